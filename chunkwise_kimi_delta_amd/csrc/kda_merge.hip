// Prefix merge of segment summaries ("KDA Context Parallelism (KCP)",
// algorithm step 4; "Hyper-Parallel Chunk KDA" section 5.3, forward merge):
// for j = 0..P-1 in order, state <- M_j state + S~_j, in fp32.
// One workgroup per (value head, 32-column tile of the state); the state tile
// stays in LDS across the P steps and each M_j is staged through LDS.
#include "kda_launch.h"

namespace kda {

namespace {

// BWD: the reverse merge of the backward, state <- M_j^T state + S_j for
// j = P-1 down to 0 ("Hyper-Parallel Chunk KDA" section 6.4; "KDA Chunk
// Backward — TPU/Pallas Kernel Design" section 2.4): M_j is staged transposed.
template <int KD, int VD, bool BWD>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int BVm = 32, PS = BVm + 4, PM = KD + 4;
  constexpr int RPT = KD * BVm / 256;            // outputs per thread
  __shared__ __attribute__((aligned(16))) float sS[KD * PS];
  __shared__ __attribute__((aligned(16))) float sM[KD * PM];
  const int tile = blockIdx.x % (VD / BVm), h = blockIdx.x / (VD / BVm);
  const int v0 = tile * BVm, tid = threadIdx.x;
  const int col = tid % BVm, rg = tid / BVm;     // rows rg, rg + 8, ...
  float* st = a.state + (int64_t)h * KD * VD;
  for (int i = tid; i < KD * BVm; i += 256) sS[(i / BVm) * PS + i % BVm] = st[(i / BVm) * VD + v0 + i % BVm];
  for (int jj = 0; jj < a.P; ++jj) {
    const int j = BWD ? a.P - 1 - jj : jj;
    const float* Mj = a.M + ((int64_t)j * a.Hv + h) * KD * KD;
    const float* Sj = a.S + ((int64_t)j * a.Hv + h) * KD * VD;
    for (int i = tid * 4; i < KD * KD; i += 256 * 4) {
      f32x4 x = *reinterpret_cast<const f32x4*>(Mj + i);
      if (BWD) {   // row r of M^T is column r of M
#pragma unroll
        for (int e = 0; e < 4; ++e) sM[((i + e) % KD) * PM + (i + e) / KD] = x[e];
      } else {
        *reinterpret_cast<f32x4*>(sM + (i / KD) * PM + i % KD) = x;
      }
    }
    __syncthreads();
    float acc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) acc[r] = Sj[(int64_t)(rg + 8 * r) * VD + v0 + col];
    for (int m = 0; m < KD; m += 4) {
      float s0 = sS[(m + 0) * PS + col], s1 = sS[(m + 1) * PS + col];
      float s2 = sS[(m + 2) * PS + col], s3 = sS[(m + 3) * PS + col];
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        f32x4 mv = *reinterpret_cast<const f32x4*>(sM + (rg + 8 * r) * PM + m);
        acc[r] += mv.x * s0 + mv.y * s1 + mv.z * s2 + mv.w * s3;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RPT; ++r) sS[(rg + 8 * r) * PS + col] = acc[r];
    __syncthreads();
  }
  for (int i = tid; i < KD * BVm; i += 256) st[(i / BVm) * VD + v0 + i % BVm] = sS[(i / BVm) * PS + i % BVm];
}

// Incoming states of the segments of each sequence (segment-parallel scan):
// h_in[s + 1] = M_s h_in[s] + S~_s for s = 0 .. nseg - 2, h_in[0] the
// sequence's initial state (dense row, cache row or zero) -- the forward merge
// of "KDA Context Parallelism (KCP)", algorithm step 4, with every prefix
// kept.  One workgroup per (sequence, value head, 32-column tile), the state
// tile in LDS, each M_s staged through LDS, fp32 FMA.
template <int KD, int VD>
__global__ __launch_bounds__(256) void prefix_merge_kernel(PrefixMergeArgs a) {
  constexpr int BVm = 32, PS = BVm + 4, PM = KD + 4;
  constexpr int RPT = KD * BVm / 256;
  __shared__ __attribute__((aligned(16))) float sS[KD * PS];
  __shared__ __attribute__((aligned(16))) float sM[KD * PM];
  constexpr int NT = VD / BVm;
  const int tile = blockIdx.x % NT, h = (blockIdx.x / NT) % a.Hv, n = blockIdx.x / (NT * a.Hv);
  int64_t tok0;
  int len;
  seq_range(a.seq, n, tok0, len);
  const int nck = (len + BT - 1) / BT;
  const int nseg = (nck + a.seg_len - 1) / a.seg_len;
  if (nseg < 2) return;
  const float* src = nullptr;
  if (a.state_rows > 0) {
    const int r = a.state_idx[n];
    if (r >= 0 && r < a.state_rows && a.h0) src = a.h0 + ((int64_t)r * a.Hv + h) * (KD * VD);
  } else if (a.h0) {
    src = a.h0 + ((int64_t)n * a.Hv + h) * (KD * VD);
  }
  const int v0 = tile * BVm, tid = threadIdx.x;
  const int col = tid % BVm, rg = tid / BVm;     // rows rg, rg + 8, ...
  for (int i = tid; i < KD * BVm; i += 256)
    sS[(i / BVm) * PS + i % BVm] = src ? src[(i / BVm) * VD + v0 + i % BVm] : 0.f;
  for (int s = 0; s + 1 < nseg; ++s) {
    const int64_t j = (int64_t)n * a.seg_max + s;
    const float* Mj = a.M + (j * a.Hv + h) * (KD * KD);
    const float* Sj = a.S + (j * a.Hv + h) * (KD * VD);
    for (int i = tid * 4; i < KD * KD; i += 256 * 4) {
      f32x4 x = *reinterpret_cast<const f32x4*>(Mj + i);
      *reinterpret_cast<f32x4*>(sM + (i / KD) * PM + i % KD) = x;
    }
    __syncthreads();
    float acc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) acc[r] = Sj[(int64_t)(rg + 8 * r) * VD + v0 + col];
    for (int m = 0; m < KD; m += 4) {
      float s0 = sS[(m + 0) * PS + col], s1 = sS[(m + 1) * PS + col];
      float s2 = sS[(m + 2) * PS + col], s3 = sS[(m + 3) * PS + col];
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        f32x4 mv = *reinterpret_cast<const f32x4*>(sM + (rg + 8 * r) * PM + m);
        acc[r] += mv.x * s0 + mv.y * s1 + mv.z * s2 + mv.w * s3;
      }
    }
    __syncthreads();
    float* out = a.h_in + ((j + 1) * a.Hv + h) * (KD * VD);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      sS[(rg + 8 * r) * PS + col] = acc[r];
      out[(int64_t)(rg + 8 * r) * VD + v0 + col] = acc[r];
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_prefix_merge(int K, int V, const PrefixMergeArgs& a, hipStream_t s) {
  if (a.seq.N == 0 || a.Hv == 0 || a.seg_max < 2) return hipSuccess;
  const long nb = (long)a.seq.N * a.Hv * (V / 32);
  if (nb > 0x7fffffffL) return hipErrorInvalidValue;
#define KDA_PMERGE_CASE(KK, VV) \
  if (K == KK && V == VV) return launch(prefix_merge_kernel<KK, VV>, dim3((unsigned)nb), dim3(256), s, a);
  KDA_PMERGE_CASE(128, 128)
  KDA_PMERGE_CASE(64, 64)
  KDA_PMERGE_CASE(128, 64)
  KDA_PMERGE_CASE(64, 128)
#undef KDA_PMERGE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_merge(int K, int V, const MergeArgs& a, hipStream_t s, bool backward) {
  if (a.P == 0 || a.Hv == 0) return hipSuccess;
#define KDA_MERGE_CASE(KK, VV)                                                                       \
  if (K == KK && V == VV) {                                                                          \
    return backward ? launch(merge_kernel<KK, VV, true>, dim3(a.Hv * (VV / 32)), dim3(256), s, a)    \
                    : launch(merge_kernel<KK, VV, false>, dim3(a.Hv * (VV / 32)), dim3(256), s, a);  \
  }
  KDA_MERGE_CASE(128, 128)
  KDA_MERGE_CASE(64, 64)
  KDA_MERGE_CASE(128, 64)
  KDA_MERGE_CASE(64, 128)
#undef KDA_MERGE_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
