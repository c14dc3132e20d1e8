// Token-by-token KDA forward for decode and other short sequences: the
// recurrent form of the method, with the state held in registers.
//
// Follows the recurrent decode step of the vllm-ascend KDA prefill state-copy
// page (background section: one token per sequence, the state cache read and
// written in place) and the token recurrence itself ("KDA Context Parallelism
// (KCP)", notation; "KDA Chunk Backward — TPU/Pallas Kernel Design", section 1):
//     S' = Diag(alpha_t) S;  e = v_t - S'^T k_t;  S = S' + beta_t k_t e^T;  o_t = scale S^T q_t
// with the gate, L2Norm and sigmoid of "Hyper-Parallel Chunk KDA" section 4.
//
// One wave per (sequence, value head, 64-column slice of the state).  Lane l
// holds columns c0 + 4*(l % 16) .. +3 of the rows r = 4*i + l/16 (i = 0 ..
// K/4 - 1): the state slice is read and written with 16-byte accesses, one
// coalesced 1 KiB block per four rows.  Sums over the K rows are a lane's own
// partial sum plus two cross-lane steps (lanes l, l^16, l^32, l^48).  Per
// token the 128 per-channel values (decay, normalised k and q) are formed two
// per lane and shared through LDS.  Everything is fp32; the cost is the state's
// HBM round trip (K*V*8 bytes per sequence and head).
#include "kda_launch.h"

namespace kda {

namespace {

template <typename T> __device__ __forceinline__ float ld1(const T* p);
template <> __device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld1<bf16_t>(const bf16_t* p) { return bf2f(*p); }

__device__ __forceinline__ float softplus(float x) {
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}

template <int KD, int VD, typename IT>
__global__ __launch_bounds__(64) void recurrent_kernel(RecurrentArgs a) {
  constexpr int RPL = KD / 4;                       // state rows per lane
  __shared__ float sAlpha[KD], sK[KD], sQ[KD];
  const int lane = threadIdx.x;
  constexpr int NSL = VD / 64;                      // column slices per head
  const int slice = blockIdx.x % NSL;
  const int h = (blockIdx.x / NSL) % a.Hv;
  const int n = blockIdx.x / (NSL * a.Hv);
  const int hk = h / (a.Hv / a.Hk);
  const int c0 = 64 * slice + 4 * (lane & 15), rg = lane >> 4;

  int64_t tok0;
  int len;
  seq_range(a.seq, n, tok0, len);

  // ---- initial state (cache row, dense row or zero)
  const float* src = nullptr;
  float* dst = nullptr;
  if (a.state_rows > 0) {
    const int r = a.state_idx[n];
    if (r >= 0 && r < a.state_rows) {
      if (a.h0) src = a.h0 + ((int64_t)r * a.Hv + h) * (int64_t)(KD * VD);
      if (a.hT) dst = a.hT + ((int64_t)r * a.Hv + h) * (int64_t)(KD * VD);
    }
  } else {
    if (a.h0) src = a.h0 + ((int64_t)n * a.Hv + h) * (int64_t)(KD * VD);
    if (a.hT) dst = a.hT + ((int64_t)n * a.Hv + h) * (int64_t)(KD * VD);
  }
  f32x4 S[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i)
    S[i] = src ? *reinterpret_cast<const f32x4*>(src + (int64_t)(4 * i + rg) * VD + c0) : zero4();

  const bool gik = a.flags & F_GATE, l2 = a.flags & F_L2;
  const float lb = (a.flags & F_SAFE) ? a.lower_bound : -INFINITY;
  const float Aexp = gik ? expf(a.A_log[h]) : 0.f;
  float bias[2] = {0.f, 0.f};
  if (gik && a.dt_bias) {
    bias[0] = a.dt_bias[h * KD + lane];
    if (KD > 64) bias[1] = a.dt_bias[h * KD + 64 + lane];
  }
  const IT* q = static_cast<const IT*>(a.q);
  const IT* k = static_cast<const IT*>(a.k);
  const IT* v = static_cast<const IT*>(a.v);
  const IT* g = static_cast<const IT*>(a.g);
  const IT* bt = static_cast<const IT*>(a.beta);
  IT* o = static_cast<IT*>(a.o);

  for (int t = 0; t < len; ++t) {
    const int64_t tok = tok0 + t;
    // ---- per-channel values of this token: two channels per lane
    float kc[2], qc[2], al[2];
    float skk = 0.f, sqq = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = lane + 64 * j;
      kc[j] = qc[j] = al[j] = 0.f;
      if (c < KD) {
        kc[j] = ld1(k + (tok * a.Hk + hk) * KD + c);
        qc[j] = ld1(q + (tok * a.Hk + hk) * KD + c);
        float gv = ld1(g + (tok * a.Hv + h) * KD + c);
        if (gik) gv = -Aexp * softplus(gv + bias[j]);
        al[j] = expf(gv < lb ? lb : gv);          // (a NaN gate stays NaN)
      }
      skk += kc[j] * kc[j];
      sqq += qc[j] * qc[j];
    }
    if (l2) {
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        skk += __shfl_xor(skk, m);
        sqq += __shfl_xor(sqq, m);
      }
    }
    const float rk = l2 ? 1.f / sqrtf(skk + a.eps) : 1.f;
    const float rq = a.scale * (l2 ? 1.f / sqrtf(sqq + a.eps) : 1.f);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = lane + 64 * j;
      if (c < KD) {
        sAlpha[c] = al[j];
        sK[c] = kc[j] * rk;
        sQ[c] = qc[j] * rq;
      }
    }
    float beta = ld1(bt + tok * a.Hv + h);
    if (a.flags & F_SIGMOID) beta = 1.f / (1.f + expf(-beta));
    f32x4 vv;
    {
      const IT* vp = v + (tok * a.Hv + h) * VD + c0;
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[e] = ld1(vp + e);
    }
    __syncthreads();
    // ---- decay, then the prediction S'^T k of this lane's columns
    f32x4 pred = zero4();
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int r = 4 * i + rg;
      const float ar = sAlpha[r], kr = sK[r];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[i][e] *= ar;
        pred[e] += S[i][e] * kr;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pred[e] += __shfl_xor(pred[e], 16);
      pred[e] += __shfl_xor(pred[e], 32);
    }
    f32x4 ev;
#pragma unroll
    for (int e = 0; e < 4; ++e) ev[e] = beta * (vv[e] - pred[e]);
    // ---- write and read out
    f32x4 out = zero4();
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int r = 4 * i + rg;
      const float kr = sK[r], qr = sQ[r];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[i][e] += kr * ev[e];
        out[e] += S[i][e] * qr;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[e] += __shfl_xor(out[e], 16);
      out[e] += __shfl_xor(out[e], 32);
    }
    if (rg == 0) {
      IT* op = o + (tok * a.Hv + h) * VD + c0;
#pragma unroll
      for (int e = 0; e < 4; ++e) op[e] = from_f<IT>(out[e]);
    }
    __syncthreads();   // the next token overwrites the shared channel values
  }

  if (dst) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) *reinterpret_cast<f32x4*>(dst + (int64_t)(4 * i + rg) * VD + c0) = S[i];
  }
}

}  // namespace

hipError_t launch_recurrent(int K, int V, int dtype, const RecurrentArgs& a, hipStream_t s) {
  if (a.seq.N == 0 || a.Hv == 0) return hipSuccess;
  const long nb = (long)a.seq.N * a.Hv * (V / 64);
  if (nb > 0x7fffffffL) return hipErrorInvalidValue;
#define KDA_REC_CASE(KK, VV, TT)                                                                  \
  if (K == KK && V == VV) return launch(recurrent_kernel<KK, VV, TT>, dim3((unsigned)nb), dim3(64), s, a);
  if (dtype == 1) {
    KDA_REC_CASE(128, 128, bf16_t)
    KDA_REC_CASE(64, 64, bf16_t)
    KDA_REC_CASE(128, 64, bf16_t)
    KDA_REC_CASE(64, 128, bf16_t)
  } else {
    KDA_REC_CASE(128, 128, float)
    KDA_REC_CASE(64, 64, float)
    KDA_REC_CASE(128, 64, float)
    KDA_REC_CASE(64, 128, float)
  }
#undef KDA_REC_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
