// Inter-chunk KDA state scan with the fused chunk output, one workgroup
// (4 waves) per (value tile of BV columns, value head, sequence).
//
// Follows "KDA Chunk Backward — TPU/Pallas Kernel Design", sections 1 and 1.2
// (the forward output, v_new = u - w h, the inter-chunk recurrence) and the
// state / finalize stages of "Hyper-Parallel Chunk KDA" section 5.1.  For
// each chunk in order, with h the K x BV state tile at the chunk entry:
//   v_new = u - w h
//   o     = qg h + tril(Aqk) v_new               (forward mode only)
//   h     = Diag(gdec) h + kg^T v_new
// The state stays in the matrix-core accumulators (fp32) for the whole
// sequence; it is rounded to a bf16 hi/lo pair only as an operand, and u,
// kg^T and v_new enter the state update as fp32 (hi/lo pairs), so each
// state-feeding product carries ~16 significant bits.  The next chunk's
// inputs are prefetched into registers while the current chunk computes.
//
// Summary mode scans the augmented state [S~ | M] (K x (V + K)) from [0 | I]
// with u = [u | 0] and writes S~ and M ("KDA Context Parallelism (KCP)",
// notation and algorithm steps 1-2): the M columns see zero values, so they
// accumulate the product of the per-token transitions.
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
constexpr int imax(int a, int b) { return a > b ? a : b; }

template <int KD, int VD, int BV, typename ST, bool SUM>
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
  constexpr int NTH = 256;
  constexpr bool F32 = sizeof(ST) == 4;
  constexpr int ES = sizeof(ST);
  constexpr int EI = 16 / ES;
  constexpr int PK = KD + EI;          // rows of K elements (w, qg), ST
  constexpr int PT = 64 + EI;          // rows of 64 elements (Aqk), ST
  constexpr int PKG = 64 + 4;          // kg^T rows (fp32)
  constexpr int PU = BV + 4;           // u tile rows (fp32)
  constexpr int PH = KD + 8;           // h^T rows (bf16)
  constexpr int PV = 64 + 8;           // v_new^T rows (bf16)
  constexpr int VA = SUM ? VD + KD : VD;
  constexpr int NTILE = VA / BV;
  constexpr int RT = KD / 64;          // h row tiles per wave
  constexpr int CT = BV / 16;          // column tiles

  __shared__ __attribute__((aligned(16))) ST sW[64 * PK];
  __shared__ __attribute__((aligned(16))) float sKg[KD * PKG];
  __shared__ __attribute__((aligned(16))) ST sQg[SUM ? 8 : 64 * PK];
  __shared__ __attribute__((aligned(16))) ST sAq[SUM ? 8 : 64 * PT];
  __shared__ __attribute__((aligned(16))) float sU[64 * PU];
  __shared__ __attribute__((aligned(16))) float sGd[KD];
  __shared__ __attribute__((aligned(16))) bf16_t sHhi[BV * PH];
  __shared__ __attribute__((aligned(16))) bf16_t sHlo[BV * PH];
  __shared__ __attribute__((aligned(16))) bf16_t sVhi[BV * PV];
  __shared__ __attribute__((aligned(16))) bf16_t sVlo[BV * PV];

  // ---- block -> (tile, head, sequence); tiles of one (head, sequence) share an XCD
  int lid = blockIdx.x;
  const int NB = gridDim.x;
  if ((NB & 7) == 0) lid = (lid & 7) * (NB >> 3) + (lid >> 3);
  const int tv = lid % NTILE;
  const int h = (lid / NTILE) % a.Hv;
  const int n = lid / (NTILE * a.Hv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, quad = lane >> 4;

  int64_t tok0s;
  int len;
  seq_range(a.seq, n, tok0s, len);
  const int nck = (len + BT - 1) / BT;
  const int cb = chunk_base(a.seq, n);
  const bool mtile = SUM && tv * BV >= VD;              // columns of M
  const int v0 = mtile ? tv * BV - VD : tv * BV;        // first column inside S~ or M

  // ---- register staging of one chunk's inputs (16-byte pieces)
  constexpr int NWp = 64 * KD * ES / 16, NKp = KD * 64 * 4 / 16;
  constexpr int NQp = SUM ? 0 : 64 * KD * ES / 16, NAp = SUM ? 0 : 64 * 64 * ES / 16;
  constexpr int NUp = 64 * BV * 4 / 16, NGp = KD * 4 / 16;
  constexpr int CW = cdiv(NWp, NTH), CK = cdiv(NKp, NTH), CQ = imax(1, cdiv(NQp, NTH));
  constexpr int CA = imax(1, cdiv(NAp, NTH)), CU = cdiv(NUp, NTH), CG = cdiv(NGp, NTH);
  u32x4 rW[CW], rK[CK], rQ[CQ], rA[CA], rU[CU], rG[CG];

  auto load_chunk = [&](int c) __attribute__((always_inline)) {
    const int64_t ch = (int64_t)h * a.nchunks + cb + c;
    const u32x4* gw = reinterpret_cast<const u32x4*>(static_cast<const ST*>(a.w) + ch * (64 * KD));
    const u32x4* gk = reinterpret_cast<const u32x4*>(static_cast<const float*>(a.kgT) + ch * (64 * KD));
#pragma unroll
    for (int i = 0; i < CW; ++i) { int p = tid + i * NTH; if (p < NWp) rW[i] = gw[p]; }
#pragma unroll
    for (int i = 0; i < CK; ++i) { int p = tid + i * NTH; if (p < NKp) rK[i] = gk[p]; }
    if (!SUM) {
      const u32x4* gq = reinterpret_cast<const u32x4*>(static_cast<const ST*>(a.qg) + ch * (64 * KD));
      const u32x4* ga = reinterpret_cast<const u32x4*>(static_cast<const ST*>(a.Aqk) + ch * (64 * 64));
#pragma unroll
      for (int i = 0; i < CQ; ++i) { int p = tid + i * NTH; if (p < NQp) rQ[i] = gq[p]; }
#pragma unroll
      for (int i = 0; i < CA; ++i) { int p = tid + i * NTH; if (p < NAp) rA[i] = ga[p]; }
    }
    const float* gu = static_cast<const float*>(a.u) + ch * (64 * VD) + v0;
    constexpr int UPR = BV / 4;           // pieces per u row
#pragma unroll
    for (int i = 0; i < CU; ++i) {
      int p = tid + i * NTH;
      if (p < NUp) {
        if (mtile) rU[i] = u32x4{0u, 0u, 0u, 0u};
        else rU[i] = *reinterpret_cast<const u32x4*>(gu + (p / UPR) * VD + (p % UPR) * 4);
      }
    }
    const u32x4* gg = reinterpret_cast<const u32x4*>(a.gdec + ch * KD);
#pragma unroll
    for (int i = 0; i < CG; ++i) { int p = tid + i * NTH; if (p < NGp) rG[i] = gg[p]; }
  };
  auto stage_chunk = [&]() __attribute__((always_inline)) {
    constexpr int WPR = KD * ES / 16, KPR = 64 * ES / 16, KGPR = 64 / 4, UPR = BV / 4;
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      int p = tid + i * NTH;
      if (p < NWp) *reinterpret_cast<u32x4*>(sW + (p / WPR) * PK + (p % WPR) * EI) = rW[i];
    }
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      int p = tid + i * NTH;
      if (p < NKp) *reinterpret_cast<u32x4*>(sKg + (p / KGPR) * PKG + (p % KGPR) * 4) = rK[i];
    }
    if (!SUM) {
#pragma unroll
      for (int i = 0; i < CQ; ++i) {
        int p = tid + i * NTH;
        if (p < NQp) *reinterpret_cast<u32x4*>(sQg + (p / WPR) * PK + (p % WPR) * EI) = rQ[i];
      }
#pragma unroll
      for (int i = 0; i < CA; ++i) {
        int p = tid + i * NTH;
        if (p < NAp) *reinterpret_cast<u32x4*>(sAq + (p / KPR) * PT + (p % KPR) * EI) = rA[i];
      }
    }
#pragma unroll
    for (int i = 0; i < CU; ++i) {
      int p = tid + i * NTH;
      if (p < NUp) *reinterpret_cast<u32x4*>(sU + (p / UPR) * PU + (p % UPR) * 4) = rU[i];
    }
#pragma unroll
    for (int i = 0; i < CG; ++i) {
      int p = tid + i * NTH;
      if (p < NGp) *reinterpret_cast<u32x4*>(sGd + p * 4) = rG[i];
    }
  };

  // ---- state tile in accumulators: rows 16*(RT*wave+rt) + 4*quad + e, col 16*ct + r16
  f32x4 hs[RT][CT];
  const float* h0p = nullptr;
  bool valid_row = true;
  int64_t srow = n;
  if (!SUM) {
    if (a.state_rows > 0) {
      const int r = a.state_idx[n];
      valid_row = r >= 0 && r < a.state_rows;
      srow = r;
      if (valid_row && a.h0) h0p = a.h0 + (srow * a.Hv + h) * (int64_t)(KD * VD);
    } else if (a.h0) {
      h0p = a.h0 + ((int64_t)n * a.Hv + h) * (int64_t)(KD * VD);
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * (RT * wave + rt) + 4 * quad + e, col = 16 * ct + r16;
        float x = 0.f;
        if (mtile) x = (row == v0 + col) ? 1.f : 0.f;
        else if (h0p) x = h0p[(int64_t)row * VD + v0 + col];
        hs[rt][ct][e] = x;
      }

  if (nck > 0) load_chunk(0);
  for (int c = 0; c < nck; ++c) {
    stage_chunk();
    // h^T as bf16 hi/lo operand
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int row0 = 16 * (RT * wave + rt) + 4 * quad, col = 16 * ct + r16;
        uint32_t hi01, hi23, lo01, lo23;
        float hv[4], lv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hv[e] = hs[rt][ct][e];
          lv[e] = hv[e] - bf2f(f2bf(hv[e]));
        }
        hi01 = pack_bf16x2(hv[0], hv[1]);
        hi23 = pack_bf16x2(hv[2], hv[3]);
        lo01 = pack_bf16x2(lv[0], lv[1]);
        lo23 = pack_bf16x2(lv[2], lv[3]);
        *reinterpret_cast<u32x2*>(sHhi + col * PH + row0) = u32x2{hi01, hi23};
        *reinterpret_cast<u32x2*>(sHlo + col * PH + row0) = u32x2{lo01, lo23};
      }
    __syncthreads();
    if (c + 1 < nck) load_chunk(c + 1);

    // ---- v_new = u - w h   (wave: token rows 16*wave .. +15)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < KD / 32; ++ks) {
        const int k0 = ks * 32 + 8 * quad;
        acc = mma_a_bsplit(sW + (16 * wave + r16) * PK + k0, sHhi + (16 * ct + r16) * PH + k0,
                           sHlo + (16 * ct + r16) * PH + k0, acc);
      }
      const int t0 = 16 * wave + 4 * quad, col = 16 * ct + r16;
      float vn[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vn[e] = sU[(t0 + e) * PU + col] - acc[e];
      float lv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) lv[e] = vn[e] - bf2f(f2bf(vn[e]));
      *reinterpret_cast<u32x2*>(sVhi + col * PV + t0) =
          u32x2{pack_bf16x2(vn[0], vn[1]), pack_bf16x2(vn[2], vn[3])};
      *reinterpret_cast<u32x2*>(sVlo + col * PV + t0) =
          u32x2{pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3])};
    }
    __syncthreads();

    // ---- o = qg h + tril(Aqk) v_new
    if (!SUM) {
      const int Cn = min(BT, len - c * BT);
      const int64_t tokc = tok0s + (int64_t)c * BT;
      ST* op = static_cast<ST*>(a.o);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < KD / 32; ++ks) {
          const int k0 = ks * 32 + 8 * quad;
          if (F32)
            acc = mma_a_bsplit(sQg + (16 * wave + r16) * PK + k0, sHhi + (16 * ct + r16) * PH + k0,
                               sHlo + (16 * ct + r16) * PH + k0, acc);
          else
            acc = mma_a_bhi(sQg + (16 * wave + r16) * PK + k0, sHhi + (16 * ct + r16) * PH + k0, acc);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks * 2 <= wave) {     // Aqk is lower triangular
            const int k0 = ks * 32 + 8 * quad;
            if (F32)
              acc = mma_a_bsplit(sAq + (16 * wave + r16) * PT + k0, sVhi + (16 * ct + r16) * PV + k0,
                                 sVlo + (16 * ct + r16) * PV + k0, acc);
            else
              acc = mma_a_bhi(sAq + (16 * wave + r16) * PT + k0, sVhi + (16 * ct + r16) * PV + k0, acc);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * wave + 4 * quad + e;
          if (t < Cn)
            op[(tokc + t) * (int64_t)(a.Hv * VD) + (int64_t)h * VD + v0 + 16 * ct + r16] = from_f<ST>(acc[e]);
        }
      }
    }

    // ---- h = Diag(gdec) h + kg^T v_new
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int R = RT * wave + rt;
      float gd[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) gd[e] = sGd[16 * R + 4 * quad + e];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        f32x4 acc = hs[rt][ct];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= gd[e];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int k0 = ks * 32 + 8 * quad;
          acc = mma_a_bsplit(sKg + (16 * R + r16) * PKG + k0, sVhi + (16 * ct + r16) * PV + k0,
                             sVlo + (16 * ct + r16) * PV + k0, acc);
        }
        hs[rt][ct] = acc;
      }
    }
    __syncthreads();
  }

  // ---- final state
  float* dst = nullptr;
  int64_t ld = VD;
  if (SUM) {
    if (mtile) { dst = a.M + ((int64_t)n * a.Hv + h) * (int64_t)(KD * KD); ld = KD; }
    else dst = a.hT + ((int64_t)n * a.Hv + h) * (int64_t)(KD * VD);
  } else if (a.hT) {
    if (a.state_rows > 0) {
      if (valid_row) dst = a.hT + (srow * a.Hv + h) * (int64_t)(KD * VD);
    } else {
      dst = a.hT + ((int64_t)n * a.Hv + h) * (int64_t)(KD * VD);
    }
  }
  if (dst) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * (RT * wave + rt) + 4 * quad + e, col = 16 * ct + r16;
          dst[(int64_t)row * ld + v0 + col] = hs[rt][ct][e];
        }
  }
}

// Exclusive prefix of per-sequence chunk counts (one workgroup).
__global__ __launch_bounds__(256) void chunk_offsets_kernel(const int32_t* cu, int N, int32_t* off) {
  __shared__ int32_t part[256];
  const int t = threadIdx.x;
  const int per = (N + 255) / 256;
  const int b = t * per, e = min(N, b + per);
  int32_t s = 0;
  for (int i = b; i < e; ++i) s += (cu[i + 1] - cu[i] + BT - 1) / BT;
  part[t] = s;
  __syncthreads();
  if (t == 0) {
    int32_t run = 0;
    for (int i = 0; i < 256; ++i) { int32_t x = part[i]; part[i] = run; run += x; }
  }
  __syncthreads();
  int32_t run = part[t];
  for (int i = b; i < e; ++i) {
    off[i] = run;
    run += (cu[i + 1] - cu[i] + BT - 1) / BT;
  }
  if (e == N && b < e) off[N] = run;
  if (N == 0 && t == 0) off[0] = 0;
}

}  // namespace

hipError_t launch_chunk_offsets(const int32_t* cu, int N, int32_t* chunk_off, hipStream_t s) {
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(256), 0, s, cu, N, chunk_off);
  return hipGetLastError();
}

hipError_t launch_scan(int K, int V, int dtype, const ScanArgs& a, hipStream_t s) {
  constexpr int BV = 32;
  if (a.seq.N == 0 || a.Hv == 0) return hipSuccess;
  const int VA = a.summary ? V + K : V;
  const long nb = (long)(VA / BV) * a.Hv * a.seq.N;
  if (nb > 0x7fffffffL) return hipErrorInvalidValue;
  dim3 grid((unsigned)nb), block(256);
#define KDA_SCAN_CASE(KK, VV, TT)                                                    \
  if (K == KK && V == VV) {                                                          \
    if (a.summary) hipLaunchKernelGGL((scan_kernel<KK, VV, BV, TT, true>), grid, block, 0, s, a); \
    else hipLaunchKernelGGL((scan_kernel<KK, VV, BV, TT, false>), grid, block, 0, s, a);          \
    return hipGetLastError();                                                        \
  }
  if (dtype == 1) {
    KDA_SCAN_CASE(128, 128, bf16_t)
    KDA_SCAN_CASE(64, 64, bf16_t)
    KDA_SCAN_CASE(128, 64, bf16_t)
    KDA_SCAN_CASE(64, 128, bf16_t)
  } else {
    KDA_SCAN_CASE(64, 64, float)
    KDA_SCAN_CASE(64, 128, float)
  }
#undef KDA_SCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
