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
// sequence.  It is rounded to a bf16 hi/lo pair as an operand, and u, kg^T and
// v_new enter the state update as fp32 (hi/lo pairs), so each state-feeding
// product carries ~16 significant bits.  Every per-chunk operand is read from
// the workspace straight into registers in the matrix-core layout, one chunk
// ahead of its use; only h^T and v_new^T, which the workgroup produces itself,
// pass through LDS.
//
// Each workgroup has 4 state waves, which carry the recurrence, and in forward
// mode 4 output waves, which form o from the same h^T and v_new^T off the
// critical path.  Two workgroup barriers per chunk order the roles: h^T is
// published before the first, v_new^T before the second.
//
// Summary mode scans the augmented state [S~ | M] (K x (V + K)) from [0 | I]
// with u = [u | 0] and writes S~ and M ("KDA Context Parallelism (KCP)",
// notation and algorithm steps 1-2): the M columns see zero values, so they
// accumulate the product of the per-token transitions.
#include "kda_launch.h"

namespace kda {

namespace {

// One 8-element matrix-core operand fragment as stored in the workspace.
template <typename ST> struct Op;
template <> struct Op<bf16_t> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const bf16x8*>(p); }
};
template <> struct Op<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ Frag split() const {
    float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return split8(x);
  }
};

// acc += op * (bhi + blo)
__device__ __forceinline__ f32x4 mma_bsplit(const Op<bf16_t>& op, const bf16x8& bhi, const bf16x8& blo,
                                            f32x4 acc) {
  acc = mfma(op.v, bhi, acc);
  return mfma(op.v, blo, acc);
}
__device__ __forceinline__ f32x4 mma_bsplit(const Op<float>& op, const bf16x8& bhi, const bf16x8& blo,
                                            f32x4 acc) {
  Frag f = op.split();
  acc = mfma(f.hi, bhi, acc);
  acc = mfma(f.hi, blo, acc);
  return mfma(f.lo, bhi, acc);
}
// acc += (ahi [+ alo]) * op for the output terms: bf16 operands use the hi
// part of the LDS operand only, fp32 operands keep full precision.
__device__ __forceinline__ f32x4 mma_out_t(const bf16x8& ahi, const bf16x8&, const Op<bf16_t>& op, f32x4 acc) {
  return mfma(ahi, op.v, acc);
}
__device__ __forceinline__ f32x4 mma_out_t(const bf16x8& ahi, const bf16x8& alo, const Op<float>& op, f32x4 acc) {
  Frag f = op.split();
  acc = mfma(ahi, f.hi, acc);
  acc = mfma(alo, f.hi, acc);
  return mfma(ahi, f.lo, acc);
}
// Store 4 consecutive values.
__device__ __forceinline__ void store4(bf16_t* p, const f32x4& v) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void store4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }

template <int KD, int BV, typename ST>
struct StateFrags {
  static constexpr int NKS = KD / 32, RT = KD / 64, CT = BV / 16;
  Op<ST> w[NKS];          // w rows 16*sw + r16, channels 32*ks + 8*quad
  Op<float> kg[RT][2];    // kg^T rows 16*(RT*sw + rt) + r16, tokens 32*ks + 8*quad
  f32x4 u[CT];            // u^T row (value column) v0 + 16*ct + r16, tokens 16*sw + 4*quad .. +3
  f32x4 gd[RT];           // gdec for channels 16*(RT*sw + rt) + 4*quad .. +3
};
// Per-chunk operands of an output wave.
template <int KD, typename ST>
struct OutFrags {
  static constexpr int NKS = KD / 32;
  Op<ST> q[NKS];          // qg rows 16*ow + r16, channels 32*ks + 8*quad
  Op<ST> aq[2];           // Aqk rows 16*ow + r16, tokens 32*ks + 8*quad
};

// Workgroup: 4 state waves (v_new and the state update: the recurrence's
// critical path) and, in forward mode, 4 output waves that compute o from the
// same h^T and v_new^T while the state waves move on.
template <int KD, int VD, int BV, typename ST, bool SUM>
__global__ __launch_bounds__(SUM ? 256 : 512) void scan_kernel(ScanArgs a) {
  using SF = StateFrags<KD, BV, ST>;
  using OF = OutFrags<KD, ST>;
  constexpr int NKS = SF::NKS, RT = SF::RT, CT = SF::CT;
  constexpr int PH = KD + 8;           // h^T rows (bf16)
  constexpr int PV = 64 + 8;           // v_new^T rows (bf16)
  constexpr int VA = SUM ? VD + KD : VD;
  constexpr int NTILE = VA / BV;

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
  const int rw = wave & 3;                              // wave index within its role

  int64_t tok0s;
  int len;
  seq_range(a.seq, n, tok0s, len);
  const int nck = (len + BT - 1) / BT;
  const int cb = chunk_base(a.seq, n);
  const bool mtile = SUM && tv * BV >= VD;              // columns of M
  const int v0 = mtile ? tv * BV - VD : tv * BV;        // first column inside S~ or M

  if (wave < 4) {
    // =========================== state waves ===========================
    auto load = [&](SF& f, int c) __attribute__((always_inline)) {
      const int64_t ch = (int64_t)h * a.nchunks + cb + c;
      const ST* w = static_cast<const ST*>(a.w) + ch * (64 * KD) + (16 * rw + r16) * KD + 8 * quad;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) f.w[ks].load(w + 32 * ks);
      const float* kg = static_cast<const float*>(a.kgT) + ch * (KD * 64) + 8 * quad;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) f.kg[rt][ks].load(kg + (16 * (RT * rw + rt) + r16) * 64 + 32 * ks);
      const float* u = static_cast<const float*>(a.u) + ch * (VD * 64) + 16 * rw + 4 * quad;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        f.u[ct] = mtile ? zero4() : *reinterpret_cast<const f32x4*>(u + (v0 + 16 * ct + r16) * 64);
      const float* gd = a.gdec + ch * KD + 4 * quad;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) f.gd[rt] = *reinterpret_cast<const f32x4*>(gd + 16 * (RT * rw + rt));
    };

    // state tile in accumulators: rows 16*(RT*rw+rt) + 4*quad + e, col 16*ct + r16
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
          const int row = 16 * (RT * rw + rt) + 4 * quad + e, col = 16 * ct + r16;
          float x = 0.f;
          if (mtile) x = (row == v0 + col) ? 1.f : 0.f;
          else if (h0p) x = h0p[(int64_t)row * VD + v0 + col];
          hs[rt][ct][e] = x;
        }

    auto step = [&](const SF& cur, SF& nxt, int c) __attribute__((always_inline)) {
      // Unconditional prefetch (the last chunk reloads itself) so that the
      // compiler's wait counters stay exact across the loop back-edge.
      load(nxt, min(c + 1, nck - 1));
      // h^T as a bf16 hi/lo operand
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int row0 = 16 * (RT * rw + rt) + 4 * quad, col = 16 * ct + r16;
          float hv[4], lv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hv[e] = hs[rt][ct][e];
            lv[e] = hv[e] - bf2f(f2bf(hv[e]));
          }
          *reinterpret_cast<u32x2*>(sHhi + col * PH + row0) = u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
          *reinterpret_cast<u32x2*>(sHlo + col * PH + row0) = u32x2{pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3])};
        }
      __syncthreads();

      // ---- v_new = u - w h   (token rows 16*rw .. +15)
      bf16x8 bh[CT][NKS], bl[CT][NKS];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int off = (16 * ct + r16) * PH + 32 * ks + 8 * quad;
          bh[ct][ks] = load_bf16x8(sHhi + off);
          bl[ct][ks] = load_bf16x8(sHlo + off);
        }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc = mma_bsplit(cur.w[ks], bh[ct][ks], bl[ct][ks], acc);
        const int t0 = 16 * rw + 4 * quad, col = 16 * ct + r16;
        float vn[4], lv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vn[e] = cur.u[ct][e] - acc[e];
          lv[e] = vn[e] - bf2f(f2bf(vn[e]));
        }
        *reinterpret_cast<u32x2*>(sVhi + col * PV + t0) = u32x2{pack_bf16x2(vn[0], vn[1]), pack_bf16x2(vn[2], vn[3])};
        *reinterpret_cast<u32x2*>(sVlo + col * PV + t0) = u32x2{pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3])};
      }
      __syncthreads();

      // ---- h = Diag(gdec) h + kg^T v_new
      bf16x8 vh[CT][2], vl[CT][2];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int off = (16 * ct + r16) * PV + 32 * ks + 8 * quad;
          vh[ct][ks] = load_bf16x8(sVhi + off);
          vl[ct][ks] = load_bf16x8(sVlo + off);
        }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const Frag kf[2] = {cur.kg[rt][0].split(), cur.kg[rt][1].split()};
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          f32x4 acc = hs[rt][ct];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] *= cur.gd[rt][e];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            acc = mfma(kf[ks].hi, vh[ct][ks], acc);
            acc = mfma(kf[ks].hi, vl[ct][ks], acc);
            acc = mfma(kf[ks].lo, vh[ct][ks], acc);
          }
          hs[rt][ct] = acc;
        }
      }
    };

    SF fa, fb;
    if (nck > 0) load(fa, 0);
    for (int c = 0; c < nck; c += 2) {
      step(fa, fb, c);
      if (c + 1 < nck) step(fb, fa, c + 1);
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
            const int row = 16 * (RT * rw + rt) + 4 * quad + e, col = 16 * ct + r16;
            dst[(int64_t)row * ld + v0 + col] = hs[rt][ct][e];
          }
    }
  } else if constexpr (!SUM) {
    // =========================== output waves ==========================
    auto load = [&](OF& f, int c) __attribute__((always_inline)) {
      const int64_t ch = (int64_t)h * a.nchunks + cb + c;
      const ST* q = static_cast<const ST*>(a.qg) + ch * (64 * KD) + (16 * rw + r16) * KD + 8 * quad;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) f.q[ks].load(q + 32 * ks);
      const ST* aq = static_cast<const ST*>(a.Aqk) + ch * (64 * 64) + (16 * rw + r16) * 64 + 8 * quad;
      f.aq[0].load(aq);
      f.aq[1].load(aq + 32);
    };
    ST* op = static_cast<ST*>(a.o);
    auto step = [&](const OF& cur, OF& nxt, int c) __attribute__((always_inline)) {
      // Unconditional prefetch (the last chunk reloads itself) so that the
      // compiler's wait counters stay exact across the loop back-edge.
      load(nxt, min(c + 1, nck - 1));
      __syncthreads();
      // o^T = h^T qg^T (needs only h^T; overlaps the state waves' v_new).  The
      // transposed tile gives each lane 4 consecutive value columns of one
      // token, stored as one 8-byte (bf16) or 16-byte (fp32) write.
      f32x4 acc[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        acc[ct] = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int off = (16 * ct + r16) * PH + 32 * ks + 8 * quad;
          acc[ct] = mma_out_t(load_bf16x8(sHhi + off), load_bf16x8(sHlo + off), cur.q[ks], acc[ct]);
        }
      }
      __syncthreads();
      // o^T += v_new^T tril(Aqk)^T
      const int t = 16 * rw + r16;                       // this lane's token
      const bool tok_ok = t < min(BT, len - c * BT);
      ST* orow = op + (tok0s + (int64_t)c * BT + t) * (int64_t)(a.Hv * VD) + (int64_t)h * VD + v0 + 4 * quad;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks * 2 <= rw) {     // Aqk is lower triangular
            const int off = (16 * ct + r16) * PV + 32 * ks + 8 * quad;
            acc[ct] = mma_out_t(load_bf16x8(sVhi + off), load_bf16x8(sVlo + off), cur.aq[ks], acc[ct]);
          }
        }
        if (tok_ok) store4(orow + 16 * ct, acc[ct]);
      }
    };
    OF fa, fb;
    if (nck > 0) load(fa, 0);
    for (int c = 0; c < nck; c += 2) {
      step(fa, fb, c);
      if (c + 1 < nck) step(fb, fa, c + 1);
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
  dim3 grid((unsigned)nb), block(a.summary ? 256 : 512);
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
