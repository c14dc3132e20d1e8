// Chunk-local KDA work, one workgroup (8 waves) per (64-token chunk, value head).
//
// Follows "KDA Chunk Backward — TPU/Pallas Kernel Design", section 1.2 (WY
// representation, log2-space chunk-local gate) and section 3.7 (sub-block
// normalisation with a reference gate), and the prepare stage of
// "Hyper-Parallel Chunk KDA" section 5.1 (gate, L2Norm, beta, Akk/Aqk, w, u,
// qg, kg).  Per chunk with tokens i = 0..63 (rows >= C of a partial chunk are
// zero-padded and inert):
//   gamma_i   = log2(e) * sum_{r<=i} g_r         (inclusive, per channel)
//   L_ij      = beta_i * sum_c k_ic k_jc 2^(gamma_ic - gamma_jc)   (i > j)
//   Aqk_ij    = scale  * sum_c q_ic k_jc 2^(gamma_ic - gamma_jc)   (i >= j)
//   A         = (I + L)^-1
//   u = A (beta * v),  w = A (beta * k * 2^gamma)
//   kgT = (k * 2^(gamma_C - gamma))^T,  qg = scale * q * 2^gamma,  gdec = 2^gamma_C
// u and kgT feed the state update directly and are kept in fp32; w, qg and
// Aqk are stored in the token dtype.
//
// Range safety of the decay products.  Within one chunk gamma can fall by
// hundreds, so 2^gamma_i * 2^-gamma_j overflows fp32.  Every pair i > j is
// instead evaluated at the level of a binary split of the chunk where i lies
// in the upper half and j in the lower half of one block, with the reference
// r = first row of the upper half:
//   2^(gamma_i - gamma_j) = 2^(gamma_i - gamma_r) * 2^(gamma_r - gamma_j),
// both factors <= 1.  Level 64 and 32 blocks are full 16x16 matrix-core tiles;
// levels 16, 8, 4, 2 live inside the diagonal tiles and are masked per entry.
// The diagonal of Aqk (factor 1) is a plain dot product.
#include "kda_launch.h"

namespace kda {

namespace {

template <int KD, int VD, typename IT>
__global__ __launch_bounds__(512) void intra_kernel(IntraArgs a) {
  using ST = IT;                                   // workspace element type
  constexpr int NTH = 512;
  constexpr bool F32 = sizeof(IT) == 4;
  constexpr int EI = 16 / sizeof(IT);              // elements per 16 bytes
  constexpr int PQ = KD + EI;                      // row stride of sQ / sK
  constexpr int PG = KD + 4;                       // row stride of sG (floats)
  constexpr int P64 = 64 + 4;                      // row stride of sL / sA
  constexpr int PT = 64 + EI;                      // row stride of transposed operands
  constexpr int UQ = 64 * PQ > VD * PT ? 64 * PQ : VD * PT;

  __shared__ __attribute__((aligned(16))) IT sQV[UQ];        // q, later v^T
  __shared__ __attribute__((aligned(16))) IT sK[64 * PQ];
  __shared__ __attribute__((aligned(16))) float sG[64 * PG];  // gamma (log2)
  __shared__ __attribute__((aligned(16))) float sL[64 * P64];
  __shared__ __attribute__((aligned(16))) float sA[64 * P64];
  __shared__ __attribute__((aligned(16))) ST sXT[KD * PT];    // (beta-free) k*2^gamma, transposed
  __shared__ float sTot[NTH];
  __shared__ float sX[3 * 256];
  __shared__ float sBeta[64], sRq[64], sRk[64], sDg[64];

  const int gc = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = seq_of_chunk(a.seq, gc);
  int64_t tok0s;
  int len;
  seq_range(a.seq, n, tok0s, len);
  const int cidx = gc - chunk_base(a.seq, n);
  const int64_t tok0 = tok0s + (int64_t)cidx * BT;
  const int C = min(BT, len - cidx * BT);
  const int hk = h / (a.Hv / a.Hk);
  const int64_t ch = (int64_t)h * a.nchunks + gc;      // head-major chunk slot
  const bool has_q = a.q != nullptr;

  for (int i = tid; i < 64 * P64; i += NTH) sA[i] = 0.f;

  // ---- gate activation + chunk-local inclusive cumsum (log2 units)
  {
    constexpr int G = NTH / KD, RPG = BT / G;
    const int c = tid % KD, grp = tid / KD;
    const IT* gp = static_cast<const IT*>(a.g);
    const bool gik = a.flags & F_GATE, safe = a.flags & F_SAFE;
    float Aexp = 0.f, bias = 0.f;
    if (gik) {
      Aexp = expf(a.A_log[h]);
      bias = a.dt_bias ? a.dt_bias[h * KD + c] : 0.f;
    }
    const int64_t gstride = (int64_t)a.Hv * KD;
    float run = 0.f;
#pragma unroll 4
    for (int r = 0; r < RPG; ++r) {
      const int i = grp * RPG + r;
      float gl = 0.f;
      if (i < C) {
        float x = to_f<IT>(gp[(tok0 + i) * gstride + h * KD + c]);
        float gn;
        if (gik) {
          float z = x + bias;
          float sp = fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
          gn = -Aexp * sp;
        } else {
          gn = x;
        }
        if (safe) gn = fmaxf(gn, a.lower_bound);
        gl = gn * LOG2E;
      }
      run += gl;
      sG[i * PG + c] = run;
    }
    sTot[grp * KD + c] = run;
  }

  // ---- q, k rows (raw) + squared norms + q.k dot; beta
  {
    constexpr int CPR = KD / EI, TOT = 64 * CPR;
    const IT* qp = static_cast<const IT*>(a.q);
    const IT* kp = static_cast<const IT*>(a.k);
    const int64_t qstride = (int64_t)a.Hk * KD;
    const bool l2 = a.flags & F_L2;
    for (int id = tid; id < TOT; id += NTH) {
      const int row = id / CPR, part = id % CPR;
      u32x4 uq = u32x4{0u, 0u, 0u, 0u}, uk = u32x4{0u, 0u, 0u, 0u};
      if (row < C) {
        const int64_t off = (tok0 + row) * qstride + hk * KD + part * EI;
        if (has_q) uq = *reinterpret_cast<const u32x4*>(qp + off);
        uk = *reinterpret_cast<const u32x4*>(kp + off);
      }
      *reinterpret_cast<u32x4*>(sQV + row * PQ + part * EI) = uq;
      *reinterpret_cast<u32x4*>(sK + row * PQ + part * EI) = uk;
      const IT* eq = reinterpret_cast<const IT*>(&uq);
      const IT* ek = reinterpret_cast<const IT*>(&uk);
      float sqq = 0.f, skk = 0.f, sqk = 0.f;
#pragma unroll
      for (int e = 0; e < EI; ++e) {
        float xq = to_f<IT>(eq[e]), xk = to_f<IT>(ek[e]);
        sqq += xq * xq;
        skk += xk * xk;
        sqk += xq * xk;
      }
#pragma unroll
      for (int o = CPR / 2; o >= 1; o >>= 1) {
        sqq += __shfl_xor(sqq, o);
        skk += __shfl_xor(skk, o);
        sqk += __shfl_xor(sqk, o);
      }
      if (part == 0) {
        sRq[row] = l2 ? 1.f / sqrtf(sqq + a.eps) : 1.f;
        sRk[row] = l2 ? 1.f / sqrtf(skk + a.eps) : 1.f;
        sDg[row] = sqk;
      }
    }
    if (tid < 64) {
      float b = 0.f;
      if (tid < C) {
        b = to_f<IT>(static_cast<const IT*>(a.beta)[(tok0 + tid) * a.Hv + h]);
        if (a.flags & F_SIGMOID) b = 1.f / (1.f + expf(-b));
      }
      sBeta[tid] = b;
    }
  }
  __syncthreads();
  {  // add the totals of the preceding row groups to finish the cumsum
    constexpr int G = NTH / KD, RPG = BT / G;
    const int c = tid % KD, grp = tid / KD;
    float off = 0.f;
    for (int g2 = 0; g2 < grp; ++g2) off += sTot[g2 * KD + c];
    if (grp > 0)
      for (int r = 0; r < RPG; ++r) sG[(grp * RPG + r) * PG + c] += off;
  }
  __syncthreads();

  // ---- Akk (L) and Aqk tiles on the matrix cores
  ST* Aqk_out = static_cast<ST*>(a.Aqk) + ch * (BT * BT);
  {
    const int r16 = lane & 15, quad = lane >> 4;
    // acc_kk/acc_qk += (row operand at level L) x (col operand at level L)^T
    auto tile_level = [&](int I, int J, int L, f32x4& akk, f32x4& aqk) {
      const int i = 16 * I + r16, j = 16 * J + r16;
      const bool irow = (i % L) >= (L >> 1), jcol = (j % L) < (L >> 1);
      const int ri = (i / L) * L + (L >> 1), rj = (j / L) * L + (L >> 1);
      const float rki = sRk[i], rqi = sRq[i], rkj = sRk[j];
#pragma unroll
      for (int ks = 0; ks < KD / 32; ++ks) {
        const int c0 = ks * 32 + 8 * quad;
        float ka[8], qa[8], kb[8];
        if (irow) {
          float x[8], gi[8], gr[8];
          load8(&sK[i * PQ + c0], x);
          load8(&sG[i * PG + c0], gi);
          load8(&sG[ri * PG + c0], gr);
          float xq[8];
          if (has_q) load8(&sQV[i * PQ + c0], xq);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float f = exp2f(gi[e] - gr[e]);
            ka[e] = x[e] * rki * f;
            qa[e] = has_q ? xq[e] * rqi * f : 0.f;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) { ka[e] = 0.f; qa[e] = 0.f; }
        }
        if (jcol) {
          float x[8], gj[8], gr[8];
          load8(&sK[j * PQ + c0], x);
          load8(&sG[j * PG + c0], gj);
          load8(&sG[rj * PG + c0], gr);
#pragma unroll
          for (int e = 0; e < 8; ++e) kb[e] = x[e] * rkj * exp2f(gr[e] - gj[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) kb[e] = 0.f;
        }
        Frag fa = split8(ka), fb = split8(kb);
        akk = mfma(fa.hi, fb.hi, akk);
        akk = mfma(fa.lo, fb.hi, akk);
        akk = mfma(fa.hi, fb.lo, akk);
        if (has_q) {
          if (F32) {
            Frag fq = split8(qa);
            aqk = mfma(fq.hi, fb.hi, aqk);
            aqk = mfma(fq.lo, fb.hi, aqk);
            aqk = mfma(fq.hi, fb.lo, aqk);
          } else {
            aqk = mfma(round8(qa), fb.hi, aqk);
          }
        }
      }
    };
    // full tile at one level: every entry valid
    auto full_tile = [&](int I, int J, int L) {
      f32x4 akk = zero4(), aqk = zero4();
      tile_level(I, J, L, akk, aqk);
      const int j = 16 * J + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * I + 4 * quad + e;
        sL[i * P64 + j] = sBeta[i] * akk[e];
        if (has_q) Aqk_out[i * BT + j] = from_f<ST>(a.scale * aqk[e]);
      }
    };
    if (wave < 4) {
      // diagonal tile I = wave: levels 16, 8, 4, 2 (index b: L = 2 << b)
      const int I = wave;
      f32x4 kk[4], qk[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        kk[b] = zero4();
        qk[b] = zero4();
        tile_level(I, I, 2 << b, kk[b], qk[b]);
      }
      const int j = 16 * I + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * I + 4 * quad + e;
        float vk = 0.f, vq = 0.f;
        if (i > j) {
          const int b = 31 - __clz(i ^ j);
          vk = b == 0 ? kk[0][e] : b == 1 ? kk[1][e] : b == 2 ? kk[2][e] : kk[3][e];
          vq = b == 0 ? qk[0][e] : b == 1 ? qk[1][e] : b == 2 ? qk[2][e] : qk[3][e];
          vk *= sBeta[i];
          vq *= a.scale;
        } else if (i == j) {
          vq = a.scale * sRq[i] * sRk[i] * sDg[i];
        }
        sL[i * P64 + j] = vk;
        if (has_q) Aqk_out[i * BT + j] = from_f<ST>(vq);
      }
    } else {
      const int w4 = wave - 4;
      full_tile(2 + (w4 >> 1), w4 & 1, 64);
      if (w4 == 0) full_tile(1, 0, 32);
      if (w4 == 1) full_tile(3, 2, 32);
      if (w4 >= 2 && has_q) {  // upper-triangle tiles of Aqk are zero
        for (int idx = (w4 - 2) * 64 + lane; idx < 6 * 256; idx += 128) {
          const int t = idx >> 8, e = idx & 255;
          const int I = t < 3 ? 0 : (t < 5 ? 1 : 2);
          const int J = t < 3 ? t + 1 : (t < 5 ? t - 1 : 3);
          Aqk_out[(16 * I + (e >> 4)) * BT + 16 * J + (e & 15)] = from_f<ST>(0.f);
        }
      }
    }
  }

  // ---- elementwise outputs: qg, kgT, X^T (LDS), gdec
  {
    constexpr int CG = KD / 8;
    if (has_q) {
      ST* qg = static_cast<ST*>(a.qg) + ch * (BT * KD);
      for (int idx = tid; idx < BT * CG; idx += NTH) {
        const int i = idx / CG, c0 = (idx % CG) * 8;
        float x[8], gi[8];
        load8(&sQV[i * PQ + c0], x);
        load8(&sG[i * PG + c0], gi);
        const float s = a.scale * sRq[i];
        float outv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) outv[e] = x[e] * s * exp2f(gi[e]);
        store8(qg + i * KD + c0, outv);
      }
    }
    float* kgT = static_cast<float*>(a.kgT) + ch * (KD * BT);
    for (int idx = tid; idx < KD * 8; idx += NTH) {
      const int c = idx >> 3, t0 = (idx & 7) * 8;
      const float gC = sG[63 * PG + c];
      float kv[8], xv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = t0 + e;
        const float kn = to_f<IT>(sK[t * PQ + c]) * sRk[t];
        const float gt = sG[t * PG + c];
        kv[e] = kn * exp2f(gC - gt);
        xv[e] = kn * exp2f(gt);
      }
      store8(kgT + c * BT + t0, kv);
      store8(sXT + c * PT + t0, xv);
    }
    if (tid < KD) a.gdec[ch * KD + tid] = exp2f(sG[63 * PG + tid]);
  }
  __syncthreads();

  // ---- diagonal 16x16 inverses (wave 0) | v^T into LDS (waves 1..7)
  if (wave == 0) {
    const int b = lane >> 4, jj = lane & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == jj) ? 1.f : 0.f;
#pragma unroll
      for (int kq = 0; kq < i; ++kq) s -= sL[(16 * b + i) * P64 + 16 * b + kq] * x[kq];
      x[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sA[(16 * b + i) * P64 + 16 * b + jj] = x[i];
  } else {
    constexpr int CPRV = VD / EI, TOTV = 64 * CPRV;
    const IT* vp = static_cast<const IT*>(a.v);
    const int64_t vstride = (int64_t)a.Hv * VD;
    for (int id = tid - 64; id < TOTV; id += NTH - 64) {
      const int row = id / CPRV, part = id % CPRV;
      u32x4 uv = u32x4{0u, 0u, 0u, 0u};
      if (row < C) uv = *reinterpret_cast<const u32x4*>(vp + (tok0 + row) * vstride + h * VD + part * EI);
      const IT* ev = reinterpret_cast<const IT*>(&uv);
#pragma unroll
      for (int e = 0; e < EI; ++e) sQV[(part * EI + e) * PT + row] = ev[e];
    }
  }
  __syncthreads();

  // ---- off-diagonal blocks of (I+L)^-1, by block distance d
  {
    const int jj = lane & 15, i0 = 4 * (lane >> 4);
    for (int d = 1; d <= 3; ++d) {
      if (wave <= 3 - d) {
        const int I = wave + d, J = wave;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int m = J; m < I; ++m) {
          for (int kq = 0; kq < 16; ++kq) {
            const float av = sA[(16 * m + kq) * P64 + 16 * J + jj];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += sL[(16 * I + i0 + e) * P64 + 16 * m + kq] * av;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sX[wave * 256 + (i0 + e) * 16 + jj] = acc[e];
      }
      __syncthreads();
      if (wave <= 3 - d) {
        const int I = wave + d, J = wave;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int kq = 0; kq < 16; ++kq) {
          const float xv = sX[wave * 256 + kq * 16 + jj];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] -= sA[(16 * I + i0 + e) * P64 + 16 * I + kq] * xv;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sA[(16 * I + i0 + e) * P64 + 16 * J + jj] = acc[e];
      }
      __syncthreads();
    }
  }

  // ---- u = A diag(beta) v,  w = A diag(beta) X   (X = k * 2^gamma)
  {
    const int I = wave & 3, isw = wave >> 2;
    const int r16 = lane & 15, quad = lane >> 4;
    const int nks = I >= 2 ? 2 : 1;                // A is lower triangular
    Frag fa[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks < nks) {
        const int j0 = ks * 32 + 8 * quad;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = sA[(16 * I + r16) * P64 + j0 + e] * sBeta[j0 + e];
        fa[ks] = split8(x);
      }
    }
    const int ND = isw ? KD : VD;
    const ST* Bsrc = isw ? sXT : sQV;
    ST* dstw = static_cast<ST*>(a.w) + ch * (BT * KD);       // w in the token dtype
    float* dstu = static_cast<float*>(a.u) + ch * (BT * VD);  // u in fp32
    for (int ct = 0; ct < ND / 16; ++ct) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks < nks) {
          const ST* bp = Bsrc + (16 * ct + r16) * PT + ks * 32 + 8 * quad;
          if (F32) {
            float xb[8];
            load8(reinterpret_cast<const float*>(bp), xb);
            Frag fb = split8(xb);
            acc = mfma(fa[ks].hi, fb.hi, acc);
            acc = mfma(fa[ks].lo, fb.hi, acc);
            acc = mfma(fa[ks].hi, fb.lo, acc);
          } else {
            bf16x8 b = load_bf16x8(reinterpret_cast<const bf16_t*>(bp));
            acc = mfma(fa[ks].hi, b, acc);
            acc = mfma(fa[ks].lo, b, acc);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = (16 * I + 4 * quad + e) * ND + 16 * ct + r16;
        if (isw) dstw[idx] = from_f<ST>(acc[e]);
        else dstu[idx] = acc[e];
      }
    }
  }
}

}  // namespace

hipError_t launch_intra(int K, int V, int dtype, const IntraArgs& a, hipStream_t s) {
  if (a.nchunks == 0 || a.Hv == 0) return hipSuccess;
  dim3 grid(a.nchunks, a.Hv), block(512);
#define KDA_INTRA_CASE(KK, VV, TT)                                          \
  if (K == KK && V == VV) {                                                 \
    hipLaunchKernelGGL((intra_kernel<KK, VV, TT>), grid, block, 0, s, a);   \
    return hipGetLastError();                                               \
  }
  if (dtype == 1) {
    KDA_INTRA_CASE(128, 128, bf16_t)
    KDA_INTRA_CASE(64, 64, bf16_t)
    KDA_INTRA_CASE(128, 64, bf16_t)
    KDA_INTRA_CASE(64, 128, bf16_t)
  } else {
    KDA_INTRA_CASE(64, 64, float)
    KDA_INTRA_CASE(64, 128, float)
  }
#undef KDA_INTRA_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
