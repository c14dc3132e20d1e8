// Chunk-local KDA work, one workgroup (4 waves) per (64-token chunk, value head).
//
// Follows "KDA Chunk Backward — TPU/Pallas Kernel Design", section 1.2 (WY
// representation, log2-space chunk-local gate) and section 3.7 (sub-block
// normalisation with a reference gate), and the prepare stage of
// "Hyper-Parallel Chunk KDA" section 5.1 (gate, L2Norm, beta, Akk/Aqk, w, u,
// qg, kg).  Per chunk with tokens i = 0..63 (rows >= C of a partial chunk are
// zero and inert):
//   gamma_i   = log2(e) * sum_{r<=i} g_r         (inclusive, per channel)
//   L_ij      = beta_i * sum_c k_ic k_jc 2^(gamma_ic - gamma_jc)   (i > j)
//   Aqk_ij    = scale  * sum_c q_ic k_jc 2^(gamma_ic - gamma_jc)   (i >= j)
//   A         = (I + L)^-1
//   u = A (beta * v),  w = A (beta * k * 2^gamma)
//   kg = k * 2^(gamma_C - gamma),  qg = scale * q * 2^gamma,  gdec = 2^gamma_C
// Workspace per (head, chunk): gdec [K] in fp32; with bf16 tokens w, qg [64][K],
// kg^T [K][64], Aqk [64][64] and u [64][V] in fp16 (11 significant bits); with
// fp32 tokens w, qg, Aqk and u in fp32 and kg^T as a bf16 hi part and an e4m3
// lo part (together ~13 significant bits).
//
// Each wave owns 16 token rows and keeps them in registers in the matrix-core
// operand layout (lane: row 16*wave + lane%16, channels 32*ks + 8*(lane/16) + e),
// so a row is both the A operand of its own row tile and the B operand of its
// own column tile.
//
// Range safety of the decay products.  Within one chunk gamma can fall by
// hundreds, so 2^gamma_i * 2^-gamma_j overflows fp32.  Every pair i > j is
// evaluated at the level of a binary split of the chunk where i lies in the
// upper half and j in the lower half of one block, with the reference
// r = first row of the upper half:
//   2^(gamma_i - gamma_j) = 2^(gamma_i - gamma_r) * 2^(gamma_r - gamma_j),
// both factors <= 1.  Levels 64 and 32 are full 16x16 tiles; levels 16, 8, 4
// and 2 live inside the diagonal tiles and are masked per entry.  The diagonal
// of Aqk (factor 1) is a plain dot product.
//
// Precision of the matrix-core products.  With bf16 token tensors every
// factor of Akk and Aqk enters as one bf16 rounding (single pass): an
// error of 2^-9 relative per entry of L moves (I + L)^-1, u and w by far less
// than the state tolerance, since L only reaches the state through them.
// With fp32 token tensors Akk and Aqk use bf16 hi/lo pairs (three passes).
#include "kda_launch.h"

#include <type_traits>

namespace kda {

namespace {

constexpr float LN2 = 0.6931471805599453f;

template <int N>
__device__ __forceinline__ float dpp_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, true));
}
// Inclusive prefix sum across the 16 lanes of each DPP row.
__device__ __forceinline__ float row_scan16(float x) {
  x += dpp_shr<1>(x);
  x += dpp_shr<2>(x);
  x += dpp_shr<4>(x);
  x += dpp_shr<8>(x);
  return x;
}

// Value of x in another lane: a DPP move with control CTRL (row_shl, quad_perm)
// or a swizzle with bit-mode PATTERN (and/or masks within 32-lane groups).
template <int CTRL>
__device__ __forceinline__ float lane_from(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
template <int PATTERN>
__device__ __forceinline__ float swizzle(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), PATTERN));
}

// 2^x and log2(x) on the transcendental unit (v_exp_f32 / v_log_f32).  Every
// exponent used here is <= 0; results below the normal range flush towards
// zero, where the products they scale are negligible.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ void zero8(float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = 0.f;
}

// acc += A * B with both operands split into bf16 hi/lo (three passes).
__device__ __forceinline__ f32x4 mma3(const Frag& A, const Frag& B, f32x4 acc) {
  acc = mfma(A.hi, B.hi, acc);
  acc = mfma(A.lo, B.hi, acc);
  acc = mfma(A.hi, B.lo, acc);
  return acc;
}

// Transposes on the matrix cores.  With B = S_half (32 x 16, one where the
// reduction index equals 16*half + column), the product A S_half of a row
// tile A (16 rows x 32 reduction, bf16) is A's columns 16*half .. +15 as an
// accumulator tile: lane l gets column 16*half + l%16 of rows 4*(l/16) .. +3.
// Every product term is one bf16 value times 1, so the result is exact.  Two
// such tiles of consecutive 16-row tiles are the two halves of one operand
// fragment in the stored lane order (slots 8g .. 8g+3 and 8g+4 .. 8g+7 hold
// rows 4g .. 4g+3 of the first and of the second tile).
__device__ __forceinline__ bf16x8 select_operand(int half, int lane) {
  const int col = 16 * half + (lane & 15), k0 = 8 * (lane >> 4);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = (k0 + 2 * j == col ? 0x3f80u : 0u) | (k0 + 2 * j + 1 == col ? 0x3f800000u : 0u);
  return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
}
// The same with fp16 operands (1.0 = 0x3c00): A S_half on the fp16 matrix cores.
__device__ __forceinline__ f16x8 select_operand_f16(int half, int lane) {
  const int col = 16 * half + (lane & 15), k0 = 8 * (lane >> 4);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = (k0 + 2 * j == col ? 0x3c00u : 0u) | (k0 + 2 * j + 1 == col ? 0x3c000000u : 0u);
  return __builtin_bit_cast(f16x8, u32x4{w[0], w[1], w[2], w[3]});
}
__device__ __forceinline__ u32x2 pack4(const f32x4& v) {
  return u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// Eight consecutive elements through a buffer descriptor (zeros past its end).
template <typename T> __device__ __forceinline__ void load8b(rsrc_t r, uint32_t off, float (&x)[8]);
template <> __device__ __forceinline__ void load8b<bf16_t>(rsrc_t r, uint32_t off, float (&x)[8]) {
  const u32x4 u = buf_load16(r, off);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(w[j] << 16);
    x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void load8b<float>(rsrc_t r, uint32_t off, float (&x)[8]) {
  const f32x4 a = __builtin_bit_cast(f32x4, buf_load16(r, off));
  const f32x4 b = __builtin_bit_cast(f32x4, buf_load16(r, off + 16));
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <typename T> __device__ __forceinline__ float load1b(rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ float load1b<bf16_t>(rsrc_t r, uint32_t off) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0) << 16);
}
template <> __device__ __forceinline__ float load1b<float>(rsrc_t r, uint32_t off) {
  return __uint_as_float(buf_load4(r, off));
}

// Store 4 consecutive values (8 bytes as bf16, 16 bytes as fp32).
__device__ __forceinline__ void store4(bf16_t* p, const f32x4& v) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void store4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }
// The fp16 record sections w, qg, Aqk (and u, below) are written with
// non-temporal stores: the scan that reads them back after this kernel then
// runs about 10% faster at the layer shape; the same hint on kg^T moved time
// from the scan into this kernel instead.
__device__ __forceinline__ void store4(_Float16* p, const f32x4& v) {
  __builtin_nontemporal_store(pack4_f16(v), reinterpret_cast<u32x2*>(p));
}

// Three workgroups per CU with bf16 tokens (at most 53 KB of LDS and 168
// registers each); fp32 tokens need more LDS: two with K = V = 64, one otherwise.
template <int KD, int VD, typename IT> constexpr int intra_min_blocks() {
  return sizeof(IT) == 2 ? 3 : (KD == 128 || VD == 128) ? 1 : 2;
}

template <int KD, int VD, typename IT, bool FWD>
__global__ __launch_bounds__(256, (intra_min_blocks<KD, VD, IT>())) void intra_kernel(IntraArgs a) {
  using ST = IT;                                   // staging type of v^T and X^T (fp32 tokens)
  constexpr bool F32 = sizeof(IT) == 4;
  constexpr int NKS = KD / 32, NVS = VD / 32;
  constexpr int P64 = 64 + 4;                      // row stride of sLA (floats)
  constexpr int PB = KD + 8;                       // row stride of bf16 column operands
  constexpr int PT = 64 + 16 / (int)sizeof(ST);    // row stride of v^T / X^T (fp32 tokens)
  constexpr int NP = F32 ? 2 : 1;                  // bf16 parts of a column operand (hi [, lo])
  constexpr int BOP_BYTES = (32 + 16 + 16 + 32) * PB * 2 * NP;   // + rows 48..63 as row operand (k, q)
  // v^T / X^T: fp32 tokens as [channel][token] rows; bf16 tokens as operand
  // fragments (16 channels x 32 tokens, 1 KiB each, stored lane order)
  constexpr int VX_BYTES = F32 ? (VD + KD) * PT * 4 : (VD + KD) / 16 * 2 * 1024;
  constexpr int UB = BOP_BYTES > VX_BYTES ? BOP_BYTES : VX_BYTES;

  __shared__ __attribute__((aligned(16))) float sTot[3][KD];   // gate totals of waves 0..2
  __shared__ __attribute__((aligned(16))) float sRef[4][KD];   // gamma of rows 16, 32, 48 and the chunk total
  // L (strictly lower part, row-major) and A = (I+L)^-1 transposed (upper part
  // and diagonal: A_ij at sLA[j][i] for i >= j) share one 64 x 64 array
  __shared__ __attribute__((aligned(16))) float sLA[64 * P64];
  float* sL = sLA;
  // beta of row r in the row's padding column (sLA[r][64]; the padding is never
  // touched otherwise), which keeps the LDS within a third of the CU's
  auto sBeta = [&](int r) -> float& { return sLA[r * P64 + 64]; };
  // column operands of the off-diagonal levels, later reused for v^T and X^T
  __shared__ __attribute__((aligned(16))) unsigned char sU8[UB];
  bf16_t* b64hi = reinterpret_cast<bf16_t*>(sU8);  // rows 0..31, reference row 32
  bf16_t* b64lo = b64hi + 32 * PB;                 // (lo parts: fp32 tokens only)
  bf16_t* b32ahi = b64hi + NP * 32 * PB;           // rows 0..15, reference row 16
  bf16_t* b32alo = b32ahi + 16 * PB;
  bf16_t* b32bhi = b32ahi + NP * 16 * PB;          // rows 32..47, reference row 48
  bf16_t* b32blo = b32bhi + 16 * PB;
  bf16_t* r32khi = b32bhi + NP * 16 * PB;          // rows 48..63 against reference row 48 (row operand)
  bf16_t* r32klo = r32khi + 16 * PB;
  bf16_t* r32qhi = r32khi + NP * 16 * PB;          // the same rows of q
  bf16_t* r32qlo = r32qhi + 16 * PB;
  ST* sVT = reinterpret_cast<ST*>(sU8);            // fp32 tokens: [VD][PT]
  ST* sXT = sVT + VD * PT;                         //              [KD][PT]
  u32x4* sVF = reinterpret_cast<u32x4*>(sU8);      // bf16 tokens: fragment (ct, ks) at [(2ct + ks) * 64]
  u32x4* sXF = sVF + (VD / 16) * 2 * 64;

  int gc, h;
  chunk_head_of_block(blockIdx.x, gridDim.x, a.nchunks, a.Hv, a.Hk, gc, h);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: wave branches are scalar
  const int r16 = lane & 15, quad = lane >> 4;
  const int n = seq_of_chunk(a.seq, gc);
  int64_t tok0s;
  int len;
  seq_range(a.seq, n, tok0s, len);
  const int cidx = gc - chunk_base(a.seq, n);
  const int64_t tok0 = tok0s + (int64_t)cidx * BT;
  const int C = min(BT, len - cidx * BT);
  const int hk = h / (a.Hv / a.Hk);
  const int64_t ch = (int64_t)h * a.nchunks + gc;      // head-major chunk slot
  constexpr RecLayout RL = rec_layout(KD, VD, (int)sizeof(IT), FWD);
  unsigned char* rec = a.ws + ch * RL.bytes;
  constexpr bool has_q = FWD;                          // q (and the output terms) present
  const int i = 16 * wave + r16;                       // this lane's token row
  const bool live = i < C;

  // ---- loads, in the order of use (loads complete in order): gate bias and
  // gate rows first, then k, q rows of this lane, beta, v rows.  Buffer loads with
  // per-tensor descriptors bounded at the chunk's last valid row: rows past the
  // sequence end read as zeros without a branch, so all loads issue back to
  // back (a conditional load would make the compiler wait for each one).
  const bool gik = a.flags & F_GATE;
  constexpr int ES = (int)sizeof(IT);
  // gate bias rows: read per channel slice where they are used (L2-resident)
  const rsrc_t rb = make_rsrc(a.dt_bias ? a.dt_bias + h * KD : a.A_log, (gik && a.dt_bias) ? KD * 4 : 0);
  float gl[NKS][8], kx[NKS][8], qx[NKS][8];
  float beta;
  {
    const rsrc_t rg = make_rsrc(static_cast<const IT*>(a.g) + (tok0 * a.Hv + h) * KD, (uint32_t)(C * a.Hv * KD * ES));
    const rsrc_t rk = make_rsrc(static_cast<const IT*>(a.k) + (tok0 * a.Hk + hk) * KD, (uint32_t)(C * a.Hk * KD * ES));
    const rsrc_t rq = make_rsrc(has_q ? static_cast<const IT*>(a.q) + (tok0 * a.Hk + hk) * KD : nullptr,
                                has_q ? (uint32_t)(C * a.Hk * KD * ES) : 0u);
    const rsrc_t rbeta = make_rsrc(static_cast<const IT*>(a.beta) + tok0 * a.Hv + h, (uint32_t)(C * a.Hv * ES));
    const uint32_t ok = (uint32_t)(i * a.Hk * KD) * ES, og = (uint32_t)(i * a.Hv * KD) * ES;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) load8b<IT>(rg, og + (32 * ks + 8 * quad) * ES, gl[ks]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      load8b<IT>(rk, ok + (32 * ks + 8 * quad) * ES, kx[ks]);
      load8b<IT>(rq, ok + (32 * ks + 8 * quad) * ES, qx[ks]);
    }
    beta = load1b<IT>(rbeta, (uint32_t)(i * a.Hv) * ES);
  }
  // (after the row loads: its scalar read and exponential would hold them back)
  __builtin_amdgcn_sched_barrier(0);
  const float Aexp = gik ? expf(a.A_log[h]) : 0.f;

  // ---- gate activation (log2 units), in-wave row prefix sums, norms
  {
    // The flag tests sit outside the element loops (one uniform branch), so
    // that the per-element work forms one straight-line block.  Results are in
    // log2 units: log2(e) * max(g, lb) = max(log2(e) * g, log2(e) * lb), with
    // the unit change and the zero of rows past the sequence end folded into
    // one per-row coefficient (lb = -inf without the clamp: max(x, -inf) = x).
    const float lb2 = !live ? 0.f : (a.flags & F_SAFE) ? a.lower_bound * LOG2E : -INFINITY;
    if (gik) {
      const float cA = live ? -Aexp * LOG2E : 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        float bias[8];
        load8b<float>(rb, (uint32_t)(32 * ks + 8 * quad) * 4, bias);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float z = gl[ks][e] + bias[e];
          // softplus(z) = max(z, 0) + ln(1 + e^-|z|)
          gl[ks][e] = fmaxf(cA * (fmaxf(z, 0.f) + LN2 * flog2(1.f + fexp2(-LOG2E * fabsf(z)))), lb2);
        }
      }
    } else {
      const float cL = live ? LOG2E : 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) gl[ks][e] = fmaxf(cL * gl[ks][e], lb2);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) gl[ks][e] = row_scan16(gl[ks][e]);
  }
  // total decay of this wave's 16 rows (log2 units, largest over the channels):
  // the row-15 lanes hold the tile totals; it decides the diagonal tile's form
  float span = 0.f;
  if (r16 == 15) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) span = fmaxf(span, -gl[ks][e]);
  }
  span = fmaxf(span, __shfl_xor(span, 16));
  span = fmaxf(span, __shfl_xor(span, 32));
  span = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(span), 15));
  float rq, rk, dqk;
  {
    float sqq = 0.f, skk = 0.f, sqk = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sqq += qx[ks][e] * qx[ks][e];
        skk += kx[ks][e] * kx[ks][e];
        sqk += qx[ks][e] * kx[ks][e];
      }
    sqq += __shfl_xor(sqq, 16); sqq += __shfl_xor(sqq, 32);
    skk += __shfl_xor(skk, 16); skk += __shfl_xor(skk, 32);
    sqk += __shfl_xor(sqk, 16); sqk += __shfl_xor(sqk, 32);
    const bool l2 = a.flags & F_L2;
    // the attention scale rides on q's normalisation (q enters only Aqk and qg)
    // (rows past the sequence end get zero factors: with eps = 0 their zero
    // norms would otherwise turn into 0 * inf = NaN)
    rq = live ? a.scale * (l2 ? 1.f / sqrtf(sqq + a.eps) : 1.f) : 0.f;
    rk = live ? (l2 ? 1.f / sqrtf(skk + a.eps) : 1.f) : 0.f;
    dqk = sqk;
  }
  if (r16 == 15 && wave < 3) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) store8(&sTot[wave][32 * ks + 8 * quad], gl[ks]);
  }
  // beta activation here, not at its load: the gate work above needs only the
  // gate rows, and waiting on beta means waiting on every load before it
  if (a.flags & F_SIGMOID) beta = live ? 1.f / (1.f + expf(-beta)) : 0.f;
  if (quad == 0) sBeta(i) = beta;
  __syncthreads();

  // ---- finish the chunk cumsum; publish reference rows and the chunk decay
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int c0 = 32 * ks + 8 * quad;
    // offset of this wave's rows: the sum of the earlier waves' totals
    float off[8];
    zero8(off);
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      if (w >= wave) break;
      float t[8];
      load8(&sTot[w][c0], t);
#pragma unroll
      for (int e = 0; e < 8; ++e) off[e] += t[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) gl[ks][e] += off[e];
    // reference rows 16, 32, 48 and row 63 (the chunk total gamma_C)
    if (r16 == 0 && wave >= 1) store8(&sRef[wave - 1][c0], gl[ks]);
    if (r16 == 15 && wave == 3) store8(&sRef[3][c0], gl[ks]);
  }
  // normalised rows
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kx[ks][e] *= rk;
      qx[ks][e] *= rq;
    }
  __syncthreads();

  // ---- column operands of levels 64 / 32 (LDS), qg and kg^T (global)
  const bf16x8 sel[2] = {select_operand(0, lane), select_operand(1, lane)};
  {
    auto put_col = [&](const float* gref, bf16_t* hi, bf16_t* lo, int row) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c0 = 32 * ks + 8 * quad;
        float gr[8], x[8];
        load8(gref + c0, gr);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = kx[ks][e] * fexp2(gr[e] - gl[ks][e]);
        if constexpr (F32) {
          Frag f = split8(x);
          *reinterpret_cast<bf16x8*>(hi + row * PB + c0) = f.hi;
          *reinterpret_cast<bf16x8*>(lo + row * PB + c0) = f.lo;
        } else {
          *reinterpret_cast<bf16x8*>(hi + row * PB + c0) = round8(x);
        }
      }
    };
    if (wave == 3 && r16 == 0) {   // the chunk decay 2^gamma_C (wave 3 builds no column operand)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        float d[8];
        load8(sRef[3] + 32 * ks + 8 * quad, d);
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = fexp2(d[e]);
        store8(reinterpret_cast<float*>(rec + RL.gd) + 32 * ks + 8 * quad, d);
      }
    }
    if (wave <= 1) put_col(sRef[1], b64hi, b64lo, i);
    if (wave == 0) put_col(sRef[0], b32ahi, b32alo, i);
    if (wave == 2) put_col(sRef[2], b32bhi, b32blo, i - 32);
    if (wave == 3) {
      // rows 48..63 against reference row 48 (factor 2^(gamma_i - gamma_48) <= 1),
      // k and q: the level-32 tile (3, 2) is formed by wave 0, idle there
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c0 = 32 * ks + 8 * quad;
        float gr[8], kv[8], qv[8];
        load8(sRef[2] + c0, gr);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = fexp2(gl[ks][e] - gr[e]);
          kv[e] = kx[ks][e] * f;
          qv[e] = qx[ks][e] * f;
        }
        if constexpr (F32) {
          const Frag fk = split8(kv), fq = split8(qv);
          *reinterpret_cast<bf16x8*>(r32khi + r16 * PB + c0) = fk.hi;
          *reinterpret_cast<bf16x8*>(r32klo + r16 * PB + c0) = fk.lo;
          if (has_q) {
            *reinterpret_cast<bf16x8*>(r32qhi + r16 * PB + c0) = fq.hi;
            *reinterpret_cast<bf16x8*>(r32qlo + r16 * PB + c0) = fq.lo;
          }
        } else {
          *reinterpret_cast<bf16x8*>(r32khi + r16 * PB + c0) = round8(kv);
          if (has_q) *reinterpret_cast<bf16x8*>(r32qhi + r16 * PB + c0) = round8(qv);
        }
      }
    }
    if (has_q) {
      // qg: fp16 with bf16 tokens (the scan's h operand is an fp16 hi/lo pair)
      using QT = typename std::conditional<F32, float, _Float16>::type;
      QT* qg = reinterpret_cast<QT*>(rec + RL.qg);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        f32x4 x0, x1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x0[e] = qx[ks][e] * fexp2(gl[ks][e]);
          x1[e] = qx[ks][e + 4] * fexp2(gl[ks][e + 4]);
        }
        store4(qg + frag_off(i, 32 * ks + 8 * quad, NKS), x0);
        store4(qg + frag_off(i, 32 * ks + 8 * quad + 4, NKS), x1);
      }
    }
    // kg = k * 2^(gamma_C - gamma), transposed on the matrix cores into kg^T
    // fragments (16 channels x 32 tokens): this wave's 16 tokens are half of
    // fragment (kt, wave / 2), 8 bytes of each lane.  bf16 tokens: fp16 rows
    // (|kg| <= 1, 11 significant bits).  fp32 tokens: bf16 hi rows, and the
    // lo parts as e4m3 after scaling by 2^10 (clamped to its range), the lo
    // bytes of the four waves interleaved into 16-byte lane words.
    unsigned char* kgh = rec + RL.kgh;
    const uint32_t kg_off = (uint32_t)((wave >> 1) * 64 + lane) * 16 + (wave & 1) * 8;
    const uint32_t kl_off = (uint32_t)lane * 16 + (wave >> 1) * 8 + (wave & 1) * 4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float x[8], gc[8];
      load8(sRef[3] + 32 * ks + 8 * quad, gc);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = kx[ks][e] * fexp2(gc[e] - gl[ks][e]);
      if constexpr (F32) {
        const Frag f = split8(x);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kt = 2 * ks + half;
          const f32x4 th = mfma(f.hi, sel[half], zero4());
          const f32x4 tl = mfma(f.lo, sel[half], zero4());
          *reinterpret_cast<u32x2*>(kgh + kt * 2 * 1024 + kg_off) = pack4(th);
          *reinterpret_cast<uint32_t*>(rec + RL.kgl + kt * 1024 + kl_off) = pack4_fp8(tl * KGL_SCALE);
        }
      } else {
        const f16x8 f = round8_f16(x);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kt = 2 * ks + half;
          const f32x4 th = mfma(f, select_operand_f16(half, lane), zero4());
          *reinterpret_cast<u32x2*>(kgh + kt * 2 * 1024 + kg_off) = pack4_f16(th);
        }
      }
    }
  }
  __syncthreads();

  // v rows (8 values of the token dtype per slice), read after the diagonal
  // tiles: loaded with the other rows at the top they would stay live through
  // every phase (the register count that allows three workgroups per CU)
  u32x4 vr[NVS][ES / 2];
  // ---- Akk (L) and Aqk tiles on the matrix cores
  // Aqk: fp16 with bf16 tokens, fp32 with fp32 tokens
  using AT = typename std::conditional<F32, float, _Float16>::type;
  AT* Aqk_out = reinterpret_cast<AT*>(rec + RL.aqk);
  {
    // Diagonal tile of this wave: levels L = 2 << b for b = 0..3 (blocks of 2,
    // 4, 8, 16 rows).  At level b every row carries one factor, relative to the
    // first row of the upper half of its block: 2^(gamma_r - gamma_ref) in the
    // upper half, 2^(gamma_ref - gamma_r) in the lower half.  The operand built
    // from these rows serves as both matrix-core operands: the entries (i, j)
    // with i in the upper and j in the lower half are exactly the wanted ones;
    // the rest of the tile is ignored.  The reference gamma comes from the lane
    // of the reference row by a DPP move (b = 0, 1) or a swizzle (b = 2, 3);
    // the 16 lanes of a DPP row are the 16 rows of the tile.
    //
    // Small-decay form.  With the in-kernel gate every g is <= 0, so within
    // the tile |gamma_r - gamma_8| never exceeds the tile's total decay D.
    // When D < 112 (log2 units) one reference serves every pair: with
    // F_i = k_i 2^(gamma_i - gamma_8) and G_j = k_j 2^(gamma_8 - gamma_j), both
    // below 2^112 in scale, L_ij = beta_i F_i . G_j exactly as at the split
    // levels (entries with i <= j may overflow and are never read).  Decided
    // per wave from its own rows' totals (span, taken after the row scans).
    const bool one_ref = gik && span < 112.f;
    // dk, dq: the tile's entries (i > j for L, i >= j for Aqk); the split
    // levels are formed one after another and each keeps only its own entries
    f32x4 dk = zero4(), dq = zero4();
    if (one_ref) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        float kf[8], kb[8], qf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float g = gl[ks][e];
          const float d = g - swizzle<0x110>(g);   // gamma_r - gamma_8 (row 8 of the tile)
          const float f = fexp2(d), fb = fexp2(-d);
          kf[e] = kx[ks][e] * f;
          kb[e] = kx[ks][e] * fb;
          qf[e] = qx[ks][e] * f;
        }
        // A = G (rows j), B = F (columns i): this lane gets (i = r16, j = 4*quad + e)
        if constexpr (F32) {
          const Frag F = split8(kf), G = split8(kb);
          dk = mma3(G, F, dk);
          if (has_q) dq = mma3(G, split8(qf), dq);
        } else {
          const bf16x8 F = round8(kf), G = round8(kb);
          dk = mfma(G, F, dk);
          if (has_q) dq = mfma(G, round8(qf), dq);
        }
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bool up = (r16 >> b) & 1;
        // lane-uniform arithmetic only: a cross-lane move under a lane-dependent
        // branch would read from disabled lanes
        const float sgn = up ? 1.f : -1.f;
        f32x4 tk = zero4(), tq = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          float kv[8], qv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float g = gl[ks][e];
            float ex;
            if (b == 0) ex = (up ? 0.f : 1.f) * (lane_from<0x101>(g) - g);   // lower rows: row r + 1 (row_shl:1)
            else if (b == 1) ex = sgn * (g - lane_from<0xAA>(g));           // row (r & ~3) | 2 (quad_perm 2,2,2,2)
            else if (b == 2) ex = sgn * (g - swizzle<0x98>(g));             // row (r & ~7) | 4
            else ex = sgn * (g - swizzle<0x110>(g));                        // row 8
            const float f = fexp2(ex);
            kv[e] = kx[ks][e] * f;
            qv[e] = qx[ks][e] * f;
          }
          if constexpr (F32) {
            const Frag F = split8(kv);
            tk = mma3(F, F, tk);
            if (has_q) tq = mma3(F, split8(qv), tq);
          } else {
            const bf16x8 F = round8(kv);
            tk = mfma(F, F, tk);
            if (has_q) tq = mfma(F, round8(qv), tq);
          }
        }
        // entries (i, j) with i > j whose highest differing bit is b
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int il = r16, jl = 4 * quad + e;
          if (il > jl && 31 - __clz(il ^ jl) == b) {
            dk[e] = tk[e];
            dq[e] = tq[e];
          }
        }
      }
    }
    // diagonal tile output: this lane holds row i = r16, columns 4*quad .. +3,
    // and owns row i's beta, norms and q.k dot
    {
      f32x4 vk4, vq4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int il = r16, jl = 4 * quad + e;
        float vk = 0.f, vq = 0.f;
        if (il > jl) {
          vk = beta * dk[e];
          vq = dq[e];
        } else if (il == jl) {
          vq = rq * rk * dqk;
        }
        vk4[e] = vk;
        vq4[e] = vq;
      }
      *reinterpret_cast<f32x4*>(&sL[i * P64 + 16 * wave + 4 * quad]) = vk4;
      if (has_q) store4(Aqk_out + frag_off(i, 16 * wave + 4 * quad, 2), vq4);
    }
    {
    const rsrc_t rv = make_rsrc(static_cast<const IT*>(a.v) + (tok0 * a.Hv + h) * VD, (uint32_t)(C * a.Hv * VD * ES));
    const uint32_t ov = (uint32_t)(i * a.Hv * VD) * ES;
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
      for (int j = 0; j < ES / 2; ++j) vr[vs][j] = buf_load16(rv, ov + (32 * vs + 8 * quad) * ES + 16 * j);
  }
    // Off-diagonal tiles: row operands (one per reference, shared by the column
    // tiles it meets) against column operands in LDS.  Level 64: tiles 2, 3
    // against 0, 1 (reference row 32) -> acc[0], acc[1], waves 2 and 3; level 32:
    // tile 1 against 0 (row 16) -> acc[2], wave 1, and tile 3 against 2 (row 48)
    // by wave 0 from the row operand wave 3 left in LDS.
    {
      f32x4 ak[3], aq[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        ak[j] = zero4();
        aq[j] = zero4();
      }
      const bool l64 = wave >= 2, l32 = wave == 1;
      const float* gref32 = sRef[0];
      const bf16_t* c32hi = b32ahi;
      const bf16_t* c32lo = b32alo;
      auto row_op = [&](const float* gref, int ks, Frag& R, bf16x8& Rq, Frag& Rqf) __attribute__((always_inline)) {
        const int c0 = 32 * ks + 8 * quad;
        float gr[8], kv[8], qv[8];
        load8(gref + c0, gr);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = fexp2(gl[ks][e] - gr[e]);
          kv[e] = kx[ks][e] * f;
          qv[e] = qx[ks][e] * f;
        }
        if constexpr (F32) {
          R = split8(kv);
          Rqf = split8(qv);
        } else {
          R.hi = round8(kv);
          Rq = round8(qv);
        }
      };
      auto tile = [&](const Frag& R, const bf16x8& Rq, const Frag& Rqf, const bf16_t* bhi, const bf16_t* blo,
                      int brow0, int ks, f32x4& akk, f32x4& aqk) __attribute__((always_inline)) {
        const int c0 = 32 * ks + 8 * quad;
        // transposed tiles: row i = r16, columns 4*quad .. +3
        if constexpr (F32) {
          Frag Cs;
          Cs.hi = load_bf16x8(bhi + (brow0 + r16) * PB + c0);
          Cs.lo = load_bf16x8(blo + (brow0 + r16) * PB + c0);
          akk = mma3(Cs, R, akk);
          if (has_q) aqk = mma3(Cs, Rqf, aqk);
        } else {
          const bf16x8 Ch = load_bf16x8(bhi + (brow0 + r16) * PB + c0);
          akk = mfma(Ch, R.hi, akk);
          if (has_q) aqk = mfma(Ch, Rq, aqk);
        }
      };
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        Frag R, Rqf;
        bf16x8 Rq;
        if (l64) {
          row_op(sRef[1], ks, R, Rq, Rqf);
          tile(R, Rq, Rqf, b64hi, b64lo, 0, ks, ak[0], aq[0]);
          tile(R, Rq, Rqf, b64hi, b64lo, 16, ks, ak[1], aq[1]);
        }
        if (l32) {
          row_op(gref32, ks, R, Rq, Rqf);
          tile(R, Rq, Rqf, c32hi, c32lo, 0, ks, ak[2], aq[2]);
        }
        if (wave == 0) {
          const int c0 = 32 * ks + 8 * quad;
          R.hi = load_bf16x8(r32khi + r16 * PB + c0);
          if constexpr (F32) {
            R.lo = load_bf16x8(r32klo + r16 * PB + c0);
            if (has_q) {
              Rqf.hi = load_bf16x8(r32qhi + r16 * PB + c0);
              Rqf.lo = load_bf16x8(r32qlo + r16 * PB + c0);
            }
          } else if (has_q) {
            Rq = load_bf16x8(r32qhi + r16 * PB + c0);
          }
          tile(R, Rq, Rqf, b32bhi, b32blo, 0, ks, ak[2], aq[2]);
        }
      }
      // tile J of row tile `row / 16` (row = this lane's row of it), scaled
      auto put = [&](int J, int row, float brow, const f32x4& akk, const f32x4& aqk) __attribute__((always_inline)) {
        f32x4 vk4, vq4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vk4[e] = brow * akk[e];
          vq4[e] = aqk[e];
        }
        *reinterpret_cast<f32x4*>(&sL[row * P64 + 16 * J + 4 * quad]) = vk4;
        if (has_q) store4(Aqk_out + frag_off(row, 16 * J + 4 * quad, 2), vq4);
      };
      if (l64) {
        put(0, i, beta, ak[0], aq[0]);
        put(1, i, beta, ak[1], aq[1]);
      }
      if (l32) put(0, i, beta, ak[2], aq[2]);
      if (wave == 0) put(2, 48 + r16, sBeta(48 + r16), ak[2], aq[2]);
    }
    if (has_q) {  // upper-triangle tiles of this row tile are zero (those of the
                  // all-zero 32 x 32 block, rows < 32 and tokens >= 32, are never read)
      for (int J = wave + 1; J < (wave < 2 ? 2 : 4); ++J) store4(Aqk_out + frag_off(i, 16 * J + 4 * quad, 2), zero4());
    }
  }
  __syncthreads();

  // ---- v^T and X^T = (k * 2^gamma)^T into LDS; diagonal 16x16 inverses
  if constexpr (F32) {
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
      for (int e = 0; e < 8; ++e) sVT[(32 * vs + 8 * quad + e) * PT + i] = __uint_as_float(vr[vs][e >> 2][e & 3]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) sXT[(32 * ks + 8 * quad + e) * PT + i] = kx[ks][e] * fexp2(gl[ks][e]);
  } else {
    // transposed on the matrix cores into operand fragments (16 channels x 32
    // tokens); v enters as the token's own bf16 values
    const uint32_t f_off = (uint32_t)(wave >> 1) * 64 + lane;   // fragment (ct, wave / 2), in u32x4
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs) {
      const bf16x8 vrow = __builtin_bit_cast(bf16x8, vr[vs][0]);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ct = 2 * vs + half;
        *reinterpret_cast<u32x2*>(reinterpret_cast<unsigned char*>(sVF + ct * 2 * 64 + f_off) + (wave & 1) * 8) =
            pack4(mfma(vrow, sel[half], zero4()));
      }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // 2^gamma is formed again here: otherwise the compiler keeps the qg
        // phase's values live (32 registers) through every phase in between
        float gg = gl[ks][e];
        asm volatile("" : "+v"(gg));
        x[e] = kx[ks][e] * fexp2(gg);
      }
      const bf16x8 xrow = round8(x);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ct = 2 * ks + half;
        *reinterpret_cast<u32x2*>(reinterpret_cast<unsigned char*>(sXF + ct * 2 * 64 + f_off) + (wave & 1) * 8) =
            pack4(mfma(xrow, sel[half], zero4()));
      }
    }
  }
  if (quad == 0) {
    const int b = wave, jj = r16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == jj) ? 1.f : 0.f;
#pragma unroll
      for (int kq = 0; kq < r; ++kq) s -= sL[(16 * b + r) * P64 + 16 * b + kq] * x[kq];
      x[r] = s;
    }
    // column jj of A_bb (x[r] = A_bb[r][jj], zero for r < jj) as row 16b + jj of
    // sLA: the upper part and the diagonal of the block take A_bb transposed,
    // and its strictly lower part (L_bb, read only above) becomes zero
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<f32x4*>(&sLA[(16 * b + jj) * P64 + 16 * b + 4 * r4]) =
          f32x4{x[4 * r4], x[4 * r4 + 1], x[4 * r4 + 2], x[4 * r4 + 3]};
  }
  __syncthreads();

  // ---- off-diagonal blocks of (I+L)^-1: A_IJ = -A_II sum_{J<=m<I} L_Im A_mJ.
  // Wave J forms the blocks of its own block column J (I = J+1 .. 3) in order,
  // on the fp32 matrix cores (16x16x4 per pass, four passes per 16-wide
  // reduction).  Pass p of a product gives lane l the reduction index
  // 4*(l/16) + p, so an accumulator tile (lane l: rows 4*(l/16) .. +3, column
  // l%16) is, element p, exactly the B operand of pass p: the column blocks
  // stay in registers and only the diagonal inverses (other waves) and L come
  // from LDS.
  if (wave < 3) {
    const int J = wave;
    f32x4 col[4];   // col[m] = A_mJ as an accumulator tile (m >= J)
#pragma unroll
    for (int m = 0; m < 3; ++m)
      if (m == J)
        col[m] = *reinterpret_cast<const f32x4*>(&sLA[(16 * J + r16) * P64 + 16 * J + 4 * quad]);
#pragma unroll
    for (int I = 1; I < 4; ++I) {
      if (I <= J) continue;
      f32x4 x = zero4();
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        if (m < J || m >= I) continue;
        const f32x4 lrow = *reinterpret_cast<const f32x4*>(&sL[(16 * I + r16) * P64 + 16 * m + 4 * quad]);
#pragma unroll
        for (int pss = 0; pss < 4; ++pss) x = __builtin_amdgcn_mfma_f32_16x16x4f32(lrow[pss], col[m][pss], x, 0, 0, 0);
      }
      // row r16 of A_II (the block's lower part holds zeros where A_II has them)
      f32x4 arow;
#pragma unroll
      for (int e = 0; e < 4; ++e) arow[e] = sLA[(16 * I + 4 * quad + e) * P64 + 16 * I + r16];
      f32x4 y = zero4();
#pragma unroll
      for (int pss = 0; pss < 4; ++pss) y = __builtin_amdgcn_mfma_f32_16x16x4f32(arow[pss], x[pss], y, 0, 0, 0);
      col[I] = -y;
      // A_IJ (I > J) transposed into block (J, I) of sLA, above L
      *reinterpret_cast<f32x4*>(&sLA[(16 * J + r16) * P64 + 16 * I + 4 * quad]) = -y;
    }
  }
  __syncthreads();

  // ---- u^T = (A diag(beta) v)^T (fp16 | fp32),  w = A diag(beta) X (token dtype)
  // Both reduction slices are used by every wave: the strictly upper blocks
  // of A are zero in LDS, so the products need no per-wave bounds.
  {
    const int I = wave;
    // rows of A diag(beta): reduction slots in the stored fragment order for
    // bf16 tokens (slots 8g .. 8g+3: tokens 4g .. 4g+3, 8g+4 .. 8g+7: tokens
    // 16+4g .. 16+4g+3 of each 32), in natural order for fp32 tokens
    Frag fa[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int j0 = F32 ? 32 * ks + 8 * quad : 32 * ks + 4 * quad;
      const int j1 = F32 ? j0 + 4 : j0 + 16;
      float ar[8], bt[8], x[8];
      const int ia = 16 * I + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ar[e] = j0 + e <= ia ? sLA[(j0 + e) * P64 + ia] : 0.f;
        ar[4 + e] = j1 + e <= ia ? sLA[(j1 + e) * P64 + ia] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bt[e] = sBeta(j0 + e);
        bt[4 + e] = sBeta(j1 + e);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = ar[e] * bt[e];
      fa[ks] = split8(x);
    }
    auto tile = [&](const ST* bsrc, const u32x4* fsrc, int ct, bool a_left) __attribute__((always_inline)) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if constexpr (F32) {
          const ST* bp = bsrc + (16 * ct + r16) * PT + 32 * ks + 8 * quad;
          float xb[8];
          load8(reinterpret_cast<const float*>(bp), xb);
          acc = a_left ? mma3(fa[ks], split8(xb), acc) : mma3(split8(xb), fa[ks], acc);
        } else {
          const bf16x8 b = __builtin_bit_cast(bf16x8, fsrc[(2 * ct + ks) * 64 + lane]);
          if (a_left) {
            acc = mfma(fa[ks].hi, b, acc);
            acc = mfma(fa[ks].lo, b, acc);
          } else {
            acc = mfma(b, fa[ks].hi, acc);
            acc = mfma(b, fa[ks].lo, acc);
          }
        }
      }
      return acc;
    };
#pragma unroll
    for (int ct = 0; ct < VD / 16; ++ct) {
      const f32x4 acc = tile(sVT, sVF, ct, true);
      const int uo = cfrag_off(16 * I + 4 * quad, 16 * ct + r16, VD / 16);
      if constexpr (F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(rec + RL.ut) + uo) = acc;
      } else {
        __builtin_nontemporal_store(pack4_f16(acc), reinterpret_cast<u32x2*>(reinterpret_cast<_Float16*>(rec + RL.ut) + uo));
      }
    }
    // w^T tiles (X^T rows as the A operand): this lane holds token 16*I + r16,
    // channels 16*ct + 4*quad .. +3 -> one vector store
    using WT = typename std::conditional<F32, float, _Float16>::type;   // w: fp16 with bf16 tokens
    WT* wbase = reinterpret_cast<WT*>(rec + RL.w);
#pragma unroll
    for (int ct = 0; ct < KD / 16; ++ct) {
      const f32x4 acc = tile(sXT, sXF, ct, false);
      store4(wbase + frag_off(16 * I + r16, 16 * ct + 4 * quad, NKS), acc);
    }
  }
}

}  // namespace

hipError_t launch_intra(int K, int V, int dtype, const IntraArgs& a, hipStream_t s) {
  if (a.nchunks == 0 || a.Hv == 0) return hipSuccess;
  const long nb = (long)a.nchunks * a.Hv;
  if (nb > 0x7fffffffL) return hipErrorInvalidValue;
  dim3 grid((unsigned)nb), block(256);
#define KDA_INTRA_CASE(KK, VV, TT)                                          \
  if (K == KK && V == VV) {                                                 \
    return a.q ? launch(intra_kernel<KK, VV, TT, true>, grid, block, s, a)  \
               : launch(intra_kernel<KK, VV, TT, false>, grid, block, s, a); \
  }
  if (dtype == 1) {
    KDA_INTRA_CASE(128, 128, bf16_t)
    KDA_INTRA_CASE(64, 64, bf16_t)
    KDA_INTRA_CASE(128, 64, bf16_t)
    KDA_INTRA_CASE(64, 128, bf16_t)
  } else {
    KDA_INTRA_CASE(128, 128, float)
    KDA_INTRA_CASE(64, 64, float)
    KDA_INTRA_CASE(128, 64, float)
    KDA_INTRA_CASE(64, 128, float)
  }
#undef KDA_INTRA_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
