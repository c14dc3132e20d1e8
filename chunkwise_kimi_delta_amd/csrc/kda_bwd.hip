// Chunkwise KDA backward: gradients of the forward with respect to q, k, v,
// the gate input, beta, A_log, dt_bias and the initial state.
//
// Follows "KDA Chunk Backward — TPU/Pallas Kernel Design": section 1.1 (what
// the backward recomputes instead of storing), 2.2 (dAv: the output's
// gradient into the intra-chunk attention and v_new), 2.3 (the reverse
// inter-chunk recurrence of the state gradient, the WY / intra-chunk
// backward and the reverse cumsum of the gate gradient) and 2.5 (the gate
// backward), and "Hyper-Parallel Chunk KDA" section 5.2 (backward stages).
// Arithmetic is fp32.  Stored in fp16 (11 significant bits; magnitudes up to
// 65504, the forward's bound on v_new with bf16 tokens): the record's w, u,
// kg and qg, and the chunk-entry states and exit gradients that the scans
// hand to the chunk kernel; the rest of the record (G, A, Aqk, beta, the norm
// factors) stays fp32.  The two state scans and the chunk kernel's passes over K and V
// multiply bf16 hi/lo operand pairs (~16 significant bits per operand, fp32
// accumulation, three passes per product); the other chunk-local products run
// on the fp32 matrix cores.  The decay
// ratios exp(G_i - G_j) of a chunk are never formed from a positive exponent:
// a block of rows against an earlier block splits at the later block's first
// row r into 2^(G_i - G_r) 2^(G_r - G_j), both <= 1 (G is the in-chunk cumsum,
// non-increasing), and the pairs inside a 16-row block use its row 8 as the
// reference when no factor that makes exceeds 2^96, else the levels of a
// binary split, so prescaled operands turn the pair sums into plain matrix
// products for any decay.
//
// Per chunk (rows i < C, h the chunk-entry state, h' its exit state):
//   v_new = u - w h,   o = qg h + Aqk v_new,   h' = D h + kg^T v_new
// with u = A (b v), w = A (b k e^G), A = (I + L)^-1, L_ij = b_i sum_c
// k_ic k_jc e^(G_ic - G_jc) (i > j), Aqk_ij = s sum_c q_ic k_jc e^(G_ic -
// G_jc) (i >= j), qg = s q e^G, kg = k e^(G_C - G), D = diag(e^G_C).  Given
// dh' and do:
//   dv_new = Aqk^T do + kg dh',   dh = qg^T do + D dh' - w^T dv_new
//   dAqk = tril(do v_new^T),  dqg = do h^T,  dkg = v_new dh'^T,  dD = rowsum(h . dh')
//   dw = -dv_new h^T,  d(b v) = A^T dv_new,  d(b k e^G) = A^T dw
//   dA = tril(dv_new (b v)^T + dw (b k e^G)^T),  dL = -strict_tril(A^T dA A^T)
// and the pair sums of dL and dAqk back into k, q, b and G.
//
// Kernels:
//   bwd_prep_kernel   (chunk, head): gate, norms, sigmoid, G, L, Aqk, A, u, w, kg, qg
//                     -> fp32 record
//   bwd_state_kernel  (sequence, head): the forward state recurrence, storing every
//                     chunk-entry state
//   bwd_scan_kernel   (sequence, head): the reverse recurrence of dh, storing each
//                     chunk's exit gradient; dh0 at the end
//   bwd_chunk_kernel  (chunk, head): the chunk-local products; dL and dAqk out, partial
//                     gradients of q, k, G and beta
//   bwd_pairs_kernel  (chunk, head): the pair sums of dL and dAqk into those partials,
//                     then the reverse cumsum of the gate gradient
//   bwd_qk_kernel     (token, q/k head): grouped-head sum and L2Norm backward
//   bwd_gate_kernel / bwd_gate_sum_kernel: gate and sigmoid backward, dA_log and
//                     dt_bias sums (two passes, fixed order: deterministic)
#include "kda_bwd_launch.h"

#include <type_traits>

namespace kda {

namespace {

template <typename T> __device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<bf16_t>(const bf16_t* p) { return bf2f(*p); }
// One element through a buffer descriptor (zero past its end), as a float.
template <typename T> __device__ __forceinline__ float ldb(rsrc_t r, uint32_t byte_off);
template <> __device__ __forceinline__ float ldb<float>(rsrc_t r, uint32_t o) { return __uint_as_float(buf_load4(r, o)); }
template <> __device__ __forceinline__ float ldb<bf16_t>(rsrc_t r, uint32_t o) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)o, 0, 0) << 16);
}
template <typename T> __device__ __forceinline__ f32x4 ldb4(rsrc_t r, uint32_t byte_off);
template <> __device__ __forceinline__ f32x4 ldb4<float>(rsrc_t r, uint32_t o) { return __builtin_bit_cast(f32x4, buf_load16(r, o)); }
template <> __device__ __forceinline__ f32x4 ldb4<bf16_t>(rsrc_t r, uint32_t o) {
  const u32x2 u = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)o, 0, 0));
  f32x4 x;
  x[0] = __uint_as_float(u.x << 16);
  x[1] = __uint_as_float(u.x & 0xffff0000u);
  x[2] = __uint_as_float(u.y << 16);
  x[3] = __uint_as_float(u.y & 0xffff0000u);
  return x;
}
// Four consecutive fp16 elements (8 bytes, aligned) as floats.
__device__ __forceinline__ f32x4 ld4h(const _Float16* p) { return unpack4_f16(*reinterpret_cast<const u32x2*>(p)); }
// Four consecutive elements as floats (8 bytes of bf16 or 16 bytes of fp32, aligned).
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4(const bf16_t* p) {
  const u32x2 u = *reinterpret_cast<const u32x2*>(p);
  f32x4 r;
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xffff0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xffff0000u);
  return r;
}

__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }
// 2^x on the transcendental unit; every decay exponent here is <= 0
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float LOG2E_F = 1.4426950408889634f;
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

// Workgroups of NTH threads: 16 waves, four per SIMD.  The kernels run one
// workgroup per CU (their LDS is 100 - 160 KB), so the extra waves are what
// hides the latency of each phase's loads; each wave owns fewer output tiles,
// which keeps its accumulators within 128 registers.
constexpr int NTH = 1024;

struct ChunkPos {
  int n, C;
  int64_t tok0;     // first token of the chunk
  int64_t slot;     // head-major (head, global chunk) slot
  int gc;
};
__device__ __forceinline__ ChunkPos chunk_pos(const SeqInfo& s, int gc, int h, int nchunks) {
  ChunkPos p;
  p.gc = gc;
  p.n = seq_of_chunk(s, gc);
  int64_t t0;
  int len;
  seq_range(s, p.n, t0, len);
  const int cidx = gc - chunk_base(s, p.n);
  p.tok0 = t0 + (int64_t)cidx * BT;
  p.C = min(BT, len - cidx * BT);
  p.slot = (int64_t)h * nchunks + gc;
  return p;
}

// acc += a * b on the fp32 matrix cores (16 x 16 x 4 per instruction)
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------ tile ownership
// Tiles of a R x V output (R = 64 or K rows, V columns) over NW waves: wave w owns tiles w * TPW + t (t < TPW), so that all its tiles lie in
// one block of 16 rows (rb) and consecutive column blocks (cb).
template <int R, int V, int NW = NTH / 64>
struct STiles {
  static constexpr int NCB = V / 16, NT = (R / 16) * NCB, TPW = NT / NW;
  static_assert(NCB % TPW == 0 || TPW % NCB == 0, "a wave's tiles share one row block");
  int rb, cb0, r16, q;
  __device__ explicit STiles(int tid) : r16(tid & 15), q((tid >> 4) & 3) {
    const int T0 = (tid >> 6) * TPW;
    rb = T0 / NCB;
    cb0 = T0 % NCB;
  }
};
static_assert(STiles<128, 128>::TPW == 4 && STiles<64, 128>::TPW == 2 && STiles<64, 64>::TPW == 1,
              "tile counts per wave");

// ------------------------------------------------------ state scans
// Both state scans run one workgroup per (sequence, head) with VD / 16 waves
// and keep the K x V state in registers: wave w owns column block w (16
// columns), KD / 16 accumulator tiles in which lane l holds rows
// 16 t + 4 (l / 16) + e of column 16 w + l % 16.  A chunk's operands are
// staged once in LDS as matrix-core fragments of bf16 hi/lo pairs (hi =
// bf16(x), lo = bf16(x - hi): ~16 significant bits), and every product is
// three passes of v_mfma_f32_16x16x32_bf16 (hi.hi + lo.hi + hi.lo) into fp32
// accumulators.  Inside each aligned block of 32 the reduction index x sits
// in lane group (x & 15) >> 2, slot 4 (x >> 4) + (x & 3) of a fragment, so
// that two accumulator tiles of 16 rows are, as they are, the B operand of a
// product that reduces over those 32 rows: the state and v_new (dv_new) feed
// the next product without leaving the registers, and nothing but the
// chunk's operand staging needs a barrier.
// The stored chunk states and gradients (K x V fp32 per chunk) keep four
// consecutive rows of a column together: element (k, v) at sq_index(k, v), so
// that an accumulator tile's four rows of a column are one 16-byte store.
__host__ __device__ constexpr int sq_index(int k, int v, int V) { return ((k >> 2) * V + v) * 4 + (k & 3); }
constexpr int FRB = 2048;   // bytes of one fragment in LDS: hi (64 lanes x 16 B), then lo

// reduction index (inside its block of 32) of slot j of lane group g
__device__ __forceinline__ int sg_index(int g, int j) { return ((j >> 2) << 4) | (g << 2) | (j & 3); }

__device__ __forceinline__ Frag frag_get(const unsigned char* f, int lane) {
  Frag r;
  r.hi = *reinterpret_cast<const bf16x8*>(f + 16 * lane);
  r.lo = *reinterpret_cast<const bf16x8*>(f + 1024 + 16 * lane);
  return r;
}
__device__ __forceinline__ void frag_put(unsigned char* f, int lane, const Frag& x) {
  *reinterpret_cast<bf16x8*>(f + 16 * lane) = x.hi;
  *reinterpret_cast<bf16x8*>(f + 1024 + 16 * lane) = x.lo;
}
// acc += a b, both operands split (the lo.lo term, below 2^-16 of the
// product, is dropped)
__device__ __forceinline__ f32x4 mma3(const Frag& a, const Frag& b, f32x4 acc) {
  acc = mfma(a.hi, b.hi, acc);
  acc = mfma(a.lo, b.hi, acc);
  return mfma(a.hi, b.lo, acc);
}
// This wave's LDS writes done before its next LDS reads (a wave's LDS
// operations complete in order; this also keeps the compiler from moving
// reads above the writes)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}
// Fragments whose reduction runs along the rows of a row-major source S
// (A[c][t] = S[t][c], or a B operand B[t][c]) for the 16 columns c and 32
// rows t of one block of S are transposed in their own LDS: the wave first
// stages the block there (row t at 64 t bytes; lane l holds row l / 2,
// columns 8 (l % 2) .. +7), then each lane reads its column at its eight
// rows and overwrites the staging with the split fragment.
__device__ __forceinline__ void stage_t(unsigned char* f, int lane, const float (&x)[8]) {
  float* st = reinterpret_cast<float*>(f) + 8 * lane;
  *reinterpret_cast<f32x4*>(st) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(st + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void gather_t(const unsigned char* f, int lane, float (&y)[8]) {
  const float* st = reinterpret_cast<const float*>(f);
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = st[16 * sg_index(lane >> 4, j) + (lane & 15)];
}
// the same for a bf16 source, hi part only (1 KiB: row t at 32 t bytes)
__device__ __forceinline__ void stage_t16(unsigned char* f, int lane, const u32x4& x) {
  *reinterpret_cast<u32x4*>(f + 16 * lane) = x;
}
__device__ __forceinline__ bf16x8 gather_t16(const unsigned char* f, int lane) {
  const bf16_t* st = reinterpret_cast<const bf16_t*>(f);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = (uint32_t)st[16 * sg_index(lane >> 4, 2 * j) + (lane & 15)] |
           ((uint32_t)st[16 * sg_index(lane >> 4, 2 * j + 1) + (lane & 15)] << 16);
  return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
}
__device__ __forceinline__ void ld8(const float* p, float (&x)[8]) {
  const f32x4 a = ld4(p), b = ld4(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
// The same from fp16 sections of the record.
__device__ __forceinline__ void ld8h(const _Float16* p, float (&x)[8]) {
  const f32x4 a = ld4h(p), b = ld4h(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
__device__ __forceinline__ void ld8sh(const _Float16* p, float (&x)[8]) {
  const f32x4 a = ld4h(p), b = ld4h(p + 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
// fp16 section of a record
__device__ __forceinline__ const _Float16* h16(const float* p) { return reinterpret_cast<const _Float16*>(p); }
__device__ __forceinline__ _Float16* h16(float* p) { return reinterpret_cast<_Float16*>(p); }
// eight values at p[0..3] and p[16..19]: the slots of lane group g of a
// fragment whose reduction index runs along the row (p = row + 32 kb + 4 g)
__device__ __forceinline__ void ld8s(const float* p, float (&x)[8]) {
  const f32x4 a = ld4(p), b = ld4(p + 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

// 4 x 4 transpose across the four lanes of a quad (b = lane & 3): lane b's
// x[j] becomes lane j's x[b].  Two exchanges of 2 x 2 blocks through DPP quad
// permutations (xor 1, then xor 2), every lane active.
template <int CTRL> __device__ __forceinline__ float dpp_q(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ void quad_transpose(f32x4& x, int b) {
  const bool o1 = b & 1, o2 = b & 2;
  float r = dpp_q<0xB1>(o1 ? x[0] : x[1]);   // quad_perm [1, 0, 3, 2]
  x[0] = o1 ? r : x[0];
  x[1] = o1 ? x[1] : r;
  r = dpp_q<0xB1>(o1 ? x[2] : x[3]);
  x[2] = o1 ? r : x[2];
  x[3] = o1 ? x[3] : r;
  r = dpp_q<0x4E>(o2 ? x[0] : x[2]);         // quad_perm [2, 3, 0, 1]
  x[0] = o2 ? r : x[0];
  x[2] = o2 ? x[2] : r;
  r = dpp_q<0x4E>(o2 ? x[1] : x[3]);
  x[1] = o2 ? r : x[1];
  x[3] = o2 ? x[3] : r;
}

// The chunk-entry states for the backward, in fp32 from the fp32 records:
// h <- D h + kg^T (u - w h), every entry state stored (in fp16).  Operands per chunk:
// -w as A[token][K] and kg^T = (k 2^(G_C - G))^T as A[K][token].
template <int KD, int VD>
__global__ __launch_bounds__(VD * 4) void bwd_state_kernel(BwdArgs a) {
  constexpr int NW = VD / 16, NKT = KD / 16, NKB = KD / 32;
  constexpr int NFW = 4 * NKB, NFK = 2 * NKT;
  constexpr int IW = (NFW + NW - 1) / NW, IK = (NFK + NW - 1) / NW;   // fragments per wave
  __shared__ __attribute__((aligned(16))) unsigned char sF[(NFW + NFK) * FRB];
  __shared__ __attribute__((aligned(16))) float sD[KD];   // 2^(G_C) per channel
  constexpr BwdRec R = bwd_rec(KD, VD);
  const int h = blockIdx.x % a.Hv, n = blockIdx.x / a.Hv, tid = threadIdx.x;
  // (the wave index is uniform: per-wave branches stay scalar)
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), r16 = lane & 15, g = lane >> 4;
  const int col = 16 * wave + r16;
  unsigned char* fW = sF;
  unsigned char* fK = sF + NFW * FRB;
  int64_t tok0s;
  int len;
  seq_range(a.seq, n, tok0s, len);
  const int nck = (len + BT - 1) / BT;
  const int cb = chunk_base(a.seq, n);
  f32x4 H[NKT];
  {
    const float* h0 = a.h0 ? a.h0 + ((int64_t)n * a.Hv + h) * (KD * VD) : nullptr;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) H[t][e] = h0 ? h0[(16 * t + 4 * g + e) * VD + col] : 0.f;
  }
  for (int c = 0; c < nck; ++c) {
    const int64_t slot = (int64_t)h * a.nchunks + cb + c;
    const float* rec = a.rec + slot * (int64_t)(R.bytes / 4);
    const float* Gc = rec + R.G + (min(BT, len - c * BT) - 1) * KD;
    {  // the chunk-entry state out
      _Float16* dst = a.h_store_w + slot * (int64_t)(KD * VD);
#pragma unroll
      for (int t = 0; t < NKT; ++t) *reinterpret_cast<u32x2*>(dst + sq_index(16 * t + 4 * g, col, VD)) = pack4_f16(H[t]);
    }
    // then the loads: u (v_new starts at u), -w and kg
    f32x4 vn[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) vn[rt] = ld4h(h16(rec + R.u) + sq_index(16 * rt + 4 * g, col, VD));
    const float gcv = tid < KD ? Gc[tid] : 0.f;
    // (a wave past the last fragment loads the last one again and skips its write)
    float xw[IW][8], xk[IK][8];
#pragma unroll
    for (int i = 0; i < IW; ++i) {
      const int f = min(wave + NW * i, NFW - 1);
      ld8sh(h16(rec + R.w) + (16 * (f / NKB) + r16) * KD + 32 * (f % NKB) + 4 * g, xw[i]);
    }
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int f = min(wave + NW * i, NFK - 1);
      const int t = 32 * (f % 2) + (lane >> 1), k0 = 16 * (f / 2) + 8 * (lane & 1);
      ld8h(h16(rec + R.kg) + t * KD + k0, xk[i]);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load issued before the first use
#pragma unroll
    for (int i = 0; i < IW; ++i) {
      const int f = wave + NW * i;
      if (f < NFW) {
#pragma unroll
        for (int j = 0; j < 8; ++j) xw[i][j] = -xw[i][j];
        frag_put(fW + f * FRB, lane, split8(xw[i]));
      }
    }
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int f = wave + NW * i;
      if (f < NFK) stage_t(fK + f * FRB, lane, xk[i]);
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int f = wave + NW * i;
      if (f < NFK) gather_t(fK + f * FRB, lane, xk[i]);
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < IK; ++i) {
      const int f = wave + NW * i;
      if (f < NFK) frag_put(fK + f * FRB, lane, split8(xk[i]));
    }
    if (tid < KD) sD[tid] = ex2(gcv);
    __syncthreads();
    // v_new = u - w h: the state is the B operand as it sits in the accumulators
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const Frag b = split_pair(H[2 * kb], H[2 * kb + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) vn[rt] = mma3(frag_get(fW + (rt * NKB + kb) * FRB, lane), b, vn[rt]);
    }
    // h = D h + kg^T v_new
    const Frag vb0 = split_pair(vn[0], vn[1]), vb1 = split_pair(vn[2], vn[3]);
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const f32x4 d = *reinterpret_cast<const f32x4*>(sD + 16 * t + 4 * g);
      f32x4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = d[e] * H[t][e];
      acc = mma3(frag_get(fK + (2 * t) * FRB, lane), vb0, acc);
      H[t] = mma3(frag_get(fK + (2 * t + 1) * FRB, lane), vb1, acc);
    }
    __syncthreads();   // every wave done with this chunk's fragments
  }
}

// ------------------------------------------------------ reverse state scan
// dh over the chunks in reverse: dv_new = Aqk^T do + kg dh',
// dh = qg^T do + D dh' - w^T dv_new, every chunk's exit gradient stored.
// Operands per chunk: kg as A[token][K], Aqk^T as A[token i][token r], qg^T
// and -w^T as A[K][token], do as B[token][column] (bf16 tokens are exact in
// one bf16 part; fp32 tokens are split like the rest).
template <int KD, int VD, typename IT>
__global__ __launch_bounds__(VD * 4) void bwd_scan_kernel(BwdArgs a) {
  constexpr bool F32 = sizeof(IT) == 4;
  constexpr int NW = VD / 16, NKT = KD / 16, NKB = KD / 32;
  constexpr int NFG = 4 * NKB, NFA = 8, NFQ = 2 * NKT, NFD = 2 * NW;
  constexpr int DOB = F32 ? FRB : FRB / 2;   // bytes of a do fragment
  constexpr int IG = (NFG + NW - 1) / NW, IA = (NFA + NW - 1) / NW, IQ = (NFQ + NW - 1) / NW;
  __shared__ __attribute__((aligned(16))) unsigned char sF[(NFG + NFA + 2 * NFQ) * FRB + NFD * DOB];
  __shared__ __attribute__((aligned(16))) float sD[KD];
  constexpr BwdRec R = bwd_rec(KD, VD);
  const int h = blockIdx.x % a.Hv, n = blockIdx.x / a.Hv, tid = threadIdx.x;
  // (the wave index is uniform: per-wave branches stay scalar)
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), r16 = lane & 15, g = lane >> 4;
  const int col = 16 * wave + r16;
  unsigned char* fG = sF;
  unsigned char* fA = fG + NFG * FRB;
  unsigned char* fQ = fA + NFA * FRB;
  unsigned char* fWT = fQ + NFQ * FRB;
  unsigned char* fD = fWT + NFQ * FRB;
  int64_t tok0s;
  int len;
  seq_range(a.seq, n, tok0s, len);
  const int nck = (len + BT - 1) / BT;
  const int cb = chunk_base(a.seq, n);
  const IT* dout = static_cast<const IT*>(a.dout);
  f32x4 DH[NKT];   // dh' of the last chunk: the final state's gradient
  {
    const float* dht = a.dht ? a.dht + ((int64_t)n * a.Hv + h) * (KD * VD) : nullptr;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) DH[t][e] = dht ? dht[(16 * t + 4 * g + e) * VD + col] : 0.f;
  }
  for (int c = nck - 1; c >= 0; --c) {
    const int64_t slot = (int64_t)h * a.nchunks + cb + c;
    const float* rec = a.rec + slot * (int64_t)(R.bytes / 4);
    const int C = min(BT, len - c * BT);
    const int64_t tok0 = tok0s + (int64_t)c * BT;
    const float* Gc = rec + R.G + (C - 1) * KD;
    // the exit gradient of this chunk out
    if (a.dh_store) {
      _Float16* dst = a.dh_store + slot * (int64_t)(KD * VD);
#pragma unroll
      for (int t = 0; t < NKT; ++t) *reinterpret_cast<u32x2*>(dst + sq_index(16 * t + 4 * g, col, VD)) = pack4_f16(DH[t]);
    }
    // then the loads (a wave past the last fragment of a kind loads the last
    // one again and skips its write)
    const float gcv = tid < KD ? Gc[tid] : 0.f;
    float xg[IG][8], xa[IA][8], xq[IQ][8], xw[IQ][8];
#pragma unroll
    for (int i = 0; i < IG; ++i) {
      const int f = min(wave + NW * i, NFG - 1);
      ld8sh(h16(rec + R.kg) + (16 * (f / NKB) + r16) * KD + 32 * (f % NKB) + 4 * g, xg[i]);
    }
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const int f = min(wave + NW * i, NFA - 1);   // f = 2 * (block of 16 i) + (block of 32 r)
      ld8(rec + R.aqk + (32 * (f % 2) + (lane >> 1)) * BT + 16 * (f / 2) + 8 * (lane & 1), xa[i]);
    }
#pragma unroll
    for (int i = 0; i < IQ; ++i) {
      const int f = min(wave + NW * i, NFQ - 1);   // f = 2 * (block of 16 K) + (block of 32 tokens)
      const int o = (32 * (f % 2) + (lane >> 1)) * KD + 16 * (f / 2) + 8 * (lane & 1);
      ld8h(h16(rec + R.qg) + o, xq[i]);
      ld8h(h16(rec + R.w) + o, xw[i]);
    }
    // do: this wave's two fragments (column block = wave), rows past the chunk zero
    float xd[2][8];
    u32x4 xd16[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int t = 32 * tb + (lane >> 1);
      const IT* p = dout + ((tok0 + t) * a.Hv + h) * VD + 16 * wave + 8 * (lane & 1);
      if constexpr (F32) {
        if (t < C) ld8(reinterpret_cast<const float*>(p), xd[tb]);
        else
#pragma unroll
          for (int j = 0; j < 8; ++j) xd[tb][j] = 0.f;
      } else {
        xd16[tb] = t < C ? *reinterpret_cast<const u32x4*>(p) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // every load issued before the first use
    // kg fragments (reduction along the row: no transposition)
#pragma unroll
    for (int i = 0; i < IG; ++i) {
      const int f = wave + NW * i;
      if (f < NFG) frag_put(fG + f * FRB, lane, split8(xg[i]));
    }
    // transposed fragments: stage, gather, split
#pragma unroll
    for (int i = 0; i < IA; ++i)
      if (wave + NW * i < NFA) stage_t(fA + (wave + NW * i) * FRB, lane, xa[i]);
#pragma unroll
    for (int i = 0; i < IQ; ++i) {
      const int f = wave + NW * i;
      if (f < NFQ) {
#pragma unroll
        for (int j = 0; j < 8; ++j) xw[i][j] = -xw[i][j];
        stage_t(fQ + f * FRB, lane, xq[i]);
        stage_t(fWT + f * FRB, lane, xw[i]);
      }
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      if constexpr (F32) stage_t(fD + (2 * wave + tb) * DOB, lane, xd[tb]);
      else stage_t16(fD + (2 * wave + tb) * DOB, lane, xd16[tb]);
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < IA; ++i)
      if (wave + NW * i < NFA) gather_t(fA + (wave + NW * i) * FRB, lane, xa[i]);
#pragma unroll
    for (int i = 0; i < IQ; ++i)
      if (wave + NW * i < NFQ) {
        gather_t(fQ + (wave + NW * i) * FRB, lane, xq[i]);
        gather_t(fWT + (wave + NW * i) * FRB, lane, xw[i]);
      }
    bf16x8 dh16[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      if constexpr (F32) gather_t(fD + (2 * wave + tb) * DOB, lane, xd[tb]);
      else dh16[tb] = gather_t16(fD + (2 * wave + tb) * DOB, lane);
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < IA; ++i)
      if (wave + NW * i < NFA) frag_put(fA + (wave + NW * i) * FRB, lane, split8(xa[i]));
#pragma unroll
    for (int i = 0; i < IQ; ++i)
      if (wave + NW * i < NFQ) {
        frag_put(fQ + (wave + NW * i) * FRB, lane, split8(xq[i]));
        frag_put(fWT + (wave + NW * i) * FRB, lane, split8(xw[i]));
      }
    // do stays in this wave's registers: its fragments are its own column block
    Frag dof[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      if constexpr (F32) dof[tb] = split8(xd[tb]);
      else dof[tb].hi = dh16[tb];
    }
    if (tid < KD) sD[tid] = ex2(gcv);
    __syncthreads();
    // dv_new = Aqk^T do + kg dh' (this wave's columns)
    f32x4 dv[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) dv[rt] = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const Frag A = frag_get(fA + (2 * rt + kb) * FRB, lane);
        if constexpr (F32) dv[rt] = mma3(A, dof[kb], dv[rt]);
        else dv[rt] = mfma(A.lo, dof[kb].hi, mfma(A.hi, dof[kb].hi, dv[rt]));
      }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const Frag b = split_pair(DH[2 * kb], DH[2 * kb + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) dv[rt] = mma3(frag_get(fG + (rt * NKB + kb) * FRB, lane), b, dv[rt]);
    }
    // dh = D dh' + qg^T do - w^T dv_new
    const Frag vb0 = split_pair(dv[0], dv[1]), vb1 = split_pair(dv[2], dv[3]);
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const f32x4 d = *reinterpret_cast<const f32x4*>(sD + 16 * t + 4 * g);
      f32x4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = d[e] * DH[t][e];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const Frag Q = frag_get(fQ + (2 * t + tb) * FRB, lane);
        if constexpr (F32) acc = mma3(Q, dof[tb], acc);
        else acc = mfma(Q.lo, dof[tb].hi, mfma(Q.hi, dof[tb].hi, acc));
        acc = mma3(frag_get(fWT + (2 * t + tb) * FRB, lane), tb ? vb1 : vb0, acc);
      }
      DH[t] = acc;
    }
    __syncthreads();   // every wave done with this chunk's fragments
  }
  if (a.dh0) {
    float* d0 = a.dh0 + ((int64_t)n * a.Hv + h) * (KD * VD);
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) d0[(16 * t + 4 * g + e) * VD + col] = DH[t][e];
  }
}

// ------------------------------------------------------------------ prep
// The fp32 record of one (chunk, head): gate, norms, sigmoid, the in-chunk
// cumsum G (log2 units), L = tril(beta k k^T decayed), Aqk, A = (I + L)^-1,
// u = A (beta v), w = A (beta k 2^G).  L and Aqk are formed on the fp32 matrix
// cores in 16 x 16 tiles: a tile below the diagonal blocks against the first
// row r of its row block (factors 2^(G_i - G_r) and 2^(G_r - G_j), both <= 1);
// a diagonal tile in four split levels (blocks of 16, 8, 4 and 2 rows: the
// pairs with i in the upper and j in the lower half of one block, against
// that upper half's first row), every pair i > j meeting exactly one level.
template <int KD, int VD, typename IT>
__global__ __launch_bounds__(NTH) void bwd_prep_kernel(BwdArgs a) {
  constexpr int MX = KD > VD ? KD : VD;
  constexpr int LX = MX + 4, LS = BT + 4;
  __shared__ __attribute__((aligned(16))) float sG[BT * LX];
  __shared__ __attribute__((aligned(16))) float sK[BT * LX];
  __shared__ __attribute__((aligned(16))) float sX[BT * LX];   // q, then beta v, then beta k 2^G
  __shared__ __attribute__((aligned(16))) float sL[BT * LS];
  __shared__ __attribute__((aligned(16))) float sA[BT * LS];
  __shared__ float sB[BT], sDiag[BT];
  constexpr BwdRec R = bwd_rec(KD, VD);
  int gc, h;
  chunk_head_of_block(blockIdx.x, gridDim.x, a.nchunks, a.Hv, a.Hk, gc, h);
  const ChunkPos P = chunk_pos(a.seq, gc, h, a.nchunks);
  const int hk = h / (a.Hv / a.Hk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, quad = lane >> 4;
  float* rec = a.rec + P.slot * (int64_t)(R.bytes / 4);
  const IT* q = static_cast<const IT*>(a.q);
  const IT* k = static_cast<const IT*>(a.k);
  const IT* g = static_cast<const IT*>(a.g);
  const IT* bt = static_cast<const IT*>(a.beta);
  const IT* v = static_cast<const IT*>(a.v);
  const bool gik = a.flags & F_GATE, l2 = a.flags & F_L2;
  const float lb = (a.flags & F_SAFE) ? a.lower_bound : -INFINITY;
  const float Aexp = gik ? expf(a.A_log[h]) : 0.f;

  // ---- gate, norms, beta: rows r = tid / TPR, channels CPT * (tid % TPR) .. +CPT-1.
  // softplus in log2 form on the transcendental unit: softplus(z) = max(z, 0)
  // + ln2 log2(1 + 2^(-|z| log2 e)); the decay is kept in log2 units
  {
    constexpr int TPR = NTH / BT, CPT = KD / TPR;   // threads per row, channels per thread
    static_assert(CPT % 4 == 0 && (TPR & (TPR - 1)) == 0, "whole 4-channel pieces per thread");
    const int r = tid / TPR, part = tid % TPR;
    const bool live = r < P.C;
    float kr[CPT], qr[CPT], gr[CPT], br[CPT];
    if (live) {
      const IT* kp = k + ((P.tok0 + r) * a.Hk + hk) * KD + part * CPT;
      const IT* qp = q + ((P.tok0 + r) * a.Hk + hk) * KD + part * CPT;
      const IT* gp = g + ((P.tok0 + r) * a.Hv + h) * KD + part * CPT;
#pragma unroll
      for (int e4 = 0; e4 < CPT; e4 += 4) {
        const f32x4 kv = ld4(kp + e4), qv = ld4(qp + e4), gv = ld4(gp + e4);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          kr[e4 + p] = kv[p];
          qr[e4 + p] = qv[p];
          gr[e4 + p] = gv[p];
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < CPT; ++e) kr[e] = qr[e] = gr[e] = 0.f;
    }
#pragma unroll
    for (int e4 = 0; e4 < CPT; e4 += 4) {
      const f32x4 bv = (gik && a.dt_bias) ? ld4(a.dt_bias + h * KD + part * CPT + e4) : zero4();
#pragma unroll
      for (int p = 0; p < 4; ++p) br[e4 + p] = bv[p];
    }
    float skk = 0.f, sqq = 0.f, sqk = 0.f;
    const float lb2 = !live ? 0.f : lb * LOG2E_F;     // (lb = -inf: no clamp)
    const float cA = live ? -Aexp * LOG2E_F : 0.f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      skk += kr[e] * kr[e];
      sqq += qr[e] * qr[e];
      sqk += qr[e] * kr[e];
      float gl;
      if (gik) {
        const float z = gr[e] + br[e];
        gl = cA * (fmaxf(z, 0.f) + 0.6931471805599453f * __builtin_amdgcn_logf(1.f + ex2(-LOG2E_F * fabsf(z))));
      } else {
        gl = live ? gr[e] * LOG2E_F : 0.f;
      }
      sG[r * LX + part * CPT + e] = fmaxf(gl, lb2);    // log2 units
    }
    for (int m = 1; m < TPR; m <<= 1) {
      skk += __shfl_xor(skk, m);
      sqq += __shfl_xor(sqq, m);
      sqk += __shfl_xor(sqk, m);
    }
    const float rk = live ? (l2 ? 1.f / sqrtf(skk + a.eps) : 1.f) : 0.f;
    const float rq = live ? (l2 ? 1.f / sqrtf(sqq + a.eps) : 1.f) : 0.f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const int c = part * CPT + e;
      sK[r * LX + c] = kr[e] * rk;
      sX[r * LX + c] = qr[e] * rq;
    }
    if (part == 0) {
      float b = live ? ldf(bt + (P.tok0 + r) * a.Hv + h) : 0.f;
      if (live && (a.flags & F_SIGMOID)) b = sigmoid_f(b);
      sB[r] = b;
      sDiag[r] = a.scale * rq * rk * sqk;      // Aqk_rr (decay factor 1)
      rec[R.rk + r] = rk;
      rec[R.rq + r] = rq;
    }
  }
  __syncthreads();
  {  // in-chunk cumsum of the decay: KD channels x NSG segments of SR rows
    constexpr int NSG = NTH / KD, SR = BT / NSG;
    float* sTot = sL;   // [NSG][KD] (sL unused until the tiles)
    const int cc = tid % KD, sg = tid / KD, r0 = sg * SR;
    float x[SR], run = 0.f;
#pragma unroll
    for (int r = 0; r < SR; ++r) {
      run += sG[(r0 + r) * LX + cc];
      x[r] = run;
    }
    sTot[sg * KD + cc] = run;
    __syncthreads();
    float off = 0.f;
    for (int s2 = 0; s2 < sg; ++s2) off += sTot[s2 * KD + cc];
#pragma unroll
    for (int r = 0; r < SR; ++r) sG[(r0 + r) * LX + cc] = x[r] + off;
  }
  __syncthreads();
  // store G, kg, qg and beta
#pragma unroll
  for (int s2 = 0; s2 < BT * KD / 4 / NTH; ++s2) {
    const int i = 4 * (tid + NTH * s2), r = i / KD, c = i % KD;
    *reinterpret_cast<f32x4*>(rec + R.G + i) = *reinterpret_cast<const f32x4*>(&sG[r * LX + c]);
    const f32x4 gv = *reinterpret_cast<const f32x4*>(&sG[r * LX + c]);
    const f32x4 gC = *reinterpret_cast<const f32x4*>(&sG[(P.C - 1) * LX + c]);
    const f32x4 kv = *reinterpret_cast<const f32x4*>(&sK[r * LX + c]);
    const f32x4 qv = *reinterpret_cast<const f32x4*>(&sX[r * LX + c]);
    f32x4 kgv, qgv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kgv[e] = kv[e] * ex2(gC[e] - gv[e]);
      qgv[e] = a.scale * qv[e] * ex2(gv[e]);
    }
    *reinterpret_cast<u32x2*>(h16(rec + R.kg) + i) = pack4_f16(kgv);
    *reinterpret_cast<u32x2*>(h16(rec + R.qg) + i) = pack4_f16(qgv);
  }
  if (tid < BT) rec[R.beta + tid] = sB[tid];

  // ---- L (beta-scaled, strict lower) and Aqk (scaled, lower): 6 tiles below
  // the diagonal blocks and the 4 diagonal tiles, one job each.  A diagonal
  // tile takes one reference row (its row 8) for every pair when none of the
  // factors that makes exceeds 2^96 in any channel; otherwise its job runs
  // the four split levels one after the other.
  float* aqk = rec + R.aqk;
  for (int job = wave; job < 10; job += NTH / 64) {
    f32x4 accL = zero4(), accQ = zero4();
    bool one_ref = false;
    if (job >= 6) {
      const int r0 = 16 * (job - 6);
      bool ok1 = true;
      for (int cc = lane; cc < KD; cc += 64) {
        const float gm = sG[(r0 + 8) * LX + cc];
        ok1 = ok1 && fmaxf(sG[r0 * LX + cc] - gm, gm - sG[(r0 + 15) * LX + cc]) < 96.f;
      }
      one_ref = __all(ok1);
    }
    if (job >= 6 && one_ref) {
      const int I = job - 6, ry = 16 * I + r16, rr = 16 * I + 8;
#pragma unroll 2
      for (int kk = 0; kk < KD; kk += 16) {
        const int c0 = kk + 4 * quad;
        const f32x4 gy = *reinterpret_cast<const f32x4*>(&sG[ry * LX + c0]);
        const f32x4 gr = *reinterpret_cast<const f32x4*>(&sG[rr * LX + c0]);
        const f32x4 ky = *reinterpret_cast<const f32x4*>(&sK[ry * LX + c0]);
        const f32x4 qy = *reinterpret_cast<const f32x4*>(&sX[ry * LX + c0]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float fa = ex2(gy[p] - gr[p]), fb = ky[p] * ex2(gr[p] - gy[p]);
          accL = mfma4(ky[p] * fa, fb, accL);
          accQ = mfma4(qy[p] * fa, fb, accQ);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int il = 4 * quad + e, jl = r16;
        const int i = 16 * I + il, j = 16 * I + jl;
        sL[i * LS + j] = il > jl ? sB[i] * accL[e] : 0.f;
        aqk[i * BT + j] = il > jl ? a.scale * accQ[e] : il == jl ? sDiag[i] : 0.f;
      }
    } else if (job < 6) {
      const int I = job < 1 ? 1 : job < 3 ? 2 : 3, J = job < 1 ? 0 : job < 3 ? job - 1 : job - 3;
      const int ri = 16 * I + r16, rj = 16 * J + r16, rr = 16 * I;
#pragma unroll 2
      for (int kk = 0; kk < KD; kk += 16) {
        const int c0 = kk + 4 * quad;
        const f32x4 gi = *reinterpret_cast<const f32x4*>(&sG[ri * LX + c0]);
        const f32x4 gj = *reinterpret_cast<const f32x4*>(&sG[rj * LX + c0]);
        const f32x4 gr = *reinterpret_cast<const f32x4*>(&sG[rr * LX + c0]);
        const f32x4 ki = *reinterpret_cast<const f32x4*>(&sK[ri * LX + c0]);
        const f32x4 qi = *reinterpret_cast<const f32x4*>(&sX[ri * LX + c0]);
        const f32x4 kj = *reinterpret_cast<const f32x4*>(&sK[rj * LX + c0]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float fa = ex2(gi[p] - gr[p]), b = kj[p] * ex2(gr[p] - gj[p]);
          accL = mfma4(ki[p] * fa, b, accL);
          accQ = mfma4(qi[p] * fa, b, accQ);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * I + 4 * quad + e, j = 16 * J + r16;
        sL[i * LS + j] = sB[i] * accL[e];
        aqk[i * BT + j] = a.scale * accQ[e];
        sL[j * LS + i] = 0.f;          // the mirrored tile above the diagonal
        aqk[j * BT + i] = 0.f;
      }
    } else {
      const int I = job - 6;
#pragma unroll 1
      for (int lv = 0; lv < 4; ++lv) {
      accL = zero4();
      accQ = zero4();
      const int y = r16, ry = 16 * I + y;
      const bool up = (y >> lv) & 1;
      const int rref = 16 * I + ((y >> (lv + 1)) << (lv + 1)) + (1 << lv);
#pragma unroll 2
      for (int kk = 0; kk < KD; kk += 16) {
        const int c0 = kk + 4 * quad;
        const f32x4 gy = *reinterpret_cast<const f32x4*>(&sG[ry * LX + c0]);
        const f32x4 gr = *reinterpret_cast<const f32x4*>(&sG[rref * LX + c0]);
        const f32x4 ky = *reinterpret_cast<const f32x4*>(&sK[ry * LX + c0]);
        const f32x4 qy = *reinterpret_cast<const f32x4*>(&sX[ry * LX + c0]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float f = ex2(up ? gy[p] - gr[p] : gr[p] - gy[p]);
          const float fk = ky[p] * f;
          accL = mfma4(fk, fk, accL);
          accQ = mfma4(qy[p] * f, fk, accQ);
        }
      }
      // entries (i upper, j lower) of one block at this level
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int il = 4 * quad + e, jl = r16;
        const int i = 16 * I + il, j = 16 * I + jl;
        if ((il >> (lv + 1)) == (jl >> (lv + 1)) && ((il >> lv) & 1) && !((jl >> lv) & 1)) {
          sL[i * LS + j] = sB[i] * accL[e];
          aqk[i * BT + j] = a.scale * accQ[e];
        } else if (lv == 0 && il <= jl) {   // diagonal and upper entries of the tile, once
          sL[i * LS + j] = 0.f;
          aqk[i * BT + j] = il == jl ? sDiag[i] : 0.f;
        }
      }
      }
    }
  }
  __syncthreads();

  // ---- A = (I + L)^-1: diagonal 16 x 16 blocks by substitution (16 lanes of
  // waves 0..3, one column each), then the blocks below them column block by
  // column block, A_IJ = -A_II sum_{J <= m < I} L_Im A_mJ, on the matrix cores
  if (wave < 4 && quad == 0) {
    const int b = wave, jj = r16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == jj) ? 1.f : 0.f;
#pragma unroll
      for (int kq = 0; kq < r; ++kq) s -= sL[(16 * b + r) * LS + 16 * b + kq] * x[kq];
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sA[(16 * b + r) * LS + 16 * b + jj] = x[r];
  }
  for (int idx = tid; idx < 6 * 256; idx += NTH) {   // the blocks above the diagonal are zero
    const int t = idx >> 8, e = idx & 255;
    const int I = t < 3 ? 0 : (t < 5 ? 1 : 2);
    const int J = t < 3 ? t + 1 : (t < 5 ? t - 1 : 3);
    sA[(16 * I + (e >> 4)) * LS + 16 * J + (e & 15)] = 0.f;
  }
  __syncthreads();
  if (wave < 3) {
    const int J = wave;
    f32x4 col[4];
#pragma unroll
    for (int m = 0; m < 3; ++m)
      if (m == J)
#pragma unroll
        for (int e = 0; e < 4; ++e) col[m][e] = sA[(16 * J + 4 * quad + e) * LS + 16 * J + r16];
#pragma unroll
    for (int I = 1; I < 4; ++I) {
      if (I <= J) continue;
      f32x4 x = zero4();
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        if (m < J || m >= I) continue;
        const f32x4 lrow = *reinterpret_cast<const f32x4*>(&sL[(16 * I + r16) * LS + 16 * m + 4 * quad]);
#pragma unroll
        for (int p = 0; p < 4; ++p) x = mfma4(lrow[p], col[m][p], x);
      }
      const f32x4 arow = *reinterpret_cast<const f32x4*>(&sA[(16 * I + r16) * LS + 16 * I + 4 * quad]);
      f32x4 y = zero4();
#pragma unroll
      for (int p = 0; p < 4; ++p) y = mfma4(arow[p], x[p], y);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        col[I][e] = -y[e];
        sA[(16 * I + 4 * quad + e) * LS + 16 * J + r16] = -y[e];
      }
    }
  }
  {  // beta v into sX (q is no longer needed): every load issued first
    constexpr int NV = BT * VD / 4 / NTH;
    f32x4 xv[NV];
#pragma unroll
    for (int s2 = 0; s2 < NV; ++s2) {
      const int i4 = tid + NTH * s2, r = 4 * i4 / VD, c = 4 * i4 % VD;
      xv[s2] = r < P.C ? ld4(v + ((P.tok0 + r) * a.Hv + h) * VD + c) : zero4();
    }
#pragma unroll
    for (int s2 = 0; s2 < NV; ++s2) {
      const int i4 = tid + NTH * s2, r = 4 * i4 / VD, c = 4 * i4 % VD;
      *reinterpret_cast<f32x4*>(&sX[r * LX + c]) = sB[r] * xv[s2];
    }
  }
  __syncthreads();
#pragma unroll
  for (int s2 = 0; s2 < BT * BT / 4 / NTH; ++s2) {
    const int i = 4 * (tid + NTH * s2), r = i / BT, c = i % BT;
    *reinterpret_cast<f32x4*>(rec + R.A + i) = *reinterpret_cast<const f32x4*>(&sA[r * LS + c]);
  }
  {  // u = A (beta v)
    using TV = STiles<BT, VD>;
    const TV tv(tid);
    f32x4 acc[TV::TPW];
#pragma unroll
    for (int t = 0; t < TV::TPW; ++t) acc[t] = zero4();
    for (int kk = 0; kk < BT; kk += 16) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(&sA[(16 * tv.rb + tv.r16) * LS + kk + 4 * tv.q]);
#pragma unroll
      for (int t = 0; t < TV::TPW; ++t)
#pragma unroll
        for (int p = 0; p < 4; ++p)
          acc[t] = mfma4(av[p], sX[(kk + 4 * tv.q + p) * LX + 16 * (tv.cb0 + t) + tv.r16], acc[t]);
    }
#pragma unroll
    for (int t = 0; t < TV::TPW; ++t)   // (u keeps four rows of a column together)
      *reinterpret_cast<u32x2*>(h16(rec + R.u) + sq_index(16 * tv.rb + 4 * tv.q, 16 * (tv.cb0 + t) + tv.r16, VD)) = pack4_f16(acc[t]);
  }
  __syncthreads();
#pragma unroll 4
  for (int i = tid; i < BT * KD; i += NTH) {
    const int r = i / KD, c = i % KD;
    sX[r * LX + c] = sB[r] * sK[r * LX + c] * ex2(sG[r * LX + c]);
  }
  __syncthreads();
  {  // w = A (beta k 2^G)
    using TK = STiles<BT, KD>;
    const TK tk(tid);
    f32x4 acc[TK::TPW];
#pragma unroll
    for (int t = 0; t < TK::TPW; ++t) acc[t] = zero4();
    for (int kk = 0; kk < BT; kk += 16) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(&sA[(16 * tk.rb + tk.r16) * LS + kk + 4 * tk.q]);
#pragma unroll
      for (int t = 0; t < TK::TPW; ++t)
#pragma unroll
        for (int p = 0; p < 4; ++p)
          acc[t] = mfma4(av[p], sX[(kk + 4 * tk.q + p) * LX + 16 * (tk.cb0 + t) + tk.r16], acc[t]);
    }
#pragma unroll
    for (int t = 0; t < TK::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        h16(rec + R.w)[(16 * tk.rb + 4 * tk.q + e) * KD + 16 * (tk.cb0 + t) + tk.r16] = (_Float16)acc[t][e];
  }
}

// --------------------------------------------------------- chunk backward
// fp32 matrix-core products (v_mfma_f32_16x16x4_f32, exact fp32 products)
// for 64-row outputs.  A 64 x N output is cut into 16 x 16 tiles; wave w owns
// tiles w + 8 t (t < TPW), all in tile column w % (N / 16), at tile rows
// (w + 8 t) / (N / 16).  In a tile, lane l holds rows 4 (l / 16) + e (e =
// 0..3) of column l % 16.  Pass p of a 16-wide reduction step gives lane l the
// reduction index 4 (l / 16) + p, so each operand is read as four
// consecutive reduction values per lane.
template <int N, int NW = NTH / 64>
struct Own {
  static constexpr int NT = N / 16, TPW = 4 * NT / NW;
  static_assert(TPW >= 1 && NW % NT == 0, "whole tiles per wave, one column block per wave");
  int w, r16, q;
  __device__ explicit Own(int tid) : w(tid >> 6), r16(tid & 15), q((tid >> 4) & 3) {}
  __device__ int ti(int t) const { return (w + NW * t) / NT; }
  __device__ int col() const { return 16 * (w % NT) + r16; }
  __device__ int row(int t, int e) const { return 16 * ti(t) + 4 * q + e; }
};
static_assert(Own<64>::TPW == 1 && Own<128>::TPW == 2, "sixteen waves cover a 64-row output");


// acc += A (64 x kr) * B (kr x N) with both operands read element by element
// (from LDS) through accessors.
template <int N, int NW, typename FA, typename FB>
__device__ __forceinline__ void mf_lds(f32x4 (&acc)[(Own<N, NW>::TPW)], int kr, int tid, FA A, FB B) {
  const Own<N, NW> o(tid);
  for (int kk = 0; kk < kr; kk += 16) {
    float b[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) b[p] = B(kk + 4 * o.q + p, o.col());
#pragma unroll
    for (int t = 0; t < Own<N>::TPW; ++t)
#pragma unroll
      for (int p = 0; p < 4; ++p) acc[t] = mfma4(A(16 * o.ti(t) + o.r16, kk + 4 * o.q + p), b[p], acc[t]);
  }
}
template <int T>
__device__ __forceinline__ void zero(f32x4 (&x)[T]) {
#pragma unroll
  for (int t = 0; t < T; ++t) x[t] = zero4();
}
// Sum over the 16 lanes of a DPP row (lanes sharing l / 16).
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

template <int KD, int VD, typename IT>
__global__ __launch_bounds__(NTH) void bwd_chunk_kernel(BwdArgs a) {
  static_assert(KD == 128 || KD == 64, "K");
  constexpr int MX = KD > VD ? KD : VD;
  constexpr int LX = MX + 4;        // row stride of the 64-row matrices (16-byte aligned rows)
  constexpr int LS = BT + 4;        // row stride of the 64 x 64 matrices
  __shared__ __attribute__((aligned(16))) float sB1[BT * LX];
  __shared__ __attribute__((aligned(16))) float sB2[BT * LX];
  __shared__ __attribute__((aligned(16))) float sB3[BT * LX];
  // the three 64 x 64 matrices; before them the same space holds kg and Aqk
  __shared__ __attribute__((aligned(16))) float sSm[3 * BT * LS];
  __shared__ float sBeta[BT], sRk[BT], sGC[KD], sDD[KD];
  float* sS1 = sSm;
  float* sS2 = sSm + BT * LS;
  float* sS3 = sSm + 2 * BT * LS;
  float* sKG = sSm;                 // [64][LX] kg = k 2^(G_C - G) (until dv_new)
  float* sAq = sSm + BT * LX;       // [64][LS] Aqk (until dv_new)
  static_assert(BT * LX + BT * LS <= 3 * BT * LS, "kg and Aqk fit the small matrices' space");
  using OK = Own<KD>;
  using OV = Own<VD>;
  using OS = Own<BT>;
  static_assert((OK::NT + OV::NT) * BT <= BT * LS && (NTH / 64 / OK::NT) * KD <= BT * LS,
                "reduction buffers fit the small matrices");
  constexpr BwdRec R = bwd_rec(KD, VD);
  int gc, h;
  chunk_head_of_block(blockIdx.x, gridDim.x, a.nchunks, a.Hv, a.Hk, gc, h);
  const ChunkPos P = chunk_pos(a.seq, gc, h, a.nchunks);
  const int tid = threadIdx.x;
  const OK ok(tid);
  const OV ov(tid);
  const OS os(tid);
  const float* rec = a.rec + P.slot * (int64_t)(R.bytes / 4);
  const _Float16* hc = a.h_store + P.slot * (int64_t)(KD * VD);
  const _Float16* dh = a.dh_store + P.slot * (int64_t)(KD * VD);
  const IT* dout = static_cast<const IT*>(a.dout);
  const IT* vin = static_cast<const IT*>(a.v);
  const float* G = rec + R.G;
  const _Float16* kgr = h16(rec + R.kg);
  const _Float16* qgr = h16(rec + R.qg);
  auto VV = [&](int i, int c) { return i < P.C ? ldf(vin + ((P.tok0 + i) * a.Hv + h) * VD + c) : 0.f; };
  // normalised k: the chunk's raw k rows through a descriptor bounded at its
  // last token (rows past it read as zero), times each row's factor
  const rsrc_t rk_in = make_rsrc(static_cast<const IT*>(a.k) + (P.tok0 * a.Hk + h / (a.Hv / a.Hk)) * KD,
                                 (uint32_t)(P.C * a.Hk * KD * (int)sizeof(IT)));
  auto KN = [&](int i, int c) { return ldb<IT>(rk_in, (uint32_t)((i * a.Hk * KD + c) * (int)sizeof(IT))) * sRk[i]; };
  if (tid < BT) {
    sBeta[tid] = rec[R.beta + tid];
    sRk[tid] = rec[R.rk + tid];
  }
  if (tid < KD) sGC[tid] = G[(P.C - 1) * KD + tid];
  __syncthreads();
  // staged once: do (fp32) into B3, kg and Aqk into the small matrices' space
  float* sDo = sB3;
  float* sBX = sB3;   // b k 2^G once do is no longer needed
  {  // every load issued before any use
    constexpr int ND = BT * VD / 4 / NTH, NK = BT * KD / 4 / NTH, NQ = BT * BT / 4 / NTH;
    f32x4 xd[ND], xk[NK], xq[NQ];
#pragma unroll
    for (int s2 = 0; s2 < ND; ++s2) {
      const int i4 = tid + NTH * s2, r = 4 * i4 / VD, cc = 4 * i4 % VD;
      xd[s2] = r < P.C ? ld4(dout + ((P.tok0 + r) * a.Hv + h) * VD + cc) : zero4();
    }
#pragma unroll
    for (int s2 = 0; s2 < NK; ++s2) {
      const int i4 = tid + NTH * s2;
      xk[s2] = ld4h(kgr + 4 * i4);
    }
#pragma unroll
    for (int s2 = 0; s2 < NQ; ++s2) xq[s2] = *reinterpret_cast<const f32x4*>(rec + R.aqk + 4 * (tid + NTH * s2));
#pragma unroll
    for (int s2 = 0; s2 < ND; ++s2) {
      const int i4 = tid + NTH * s2, r = 4 * i4 / VD, cc = 4 * i4 % VD;
      *reinterpret_cast<f32x4*>(&sDo[r * LX + cc]) = xd[s2];
    }
#pragma unroll
    for (int s2 = 0; s2 < NK; ++s2) {
      const int i4 = tid + NTH * s2, r = 4 * i4 / KD, cc = 4 * i4 % KD;
      *reinterpret_cast<f32x4*>(&sKG[r * LX + cc]) = xk[s2];
    }
#pragma unroll
    for (int s2 = 0; s2 < NQ; ++s2) {
      const int i4 = tid + NTH * s2, r = 4 * i4 / BT, cc = 4 * i4 % BT;
      *reinterpret_cast<f32x4*>(&sAq[r * LS + cc]) = xq[s2];
    }
  }

  // gradients of q, k and G in the 64 x K ownership; partial sums of dbeta
  // (64 x K and 64 x V ownership) and of dG_C (this lane's column)
  f32x4 dq[OK::TPW], dk[OK::TPW], dG[OK::TPW], dbK[OK::TPW], dbV[OV::TPW];
  zero(dq);
  zero(dk);
  zero(dG);
  zero(dbK);
  zero(dbV);
  float dGCp = 0.f;

  const int vc = ov.col();   // this lane's column in the 64 x V products
  __syncthreads();   // do, kg and Aqk staged
  {  // v_new = u - w h  -> B1 and dv_new = kg dh' + Aqk^T do  -> B2: one pass over K for
     // both K-reductions (w rows from global memory, kg rows from LDS, h and dh' columns
     // from global memory), then the Aqk^T do part
    f32x4 an[OV::TPW], ad[OV::TPW];
    zero(an);
    zero(ad);
    // the K reductions as bf16 hi/lo products (three passes each): lane group q
    // takes rows 32 kb + 8 q .. +7 of h and dh' (two 16-byte loads in their
    // four-row layout) and the same channels of the w and kg rows
    const _Float16* wr = h16(rec + R.w) + ov.r16 * KD + 8 * ov.q;
#pragma unroll
    for (int kb = 0; kb < KD / 32; ++kb) {
      const int k0 = 32 * kb + 8 * ov.q;
      float x[8];
      *reinterpret_cast<f32x4*>(x) = ld4h(hc + sq_index(k0, vc, VD));
      *reinterpret_cast<f32x4*>(x + 4) = ld4h(hc + sq_index(k0 + 4, vc, VD));
      const Frag bh = split8(x);
      *reinterpret_cast<f32x4*>(x) = ld4h(dh + sq_index(k0, vc, VD));
      *reinterpret_cast<f32x4*>(x + 4) = ld4h(dh + sq_index(k0 + 4, vc, VD));
      const Frag bd = split8(x);
#pragma unroll
      for (int t = 0; t < OV::TPW; ++t) {
        ld8h(wr + 16 * ov.ti(t) * KD + 32 * kb, x);
        an[t] = mma3(split8(x), bh, an[t]);
        ld8(&sKG[(16 * ov.ti(t) + ov.r16) * LX + k0], x);
        ad[t] = mma3(split8(x), bd, ad[t]);
      }
    }
#pragma unroll 2
    for (int r0 = 0; r0 < BT; r0 += 16) {
      float b[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) b[p] = sDo[(r0 + 4 * ov.q + p) * LX + vc];
#pragma unroll
      for (int t = 0; t < OV::TPW; ++t)
#pragma unroll
        for (int p = 0; p < 4; ++p)
          ad[t] = mfma4(sAq[(r0 + 4 * ov.q + p) * LS + 16 * ov.ti(t) + ov.r16], b[p], ad[t]);
    }
#pragma unroll
    for (int t = 0; t < OV::TPW; ++t) {
      const f32x4 u4 = ld4h(h16(rec + R.u) + sq_index(16 * ov.ti(t) + 4 * ov.q, vc, VD));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = ov.row(t, e);
        sB1[i * LX + vc] = u4[e] - an[t][e];
        sB2[i * LX + vc] = ad[t][e];
      }
    }
  }
  __syncthreads();   // (kg and Aqk give their space to the small matrices)
  {  // dAqk = tril(do v_new^T)  -> S1
    f32x4 acc[OS::TPW];
    zero(acc);
    const int j = os.col();
#pragma unroll 2
    for (int c0 = 0; c0 < VD; c0 += 16) {
      const f32x4 b = *reinterpret_cast<const f32x4*>(&sB1[j * LX + c0 + 4 * os.q]);
#pragma unroll
      for (int t = 0; t < OS::TPW; ++t) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(&sDo[(16 * os.ti(t) + os.r16) * LX + c0 + 4 * os.q]);
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[t] = mfma4(av[p], b[p], acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < OS::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = os.row(t, e);
        sS1[i * LS + j] = i >= j ? acc[t][e] : 0.f;
      }
  }
  const int kc = ok.col();   // this lane's channel in the 64 x K products
  {  // dkg = v_new dh'^T (k, G, G_C), dqg = do h^T (q, G) and dw = -dv_new h^T (-> B1) in
     // one pass over the V columns: h and dh' rows of this lane's channel straight from
     // global memory; dD = rowsum(h . dh') on the way
    f32x4 ak[OK::TPW], aq[OK::TPW], aw[OK::TPW];
    zero(ak);
    zero(aq);
    zero(aw);
    // bf16 hi/lo products over the V columns: lane group q takes columns
    // 32 kb + 8 q .. +7.  h and dh' come in their four-row layout, one 16-byte
    // load per column for the four channels of the lane's quad, and a 4 x 4
    // transpose across the quad leaves each lane its own channel's columns.
    const int qb = ok.r16 & 3;   // this lane's place in its quad (= kc & 3)
    const _Float16* hq = hc + sq_index(kc & ~3, 8 * ok.q + qb, VD);
    const _Float16* dhq = dh + sq_index(kc & ~3, 8 * ok.q + qb, VD);
    float dd = 0.f;   // this lane's quarter of the columns
#pragma unroll
    for (int kb = 0; kb < VD / 32; ++kb) {
      f32x4 h0 = ld4h(hq + 4 * (32 * kb)), h1 = ld4h(hq + 4 * (32 * kb + 4));
      f32x4 d0 = ld4h(dhq + 4 * (32 * kb)), d1 = ld4h(dhq + 4 * (32 * kb + 4));
      quad_transpose(h0, qb);
      quad_transpose(h1, qb);
      quad_transpose(d0, qb);
      quad_transpose(d1, qb);
      float xh[8], xd[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xh[j] = h0[j];
        xh[4 + j] = h1[j];
        xd[j] = d0[j];
        xd[4 + j] = d1[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) dd += xh[j] * xd[j];
      const Frag bh = split8(xh), bd = split8(xd);
#pragma unroll
      for (int t = 0; t < OK::TPW; ++t) {
        const int ro = (16 * ok.ti(t) + ok.r16) * LX + 32 * kb + 8 * ok.q;
        float x[8];
        ld8(&sB1[ro], x);
        ak[t] = mma3(split8(x), bd, ak[t]);
        ld8(&sDo[ro], x);
        aq[t] = mma3(split8(x), bh, aq[t]);
        ld8(&sB2[ro], x);
        aw[t] = mma3(split8(x), bh, aw[t]);
      }
    }
    dd += __shfl_xor(dd, 16);
    dd += __shfl_xor(dd, 32);
    if (ok.q == 0 && ok.ti(0) == 0) sDD[kc] = dd;
#pragma unroll
    for (int t = 0; t < OK::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = ok.row(t, e);
        const float gi = G[i * KD + kc];
        const float ex = ex2(sGC[kc] - gi);
        const float kgv = (float)kgr[i * KD + kc];   // k^ 2^(G_C - G)
        const float eq = a.scale * ex2(gi);
        dk[t][e] += ex * ak[t][e];
        dG[t][e] += (float)qgr[i * KD + kc] * aq[t][e] - kgv * ak[t][e];
        dGCp += kgv * ak[t][e];
        dq[t][e] += eq * aq[t][e];
      }
    // the sums formed here, not where they are next used: deferred, they would
    // keep this pass's loaded G, kg and qg values alive (and spilled) until the end
#pragma unroll
    for (int t = 0; t < OK::TPW; ++t) asm volatile("" : "+v"(dq[t]), "+v"(dk[t]), "+v"(dG[t]));
    asm volatile("" : "+v"(dGCp));
    __syncthreads();   // every wave is done with v_new (B1) before dw replaces it
#pragma unroll
    for (int t = 0; t < OK::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) sB1[ok.row(t, e) * LX + kc] = -aw[t][e];
  }
#pragma unroll 8
  for (int i = tid; i < BT * BT; i += NTH) sS2[(i / BT) * LS + i % BT] = rec[R.A + i];
  __syncthreads();
  {  // d(b k e^G) = A^T dw: k, b, G
    f32x4 acc[OK::TPW];
    zero(acc);
    mf_lds<KD, NTH / 64>(acc, BT, tid, [&](int j, int i) { return sS2[i * LS + j]; },
               [&](int i, int kk) { return sB1[i * LX + kk]; });
#pragma unroll
    for (int t = 0; t < OK::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = ok.row(t, e), kk = ok.col();
        const float ex = ex2(G[j * KD + kk]), X = KN(j, kk) * ex;
        const float dX = sBeta[j] * acc[t][e];
        dbK[t][e] += X * acc[t][e];
        dk[t][e] += ex * dX;
        dG[t][e] += X * dX;
        sBX[j * LX + kk] = sBeta[j] * X;   // b k 2^G for dA (do's space is free)
      }
#pragma unroll
    for (int t = 0; t < OK::TPW; ++t) asm volatile("" : "+v"(dbK[t]), "+v"(dk[t]), "+v"(dG[t]));   // (as above)
  }
  {  // d(b v) = A^T dv_new: dv and b
    f32x4 acc[OV::TPW];
    zero(acc);
    mf_lds<VD, NTH / 64>(acc, BT, tid, [&](int j, int i) { return sS2[i * LS + j]; },
               [&](int i, int c) { return sB2[i * LX + c]; });
    f32x4 vv[OV::TPW];   // (all loads before the stores)
#pragma unroll
    for (int t = 0; t < OV::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[t][e] = VV(ov.row(t, e), ov.col());
#pragma unroll
    for (int t = 0; t < OV::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = ov.row(t, e), c = ov.col();
        dbV[t][e] += vv[t][e] * acc[t][e];
        if (j < P.C) a.dv[((P.tok0 + j) * a.Hv + h) * VD + c] = sBeta[j] * acc[t][e];
      }
#pragma unroll
    for (int t = 0; t < OV::TPW; ++t) asm volatile("" : "+v"(dbV[t]));
  }
  __syncthreads();   // b k 2^G staged
  {  // dA = tril(dv_new (b v)^T + dw (b k e^G)^T)  -> S3 (b v straight from global memory, b k e^G from LDS)
    f32x4 acc[OS::TPW];
    zero(acc);
    const int j = os.col();
    const float bj = sBeta[j];
#pragma unroll 4
    for (int c0 = 0; c0 < VD; c0 += 16) {
      const f32x4 vv = j < P.C ? ld4(vin + ((P.tok0 + j) * a.Hv + h) * VD + c0 + 4 * os.q) : zero4();
#pragma unroll
      for (int t = 0; t < OS::TPW; ++t) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(&sB2[(16 * os.ti(t) + os.r16) * LX + c0 + 4 * os.q]);
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[t] = mfma4(av[p], bj * vv[p], acc[t]);
      }
    }
#pragma unroll 4
    for (int c0 = 0; c0 < KD; c0 += 16) {
      const f32x4 xv = *reinterpret_cast<const f32x4*>(&sBX[j * LX + c0 + 4 * os.q]);
#pragma unroll
      for (int t = 0; t < OS::TPW; ++t) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(&sB1[(16 * os.ti(t) + os.r16) * LX + c0 + 4 * os.q]);
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[t] = mfma4(av[p], xv[p], acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < OS::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = os.row(t, e);
        sS3[i * LS + j] = i >= j ? acc[t][e] : 0.f;
      }
  }
  __syncthreads();
  {  // dL = -strict_tril(A^T (dA A^T))  -> S3
    f32x4 acc[OS::TPW];
    zero(acc);
    mf_lds<BT, NTH / 64>(acc, BT, tid, [&](int i, int j) { return sS3[i * LS + j]; },
               [&](int j, int m) { return sS2[m * LS + j]; });
    __syncthreads();
#pragma unroll
    for (int t = 0; t < OS::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) sS3[os.row(t, e) * LS + os.col()] = acc[t][e];
    __syncthreads();
    zero(acc);
    mf_lds<BT, NTH / 64>(acc, BT, tid, [&](int l, int i) { return sS2[i * LS + l]; },
               [&](int i, int m) { return sS3[i * LS + m]; });
    __syncthreads();
#pragma unroll
    for (int t = 0; t < OS::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int l = os.row(t, e), m = os.col();
        sS3[l * LS + m] = l > m ? -acc[t][e] : 0.f;
      }
  }
  __syncthreads();
  {  // dL and dAqk to the workspace for the pair sums
    float* pr = a.pairs + P.slot * (int64_t)(2 * BT * BT);
#pragma unroll
    for (int s = 0; s < BT * BT / 4 / NTH; ++s) {
      const int i = 4 * (tid + NTH * s), r = i / BT, cc = i % BT;
      *reinterpret_cast<f32x4*>(pr + i) = *reinterpret_cast<const f32x4*>(&sS3[r * LS + cc]);
      *reinterpret_cast<f32x4*>(pr + BT * BT + i) = *reinterpret_cast<const f32x4*>(&sS1[r * LS + cc]);
    }
  }
  // dbeta partial sums in a fixed order (per ownership, the 16 lanes of a row
  // first), dG_C over rows (the four lane groups first)
  __syncthreads();
  float* sRedB = sS1;   // [OK::NT + OV::NT][BT]
  float* sRedK = sS2;   // [waves per column block][KD]
#pragma unroll
  for (int t = 0; t < OK::TPW; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s = sum16(dbK[t][e]);
      if (ok.r16 == 0) sRedB[(ok.w % OK::NT) * BT + ok.row(t, e)] = s;
    }
#pragma unroll
  for (int t = 0; t < OV::TPW; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s = sum16(dbV[t][e]);
      if (ov.r16 == 0) sRedB[(OK::NT + ov.w % OV::NT) * BT + ov.row(t, e)] = s;
    }
  {
    float s = dGCp;
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (ok.q == 0) sRedK[(ok.w / OK::NT) * KD + ok.col()] = s;
  }
  // dG into LDS (v_new / dw no longer needed)
#pragma unroll
  for (int t = 0; t < OK::TPW; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) sB1[ok.row(t, e) * LX + ok.col()] = dG[t][e];
  __syncthreads();
  if (tid < BT) {
    float s = 0.f;
    for (int r = 0; r < OK::NT + OV::NT; ++r) s += sRedB[r * BT + tid];
    if (tid < P.C) a.dbeta_act[(P.tok0 + tid) * a.Hv + h] = s;
  }
  if (tid < KD) {
    // dG_C (the chunk decay's gradient) joins the last row: the reverse cumsum
    // over the rows then hands it to every row
    float s = 0.f;
    for (int r = 0; r < NTH / 64 / OK::NT; ++r) s += sRedK[r * KD + tid];
    sB1[(P.C - 1) * LX + tid] += s + ex2(sGC[tid]) * sDD[tid];
  }
  __syncthreads();
  // partial gradients (the pair sums add to them): dG rows, dq, dk
#pragma unroll 4
  for (int i = tid; i < BT * KD; i += NTH) {
    const int r = i / KD, cc = i % KD;
    if (r < P.C) a.dg_nat[((P.tok0 + r) * a.Hv + h) * KD + cc] = sB1[r * LX + cc];
  }
#pragma unroll
  for (int t = 0; t < OK::TPW; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = ok.row(t, e);
      if (i >= P.C) continue;
      a.dqn[((P.tok0 + i) * a.Hv + h) * KD + ok.col()] = dq[t][e];
      a.dkn[((P.tok0 + i) * a.Hv + h) * KD + ok.col()] = dk[t][e];
    }
}

// Pair sums of the chunk backward: the gradients dL and dAqk of the decayed
// key-key and query-key products, back into k, q, beta and the gate cumsum,
// added to the partial gradients the chunk kernel left; then the reverse
// cumsum of the gate gradient over the chunk's rows.
template <int KD, int VD, typename IT>
__global__ __launch_bounds__(NTH) void bwd_pairs_kernel(BwdArgs a) {
  static_assert(KD == 128 || KD == 64, "K");
  constexpr int LX = KD + 4;        // row stride of the 64 x K matrices
  constexpr int LS = BT + 4;        // row stride of the 64 x 64 matrices
  __shared__ __attribute__((aligned(16))) float sB1[BT * LX];
  __shared__ __attribute__((aligned(16))) float sB2[BT * LX];
  __shared__ __attribute__((aligned(16))) float sB3[BT * LX];
  __shared__ __attribute__((aligned(16))) float sS1[BT * LS];
  __shared__ __attribute__((aligned(16))) float sS3[BT * LS];
  __shared__ float sBeta[BT];
  using OK = Own<KD>;
  static_assert(OK::NT * BT <= BT * LS && (NTH / KD) * KD <= BT * LS, "reduction buffers fit");
  constexpr BwdRec R = bwd_rec(KD, VD);
  int gc, h;
  chunk_head_of_block(blockIdx.x, gridDim.x, a.nchunks, a.Hv, a.Hk, gc, h);
  const ChunkPos P = chunk_pos(a.seq, gc, h, a.nchunks);
  const int tid = threadIdx.x;
  const OK ok(tid);
  const float* rec = a.rec + P.slot * (int64_t)(R.bytes / 4);
  const float* G = rec + R.G;
  // the chunk's raw q and k rows, bounded at its last token (rows past it read as zero)
  const int64_t qk0 = (P.tok0 * a.Hk + h / (a.Hv / a.Hk)) * KD;
  const uint32_t qk_bytes = (uint32_t)(P.C * a.Hk * KD * (int)sizeof(IT));
  const rsrc_t rk_in = make_rsrc(static_cast<const IT*>(a.k) + qk0, qk_bytes);
  const rsrc_t rq_in = make_rsrc(static_cast<const IT*>(a.q) + qk0, qk_bytes);
  if (tid < BT) sBeta[tid] = rec[R.beta + tid];
  {  // dL and dAqk
    const float* pr = a.pairs + P.slot * (int64_t)(2 * BT * BT);
#pragma unroll
    for (int s = 0; s < BT * BT / 4 / NTH; ++s) {
      const int i = 4 * (tid + NTH * s), r = i / BT, cc = i % BT;
      *reinterpret_cast<f32x4*>(&sS3[r * LS + cc]) = *reinterpret_cast<const f32x4*>(pr + i);
      *reinterpret_cast<f32x4*>(&sS1[r * LS + cc]) = *reinterpret_cast<const f32x4*>(pr + BT * BT + i);
    }
  }
  // stage G and the normalised k and q (raw rows times their factors) for the
  // pair sums (4-element pieces, all issued at once; rows past the sequence
  // end are zero)
  {
    constexpr int NP4 = BT * KD / 4 / NTH;
    f32x4 xg[NP4], xk[NP4], xq[NP4];
    float fk[NP4], fq[NP4];
#pragma unroll
    for (int s = 0; s < NP4; ++s) {
      const int i = 4 * (tid + NTH * s), r = i / KD, cc = i % KD;
      const uint32_t o = (uint32_t)((r * a.Hk * KD + cc) * (int)sizeof(IT));
      xg[s] = *reinterpret_cast<const f32x4*>(G + i);
      xk[s] = ldb4<IT>(rk_in, o);
      xq[s] = ldb4<IT>(rq_in, o);
      fk[s] = rec[R.rk + r];
      fq[s] = rec[R.rq + r];
    }
#pragma unroll
    for (int s = 0; s < NP4; ++s) {
      const int i = 4 * (tid + NTH * s), r = i / KD, cc = i % KD;
      *reinterpret_cast<f32x4*>(&sB1[r * LX + cc]) = xg[s];
      *reinterpret_cast<f32x4*>(&sB2[r * LX + cc]) = xk[s] * fk[s];
      *reinterpret_cast<f32x4*>(&sB3[r * LX + cc]) = xq[s] * fq[s];
    }
  }
  __syncthreads();
  f32x4 dq[OK::TPW], dk[OK::TPW], dG[OK::TPW], dbK[OK::TPW];
  zero(dq);
  zero(dk);
  zero(dG);
  zero(dbK);
  // Pair sums of dL (S3) and dAqk (S1) back into k, q, b and G in this lane's
  // channel c, on the matrix cores.  For a pair i >= j the decay factor
  // 2^(G_ic - G_jc) splits at a reference row r with j <= r <= i into
  // 2^(G_ic - G_rc) 2^(G_rc - G_jc), both <= 1 (G is non-increasing), so a
  // block of rows against another block is a plain product of prescaled
  // operands.  Off-diagonal blocks use the first row of the later block as r;
  // the diagonal blocks split further (below).
  const int c = ok.col();
  // The diagonal blocks take one reference row (i0 + 8) for every pair when
  // none of the factors it makes exceeds 2^96 in any channel of the wave's
  // tiles (a wave-uniform choice): one product per side instead of four split
  // levels.  Each choice is its own copy of the loop (separate registers).
  auto pair_tiles = [&](auto one_ref) __attribute__((always_inline)) {
    constexpr bool ONE_REF = decltype(one_ref)::value;
#pragma unroll
  for (int t = 0; t < OK::TPW; ++t) {
    const int I = ok.ti(t), i0 = 16 * I, iq = i0 + 4 * ok.q;   // rows iq .. iq + 3 of block I
    float gq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) gq[e] = sB1[(iq + e) * LX + c];
    f32x4 rL = zero4(), rA = zero4(), cL = zero4(), cA = zero4();
    // row side, earlier blocks: sum over j < i0 against reference row i0
    if (I > 0) {
      const float gr = sB1[i0 * LX + c];
      f32x4 pL = zero4(), pA = zero4();
      for (int kk = 0; kk < i0; kk += 16) {
        float b[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int j = kk + 4 * ok.q + p;
          b[p] = sB2[j * LX + c] * ex2(gr - sB1[j * LX + c]);
        }
        const f32x4 aL = *reinterpret_cast<const f32x4*>(&sS3[(i0 + ok.r16) * LS + kk + 4 * ok.q]);
        const f32x4 aA = *reinterpret_cast<const f32x4*>(&sS1[(i0 + ok.r16) * LS + kk + 4 * ok.q]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          pL = mfma4(aL[p], b[p], pL);
          pA = mfma4(aA[p], b[p], pA);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = ex2(gq[e] - gr);
        rL[e] += f * pL[e];
        rA[e] += f * pA[e];
      }
    }
    // column side, later blocks: sum over i >= i0 + 16 against reference row i0 + 16
    if (I < 3) {
      const int r = i0 + 16;
      const float gr = sB1[r * LX + c];
      f32x4 pL = zero4(), pA = zero4();
      for (int kk = r; kk < BT; kk += 16) {
        float bL[4], bA[4], aL[4], aA[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int i = kk + 4 * ok.q + p;
          const float ex = ex2(sB1[i * LX + c] - gr);
          bL[p] = sBeta[i] * sB2[i * LX + c] * ex;
          bA[p] = sB3[i * LX + c] * ex;
          aL[p] = sS3[i * LS + i0 + ok.r16];
          aA[p] = sS1[i * LS + i0 + ok.r16];
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          pL = mfma4(aL[p], bL[p], pL);
          pA = mfma4(aA[p], bA[p], pA);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = ex2(gr - gq[e]);
        cL[e] += f * pL[e];
        cA[e] += f * pA[e];
      }
    }
    // the diagonal block: binary split levels b = 3 .. 0 (blocks of 16, 8, 4
    // and 2 rows).  At level b the pairs (i, j) with i in the upper and j in
    // the lower half of one block use that upper half's first row as the
    // reference; every pair i > j of the block meets exactly one level, and
    // both factors are <= 1, whatever the decay.  Rows on the other side get
    // a zero operand before any product (their factor may overflow).
    const int xr = 4 * ok.q;   // this lane's reduction rows x = i0 + xr + p
    if constexpr (ONE_REF) {
      const float gm = sB1[(i0 + 8) * LX + c];
      f32x4 pL = zero4(), pA = zero4(), qL = zero4(), qA = zero4();
      const int y = ok.r16;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int x = xr + p, xg = i0 + x;
        const float gx = sB1[xg * LX + c], kx = sB2[xg * LX + c];
        const float bR = kx * ex2(gm - gx);         // row side: j = x
        pL = mfma4(x < y ? sS3[(i0 + y) * LS + xg] : 0.f, bR, pL);   // i = y > j = x
        pA = mfma4(x < y ? sS1[(i0 + y) * LS + xg] : 0.f, bR, pA);
        const float eu = ex2(gx - gm);              // column side: i = x > j = y
        qL = mfma4(x > y ? sS3[xg * LS + i0 + y] : 0.f, sBeta[xg] * kx * eu, qL);
        qA = mfma4(x > y ? sS1[xg * LS + i0 + y] : 0.f, sB3[xg * LX + c] * eu, qA);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float fr = ex2(gq[e] - gm), fc = ex2(gm - gq[e]);
        rL[e] += fr * pL[e];
        rA[e] += fr * pA[e];
        cL[e] += fc * qL[e];
        cA[e] += fc * qA[e];
      }
    } else {
#pragma unroll 1
      for (int lv = 3; lv >= 0; --lv) {
        const int hb = 1 << lv;
        f32x4 pL = zero4(), pA = zero4(), qL = zero4(), qA = zero4();
        float bR[4], bL[4], bA[4], aL[4], aA[4], aC[4], aD[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int x = xr + p, xg = i0 + x;
          const bool lo = !((x >> lv) & 1);                       // x in a lower half
          const float gref = sB1[(i0 + ((x >> (lv + 1)) << (lv + 1)) + hb) * LX + c];
          const float gx = sB1[xg * LX + c], kx = sB2[xg * LX + c];
          bR[p] = lo ? kx * ex2(gref - gx) : 0.f;                   // row side: j = x (lower)
          const float eu = !lo ? ex2(gx - gref) : 0.f;              // column side: i = x (upper)
          bL[p] = sBeta[xg] * kx * eu;
          bA[p] = sB3[xg * LX + c] * eu;
          // A operands, row i0 + r16 against reduction row x (same block, opposite halves)
          const int y = ok.r16;
          const bool pair_rows = (y >> (lv + 1)) == (x >> (lv + 1));
          const bool row_up = pair_rows && ((y >> lv) & 1) && lo;    // i = y upper, j = x lower
          const bool col_lo = pair_rows && !((y >> lv) & 1) && !lo;  // j = y lower, i = x upper
          aL[p] = row_up ? sS3[(i0 + y) * LS + xg] : 0.f;
          aA[p] = row_up ? sS1[(i0 + y) * LS + xg] : 0.f;
          aC[p] = col_lo ? sS3[xg * LS + i0 + y] : 0.f;
          aD[p] = col_lo ? sS1[xg * LS + i0 + y] : 0.f;
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          pL = mfma4(aL[p], bR[p], pL);
          pA = mfma4(aA[p], bR[p], pA);
          qL = mfma4(aC[p], bL[p], qL);
          qA = mfma4(aD[p], bA[p], qA);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int y = 4 * ok.q + e;   // output row iq + e
          const bool up = (y >> lv) & 1;
          const float gref = sB1[(i0 + ((y >> (lv + 1)) << (lv + 1)) + hb) * LX + c];
          const float fr = up ? ex2(gq[e] - gref) : 0.f;      // row side: i upper
          const float fc = !up ? ex2(gref - gq[e]) : 0.f;     // column side: j lower
          rL[e] += fr * pL[e];
          rA[e] += fr * pA[e];
          cL[e] += fc * qL[e];
          cA[e] += fc * qA[e];
        }
      }
    }
    // the diagonal of dAqk (factor 1): row side j = i, column side i = j
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = iq + e;
      const float d = sS1[i * LS + i];
      rA[e] += d * sB2[i * LX + c];
      cA[e] += d * sB3[i * LX + c];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = iq + e;
      const float ki = sB2[i * LX + c], qi = sB3[i * LX + c];
      const float s = cL[e] + a.scale * cA[e];
      dk[t][e] += sBeta[i] * rL[e] + s;
      dq[t][e] += a.scale * rA[e];
      dG[t][e] += sBeta[i] * ki * rL[e] + a.scale * qi * rA[e] - ki * s;
      dbK[t][e] += ki * rL[e];
    }
  }
  };
  bool one_ref = true;
#pragma unroll
  for (int t = 0; t < OK::TPW; ++t) {
    const int i0 = 16 * ok.ti(t);
    const float gm = sB1[(i0 + 8) * LX + c];
    one_ref = one_ref && fmaxf(sB1[i0 * LX + c] - gm, gm - sB1[(i0 + 15) * LX + c]) < 96.f;
  }
  if (__all(one_ref)) pair_tiles(std::true_type{});
  else pair_tiles(std::false_type{});
  __syncthreads();   // (the pair sums read sB3 and sS3, reused below)
  // dbeta: this kernel's share, added to the chunk kernel's partial sums
  float* sRedB = sS1;   // [OK::NT][BT]
#pragma unroll
  for (int t = 0; t < OK::TPW; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s = sum16(dbK[t][e]);
      if (ok.r16 == 0) sRedB[(ok.w % OK::NT) * BT + ok.row(t, e)] = s;
    }
  // dq, dk: added to the partial gradients; dG: the whole row into LDS.  All
  // partials are loaded before any store (the output buffers may alias as far
  // as the compiler knows, which would otherwise order every load after the
  // previous store)
  {
    f32x4 pq[OK::TPW], pk[OK::TPW], pg[OK::TPW];
#pragma unroll
    for (int t = 0; t < OK::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = ok.row(t, e);
        const int64_t o = ((P.tok0 + i) * a.Hv + h) * KD + c;
        const bool in = i < P.C;
        pq[t][e] = in ? a.dqn[o] : 0.f;
        pk[t][e] = in ? a.dkn[o] : 0.f;
        pg[t][e] = in ? a.dg_nat[o] : 0.f;
      }
#pragma unroll
    for (int t = 0; t < OK::TPW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = ok.row(t, e);
        if (i < P.C) {
          const int64_t o = ((P.tok0 + i) * a.Hv + h) * KD + c;
          a.dqn[o] = pq[t][e] + dq[t][e];
          a.dkn[o] = pk[t][e] + dk[t][e];
        }
        sB3[i * LX + c] = pg[t][e] + dG[t][e];
      }
  }
  __syncthreads();
  if (tid < BT && tid < P.C) {
    float s = 0.f;
    for (int r = 0; r < OK::NT; ++r) s += sRedB[r * BT + tid];
    a.dbeta_act[(P.tok0 + tid) * a.Hv + h] += s;
  }
  {  // dG -> dg: reverse cumsum over the chunk's rows (dG_C is in the last
     // row); NTH / KD threads per channel, each a segment of SR rows
    constexpr int NSG = NTH / KD, SR = BT / NSG;
    float* sSeg = sS3;   // [NSG][KD] segment totals
    const int cc = tid % KD, sg = tid / KD, r0 = sg * SR;
    float x[SR], run = 0.f;
#pragma unroll
    for (int r = SR - 1; r >= 0; --r) {
      run += r0 + r < P.C ? sB3[(r0 + r) * LX + cc] : 0.f;
      x[r] = run;
    }
    sSeg[sg * KD + cc] = run;
    __syncthreads();
    float off = 0.f;
    for (int g = sg + 1; g < NSG; ++g) off += sSeg[g * KD + cc];
#pragma unroll
    for (int r = 0; r < SR; ++r)
      if (r0 + r < P.C) a.dg_nat[((P.tok0 + r0 + r) * a.Hv + h) * KD + cc] = x[r] + off;
  }
}

// ------------------------------------------- grouped heads and L2Norm
// One wave per (token, q/k head): lanes 0..31 take q, lanes 32..63 take k,
// KD / 32 consecutive channels per lane (16- or 8-byte accesses); the sum over
// the group's value heads, then the L2Norm backward.
constexpr int QK_THREADS = 256;

template <int KD, typename IT>
__global__ __launch_bounds__(QK_THREADS) void bwd_qk_kernel(BwdArgs a, int64_t tokens) {
  constexpr int CPL = KD / 32;
  const int lane = threadIdx.x & 63, half = lane >> 5, c0 = CPL * (lane & 31);
  const int64_t item = (int64_t)blockIdx.x * (QK_THREADS / 64) + (threadIdx.x >> 6);
  if (item >= tokens * a.Hk) return;   // (whole waves: no barrier follows)
  const int64_t tok = item / a.Hk;
  const int hk = (int)(item % a.Hk), rep = a.Hv / a.Hk;
  const bool l2 = a.flags & F_L2;
  const IT* x = static_cast<const IT*>(half ? a.k : a.q) + (tok * a.Hk + hk) * KD + c0;
  const float* d = (half ? a.dkn : a.dqn) + (tok * a.Hv + (int64_t)hk * rep) * KD + c0;
  float* out = (half ? a.dk : a.dq) + (tok * a.Hk + hk) * KD + c0;
  float xs[CPL], ds[CPL];
  if constexpr (CPL == 4) {
    const f32x4 xv = ld4(x);
    f32x4 dv = ld4(d);
    for (int r = 1; r < rep; ++r) dv += ld4(d + (int64_t)r * KD);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xs[j] = xv[j];
      ds[j] = dv[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      xs[j] = ldf(x + j);
      ds[j] = d[j];
    }
    for (int r = 1; r < rep; ++r)
#pragma unroll
      for (int j = 0; j < CPL; ++j) ds[j] += d[(int64_t)r * KD + j];
  }
  float sxx = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) sxx += xs[j] * xs[j];
  for (int m = 1; m < 32; m <<= 1) sxx += __shfl_xor(sxx, m);
  const float rr = l2 ? 1.f / sqrtf(sxx + a.eps) : 1.f;
  float sxd = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) sxd += xs[j] * rr * ds[j];
  for (int m = 1; m < 32; m <<= 1) sxd += __shfl_xor(sxd, m);
  float o[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) o[j] = l2 ? rr * (ds[j] - xs[j] * rr * sxd) : ds[j];
  if constexpr (CPL == 4) *reinterpret_cast<f32x4*>(out) = f32x4{o[0], o[1], o[2], o[3]};
  else
#pragma unroll
    for (int j = 0; j < CPL; ++j) out[j] = o[j];
}

// -------------------------------------------------- gate and sigmoid
// One workgroup per (value head, block of tokens): four channels per thread
// (16-byte accesses), KD / 4 threads per token row and 128 / (KD / 4) rows in
// flight; the gate input's gradient, and this block's partial sums of dA_log
// and dt_bias (summed in block order by bwd_gate_sum_kernel).
constexpr int GATE_TOKENS = BWD_GATE_TOKENS;
constexpr int GATE_THREADS = 128;

template <int KD, typename IT>
__global__ __launch_bounds__(GATE_THREADS) void bwd_gate_kernel(BwdArgs a, int64_t tokens, float* part) {
  constexpr int LPR = KD / 4, RP = GATE_THREADS / LPR;   // threads per token row, rows in flight
  const int h = blockIdx.x % a.Hv, blk = blockIdx.x / a.Hv, tid = threadIdx.x;
  const int rg = tid / LPR, c0 = 4 * (tid % LPR);
  const IT* g = static_cast<const IT*>(a.g);
  const IT* bt = static_cast<const IT*>(a.beta);
  const bool gik = a.flags & F_GATE;
  const float lb = (a.flags & F_SAFE) ? a.lower_bound : -INFINITY;
  const float Aexp = gik ? expf(a.A_log[h]) : 0.f;
  const f32x4 bias = (gik && a.dt_bias) ? ld4(a.dt_bias + h * KD + c0) : zero4();
  f32x4 sB = zero4();
  float sA = 0.f;
  const int64_t t0 = (int64_t)blk * GATE_TOKENS, t1 = min(tokens, t0 + GATE_TOKENS);
  // batches of GB tokens per row group, every load of a batch issued before
  // its stores (the output may alias the inputs as far as the compiler knows)
  constexpr int GB = 4;
  for (int64_t tb = t0 + rg; tb < t1; tb += RP * GB) {
    f32x4 dgn[GB], x[GB];
#pragma unroll
    for (int u = 0; u < GB; ++u) {
      const int64_t t = tb + RP * u;
      const int64_t i = (t * a.Hv + h) * KD + c0;
      dgn[u] = t < t1 ? ld4(a.dg_nat + i) : zero4();
      x[u] = t < t1 ? ld4(g + i) : zero4();
    }
#pragma unroll
    for (int u = 0; u < GB; ++u) {
      const int64_t t = tb + RP * u;
      if (t >= t1) break;
      f32x4 dz;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float gact = x[u][j], d = dgn[u][j];
        if (gik) {
          // softplus(z) = max(z, 0) + ln(1 + e^-|z|) and its derivative sigmoid(z)
          // from one exponential: e = e^-|z|, sigmoid = 1 / (1 + e) for z >= 0
          // and e / (1 + e) below
          const float z = x[u][j] + bias[j];
          const float e = ex2(-LOG2E_F * fabsf(z));
          const float r = 1.f / (1.f + e);
          gact = -Aexp * (fmaxf(z, 0.f) + 0.6931471805599453f * __builtin_amdgcn_logf(1.f + e));
          d = dgn[u][j] * -Aexp * (z >= 0.f ? r : e * r);
        }
        const bool clamped = gact < lb;
        dz[j] = clamped ? 0.f : d;
        sA += clamped ? 0.f : dgn[u][j] * gact;
      }
      sB += dz;
      *reinterpret_cast<f32x4*>(a.dg + (t * a.Hv + h) * KD + c0) = dz;
    }
  }
  // beta: one token per thread
  for (int64_t t = t0 + tid; t < t1; t += GATE_THREADS) {
    const int64_t jb = t * a.Hv + h;
    float d = a.dbeta_act[jb];
    if (a.flags & F_SIGMOID) {
      const float sg = sigmoid_f(ldf(bt + jb));
      d *= sg * (1.f - sg);
    }
    a.dbeta[jb] = d;
  }
  // partial sums: [blk][Hv][KD + 1] (dt_bias per channel, then A_log), each
  // summed over the row groups / threads in a fixed order
  __shared__ __attribute__((aligned(16))) f32x4 redB[RP][LPR];
  __shared__ float redA[GATE_THREADS];
  redB[rg][tid % LPR] = sB;
  redA[tid] = sA;
  __syncthreads();
  float* pp = part + ((int64_t)blk * a.Hv + h) * (KD + 1);
  if (rg == 0) {
    f32x4 s = redB[0][tid];
    for (int r = 1; r < RP; ++r) s += redB[r][tid];
#pragma unroll
    for (int j = 0; j < 4; ++j) pp[c0 + j] = s[j];
  }
  if (tid == 0) {
    float s = 0.f;
    for (int i = 0; i < GATE_THREADS; ++i) s += redA[i];
    pp[KD] = s;
  }
}

template <int KD>
__global__ __launch_bounds__(KD) void bwd_gate_sum_kernel(BwdArgs a, int nblk, const float* part) {
  const int h = blockIdx.x, c = threadIdx.x;
  float sB = 0.f, sA = 0.f;
  for (int b = 0; b < nblk; ++b) {
    const float* pp = part + ((int64_t)b * a.Hv + h) * (KD + 1);
    sB += pp[c];
    if (c == 0) sA += pp[KD];
  }
  if (a.ddt_bias) a.ddt_bias[h * KD + c] = sB;
  if (c == 0 && a.dA_log) a.dA_log[h] = sA;
}

}  // namespace

hipError_t launch_bwd(int K, int V, int dtype, const BwdArgs& a, int stage, int64_t tokens, float* part,
                      hipStream_t s) {
  const long nb_chunk = (long)a.nchunks * a.Hv;
  const long nb_scan = (long)a.seq.N * a.Hv;
  const long nb_qk = (long)tokens * a.Hk;
  const int nblk = (int)((tokens + GATE_TOKENS - 1) / GATE_TOKENS);
  if (nb_chunk > 0x7fffffffL || nb_qk > 0x7fffffffL || (long)nblk * a.Hv > 0x7fffffffL) return hipErrorInvalidValue;
#define KDA_BWD_CASE(KK, VV, TT)                                                                        \
  if (K == KK && V == VV) {                                                                             \
    switch (stage) {                                                                                    \
      case 0: return nb_chunk ? launch(bwd_prep_kernel<KK, VV, TT>, dim3(nb_chunk), dim3(NTH), s, a) : hipSuccess; \
      case 1: return nb_scan ? launch(bwd_scan_kernel<KK, VV, TT>, dim3(nb_scan), dim3(VV * 4), s, a) : hipSuccess;  \
      case 2: return nb_chunk ? launch(bwd_chunk_kernel<KK, VV, TT>, dim3(nb_chunk), dim3(NTH), s, a) : hipSuccess; \
      case 3: return nb_qk ? launch(bwd_qk_kernel<KK, TT>, dim3((nb_qk + 3) / 4), dim3(QK_THREADS), s, a, tokens) : hipSuccess; \
      case 4: return nblk ? launch(bwd_gate_kernel<KK, TT>, dim3(nblk * a.Hv), dim3(GATE_THREADS), s, a, tokens, part) \
                          : hipSuccess;                                                                 \
      case 5: return launch(bwd_gate_sum_kernel<KK>, dim3(a.Hv), dim3(KK), s, a, nblk, (const float*)part);       \
      case 6: return nb_scan ? launch(bwd_state_kernel<KK, VV>, dim3(nb_scan), dim3(VV * 4), s, a) : hipSuccess;      \
      case 7: return nb_chunk ? launch(bwd_pairs_kernel<KK, VV, TT>, dim3(nb_chunk), dim3(NTH), s, a) : hipSuccess; \
    }                                                                                                   \
    return hipErrorInvalidValue;                                                                        \
  }
  if (dtype == 1) {
    KDA_BWD_CASE(128, 128, bf16_t)
    KDA_BWD_CASE(64, 64, bf16_t)
    KDA_BWD_CASE(128, 64, bf16_t)
    KDA_BWD_CASE(64, 128, bf16_t)
  } else {
    KDA_BWD_CASE(128, 128, float)
    KDA_BWD_CASE(64, 64, float)
    KDA_BWD_CASE(128, 64, float)
    KDA_BWD_CASE(64, 128, float)
  }
#undef KDA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
