// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
//
// Matrix-core tiles use v_mfma_f32_16x16x32_bf16.  Operand and result
// fragments, for lane l of the wave:
//   A (16 x 32, rows x reduction): row  l % 16, reduction slots 8*(l/16) .. +7
//   B (32 x 16, reduction x cols): col  l % 16, reduction slots 8*(l/16) .. +7
//   C (16 x 16):                   col  l % 16, rows 4*(l/16) .. +3
// A and B always load the same reduction slots, so the order of the 32
// reduction terms inside one instruction does not affect the result.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native vector types (HIP's uint4/float4 wrapper structs defeat scalar
// replacement of register arrays, which then land in scratch or LDS).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t bf16_t;   // bf16 storage (raw bits)

constexpr int BT = 64;     // chunk length (tokens)
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 b = (__bf16)f;                     // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(bf16_t, b);
}
template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t x) { return bf2f(x); }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return f2bf(x); }

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// The same tile shape on fp16 operands (11 significant bits each).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// Block b of nb = nchunks * Hv chunk-local workgroups -> (chunk gc, value head
// h).  Without grouped heads: head-major (consecutive blocks take consecutive
// chunks of one head).  With Hv / Hk = R > 1 value heads per q/k head: the
// dispatcher deals consecutive blocks to the 8 XCDs in turn, so block b is taken
// as entry (b % 8) * nb / 8 + b / 8 of one list per XCD, and within that list
// the R value heads that read the same q/k rows at the same chunk are adjacent:
// those rows then come from HBM once into the XCD's L2 instead of once per
// value head.
__device__ __forceinline__ void chunk_head_of_block(int b, int nb, int nchunks, int Hv, int Hk, int& gc, int& h) {
  const int R = Hv / Hk;
  if (R == 1) {
    gc = b % nchunks;
    h = b / nchunks;
    return;
  }
  const int L = (nb & 7) == 0 ? (b & 7) * (nb >> 3) + (b >> 3) : b;
  const int rest = L / R;
  gc = rest / Hk;
  h = (rest % Hk) * R + L % R;
}

// Four floats -> four e4m3 bytes (round to nearest even), clamped to +-448 so
// that no value converts to NaN.
__device__ __forceinline__ uint32_t pack4_fp8(const f32x4& v) {
  f32x4 c;
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = fminf(fmaxf(v[e], -448.f), 448.f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
}
// acc += A * B on 8-bit e4m3 operands (eight per lane, same lane layout as bf16)
__device__ __forceinline__ f32x4 mfma_fp8(uint64_t a, uint64_t b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)a, (long)b, c, 0, 0, 0);
}

// fp32 -> bf16 hi/lo pairs: hi = RNE(x), lo = RNE(x - hi), so that hi + lo
// carries ~16 significant bits of x (x - hi is exact in fp32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two floats -> two bf16 (round to nearest even) in one word, a in the low
// half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const bf16x2_t h = {(__bf16)a, (__bf16)b};
  const uint32_t hb = __builtin_bit_cast(uint32_t, h);
  const bf16x2_t l = {(__bf16)(a - __uint_as_float(hb << 16)), (__bf16)(b - __uint_as_float(hb & 0xffff0000u))};
  hi = hb;
  lo = __builtin_bit_cast(uint32_t, l);
}

// Eight values -> bf16 fragment (hi) and the rounding remainder (lo).
struct Frag { bf16x8 hi, lo; };

__device__ __forceinline__ Frag split8(const float (&x)[8]) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  split2(x[0], x[1], h0, l0);
  split2(x[2], x[3], h1, l1);
  split2(x[4], x[5], h2, l2);
  split2(x[6], x[7], h3, l3);
  Frag f;
  f.hi = __builtin_bit_cast(bf16x8, u32x4{h0, h1, h2, h3});
  f.lo = __builtin_bit_cast(bf16x8, u32x4{l0, l1, l2, l3});
  return f;
}
// Two accumulator tiles (rows 4g..4g+3 and 16+4g..16+4g+3 of a 32-row block)
// as one hi/lo operand fragment.
__device__ __forceinline__ Frag split_pair(const f32x4& x, const f32x4& y) {
  const float v[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return split8(v);
}
__device__ __forceinline__ bf16x8 round8(const float (&x)[8]) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
  return r;
}

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32) as floats.
__device__ __forceinline__ void load8(const bf16_t* p, float (&x)[8]) {
  u32x4 u = *reinterpret_cast<const u32x4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
// Store 8 floats as 8 consecutive elements of type bf16 (16-byte aligned) or fp32.
__device__ __forceinline__ void store8(bf16_t* p, const float (&x)[8]) {
  u32x4 u = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
             pack_bf16x2(x[6], x[7])};
  *reinterpret_cast<u32x4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  f32x4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}
__device__ __forceinline__ bf16x8 load_bf16x8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Four floats <-> four fp16 values (round to nearest even), 8 bytes.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// fp32 -> fp16 hi/lo pairs: hi = RNE(x), lo = RNE(x - hi) (about 22 significant bits)
struct Frag16 { f16x8 hi, lo; };
__device__ __forceinline__ void split2_f16(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f16x2 h = {(_Float16)a, (_Float16)b};
  const f16x2 l = {(_Float16)(a - (float)h[0]), (_Float16)(b - (float)h[1])};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}
// Two stacked accumulator tiles as one fp16 hi/lo operand fragment.
__device__ __forceinline__ Frag16 split_pair16(const f32x4& x, const f32x4& y) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  split2_f16(x[0], x[1], h0, l0);
  split2_f16(x[2], x[3], h1, l1);
  split2_f16(y[0], y[1], h2, l2);
  split2_f16(y[2], y[3], h3, l3);
  Frag16 f;
  f.hi = __builtin_bit_cast(f16x8, u32x4{h0, h1, h2, h3});
  f.lo = __builtin_bit_cast(f16x8, u32x4{l0, l1, l2, l3});
  return f;
}
__device__ __forceinline__ f16x8 round8_f16(const float (&x)[8]) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (_Float16)x[i];
  return r;
}
__device__ __forceinline__ u32x2 pack4_f16(const f32x4& v) {
  const f16x2 a = {(_Float16)v[0], (_Float16)v[1]}, b = {(_Float16)v[2], (_Float16)v[3]};
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}
__device__ __forceinline__ f32x4 unpack4_f16(const u32x2& u) {
  // (the words are copied to scalars first: a bit cast taken straight from a
  // vector element expression has been compiled as a cast of element 0)
  const uint32_t w0 = u.x, w1 = u.y;
  const f16x2 a = __builtin_bit_cast(f16x2, w0), b = __builtin_bit_cast(f16x2, w1);
  return f32x4{(float)a[0], (float)a[1], (float)b[0], (float)b[1]};
}

// Raw buffer loads: a resource descriptor for a byte range (base in SGPRs,
// bounds checked by the hardware: reads past num_bytes return zeros) and a
// 32-bit per-lane byte offset, so that per-lane addresses are computed once.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)num_bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// acc += A * B where the operands are stored as T (bf16: exact single pass;
// fp32: split into hi/lo and accumulated in three passes, dropping lo*lo).
__device__ __forceinline__ f32x4 mma_stored(const bf16_t* a, const bf16_t* b, f32x4 acc) {
  return mfma(load_bf16x8(a), load_bf16x8(b), acc);
}
__device__ __forceinline__ f32x4 mma_stored(const float* a, const float* b, f32x4 acc) {
  float xa[8], xb[8];
  load8(a, xa);
  load8(b, xb);
  Frag fa = split8(xa), fb = split8(xb);
  acc = mfma(fa.hi, fb.hi, acc);
  acc = mfma(fa.lo, fb.hi, acc);
  acc = mfma(fa.hi, fb.lo, acc);
  return acc;
}

// Stored-operand A against a B operand kept as bf16 hi/lo pair in LDS.
__device__ __forceinline__ f32x4 mma_a_bsplit(const bf16_t* a, const bf16_t* bhi, const bf16_t* blo,
                                              f32x4 acc) {
  bf16x8 fa = load_bf16x8(a);
  acc = mfma(fa, load_bf16x8(bhi), acc);
  acc = mfma(fa, load_bf16x8(blo), acc);
  return acc;
}
__device__ __forceinline__ f32x4 mma_a_bsplit(const float* a, const bf16_t* bhi, const bf16_t* blo,
                                              f32x4 acc) {
  float xa[8];
  load8(a, xa);
  Frag fa = split8(xa);
  bf16x8 h = load_bf16x8(bhi), l = load_bf16x8(blo);
  acc = mfma(fa.hi, h, acc);
  acc = mfma(fa.hi, l, acc);
  acc = mfma(fa.lo, h, acc);
  return acc;
}
// Stored-operand A against the hi part only of a split B operand.
__device__ __forceinline__ f32x4 mma_a_bhi(const bf16_t* a, const bf16_t* bhi, f32x4 acc) {
  return mfma(load_bf16x8(a), load_bf16x8(bhi), acc);
}
__device__ __forceinline__ f32x4 mma_a_bhi(const float* a, const bf16_t* bhi, f32x4 acc) {
  float xa[8];
  load8(a, xa);
  Frag fa = split8(xa);
  bf16x8 h = load_bf16x8(bhi);
  acc = mfma(fa.hi, h, acc);
  acc = mfma(fa.lo, h, acc);
  return acc;
}

// Sequence bookkeeping shared by the kernels.  BSND: sequence n = batch n,
// tokens [n*T, n*T + T).  TND: tokens [cu[n], cu[n+1]); chunk_off[n] is the
// first global chunk of sequence n (chunk_off[N] = total chunks).
struct SeqInfo {
  int tnd;                    // 0: BSND, 1: TND
  int T;                      // BSND tokens per sequence
  int N;                      // sequences
  const int32_t* cu;          // TND device cu_seqlens [N+1]
  const int32_t* chunk_off;   // TND device chunk offsets [N+1]
};

__device__ __forceinline__ void seq_range(const SeqInfo& s, int n, int64_t& tok0, int& len) {
  if (s.tnd) {
    int a = s.cu[n], b = s.cu[n + 1];
    tok0 = a;
    len = b - a;
  } else {
    tok0 = (int64_t)n * s.T;
    len = s.T;
  }
}
__device__ __forceinline__ int chunk_base(const SeqInfo& s, int n) {
  return s.tnd ? s.chunk_off[n] : n * ((s.T + BT - 1) / BT);
}
// Sequence owning global chunk gc: the n with chunk_base(n) <= gc < chunk_base(n+1).
__device__ __forceinline__ int seq_of_chunk(const SeqInfo& s, int gc) {
  if (!s.tnd) return gc / ((s.T + BT - 1) / BT);
  int lo = 0, hi = s.N - 1;            // largest n with chunk_off[n] <= gc
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s.chunk_off[mid] <= gc) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace kda
