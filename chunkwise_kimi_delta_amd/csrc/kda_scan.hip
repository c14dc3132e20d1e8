// Inter-chunk KDA state scan with the fused chunk output.  One workgroup per
// (value tile of 16 columns, or of 32 when the grid holds two rounds or more,
// value head, sequence).
//
// Follows "KDA Chunk Backward — TPU/Pallas Kernel Design", sections 1 and 1.2
// (the forward output, v_new = u - w h, the inter-chunk recurrence) and the
// state / finalize stages of "Hyper-Parallel Chunk KDA" section 5.1.  For
// each chunk in order, with h the K x 16 state tile at the chunk entry:
//   v_new = u - w h
//   o     = qg h + tril(Aqk) v_new               (forward mode only)
//   h     = Diag(gdec) h + kg^T v_new
//
// Work split.  K/32 state waves each own 32 rows of the state (fp32, in
// matrix-core accumulators for the whole sequence).  Per chunk:
//   1. each state wave forms its 32-row share of w h straight from its
//      accumulators (two stacked accumulator tiles are one reduction slice of
//      the next product; the workspace stores w, kg^T, qg and Aqk with the
//      matching index permutation) and leaves it in LDS;       -- barrier A
//   2. each state wave sums the shares of its own token tile(s), subtracts
//      from u and leaves v_new as a hi/lo fragment in LDS;     -- barrier B
//   3. every state wave updates its rows with the whole v_new, while two
//      output waves form o from the same h and v_new fragments.
// The output waves run their loads two chunks ahead and touch the workspace
// four chunks ahead, so the state waves' own loads (one chunk ahead) are
// served from L2; they store chunk c's output one step later, between the
// barriers of chunk c + 1, where they would otherwise wait.
//
// Precision.  With bf16 tokens w, qg, Aqk and kg^T are stored in fp16 (11
// bits, |kg| <= 1); h enters w h as an fp16 hi/lo pair (~22 bits), kg^T meets
// v_new as an fp16 hi/lo pair, and the output takes qg h and Aqk v_new in fp16
// (the hi parts of h and v_new).  With fp32 tokens h and v_new are bf16 hi/lo
// pairs (~16 bits) against fp32 w, qg and Aqk, and kg^T is a bf16 hi part plus
// an e4m3 lo part (scaled by 2^10) that meets v_new in e4m3 in an accumulator of
// its own (~13 bits).
//
// Summary mode scans the augmented state [S~ | M] (K x (V + K)) from [0 | I]
// with u = [u | 0] and writes S~ and M ("KDA Context Parallelism (KCP)",
// notation and algorithm steps 1-2): the M columns see zero values, so they
// accumulate the product of the per-token transitions.
//
// Segments.  A sequence of nck chunks may be cut into segments of seg_len
// chunks, one workgroup per (tile, head, sequence, segment) -- the same
// decomposition applied across CUs ("KDA Context Parallelism (KCP)",
// algorithm): the summary mode writes each segment's (M, S~) at index
// n * seg_max + s (optionally skipping last segments, whose summary nobody
// needs); the forward mode starts segment s > 0 from h_in[n * seg_max + s]
// (the prefix merge of the earlier segments' summaries) and only the last
// segment writes the sequence's final state.
#include "kda_launch.h"

#include <type_traits>

namespace kda {

namespace {

// One 8-element matrix-core operand fragment as stored in the workspace: fp32
// with fp32 tokens (split into bf16 hi/lo on use), fp16 with bf16 tokens (Op16).
template <typename ST> struct Op;
template <> struct Op<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
    a = __builtin_bit_cast(f32x4, buf_load16(r, off));
    b = __builtin_bit_cast(f32x4, buf_load16(r, off + 16));
  }
  __device__ __forceinline__ Frag split() const {
    float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return split8(x);
  }
};

// An fp16 operand fragment as stored with bf16 tokens (w, qg, Aqk).
struct Op16 {
  f16x8 v;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { v = __builtin_bit_cast(f16x8, buf_load16(r, off)); }
};
// acc += A * (B.hi + B.lo) with A stored in the workspace
__device__ __forceinline__ f32x4 mma_sb(const Op<float>& A, const Frag& B, f32x4 acc) {
  const Frag f = A.split();
  acc = mfma(f.hi, B.hi, acc);
  acc = mfma(f.lo, B.hi, acc);
  return mfma(f.hi, B.lo, acc);
}
__device__ __forceinline__ f32x4 mma_sb(const Op16& A, const Frag16& B, f32x4 acc) {
  acc = mfma(A.v, B.hi, acc);
  return mfma(A.v, B.lo, acc);
}
// Output products, A from LDS (hi [, lo]) and B stored: bf16 tokens use the
// hi part only, fp32 tokens keep ~16 bits on both sides.
__device__ __forceinline__ f32x4 mma_out(const f16x8& ahi, const f16x8&, const Op16& B, f32x4 acc) {
  return mfma(ahi, B.v, acc);
}
__device__ __forceinline__ f32x4 mma_out(const bf16x8& ahi, const bf16x8& alo, const Op<float>& B, f32x4 acc) {
  const Frag f = B.split();
  acc = mfma(ahi, f.hi, acc);
  acc = mfma(alo, f.hi, acc);
  return mfma(ahi, f.lo, acc);
}

__device__ __forceinline__ void store4(bf16_t* p, const f32x4& v) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void store4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }

// Half of a v_new fragment: one accumulator tile (4 values per lane) as bf16
// hi (x, y) and lo (z, w).
__device__ __forceinline__ u32x4 half_frag(const f32x4& v) {
  uint32_t h0, l0, h1, l1;
  split2(v[0], v[1], h0, l0);
  split2(v[2], v[3], h1, l1);
  return u32x4{h0, h1, l0, l1};
}
// The same split into fp16 hi (x, y) and lo (z, w).
__device__ __forceinline__ u32x4 half_frag16(const f32x4& v) {
  uint32_t h0, l0, h1, l1;
  split2_f16(v[0], v[1], h0, l0);
  split2_f16(v[2], v[3], h1, l1);
  return u32x4{h0, h1, l0, l1};
}
__device__ __forceinline__ Frag16 join_halves16(const u32x4& a, const u32x4& b) {
  Frag16 f;
  f.hi = __builtin_bit_cast(f16x8, u32x4{a.x, a.y, b.x, b.y});
  f.lo = __builtin_bit_cast(f16x8, u32x4{a.z, a.w, b.z, b.w});
  return f;
}
__device__ __forceinline__ Frag join_halves(const u32x4& a, const u32x4& b) {
  Frag f;
  f.hi = __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
  f.lo = __builtin_bit_cast(bf16x8, u32x4{a.z, a.w, b.z, b.w});
  return f;
}

// Lane K of each 16-lane row, broadcast to the row (DPP row_newbcast; every
// lane active).
template <int K>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + K, 0xf, 0xf, false));
}

constexpr int TOUCH_AHEAD = 4;   // chunks between an L2 touch and its chunk's loads
constexpr int SPF = 1;           // state waves: chunks between an operand load and its use
constexpr int OPF = 2;           // output waves: the same
constexpr int NOW = 2;             // output waves (forward mode)
constexpr int TPO = 4 / NOW;       // token tiles per output wave

// RF: the records hold the forward sections (qg, Aqk), i.e. the chunk-local
// kernel ran in forward mode; a summary scan inside a forward call reads them.
template <int KD, int VD, typename ST, bool SUM, int CT, bool RF>
__global__ __launch_bounds__(SUM ? KD * 2 : KD * 2 + 64 * NOW) void scan_kernel(ScanArgs a) {
  static_assert(SUM || RF, "the forward scan reads forward records");
  constexpr RecLayout L = rec_layout(KD, VD, (int)sizeof(ST), RF);
  constexpr bool F32 = sizeof(ST) == 4;
  constexpr int ES = (int)sizeof(ST);
  // w and qg fragments: fp16 with bf16 tokens, fp32 (split on use) with fp32 tokens
  using OW = typename std::conditional<F32, Op<ST>, Op16>::type;
  constexpr int NS = KD / 32;         // state waves, 32 state rows each
  constexpr int TPW = 4 / NS;         // token tiles each state wave reduces
  constexpr int BV = 16 * CT;         // state columns per workgroup
  constexpr int VA = SUM ? VD + KD : VD;
  constexpr int NTILE = VA / BV;
  static_assert(VD % BV == 0, "a workgroup's columns lie in one of S~ and M");

  __shared__ f32x4 sP[NS][4][CT][64];                       // per-wave shares of w h
  __shared__ u32x4 sV[2][4][CT][64];                        // v_new half fragments, by chunk parity
  __shared__ uint32_t sV8[2][F32 ? 4 : 1][CT][64];          // v_new as e4m3 (fp32 tokens: the kg^T lo pass)
  // h fragments (hi) for the output: fp16 with bf16 tokens, bf16 with fp32 tokens
  using HT = typename std::conditional<F32, bf16x8, f16x8>::type;
  __shared__ HT sHh[SUM ? 1 : 2][NS][CT][64];
  __shared__ bf16x8 sHl[(F32 && !SUM) ? 2 : 1][NS][CT][64]; // h fragments (lo), fp32 tokens

  // ---- block -> (tile, head, sequence); tiles of one (head, sequence) share an XCD
  int lid = blockIdx.x;
  const int NB = gridDim.x;
  if ((NB & 7) == 0) lid = (lid & 7) * (NB >> 3) + (lid >> 3);
  const int tv = lid % NTILE;
  const int h = (lid / NTILE) % a.Hv;
  const int ns = lid / (NTILE * a.Hv);                  // (sequence, segment)
  const int n = ns / a.seg_max, seg = ns % a.seg_max;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, quad = lane >> 4;

  int64_t tok0s;
  int len;
  seq_range(a.seq, n, tok0s, len);
  // this segment's chunks [c_lo, c_hi) of the sequence; segment 0 always runs
  // (an empty sequence still passes its initial state through)
  const int nck_seq = (len + BT - 1) / BT;
  const int c_lo = (int)min((int64_t)seg * a.seg_len, (int64_t)nck_seq);
  const int c_hi = (int)min((int64_t)c_lo + a.seg_len, (int64_t)nck_seq);
  const bool last_seg = c_hi == nck_seq;
  if (seg > 0 && c_lo >= nck_seq) return;               // past the sequence: no work
  if (SUM && a.skip_last && last_seg) return;           // summary not needed
  tok0s += (int64_t)c_lo * BT;
  len = min(len - c_lo * BT, (c_hi - c_lo) * BT);
  const int nck = c_hi - c_lo;
  const int64_t sidx = (int64_t)n * a.seg_max + seg;    // summary output / h_in index
  const int cb = chunk_base(a.seq, n) + c_lo;
  const bool mtile = SUM && tv * BV >= VD;              // columns of M
  const int v0 = mtile ? tv * BV - VD : tv * BV;        // first column inside S~ or M
  const unsigned char* recs = a.ws + ((size_t)h * a.nchunks + cb) * L.bytes;

  if (wave < NS) {
    // =========================== state waves ===========================
    const int s = wave;
    const int row0 = 32 * s;
    constexpr int UB = ut_bytes(ES);                      // bytes per element of u
    // u as stored (four fp16 or fp32 values), converted where it is used
    using URaw = typename std::conditional<UB == 2, u32x2, u32x4>::type;
    // kg^T: fp16 with bf16 tokens; bf16 hi + e4m3 lo with fp32 tokens
    using KG = typename std::conditional<F32, bf16x8, f16x8>::type;
    struct Ops {
      OW w[4];                        // w rows 16*tt + r16, channels row0 + (slots of lane / 16)
      URaw u[TPW][CT];                // u rows 16*(TPW*s + j) + 4*quad .. +3, column v0 + 16*ct + r16
      KG kh[2][2];                    // kg^T rows row0 + 16*kt + r16, tokens 32*ks + (slots)
      uint64_t kl[2][2];              // fp32 tokens: the lo part (e4m3, scaled by 2^10)
      float gd;                       // gdec row row0 + 16*((r16 >> 2) & 1) + 4*quad + (r16 & 3)
    };
    // fragment (tt, K-block s) of w; fragments (2s + kt, ks) of kg^T; u tiles
    // (TPW*s + j, v0/16 + ct).  M columns (summary mode) see u = 0: their
    // offset lies past the record, where the buffer load returns zeros.
    constexpr uint32_t FW = 512 * ES;                     // bytes per operand fragment
    const uint32_t o_w = L.w + (uint32_t)(s * 512 + lane * 8) * ES;
    const uint32_t o_u = mtile ? (uint32_t)L.bytes
                               : L.ut + (uint32_t)((TPW * s * (VD / 16) + v0 / 16) * 256 + lane * 4) * UB;
    const uint32_t o_kg = (uint32_t)(2 * s * 2 * 512 + lane * 8) * 2;
    const uint32_t o_kl = (uint32_t)(2 * s * 1024 + lane * 16);     // e4m3: both token blocks per lane
    // (one gdec row per lane: lanes 0..7 of each 16-lane row hold the eight
    // rows that row's accumulator tiles need, handed out by DPP broadcasts)
    const uint32_t o_gd = L.gd + (uint32_t)(row0 + 16 * ((r16 >> 2) & 1) + 4 * quad + (r16 & 3)) * 4;
    // operands of the first half of a step (w h and v_new) ...
    auto load_a = [&](Ops& f, int c) __attribute__((always_inline)) {
      const rsrc_t r = make_rsrc(recs + (size_t)c * L.bytes, (uint32_t)L.bytes);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) f.w[tt].load(r, o_w + FW * NS * tt);
#pragma unroll
      for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const uint32_t o = o_u + (mtile ? 0 : 256 * UB * ((VD / 16) * j + ct));
          if constexpr (UB == 2) f.u[j][ct] = buf_load8(r, o);
          else f.u[j][ct] = buf_load16(r, o);
        }
    };
    // ... and of the state update
    auto load_b = [&](Ops& f, int c) __attribute__((always_inline)) {
      const rsrc_t r = make_rsrc(recs + (size_t)c * L.bytes, (uint32_t)L.bytes);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          f.kh[kt][ks] = __builtin_bit_cast(KG, buf_load16(r, L.kgh + o_kg + 1024 * (2 * kt + ks)));
        if constexpr (F32) {
          const u32x4 l = buf_load16(r, L.kgl + o_kl + 1024 * kt);
          f.kl[kt][0] = (uint64_t)l.y << 32 | l.x;
          f.kl[kt][1] = (uint64_t)l.w << 32 | l.z;
        }
      }
      f.gd = __uint_as_float(buf_load4(r, o_gd));
    };
    auto load = [&](Ops& f, int c) __attribute__((always_inline)) {
      load_a(f, c);
      load_b(f, c);
    };

    // state rows row0 + 16*kt + 4*quad + e, column v0 + 16*ct + r16
    f32x4 hs[2][CT];
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
      // a later segment starts from the prefix merge of the earlier ones
      if (seg > 0) h0p = a.h_in + (sidx * a.Hv + h) * (int64_t)(KD * VD);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = row0 + 16 * kt + 4 * quad + e, col = v0 + 16 * ct + r16;
          float x = 0.f;
          if (mtile) x = (row == col) ? 1.f : 0.f;
          else if (h0p) x = h0p[(int64_t)row * VD + col];
          hs[kt][ct][e] = x;
        }

    auto step = [&](const Ops& cur, Ops& nxt, int c) __attribute__((always_inline)) {
      // Unconditional prefetch (the last chunk reloads itself) so that the
      // compiler's wait counters stay exact across the loop back-edge; the
      // scheduling barrier keeps the loads at the top of the step.
      load(nxt, min(c + SPF, nck - 1));
      __builtin_amdgcn_sched_barrier(0);
      // ---- 1. this wave's share of w h
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        using HF = typename std::conditional<F32, Frag, Frag16>::type;
        HF hb;
        if constexpr (F32) hb = split_pair(hs[0][ct], hs[1][ct]);
        else hb = split_pair16(hs[0][ct], hs[1][ct]);
        if constexpr (!SUM) {
          sHh[c & 1][s][ct][lane] = hb.hi;
          if constexpr (F32) sHl[c & 1][s][ct][lane] = hb.lo;
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) sP[s][tt][ct][lane] = mma_sb(cur.w[tt], hb, zero4());
      }
      __syncthreads();                                           // A
      // ---- 2. v_new of this wave's token tiles (shares summed in wave order)
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int tt = TPW * s + j;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          f32x4 sum = sP[0][tt][ct][lane];
#pragma unroll
          for (int w2 = 1; w2 < NS; ++w2) {
            const f32x4 x = sP[w2][tt][ct][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[e] += x[e];
          }
          f32x4 v, uv;
          if constexpr (UB == 2) uv = unpack4_f16(cur.u[j][ct]);
          else uv = __builtin_bit_cast(f32x4, cur.u[j][ct]);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = uv[e] - sum[e];
          if constexpr (F32) {
            sV[c & 1][tt][ct][lane] = half_frag(v);
            sV8[c & 1][tt][ct][lane] = pack4_fp8(v);
          } else {
            sV[c & 1][tt][ct][lane] = half_frag16(v);
          }
        }
      }
      __syncthreads();                                           // B
      // ---- 3. h = Diag(gdec) h + kg^T v_new
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        using VF = typename std::conditional<F32, Frag, Frag16>::type;
        VF vb[2];
        uint64_t v8[2] = {0, 0};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if constexpr (F32) {
            vb[ks] = join_halves(sV[c & 1][2 * ks][ct][lane], sV[c & 1][2 * ks + 1][ct][lane]);
            v8[ks] = (uint64_t)sV8[c & 1][2 * ks][ct][lane] | ((uint64_t)sV8[c & 1][2 * ks + 1][ct][lane] << 32);
          } else {
            vb[ks] = join_halves16(sV[c & 1][2 * ks][ct][lane], sV[c & 1][2 * ks + 1][ct][lane]);
          }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          f32x4 acc = hs[kt][ct], acc8 = zero4();
          acc[0] *= kt ? row_bcast<4>(cur.gd) : row_bcast<0>(cur.gd);
          acc[1] *= kt ? row_bcast<5>(cur.gd) : row_bcast<1>(cur.gd);
          acc[2] *= kt ? row_bcast<6>(cur.gd) : row_bcast<2>(cur.gd);
          acc[3] *= kt ? row_bcast<7>(cur.gd) : row_bcast<3>(cur.gd);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            acc = mfma(cur.kh[kt][ks], vb[ks].hi, acc);
            acc = mfma(cur.kh[kt][ks], vb[ks].lo, acc);
            if constexpr (F32) acc8 = mfma_fp8(cur.kl[kt][ks], v8[ks], acc8);
          }
          if constexpr (F32) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += acc8[e] * (1.f / KGL_SCALE);
          }
          hs[kt][ct] = acc;
        }
      }
    };

    if (nck > 0) {
      // operands of chunk c live in f[c % (SPF + 1)], loaded SPF steps ahead
      Ops f[SPF + 1];
#pragma unroll
      for (int i = 0; i < SPF; ++i) load(f[i], min(i, nck - 1));
      for (int c = 0; c < nck; c += SPF + 1) {
#pragma unroll
        for (int i = 0; i <= SPF; ++i)
          if (c + i < nck) step(f[i], f[(i + SPF) % (SPF + 1)], c + i);
      }
    }

    // ---- final state
    float* dst = nullptr;
    int64_t ld = VD;
    if (SUM) {
      if (mtile) { dst = a.M + (sidx * a.Hv + h) * (int64_t)(KD * KD); ld = KD; }
      else dst = a.hT + (sidx * a.Hv + h) * (int64_t)(KD * VD);
    } else if (a.hT && last_seg) {
      if (a.state_rows > 0) {
        if (valid_row) dst = a.hT + (srow * a.Hv + h) * (int64_t)(KD * VD);
      } else {
        dst = a.hT + ((int64_t)n * a.Hv + h) * (int64_t)(KD * VD);
      }
    }
    if (dst) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = row0 + 16 * kt + 4 * quad + e;
            dst[(int64_t)row * ld + v0 + 16 * ct + r16] = hs[kt][ct][e];
          }
    }
  } else if constexpr (!SUM) {
    // =========================== output waves ==========================
    // output wave ow forms token tiles TPO*ow .. TPO*ow + TPO - 1.  Chunk c's
    // output is formed between the state waves' barriers B(c) and A(c+1).
    const int ow = wave - NS;
    const int owu = __builtin_amdgcn_readfirstlane(ow);   // uniform: the Aqk block tests are scalar branches
    auto aqk_live = [](int tt, int ks) { return 32 * ks <= 16 * tt + 15; };
    using AQ = typename std::conditional<F32, Op<ST>, Op16>::type;   // Aqk: fp16 with bf16 tokens
    struct OF {
      OW q[TPO][NS];        // qg rows 16*(TPO*ow + j) + r16, channels 32*kb + (slots of lane / 16)
      AQ aq[TPO][2];        // Aqk rows 16*(TPO*ow + j) + r16, tokens 32*ks + (slots)
    };
    // fragments (TPO*ow + j, kb) of qg and (TPO*ow + j, ks) of Aqk
    constexpr uint32_t FW = 512 * ES;
    const uint32_t o_q = L.qg + (uint32_t)(TPO * ow * NS * 512 + lane * 8) * ES;
    const uint32_t o_a = L.aqk + (uint32_t)(TPO * ow * 2 * 512 + lane * 8) * ES;
    auto load = [&](OF& f, int c) __attribute__((always_inline)) {
      const rsrc_t r = make_rsrc(recs + (size_t)c * L.bytes, (uint32_t)L.bytes);
#pragma unroll
      for (int j = 0; j < TPO; ++j) {
#pragma unroll
        for (int kb = 0; kb < NS; ++kb) f.q[j][kb].load(r, o_q + FW * (NS * j + kb));
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          // token block ks of Aqk rows 16*tt .. +15 is zero when it lies wholly
          // above the diagonal: not loaded, and its product skipped
          if (aqk_live(TPO * owu + j, ks)) f.aq[j][ks].load(r, o_a + FW * (2 * j + ks));
          else f.aq[j][ks] = AQ{};
        }
      }
    };
    // L2 warm-up: this tile touches its share of the 128-byte lines of the
    // record four chunks ahead (one line per lane; the sibling tiles of the
    // head cover the rest).  The loaded word is consumed three steps later,
    // so the touch never makes this wave wait.
    constexpr int NL = (int)(L.bytes / 128);
    const int l0 = tv * NL / NTILE, l1 = (tv + 1) * NL / NTILE;
    const int tline = l0 + ow * 64 + lane;   // NOW*64 lanes cover a tile's share
    const uint32_t toff = tline < l1 ? (uint32_t)tline * 128 : (uint32_t)L.bytes;   // past the end: no access
    auto touch = [&](int c) __attribute__((always_inline)) -> uint32_t {
      return buf_load4(make_rsrc(recs + (size_t)min(c, nck - 1) * L.bytes, (uint32_t)L.bytes), toff);
    };
    ST* op = static_cast<ST*>(a.o);
    // Chunk c's output tiles wait in registers and are stored between the
    // barriers A(c+1) and B(c+1), where this wave would otherwise sit idle for
    // the state waves' reduction: a store that waits for a slot in the memory
    // queue then delays no barrier.
    f32x4 pend[TPO][CT];
    auto flush = [&](int c) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < TPO; ++j)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int t = 16 * (TPO * ow + j) + r16;
          if (op && t < len - c * BT)
            store4(op + (tok0s + (int64_t)c * BT + t) * (int64_t)(a.Hv * VD) + (int64_t)h * VD + v0 + 16 * ct + 4 * quad,
                   pend[j][ct]);
        }
    };
    // Each step loads chunk c + 2 into `ld`, stores chunk c - 1 and forms
    // chunk c from `use`.
    uint32_t pf[TOUCH_AHEAD - 1];
    auto ostep = [&](OF& ld, const OF& use, int c) __attribute__((always_inline)) {
      load(ld, min(c + OPF, nck - 1));
      asm volatile("; prefetch sink %0" ::"v"(pf[0]));
#pragma unroll
      for (int i = 0; i + 1 < TOUCH_AHEAD - 1; ++i) pf[i] = pf[i + 1];
      pf[TOUCH_AHEAD - 2] = touch(c + TOUCH_AHEAD);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();                                           // A(c)
      if (c > 0) flush(c - 1);
      __syncthreads();                                           // B(c)
      const int b = c & 1;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        HT hh[NS], hl[NS];
#pragma unroll
        for (int kb = 0; kb < NS; ++kb) {
          hh[kb] = sHh[b][kb][ct][lane];
          if constexpr (F32) hl[kb] = sHl[b][kb][ct][lane];
          else hl[kb] = hh[kb];
        }
        using VF = typename std::conditional<F32, Frag, Frag16>::type;
        VF vf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if constexpr (F32) vf[ks] = join_halves(sV[b][2 * ks][ct][lane], sV[b][2 * ks + 1][ct][lane]);
          else vf[ks] = join_halves16(sV[b][2 * ks][ct][lane], sV[b][2 * ks + 1][ct][lane]);
        }
#pragma unroll
        for (int j = 0; j < TPO; ++j) {
          // o^T tile tt = TPO*ow + j: this lane holds token 16*tt + r16, columns
          // v0 + 16*ct + 4*quad .. +3
          f32x4 acc = zero4();
#pragma unroll
          for (int kb = 0; kb < NS; ++kb) acc = mma_out(hh[kb], hl[kb], use.q[j][kb], acc);
          // (the strictly upper 16 x 16 blocks of Aqk are stored as zeros; whole
          // zero 32-token blocks are skipped)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            if (aqk_live(TPO * owu + j, ks)) {
              if constexpr (F32) acc = mma_out(vf[ks].hi, vf[ks].lo, use.aq[j][ks], acc);
              else acc = mfma(vf[ks].hi, use.aq[j][ks].v, acc);
            }
          pend[j][ct] = acc;
        }
      }
    };
    if (nck > 0) {
      // (the first touches, like every load here, only for a sequence with chunks:
      // for an empty one the clamped chunk index would be -1)
#pragma unroll
      for (int i = 0; i < TOUCH_AHEAD - 1; ++i) pf[i] = touch(i + 1);
      // operands of chunk c live in f[c % (OPF + 1)], loaded OPF steps ahead
      OF f[OPF + 1];
#pragma unroll
      for (int i = 0; i < OPF; ++i) load(f[i], min(i, nck - 1));
      for (int c = 0; c < nck; c += OPF + 1) {
#pragma unroll
        for (int i = 0; i <= OPF; ++i)
          if (c + i < nck) ostep(f[(i + OPF) % (OPF + 1)], f[i], c + i);
      }
      flush(nck - 1);
#pragma unroll
      for (int i = 0; i < TOUCH_AHEAD - 1; ++i) asm volatile("; prefetch sink %0" ::"v"(pf[i]));
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
  return launch(chunk_offsets_kernel, dim3(1), dim3(256), s, cu, N, chunk_off);
}

hipError_t launch_scan(int K, int V, int dtype, const ScanArgs& a, hipStream_t s) {
  if (a.seq.N == 0 || a.Hv == 0) return hipSuccess;
  if (a.seg_max < 1 || a.seg_len < 1) return hipErrorInvalidValue;
  const int VA = a.summary ? V + K : V;
  // 16-column tiles; the forward scan runs one workgroup per CU at a time.
  // When its grid holds two or more rounds of those (bf16, K = V = 128),
  // 32-column tiles: a workgroup then loads each chunk's shared operands once
  // for twice the columns, and the scan is bound per CU by those loads (gqa
  // 1912 -> 1564 us, varlen 1568 -> 1220 us).  With fewer tiles, wider tiles
  // would leave CUs idle (the 32-head layer: 159 -> 261 us); the summary scan,
  // without output waves, already runs several workgroups per CU and measured
  // slower with them (2441 -> 2629 us at 512 summary tiles).
  const long nb1 = (long)(VA / 16) * a.Hv * a.seq.N * a.seg_max;
  int CTsel = 1;
  if (!a.summary && dtype == 1 && K == 128 && V == 128) {
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (nb1 >= 2L * ncu) CTsel = 2;
  }
  const long nb = nb1 / CTsel;
  if (nb > 0x7fffffffL) return hipErrorInvalidValue;
  // K/32 state waves, plus the output waves in forward mode
  dim3 grid((unsigned)nb), block(K * 2 + (a.summary ? 0 : 64 * NOW));
#define KDA_SCAN_CASE(KK, VV, TT, CC)                                                             \
  if (K == KK && V == VV && CTsel == CC) {                                                        \
    if (!a.summary) return launch(scan_kernel<KK, VV, TT, false, CC, true>, grid, block, s, a);   \
    return a.fwd_records ? launch(scan_kernel<KK, VV, TT, true, CC, true>, grid, block, s, a)     \
                         : launch(scan_kernel<KK, VV, TT, true, CC, false>, grid, block, s, a);   \
  }
  if (dtype == 1 && CTsel == 2 && K == 128 && V == 128)
    return launch(scan_kernel<128, 128, bf16_t, false, 2, true>, grid, block, s, a);
  if (dtype == 1) {
    KDA_SCAN_CASE(128, 128, bf16_t, 1)
    KDA_SCAN_CASE(64, 64, bf16_t, 1)
    KDA_SCAN_CASE(128, 64, bf16_t, 1)
    KDA_SCAN_CASE(64, 128, bf16_t, 1)
  } else {
    KDA_SCAN_CASE(128, 128, float, 1)
    KDA_SCAN_CASE(64, 64, float, 1)
    KDA_SCAN_CASE(128, 64, float, 1)
    KDA_SCAN_CASE(64, 128, float, 1)
  }
#undef KDA_SCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
