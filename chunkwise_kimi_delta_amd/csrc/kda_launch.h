// Internal interface between the C ABI (kda_api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_common.h"

namespace kda {

enum : uint32_t { F_GATE = 1u, F_SAFE = 2u, F_L2 = 4u, F_SIGMOID = 8u };

// Per-(value head, chunk) workspace record written by the chunk-local kernel
// and read by the state scan.  Sections are 256-byte aligned; a record is one
// contiguous span so that a whole chunk can be prefetched as a byte range.
// Matrices are stored as matrix-core fragments in lane order, so that every
// operand load of the scan is one contiguous 1 KiB (2 KiB for fp32) block; the
// fp8 kgl keeps the two token blocks of a channel tile side by side per lane
// (8 bytes each), so one 1 KiB load fetches both:
//   w   [64][K]  fp16 | fp32   operand fragments, rows = tokens, reduction = channels
//                              (fp16 with bf16 tokens)
//   kgh [K][64]  fp16 | bf16   kg^T, rows = channels, reduction = tokens: fp16 with
//                              bf16 tokens; with fp32 tokens its bf16 hi part and
//   kgl [K][64]  fp8 e4m3      the lo part, 2^10 (kg^T - hi) (one byte per element;
//                              channel tile kt, lane l, token block tb at
//                              1024 kt + 16 l + 8 tb; fp32 tokens only)
//   qg  [64][K]  fp16 | fp32   scale * q * 2^gamma, like w (forward only)
//   aqk [64][64] fp16 | fp32   tril(Aqk), rows = tokens, reduction = tokens (forward
//                              only; fp16 with bf16 tokens)
//   gd  [K]      fp32          2^gamma_C, the chunk decay (plain vector)
//   ut  [64][V]  fp16 | fp32   u as accumulator tiles (16 x 16, four values per lane):
//                              fp16 with bf16 tokens (11 significant bits, 8 bytes
//                              per lane and tile), fp32 with fp32 tokens
// The strictly upper 32 x 32 block of aqk (rows 0..31, tokens 32..63) is zero and
// neither written nor read.
// Inside an operand fragment the reduction index is permuted by sigma: within
// each aligned block of 32, index x sits in slot sig32(x), so that reduction
// slot 8*g + i (g = lane / 16, i = 0..7) holds index 4*g + i for i < 4 and
// 16 + 4*g + (i - 4) for i >= 4 -- the rows of two stacked accumulator tiles
// as one lane holds them.
struct RecLayout {
  size_t w, kgh, kgl, qg, aqk, gd, ut, bytes;
};
__host__ __device__ constexpr size_t al256(size_t x) { return (x + 255) & ~size_t(255); }
// bytes per element of u in the record, by token element size
__host__ __device__ constexpr int ut_bytes(int es) { return es == 2 ? 2 : 4; }
__host__ __device__ constexpr RecLayout rec_layout(int K, int V, int es, bool fwd) {
  RecLayout r{};
  r.w = 0;
  r.kgh = al256(r.w + (size_t)64 * K * es);
  r.kgl = al256(r.kgh + (size_t)K * 64 * 2);
  r.qg = al256(r.kgl + (es == 2 ? 0 : (size_t)K * 64));
  r.aqk = al256(r.qg + (fwd ? (size_t)64 * K * es : 0));
  r.gd = al256(r.aqk + (fwd ? (size_t)64 * 64 * es : 0));
  r.ut = al256(r.gd + (size_t)K * 4);
  r.bytes = al256(r.ut + (size_t)V * 64 * ut_bytes(es));
  return r;
}
// Scale of the fp8 kgl values (2^10): kg^T - hi is below 2^-8 |kg| <= 2^-8
// for unit-norm keys, well inside e4m3's range after scaling.
constexpr float KGL_SCALE = 1024.f;
__host__ __device__ constexpr int sig32(int x) { return 8 * ((x & 15) >> 2) + 4 * (x >> 4) + (x & 3); }
// Element offset of (row, red) in a matrix stored as 16 x 32 operand fragments
// (nrb fragments along the reduction index): 512 elements per fragment, eight
// per lane, lane = row % 16 + 16 * (slot / 8).
__host__ __device__ constexpr int frag_off(int row, int red, int nrb) {
  return (((row >> 4) * nrb + (red >> 5)) << 9) + (((row & 15) + 16 * (sig32(red & 31) >> 3)) << 3) +
         (sig32(red & 31) & 7);
}
// Element offset of (row, col) in a matrix stored as 16 x 16 accumulator tiles
// (ncb tiles along col): 256 elements per tile, lane = col % 16 + 16 * (row % 16 / 4),
// four consecutive rows per lane.
__host__ __device__ constexpr int cfrag_off(int row, int col, int ncb) {
  return (((row >> 4) * ncb + (col >> 4)) << 8) + (((col & 15) + 16 * ((row & 15) >> 2)) << 2) + (row & 3);
}

// Chunk-local ("intra") kernel: gate + cumsum, L2Norm, beta, Akk/Aqk,
// (I+L)^-1, WY factors.  One workgroup per (chunk, value head).
struct IntraArgs {
  SeqInfo seq;
  const void *q, *k, *v, *g, *beta;   // q may be null (summary)
  const float *A_log, *dt_bias;
  int Hk, Hv, nchunks;
  uint32_t flags;
  float scale, eps, lower_bound;
  unsigned char* ws;                  // records, [Hv][nchunks]
};

// Inter-chunk state scan + output.  One workgroup per (16-column value tile,
// head, sequence).
struct ScanArgs {
  SeqInfo seq;
  int Hv, nchunks, state_rows, summary;
  int fwd_records;                    // summary mode on records written in forward mode
  int seg_len, seg_max;               // chunks per segment (>= 1), segments per sequence in the grid
  int skip_last;                      // summary mode: no workgroup for a sequence's last segment
  const float* h_in;                  // forward, segment s > 0: [N*seg_max][Hv][K][V] incoming state
  const unsigned char* ws;            // records, [Hv][nchunks]
  const float* h0;                    // [N,Hv,K,V] | cache | null
  const int32_t* state_idx;           // cache mode
  float* hT;                          // final [N,Hv,K,V] | cache | null ; summary: S~
  float* M;                           // summary only: [N*seg_max,Hv,K,K] (S~ in hT alike)
  void* o;                            // [tokens,Hv,V] (null: not written)
};

// Token-by-token forward (decode).  One wave per (64-column slice, head, sequence).
struct RecurrentArgs {
  SeqInfo seq;
  const void *q, *k, *v, *g, *beta;
  const float *A_log, *dt_bias;
  int Hk, Hv, state_rows;
  uint32_t flags;
  float scale, eps, lower_bound;
  const float* h0;                    // [N,Hv,K,V] | cache | null
  const int32_t* state_idx;           // cache mode
  float* hT;                          // final [N,Hv,K,V] | cache | null (may equal h0)
  void* o;                            // [tokens,Hv,V]
};

struct MergeArgs {
  int P, Hv;
  const float *M, *S;
  float* state;
};

// Prefix merge over the segments of each sequence: h_in[n*seg_max + s + 1] =
// M[..s] h_in[..s] + S~[..s], from the sequence's initial state.
struct PrefixMergeArgs {
  SeqInfo seq;
  int Hv, seg_len, seg_max, state_rows;
  const float *M, *S;                 // [N*seg_max][Hv][K][K], [..][K][V]
  const float* h0;                    // [N,Hv,K,V] | cache | null
  const int32_t* state_idx;
  float* h_in;                        // [N*seg_max][Hv][K][V]
};

// Launch a kernel and return the status of this launch alone (hipLaunchKernel
// reports its own failure; hipGetLastError would also return an error left
// behind by the caller's earlier work).
template <typename... A>
inline hipError_t launch(void (*kern)(A...), dim3 grid, dim3 block, hipStream_t s, A... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, 0, s);
}

// dtype: 0 = fp32, 1 = bf16
hipError_t launch_chunk_offsets(const int32_t* cu, int N, int32_t* chunk_off, hipStream_t s);
hipError_t launch_intra(int K, int V, int dtype, const IntraArgs& a, hipStream_t s);
hipError_t launch_scan(int K, int V, int dtype, const ScanArgs& a, hipStream_t s);
hipError_t launch_merge(int K, int V, const MergeArgs& a, hipStream_t s, bool backward = false);
hipError_t launch_prefix_merge(int K, int V, const PrefixMergeArgs& a, hipStream_t s);
hipError_t launch_recurrent(int K, int V, int dtype, const RecurrentArgs& a, hipStream_t s);
// Device address of the fixed scratch on the stream's device (kda_noalloc.hip);
// on failure `why` names the step that failed.
hipError_t noalloc_scratch(hipStream_t stream, void** out, char* why, size_t why_len);

}  // namespace kda
