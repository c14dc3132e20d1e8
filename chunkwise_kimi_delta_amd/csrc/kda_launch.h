// Internal interface between the C ABI (kda_api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_common.h"

namespace kda {

enum : uint32_t { F_GATE = 1u, F_SAFE = 2u, F_L2 = 4u, F_SIGMOID = 8u };

// Chunk-local ("intra") kernel: gate + cumsum, L2Norm, beta, Akk/Aqk,
// (I+L)^-1, WY factors.  One workgroup per (chunk, value head).
struct IntraArgs {
  SeqInfo seq;
  const void *q, *k, *v, *g, *beta;   // q may be null (summary)
  const float *A_log, *dt_bias;
  int Hk, Hv, nchunks;
  uint32_t flags;
  float scale, eps, lower_bound;
  // outputs, head-major [Hv][nchunks][...]; element type = token dtype
  void *w, *u, *kgT, *qg, *Aqk;       // qg/Aqk unused when q is null
  float* gdec;                        // [Hv][nchunks][K]  2^(chunk log2 decay)
};

// Inter-chunk state scan + output.  One workgroup per (dv tile, head, sequence).
struct ScanArgs {
  SeqInfo seq;
  int Hv, nchunks, state_rows, summary;
  const void *w, *u, *kgT, *qg, *Aqk;
  const float* gdec;
  const float* h0;                    // [N,Hv,K,V] | cache | null
  const int32_t* state_idx;           // cache mode
  float* hT;                          // final [N,Hv,K,V] | cache | null ; summary: S~
  float* M;                           // summary only: [N,Hv,K,K]
  void* o;                            // [tokens,Hv,V]
};

struct MergeArgs {
  int P, Hv;
  const float *M, *S;
  float* state;
};

// dtype: 0 = fp32, 1 = bf16
hipError_t launch_chunk_offsets(const int32_t* cu, int N, int32_t* chunk_off, hipStream_t s);
hipError_t launch_intra(int K, int V, int dtype, const IntraArgs& a, hipStream_t s);
hipError_t launch_scan(int K, int V, int dtype, const ScanArgs& a, hipStream_t s);
hipError_t launch_merge(int K, int V, const MergeArgs& a, hipStream_t s);

}  // namespace kda
