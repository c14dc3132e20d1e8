// Backward launch interface: the per-(head, chunk) record, the arguments of
// the backward kernels (kda_bwd.hip) and their launcher.  Kept apart from the
// forward's kda_launch.h so that the forward's sources change only with the
// forward.
#pragma once
#include "kda_launch.h"

namespace kda {

// Backward record per (head, chunk), row-major, section offsets in floats:
//   fp32: G [64][K] in-chunk cumsum of the decay in log2 units (rows past the
//   end keep the last value), beta [64] (activated), rk / rq [64] the factors
//   that normalise each row of k and q (0 past the end; the normalised rows are
//   the raw rows times these, formed where they are read), A [64][64] =
//   (I + L)^-1, aqk [64][64] (scaled, zero above the diagonal);
//   fp16 (11 significant bits; magnitudes up to 65504): w [64][K], u [64][V]
//   stored [16][V][4] (four consecutive rows of a column together),
//   kg = k^ 2^(G_C - G) and qg = scale q^ 2^G [64][K] (k^, q^ the normalised
//   rows, G_C the last row of G) for the state scans and the chunk kernel.
struct BwdRec {
  size_t G, beta, rk, rq, A, aqk, w, u, kg, qg, bytes;
};
__host__ __device__ constexpr BwdRec bwd_rec(int K, int V) {
  BwdRec r{};
  r.G = 0;
  r.beta = r.G + 64 * (size_t)K;
  r.rk = r.beta + 64;
  r.rq = r.rk + 64;
  r.A = r.rq + 64;
  r.aqk = r.A + 64 * 64;
  r.w = r.aqk + 64 * 64;
  r.u = r.w + 32 * (size_t)K;           // (fp16 sections: half a float per element)
  r.kg = r.u + 32 * (size_t)V;
  r.qg = r.kg + 32 * (size_t)K;
  r.bytes = al256((r.qg + 32 * (size_t)K) * 4);
  return r;
}

struct BwdArgs {
  SeqInfo seq;
  const void *q, *k, *v, *g, *beta, *dout;   // token tensors (dtype of q)
  const float *A_log, *dt_bias, *dht;        // dht [N][Hv][K][V] or null
  int Hk, Hv, nchunks;
  uint32_t flags;
  float scale, eps, lower_bound;
  float* rec;                 // [Hv * nchunks] backward records
  const float* h0;            // [N][Hv][K][V] or null (zero)
  // fp16 [Hv * nchunks][K/4][V][4] chunk-entry states (four rows of a column together)
  const _Float16* h_store;
  _Float16* h_store_w;        // the same buffer, written by the state kernel
  _Float16* dh_store;         // fp16 [Hv * nchunks][K/4][V][4] gradients of the chunk-exit states (or null)
  float* dh0;                 // [N][Hv][K][V] or null
  float *dqn, *dkn;           // [tokens][Hv][K]: per value head, w.r.t. normalised q / k
  float *dbeta_act, *dg_nat;  // [tokens][Hv] w.r.t. activated beta, [tokens][Hv][K] w.r.t. the decay
  float *dq, *dk;             // [tokens][Hk][K]
  float *dv, *dg, *dbeta;     // [tokens][Hv][V], [tokens][Hv][K], [tokens][Hv]
  float *dA_log, *ddt_bias;   // [Hv], [Hv][K] or null
  float* pairs;               // [Hv * nchunks][2][64][64]: dL and dAqk of each chunk
};

// Backward stage: 0 prep, 6 forward state scan, 1 reverse state scan, 2
// chunk-local backward (products), 7 its pair sums, 3 grouped heads + L2Norm,
// 4 gate/sigmoid with block partial sums (into `part`), 5 the sums of those
// partials.
hipError_t launch_bwd(int K, int V, int dtype, const BwdArgs& a, int stage, int64_t tokens, float* part,
                      hipStream_t s);
constexpr int BWD_GATE_TOKENS = 512;   // tokens per gate workgroup (one partial each)

}  // namespace kda
