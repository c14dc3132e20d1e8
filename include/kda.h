/*
 * kda.h — C ABI of the MI355X (gfx950) chunkwise Kimi Delta Attention library.
 *
 * KDA is a gated delta rule with a per-channel decay.  For one sequence and one
 * value head, with state S (K x V, fp32), per token t:
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t,          alpha_t = exp(g_t)  (one per key channel)
 * The library computes it in 64-token chunks with the WY representation, as in
 * "KDA Chunk Backward — TPU/Pallas Kernel Design", sections 1 and 1.2 (forward
 * output = inter-chunk part from the chunk-entry state + lower-triangular
 * intra-chunk part; u/w WY factors; log2-space chunk-local gate cumsum;
 * inter-chunk state recurrence).
 *
 * Conventions shared by every call
 *  - Tensor pointers are DEVICE pointers unless the name ends in _host.  All
 *    tensors are dense row-major (the last axis is contiguous) and 16-byte
 *    aligned.  The caller owns all memory; the library allocates nothing and
 *    keeps no pointer, stream or tensor after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *    are asynchronous on it; nothing synchronises the host.
 *  - Fail-closed: every argument visible on the host is validated before any
 *    launch.  On error the call returns a status, launches nothing and records
 *    a message readable with kda_last_error() (thread-local).  There is no
 *    fallback path.  A failed kernel launch returns KDA_ERR_HIP.
 *  - Device-resident index values (cu_seqlens, state_indices) are not read by
 *    the host.  Kernels treat a state index that is negative or >= state_rows
 *    as invalid: that sequence starts from a zero state and its final state is
 *    not written.  Valid indices must be unique when final states are written
 *    into a cache (caller precondition; vllm-ascend KDA prefill state copy
 *    page, numeric-contract section).  Address arithmetic is 64-bit.
 *  - Token layouts ("Hyper-Parallel Chunk KDA" section 4.2):
 *        BSND: q,k [B,T,Hk,K]  v [B,T,Hv,V]  g [B,T,Hv,K]  beta [B,T,Hv]  o [B,T,Hv,V]
 *        TND : the same without B; sequences are packed and delimited by
 *              cu_seqlens [N+1] (int32, cu[0]=0, non-decreasing, cu[N]=T).
 *    Every sequence starts from its own initial state ("Hyper-Parallel Chunk
 *    KDA" section 6.5).  Value head h reads query/key head h / (Hv/Hk)
 *    (section 4.2, grouped heads).
 */
#ifndef KDA_MI355X_H
#define KDA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 2

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1,   /* a shape, pointer, flag or size is wrong */
  KDA_ERR_UNSUPPORTED = 2,        /* valid request outside the built envelope */
  KDA_ERR_WORKSPACE_TOO_SMALL = 3,
  KDA_ERR_HIP = 4                 /* a HIP launch or runtime call failed */
} kda_status_t;

typedef enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;
typedef enum kda_layout { KDA_LAYOUT_BSND = 0, KDA_LAYOUT_TND = 1 } kda_layout_t;

/* Flags ("Hyper-Parallel Chunk KDA" section 4: use_gate_in_kernel, safe_gate,
 * use_qk_l2norm_in_kernel, use_beta_sigmoid_in_kernel). */
enum {
  /* g holds the raw gate; the decay is g = -exp(A_log[h]) * softplus(g + dt_bias[h,:]).
   * Without it g holds the natural-log decay itself (g <= 0). */
  KDA_GATE_IN_KERNEL = 1u,
  /* clamp the natural-log decay below at lower_bound, per token and channel */
  KDA_SAFE_GATE = 2u,
  /* q and k are divided by sqrt(sum x^2 + eps) per token and head */
  KDA_QK_L2NORM = 4u,
  /* beta holds a logit; the write strength is sigmoid(beta) */
  KDA_BETA_SIGMOID = 8u
};

/* Number of stage events a token-level call records (see kda_chunk_fwd). */
#define KDA_STAGE_EVENTS 3

/* Problem description, passed by pointer to every token-level call. */
typedef struct kda_problem {
  int32_t layout;       /* kda_layout_t */
  int32_t dtype;        /* kda_dtype_t of q, k, v, g, beta and o */
  int32_t B, T;         /* BSND: batch and tokens per sequence.  TND: B = 1, T = packed tokens */
  int32_t Hk, Hv;       /* query/key heads and value heads; Hv % Hk == 0 */
  int32_t K, V;         /* key and value head dims; each 64 or 128 (bf16 or fp32 tokens) */
  int32_t chunk_size;   /* must be 64 */
  uint32_t flags;       /* KDA_* flags above */
  float scale;          /* output scale, usually K^-1/2 */
  float eps;            /* L2Norm epsilon (inside the square root), e.g. 1e-6 */
  float lower_bound;    /* safe-gate floor for the natural-log decay, finite and <= 0, e.g. -5 */
  int32_t num_seqs;     /* N: BSND must equal B; TND = number of packed sequences */
  const int32_t* cu_seqlens_host; /* TND: HOST copy of cu_seqlens [N+1]; NULL for BSND */
  int32_t state_rows;   /* 0: states are [N,Hv,K,V]; > 0: state cache rows, see kda_chunk_fwd */
  /* Segment-parallel state scan of kda_chunk_fwd / kda_chunk_fwd_noalloc
   * ("KDA Context Parallelism (KCP)", algorithm, applied across the GPU's
   * compute units): 0 = the library decides (it splits long sequences when too
   * few (sequence, head) scans would occupy the GPU), 1 = one sequential scan
   * per sequence, n > 1 = cut each sequence's chunks into at most n segments
   * that are summarised in parallel, merged in order and rescanned in
   * parallel.  The result is the same computation; other calls ignore it. */
  int32_t scan_segments;
} kda_problem_t;

/* Bytes of device workspace kda_chunk_fwd needs for this problem. */
kda_status_t kda_chunk_fwd_workspace_size(const kda_problem_t* p, size_t* bytes);

/*
 * Chunkwise KDA forward ("Hyper-Parallel Chunk KDA" section 4, the fused
 * interface, and section 5.1, the prepare / state / finalize stages it fuses;
 * "KDA Chunk Backward — TPU/Pallas Kernel Design" section 1.2 for the chunk
 * formulas).
 *
 *  q, k, v, g, beta : token tensors in p->layout and p->dtype (see above).
 *  A_log [Hv], dt_bias [Hv,K] : fp32 gate parameters, used with
 *                     KDA_GATE_IN_KERNEL (A_log required, dt_bias may be NULL = 0;
 *                     dt_bias is read 16 bytes at a time and must be 16-byte aligned).
 *  cu_seqlens       : device int32 [N+1] for TND (must equal cu_seqlens_host); NULL for BSND.
 *  initial_state    : state_rows == 0: fp32 [N,Hv,K,V] or NULL (zero start).
 *                     state_rows  > 0: fp32 state cache [state_rows,Hv,K,V]; sequence n
 *                     starts from row state_indices[n] (zero when that index is invalid).
 *  state_indices    : device int32 [N]; required iff state_rows > 0.
 *  o                : output [.., Hv, V] in p->dtype (every token row is written).
 *  final_state      : state_rows == 0: fp32 [N,Hv,K,V] or NULL (not produced).
 *                     state_rows  > 0: fp32 cache [state_rows,Hv,K,V] or NULL; the final
 *                     state of sequence n is written to row state_indices[n] when that
 *                     index is valid, other rows are untouched.  May equal initial_state.
 *  workspace        : device buffer of at least kda_chunk_fwd_workspace_size bytes.
 *  stage_events     : NULL, or KDA_STAGE_EVENTS hipEvent_t handles (as void*, any may be
 *                     NULL) recorded on `stream` before the first kernel, after the
 *                     chunk-local kernel and after the last kernel of this call; a
 *                     caller times each kernel with them.  Not kept after the call.
 * Inputs are not modified (except the cache when final_state == initial_state).
 * Numeric range with bf16 tokens: the workspace keeps u = (I+L)^-1 (beta v), w,
 * qg, Aqk and kg^T in fp16, and the state update takes v_new = u - w h as an fp16
 * hi/lo pair; these stay exact to about 11 bits for magnitudes from 6.1e-5 to
 * 65504 (with unit-norm keys, |v| up to about 1e4; without KDA_QK_L2NORM, |scale q|
 * and |k| up to 65504).  Larger magnitudes become infinities, so o and the final
 * state turn non-finite rather than silently inexact.  fp32 token runs carry
 * these values in fp32 and bf16 hi/lo pairs (no such bound).
 */
kda_status_t kda_chunk_fwd(const kda_problem_t* p,
                           const void* q, const void* k, const void* v,
                           const void* g, const void* beta,
                           const float* A_log, const float* dt_bias,
                           const float* initial_state, const int32_t* cu_seqlens,
                           const int32_t* state_indices,
                           void* o, float* final_state,
                           void* workspace, size_t workspace_bytes, void* stream,
                           void* const* stage_events);

/* Bytes of device workspace kda_chunk_bwd needs for this problem. */
kda_status_t kda_chunk_bwd_workspace_size(const kda_problem_t* p, size_t* bytes);

/*
 * Chunkwise KDA backward ("KDA Chunk Backward — TPU/Pallas Kernel Design",
 * sections 1.1, 2.2, 2.3 and 2.5; "Hyper-Parallel Chunk KDA" section 5.2):
 * the gradients of L = sum(do * o) + sum(dht * final_state) for the forward
 * kda_chunk_fwd computes with the same arguments.  The forward quantities are
 * recomputed (the call runs the forward's kernels first, keeping every
 * chunk-entry state in the workspace), then the state gradient is carried
 * backwards over the chunks and every chunk's local backward runs in
 * parallel.  All gradients are fp32, computed in fp32; the chunk-entry states,
 * the state gradients and the per-chunk w, u, kg and qg are handed between the
 * kernels in fp16 with either token dtype, so a state or state-gradient entry
 * beyond 65504 turns the gradients non-finite rather than silently inexact.
 *  q ... cu_seqlens : as in kda_chunk_fwd; p->state_rows must be 0 (dense states).
 *  dout  : dL/do, [.., Hv, V] in p->dtype.   dht : fp32 [N,Hv,K,V] or NULL (zero).
 *  dq, dk : fp32 [.., Hk, K] (grouped heads summed over their value heads; with
 *           KDA_QK_L2NORM, with respect to the raw q and k); 16-byte aligned.
 *  dv     : fp32 [.., Hv, V].
 *  dg     : fp32 [.., Hv, K], with respect to g as passed (the raw gate with
 *           KDA_GATE_IN_KERNEL, else the natural-log decay); zero where the
 *           safe-gate clamp is active; 16-byte aligned.
 *  dbeta  : fp32 [.., Hv], with respect to beta as passed (the logit with
 *           KDA_BETA_SIGMOID).
 *  dA_log : fp32 [Hv] or NULL; ddt_bias : fp32 [Hv,K] or NULL (KDA_GATE_IN_KERNEL;
 *           ddt_bias needs dt_bias).  dh0 : fp32 [N,Hv,K,V] or NULL.
 *  workspace : at least kda_chunk_bwd_workspace_size bytes.
 * Every output is overwritten; nothing is accumulated into.
 */
kda_status_t kda_chunk_bwd(const kda_problem_t* p,
                           const void* q, const void* k, const void* v,
                           const void* g, const void* beta,
                           const float* A_log, const float* dt_bias,
                           const float* initial_state, const int32_t* cu_seqlens,
                           const void* dout, const float* dht,
                           float* dq, float* dk, float* dv, float* dg, float* dbeta,
                           float* dA_log, float* ddt_bias, float* dh0,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace kda_segment_summary_bwd needs for this problem. */
kda_status_t kda_segment_summary_bwd_workspace_size(const kda_problem_t* p, size_t* bytes);

/*
 * Backward summary of each sequence ("Hyper-Parallel Chunk KDA" sections 5.2
 * and 6.4, the backward pre-process; "KDA Chunk Backward — TPU/Pallas Kernel
 * Design" section 2.4): local[n] = the gradient of sum(do * o) over sequence n
 * with respect to its initial state when no gradient flows in from its final
 * state.  The state gradient's recursion does not involve the states, so for
 * any gradient dS_T of the final state the initial state's gradient is
 *     M[n]^T dS_T + local[n]
 * with M the forward summary's transition (kda_segment_summary).  Sequence
 * parallelism: each segment computes its (M, local) independently, then
 * kda_summary_merge_bwd hands each segment the gradient of its final state.
 *  q ... cu_seqlens : as in kda_chunk_fwd (p->state_rows must be 0; no state).
 *  dout  : dL/do, [.., Hv, V] in p->dtype.   local : fp32 [N,Hv,K,V] output.
 */
kda_status_t kda_segment_summary_bwd(const kda_problem_t* p,
                                     const void* q, const void* k, const void* v,
                                     const void* g, const void* beta,
                                     const float* A_log, const float* dt_bias,
                                     const int32_t* cu_seqlens, const void* dout,
                                     float* local, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Reverse merge of backward summaries ("Hyper-Parallel Chunk KDA" section 6.4;
 * "KDA Chunk Backward — TPU/Pallas Kernel Design" section 2.4), in place on
 * state [Hv,K,V] (fp32), in reverse time order:
 *     for j = P-1 down to 0:  state <- M[j]^T state + local[j]
 * with M fp32 [P,Hv,K,K] (the forward summaries' transitions) and local fp32
 * [P,Hv,K,V].  Start from the gradient of the last segment's final state
 * (zero if none); after the step for segment j the state is the gradient of
 * segment j-1's final state.  P = 0 launches nothing.
 */
kda_status_t kda_summary_merge_bwd(int32_t P, int32_t Hv, int32_t K, int32_t V,
                                   const float* M, const float* local, float* state,
                                   void* stream);

/* Bytes of the fixed device scratch behind kda_chunk_fwd_noalloc (64 MiB). */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * kda_chunk_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same computation, arguments and results as kda_chunk_fwd (no stage events),
 * with the workspace taken from a fixed KDA_NOALLOC_SCRATCH_BYTES array that
 * the library holds on each GPU it runs on until the process ends.  It calls
 * no allocating routine.  Problems whose kda_chunk_fwd_workspace_size exceeds
 * KDA_NOALLOC_SCRATCH_BYTES are rejected with KDA_ERR_UNSUPPORTED (at K = V =
 * 128 in bf16 that is about 900 (head, 64-token chunk) pairs, e.g. 32 heads x
 * 1792 tokens).  Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (two streams, two threads) race and must be serialised
 * by the caller.  The first call on a device looks up the scratch address on
 * that device (the stream's device is made current for the lookup and then
 * restored).
 */
kda_status_t kda_chunk_fwd_noalloc(const kda_problem_t* p,
                                   const void* q, const void* k, const void* v,
                                   const void* g, const void* beta,
                                   const float* A_log, const float* dt_bias,
                                   const float* initial_state, const int32_t* cu_seqlens,
                                   const int32_t* state_indices,
                                   void* o, float* final_state, void* stream);

/* Bytes of device workspace kda_segment_summary needs for this problem. */
kda_status_t kda_segment_summary_workspace_size(const kda_problem_t* p, size_t* bytes);

/*
 * Affine summary of each sequence ("KDA Context Parallelism (KCP)", notation,
 * composition and algorithm steps 1-2; "Hyper-Parallel Chunk KDA" section 5.1,
 * pre_process_fwd): a state X entering sequence n leaves it as
 *     M[n] X + S_tilde[n],
 * M[n] = the ordered product of the per-token transitions (I - beta k k^T) Diag(alpha),
 * later tokens on the left; S_tilde[n] = the state reached from a zero state.
 *  k, v, g, beta, A_log, dt_bias, cu_seqlens : as in kda_chunk_fwd (no q is needed).
 *  M       : fp32 [N,Hv,K,K] output.   S_tilde : fp32 [N,Hv,K,V] output.
 *  stage_events : as in kda_chunk_fwd.
 * p->state_rows must be 0.
 */
kda_status_t kda_segment_summary(const kda_problem_t* p,
                                 const void* k, const void* v, const void* g, const void* beta,
                                 const float* A_log, const float* dt_bias,
                                 const int32_t* cu_seqlens,
                                 float* M, float* S_tilde,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* stage_events);

/*
 * Prefix merge of preceding summaries ("KDA Context Parallelism (KCP)",
 * algorithm step 4; "Hyper-Parallel Chunk KDA" section 5.3, merge in the
 * forward direction): in place on state [Hv,K,V] (fp32),
 *     for j = 0 .. P-1 in order:  state <- M[j] state + S_tilde[j]
 * with M fp32 [P,Hv,K,K] and S_tilde fp32 [P,Hv,K,V].  Pass a zeroed state to
 * start from zero.  P = 0 leaves the state unchanged and launches nothing.
 * K and V must each be 64 or 128.
 */
kda_status_t kda_summary_merge(int32_t P, int32_t Hv, int32_t K, int32_t V,
                               const float* M, const float* S_tilde, float* state,
                               void* stream);

/*
 * Token-by-token KDA forward for decode ("vllm-ascend KDA prefill state copy"
 * page, background section: the recurrent step that follows a prefill, one
 * token per sequence with the state cache updated in place).  Same problem
 * descriptor, tensors and state conventions as kda_chunk_fwd, any sequence
 * length (each sequence's tokens are applied in order, the state kept in
 * registers), no workspace.  It is meant for a few tokens per sequence: its
 * cost is the state's round trip through HBM plus K*V*8 flop per token and
 * head; longer sequences belong to kda_chunk_fwd.  With a state cache,
 * initial_state and final_state may be the same buffer (in place).
 */
kda_status_t kda_recurrent_fwd(const kda_problem_t* p,
                               const void* q, const void* k, const void* v,
                               const void* g, const void* beta,
                               const float* A_log, const float* dt_bias,
                               const float* initial_state, const int32_t* cu_seqlens,
                               const int32_t* state_indices,
                               void* o, float* final_state, void* stream);

/* Chunk map of packed sequences (host only, no device work): given host
 * cu_seqlens [N+1] and a chunk size, writes chunk_offsets_host [N+1] with the
 * index of each sequence's first chunk (a chunk never spans two sequences and
 * the last chunk of a sequence may be partial); chunk_offsets_host[N] is the
 * total chunk count ("KDA Chunk Backward — TPU/Pallas Kernel Design" section
 * 3.8, chunk-to-segment map). */
kda_status_t kda_chunk_offsets_host(const int32_t* cu_seqlens_host, int32_t N,
                                    int32_t chunk_size, int32_t* chunk_offsets_host);

/* Static description of a status code. */
const char* kda_status_string(kda_status_t s);
/* Detail of the last failure on the calling thread ("" if none). */
const char* kda_last_error(void);
/* KDA_ABI_VERSION of the built library. */
int32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_MI355X_H */
