// C ABI of the KDA library: host-side validation, workspace carving and
// kernel launches.  No arithmetic of the method happens here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>

#include "../../include/kda.h"
#include "kda_bwd_launch.h"

namespace {

thread_local std::string g_last_error;

// Stage events of one call (caller-owned, recorded on the call's stream).
hipError_t record_stage(void* const* ev, int i, hipStream_t s) {
  return (ev && ev[i]) ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) : hipSuccess;
}

kda_status_t fail(kda_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kda_status_t fail(kda_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}
kda_status_t ok() {
  g_last_error.clear();
  return KDA_OK;
}

constexpr int kBT = 64;
constexpr uint32_t kAllFlags = KDA_GATE_IN_KERNEL | KDA_SAFE_GATE | KDA_QK_L2NORM | KDA_BETA_SIGMOID;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Plan {
  int64_t tokens = 0;     // tokens in the token tensors
  int64_t nchunks = 0;    // chunks over all sequences
  int N = 0;
  size_t es = 0;          // element size of token tensors
  int seg_len = 0x7fffffff, seg_max = 1;   // segment-parallel scan (seg_max > 1)
  // workspace offsets
  size_t off_chunk = 0, off_rec = 0, off_mseg = 0, off_sseg = 0, off_hin = 0;
  size_t bytes = 0;
};

// Segment plan of the forward scan.  Automatic: split when fewer than half the
// compute units would hold a (sequence, head, 16-column tile) scan, into
// segments of at least 8 chunks, aiming at about 256 workgroups.
void plan_segments(const kda_problem_t* p, int64_t max_nck, int N, Plan& pl) {
  int target = 1;
  if (p->scan_segments > 1) {
    target = p->scan_segments;
  } else if (p->scan_segments == 0) {
    const int64_t wg = (int64_t)N * p->Hv * (p->V / 16);
    if (wg > 0 && wg < 128) target = (int)std::min<int64_t>(16, 256 / wg);
  }
  if (target < 2 || max_nck < 2) return;
  int64_t len = (max_nck + target - 1) / target;
  if (p->scan_segments == 0) len = std::max<int64_t>(len, 8);
  const int64_t nseg = (max_nck + len - 1) / len;
  if (nseg < 2) return;
  pl.seg_len = (int)len;
  pl.seg_max = (int)nseg;
}

// Shape / flag validation shared by every token-level call; fills the plan.
kda_status_t plan_problem(const kda_problem_t* p, bool forward, Plan& pl) {
  if (!p) return fail(KDA_ERR_INVALID_ARGUMENT, "problem descriptor is NULL");
  if (p->layout != KDA_LAYOUT_BSND && p->layout != KDA_LAYOUT_TND)
    return fail(KDA_ERR_INVALID_ARGUMENT, "layout %d is neither BSND (0) nor TND (1)", p->layout);
  if (p->dtype != KDA_F32 && p->dtype != KDA_BF16)
    return fail(KDA_ERR_INVALID_ARGUMENT, "dtype %d is neither F32 (0) nor BF16 (1)", p->dtype);
  if (p->chunk_size != kBT)
    return fail(KDA_ERR_UNSUPPORTED, "chunk_size %d: only 64 is built", p->chunk_size);
  if (p->Hk < 1 || p->Hv < 1 || p->Hv % p->Hk != 0)
    return fail(KDA_ERR_INVALID_ARGUMENT, "heads Hk=%d Hv=%d: need Hk >= 1 and Hv %% Hk == 0", p->Hk, p->Hv);
  if (p->Hv > 65535) return fail(KDA_ERR_UNSUPPORTED, "Hv=%d exceeds 65535", p->Hv);
  if ((p->K != 64 && p->K != 128) || (p->V != 64 && p->V != 128))
    return fail(KDA_ERR_UNSUPPORTED, "head dims K=%d V=%d: each must be 64 or 128", p->K, p->V);
  if (p->flags & ~kAllFlags) return fail(KDA_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", p->flags & ~kAllFlags);
  if (!std::isfinite(p->scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (!std::isfinite(p->eps) || p->eps < 0.f) return fail(KDA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if ((p->flags & KDA_SAFE_GATE) && !(std::isfinite(p->lower_bound) && p->lower_bound <= 0.f))
    return fail(KDA_ERR_INVALID_ARGUMENT, "lower_bound must be finite and <= 0 (a decay, in natural log)");
  if (p->B < 0 || p->T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "negative B=%d or T=%d", p->B, p->T);
  if (p->state_rows < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "negative state_rows");
  if (p->scan_segments < 0 || p->scan_segments > 4096)
    return fail(KDA_ERR_INVALID_ARGUMENT, "scan_segments %d outside 0 .. 4096", p->scan_segments);
  if (!forward && p->state_rows != 0)
    return fail(KDA_ERR_INVALID_ARGUMENT, "summaries take no state cache (state_rows must be 0)");

  pl.es = p->dtype == KDA_BF16 ? 2 : 4;
  int64_t max_nck = 0;
  if (p->layout == KDA_LAYOUT_BSND) {
    if (p->num_seqs != p->B)
      return fail(KDA_ERR_INVALID_ARGUMENT, "BSND needs num_seqs == B (got %d vs %d)", p->num_seqs, p->B);
    if (p->cu_seqlens_host) return fail(KDA_ERR_INVALID_ARGUMENT, "BSND takes no cu_seqlens");
    pl.N = p->B;
    pl.tokens = (int64_t)p->B * p->T;
    pl.nchunks = (int64_t)p->B * ((p->T + kBT - 1) / kBT);
    max_nck = (p->T + kBT - 1) / kBT;
  } else {
    if (p->B != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "TND needs B == 1 (got %d)", p->B);
    if (p->num_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "negative num_seqs");
    if (!p->cu_seqlens_host) return fail(KDA_ERR_INVALID_ARGUMENT, "TND needs the host copy of cu_seqlens");
    const int32_t* cu = p->cu_seqlens_host;
    if (cu[0] != 0) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens[0] = %d, must be 0", cu[0]);
    int64_t nc = 0;
    for (int i = 0; i < p->num_seqs; ++i) {
      if (cu[i + 1] < cu[i])
        return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %d (%d -> %d)", i, cu[i], cu[i + 1]);
      const int64_t c = (cu[i + 1] - cu[i] + kBT - 1) / kBT;
      nc += c;
      max_nck = std::max(max_nck, c);
    }
    if (cu[p->num_seqs] != p->T)
      return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens[N] = %d differs from T = %d", cu[p->num_seqs], p->T);
    pl.N = p->num_seqs;
    pl.tokens = p->T;
    pl.nchunks = nc;
  }
  if (pl.nchunks > 0x7fffffffLL) return fail(KDA_ERR_UNSUPPORTED, "too many chunks (%lld)", (long long)pl.nchunks);
  const int VA = forward ? p->V : p->V + p->K;
  if ((int64_t)(VA / 16) * p->Hv * pl.N > 0x7fffffffLL || pl.nchunks * (int64_t)p->Hv > 0x7fffffffLL)
    return fail(KDA_ERR_UNSUPPORTED, "too many (sequence, head, tile) workgroups");

  if (forward) plan_segments(p, max_nck, pl.N, pl);
  if ((int64_t)(p->V + p->K) / 16 * p->Hv * pl.N * pl.seg_max > 0x7fffffffLL)
    return fail(KDA_ERR_UNSUPPORTED, "too many (sequence, segment, head, tile) workgroups");

  const size_t slots = (size_t)p->Hv * (size_t)pl.nchunks;
  size_t off = 0;
  pl.off_chunk = off;  off = align256(off + sizeof(int32_t) * (size_t)(pl.N + 1));
  pl.off_rec = off;    off = align256(off + slots * kda::rec_layout(p->K, p->V, (int)pl.es, forward).bytes);
  if (pl.seg_max > 1) {
    const size_t segs = (size_t)pl.N * pl.seg_max * p->Hv;
    pl.off_mseg = off;  off = align256(off + segs * p->K * p->K * sizeof(float));
    pl.off_sseg = off;  off = align256(off + segs * p->K * p->V * sizeof(float));
    pl.off_hin = off;   off = align256(off + segs * p->K * p->V * sizeof(float));
  }
  pl.bytes = off;
  return KDA_OK;
}

kda_status_t check_token_ptr(const void* ptr, const char* name, size_t align) {
  if (!ptr) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned(ptr, align)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not %zu-byte aligned", name, align);
  return KDA_OK;
}

kda::SeqInfo seq_info(const kda_problem_t* p, const Plan& pl, const int32_t* cu, void* ws) {
  kda::SeqInfo s;
  s.tnd = p->layout == KDA_LAYOUT_TND;
  s.T = p->T;
  s.N = pl.N;
  s.cu = cu;
  s.chunk_off = s.tnd ? reinterpret_cast<const int32_t*>(static_cast<char*>(ws) + pl.off_chunk) : nullptr;
  return s;
}

kda_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return KDA_OK;
}

// Launch the chunk-offset prologue (TND) and the chunk-local kernel.
kda_status_t run_intra(const kda_problem_t* p, const Plan& pl, const kda::SeqInfo& si, const int32_t* cu,
                       const void* q, const void* k, const void* v, const void* g, const void* beta,
                       const float* A_log, const float* dt_bias, char* ws, hipStream_t s) {
  if (si.tnd && pl.N > 0) {
    kda_status_t st = hip_status(
        kda::launch_chunk_offsets(cu, pl.N, reinterpret_cast<int32_t*>(ws + pl.off_chunk), s),
        "chunk offsets launch");
    if (st != KDA_OK) return st;
  }
  kda::IntraArgs a{};
  a.seq = si;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.A_log = A_log; a.dt_bias = dt_bias;
  a.Hk = p->Hk; a.Hv = p->Hv; a.nchunks = (int)pl.nchunks;
  a.flags = p->flags; a.scale = p->scale; a.eps = p->eps; a.lower_bound = p->lower_bound;
  a.ws = reinterpret_cast<unsigned char*>(ws + pl.off_rec);
  return hip_status(kda::launch_intra(p->K, p->V, p->dtype, a, s), "intra-chunk kernel launch");
}

kda_status_t common_inputs(const kda_problem_t* p, const Plan& pl, const void* k, const void* v,
                           const void* g, const void* beta, const float* A_log, const float* dt_bias,
                           const int32_t* cu) {
  if (pl.tokens > 0) {
    kda_status_t st;
    if ((st = check_token_ptr(k, "k", 16)) != KDA_OK) return st;
    if ((st = check_token_ptr(v, "v", 16)) != KDA_OK) return st;
    if ((st = check_token_ptr(g, "g", 16)) != KDA_OK) return st;
    if ((st = check_token_ptr(beta, "beta", pl.es)) != KDA_OK) return st;
    if ((p->flags & KDA_GATE_IN_KERNEL) && !A_log)
      return fail(KDA_ERR_INVALID_ARGUMENT, "KDA_GATE_IN_KERNEL needs A_log");
    if ((p->flags & KDA_GATE_IN_KERNEL) && dt_bias && !aligned(dt_bias, 16))
      return fail(KDA_ERR_INVALID_ARGUMENT, "dt_bias must be 16-byte aligned");
  }
  if (p->layout == KDA_LAYOUT_TND && !cu) return fail(KDA_ERR_INVALID_ARGUMENT, "TND needs device cu_seqlens");
  return KDA_OK;
}

}  // namespace

extern "C" {

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status_t s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KDA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

kda_status_t kda_chunk_offsets_host(const int32_t* cu, int32_t N, int32_t chunk, int32_t* out) {
  if (!cu || !out || N < 0 || chunk < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "bad chunk-offset arguments");
  if (cu[0] != 0) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens[0] must be 0");
  int64_t run = 0;
  for (int i = 0; i < N; ++i) {
    if (cu[i + 1] < cu[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %d", i);
    out[i] = (int32_t)run;
    run += (cu[i + 1] - cu[i] + chunk - 1) / chunk;
    if (run > 0x7fffffffLL) return fail(KDA_ERR_UNSUPPORTED, "too many chunks");
  }
  out[N] = (int32_t)run;
  return ok();
}

kda_status_t kda_chunk_fwd_workspace_size(const kda_problem_t* p, size_t* bytes) {
  if (!bytes) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Plan pl;
  kda_status_t st = plan_problem(p, true, pl);
  if (st != KDA_OK) return st;
  *bytes = pl.bytes;
  return ok();
}

kda_status_t kda_segment_summary_workspace_size(const kda_problem_t* p, size_t* bytes) {
  if (!bytes) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Plan pl;
  kda_status_t st = plan_problem(p, false, pl);
  if (st != KDA_OK) return st;
  *bytes = pl.bytes;
  return ok();
}

kda_status_t kda_chunk_fwd(const kda_problem_t* p, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, const float* A_log, const float* dt_bias,
                           const float* initial_state, const int32_t* cu_seqlens,
                           const int32_t* state_indices, void* o, float* final_state,
                           void* workspace, size_t workspace_bytes, void* stream,
                           void* const* stage_events) {
  Plan pl;
  kda_status_t st = plan_problem(p, true, pl);
  if (st != KDA_OK) return st;
  if ((st = common_inputs(p, pl, k, v, g, beta, A_log, dt_bias, cu_seqlens)) != KDA_OK) return st;
  if (pl.tokens > 0) {
    if ((st = check_token_ptr(q, "q", 16)) != KDA_OK) return st;
    if ((st = check_token_ptr(o, "o", 16)) != KDA_OK) return st;
  }
  if (p->state_rows > 0 && !state_indices)
    return fail(KDA_ERR_INVALID_ARGUMENT, "state_rows > 0 needs state_indices");
  if (p->state_rows == 0 && state_indices)
    return fail(KDA_ERR_INVALID_ARGUMENT, "state_indices given without a state cache (state_rows == 0)");
  if ((initial_state && !aligned(initial_state, 16)) || (final_state && !aligned(final_state, 16)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "states must be 16-byte aligned");
  if (workspace_bytes < pl.bytes)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.bytes);
  if (pl.bytes && !workspace) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (pl.N == 0) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  kda::SeqInfo si = seq_info(p, pl, cu_seqlens, ws);
  if ((st = hip_status(record_stage(stage_events, 0, s), "stage event")) != KDA_OK) return st;
  if ((st = run_intra(p, pl, si, cu_seqlens, q, k, v, g, beta, A_log, dt_bias, ws, s)) != KDA_OK) return st;
  if ((st = hip_status(record_stage(stage_events, 1, s), "stage event")) != KDA_OK) return st;
  kda::ScanArgs a{};
  a.seq = si;
  a.Hv = p->Hv; a.nchunks = (int)pl.nchunks; a.state_rows = p->state_rows;
  a.ws = reinterpret_cast<const unsigned char*>(ws + pl.off_rec);
  a.seg_len = pl.seg_len; a.seg_max = pl.seg_max;
  if (pl.seg_max > 1) {
    // segment-parallel scan: summaries of every segment but each sequence's
    // last, their prefix merge, then all segments' scans from their incoming states
    float* Mseg = reinterpret_cast<float*>(ws + pl.off_mseg);
    float* Sseg = reinterpret_cast<float*>(ws + pl.off_sseg);
    float* hin = reinterpret_cast<float*>(ws + pl.off_hin);
    kda::ScanArgs sa = a;
    sa.summary = 1; sa.fwd_records = 1; sa.skip_last = 1; sa.state_rows = 0;
    sa.hT = Sseg; sa.M = Mseg;
    if ((st = hip_status(kda::launch_scan(p->K, p->V, p->dtype, sa, s), "segment summary scan launch")) != KDA_OK)
      return st;
    kda::PrefixMergeArgs ma{};
    ma.seq = si; ma.Hv = p->Hv; ma.seg_len = pl.seg_len; ma.seg_max = pl.seg_max;
    ma.state_rows = p->state_rows; ma.M = Mseg; ma.S = Sseg; ma.h0 = initial_state;
    ma.state_idx = state_indices; ma.h_in = hin;
    if ((st = hip_status(kda::launch_prefix_merge(p->K, p->V, ma, s), "segment prefix merge launch")) != KDA_OK)
      return st;
    a.h_in = hin;
  }
  a.summary = 0;
  a.h0 = initial_state; a.state_idx = state_indices; a.hT = final_state; a.M = nullptr; a.o = o;
  if ((st = hip_status(kda::launch_scan(p->K, p->V, p->dtype, a, s), "state-scan kernel launch")) != KDA_OK)
    return st;
  if ((st = hip_status(record_stage(stage_events, 2, s), "stage event")) != KDA_OK) return st;
  return ok();
}

kda_status_t kda_segment_summary(const kda_problem_t* p, const void* k, const void* v, const void* g,
                                 const void* beta, const float* A_log, const float* dt_bias,
                                 const int32_t* cu_seqlens, float* M, float* S_tilde, void* workspace,
                                 size_t workspace_bytes, void* stream, void* const* stage_events) {
  Plan pl;
  kda_status_t st = plan_problem(p, false, pl);
  if (st != KDA_OK) return st;
  if ((st = common_inputs(p, pl, k, v, g, beta, A_log, dt_bias, cu_seqlens)) != KDA_OK) return st;
  if (pl.N > 0 && (!M || !S_tilde)) return fail(KDA_ERR_INVALID_ARGUMENT, "M and S_tilde are required");
  if ((M && !aligned(M, 16)) || (S_tilde && !aligned(S_tilde, 16)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "M and S_tilde must be 16-byte aligned");
  if (workspace_bytes < pl.bytes)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, pl.bytes);
  if (pl.bytes && !workspace) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (pl.N == 0) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  kda::SeqInfo si = seq_info(p, pl, cu_seqlens, ws);
  if ((st = hip_status(record_stage(stage_events, 0, s), "stage event")) != KDA_OK) return st;
  if ((st = run_intra(p, pl, si, cu_seqlens, nullptr, k, v, g, beta, A_log, dt_bias, ws, s)) != KDA_OK)
    return st;
  if ((st = hip_status(record_stage(stage_events, 1, s), "stage event")) != KDA_OK) return st;
  kda::ScanArgs a{};
  a.seq = si;
  a.Hv = p->Hv; a.nchunks = (int)pl.nchunks; a.state_rows = 0; a.summary = 1;
  a.seg_len = 0x7fffffff; a.seg_max = 1;
  a.ws = reinterpret_cast<const unsigned char*>(ws + pl.off_rec);
  a.hT = S_tilde; a.M = M;
  if ((st = hip_status(kda::launch_scan(p->K, p->V, p->dtype, a, s), "summary scan kernel launch")) != KDA_OK)
    return st;
  if ((st = hip_status(record_stage(stage_events, 2, s), "stage event")) != KDA_OK) return st;
  return ok();
}

namespace {

// Workspace of the backward: the chunk map, then the backward records, the
// chunk-entry states, the chunk-exit state gradients, the per-value-head q/k
// gradients, beta and decay gradients, the gate's block partial sums and
// each chunk's dL / dAqk for the pair sums.
struct BwdPlan {
  Plan fwd;
  size_t off_rec = 0, off_h = 0, off_dh = 0, off_dqn = 0, off_dkn = 0, off_db = 0, off_dg = 0, off_part = 0;
  size_t off_pairs = 0;
  size_t bytes = 0;
  int64_t tokens = 0;
};

kda_status_t plan_bwd(const kda_problem_t* p, BwdPlan& bp) {
  kda_problem_t q = *p;
  q.scan_segments = 1;                       // (the forward's segment plan plays no part here)
  kda_status_t st = plan_problem(&q, true, bp.fwd);
  if (st != KDA_OK) return st;
  if (p->state_rows != 0)
    return fail(KDA_ERR_UNSUPPORTED, "the backward takes dense initial states (state_rows must be 0)");
  const Plan& f = bp.fwd;
  bp.tokens = f.tokens;
  const size_t slots = (size_t)p->Hv * (size_t)f.nchunks;
  const size_t th = (size_t)f.tokens * p->Hv;
  const size_t nblk = (size_t)((f.tokens + kda::BWD_GATE_TOKENS - 1) / kda::BWD_GATE_TOKENS);
  size_t off = align256(f.off_rec);            // the chunk map only; no forward records
  bp.off_rec = off;  off = align256(off + slots * kda::bwd_rec(p->K, p->V).bytes);
  // the chunk-entry states and the exit gradients in fp16 (2 bytes per element)
  bp.off_h = off;    off = align256(off + slots * p->K * p->V * 2);
  bp.off_dh = off;   off = align256(off + slots * p->K * p->V * 2);
  bp.off_dqn = off;  off = align256(off + th * p->K * sizeof(float));
  bp.off_dkn = off;  off = align256(off + th * p->K * sizeof(float));
  bp.off_db = off;   off = align256(off + th * sizeof(float));
  bp.off_dg = off;   off = align256(off + th * p->K * sizeof(float));
  bp.off_part = off; off = align256(off + nblk * p->Hv * (p->K + 1) * sizeof(float));
  bp.off_pairs = off; off = align256(off + slots * 2 * kda::BT * kda::BT * sizeof(float));
  bp.bytes = off;
  return KDA_OK;
}

}  // namespace

kda_status_t kda_chunk_bwd_workspace_size(const kda_problem_t* p, size_t* bytes) {
  if (!bytes) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  BwdPlan bp;
  kda_status_t st = plan_bwd(p, bp);
  if (st != KDA_OK) return st;
  *bytes = bp.bytes;
  return ok();
}

kda_status_t kda_chunk_bwd(const kda_problem_t* p, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, const float* A_log, const float* dt_bias,
                           const float* initial_state, const int32_t* cu_seqlens, const void* dout,
                           const float* dht, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                           float* dA_log, float* ddt_bias, float* dh0, void* workspace,
                           size_t workspace_bytes, void* stream) {
  BwdPlan bp;
  kda_status_t st = plan_bwd(p, bp);
  if (st != KDA_OK) return st;
  const Plan& pl = bp.fwd;
  if ((st = common_inputs(p, pl, k, v, g, beta, A_log, dt_bias, cu_seqlens)) != KDA_OK) return st;
  if (pl.tokens > 0) {
    if ((st = check_token_ptr(q, "q", 16)) != KDA_OK) return st;
    if ((st = check_token_ptr(dout, "do", 16)) != KDA_OK) return st;
    // dq, dk and dg are written 16 bytes at a time
    const struct { const void* ptr; const char* name; size_t align; } outs[] = {
        {dq, "dq", 16}, {dk, "dk", 16}, {dv, "dv", 4}, {dg, "dg", 16}, {dbeta, "dbeta", 4}};
    for (const auto& o : outs)
      if ((st = check_token_ptr(o.ptr, o.name, o.align)) != KDA_OK) return st;
  }
  for (const float* s : {initial_state, dht, (const float*)dh0, (const float*)dA_log, (const float*)ddt_bias})
    if (s && !aligned(s, 4)) return fail(KDA_ERR_INVALID_ARGUMENT, "fp32 arguments must be 4-byte aligned");
  if (workspace_bytes < bp.bytes)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, bp.bytes);
  if (bp.bytes && !workspace) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (pl.N == 0) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  kda::SeqInfo si = seq_info(p, pl, cu_seqlens, ws);
  if (si.tnd) {   // chunk map of the packed sequences
    if ((st = hip_status(kda::launch_chunk_offsets(cu_seqlens, pl.N, reinterpret_cast<int32_t*>(ws + pl.off_chunk), s),
                         "chunk offsets launch")) != KDA_OK)
      return st;
  }
  // 2. - 6. backward stages
  kda::BwdArgs a{};
  a.seq = si;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.dout = dout;
  a.A_log = A_log; a.dt_bias = dt_bias; a.dht = dht;
  a.Hk = p->Hk; a.Hv = p->Hv; a.nchunks = (int)pl.nchunks;
  a.flags = p->flags; a.scale = p->scale; a.eps = p->eps; a.lower_bound = p->lower_bound;
  a.rec = reinterpret_cast<float*>(ws + bp.off_rec);
  a.h0 = initial_state;
  a.h_store = reinterpret_cast<const _Float16*>(ws + bp.off_h);
  a.h_store_w = reinterpret_cast<_Float16*>(ws + bp.off_h);
  a.dh_store = reinterpret_cast<_Float16*>(ws + bp.off_dh);
  a.dh0 = dh0;
  a.dqn = reinterpret_cast<float*>(ws + bp.off_dqn);
  a.dkn = reinterpret_cast<float*>(ws + bp.off_dkn);
  a.dbeta_act = reinterpret_cast<float*>(ws + bp.off_db);
  a.dg_nat = reinterpret_cast<float*>(ws + bp.off_dg);
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta;
  a.dA_log = (p->flags & KDA_GATE_IN_KERNEL) ? dA_log : nullptr;
  a.ddt_bias = ((p->flags & KDA_GATE_IN_KERNEL) && dt_bias) ? ddt_bias : nullptr;
  a.pairs = reinterpret_cast<float*>(ws + bp.off_pairs);
  float* part = reinterpret_cast<float*>(ws + bp.off_part);
  // prep (records), forward states, reverse state scan, chunk backward and its
  // pair sums, q/k, gate, gate sums
  static const int order[] = {0, 6, 1, 2, 7, 3, 4, 5};
  static const char* what[] = {"backward prep launch", "backward reverse scan launch", "backward chunk launch",
                               "backward q/k launch", "backward gate launch", "backward gate sum launch",
                               "backward state scan launch", "backward pair sums launch"};
  for (int stage : order)
    if ((st = hip_status(kda::launch_bwd(p->K, p->V, p->dtype, a, stage, bp.tokens, part, s), what[stage])) != KDA_OK)
      return st;
  return ok();
}

kda_status_t kda_segment_summary_bwd_workspace_size(const kda_problem_t* p, size_t* bytes) {
  if (!bytes) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  BwdPlan bp;
  kda_status_t st = plan_bwd(p, bp);
  if (st != KDA_OK) return st;
  *bytes = bp.off_h;     // the chunk map and the backward records
  return ok();
}

kda_status_t kda_segment_summary_bwd(const kda_problem_t* p, const void* q, const void* k, const void* v,
                                     const void* g, const void* beta, const float* A_log, const float* dt_bias,
                                     const int32_t* cu_seqlens, const void* dout, float* local, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  BwdPlan bp;
  kda_status_t st = plan_bwd(p, bp);
  if (st != KDA_OK) return st;
  const Plan& pl = bp.fwd;
  if ((st = common_inputs(p, pl, k, v, g, beta, A_log, dt_bias, cu_seqlens)) != KDA_OK) return st;
  if (pl.tokens > 0) {
    if ((st = check_token_ptr(q, "q", 16)) != KDA_OK) return st;
    if ((st = check_token_ptr(dout, "do", 16)) != KDA_OK) return st;
  }
  if (pl.N > 0 && (!local || !aligned(local, 4)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "local is NULL or misaligned");
  if (workspace_bytes < bp.off_h)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, bp.off_h);
  if (bp.off_h && !workspace) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (pl.N == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  kda::SeqInfo si = seq_info(p, pl, cu_seqlens, ws);
  if (si.tnd) {
    if ((st = hip_status(kda::launch_chunk_offsets(cu_seqlens, pl.N, reinterpret_cast<int32_t*>(ws + pl.off_chunk), s),
                         "chunk offsets launch")) != KDA_OK)
      return st;
  }
  kda::BwdArgs a{};
  a.seq = si;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.dout = dout;
  a.A_log = A_log; a.dt_bias = dt_bias; a.dht = nullptr;
  a.Hk = p->Hk; a.Hv = p->Hv; a.nchunks = (int)pl.nchunks;
  a.flags = p->flags; a.scale = p->scale; a.eps = p->eps; a.lower_bound = p->lower_bound;
  a.rec = reinterpret_cast<float*>(ws + bp.off_rec);
  a.dh_store = nullptr;
  a.dh0 = local;
  if ((st = hip_status(kda::launch_bwd(p->K, p->V, p->dtype, a, 0, bp.tokens, nullptr, s), "backward prep launch")) != KDA_OK)
    return st;
  if ((st = hip_status(kda::launch_bwd(p->K, p->V, p->dtype, a, 1, bp.tokens, nullptr, s),
                       "backward reverse scan launch")) != KDA_OK)
    return st;
  return ok();
}

kda_status_t kda_summary_merge_bwd(int32_t P, int32_t Hv, int32_t K, int32_t V, const float* M,
                                   const float* local, float* state, void* stream) {
  if (P < 0 || Hv < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "need P >= 0 and Hv >= 1 (P=%d Hv=%d)", P, Hv);
  if ((K != 64 && K != 128) || (V != 64 && V != 128))
    return fail(KDA_ERR_UNSUPPORTED, "head dims K=%d V=%d: each must be 64 or 128", K, V);
  if ((int64_t)Hv * (V / 32) > 0x7fffffffLL) return fail(KDA_ERR_UNSUPPORTED, "too many heads");
  if (!state || !aligned(state, 16)) return fail(KDA_ERR_INVALID_ARGUMENT, "state is NULL or misaligned");
  if (P == 0) return ok();
  if (!M || !local || !aligned(M, 16) || !aligned(local, 16))
    return fail(KDA_ERR_INVALID_ARGUMENT, "M and local must be non-NULL and 16-byte aligned");
  kda::MergeArgs a{P, Hv, M, local, state};
  kda_status_t st = hip_status(kda::launch_merge(K, V, a, static_cast<hipStream_t>(stream), true),
                               "reverse merge kernel launch");
  if (st != KDA_OK) return st;
  return ok();
}

kda_status_t kda_chunk_fwd_noalloc(const kda_problem_t* p, const void* q, const void* k, const void* v,
                                   const void* g, const void* beta, const float* A_log, const float* dt_bias,
                                   const float* initial_state, const int32_t* cu_seqlens,
                                   const int32_t* state_indices, void* o, float* final_state, void* stream) {
  Plan pl;
  kda_status_t st = plan_problem(p, true, pl);
  if (st != KDA_OK) return st;
  if (pl.bytes > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
    return fail(KDA_ERR_UNSUPPORTED,
                "this problem needs %zu bytes of workspace; the fixed scratch holds %zu "
                "(call kda_chunk_fwd with a workspace instead)",
                pl.bytes, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
  if (pl.N == 0) return kda_chunk_fwd(p, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens,
                                      state_indices, o, final_state, nullptr, 0, stream, nullptr);
  void* ws = nullptr;
  char why[160] = "";
  const hipError_t e = kda::noalloc_scratch(static_cast<hipStream_t>(stream), &ws, why, sizeof why);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "fixed scratch: %s: %s", why, hipGetErrorString(e));
  return kda_chunk_fwd(p, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens, state_indices, o,
                       final_state, ws, KDA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

kda_status_t kda_recurrent_fwd(const kda_problem_t* p, const void* q, const void* k, const void* v,
                               const void* g, const void* beta, const float* A_log, const float* dt_bias,
                               const float* initial_state, const int32_t* cu_seqlens,
                               const int32_t* state_indices, void* o, float* final_state, void* stream) {
  Plan pl;
  kda_status_t st = plan_problem(p, true, pl);
  if (st != KDA_OK) return st;
  if ((st = common_inputs(p, pl, k, v, g, beta, A_log, dt_bias, cu_seqlens)) != KDA_OK) return st;
  if (pl.tokens > 0) {
    if ((st = check_token_ptr(q, "q", 16)) != KDA_OK) return st;
    if ((st = check_token_ptr(o, "o", 16)) != KDA_OK) return st;
  }
  if (p->state_rows > 0 && !state_indices)
    return fail(KDA_ERR_INVALID_ARGUMENT, "state_rows > 0 needs state_indices");
  if (p->state_rows == 0 && state_indices)
    return fail(KDA_ERR_INVALID_ARGUMENT, "state_indices given without a state cache (state_rows == 0)");
  if ((initial_state && !aligned(initial_state, 16)) || (final_state && !aligned(final_state, 16)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "states must be 16-byte aligned");
  if (pl.N == 0) return ok();
  kda::RecurrentArgs a{};
  a.seq.tnd = p->layout == KDA_LAYOUT_TND;
  a.seq.T = p->T;
  a.seq.N = pl.N;
  a.seq.cu = cu_seqlens;
  a.seq.chunk_off = nullptr;   // the recurrent kernel walks tokens, not chunks
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.A_log = A_log; a.dt_bias = dt_bias;
  a.Hk = p->Hk; a.Hv = p->Hv; a.state_rows = p->state_rows;
  a.flags = p->flags; a.scale = p->scale; a.eps = p->eps; a.lower_bound = p->lower_bound;
  a.h0 = initial_state; a.state_idx = state_indices; a.hT = final_state; a.o = o;
  if ((st = hip_status(kda::launch_recurrent(p->K, p->V, p->dtype, a, static_cast<hipStream_t>(stream)),
                       "recurrent kernel launch")) != KDA_OK)
    return st;
  return ok();
}

kda_status_t kda_summary_merge(int32_t P, int32_t Hv, int32_t K, int32_t V, const float* M,
                               const float* S_tilde, float* state, void* stream) {
  if (P < 0 || Hv < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "need P >= 0 and Hv >= 1 (P=%d Hv=%d)", P, Hv);
  if ((K != 64 && K != 128) || (V != 64 && V != 128))
    return fail(KDA_ERR_UNSUPPORTED, "head dims K=%d V=%d: each must be 64 or 128", K, V);
  if ((int64_t)Hv * (V / 32) > 0x7fffffffLL) return fail(KDA_ERR_UNSUPPORTED, "too many heads");
  if (!state || !aligned(state, 16)) return fail(KDA_ERR_INVALID_ARGUMENT, "state is NULL or misaligned");
  if (P == 0) return ok();
  if (!M || !S_tilde || !aligned(M, 16) || !aligned(S_tilde, 16))
    return fail(KDA_ERR_INVALID_ARGUMENT, "M and S_tilde must be non-NULL and 16-byte aligned");
  kda::MergeArgs a{P, Hv, M, S_tilde, state};
  kda_status_t st = hip_status(kda::launch_merge(K, V, a, static_cast<hipStream_t>(stream)), "merge kernel launch");
  if (st != KDA_OK) return st;
  return ok();
}

}  // extern "C"
