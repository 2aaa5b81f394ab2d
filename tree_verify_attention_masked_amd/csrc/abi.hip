// extern "C" entry points of libspectree: host-side validation, planning and
// launches on the caller's stream.  No call allocates, synchronises or copies
// to the host.
#include <cmath>

#include "common.h"

using namespace spectree;

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool dtype_ok(int dtype, int D) {
  if (dtype == SPEC_BF16) return D == 128;
  if (dtype == SPEC_F32) return D == 64 || D == 128;
  return false;
}

// Rows of queries, keys, values and outputs move with 16-byte vector accesses.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by attention and compaction.  Returns SPEC_OK or an error.
int check_kv_shapes(int B, int T, int Hkv, int D, int block_size, int max_blocks, int num_blocks, int dtype) {
  if (B < 0 || T < 1 || Hkv < 1 || D < 1 || max_blocks < 1 || num_blocks < 1) return SPEC_ERR_INVALID_ARG;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_INVALID_ARG;
  if (block_size != kBlockSize || T > kMaxT || !dtype_ok(dtype, D)) return SPEC_ERR_UNSUPPORTED;
  if (static_cast<long>(max_blocks) * kBlockSize < T) return SPEC_ERR_INVALID_ARG;
  if (static_cast<long>(max_blocks) * kBlockSize > (1L << 30)) return SPEC_ERR_UNSUPPORTED;
  return SPEC_OK;
}

}  // namespace

extern "C" {

const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK:
      return "SPEC_OK";
    case SPEC_ERR_INVALID_ARG:
      return "SPEC_ERR_INVALID_ARG: null pointer or inconsistent size";
    case SPEC_ERR_UNSUPPORTED:
      return "SPEC_ERR_UNSUPPORTED: dtype, head dim, block size or tree size not supported";
    case SPEC_ERR_WORKSPACE:
      return "SPEC_ERR_WORKSPACE: workspace missing or too small";
    case SPEC_ERR_HIP:
      return "SPEC_ERR_HIP: HIP launch failed";
    default:
      return "unknown spec_status";
  }
}

int spec_version(void) { return kVersion; }

size_t spec_tree_attn_workspace_size(int B, int T, int Hq, int Hkv, int D, int max_blocks_per_seq, int dtype) {
  if (B <= 0 || T < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || max_blocks_per_seq < 1 || !dtype_ok(dtype, D))
    return 0;
  return plan_attn(B, T, Hq, Hkv, D, max_blocks_per_seq, dtype).ws_bytes;
}

int spec_tree_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                   const int32_t* prefix_lens, const int32_t* parent, void* out, int B, int T, int Hq, int Hkv,
                   int D, int block_size, int max_blocks_per_seq, int num_blocks, float scale, int dtype,
                   int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_kv_shapes(B, T, Hkv, D, block_size, max_blocks_per_seq, num_blocks, dtype);
  if (rc != SPEC_OK) return rc;
  if (Hq < Hkv || Hq % Hkv != 0) return SPEC_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return SPEC_ERR_INVALID_ARG;  // the kernels track the largest score
  if (B == 0) return SPEC_OK;
  if (!q || !k_cache || !v_cache || !block_table || !prefix_lens || !parent || !out) return SPEC_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return SPEC_ERR_INVALID_ARG;
  const AttnPlan plan = plan_attn(B, T, Hq, Hkv, D, max_blocks_per_seq, dtype);
  if (plan.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.ws_bytes)) return SPEC_ERR_WORKSPACE;
  AttnLaunch L{};
  L.q = q;
  L.k = k_cache;
  L.v = v_cache;
  L.block_table = block_table;
  L.prefix_lens = prefix_lens;
  L.parent = parent;
  L.out = out;
  L.status = status;
  L.workspace = workspace;
  L.B = B;
  L.T = T;
  L.Hq = Hq;
  L.Hkv = Hkv;
  L.D = D;
  L.max_blocks = max_blocks_per_seq;
  L.num_blocks = num_blocks;
  L.scale = scale;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = (dtype == SPEC_BF16) ? launch_attn_bf16(plan, L, s) : launch_attn_f32(plan, L, s);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

size_t spec_tree_reject_workspace_size(int B, int T, int V) {
  if (B <= 0 || T < 1 || V < 1) return 0;
  return reject_workspace_bytes(B, T, V);
}

int spec_tree_reject_plan(int B, int T, int V, int64_t max_resident_workgroups, int* team_size, int* slice_len) {
  if (B < 1 || T < 1 || V < 1 || max_resident_workgroups < 1 || !team_size || !slice_len)
    return SPEC_ERR_INVALID_ARG;
  if (T > kMaxT || V > kMaxV) return SPEC_ERR_UNSUPPORTED;
  reject_plan(B, T, V, static_cast<long>(max_resident_workgroups), team_size, slice_len);
  return SPEC_OK;
}

int64_t spec_tree_reject_max_resident(void) { return reject_resident_capacity(); }

size_t spec_tree_reject_truncated_workspace_size(int B, int T, int V, int top_k) {
  if (B <= 0 || T < 1 || V < 1 || top_k < 1 || top_k > kTruncTopKMax) return 0;
  return reject_trunc_workspace_bytes(B, T, V, top_k);
}

int spec_tree_reject_truncated_plan(int B, int T, int V, int top_k, int64_t max_resident_workgroups, int* team_size,
                                    int* list_len) {
  if (B < 1 || T < 1 || V < 1 || max_resident_workgroups < 1 || !team_size || !list_len)
    return SPEC_ERR_INVALID_ARG;
  if (T > kMaxT || V > kMaxV || top_k < 1 || top_k > kTruncTopKMax) return SPEC_ERR_UNSUPPORTED;
  reject_trunc_plan(B, T, V, top_k, static_cast<long>(max_resident_workgroups), team_size, list_len);
  return SPEC_OK;
}

}  // extern "C"

namespace {

// Stand-in for the workspace pointer of the allocation-free entry point during
// validation (never dereferenced: launch_reject_static puts the device address
// of its static array in its place).
void* const kStaticWorkspace = reinterpret_cast<void*>(static_cast<uintptr_t>(1));

// Host validation of the sampler's arguments and its launch description.
int make_reject(const float* target_logits, const float* draft_probs, const int32_t* draft_tokens,
                const int32_t* parent, int B, int T, int V, float temperature, int without_replacement, uint64_t seed,
                uint64_t offset, int32_t* accepted_nodes, int32_t* out_tokens, int32_t* num_accepted,
                int32_t* status, void* workspace, size_t workspace_bytes, RejectLaunch* L) {
  if (B < 0 || T < 1 || V < 1) return SPEC_ERR_INVALID_ARG;
  if (T > kMaxT || V > kMaxV) return SPEC_ERR_UNSUPPORTED;
  if (!(temperature >= 0.0f) || !std::isfinite(temperature)) return SPEC_ERR_INVALID_ARG;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !draft_tokens || !parent || !accepted_nodes || !out_tokens || !num_accepted)
    return SPEC_ERR_INVALID_ARG;
  if (temperature > 0.0f && !draft_probs) return SPEC_ERR_INVALID_ARG;
  const size_t need = reject_workspace_bytes(B, T, V);
  if (workspace == nullptr || workspace_bytes < need) return SPEC_ERR_WORKSPACE;  // (see kStaticWorkspace)
  *L = RejectLaunch{};
  L->logits = target_logits;
  L->q = draft_probs;
  L->tokens = draft_tokens;
  L->parent = parent;
  L->B = B;
  L->T = T;
  L->V = V;
  L->temperature = temperature;
  L->without_replacement = without_replacement;
  L->seed = seed;
  L->offset = offset;
  L->accepted = accepted_nodes;
  L->out_tokens = out_tokens;
  L->num_accepted = num_accepted;
  L->status = status;
  L->workspace = workspace;
  L->workspace_bytes = workspace_bytes;
  return SPEC_OK;
}

// Host validation of the compaction's arguments (the path pointers are checked
// by the caller when they are inputs) and its launch description.
int make_compact(void* k_cache, void* v_cache, const int32_t* block_table, const int32_t* prefix_lens,
                 int32_t* new_lens, int B, int T, int Hkv, int D, int block_size, int max_blocks_per_seq,
                 int num_blocks, int dtype, int32_t* status, CompactLaunch* L) {
  const int rc = check_kv_shapes(B, T, Hkv, D, block_size, max_blocks_per_seq, num_blocks, dtype);
  if (rc != SPEC_OK) return rc;
  if (B == 0) return SPEC_OK;
  if (!k_cache || !v_cache || !block_table || !prefix_lens) return SPEC_ERR_INVALID_ARG;
  *L = CompactLaunch{};
  L->k = k_cache;
  L->v = v_cache;
  L->block_table = block_table;
  L->prefix_lens = prefix_lens;
  L->new_lens = new_lens;
  L->status = status;
  L->B = B;
  L->T = T;
  L->Hkv = Hkv;
  L->D = D;
  L->max_blocks = max_blocks_per_seq;
  L->num_blocks = num_blocks;
  L->elem_bytes = dtype == SPEC_BF16 ? 2 : 4;
  return SPEC_OK;
}

}  // namespace

extern "C" {

int spec_tree_reject(const float* target_logits, const float* draft_probs, const int32_t* draft_tokens,
                     const int32_t* parent, int B, int T, int V, float temperature, int without_replacement,
                     uint64_t seed, uint64_t offset, int32_t* accepted_nodes, int32_t* out_tokens,
                     int32_t* num_accepted, int32_t* status, void* workspace, size_t workspace_bytes,
                     void* stream) {
  RejectLaunch L;
  const int rc = make_reject(target_logits, draft_probs, draft_tokens, parent, B, T, V, temperature,
                             without_replacement, seed, offset, accepted_nodes, out_tokens, num_accepted, status,
                             workspace, workspace_bytes, &L);
  if (rc != SPEC_OK || B == 0) return rc;
  const hipError_t e = launch_reject(L, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int spec_kv_compact(void* k_cache, void* v_cache, const int32_t* block_table, const int32_t* prefix_lens,
                    const int32_t* accepted_nodes, const int32_t* num_accepted, int32_t* new_lens, int B, int T,
                    int Hkv, int D, int block_size, int max_blocks_per_seq, int num_blocks, int dtype,
                    int32_t* status, void* stream) {
  CompactLaunch L;
  const int rc = make_compact(k_cache, v_cache, block_table, prefix_lens, new_lens, B, T, Hkv, D, block_size,
                              max_blocks_per_seq, num_blocks, dtype, status, &L);
  if (rc != SPEC_OK || B == 0) return rc;
  if (!accepted_nodes || !num_accepted) return SPEC_ERR_INVALID_ARG;
  L.accepted = accepted_nodes;
  L.num_accepted = num_accepted;
  const hipError_t e = launch_compact(L, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int spec_tree_reject_compact(const float* target_logits, const float* draft_probs, const int32_t* draft_tokens,
                             const int32_t* parent, int B, int T, int V, float temperature, int without_replacement,
                             uint64_t seed, uint64_t offset, int32_t* accepted_nodes, int32_t* out_tokens,
                             int32_t* num_accepted, int32_t* status, void* workspace, size_t workspace_bytes,
                             void* k_cache, void* v_cache, const int32_t* block_table, const int32_t* prefix_lens,
                             int32_t* new_lens, int Hkv, int D, int block_size, int max_blocks_per_seq,
                             int num_blocks, int dtype, void* stream) {
  RejectLaunch R;
  int rc = make_reject(target_logits, draft_probs, draft_tokens, parent, B, T, V, temperature, without_replacement,
                       seed, offset, accepted_nodes, out_tokens, num_accepted, status, workspace, workspace_bytes,
                       &R);
  if (rc != SPEC_OK) return rc;
  CompactLaunch C;
  rc = make_compact(k_cache, v_cache, block_table, prefix_lens, new_lens, B, T, Hkv, D, block_size,
                    max_blocks_per_seq, num_blocks, dtype, status, &C);
  if (rc != SPEC_OK || B == 0) return rc;
  R.compact = &C;  // copied into the kernel arguments at launch
  const hipError_t e = launch_reject(R, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int spec_tree_reject_truncated(const float* target_logits, const float* draft_probs, const int32_t* draft_tokens,
                               const int32_t* parent, int B, int T, int V, float temperature, int top_k, float top_p,
                               int without_replacement, uint64_t seed, uint64_t offset, int32_t* accepted_nodes,
                               int32_t* out_tokens, int32_t* num_accepted, int32_t* status, void* workspace,
                               size_t workspace_bytes, void* k_cache, void* v_cache, const int32_t* block_table,
                               const int32_t* prefix_lens, int32_t* new_lens, int Hkv, int D, int block_size,
                               int max_blocks_per_seq, int num_blocks, int dtype, void* stream) {
  if (B < 0 || T < 1 || V < 1) return SPEC_ERR_INVALID_ARG;
  if (top_k < 1 || top_k > kTruncTopKMax) return SPEC_ERR_UNSUPPORTED;
  if (!(top_p > 0.0f)) return SPEC_ERR_INVALID_ARG;  // also NaN
  RejectLaunch R;
  int rc = make_reject(target_logits, draft_probs, draft_tokens, parent, B, T, V, temperature, without_replacement,
                       seed, offset, accepted_nodes, out_tokens, num_accepted, status, workspace, workspace_bytes,
                       &R);
  if (rc != SPEC_OK) return rc;
  if (B > 0 && workspace_bytes < reject_trunc_workspace_bytes(B, T, V, top_k)) return SPEC_ERR_WORKSPACE;
  CompactLaunch C;
  if (k_cache != nullptr) {
    rc = make_compact(k_cache, v_cache, block_table, prefix_lens, new_lens, B, T, Hkv, D, block_size,
                      max_blocks_per_seq, num_blocks, dtype, status, &C);
    if (rc != SPEC_OK) return rc;
  }
  if (B == 0) return SPEC_OK;
  R.top_k = top_k;
  R.top_p = top_p;
  if (k_cache != nullptr) R.compact = &C;
  const hipError_t e = launch_reject(R, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int spec_tree_reject_compact_noalloc(const float* target_logits, const float* draft_probs,
                                     const int32_t* draft_tokens, const int32_t* parent, int B, int T, int V,
                                     float temperature, int without_replacement, uint64_t seed, uint64_t offset,
                                     int32_t* accepted_nodes, int32_t* out_tokens, int32_t* num_accepted,
                                     int32_t* status, void* k_cache, void* v_cache, const int32_t* block_table,
                                     const int32_t* prefix_lens, int32_t* new_lens, int Hkv, int D, int block_size,
                                     int max_blocks_per_seq, int num_blocks, int dtype, void* stream) {
  RejectLaunch R;
  int rc = make_reject(target_logits, draft_probs, draft_tokens, parent, B, T, V, temperature, without_replacement,
                       seed, offset, accepted_nodes, out_tokens, num_accepted, status, kStaticWorkspace,
                       reject_static_scratch_bytes(), &R);
  if (rc != SPEC_OK) return rc;
  CompactLaunch C;
  rc = make_compact(k_cache, v_cache, block_table, prefix_lens, new_lens, B, T, Hkv, D, block_size,
                    max_blocks_per_seq, num_blocks, dtype, status, &C);
  if (rc != SPEC_OK || B == 0) return rc;
  R.compact = &C;
  const hipError_t e = launch_reject_static(R, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int spec_tree_kv_write(const void* k_new, const void* v_new, void* q, void* k_cache, void* v_cache,
                       const int32_t* block_table, const int32_t* prefix_lens, const int32_t* parent,
                       int32_t* status, int B, int T, int Hq, int Hkv, int D, int block_size,
                       int max_blocks_per_seq, int num_blocks, float rope_theta, int dtype, void* stream) {
  const int rc = check_kv_shapes(B, T, Hkv, D, block_size, max_blocks_per_seq, num_blocks, dtype);
  if (rc != SPEC_OK) return rc;
  if (q != nullptr && (Hq < 1 || Hq % Hkv != 0)) return SPEC_ERR_INVALID_ARG;
  if (!(rope_theta >= 0.0f) || std::isinf(rope_theta)) return SPEC_ERR_INVALID_ARG;
  if (B == 0) return SPEC_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !prefix_lens || !parent) {
    return SPEC_ERR_INVALID_ARG;
  }
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return SPEC_ERR_INVALID_ARG;
  KvWriteLaunch L{};
  L.k_new = k_new;
  L.v_new = v_new;
  L.q = q;
  L.k_cache = k_cache;
  L.v_cache = v_cache;
  L.block_table = block_table;
  L.prefix_lens = prefix_lens;
  L.parent = parent;
  L.status = status;
  L.B = B;
  L.T = T;
  L.Hq = Hq;
  L.Hkv = Hkv;
  L.D = D;
  L.max_blocks = max_blocks_per_seq;
  L.num_blocks = num_blocks;
  L.bf16 = dtype == SPEC_BF16 ? 1 : 0;
  L.theta = rope_theta;
  const hipError_t e = launch_kv_write(L, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

size_t spec_tree_write_attn_workspace_size(int B, int T, int Hq, int Hkv, int D, int max_blocks_per_seq, int dtype) {
  if (B <= 0 || T < 1 || T > kMaxT || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || max_blocks_per_seq < 1 ||
      dtype != SPEC_BF16 || D != 128)
    return 0;
  return plan_attn_write(B, T, Hq, Hkv, max_blocks_per_seq).ws_bytes;
}

int spec_tree_write_attn(const void* k_new, const void* v_new, const void* q, void* k_cache, void* v_cache,
                         const int32_t* block_table, const int32_t* prefix_lens, const int32_t* parent, void* out,
                         int B, int T, int Hq, int Hkv, int D, int block_size, int max_blocks_per_seq, int num_blocks,
                         float rope_theta, float scale, int dtype, int32_t* status, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const int rc = check_kv_shapes(B, T, Hkv, D, block_size, max_blocks_per_seq, num_blocks, dtype);
  if (rc != SPEC_OK) return rc;
  if (dtype != SPEC_BF16) return SPEC_ERR_UNSUPPORTED;
  if (Hq < Hkv || Hq % Hkv != 0) return SPEC_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.0f) || !(rope_theta >= 0.0f) || std::isinf(rope_theta))
    return SPEC_ERR_INVALID_ARG;
  if (B == 0) return SPEC_OK;
  if (!k_new || !v_new || !q || !k_cache || !v_cache || !block_table || !prefix_lens || !parent || !out)
    return SPEC_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(out))
    return SPEC_ERR_INVALID_ARG;
  const AttnPlan plan = plan_attn_write(B, T, Hq, Hkv, max_blocks_per_seq);
  if (workspace == nullptr || workspace_bytes < plan.ws_bytes) return SPEC_ERR_WORKSPACE;
  AttnWriteLaunch W{};
  AttnLaunch& L = W.attn;
  L.q = q;
  L.k = k_cache;
  L.v = v_cache;
  L.block_table = block_table;
  L.prefix_lens = prefix_lens;
  L.parent = parent;
  L.out = out;
  L.status = status;
  L.workspace = workspace;
  L.B = B;
  L.T = T;
  L.Hq = Hq;
  L.Hkv = Hkv;
  L.D = D;
  L.max_blocks = max_blocks_per_seq;
  L.num_blocks = num_blocks;
  L.scale = scale;
  W.k_new = k_new;
  W.v_new = v_new;
  W.theta = rope_theta;
  const hipError_t e = launch_attn_write(plan, W, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int spec_tree_truncate(const float* logits_in, float* logits_out, int B, int T, int V, float temperature,
                       int top_k, float top_p, int32_t* status, void* stream) {
  if (B < 0 || T < 1 || V < 1) return SPEC_ERR_INVALID_ARG;
  if (V > (1 << 24)) return SPEC_ERR_UNSUPPORTED;
  if (!(temperature >= 0.0f) || std::isinf(temperature)) return SPEC_ERR_INVALID_ARG;
  if (!(top_p > 0.0f)) return SPEC_ERR_INVALID_ARG;  // also NaN
  if (B == 0) return SPEC_OK;
  if (!logits_in || !logits_out) return SPEC_ERR_INVALID_ARG;
  if (static_cast<long long>(B) * T > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  TruncateLaunch L{};
  L.in = logits_in;
  L.out = logits_out;
  L.status = status;
  L.B = B;
  L.T = T;
  L.V = V;
  L.temperature = temperature;
  L.top_k = top_k;
  L.top_p = top_p;
  const hipError_t e = launch_truncate(L, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // extern "C"
