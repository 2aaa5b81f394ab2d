/*
 * spectree.h — C ABI of the tree-verification hot path of tree-based
 * speculative decoding, for AMD Instinct MI355X (gfx950).
 *
 * Three calls, one per step of verifying a flattened draft tree in one target
 * pass:
 *   spec_tree_attn    tree-masked verify attention over a paged KV prefix
 *   spec_tree_reject  tree rejection sampling (greedy, with replacement,
 *                     or Sequoia-style without replacement)
 *   spec_kv_compact   keep only the accepted root-to-leaf path in the KV cache
 * and spec_tree_reject_compact, the last two in one launch; and, for the step
 * before them, spec_tree_kv_write (the tree's K/V rows into the paged cache,
 * keys and queries rotated for their tree positions), also fused with the
 * attention in one launch as spec_tree_write_attn; spec_tree_truncate
 * applies top-k / top-p to the target logits before the sampler.
 *
 * Conventions shared by every call
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing and is reentrant; the only state it keeps between
 *     calls is a per-device cache of one occupancy query (the sampler's).
 *   - Each call only enqueues work on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream).  No call synchronises or copies to the host,
 *     so a caller can chain draft and verify steps without a CPU round trip.
 *   - Shapes and pointers are checked on the host before anything is launched;
 *     a failed check returns a negative spec_status and launches nothing.
 *     Queries, keys, values (new rows and caches) and attention outputs must
 *     start on a 16-byte boundary (they move with 16-byte accesses); a pointer
 *     that does not is SPEC_ERR_INVALID_ARG.
 *   - Device contents that the host cannot see without a copy (the parent
 *     array, block-table entries, prefix lengths, draft tokens, NaN logits,
 *     accepted paths) are checked by the kernels.  A kernel that finds a bad
 *     value never reads or writes out of bounds; it ORs a SPEC_DEV_* bit into
 *     `status[b]` (when `status` is not NULL) and writes a defined result for
 *     that sequence (documented per call).  `status` must be zero-filled by
 *     the caller before the first call that should report into it.
 *   - Draft tree: T nodes flattened in topological order.  Node 0 is the root
 *     (the last committed token); parent[b][0] = -1 and 0 <= parent[b][i] < i.
 *     Node i may attend to tree node j iff j is i or an ancestor of i (the
 *     tree_mask of "Report: Support nextn speculative decoding", EAGLE
 *     implementation summary, step 3).
 *   - Paged KV cache: [num_blocks, Hkv, block_size, D] for K and for V, with
 *     block_size = 16.  Logical position t of sequence b lives at
 *     cache[block_table[b][t / 16]][kv_head][t % 16][:].  Tree node i's K/V row
 *     is at logical position prefix_lens[b] + i, written by the caller before
 *     spec_tree_attn (with its rotary position prefix_lens[b] + depth(i)), for
 *     instance with spec_tree_kv_write.
 */
#ifndef SPECTREE_H
#define SPECTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPEC_OK = 0,
  SPEC_ERR_INVALID_ARG = -1, /* null pointer, non-positive or inconsistent size */
  SPEC_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype, D, block size, T > 512) */
  SPEC_ERR_WORKSPACE = -3,   /* workspace pointer NULL or smaller than the *_workspace_size */
  SPEC_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} spec_status;

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* Device-detected input errors, OR-ed into status[b]. */
enum {
  SPEC_DEV_PARENT = 1,     /* parent[b] is not a topological parent array */
  SPEC_DEV_BLOCK = 2,      /* a needed block_table entry is outside [0, num_blocks) */
  SPEC_DEV_LENGTH = 4,     /* prefix_lens[b] < 0 or prefix_lens[b] + T > max_blocks_per_seq * 16 */
  SPEC_DEV_TOKEN = 8,      /* a draft token outside [0, V) */
  SPEC_DEV_NONFINITE = 16, /* NaN/Inf in a target-logit row or a draft probability that was read */
  SPEC_DEV_EMPTY = 32,     /* a distribution with zero total mass had to be sampled */
  SPEC_DEV_PATH = 64,      /* accepted path not of the form 0 = n_0 < n_1 < ... < n_L < T */
  SPEC_DEV_TIMEOUT = 128   /* a bounded wait between the workgroups sampling one sequence
                              expired (other work held the CUs); the sequence gets the
                              error outputs of spec_tree_reject */
};

/* Human-readable name of a spec_status value. */
const char* spec_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int spec_version(void);

/* ------------------------------------------------------------------------
 * spec_tree_attn — tree-masked verify attention.
 *
 * For every sequence b, tree node i and query head h (kv head g = h / (Hq/Hkv)):
 *   keys K(i) = prefix positions 0 .. prefix_lens[b]-1, plus positions
 *               prefix_lens[b] + j for every ancestor-or-self j of i;
 *   out[b,i,h,:] = softmax_t(scale * <q[b,i,h,:], k_t>) . v_t  over t in K(i).
 * This is the multi-query paged attention used to score all drafted tokens in
 * one pass (vLLM PR "[WIP] Speculative decoding using a draft model", future
 * work list; EAGLE report, step 3: attention is skipped for unrelated draft
 * tokens).  Accumulation is fp32; bf16 inputs use bf16 matrix-core products.
 *
 *   q            [B, T, Hq, D] dtype, contiguous
 *   k_cache      [num_blocks, Hkv, 16, D] dtype
 *   v_cache      [num_blocks, Hkv, 16, D] dtype
 *   block_table  [B, max_blocks_per_seq] int32; must cover prefix_lens[b] + T
 *   prefix_lens  [B] int32, >= 0
 *   parent       [B, T] int32
 *   out          [B, T, Hq, D] dtype (written)
 *   scale        softmax scale, finite and > 0 (callers normally pass 1/sqrt(D))
 *   status       [B] int32 or NULL; on a device-detected error the rows of the
 *                affected sequence are still written, from the subset of keys
 *                that could be read safely
 *   workspace    device scratch of at least spec_tree_attn_workspace_size(...)
 *                bytes (may be NULL when that size is 0).  When the KV range
 *                is split over several workgroups, the first bytes hold one
 *                arrival counter per (sequence, kv head, block of query rows),
 *                which must be zero before the first call; every call that
 *                completes leaves them zero, so for one shape a workspace is
 *                zero-filled once and then reused.  The rest holds the splits'
 *                partial results.  Where the counters end depends on (B, T,
 *                Hq, Hkv, max_blocks_per_seq): zero-fill the workspace again
 *                before a call with another shape (or keep one per shape).
 *                Calls that overlap in time must not share a workspace.
 * Supported: dtype SPEC_BF16 with D = 128, dtype SPEC_F32 with D in {64, 128};
 * block_size = 16; 1 <= T <= 512; Hq % Hkv == 0.  B == 0 is a no-op.
 * ---------------------------------------------------------------------- */
size_t spec_tree_attn_workspace_size(int B, int T, int Hq, int Hkv, int D,
                                     int max_blocks_per_seq, int dtype);

int spec_tree_attn(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* prefix_lens,
                   const int32_t* parent, void* out,
                   int B, int T, int Hq, int Hkv, int D, int block_size,
                   int max_blocks_per_seq, int num_blocks, float scale, int dtype,
                   int32_t* status, void* workspace, size_t workspace_bytes,
                   void* stream);

/* ------------------------------------------------------------------------
 * spec_tree_reject — tree rejection sampling.
 *
 * Per sequence, walk the tree from the root.  At the current node u, with
 * p = softmax(target_logits[b,u,:] / temperature) and q = draft_probs[b,u,:]:
 * try the children c of u in increasing index order with x = draft_tokens[b,c]
 * and a uniform r: accept iff r * q(x) < p(x) ("Speculative Decoding" notes,
 * "Draft Token Validation": accept when p >= q, else with probability p/q).
 * After each rejected child p becomes max(p - q, 0) renormalised (left as is if
 * that mass is 0); with without_replacement != 0, q also loses x and is
 * renormalised (Sequoia summary, "Robust Sampling").  An accepted child becomes
 * the current node.  When the current node has no untried child left, one
 * token is drawn from the current p by inverse CDF in vocabulary order (the
 * residual token, or the bonus token after a fully accepted branch).
 * temperature == 0 is greedy: accept the first child whose token equals the
 * argmax of the target logits (lowest index on ties), else emit that argmax.
 *
 * Randomness: Philox4x32-10 (Salmon et al., SC'11) with key = (seed lo, seed
 * hi) and counter = (node, b, purpose + 2*(offset >> 32), offset lo), purpose
 * 0 for the accept test of child `node`, 1 for the final draw at `node`;
 * uniform = (word0 >> 8) * 2^-24.  A draw depends only on (seed, offset, b,
 * node, purpose).  Decisions are taken in fp64 from the fp32 inputs.
 *
 *   target_logits [B, T, V] float32; row u = logits of the token after node u
 *   draft_probs   [B, T, V] float32; row u = draft distribution the children
 *                 of u were drafted from, used as given (not renormalised)
 *   draft_tokens  [B, T] int32; token of node i (entry 0 ignored)
 *   parent        [B, T] int32
 *   accepted_nodes[B, T] int32 out: n_0 = 0, n_1 .. n_L, then -1
 *   out_tokens    [B, T] int32 out: tokens of n_1 .. n_L, the drawn token, then -1
 *   num_accepted  [B] int32 out: L
 *   status        [B] int32 or NULL; on a device-detected error the sequence
 *                 gets L = 0, accepted_nodes = [0, -1, ...], out_tokens all -1
 *   workspace     >= spec_tree_reject_workspace_size(B, T, V) bytes, all of it
 *                 zero before the first call.  Its first 256 bytes hold the
 *                 grid's exit counter and a call epoch; the rest holds the
 *                 exchange slots, each tagged with the epoch of the call that
 *                 wrote it, so a slot is only ever read by that call.  Every
 *                 call that completes leaves the workspace ready for the next
 *                 call of any shape it is large enough for: zero-fill it once,
 *                 then reuse it.  Calls that overlap in time must not share a
 *                 workspace.
 * Execution: each sequence is sampled by a team of up to 64 cooperating
 * workgroups that exchange partial sums through the workspace.  Before the
 * launch the team is sized so that the whole grid (B x team size) fits on the
 * device at once (spec_tree_reject_plan with spec_tree_reject_max_resident);
 * when not even two members per sequence fit, each sequence gets one
 * workgroup, which waits for nobody.  Waits are bounded; a wait can run out
 * only if other work holds the device's CUs for the whole bound, and then the
 * sequence reports SPEC_DEV_TIMEOUT with the error outputs below.  Member 0
 * of a team alone writes the sequence's outputs (and, in
 * spec_tree_reject_compact, moves its KV rows), so they are always one
 * consistent result.
 * Supported: 1 <= T <= 512, 1 <= V <= 262144, temperature >= 0 and finite.
 * ---------------------------------------------------------------------- */
size_t spec_tree_reject_workspace_size(int B, int T, int V);

/* Team plan of spec_tree_reject on a device that holds
 * `max_resident_workgroups` of its workgroups at once: the number of
 * workgroups per sequence (*team_size) and the vocabulary entries each owns
 * (*slice_len).  B * *team_size <= max_resident_workgroups whenever
 * *team_size > 1.  Host only; no GPU needed.  Returns SPEC_OK, or
 * SPEC_ERR_INVALID_ARG / SPEC_ERR_UNSUPPORTED as spec_tree_reject would. */
int spec_tree_reject_plan(int B, int T, int V, int64_t max_resident_workgroups, int* team_size, int* slice_len);

/* Workgroups of the sampler kernel the current HIP device holds at once (its
 * occupancy per CU times the CU count), as used by spec_tree_reject; 0 if the
 * device cannot be queried. */
int64_t spec_tree_reject_max_resident(void);

int spec_tree_reject(const float* target_logits, const float* draft_probs,
                     const int32_t* draft_tokens, const int32_t* parent,
                     int B, int T, int V, float temperature, int without_replacement,
                     uint64_t seed, uint64_t offset,
                     int32_t* accepted_nodes, int32_t* out_tokens, int32_t* num_accepted,
                     int32_t* status, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ------------------------------------------------------------------------
 * spec_kv_compact — selective KV-cache compaction (in place).
 *
 * For d = 1 .. L (L = num_accepted[b], path n_d = accepted_nodes[b][d]) and
 * every kv head, the K and V rows at logical position prefix_lens[b] + n_d are
 * moved to prefix_lens[b] + d, with the result of doing so in increasing d
 * (a destination that is also a later source is read before it is written).
 * Nothing else is written; slots past the new length keep stale data (the
 * rejected tokens' KV is evicted: EAGLE report, "Important Implementation
 * Detail"; SGLang doc, "Prefix Match").  new_lens[b] = prefix_lens[b] + L + 1.
 *
 *   k_cache, v_cache [num_blocks, Hkv, 16, D] dtype, modified in place
 *   block_table, prefix_lens as for spec_tree_attn
 *   accepted_nodes [B, T] int32, num_accepted [B] int32 (spec_tree_reject's output)
 *   new_lens       [B] int32 out, or NULL
 *   status         [B] int32 or NULL; a sequence with a bad path or table is
 *                  left untouched and new_lens[b] = prefix_lens[b]
 * Supported: as spec_tree_attn.  Sequences must not share blocks.
 * ---------------------------------------------------------------------- */
int spec_kv_compact(void* k_cache, void* v_cache, const int32_t* block_table,
                    const int32_t* prefix_lens, const int32_t* accepted_nodes,
                    const int32_t* num_accepted, int32_t* new_lens,
                    int B, int T, int Hkv, int D, int block_size,
                    int max_blocks_per_seq, int num_blocks, int dtype,
                    int32_t* status, void* stream);

/* ----------------------------------------------------------------------
 * spec_tree_reject_compact — spec_tree_reject followed by spec_kv_compact
 * along the path it accepted, in one launch.
 *
 * The vLLM PR ("[WIP] Speculative decoding using a draft model", guide for
 * reviewers) asks that the verifier and the cache update run without a host
 * round trip between them; here they also share one kernel: once a team has
 * walked a sequence's tree, its workgroups move the accepted rows of the kv
 * heads they own, from the path they already hold.  Every output equals that of
 * calling spec_tree_reject and then spec_kv_compact on its accepted_nodes and
 * num_accepted (after a sampler error, L = 0: the cache is left as it is and
 * new_lens[b] = prefix_lens[b] + 1).
 *
 *   the first 17 arguments  as for spec_tree_reject
 *   k_cache .. num_blocks, dtype  as for spec_kv_compact (T is the sampler's)
 *   status  receives both kernels' device error bits
 * Supported: as spec_tree_reject and spec_kv_compact together.
 * ---------------------------------------------------------------------- */
int spec_tree_reject_compact(const float* target_logits, const float* draft_probs,
                             const int32_t* draft_tokens, const int32_t* parent,
                             int B, int T, int V, float temperature, int without_replacement,
                             uint64_t seed, uint64_t offset,
                             int32_t* accepted_nodes, int32_t* out_tokens, int32_t* num_accepted,
                             int32_t* status, void* workspace, size_t workspace_bytes,
                             void* k_cache, void* v_cache, const int32_t* block_table,
                             const int32_t* prefix_lens, int32_t* new_lens,
                             int Hkv, int D, int block_size, int max_blocks_per_seq,
                             int num_blocks, int dtype, void* stream);

/* ----------------------------------------------------------------------
 * spec_tree_reject_compact_noalloc — spec_tree_reject_compact without a
 * caller-supplied workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The call itself allocates nothing: the sampler's workspace is
 * a static device array of the library, 8 MiB per GPU (one copy on every GPU
 * the library runs on, held until the process ends), zero-filled at load.
 *
 *   arguments  as for spec_tree_reject_compact, without workspace and
 *              workspace_bytes; the caller still passes every input and output
 *   returns    SPEC_ERR_WORKSPACE when spec_tree_reject_workspace_size(B, T, V)
 *              exceeds 8 MiB (e.g. B * team size * (2T + 10) * 32 bytes past
 *              that); otherwise as spec_tree_reject_compact
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents; each completed call leaves it ready for the next call of any
 * shape.  Calls that overlap in time on one GPU (several streams or threads)
 * race on it and must not be issued.
 * ---------------------------------------------------------------------- */
int spec_tree_reject_compact_noalloc(const float* target_logits, const float* draft_probs,
                                     const int32_t* draft_tokens, const int32_t* parent,
                                     int B, int T, int V, float temperature, int without_replacement,
                                     uint64_t seed, uint64_t offset,
                                     int32_t* accepted_nodes, int32_t* out_tokens, int32_t* num_accepted,
                                     int32_t* status, void* k_cache, void* v_cache,
                                     const int32_t* block_table, const int32_t* prefix_lens,
                                     int32_t* new_lens, int Hkv, int D, int block_size,
                                     int max_blocks_per_seq, int num_blocks, int dtype, void* stream);

/* ----------------------------------------------------------------------
 * spec_tree_kv_write — the step before verify attention: write every tree
 * node's K and V rows into the paged cache, the key (and, if given, the
 * queries, in place) rotated for the node's position.
 *
 * Node i of sequence b is at position prefix_lens[b] + depth(i): the tree is
 * scored in one flattened pass ("Report: Support nextn speculative decoding",
 * implementation summary, step 3), each token at the position it would have
 * along its own path (the position_ids of "Issue: Speculative Decoding on
 * vLLM").  Its rows go to logical slot prefix_lens[b] + i, where
 * spec_tree_attn reads them.  Rotation: RoFormer's rotary position embedding
 * in the half-split layout -- for j < D/2 the pair (x_j, x_{j+D/2}) at position
 * p turns by p * rope_theta^(-2j/D) (angles in fp64) -- or none when
 * rope_theta == 0.  V rows are copied bit for bit.
 *
 *   k_new, v_new [B, T, Hkv, D] dtype: the nodes' keys (before rotation) and values
 *   q            [B, T, Hq, D] dtype, rotated in place, or NULL
 *   k_cache, v_cache, block_table, prefix_lens, parent  as for spec_tree_attn;
 *                the caches are written at the T slots of each sequence only
 *   status       [B] int32 or NULL; a bad parent row or prefix length leaves
 *                the sequence unwritten, a bad block index skips that slot's rows
 *   rope_theta   >= 0 and finite (10000 for Llama-2 layers, 500000 for Llama-3)
 * Supported: as spec_tree_attn; Hq % Hkv == 0 when q is given.
 * ---------------------------------------------------------------------- */
int spec_tree_kv_write(const void* k_new, const void* v_new, void* q, void* k_cache, void* v_cache,
                       const int32_t* block_table, const int32_t* prefix_lens, const int32_t* parent,
                       int32_t* status, int B, int T, int Hq, int Hkv, int D, int block_size,
                       int max_blocks_per_seq, int num_blocks, float rope_theta, int dtype, void* stream);

/* ----------------------------------------------------------------------
 * spec_tree_write_attn — spec_tree_kv_write and spec_tree_attn in one launch:
 * the step before verify attention (the tree's K/V rows into the paged cache,
 * keys and queries rotated for the nodes' positions prefix_lens[b] +
 * depth(i); "Report: Support nextn speculative decoding", implementation
 * summary, step 3, and the position_ids of "Issue: Speculative Decoding on
 * vLLM") fused with the tree attention over the prefix and the tree.
 *
 * Writes the same cache rows, bit for bit, as spec_tree_kv_write, and the same
 * `out` as spec_tree_attn called after it on the queries it rotated (bit for
 * bit except on the batched launch below, whose KV splits fall elsewhere, so
 * its outputs differ by the bf16 rounding of the probabilities).  The
 * caller's `q` is not modified.  With at most 16 query rows per kv head (the
 * streaming kernel) it is one launch: every work item rotates its own queries,
 * and an item whose KV range holds tree keys first writes its kv head's T key
 * and value rows.  On a ragged batch of up to 64 sequences with at most 64
 * query rows per kv head and more work items than the device holds at once
 * (batched serving), the write also runs inside the attention launch: its
 * first work items write the tree's K/V rows of one sequence 64 rows at a
 * time and count them, the attention items rotate their own queries, and an
 * item that reads the tree's keys starts once its sequence's rows are all
 * written (work items are claimed from a counter in the workspace, writers
 * first, so this wait always ends).  Every other shape takes two launches,
 * which measured faster there: the write, with the rotated queries going to
 * the workspace, then the attention.
 *
 *   k_new, v_new [B, T, Hkv, D] bf16: the nodes' keys (before rotation) and values
 *   q            [B, T, Hq, D] bf16: the queries before rotation (read only)
 *   k_cache, v_cache, block_table, prefix_lens, parent, out, scale, status
 *                as for spec_tree_attn; the caches are written at the T slots
 *                of each sequence only
 *   rope_theta   >= 0 and finite; 0 writes and uses the rows unrotated
 *   workspace    >= spec_tree_write_attn_workspace_size(...) bytes, never
 *                NULL (the work counter, B counts of written rows and the
 *                split partials; spec_tree_attn's workspace on the streaming
 *                launch; or the rotated queries and spec_tree_attn's
 *                workspace), zero-filled before the first call;
 *                each completed call leaves its counters zero, so a workspace
 *                serves later calls of the same shape as it is (re-zero it
 *                when the shape changes, as for spec_tree_attn)
 * Errors: a bad parent row or prefix length writes no cache row of that
 * sequence (status reports it; that sequence's outputs are then not
 * meaningful, the other sequences' are exact); a bad block index skips that
 * slot (SPEC_DEV_BLOCK).
 * Supported: bf16, D = 128, block_size = 16, 1 <= T <= 512, Hq % Hkv == 0.
 * ---------------------------------------------------------------------- */
size_t spec_tree_write_attn_workspace_size(int B, int T, int Hq, int Hkv, int D, int max_blocks_per_seq,
                                           int dtype);
int spec_tree_write_attn(const void* k_new, const void* v_new, const void* q, void* k_cache, void* v_cache,
                         const int32_t* block_table, const int32_t* prefix_lens, const int32_t* parent, void* out,
                         int B, int T, int Hq, int Hkv, int D, int block_size, int max_blocks_per_seq,
                         int num_blocks, float rope_theta, float scale, int dtype, int32_t* status,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * spec_tree_truncate — top-k / top-p truncation of the target logits, for a
 * sampler that verifies against a truncated target (the Sequoia summary,
 * "Sequoia: Scalable and Robust Speculative Decoding", robustness to the top-p
 * hyperparameter).  Run it on target_logits before spec_tree_reject.
 *
 * Every row (b, u) keeps {x : logit >= t} and sets the other entries to -inf,
 * so the sampler gives them probability 0 in every acceptance test, residual
 * and final draw.  t is the k-th largest finite logit for top-k (Fan et al.
 * 2018) and, for top-p (Holtzman et al. 2020), the largest logit value v such
 * that {logit >= v} holds at least top_p of softmax(logits / temperature);
 * equal logits are never split.  Both rules: top-k first, then top-p over the
 * top-k set renormalised.  Temperature 0: top-p keeps the logits tied at the
 * maximum.  The top-p masses are fp32 exponentials summed in fp64 (about 1e-7
 * relative): a top_p within that distance of a cumulative mass may keep one
 * group of equal logits more or fewer than exact arithmetic would.
 *
 *   logits_in    [B, T, V] float32
 *   logits_out   [B, T, V] float32: == logits_in for in place (only dropped
 *                entries are written), else disjoint from it (every entry
 *                written)
 *   temperature  >= 0 and finite, the sampler's
 *   top_k        <= 0: off; >= the row's count of finite logits keeps them all
 *   top_p        > 0; >= 1: off
 *   status       [B] int32 or NULL; a row holding NaN or +inf gets
 *                SPEC_DEV_NONFINITE and is left as it is (copied when out of place)
 * Supported: any B, T >= 1, 1 <= V <= 2^24.  Caller-side -inf entries count as
 * dropped already.
 * ---------------------------------------------------------------------- */
int spec_tree_truncate(const float* logits_in, float* logits_out, int B, int T, int V,
                       float temperature, int top_k, float top_p, int32_t* status, void* stream);

/* ----------------------------------------------------------------------
 * spec_tree_reject_truncated — spec_tree_reject against the target truncated
 * to top_k then top_p (the rules of spec_tree_truncate), with the truncation
 * taken inside the sampler and only for the rows its walk visits, and
 * optionally the compaction of spec_tree_reject_compact in the same launch.
 * The Sequoia summary ("Sequoia: Scalable and Robust Speculative Decoding",
 * the top-p robustness table) verifies against a nucleus-truncated target;
 * nothing is written back to target_logits.
 *
 * Results equal those of spec_tree_truncate followed by spec_tree_reject
 * (or spec_tree_reject_compact), except that the top-p masses here are fp64
 * exponentials: a top_p within about 1e-15 relative of a cumulative mass may
 * keep one group of equal logits more or fewer than exact arithmetic would.
 * Each team member lists the largest values of its slice of a visited row;
 * the members exchange the lists through the workspace (a second exchange,
 * with K values each, when one slice held more of the row's top values than
 * its first list) and every member finds the same threshold from them.
 *
 *   the first 7 arguments, temperature, without_replacement, seed, offset and
 *     the outputs up to status  as for spec_tree_reject
 *   top_k        1 .. 64 (>= the row's count of finite logits keeps them all)
 *   top_p        > 0; >= 1: top-k only
 *   workspace    >= spec_tree_reject_truncated_workspace_size(B, T, V, top_k)
 *                bytes, zero before the first call, reusable as for
 *                spec_tree_reject (the same epoch-tagged layout, with the
 *                members' lists after the slots)
 *   k_cache      NULL: no compaction (the arguments up to dtype are ignored);
 *                otherwise k_cache .. dtype as for spec_tree_reject_compact
 * temperature == 0 is greedy, which truncation does not change (the argmax is
 * always kept).  Returns SPEC_ERR_UNSUPPORTED for top_k outside 1 .. 64 (use
 * spec_tree_truncate, then spec_tree_reject), SPEC_ERR_INVALID_ARG for top_p
 * <= 0 or NaN, otherwise as spec_tree_reject (and spec_kv_compact).
 * ---------------------------------------------------------------------- */
size_t spec_tree_reject_truncated_workspace_size(int B, int T, int V, int top_k);

/* Team plan of spec_tree_reject_truncated (as spec_tree_reject_plan) and the
 * length of the members' first lists (<= top_k).  Host only. */
int spec_tree_reject_truncated_plan(int B, int T, int V, int top_k, int64_t max_resident_workgroups,
                                    int* team_size, int* list_len);

int spec_tree_reject_truncated(const float* target_logits, const float* draft_probs,
                               const int32_t* draft_tokens, const int32_t* parent,
                               int B, int T, int V, float temperature, int top_k, float top_p,
                               int without_replacement, uint64_t seed, uint64_t offset,
                               int32_t* accepted_nodes, int32_t* out_tokens, int32_t* num_accepted,
                               int32_t* status, void* workspace, size_t workspace_bytes,
                               void* k_cache, void* v_cache, const int32_t* block_table,
                               const int32_t* prefix_lens, int32_t* new_lens,
                               int Hkv, int D, int block_size, int max_blocks_per_seq,
                               int num_blocks, int dtype, void* stream);

/* ----------------------------------------------------------------------
 * spec_sequoia_tree — Sequoia's tree construction: the draft-tree shape of n
 * nodes and depth <= max_depth that maximises the expected number of tokens
 * one verification step generates ("Sequoia: Scalable and Robust Speculative
 * Decoding" summary, "Scalable Speculative Decoding", "Dynamic Programming";
 * the objective and the dynamic program are those of the published Sequoia
 * paper).  Positional acceptance: the k-th child of an accepted node, in the
 * order the verifier tries siblings, is the one accepted with probability
 * accept[k-1] (0 past the vector), whatever the node; a node is accepted with
 * the product of those probabilities along its path, and the tree generates
 * their sum (root: 1) tokens in expectation.  Host code: runs on the CPU, no
 * GPU needed; every pointer is a HOST pointer.
 *
 *   accept    [K] double in [0, 1] (measured per-rank acceptance; K may be 0)
 *   n         tree size, 1 <= n <= 4096
 *   max_depth deepest node's depth in edges from the root (>= 1 when n > 1)
 *   parent    [n] int32 out: parent array numbered breadth first, siblings in
 *             rank order (parent[0] = -1, parent[i] < i), ready for the other
 *             calls' `parent` argument
 *   expected  out (nullable): the optimum's expected tokens per step
 * Returns SPEC_OK; SPEC_ERR_INVALID_ARG for a bad argument or no feasible
 * tree; SPEC_ERR_UNSUPPORTED when n > 4096 or the tables (about
 * min(max_depth, n-1) * (min(K, n-1) + 2) * n entries) pass 16 Mi entries.
 * ---------------------------------------------------------------------- */
int spec_sequoia_tree(const double* accept, int K, int n, int max_depth, int32_t* parent, double* expected);

#ifdef __cplusplus
}
#endif

#endif /* SPECTREE_H */
