/*
 * tav.h — tree-attention verification on AMD MI355X (gfx950).
 *
 * C ABI of the verification step of tree-based speculative decoding:
 *   tree_mask_build     parent[] -> packed ancestor-or-self bitmasks
 *   tree_attn_verify    tree attention over a paged KV prefix plus ancestors
 *   tree_attn_verify_tree  the same from parent[] (mask built in the launch)
 *   spec_verify_sample  target/draft softmax and the rejection-sampling walk
 *   spec_verify_sample_wor  the same walk for siblings drawn without replacement
 *   spec_verify_sample_probe  the walk, also writing the p and q it decides with
 *   spec_verify_sample_noalloc  the walk on the library's fixed scratch (no workspace)
 *   spec_verify_sample_commit  the walk and kv_commit_path in one launch
 *   kv_commit_path      copy the accepted path's K/V into the paged cache
 *   kv_commit_inplace   the same when the tree's K/V already sit in the cache
 *   tree_expand_topk    top-k draft tokens, log q and entropy per frontier row
 *   tree_expand_sample  the same with the k tokens drawn without replacement
 *   tree_select_topm    the budget's best M-node subtree of a candidate tree
 *   tree_widths_by_entropy  branching widths from the frontier's entropy ranks
 *   tree_topology_dp    the budget's best topology under acceptance by sibling rank
 *   tav_sampler_plan    how the walk lays out a batch on the device
 *   tav_sampler_plan_for  the same rule for a given device shape (host only)
 *   tav_model_speedup, tav_best_chain_length, tav_fit_alpha
 *                       the speedup model, on the host, fed by measured times
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless stated otherwise. All tensors are
 *     owned by the caller; the library keeps no pointer after a call returns
 *     and holds no mutable global state, except the fixed per-device scratch
 *     of spec_verify_sample_noalloc. Buffers must stay alive until the work
 *     queued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call is asynchronous; the four calls chain on one stream with no
 *     host synchronisation.
 *   - The return value reports host-checkable argument errors only; nothing
 *     is launched when it is not TAV_OK. Faults found in device data (a bad
 *     tree, a bad block-table entry, non-finite logits) are OR-ed into
 *     `*dev_flags` (a device uint32 the caller zeroes and reads when it
 *     chooses; may be NULL to ignore them). Kernels never trap; outputs are
 *     unspecified for a sequence whose data raised a flag.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Tree nodes are numbered topologically: node 0 is the root
 *     (parent -1) and 0 <= parent[i] < i for i >= 1. 1 <= N <= 256.
 *   - Paged KV: 16-token blocks. K cache [num_blocks][Hkv][16][D]
 *     (token-major), V cache [num_blocks][Hkv][D][16] (feature-major).
 *     block_table[b][j] is the physical block of logical block j of sequence b
 *     (token position pos lives in block block_table[b][pos/16], slot pos%16).
 */
#ifndef TAV_H
#define TAV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tav_status;

#define TAV_OK 0
#define TAV_ERR_ARG 1          /* null or misaligned pointer, size out of range */
#define TAV_ERR_UNSUPPORTED 2  /* valid but unsupported shape (D, block size, N, ...) */
#define TAV_ERR_WORKSPACE 3    /* workspace missing or smaller than required */
#define TAV_ERR_LAUNCH 4       /* the HIP runtime refused a launch */

/* Bits OR-ed into *dev_flags by the kernels. */
#define TAV_FLAG_BAD_PARENT 0x1u        /* parent[] is not a rooted topological tree */
#define TAV_FLAG_BAD_BLOCK 0x2u         /* block-table entry outside [0, num_blocks) */
#define TAV_FLAG_NONFINITE_LOGITS 0x4u  /* NaN logit, or a row with no finite logit */
#define TAV_FLAG_CAPACITY 0x8u          /* prefix/commit beyond max_prefix_len or the table */
#define TAV_FLAG_BAD_TOKEN 0x10u        /* token[b][i] outside [0, V) for i >= 1 */
#define TAV_FLAG_SYNC_TIMEOUT 0x20u     /* a bounded inter-workgroup wait ran out */
#define TAV_FLAG_ATTN_RANGE 0x40u       /* an attention output is not finite (a V entry of
                                           magnitude >= 65520, or a non-finite input) */

#define TAV_ABI_VERSION 1

/* Version of this ABI (TAV_ABI_VERSION of the library that was built). */
int32_t tav_abi_version(void);

/* Static text naming a status code. */
const char *tav_status_string(tav_status status);

/*
 * tree_mask_build — ancestor-or-self masks of a batch of candidate trees.
 *
 * Defined by the jisaku.com glossary ("tree-based speculative decoding",
 * tree-attention section: M[i][j] = 1 exactly when node j is node i or one of
 * its ancestors) with the 5-node instance printed in the radar-34b blog §3
 * (Tree Attention Verification Matrix).
 *
 *   parent  int32 [B][N]        parent of each node (-1 for node 0)
 *   mask    uint64 [B][N][W]    out, W = ceil(N/64); bit j%64 of word j/64 of
 *                               row i is M[i][j]; unused bits are zero
 *   depth   int32 [B][N]        out, nullable; number of proper ancestors
 *   B >= 1, 1 <= N <= 256. mask must be 8-byte aligned.
 *   Sets TAV_FLAG_BAD_PARENT for a tree that breaks the numbering rule.
 */
tav_status tree_mask_build(const int32_t *parent, int32_t B, int32_t N, uint64_t *mask,
                           int32_t *depth, uint32_t *dev_flags, void *stream);

/*
 * tree_attn_workspace_bytes — device workspace tree_attn_verify needs for
 * these sizes on the current device (may be 0). Returns 0 for sizes that
 * tree_attn_verify would reject.
 */
size_t tree_attn_workspace_bytes(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t max_prefix_len);

/*
 * tav_attn_plan — how tree_attn_verify divides the work for these sizes on a
 * device of `cus` compute units holding `per_cu` of its workgroups each. A
 * host function (nothing launched, no device needed), for checking the plan:
 *   plan[0] waves per workgroup: 8 in both forms, eight row waves of 32
 *   query rows (row blocks of 256 rows), or four row waves in two sets that
 *   split each tile's keys (row blocks of 128 rows; taken up to 128 rows per
 *   KV head, and above that where the first form's plan is dominated by
 *   prefix splits),
 *   plan[1] row blocks per (sequence, KV head), plan[2] prefix splits,
 *   plan[3] the most block-table entries any split stages, over every prefix
 *   length up to max_prefix_len, plan[4] the capacity of that staging copy
 *   (plan[3] <= plan[4] for every supported shape).
 * TAV_ERR_ARG for a NULL plan or cus, per_cu < 1; TAV_ERR_UNSUPPORTED for
 * sizes tree_attn_verify rejects.
 */
tav_status tav_attn_plan(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t max_prefix_len, int32_t cus, int32_t per_cu, int32_t *plan);

/*
 * tav_sampler_plan — how spec_verify_sample and its variants lay out B
 * sequences of vocabulary V on the current device (a host call that reads
 * the device's CU count and the kernels' occupancy; nothing launched).
 * greedy: 0 the sampling walks (temperature > 0), 1 greedy verification.
 *   plan[0] vocabulary entries per thread: 4, 8 or 16 (held in registers) or
 *           28 (16 in registers, 12 in LDS); 28 only where it cuts the
 *           sequences per group by more than a third (a sequence costs about
 *           1.5 times as much with it), else the fewest sequences per group,
 *           the smallest among equals;
 *   plan[1] workgroups per sequence (a group), ceil(V / (512 plan[0]));
 *   plan[2] groups walking at once, each taking sequences g, g + plan[2],
 *           ... in turn (ceil(B / plan[2]) of them);
 *   plan[3] vocabulary entries per workgroup.
 * TAV_ERR_ARG for a NULL plan, B < 1, V < 1 or greedy outside {0, 1};
 * TAV_ERR_UNSUPPORTED for V > 2^21; TAV_ERR_LAUNCH if no plan fits the
 * device (or there is none).
 */
tav_status tav_sampler_plan(int32_t B, int32_t V, int32_t greedy, int32_t *plan);

/*
 * tav_sampler_plan_for — the same layout rule on a device of `cus` compute
 * units holding per_cu[i] workgroups of each walk kernel at once (per_cu[0..3]
 * the sampling walk with 4, 8, 16 and 28 entries per thread, per_cu[4] greedy
 * verification; host arithmetic only, nothing queried or launched), so the
 * rule can be checked without a device. plan as for tav_sampler_plan.
 * TAV_ERR_ARG for a NULL pointer, B < 1, V < 1, cus < 1, a negative per_cu
 * entry or greedy outside {0, 1}; TAV_ERR_UNSUPPORTED for V > 2^21;
 * TAV_ERR_LAUNCH if no layout fits.
 */
tav_status tav_sampler_plan_for(int32_t B, int32_t V, int32_t greedy, int32_t cus,
                                const int32_t *per_cu, int32_t *plan);

/*
 * tree_attn_verify — one attention layer of the verification forward pass.
 *
 * The target scores all candidates in one pass over the prefix with the
 * candidates appended (LLM Primer ch. 9, §9.1); each candidate attends only
 * along its root-to-node path (jisaku.com glossary, tree-attention section;
 * radar-34b blog §3); the prefix is read from a paged cache through a block
 * table (radar-34b blog §5; jisaku.com glossary, KV-cache section).
 *
 * For sequence b, query head h (KV head h / (Hq/Hkv)) and node i:
 *   keys = prefix positions [0, prefix_len[b]) and tree nodes j with bit j of
 *          mask[b][i] set;
 *   out[b][i][h] = softmax(scale * q·k over keys) · v, in fp32.
 *
 *   q              bf16 [B][N][Hq][D]
 *   k_tree,v_tree  bf16 [B][N][Hkv][D]    K/V of the tree nodes themselves
 *   k_cache        bf16 [num_blocks][Hkv][16][D]
 *   v_cache        bf16 [num_blocks][Hkv][D][16]
 *   block_table    int32 [B][max_blocks]
 *   prefix_len     int32 [B], each in [0, max_prefix_len]
 *   mask           uint64 [B][N][ceil(N/64)] from tree_mask_build
 *   out            fp32 [B][N][Hq][D]
 *   workspace      device buffer of >= tree_attn_workspace_bytes(...) bytes,
 *                  256-byte aligned, zero-filled before its first use; every
 *                  call leaves it zero-filled again (NULL allowed when the size
 *                  is 0). It holds the split partials and the counters the
 *                  splits of a (sequence, KV head) merge by, so calls that
 *                  share a workspace must not overlap.
 *   Supported: D in {64, 128}, block_size == 16, Hq % Hkv == 0,
 *   1 <= N <= 256, Hq/Hkv * N <= 4096, num_blocks * Hkv < 2^32 (cache
 *   block-heads are indexed with 32 bits). bf16 tensors 16-byte aligned.
 *   Precision: Q·K runs as a bf16 MFMA with fp32 accumulation; the weights
 *   and V enter the P·V MFMA as fp16 (V converts from bf16 exactly while
 *   |v| < 65520), accumulating in fp32.
 *   Flags: TAV_FLAG_BAD_BLOCK for a needed block outside [0, num_blocks);
 *   TAV_FLAG_CAPACITY for prefix_len beyond max_prefix_len or the table;
 *   TAV_FLAG_ATTN_RANGE for a non-finite output; TAV_FLAG_SYNC_TIMEOUT if a
 *   split's bounded wait for the other splits' partials ran out.
 */
tav_status tree_attn_verify(const uint16_t *q, const uint16_t *k_tree, const uint16_t *v_tree,
                            const uint16_t *k_cache, const uint16_t *v_cache, int32_t num_blocks,
                            const int32_t *block_table, int32_t max_blocks,
                            const int32_t *prefix_len, int32_t max_prefix_len,
                            const uint64_t *mask, int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t block_size, float scale, float *out,
                            void *workspace, size_t ws_bytes, uint32_t *dev_flags, void *stream);

/*
 * tree_attn_verify_tree — tree_attn_verify with the tree given as parent[]
 * instead of a mask: the attention launch builds the ancestor-or-self bits
 * itself (the rule of tree_mask_build: node j is visible to node i exactly
 * when j is i or one of its ancestors; jisaku.com glossary, tree-attention
 * section), so a step needs no separate mask launch. Outputs and every
 * other argument are those of tree_attn_verify; out is bit-identical to
 * tree_attn_verify's with the mask tree_mask_build makes from the same
 * parent[].
 *   parent     int32 [B][N], topological (parent[0] = -1, parent[i] < i)
 *   mask_out   optional uint64 [B][N][ceil(N/64)]: the mask, as tree_mask_build
 *              writes it (NULL: not written)
 *   depth_out  optional int32 [B][N]: node depths, as tree_mask_build
 * Flags: those of tree_attn_verify, and TAV_FLAG_BAD_PARENT for a parent
 * entry that breaks the numbering (as tree_mask_build; the bits of such a
 * node stop where its climb stops).
 */
tav_status tree_attn_verify_tree(const uint16_t *q, const uint16_t *k_tree,
                                 const uint16_t *v_tree, const uint16_t *k_cache,
                                 const uint16_t *v_cache, int32_t num_blocks,
                                 const int32_t *block_table, int32_t max_blocks,
                                 const int32_t *prefix_len, int32_t max_prefix_len,
                                 const int32_t *parent, uint64_t *mask_out, int32_t *depth_out,
                                 int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t block_size, float scale, float *out, void *workspace,
                                 size_t ws_bytes, uint32_t *dev_flags, void *stream);

/*
 * spec_verify_workspace_bytes — device workspace spec_verify_sample needs
 * for these sizes on the current device. Returns 0 for unsupported sizes.
 */
size_t spec_verify_workspace_bytes(int32_t B, int32_t N, int32_t V);

/*
 * spec_verify_sample — lossless rejection-sampling verification of a batch of
 * candidate trees, walked from the root down.
 *
 * Acceptance with probability min(1, p(x)/q(x)) and redraw from the
 * normalised positive part of p - q on rejection: radar-34b blog §2
 * (rejection-sampling acceptance condition). N+1 target distributions per
 * pass, so a fully accepted path still emits a bonus token: LLM Primer ch. 9,
 * §9.1. Root-down depth-first decisions: jisaku.com glossary, SpecInfer.
 *
 * For each sequence, starting at u = 0 (the root, never tested):
 *   p_u = softmax(target_logits[b][u] / T), q_u = softmax(draft_logits[b][u] / T);
 *   the children of u are tried in ascending node index: child c with token x
 *   is accepted iff r_acc(b,c) * q_u(x) < p_res(x), where p_res starts at p_u
 *   and, after each rejection, becomes max(0, p_res - q_u) / sum(...)
 *   (unchanged if that sum is 0); an accepted child becomes u;
 *   when u has no children, or all were rejected, one token is drawn from
 *   p_res (p_u at a leaf): the smallest k with C(k) > r_res(b,u) * sum(p_res).
 * Uniforms: Philox4x64-10 on counter (offset, b, i, 0), key (seed, 0); word 0
 * gives r_acc(b,i), word 1 gives r_res(b,i), as (w >> 40) * 2^-24.
 * All softmax, residual and CDF arithmetic is float64.
 *
 * temperature == 0 selects greedy verification (LLM Primer ch. 9, §9.1: the
 * longest prefix matching the target's own choice is accepted, then the
 * target's choice is committed): at u the choice x* is the argmax of
 * target_logits[b][u], the lowest token among equal maxima; the first child
 * (ascending node index) whose token is x* is accepted and becomes u; if
 * none is, x* is emitted and the walk stops (at a leaf, x* is the bonus).
 * No draft row and no uniform is read; draft_logits may be NULL.
 *
 *   target_logits, draft_logits  fp32 [B][N][V]; draft row u is the
 *                                distribution u's children were drawn from
 *   parent, token                int32 [B][N]; token[b][0] is ignored
 *   temperature                  >= 0 and finite (float64, used as given);
 *                                0 is greedy verification
 *   path        int32 [B][N] out: accepted nodes from the root (path[b][0] = 0), -1 padded
 *   n_accepted  int32 [B] out: accepted children (path length - 1)
 *   out_tokens  int32 [B][N] out: emitted tokens, n_accepted[b] + 1 of them, -1 padded
 *   workspace   device buffer of >= spec_verify_workspace_bytes(B, N, V) bytes,
 *               256-byte aligned, zero-filled before its first use; every call
 *               leaves it zero-filled again. Calls that share a workspace must
 *               not overlap in time (e.g. keep them on one stream).
 *   Supported: 1 <= N <= 256, 1 <= V <= 2^21, fp32 logits 4-byte aligned.
 *   Flags: TAV_FLAG_BAD_PARENT, TAV_FLAG_BAD_TOKEN, TAV_FLAG_NONFINITE_LOGITS,
 *   TAV_FLAG_SYNC_TIMEOUT.
 */
tav_status spec_verify_sample(const float *target_logits, const float *draft_logits,
                              const int32_t *parent, const int32_t *token, int32_t B, int32_t N,
                              int32_t V, double temperature, uint64_t seed, uint64_t offset,
                              int32_t *path, int32_t *n_accepted, int32_t *out_tokens,
                              void *workspace, size_t ws_bytes, uint32_t *dev_flags,
                              void *stream);

/*
 * spec_verify_sample_wor — spec_verify_sample for trees whose siblings were
 * drawn from q_u without replacement (distinct tokens per parent).
 *
 * The rejection step is the one above (radar-34b blog §2: accept with
 * min(1, p/q), else continue from the normalised positive part of p - q);
 * what changes is the draft distribution the next sibling is tested with. The
 * pages give top-k branching (jisaku.com glossary, tree-topology strategies) but no
 * sibling rule; testing every sibling against q_u is lossless only for
 * independent draws, so for draws without replacement the rejected token is
 * taken out of q: after sibling j (token x_j) is rejected at u,
 *   p_res <- max(0, p_res - q_j) / sum(...)   (as above, with the current q_j)
 *   q_{j+1}(y) = q_j(y) / sum_{z != x_j} q_j(z) for y != x_j, q_{j+1}(x_j) = 0,
 * with q_0 = q_u; if no draft mass is left q_{j+1} is zero, and a later
 * sibling with q(x) = 0 is accepted iff p_res(x) > 0. Sibling c after j
 * rejections is accepted iff r_acc(b,c) * q_j(x_c) < p_res(x_c). A repeated
 * token (not a draw without replacement) has q = 0 from its second
 * occurrence on. Everything else (uniforms, final draw, outputs, workspace,
 * greedy at temperature 0, flags, limits) is as for spec_verify_sample; the
 * workspace size is spec_verify_workspace_bytes(B, N, V).
 */
tav_status spec_verify_sample_wor(const float *target_logits, const float *draft_logits,
                                  const int32_t *parent, const int32_t *token, int32_t B,
                                  int32_t N, int32_t V, double temperature, uint64_t seed,
                                  uint64_t offset, int32_t *path, int32_t *n_accepted,
                                  int32_t *out_tokens, void *workspace, size_t ws_bytes,
                                  uint32_t *dev_flags, void *stream);

/*
 * spec_verify_sample_probe — spec_verify_sample (the independent-sibling
 * rule, temperature > 0) that also writes the softmax values its decisions
 * are taken with, so they can be checked against an exact softmax
 * (radar-34b blog §2 defines the walk on p and q; LLM Primer ch. 9, §9.1 has
 * one target distribution per node).
 *
 * For every node u the walk visits in sequence b:
 *   p_rows[b][u][y]  p_u(y) = softmax(target_logits[b][u] / T)(y), y < V,
 *                    as the walk holds it: each entry's exponential in fp32
 *                    relative to its wave's maximum, rebased to the row's
 *                    maximum and normalised in fp64;
 *   q_rows[b][u][y]  the same for the draft row, if u has children;
 *   child_pq[b][c][0..1]  for each child c of u: p_u(token[b][c]) and
 *                    q_u(token[b][c]) as the child tests read them.
 * Rows and entries of nodes the walk does not visit are left untouched.
 * path, n_accepted and out_tokens are those spec_verify_sample returns for
 * the same arguments. The probe writes 8 bytes per vocabulary entry of each
 * visited row: a checking tool, not the hot path.
 *
 *   p_rows, q_rows  fp64 [B][N][V] (8-byte aligned); child_pq fp64 [B][N][2]
 *   temperature > 0 (no greedy mode); everything else as spec_verify_sample,
 *   whose workspace size applies.
 */
tav_status spec_verify_sample_probe(const float *target_logits, const float *draft_logits,
                                    const int32_t *parent, const int32_t *token, int32_t B,
                                    int32_t N, int32_t V, double temperature, uint64_t seed,
                                    uint64_t offset, int32_t *path, int32_t *n_accepted,
                                    int32_t *out_tokens, double *p_rows, double *q_rows,
                                    double *child_pq, void *workspace, size_t ws_bytes,
                                    uint32_t *dev_flags, void *stream);

/*
 * spec_verify_sample_noalloc — spec_verify_sample (the independent-sibling
 * rule, or greedy at temperature 0) for callers that cannot allocate: code
 * under stream capture, tight serving loops, harnesses that forbid
 * allocation. It takes no workspace; its scratch (the exit counter and the
 * group mailbox) is a fixed 256 KiB array of the library, one per device,
 * held until the process ends. The call allocates nothing (no hipMalloc, no
 * allocating library routine). The first call on a device looks the array
 * up and queues a clearing fill kernel on `stream` ahead of its own kernel;
 * every call leaves the array zero-filled again. Calls on one device share
 * the array, so calls that overlap in time on one device race: keep them on
 * one stream. Results are those of spec_verify_sample for the same
 * arguments. TAV_ERR_WORKSPACE if the plan's mailbox exceeded the array
 * (no supported shape does: it needs at most 64 KiB); argument errors as
 * spec_verify_sample.
 */
tav_status spec_verify_sample_noalloc(const float *target_logits, const float *draft_logits,
                                      const int32_t *parent, const int32_t *token, int32_t B,
                                      int32_t N, int32_t V, double temperature, uint64_t seed,
                                      uint64_t offset, int32_t *path, int32_t *n_accepted,
                                      int32_t *out_tokens, uint32_t *dev_flags, void *stream);

/*
 * kv_commit_path — keep the accepted path's K/V, discarding the rest.
 *
 * Only the accepted path survives verification; rejected branches are pruned
 * and the cache rolls back to the accepted length, which paged blocks make
 * cheap: radar-34b blog §5 (KV-cache management); jisaku.com glossary,
 * KV-cache section.
 *
 * For t = 0..n_accepted[b], node path[b][t] is written at position
 * prefix_len[b] + t of sequence b (block block_table[b][pos/16], slot pos%16);
 * commit_slots[b][t] = block * 16 + pos % 16 (-1 beyond the path);
 * new_prefix_len[b] = prefix_len[b] + n_accepted[b] + 1. Nothing else in the
 * caches is written.
 *
 *   k_tree, v_tree   bf16 [B][N][Hkv][D]
 *   path, n_accepted as written by spec_verify_sample (read on the device)
 *   k_cache, v_cache the paged caches, updated in place
 *   commit_slots     int32 [B][N] out;  new_prefix_len int32 [B] out
 *   Supported: D in {64, 128}, block_size == 16, 1 <= N <= 256.
 *   Flags: TAV_FLAG_BAD_BLOCK, TAV_FLAG_CAPACITY (table too short),
 *   TAV_FLAG_BAD_PARENT (path entry outside [0, N) or n_accepted outside [0, N)).
 */
tav_status kv_commit_path(const uint16_t *k_tree, const uint16_t *v_tree, const int32_t *path,
                          const int32_t *n_accepted, int32_t num_blocks,
                          const int32_t *block_table, int32_t max_blocks,
                          const int32_t *prefix_len, uint16_t *k_cache, uint16_t *v_cache,
                          int32_t B, int32_t N, int32_t Hkv, int32_t D, int32_t block_size,
                          int32_t *commit_slots, int32_t *new_prefix_len, uint32_t *dev_flags,
                          void *stream);

/*
 * spec_verify_sample_commit — spec_verify_sample (or spec_verify_sample_wor
 * with without_replacement = 1; greedy at temperature 0) followed by
 * kv_commit_path, in one launch: the walk's workgroups copy each sequence's
 * accepted path into the paged cache as soon as that sequence is decided
 * (radar-34b blog §5 and jisaku.com glossary, KV-cache section: only the
 * accepted root-to-node path is kept, at the sequence's next positions).
 * Every output is the bytes the two separate calls write for the same
 * arguments: path, n_accepted, out_tokens as spec_verify_sample; the caches,
 * commit_slots and new_prefix_len as kv_commit_path given that path (a
 * sequence whose walk raised a flag commits its root row, as there).
 * Arguments are the union of the two calls' and mean the same; the commit's
 * are checked first (kv_commit_path's rules: D 64 or 128, block_size 16,
 * 16-byte aligned k_tree, v_tree, k_cache), then the walk's. The workspace is
 * spec_verify_workspace_bytes(B, N, V) bytes, as for spec_verify_sample.
 * Flags: the union of the two calls' flags.
 */
tav_status spec_verify_sample_commit(
    const float *target_logits, const float *draft_logits, const int32_t *parent,
    const int32_t *token, int32_t B, int32_t N, int32_t V, double temperature, uint64_t seed,
    uint64_t offset, int32_t without_replacement, int32_t *path, int32_t *n_accepted,
    int32_t *out_tokens, const uint16_t *k_tree, const uint16_t *v_tree, int32_t num_blocks,
    const int32_t *block_table, int32_t max_blocks, const int32_t *prefix_len, uint16_t *k_cache,
    uint16_t *v_cache, int32_t Hkv, int32_t D, int32_t block_size, int32_t *commit_slots,
    int32_t *new_prefix_len, void *workspace, size_t ws_bytes, uint32_t *dev_flags, void *stream);

/*
 * kv_commit_inplace — zero-copy rollback: the tree's K/V already sit in the
 * cache, node i of sequence b at position prefix_len[b] + i (written there
 * by the forward pass), and only the accepted path's rows that are out of
 * place move.
 *
 * Engines branch and roll back the tree through paged block-table operations
 * without copying: radar-34b blog §5 (KV-cache management); entries off the
 * accepted path are pruned and the cache rolled back to the right position:
 * jisaku.com glossary, KV-cache section.
 *
 * For t = 0..n_accepted[b], position prefix_len[b] + t receives what position
 * prefix_len[b] + path[b][t] held (every such row is read before any is
 * written, so overlapping moves are safe); rows with path[b][t] == t do not
 * move. new_prefix_len[b] = prefix_len[b] + n_accepted[b] + 1; positions past
 * it are abandoned (left as they are, not freed). commit_slots as in
 * kv_commit_path. Nothing else in the caches is written.
 *
 *   path, n_accepted as written by spec_verify_sample (read on the device)
 *   block_table      must map positions prefix_len[b] .. prefix_len[b] + N - 1
 *   k_cache, v_cache the paged caches, updated in place
 *   commit_slots     int32 [B][N] out;  new_prefix_len int32 [B] out
 *   Supported: D in {64, 128}, block_size == 16, 1 <= N <= 256, B <= 65535.
 *   Flags: TAV_FLAG_CAPACITY (table shorter than the tree: nothing moves),
 *   TAV_FLAG_BAD_BLOCK, TAV_FLAG_BAD_PARENT (path entry outside [0, N) or
 *   n_accepted outside [0, N)).
 */
tav_status kv_commit_inplace(const int32_t *path, const int32_t *n_accepted, int32_t num_blocks,
                             const int32_t *block_table, int32_t max_blocks,
                             const int32_t *prefix_len, uint16_t *k_cache, uint16_t *v_cache,
                             int32_t B, int32_t N, int32_t Hkv, int32_t D, int32_t block_size,
                             int32_t *commit_slots, int32_t *new_prefix_len, uint32_t *dev_flags,
                             void *stream);

/*
 * tree_expand_workspace_bytes — device workspace tree_expand_topk needs for
 * R rows of V logits and k tokens per row. Returns 0 for unsupported sizes.
 */
size_t tree_expand_workspace_bytes(int64_t R, int32_t V, int32_t k);

/*
 * tree_expand_topk — what tree construction reads from each frontier node's
 * draft row: its k most likely tokens with their log-probabilities, and the
 * entropy of the draft distribution. Top-k branching expands a node by its
 * draft's k most likely tokens; entropy-based branching gives a node more
 * branches the higher its entropy (jisaku.com glossary, tree-topology
 * strategies).
 *
 * For row r, q = softmax(draft_logits[r] / T):
 *   top_token[r][i]  the i-th most likely token (i < k), the lower token
 *                    first among equal logits;
 *   top_logq[r][i]   log q of that token (fp64);
 *   entropy[r]       -sum q log q over tokens with q > 0 (fp64).
 * Each token's exponential is taken in fp32 and the sums in fp64, so log q
 * and the entropy are within about 1e-6 of exact arithmetic; the token
 * ranking compares the fp32 logits themselves and is exact.
 *
 *   draft_logits  fp32 [R][V], 4-byte aligned
 *   k             1 <= k <= min(16, V);  temperature > 0 and finite
 *   workspace     device buffer of >= tree_expand_workspace_bytes(R, V, k)
 *                 bytes, 16-byte aligned (no initial contents needed)
 *   Supported: V <= 2^21.
 *   Flags: TAV_FLAG_NONFINITE_LOGITS for a row with a NaN or a maximum that
 *   is not finite (its tokens are -1, its log q and entropy NaN).
 */
tav_status tree_expand_topk(const float *draft_logits, int64_t R, int32_t V, int32_t k,
                            double temperature, int32_t *top_token, double *top_logq,
                            double *entropy, void *workspace, size_t ws_bytes,
                            uint32_t *dev_flags, void *stream);

/*
 * tav_philox_uniforms — the uniforms spec_verify_sample draws, for checking:
 * u[b][i][0] = r_acc(b, i), u[b][i][1] = r_res(b, i) (fp32, exact).
 */
tav_status tav_philox_uniforms(uint64_t seed, uint64_t offset, int32_t B, int32_t N, float *u,
                               void *stream);

/*
 * tav_target_probs — p = softmax(logits / T) per row, every exponential and
 * sum in float64 on the device (radar-34b blog §2 names p and q). A reference
 * for the device's fp64 exponential; the walk itself takes its per-entry
 * exponentials in fp32 (see spec_verify_sample_probe, which exposes the
 * values the walk decides with).
 *   logits fp32 [rows][V] (16-byte aligned), p fp64 [rows][V].
 */
tav_status tav_target_probs(const float *logits, int64_t rows, int32_t V, double temperature,
                            double *p, uint32_t *dev_flags, void *stream);

/*
 * tree_expand_sample — tree_expand_topk for a sampled tree: the k tokens of
 * each row are drawn from q = softmax(row / T) without replacement, the
 * order of the draws kept, so a tree grown from them is one for which
 * spec_verify_sample_wor is lossless. The glossary's top-k branching
 * (jisaku.com glossary, tree-topology strategies) with the k most likely
 * tokens replaced by k draws; the draw is the Gumbel-top-k construction: the
 * k largest keys x/T + G, the lower token first among equal keys, are the
 * draws in order. Each key is formed in fp64 exactly as written: x/T with
 * x widened from fp32, G = -log(-log u), u = fl64(m + 1/2) 2^-53 for the
 * 53-bit integer m = hi 2^21 + lo of token t in row r:
 *   hi  SplitMix64 (Steele, Lea, Flood 2014) seeded with K, output number
 *       r 2^20 + t/2 + 1 (its high half for even t, low half for odd t),
 *       K = word 0 of Philox4x64-10 at counter (offset, 0, 0, 3), key (seed, 0);
 *   lo  the top 21 bits of 32-bit half (t mod 8)/4 (0: high) of word
 *       (t mod 8) mod 4 of Philox4x64-10 at counter (offset, r, t/8, 2),
 *       key (seed, 0)
 * (the node uniforms of spec_verify_sample use counter word 3 = 0). The
 * kernels bound every key from hi alone in fp32 and form the exact fp64 key
 * only for the few tokens whose bounds reach the k-th; a result differs from
 * exact arithmetic only where two keys agree to the last bits of the fp64
 * log. top_logq and entropy are as in tree_expand_topk; arguments, workspace
 * (tree_expand_workspace_bytes), limits and flags too; R < 2^44.
 */
tav_status tree_expand_sample(const float *draft_logits, int64_t R, int32_t V, int32_t k,
                              double temperature, uint64_t seed, uint64_t offset,
                              int32_t *top_token, double *top_logq, double *entropy,
                              void *workspace, size_t ws_bytes, uint32_t *dev_flags,
                              void *stream);

/*
 * tree_select_topm — the budget step of tree construction: keep the M best
 * nodes of each candidate tree and renumber them as a tree.
 *
 * The budget rule caps the node count and allots branches to maximise the
 * expected number of accepted tokens (jisaku.com glossary, tree-topology
 * strategies, budget-constrained optimisation); EAGLE-2 grows the draft
 * tree dynamically and keeps the most promising paths (LLM Primer ch. 9,
 * §9.2). A node's acceptance is estimated by the draft as the product of q
 * along its path: score(0) = 0, score(i) = score(parent[i]) + min(logq[i], 0)
 * in fp64, one addition per node. The kept set is the M nodes of largest
 * score, the lower index first among equal scores; since no child scores
 * above its parent it is a subtree, and it maximises the sum of exp(score)
 * over all M-node subtrees.
 *
 *   parent  int32 [B][Nc] candidate trees (topological, as for every call)
 *   token   int32 [B][Nc] candidate tokens (copied through, not checked)
 *   logq    fp64 [B][Nc] log q of node i's token in its parent's draft row
 *           (e.g. tree_expand_topk's top_logq); entry 0 is ignored; -inf allowed
 *   out_parent int32 [B][M] out: the kept nodes' parents, as new indices
 *   out_token  int32 [B][M] out: their tokens
 *   out_src    int32 [B][M] out: their candidate indices, ascending
 * The kept nodes keep their relative order, so the output is topological
 * with the root at 0. 1 <= M <= Nc <= 1024.
 * Flags: TAV_FLAG_BAD_PARENT, TAV_FLAG_NONFINITE_LOGITS (a NaN log q); the
 * sequence's outputs are then not written.
 */
tav_status tree_select_topm(const int32_t *parent, const int32_t *token, const double *logq,
                            int32_t B, int32_t Nc, int32_t M, int32_t *out_parent,
                            int32_t *out_token, int32_t *out_src, uint32_t *dev_flags,
                            void *stream);

/*
 * tree_topology_workspace_bytes — device workspace tree_topology_dp needs
 * (0 for unsupported sizes).
 */
size_t tree_topology_workspace_bytes(int32_t K, int32_t n, int32_t depth);

/*
 * tree_topology_dp — the budget-constrained tree topology by dynamic
 * programming: the node count is capped at n and branches are allotted to
 * maximise the expected number of accepted tokens (jisaku.com glossary,
 * tree-topology strategies, budget-constrained optimisation; the Sequoia
 * paragraph: a topology chosen for the hardware and the draft's behaviour).
 * Acceptance model by sibling rank: the k-th child of a node, once reached,
 * is accepted with probability p_rank[k-1] at any depth, so the expected
 * accepted count of a tree is the sum over non-root nodes of the product of
 * p over the ranks along the node's path. Among all trees of n nodes, depth
 * at most `depth` and at most K children per node, the one of largest
 * expected count, from
 *   F(1, r) = 0, F(m, 0) = -inf (m > 1), F(m, r) = C(m - 1, r - 1, 1),
 *   C(0, r, j) = 0, C(s, r, j) = -inf for j > K,
 *   C(s, r, j) = max_{t=1..s} p_j (1 + F(t, r)) + C(s - t, r, j + 1)
 * in fp64, each value formed as (1 + F), times p_j, plus C, the smallest t
 * among equal maxima (C places s nodes in the subtrees of children j, j+1,
 * ...). The tree is written breadth-first: node 0 the root, each node's
 * children in rank order as nodes are reached (topological; siblings in the
 * order the walk tries them).
 *
 *   p_rank  host array of K probabilities in [0, 1]
 *   parent  int32 [n] out (device): parent of each node, -1 for node 0
 *   rank    int32 [n] out (device): 1-based position among its siblings (0 for the root)
 *   value   fp64 [1] out (device): the expected accepted count
 *   workspace  device buffer of >= tree_topology_workspace_bytes(K, n, depth)
 *   Supported: 1 <= K <= 16, 1 <= n <= 256, 0 <= depth <= 64.
 *   TAV_ERR_ARG for a p outside [0, 1] or NaN; TAV_ERR_UNSUPPORTED when no
 *   n-node tree fits within the depth and K children per node.
 */
tav_status tree_topology_dp(const double *p_rank, int32_t K, int32_t n, int32_t depth,
                            int32_t *parent, int32_t *rank, double *value, void *workspace,
                            size_t ws_bytes, void *stream);

/*
 * tree_widths_by_entropy — entropy-based branching: a frontier node whose
 * draft distribution has higher entropy gets more branches (jisaku.com
 * glossary, tree-topology strategies). The F frontier nodes of row b are
 * ranked by entropy, ascending, the lower index first among equal values;
 * the node of rank r gets w_min + floor((w_max - w_min + 1) * r / F)
 * branches, so with widths 1..4 each quartile of the frontier gets one width.
 *
 *   entropy  fp64 [B][F] (e.g. tree_expand_topk's entropy of the frontier rows)
 *   width    int32 [B][F] out
 * 1 <= F <= 1024, 0 <= w_min <= w_max. Flags: TAV_FLAG_NONFINITE_LOGITS (a
 * NaN entropy; the row's widths are then not written).
 */
tav_status tree_widths_by_entropy(const double *entropy, int32_t B, int32_t F, int32_t w_min,
                                  int32_t w_max, int32_t *width, uint32_t *dev_flags,
                                  void *stream);

/*
 * The speedup model of a speculative step (LLM Primer ch. 9, §9.3): speedup =
 * E[emitted] / (T_draft/T_decode + 1 + alpha*N), alpha the verification
 * overhead per candidate position. Host functions: no device pointer, no
 * stream, nothing launched.
 *
 * tav_model_speedup — that ratio; NaN for n < 0, a negative or NaN argument
 * or a non-positive denominator.
 *
 * tav_best_chain_length — the chain length N in [1, n_max] with the largest
 * model speedup when each candidate is accepted with probability p, so a
 * chain emits sum_{i<=N} p^i tokens on average (jisaku.com glossary,
 * linear-speculation closed form); the smallest such N on ties. Writes the
 * speedup to *speedup_out if it is not NULL. Returns 0 for p outside [0, 1],
 * n_max < 1 or a negative or non-finite ratio or alpha.
 *
 * tav_fit_alpha — alpha from verification times t_us[k] measured at tree
 * sizes n[k] (host arrays, count >= 2, n[0] = 1): the least-squares slope of
 * t(N)/t(1) - 1 against N - 1, through the origin. NaN on bad input.
 */
double tav_model_speedup(double expected_emitted, double draft_ratio, double alpha, int32_t n);

/*
 * tav_verify_speedup — the same model at batch B with a whole decode step as
 * the baseline of alpha (LLM Primer ch. 9, §9.3; the yuuk.io wiki notes the
 * speedup falls as the batch grows). With lin(T) = max(2 params / HBM,
 * 2 params T / MFMA) the roofline time of a bf16 product over T tokens:
 *   T_decode = layers (lin_layer(B) + attn_decode) + lin_head(B) + sampler_decode
 *   T_verify = layers (lin_layer(B n) + attn_verify) + lin_head(B n) + sampler_verify
 *   alpha = (T_verify / T_decode - 1) / n,
 *   speedup = expected_emitted / (draft_ratio + 1 + alpha n).
 * attn_* are one layer's attention times and sampler_* the walk's, in us (as
 * measured); params counts of a layer's projections and of the vocabulary
 * head; hbm_gbs in GB/s, mfma_tflops in TFLOP/s. Writes alpha, T_decode and
 * T_verify (us) to out[0..2] if out is not NULL. NaN for a negative or
 * non-finite argument, layers, batch or n below 1, or a non-positive rate.
 */
double tav_verify_speedup(double expected_emitted, double draft_ratio, int32_t layers,
                          double layer_params, double head_params, int32_t batch, int32_t n,
                          double attn_verify_us, double sampler_verify_us, double attn_decode_us,
                          double sampler_decode_us, double hbm_gbs, double mfma_tflops,
                          double *out);
int32_t tav_best_chain_length(double p, double draft_ratio, double alpha, int32_t n_max,
                              double *speedup_out);
double tav_fit_alpha(const int32_t *n, const double *t_us, int32_t count);

#ifdef __cplusplus
}
#endif

#endif /* TAV_H */
