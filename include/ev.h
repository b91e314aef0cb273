/*
 * ev.h — one-pass verification of a drafted token tree on AMD MI355X (gfx950).
 *
 * What the library computes (sources, all web pages on EAGLE speculative decoding):
 *   [TR] "Tech Radar: SGLang EAGLE-2 speculative decoding" (learn.tanhdev.com),
 *        sec. 2: sequence diagram (draft a tree of at most 64 nodes plus its mask, run
 *        ONE target forward over the whole tree, keep the accepted branch's KV, drop the
 *        rest) and the dynamic tree-attention mask equation M.
 *   [EX] "EAGLE — Draft head attached to an internal layer, 3x speedup" (troisinh.com),
 *        "Core idea" (verify all branches at once for the longest accepted prefix) and
 *        "Why it works" (rejection sampling keeps the target's output distribution).
 *   [SN] "EAGLE — guessing the next step in feature space" (estelledc.github.io),
 *        case 1 (k accepted drafts advance k + 1 tokens) and case 3 (lossless argument).
 *
 * Conventions shared by every call
 *   - Every pointer argument is DEVICE memory owned by the caller unless marked (host).
 *   - Calls enqueue work on `stream` and return without synchronising.  No call
 *     allocates memory or keeps state between calls; workspace comes from the caller,
 *     sized by the matching *_workspace() query.
 *   - Argument errors visible on the host (NULL pointers, sizes out of range, workspace
 *     too small, bad scalars) return a non-zero ev_status before anything is launched.
 *   - Errors that depend on device data (a bad parent[] array, a prefix that does not
 *     fit the cache, a block id or token id out of range) are reported through the
 *     optional device word *dev_status (may be NULL): the first error code stored there
 *     wins (the caller zeroes it beforehand and reads it after synchronising).  Outputs of
 *     an offending sequence are then unspecified, but no out-of-bounds access is made.
 *   - Arrays of queries, outputs and cache rows must start on a 16-byte boundary (any
 *     device allocator's alignment); a misaligned one returns EV_ERR_ARG.
 *   - Tree encoding: parent[B][T] int32, node 0 is the root (the last committed token,
 *     parent -1) and 0 <= parent[i] < i for i >= 1; 1 <= T <= 64.
 *   - Draft tokens: tokens[B][T] int32; tokens[b][i] is the token drafted at node i.
 *   - KV slots: the tree's own keys/values occupy logical slots L_b .. L_b+T-1 in node
 *     order, right after the committed prefix of length L_b = prefix_len[b].
 */
#ifndef EV_H
#define EV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ev_status;

enum {
  EV_OK = 0,
  EV_ERR_NULL = 1,        /* a required pointer is NULL */
  EV_ERR_SHAPE = 2,       /* a size is out of range (T, heads, head_dim, V, layout) */
  EV_ERR_DTYPE = 3,       /* unsupported element type */
  EV_ERR_WORKSPACE = 4,   /* ws_bytes smaller than the *_workspace() query */
  EV_ERR_ARG = 5,         /* invalid scalar (temperature, softmax scale) or misaligned array */
  EV_ERR_LAUNCH = 6,      /* a kernel launch failed */
  EV_ERR_SCRATCH = 7,     /* the call does not fit the fixed scratch of a no-allocation entry point */
  /* device-side codes, stored into *dev_status */
  EV_DERR_PARENT = 101,   /* parent[] is not a topological tree rooted at node 0 */
  EV_DERR_BOUNDS = 102,   /* prefix + tree does not fit the cache, or a block id is out of range */
  EV_DERR_TOKEN = 103,    /* a draft token id is outside [0, V) */
  EV_DERR_PATH = 104,     /* path / accept_len given to compaction is not a valid root path */
  EV_DERR_WIDTH = 105     /* a node has more children than the max_children bound */
};

typedef enum { EV_F32 = 0, EV_BF16 = 1, EV_INT4 = 2 } ev_dtype;

/* (host) KV-cache descriptor shared by attention and compaction.
 *   contiguous (paged = 0): k, v are [B][n_kv_heads][cap][head_dim]
 *   paged      (paged = 1): k, v are [n_blocks][n_kv_heads][block_size][head_dim];
 *              logical slot s of sequence b lives in block block_table[b][s / block_size]
 *              (block_table is device int32 [B][max_blocks_per_seq]) at offset
 *              s % block_size.
 *   Compaction touches n_layers layers found at k + l * layer_stride (elements), same for v;
 *   attention reads layer 0 only.
 *   EV_INT4 (an INT4-quantised cache; [EX] pairs EAGLE with KV-cache quantisation): each
 *   (slot, KV head) row holds head_dim signed 4-bit values q in [-8, 7], two per byte
 *   (element 2j in the low nibble of byte j, two's complement), so k and v are uint8 with
 *   head_dim / 2 bytes per row in the layouts above; k_scale and v_scale hold one float32
 *   scale s per row ([B][n_kv_heads][cap] or [n_blocks][n_kv_heads][block_size]).  The
 *   value used is bf16(s * q), the float32 product rounded to the nearest bfloat16.
 *   layer_stride still counts values (a multiple of head_dim); the scales of layer l
 *   start layer_stride / head_dim floats after layer 0's.  Queries and outputs of
 *   attention over an EV_INT4 cache are bfloat16. */
typedef struct {
  int32_t dtype;              /* ev_dtype of K and V (and of Q / O for attention) */
  int32_t n_kv_heads;
  int32_t head_dim;           /* 64 or 128 */
  int32_t paged;              /* 0 contiguous, 1 paged */
  void *k;
  void *v;
  int32_t n_layers;           /* >= 1 */
  int64_t layer_stride;       /* elements between consecutive layers */
  int64_t cap;                /* contiguous: slots per sequence */
  const int32_t *block_table; /* paged only */
  int32_t block_size;         /* paged: slots per block, a power of two in [1, 256] */
  int32_t max_blocks_per_seq; /* paged: columns of block_table */
  int32_t n_blocks;           /* paged: blocks in the pool */
  const float *k_scale;       /* EV_INT4 only: per-row scales of k */
  const float *v_scale;       /* EV_INT4 only: per-row scales of v */
} ev_kv_desc;

/* ev_tree_mask_build — ancestor mask of each tree ([TR] sec. 2, mask equation M).
 *   anc_mask[B][T] uint64: bit j of anc_mask[b][i] is set iff node j is node i or one of
 *   its ancestors.  depth[B][T] int32 (may be NULL): edges from the root.
 *   A parent[] that is not topological sets EV_DERR_PARENT. */
ev_status ev_tree_mask_build(const int32_t *parent, int32_t B, int32_t T,
                             uint64_t *anc_mask, int32_t *depth,
                             int32_t *dev_status, hipStream_t stream);

/* Bytes of workspace ev_tree_attention needs for these shapes (0 when none, and 0 for
 * invalid arguments): the split-L partial results when the key range is split across
 * workgroups.  max_prefix_len (host) is the largest prefix_len[b] the call will see; the
 * key range [0, max_prefix_len + T) is what the work is split over, so pass the batch's
 * real longest prefix, not the cache capacity (a bound beyond the cache counts as the
 * cache's capacity).  The same value must be passed to ev_tree_attention.  The workspace
 * needs no initialisation; calls that overlap in time must not share one. */
size_t ev_tree_attention_workspace(const ev_kv_desc *kv, int32_t B, int32_t T, int32_t Hq,
                                   int64_t max_prefix_len);

/* ev_tree_attention — tree-masked attention of the T node queries of each sequence
 * ([TR] sec. 2: every node attends to the whole committed prefix and, among the tree
 * slots, exactly to those with M[i][j] = 1; [EX] "Core idea": all branches in one pass).
 *   q    [B][T][Hq][head_dim], dtype kv->dtype;  query head h reads KV head h / (Hq / Hkv)
 *   kv   layer 0 of the cache (slots L_b .. L_b+T-1 already hold the tree's own K/V)
 *   prefix_len [B] int32, anc_mask [B][T] from ev_tree_mask_build
 *   max_prefix_len (host) an upper bound of every prefix_len[b], as given to
 *        ev_tree_attention_workspace (>= 0, else EV_ERR_SHAPE)
 *   sm_scale   score scale (pass 1/sqrt(head_dim) for the usual attention)
 *   out  [B][T][Hq][head_dim], dtype kv->dtype;  lse [B][T][Hq] float, natural log of the
 *        softmax normaliser of the scaled scores.
 *   ws, ws_bytes: workspace of at least ev_tree_attention_workspace() bytes.
 *   bf16 is computed with bf16 matrix-core products and float32 softmax/accumulation;
 *   f32 in float32 throughout.  EV_DERR_BOUNDS when L_b + T exceeds the cache or L_b
 *   exceeds max_prefix_len. */
ev_status ev_tree_attention(const void *q, const ev_kv_desc *kv, const int32_t *prefix_len,
                            const uint64_t *anc_mask, int32_t B, int32_t T, int32_t Hq,
                            int64_t max_prefix_len, float sm_scale, void *out, float *lse,
                            void *ws, size_t ws_bytes, int32_t *dev_status, hipStream_t stream);

/* ev_tree_attention_noalloc — ev_tree_attention for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as ev_tree_attention, without ws and
 * ws_bytes: the split partials go to a fixed array of ev_tree_attention_noalloc_limit()
 * bytes (32 MiB) that the library holds on each GPU it runs on until the process ends.
 * The call allocates nothing; it runs on the current device (pass a stream of that
 * device).  A call whose plan needs more than the array returns EV_ERR_SCRATCH before
 * launching (the Llama-3-70B-shaped layer needs 14 MB; a paged batch with one split per
 * work unit needs none).  Every call on a GPU shares that GPU's array: calls that overlap
 * in time on one GPU (other streams, other host threads) race and must be serialised by
 * the caller. */
ev_status ev_tree_attention_noalloc(const void *q, const ev_kv_desc *kv, const int32_t *prefix_len,
                                    const uint64_t *anc_mask, int32_t B, int32_t T, int32_t Hq,
                                    int64_t max_prefix_len, float sm_scale, void *out, float *lse,
                                    int32_t *dev_status, hipStream_t stream);

/* (host) Bytes of the fixed scratch array ev_tree_attention_noalloc uses. */
size_t ev_tree_attention_noalloc_limit(void);

/* ev_tree_mask_attention — ev_tree_mask_build followed by ev_tree_attention, in one call
 * ([TR] sec. 2: the mask M is derived from the tree and applied in the same forward).
 *   parent [B][T] int32 as for ev_tree_mask_build; anc_mask [B][T] uint64 (output, required)
 *   and depth [B][T] int32 (output, may be NULL) receive what ev_tree_mask_build writes;
 *   every other argument, the workspace (ev_tree_attention_workspace) and the outputs are
 *   those of ev_tree_attention.  For bf16 caches with head_dim 128 the attention launch
 *   itself builds the masks from parent[] (the workgroups whose keys reach the tree slots
 *   build them, one per sequence stores them), so mask and attention cost one launch;
 *   otherwise the mask kernel runs first.  A parent[] that is not a tree sets
 *   EV_DERR_PARENT; that sequence's outputs are then unspecified. */
ev_status ev_tree_mask_attention(const void *q, const ev_kv_desc *kv, const int32_t *prefix_len,
                                 const int32_t *parent, uint64_t *anc_mask, int32_t *depth,
                                 int32_t B, int32_t T, int32_t Hq, int64_t max_prefix_len,
                                 float sm_scale, void *out, float *lse, void *ws, size_t ws_bytes,
                                 int32_t *dev_status, hipStream_t stream);

/* Bytes of workspace the acceptance calls need (B * T <= 65535, V <= 262144).
 * The acceptance workspace holds arrival counters: zero-fill it (for example with
 * hipMemset) before its first use.  Every call that launches leaves the counters at zero
 * again, whatever B, T and V were, so one zeroed workspace of the largest size serves
 * calls of every smaller shape.  Calls that overlap in time must not share a workspace. */
size_t ev_accept_workspace(int32_t B, int32_t T, int32_t V);

/* ev_accept_greedy — greedy longest-matching-path acceptance ([EX] "Core idea";
 * [SN] case 1).  From the root, the target's token at node a is the lowest-index argmax of
 * the float32 row logits[b][a][:]; the walk moves to the lowest-index child drafted with
 * that token and stops at the first node with no such child.
 *   logits [B][T][V] float: row i is the target's next-token logits after node i.
 *   accept_len[B]: k, the number of accepted drafts.
 *   path[B][T]: accepted node indices (path[b][0] = 0), -1 after k + 1 entries.
 *   out_tokens[B][T]: the k + 1 emitted tokens (k drafts and the target's own next
 *   token at the last accepted node), -1 afterwards. */
ev_status ev_accept_greedy(const float *logits, const int32_t *tokens, const int32_t *parent,
                           int32_t B, int32_t T, int32_t V,
                           int32_t *accept_len, int32_t *path, int32_t *out_tokens,
                           void *ws, size_t ws_bytes, int32_t *dev_status, hipStream_t stream);

/* ev_accept_rejection — distribution-preserving rejection sampling walked down the tree
 * ([EX] "Why it works"; [SN] case 3) for deterministic (point-mass) drafts.
 *   p_a = softmax(logits[b][a] / temperature), evaluated in float64:
 *     s_y = double(logit_y) * (1.0 / double(temperature)), p(y) = exp(s_y - max s) / sum.
 *   At node a the children c are tried in ascending index; a child whose token was
 *   already rejected at a is skipped; child c is accepted iff uniforms[b][c] * Z < p_a(x)
 *   with Z the residual mass (1 minus the mass of tokens rejected so far at a).  When
 *   no child is accepted the emitted token is drawn from the residual distribution by
 *   inverse CDF in ascending token id with t = uniforms[b][0] * Z.
 *   uniforms [B][T] double in [0, 1).  Outputs as for ev_accept_greedy.
 *   EV_ERR_ARG unless temperature is finite and > 0. */
ev_status ev_accept_rejection(const float *logits, const int32_t *tokens, const int32_t *parent,
                              int32_t B, int32_t T, int32_t V, float temperature,
                              const double *uniforms,
                              int32_t *accept_len, int32_t *path, int32_t *out_tokens,
                              void *ws, size_t ws_bytes, int32_t *dev_status, hipStream_t stream);

/* ev_accept_greedy_compact, ev_accept_rejection_compact — ev_accept_greedy /
 * ev_accept_rejection followed by ev_kv_compact of each accepted path ([TR] sec. 2: keep
 * the accepted branch's KV) in the same launch: the workgroup that walks a sequence's tree
 * then moves its accepted rows.  Arguments and outputs are those of the acceptance call,
 * plus kv, prefix_len and new_len as for ev_kv_compact (the path and accept_len written
 * here are what it compacts).  When one accepted node's rows (all layers, KV heads, K and
 * V) exceed 4 KB, the ev_kv_compact kernel is launched after the acceptance instead.
 * Device errors as for both calls. */
ev_status ev_accept_greedy_compact(const float *logits, const int32_t *tokens,
                                   const int32_t *parent, int32_t B, int32_t T, int32_t V,
                                   int32_t *accept_len, int32_t *path, int32_t *out_tokens,
                                   const ev_kv_desc *kv, const int32_t *prefix_len,
                                   int32_t *new_len, void *ws, size_t ws_bytes,
                                   int32_t *dev_status, hipStream_t stream);
ev_status ev_accept_rejection_compact(const float *logits, const int32_t *tokens,
                                      const int32_t *parent, int32_t B, int32_t T, int32_t V,
                                      float temperature, const double *uniforms,
                                      int32_t *accept_len, int32_t *path, int32_t *out_tokens,
                                      const ev_kv_desc *kv, const int32_t *prefix_len,
                                      int32_t *new_len, void *ws, size_t ws_bytes,
                                      int32_t *dev_status, hipStream_t stream);

/* Bytes of workspace ev_accept_sampled needs (same limits and zero-fill contract as the
 * acceptance workspace above). */
size_t ev_accept_sampled_workspace(int32_t B, int32_t T, int32_t V);

/* ev_accept_sampled — the accept-or-resample rule ([EX] "Why it works"; [SN] case 3) for
 * drafts that were SAMPLED from a draft distribution instead of taken by argmax.
 *   draft_logits [B][T][V] float: row a is the drafter's logits at node a; its children
 *   were drawn independently from q_a = softmax(draft_logits[b][a] / draft_temperature)
 *   (duplicate siblings allowed, each tested on its own).
 *   p_a as in ev_accept_rejection; q_a by the same float64 contract with draft_temperature.
 *   At node a the children are tried in ascending index against the residual
 *   r = W / Z, W(y) = max(0, p_a(y) - s q_a(y)), Z = sum_y W(y), starting at s = 0: child c
 *   drafting x is accepted iff uniforms[b][c] * q_a(x) * Z < W(x) (probability
 *   min(1, r(x) / q_a(x))); a rejection adds Z to s (r becomes max(0, r - q_a),
 *   renormalised).  When no child is accepted the emitted token is the inverse-CDF draw of
 *   W in ascending token id with t = uniforms[b][0] * Z.
 *   max_children: (host) bound on the children of any node, 0 <= max_children <= T; it
 *   fixes the number of launches: one pass over every row (which also takes each node's
 *   first decision), then max_children passes over the rows still undecided.  A node
 *   with more children sets EV_DERR_WIDTH.
 *   Outputs as for ev_accept_greedy.  EV_ERR_ARG unless both temperatures are finite and
 *   > 0. */
ev_status ev_accept_sampled(const float *logits, const float *draft_logits, const int32_t *tokens,
                            const int32_t *parent, int32_t B, int32_t T, int32_t V,
                            float temperature, float draft_temperature, const double *uniforms,
                            int32_t max_children, int32_t *accept_len, int32_t *path,
                            int32_t *out_tokens, void *ws, size_t ws_bytes, int32_t *dev_status,
                            hipStream_t stream);

/* ev_kv_compact — keep the accepted branch's KV ([TR] sec. 2 sequence diagram).
 * For m = 1..k (k = accept_len[b], path from an acceptance call), logical slot
 * L_b + path[b][m] is copied to slot L_b + m, for K and V, every KV head and all
 * kv->n_layers layers, in place; every source is read before any slot is written.
 * new_len[B] = L_b + k + 1.  Slots at or beyond L_b + k + 1 are left untouched.
 * EV_DERR_PATH when path is not strictly increasing within [0, T) from node 0. */
ev_status ev_kv_compact(const ev_kv_desc *kv, const int32_t *prefix_len, const int32_t *path,
                        const int32_t *accept_len, int32_t B, int32_t T,
                        int32_t *new_len, int32_t *dev_status, hipStream_t stream);

/* Bytes of workspace ev_kv_compact_remap needs for B sequences (no zero-fill needed). */
size_t ev_kv_compact_remap_workspace(int32_t B);

/* ev_kv_compact_remap — zero-copy pruning of a PAGED cache ([TR] sec. 2: keep the accepted
 * branch's KV and drop the rest; sec. 4: KV fragmentation and the radix prefix cache):
 * the same logical result as ev_kv_compact, with block-table entries remapped instead of
 * rows copied wherever the moves allow it.
 *   Destination slots L_b + m (m = 1..k) lie in logical blocks X.  A block wholly past the
 *   root (X * block_size > L_b) whose moves share one offset D = path[m] - m, a multiple
 *   of block_size, moves no data: D = 0 leaves it in place; D > 0 points its entry at the
 *   physical block of X + D / block_size.  Every other destination block is written by
 *   copying rows (K and V, every KV head and layer).  A remap whose source block receives
 *   such copies is copied instead, repeated until none is left.  With block_size 1 (pages
 *   of one token) nothing is copied.
 *   The table kv->block_table points to is updated in place (writable device memory):
 *   remapped entries change, and entries of blocks from ceil(new_len / block_size) up to
 *   ceil((L_b + T) / block_size) become -1.  Blocks before L_b / block_size are untouched.
 *   Outputs: new_len[B] = L_b + k + 1; freed [B][max_blocks_per_seq]: in ascending logical
 *   block order, the distinct physical blocks of the tree's blocks (from L_b / block_size
 *   on) that no live block references any more, freed_count[B] of them; copied[B]: slots
 *   moved by copying.  The caller returns the freed blocks to its pool.  The table entries
 *   of a sequence's tree blocks must be distinct (as an allocator hands them out).
 *   EV_ERR_ARG for a contiguous cache; device errors as ev_kv_compact (EV_DERR_PATH,
 *   EV_DERR_BOUNDS, also for a table entry outside [0, n_blocks)); a sequence with a device
 *   error is left unchanged. */
ev_status ev_kv_compact_remap(const ev_kv_desc *kv, const int32_t *prefix_len,
                              const int32_t *path, const int32_t *accept_len, int32_t B,
                              int32_t T, int32_t *new_len, int32_t *freed, int32_t *freed_count,
                              int32_t *copied, void *ws, size_t ws_bytes, int32_t *dev_status,
                              hipStream_t stream);

/* ---- Draft-tree construction ([TR] sec. 2: sequence diagram, "Dynamic Tree-Attention
 * Masking") ----
 * The drafter grows the tree depth by depth: after each expansion it runs on the new
 * frontier and hands its next-token logits back.  Frontier node n, with
 * q_n = softmax(draft_logits_n / temperature) (float64 as in ev_accept_rejection), gets
 * k_n = min(k_max, max(1, floor(exp(H(q_n)) + 1/2))) children, where H is the entropy in
 * nats.  They are its k_n most probable tokens; equal logits go to the lower token id.
 * A node's value is the product of q along its path (root 1).  Each depth keeps the
 * `beam` best new candidates as the next frontier.  The tree is the root plus the
 * n_nodes - 1 best candidates of all depths, numbered by depth and then by value rank.
 * Equal values go to the lower candidate id: depth first, then frontier slot, then
 * child rank.  A child's value never exceeds its parent's, so every chosen node's
 * ancestors are chosen too.
 * The workspace carries the tree under construction from call to call: zero-fill it
 * before its first use (it is left with its counters at zero), and use one workspace
 * per tree being built at a time. */

/* Bytes of workspace for B sequences, beam width `beam` (1..8) and V-token logit rows. */
size_t ev_draft_tree_workspace(int32_t B, int32_t beam, int32_t V);

/* ev_draft_tree_expand — one depth of the beam expansion.  Calls go depth = 0, 1, 2, ...
 * (< 16) on the same workspace.  Depth 0 expands the root.
 *   draft_logits [B][beam][V] float: row w is the drafter's logits after frontier slot w
 *   of this depth (depth 0: row 0 is the root's; rows at or beyond the frontier count are
 *   not read).
 *   k_max in 1..8: most children per node.
 *   Outputs, the next frontier, for the drafter: frontier_tokens [B][beam] (its tokens,
 *   best first), frontier_slots [B][beam] (the slot of each one's parent at this depth),
 *   both -1 beyond frontier_count [B].
 *   EV_ERR_ARG unless temperature is finite and > 0.  EV_DERR_TOKEN when NaN logits
 *   leave fewer real tokens than a node's width (the token is clamped to V - 1). */
ev_status ev_draft_tree_expand(const float *draft_logits, int32_t B, int32_t beam, int32_t V,
                               int32_t depth, float temperature, int32_t k_max,
                               int32_t *frontier_tokens, int32_t *frontier_slots,
                               int32_t *frontier_count, void *ws, size_t ws_bytes,
                               int32_t *dev_status, hipStream_t stream);

/* ev_draft_tree_finalize — the tree after the expansions made so far.  B, beam and V are
 * those of the expansions.
 *   root_tokens [B]: the last committed token of each sequence (node 0's token).
 *   Outputs parent [B][n_nodes] (parent[0] = -1, 0 <= parent[i] < i) and tokens
 *   [B][n_nodes], both -1 beyond tree_size [B] (at most n_nodes, 1..64); ready for
 *   ev_tree_mask_build and the verification pass. */
ev_status ev_draft_tree_finalize(const int32_t *root_tokens, int32_t B, int32_t beam, int32_t V,
                                 int32_t n_nodes, int32_t *parent, int32_t *tokens,
                                 int32_t *tree_size, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/* (host) Static description of a status code. */
const char *ev_status_string(ev_status s);

#ifdef __cplusplus
}
#endif

#endif /* EV_H */
