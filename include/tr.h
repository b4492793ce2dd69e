/*
 * tr.h -- C ABI of libtr: the data-parallel hot path of Token Recycling (TR)
 * speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * TR keeps a |V| x k matrix M of candidate successor tokens ("Token
 * Recycling" summary, section Method, first module).  One decoding step:
 *   1. retrieve a static draft tree from M, starting at the last committed
 *      token (Method, second module);
 *   2. verify the tree's merged sequence against the prefix with tree
 *      attention: each node sees the prefix, its ancestors and itself, never
 *      a sibling branch (Method, third module; walk-through, workflow step 3);
 *   3. accept the longest correct path plus the target's token after it
 *      (walk-through, workflow step 4);
 *   4. overwrite, for every tree node x~_i, the row M[x~_i] with
 *      argtopk(p~_{i+1}) of that node's next-token distribution (Chinese
 *      summary, section Method, the update equation; walk-through, "why it
 *      is called Token Recycling").
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or keeps them.  Buffers must not alias
 *     unless a call says so.  Layouts are dense, row-major, innermost last.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous: outputs are valid once the stream has been synchronised.
 *   - Host-side checks (null pointers, sizes, dtype pairs, tree/k mismatch,
 *     workspace size) return a non-OK status and launch nothing; the reason
 *     is in tr_last_error().  A failed launch returns TR_ERR_HIP.
 *   - Data errors only the device can see set sticky bits in the workspace
 *     status word (tr_read_device_status) and skip the offending write:
 *     a token outside [0, V) (TR_FLAG_BAD_TOKEN), a commit that would
 *     overflow the cache capacity (TR_FLAG_CACHE_FULL) and a prefix_len
 *     outside [0, cap] given to tr_tree_attn (TR_FLAG_BAD_PREFIX; the
 *     length is clamped to that range).  TR_FLAG_HANDOVER reports that a
 *     wait of one block of a launch for another gave up (bounded at about
 *     seconds; it does not occur in normal operation): that call's outputs
 *     are unspecified and the workspace must be zeroed again
 *     (tr_workspace_init).
 *   - Tie and duplicate rules (fixed here; the pages leave them open):
 *     top-k orders by value descending, then token id ascending, with
 *     -0.0 == +0.0; when two tree nodes carry the same token, the node with
 *     the highest merged-sequence index writes M; the accepted path is the
 *     deepest accepted node, ties to the smallest index.
 *   - Logits must not be NaN (+-inf are fine).
 *
 * Limits: 1 <= k <= 16, 1 <= tree nodes <= 128, head dimension d = 128,
 * Hq a multiple of Hkv.  The top-k of a logits row (tr_update_topk, tr_step
 * and its variants) holds V <= 1,048,576 (bfloat16 logits, k <= 8),
 * 524,288 (bfloat16 with k > 8, or float32 with k <= 8) or 262,144 (float32,
 * k > 8); a longer row is TR_ERR_UNSUPPORTED.  bf16 tree attention takes
 * B <= 2048 sequences.
 */
#ifndef TR_H
#define TR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TR_OK = 0,
  TR_ERR_INVALID_ARGUMENT = 1,
  TR_ERR_UNSUPPORTED = 2,
  TR_ERR_INVALID_TREE = 3,
  TR_ERR_WORKSPACE_TOO_SMALL = 4,
  TR_ERR_HIP = 5
} tr_status;

typedef enum { TR_INT32 = 0, TR_INT64 = 1, TR_FLOAT32 = 2, TR_BFLOAT16 = 3 } tr_dtype;

enum { TR_FLAG_BAD_TOKEN = 1u, TR_FLAG_CACHE_FULL = 2u, TR_FLAG_BAD_PREFIX = 4u,
       TR_FLAG_BAD_PAGE = 8u, TR_FLAG_HANDOVER = 16u };

/* Opaque, immutable draft-tree template (host memory, library-owned).
 * Shareable across streams and threads. */
typedef struct tr_tree tr_tree;

/* Human-readable name of a status code (static string). */
const char* tr_status_string(tr_status s);

/* Detail of the last non-OK status returned on the calling thread
 * (thread-local, static storage; empty string if none). */
const char* tr_last_error(void);

/* ------------------------------------------------------------------------
 * Tree template (host only; no GPU needed).
 * The tree is static and imbalanced ("Token Recycling" summary, Method,
 * second module): children counts are fixed across steps; a node with c
 * children expands the c best candidates (ranks 0..c-1) of its row.
 * Nodes are numbered in merged-sequence order: layer by layer, inside a
 * layer by (parent index, rank) (Method, "merged sequence"; walk-through
 * step 3 prints [guest, speaker, speak, event, at, for, ing]).
 * ------------------------------------------------------------------------ */

/* parent[0] = -1 and rank[0] = -1 (root); for n > 0: 0 <= parent[n] < n,
 * 0 <= rank[n] < k, ranks distinct under one parent, nodes in layer order.
 * Host arrays of n_nodes entries, copied.  *out receives the template;
 * release it with tr_tree_destroy.  Errors: TR_ERR_INVALID_TREE,
 * TR_ERR_INVALID_ARGUMENT (null pointer, n_nodes outside 1..128, k outside
 * 1..16). */
tr_status tr_tree_create(int32_t n_nodes, const int32_t* parent, const int32_t* rank, int32_t k,
                         tr_tree** out);

/* Same from per-layer child counts: layer l (0 = the root's layer) has
 * level_len[l] counts, stored one layer after another in `counts`; entry i
 * of layer l is the number of children of the i-th node of that layer
 * (missing entries: no children).  Host arrays, copied. */
tr_status tr_tree_create_levels(int32_t n_levels, const int32_t* level_len, const int32_t* counts,
                                int32_t k, tr_tree** out);

void tr_tree_destroy(tr_tree* t);

/* Template facts, to host memory.  Any output pointer may be NULL.
 * parent_out/rank_out/depth_out: [n_nodes] int32; anc_out: [n_nodes][2]
 * uint64 ancestor bitmask (bit j of row n set iff node j is n or one of
 * its ancestors: the tree-attention mask). */
tr_status tr_tree_info(const tr_tree* t, int32_t* n_nodes, int32_t* depth, int32_t* k,
                       int32_t* parent_out, int32_t* rank_out, int32_t* depth_out,
                       uint64_t* anc_out);

/* ------------------------------------------------------------------------
 * Workspace.  One device buffer per stream holds counters, partial results
 * and the device status word.  Size it with tr_workspace_size for the
 * largest (B, V, heads, capacity) it will serve, zero it once with
 * tr_workspace_init; afterwards every call leaves it ready for the next
 * (counters return to zero), so it can be reused across calls and
 * captured in a HIP graph.  Calls sharing one workspace must be ordered
 * on one stream.
 * ------------------------------------------------------------------------ */
size_t tr_workspace_size(const tr_tree* t, int32_t B, int64_t V, int32_t k, int32_t Hq,
                         int32_t Hkv, int32_t d, int64_t cap);

/* Zero-fills ws (a kernel, not a memset).  ws must be 256-byte aligned. */
tr_status tr_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Copies the sticky status word (TR_FLAG_* bits) to *flags and clears it.
 * Synchronises `stream`. */
tr_status tr_read_device_status(void* ws, uint32_t* flags, void* stream);

/* ------------------------------------------------------------------------
 * Hot path.
 * ------------------------------------------------------------------------ */

/* Draft tree retrieval ("Token Recycling" summary, Method, second module;
 * walk-through, workflow steps 1-2): tree_tok[b][0] = root_tok[b] and,
 * layer by layer, tree_tok[b][n] = M[b][tree_tok[b][parent n]][rank n].
 *   M        [B][V][k] int32 or int64 (m_dtype), read only.
 *   root_tok [B] int32.  tree_tok [B][T] int32, written.
 *   ws       workspace (for the status word).
 * A token outside [0, V) sets TR_FLAG_BAD_TOKEN; its children get -1. */
tr_status tr_retrieve(const tr_tree* t, int32_t B, const void* M, tr_dtype m_dtype, int64_t V,
                      int32_t k, const int32_t* root_tok, int32_t* tree_tok, void* ws,
                      size_t ws_bytes, void* stream);

/* Tree attention over the prefix cache (Method, third module; walk-through
 * step 3): for every node n, query head h (key/value head h / (Hq/Hkv)):
 *   out[b][n][h] = sum_j softmax_j(scale * q[b][n][h] . key_j) value_j
 * with j over cache positions 0..prefix_len[b]-1 and the tree nodes that
 * are n or its ancestors.
 *   q         [B][T][Hq][d]      dt (TR_FLOAT32 or TR_BFLOAT16)
 *   k_tree,
 *   v_tree    [B][T][Hkv][d]     dt: the tree nodes' own keys/values
 *   k_cache,
 *   v_cache   [B][Hkv][cap][d]   dt: positions >= prefix_len[b] unread
 *   prefix_len [B] int32 (device; 0 <= prefix_len <= cap)
 *   scale     > 0 and finite (1/sqrt(d) in the usual reading)
 *   out       [B][T][Hq][d]      dt, written
 * Arithmetic: float32 accumulation; bf16 inputs use bf16 matrix cores for
 * both products.  The result does not depend on how the prefix is split. */
tr_status tr_tree_attn(const tr_tree* t, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, tr_dtype dt,
                       const void* q, const void* k_tree, const void* v_tree, const void* k_cache,
                       const void* v_cache, int64_t cap, const int32_t* prefix_len, float scale,
                       void* out, void* ws, size_t ws_bytes, void* stream);

/* tr_tree_attn for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, arithmetic, results and errors as
 * tr_tree_attn, without ws / ws_bytes: the call's scratch (prefix partials,
 * merge records) lives in a 48 MiB array of device memory that the library
 * holds on every GPU it runs on from the first call there until the process
 * ends; the call itself allocates nothing.  A call needing more scratch than
 * that (tr_workspace_size's attention part above 48 MiB) returns
 * TR_ERR_UNSUPPORTED and launches nothing.  Every call on one GPU shares that
 * GPU's array, so calls that overlap on one GPU (different streams or host
 * threads without ordering) race: order them on one stream.
 *   flags  device uint32 (nullable): the sticky TR_FLAG_* bits of the call
 *          are OR-ed into it (TR_FLAG_BAD_PREFIX); the caller clears it. */
tr_status tr_tree_attn_noalloc(const tr_tree* t, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                               tr_dtype dt, const void* q, const void* k_tree, const void* v_tree,
                               const void* k_cache, const void* v_cache, int64_t cap,
                               const int32_t* prefix_len, float scale, void* out, uint32_t* flags,
                               void* stream);

/* argtopk of every node's next-token logits and the recycling update
 * M[tree_tok[b][n]] = argtopk(logits[b][n]) for every node n, in merged
 * order (Chinese summary, Method, update equation; walk-through "why it is
 * called Token Recycling": rejected nodes update M too).
 *   logits   [B][T][V]  l_dtype (TR_FLOAT32 or TR_BFLOAT16)
 *   tree_tok [B][T] int32 (may be NULL when M is NULL)
 *   M        [B][V][k]  m_dtype, updated in place; NULL: top-k only
 *   topk_out [B][T][k] int32 token ids, best first; may be NULL when M
 *            is given. */
tr_status tr_update_topk(const tr_tree* t, int32_t B, const void* logits, tr_dtype l_dtype,
                         int64_t V, int32_t k, const int32_t* tree_tok, void* M, tr_dtype m_dtype,
                         int32_t* topk_out, void* ws, size_t ws_bytes, void* stream);

/* Greedy verification (Method, third module: the longest correct sequence
 * is the step's output; walk-through step 4: the target's own token follows
 * it).  It reads the target's greedy token of every node from topk; a caller
 * holding only the logits gets them first with tr_update_topk (M = NULL,
 * topk_out given), then calls this (tr_step does both in one launch).
 * g(n) = topk[b][n][0]; node n > 0 is accepted iff its parent is and
 * tree_tok[b][n] == g(parent).  best = deepest accepted node (ties: lowest
 * index).  Outputs (Dmax = tree depth):
 *   accept_len  [B]         L = depth(best)
 *   accept_path [B][Dmax+1] node ids root..best, then -1 (may be NULL)
 *   bonus       [B]         g(best)
 *   emitted     [B][Dmax+1] tree_tok of path[1..L], then bonus, then -1
 *                           (may be NULL) */
tr_status tr_verify(const tr_tree* t, int32_t B, const int32_t* topk, int32_t k,
                    const int32_t* tree_tok, int32_t* accept_len, int32_t* accept_path,
                    int32_t* bonus, int32_t* emitted, void* stream);

/* One whole TR step after the target's forward pass, fused:
 *   top-k of every node -> verify -> update M -> commit the accepted path's
 *   key/value rows -> next root = bonus -> retrieve the next tree.
 * The current tree was retrieved from M before this update; the next tree
 * sees the update (walk-through step 2).
 *   tree_tok  [B][T] in: this step's tree; out: the next step's tree
 *   root_tok  [B]    out: the bonus token (the next root)
 *   accept_len [B], accept_path [B][Dmax+1] (nullable),
 *   emitted [B][Dmax+1] (nullable) as tr_verify
 *   k_tree, v_tree [B][T][Hkv][d], k_cache, v_cache [B][Hkv][cap][d] in
 *   kv_dtype; prefix_len [B] in/out: rows path[0..L] are copied to cache
 *   positions prefix_len .. prefix_len+L and prefix_len grows by L+1.
 *   If k_cache is NULL no commit is done.
 *   topk_out  [B][T][k] (nullable).
 * With fewer than 256 logit rows (B*T) of at most 32768 logits, the step
 * runs as one launch of row blocks, a tail block per sequence and copy
 * blocks that wait for one another through the workspace; setting the
 * environment variable TR_FEW_ROW_STEP=0 selects the general kernel
 * instead (same results; a diagnostic switch).  tr_update_topk with M
 * follows the same rule. */
tr_status tr_step(const tr_tree* t, int32_t B, int64_t V, int32_t k, const void* logits,
                  tr_dtype l_dtype, void* M, tr_dtype m_dtype, int32_t* tree_tok, int32_t* root_tok,
                  int32_t* accept_len, int32_t* accept_path, int32_t* emitted, int32_t Hkv,
                  int32_t d, tr_dtype kv_dtype, const void* k_tree, const void* v_tree,
                  void* k_cache, void* v_cache, int64_t cap, int32_t* prefix_len, int32_t* topk_out,
                  void* ws, size_t ws_bytes, void* stream);

/* Which nodes recycle their top-k into M (Token Recycling, Experiment,
 * ablation of the update: every draft token against the accepted ones
 * only; every draft token gives the longer mean accepted length and is the
 * method's default). */
typedef enum {
  TR_UPDATE_ALL = 0,        /* every node of the tree (tr_step) */
  TR_UPDATE_ACCEPTED = 1    /* the accepted path only, root included:
                               M[tok path[i]] = topk[path[i]], i = 0..L; on a
                               repeated token the deeper node wins */
} tr_update_mode;

/* tr_step with a choice of update (tr_update_mode); everything else,
 * including arguments, errors and the retrieval of the next tree from the
 * updated M, as tr_step.  An unknown mode is TR_ERR_INVALID_ARGUMENT. */
tr_status tr_step_ex(const tr_tree* t, int32_t B, int64_t V, int32_t k, const void* logits,
                     tr_dtype l_dtype, void* M, tr_dtype m_dtype, int32_t* tree_tok,
                     int32_t* root_tok, int32_t* accept_len, int32_t* accept_path,
                     int32_t* emitted, int32_t Hkv, int32_t d, tr_dtype kv_dtype,
                     const void* k_tree, const void* v_tree, void* k_cache, void* v_cache,
                     int64_t cap, int32_t* prefix_len, int32_t* topk_out, tr_update_mode mode,
                     void* ws, size_t ws_bytes, void* stream);

/* tr_step with verification by sampling instead of greedy matching
 * (speculative-decoding lesson: accept a draft x with min(1, p(x)/q(x)),
 * else draw from the normalised positive part of p - q and stop; after a
 * fully accepted draft the bonus is drawn from p; Token Recycling,
 * Experiment: TR is also evaluated with sampling).
 *   p_n = softmax(logits[b][n] / temperature), temperature > 0 and finite.
 *   TR's drafts come from M, so q is a point mass on each drafted token.
 *   From the root, the children of the current node are tried in rank
 *   order: child c with token x is accepted when u[b][c][0] < r(x), r the
 *   current residual (p_n at first; each rejected sibling's token is taken
 *   out and r renormalised), and the walk moves to c.  When no child is
 *   accepted (a leaf has none) the bonus is drawn from r with u[b][n][1]:
 *   the smallest id whose cumulative residual probability, ids in
 *   increasing order, exceeds u[b][n][1].  The path root..stop node is the
 *   accepted path (accept_len, accept_path, emitted, commit, next root as
 *   tr_step).  The update of M (mode) still writes each node's top-k.
 *   uniforms [B][T][2] float32 in [0, 1), device memory (the caller draws
 *   them, e.g. from its own generator).  Probabilities are computed in
 *   float32; a uniform within float32 rounding of a threshold may decide
 *   either way.
 * Extra errors: TR_ERR_INVALID_ARGUMENT for a null uniforms pointer or a
 * temperature that is not positive and finite; TR_ERR_UNSUPPORTED for
 * V > 262144.  Workspace as tr_step. */
tr_status tr_step_sample(const tr_tree* t, int32_t B, int64_t V, int32_t k, const void* logits,
                         tr_dtype l_dtype, float temperature, const float* uniforms, void* M,
                         tr_dtype m_dtype, int32_t* tree_tok, int32_t* root_tok,
                         int32_t* accept_len, int32_t* accept_path, int32_t* emitted, int32_t Hkv,
                         int32_t d, tr_dtype kv_dtype, const void* k_tree, const void* v_tree,
                         void* k_cache, void* v_cache, int64_t cap, int32_t* prefix_len,
                         int32_t* topk_out, tr_update_mode mode, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------
 * Paged prefix cache, all layers of a model.  The pages fix no cache
 * layout; this one stores the same prefix rows as the contiguous
 * [B][Hkv][cap][d] cache, so every result equals the contiguous one.
 * Position p of sequence b is row p % page_size of page
 * block_table[b][p / page_size].  All pointers inside are device memory
 * owned by the caller; the struct itself is read on the host during the
 * call only.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t n_layers;            /* layers in the pools and tree rows, >= 1 */
  int32_t Hkv;                 /* key/value heads */
  int32_t d;                   /* head dimension: 128 */
  tr_dtype dtype;              /* TR_BFLOAT16 */
  int32_t page_size;           /* rows per page: a power of two, >= 64 */
  int64_t num_pages;           /* pages in each layer's pool */
  int32_t max_pages;           /* block-table entries per sequence */
  const int32_t* block_table;  /* [B][max_pages] page ids in [0, num_pages) */
  void* k_pages;               /* [n_layers][num_pages][Hkv][page_size][d] */
  void* v_pages;
  const void* k_tree;          /* [n_layers][B][T][Hkv][d]: this step's tree rows */
  const void* v_tree;
  int32_t* prefix_len;         /* [B], capacity max_pages * page_size */
} tr_paged_kv;

/* tr_tree_attn for layer `layer` of a paged cache: q [B][T][Hq][d] and out
 * [B][T][Hq][d] of that layer; the tree rows and the prefix pages are the
 * layer's slices of kv.  A page id outside [0, num_pages) reads page 0 and
 * sets TR_FLAG_BAD_PAGE.  Errors as tr_tree_attn, plus
 * TR_ERR_INVALID_ARGUMENT for a layer outside [0, n_layers) or a page size
 * that is not a power of two of at least 64, and TR_ERR_UNSUPPORTED for
 * float32 pages or a prefix chunk spanning more than 256 pages.  Workspace:
 * tr_workspace_size with cap = max_pages * page_size. */
tr_status tr_tree_attn_paged(const tr_tree* t, int32_t B, int32_t Hq, const void* q,
                             const tr_paged_kv* kv, int32_t layer, float scale, void* out,
                             void* ws, size_t ws_bytes, void* stream);

/* tr_step_ex with a paged cache: the commit copies the accepted rows of
 * every layer (kv->k_tree / v_tree) into positions prefix_len ..
 * prefix_len+L of each layer's pages; a commit past max_pages * page_size
 * is skipped with TR_FLAG_CACHE_FULL, a bad page id writes page 0 and sets
 * TR_FLAG_BAD_PAGE.  Everything else as tr_step_ex. */
tr_status tr_step_paged(const tr_tree* t, int32_t B, int64_t V, int32_t k, const void* logits,
                        tr_dtype l_dtype, void* M, tr_dtype m_dtype, int32_t* tree_tok,
                        int32_t* root_tok, int32_t* accept_len, int32_t* accept_path,
                        int32_t* emitted, const tr_paged_kv* kv, int32_t* topk_out,
                        tr_update_mode mode, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * LM head fused with the top-k (the logits are never written).  The update
 * M[x~_i] = argtopk(p~_{i+1}) needs only the k best ids of each node's
 * next-token distribution (Token Recycling, Chinese summary, Method), and
 * softmax is increasing, so they are the k best of the logits z = h W^T:
 *   h [rows][H] hidden states, W [V][H] output embedding, both bfloat16,
 *   device memory, 16-byte aligned; products accumulate in float32; ids
 *   ordered by z descending, ties to the lower id; H a multiple of 128,
 *   k <= 8.  Built for decode-sized rows (W is streamed once per 96 rows).
 * Workspace: tr_lmhead_workspace_size(rows, V, k) bytes (rows = B * nodes
 * for tr_step_lmhead), zeroed once with tr_workspace_init.
 * ------------------------------------------------------------------------ */
size_t tr_lmhead_workspace_size(int64_t rows, int64_t V, int32_t k);

/* topk_out [rows][k] int32.  Errors: TR_ERR_INVALID_ARGUMENT (null or
 * misaligned pointer, V outside k..2^31-1), TR_ERR_UNSUPPORTED (dtype not
 * bfloat16, H not a multiple of 128, k > 8, rows > 32768),
 * TR_ERR_WORKSPACE_TOO_SMALL. */
tr_status tr_lmhead_topk(int32_t rows, int32_t H, int64_t V, int32_t k, const void* h,
                         const void* W, tr_dtype dtype, int32_t* topk_out, void* ws,
                         size_t ws_bytes, void* stream);

/* tr_step_ex with the LM head in front: the top-k of every node comes from
 * h [B][T][H] and W instead of a logits tensor; everything after it
 * (verification, update, commit, next retrieval) and every other argument
 * as tr_step_ex.  Greedy verification only.  With fewer than 256 rows (B*T)
 * and V <= 32768 the slices' candidates are merged by the few-row step
 * launch of tr_step (TR_FEW_ROW_STEP=0 selects one merge block per row
 * instead; same results). */
tr_status tr_step_lmhead(const tr_tree* t, int32_t B, int32_t H, int64_t V, int32_t k,
                         const void* h, const void* W, tr_dtype dtype, void* M, tr_dtype m_dtype,
                         int32_t* tree_tok, int32_t* root_tok, int32_t* accept_len,
                         int32_t* accept_path, int32_t* emitted, int32_t Hkv, int32_t d,
                         tr_dtype kv_dtype, const void* k_tree, const void* v_tree, void* k_cache,
                         void* v_cache, int64_t cap, int32_t* prefix_len, int32_t* topk_out,
                         tr_update_mode mode, void* ws, size_t ws_bytes, void* stream);

/* Initial contents of M (Token Recycling, Method, first module: a hot start
 * inherits the matrix left by earlier inference instead of an empty one;
 * Experiment, initialisation ablation: all-zero, random ids, and prior
 * matrices, fixed, shuffled or inherited).  Not part of a step: called once
 * before decoding starts.
 *   M [B][V][k] in m_dtype (int32 or int64), device memory, 16-byte aligned.
 *   TR_INIT_ZERO    every id 0.
 *   TR_INIT_RANDOM  id e (flat index over [B][V][k]) = floor(u_e * V), u_e =
 *                   (z_e >> 32) / 2^32, z_e = output e of SplitMix64 seeded
 *                   with seed: the mix of seed + (e+1) * 0x9E3779B97F4A7C15
 *                   (Steele, Lea and Flood, OOPSLA 2014).
 *   TR_INIT_PRIOR   M[b] = prior[prior_batches == 1 ? 0 : b]; prior is
 *                   [prior_batches][V][k] in prior_dtype (int32 or int64),
 *                   device memory, 16-byte aligned, prior_batches 1 (one
 *                   prior for every sequence: fixed or shuffled priors) or B
 *                   (each sequence its own: inherited).  Ids are converted to
 *                   m_dtype as they are; ids outside [0, V) are flagged by
 *                   the retrieval that reads them.  prior must not overlap M.
 * prior and prior_dtype are ignored by the other modes, seed by all but
 * RANDOM.  Errors: TR_ERR_INVALID_ARGUMENT for a null or misaligned tensor,
 * B, V or k below 1, V above 2^31-1, an unknown mode or prior_batches not 1
 * or B; TR_ERR_UNSUPPORTED for other dtypes.  Launches one kernel on stream. */
typedef enum {
  TR_INIT_ZERO = 0,
  TR_INIT_RANDOM = 1,
  TR_INIT_PRIOR = 2
} tr_init_mode;

tr_status tr_init_matrix(int32_t B, int64_t V, int32_t k, void* M, tr_dtype m_dtype,
                         tr_init_mode mode, const void* prior, tr_dtype prior_dtype,
                         int32_t prior_batches, uint64_t seed, void* stream);

/* ------------------------------------------------------------------------
 * Profiling aid (outside the TR step).  While enabled, each kernel the
 * library launches is bracketed by two HIP events recorded on the stream it
 * is launched on, so the elapsed time between them is that launch's time on
 * the device.  tr_profile_read synchronises on the recorded events, writes
 * up to max (kernel, milliseconds) records in launch order, forgets all
 * records and returns how many it wrote.  At most 16384 launches are kept
 * between reads (later ones are not recorded).  tr_profile_enable creates
 * the events (hipEventCreate) the first time it is turned on.  Not
 * thread-safe: one host thread drives the library while profiling.
 * ------------------------------------------------------------------------ */
typedef enum {
  TR_KERNEL_ATTN_PREFIX = 1,   /* tr_tree_attn, prefix chunks */
  TR_KERNEL_ATTN_COMBINE = 2,  /* tr_tree_attn, merge of chunks and tree keys */
  TR_KERNEL_TOPK = 3,          /* tr_step / tr_update_topk (top-k and tail) */
  TR_KERNEL_RETRIEVE = 4,      /* tr_retrieve */
  TR_KERNEL_VERIFY = 5,        /* tr_verify */
  TR_KERNEL_FILL = 6,          /* tr_workspace_init */
  TR_KERNEL_INIT = 7,          /* tr_init_matrix */
  TR_KERNEL_LMHEAD = 8,        /* tr_lmhead_topk / tr_step_lmhead: product and slice top-k */
  TR_KERNEL_LMHEAD_MERGE = 9,  /* tr_lmhead_topk / tr_step_lmhead: merge (and tail) */
  TR_KERNEL_READ_PROBE = 10    /* tr_read_probe */
} tr_kernel_id;

typedef struct {
  int32_t kernel;              /* tr_kernel_id */
  float ms;
} tr_launch_time;

tr_status tr_profile_enable(int32_t on);
int32_t tr_profile_read(tr_launch_time* out, int32_t max);

/* Achievable streaming-read bandwidth (a sanity denominator for the
 * kernels' HBM figures, not a TR step): one kernel reads every byte of
 * src [bytes] once with non-temporal 16-byte loads and folds them into
 * sink [2048] uint32 (device memory, XOR-accumulated, contents meaningless).
 * Time it with tr_profile_enable (kernel TR_KERNEL_READ_PROBE).  Errors:
 * TR_ERR_INVALID_ARGUMENT for a null or misaligned pointer or a size that
 * is not a positive multiple of 16. */
tr_status tr_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TR_H */
