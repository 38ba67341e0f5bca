/*
 * eagle_mi355x.h -- C ABI of the MI355X (gfx950) EAGLE-2 draft-round library.
 *
 * One round of EAGLE feature-level drafting with EAGLE-2 dynamic draft trees:
 *   eagle_draft_level(level = 1)          LM-head tail on the root's draft feature
 *   eagle_draft_level(level = 2..depth)   draft forward on the k frontier nodes,
 *                                         LM head, softmax, top-k, k*k -> k select
 *   eagle_rerank_build_tree               top m-1 of every candidate + the root,
 *                                         flattened, ancestor-only mask, positions
 *   eagle_draft_level_static,             a static (fixed-shape) tree instead: the
 *   eagle_build_static_tree               template picks each level's children
 *   eagle_verify_greedy                   greedy longest-accepted-path walk
 *   eagle_verify_rejection                recursive rejection sampling of sampled
 *                                         children (lossless for i.i.d. draws)
 *   eagle_verify_rejection_topk           the same for deterministic (top-k or
 *                                         template) children (lossless)
 *   eagle_verify_relaxed                  threshold acceptance on the target's
 *                                         probabilities, residual draw for the bonus
 *   eagle_draft_extend                    draft forward over the accepted path with
 *                                         the target's true features, KV append
 *
 * Sources, cited by title and section:
 *   [P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）" (study notes)
 *   [P2] "(EAGLE 1)EAGLE: Speculative Sampling Requires Rethinking Feature Uncertainty"
 *   [P3] Medusa -> EAGLE -> EAGLE-2 notes, zdszero.github.io "spec_medusa_eagle"
 *   [P4] "投机解码：从eagle1到dflash" (EAGLE-2 flow diagram)
 *
 * Conventions shared by every entry point
 *   Ownership  Every pointer is a device buffer owned by the caller (weights,
 *              state, outputs, workspace).  The library allocates no device
 *              memory and keeps no state between calls except a thread-local
 *              error string.
 *   Execution  Calls are asynchronous on `stream` (a hipStream_t; NULL = the
 *              default stream) and never synchronise.  A round's calls must be
 *              issued in round order on one stream; `ws` carries the round's
 *              state (frontier, candidate pool, draft features, in-tree KV)
 *              between calls and must not be used by two rounds at once.
 *              Nothing in a round waits on the host, so a whole round can be
 *              captured into one HIP graph.
 *   Errors     0 = OK, negative = eagle_status.  Every shape, pointer and size
 *              check runs on the host before any launch; a failing call
 *              launches nothing.  Launch failures return EAGLE_ERR_HIP.  The
 *              reason is in eagle_last_error().  Bad data found on the device
 *              (a token id outside [0, vocab), a prefix length outside
 *              [1, max_prefix - m]) is clamped and recorded in the workspace
 *              error word (eagle_ws_view(EAGLE_WS_ERROR)); it never traps.
 *   Types      dims.dtype applies to weights, features, K/V and the workspace
 *              feature/KV regions.  Logits, scores and log-probabilities are
 *              fp32; indices are int32; the tree mask is uint8.  All matrices
 *              are row-major.
 */
#ifndef EAGLE_MI355X_H
#define EAGLE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EAGLE_OK = 0,
    EAGLE_ERR_ARG = -1,          /* null pointer, bad enum, level out of range   */
    EAGLE_ERR_SHAPE = -2,        /* dims / tree config inconsistent              */
    EAGLE_ERR_UNSUPPORTED = -3,  /* valid but outside what the kernels cover     */
    EAGLE_ERR_WORKSPACE = -4,    /* ws_bytes < eagle_workspace_bytes()           */
    EAGLE_ERR_HIP = -5           /* a HIP launch failed                          */
} eagle_status;

typedef enum { EAGLE_F32 = 0, EAGLE_BF16 = 1 } eagle_dtype;

#define EAGLE_MAX_DEPTH 16
#define EAGLE_MAX_TOPK 16
#define EAGLE_MAX_TREE 64

/* Model shapes.  d == n_heads * head_dim; n_heads % n_kv_heads == 0 (GQA when
 * n_kv_heads < n_heads); head_dim in {64, 128}; ffn % 8 == 0.  The draft head
 * is FC(2d -> d, bias) + one Llama decoder layer whose first input norm is the
 * identity and which has no final norm ([P3] "在 SGLang 里"); embedding and LM
 * head are the target's ([P1] §4.1 components).  rms_eps (e.g. 1e-6) is the
 * post-attention RMSNorm epsilon; rope_theta (e.g. 1e4) the rotary base. */
typedef struct {
    int32_t d, n_heads, n_kv_heads, head_dim, ffn, vocab;
    int32_t dtype;               /* eagle_dtype */
    float rms_eps, rope_theta;
} eagle_dims;

/* Draft-head weights (all dims.dtype).  As the caller holds them (row-major,
 * Linear convention [out][in]):
 *   fc_w [d][2d]   columns 0..d-1 take the feature, d..2d-1 the token embedding
 *                  ([P1] §4.1 input = [f_j || e(t_{j+1})]);
 *   fc_b [d];  wq [H*hd][d];  wk, wv [Hkv*hd][d];  wo [d][H*hd];
 *   post_norm [d] (RMSNorm gain);  w_gate, w_up [ffn][d];  w_down [d][ffn];
 *   embed [vocab][d] and lm_head [vocab][d]: the target's, shared and frozen.
 * The drafting calls stream wq, wk, wv, wo, w_gate, w_up, w_down, lm_head and
 * the feature half of fc_w once per pass and take them in the packed layout
 * that eagle_pack_weights writes (packed == EAGLE_PACKED_WEIGHTS); fc_b,
 * post_norm and embed stay row-major.  `packed` is 0 for row-major sources,
 * whose tok_proj is ignored. */
typedef struct {
    const void *fc_w, *fc_b, *wq, *wk, *wv, *wo, *post_norm, *w_gate, *w_up, *w_down;
    const void *embed, *lm_head;
    const void *tok_proj;        /* packed only: fp32 [vocab][d], see eagle_pack_weights */
    int32_t packed;
} eagle_weights;

#define EAGLE_PACKED_WEIGHTS 0x45505731  /* marks a struct filled by eagle_pack_weights */

/* Tree shape: (depth, topk, m) = SGLang's (num-steps, eagle-topk,
 * num-draft-tokens) ([P3] "在 SGLang 里"); m counts the root.
 * 1 <= batch; 2 <= depth <= 16; 1 <= topk <= 16; 2 <= m <= 64;
 * m - 1 <= topk + (depth - 1) * topk^2; max_prefix = rows of the KV cache. */
typedef struct {
    int32_t batch, depth, topk, m, max_prefix;
} eagle_tree_cfg;

/* Per-sequence decoding state, owned by the caller and updated by the extend.
 *   k_cache, v_cache [batch][max_prefix][Hkv][hd] (dtype): the draft's KV for
 *       the accepted prefix, keys stored after RoPE.  Rows 0..prefix_len-1 are
 *       valid; the last of them is the root row.
 *   prefix_len [batch] int32; needs 1 <= prefix_len <= max_prefix - m.
 *   root_feat [batch][d] (dtype): the draft feature predicted at the root row,
 *       whose LM head gives level 1 (written by the previous extend).
 *   root_token [batch] int32: the root token (the previous round's bonus). */
typedef struct {
    void *k_cache, *v_cache;
    int32_t *prefix_len;
    void *root_feat;
    int32_t *root_token;
} eagle_seq_state;

/* Workspace records (readable through eagle_ws_view). */
typedef struct {
    float score;      /* sum of draft log-probabilities along the root path     */
    float logp;       /* this node's own draft log-probability                  */
    int32_t token;
    int32_t parent;   /* pool index of the parent; -1 for children of the root  */
    int32_t depth;    /* 1..depth                                               */
    int32_t pslot;    /* frontier slot of the parent at its level; -1: the root */
} eagle_pool_entry;   /* pool of a sequence: [topk + (depth-1)*topk^2] entries  */

typedef struct {
    int32_t token;
    float score;
    int32_t pool_idx;
    int32_t pslot;                   /* frontier slot of the parent (-1: root)  */
    int32_t anc[EAGLE_MAX_DEPTH];    /* anc[i] = frontier slot of the ancestor  */
                                     /* at depth i+1 (the last one is itself)   */
} eagle_frontier_node;

/* Packed weights (one-time set-up, like loading a checkpoint).  Each streamed
 * matrix W [N][K] becomes tiles of 16 output rows x KS inputs (KS = 32 for
 * bf16, 16 for fp32): one kilobyte, the operand of one 16x16 MFMA step, stored
 * in the order the 64 lanes of a wave load it (lane l = 16g + c holds row c,
 * inputs g*16/elem .. of the tile), tiles of one row block consecutive along K
 * (tile (t, s) at ((t * ceil(K/KS)) + s) * 16 * KS elements).  A wave's load
 * is then one contiguous kilobyte instead of 16 rows of 64 bytes.  Rows and K
 * are padded with zeros to whole tiles.  wq, wk, wv tiles hold 8 RoPE pairs of
 * one head: tile j of a head holds its rows 8j..8j+7 and hd/2+8j..hd/2+8j+7,
 * so that the rotation stays within a lane's columns; every other matrix's
 * tile t holds rows 16t..16t+15.  Only the feature half of fc_w (its columns
 * 0..d-1, as a [d][d] matrix) is packed.  The token half enters through the
 * token-projection table tok_proj [vocab][d] fp32, tok_proj[v] = fc_w[:, d:2d]
 * * embed[v] (fp32 sums of the exact products), written here: the FC of a
 * row [f || e(t)] is W_fc[:, :d] f + tok_proj[t] + fc_b ([P1] §4.1 input
 * equation; the product of a matrix with a concatenation is the sum of its
 * column blocks' products), so the drafting calls read one table row per row
 * instead of streaming the token half of fc_w.
 * eagle_packed_weights_bytes: bytes of the packed buffer (each matrix and
 * the table at a 256-byte-aligned offset); 0 if dims are invalid.
 * eagle_pack_weights: src holds the row-major matrices (src->packed == 0);
 * dst is device memory of at least that many bytes, 256-byte aligned, owned
 * by the caller and left untouched by the drafting calls.  Fills *out with
 * pointers into dst (and src's fc_b, post_norm, embed) and sets out->packed.
 * src's matrices are read by kernels on `stream`: keep them until that work
 * is done.
 * Returns EAGLE_ERR_ARG on NULL pointers or a misaligned dst,
 * EAGLE_ERR_WORKSPACE if dst_bytes is too small; launches on `stream`. */
size_t eagle_packed_weights_bytes(const eagle_dims *dims);
int eagle_pack_weights(const eagle_dims *dims, const eagle_weights *src, void *dst, size_t dst_bytes,
                       eagle_weights *out, void *stream);

/* Bytes of workspace for (dims, cfg); 0 if they are invalid. */
size_t eagle_workspace_bytes(const eagle_dims *dims, const eagle_tree_cfg *cfg);

/* Zero the workspace (counters and error word must start at zero) and write
 * the RoPE frequency table (theta^(-2i/hd) in fp64) it holds.  Call once after
 * allocating it; every kernel leaves its counters at zero again. */
int eagle_workspace_init(const eagle_dims *dims, const eagle_tree_cfg *cfg, void *ws,
                         size_t ws_bytes, void *stream);

#define EAGLE_LEVEL_FULL 0
#define EAGLE_LEVEL_TAIL_ONLY 1   /* level >= 2: skip the forward and run the LM-head
                                     tail + select on the features already in the
                                     workspace (EAGLE_WS_FEAT, depth level-1) */
#define EAGLE_LEVEL_LMHEAD_ONLY 2 /* timing and counter runs: launch only the LM-head
                                     GEMM stage of the tail (per-slab softmax and
                                     top-k partials in the workspace); the pool and
                                     frontier are NOT updated, so a level run this way
                                     must be run again with FULL or TAIL_ONLY before
                                     the round continues */
#define EAGLE_LEVEL_FULL_FC 3     /* level >= 2: FULL, and compute this level's FC input
                                     x0 in this call (see "FC hand-over" below) */

/* One tree level ([P1] §10.3 expansion; [P3] select_top_k_tokens).
 * level 1: LM head + softmax + top-k on root_feat; the k children of each
 *   root enter the pool and form frontier depth 1.  The first level's top-k
 *   comes from the previous round's extend ([P3] "在 SGLang 里").
 * level L >= 2: for each node x of frontier depth L-1 the row
 *   [feature of x's parent || embed[token(x)]] goes through FC + bias, q/k/v,
 *   RoPE at position prefix_len-1+(L-1), attention over all prefix rows plus
 *   the in-tree K/V of x's ancestors and x itself (ancestor-only mask,
 *   [P1] §12 item 5), o-projection + residual, RMSNorm, SwiGLU + residual
 *   ([P1] §4.1; [P2] Core Idea; [P3]).  The predicted features go to
 *   EAGLE_WS_FEAT depth L-1 and the row's K/V to the in-tree slots.  Then LM
 *   head, softmax, top-k per row; child score = parent score + log p (the
 *   path product of [P1] §10.3 in the log domain); all k*k children join the
 *   pool in (frontier slot, rank) order, and the best k by (score desc, pool
 *   index asc) form frontier depth L.
 * Levels must run 1, 2, ..., depth in order within a round.  w: packed
 * weights (eagle_pack_weights; EAGLE_ERR_ARG otherwise).
 * FC hand-over: when batch * topk <= 16, the FC input of level L+1 (x0 of the
 * next frontier) is computed by level L's call (FULL or TAIL_ONLY, L < depth):
 * its LM-head merge launch also streams the feature half of the FC over level
 * L's rows, and once the next frontier is chosen forms x0 = W_fc[:, :d] h(parent)
 * + tok_proj[token] + fc_b.  Level L+1 (FULL) then starts at q/k/v.  A caller
 * that writes the frontier or the features of the parents into the workspace
 * itself runs level L+1 with EAGLE_LEVEL_FULL_FC, which computes x0 in that
 * call.  With batch * topk > 16 every FULL level computes its own FC. */
int eagle_draft_level(const eagle_dims *dims, const eagle_weights *w,
                      const eagle_tree_cfg *cfg, const eagle_seq_state *state,
                      int32_t level, int32_t flags, void *ws, size_t ws_bytes,
                      void *stream);

/* eagle_draft_level, with the LM-head GEMM kernel of the call launched so that
 * start_event and stop_event (hipEvent_t, created by the caller with timing
 * enabled; either may be NULL) are stamped when that one kernel starts and
 * when it ends (hipExtLaunchKernel), rather than where the events would sit
 * in the stream's queue: it times the kernel alone, with no queue overhead.
 * Same arguments, outputs and errors as eagle_draft_level otherwise.  For
 * timing runs; not meant for graph capture. */
int eagle_draft_level_timed(const eagle_dims *dims, const eagle_weights *w,
                            const eagle_tree_cfg *cfg, const eagle_seq_state *state,
                            int32_t level, int32_t flags, void *ws, size_t ws_bytes,
                            void *start_event, void *stop_event, void *stream);

/* Target-side tree-verify attention ([P1] §6.2: the target scores every tree
 * node in one forward with tree attention; [P4] EAGLE-2 diagram, stage two: the
 * flattened tree is fed with the ancestor-only mask and per-node positions).
 * The target's attention over the m flattened tree tokens of each sequence:
 *   q        device fp32 [batch][m][n_heads][head_dim], post-RoPE at the node
 *            positions (prefix_len-1+depth), row i = flat node i;
 *   k_cache, v_cache  device dtype [batch][max_prefix][n_kv_heads][head_dim]:
 *            rows 0..prefix_len-1 hold the prefix, rows prefix_len..prefix_len+m-1
 *            the tree tokens' keys and values (flat order, post-RoPE);
 *   prefix_len  device int32 [batch] (clamped to 1..max_prefix-m and flagged in
 *            the workspace error word, as everywhere);
 *   mask     device uint8 [batch][m][m], as eagle_rerank_build_tree writes it
 *            (nonzero: the column node is an ancestor of the row node or itself);
 *   out      device dtype [batch][m][n_heads*head_dim].
 * Query (i, head h) attends, scaled by 1/sqrt(head_dim), to every prefix row and
 * to tree row j iff mask[i][j] != 0, with KV head h*n_kv_heads/n_heads.  Uses
 * the workspace of (dims, cfg) for split partials; depth and topk of cfg are
 * validated but not used.  Errors: EAGLE_ERR_ARG for NULL pointers, the usual
 * shape/workspace errors, EAGLE_ERR_HIP if the launch fails. */
int eagle_tree_verify_attention(const eagle_dims *dims, const eagle_tree_cfg *cfg, const float *q,
                                const void *k_cache, const void *v_cache, const int32_t *prefix_len,
                                const uint8_t *mask, void *out, void *ws, size_t ws_bytes,
                                void *stream);

/* Static draft tree ([P1] §10.1: EAGLE-1 and Medusa draft on a tree of fixed
 * shape, a fixed number of candidates per level, chosen once for every
 * input).  The tree is a template of topk slots per depth: depth 1 is the
 * root's top-k in rank order; slot j of depth L >= 2 is the child of rank
 * tmpl[L-1][j][1] (in its parent's top-k order, logit desc, id asc) of slot
 * tmpl[L-1][j][0] of depth L-1, whatever its score.
 * eagle_draft_level_static is eagle_draft_level with that selection in place
 * of the k*k -> k select (the draft forward, LM head, softmax, top-k and the
 * pool are unchanged).  tmpl: device int32 [depth][topk][2] (row 0 unused),
 * entries clamped into 0..topk-1; the pairs of one depth should be distinct.
 * Level 1 ignores tmpl.  eagle_build_static_tree then writes the tree from
 * the frontiers the levels left in ws: root first, then depth-major, then
 * slot order (node (L, j) at flat index 1 + (L-1)*topk + j), the first m
 * nodes (m <= 1 + depth*topk); outputs as for eagle_rerank_build_tree
 * (node_logscore = the node's path score). */
int eagle_draft_level_static(const eagle_dims *dims, const eagle_weights *w,
                             const eagle_tree_cfg *cfg, const eagle_seq_state *state,
                             int32_t level, int32_t flags, const int32_t *tmpl, void *ws,
                             size_t ws_bytes, void *stream);
int eagle_build_static_tree(const eagle_dims *dims, const eagle_tree_cfg *cfg,
                            const eagle_seq_state *state, void *ws, size_t ws_bytes,
                            int32_t *tokens, int32_t *parents, int32_t *depth, int32_t *positions,
                            uint8_t *mask, float *node_logscore, void *stream);

/* Rerank and build ([P1] §10.3 rerank; [P3] organize_draft_results and
 * build_tree_kernel_efficient; [P4] EAGLE-2 diagram).  Per sequence: the best
 * m-1 pool entries by (score desc, depth asc, pool index asc) plus the root;
 * flattened root first, then depth-major, then by parent's flat index, then
 * by child rank.  Outputs (device, [batch][m] unless noted):
 *   tokens, parents (flat index, -1 for the root), depth, positions
 *   (prefix_len-1+depth), mask [batch][m][m] uint8 (1 iff column is an
 *   ancestor of the row or the row itself), node_logscore (0 for the root).
 * Any output pointer except tokens and parents may be NULL. */
int eagle_rerank_build_tree(const eagle_dims *dims, const eagle_tree_cfg *cfg,
                            const eagle_seq_state *state, void *ws, size_t ws_bytes,
                            int32_t *tokens, int32_t *parents, int32_t *depth,
                            int32_t *positions, uint8_t *mask, float *node_logscore,
                            void *stream);

/* Greedy verification ([P4] EAGLE-2 diagram: accept the longest consistent
 * path, back off to the last accepted node).  target_logits [batch][m][vocab]
 * fp32 are the target's logits at each flat tree node.  From the root: t* =
 * argmax of the current node's row (lowest id on exact ties); if a child has
 * token t*, descend, else stop.  Outputs: accept_len [batch] = nodes on the
 * path including the root (accepted drafts + 1); accept_path [batch][depth+1]
 * flat indices, -1 after the end; bonus [batch] = t* at the stop. */
int eagle_verify_greedy(const eagle_tree_cfg *cfg, int32_t vocab, const float *target_logits,
                        const int32_t *tokens, const int32_t *parents, int32_t *accept_len,
                        int32_t *accept_path, int32_t *bonus, void *stream);

/* Strict verification by recursive rejection sampling ([P1] §6.2: accept a
 * drafted token t iff u <= min(1, p(t)/q(t)), otherwise resample from
 * norm(max(0, p - q)), node by node).  Precondition for losslessness: the
 * children of each node were drawn independently from q at that node (a
 * sampled tree).  The result is then distributed exactly as the target.  The
 * trees this library builds are deterministic (EAGLE-2's top-k, or a static
 * template): verify those with eagle_verify_rejection_topk below, for which
 * this call's output is NOT distributed as the target (a single child t with
 * q(t) = p(t) = 0.5 is always emitted, not half of the time).
 * p = softmax(target_logits[node] / temperature) and q =
 * softmax(draft_logits[node] / temperature), both [batch][m][vocab] fp32 (the
 * draft's logits at every flat tree node, kept by the caller; every row is
 * read).  From the root, the node's children are tried in flat order,
 * child c accepted iff p(t_c) > 0 and uniforms[b][c] * q(t_c) <= p(t_c)
 * (a token the current p gives no mass is never accepted, whatever q is);
 * after each rejection p <- norm(max(0, p - q)) (kept when that has no mass); when every
 * child is rejected (or the node is a leaf, or the path already holds depth+1
 * nodes) the bonus is the smallest id whose cumulative p exceeds
 * uniforms[b][m] (clamped into [0, 1)).  uniforms: device fp32
 * [batch][m+1], the caller's random numbers.  scratch: device buffer of at
 * least eagle_verify_rejection_scratch_bytes(cfg, vocab) bytes, 8-byte
 * aligned (softmax statistics of every row, per id range), owned by the caller
 * and overwritten.  Outputs as for
 * eagle_verify_greedy.  batch*m at most 65535. */
size_t eagle_verify_rejection_scratch_bytes(const eagle_tree_cfg *cfg, int32_t vocab);
int eagle_verify_rejection(const eagle_tree_cfg *cfg, int32_t vocab, const float *target_logits,
                           const float *draft_logits, const int32_t *tokens,
                           const int32_t *parents, float temperature, const float *uniforms,
                           int32_t *accept_len, int32_t *accept_path, int32_t *bonus,
                           void *scratch, size_t scratch_bytes, void *stream);

/* Strict rejection sampling of deterministic candidates ([P1] §6.2, with
 * each drafted child taken as a point-mass proposal: the draft's top-k
 * children, or a static template's, are a fixed list and not draws from q).
 * p = softmax(target_logits[node] / temperature).  From the root, the node's
 * children are tried in flat order: child c is accepted iff
 * uniforms[b][c] * (1 - mass of the tokens of the children tried before it)
 * <= p(t_c) and p(t_c) > 0, i.e. with the probability the current residual
 * (p with the rejected tokens removed, renormalised) gives t_c; a token that
 * an earlier sibling already carries is rejected.  When every child is
 * rejected (or the node is a leaf, or the path already holds depth+1 nodes)
 * the bonus is drawn from that residual (p with the node's children removed;
 * p itself if they held all the mass) by inverse CDF with uniforms[b][m]: the
 * emitted token is distributed exactly as the target for any fixed list of
 * candidates.  Same arguments as eagle_verify_relaxed (its scratch size too),
 * without the threshold, and uniforms [batch][m+1] as for
 * eagle_verify_rejection.  Outputs as for eagle_verify_greedy.  batch*m at
 * most 65535. */
int eagle_verify_rejection_topk(const eagle_tree_cfg *cfg, int32_t vocab, const float *target_logits,
                                const int32_t *tokens, const int32_t *parents, float temperature,
                                const float *uniforms, int32_t *accept_len, int32_t *accept_path,
                                int32_t *bonus, void *scratch, size_t scratch_bytes, void *stream);

/* eagle_verify_rejection_topk for callers that cannot allocate (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same call without the scratch argument.  Its per-segment softmax
 * statistics live in a device array inside the library, of
 * EAGLE_NOALLOC_MAX_ROWS * 128 bytes (512 KB) on each device it runs on, kept
 * until the process ends; the call allocates nothing (no hipMalloc or
 * allocating library routine).  batch * m must be at most
 * EAGLE_NOALLOC_MAX_ROWS, else EAGLE_ERR_UNSUPPORTED.  The array is found on
 * the calling thread's current device, which must be the stream's.  Every
 * call on a device shares that device's array: calls that overlap on one
 * device (other streams, other threads) race and must be ordered by the
 * caller.  Nothing in it needs to start at zero (every statistic is written
 * before it is read).  Errors and outputs as for eagle_verify_rejection_topk,
 * plus EAGLE_ERR_HIP if the array's address cannot be obtained. */
#define EAGLE_NOALLOC_MAX_ROWS 4096
int eagle_verify_rejection_topk_noalloc(const eagle_tree_cfg *cfg, int32_t vocab, const float *target_logits,
                                        const int32_t *tokens, const int32_t *parents, float temperature,
                                        const float *uniforms, int32_t *accept_len, int32_t *accept_path,
                                        int32_t *bonus, void *stream);

/* Relaxed acceptance ([P2] closing notes on SGLang's verification: the
 * target's probabilities and a probability threshold decide whether a token
 * is accepted; only when every candidate of a level fails is one
 * rejection-sampling draw made there, for the bonus token).  From the root:
 * p = softmax(target_logits[node] / temperature) in fp32; the node's children
 * are tried in flat order and the walk descends to the first child c with
 * p(c) >= threshold.  When none passes (or the node has no children, or the
 * path already holds depth+1 nodes) the bonus is drawn from p with the
 * node's children removed and the rest renormalised: the smallest token id
 * whose cumulative residual mass exceeds u * (residual total), u =
 * uniforms[b] clamped into [0, 1); if the children held all of p's mass the
 * draw is from p itself.  Inputs as for eagle_verify_greedy, plus
 * temperature (> 0, finite), threshold (finite; <= 0 accepts every first
 * child, > 1 none) and uniforms [batch] fp32 (device; the caller's random
 * numbers, one per sequence).  scratch: device buffer of at least
 * eagle_verify_relaxed_scratch_bytes(cfg) bytes, 8-byte aligned, owned by the
 * caller and overwritten (the per-segment softmax statistics of every tree
 * row).  Outputs as for eagle_verify_greedy.  Logits of -inf carry no
 * probability; a stop row whose logits are all -inf (no distribution) gives
 * bonus 0.  batch*m at most 65535. */
size_t eagle_verify_relaxed_scratch_bytes(const eagle_tree_cfg *cfg);   /* 0 if cfg is invalid */
int eagle_verify_relaxed(const eagle_tree_cfg *cfg, int32_t vocab, const float *target_logits,
                         const int32_t *tokens, const int32_t *parents, float temperature,
                         float threshold, const float *uniforms, int32_t *accept_len,
                         int32_t *accept_path, int32_t *bonus, void *scratch, size_t scratch_bytes,
                         void *stream);

/* Draft extend ([P3] "在 SGLang 里": rerun the draft over the accepted
 * positions with the target's true hidden states, take row accept_len-1 as
 * the next start; [P2] Core Idea; [P1] §12 item 3).  Row i < accept_len
 * carries [true_feat[path_i] || embed[token of path_{i+1}, or the bonus for
 * the last row]] at position prefix_len+i and attends the prefix plus extend
 * rows 0..i.  An accepted path has at most min(m, depth+1) nodes, so each
 * sequence forwards re = min(m, depth+1) rows (rows past accept_len are
 * computed and ignored).  Updates the state: K/V rows
 * prefix_len..prefix_len+re-1 written (the first accept_len are valid),
 * prefix_len += accept_len, root_feat = feature of row accept_len-1,
 * root_token = bonus.  accept_len is clamped to 1..re.
 * true_feat [batch][m][d] (dtype) are the target's features at each flat
 * tree node; tokens [batch][m], accept_len, accept_path, bonus as produced
 * by the calls above.  w: packed weights, as for eagle_draft_level. */
int eagle_draft_extend(const eagle_dims *dims, const eagle_weights *w,
                       const eagle_tree_cfg *cfg, const eagle_seq_state *state,
                       const void *true_feat, const int32_t *tokens, const int32_t *accept_len,
                       const int32_t *accept_path, const int32_t *bonus, void *ws,
                       size_t ws_bytes, void *stream);

const char *eagle_status_str(int status);
const char *eagle_last_error(void);   /* thread-local text of the last failure */

/* Workspace regions, for tests and debugging. */
typedef enum {
    EAGLE_WS_ERROR = 0,     /* int32[4]; [0] bit 0: token id clamped, bit 1: prefix_len clamped,
                               bit 2: a bounded wait of the FC hand-over gave up (never
                               expected; the next level's input is then not valid) */
    EAGLE_WS_POOL = 1,      /* eagle_pool_entry [batch][pool]                        */
    EAGLE_WS_FRONTIER = 2,  /* eagle_frontier_node [depth+1][batch][topk] (by depth)  */
    EAGLE_WS_FEAT = 3,      /* dtype [depth][batch][topk][d]: features of frontier nodes */
    EAGLE_WS_TREE_K = 4,    /* fp32 [batch][depth][topk][Hkv][hd]: in-tree keys (post-RoPE) */
    EAGLE_WS_TREE_V = 5,    /* fp32 [batch][depth][topk][Hkv][hd]: in-tree values     */
    EAGLE_WS_EXT_H = 6,     /* dtype [batch][min(m, depth+1)][d]: extend output features */
    /* the last layer pass's intermediates (a level's or the extend's rows, R of them:
       batch*topk, batch*min(m, depth+1) or batch), row-major over the first R rows */
    EAGLE_WS_X0 = 7,        /* fp32 [R][d]: FC output x0 (after the bias)            */
    EAGLE_WS_ATTN = 8,      /* dtype [R][n_heads*head_dim]: attention output          */
    EAGLE_WS_Y = 9          /* fp32 [R][d]: x0 + o-projection (the post-attention stream) */
} eagle_ws_region;

int eagle_ws_view(const eagle_dims *dims, const eagle_tree_cfg *cfg, const void *ws,
                  int32_t what, void **ptr, size_t *bytes);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE_MI355X_H */
