/*
 * tree_verify.h -- C ABI of libtv.so: DDTree tree-verify attention and greedy
 * acceptance on MI355X (gfx950).
 *
 * The method (Luce DFlash pages: "Luce DFlash: 単一RTX 3090で最大2倍の
 * スループットを目指すQwen3.6-27B", feature list; "We got 207 tok/s with
 * Qwen3.5-27B on an RTX 3090", claims and "What we built vs what we didn't"):
 * a DFlash draft proposes a DDTree of draft tokens (budget 22, i.e. 23 nodes
 * with the root, block size 16); the target model scores every node of the
 * tree in a single verify pass; verification is greedy. The KV cache of the
 * target is F16 or Q4_0 (the Q4_0 path reaches about 128K context), and decode
 * may restrict attention to a sliding window of 2048 tokens.
 *
 * This library implements the data-parallel core of that verify pass:
 *   tree_verify_attn  one attention layer of the verify pass: every tree node
 *                     attends to the committed cache rows (inside the window)
 *                     and to its own tree ancestors, itself included;
 *   tree_accept       greedy acceptance: per-node argmax over the vocabulary
 *                     and the longest root path whose draft tokens match;
 *   tree_commit_kv    the step after acceptance: the accepted path's K/V
 *                     rows appended to one layer's cache (Q4_0 or F16);
 *                     tree_commit_kv_layers does every layer in one launch.
 *
 * Conventions shared by all calls
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream). Results are valid once the stream has been synchronised.
 *   - The library allocates no device memory. Inputs, outputs and workspaces
 *     belong to the caller and must stay alive until the stream reaches them.
 *   - Host arrays passed in (parent, tokens) are read during the call only.
 *   - Every argument check runs on the host before anything is launched; on
 *     an error nothing is launched and no output is written.
 *   - Apart from tree_accept_noalloc's per-device acceptance array (see
 *     there) and a per-device cache of the compute-unit count, the library
 *     keeps no mutable global state; calls from several threads on
 *     different streams with their own outputs and workspaces are safe.
 */
#ifndef TREE_VERIFY_H
#define TREE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_API __attribute__((visibility("default")))

/* Status codes. */
#define TV_OK 0
#define TV_E_ARG (-1)       /* null pointer, bad enum, non-positive scale, ... */
#define TV_E_TREE (-2)      /* parent array is not a rooted topological tree   */
#define TV_E_SHAPE (-3)     /* head counts / head_dim / sizes not supported    */
#define TV_E_ALIGN (-4)     /* pointer or stride misaligned                    */
#define TV_E_WORKSPACE (-5) /* workspace missing or too small                  */
#define TV_E_HIP (-6)       /* a HIP runtime call or kernel launch failed      */

/* KV cache storage types. */
#define TV_KV_F16 0  /* IEEE binary16, one row = head_dim values             */
#define TV_KV_Q4_0 1 /* ggml Q4_0: per 32 values an 18-byte block = fp16
                        scale (little endian) + 16 code bytes; element e
                        (0..15) of a block is the low nibble of code byte e,
                        element e+16 its high nibble; value = scale*(code-8) */

#define TV_MAX_NODES 64

/*
 * Shape of one verify-attention layer.
 *
 * n_nodes      tree size, 1..TV_MAX_NODES (budget 22 -> 23). Node 0 is the
 *              root: the last emitted token, whose K/V are not yet in the
 *              cache.
 * parent       HOST int32[n_nodes]: parent[0] == -1 and 0 <= parent[i] < i
 *              (topological numbering); anything else is TV_E_TREE.
 * n_q_heads    query heads H_q; n_kv_heads H_kv divides it. Query head h
 *              reads KV head h / (H_q / H_kv).
 * head_dim     64, 128 or 256.
 * kv_type      TV_KV_F16 or TV_KV_Q4_0.
 * n_ctx        committed cache rows (>= 0).
 * window       0: attend to all rows; W > 0: only to rows
 *              [max(0, n_ctx - W), n_ctx). The window counts cache rows only;
 *              every node also sees all of its ancestors.
 * window_mode  0: the window above, the same for every node. 1: per
 *              position: a node at depth k (position n_ctx + k) sees the
 *              positions [n_ctx + k - W, n_ctx + k] of its own sequence, i.e.
 *              cache rows [max(0, n_ctx + k - W), n_ctx) and its ancestors at
 *              depth >= k - W: the keys that position has in token-by-token
 *              decoding with window W. No effect when window == 0.
 * kv_token_stride  bytes from row j to row j+1 of one KV head (>= row size,
 *              multiple of 4 for Q4_0 and of 16 for F16).
 * kv_head_stride   bytes from KV head g to g+1 (multiple of 4 / 16 likewise).
 *              Head-major caches use token_stride = row bytes and
 *              head_stride = n_rows_allocated * row bytes.
 * scale        softmax scale applied to q.k (finite, > 0), usually
 *              1/sqrt(head_dim).
 */
typedef struct tv_attn_desc {
    int32_t n_nodes;
    const int32_t *parent;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t kv_type;
    int64_t n_ctx;
    int64_t window;
    int64_t kv_token_stride;
    int64_t kv_head_stride;
    float scale;
    int32_t window_mode;
} tv_attn_desc;

/*
 * Device buffers of one layer (all caller-owned, base pointers 16-byte
 * aligned).
 *
 * k_cache, v_cache  the committed cache, laid out by the strides above.
 *                   May be NULL when n_ctx == 0.
 * q                 fp16 [n_nodes][n_q_heads][head_dim]
 * k_tree, v_tree    fp16 [n_nodes][n_kv_heads][head_dim]: K/V of the tree
 *                   nodes themselves (after any positional encoding).
 * out               fp32 [n_nodes][n_q_heads][head_dim]
 */
typedef struct tv_attn_ptrs {
    const void *k_cache;
    const void *v_cache;
    const void *q;
    const void *k_tree;
    const void *v_tree;
    float *out;
} tv_attn_ptrs;

/*
 * Device workspace (bytes) tree_verify_attn needs for `d`: partial softmax
 * states of the key-range splits (per split and output row, the normalised
 * partial output in fp16 and the log2 of its softmax denominator in fp32). 0 when `d` is invalid or no split is
 * needed (n_ctx == 0 after the window). Depends on the device's compute-unit
 * count, so query it for the device the call will run on (the current one).
 */
TV_API size_t tv_attn_workspace_bytes(const tv_attn_desc *d);

/* Split kernels a plan may launch (tv_attn_plan_info.kernel). */
#define TV_SPLIT_NONE 0  /* no whole 64-row chunk: the merge kernel scores every key */
#define TV_SPLIT_F16 1   /* F16 cache, one wave per SIMD */
#define TV_SPLIT_Q4_0 2  /* Q4_0 cache, one wave per SIMD, dequantisation interleaved with the MFMAs */
#define TV_SPLIT_Q4_0_WS 3 /* Q4_0 cache, head_dim 256: two waves per SIMD, one running the MFMAs,
                              the other dequantising the next chunks */
#define TV_SPLIT_F16_WS 4  /* F16 cache, head_dim 256: the same two roles, the other wave moving
                              the next chunks into LDS (at most one shared tile) */

/*
 * How tree_verify_attn would run `d` on a device with `n_cu` compute units
 * (n_cu <= 0: the current device's count, which needs the HIP runtime). A
 * host-only query: it checks `d` like tree_verify_attn, launches nothing and
 * touches no device memory, so callers and tests can see the split plan
 * (and size the workspace) without a GPU.
 *
 * splits        key-range splits per (KV head, row group); 0 when no whole
 *               64-row chunk is left for the split kernel
 * row_groups    groups the G * n_nodes packed query rows of a KV head are cut
 *               into (16-row tiles; each group is one workgroup per split)
 * own_tiles     most 16-row tiles one wave holds for all keys
 * shared_tiles  tiles whose keys are divided among the waves
 * masked        1 when the split kernel masks keys (a window end or start
 *               that is not on a chunk boundary)
 * kernel        TV_SPLIT_*
 * chunks        64-row chunks the split kernel covers per KV head
 * merge_rows    cache rows per node the merge kernel scores one by one
 * workspace_bytes  tv_attn_workspace_bytes for that device
 * Returns TV_OK or the TV_E_* code tree_verify_attn would return for `d`.
 */
typedef struct tv_attn_plan_info {
    int32_t splits;
    int32_t row_groups;
    int32_t own_tiles;
    int32_t shared_tiles;
    int32_t masked;
    int32_t kernel;
    int64_t chunks;
    int64_t merge_rows;
    uint64_t workspace_bytes;
} tv_attn_plan_info;

TV_API int tv_attn_plan(const tv_attn_desc *d, int32_t n_cu, tv_attn_plan_info *out);

/*
 * One layer of tree-verify attention, asynchronous on `stream`:
 *   out[i][h] = softmax over keys k of scale * q[i][h] . k, applied to the
 *   matching values, where the keys are the cache rows of the window and the
 *   tree nodes j that are ancestors of i or i itself.
 * Computation: fp16 products with fp32 accumulation; probabilities are
 * rounded to fp16 before they weight the cache values.
 * Accuracy (tested, not proven): the outputs are within 2e-3 of exact
 * attention, per output row relative to that row's largest value, while
 * every scaled score |scale * q.k| (q a query row, k a cache or tree key) is
 * at most 20 (29 in log2 units). For a Q4_0 cache each dequantised value scale*(code-8) is
 * rounded to fp16 once (relative 2^-11), which moves a score by up to 2^-11
 * of the sum of its terms' magnitudes; beyond that range the row error grows
 * about in proportion to the scores (measured: 8e-4 at 11, 2e-3 at 21, 8.5e-3
 * at 171). F16 caches are used as stored.
 * Non-finite inputs: a NaN or infinity in q, k_tree, v_tree or a cache row
 * (also a Q4_0 block whose fp16 scale is +-inf or NaN, which tree_commit_kv
 * writes for a block holding +-inf) leaves unspecified the outputs of every
 * query row of the KV head that reads it; other KV heads' rows are exact as
 * above.
 * `workspace` must hold tv_attn_workspace_bytes(d) bytes (NULL allowed when
 * that is 0), 16-byte aligned, and is overwritten.
 * Returns TV_OK or a TV_E_* code (nothing is launched on error).
 */
TV_API int tree_verify_attn(const tv_attn_desc *d, const tv_attn_ptrs *p, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * Device workspace (bytes) tree_accept needs for n_nodes x vocab logits:
 * completion counters and one running maximum per node, 832 bytes for any
 * valid shape. 0 for n_nodes outside 1..TV_MAX_NODES or vocab < 1.
 */
TV_API size_t tv_accept_workspace_bytes(int32_t n_nodes, int32_t vocab);

/*
 * Greedy acceptance of one verify step, asynchronous on `stream`.
 *
 * logits      device fp32 [n_nodes][vocab], 16-byte aligned, vocab >= 1.
 * parent      HOST int32[n_nodes], as in tv_attn_desc.
 * tokens      HOST int32[n_nodes]: draft token of each node (tokens[0], the
 *             root's, is not used).
 * argmax_out  device int32[n_nodes]: a[i] = argmax_v logits[i][v] with -0 ==
 *             +0, NaN below every number, ties to the smallest v, an all-NaN
 *             row giving 0.
 * result_out  device int32[2 + 2*n_nodes]:
 *               [0] n_acc, the number of accepted draft tokens;
 *               [1] the bonus token, a[last accepted node];
 *               [2 .. 2+n) the accepted path, node indices from the root,
 *                          padded with -1;
 *               [2+n .. 2+2n) the emitted tokens: tokens of path[1..n_acc],
 *                          then the bonus token, padded with -1.
 *             The accepted path is the longest root path along which every
 *             child's token equals its parent's argmax; among equally long
 *             ones, the one with the smaller child index where they diverge.
 * workspace   device, tv_accept_workspace_bytes(n_nodes, vocab) bytes,
 *             8-byte aligned, all zero before the first call that uses it
 *             (e.g. zeroed once when allocated); every call leaves it zero
 *             again, so a workspace can be reused call after call on one
 *             stream. Calls that share a workspace must not overlap (one
 *             stream, or ordered streams).
 * One launch: every workgroup reduces one 16384-logit slice of one row into
 * the row's maximum with device-scope atomics; the workgroup that completes
 * the last row runs the walk.
 */
TV_API int tree_accept(const float *logits, int32_t n_nodes, int32_t vocab, const int32_t *parent,
                const int32_t *tokens, int32_t *argmax_out, int32_t *result_out, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * tree_accept without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation). Same arguments, checks and results as tree_accept
 * (n_nodes up to TV_MAX_NODES, any vocab >= 1; anything larger is
 * TV_E_SHAPE). The acceptance state (832 bytes of counters and row maxima)
 * lives in a static array of the library, one per device, held until the
 * process ends: zero when the library loads, and every call leaves it zero.
 * All calls on one device share that array, so calls that overlap on one
 * device race: serialise them (one stream, or ordered streams). Nothing is
 * allocated; the first call on a device looks up the array's address there.
 */
TV_API int tree_accept_noalloc(const float *logits, int32_t n_nodes, int32_t vocab, const int32_t *parent,
                               const int32_t *tokens, int32_t *argmax_out, int32_t *result_out, void *stream);

/*
 * Shape of one layer's KV commit.
 *
 * n_nodes      size of the verified tree, 1..TV_MAX_NODES.
 * n_kv_heads   KV heads H_kv (>= 1).
 * head_dim     64, 128 or 256.
 * kv_type      TV_KV_F16 or TV_KV_Q4_0.
 * n_ctx        rows committed before this step (>= 0): position r of the
 *              accepted path (r = 0 is the root) goes to row n_ctx + r.
 * capacity     rows allocated per KV head; n_ctx + n_nodes <= capacity, so
 *              every possible path fits.
 * kv_token_stride, kv_head_stride  as in tv_attn_desc (same rules).
 */
typedef struct tv_commit_desc {
    int32_t n_nodes;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t kv_type;
    int64_t n_ctx;
    int64_t capacity;
    int64_t kv_token_stride;
    int64_t kv_head_stride;
} tv_commit_desc;

/*
 * Appends the accepted path of a verify step to one layer's KV cache,
 * asynchronous on `stream`. After greedy acceptance the root and the accepted
 * nodes are committed tokens (Luce DFlash pages: the verify state keeps the
 * target's cache in Q4_0 or F16); their K and V rows move from the tree
 * buffers into the cache.
 *
 * result      device int32[2 + 2*n_nodes], the result_out of tree_accept for
 *             the same tree (read on the device: the commit may follow the
 *             acceptance on the stream without a host round trip). n_acc =
 *             result[0]; the path is result[2 .. 2 + n_acc].
 * k_tree, v_tree  device fp16 [n_nodes][n_kv_heads][head_dim], 16-byte
 *             aligned: the K/V rows the verify pass used for the nodes.
 * k_cache, v_cache  device caches laid out by the strides, 16-byte aligned.
 *             For r = 0 .. n_acc, row n_ctx + r of every KV head receives
 *             node result[2 + r]'s row: copied for F16; for Q4_0 quantised
 *             per 32-value block with m = the value of largest magnitude
 *             (the first on ties), scale d = m / -8 stored as fp16 (nearest,
 *             ties to even), and code = floor(x * (1/d) + 8.5) clamped to
 *             0..15 (product and sum rounded separately in fp32; a zero
 *             block gets scale +0 and codes 8; NaN gets code 0). No other row is written.
 *             A result whose n_acc or path node is out of range writes
 *             nothing.
 * Returns TV_OK or a TV_E_* code (nothing is launched on error).
 */
TV_API int tree_commit_kv(const tv_commit_desc *d, const int32_t *result, const void *k_tree, const void *v_tree,
                   void *k_cache, void *v_cache, void *stream);

/*
 * tree_commit_kv for n_layers layers of the same shape at once (one launch
 * per 64 layers): k_tree, v_tree, k_cache, v_cache are HOST arrays of
 * n_layers device pointers, layer l's buffers at index l, each as in
 * tree_commit_kv; all layers share `d` (so the same strides and n_ctx) and
 * the acceptance result. The arrays are read during the call only.
 * Returns TV_OK or a TV_E_* code (nothing is launched on error; every layer's
 * pointers are checked before the first launch).
 */
TV_API int tree_commit_kv_layers(const tv_commit_desc *d, int32_t n_layers, const int32_t *result,
                          const void *const *k_tree, const void *const *v_tree, void *const *k_cache,
                          void *const *v_cache, void *stream);

/* Layers one tree_verify_step call takes. */
#define TV_MAX_LAYERS 16

/*
 * Device workspace (bytes) of tree_verify_step for n_layers layers of shape
 * `d` and `vocab` logits per node: a 2048-byte work-queue header (counters,
 * a status word and the acceptance state), then per layer one block of split
 * partials of tv_attn_workspace_bytes(d) bytes rounded up to a multiple of
 * 256. 0 when d is invalid, n_layers is outside 1..TV_MAX_LAYERS or
 * vocab < 1.
 */
TV_API size_t tv_step_workspace_bytes(const tv_attn_desc *d, int32_t n_layers, int32_t vocab);

/* How tree_verify_step runs a shape (host only, launches nothing). */
typedef struct tv_step_plan_info {
    int32_t launches;   /* kernel launches per call: 1 with the work-queue kernel,
                           2 for one layer of head_dim 256 with whole chunks */
    int32_t workgroups; /* workgroups of the work-queue kernel, or of the two
                           launches of one layer; 0 for the separate launches */
    int32_t splits;     /* key-range splits per KV head and row group of every layer */
    int32_t row_groups;
    int64_t items;      /* work items of the work-queue kernel (0 without it) */
    uint64_t workspace_bytes;
} tv_step_plan_info;

/* n_cu <= 0 asks the current device for its compute-unit count. */
TV_API int tv_step_plan(const tv_attn_desc *d, int32_t n_layers, int32_t vocab, int32_t n_cu,
                        tv_step_plan_info *out);

/*
 * One verify step over n_layers attention layers and the acceptance,
 * asynchronous on `stream`: the results of tree_verify_attn(d, &layers[l],
 * ...) for l = 0 .. n_layers-1 followed by tree_accept(logits, d->n_nodes,
 * vocab, d->parent, tokens, argmax_out, result_out, ...), with the same
 * checks, error codes and accuracy. The acceptance is bit for bit the same;
 * the attention is too where the step splits the keys as tree_verify_attn
 * does (tv_step_plan's splits equal tv_attn_plan's: one layer, long
 * contexts), and otherwise differs only by the rounding of the per-split
 * partial states (several layers share the device, so each layer's keys are
 * cut into fewer, longer splits).
 *
 * d           one descriptor for every layer (tree, heads, head_dim, context,
 *             window, scale, cache type and strides).
 * layers      HOST array of n_layers (1..TV_MAX_LAYERS) tensor sets, each as
 *             in tree_verify_attn.
 * logits, vocab, tokens, argmax_out, result_out   as in tree_accept; the
 *             logits are an input of the step, so a caller whose logits
 *             depend on these layers' outputs calls tree_verify_attn per
 *             layer instead.
 * workspace   device, tv_step_workspace_bytes(d, n_layers, vocab) bytes,
 *             256-byte aligned; its first 2048 bytes all zero before the
 *             first call (e.g. zeroed once when allocated). Every call leaves
 *             them zero again, except the status word (uint32 at byte 8),
 *             which a call sets to 1 if a merge item's wait ever ran out
 *             (not expected to happen: that call's outputs are then not
 *             valid) and which only the caller clears. Calls that share a
 *             workspace must not overlap.
 *
 * One layer of head_dim 256 with at least one whole chunk takes two
 * launches: its split kernel (as in tree_verify_attn), then one kernel whose
 * workgroups merge the output rows or scan the acceptance slices side by
 * side (the merge and the acceptance do not depend on each other), which
 * saves the acceptance its own launch. Otherwise, where the plan's split
 * kernel is TV_SPLIT_Q4_0_WS, the step is one launch of a persistent kernel (at most one workgroup per compute unit) that takes
 * work items from a device-side queue in ticket order: the acceptance
 * slices, then every layer's split items, each layer's merge items queued
 * behind the next layer's splits. A merge item waits (a bounded spin) for
 * its layer's split items, which hold lower tickets and so are already
 * running or done: no wait depends on a workgroup that has not started.
 * Other plans make the same launches as the separate calls, in order on
 * `stream`. The persistent kernel is the idea of "We got 207 tok/s with
 * Qwen3.5-27B on an RTX 3090", "What makes it work" (one kernel instead of
 * many launches per token).
 */
TV_API int tree_verify_step(const tv_attn_desc *d, int32_t n_layers, const tv_attn_ptrs *layers,
                            const float *logits, int32_t vocab, const int32_t *tokens, int32_t *argmax_out,
                            int32_t *result_out, void *workspace, size_t workspace_bytes, void *stream);

/* Kinds of tv_stream_probe. */
#define TV_PROBE_READ 0        /* read every byte */
#define TV_PROBE_Q4_0_DECODE 1 /* read, and unpack every byte as Q4_0 codes times a scale */

/*
 * Diagnostic: streams `bytes` bytes of device memory from `buf` (16-byte
 * aligned, a multiple of 16 bytes) with no attention arithmetic, to measure
 * the rate a streaming kernel reaches on this GPU next to the attention
 * kernels' own. TV_PROBE_READ only reads; TV_PROBE_Q4_0_DECODE also turns
 * every 4-bit code into fp16 (code - 8) * scale, with the instruction mix
 * the split kernels use (the scale is a constant; block scales are not
 * parsed). n_checksums workgroups (1 .. 2^20) each read one of
 * n_checksums near-equal contiguous ranges with streaming loads and write one
 * checksum word to the device array `checksums` (4-byte aligned), whose
 * values only keep the reads from being optimised away. Asynchronous on
 * `stream`.
 * Returns TV_OK or a TV_E_* code (nothing is launched on error).
 */
TV_API int tv_stream_probe(const void *buf, uint64_t bytes, int32_t kind, uint32_t *checksums,
                           int32_t n_checksums, void *stream);

/* Static string for a status code. */
TV_API const char *tv_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* TREE_VERIFY_H */
