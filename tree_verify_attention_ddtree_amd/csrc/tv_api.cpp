// C ABI of libtv.so: argument checks, planning, workspace sizes, launches.
// Every check runs on the host before anything is launched.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "tv_internal.h"

namespace tv {

int launch_attn(const tv_attn_desc *d, const tv_attn_ptrs *p, const SplitPlan &plan, void *ws,
                hipStream_t stream);
int launch_accept(const float *logits, int n, int vocab, const int32_t *parent, const int32_t *tokens,
                  int32_t *argmax_out, int32_t *result_out, void *ws, hipStream_t stream);
int launch_accept_noalloc(const float *logits, int n, int vocab, const int32_t *parent, const int32_t *tokens,
                          int32_t *argmax_out, int32_t *result_out, hipStream_t stream);
int launch_stream_probe(const void *buf, uint64_t bytes, int kind, uint32_t *checksums, int n_wg,
                        hipStream_t stream);
int launch_step(const tv_attn_desc *d, int n_layers, const tv_attn_ptrs *layers, const float *logits, int vocab,
                const int32_t *tokens, int32_t *argmax_out, int32_t *result_out, void *ws, int n_cu,
                const SplitPlan &plan, hipStream_t stream);
int launch_commit(const tv_commit_desc *d, int n_layers, const int32_t *result, const void *const *k_tree,
                  const void *const *v_tree, void *const *k_cache, void *const *v_cache, hipStream_t stream);

// Splits are sized so one launch fills the device with about one workgroup
// per compute unit, down to one chunk per split: a split's fixed cost (Q
// fragments, pipeline fill, writing its partial state) is paid in parallel,
// which beats fewer, longer splits while the device is not full.
constexpr int kMinChunks = 1;

static int check_tree(int n, const int32_t *parent)
{
    if (n < 1 || n > TV_MAX_NODES) return TV_E_SHAPE;
    if (!parent) return TV_E_ARG;
    if (parent[0] != -1) return TV_E_TREE;
    for (int i = 1; i < n; ++i)
        if (parent[i] < 0 || parent[i] >= i) return TV_E_TREE;
    return TV_OK;
}

static int check_desc(const tv_attn_desc *d)
{
    if (!d) return TV_E_ARG;
    int rc = check_tree(d->n_nodes, d->parent);
    if (rc) return rc;
    if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads) return TV_E_SHAPE;
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return TV_E_SHAPE;
    if (d->kv_type != TV_KV_F16 && d->kv_type != TV_KV_Q4_0) return TV_E_ARG;
    if (d->n_ctx < 0 || d->window < 0) return TV_E_SHAPE;
    if (d->window_mode != 0 && d->window_mode != 1) return TV_E_ARG;
    if (!(d->scale > 0.0f) || !isfinite(d->scale)) return TV_E_ARG;
    // the kernels address q, out and a split's block of the workspace with
    // 32-bit buffer offsets: n * H_q rows of 2 * head_dim bytes stay below 2^31
    if ((int64_t)d->n_nodes * d->n_q_heads * 2 * d->head_dim >= ((int64_t)1 << 31)) return TV_E_SHAPE;
    // grid dimension y of the split kernel
    if (d->n_kv_heads > 65535) return TV_E_SHAPE;
    if (d->n_ctx > 0) {
        const int64_t row = d->kv_type == TV_KV_Q4_0 ? (int64_t)d->head_dim / 32 * 18 : (int64_t)d->head_dim * 2;
        const int64_t al = d->kv_type == TV_KV_Q4_0 ? 4 : 16;
        if (d->kv_token_stride < row || d->kv_head_stride < 0) return TV_E_SHAPE;
        // per-thread row offsets inside a 64-row chunk are 32-bit
        if (d->kv_token_stride > ((int64_t)1 << 24)) return TV_E_SHAPE;
        if (d->kv_token_stride % al || d->kv_head_stride % al) return TV_E_ALIGN;
    }
    return TV_OK;
}

// Tile roles for T tiles cut into RG row groups; false when a group needs
// more tile slots per wave than the kernels have.
static bool rows_for_groups(int T, int RG, bool three_shared, RowPlan *rp)
{
    int nown = 0, nsh = 0;
    for (int g = 0; g < RG; ++g) {
        const int Tg = T / RG + (g < T % RG ? 1 : 0);
        int o, s;
        group_roles(Tg, &o, &s, three_shared);
        nown = o > nown ? o : nown;
        nsh = s > nsh ? s : nsh;
    }
    if (nown + nsh > kMaxSlots || nown + nsh < 1) return false;
    rp->tiles = T;
    rp->groups = RG;
    rp->nown = nown;
    rp->nsh = nsh;
    return true;
}

static int plan_rows(int M, bool three_shared, RowPlan *rp)
{
    const int T = (M + 15) / 16;
    for (int RG = 1; RG <= T; ++RG)
        if (rows_for_groups(T, RG, three_shared, rp)) return TV_OK;
    return TV_E_SHAPE;
}

int plan_attn(const tv_attn_desc *d, int n_cu, SplitPlan *out)
{
    const int G = d->n_q_heads / d->n_kv_heads;
    const int M = G * d->n_nodes;
    // the Q4_0 kernels have an all-shared layout for three tiles
    const bool three_shared = d->kv_type == TV_KV_Q4_0;
    int rc = plan_rows(M, three_shared, &out->rows);
    if (rc) return rc;
    out->s0 = (d->window > 0 && d->n_ctx > d->window) ? d->n_ctx - d->window : 0;
    out->R = d->n_ctx - out->s0;
    int max_depth = 0;
    const bool per_pos = d->window_mode == 1 && d->window > 0;
    if (per_pos) {
        int depth[TV_MAX_NODES];
        depth[0] = 0;
        for (int i = 1; i < d->n_nodes; ++i) {
            depth[i] = depth[d->parent[i]] + 1;
            max_depth = depth[i] > max_depth ? depth[i] : max_depth;
        }
    }
    const int64_t per = (int64_t)d->n_kv_heads * out->rows.groups;
    // At most two chunks a split (short contexts): half the splits, and the
    // row-group step below gives the rows two groups instead. The grid keeps
    // one workgroup per CU, each with twice the chunks and about half the
    // rows, and the merge reads half the partials (27B layer, Q4_0, 23
    // nodes: 4K 25.3 -> 19.8 us, 8K 26.5 -> 23.5 us; no gain from 16K; F16
    // at 8K: 25.5 -> 23.1 us). Taken where both groups fit a warp-specialised
    // kernel (the one-wave F16 kernel gained nothing from it).
    RowPlan two;
    const bool halve = out->rows.groups == 1 && out->rows.tiles >= 2 &&
                       rows_for_groups(out->rows.tiles, 2, three_shared, &two) &&
                       (d->kv_type == TV_KV_Q4_0 ? ws_layout(d->head_dim, two.nown, two.nsh)
                                                 : ws_layout_f16(d->head_dim, two.nown, two.nsh));
    auto splits = [&](int64_t n_chunks, bool may_halve) -> int {
        int64_t S = (n_cu + per - 1) / per;
        if (may_halve && halve && n_chunks <= 2 * S && (S + 1) / 2 * 2 * per <= n_cu) S = (S + 1) / 2;
        int64_t cap = n_chunks / kMinChunks;
        if (cap < 1) cap = 1;
        if (S > cap) S = cap;
        if (S < 1) S = 1;
        if (S > 65535) S = 65535;
        return (int)S;
    };
    // Two ways to attend the window rows that do not make a whole chunk of
    // the same keys for every row: the per-node first rows of a per-position
    // window (as many as the tree is deep) and a remainder of fewer than
    // kChunk rows at the window's end.
    //  - masked split kernel: whole chunks from s0, then one chunk ending at
    //    the window's end; per row, keys it may not see (before its node's
    //    window start, or already counted) score -inf. The masking code
    //    costs every chunk about 3% (register allocation), so it is a
    //    separate instantiation, taken while splits are short (up to 8
    //    chunks), where the merge kernel's rows would cost more.
    //  - otherwise the merge kernel scores those rows (head rows per node,
    //    then the tail) and the split kernel takes the whole chunks between.
    out->mask = 0;
    out->tail = 0;
    const int64_t rem = out->R % kChunk;
    // a node at depth k starts seeing the window k - (W - R) rows in: some
    // node skips rows when the tree is deeper than W - R
    const bool skips = per_pos && out->R > 0 && max_depth > d->window - out->R;
    const bool ragged = rem > 0 || skips;
    if (ragged && d->n_ctx >= kChunk) {
        const int64_t nc = out->R / kChunk + (rem ? 1 : 0);
        const int S = splits(nc, false);
        if ((nc + S - 1) / S <= 8) {
            out->mask = 1;
            out->head = 0;
            out->n_whole = out->R / kChunk;
            out->n_chunks = nc;
            out->S = S;
        }
    }
    if (!out->mask) {
        out->head = per_pos ? (out->R < max_depth ? out->R : max_depth) : 0;
        out->n_chunks = (out->R - out->head) / kChunk;
        out->n_whole = out->n_chunks;
        out->tail = out->R - out->head - out->n_chunks * kChunk;
        if (out->n_chunks == 0) {
            out->S = 0;
            return TV_OK;
        }
        out->S = splits(out->n_chunks, true);
    }
    // A key range too short to give every CU a split (S capped by the chunk
    // count, e.g. a 2048-row window) leaves CUs idle: cut the rows into more
    // groups as well, up to one workgroup per CU. Each group dequantises the
    // same chunks again, but on a CU that would otherwise wait.
    for (int RG = out->rows.groups + 1; RG <= out->rows.tiles; ++RG) {
        if ((int64_t)out->S * d->n_kv_heads * RG > n_cu) break;
        RowPlan rp;
        if (rows_for_groups(out->rows.tiles, RG, three_shared, &rp)) out->rows = rp;
    }
    // Small layouts the warp-specialised kernels lack, moved onto one they
    // have with idle tile slots (a slot past the group's last tile computes
    // zero query rows and writes nothing). Measured on the budget sweep (24 q
    // / 4 kv heads, head_dim 256):
    //   F16, up to 8 tiles: one or two own tiles per wave instead of the
    //   all-shared or (1, 2) layouts of the one-wave kernel (128K: 4 nodes
    //   122 -> 97 us, 16 nodes 135 -> 105; 8K: 4 nodes 27.0 -> 16.2);
    //   Q4_0, three tiles: one own tile per wave instead of three shared (8
    //   nodes at 128K: 67.4 -> 61.3 us); six tiles: two own tiles per wave
    //   instead of one own and two shared, which takes the two shared tiles
    //   off the load waves (16 nodes at 128K: 83.9 -> 81.8 us, at 32K 31.3
    //   -> 30.5; five tiles measured slower that way). One or two Q4_0 tiles
    //   stay on the one-wave kernel, which measured faster there (1 node:
    //   55.8 against 61.7 us).
    RowPlan &r = out->rows;
    if (!out->mask && r.groups == 1) {
        if (d->kv_type == TV_KV_F16 && r.tiles <= 8 && !ws_layout_f16(d->head_dim, r.nown, r.nsh) &&
            ws_layout_f16(d->head_dim, 2, 0)) {
            r.nown = r.tiles <= 4 ? 1 : 2;
            r.nsh = 0;
        } else if (d->kv_type == TV_KV_Q4_0 && r.tiles == 3 && r.nown == 0 && ws_layout(d->head_dim, 1, 0)) {
            r.nown = 1;
            r.nsh = 0;
        } else if (d->kv_type == TV_KV_Q4_0 && r.tiles == 6 && r.nown == 1 && r.nsh == 2 &&
                   ws_layout(d->head_dim, 2, 0)) {
            r.nown = 2;
            r.nsh = 0;
        }
    }
    return TV_OK;
}

size_t attn_ws_bytes(const tv_attn_desc *d, const SplitPlan &p)
{
    const size_t NR = (size_t)d->n_nodes * d->n_q_heads;
    // fp16 normalised outputs [S][NR][D], then fp32 log2 denominators [S][NR]
    return (size_t)p.S * NR * ((size_t)d->head_dim * 2 + sizeof(float));
}

int split_kernel_kind(const tv_attn_desc *d, const SplitPlan &p)
{
    if (p.S == 0) return TV_SPLIT_NONE;
    if (d->kv_type == TV_KV_Q4_0 && !p.mask && ws_layout(d->head_dim, p.rows.nown, p.rows.nsh))
        return TV_SPLIT_Q4_0_WS;
    if (d->kv_type == TV_KV_F16 && !p.mask && ws_layout_f16(d->head_dim, p.rows.nown, p.rows.nsh))
        return TV_SPLIT_F16_WS;
    return d->kv_type == TV_KV_Q4_0 ? TV_SPLIT_Q4_0 : TV_SPLIT_F16;
}

// A layer's merge items are queued behind about one round of later split
// items (one per compute unit), so that its own splits have finished when
// they start: ceil(n_cu / split items per layer) + 1 layers, at least 2.
int step_lag(int n_cu, int n_split)
{
    const int l = (n_cu + n_split - 1) / n_split + 1;
    return l < 2 ? 2 : l;
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t step_layer_bytes(const tv_attn_desc *d, const SplitPlan &p) { return round256(attn_ws_bytes(d, p)); }

size_t step_ws_bytes(const tv_attn_desc *d, const SplitPlan &p, int n_layers)
{
    return kStepHeader + (size_t)n_layers * step_layer_bytes(d, p);
}

// Launches of one step call (1 with the work-queue kernel) and its work
// items (one workgroup each); 0 workgroups when the plan has no work-queue
// kernel (then the step makes the separate launches).
StepForm step_shape(const tv_attn_desc *d, const SplitPlan &p, int n_layers, int vocab, int *launches, int *workgroups,
                    int64_t *items)
{
    // (the merge items address a layer's partials with 31-bit offsets)
    const bool fits = (int64_t)p.S * d->n_nodes * d->n_q_heads * (2 * d->head_dim) < ((int64_t)1 << 31);
    const int64_t NR = (int64_t)d->n_nodes * d->n_q_heads;
    const int64_t n_split = (int64_t)p.S * d->n_kv_heads * p.rows.groups;
    const int64_t n_merge = (NR + kMergeRowsMid - 1) / kMergeRowsMid;
    const int64_t n_last = (NR + kMergeRowsLast - 1) / kMergeRowsLast;
    const int64_t slices = (int64_t)d->n_nodes * (((int64_t)vocab + kSliceFloats - 1) / kSliceFloats);
    const int64_t total = (slices + 1) / 2 + n_layers * n_split + (n_layers - 1) * n_merge + n_last;
    if (n_layers == 1 && d->head_dim == 256 && p.S > 0 && NR + slices <= INT32_MAX) {
        // one layer: its split kernel, then its merge and the acceptance in
        // one launch of 256-thread workgroups
        *items = 0;
        *workgroups = (int)(n_split + NR + slices);
        *launches = 2;
        return kStepTwo;
    }
    if (split_kernel_kind(d, p) == TV_SPLIT_Q4_0_WS && fits && total <= INT32_MAX) {
        *items = total;
        *workgroups = (int)total;
        *launches = 1;
        return kStepQueue;
    }
    *items = 0;
    *workgroups = 0;
    *launches = n_layers * (p.S > 0 ? 2 : 1) + 1;
    return kStepSeparate;
}

int device_cu_count(int *n_cu)
{
    // cached per device; the count of a device never changes
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TV_E_HIP;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *n_cu = c;
            return TV_OK;
        }
    }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
        return TV_E_HIP;
    if (dev >= 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
    *n_cu = v;
    return TV_OK;
}

}  // namespace tv

extern "C" {

const char *tv_strerror(int code)
{
    switch (code) {
    case TV_OK: return "ok";
    case TV_E_ARG: return "invalid argument";
    case TV_E_TREE: return "parent array is not a rooted tree in topological order";
    case TV_E_SHAPE: return "unsupported shape";
    case TV_E_ALIGN: return "misaligned pointer or stride";
    case TV_E_WORKSPACE: return "workspace missing or too small";
    case TV_E_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

size_t tv_attn_workspace_bytes(const tv_attn_desc *d)
{
    if (tv::check_desc(d)) return 0;
    int n_cu = 0;
    if (tv::device_cu_count(&n_cu)) return 0;
    tv::SplitPlan plan;
    if (tv::plan_attn(d, n_cu, &plan)) return 0;
    return tv::attn_ws_bytes(d, plan);
}

static bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int tv_attn_plan(const tv_attn_desc *d, int32_t n_cu, tv_attn_plan_info *out)
{
    int rc = tv::check_desc(d);
    if (rc) return rc;
    if (!out) return TV_E_ARG;
    int cu = n_cu;
    if (cu <= 0) {
        rc = tv::device_cu_count(&cu);
        if (rc) return rc;
    }
    tv::SplitPlan plan;
    rc = tv::plan_attn(d, cu, &plan);
    if (rc) return rc;
    memset(out, 0, sizeof(*out));
    out->splits = plan.S;
    out->row_groups = plan.rows.groups;
    out->own_tiles = plan.rows.nown;
    out->shared_tiles = plan.rows.nsh;
    out->masked = plan.mask;
    out->kernel = tv::split_kernel_kind(d, plan);
    out->chunks = plan.S > 0 ? plan.n_chunks : 0;
    out->merge_rows = plan.head + plan.tail;
    out->workspace_bytes = tv::attn_ws_bytes(d, plan);
    return TV_OK;
}

static int check_ptrs(const tv_attn_desc *d, const tv_attn_ptrs *p)
{
    if (!p || !p->q || !p->k_tree || !p->v_tree || !p->out) return TV_E_ARG;
    if (d->n_ctx > 0 && (!p->k_cache || !p->v_cache)) return TV_E_ARG;
    if (!aligned(p->q, 16) || !aligned(p->k_tree, 16) || !aligned(p->v_tree, 16) || !aligned(p->out, 16))
        return TV_E_ALIGN;
    if (d->n_ctx > 0 && (!aligned(p->k_cache, 16) || !aligned(p->v_cache, 16))) return TV_E_ALIGN;
    return TV_OK;
}

int tree_verify_attn(const tv_attn_desc *d, const tv_attn_ptrs *p, void *workspace, size_t workspace_bytes,
                     void *stream)
{
    int rc = tv::check_desc(d);
    if (rc) return rc;
    rc = check_ptrs(d, p);
    if (rc) return rc;
    int n_cu = 0;
    rc = tv::device_cu_count(&n_cu);
    if (rc) return rc;
    tv::SplitPlan plan;
    rc = tv::plan_attn(d, n_cu, &plan);
    if (rc) return rc;
    const size_t need = tv::attn_ws_bytes(d, plan);
    if (need > 0 && (!workspace || workspace_bytes < need)) return TV_E_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return TV_E_ALIGN;
    return tv::launch_attn(d, p, plan, workspace, (hipStream_t)stream);
}

size_t tv_accept_workspace_bytes(int32_t n_nodes, int32_t vocab)
{
    if (n_nodes < 1 || n_nodes > TV_MAX_NODES || vocab < 1) return 0;
    return tv::kAcceptWsBytes;
}

static int check_accept(const float *logits, int32_t n_nodes, int32_t vocab, const int32_t *parent,
                        const int32_t *tokens, const int32_t *argmax_out, const int32_t *result_out)
{
    int rc = tv::check_tree(n_nodes, parent);
    if (rc) return rc;
    if (vocab < 1) return TV_E_SHAPE;
    if (!logits || !tokens || !argmax_out || !result_out) return TV_E_ARG;
    if (!aligned(logits, 16) || !aligned(argmax_out, 4) || !aligned(result_out, 4)) return TV_E_ALIGN;
    return TV_OK;
}

int tree_accept(const float *logits, int32_t n_nodes, int32_t vocab, const int32_t *parent, const int32_t *tokens,
                int32_t *argmax_out, int32_t *result_out, void *workspace, size_t workspace_bytes, void *stream)
{
    int rc = check_accept(logits, n_nodes, vocab, parent, tokens, argmax_out, result_out);
    if (rc) return rc;
    const size_t need = tv::kAcceptWsBytes;
    if (!workspace || workspace_bytes < need) return TV_E_WORKSPACE;
    if (!aligned(workspace, 8)) return TV_E_ALIGN;
    return tv::launch_accept(logits, n_nodes, vocab, parent, tokens, argmax_out, result_out, workspace,
                             (hipStream_t)stream);
}

int tree_accept_noalloc(const float *logits, int32_t n_nodes, int32_t vocab, const int32_t *parent,
                        const int32_t *tokens, int32_t *argmax_out, int32_t *result_out, void *stream)
{
    int rc = check_accept(logits, n_nodes, vocab, parent, tokens, argmax_out, result_out);
    if (rc) return rc;
    return tv::launch_accept_noalloc(logits, n_nodes, vocab, parent, tokens, argmax_out, result_out,
                                     (hipStream_t)stream);
}

static int step_setup(const tv_attn_desc *d, int32_t n_layers, int32_t vocab, int32_t n_cu_in, int *n_cu,
                      tv::SplitPlan *plan)
{
    int rc = tv::check_desc(d);
    if (rc) return rc;
    if (n_layers < 1 || n_layers > TV_MAX_LAYERS || vocab < 1) return TV_E_SHAPE;
    *n_cu = n_cu_in;
    if (*n_cu <= 0) {
        rc = tv::device_cu_count(n_cu);
        if (rc) return rc;
    }
    rc = tv::plan_attn(d, *n_cu, plan);
    if (rc || n_layers < 2 || plan->S == 0) return rc;
    // With several layers in one queue the grid need not be filled by one
    // layer's splits: fewer, longer split items pay the per-item cost
    // (query rows, pipeline fill, partial state, ticket: about 6 us) less
    // often and leave fewer partials to merge. The split count drops to the
    // larger of two floors: at least two rounds of split items over the
    // device (short of that the step's tail has idle compute units) and at
    // most 16 chunks per item (longer items end the step unevenly). Measured
    // (one launch, against the single-layer split count): 16 layers at 8K
    // 191 against 337 us, at 32K 462 against 532, 4 layers at 32K 134
    // against 162.
    const int64_t lk = (int64_t)n_layers * d->n_kv_heads;
    const int64_t s_rounds = (2 * (int64_t)*n_cu + lk - 1) / lk;
    const int64_t s_chunks = (plan->n_chunks + 15) / 16;
    const int64_t st = s_rounds > s_chunks ? s_rounds : s_chunks;
    if (st >= plan->S) return TV_OK;
    return tv::plan_attn(d, (int)(st * d->n_kv_heads), plan);
}

size_t tv_step_workspace_bytes(const tv_attn_desc *d, int32_t n_layers, int32_t vocab)
{
    int n_cu = 0;
    tv::SplitPlan plan;
    if (step_setup(d, n_layers, vocab, 0, &n_cu, &plan)) return 0;
    return tv::step_ws_bytes(d, plan, n_layers);
}

int tv_step_plan(const tv_attn_desc *d, int32_t n_layers, int32_t vocab, int32_t n_cu, tv_step_plan_info *out)
{
    int cu = 0;
    tv::SplitPlan plan;
    int rc = step_setup(d, n_layers, vocab, n_cu, &cu, &plan);
    if (rc) return rc;
    if (!out) return TV_E_ARG;
    memset(out, 0, sizeof(*out));
    int launches = 0, wgs = 0;
    int64_t items = 0;
    tv::step_shape(d, plan, n_layers, vocab, &launches, &wgs, &items);
    out->launches = launches;
    out->workgroups = wgs;
    out->splits = plan.S;
    out->row_groups = plan.rows.groups;
    out->items = items;
    out->workspace_bytes = tv::step_ws_bytes(d, plan, n_layers);
    return TV_OK;
}

int tree_verify_step(const tv_attn_desc *d, int32_t n_layers, const tv_attn_ptrs *layers, const float *logits,
                     int32_t vocab, const int32_t *tokens, int32_t *argmax_out, int32_t *result_out,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    int rc = tv::check_desc(d);
    if (rc) return rc;
    if (n_layers < 1 || n_layers > TV_MAX_LAYERS) return TV_E_SHAPE;
    if (!layers) return TV_E_ARG;
    for (int l = 0; l < n_layers; ++l) {
        rc = check_ptrs(d, &layers[l]);
        if (rc) return rc;
    }
    rc = check_accept(logits, d->n_nodes, vocab, d->parent, tokens, argmax_out, result_out);
    if (rc) return rc;
    if (!workspace) return TV_E_WORKSPACE;
    if (!aligned(workspace, 256)) return TV_E_ALIGN;
    int n_cu = 0;
    tv::SplitPlan plan;
    rc = step_setup(d, n_layers, vocab, 0, &n_cu, &plan);
    if (rc) return rc;
    if (workspace_bytes < tv::step_ws_bytes(d, plan, n_layers)) return TV_E_WORKSPACE;
    return tv::launch_step(d, n_layers, layers, logits, vocab, tokens, argmax_out, result_out, workspace, n_cu, plan,
                           (hipStream_t)stream);
}

int tv_stream_probe(const void *buf, uint64_t bytes, int32_t kind, uint32_t *checksums, int32_t n_checksums,
                    void *stream)
{
    if (!buf || !checksums) return TV_E_ARG;
    if (kind != TV_PROBE_READ && kind != TV_PROBE_Q4_0_DECODE) return TV_E_ARG;
    if (bytes == 0 || n_checksums < 1 || n_checksums > (1 << 20)) return TV_E_SHAPE;
    if (bytes % 16 || !aligned(buf, 16) || !aligned(checksums, 4)) return TV_E_ALIGN;
    return tv::launch_stream_probe(buf, bytes, kind, checksums, n_checksums, (hipStream_t)stream);
}

static int check_commit_desc(const tv_commit_desc *d)
{
    if (!d) return TV_E_ARG;
    if (d->n_nodes < 1 || d->n_nodes > TV_MAX_NODES || d->n_kv_heads < 1) return TV_E_SHAPE;
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return TV_E_SHAPE;
    if (d->kv_type != TV_KV_F16 && d->kv_type != TV_KV_Q4_0) return TV_E_ARG;
    if (d->n_ctx < 0 || d->capacity < 0 || d->n_ctx > d->capacity - d->n_nodes) return TV_E_SHAPE;
    const int64_t row = d->kv_type == TV_KV_Q4_0 ? (int64_t)d->head_dim / 32 * 18 : (int64_t)d->head_dim * 2;
    const int64_t al = d->kv_type == TV_KV_Q4_0 ? 4 : 16;
    if (d->kv_token_stride < row || d->kv_head_stride < 0) return TV_E_SHAPE;
    if (d->kv_token_stride % al || d->kv_head_stride % al) return TV_E_ALIGN;
    return TV_OK;
}

static int check_commit_layer(const void *k_tree, const void *v_tree, const void *k_cache, const void *v_cache)
{
    if (!k_tree || !v_tree || !k_cache || !v_cache) return TV_E_ARG;
    if (!aligned(k_tree, 16) || !aligned(v_tree, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
        return TV_E_ALIGN;
    return TV_OK;
}

int tree_commit_kv(const tv_commit_desc *d, const int32_t *result, const void *k_tree, const void *v_tree,
                   void *k_cache, void *v_cache, void *stream)
{
    int rc = check_commit_desc(d);
    if (rc) return rc;
    if (!result) return TV_E_ARG;
    if (!aligned(result, 4)) return TV_E_ALIGN;
    rc = check_commit_layer(k_tree, v_tree, k_cache, v_cache);
    if (rc) return rc;
    return tv::launch_commit(d, 1, result, &k_tree, &v_tree, &k_cache, &v_cache, (hipStream_t)stream);
}

int tree_commit_kv_layers(const tv_commit_desc *d, int32_t n_layers, const int32_t *result,
                          const void *const *k_tree, const void *const *v_tree, void *const *k_cache,
                          void *const *v_cache, void *stream)
{
    int rc = check_commit_desc(d);
    if (rc) return rc;
    if (n_layers < 1) return TV_E_SHAPE;
    if (!result || !k_tree || !v_tree || !k_cache || !v_cache) return TV_E_ARG;
    if (!aligned(result, 4)) return TV_E_ALIGN;
    for (int l = 0; l < n_layers; ++l) {
        rc = check_commit_layer(k_tree[l], v_tree[l], k_cache[l], v_cache[l]);
        if (rc) return rc;
    }
    return tv::launch_commit(d, n_layers, result, k_tree, v_tree, k_cache, v_cache, (hipStream_t)stream);
}

}  // extern "C"
