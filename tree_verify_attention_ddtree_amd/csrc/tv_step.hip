// One verify step in one launch (gfx950): the tree-verify attention of every
// layer (split and merge) and the greedy acceptance, as the work items of one
// kernel, handed out by a device-side ticket queue.
//
// Method: the target verifies the whole DDTree draft tree in one pass per
// step ("Luce DFlash: 単一RTX 3090で最大2倍のスループットを目指す
// Qwen3.6-27B", feature list: DDTree tree verify, greedy verify, Q4_0 KV up
// to about 128K); the persistent kernel that replaces many launches per token
// with one is the idea of "We got 207 tok/s with Qwen3.5-27B on an RTX 3090",
// "What makes it work" (there with a cooperative grid sync over a whole
// model; here a ticket queue over the verify step's attention layers and its
// acceptance).
//
// Queue: the grid has one workgroup per item; a workgroup takes ticket t with
// a device-scope atomic add when it starts and runs item t, so items start in
// ticket order whatever order the hardware dispatches workgroups in.
// (A persistent loop over items would keep per-thread values live across the
// split body, whose math waves use every register.) Items in ticket order:
//   S_0 .. S_{g-1}          the split items of the first g layers (split,
//                           KV head, row group): the warp-specialised split
//                           body of tv_split_q4ws.h;
//   S_k, M_{k-g}            for k = g .. L-1: layer k's split items, then the
//                           merge items of layer k - g (8 output rows each,
//                           two at a time, one per half workgroup); the lag g
//                           puts about one round of split items (one per
//                           compute unit) between a layer's splits and its
//                           merges, so the merges rarely wait;
//   M_{L-g} .. M_{L-2}, A, M_{L-1}
//                           the remaining merges (4 rows per item for the
//                           last layer) around the acceptance items (one
//                           16384-logit slice per half workgroup), so that
//                           the workgroups freed by the last splits have
//                           work while the slowest of them finish.
// The first wave of workgroups takes split items only: workgroups are handed
// to the device's L2 partitions (XCDs) in turn, and a partition without a
// free compute unit holds back the next workgroup, so short items at the
// start leave compute units idle until the long ones end (measured at 128K
// rows: 190 us with the acceptance first, against 110 us as separate
// launches).
// A split item stores its partial state with device-coherent stores, waits
// for them to complete and then increments its layer's counter; a merge item
// waits (thread 0, bounded spin) until the counter of its layer has every
// split item, then reads the partials with device-coherent loads (no cache
// of the device can hand it a stale copy). Every item a merge waits for holds
// a lower ticket, so a workgroup that started earlier took it and is running
// or has finished it: no wait depends on a workgroup that has not started,
// and the lowest unfinished item never waits. The spin is bounded all the
// same (a status word records a wait that ran out). The workgroup that exits
// last sets the queue counters back to zero; the acceptance's own counters
// are reset by the workgroup that runs its walk.

#include <string.h>

#include "tv_accept.h"
#include "tv_merge.h"
#include "tv_split_q4ws.h"

namespace tv {

// Work-queue header at the start of the step workspace (all zero between
// calls, except the status word, which only the caller clears).
constexpr size_t kQTicket = 0;      // u32 next ticket
constexpr size_t kQExited = 4;      // u32 workgroups that left the loop
constexpr size_t kQStatus = 8;      // u32 1 if a merge wait ran out
constexpr size_t kQDone = 64;       // u32[TV_MAX_LAYERS] split items done per layer
constexpr size_t kQAccept = 1024;   // acceptance state (kAcceptWsBytes)
static_assert(kQDone + 4 * TV_MAX_LAYERS <= kQAccept && kQAccept + kAcceptWsBytes <= kStepHeader,
              "work-queue header layout");

// Output rows per merge item (kMergeRowsMid, kMergeRowsLast), two at a time,
// one per half workgroup. A merge row takes about 4 us at one workgroup per
// compute unit (latency bound), and every item pays about 2 us of dispatch
// and ticket: merges that run beside later layers' splits take 8 rows, the
// last layer's merges, which end the step, 4 (16 layers at 32K rows: 533 us
// with 8 rows, 585 with 4, 691 with 2; one layer at 128K rows: 111, 107 and
// 114 us).

struct StepLayer {
    SplitPtrs sp;
    const _Float16 *k_tree;
    const _Float16 *v_tree;
    float *out;
};

struct StepArgs {
    SplitArgs sa;   // layer-independent split fields (tensors per layer below)
    MergeArgs ma;   // layer-independent merge fields
    AcceptArgs ac;  // acceptance of the step
    StepLayer layer[TV_MAX_LAYERS];
    uint32_t *queue;  // work-queue header
    uint32_t spin_limit;
    int32_t n_layers;
    int32_t n_accept;  // acceptance items (two slices each)
    int32_t n_split;   // split items per layer: S * H_kv * row groups
    int32_t n_merge;   // merge items per layer (kMergeRowsMid rows each)
    int32_t n_merge_last;  // merge items of the last layer (kMergeRowsLast rows each)
    int32_t H_kv;
    int32_t lag;  // layers between a layer's split items and its merge items
    int32_t total;
};
static_assert(sizeof(StepArgs) <= 4096, "kernel arguments of the step kernel");

// Role of ticket t (see the queue order above).
struct Item {
    int kind;  // 0 acceptance, 1 split, 2 merge
    int layer;
    int index;
    int rows;  // output rows per merge item
};

__device__ __forceinline__ Item decode(const StepArgs &s, int t)
{
    const int L = s.n_layers, S = s.n_split, M = s.n_merge, lag = s.lag;
    int u = t;
    const int nh = L < lag ? L : lag;  // blocks S_k alone, k < lag
    if (u < nh * S) return {1, u / S, u % S, 0};
    u -= nh * S;
    const int blk = S + M;
    const int nb = L - nh;  // blocks S_k, M_{k-lag} for k = lag .. L-1
    if (u < nb * blk) {
        const int k = lag + u / blk, r = u % blk;
        return r < S ? Item{1, k, r, 0} : Item{2, k - lag, r - S, kMergeRowsMid};
    }
    u -= nb * blk;
    const int nt = L - 1 - nb;  // merges of layers nb .. L-2 after every split
    if (u < nt * M) return {2, nb + u / M, u % M, kMergeRowsMid};
    u -= nt * M;
    if (u < s.n_accept) return {0, 0, u, 0};
    return {2, L - 1, u - s.n_accept, kMergeRowsLast};
}

template <int NOWN, int NSH>
__global__ void __launch_bounds__(kWsThreads, 1) step_kernel(const StepArgs s)
{
    __shared__ uint32_t tick;
    const int tid = threadIdx.x;
    if (tid == 0)
        tick = __hip_atomic_fetch_add(s.queue + kQTicket / 4, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const Item it = decode(s, (int)tick);
    if (it.kind == 1) {
        // -------------------------------------------------------- split item
        const StepLayer &ly = s.layer[it.layer];
        const int S = s.sa.S;
        const int split = it.index % S, gkv = (it.index / S) % s.H_kv, rg = it.index / (S * s.H_kv);
        const int RG = s.n_split / (S * s.H_kv);
        uint32_t unused = 0;
        ws_split<NOWN, NSH, kCpolSc1>(s.sa, ly.sp, split, gkv, rg, RG, nullptr, unused);
        // The partial state went out with device-coherent stores. Every wave
        // waits until its stores are complete (a barrier does not wait for
        // them), then thread 0 counts the item done: a merge that sees the
        // count sees the stores. (A release fence would write back the whole
        // L2 instead, about 5 us per split item.)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            __hip_atomic_fetch_add(s.queue + kQDone / 4 + it.layer, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (it.kind == 2) {
        // -------------------------------------------------------- merge item
        if (tid == 0) {
            const uint32_t *done = s.queue + kQDone / 4 + it.layer;
            uint32_t spins = 0;
            while (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)s.n_split) {
                if (++spins > s.spin_limit) {
                    __hip_atomic_fetch_or(s.queue + kQStatus / 4, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        // the partials are read with device-coherent loads after this
        // barrier, so they see every store the count covers
        __syncthreads();
        const StepLayer &ly = s.layer[it.layer];
        const MergePtrs p = {ly.sp.q, ly.k_tree, ly.v_tree, ly.sp.ws_o, ly.sp.ws_m, ly.out, ly.sp.k_cache,
                             ly.sp.v_cache};
        static_assert(2 * sizeof(MergeLds<256>) <= sizeof(ws_lds), "two merge rows in the split items' LDS");
        MergeLds<256> *ml = (MergeLds<256> *)ws_lds;
        const int half = tid >> 8;
        const int NR = s.ma.NR;
#pragma unroll 1
        for (int j = 0; j < it.rows / 2; ++j) {
            const int row = it.index * it.rows + 2 * j + half;
            if (j > 0) __syncthreads();  // the LDS of the previous row is free
            merge_row<256, kCpolSc1>(s.ma, p, row < NR ? row : NR - 1, tid & 255, row < NR, ml[half]);
        }
    } else {
        // --------------------------------------------------- acceptance item
        static_assert(2 * sizeof(AcceptLds) <= sizeof(ws_lds), "two acceptance slices in the split items' LDS");
        AcceptLds *al = (AcceptLds *)ws_lds;
        const int half = tid >> 8;
        const int f = 2 * it.index + half;
        const bool valid = f < s.ac.n * s.ac.n_slices;
        const int row = valid ? f / s.ac.n_slices : 0, sl = valid ? f % s.ac.n_slices : 0;
        accept_slice(s.ac, row, sl, tid & 255, valid, al[half]);
    }
    // the workgroup that finishes last sets the queue back to zero (every
    // other workgroup has taken its ticket and finished its item)
    __syncthreads();
    if (tid == 0) {
        const uint32_t e =
            __hip_atomic_fetch_add(s.queue + kQExited / 4, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (e == gridDim.x - 1) {
            for (int l = 0; l < s.n_layers; ++l)
                __hip_atomic_store(s.queue + kQDone / 4 + l, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(s.queue + kQTicket / 4, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(s.queue + kQExited / 4, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// One layer's merge and the acceptance in one launch (the step of a single
// layer, after its split kernel): the first n * n_slices workgroups scan one
// acceptance slice each (row-major over the rows' slices), the rest merge an
// output row each. The two parts share nothing but the launch; the
// acceptance, the longer chain of the two, is dispatched first (128K layer:
// 97.9 against 99.2 us a step).
__global__ void __launch_bounds__(256) merge_accept_kernel(const MergeArgs m, const AcceptArgs ac)
{
    static_assert(kAccThreads == 256, "a merge row and an acceptance slice take 256 threads each");
    __shared__ union {
        MergeLds<256> mg;
        AcceptLds acc;
    } sm;
    const int b = blockIdx.x;
    const int na = ac.n * ac.n_slices;
    if (b >= na) {
        merge_row<256>(m, m.p, b - na, threadIdx.x, true, sm.mg);
        return;
    }
    accept_slice(ac, b / ac.n_slices, b % ac.n_slices, threadIdx.x, true, sm.acc);
}

// step kernel of a tile layout (every layout ws_layout accepts)
static const void *pick_step(int nown, int nsh)
{
#define TV_CASE(O, S) \
    if (nown == O && nsh == S) return (const void *)step_kernel<O, S>;
    TV_CASE(1, 0) TV_CASE(1, 1) TV_CASE(1, 2) TV_CASE(2, 0) TV_CASE(2, 1)
#undef TV_CASE
    return nullptr;
}

int launch_attn(const tv_attn_desc *d, const tv_attn_ptrs *p, const SplitPlan &plan, void *ws, hipStream_t stream);
int launch_split(const tv_attn_desc *d, const tv_attn_ptrs *p, const SplitPlan &plan, void *ws, hipStream_t stream);
int launch_accept(const float *logits, int n, int vocab, const int32_t *parent, const int32_t *tokens,
                  int32_t *argmax_out, int32_t *result_out, void *ws, hipStream_t stream);
void fill_accept_args(const float *logits, int n, int vocab, const int32_t *parent, const int32_t *tokens,
                      int32_t *argmax_out, int32_t *result_out, uint8_t *ws, AcceptArgs *a);

int launch_step(const tv_attn_desc *d, int n_layers, const tv_attn_ptrs *layers, const float *logits, int vocab,
                const int32_t *tokens, int32_t *argmax_out, int32_t *result_out, void *ws, int n_cu,
                const SplitPlan &plan, hipStream_t stream)
{
    uint8_t *const base = (uint8_t *)ws;
    const size_t lb = step_layer_bytes(d, plan);
    int launches = 0, wgs = 0;
    int64_t items = 0;
    const StepForm form = step_shape(d, plan, n_layers, vocab, &launches, &wgs, &items);
    if (form == kStepTwo) {
        // one layer: its split kernel, then its merge and the acceptance in
        // one launch
        const int rc = launch_split(d, &layers[0], plan, base + kStepHeader, stream);
        if (rc) return rc;
        MergeArgs m;
        AcceptArgs ac;
        fill_merge_args(d, &layers[0], plan, base + kStepHeader, &m);
        fill_accept_args(logits, d->n_nodes, vocab, d->parent, tokens, argmax_out, result_out, base + kQAccept, &ac);
        void *args[] = {(void *)&m, (void *)&ac};
        const int nwg = m.NR + ac.n * ac.n_slices;
        if (hipLaunchKernel((const void *)merge_accept_kernel, dim3(nwg), dim3(256), args, 0, stream) != hipSuccess)
            return TV_E_HIP;
        return TV_OK;
    }
    if (form == kStepSeparate) {
        // per-layer launches, then the acceptance, on the same stream
        for (int l = 0; l < n_layers; ++l) {
            const int rc = launch_attn(d, &layers[l], plan, base + kStepHeader + l * lb, stream);
            if (rc) return rc;
        }
        return launch_accept(logits, d->n_nodes, vocab, d->parent, tokens, argmax_out, result_out, base + kQAccept,
                             stream);
    }
    StepArgs s;
    memset(&s, 0, sizeof(s));
    fill_split_args(d, &layers[0], plan, base + kStepHeader, &s.sa);
    fill_merge_args(d, &layers[0], plan, base + kStepHeader, &s.ma);
    fill_accept_args(logits, d->n_nodes, vocab, d->parent, tokens, argmax_out, result_out, base + kQAccept, &s.ac);
    for (int l = 0; l < n_layers; ++l) {
        SplitArgs a;
        fill_split_args(d, &layers[l], plan, base + kStepHeader + l * lb, &a);
        s.layer[l].sp = {a.k_cache, a.v_cache, a.q, a.ws_o, a.ws_m};
        s.layer[l].k_tree = (const _Float16 *)layers[l].k_tree;
        s.layer[l].v_tree = (const _Float16 *)layers[l].v_tree;
        s.layer[l].out = layers[l].out;
    }
    s.queue = (uint32_t *)base;
    // 2^22 polls, each a load from memory (about a microsecond) and a short
    // sleep: seconds, far beyond the longest split item (about 0.1 ms at
    // 128K rows)
    s.spin_limit = 1u << 22;
    s.n_layers = n_layers;
    s.n_split = plan.S * d->n_kv_heads * plan.rows.groups;
    const int NR = d->n_nodes * d->n_q_heads;
    s.n_merge = (NR + kMergeRowsMid - 1) / kMergeRowsMid;
    s.n_merge_last = (NR + kMergeRowsLast - 1) / kMergeRowsLast;
    s.n_accept = (s.ac.n * s.ac.n_slices + 1) / 2;
    s.H_kv = d->n_kv_heads;
    s.lag = step_lag(n_cu, s.n_split);
    s.total = (int32_t)items;
    const void *fn = pick_step(plan.rows.nown, plan.rows.nsh);
    if (!fn) return TV_E_SHAPE;
    void *args[] = {(void *)&s};
    if (hipLaunchKernel(fn, dim3(wgs), dim3(kWsThreads), args, 0, stream) != hipSuccess) return TV_E_HIP;
    return TV_OK;
}

}  // namespace tv
