// Internal declarations shared by the HIP sources of libtv.so (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tree_verify.h"

namespace tv {

// Keys per pipeline stage of the split kernel.
constexpr int kChunk = 64;
// Query tiles (16 rows each) a wave may hold: own tiles + shared tiles.
constexpr int kMaxSlots = 3;

// How the packed query rows of one KV head are cut into row groups and how a
// group's 16-row tiles are spread over the 4 waves of a workgroup.
struct RowPlan {
    int tiles;   // ceil(M / 16), M = G * n_nodes
    int groups;  // row groups (grid z)
    int nown;    // max own tiles per wave over groups
    int nsh;     // max shared tiles per group
};

// Per-group tile roles: a group of Tg tiles gives every wave Tg/4 own tiles;
// of the Tg%4 left over, 1 or 2 are shared (each split by keys over the four
// waves) and 3 become one more own tile for waves 0..2.
inline void group_roles(int Tg, int *own_max, int *sh, bool three_shared)
{
    const int a = Tg / 4, r = Tg % 4;
    if (r == 3 && a == 0 && three_shared) {
        // three tiles: all shared (each wave scores one key tile of each)
        // rather than one own tile for three waves and none for the fourth
        *own_max = 0;
        *sh = 3;
    } else if (r == 3) {
        *own_max = a + 1;
        *sh = 0;
    } else {
        *own_max = a;
        *sh = r;
    }
}

struct SplitPlan {
    RowPlan rows;
    int64_t s0;       // first cache row in the window
    int64_t R;        // cache rows in the window
    int64_t head;     // rows [s0, s0 + head) scored per node by the merge kernel (<= tree depth)
    int64_t n_chunks; // chunks of the split kernel (from s0 + head)
    int64_t n_whole;  // of which whole chunks; a chunk after them ends at the window's end
    int64_t tail;     // last rows of the window scored by the merge kernel
    int mask;         // the split kernel masks keys (its last chunk, per-node window starts)
    int S;            // key-range splits per (KV head, row group)
};

// Tile layouts (own tiles per wave, shared tiles per workgroup) for which the
// warp-specialised Q4_0 split kernel and the work-queue step kernel are
// built (head_dim 256): the kernels' dispatch tables and the host planner
// both read this.
inline bool ws_layout(int D, int nown, int nsh)
{
    return D == 256 && ((nown == 1 && nsh >= 0 && nsh <= 2) || (nown == 2 && nsh >= 0 && nsh <= 1));
}

// ... and of its F16 form (at most one shared tile: the load waves' raw F16
// rows take the registers a second one would need).
inline bool ws_layout_f16(int D, int nown, int nsh)
{
    return D == 256 && (nown == 1 || nown == 2) && nsh >= 0 && nsh <= 1;
}

// Sizes the host side needs from the kernels' layouts.
constexpr size_t kAcceptWsBytes = 832;  // acceptance state: counters, per-row maxima
constexpr int kSliceFloats = 16384;     // logits per acceptance workgroup (slice)
constexpr size_t kStepHeader = 2048;    // work-queue header of the step workspace
constexpr int kMergeRowsMid = 8;        // output rows per step merge item (all but the last layer)
constexpr int kMergeRowsLast = 4;       // ... of the last layer

int plan_attn(const tv_attn_desc *d, int n_cu, SplitPlan *out);
// Which split kernel a plan launches (TV_SPLIT_* of tree_verify.h).
int split_kernel_kind(const tv_attn_desc *d, const SplitPlan &p);
size_t attn_ws_bytes(const tv_attn_desc *d, const SplitPlan &p);
int device_cu_count(int *n_cu);
// The step's plan: its workspace, launches and work items, and the lag of
// its merge items (see tv_step.hip).
size_t step_layer_bytes(const tv_attn_desc *d, const SplitPlan &p);
size_t step_ws_bytes(const tv_attn_desc *d, const SplitPlan &p, int n_layers);
// How tree_verify_step runs: the separate per-layer launches, one launch of
// the work-queue kernel, or (one layer of head_dim 256 with at least one
// whole chunk) the split kernel then merge_accept_kernel.
enum StepForm { kStepSeparate = 0, kStepQueue = 1, kStepTwo = 2 };
StepForm step_shape(const tv_attn_desc *d, const SplitPlan &p, int n_layers, int vocab, int *launches, int *workgroups,
                    int64_t *items);
int step_lag(int n_cu, int n_split);

}  // namespace tv
