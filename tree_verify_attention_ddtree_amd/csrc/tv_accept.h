// Greedy acceptance pieces (internal header of libtv.so): the per-slice
// argmax and the walk, shared by accept_kernel and the work-queue step kernel.
//
// Method: verification is greedy; the engine accepts the draft tokens along
// the tree while they equal the target's argmax, and the target's argmax at
// the last accepted node is emitted as well ("Luce DFlash: 単一RTX 3090で最大
// 2倍のスループットを目指すQwen3.6-27B", feature list and constraints: greedy
// verify only, sampling parameters ignored).
#pragma once

#include "tv_internal.h"

namespace tv {

constexpr int kAccThreads = 256;

// Integer tests only, so that the order holds whatever floating-point
// options the including file is compiled with.
__device__ __forceinline__ uint32_t order_code(float x)
{
    uint32_t b = __builtin_bit_cast(uint32_t, x);
    const uint32_t mag = b & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return 0u;  // NaN: below every number
    if (mag == 0u) b = 0u;             // -0 -> +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t pack_key(float x, uint32_t idx)
{
    return ((uint64_t)order_code(x) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_umax64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, off);
        const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
        v = umax64(v, ((uint64_t)hi << 32) | lo);
    }
    return v;
}

// Workspace (all of it zero before the first call; the last workgroup of
// every call sets it back to zero): the count of rows done, then one slice
// counter and one running maximum key per row.
constexpr size_t kRowsDoneOff = 0;
constexpr size_t kRowCountOff = 64;
constexpr size_t kRowKeyOff = kRowCountOff + 4 * TV_MAX_NODES;
static_assert(kRowKeyOff + 8 * TV_MAX_NODES == kAcceptWsBytes, "acceptance state layout");

struct AcceptArgs {
    const float *logits;
    uint32_t *rows_done;
    uint32_t *row_count;  // [n] slices done per row
    uint64_t *row_key;    // [n] maximum key per row
    int32_t *argmax_out;
    int32_t *result_out;
    int32_t vocab;
    int32_t n;
    int32_t n_slices;
    int32_t parent[TV_MAX_NODES];
    int32_t tokens[TV_MAX_NODES];
    uint64_t anc[TV_MAX_NODES];  // ancestor-or-self mask of each node
};

// The walk, by one wave; lane i stands for tree node i and holds its parent,
// token and ancestor-or-self mask (par, tok, anc; -1, -1, 0 past the last
// node), read from the kernel arguments when the workgroup started.
//   1. a[i]: lane i reads the maximum key of row i.
//   2. Node i matches when its token equals its parent's argmax; it is on an
//      accepted path when every node of its root path matches, i.e. its
//      ancestor mask lies inside the ballot of matching nodes.
//   3. The deepest such nodes mark their root paths; the descent from the
//      root takes, at every level, the smallest child on a marked path, which
//      is the lexicographically smallest of the longest accepted paths.
// Only the parent's argmax crosses lanes; the rest are ballots and lane reads
// of uniform indices.
__device__ void walk(const AcceptArgs &a, int lane, int par, int tok, uint64_t anc)
{
    const int n = a.n;
    const bool live = lane < n;
    const uint64_t b = __hip_atomic_load(a.row_key + (live ? lane : 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    int am = 0;
    if (live) {
        am = (int32_t)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFu));
        a.argmax_out[lane] = am;
    }

    const int am_parent = __shfl(am, (live && lane > 0) ? par : lane);
    const bool matched = live && (lane == 0 || tok == am_parent);
    const uint64_t M = __builtin_amdgcn_ballot_w64(matched);
    const bool ok = live && (anc & ~M) == 0;
    const int depth = __builtin_popcountll(anc) - 1;
    // deepest accepted depth, one bit at a time from the top
    int best = 0;
#pragma unroll
    for (int bit = 5; bit >= 0; --bit) {
        const int cand = best | (1 << bit);
        if (__builtin_amdgcn_ballot_w64(ok && depth >= cand)) best = cand;
    }
    // root paths of the deepest accepted nodes
    uint64_t deepest = __builtin_amdgcn_ballot_w64(ok && depth == best);
    uint64_t onpath = 0;
    const uint32_t anc_lo = (uint32_t)anc, anc_hi = (uint32_t)(anc >> 32);
    while (deepest) {
        const int d = __builtin_ctzll(deepest);
        deepest &= deepest - 1;
        onpath |= ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(anc_hi, d) << 32) |
                  (uint32_t)__builtin_amdgcn_readlane(anc_lo, d);
    }
    // descent from the root
    int u = 0, n_acc = 0;
    uint64_t chosen = 1ull;
    for (;;) {
        const uint64_t cand = __builtin_amdgcn_ballot_w64(live && lane > 0 && par == u && ((onpath >> lane) & 1));
        if (!cand) break;
        u = __builtin_ctzll(cand);
        chosen |= 1ull << u;
        ++n_acc;
    }
    const int bonus = __builtin_amdgcn_readlane(am, u);
    // result layout: [n_acc, bonus, path nodes (n, -1 padded), emitted tokens
    // (n: the path's draft tokens, then the bonus, -1 padded)]. The nodes of
    // the chosen path write their own entries; every other position is
    // written by the lane of that index.
    int32_t *res = a.result_out;
    if ((chosen >> lane) & 1) {
        res[2 + depth] = lane;
        if (depth >= 1) res[2 + n + depth - 1] = tok;
    }
    for (int pos = lane; pos < 2 + 2 * n; pos += 64) {
        if (pos == 0) {
            res[0] = n_acc;
        } else if (pos == 1) {
            res[1] = bonus;
        } else if (pos < 2 + n) {
            if (pos - 2 > n_acc) res[pos] = -1;
        } else {
            const int je = pos - 2 - n;
            if (je == n_acc) res[pos] = bonus;
            else if (je > n_acc) res[pos] = -1;
        }
    }
}

struct AcceptLds {
    uint64_t red[kAccThreads / 64];
    int last;
};

// Slice `sl` of logits row `row` by kAccThreads threads (t = 0..255) with LDS
// `sm`; a caller with more threads runs one slice per group of kAccThreads,
// each with its own `sm`, all through the same two barriers (a group with no
// slice passes valid = false and only meets them).
__device__ __forceinline__ void accept_slice(const AcceptArgs &a, int row, int sl, int t, bool valid, AcceptLds &sm)
{
    constexpr int PER = kSliceFloats / (4 * kAccThreads);  // 16-byte loads per thread
    const int vocab = a.vocab;
    const int64_t lo = (int64_t)sl * kSliceFloats;
    const int64_t hi = !valid ? lo : lo + kSliceFloats < vocab ? lo + kSliceFloats : vocab;
    const float *r = a.logits + (int64_t)row * vocab;
    // The walk's per-node data, in case this workgroup runs it: lane-indexed
    // reads of the kernel arguments are memory loads, so they are issued now
    // and wait behind the scan, not at the end of the acceptance (about
    // 0.3 us less per call on gfx950).
    int par = -1, tok = -1;
    uint64_t anc = 0;
    if (t < a.n) {
        par = a.parent[t];
        tok = a.tokens[t];
        anc = a.anc[t];
    }
    uint64_t best = 0;  // below every key
    // 16-byte loads where the row allows them (rows start 16-byte aligned
    // only when vocab is a multiple of 4); all of a thread's loads are issued
    // before the first compare.
    if ((vocab & 3) == 0) {
        float4 x[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int64_t v = lo + 4 * t + 4 * kAccThreads * k;
            x[k] = v < hi ? *(const float4 *)(r + v) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int64_t v = lo + 4 * t + 4 * kAccThreads * k;
            if (v < hi) {
                best = umax64(best, pack_key(x[k].x, (uint32_t)v));
                best = umax64(best, pack_key(x[k].y, (uint32_t)v + 1));
                best = umax64(best, pack_key(x[k].z, (uint32_t)v + 2));
                best = umax64(best, pack_key(x[k].w, (uint32_t)v + 3));
            }
        }
    } else {
        for (int64_t v = lo + t; v < hi; v += kAccThreads) best = umax64(best, pack_key(r[v], (uint32_t)v));
    }
    best = wave_umax64(best);
    if ((t & 63) == 0) sm.red[t >> 6] = best;
    __syncthreads();
    if (t == 0 && valid) {
        uint64_t b = sm.red[0];
        for (int w = 1; w < kAccThreads / 64; ++w) b = umax64(b, sm.red[w]);
        // Device-scope atomics only, each finished (returned) before the
        // next is issued: the slice key into the row's maximum, then the
        // row's slice count; the row's last slice counts the row done, and
        // the workgroup that counts the last row runs the walk. Every
        // maximum is in place before its row counts as done, and every row
        // before the last count, so the walk reads final keys.
        const uint64_t prev =
            __hip_atomic_fetch_max(a.row_key + row, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // (no key has all 64 bits set: NaN maps to code 0; the test only
        // makes the count wait for the maximum's return)
        const uint32_t inc = prev == ~0ull ? 2u : 1u;
        const uint32_t d = __hip_atomic_fetch_add(a.row_count + row, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int is_last = 0;
        if (d == (uint32_t)a.n_slices - 1) {
            const uint32_t r = __hip_atomic_fetch_add(a.rows_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            is_last = r == (uint32_t)a.n - 1;
        }
        sm.last = is_last;
    } else if (t == 0) {
        sm.last = 0;
    }
    __syncthreads();
    if (!sm.last) return;
    if (t < 64) {
        walk(a, t, par, tok, anc);
        // leave the workspace zero for the next call
        if (t < a.n) {
            __hip_atomic_store(a.row_key + t, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.row_count + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (t == 0) __hip_atomic_store(a.rows_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace tv
