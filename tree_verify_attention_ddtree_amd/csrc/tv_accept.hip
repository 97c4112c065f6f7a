// Greedy acceptance for gfx950: per-node argmax over the vocabulary, then the
// walk down the draft tree.
//
// Method: verification is greedy; the engine accepts the draft tokens along
// the tree while they equal the target's argmax, and the target's argmax at
// the last accepted node is emitted as well ("Luce DFlash: 単一RTX 3090で最大
// 2倍のスループットを目指すQwen3.6-27B", feature list and constraints: greedy
// verify only, sampling parameters ignored).
//
// Kernel 1 (argmax_partial): grid (chunks, n). Each workgroup scans one slice
// of one logits row with 16-byte loads and reduces a 64-bit key
// (order-preserving float code << 32 | ~index) so that the maximum key is the
// largest value with the smallest index; NaN maps to the lowest code and -0 to
// the code of +0.
// Kernel 2 (finish_walk): one wave, lane i = node i: reduces the slices of
// row i, then finds the accepted path with wave-wide pointer jumping.

#include "tv_internal.h"

namespace tv {

constexpr int kAccThreads = 256;
constexpr int kSliceFloats = 8192;  // logits per workgroup of kernel 1

__device__ __forceinline__ uint32_t order_code(float x)
{
    if (x != x) return 0u;    // NaN: below every number
    if (x == 0.0f) x = 0.0f;  // -0 -> +0
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
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

__global__ void __launch_bounds__(kAccThreads) argmax_partial(const float *logits, int vocab, int n_slices,
                                                              uint64_t *part)
{
    const int row = blockIdx.y, sl = blockIdx.x;
    const int64_t lo = (int64_t)sl * kSliceFloats;
    const int64_t hi = lo + kSliceFloats < vocab ? lo + kSliceFloats : vocab;
    const float *r = logits + (int64_t)row * vocab;
    uint64_t best = 0;
    // 16-byte loads where the row allows them; rows start 16-byte aligned
    // only when vocab is a multiple of 4.
    if ((vocab & 3) == 0) {
        for (int64_t v = lo + 4 * threadIdx.x; v < hi; v += 4 * kAccThreads) {
            const float4 x = *(const float4 *)(r + v);
            best = umax64(best, pack_key(x.x, (uint32_t)v));
            best = umax64(best, pack_key(x.y, (uint32_t)v + 1));
            best = umax64(best, pack_key(x.z, (uint32_t)v + 2));
            best = umax64(best, pack_key(x.w, (uint32_t)v + 3));
        }
    } else {
        for (int64_t v = lo + threadIdx.x; v < hi; v += kAccThreads) best = umax64(best, pack_key(r[v], (uint32_t)v));
    }
    best = wave_umax64(best);
    __shared__ uint64_t red[kAccThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t b = red[0];
        for (int w = 1; w < kAccThreads / 64; ++w) b = umax64(b, red[w]);
        part[(int64_t)row * n_slices + sl] = b;
    }
}

struct WalkArgs {
    const uint64_t *part;
    int32_t *argmax_out;
    int32_t *result_out;
    int32_t n;
    int32_t n_slices;
    int32_t parent[TV_MAX_NODES];
    int32_t tokens[TV_MAX_NODES];
};

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src)
{
    const uint32_t lo = __shfl((uint32_t)v, src), hi = __shfl((uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

// One wave; lane i stands for tree node i.
//   1. a[i]: lane i reduces the slice maxima of row i.
//   2. Pointer jumping over parents (6 rounds cover depth 63): depth, whether
//      every edge of the root path matches (child token == parent's argmax),
//      and the ancestor-or-self bitmask.
//   3. The deepest matched nodes mark their root paths; the descent from the
//      root takes, at every level, the smallest child on a marked path, which
//      is the lexicographically smallest of the longest accepted paths.
__global__ void __launch_bounds__(64) finish_walk(const WalkArgs a)
{
    const int lane = threadIdx.x;
    const int n = a.n;
    int par = -1, tok = -1;
#pragma unroll
    for (int i = 0; i < TV_MAX_NODES; ++i)
        if (lane == i) {
            par = a.parent[i];
            tok = a.tokens[i];
        }
    const bool live = lane < n;

    int am = 0;
    if (live) {
        // the slice maxima of row `lane`, loaded 32 at a time
        uint64_t b = 0;
        const uint64_t *pr = a.part + (int64_t)lane * a.n_slices;
        for (int s0 = 0; s0 < a.n_slices; s0 += 32) {
            uint64_t v[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) v[k] = s0 + k < a.n_slices ? pr[s0 + k] : 0ull;
#pragma unroll
            for (int k = 0; k < 32; ++k) b = umax64(b, v[k]);
        }
        am = (int32_t)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFu));
        a.argmax_out[lane] = am;
    }

    const int p0 = (live && lane > 0) ? par : lane;  // root and dead lanes point to themselves
    const int am_parent = __shfl(am, p0);
    bool ok = !live ? false : (lane == 0 ? true : tok == am_parent);
    int nxt = p0;
    int depth = (live && lane > 0) ? 1 : 0;
    uint64_t msk = 1ull << lane;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
        const bool ok_n = __shfl((int)ok, nxt) != 0;
        const int d_n = __shfl(depth, nxt);
        const uint64_t m_n = shfl64(msk, nxt);
        const int nxt_n = __shfl(nxt, nxt);
        if (nxt != lane) {
            ok = ok && ok_n;
            depth += d_n;
            msk |= m_n;
        }
        nxt = nxt_n;
    }
    const bool matched = live && ok;
    int best = matched ? depth : -1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) best = max(best, __shfl_xor(best, off));
    uint64_t onpath = (matched && depth == best) ? msk : 0ull;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) onpath |= shfl64(onpath, lane ^ off);

    // descent; lane k records the k-th node of the path
    int u = 0, len = 1, mypath = lane == 0 ? 0 : -1;
    for (;;) {
        const uint64_t cand = __builtin_amdgcn_ballot_w64(live && lane > 0 && par == u && ((onpath >> lane) & 1));
        if (!cand) break;
        u = __builtin_ctzll(cand);
        if (lane == len) mypath = u;
        ++len;
    }
    const int n_acc = len - 1;
    const int bonus = __shfl(am, u);
    // every output position is written exactly once; the shuffles run with
    // all lanes active
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const int pos = lane + 64 * r;
        const int jp = pos - 2;      // index into the path
        const int je = pos - 2 - n;  // index into the emitted tokens
        const int pj = __shfl(mypath, (jp >= 0 && jp < 64) ? jp : 0);
        const int pe = __shfl(mypath, (je + 1 >= 0 && je + 1 < 64) ? je + 1 : 0);
        const int te = __shfl(tok, (pe >= 0 && pe < 64) ? pe : 0);
        int v;
        if (pos == 0)
            v = n_acc;
        else if (pos == 1)
            v = bonus;
        else if (pos < 2 + n)
            v = jp <= n_acc ? pj : -1;
        else
            v = je < n_acc ? te : (je == n_acc ? bonus : -1);
        if (pos < 2 + 2 * n) a.result_out[pos] = v;
    }
}

static int64_t n_slices_for(int vocab) { return ((int64_t)vocab + kSliceFloats - 1) / kSliceFloats; }

size_t accept_ws_bytes(int n, int vocab) { return (size_t)n * (size_t)n_slices_for(vocab) * sizeof(uint64_t); }

int launch_accept(const float *logits, int n, int vocab, const int32_t *parent, const int32_t *tokens,
                  int32_t *argmax_out, int32_t *result_out, void *ws, hipStream_t stream)
{
    const int ns = (int)n_slices_for(vocab);
    uint64_t *part = (uint64_t *)ws;
    hipLaunchKernelGGL(argmax_partial, dim3(ns, n), dim3(kAccThreads), 0, stream, logits, vocab, ns, part);
    if (hipGetLastError() != hipSuccess) return TV_E_HIP;
    WalkArgs w;
    w.part = part;
    w.argmax_out = argmax_out;
    w.result_out = result_out;
    w.n = n;
    w.n_slices = ns;
    for (int i = 0; i < TV_MAX_NODES; ++i) {
        w.parent[i] = i < n ? parent[i] : -1;
        w.tokens[i] = i < n ? tokens[i] : -1;
    }
    hipLaunchKernelGGL(finish_walk, dim3(1), dim3(64), 0, stream, w);
    if (hipGetLastError() != hipSuccess) return TV_E_HIP;
    return TV_OK;
}

}  // namespace tv
