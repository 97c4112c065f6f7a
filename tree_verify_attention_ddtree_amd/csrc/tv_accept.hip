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
// Kernel 2 (finish_walk): one wave. Reduces the slices of every row, writes
// the argmax, then one lane walks the tree (n <= 64).

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

__global__ void __launch_bounds__(64) finish_walk(const WalkArgs a)
{
    __shared__ int32_t am[TV_MAX_NODES];
    const int lane = threadIdx.x;
    // one row per iteration, slices spread over the wave
    for (int i = 0; i < a.n; ++i) {
        uint64_t b = 0;
        for (int s = lane; s < a.n_slices; s += 64) b = umax64(b, a.part[(int64_t)i * a.n_slices + s]);
        b = wave_umax64(b);
        if (lane == 0) {
            const int32_t idx = (int32_t)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFu));
            am[i] = idx;
            a.argmax_out[i] = idx;
        }
    }
    __syncthreads();
    if (lane != 0) return;
    // matched: node i lies on an accepted path from the root
    bool matched[TV_MAX_NODES];
    int depth[TV_MAX_NODES], reach[TV_MAX_NODES];
    matched[0] = true;
    depth[0] = 0;
    for (int i = 1; i < a.n; ++i) {
        const int p = a.parent[i];
        depth[i] = depth[p] + 1;
        matched[i] = matched[p] && a.tokens[i] == am[p];
    }
    // reach[u]: deepest matched depth below (or at) matched node u
    for (int i = 0; i < a.n; ++i) reach[i] = matched[i] ? depth[i] : -1;
    for (int i = a.n - 1; i > 0; --i)
        if (matched[i] && reach[i] > reach[a.parent[i]]) reach[a.parent[i]] = reach[i];
    // descend: at every node take the smallest child that still reaches the
    // deepest matched depth
    int path[TV_MAX_NODES];
    int len = 0, u = 0;
    path[len++] = 0;
    for (;;) {
        int next = -1;
        for (int c = u + 1; c < a.n; ++c)
            if (a.parent[c] == u && matched[c] && reach[c] == reach[0]) {
                next = c;
                break;
            }
        if (next < 0) break;
        path[len++] = next;
        u = next;
    }
    const int n = a.n;
    const int n_acc = len - 1;
    const int bonus = am[path[len - 1]];
    int32_t *res = a.result_out;
    for (int k = 0; k < 2 + 2 * n; ++k) res[k] = -1;
    res[0] = n_acc;
    res[1] = bonus;
    for (int k = 0; k < len; ++k) res[2 + k] = path[k];
    for (int k = 1; k < len; ++k) res[2 + n + k - 1] = a.tokens[path[k]];
    res[2 + n + n_acc] = bonus;
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
