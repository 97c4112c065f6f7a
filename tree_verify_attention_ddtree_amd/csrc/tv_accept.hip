// Greedy acceptance for gfx950: per-node argmax over the vocabulary, then the
// walk down the draft tree, in one launch.
//
// Method: verification is greedy; the engine accepts the draft tokens along
// the tree while they equal the target's argmax, and the target's argmax at
// the last accepted node is emitted as well ("Luce DFlash: 単一RTX 3090で最大
// 2倍のスループットを目指すQwen3.6-27B", feature list and constraints: greedy
// verify only, sampling parameters ignored).
//
// accept_kernel, grid (slices, n): each workgroup scans one slice of one
// logits row with 16-byte loads and reduces a 64-bit key (order-preserving
// float code << 32 | ~index), so that the maximum key is the largest value
// with the smallest index (NaN maps to the lowest code, -0 to the code of
// +0), and stores it. A completion counter then picks the workgroup that
// finishes last; its first wave (lane i = node i) reduces every row's slice
// keys and finds the accepted path from ballots over the nodes' ancestor
// masks (built on the host from the parent array), and sets the counter back
// to zero for the next call.

#include <mutex>

#include "tv_accept.h"

namespace tv {

// One workgroup per (slice, row).
__global__ void __launch_bounds__(kAccThreads) accept_kernel(const AcceptArgs a)
{
    __shared__ AcceptLds sm;
    accept_slice(a, blockIdx.y, blockIdx.x, threadIdx.x, true, sm);
}

static int64_t n_slices_for(int vocab) { return ((int64_t)vocab + kSliceFloats - 1) / kSliceFloats; }

void fill_accept_args(const float *logits, int n, int vocab, const int32_t *parent, const int32_t *tokens,
                      int32_t *argmax_out, int32_t *result_out, uint8_t *ws, AcceptArgs *out)
{
    AcceptArgs &a = *out;
    a.logits = logits;
    a.rows_done = (uint32_t *)(ws + kRowsDoneOff);
    a.row_count = (uint32_t *)(ws + kRowCountOff);
    a.row_key = (uint64_t *)(ws + kRowKeyOff);
    a.argmax_out = argmax_out;
    a.result_out = result_out;
    a.vocab = vocab;
    a.n = n;
    a.n_slices = (int)n_slices_for(vocab);
    for (int i = 0; i < TV_MAX_NODES; ++i) {
        a.parent[i] = i < n ? parent[i] : -1;
        a.tokens[i] = i < n ? tokens[i] : -1;
        uint64_t m = 0;
        if (i < n)
            for (int v = i; v >= 0; v = parent[v]) m |= 1ull << v;
        a.anc[i] = m;
    }
}

static int launch_accept_on(const float *logits, int n, int vocab, const int32_t *parent, const int32_t *tokens,
                            int32_t *argmax_out, int32_t *result_out, uint8_t *ws, hipStream_t stream)
{
    AcceptArgs a;
    fill_accept_args(logits, n, vocab, parent, tokens, argmax_out, result_out, ws, &a);
    void *args[] = {(void *)&a};
    if (hipLaunchKernel((const void *)accept_kernel, dim3(a.n_slices, n), dim3(kAccThreads), args, 0, stream) !=
        hipSuccess)
        return TV_E_HIP;
    return TV_OK;
}

int launch_accept(const float *logits, int n, int vocab, const int32_t *parent, const int32_t *tokens,
                  int32_t *argmax_out, int32_t *result_out, void *ws, hipStream_t stream)
{
    return launch_accept_on(logits, n, vocab, parent, tokens, argmax_out, result_out, (uint8_t *)ws, stream);
}

// State of tree_accept_noalloc: the acceptance workspace as a static device
// array, one per device (zero when the module loads; every call leaves it
// zero). Host code never passes the array's name to a kernel: the device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current.
static __device__ __align__(256) uint64_t scratch[kAcceptWsBytes / sizeof(uint64_t)];

static int scratch_ptr(uint8_t **out)
{
    static std::mutex mu;
    static void *ptrs[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return TV_E_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TV_E_HIP;
        ptrs[dev] = p;
    }
    *out = (uint8_t *)ptrs[dev];
    return TV_OK;
}

int launch_accept_noalloc(const float *logits, int n, int vocab, const int32_t *parent, const int32_t *tokens,
                          int32_t *argmax_out, int32_t *result_out, hipStream_t stream)
{
    uint8_t *ws = nullptr;
    const int rc = scratch_ptr(&ws);
    if (rc) return rc;
    return launch_accept_on(logits, n, vocab, parent, tokens, argmax_out, result_out, ws, stream);
}

}  // namespace tv
