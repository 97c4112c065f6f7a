// Warp-specialised split kernel for Q4_0 caches with head_dim 256 (gfx950):
// one workgroup per (key-range split, KV head, row group); the body and its
// design notes are in tv_split_q4ws.h.

#include "tv_split_q4ws.h"

namespace tv {

template <int NOWN, int NSH>
__global__ void __launch_bounds__(kWsThreads, 1) split_q4ws_kernel(const SplitArgs a)
{
    const SplitPtrs p = {a.k_cache, a.v_cache, a.q, a.ws_o, a.ws_m};
    uint32_t next = 0;
    // partial state through device-coherent stores (see kCpolSc1)
    ws_split<NOWN, NSH, kCpolSc1>(a, p, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.z, nullptr, next);
}

split_fn pick_split_q4ws(int D, int nown, int nsh)
{
    if (D != 256) return nullptr;
#define TV_CASE(O, S) \
    if (nown == O && nsh == S) return split_q4ws_kernel<O, S>;
    TV_CASE(1, 0) TV_CASE(1, 1) TV_CASE(1, 2) TV_CASE(2, 0) TV_CASE(2, 1)
#undef TV_CASE
    return nullptr;
}

}  // namespace tv
