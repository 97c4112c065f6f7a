// Warp-specialised split kernel for F16 caches with head_dim 256 (gfx950):
// one workgroup per (key-range split, KV head, row group); the body is the
// one of the Q4_0 kernel (tv_split_q4ws.h), whose load waves here move each
// F16 chunk into the fragment-order stage without decoding (F16WsLoader).
// Built for the layouts with at most one shared tile: the load waves hold
// two chunks of raw F16 rows (128 registers), which leaves room for one
// shared tile's state, not two.

#include "tv_split_q4ws.h"

namespace tv {

template <int NOWN, int NSH>
__global__ void __launch_bounds__(kWsThreads, 1) split_f16ws_kernel(const SplitArgs a)
{
    const SplitPtrs p = {a.k_cache, a.v_cache, a.q, a.ws_o, a.ws_m};
    uint32_t next = 0;
    // partial state through device-coherent stores (see kCpolSc1)
    ws_split<NOWN, NSH, kCpolSc1, TV_KV_F16>(a, p, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.z, nullptr, next);
}

split_fn pick_split_f16ws(int D, int nown, int nsh)
{
    if (!ws_layout_f16(D, nown, nsh)) return nullptr;
#define TV_CASE(O, S) \
    if (nown == O && nsh == S) return split_f16ws_kernel<O, S>;
    TV_CASE(1, 0) TV_CASE(1, 1) TV_CASE(2, 0) TV_CASE(2, 1)
#undef TV_CASE
    return nullptr;
}

}  // namespace tv
