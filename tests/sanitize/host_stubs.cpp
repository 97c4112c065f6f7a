// Launch functions of libtv.so for the host-only sanitizer build
// (run_cpu_suite.sh): that build holds the C ABI, its argument checks, the
// planner and the workspace sizes (tv_api.cpp) under ASan and UBSan, and no
// GPU code. Every launch reports TV_E_HIP; the CPU tests never reach one,
// since each call they make fails a host check first or finds no device.

#include "tv_internal.h"

namespace tv {

int launch_attn(const tv_attn_desc *, const tv_attn_ptrs *, const SplitPlan &, void *, hipStream_t) { return TV_E_HIP; }

int launch_accept(const float *, int, int, const int32_t *, const int32_t *, int32_t *, int32_t *, void *, hipStream_t)
{
    return TV_E_HIP;
}

int launch_accept_noalloc(const float *, int, int, const int32_t *, const int32_t *, int32_t *, int32_t *, hipStream_t)
{
    return TV_E_HIP;
}

int launch_stream_probe(const void *, uint64_t, int, uint32_t *, int, hipStream_t) { return TV_E_HIP; }

int launch_commit(const tv_commit_desc *, int, const int32_t *, const void *const *, const void *const *,
                  void *const *, void *const *, hipStream_t)
{
    return TV_E_HIP;
}

int launch_step(const tv_attn_desc *, int, const tv_attn_ptrs *, const float *, int, const int32_t *, int32_t *,
                int32_t *, void *, int, const SplitPlan &, hipStream_t)
{
    return TV_E_HIP;
}

}  // namespace tv
