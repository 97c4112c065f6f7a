// Stream probes: how fast this GPU streams a buffer the size of a KV cache,
// with no attention arithmetic. The attention kernels are measured against
// them: the plain read gives the HBM rate a streaming kernel reaches, the
// decoding read the rate when every code byte also goes through the Q4_0
// unpacking (the per-value vector work the split kernels do before their
// MFMAs).
//
// Method context: the verify step streams a Q4_0 (or F16) KV cache ("Luce
// DFlash: 単一RTX 3090で最大2倍のスループットを目指すQwen3.6-27B", feature list:
// Q4_0 KV as the route to about 128K context).

#include "tv_internal.h"

namespace tv {

typedef _Float16 ph2 __attribute__((ext_vector_type(2)));
typedef uint32_t pu4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;

// fp16 pairs of the codes of one dword (8 nibbles, offset by 8), times a scale:
// the instruction mix of the Q4_0 dequantisation (bit masks into fp16 1024 +
// code, one subtraction or fused multiply-add for the offset, one multiply)
__device__ __forceinline__ ph2 decode_dword(uint32_t x, ph2 s, ph2 acc)
{
    const uint32_t y = x >> 8;
    const ph2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const ph2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const ph2 off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const ph2 v0 = __builtin_bit_cast(ph2, (x & 0x000F000Fu) | 0x64006400u) - off;
    const ph2 v1 = __builtin_bit_cast(ph2, (y & 0x000F000Fu) | 0x64006400u) - off;
    const ph2 v2 = __builtin_elementwise_fma(__builtin_bit_cast(ph2, (x & 0x00F000F0u) | 0x64006400u), sixteenth, off_hi);
    const ph2 v3 = __builtin_elementwise_fma(__builtin_bit_cast(ph2, (y & 0x00F000F0u) | 0x64006400u), sixteenth, off_hi);
    return acc + (v0 * s + v1 * s) + (v2 * s + v3 * s);
}

// Each workgroup streams its own contiguous range of 16-byte pieces (the
// first n16 % gridDim.x workgroups one piece more) with streaming
// (nontemporal) loads, U per thread issued before any is used (8 for the
// plain read, 4 for the decoding read, which is bound by its vector work);
// one checksum word per workgroup (so that no load can be dropped). On gfx950
// this reads 1 GiB at about 6.9 TB/s, where a grid-stride loop with ordinary
// loads reads 5.1-5.6 TB/s.
template <int KIND>
__global__ void __launch_bounds__(kProbeThreads) stream_probe(const pu4 *base, uint64_t n16, uint32_t *checksums)
{
    const uint64_t per = n16 / gridDim.x, extra = n16 % gridDim.x;
    const uint64_t begin = (uint64_t)blockIdx.x * per + (blockIdx.x < extra ? blockIdx.x : extra);
    const uint64_t len = per + (blockIdx.x < extra ? 1 : 0);
    constexpr int U = KIND == 0 ? 8 : 4;
    const pu4 *b = base + begin;
    uint32_t acc = 0;
    ph2 hacc = {(_Float16)0.f, (_Float16)0.f};
    const ph2 s = {(_Float16)0.05f, (_Float16)0.05f};
    for (uint64_t i = threadIdx.x; i < len; i += U * kProbeThreads) {
        pu4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint64_t j = i + k * kProbeThreads;
            v[k] = j < len ? __builtin_nontemporal_load(b + j) : (pu4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if constexpr (KIND == 0) {
                acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
            } else {
                hacc = decode_dword(v[k].x, s, hacc);
                hacc = decode_dword(v[k].y, s, hacc);
                hacc = decode_dword(v[k].z, s, hacc);
                hacc = decode_dword(v[k].w, s, hacc);
            }
        }
    }
    if constexpr (KIND != 0) acc = __builtin_bit_cast(uint32_t, hacc);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
    __shared__ uint32_t red[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < kProbeThreads / 64; ++w) r ^= red[w];
        checksums[blockIdx.x] = r;
    }
}

int launch_stream_probe(const void *buf, uint64_t bytes, int kind, uint32_t *checksums, int n_wg,
                        hipStream_t stream)
{
    const pu4 *base = (const pu4 *)buf;
    uint64_t n16 = bytes / 16;
    void *args[] = {(void *)&base, (void *)&n16, (void *)&checksums};
    const void *fn = kind == 0 ? (const void *)stream_probe<0> : (const void *)stream_probe<1>;
    return hipLaunchKernel(fn, dim3(n_wg), dim3(kProbeThreads), args, 0, stream) == hipSuccess ? TV_OK : TV_E_HIP;
}

}  // namespace tv
