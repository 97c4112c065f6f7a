// KV commit of the accepted path for gfx950: after greedy acceptance the root
// and the accepted nodes become committed tokens, so their K and V rows are
// appended to the layer's cache, quantised to Q4_0 or copied as F16.
//
// Method: the verify state of the target keeps its KV cache in Q4_0 (to
// reach about 128K tokens) or F16 ("Luce DFlash: 単一RTX 3090で最大2倍の
// スループットを目指すQwen3.6-27B", feature list; "We got 207 tok/s with
// Qwen3.5-27B on an RTX 3090", "What we built vs what we didn't"). The pages
// give no quantiser; the one used here, per 32-value block and in fp32:
// m = the value of largest magnitude (the first on ties), d = m / -8 stored
// as fp16 (nearest, ties to even; +0 for a block of zeros), id = 1/d (0 when
// d == 0), and each value
// gets code floor(x*id + 8.5) clamped to 0..15, with the product and the sum
// rounded separately and NaN giving code 0.
//
// One workgroup (one wave) per (path position r, KV head g, layer); positions
// past the accepted length exit at once. The accepted length and the path
// are read from the acceptance result on the device, so the commit can follow
// the acceptance on the stream without a host round trip. A Q4_0 block is
// quantised by two lanes (16 values each: lane h holds elements 8h..8h+7 and
// 16+8h..16+8h+7, so its codes fill code bytes 8h..8h+7); the lanes agree on
// the value of largest magnitude through one exchange.

#include "tv_internal.h"

namespace tv {

typedef _Float16 c_h8 __attribute__((ext_vector_type(8)));

constexpr int kMaxCommitLayers = 64;

template <int ML>
struct CommitArgs {
    const int32_t *result;  // acceptance result: [0] n_acc, [2 ..] path nodes
    int64_t n_ctx;
    int64_t tok_stride;
    int64_t head_stride;
    int32_t n;
    int32_t H_kv;
    int32_t D;
    int32_t kv_type;
    const _Float16 *k_tree[ML];
    const _Float16 *v_tree[ML];
    uint8_t *k_cache[ML];
    uint8_t *v_cache[ML];
};

// Code of one value: floor(x*id + 8.5) clamped to 0..15 (product and sum
// rounded separately; NaN gives 0, as fmaxf returns the other operand).
__device__ __forceinline__ uint32_t q4_code(float x, float id)
{
#pragma clang fp contract(off)
    const float p = x * id;
    const float c = p + 8.5f;
    return (uint32_t)fminf(fmaxf(floorf(c), 0.0f), 15.0f);
}

template <int ML>
__global__ void __launch_bounds__(64) commit_kernel(const CommitArgs<ML> a)
{
    const int r = blockIdx.x, g = blockIdx.y, layer = blockIdx.z, t = threadIdx.x;
    // both words of the result are requested at once (2 + r < 2 + 2n is in
    // bounds whatever n_acc is); one branch on the combined test
    const int n_acc = a.result[0];
    const int node = a.result[2 + r];
    const bool skip = (n_acc < 0) | (n_acc >= a.n) | (r > n_acc) | (node < 0) | (node >= a.n);
    if (skip) return;
    const int64_t src_off = ((int64_t)node * a.H_kv + g) * a.D;
    const int64_t dst_off = (int64_t)g * a.head_stride + (a.n_ctx + r) * a.tok_stride;
    if (a.kv_type == TV_KV_Q4_0) {
        const int nb = a.D / 32;        // blocks per row
        const int blk = t >> 1, h = t & 1;  // lanes [0, 2nb): K blocks, [2nb, 4nb): V blocks
        const bool active = blk < 2 * nb;
        const bool isv = blk >= nb;
        const int b = isv ? blk - nb : blk;
        float x[16];
        if (active) {
            const _Float16 *src = (isv ? a.v_tree[layer] : a.k_tree[layer]) + src_off + 32 * b + 8 * h;
            const c_h8 lo = *(const c_h8 *)src;
            const c_h8 hi = *(const c_h8 *)(src + 16);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                x[k] = (float)lo[k];
                x[8 + k] = (float)hi[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) x[k] = 0.0f;
        }
        // largest magnitude, the first in element order on ties: each lane
        // scans its values in element order, then the two lanes compare
        float amax = 0.0f, m = 0.0f;
        int idx = 32;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const float v = fabsf(x[k]);
            if (amax < v) {
                amax = v;
                m = x[k];
                idx = k < 8 ? 8 * h + k : 16 + 8 * h + (k - 8);
            }
        }
        const float amax_p = __shfl_xor(amax, 1);
        const float m_p = __shfl_xor(m, 1);
        const int idx_p = __shfl_xor(idx, 1);
        if (amax_p > amax || (amax_p == amax && idx_p < idx)) m = m_p;
        const float d = m != 0.0f ? m / -8.0f : 0.0f;
        const float id = d != 0.0f ? 1.0f / d : 0.0f;
        if (active) {
            uint16_t *dst = (uint16_t *)((isv ? a.v_cache[layer] : a.k_cache[layer]) + dst_off + 18 * b);
            if (h == 0) dst[0] = __builtin_bit_cast(uint16_t, (_Float16)d);
#pragma unroll
            for (int k = 0; k < 8; k += 2) {
                const uint32_t b0 = q4_code(x[k], id) | (q4_code(x[8 + k], id) << 4);
                const uint32_t b1 = q4_code(x[k + 1], id) | (q4_code(x[9 + k], id) << 4);
                dst[1 + 4 * h + k / 2] = (uint16_t)(b0 | (b1 << 8));
            }
        }
    } else {
        const int nv = a.D / 8;  // 16-byte pieces per row
        for (int i = t; i < 2 * nv; i += 64) {
            const bool isv = i >= nv;
            const int p = isv ? i - nv : i;
            const uint4 v = *(const uint4 *)((isv ? a.v_tree[layer] : a.k_tree[layer]) + src_off + 8 * p);
            *(uint4 *)((isv ? a.v_cache[layer] : a.k_cache[layer]) + dst_off + 16 * p) = v;
        }
    }
}

template <int ML>
static int launch_commit_t(const tv_commit_desc *d, int n_layers, const int32_t *result,
                           const void *const *k_tree, const void *const *v_tree, void *const *k_cache,
                           void *const *v_cache, hipStream_t stream)
{
    CommitArgs<ML> a;
    a.result = result;
    a.n_ctx = d->n_ctx;
    a.tok_stride = d->kv_token_stride;
    a.head_stride = d->kv_head_stride;
    a.n = d->n_nodes;
    a.H_kv = d->n_kv_heads;
    a.D = d->head_dim;
    a.kv_type = d->kv_type;
    for (int l = 0; l < ML; ++l) {
        const bool on = l < n_layers;
        a.k_tree[l] = on ? (const _Float16 *)k_tree[l] : nullptr;
        a.v_tree[l] = on ? (const _Float16 *)v_tree[l] : nullptr;
        a.k_cache[l] = on ? (uint8_t *)k_cache[l] : nullptr;
        a.v_cache[l] = on ? (uint8_t *)v_cache[l] : nullptr;
    }
    void *args[] = {(void *)&a};
    return hipLaunchKernel((const void *)commit_kernel<ML>, dim3(d->n_nodes, d->n_kv_heads, n_layers), dim3(64),
                           args, 0, stream) == hipSuccess
               ? TV_OK
               : TV_E_HIP;
}

int launch_commit(const tv_commit_desc *d, int n_layers, const int32_t *result, const void *const *k_tree,
                  const void *const *v_tree, void *const *k_cache, void *const *v_cache, hipStream_t stream)
{
    for (int l0 = 0; l0 < n_layers; l0 += kMaxCommitLayers) {
        const int nl = n_layers - l0 < kMaxCommitLayers ? n_layers - l0 : kMaxCommitLayers;
        const int rc = nl == 1 ? launch_commit_t<1>(d, 1, result, k_tree + l0, v_tree + l0, k_cache + l0,
                                                    v_cache + l0, stream)
                               : launch_commit_t<kMaxCommitLayers>(d, nl, result, k_tree + l0, v_tree + l0,
                                                                   k_cache + l0, v_cache + l0, stream);
        if (rc) return rc;
    }
    return TV_OK;
}

}  // namespace tv
