// Merge of the split partials with each node's tree ancestors and the
// window rows left to it (internal header of libtv.so): the body shared by
// merge_kernel and the work-queue step kernel.
//
// Method: a node's softmax runs over the committed cache rows it sees and its
// tree ancestors (itself included), the DDTree verify of "Luce DFlash: 単一
// RTX 3090で最大2倍のスループットを目指すQwen3.6-27B", feature list; the
// split-K partials are combined by their log-sum-exp weights.
#pragma once

#include "tv_split_common.h"

namespace tv {

// ---------------------------------------------------------------------------
// Merge: per output row (node i, query head h), the tree ancestors' scores in
// fp32, then the log-sum-exp combination of the split partials and the tree.

// The tensors of one layer's merge (device memory): query rows, the tree's
// K / V rows, the split partials, the output, the KV cache.
struct MergePtrs {
    const _Float16 *q;
    const _Float16 *k_tree;
    const _Float16 *v_tree;
    const _Float16 *ws_o;
    const float *ws_m;
    float *out;
    const uint8_t *k_cache;
    const uint8_t *v_cache;
};

struct MergeArgs {
    MergePtrs p;
    int32_t NR;
    int32_t H_q;
    int32_t H_kv;
    int32_t G;
    int32_t S;
    float c;  // scale * log2(e)
    // per-position window: cache rows [head_begin, head_begin + n_head) are
    // scored here, node i skipping the first head_skip[i] of them
    int64_t head_begin;
    int32_t n_head;
    int32_t head_skip[TV_MAX_NODES];  // 32-bit entries: a scalar load per node
    // cache rows [tail_begin, tail_end) of the window that do not fill a
    // whole chunk of the split kernel
    int64_t tok_stride;
    int64_t head_stride;
    int64_t tail_begin;
    int32_t n_tail;
    int32_t kv_type;
    uint64_t anc[TV_MAX_NODES];
};

// Values d0 .. d0+n-1 (inside one 32-wide block) of one cache row, decoded
// exactly in fp32.
template <int N>
__device__ __forceinline__ void cache_values(const uint8_t *row, int kv_type, int d0, float (&out)[N])
{
    if (kv_type == TV_KV_Q4_0) {
        const uint8_t *blk = row + 18 * (d0 / 32);
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(blk[0] | (blk[1] << 8)));
#pragma unroll
        for (int p = 0; p < N; ++p) {
            const int e = (d0 + p) % 32;
            const int byte = blk[2 + (e % 16)];
            const int code = e < 16 ? (byte & 15) : (byte >> 4);
            out[p] = s * (float)(code - 8);
        }
    } else {
        const _Float16 *h = (const _Float16 *)row + d0;
#pragma unroll
        for (int p = 0; p < N; ++p) out[p] = (float)h[p];
    }
}

// One workgroup of 256 threads per output row (node i, query head h), in
// three steps of independent loads:
//   1. thread (split group sg, d-octet dq) loads the partial states of its
//      splits s = sg, sg + NGR, ... and folds them against their own maximum;
//      at the same time the threads score the row's extra keys (its tree
//      ancestors, then the window's tail rows), KL lanes per key;
//   2. the maximum over splits and extra keys;
//   3. the extra keys' V rows are spread over the split groups (the first
//      VPF of each group are loaded during step 1, as they do not depend on
//      the scores); the groups' sums meet in LDS.
// A split's weight is 2^(lse_s - m*) with lse_s the log2 of its softmax
// denominator, an extra key's 2^(score - m*); the output is the weighted sum
// of the splits' normalised outputs and the keys' V rows over the sum of the
// weights.
template <int D>
struct MergeLds {
    float sk[TV_MAX_NODES + 2 * kChunk];
    float red_s[256 / (D / 8)];
    float red_k[4];
    __attribute__((aligned(16))) float acc_s[256 / (D / 8)][D];
    float l_s[256 / (D / 8)];
};

// Output row `row` by 256 threads (t = 0..255) with LDS `sm`; the caller's
// other threads, if any, pass the same barriers. With `store` false the row
// is computed (row must still be valid) but not written. With CPOL set
// (kCpolSc1) the split partials are read with device-coherent loads, which
// see partials that device-coherent stores of other workgroups of the same
// launch completed (their byte offsets must fit 31 bits).
template <int D, int CPOL = 0>
__device__ __forceinline__ void merge_row(const MergeArgs &a, const MergePtrs &p, int row, int t, bool store,
                                          MergeLds<D> &sm)
{
    constexpr int QD = D / 8;       // d-octets per row
    constexpr int NGR = 256 / QD;   // split groups
    constexpr int KL = 16;          // lanes per extra key
    constexpr int KPT = D / KL;     // values per lane of a key's dot product
    constexpr int KPASS = 256 / KL; // extra keys per pass
    constexpr int SMAX = 8;         // splits per thread held in registers
    constexpr int VPF = 2;          // extra keys per split group whose V is loaded early
    static_assert(32 % KPT == 0, "a lane's key slice lies inside one 32-value block");
    float *const sk = sm.sk;
    float *const red_s = sm.red_s;
    float *const red_k = sm.red_k;
    auto &acc_s = sm.acc_s;
    float *const l_s = sm.l_s;

    const int lane = t & 63, w = t >> 6;
    const int dq = t % QD, sg = t / QD;
    // the node index is uniform: its ancestor mask and head skip come
    // through scalar loads, which do not wait behind the vector loads above
    const int i = __builtin_amdgcn_readfirstlane(row / a.H_q), h = row % a.H_q, g = h / a.G;
    const uint64_t anc = a.anc[i];
    const int na = __builtin_popcountll(anc);
    const int hs = a.head_skip[i];
    const int nh = a.n_head - hs;     // head rows this node sees
    const int nk = na + nh + a.n_tail;
    // extra key kk -> cache row (head rows, then tail rows) for kk >= na
    auto extra_row = [&](int kk) -> int64_t {
        return kk < na + nh ? a.head_begin + hs + (kk - na) : a.tail_begin + (kk - na - nh);
    };
    const uint8_t *kh = p.k_cache + (int64_t)g * a.head_stride;
    const uint8_t *vh = p.v_cache + (int64_t)g * a.head_stride;

    const int kl = t % KL;
    // row of the kk-th ancestor (kk < na) in the tree's [node][H_kv][D] rows
    auto tree_row = [&](int kk) -> int64_t {
        uint64_t mm = anc;
        for (int r = 0; r < kk; ++r) mm &= mm - 1;
        return (int64_t)__builtin_ctzll(mm) * a.H_kv + g;
    };
    // V values of extra key kk, for the cache rows (kk >= na), decoded exactly
    auto cache_v = [&](int kk, float (&vv)[8]) {
        cache_values<8>(vh + extra_row(kk) * a.tok_stride, a.kv_type, 8 * dq, vv);
    };
    auto cache_k = [&](int kk, float (&kv)[KPT]) {
        cache_values<KPT>(kh + extra_row(kk) * a.tok_stride, a.kv_type, kl * KPT, kv);
    };
    // Requested before anything waits on memory: the V rows of this group's
    // first extra keys (they do not depend on the scores), the query slice
    // and the key slices of the first score pass. Tree rows are loaded raw
    // and converted where they are used, so that no load waits at its branch;
    // cache rows (window head or tail), decoded where they are loaded, only
    // occur with a window or a partial last chunk.
    float vpf[VPF][8];
    h8 vtr[VPF];
#pragma unroll
    for (int j = 0; j < VPF; ++j) {
        const int kk = sg + NGR * j;
        if (kk < na) vtr[j] = *(const h8 *)(p.v_tree + tree_row(kk) * D + 8 * dq);
        else if (kk < nk) cache_v(kk, vpf[j]);
    }
    typedef _Float16 hk __attribute__((ext_vector_type(KPT)));  // a lane's slice of a row
    const hk qr = *(const hk *)(p.q + (int64_t)row * D + kl * KPT);
    const int kk0 = t / KL;
    hk ktr;
    float kc0[KPT];
    if (kk0 < na) ktr = *(const hk *)(p.k_tree + tree_row(kk0) * D + kl * KPT);
    else if (kk0 < nk) cache_k(kk0, kc0);

    // step 1a's loads for this thread's first SMAX splits, behind those
    // above (the scores need their loads sooner); no branch around a load: a
    // split past the last reads split 0, and the fold gives it no weight.
    // Without splits (no whole chunk of keys) the workspace may be absent:
    // nothing is read from it.
    float mv[SMAX];
    h8 ov[SMAX];
    // partial of split s (loads only)
    auto load_part = [&](int s, float &m, h8 &o) {
        if constexpr (CPOL == 0) {
            const int64_t base = (int64_t)s * a.NR + row;
            m = p.ws_m[base];
            o = *(const h8 *)(p.ws_o + base * D + 8 * dq);
        } else {
            const u32 base = (u32)s * (u32)a.NR + (u32)row;
            const __amdgpu_buffer_rsrc_t rm = raw_rsrc(p.ws_m, 0x7FFFFFFFu);
            const __amdgpu_buffer_rsrc_t ro = raw_rsrc(p.ws_o, 0x7FFFFFFFu);
            m = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rm, base * 4u, 0, CPOL));
            o = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(ro, base * (u32)(2 * D) + 16u * (u32)dq,
                                                                            0, CPOL));
        }
    };
    if (a.S > 0) {
#pragma unroll
        for (int k = 0; k < SMAX; ++k) {
            const int s = sg + NGR * k;
            load_part(s < a.S ? s : 0, mv[k], ov[k]);
        }
    }

    // ---- step 1a: this thread's splits, folded against their maximum
    float ms = kNegBig;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    for (int s0 = sg; s0 < a.S; s0 += NGR * SMAX) {
        if (s0 != sg) {
#pragma unroll
            for (int k = 0; k < SMAX; ++k) {
                const int s = s0 + NGR * k;
                load_part(s < a.S ? s : 0, mv[k], ov[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < SMAX; ++k) mv[k] = s0 + NGR * k < a.S ? mv[k] : kNegBig;
        float mb = ms;
#pragma unroll
        for (int k = 0; k < SMAX; ++k) mb = fmaxf(mb, mv[k]);
        const float r = exp2f(ms - mb);
        L *= r;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= r;
#pragma unroll
        for (int k = 0; k < SMAX; ++k) {
            const float f = exp2f(mv[k] - mb);
            L += f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(f, (float)ov[k][e], acc[e]);
        }
        ms = mb;
    }
    // ---- step 1b: scores of the extra keys (ancestors, then tail rows)
    float mk = -INFINITY;
    {
        float qv[KPT];
#pragma unroll
        for (int p = 0; p < KPT; ++p) qv[p] = (float)qr[p];
        for (int base = 0; base < nk; base += KPASS) {
            const int kk = base + t / KL;
            float part = 0.f;
            if (kk < nk) {
                float kv[KPT];
                if (kk < na) {
                    const hk kr = base == 0 ? ktr : *(const hk *)(p.k_tree + tree_row(kk) * D + kl * KPT);
#pragma unroll
                    for (int p = 0; p < KPT; ++p) kv[p] = (float)kr[p];
                } else if (base == 0) {
#pragma unroll
                    for (int p = 0; p < KPT; ++p) kv[p] = kc0[p];
                } else {
                    cache_k(kk, kv);
                }
#pragma unroll
                for (int p = 0; p < KPT; ++p) part = __builtin_fmaf(qv[p], kv[p], part);
            }
#pragma unroll
            for (int off = KL / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off);
            if (kk < nk) {
                const float sj = part * a.c;
                if (kl == 0) sk[kk] = sj;
                mk = fmaxf(mk, sj);
            }
        }
    }
    // ---- step 2: maxima
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mk = fmaxf(mk, __shfl_xor(mk, off));
    if (lane == 0) red_k[w] = mk;
    if (dq == 0) red_s[sg] = ms;
    __syncthreads();
    float mstar = fmaxf(fmaxf(red_k[0], red_k[1]), fmaxf(red_k[2], red_k[3]));
#pragma unroll
    for (int k = 0; k < NGR; ++k) mstar = fmaxf(mstar, red_s[k]);
    {
        const float r = exp2f(ms - mstar);
        L *= r;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= r;
    }
    // ---- step 3: the extra keys' V rows, spread over the split groups
#pragma unroll
    for (int j = 0; j < VPF; ++j) {
        const int kk = sg + NGR * j;
        if (kk < nk) {
            const float f = exp2f(sk[kk] - mstar);
            L += f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(f, kk < na ? (float)vtr[j][e] : vpf[j][e], acc[e]);
        }
    }
    for (int kk = sg + NGR * VPF; kk < nk; kk += NGR) {
        const float f = exp2f(sk[kk] - mstar);
        L += f;
        float vv[8];
        if (kk < na) {
            const h8 vr = *(const h8 *)(p.v_tree + tree_row(kk) * D + 8 * dq);
#pragma unroll
            for (int e = 0; e < 8; ++e) vv[e] = (float)vr[e];
        } else {
            cache_v(kk, vv);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(f, vv[e], acc[e]);
    }
    *(f4 *)&acc_s[sg][8 * dq] = (f4){acc[0], acc[1], acc[2], acc[3]};
    *(f4 *)&acc_s[sg][8 * dq + 4] = (f4){acc[4], acc[5], acc[6], acc[7]};
    if (dq == 0) l_s[sg] = L;
    __syncthreads();
    if (t < D && store) {
        float sum = 0.f, Ls = 0.f;
#pragma unroll
        for (int k = 0; k < NGR; ++k) {
            sum += acc_s[k][t];
            Ls += l_s[k];
        }
        p.out[(int64_t)row * D + t] = sum / Ls;
    }
}

// Host side (tv_attn.hip): the arguments of one layer's split and merge
// launches, with its split partials at `ws`.
void fill_split_args(const tv_attn_desc *d, const tv_attn_ptrs *p, const SplitPlan &plan, void *ws, SplitArgs *out);
void fill_merge_args(const tv_attn_desc *d, const tv_attn_ptrs *p, const SplitPlan &plan, void *ws, MergeArgs *out);
// The warp-specialised split kernel of a plan, or null.
split_fn pick_ws(const tv_attn_desc *d, const SplitPlan &p);

}  // namespace tv
