// Tree-verify attention for gfx950: split-K flash decode over the committed
// KV cache with the whole packed (GQA group x tree node) query block of one KV
// head held by one workgroup, then a merge kernel that adds each node's tree
// ancestors and combines the splits.
//
// Method: the target model scores all nodes of a DDTree draft tree in one
// verify pass; each node attends to the committed KV cache (F16 or Q4_0,
// optionally limited to a 2048-token sliding window at decode) and, inside
// the tree, to its ancestors. Sources: "Luce DFlash: 単一RTX 3090で最大2倍の
// スループットを目指すQwen3.6-27B", feature list (DDTree tree verify with
// budget 22 and block size 16, greedy verify, Q4_0 KV up to about 128K,
// sliding-window flash attention with a 2048-token window); "We got 207 tok/s
// with Qwen3.5-27B on an RTX 3090", "What we built vs what we didn't" (DDTree
// tree-structured verify; Q4_0 KV cache to fit 128K).
//
// Split kernel, one workgroup = 4 wave64s per (key-range split, KV head, row
// group):
//   * Rows: the M = G * n query rows of a KV head (row r = node r/G, query
//     head g*G + r%G) are cut into 16-row tiles. Each wave owns whole tiles;
//     one or two left-over tiles are "shared": every wave computes them over
//     its own quarter (16 keys) of each 64-key chunk and the four partial
//     softmax states are merged through LDS at the end.
//   * Keys stream in 64-row chunks, double-buffered in LDS. Every thread
//     loads raw Q4_0 bytes (or fp16) for the next chunk into registers while
//     the current chunk is computed, then dequantises in registers (fp16 bit
//     tricks, exact code - 8, one rounding when the fp16 scale is applied)
//     and writes K row-major and V transposed into LDS.
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_f16 with fp32
//     accumulation; Q fragments stay in registers, the O accumulators too.
//   * Online softmax in the exp2 domain with a lazy rescale (the running max
//     only moves when a chunk's max exceeds it by more than 2^8), P rounded to
//     fp16 and its row sums taken from the rounded values.

#include <string.h>

#include "tv_merge.h"
#include "tv_split_common.h"

namespace tv {

// Thread t of the 256 handles K (t < 128) or V (t >= 128), NK consecutive
// keys of the chunk and one 32-value block of those rows.
template <int D, int KVT>
__device__ __forceinline__ void load_raw(const SplitArgs &a, int gkv, int64_t kbase, int tid, u32 *raw)
{
    using St = Stage<D, KVT>;
    const int isv = tid >> 7, u = tid & 127;
    const int b = u % St::NB, key0 = (u / St::NB) * St::NK;
    const uint8_t *base = (isv ? a.v_cache : a.k_cache) + (int64_t)gkv * a.head_stride;
#pragma unroll
    for (int kk = 0; kk < St::NK; ++kk) {
        const int64_t row = kbase + key0 + kk;
        if constexpr (KVT == TV_KV_Q4_0) {
            const u32 *p = (const u32 *)(base + row * a.tok_stride + ((18 * b) & ~3));
#pragma unroll
            for (int j = 0; j < 5; ++j) raw[kk * 5 + j] = p[j];
        } else {
            const uint4 *p = (const uint4 *)(base + row * a.tok_stride + 64 * b);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 t = p[j];
                raw[kk * 16 + 4 * j + 0] = t.x;
                raw[kk * 16 + 4 * j + 1] = t.y;
                raw[kk * 16 + 4 * j + 2] = t.z;
                raw[kk * 16 + 4 * j + 3] = t.w;
            }
        }
    }
}

// Dequantise the raw registers and write them into one LDS stage:
//   K:   ks[key][32b + 8k + j], for Q4_0 the 8 values of code dword k in the
//        order of q4_unpack; for F16 the natural order.
//   V^T: vt[d][vpos(key)].
template <int D, int KVT>
__device__ __forceinline__ void store_stage(const u32 *raw, _Float16 *ks, _Float16 *vt, int tid)
{
    using St = Stage<D, KVT>;
    const int isv = tid >> 7, u = tid & 127;
    const int b = u % St::NB, key0 = (u / St::NB) * St::NK;
    if constexpr (KVT == TV_KV_Q4_0) {
        // code dwords and scale of key kk: block starts at byte 18b of the row;
        // the 5 raw dwords start at (18b & ~3).
        u32 cw[St::NK][4];
        _Float16 sc[St::NK];
#pragma unroll
        for (int kk = 0; kk < St::NK; ++kk) {
            const u32 *r = raw + kk * 5;
            if (b & 1) {  // block at 2 mod 4: scale in the high half of r[0]
                sc[kk] = __builtin_bit_cast(_Float16, (uint16_t)(r[0] >> 16));
#pragma unroll
                for (int k = 0; k < 4; ++k) cw[kk][k] = r[k + 1];
            } else {  // block at 0 mod 4: codes start 2 bytes into r[0]
                sc[kk] = __builtin_bit_cast(_Float16, (uint16_t)(r[0] & 0xFFFFu));
#pragma unroll
                for (int k = 0; k < 4; ++k) cw[kk][k] = (r[k] >> 16) | (r[k + 1] << 16);
            }
        }
        if (!isv) {
#pragma unroll
            for (int kk = 0; kk < St::NK; ++kk) {
                const h2 s2 = {sc[kk], sc[kk]};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    h2 v[4];
                    q4_unpack(cw[kk][k], v);
                    h8 o;
                    o.s01 = v[0] * s2;
                    o.s23 = v[1] * s2;
                    o.s45 = v[2] * s2;
                    o.s67 = v[3] * s2;
                    *(h8 *)(ks + (key0 + kk) * St::KSTR + 32 * b + 8 * k) = o;
                }
            }
        } else {
            const int p0 = vpos(key0);
            if constexpr (St::NK >= 2) {
                // pairs of keys: interleave their code bytes so every fp16
                // pair holds one element of two keys
#pragma unroll
                for (int pr = 0; pr < St::NK / 2; ++pr) {
                    const h2 s2 = {sc[2 * pr], sc[2 * pr + 1]};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const u32 x0 = cw[2 * pr][k], x1 = cw[2 * pr + 1][k];
                        const u32 za = __builtin_amdgcn_perm(x1, x0, 0x05040100u);
                        const u32 zb = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
                        h2 va[4], vb[4];
                        q4_unpack(za, va);  // elements 4k, 4k+1, 4k+16, 4k+17
                        q4_unpack(zb, vb);  // elements 4k+2, 4k+3, 4k+18, 4k+19
                        const int e[8] = {4 * k, 4 * k + 1, 4 * k + 16, 4 * k + 17,
                                          4 * k + 2, 4 * k + 3, 4 * k + 18, 4 * k + 19};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            *(h2 *)(vt + (32 * b + e[t]) * St::VSTR + p0 + 2 * pr) = va[t] * s2;
                            *(h2 *)(vt + (32 * b + e[4 + t]) * St::VSTR + p0 + 2 * pr) = vb[t] * s2;
                        }
                    }
                }
            } else {
                const h2 s2 = {sc[0], sc[0]};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    h2 v[4];
                    q4_unpack(cw[0][k], v);
                    const int e[8] = {4 * k, 4 * k + 2, 4 * k + 1, 4 * k + 3,
                                      4 * k + 16, 4 * k + 18, 4 * k + 17, 4 * k + 19};
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const h2 w = v[t] * s2;
                        vt[(32 * b + e[2 * t]) * St::VSTR + p0] = w.x;
                        vt[(32 * b + e[2 * t + 1]) * St::VSTR + p0] = w.y;
                    }
                }
            }
        }
    } else {
        if (!isv) {
#pragma unroll
            for (int kk = 0; kk < St::NK; ++kk)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint4 t;
                    t.x = raw[kk * 16 + 4 * j];
                    t.y = raw[kk * 16 + 4 * j + 1];
                    t.z = raw[kk * 16 + 4 * j + 2];
                    t.w = raw[kk * 16 + 4 * j + 3];
                    *(uint4 *)(ks + (key0 + kk) * St::KSTR + 32 * b + 8 * j) = t;
                }
        } else {
            const int p0 = vpos(key0);
            if constexpr (St::NK >= 2) {
#pragma unroll
                for (int pr = 0; pr < St::NK / 2; ++pr)
#pragma unroll
                    for (int w = 0; w < 16; ++w) {
                        const u32 x0 = raw[(2 * pr) * 16 + w], x1 = raw[(2 * pr + 1) * 16 + w];
                        // dword w holds elements 2w, 2w+1 of the block
                        *(u32 *)(vt + (32 * b + 2 * w) * St::VSTR + p0 + 2 * pr) =
                            __builtin_amdgcn_perm(x1, x0, 0x05040100u);
                        *(u32 *)(vt + (32 * b + 2 * w + 1) * St::VSTR + p0 + 2 * pr) =
                            __builtin_amdgcn_perm(x1, x0, 0x07060302u);
                    }
            } else {
#pragma unroll
                for (int w = 0; w < 16; ++w) {
                    const h2 v = as_h2(raw[w]);
                    vt[(32 * b + 2 * w) * St::VSTR + p0] = v.x;
                    vt[(32 * b + 2 * w + 1) * St::VSTR + p0] = v.y;
                }
            }
        }
    }
}

template <int D, int KVT, int NOWN, int NSH, bool MASK>
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
split_kernel(const SplitArgs a)
{
    using St = Stage<D, KVT>;
    constexpr int NB = St::NB;
    constexpr int NDT = D / 16;
    constexpr int NS = NOWN + NSH;
    static_assert(NS >= 1 && NS <= kMaxSlots, "slots");
    __shared__ __attribute__((aligned(16))) _Float16 lds[2 * St::ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int split = blockIdx.x, gkv = blockIdx.y, rg = blockIdx.z;

    TileMap tm;
    tm.init(a.M, rg, gridDim.z);
    const int t_end = tm.t_end;
    int tile[NS];
#pragma unroll
    for (int k = 0; k < NOWN; ++k) tile[k] = tm.t0 + 4 * k + w;
#pragma unroll
    for (int u = 0; u < NSH; ++u) tile[NOWN + u] = tm.t0 + 4 * NOWN + u;

    const int64_t c_begin = split_chunk_begin(a, split);
    const int64_t c_end = split_chunk_begin(a, split + 1);

    // the query rows (from L2) are requested first, the first chunk's cache
    // rows (from HBM) next, so that the two are in flight together and the
    // query rows can be staged before the cache rows arrive
    QStage<D, KVT, NOWN, NSH> qs;
    qs.load(a, gkv, tm.t0, tid);
    // (every split has at least one chunk: the plan keeps S <= n_chunks)
    u32 raw[St::RAW];
    load_raw<D, KVT>(a, gkv, chunk_row<MASK>(a, c_begin), tid, raw);

    h8 qf[NS][NB];
    qs.store(tm.t0, tile, tid, col, grp, lds, qf);
    // The Q fragments are read only as MFMA B operands, which may come from
    // AGPRs; parking them there leaves the VGPRs to the accumulators.
#pragma unroll
    for (int k = 0; k < NS; ++k)
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) asm volatile("" : "+a"(qf[k][bb]));

    f4 o[NS][NDT];
    float m[NS], l[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        m[k] = kNegBig;
        l[k] = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[k][dt] = (f4){0.f, 0.f, 0.f, 0.f};
    }

    for (int64_t c = c_begin; c < c_end; ++c) {
        const int st = (int)((c - c_begin) & 1);
        _Float16 *ks = lds + st * St::ELEMS;
        _Float16 *vt = ks + St::KELEMS;
        store_stage<D, KVT>(raw, ks, vt, tid);
        if (c + 1 < c_end) load_raw<D, KVT>(a, gkv, chunk_row<MASK>(a, c + 1), tid, raw);
        __syncthreads();


        // ---- S^T tiles: 4 key tiles x own slots, key tile w x shared slots
        f4 sacc[NOWN > 0 ? NOWN : 1][4];
        f4 ssh[NSH > 0 ? NSH : 1];
#pragma unroll
        for (int k = 0; k < NOWN; ++k)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) sacc[k][kt] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NSH; ++u) ssh[u] = (f4){0.f, 0.f, 0.f, 0.f};
        // K fragments of block bb+1 are read from LDS while the MFMAs of
        // block bb run (one block of lookahead, 5 fragments per block).
        h8 kf[2][5];
        auto kload = [&](int bb, h8(&f)[5]) {
            if constexpr (NOWN > 0) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
                    f[kt] = *(const h8 *)(ks + (16 * kt + col) * St::KSTR + 32 * bb + 8 * grp);
            }
            if constexpr (NSH > 0) f[4] = *(const h8 *)(ks + (16 * w + col) * St::KSTR + 32 * bb + 8 * grp);
        };
        kload(0, kf[0]);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            if (bb + 1 < NB) kload(bb + 1, kf[(bb + 1) & 1]);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int k = 0; k < NOWN; ++k)
                    sacc[k][kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[bb & 1][kt], qf[k][bb], sacc[k][kt], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < NSH; ++u)
                ssh[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[bb & 1][4], qf[NOWN + u][bb], ssh[u], 0, 0, 0);
            TV_SCHED_FENCE();
        }
        if constexpr (MASK) {
            if (chunk_masked(a, c)) {
#pragma unroll
                for (int k = 0; k < NOWN; ++k) {
                    const int thr = masked_keys(a, c, row_skip(a, tile[k], t_end, col));
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt) mask_tile(sacc[k][kt], kt, grp, thr);
                }
#pragma unroll
                for (int u = 0; u < NSH; ++u)
                    mask_tile(ssh[u], w, grp, masked_keys(a, c, row_skip(a, tile[NOWN + u], t_end, col)));
            }
        }

        // ---- online softmax -> fp16 P^T fragments
        h8 pf[NOWN > 0 ? NOWN : 1][2];
        h8 psh[NSH > 0 ? NSH : 1];
#pragma unroll
        for (int k = 0; k < NOWN; ++k) {
            {
                float mx = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = sacc[k][kt][i];
                        sacc[k][kt][i] = v;
                        mx = fmaxf(mx, v);
                    }
                mx = wave_max_16_32(mx);
                maybe_rescale<NDT>(mx * a.c, m[k], l[k], o[k]);
                float p[4][4];
                float ls = 0.f;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) p[kt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[k][kt][i], a.c, -m[k]));
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const h2 p0 = pk_rtz(p[2 * kk][0], p[2 * kk][1]);
                    const h2 p1 = pk_rtz(p[2 * kk][2], p[2 * kk][3]);
                    const h2 p2 = pk_rtz(p[2 * kk + 1][0], p[2 * kk + 1][1]);
                    const h2 p3 = pk_rtz(p[2 * kk + 1][2], p[2 * kk + 1][3]);
                    ls = add_pair(p0, ls);
                    ls = add_pair(p1, ls);
                    ls = add_pair(p2, ls);
                    ls = add_pair(p3, ls);
                    h8 f;
                    f.s01 = p0;
                    f.s23 = p1;
                    f.s45 = p2;
                    f.s67 = p3;
                    pf[k][kk] = f;
                }
                l[k] += ls;
            }
        }
#pragma unroll
        for (int u = 0; u < NSH; ++u) {
            {
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = ssh[u][i];
                    ssh[u][i] = v;
                    mx = fmaxf(mx, v);
                }
                mx = wave_max_16_32(mx);
                maybe_rescale<NDT>(mx * a.c, m[NOWN + u], l[NOWN + u], o[NOWN + u]);
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(ssh[u][i], a.c, -m[NOWN + u]));
                const h2 p0 = pk_rtz(p[0], p[1]);
                const h2 p1 = pk_rtz(p[2], p[3]);
                float ls = add_pair(p0, 0.f);
                ls = add_pair(p1, ls);
                l[NOWN + u] += ls;
                const h2 z = {(_Float16)0.0f, (_Float16)0.0f};
                h8 f;
                if (w & 1) {  // key tile w is the upper half of k-step w/2
                    f.s01 = z; f.s23 = z; f.s45 = p0; f.s67 = p1;
                } else {
                    f.s01 = p0; f.s23 = p1; f.s45 = z; f.s67 = z;
                }
                psh[u] = f;
            }
        }

        // ---- O^T += V^T P^T; V fragments in groups of 4 with one group of
        // lookahead. Fragment idx covers k-step kk = idx / NDT, d-tile idx % NDT.
        constexpr int NG = 2 * NDT / 4;
        h8 vf[2][4];
        auto vload = [&](int g, h8(&f)[4]) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int idx = 4 * g + j, kk = idx / NDT, dt = idx % NDT;
                f[j] = *(const h8 *)(vt + (16 * dt + col) * St::VSTR + 32 * kk + 8 * grp);
            }
        };
        vload(0, vf[0]);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (g + 1 < NG) vload(g + 1, vf[(g + 1) & 1]);
            const int kk = (4 * g) / NDT;
            const bool sh_here = NSH > 0 && kk == (w >> 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int dt = (4 * g + j) % NDT;
#pragma unroll
                for (int k = 0; k < NOWN; ++k)
                    o[k][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[g & 1][j], pf[k][kk], o[k][dt], 0, 0, 0);
            }
            if (sh_here) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int dt = (4 * g + j) % NDT;
#pragma unroll
                    for (int u = 0; u < NSH; ++u)
                        o[NOWN + u][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[g & 1][j], psh[u], o[NOWN + u][dt], 0, 0, 0);
                }
            }
            TV_SCHED_FENCE();
        }
    }

    static_assert(NSH * 4 * 16 * (D + 2) * 4 <= 2 * St::ELEMS * 2, "merge scratch");
    write_partials<D, NOWN, NSH>(a, lds, 2 * St::ELEMS * 2, tid, w, col, grp, gkv, split, tm.t0, t_end, tile, o, m, l);
}

// ---------------------------------------------------------------------------
// Merge: one workgroup of 256 threads per output row (body in tv_merge.h).

template <int D>
__global__ void __launch_bounds__(256) merge_kernel(const MergeArgs a)
{
    __shared__ MergeLds<D> sm;
    merge_row<D>(a, a.p, blockIdx.x, threadIdx.x, true, sm);
}

// ---------------------------------------------------------------------------
// Host side.


template <int D, int KVT, bool MASK>
static split_fn pick_split(int nown, int nsh)
{
#define TV_CASE(O, S)              \
    if (nown == O && nsh == S) return split_kernel<D, KVT, O, S, MASK>;
    TV_CASE(0, 1) TV_CASE(0, 2) TV_CASE(1, 0) TV_CASE(1, 1) TV_CASE(1, 2) TV_CASE(2, 0) TV_CASE(2, 1)
    TV_CASE(3, 0)
#undef TV_CASE
    return nullptr;
}

template <int D>
static split_fn pick_split_f16(int nown, int nsh, bool mask)
{
    return mask ? pick_split<D, TV_KV_F16, true>(nown, nsh) : pick_split<D, TV_KV_F16, false>(nown, nsh);
}

static split_fn pick_split(int D, int kv, int nown, int nsh, bool mask)
{
    if (kv == TV_KV_Q4_0) return pick_split_q4(D, nown, nsh, mask);
    if (D == 64) return pick_split_f16<64>(nown, nsh, mask);
    if (D == 128) return pick_split_f16<128>(nown, nsh, mask);
    if (D == 256) return pick_split_f16<256>(nown, nsh, mask);
    return nullptr;
}

// The warp-specialised kernels take unmasked plans whose tile layout they
// have (head_dim 256; one or two own tiles per wave, at most two shared for
// Q4_0 and one for F16).
split_fn pick_ws(const tv_attn_desc *d, const SplitPlan &p)
{
    if (p.mask) return nullptr;
    if (d->kv_type == TV_KV_Q4_0)
        return ws_layout(d->head_dim, p.rows.nown, p.rows.nsh) ? pick_split_q4ws(d->head_dim, p.rows.nown, p.rows.nsh)
                                                                : nullptr;
    return ws_layout_f16(d->head_dim, p.rows.nown, p.rows.nsh)
               ? pick_split_f16ws(d->head_dim, p.rows.nown, p.rows.nsh)
               : nullptr;
}

void fill_split_args(const tv_attn_desc *d, const tv_attn_ptrs *p, const SplitPlan &plan, void *ws, SplitArgs *out)
{
    const int n = d->n_nodes, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim;
    const int G = Hq / Hkv;
    const int NR = n * Hq;
    SplitArgs &a = *out;
    a.k_cache = (const uint8_t *)p->k_cache;
    a.v_cache = (const uint8_t *)p->v_cache;
    a.tok_stride = d->kv_token_stride;
    a.head_stride = d->kv_head_stride;
    a.q = (const _Float16 *)p->q;
    a.ws_o = (_Float16 *)ws;
    a.ws_m = (float *)(a.ws_o + (size_t)plan.S * NR * D);
    a.s0 = plan.s0 + plan.head;
    a.n_whole = plan.n_whole;
    a.last_start = plan.s0 + plan.R - kChunk;
    a.c_per = plan.S > 0 ? plan.n_chunks / plan.S : 0;
    a.c_rem = plan.S > 0 ? (int32_t)(plan.n_chunks % plan.S) : 0;
    a.NR = NR;
    a.H_q = Hq;
    a.G = G;
    a.M = G * n;
    a.S = plan.S;
    a.c = d->scale * 1.4426950408889634f;
    a.has_skip = 0;
    for (int i = 0; i < TV_MAX_NODES; ++i) a.skip[i] = 0;
    if (plan.mask && d->window_mode == 1 && d->window > 0) {
        // per-position window: the node at depth k sees positions from
        // n_ctx + k - W on
        for (int i = 0; i < n; ++i) {
            int depth = 0;
            for (int u = d->parent[i]; u >= 0; u = d->parent[u]) ++depth;
            int64_t skip = d->n_ctx + depth - d->window - plan.s0;
            skip = skip < 0 ? 0 : (skip > plan.R ? plan.R : skip);
            a.skip[i] = (int32_t)skip;
            a.has_skip |= skip > 0;
        }
    }
}

void fill_merge_args(const tv_attn_desc *d, const tv_attn_ptrs *p, const SplitPlan &plan, void *ws, MergeArgs *out)
{
    const int n = d->n_nodes, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim;
    const int NR = n * Hq;
    MergeArgs &mg = *out;
    mg.p.q = (const _Float16 *)p->q;
    mg.p.k_tree = (const _Float16 *)p->k_tree;
    mg.p.v_tree = (const _Float16 *)p->v_tree;
    mg.p.ws_o = (const _Float16 *)ws;
    mg.p.ws_m = (const float *)((const _Float16 *)ws + (size_t)plan.S * NR * D);
    mg.p.out = p->out;
    mg.p.k_cache = (const uint8_t *)p->k_cache;
    mg.p.v_cache = (const uint8_t *)p->v_cache;
    mg.NR = NR;
    mg.H_q = Hq;
    mg.H_kv = Hkv;
    mg.G = Hq / Hkv;
    mg.S = plan.S;
    mg.c = d->scale * 1.4426950408889634f;
    mg.tok_stride = d->kv_token_stride;
    mg.head_stride = d->kv_head_stride;
    // window rows left to the merge kernel: per-node head rows, then the
    // tail (none when the masked split kernel took every row)
    mg.head_begin = plan.s0;
    mg.n_head = (int32_t)plan.head;
    mg.tail_begin = plan.s0 + plan.R - plan.tail;
    mg.n_tail = (int32_t)plan.tail;
    mg.kv_type = d->kv_type;
    for (int i = 0; i < TV_MAX_NODES; ++i) {
        mg.anc[i] = 0;
        mg.head_skip[i] = 0;
    }
    for (int i = 0; i < n; ++i) {
        uint64_t mk = 0;
        int depth = -1;
        for (int u = i; u >= 0; u = d->parent[u]) {
            mk |= 1ull << u;
            ++depth;
        }
        if (d->window_mode == 1 && d->window > 0) {
            // per-position window: the node at depth k sees positions from
            // n_ctx + k - W on, in the cache and along its path
            const int64_t start = d->n_ctx + depth - d->window;
            int64_t skip = start - plan.s0;
            skip = skip < 0 ? 0 : (skip > plan.head ? plan.head : skip);
            mg.head_skip[i] = (int32_t)skip;
            const int64_t first = (int64_t)depth - d->window;  // shallowest ancestor depth kept
            if (first > 0) {
                int du = depth;
                for (int u = i; u >= 0; u = d->parent[u], --du)
                    if (du < first) mk &= ~(1ull << u);
            }
        }
        mg.anc[i] = mk;
    }
}

// The split kernel of one layer (no launch when the plan has no split).
int launch_split(const tv_attn_desc *d, const tv_attn_ptrs *p, const SplitPlan &plan, void *ws, hipStream_t stream)
{
    const int D = d->head_dim;
    if (plan.S > 0) {
        SplitArgs a;
        fill_split_args(d, p, plan, ws, &a);
        split_fn fn = pick_ws(d, plan);
        const int threads = fn ? kWsThreads : 256;
        if (!fn) fn = pick_split(D, d->kv_type, plan.rows.nown, plan.rows.nsh, plan.mask != 0);
        if (!fn) return TV_E_SHAPE;
        dim3 grid(plan.S, d->n_kv_heads, plan.rows.groups);
        void *args[] = {(void *)&a};
        if (hipLaunchKernel((const void *)fn, grid, dim3(threads), args, 0, stream) != hipSuccess) return TV_E_HIP;
    }
    return TV_OK;
}

int launch_attn(const tv_attn_desc *d, const tv_attn_ptrs *p, const SplitPlan &plan, void *ws,
                hipStream_t stream)
{
    const int D = d->head_dim;
    const int rc = launch_split(d, p, plan, ws, stream);
    if (rc) return rc;
    MergeArgs mg;
    fill_merge_args(d, p, plan, ws, &mg);
    const void *mfn = D == 64 ? (const void *)merge_kernel<64>
                    : D == 128 ? (const void *)merge_kernel<128> : (const void *)merge_kernel<256>;
    void *margs[] = {(void *)&mg};
    // the launch's own status (hipGetLastError would also report, and
    // clear, an earlier unrelated error)
    if (hipLaunchKernel(mfn, dim3(mg.NR), dim3(256), margs, 0, stream) != hipSuccess) return TV_E_HIP;
    return TV_OK;
}

}  // namespace tv
