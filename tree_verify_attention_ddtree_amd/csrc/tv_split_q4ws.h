// Warp-specialised split workgroup for Q4_0 and F16 caches with head_dim 256
// (gfx950), internal header of libtv.so: the body shared by
// split_q4ws_kernel, split_f16ws_kernel and the work-queue step kernel. The
// notes below describe the Q4_0 form; the F16 form differs only in what the
// load waves do to a chunk (F16WsLoader: no decoding).
//
// Method: every node of a DDTree draft tree attends to the committed Q4_0 KV
// cache in one verify pass ("Luce DFlash: 単一RTX 3090で最大2倍のスループット
// を目指すQwen3.6-27B", feature list: DDTree tree verify, Q4_0 KV up to about
// 128K context; "We got 207 tok/s with Qwen3.5-27B on an RTX 3090", "What we
// built vs what we didn't"). This kernel computes, for one key-range split
// of one KV head, the partial softmax state of every packed query row over
// the cache rows of that range; the merge kernel adds the tree ancestors and
// combines the splits.
//
// Same decomposition as split_q4_kernel (the packed GQA-group x tree-node
// query rows of a KV head cut into 16-row tiles; 64-key chunks, two LDS
// stages; S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_f16 with fp32
// accumulation; online softmax in the exp2 domain with a lazy rescale), but a
// workgroup has eight wave64s in two roles, and waves w and w + 4 of a
// workgroup run on the same SIMD:
//
//   math wave q (0..3)   owns query tiles t0 + q and t0 + 4 + q (NOWN of them):
//                        Q fragments and O accumulators stay in its
//                        registers; per chunk it runs the scores, the
//                        softmax and the PV of those tiles and nothing else;
//   load wave q (4..7)   moves the raw Q4_0 bytes of chunk c + 3 from HBM
//                        into registers and dequantises chunk c + 1 into
//                        the other LDS stage: keys 16q .. 16q + 15 of K over
//                        all of D (K fragments 8q .. 8q + 7), and D-quarter
//                        q of V over all 64 keys (V^T fragments 8q .. 8q +
//                        7). It also runs the NSH
//                        shared tiles: their scores over key tile q of each
//                        chunk and their PV over D-quarter q.
//
// Within one wave, an MFMA and the vector instructions of the dequantisation
// and softmax mostly take turns. With the MFMAs in one wave and the
// dequantisation in the other, the SIMD issues the load wave's vector
// instructions while the math wave's MFMAs execute.
//
// One barrier per chunk. Iteration i (chunk c, stage st = i & 1):
//   math q: S^T(c) from stage st (two halves of 32 keys, each followed by its
//           softmax), then PV(c) from stage st;
//   load q: shared tiles: the exchange of chunk c - 1 (rescale when a wave
//           flagged one) and its PV from stage st ^ 1, V^T quarter q; scores
//           of chunk c over key tile q from stage st, P quarter to the
//           exchange buffer of parity st;
//           dequantise chunk c + 1 into stage st ^ 1 (K and V^T fragments
//           8q .. 8q + 7); request the raw bytes of chunk c + 3.
// Every LDS region a load wave writes in iteration i (stage st ^ 1: K and
// V^T fragments 8q .. 8q + 7) was last read by the math waves in iteration i - 1
// (before the barrier) and by that load wave itself earlier in iteration i;
// the math waves read it again only after the next barrier. The shared
// tiles' exchange buffers alternate with the parity, as the stages do.

#pragma once

#include <type_traits>

#include "tv_q4_common.h"

namespace tv {

template <int V>
using ic = std::integral_constant<int, V>;

// One LDS stage of a dequantised 64-key chunk (head_dim 256), in MFMA
// fragment order, so that every fragment read of a wave is one contiguous
// 1 KB (K) or four contiguous 256-byte rows (V^T), and the load waves'
// stores meet no bank conflict:
//   K: 32 fragments of 512 halves, fragment 8 t + b = keys 16t .. 16t + 15
//      and block b (values 32b .. 32b + 31); slot c + 16 g (8 halves) holds
//      key 16t + c, values 32b + 8g .. + 7 (the A operand of S^T = K Q^T);
//   V^T: 32 fragments of VFRAG halves, fragment 2j + kk = values 16j .. 16j
//      + 15 and k-step kk (keys 32kk .. 32kk + 31); row g (VROW halves: 16
//      slots and 16 bytes of padding) slot c holds value 16j + c of keys
//      32kk + 4g + (0..3) and 32kk + 16 + 4g + (0..3) (the A operand of
//      O^T += V^T P^T, in the key order of the P^T fragments). The padding
//      puts the 32 eight-byte pieces of a load wave's store (one value, 4
//      keys each) in distinct banks.
struct FmStage {
    static constexpr int KFRAG = 512;
    static constexpr int KELEMS = 32 * KFRAG;
    static constexpr int VROW = 136;
    static constexpr int VFRAG = 4 * VROW;
    static constexpr int VELEMS = 32 * VFRAG;
    static constexpr int ELEMS = KELEMS + VELEMS;
};

// Loads and stage stores of the load waves for an F16 cache (head_dim 256):
// no decoding, so a chunk moves from HBM into the fragment-order stage above
// as it is, K by plain 16-byte stores and V through an 8 x 8 transposition
// in registers. Lane mapping of load wave q:
//   K: lane l holds key 16q + (l & 15), values 8 (l >> 4) .. + 7 of every
//      block b (one 16-byte load per block, 64-byte spans of a row across
//      the lanes l, l + 16, l + 32, l + 48) and stores the piece of block b
//      at slot l of fragment 8q + b: each store instruction writes one whole
//      1 KB fragment;
//   V: lane l takes k-step kk = (l >> 2) & 1, row g = l & 3 and the
//      8 values d0 = 64q + 8 (l >> 3) .. + 7, loads them for the eight keys
//      of that slot (32kk + 4g + 0..3, 32kk + 16 + 4g + 0..3: one 16-byte
//      load per key), transposes them with byte permutes into the eight
//      slots (d0 & 15) + 0..7 of row g of fragment 2 (d0 >> 4) + kk. Eight
//      lanes that store together (one d0, all kk and g) hit 128 distinct
//      bytes of the banks (rows 272 bytes and fragments 1088 bytes apart).
struct F16WsLoader {
    const uint8_t *kbase;  // K cache of this KV head
    const uint8_t *vbase;
    int64_t tok_stride;
    u32 chunk_bytes;  // 64 rows
    u32 koff;         // K: byte offset of this lane's first piece inside a chunk
    u32 voff;         // V: byte offset of this lane's first key and values
    int lane;
    int vdst;         // V: stage offset (halves) of this lane's first slot
    u4v rk[8];        // K pieces, block b
    u4v rv[8];        // V rows of the slot's eight keys, in the P^T key order

    __device__ __forceinline__ void init_ws(const SplitArgs &a, const SplitPtrs &p, int gkv, int q, int ln)
    {
        kbase = p.k_cache + (int64_t)gkv * a.head_stride;
        vbase = p.v_cache + (int64_t)gkv * a.head_stride;
        tok_stride = a.tok_stride;
        chunk_bytes = (u32)(kChunk * a.tok_stride);
        lane = ln;
        koff = (u32)((16 * q + (ln & 15)) * tok_stride) + 16u * (u32)(ln >> 4);
        const int kk = (ln >> 2) & 1, g = ln & 3, d0 = 64 * q + 8 * (ln >> 3);
        voff = (u32)((32 * kk + 4 * g) * tok_stride) + 2u * (u32)d0;
        vdst = FmStage::KELEMS + (2 * (d0 >> 4) + kk) * FmStage::VFRAG + g * FmStage::VROW + 8 * (d0 & 15);
    }

    // A chunk past the split's end (valid false) gets an empty descriptor:
    // its loads return zeros without touching memory (as Q4Loader's).
    __device__ __forceinline__ void load_k_ws(int64_t chunk_row, bool valid)
    {
        const __amdgpu_buffer_rsrc_t r = chunk_rsrc(kbase + chunk_row * tok_stride, valid ? chunk_bytes : 0u);
#pragma unroll
        for (int b = 0; b < 8; ++b) rk[b] = __builtin_amdgcn_raw_buffer_load_b128(r, koff, 64 * b, 0);
    }

    __device__ __forceinline__ void load_v(int64_t chunk_row, bool valid)
    {
        const __amdgpu_buffer_rsrc_t r = chunk_rsrc(vbase + chunk_row * tok_stride, valid ? chunk_bytes : 0u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rv[i] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, (int)(i * tok_stride), 0);
            rv[4 + i] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, (int)((16 + i) * tok_stride), 0);
        }
    }

    // the chunk into stage `stg` (K fragments 8q .. 8q + 7, V^T D-quarter q),
    // K and V halves apart
    __device__ __forceinline__ void stage(_Float16 *stg, int q) const
    {
        stage_k(stg, q);
        stage_v(stg);
    }

    __device__ __forceinline__ void stage_k(_Float16 *stg, int q) const
    {
#pragma unroll
        for (int b = 0; b < 8; ++b) *(u4v *)(stg + (8 * q + b) * FmStage::KFRAG + 8 * lane) = rk[b];
    }

    __device__ __forceinline__ void stage_v(_Float16 *stg) const
    {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // value d0 + e of the eight keys: half e & 1 of dword e >> 1
            const u32 sel = (e & 1) ? 0x07060302u : 0x05040100u;
            u4v w;
            w.x = __builtin_amdgcn_perm(rv[1][e >> 1], rv[0][e >> 1], sel);
            w.y = __builtin_amdgcn_perm(rv[3][e >> 1], rv[2][e >> 1], sel);
            w.z = __builtin_amdgcn_perm(rv[5][e >> 1], rv[4][e >> 1], sel);
            w.w = __builtin_amdgcn_perm(rv[7][e >> 1], rv[6][e >> 1], sel);
            *(u4v *)(stg + vdst + 8 * e) = w;
        }
    }
};

// LDS of a split workgroup (module-scope arrays; each kernel that uses them
// gets its own): the two K / V^T stages (the query rows are staged there
// first and the normalised output rows gathered there last) and the shared
// tiles' exchange, by chunk parity: P^T fragments ([k-step][lane], 8 halves)
// of up to two shared tiles, the maximum each load wave's key tile was taken
// against, the rescale flags.
constexpr int kWsLdsElems = 2 * FmStage::ELEMS;
static __shared__ __attribute__((aligned(16))) _Float16 ws_lds[kWsLdsElems];
static __shared__ __attribute__((aligned(16))) _Float16 ws_psh[2][2][2 * 64 * 8];
static __shared__ float ws_shmax[2][2][4][16];
static __shared__ __attribute__((aligned(16))) int ws_shflag[2][4];

// One split (key range `split` of KV head gkv, row group rg of RG) by a
// workgroup of kWsThreads threads, in the arrays above, over the tensors `p`;
// the partial state is stored with cache policy CPOL (the buffer stores' aux
// bits: kCpolSc1 makes them coherent across the device's L2 caches). With `ticket` set, thread 0 also takes the
// next ticket of a work queue into `next`. KVT is the cache type: the load
// waves dequantise a Q4_0 chunk or move an F16 chunk into the stage; the
// math waves and the shared tiles see the same stage either way.
template <int NOWN, int NSH, int CPOL = 0, int KVT = TV_KV_Q4_0>
__device__ __forceinline__ void ws_split(const SplitArgs &a, const SplitPtrs &p, int split, int gkv, int rg, int RG,
                                         uint32_t *ticket, uint32_t &next)
{
    constexpr int D = 256;
    using St = FmStage;
    // loads and decoding (Q4_0: the stage stores are this function's)
    using L = std::conditional_t<KVT == TV_KV_Q4_0, Q4Loader<D, true>, F16WsLoader>;
    using QS = QStage<D, KVT, NOWN, NSH, kWsThreads>;
    constexpr int NB = D / 32;     // 32-value blocks per row
    constexpr int NDT = D / 16;    // D tiles
    constexpr int NDQ = NDT / 4;   // D tiles of a quarter
    constexpr int NSX = NSH > 0 ? NSH : 1;
    // the planner gives a wave at most three tile slots (own + shared)
    static_assert(NOWN >= 1 && NOWN <= 2 && NSH >= 0 && NSH <= 2 && NOWN + NSH <= kMaxSlots, "tile layouts of this kernel");
    static_assert(16 * QS::NT * QS::QSTR <= 2 * St::ELEMS, "staged query rows fit both stages");


    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool math = wv < 4;
    const int q = wv & 3;
    const int col = lane & 15, grp = lane >> 4;
    TileMap tm;
    tm.init(a.M, rg, RG);
    const int64_t c_begin = split_chunk_begin(a, split);
    const int nch = (int)(split_chunk_begin(a, split + 1) - c_begin);  // >= 1
    const u32 magic = 0x64006400u;
    const __amdgpu_buffer_rsrc_t rwm = raw_rsrc(p.ws_m + (int64_t)split * a.NR, (u32)a.NR * 4u);

    // query rows of the workgroup's tiles, requested first (from L2); the
    // load waves request the first two chunks' cache bytes behind them
    QS qrows;
    qrows.load(a, p.q, gkv, tm.t0, tid);
    // a work queue's next ticket, requested behind the query rows (its
    // latency passes while they arrive)
    if (ticket && tid == 0) next = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    if (math) {
        // ------------------------------------------------------------ math
        qrows.write_rows(tid, ws_lds);
        __syncthreads();
        h8 qf[NOWN][NB];
#pragma unroll
        for (int k = 0; k < NOWN; ++k)
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) qf[k][bb] = QS::frag(ws_lds, 16 * (4 * k + q), col, grp, bb);
        __syncthreads();
        // Q fragments are only MFMA B operands: parked in AGPRs
#pragma unroll
        for (int k = 0; k < NOWN; ++k)
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) (void)qf[k][bb];

        f4 o[NOWN][NDT];
        float m[NOWN], l[NOWN];
        const float inv_c = 1.0f / a.c;
#pragma unroll
        for (int k = 0; k < NOWN; ++k) {
            m[k] = kNegBig;
            l[k] = 0.f;
#pragma unroll
            for (int j = 0; j < NDT; ++j) o[k][j] = (f4){0.f, 0.f, 0.f, 0.f};
        }

        // One chunk in two halves of 32 keys (k-steps kk = 0, 1 of the PV):
        // scores of key tiles 2kk and 2kk + 1, their softmax, then their PV
        // over all of D, so that only one half's P fragments are live.
        auto body = [&](auto stc, bool live) {
            constexpr int st = decltype(stc)::value;
            __syncthreads();
            if (!live) return;
            const _Float16 *ks = ws_lds + st * St::ELEMS + 8 * lane;
            const _Float16 *vt = ws_lds + st * St::ELEMS + St::KELEMS + grp * St::VROW + 8 * col;
            // K fragment ii of half kk: key tile 2kk + (ii & 1), block ii >> 1;
            // V fragment j of half kk: D tile j, k-step kk
            auto kfrag = [&](int kk, int ii) -> h8 {
                return *(const h8 *)(ks + (8 * (2 * kk + (ii & 1)) + (ii >> 1)) * St::KFRAG);
            };
            auto vfrag = [&](int kk, int j) -> h8 { return *(const h8 *)(vt + (2 * j + kk) * St::VFRAG); };
            // Each fragment read feeds NOWN MFMAs, so the four math waves
            // keep the LDS busy: reads stream through 4-entry rings, three
            // ahead of use, and run on across phases (the PV's first V
            // fragments before the softmax, the next half's first K
            // fragments during the PV's last MFMAs), so that the LDS does
            // not idle while the softmax runs.
            h8 kr[4];
            kr[0] = kfrag(0, 0);
            kr[1] = kfrag(0, 1);
            kr[2] = kfrag(0, 2);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                // S^T over key tiles 2kk and 2kk + 1
                f4 s[NOWN][2];
#pragma unroll
                for (int k = 0; k < NOWN; ++k) s[k][0] = s[k][1] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ii = 0; ii < 2 * NB; ++ii) {
                    if (ii + 3 < 2 * NB) kr[(ii + 3) % 4] = kfrag(kk, ii + 3);
#pragma unroll
                    for (int k = 0; k < NOWN; ++k)
                        s[k][ii & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kr[ii % 4], qf[k][ii >> 1], s[k][ii & 1],
                                                                             0, 0, 0);
                }
                h8 vr[4];
                vr[0] = vfrag(kk, 0);
                vr[1] = vfrag(kk, 1);
                vr[2] = vfrag(kk, 2);
                TV_SCHED_FENCE();
                // does a score of these 32 keys exceed its row's running
                // maximum by more than kTau: each lane compares the largest
                // of its 8 raw scores with the row's threshold (m + kTau) / c
                // (c > 0); only the rare rescale, one wave-uniform branch,
                // takes the row maxima across lanes
                bool need = false;
                float tl[NOWN];
#pragma unroll
                for (int k = 0; k < NOWN; ++k) {
                    const float t0 = fmaxf(fmaxf(s[k][0][0], s[k][0][1]), fmaxf(s[k][0][2], s[k][0][3]));
                    const float t1 = fmaxf(fmaxf(s[k][1][0], s[k][1][1]), fmaxf(s[k][1][2], s[k][1][3]));
                    tl[k] = fmaxf(t0, t1);
                    need = need || (tl[k] > (m[k] + kTau) * inv_c);
                }
                if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
                    for (int k = 0; k < NOWN; ++k) {
                        const float mm = fmaxf(m[k], xmax_16_32(tl[k]) * a.c);
                        const float f = __builtin_amdgcn_exp2f(m[k] - mm);
                        l[k] *= f;
                        m[k] = mm;

#pragma unroll
                        for (int j = 0; j < NDT; ++j) o[k][j] *= f;
                    }
                }
                // fp16 P^T fragment of k-step kk: elements 0..3 are keys
                // 32kk + 4grp + (0..3), elements 4..7 keys 32kk + 16 + 4grp + (0..3)
                h8 pf[NOWN];
#pragma unroll
                for (int k = 0; k < NOWN; ++k) {
                    h2 p[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const f4 &sv = s[k][t >> 1];
                        const int i0 = 2 * (t & 1);
                        p[t] = pk_rtz(__builtin_amdgcn_exp2f(__builtin_fmaf(sv[i0], a.c, -m[k])),
                                      __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i0 + 1], a.c, -m[k])));
                    }
                    l[k] = add_pair(p[3], add_pair(p[2], add_pair(p[1], add_pair(p[0], l[k]))));
                    h8 fr;
                    fr.s01 = p[0];
                    fr.s23 = p[1];
                    fr.s45 = p[2];
                    fr.s67 = p[3];
                    pf[k] = fr;
                }
                // O^T += V^T P^T over k-step kk
#pragma unroll
                for (int j = 0; j < NDT; ++j) {
                    if (j + 3 < NDT)
                        vr[(j + 3) % 4] = vfrag(kk, j + 3);
                    else if (kk == 0)
                        kr[j + 3 - NDT] = kfrag(1, j + 3 - NDT);
#pragma unroll
                    for (int k = 0; k < NOWN; ++k)
                        o[k][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vr[j % 4], pf[k], o[k][j], 0, 0, 0);
                }
                TV_SCHED_FENCE();
            }
        };
        for (int i = 0; i < nch; i += 2) {
            body(ic<0>{}, true);
            body(ic<1>{}, i + 1 < nch);
        }
        __syncthreads();  // E1: every wave is past the last chunk
        __syncthreads();  // E2: the load waves' last PV has read its stage
        // normalised fp16 rows into LDS, log2 denominators to the workspace
#pragma unroll
        for (int k = 0; k < NOWN; ++k) {
            const float lt = wave_sum_16_32(l[k]);
            const float inv = lt > 0.f ? 1.0f / lt : 0.f;
            _Float16 *orow = ws_lds + (16 * (4 * k + q) + col) * QS::QSTR + 4 * grp;
#pragma unroll
            for (int j = 0; j < NDT; ++j) *(h4 *)(orow + 16 * j) = __builtin_convertvector(o[k][j] * inv, h4);
            const int tile = tm.t0 + 4 * k + q;
            const int r = 16 * tile + col;
            const bool writer = tile < tm.t_end && r < a.M && grp == 0;
            const u32 rowi = (u32)((r / a.G) * a.H_q + gkv * a.G + r % a.G);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, partial_lse2(m[k], lt)), rwm,
                                                  writer ? rowi * 4u : kOffNone, 0, CPOL);
        }
    } else {
        // ------------------------------------------------------------ load
        L ld0, ld1;  // raw bytes of even and odd chunks (relative to c_begin)
        ld0.init_ws(a, p, gkv, q, lane);
        ld1.init_ws(a, p, gkv, q, lane);
        ld0.load_k_ws(chunk_row<false>(a, c_begin), true);
        ld0.load_v(chunk_row<false>(a, c_begin), true);
        ld1.load_k_ws(chunk_row<false>(a, c_begin + 1), 1 < nch);
        ld1.load_v(chunk_row<false>(a, c_begin + 1), 1 < nch);
        qrows.write_rows(tid, ws_lds);
        __syncthreads();
        h8 qs[NSX][NB];
#pragma unroll
        for (int u = 0; u < NSH; ++u)
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) qs[u][bb] = QS::frag(ws_lds, 16 * (4 * NOWN + u), col, grp, bb);
        __syncthreads();
        // Stage stores of this lane: K pieces j (block 2u + (j >> 2), values
        // 8 (j & 3) ..) of key 16q + (lane & 15) go to fragment 8q + 2u + (j >> 2),
        // slot (lane & 15) + 16 (j & 3); V pieces (4 keys kappa = 4 (lane & 15)
        // .. + 3: k-step kappa >> 5, row (kappa >> 2) & 3, half (kappa >> 4) & 1)
        // of value 32 vb + 8 vh + e go to fragment 2 ((32 vb + 8 vh + e) >> 4)
        // + (kappa >> 5), slot (8 vh + e) & 15.
        const int kq = lane & 15;
        const int ksto = (8 * q + 2 * (lane >> 4)) * St::KFRAG + 8 * kq;
        const int vsto = [&]() {
            if constexpr (KVT == TV_KV_Q4_0)
                return St::KELEMS + (4 * ld0.vb + (kq >> 3)) * St::VFRAG + (kq & 3) * St::VROW + 64 * ld0.vh +
                       4 * ((kq >> 2) & 1);
            else
                return 0;
        }();
        // the K and V halves of a chunk into stage `stg` (Q4_0 dequantised,
        // F16 moved)
        auto deq_k = [&](const L &ld, _Float16 *stg) {
            if constexpr (KVT == TV_KV_F16) {
                ld.stage_k(stg, q);
            } else {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    int b, g;
                    const h8 o = ld.k_values(j, magic, b, g);
                    *(h8 *)(stg + ksto + (j >> 2) * St::KFRAG + 128 * (j & 3)) = o;
                }
            }
        };
        auto deq_v = [&](const L &ld, _Float16 *stg) {
            if constexpr (KVT == TV_KV_F16) {
                ld.stage_v(stg);
            } else {
#pragma unroll
                for (int pc = 0; pc < 4; ++pc) {
                    h2 vals[2][4];
                    ld.v_values(pc, magic, vals);
                    // element e = 4 (pc >> 1) + 2 (pc & 1) + {0, 1, 16, 17}[t]
                    const int de = 4 * (pc >> 1) + 2 * (pc & 1);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        h4 w4;
                        w4.s01 = vals[0][t];
                        w4.s23 = vals[1][t];
                        *(h4 *)(stg + vsto + (t >> 1) * 2 * St::VFRAG + 8 * (de + (t & 1))) = w4;
                    }
                }
            }
        };
        // chunk c_begin into stage 0; its raw registers then take chunk c_begin + 2
        deq_k(ld0, ws_lds);
        deq_v(ld0, ws_lds);
        ld0.load_k_ws(chunk_row<false>(a, c_begin + 2), 2 < nch);
        ld0.load_v(chunk_row<false>(a, c_begin + 2), 2 < nch);

        f4 osh[NSX][NDQ];
        float msh[NSX], lsh[NSX], mown[NSX];
        const float inv_c = 1.0f / a.c;
        h2 psv[NSX][2];
#pragma unroll
        for (int u = 0; u < NSX; ++u) {
            msh[u] = kNegBig;
            lsh[u] = 0.f;
            mown[u] = kNegBig;
            psv[u][0] = psv[u][1] = (h2){(_Float16)0.f, (_Float16)0.f};
#pragma unroll
            for (int j = 0; j < NDQ; ++j) osh[u][j] = (f4){0.f, 0.f, 0.f, 0.f};
        }

        // Shared tiles, the step after the chunk whose exchange has parity
        // sp: if any load wave flagged that chunk, the running maximum moves
        // to the largest of the four maxima its quarters were taken against
        // and each quarter is scaled to it in fp16; this wave's own quarter
        // (as used) goes into its row sums; then the PV of that chunk over
        // D-quarter q from its stage.
        auto shared_pv = [&](auto spc) {
            constexpr int sp = decltype(spc)::value;
            const u4v fl = *(const u4v *)ws_shflag[sp];
            h8 pfs[NSX][2];
#pragma unroll
            for (int u = 0; u < NSH; ++u) {
                pfs[u][0] = *(const h8 *)(&ws_psh[sp][u][0] + lane * 8);
                pfs[u][1] = *(const h8 *)(&ws_psh[sp][u][0] + (64 + lane) * 8);
            }
            if (__builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w)) {
#pragma unroll
                for (int u = 0; u < NSH; ++u) {
                    const float mw[4] = {ws_shmax[sp][u][0][col], ws_shmax[sp][u][1][col], ws_shmax[sp][u][2][col],
                                         ws_shmax[sp][u][3][col]};
                    const float mm = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
                    const float g = __builtin_amdgcn_exp2f(msh[u] - mm);
                    lsh[u] *= g;
                    msh[u] = mm;
#pragma unroll
                    for (int j = 0; j < NDQ; ++j) osh[u][j] *= g;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const h2 f = {(_Float16)__builtin_amdgcn_exp2f(mw[2 * kk] - mm),
                                      (_Float16)__builtin_amdgcn_exp2f(mw[2 * kk + 1] - mm)};
                        const h2 fa = {f.x, f.x}, fb = {f.y, f.y};
                        pfs[u][kk].s01 *= fa;
                        pfs[u][kk].s23 *= fa;
                        pfs[u][kk].s45 *= fb;
                        pfs[u][kk].s67 *= fb;
                    }
                    // the same fp16 products the other waves applied to this quarter
                    const _Float16 fo = (_Float16)__builtin_amdgcn_exp2f(mown[u] - mm);
                    const h2 fo2 = {fo, fo};
                    psv[u][0] *= fo2;
                    psv[u][1] *= fo2;
                }
            }
#pragma unroll
            for (int u = 0; u < NSH; ++u) lsh[u] = add_pair(psv[u][1], add_pair(psv[u][0], lsh[u]));
            const _Float16 *vt = ws_lds + sp * St::ELEMS + St::KELEMS + grp * St::VROW + 8 * col;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int j = 0; j < NDQ; ++j) {
                    const h8 vf = *(const h8 *)(vt + (2 * (NDQ * q + j) + kk) * St::VFRAG);
#pragma unroll
                    for (int u = 0; u < NSH; ++u)
                        osh[u][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pfs[u][kk], osh[u][j], 0, 0, 0);
                }
        };

        auto body = [&](auto stc, int i) {
            constexpr int st = decltype(stc)::value;
            __syncthreads();
            {
                // the K half of stage st ^ 1 is free here (its last readers,
                // chunk c - 1's scores, are past the barrier; the shared tile
                // reads only its V half), so chunk c + 1's K moves in now and
                // chunk c + 3's K is requested before the shared tile's work
                // rather than after it
                L &ldn = st == 0 ? ld1 : ld0;
                if (i + 1 < nch) deq_k(ldn, ws_lds + (st ^ 1) * St::ELEMS);
                ldn.load_k_ws(chunk_row<false>(a, c_begin + i + 3), i + 3 < nch);
            }
            if (NSH > 0 && i < nch) {
                if (i > 0) shared_pv(ic<st ^ 1>{});
                // scores of key tile q of chunk c for the shared tiles
                const _Float16 *kwb = ws_lds + st * St::ELEMS + 8 * q * St::KFRAG + 8 * lane;
                f4 ssh[NSX];
#pragma unroll
                for (int u = 0; u < NSH; ++u) ssh[u] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) {
                    const h8 kw = *(const h8 *)(kwb + bb * St::KFRAG);
#pragma unroll
                    for (int u = 0; u < NSH; ++u)
                        ssh[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kw, qs[u][bb], ssh[u], 0, 0, 0);
                }
                // this wave's P^T quarter (k-step q / 2, elements 4 (q & 1) ..
                // + 3) against the common running maximum or, when some row
                // of the key tile exceeds it by more than kTau (the flag),
                // against the larger of the two, so that no P exceeds 2^kTau
                // (each lane compares the largest of its raw scores with
                // (m + kTau) / c; the row maxima across lanes only when flagged)
                bool need_sh = false;
                float tl[NSX], mws[NSX];
#pragma unroll
                for (int u = 0; u < NSH; ++u) {
                    tl[u] = fmaxf(fmaxf(ssh[u][0], ssh[u][1]), fmaxf(ssh[u][2], ssh[u][3]));
                    need_sh = need_sh || (tl[u] > (msh[u] + kTau) * inv_c);
                    mws[u] = msh[u];
                }
                const bool flag = __builtin_amdgcn_ballot_w64(need_sh) != 0;
                if (flag) {
#pragma unroll
                    for (int u = 0; u < NSH; ++u) mws[u] = fmaxf(msh[u], xmax_16_32(tl[u]) * a.c);
                }
#pragma unroll
                for (int u = 0; u < NSH; ++u) {
                    const float mw = mws[u];
                    mown[u] = mw;
                    psv[u][0] = pk_rtz(__builtin_amdgcn_exp2f(__builtin_fmaf(ssh[u][0], a.c, -mw)),
                                       __builtin_amdgcn_exp2f(__builtin_fmaf(ssh[u][1], a.c, -mw)));
                    psv[u][1] = pk_rtz(__builtin_amdgcn_exp2f(__builtin_fmaf(ssh[u][2], a.c, -mw)),
                                       __builtin_amdgcn_exp2f(__builtin_fmaf(ssh[u][3], a.c, -mw)));
                    h4 p4;
                    p4.s01 = psv[u][0];
                    p4.s23 = psv[u][1];
                    *(h4 *)(&ws_psh[st][u][0] + ((q >> 1) * 64 + lane) * 8 + 4 * (q & 1)) = p4;
                    if (grp == 0) ws_shmax[st][u][q][col] = mw;
                }
                if (lane == 0) ws_shflag[st][q] = flag;
            }
            // dequantise chunk c + 1 (raw bytes of parity st ^ 1) into stage
            // st ^ 1, then request chunk c + 3 into the same registers (F16:
            // the V half; its K half went at the top of the step)
            _Float16 *ks_n = ws_lds + (st ^ 1) * St::ELEMS;
            auto next = [&](L &ldn) {
                if (i + 1 < nch) deq_v(ldn, ks_n);
                ldn.load_v(chunk_row<false>(a, c_begin + i + 3), i + 3 < nch);
            };
            if constexpr (st == 0)
                next(ld1);
            else
                next(ld0);
        };
        // Both bodies run on every pass, the second past the last chunk too
        // (then it only requests nothing through an empty descriptor and
        // meets the barrier), so that every path through the loop issues
        // the same loads in the same order and each wait counts only the
        // chunk it needs: with an odd last pass skipped, the wait counts at
        // the loop header had to cover both histories and waited for every
        // load in flight.
        for (int i = 0; i < nch; i += 2) {
            body(ic<0>{}, i);
            body(ic<1>{}, i + 1);
        }
        __syncthreads();  // E1: the last chunk's exchange is complete
        // the last chunk's shared update and PV; this wave's row sums meet
        // the other load waves' in the maxima buffer of the parity the last
        // chunk did not use (all of its reads were before E1)
        float(*shl)[4][16] = ws_shmax[nch & 1];
        if constexpr (NSH > 0) {
            if ((nch - 1) & 1)
                shared_pv(ic<1>{});
            else
                shared_pv(ic<0>{});
#pragma unroll
            for (int u = 0; u < NSH; ++u) {
                const float lw = wave_sum_16_32(lsh[u]);
                if (grp == 0) shl[u][q][col] = lw;
            }
        }
        __syncthreads();  // E2
#pragma unroll
        for (int u = 0; u < NSH; ++u) {
            const float lt = ((shl[u][0][col] + shl[u][1][col]) + shl[u][2][col]) + shl[u][3][col];
            const float inv = lt > 0.f ? 1.0f / lt : 0.f;
            _Float16 *orow = ws_lds + (16 * (4 * NOWN + u) + col) * QS::QSTR + 4 * grp;
#pragma unroll
            for (int j = 0; j < NDQ; ++j)
                *(h4 *)(orow + 16 * (NDQ * q + j)) = __builtin_convertvector(osh[u][j] * inv, h4);
            const int tile = tm.t0 + 4 * NOWN + u;
            const int r = 16 * tile + col;
            const bool writer = tile < tm.t_end && r < a.M && grp == 0 && q == 0;
            const u32 rowi = (u32)((r / a.G) * a.H_q + gkv * a.G + r % a.G);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, partial_lse2(msh[u], lt)), rwm,
                                                  writer ? rowi * 4u : kOffNone, 0, CPOL);
        }
    }
    __syncthreads();  // E3: every row is in LDS
    // contiguous 16-byte stores of the normalised rows (a 1 KB span per wave
    // instruction) through a buffer over this split's block of the
    // workspace; rows past the group's last drop out
    {
        const __amdgpu_buffer_rsrc_t rwo = raw_rsrc(p.ws_o + (int64_t)split * a.NR * D, (u32)a.NR * (u32)(2 * D));
        const int nrows = min(16 * tm.t_end, a.M) - 16 * tm.t0;
        const int r0 = tid / QS::PR;
        RowWalk rw(a, gkv, 16 * tm.t0 + r0, QS::RS, 2 * D);
        const u32 part = 16u * (u32)(tid % QS::PR);
        const _Float16 *src = ws_lds + r0 * QS::QSTR + 8 * (tid % QS::PR);
#pragma unroll
        for (int jj = 0; jj < QS::NQ; ++jj) {
            const u4v v = *(const u4v *)(src + jj * QS::RS * QS::QSTR);
            __builtin_amdgcn_raw_buffer_store_b128(v, rwo, r0 + jj * QS::RS < nrows ? rw.off + part : kOffNone, 0,
                                                   CPOL);
            rw.next();
        }
    }
}

}  // namespace tv
