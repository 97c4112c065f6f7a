// Split kernel for Q4_0 caches, software-pipelined for gfx950.
//
// Same decomposition as the generic split kernel (one workgroup of four
// wave64s per key-range split, KV head and row group; the packed
// GQA-group x tree-node query rows cut into 16-row MFMA tiles, own and
// shared), but the dequantisation of chunk c+1 is interleaved with the MFMAs
// of chunk c so that the VALU work runs in the shadow of the matrix cores:
//
//   iteration c:  barrier (without shared tiles)
//                 S^T(c) = K Q^T MFMAs   + dequantise K(c+1) into the other
//                                          LDS stage, one code dword per block
//                 load raw K(c+2)
//                 online softmax(c); shared tiles' P quarters to LDS
//                 barrier (with shared tiles), P quarters read back
//                 O^T += V^T P^T MFMAs   + dequantise V(c+1)
//                 load raw V(c+2)
//
// Raw Q4_0 bytes travel HBM -> registers one iteration ahead. LDS stores are
// laid out so that the writes of a wave hit distinct banks: K rows are
// written one key per lane, transposed V rows four keys (8 bytes) per lane
// with the key groups fastest across lanes.
//
// Method: DDTree tree verify over a Q4_0 KV cache ("Luce DFlash: 単一RTX 3090
// で最大2倍のスループットを目指すQwen3.6-27B", feature list; "We got 207 tok/s
// with Qwen3.5-27B on an RTX 3090", "What we built vs what we didn't").

#include "tv_q4_common.h"

namespace tv {

// Split kernel. Own tiles: each wave holds NOWN query tiles for all D.
// Shared tiles (the one or two tiles left over when the tile count is not a
// multiple of four) are split two ways: wave w scores only key tile w of
// each chunk (16 of its 64 keys) and accumulates only its quarter of D.
// The fp16 P of the four key tiles meets in LDS, so each wave's PV sees all
// 64 keys. The running maximum of a shared tile is common to the waves: a
// wave whose key tile would move it by more than kTau raises a flag, and
// when any flag is up every wave takes the largest of the four maxima,
// rescales and rewrites its P before the PV. Each wave walks the D-tiles
// rotated by its index, so that its shared quarter is the first NDT/4
// positions of every k-step and every index into the register arrays stays
// a compile-time constant.
template <int D, int NOWN, int NSH, bool MASK>
__global__ void __launch_bounds__(256, 1) split_q4_kernel(const SplitArgs a)
{
    using St = Stage<D, TV_KV_Q4_0, (NSH > 0)>;
    using L = Q4Loader<D, (NSH > 0)>;
    constexpr int NB = St::NB;
    constexpr int NDT = D / 16;
    constexpr int NDQ = NDT / 4;  // D-tiles of a shared tile per wave
    constexpr int NS = NOWN + NSH;
    static_assert(NS >= 1 && NS <= kMaxSlots, "slots");
    __shared__ __attribute__((aligned(16))) _Float16 lds[2 * St::ELEMS];
    // shared tiles, by chunk parity: P^T fragments of the chunk
    // ([k-step][lane], 8 halves), the maximum each wave's key tile was taken
    // against per row, and the waves' rescale flags
    constexpr int NSX = NSH > 0 ? NSH : 1;
    __shared__ __attribute__((aligned(16))) _Float16 psh[2][NSX][2 * 64 * 8];
    __shared__ float shmax[2][NSX][4][16];
    __shared__ __attribute__((aligned(16))) int shflag[2][4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int split = blockIdx.x, gkv = blockIdx.y, rg = blockIdx.z;

    TileMap tm;
    tm.init(a.M, rg, gridDim.z);
    int tile[NS];
#pragma unroll
    for (int k = 0; k < NOWN; ++k) tile[k] = tm.t0 + 4 * k + w;
#pragma unroll
    for (int u = 0; u < NSH; ++u) tile[NOWN + u] = tm.t0 + 4 * NOWN + u;

    const int64_t c_begin = split_chunk_begin(a, split);
    const int64_t c_end = split_chunk_begin(a, split + 1);
    const u32 magic = 0x64006400u;
    const int rot = NDQ * w;  // D-tile at loop position j is (j + rot) % NDT

    // prologue: the query rows (from L2) are requested first, the first
    // chunk's cache bytes (from HBM) next, so that the two are in flight
    // together and the query rows can be staged before the cache bytes
    // arrive; then chunk c_begin is dequantised into stage 0 and the raw
    // bytes of the next are requested
    QStage<D, TV_KV_Q4_0, NOWN, NSH> qs;
    qs.load(a, gkv, tm.t0, tid);
    L ld;
    ld.init(a, gkv, tid);
    ld.load_k(chunk_row<MASK>(a, c_begin), true);
    ld.load_v(chunk_row<MASK>(a, c_begin), true);

    h8 qf[NS][NB];
    qs.store(tm.t0, tile, tid, col, grp, lds, qf);
    // Q fragments are read only as MFMA B operands, which may live in AGPRs;
    // parking them there leaves the VGPRs to the accumulators and the pipeline.
#pragma unroll
    for (int k = 0; k < NS; ++k)
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) asm volatile("" : "+a"(qf[k][bb]));

    f4 o[NOWN > 0 ? NOWN : 1][NDT];
    f4 osh[NSH > 0 ? NSH : 1][NDQ];
    float m[NS], l[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        m[k] = kNegBig;
        l[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < NOWN; ++k)
#pragma unroll
        for (int j = 0; j < NDT; ++j) o[k][j] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NSH; ++u)
#pragma unroll
        for (int j = 0; j < NDQ; ++j) osh[u][j] = (f4){0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int j = 0; j < NB; ++j) ld.k_piece(j, lds, magic);
#pragma unroll
    for (int p = 0; p < L::V_PIECES; ++p) ld.v_piece(p, lds + St::KELEMS, magic);
    if (NSH > 0 || c_begin + 1 < c_end) {
        ld.load_k(chunk_row<MASK>(a, c_begin + 1), c_begin + 1 < c_end);
        ld.load_v(chunk_row<MASK>(a, c_begin + 1), c_begin + 1 < c_end);
    }

    // One barrier per chunk. Without shared tiles it opens the chunk: stage
    // st has been written, stage st ^ 1 read, by every wave. With shared
    // tiles it is the one before the PV (below), which orders the same
    // accesses: K(c+1) is written before it and read after the next one;
    // V(c+1) is written after it, V(c-1) was read before it. The exchange
    // buffers alternate with the stages, so a wave writing chunk c+1's
    // never meets one still reading chunk c's.
    if constexpr (NSH > 0) __syncthreads();
    for (int64_t c = c_begin; c < c_end; ++c) {
        const int st = (int)((c - c_begin) & 1);
        const _Float16 *ks = lds + st * St::ELEMS;
        const _Float16 *vt = ks + St::KELEMS;
        _Float16 *ks_n = lds + (st ^ 1) * St::ELEMS;
        _Float16 *vt_n = ks_n + St::KELEMS;
        if constexpr (NSH == 0) __syncthreads();

        // ---- S^T = K Q^T for the own slots over the 4 key tiles of the
        // chunk and for the shared slots over key tile w, with the K
        // dequantisation of chunk c+1 in between. K fragments stream through
        // a 4-entry ring, three ahead of use (an LDS read under load takes
        // longer than the 2 x 3 MFMAs a two-ahead ring covers); the shared
        // slots' fragments of key tile w through a 2-entry ring, one block
        // ahead.
        constexpr int TOT = NB * 4;
        f4 sacc[NOWN > 0 ? NOWN : 1][4];
        f4 ssh[NSX];
#pragma unroll
        for (int k = 0; k < NOWN; ++k)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) sacc[k][kt] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NSH; ++u) ssh[u] = (f4){0.f, 0.f, 0.f, 0.f};
        auto kfrag = [&](int i) -> h8 {
            const int bb = i / 4, kt = i % 4;
            return *(const h8 *)(ks + (16 * kt + col) * St::KSTR + 32 * bb + 8 * grp);
        };
        const _Float16 *kwb = ks + (16 * w + col) * St::KSTR + 8 * grp;
        h8 kr[4], kw[2];
        kr[0] = kfrag(0);
        kr[1] = kfrag(1);
        kr[2] = kfrag(2);
        if constexpr (NSH > 0) kw[0] = *(const h8 *)kwb;
#pragma unroll
        for (int i = 0; i < TOT; ++i) {
            if (i + 3 < TOT) kr[(i + 3) % 4] = kfrag(i + 3);
            const int bb = i / 4, kt = i % 4;
            if constexpr (NSH > 0)
                if (kt == 0 && bb + 1 < NB) kw[(bb + 1) & 1] = *(const h8 *)(kwb + 32 * (bb + 1));
#pragma unroll
            for (int k = 0; k < NOWN; ++k)
                sacc[k][kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kr[i % 4], qf[k][bb], sacc[k][kt], 0, 0, 0);
            if (kt == 3) {
#pragma unroll
                for (int u = 0; u < NSH; ++u)
                    ssh[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kw[bb & 1], qf[NOWN + u][bb], ssh[u], 0, 0, 0);
                ld.k_piece(bb, ks_n, magic);
                TV_SCHED_FENCE();
            }
        }
        if (NSH > 0 || c + 2 < c_end) ld.load_k(chunk_row<MASK>(a, c + 2), c + 2 < c_end);
        if constexpr (MASK) {
            if (chunk_masked(a, c)) {
#pragma unroll
                for (int k = 0; k < NS; ++k) {
                    const int thr = masked_keys(a, c, row_skip(a, tile[k], tm.t_end, col));
                    if (k < NOWN) {
#pragma unroll
                        for (int kt = 0; kt < 4; ++kt) mask_tile(sacc[k < NOWN ? k : 0][kt], kt, grp, thr);
                    } else {
                        mask_tile(ssh[k >= NOWN ? k - NOWN : 0], w, grp, thr);
                    }
                }
            }
        }

        // ---- shared slots: this wave's P^T quarter goes into the fragments
        // of k-step w / 2 (elements 4 (w & 1) .. + 3), with the maximum it was
        // taken against and the wave's rescale flag. That maximum is the
        // common running maximum, or, when some row of the key tile exceeds
        // it by more than kTau (the flag), the larger of the two per row, so
        // that no P exceeds 2^kTau. The flags are read after the barrier below.
        float mnew_sh[NSX], mown[NSX];
        h2 psv[NSX][2];
        if constexpr (NSH > 0) {
            bool need_sh = false;
#pragma unroll
            for (int u = 0; u < NSH; ++u) {
                const float t = fmaxf(fmaxf(ssh[u][0], ssh[u][1]), fmaxf(ssh[u][2], ssh[u][3]));
                const float ml = xmax_16_32(t) * a.c;
                need_sh = need_sh || (ml > m[NOWN + u] + kTau);
                mnew_sh[u] = ml;
            }
            const bool flag = __builtin_amdgcn_ballot_w64(need_sh) != 0;
#pragma unroll
            for (int u = 0; u < NSH; ++u) {
                const float mw = flag ? fmaxf(m[NOWN + u], mnew_sh[u]) : m[NOWN + u];
                mown[u] = mw;
                psv[u][0] = pk_rtz(__builtin_amdgcn_exp2f(__builtin_fmaf(ssh[u][0], a.c, -mw)),
                                   __builtin_amdgcn_exp2f(__builtin_fmaf(ssh[u][1], a.c, -mw)));
                psv[u][1] = pk_rtz(__builtin_amdgcn_exp2f(__builtin_fmaf(ssh[u][2], a.c, -mw)),
                                   __builtin_amdgcn_exp2f(__builtin_fmaf(ssh[u][3], a.c, -mw)));
                h4 p4;
                p4.s01 = psv[u][0];
                p4.s23 = psv[u][1];
                *(h4 *)(&psh[st][u][0] + ((w >> 1) * 64 + lane) * 8 + 4 * (w & 1)) = p4;
                if (grp == 0) shmax[st][u][w][col] = mw;
            }
            if (lane == 0) shflag[st][w] = flag;
        }

        // ---- running maxima of the own slots (trees: the VALU's
        // dependent-issue latency is long), one wave-uniform branch for the
        // rare rescale
        float mnew[NOWN > 0 ? NOWN : 1];
        bool need = false;
#pragma unroll
        for (int k = 0; k < NOWN; ++k) {
            float t[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                t[kt] = fmaxf(fmaxf(sacc[k][kt][0], sacc[k][kt][1]), fmaxf(sacc[k][kt][2], sacc[k][kt][3]));
            mnew[k] = xmax_16_32(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]))) * a.c;
            need = need || (mnew[k] > m[k] + kTau);
        }
        if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
            for (int k = 0; k < NOWN; ++k) {
                const float mm = fmaxf(m[k], mnew[k]);
                const float f = __builtin_amdgcn_exp2f(m[k] - mm);
                l[k] *= f;
                m[k] = mm;
#pragma unroll
                for (int j = 0; j < NDT; ++j) o[k][j] *= f;
            }
        }

        // ---- fp16 P^T fragments; k-step kk covers key tiles 2kk, 2kk+1
        h8 pf[NOWN > 0 ? NOWN : 1][2];
        auto make_p = [&](int k, int kk) {
            h2 p[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int kt = 2 * kk + (t >> 1), i0 = 2 * (t & 1);
                p[t] = pk_rtz(__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[k][kt][i0], a.c, -m[k])),
                              __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[k][kt][i0 + 1], a.c, -m[k])));
            }
            l[k] += add_pair(p[0], add_pair(p[1], 0.f)) + add_pair(p[2], add_pair(p[3], 0.f));
            h8 fr;
            fr.s01 = p[0];
            fr.s23 = p[1];
            fr.s45 = p[2];
            fr.s67 = p[3];
            pf[k][kk] = fr;
        };
#pragma unroll
        for (int k = 0; k < NOWN; ++k) make_p(k, 0);

        // ---- shared slots: once every wave's P quarter is in LDS, all waves
        // read the same full P^T fragments. If any wave raised its flag, the
        // new running maximum is the largest of the four maxima the quarters
        // were taken against, and each quarter is scaled to it in fp16 (a
        // factor of at most 1, rounded to nearest, as the products are); all
        // waves see the same flags and values, so
        // they keep identical states. Each wave sums its own key tile's P as
        // used into its row sums; the four waves' sums are added at the end.
        h8 pfs[NSX][2];
        if constexpr (NSH > 0) {
            __syncthreads();
            const u4v fl = *(const u4v *)shflag[st];
#pragma unroll
            for (int u = 0; u < NSH; ++u) {
                pfs[u][0] = *(const h8 *)(&psh[st][u][0] + lane * 8);
                pfs[u][1] = *(const h8 *)(&psh[st][u][0] + (64 + lane) * 8);
            }
            if (__builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w)) {
#pragma unroll
                for (int u = 0; u < NSH; ++u) {
                    const float m0 = m[NOWN + u];
                    const float mw[4] = {shmax[st][u][0][col], shmax[st][u][1][col], shmax[st][u][2][col],
                                         shmax[st][u][3][col]};
                    const float mm = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
                    const float g = __builtin_amdgcn_exp2f(m0 - mm);
                    l[NOWN + u] *= g;
                    m[NOWN + u] = mm;
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
                    // the same fp16 products as this wave's quarter above
                    const _Float16 fo = (_Float16)__builtin_amdgcn_exp2f(mown[u] - mm);
                    const h2 fo2 = {fo, fo};
                    psv[u][0] *= fo2;
                    psv[u][1] *= fo2;
                }
            }
#pragma unroll
            for (int u = 0; u < NSH; ++u) l[NOWN + u] += add_pair(psv[u][0], add_pair(psv[u][1], 0.f));
        }

        // ---- O^T += V^T P^T. k-step 0 runs while the P of k-step 1 is
        // computed; k-step 1 runs while V(c+1) is dequantised.
        constexpr int TV = 2 * NDT;
        // position j reads D-tile (j + rot) % NDT: from vA below the wrap,
        // from vB = vA - NDT tiles after it, both at the immediate offset of
        // position j
        const _Float16 *vA = vt + (16 * rot + col) * St::VSTR + 8 * grp;
        const _Float16 *vB = vA - NDT * 16 * St::VSTR;
        auto vfrag = [&](int i) -> h8 {
            const int kk = i / NDT, j = i % NDT;
            const _Float16 *base = j < NDT - rot ? vA : vB;
            return *(const h8 *)(base + j * 16 * St::VSTR + 32 * kk);
        };
        constexpr int VP = L::V_PIECES;
        constexpr int VSTEP = NDT / VP;
        h8 vr[4];
        vr[0] = vfrag(0);
        vr[1] = vfrag(1);
        vr[2] = vfrag(2);
#pragma unroll
        for (int i = 0; i < TV; ++i) {
            if (i + 3 < TV) vr[(i + 3) % 4] = vfrag(i + 3);
            const int kk = i / NDT, j = i % NDT;
#pragma unroll
            for (int k = 0; k < NOWN; ++k)
                o[k][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vr[i % 4], pf[k][kk], o[k][j], 0, 0, 0);
            if (j < NDQ) {
#pragma unroll
                for (int u = 0; u < NSH; ++u)
                    osh[u][j < NDQ ? j : 0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vr[i % 4], pfs[u][kk],
                                                                                   osh[u][j < NDQ ? j : 0], 0, 0, 0);
            }
            if (i == 1) {
#pragma unroll
                for (int k = 0; k < NOWN; ++k) make_p(k, 1);
            }
            if (kk == 1 && (j + 1) % VSTEP == 0) {
                ld.v_piece((j + 1) / VSTEP - 1, vt_n, magic);
                TV_SCHED_FENCE();
            }
        }
        if (NSH > 0 || c + 2 < c_end) ld.load_v(chunk_row<MASK>(a, c + 2), c + 2 < c_end);
    }

    // ---- partial states: own tiles by every wave; shared tiles by every
    // wave for its quarter of D (their row maxima and sums are identical in
    // all waves and written by wave 0). The normalised fp16 rows are gathered
    // in LDS and written as contiguous 16-byte pieces, a 1 KB span per wave
    // instruction: stored straight from the fragments, each instruction
    // would scatter 8-byte pieces over 16 rows, which costs several times
    // longer per byte. The stores go through buffers over this split's
    // blocks of the workspace; a row outside this workgroup's rows gets an
    // out-of-range offset, which drops the store.
    using QS = QStage<D, TV_KV_Q4_0, NOWN, NSH>;
    const __amdgpu_buffer_rsrc_t rwo = raw_rsrc(a.ws_o + (int64_t)split * a.NR * D, (u32)a.NR * (u32)(2 * D));
    const __amdgpu_buffer_rsrc_t rwm = raw_rsrc(a.ws_m + (int64_t)split * a.NR, (u32)a.NR * 4u);
    // the shared tiles' row sums meet in the maxima buffer of the parity
    // the last chunk did not use: every wave read it before the last
    // chunk's barrier
    float(*shl)[4][16] = shmax[((int)(c_end - c_begin) & 1)];
#pragma unroll
    for (int u = 0; u < NSH; ++u) {
        const float lw = wave_sum_16_32(l[NOWN + u]);
        if (grp == 0) shl[u][w][col] = lw;
    }
    __syncthreads();  // every wave is done with the last stage
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        float lt;
        if (k < NOWN) {
            lt = wave_sum_16_32(l[k]);
        } else {
            const int u = k >= NOWN ? k - NOWN : 0;
            lt = ((shl[u][0][col] + shl[u][1][col]) + shl[u][2][col]) + shl[u][3][col];
        }
        const int rl = 16 * (tile[k] - tm.t0) + col;
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        _Float16 *orow = lds + rl * QS::QSTR + 4 * grp;
        if (k < NOWN) {
#pragma unroll
            for (int j = 0; j < NDT; ++j)
                *(h4 *)(orow + 16 * ((j + rot) & (NDT - 1))) =
                    __builtin_convertvector(o[k < NOWN ? k : 0][j] * inv, h4);
        } else {
#pragma unroll
            for (int j = 0; j < NDQ; ++j)
                *(h4 *)(orow + 16 * (j + rot)) = __builtin_convertvector(osh[k >= NOWN ? k - NOWN : 0][j] * inv, h4);
        }
        const int r = 16 * tile[k] + col;
        const bool mwriter = tile[k] < tm.t_end && r < a.M && grp == 0 && (k < NOWN || w == 0);
        const u32 rowi = (u32)((r / a.G) * a.H_q + gkv * a.G + r % a.G);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, partial_lse2(m[k], lt)), rwm,
                                              mwriter ? rowi * 4u : kOffNone, 0, kCpolSc1);
    }
    __syncthreads();
    {
        const int nrows = min(16 * tm.t_end, a.M) - 16 * tm.t0;
        const int r0 = tid / QS::PR;
        RowWalk rw(a, gkv, 16 * tm.t0 + r0, QS::RS, 2 * D);
        const u32 part = 16u * (u32)(tid % QS::PR);
        const _Float16 *src = lds + r0 * QS::QSTR + 8 * (tid % QS::PR);
#pragma unroll
        for (int jj = 0; jj < QS::NQ; ++jj) {
            const u4v v = *(const u4v *)(src + jj * QS::RS * QS::QSTR);
            __builtin_amdgcn_raw_buffer_store_b128(v, rwo, r0 + jj * QS::RS < nrows ? rw.off + part : kOffNone, 0, kCpolSc1);
            rw.next();
        }
    }
}

template <int D, bool MASK>
static split_fn pick_q4(int nown, int nsh)
{
#define TV_CASE(O, S) \
    if (nown == O && nsh == S) return split_q4_kernel<D, O, S, MASK>;
    TV_CASE(0, 1) TV_CASE(0, 2) TV_CASE(0, 3) TV_CASE(1, 0) TV_CASE(1, 1) TV_CASE(1, 2) TV_CASE(2, 0)
    TV_CASE(2, 1) TV_CASE(3, 0)
#undef TV_CASE
    return nullptr;
}

split_fn pick_split_q4(int D, int nown, int nsh, bool mask)
{
    if (D == 64) return mask ? pick_q4<64, true>(nown, nsh) : pick_q4<64, false>(nown, nsh);
    if (D == 128) return mask ? pick_q4<128, true>(nown, nsh) : pick_q4<128, false>(nown, nsh);
    if (D == 256) return mask ? pick_q4<256, true>(nown, nsh) : pick_q4<256, false>(nown, nsh);
    return nullptr;
}

}  // namespace tv
