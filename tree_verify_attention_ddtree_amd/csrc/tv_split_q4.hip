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

#include "tv_split_common.h"

namespace tv {

// Per-thread share of one 64-key chunk.
//   K: key (tid & 63), half-blocks [u*HB, (u+1)*HB) with u = tid >> 6; one
//      half-block is 16 values (8 code bytes) of one 32-value block.
//   V: NKV consecutive keys starting at NKV * (tid % KG), one half-block
//      (block b, half h) of each.
template <int D>
struct Q4Share {
    static constexpr int NB = D / 32;
    static constexpr int HB = NB / 2;    // K half-blocks per thread
    static constexpr int NKV = NB / 2;   // V keys per thread
    static constexpr int KG = 64 / NKV;  // V key groups
    static constexpr int RAWK = 4 * HB;  // per half-block: scale dword + 3-dword code window
    static constexpr int RAWV = 4 * NKV;
};

__device__ __forceinline__ u32 and_or(u32 x, u32 m, u32 o)
{
    u32 r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
    return r;
}

// code dword (8 codes) -> the exact values code - 8 in four fp16 pairs, same
// element order as q4_unpack.
__device__ __forceinline__ void q4_unpack_ao(u32 x, u32 magic, h2 v[4])
{
    const u32 y = x >> 8;
    const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    v[0] = as_h2(and_or(x, 0x000F000Fu, magic)) - off;
    v[1] = as_h2(and_or(y, 0x000F000Fu, magic)) - off;
    v[2] = __builtin_elementwise_fma(as_h2(and_or(x, 0x00F000F0u, magic)), sixteenth, off_hi);
    v[3] = __builtin_elementwise_fma(as_h2(and_or(y, 0x00F000F0u, magic)), sixteenth, off_hi);
}

// Byte offset, inside a row, of the dword holding the scale of block b and
// of the 3-dword window holding the 8 code bytes of half h; the codes start
// 2 + 2*(b & 1) bytes into the window. Every window lies inside its row.
__device__ __forceinline__ int scale_dword_off(int b) { return 18 * b - 2 * (b & 1); }
__device__ __forceinline__ int window_off(int b, int h) { return 18 * b + 8 * h - 2 * (b & 1); }

__device__ __forceinline__ void load_half_block(const uint8_t *row, int b, int h, u32 *r)
{
    r[0] = *(const u32 *)(row + scale_dword_off(b));
    const u32 *wp = (const u32 *)(row + window_off(b, h));
    r[1] = wp[0];
    r[2] = wp[1];
    r[3] = wp[2];
}

// scale (fp16 bits) and the two code dwords of a loaded half-block
__device__ __forceinline__ void split_half_block(const u32 *r, int b, _Float16 &s, u32 &c0, u32 &c1)
{
    const bool odd = b & 1;
    s = __builtin_bit_cast(_Float16, (uint16_t)(odd ? (r[0] >> 16) : (r[0] & 0xFFFFu)));
    c0 = odd ? r[2] : __builtin_amdgcn_alignbyte(r[2], r[1], 2);
    c1 = odd ? r[3] : __builtin_amdgcn_alignbyte(r[3], r[2], 2);
}


// Raw-buffer descriptor over one chunk of cache rows: the base moves with the
// chunk (scalar arithmetic), the per-lane offsets stay constant, and reads
// past num_records return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const uint8_t *base, u32 bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, 0x00020000);
}

template <int D, bool WIDE_V>
struct Q4Loader {
    using Sh = Q4Share<D>;
    static constexpr int NB = Sh::NB;
    const uint8_t *kbase;  // K cache of this KV head
    const uint8_t *vbase;
    int64_t tok_stride;
    u32 chunk_bytes;   // 64 rows
    int kk, u;         // K: key in chunk, half-block group
    int kg, vb, vh;    // V: key group, block, half
    u32 krow;          // byte offset of this thread's K row inside a chunk
    u32 voff_s, voff_w;  // V: offsets of the scale dword and the code window of the first key
    u32 rk[Sh::RAWK];
    u32 rv[Sh::RAWV];

    __device__ __forceinline__ void init(const SplitArgs &a, int gkv, int tid)
    {
        kbase = a.k_cache + (int64_t)gkv * a.head_stride;
        vbase = a.v_cache + (int64_t)gkv * a.head_stride;
        tok_stride = a.tok_stride;
        chunk_bytes = (u32)(kChunk * a.tok_stride);
        kk = tid & 63;
        u = __builtin_amdgcn_readfirstlane(tid >> 6);
        kg = tid % Sh::KG;
        const int rest = tid / Sh::KG;
        vb = rest % NB;
        vh = rest / NB;
        krow = (u32)(kk * tok_stride);
        const u32 vrow = (u32)(Sh::NKV * kg * tok_stride);
        voff_s = vrow + (u32)scale_dword_off(vb);
        voff_w = vrow + (u32)window_off(vb, vh);
    }

    // Every row of a chunk is a cache row (a window's remainder is either
    // read as the chunk that ends at the window's end or left to the merge
    // kernel), so no bounds checks beyond the descriptor's. A chunk past the
    // split's end (valid false) gets an empty descriptor: its loads return
    // zeros without touching memory. With shared tiles the kernel issues
    // them unconditionally, so that every path through the loop has the same
    // loads in flight and each wait counts only the loads it needs (128K
    // context: 103.2 against 101.1 us); without, a branch skips them, which
    // measured faster there (32 nodes at 128K: 146.5 against 152.4 us).
    __device__ __forceinline__ void load_k(int64_t chunk_row, bool valid)
    {
        const __amdgpu_buffer_rsrc_t r = chunk_rsrc(kbase + chunk_row * tok_stride, valid ? chunk_bytes : 0u);
        if constexpr (Sh::HB == 4) {
            // blocks 2u and 2u+1: 36 contiguous bytes from a 4-byte aligned start
            const int so = 36 * u;
            const u4v d0 = __builtin_amdgcn_raw_buffer_load_b128(r, krow, so, 0);
            const u4v d1 = __builtin_amdgcn_raw_buffer_load_b128(r, krow, so + 16, 0);
            const u32 d8 = __builtin_amdgcn_raw_buffer_load_b32(r, krow, so + 32, 0);
            const u32 d[9] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w, d8};
            // half-block t: scale dword, then the 3-dword window of its codes
            const int sc[4] = {0, 0, 4, 4}, wi[4] = {0, 2, 4, 6};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                rk[4 * t] = d[sc[t]];
                rk[4 * t + 1] = d[wi[t]];
                rk[4 * t + 2] = d[wi[t] + 1];
                rk[4 * t + 3] = d[wi[t] + 2];
            }
        } else {
#pragma unroll
            for (int t = 0; t < Sh::HB; ++t) {
                const int j = u * Sh::HB + t, b = j >> 1, h = j & 1;
                rk[4 * t] = __builtin_amdgcn_raw_buffer_load_b32(r, krow, scale_dword_off(b), 0);
                const u3v w = __builtin_amdgcn_raw_buffer_load_b96(r, krow, window_off(b, h), 0);
                rk[4 * t + 1] = w.x;
                rk[4 * t + 2] = w.y;
                rk[4 * t + 3] = w.z;
            }
        }
    }

    __device__ __forceinline__ void load_v(int64_t chunk_row, bool valid)
    {
        const __amdgpu_buffer_rsrc_t r = chunk_rsrc(vbase + chunk_row * tok_stride, valid ? chunk_bytes : 0u);
#pragma unroll
        for (int q = 0; q < Sh::NKV; ++q) {
            const int so = (int)(q * tok_stride);
            rv[4 * q] = __builtin_amdgcn_raw_buffer_load_b32(r, voff_s, so, 0);
            const u3v w = __builtin_amdgcn_raw_buffer_load_b96(r, voff_w, so, 0);
            rv[4 * q + 1] = w.x;
            rv[4 * q + 2] = w.y;
            rv[4 * q + 3] = w.z;
        }
    }

    // K piece j (0..NB-1): code dword j of this thread -> one 16-byte store
    __device__ __forceinline__ void k_piece(int j, _Float16 *ks, u32 magic) const
    {
        const int t = j >> 1, k = j & 1;
        const int hbi = u * Sh::HB + t, b = hbi >> 1, h = hbi & 1;
        _Float16 s;
        u32 c0, c1;
        split_half_block(rk + 4 * t, b, s, c0, c1);
        h2 v[4];
        q4_unpack_ao(k ? c1 : c0, magic, v);
        const h2 s2 = {s, s};
        h8 o;
        o.s01 = v[0] * s2;
        o.s23 = v[1] * s2;
        o.s45 = v[2] * s2;
        o.s67 = v[3] * s2;
        // code dword index inside the block is 2h + k
        *(h8 *)(ks + kk * Stage<D, TV_KV_Q4_0, WIDE_V>::KSTR + 32 * b + 8 * (2 * h + k)) = o;
    }

    static constexpr int V_PIECES = Sh::NKV >= 2 ? 4 : 2;

    // V piece p: for NKV >= 2, code dword k = p >> 1 and element half
    // (p & 1 ? the "b" bytes : the "a" bytes) of all NKV keys
    __device__ __forceinline__ void v_piece(int p, _Float16 *vt, u32 magic) const
    {
        constexpr int VSTR = Stage<D, TV_KV_Q4_0, WIDE_V>::VSTR;
        const int pos = vpos(Sh::NKV * kg);
        if constexpr (Sh::NKV >= 2) {
            const int k = p >> 1;
            const bool second = p & 1;
            const int e0 = 8 * vh + 4 * k;
            h2 vals[Sh::NKV / 2][4];
#pragma unroll
            for (int pr = 0; pr < Sh::NKV / 2; ++pr) {
                _Float16 s0, s1;
                u32 a0, a1, b0, b1;
                split_half_block(rv + 4 * (2 * pr), vb, s0, a0, a1);
                split_half_block(rv + 4 * (2 * pr + 1), vb, s1, b0, b1);
                const u32 x0 = k ? a1 : a0, x1 = k ? b1 : b0;
                const u32 z = __builtin_amdgcn_perm(x1, x0, second ? 0x07060302u : 0x05040100u);
                q4_unpack_ao(z, magic, vals[pr]);
                const h2 s2 = {s0, s1};
#pragma unroll
                for (int t = 0; t < 4; ++t) vals[pr][t] = vals[pr][t] * s2;
            }
            // element of vals[*][t]: a-bytes give e0, e0+1, e0+16, e0+17;
            // b-bytes give e0+2, e0+3, e0+18, e0+19. One per-thread base
            // (block, half, key position), the rest immediate offsets.
            _Float16 *vrow = vt + (32 * vb + 8 * vh) * VSTR + pos;
            const int de = 4 * k + (second ? 2 : 0);
            const int ev[4] = {de, de + 1, de + 16, de + 17};
            (void)e0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                _Float16 *dst = vrow + ev[t] * VSTR;
                if constexpr (Sh::NKV == 4) {
                    h4 w4;
                    w4.s01 = vals[0][t];
                    w4.s23 = vals[1][t];
                    *(h4 *)dst = w4;
                } else {
                    *(h2 *)dst = vals[0][t];
                }
            }
        } else {
            // one key: code dword p of the half-block, fp16 stores
            _Float16 s;
            u32 c0, c1;
            split_half_block(rv, vb, s, c0, c1);
            h2 v[4];
            q4_unpack_ao(p ? c1 : c0, magic, v);
            const h2 s2 = {s, s};
            const int e0 = 8 * vh + 4 * p;
            const int ev[8] = {e0, e0 + 2, e0 + 1, e0 + 3, e0 + 16, e0 + 18, e0 + 17, e0 + 19};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const h2 w = v[t] * s2;
                vt[(32 * vb + ev[2 * t]) * VSTR + pos] = w.x;
                vt[(32 * vb + ev[2 * t + 1]) * VSTR + pos] = w.y;
            }
        }
    }
};

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
                                              mwriter ? rowi * 4u : kOffNone, 0, 0);
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
            __builtin_amdgcn_raw_buffer_store_b128(v, rwo, r0 + jj * QS::RS < nrows ? rw.off + part : kOffNone, 0, 0);
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
