// Pieces shared by the split kernels (internal header of libtv.so).
#pragma once

#include <math.h>

#include "tv_internal.h"

namespace tv {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32;
typedef u32 u2v __attribute__((ext_vector_type(2)));
typedef u32 u3v __attribute__((ext_vector_type(3)));
typedef u32 u4v __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over `bytes` bytes from `base`: loads at an offset
// past the end return zero and stores there are dropped (the range check
// covers the per-lane offset plus the immediate).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, u32 bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, 0x00020000);
}

// a per-lane buffer offset that is always out of range
constexpr u32 kOffNone = 0x80000000u;

// Cache-policy bit of a buffer store (its aux operand) that makes the store
// coherent at device scope (sc1 on gfx950): complete, it is visible to every
// workgroup of the device, with no L2 write-back. Every split kernel stores
// its partial state this way, so that none of it is left dirty in the L2s
// when the launch ends and the end-of-launch release has little to write back
// (measured on gfx950: 0.5-1 us less per split-and-merge pair).
constexpr int kCpolSc1 = 16;

// Keeps the scheduler from hoisting every LDS fragment load of an unrolled
// loop to its top, which would need a register per fragment.
#define TV_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

constexpr float kTau = 8.0f;
constexpr float kNegBig = -1.0e30f;

struct SplitArgs {
    const uint8_t *k_cache;
    const uint8_t *v_cache;
    int64_t tok_stride;
    int64_t head_stride;
    const _Float16 *q;
    _Float16 *ws_o;  // [S][NR][D] partial outputs, each divided by its row sum
    float *ws_m;     // [S][NR] log2 of the partial's softmax denominator
    int64_t s0;          // first row of the split kernel's chunks
    int64_t n_whole;     // whole chunks from s0; a chunk after them (masked kernels) ends at the window's end
    int64_t last_start;  // first row of that chunk
    int64_t c_per;  // whole chunks per split: n_chunks / S
    int32_t c_rem;  // n_chunks % S
    int32_t NR;     // n * H_q
    int32_t H_q;
    int32_t G;
    int32_t M;  // G * n
    int32_t S;
    float c;  // scale * log2(e)
    // masked kernels, per-position window: node i sees the window from row
    // s0 + skip[i] on
    int32_t has_skip;
    int32_t skip[TV_MAX_NODES];
};

// First cache row of chunk c: whole chunks from s0; for the masked kernels,
// then the chunk that ends at the window's end.
template <bool MASK>
__device__ __forceinline__ int64_t chunk_row(const SplitArgs &a, int64_t c)
{
    if constexpr (MASK) return c < a.n_whole ? a.s0 + c * kChunk : a.last_start;
    return a.s0 + c * kChunk;
}

// Whether chunk c holds keys some query row may not see: the first chunk of
// a per-position window, and the chunk that ends at the window's end (its
// rows before the end of the whole chunks are already counted).
__device__ __forceinline__ bool chunk_masked(const SplitArgs &a, int64_t c)
{
    return c == a.n_whole || (c == 0 && a.has_skip);
}

// Offset from s0 of the first window row that a slot's query row sees (0 for
// padding rows), computed where a masked chunk needs it.
__device__ __forceinline__ int row_skip(const SplitArgs &a, int tile, int t_end, int col)
{
    const int r = 16 * tile + col;
    return (a.has_skip && tile < t_end && r < a.M) ? a.skip[r / a.G] : 0;
}

// In a masked chunk, the count of leading keys a row may not see: those
// before its first visible row or before the end of the whole chunks.
__device__ __forceinline__ int masked_keys(const SplitArgs &a, int64_t c, int skip)
{
    const int64_t cs = chunk_row<true>(a, c);
    const int64_t floor_row = c == a.n_whole ? a.s0 + a.n_whole * kChunk : a.s0;
    const int64_t first = a.s0 + skip > floor_row ? a.s0 + skip : floor_row;
    return (int)(first - cs);
}

// Scores of key tile kt of a 16x16 S^T tile (lane (col, grp) holds keys
// 16kt + 4grp + e of row col) below `thr` become -inf; exp2 makes them 0.
__device__ __forceinline__ void mask_tile(f4 &s, int kt, int grp, int thr)
{
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (16 * kt + 4 * grp + e < thr) s[e] = -INFINITY;
}

// First chunk of split s (s = S gives n_chunks): floor(n_chunks * s / S),
// written as s * c_per + floor(s * c_rem / S) so that it needs no 64-bit
// division (s * c_rem < S * S fits 32 bits for S < 65536).
__device__ __forceinline__ int64_t split_chunk_begin(const SplitArgs &a, int s)
{
    return (int64_t)s * a.c_per + (int64_t)((uint32_t)s * (uint32_t)a.c_rem / (uint32_t)a.S);
}

typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(u32 x) { return __builtin_bit_cast(h2, x); }

// fp32 pair -> fp16 pair (round toward zero), one instruction
__device__ __forceinline__ h2 pk_rtz(float a, float b)
{
    return __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// acc + p.x + p.y in fp32 (exact products with 1, fp32 sums)
__device__ __forceinline__ float add_pair(h2 p, float acc)
{
    const fp16x2 one = {(__fp16)1.0f, (__fp16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2, p), one, acc, false);
}

// A split's partial state leaves the kernel normalised: O / l in fp16 (a
// convex combination of V rows, so it has the range of V) and the log2 of its
// denominator m + log2(l), which is all a log-sum-exp merge needs. A row with
// no keys gets a zero output and a weight of 2^-1e30.
__device__ __forceinline__ float partial_lse2(float m, float l)
{
    return l > 0.f ? m + __builtin_amdgcn_logf(l) : kNegBig;
}

__device__ __forceinline__ void store_h4(_Float16 *p, f4 v, float inv)
{
    *(h4 *)p = __builtin_convertvector(v * inv, h4);
}

// 8 Q4_0 codes packed in one dword (code bytes 4k..4k+3 of a block) -> the
// exact values code - 8 as four fp16 pairs: [0] = elements (4k, 4k+2),
// [1] = (4k+1, 4k+3), [2] = (4k+16, 4k+18), [3] = (4k+17, 4k+19).
// 0x6400 | c is fp16 1024 + c; 0x6400 | (c << 4) is 1024 + 16 c.
__device__ __forceinline__ void q4_unpack(u32 x, h2 v[4])
{
    const u32 y = x >> 8;
    const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    v[0] = as_h2((x & 0x000F000Fu) | 0x64006400u) - off;
    v[1] = as_h2((y & 0x000F000Fu) | 0x64006400u) - off;
    v[2] = __builtin_elementwise_fma(as_h2((x & 0x00F000F0u) | 0x64006400u), sixteenth, off_hi);
    v[3] = __builtin_elementwise_fma(as_h2((y & 0x00F000F0u) | 0x64006400u), sixteenth, off_hi);
}

// Position of chunk key kappa (0..63) in a transposed V row: inside each group
// of 32 keys, the 8 keys a lane group of the PV MFMA consumes are contiguous.
__device__ __forceinline__ int vpos(int kappa)
{
    return (kappa & ~31) + 8 * ((kappa & 15) >> 2) + 4 * ((kappa >> 4) & 1) + (kappa & 3);
}

template <int D, int KVT, bool WIDE_V = false>
struct Stage {
    static constexpr int NB = D / 32;   // 32-wide blocks per row
    static constexpr int NK = NB / 2;   // keys per thread in a chunk (K or V)
    // K row stride in LDS (halves)
    static constexpr int KSTR = D + 8;
    // V^T row stride in LDS (halves): 144 bytes, or with WIDE_V 160 bytes,
    // an odd multiple of 32, at which a PV fragment read (16 rows x 4 lane
    // groups of 16 bytes) meets no bank conflict. The Q4_0 kernels with
    // shared tiles take the wide stride (128K context: 105.5 against 107.8
    // us); those without, and the F16 kernels, measured faster at 144 bytes.
    static constexpr int VSTR = WIDE_V ? kChunk + 16 : kChunk + 8;
    static constexpr int KELEMS = kChunk * KSTR;
    static constexpr int VELEMS = D * VSTR;
    static constexpr int ELEMS = KELEMS + VELEMS;
    // raw registers per thread for the next chunk
    static constexpr int RAW = KVT == TV_KV_Q4_0 ? NK * 5 : NK * 16;
};

__device__ __forceinline__ float wave_max_16_32(float x)
{
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

// max over the four lanes {l, l^16, l^32, l^48} with the gfx950 row-swap
// permutes: each swap hands every lane the value of its partner row, one of
// the two results being the lane's own value.
__device__ __forceinline__ float xmax_16_32(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum_16_32(float x)
{
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// Rescale one query tile's state when its chunk max mnew exceeds the running
// max by more than kTau anywhere in the wave.
template <int NDT>
__device__ __forceinline__ void maybe_rescale(float mnew, float &m, float &l, f4 (&o)[NDT])
{
    const bool need = mnew > m + kTau;
    if (__builtin_amdgcn_ballot_w64(need)) {
        const float mm = fmaxf(m, mnew);
        const float f = __builtin_amdgcn_exp2f(m - mm);
        l *= f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= f;
        m = mm;
    }
}

struct SplitArgs;
typedef void (*split_fn)(const SplitArgs);

// threads of a warp-specialised split workgroup (8 wave64s)
constexpr int kWsThreads = 512;

// The tensors of one split launch that change from layer to layer (a
// multi-layer launch passes one set per layer with the other SplitArgs
// fields shared).
struct SplitPtrs {
    const uint8_t *k_cache;
    const uint8_t *v_cache;
    const _Float16 *q;
    _Float16 *ws_o;
    float *ws_m;
};

// Tiles of one row group. Own tile k of wave w is t0 + 4k + w, shared tile u
// is t0 + 4*NOWN + u; tiles at or past t_end are padding (zero queries,
// results dropped), so every wave runs the same instructions.
struct TileMap {
    int t0, t_end;
    __device__ __forceinline__ void init(int M, int rg, int RG)
    {
        const int T = (M + 15) / 16;
        const int tb = T / RG, te = T % RG;
        const int Tg = tb + (rg < te ? 1 : 0);
        t0 = rg * tb + (rg < te ? rg : te);
        t_end = t0 + Tg;
    }
};

// Byte offset of query row r of KV head gkv (node r / G, head gkv*G + r % G)
// in a [node][H_q][D] fp16 tensor, stepped `rs` rows at a time with one
// division in all (the row step is at most one carry of the head index).
struct RowWalk {
    u32 off, step, carry;
    int h, dh, G;
    __device__ __forceinline__ RowWalk(const SplitArgs &a, int gkv, int r, int rs, u32 rowb)
    {
        const u32 nodeb = (u32)a.H_q * rowb;
        G = a.G;
        h = r % G;
        off = (u32)(r / G) * nodeb + (u32)(gkv * G + h) * rowb;
        dh = rs % G;
        step = (u32)(rs / G) * nodeb + (u32)dh * rowb;
        carry = nodeb - (u32)G * rowb;
    }
    __device__ __forceinline__ void next()
    {
        h += dh;
        off += step;
        const bool wrap = h >= G;
        h = wrap ? h - G : h;
        off = wrap ? off + carry : off;
    }
};

// Q fragments of a workgroup's tiles (B operands of S^T = K Q^T), staged
// through LDS before the first chunk is dequantised there: lane (col, grp)
// of tile t ends up with query row 16*t + col, 8 values per 32-wide block.
// For Q4_0 the 8 values follow the element order of q4_unpack, for F16 the
// natural order.
//
// The workgroup reads its rows as contiguous 16-byte pieces (a 1 KB span
// per wave instruction; read straight into fragments, each instruction
// would gather 32-byte pieces of 16 rows) and writes them to LDS in the
// fragments' element order, so that each wave reads a fragment as one
// 16-byte piece. A wave runs alone on its SIMD here, so the address
// arithmetic before the loads is not hidden: one division per thread, then
// 32-bit offsets stepped row by row into a buffer over the query tensor.
//
// load() issues every load of the thread, with no branch around any of
// them; loads the caller issues after it and before store() stay in flight,
// since store() waits only for these (loads complete in issue order). Rows
// past the last query row fall past the end of the tensor and read as zero;
// every slot a lane reads in store() is written first (by the group's rows,
// the next group's rows or those zeros), and a padding row's partial state
// is never written. `lds` must be free when store() starts; it is free
// again on return (after a barrier).
template <int D, int KVT, int NOWN, int NSH, int NTH = 256>
struct QStage {
    static constexpr int NS = NOWN + NSH;
    static constexpr int NB = D / 32;
    static constexpr int QSTR = D + 16;  // row stride (halves): 16 rows x 4 lanes of 2 dwords, 2-way at most
    static constexpr int NT = 4 * NOWN + NSH;  // tiles of a workgroup
    static constexpr int PR = D / 8;           // 16-byte pieces per row
    static constexpr int RS = NTH / PR;        // rows between a thread's pieces (NTH threads)
    static constexpr int NQ = (16 * NT + RS - 1) / RS;  // pieces per thread
    static_assert(NQ * RS * QSTR <= 2 * Stage<D, KVT>::ELEMS, "staged query rows fit both stages");
    u4v pc[NQ];

    __device__ __forceinline__ void load(const SplitArgs &a, int gkv, int t0, int tid) { load(a, a.q, gkv, t0, tid); }

    __device__ __forceinline__ void load(const SplitArgs &a, const _Float16 *q, int gkv, int t0, int tid)
    {
        const __amdgpu_buffer_rsrc_t rq = raw_rsrc(q, (u32)a.NR * (u32)(2 * D));
        RowWalk rw(a, gkv, 16 * t0 + tid / PR, RS, 2 * D);
        const u32 part = 16u * (u32)(tid % PR);
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            pc[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, rw.off + part, 0, 0);
            rw.next();
        }
    }

    // the rows into LDS (no barrier)
    __device__ __forceinline__ void write_rows(int tid, _Float16 *lds) const
    {
        if constexpr (KVT == TV_KV_Q4_0) {
            // Rows go to LDS already in the fragments' element order, so that
            // a fragment is one 16-byte read: in block bb, lane group g reads
            // elements 4g + (0, 2, 1, 3), then 16 + 4g + (0, 2, 1, 3) (the
            // order of q4_unpack). This thread's piece holds elements 8s .. 8s+7
            // of block bb; its half h (4 elements, two dwords) is reordered by
            // two byte permutes and lands at 8 ((2s + h) mod 4) + 4 (s / 2).
            const int q = tid % PR, bb = q / 4, sub = q % 4;
            _Float16 *dst = lds + (tid / PR) * QSTR + 32 * bb;
            const int pos0 = 8 * ((2 * sub) % 4) + 4 * (sub / 2);
            const int pos1 = 8 * ((2 * sub + 1) % 4) + 4 * (sub / 2);
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const u4v v = pc[j];
                const u2v h0 = {__builtin_amdgcn_perm(v[1], v[0], 0x05040100u), __builtin_amdgcn_perm(v[1], v[0], 0x07060302u)};
                const u2v h1 = {__builtin_amdgcn_perm(v[3], v[2], 0x05040100u), __builtin_amdgcn_perm(v[3], v[2], 0x07060302u)};
                *(u2v *)(dst + j * RS * QSTR + pos0) = h0;
                *(u2v *)(dst + j * RS * QSTR + pos1) = h1;
            }
        } else {
            _Float16 *dst = lds + (tid / PR) * QSTR + 8 * (tid % PR);
#pragma unroll
            for (int j = 0; j < NQ; ++j) *(u4v *)(dst + j * RS * QSTR) = pc[j];
        }
    }

    // fragment of block bb for lane (col, grp) of the tile whose first row is
    // row tl0 of the group
    static __device__ __forceinline__ h8 frag(const _Float16 *lds, int tl0, int col, int grp, int bb)
    {
        return *(const h8 *)(lds + (tl0 + col) * QSTR + 8 * grp + 32 * bb);
    }

    __device__ __forceinline__ void store(int t0, const int (&tile)[NS], int tid, int col, int grp, _Float16 *lds,
                                          h8 (&qf)[NS][NB]) const
    {
        write_rows(tid, lds);
        __syncthreads();
        // every LDS read is issued before the first is used (left to itself
        // the compiler keeps one or two in flight and each waits out the
        // LDS latency)
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const _Float16 *qr = lds + (16 * (tile[k] - t0) + col) * QSTR + 8 * grp;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) qf[k][bb] = *(const h8 *)(qr + 32 * bb);
        }
        __syncthreads();
    }
};

// Writes the split's partial state (normalised output, log2 denominator) of
// every query row, for the F16 split kernel. `scratch` is the kernel's LDS
// (both stages, at least scratch_bytes long), free once every wave is past
// the last chunk. Shared tiles first: the four waves' partial states of a
// shared tile (each wave scored a quarter of the keys) are combined through
// LDS and written element by element (consecutive threads, consecutive
// values). Then the own tiles: their normalised fp16 rows are gathered in LDS
// and written as contiguous 16-byte pieces, a 1 KB span per wave instruction
// (stored straight from the fragments, each instruction would scatter 8-byte
// pieces over 16 rows). Stores go through buffers over this split's blocks of
// the workspace; a row that is not this workgroup's own gets an out-of-range
// offset, which drops the store.
template <int D, int NOWN, int NSH>
__device__ __forceinline__ void write_partials(const SplitArgs &a, _Float16 *scratch, int scratch_bytes, int tid,
                                               int w, int col, int grp, int gkv, int split, int t0, int t_end,
                                               const int (&tile)[NOWN + NSH], f4 (&o)[NOWN + NSH][D / 16],
                                               float (&m)[NOWN + NSH], float (&l)[NOWN + NSH])
{
    constexpr int NDT = D / 16;
    using QS = QStage<D, TV_KV_F16, NOWN, NSH>;
    (void)scratch_bytes;
    const __amdgpu_buffer_rsrc_t rwo = raw_rsrc(a.ws_o + (int64_t)split * a.NR * D, (u32)a.NR * (u32)(2 * D));
    const __amdgpu_buffer_rsrc_t rwm = raw_rsrc(a.ws_m + (int64_t)split * a.NR, (u32)a.NR * 4u);
    __syncthreads();  // every wave is done with the K/V stages
    if constexpr (NSH > 0) {
        float *so = (float *)scratch;            // [NSH][4][16][D]
        float *sml = so + NSH * 4 * 16 * D;      // [NSH][4][16][2]
#pragma unroll
        for (int u = 0; u < NSH; ++u) {
            const float lt = wave_sum_16_32(l[NOWN + u]);
            float *dst = so + ((u * 4 + w) * 16 + col) * D + 4 * grp;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) *(f4 *)(dst + 16 * dt) = o[NOWN + u][dt];
            if (grp == 0) {
                sml[((u * 4 + w) * 16 + col) * 2] = m[NOWN + u];
                sml[((u * 4 + w) * 16 + col) * 2 + 1] = lt;
            }
        }
        __syncthreads();
        for (int u = 0; u < NSH; ++u) {
            if (tile[NOWN + u] >= t_end) continue;
            for (int e = tid; e < 16 * D; e += 256) {
                const int qr = e / D, d = e % D;
                const int r = 16 * tile[NOWN + u] + qr;
                float mw[4], mx = kNegBig;
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) {
                    mw[ww] = sml[((u * 4 + ww) * 16 + qr) * 2];
                    mx = fmaxf(mx, mw[ww]);
                }
                float acc = 0.f, lsum = 0.f;
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) {
                    const float f = __builtin_amdgcn_exp2f(mw[ww] - mx);
                    acc += f * so[((u * 4 + ww) * 16 + qr) * D + d];
                    lsum += f * sml[((u * 4 + ww) * 16 + qr) * 2 + 1];
                }
                const u32 rowi = (u32)((r / a.G) * a.H_q + gkv * a.G + r % a.G);
                const bool valid = r < a.M;
                const _Float16 v = (_Float16)(lsum > 0.f ? acc / lsum : 0.f);
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), rwo,
                                                      valid ? rowi * (u32)(2 * D) + 2u * (u32)d : kOffNone, 0, kCpolSc1);
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, partial_lse2(mx, lsum)), rwm,
                                                      valid && d == 0 ? rowi * 4u : kOffNone, 0, kCpolSc1);
            }
        }
        __syncthreads();  // the scratch is free again
    }
    // own tiles: normalised fp16 rows into LDS, then contiguous stores
#pragma unroll
    for (int k = 0; k < NOWN; ++k) {
        const float lt = wave_sum_16_32(l[k]);
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        _Float16 *orow = scratch + (16 * (tile[k] - t0) + col) * QS::QSTR + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) *(h4 *)(orow + 16 * dt) = __builtin_convertvector(o[k][dt] * inv, h4);
        const int r = 16 * tile[k] + col;
        const bool mwriter = tile[k] < t_end && r < a.M && grp == 0;
        const u32 rowi = (u32)((r / a.G) * a.H_q + gkv * a.G + r % a.G);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, partial_lse2(m[k], lt)), rwm,
                                              mwriter ? rowi * 4u : kOffNone, 0, kCpolSc1);
    }
    __syncthreads();
    {
        // own rows are the first 16 * 4 * NOWN of the group (tiles t0 + 4k + w)
        const int nown_rows = min(min(16 * t_end, a.M) - 16 * t0, 16 * 4 * NOWN);
        const int r0 = tid / QS::PR;
        RowWalk rw(a, gkv, 16 * t0 + r0, QS::RS, 2 * D);
        const u32 part = 16u * (u32)(tid % QS::PR);
        const _Float16 *src = scratch + r0 * QS::QSTR + 8 * (tid % QS::PR);
#pragma unroll
        for (int jj = 0; jj < QS::NQ; ++jj) {
            const u4v v = *(const u4v *)(src + jj * QS::RS * QS::QSTR);
            __builtin_amdgcn_raw_buffer_store_b128(v, rwo, r0 + jj * QS::RS < nown_rows ? rw.off + part : kOffNone, 0, kCpolSc1);
            rw.next();
        }
    }
}

split_fn pick_split_q4(int D, int nown, int nsh, bool mask);
// The warp-specialised Q4_0 kernel (512 threads) for a tile layout, or null
// when it has none (head_dim other than 256, other layouts).
split_fn pick_split_q4ws(int D, int nown, int nsh);
split_fn pick_split_f16ws(int D, int nown, int nsh);

}  // namespace tv
