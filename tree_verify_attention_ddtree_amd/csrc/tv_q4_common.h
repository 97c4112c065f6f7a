// Q4_0 decoding pieces shared by the Q4_0 split kernels (internal header of
// libtv.so). A Q4_0 row is a sequence of 18-byte blocks: an fp16 scale, then
// 16 code bytes; element e (0..15) of a block is the low nibble of code byte
// e, element e + 16 its high nibble; value = scale * (code - 8).
#pragma once

#include "tv_split_common.h"

namespace tv {

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

    // Lane mapping of the warp-specialised kernel (head_dim 256), where load
    // wave q of four dequantises the chunk's keys 16q .. 16q + 15 over all of
    // D and D-quarter q (blocks 2q, 2q + 1) of all 64 keys:
    //   K: key 16q + (lane & 15), blocks 2u and 2u + 1 with u = lane >> 4
    //      (36 contiguous bytes);
    //   V: keys 4 (lane & 15) .. + 3, half-block (block 2q + (lane >> 5),
    //      half (lane >> 4) & 1).
    __device__ __forceinline__ void init_ws(const SplitArgs &a, const SplitPtrs &p, int gkv, int q, int lane)
    {
        static_assert(D == 256, "the warp-specialised mapping is for head_dim 256");
        kbase = p.k_cache + (int64_t)gkv * a.head_stride;
        vbase = p.v_cache + (int64_t)gkv * a.head_stride;
        tok_stride = a.tok_stride;
        chunk_bytes = (u32)(kChunk * a.tok_stride);
        kk = 16 * q + (lane & 15);
        u = lane >> 4;
        kg = lane & 15;
        vb = 2 * q + (lane >> 5);
        vh = (lane >> 4) & 1;
        krow = (u32)(kk * tok_stride) + (u32)(36 * u);
        const u32 vrow = (u32)(Sh::NKV * kg * tok_stride);
        voff_s = vrow + (u32)scale_dword_off(vb);
        voff_w = vrow + (u32)window_off(vb, vh);
    }

    // K bytes of the warp-specialised mapping: 36 contiguous bytes (blocks
    // 2u, 2u + 1 of key kk), split into four half-blocks as load_k does.
    __device__ __forceinline__ void load_k_ws(int64_t chunk_row, bool valid)
    {
        const __amdgpu_buffer_rsrc_t r = chunk_rsrc(kbase + chunk_row * tok_stride, valid ? chunk_bytes : 0u);
        const u4v d0 = __builtin_amdgcn_raw_buffer_load_b128(r, krow, 0, 0);
        const u4v d1 = __builtin_amdgcn_raw_buffer_load_b128(r, krow + 16u, 0, 0);
        const u32 d8 = __builtin_amdgcn_raw_buffer_load_b32(r, krow + 32u, 0, 0);
        const u32 d[9] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w, d8};
        const int sc[4] = {0, 0, 4, 4}, wi[4] = {0, 2, 4, 6};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            rk[4 * t] = d[sc[t]];
            rk[4 * t + 1] = d[wi[t]];
            rk[4 * t + 2] = d[wi[t] + 1];
            rk[4 * t + 3] = d[wi[t] + 2];
        }
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
    // the 8 dequantised values of K piece j (code dword j of this thread),
    // with their block b and 8-value group g = 2h + k inside the block
    __device__ __forceinline__ h8 k_values(int j, u32 magic, int &b, int &g) const
    {
        const int t = j >> 1, k = j & 1;
        const int hbi = u * Sh::HB + t, h = hbi & 1;
        b = hbi >> 1;
        g = 2 * h + k;
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
        return o;
    }

    // K piece j into a row-major stage (row stride KSTR)
    __device__ __forceinline__ void k_piece(int j, _Float16 *ks, u32 magic) const
    {
        int b, g;
        const h8 o = k_values(j, magic, b, g);
        *(h8 *)(ks + kk * Stage<D, TV_KV_Q4_0, WIDE_V>::KSTR + 32 * b + 8 * g) = o;
    }

    static constexpr int V_PIECES = Sh::NKV >= 2 ? 4 : 2;

    // V piece p (NKV >= 2): code dword k = p >> 1 and element half (p & 1 ?
    // the "b" bytes : the "a" bytes) of the NKV keys, dequantised; key pair
    // pr of vals[pr][t] holds element e0 + {0, 1, 16, 17}[t] + 2 (p & 1) of
    // block vb with e0 = 8 vh + 4 k (keys 2 pr and 2 pr + 1 in x and y).
    __device__ __forceinline__ void v_values(int p, u32 magic, h2 (&vals)[Sh::NKV / 2][4]) const
    {
        const int k = p >> 1;
        const bool second = p & 1;
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
    }

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
            v_values(p, magic, vals);
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

}  // namespace tv
