/*
 * tvref.c -- CPU oracle for DDTree tree-verify attention and greedy acceptance.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU library never
 * links it, and it includes nothing from the GPU library (no shared headers,
 * tables or helpers).
 *
 * What it computes is the plain definition, in double precision, with a fixed
 * order of summation, and nothing faster:
 *   - "Luce DFlash" post (Japanese / Korean translations), feature list: the
 *     target scores a DDTree draft tree of budget 22 (block size 16) in one
 *     verify pass and verification is greedy; the KV cache may be Q4_0 or F16;
 *     decode may use a 2048-token sliding-window flash attention.
 *   - Each tree node's query attends to every committed cache row in the
 *     window and to its own ancestors in the tree, itself included.
 *   - Greedy acceptance takes the argmax at every node and keeps the longest
 *     root path along which each child's draft token equals its parent's
 *     argmax; the argmax at the last accepted node is the bonus token.
 *
 * Readings where the pages are silent (each one also listed in the design
 * notes of the repository):
 *   - Q4_0 block: 18 bytes = fp16 scale, then 16 code bytes; element e (0..15)
 *     is the low nibble of code byte e, element e+16 the high nibble; value =
 *     scale * (code - 8).
 *   - Window W > 0: every node sees cache rows [max(0, n_ctx - W), n_ctx);
 *     W = 0 means all rows. Tree nodes never count against the window.
 *     Per-position window (window_mode 1): a node at depth k (position
 *     n_ctx + k) sees the positions [n_ctx + k - W, n_ctx + k] of its own
 *     sequence: cache rows [max(0, n_ctx + k - W), n_ctx) and the ancestors
 *     at depth >= k - W, the W + 1 keys a token at that position has in
 *     token-by-token decoding with the same window.
 *   - GQA: query head h reads KV head h / (H_q / H_kv).
 *   - argmax order: IEEE compare with -0 == +0, NaN below every number, ties
 *     to the smallest index, an all-NaN row gives index 0.
 *   - Longest matching path; among equally long ones the one with the smaller
 *     child index at the first divergence.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC tvref.c -o libtvref.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TVREF_OK 0
#define TVREF_EARG (-1)
#define TVREF_ETREE (-2)
#define TVREF_ESHAPE (-3)

#define TVREF_KV_F16 0
#define TVREF_KV_Q4_0 1

/* IEEE 754 binary16 -> double, from the bit layout: 1 sign bit, 5 exponent
 * bits (bias 15), 10 fraction bits; exponent 0 = zero / subnormal, 31 =
 * infinity / NaN. */
double tvref_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24); /* frac * 2^-10 * 2^-14 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
    }
    return sign ? -v : v;
}

/* One Q4_0 row of D values -> doubles. */
void tvref_q4_0_dequant_row(const uint8_t *row, int D, double *out)
{
    for (int b = 0; b < D / 32; ++b) {
        const uint8_t *blk = row + 18 * b;
        uint16_t sbits = (uint16_t)(blk[0] | (blk[1] << 8));
        double s = tvref_half_to_double(sbits);
        for (int e = 0; e < 32; ++e) {
            int byte = blk[2 + (e % 16)];
            int code = e < 16 ? (byte & 0x0f) : (byte >> 4);
            out[32 * b + e] = s * (double)(code - 8);
        }
    }
}

/* Many consecutive Q4_0 rows (row stride 18*D/32 bytes) -> doubles. */
void tvref_q4_0_dequant_rows(const uint8_t *rows, int64_t n_rows, int D, double *out)
{
    const int64_t rb = 18 * (D / 32);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) tvref_q4_0_dequant_row(rows + r * rb, D, out + r * D);
}

static void half_row(const uint16_t *src, int D, double *out)
{
    for (int d = 0; d < D; ++d) out[d] = tvref_half_to_double(src[d]);
}

/* Checks a parent array: root first, topological numbering. */
int tvref_check_tree(int n, const int32_t *parent)
{
    if (n < 1 || !parent) return TVREF_EARG;
    if (parent[0] != -1) return TVREF_ETREE;
    for (int i = 1; i < n; ++i)
        if (parent[i] < 0 || parent[i] >= i) return TVREF_ETREE;
    return TVREF_OK;
}

/* Ancestors of node i, itself included, in increasing index order (root
 * first). Returns how many were written to anc. */
int tvref_ancestors(int i, const int32_t *parent, int32_t *anc)
{
    int cnt = 0;
    for (int u = i; u >= 0; u = parent[u]) anc[cnt++] = u;
    for (int a = 0, b = cnt - 1; a < b; ++a, --b) {
        int32_t t = anc[a];
        anc[a] = anc[b];
        anc[b] = t;
    }
    return cnt;
}

/* Key/value row j (of the concatenated key list) for KV head g. */
static void load_cache_row(int kv_type, const uint8_t *base, int64_t tok_stride, int64_t head_stride,
                           int g, int64_t j, int D, double *out)
{
    const uint8_t *p = base + (int64_t)g * head_stride + j * tok_stride;
    if (kv_type == TVREF_KV_Q4_0)
        tvref_q4_0_dequant_row(p, D, out);
    else
        half_row((const uint16_t *)p, D, out);
}

/*
 * Tree-verify attention for one layer.
 *
 *   q       fp16 [n][H_q][D]
 *   k_tree  fp16 [n][H_kv][D], v_tree likewise (K/V of the tree nodes)
 *   caches  row j of KV head g at base + g*head_stride + j*tok_stride bytes,
 *           Q4_0 rows of 18*D/32 bytes or fp16 rows of D values
 *   rows    optional list of output rows r = i*H_q + h to compute (NULL: all)
 *   out     double [n][H_q][D]; rows not listed are left untouched
 *
 * For node i and head h (KV head g = h / (H_q/H_kv)) the keys are the cache
 * rows s0..n_ctx-1 in order (s0 per the window and window_mode above), then
 * anc(i) in increasing index order;
 *   s_j = scale * sum_d q[d] K_j[d]      (d ascending)
 *   m = max_j s_j,  w_j = exp(s_j - m),  l = sum_j w_j   (j ascending)
 *   out[d] = (sum_j w_j V_j[d]) / l      (j ascending)
 */
int tvref_attn(int n, const int32_t *parent, int H_q, int H_kv, int D, int64_t n_ctx, int64_t window,
               int window_mode, double scale, int kv_type, const void *k_cache, const void *v_cache,
               int64_t tok_stride, int64_t head_stride, const uint16_t *q, const uint16_t *k_tree,
               const uint16_t *v_tree, const int32_t *rows, int n_rows, double *out)
{
    int rc = tvref_check_tree(n, parent);
    if (rc) return rc;
    if (H_q < 1 || H_kv < 1 || H_q % H_kv || D < 32 || D % 32 || n_ctx < 0 || window < 0) return TVREF_ESHAPE;
    if (kv_type != TVREF_KV_F16 && kv_type != TVREF_KV_Q4_0) return TVREF_EARG;
    if (window_mode != 0 && window_mode != 1) return TVREF_EARG;
    if (n_ctx > 0 && (!k_cache || !v_cache)) return TVREF_EARG;
    const int G = H_q / H_kv;
    const int64_t s0 = (window > 0 && n_ctx > window) ? n_ctx - window : 0;
    const int64_t R = n_ctx - s0;
    const int total = n * H_q;
    const int nr = rows ? n_rows : total;
    for (int t = 0; t < nr; ++t)
        if (rows && (rows[t] < 0 || rows[t] >= total)) return TVREF_EARG;

#pragma omp parallel
    {
        double *K = malloc(sizeof(double) * D);
        double *qd = malloc(sizeof(double) * D);
        double *acc = malloc(sizeof(double) * D);
        double *sc = malloc(sizeof(double) * (size_t)(R + n));
        int32_t *anc = malloc(sizeof(int32_t) * n);
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < nr; ++t) {
            const int r = rows ? rows[t] : t;
            const int i = r / H_q, h = r % H_q, g = h / G;
            const int na = tvref_ancestors(i, parent, anc);
            /* per-position window: the node's depth k = na - 1 moves its
             * start to n_ctx + k - W, in the cache and along its path (anc[a]
             * is at depth a) */
            int64_t si = s0;
            int a0 = 0;
            if (window_mode == 1 && window > 0) {
                si = n_ctx + (na - 1) - window;
                if (si < 0) si = 0;
                const int64_t first = (int64_t)(na - 1) - window;
                a0 = first > 0 ? (int)first : 0;
            }
            half_row(q + ((int64_t)i * H_q + h) * D, D, qd);
            /* pass 1: scores */
            int64_t nk = 0;
            for (int64_t j = si; j < n_ctx; ++j) {
                load_cache_row(kv_type, (const uint8_t *)k_cache, tok_stride, head_stride, g, j, D, K);
                double s = 0.0;
                for (int d = 0; d < D; ++d) s += qd[d] * K[d];
                sc[nk++] = scale * s;
            }
            for (int a = a0; a < na; ++a) {
                half_row(k_tree + ((int64_t)anc[a] * H_kv + g) * D, D, K);
                double s = 0.0;
                for (int d = 0; d < D; ++d) s += qd[d] * K[d];
                sc[nk++] = scale * s;
            }
            /* pass 2: softmax weights and weighted values */
            double m = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) m = sc[j] > m ? sc[j] : m;
            double l = 0.0;
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            nk = 0;
            for (int64_t j = si; j < n_ctx; ++j) {
                const double w = exp(sc[nk++] - m);
                l += w;
                load_cache_row(kv_type, (const uint8_t *)v_cache, tok_stride, head_stride, g, j, D, K);
                for (int d = 0; d < D; ++d) acc[d] += w * K[d];
            }
            for (int a = a0; a < na; ++a) {
                const double w = exp(sc[nk++] - m);
                l += w;
                half_row(v_tree + ((int64_t)anc[a] * H_kv + g) * D, D, K);
                for (int d = 0; d < D; ++d) acc[d] += w * K[d];
            }
            double *o = out + (int64_t)r * D;
            for (int d = 0; d < D; ++d) o[d] = acc[d] / l;
        }
        free(K);
        free(qd);
        free(acc);
        free(sc);
        free(anc);
    }
    return TVREF_OK;
}

/* Order on float32 for the argmax: a > b in IEEE terms; +0 and -0 compare
 * equal; NaN is below every number (and equal to NaN). */
static int f_greater(float a, float b)
{
    if (isnan(a)) return 0;
    if (isnan(b)) return 1;
    return a > b;
}

/* argmax of one row; ties go to the smallest index; all-NaN gives 0. */
int32_t tvref_argmax_row(const float *row, int vocab)
{
    int32_t best = 0;
    for (int v = 1; v < vocab; ++v)
        if (f_greater(row[v], row[best])) best = v;
    return best;
}

/* Depth-first search from u over children in ascending index order. A child
 * c continues the path when tok[c] == a[u]. The first path of maximal length
 * found in this order is the one with the smaller index at the first
 * divergence. */
static void dfs_longest(int u, int n, const int32_t *parent, const int32_t *tok, const int32_t *a,
                        int32_t *cur, int depth, int32_t *best, int *best_len)
{
    cur[depth] = u;
    if (depth + 1 > *best_len) {
        *best_len = depth + 1;
        memcpy(best, cur, sizeof(int32_t) * (size_t)(depth + 1));
    }
    for (int c = u + 1; c < n; ++c)
        if (parent[c] == u && tok[c] == a[u]) dfs_longest(c, n, parent, tok, a, cur, depth + 1, best, best_len);
}

/*
 * Greedy acceptance for one verify step.
 *   logits     fp32 [n][vocab]
 *   parent     int32 [n], tokens int32 [n] (tokens[0], the root's, is unused)
 *   argmax_out int32 [n]
 *   result_out int32 [2 + 2n]:
 *       [0] n_acc (accepted draft tokens), [1] bonus token,
 *       [2 .. 2+n) accepted path node indices, root first, padded with -1,
 *       [2+n .. 2+2n) emitted tokens: tokens of path[1..n_acc], then bonus,
 *                     padded with -1.
 */
int tvref_accept(const float *logits, int n, int vocab, const int32_t *parent, const int32_t *tokens,
                 int32_t *argmax_out, int32_t *result_out)
{
    int rc = tvref_check_tree(n, parent);
    if (rc) return rc;
    if (vocab < 1 || !logits || !tokens || !argmax_out || !result_out) return TVREF_EARG;
    for (int i = 0; i < n; ++i) argmax_out[i] = tvref_argmax_row(logits + (int64_t)i * vocab, vocab);
    int32_t *cur = malloc(sizeof(int32_t) * n);
    int32_t *best = malloc(sizeof(int32_t) * n);
    int best_len = 0;
    dfs_longest(0, n, parent, tokens, argmax_out, cur, 0, best, &best_len);
    const int n_acc = best_len - 1;
    const int32_t bonus = argmax_out[best[best_len - 1]];
    for (int k = 0; k < 2 + 2 * n; ++k) result_out[k] = -1;
    result_out[0] = n_acc;
    result_out[1] = bonus;
    for (int k = 0; k < best_len; ++k) result_out[2 + k] = best[k];
    for (int k = 1; k < best_len; ++k) result_out[2 + n + k - 1] = tokens[best[k]];
    result_out[2 + n + n_acc] = bonus;
    free(cur);
    free(best);
    return TVREF_OK;
}

/* ------------------------------------------------------------------------
 * KV commit of the accepted path: after acceptance the root and the accepted
 * nodes become committed tokens, so their K and V rows are appended to the
 * cache (the pages keep the target's cache in Q4_0 or F16; they name Q4_0
 * but give no quantiser).
 *
 * Reading of the Q4_0 quantiser, per 32-value block, all in fp32 (the
 * precision in which the GPU kernel takes the same integer decisions):
 *   m     = the value of largest magnitude (the first one on ties);
 *   d     = m / -8, stored as fp16 rounded to nearest, ties to even (a block
 *           of zeros, m = 0, stores the scale +0);
 *   id    = 1 / d (0 when d == 0);
 *   c     = x * id rounded to fp32, then + 8.5 rounded to fp32 (two
 *           roundings, no fused multiply-add);
 *   code  = 15 if c >= 15, floor(c) if 0 <= c < 15, and 0 otherwise (which
 *           includes NaN).
 * So the element of largest magnitude gets code 0 and decodes to m exactly
 * whenever d is exact in fp16, and every other value lands on the nearest
 * code, ties upward.
 * ------------------------------------------------------------------------ */

/* IEEE binary32 -> binary16, round to nearest, ties to even; overflow gives
 * infinity, NaN stays NaN (quiet). From the bit layouts. */
uint16_t tvref_float_to_half(float f)
{
    uint32_t x;
    memcpy(&x, &f, sizeof x);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u) return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x0200u : 0u));
    if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u); /* |f| >= 65520 */
    if (ax >= 0x38800000u) {                                  /* |f| >= 2^-14: normal half */
        const uint32_t m = ax - 0x38000000u;                  /* exponent bias 127 -> 15 */
        const uint32_t r = m + 0x0fffu + ((m >> 13) & 1u);    /* drop 13 fraction bits, ties to even */
        return (uint16_t)(sign | (r >> 13));
    }
    if (ax <= 0x33000000u) return (uint16_t)sign; /* |f| <= 2^-25: rounds to zero */
    /* subnormal half: round |f| / 2^-24 to an integer, ties to even */
    const uint32_t e = ax >> 23;
    const uint32_t man = (ax & 0x7fffffu) | 0x800000u; /* |f| = man * 2^(e - 150) */
    const uint32_t s = 126u - e;                       /* |f| / 2^-24 = man >> s */
    uint32_t q = man >> s;
    const uint32_t rem = man & ((1u << s) - 1u), half = 1u << (s - 1u);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return (uint16_t)(sign | q);
}

static int q4_code(float x, float id)
{
    const float p = x * id;
    const float c = p + 8.5f;
    if (c >= 15.0f) return 15;
    if (c >= 0.0f) return (int)floorf(c);
    return 0;
}

/* 32 fp32 values -> one 18-byte Q4_0 block. */
void tvref_q4_0_quantize_block(const float *x, uint8_t *out)
{
    float amax = 0.0f, m = 0.0f;
    for (int j = 0; j < 32; ++j) {
        const float a = fabsf(x[j]);
        if (amax < a) {
            amax = a;
            m = x[j];
        }
    }
    const float d = m != 0.0f ? m / -8.0f : 0.0f;
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
    const uint16_t hd = tvref_float_to_half(d);
    out[0] = (uint8_t)(hd & 0xffu);
    out[1] = (uint8_t)(hd >> 8);
    for (int j = 0; j < 16; ++j) out[2 + j] = (uint8_t)(q4_code(x[j], id) | (q4_code(x[j + 16], id) << 4));
}

/* n_rows rows of D fp32 values -> n_rows Q4_0 rows of 18*D/32 bytes. */
void tvref_q4_0_quantize_rows(const float *x, int64_t n_rows, int D, uint8_t *out)
{
    for (int64_t r = 0; r < n_rows; ++r)
        for (int b = 0; b < D / 32; ++b) tvref_q4_0_quantize_block(x + r * D + 32 * b, out + r * (18 * (D / 32)) + 18 * b);
}

/*
 * Appends the accepted path to one layer's caches.
 *   result   the acceptance result (int32 [2 + 2n]): n_acc = result[0], the
 *            path's nodes result[2 .. 2 + n_acc], root first;
 *   k_tree, v_tree  fp16 bits [n][H_kv][D], the tree nodes' K and V rows;
 *   k_cache, v_cache  rows addressed as head * head_stride + row * tok_stride
 *            (bytes), capacity rows per head; F16 rows are copied, Q4_0 rows
 *            quantised with the reading above.
 * Path node path[r] goes to cache row n_ctx + r of every KV head, for
 * r = 0 .. n_acc; no other row is written.
 */
int tvref_commit(int n, int H_kv, int D, int kv_type, int64_t n_ctx, int64_t capacity, const int32_t *result,
                 const uint16_t *k_tree, const uint16_t *v_tree, uint8_t *k_cache, uint8_t *v_cache,
                 int64_t tok_stride, int64_t head_stride)
{
    if (n < 1 || n > 64 || H_kv < 1 || (D != 64 && D != 128 && D != 256)) return TVREF_ESHAPE;
    if (kv_type != TVREF_KV_F16 && kv_type != TVREF_KV_Q4_0) return TVREF_EARG;
    if (n_ctx < 0 || n_ctx + n > capacity) return TVREF_ESHAPE;
    const int n_acc = result[0];
    if (n_acc < 0 || n_acc >= n) return TVREF_EARG;
    for (int r = 0; r <= n_acc; ++r)
        if (result[2 + r] < 0 || result[2 + r] >= n) return TVREF_EARG;
    float x[256];
    for (int r = 0; r <= n_acc; ++r) {
        const int node = result[2 + r];
        for (int g = 0; g < H_kv; ++g) {
            for (int kv = 0; kv < 2; ++kv) {
                const uint16_t *src = (kv ? v_tree : k_tree) + ((int64_t)node * H_kv + g) * D;
                uint8_t *dst = (kv ? v_cache : k_cache) + g * head_stride + (n_ctx + r) * tok_stride;
                if (kv_type == TVREF_KV_F16) {
                    memcpy(dst, src, (size_t)D * 2);
                } else {
                    for (int d = 0; d < D; ++d) x[d] = (float)tvref_half_to_double(src[d]);
                    for (int b = 0; b < D / 32; ++b) tvref_q4_0_quantize_block(x + 32 * b, dst + 18 * b);
                }
            }
        }
    }
    return TVREF_OK;
}
