/*
 * oracle.c -- float64 CPU oracle for causal prefill self-attention with a
 * head-major KV-cache image.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no source,
 * header, helper or constant with the HIP library under
 * prefill_self_attention_amd/csrc, and neither side includes the other.
 *
 * Sources (the pages this oracle is written from):
 *   [P1] "Prefill不是热身：大模型推理的真正瓶颈与优化核心" (www.mhpn.cn/news/2373630)
 *   [P2] "大模型推理优化：Prefill、Decode与KV Cache的工程实践" (www.zskr.cn/news/2334369)
 *   [P3] "大模型 Prompt Prefill 阶段的高效 Batching 与算子排布" (www.nxmr.cn/news/92962)
 *   [P4] "大语言模型推理核心：Prefill与Decode原理及工程优化" (www.yfxerp.com/news/184489)
 *   [P5] untitled page at www.zwxr.cn/news/300951
 *
 * What is computed is the plain definition, not a tiled or streaming method:
 *   out_i = sum_j softmax_j(scale * q_i . k_j) v_j ,   j over the keys visible to i
 * [P1 §3 and P4 §2.2: attention is softmax(Q K^T / sqrt(d_k)) V, d_k the head
 * dimension; P4 §2.2: every row's normaliser runs over that whole row].
 * Visibility is causal: position a sees itself and every earlier position of
 * its own request [P5 §1.1; P5 §3.3 lower-triangular mask], and never a token
 * of another request in the flattened batch [P3 §2, the varlen kernel attends
 * only inside one request located by cu_seqlens].
 *
 * Arithmetic: every bf16 input is widened exactly to double; the float32
 * `scale` the GPU receives is widened to double; dot products run with d
 * ascending, sums over keys with j ascending, exp() is libm's double exp.  The
 * row maximum is subtracted before exp(), which leaves the real-number result
 * unchanged.  No -ffast-math.  OpenMP parallelises over (sequence, head)
 * pairs only; each pair is computed by the same sequential loops, so the
 * result does not depend on the thread count.
 *
 * Grouped key/value heads [P5 §2.4: grouped-query attention keeps fewer K/V
 * heads than query heads, 32 -> 8 in its example, to shrink the cache]: K, V
 * and the cache carry num_kv_heads heads, and query head h reads K/V head
 * h / (num_heads / num_kv_heads) -- consecutive query heads share one K/V head
 * (the page does not spell out the grouping; this is the plain reading).
 * num_kv_heads == num_heads is ordinary multi-head attention.
 *
 * Parity status: every function here is pinned by tests/test_oracle.py
 * (brute force, a library routine, closed forms, invariants); none is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE float32: widening is exact. */
static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Attention of one query row against an explicit list of n_keys keys.
 *   q        : D bf16 values of the query (one head)
 *   key_row  : callback-free addressing -- key j lives at kbase[j] (D bf16)
 *   out      : D doubles
 *   probs    : optional, receives the n_keys softmax weights of this row
 * The caller passes only the visible keys (causal prefix), so no mask value
 * is needed here.
 */
static void attend_row(const uint16_t *q, const uint16_t *const *kbase,
                       const uint16_t *const *vbase, int64_t n_keys, int D,
                       double scale, double *out, double *probs, double *s)
{
    /* s_j = scale * sum_d q_d k_jd  (d ascending) */
    for (int64_t j = 0; j < n_keys; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += bf16_bits_to_double(q[d]) * bf16_bits_to_double(kbase[j][d]);
        s[j] = scale * dot;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j)
        for (int d = 0; d < D; ++d)
            out[d] += s[j] * bf16_bits_to_double(vbase[j][d]);
    for (int d = 0; d < D; ++d) out[d] /= l;
    if (probs)
        for (int64_t j = 0; j < n_keys; ++j) probs[j] = s[j] / l;
}

/*
 * Where a key lives.  The key/value list seen by sequence b is its cached
 * prefix (chunked prefill: [P3 §3] a chunk attends to the already-cached part
 * of its prompt; [P5 §1.2] a decode token attends to all cached positions and
 * itself) followed by its own new tokens.  Own tokens are read from the k/v
 * inputs; prefix tokens from the cache laid out [B, H, cap, D].
 */
typedef struct {
    const uint16_t *q, *k, *v;        /* q [N, H, D]; k, v [N, HK, D] new tokens */
    const int32_t *cu;                /* [B + 1] */
    const int32_t *prefix;            /* [B] or NULL (no cached prefix) */
    const uint16_t *kc_in, *vc_in;    /* chunked cache contents before the call */
    int32_t B, H, D, cap;
    double scale;
    int32_t HK;                       /* K/V heads; H is a multiple of HK */
    /* paged cache (NULL: the [B, HK, cap, D] slab): block table [B, bt_stride]
     * of physical block indices, blocks [num_blocks, HK, PAGE, D] */
    const int32_t *bt;
    int32_t bt_stride, num_blocks;
} problem_t;

/*
 * Paged KV cache [P2 §4.2 and P5 §3.4: the cache is cut into fixed blocks of
 * 16 tokens that need not be contiguous, and a block table maps each logical
 * block of a request to a physical one; P4 §4.1 gives a block as a small
 * tokens x heads x head_dim array].  Reading taken here: physical block n
 * holds [HK, 16, D] (head-major inside the block, like the slab), and cache
 * position j of sequence b lives in block bt[b][j / 16], row j % 16.
 */
enum { PAGE = 16 };

/* element offset of cache position j of sequence b, K/V head g */
static int64_t cache_off(const problem_t *P, int64_t b, int64_t g, int64_t j)
{
    const int64_t HK = P->HK, D = P->D;
    if (!P->bt) return ((b * HK + g) * P->cap + j) * D;
    const int64_t blk = P->bt[b * P->bt_stride + j / PAGE];
    return ((blk * HK + g) * PAGE + j % PAGE) * D;
}

/* K/V head read by query head h */
static int64_t kv_head(const problem_t *P, int64_t h) { return h / (P->H / P->HK); }

static void gather_keys(const problem_t *P, int b, int h, int64_t n_keys,
                        const uint16_t **kp, const uint16_t **vp)
{
    const int64_t HK = P->HK, D = P->D, g = kv_head(P, h);
    const int64_t pre = P->prefix ? P->prefix[b] : 0;
    for (int64_t j = 0; j < n_keys; ++j) {
        if (j < pre) {
            int64_t off = cache_off(P, b, g, j);
            kp[j] = P->kc_in + off;
            vp[j] = P->vc_in + off;
        } else {
            int64_t tok = (int64_t)P->cu[b] + (j - pre);
            kp[j] = P->k + (tok * HK + g) * D;
            vp[j] = P->v + (tok * HK + g) * D;
        }
    }
}

static int64_t max_keys(const problem_t *P)
{
    int64_t mk = 0;
    for (int b = 0; b < P->B; ++b) {
        int64_t n = (int64_t)P->cu[b + 1] - P->cu[b];
        int64_t pre = P->prefix ? P->prefix[b] : 0;
        if (n + pre > mk) mk = n + pre;
    }
    return mk;
}

/* All rows of all sequences; out is [N, H, D] doubles. */
static int run_all(const problem_t *P, double *out, double *probs)
{
    const int64_t H = P->H, D = P->D;
    const int64_t mk = max_keys(P);
    const int64_t units = (int64_t)P->B * H;
    int failed = 0;
#pragma omp parallel
    {
        const uint16_t **kp = malloc(sizeof(*kp) * (size_t)(mk > 0 ? mk : 1));
        const uint16_t **vp = malloc(sizeof(*vp) * (size_t)(mk > 0 ? mk : 1));
        double *s = malloc(sizeof(double) * (size_t)(mk > 0 ? mk : 1));
        if (!kp || !vp || !s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < units; ++u) {
                const int b = (int)(u / H), h = (int)(u % H);
                const int64_t n = (int64_t)P->cu[b + 1] - P->cu[b];
                const int64_t pre = P->prefix ? P->prefix[b] : 0;
                gather_keys(P, b, h, pre + n, kp, vp);
                for (int64_t i = 0; i < n; ++i) {
                    const int64_t tok = (int64_t)P->cu[b] + i;
                    /* query i sits at absolute position pre + i and sees
                     * keys 0 .. pre + i inclusive (bottom-right alignment) */
                    double *prow = NULL;
                    if (probs) prow = probs + ((int64_t)h * n + i) * (pre + n);
                    attend_row(P->q + (tok * H + h) * D, kp, vp, pre + i + 1,
                               (int)D, P->scale, out + (tok * H + h) * D, prow, s);
                    if (prow)
                        for (int64_t j = pre + i + 1; j < pre + n; ++j) prow[j] = 0.0;
                }
            }
        }
        free(kp);
        free(vp);
        free(s);
    }
    return failed ? -1 : 0;
}

/*
 * Cache image.  The cache keeps K and V of every position of every head, not
 * Q [P2 §1.3], head-major [batch, heads, seq, head_dim] [P2 §1.3; P4 §3.2;
 * P1 §3 recommends the head-major layout].  Prefill writes them for every
 * prompt position [P5 §1.1; P1 §4].
 *   varlen : sequence b's block is [HK, len_b, D] starting at element cu_b*HK*D
 *   chunked: [B, HK, cap, D]; own token t of sequence b lands at position
 *            prefix_b + t.
 * (HK = num_kv_heads; one cache row per K/V head.)
 * Bits are copied unchanged; every other element is left as the caller
 * filled it.
 */
static void write_cache(const problem_t *P, uint16_t *kc, uint16_t *vc)
{
    const int64_t HK = P->HK, D = P->D;
    for (int b = 0; b < P->B; ++b) {
        const int64_t n = (int64_t)P->cu[b + 1] - P->cu[b];
        for (int64_t h = 0; h < HK; ++h)
            for (int64_t t = 0; t < n; ++t) {
                const int64_t src = (((int64_t)P->cu[b] + t) * HK + h) * D;
                int64_t dst;
                if (P->prefix)
                    dst = cache_off(P, b, h, P->prefix[b] + t);
                else
                    dst = (int64_t)P->cu[b] * HK * D + (h * n + t) * D;
                memcpy(kc + dst, P->k + src, sizeof(uint16_t) * (size_t)D);
                memcpy(vc + dst, P->v + src, sizeof(uint16_t) * (size_t)D);
            }
    }
}

static int check_meta(const problem_t *P)
{
    if (P->B < 0 || P->H < 1 || P->D < 1) return -2;
    if (P->HK < 1 || P->H % P->HK != 0) return -2;
    if (P->cu[0] != 0) return -3;
    for (int b = 0; b < P->B; ++b) {
        if (P->cu[b + 1] < P->cu[b]) return -3;
        if (P->prefix) {
            if (P->prefix[b] < 0) return -4;
            if ((int64_t)P->prefix[b] + (P->cu[b + 1] - P->cu[b]) > P->cap) return -4;
        }
        if (P->bt) {  /* every block the sequence touches must exist */
            const int64_t used = ((int64_t)P->prefix[b] + (P->cu[b + 1] - P->cu[b]) + PAGE - 1) / PAGE;
            for (int64_t i = 0; i < used; ++i) {
                const int32_t blk = P->bt[(int64_t)b * P->bt_stride + i];
                if (blk < 0 || blk >= P->num_blocks) return -7;
            }
        }
    }
    return 0;
}

/*
 * Varlen prefill: q, k, v are [N, H, D] bf16 bits (N = cu[B]); out is [N, H, D]
 * doubles; k_cache / v_cache hold the caller's buffer contents and receive the
 * cache image.  probs (optional, B == 1 only) receives [H, n, n] weights.
 * Returns 0, or a negative code for inconsistent metadata.
 */
int oracle_prefill_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          const int32_t *cu_seqlens, int32_t num_seqs,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, float scale,
                          double *out, uint16_t *k_cache, uint16_t *v_cache,
                          double *probs)
{
    problem_t P = {q, k, v, cu_seqlens, NULL, NULL, NULL,
                   num_seqs, num_heads, head_dim, 0, (double)scale, num_kv_heads};
    int rc = check_meta(&P);
    if (rc) return rc;
    if (probs && num_seqs != 1) return -5;
    if (run_all(&P, out, probs)) return -1;
    if (k_cache && v_cache) write_cache(&P, k_cache, v_cache);
    return 0;
}

/*
 * Chunked prefill (prompt chunks and length-1 decode rows in one batch):
 * sequence b has prefix_lens[b] tokens already in the cache [B, H, cap, D]
 * and cu[b+1]-cu[b] new tokens in q/k/v.  k_cache / v_cache are read for the
 * prefix and receive the image with the new tokens' K/V appended at
 * positions prefix_b .. prefix_b + len_b - 1.  probs (optional, B == 1)
 * receives [H, n, prefix + n].
 */
int oracle_prefill_chunked(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const int32_t *cu_seqlens, int32_t num_seqs,
                           int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t cache_capacity, const int32_t *prefix_lens,
                           float scale, double *out,
                           uint16_t *k_cache, uint16_t *v_cache, double *probs)
{
    problem_t P = {q, k, v, cu_seqlens, prefix_lens, k_cache, v_cache,
                   num_seqs, num_heads, head_dim, cache_capacity, (double)scale, num_kv_heads};
    int rc = check_meta(&P);
    if (rc) return rc;
    if (probs && num_seqs != 1) return -5;
    /* attention reads the prefix from the cache as it was before the call;
     * the new tokens' positions are written only afterwards, and they never
     * overlap the prefix region, so the order is immaterial. */
    if (run_all(&P, out, probs)) return -1;
    write_cache(&P, k_cache, v_cache);
    return 0;
}

/*
 * Sampled rows: the same definition evaluated only for the listed token
 * indices (all heads each), for parity checks at sizes where computing every
 * row would take too long.  out is [n_rows, H, D] doubles.  prefix_lens and
 * the caches may be NULL (varlen, no prefix).
 */
int oracle_prefill_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const int32_t *cu_seqlens, int32_t num_seqs,
                        int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t cache_capacity, const int32_t *prefix_lens,
                        const uint16_t *k_cache, const uint16_t *v_cache,
                        float scale, const int64_t *rows, int64_t n_rows,
                        double *out)
{
    problem_t P = {q, k, v, cu_seqlens, prefix_lens, k_cache, v_cache,
                   num_seqs, num_heads, head_dim, cache_capacity, (double)scale, num_kv_heads};
    int rc = check_meta(&P);
    if (rc) return rc;
    const int64_t H = num_heads, D = head_dim;
    const int64_t N = cu_seqlens[num_seqs];
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= N) return -6;
    const int64_t mk = max_keys(&P);
    int failed = 0;
#pragma omp parallel
    {
        const uint16_t **kp = malloc(sizeof(*kp) * (size_t)(mk > 0 ? mk : 1));
        const uint16_t **vp = malloc(sizeof(*vp) * (size_t)(mk > 0 ? mk : 1));
        double *s = malloc(sizeof(double) * (size_t)(mk > 0 ? mk : 1));
        if (!kp || !vp || !s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < n_rows * H; ++u) {
                const int64_t tok = rows[u / H];
                const int h = (int)(u % H);
                int b = 0;
                while (cu_seqlens[b + 1] <= tok) ++b; /* sequence holding tok */
                const int64_t i = tok - cu_seqlens[b];
                const int64_t pre = prefix_lens ? prefix_lens[b] : 0;
                gather_keys(&P, b, h, pre + i + 1, kp, vp);
                attend_row(q + (tok * H + h) * D, kp, vp, pre + i + 1, (int)D,
                           P.scale, out + ((u / H) * H + h) * D, NULL, s);
            }
        }
        free(kp);
        free(vp);
        free(s);
    }
    return failed ? -1 : 0;
}

/*
 * The cache image alone (no attention), for bit-exact cache checks at sizes
 * where computing every output row would take too long.  prefix_lens NULL
 * selects the varlen layout, otherwise the chunked [B, H, cap, D] layout;
 * same placement rule as write_cache above.
 */
int oracle_cache_image(const uint16_t *k, const uint16_t *v, const int32_t *cu_seqlens,
                       int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                       int32_t cache_capacity, const int32_t *prefix_lens,
                       uint16_t *k_cache, uint16_t *v_cache)
{
    /* only the K/V heads matter for the image */
    problem_t P = {NULL, k, v, cu_seqlens, prefix_lens, NULL, NULL,
                   num_seqs, num_kv_heads, head_dim, cache_capacity, 0.0, num_kv_heads};
    int rc = check_meta(&P);
    if (rc) return rc;
    write_cache(&P, k_cache, v_cache);
    return 0;
}

/*
 * INT8 rows for a quantised KV cache [P2 §4.3: only K and V are quantised,
 * Q keeps its precision; INT8 halves the cache; the scale may be per tensor,
 * per channel or per token, finer being more accurate].  The pages fix no
 * formula; the reading taken here is symmetric, one float32 scale per
 * (token, K/V head) row of D values:
 *     amax  = max_d |x_d|              (bf16 widened to float: exact)
 *     scale = amax / 127               (float32 division, round to nearest)
 *     code  = rint(x_d * (127 / amax)) (float32 division and product, ties
 *                                       to even), in [-127, 127]
 * and a row with amax < 2^-100 (127 / amax would leave float32's range for
 * the smallest bf16 values) is stored as scale 0 with all codes 0.  The
 * dequantised value is code * scale.  The integer decision is made in
 * float32 -- the precision of the kernel's epilogue -- with the same
 * operations, so codes and scales compare bit for bit.  x is rows * d bf16
 * values, row-major; codes rows * d, scales rows.
 */
int oracle_quantize_rows_int8(const uint16_t *x, int64_t rows, int32_t d,
                              int8_t *codes, float *scales)
{
    if (rows < 0 || d < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * d;
        float amax = 0.0f;
        for (int32_t i = 0; i < d; ++i) {
            const float a = fabsf((float)bf16_bits_to_double(xr[i]));
            if (a > amax) amax = a;
        }
        int8_t *cr = codes + r * d;
        if (!(amax >= 0x1p-100f)) {
            scales[r] = 0.0f;
            for (int32_t i = 0; i < d; ++i) cr[i] = 0;
            continue;
        }
        scales[r] = amax / 127.0f;
        const float inv = 127.0f / amax;
        for (int32_t i = 0; i < d; ++i) {
            float t = rintf((float)bf16_bits_to_double(xr[i]) * inv);
            if (t > 127.0f) t = 127.0f;
            if (t < -127.0f) t = -127.0f;
            cr[i] = (int8_t)t;
        }
    }
    return 0;
}

/*
 * FP8 rows for a quantised KV cache [P2 §4.3: K and V quantised, Q kept, one
 * scale per token among the granularities listed; FP8 halves the cache as
 * INT8 does].  The pages name no FP8 encoding; the reading taken here is the
 * OCP 8-bit E4M3 format ("e4m3fn"): a sign bit, 4 exponent bits with bias 7
 * and 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; there
 * are no infinities, S.1111.111 is NaN and the largest finite magnitude is
 * 1.75 * 2^8 = 448.  Symmetric, one float32 scale per (token, K/V head) row:
 *     amax  = max_d |x_d|
 *     scale = amax / 448                      (float32 division)
 *     code  = E4M3(x_d * (448 / amax))        (float32 division and product,
 *                                              then round to nearest E4M3
 *                                              value, ties to even)
 * A row with amax < 2^-100 gets scale 0 and codes of x_d * 0: zeros that keep
 * x_d's sign.  The dequantised value is decode(code) * scale.  The encoding
 * step is exact: the float32 product widens to double exactly, and the
 * rounding is done on integers of at most four bits.
 */
static uint8_t e4m3_rne(float xf)
{
    const uint8_t s = signbit(xf) ? 0x80 : 0x00;
    if (isnan(xf)) return s | 0x7f;
    const double a = fabs((double)xf);
    if (a == 0.0) return s;
    if (a < 0x1p-6) {                          /* subnormal: steps of 2^-9 */
        const double q = nearbyint(a * 512.0); /* ties to even; 8 = smallest normal */
        return s | (uint8_t)q;
    }
    int e;
    const double m = 2.0 * frexp(a, &e);       /* a = m * 2^(e-1), m in [1, 2) */
    e -= 1;
    double q = nearbyint((m - 1.0) * 8.0);     /* mantissa steps of 1/8, ties to even */
    if (q == 8.0) {
        e += 1;
        q = 0.0;
    }
    if (e > 8 || (e == 8 && q == 7.0)) return s | 0x7f; /* beyond 448: NaN */
    return s | (uint8_t)(((e + 7) << 3) | (int)q);
}

/* The value an E4M3 code stands for (NaN for S.1111.111). */
double oracle_e4m3_decode(uint8_t c)
{
    const double sgn = (c & 0x80) ? -1.0 : 1.0;
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) return sgn * ldexp((double)m, -9);
    return sgn * ldexp(1.0 + m / 8.0, e - 7);
}

uint8_t oracle_e4m3_encode(float x) { return e4m3_rne(x); }

int oracle_quantize_rows_fp8(const uint16_t *x, int64_t rows, int32_t d,
                             uint8_t *codes, float *scales)
{
    if (rows < 0 || d < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * d;
        float amax = 0.0f;
        for (int32_t i = 0; i < d; ++i) {
            const float a = fabsf((float)bf16_bits_to_double(xr[i]));
            if (a > amax) amax = a;
        }
        float inv = 0.0f;
        if (amax >= 0x1p-100f) {
            scales[r] = amax / 448.0f;
            inv = 448.0f / amax;
        } else {
            scales[r] = 0.0f;
        }
        uint8_t *cr = codes + r * d;
        for (int32_t i = 0; i < d; ++i) {
            const float t = (float)bf16_bits_to_double(xr[i]) * inv;
            cr[i] = e4m3_rne(t);
        }
    }
    return 0;
}

/*
 * Chunked prefill over a paged cache: as oracle_prefill_chunked, with the
 * prefix read from and the new tokens' K/V written to the blocks the block
 * table names (layout above).  k_cache / v_cache are [num_blocks, HK, 16, D];
 * block_table is [num_seqs, max_blocks_per_seq].  Blocks may be shared
 * between sequences (prefix sharing); new tokens must not land in a shared
 * block, as in any paged cache.
 */
int oracle_prefill_chunked_paged(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const int32_t *cu_seqlens, int32_t num_seqs,
                                 int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t num_blocks, const int32_t *block_table,
                                 int32_t max_blocks_per_seq, const int32_t *prefix_lens,
                                 float scale, double *out,
                                 uint16_t *k_cache, uint16_t *v_cache)
{
    if (!block_table || !prefix_lens || max_blocks_per_seq < 1 || num_blocks < 1) return -2;
    problem_t P = {q, k, v, cu_seqlens, prefix_lens, k_cache, v_cache,
                   num_seqs, num_heads, head_dim, max_blocks_per_seq * PAGE, (double)scale,
                   num_kv_heads, block_table, max_blocks_per_seq, num_blocks};
    int rc = check_meta(&P);
    if (rc) return rc;
    /* the prefix is read before any new token is written (positions differ) */
    if (run_all(&P, out, NULL)) return -1;
    write_cache(&P, k_cache, v_cache);
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
