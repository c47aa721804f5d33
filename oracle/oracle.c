/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for GPU-resident
 * scaled-dot-product attention: full-sequence prefill (optionally causal),
 * batched GQA decode against a preallocated KV cache, and the KV-cache append
 * scatter.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: it is used by tests/, by the smoke check and by the bench's
 * CPU-baseline leg.  It shares no code, header, table or helper with the HIP
 * library, and it is written from the definitions, not from the GPU algorithm:
 * no tiling, no online softmax, no split-KV.  Every score is formed, the full
 * row is max-subtracted, exponentiated, summed, and the weighted sum of V is
 * divided by that sum, all in double precision.  Inputs are the exact f32
 * values handed to the GPU; scale is the same f32 value widened to double.
 *
 * Sources (page title, then section):
 *  - trueno-gpu 0.4.11 src/memory/resident/attention.rs,
 *    `batched_multihead_attention`: output = softmax(Q K^T / sqrt(d_k)) V over
 *    interleaved [seq, n_heads * head_dim] activations, one head at a time.
 *  - trustformers-core 0.2.0 src/gpu_ops/cuda/oxicuda/attention.rs,
 *    `attention_prefill_gpu_to_gpu` (causal mask for a prefill with nothing
 *    cached: query i sees keys 0..=i), `softmax_causal_gpu_to_gpu` (masked cells are exactly
 *    zero) and the test helper `prefill_reference` (max-subtracted softmax,
 *    then (p / sum) * v).
 *  - trueno-gpu ..., `incremental_attention_gpu`: one query token per head
 *    against a head-first cache [heads, max_seq_len, head_dim]; an empty
 *    sequence yields zeros.
 *  - realizar 0.8.5 src/cuda/executor/cache_from_cache_from_kv_cache.rs,
 *    `init_kv_cache_gpu` (GQA cache [num_kv_heads, max_len, head_dim],
 *    num_kv_heads <= num_heads) and `init_batched_kv_cache_gpu` (batched cache
 *    [M, num_kv_heads, max_len, head_dim], per-sequence stride
 *    num_kv_heads * max_len * head_dim, 1 <= M <= 32).
 *  - trueno-gpu ..., `kv_cache_scatter_gpu`: position pos of an interleaved
 *    [n_heads * head_dim] row is written to cache[head, pos, :].
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes): GQA query head h reads KV head h / (H / Hkv) (contiguous groups);
 * prefill batch elements are independent with layout [B, S, H*d]; the decode
 * length L_m counts the keys attended (rows 0..L_m-1), L_m == 0 gives zeros;
 * scatter row r of sequence m lands at cache position cache_lens[m] + r.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared oracle.c -o liboracle.so -lm
 * (no -ffast-math: the IEEE semantics of exp and of the sums are relied on).
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One attention row, written out from the definition.
 * q: the query vector (d floats); keys/values: row j starts at
 * kbase + j * kstride (resp. vbase + j * vstride); n keys are visible.
 * out: d doubles.  scores: caller-provided scratch of n doubles. */
static void attend_row(const float *q, const float *kbase, int64_t kstride,
                       const float *vbase, int64_t vstride, int64_t n,
                       int64_t d, double scale, double *scores, double *out)
{
    int64_t j, l;
    double mu, z;
    if (n == 0) {
        for (l = 0; l < d; ++l) out[l] = 0.0;
        return;
    }
    /* s_j = scale * sum_l q[l] * k_j[l] */
    for (j = 0; j < n; ++j) {
        const float *kj = kbase + j * kstride;
        double dot = 0.0;
        for (l = 0; l < d; ++l) dot += (double)q[l] * (double)kj[l];
        scores[j] = scale * dot;
    }
    /* mu = max_j s_j ; e_j = exp(s_j - mu) ; Z = sum_j e_j */
    mu = scores[0];
    for (j = 1; j < n; ++j)
        if (scores[j] > mu) mu = scores[j];
    z = 0.0;
    for (j = 0; j < n; ++j) {
        scores[j] = exp(scores[j] - mu);
        z += scores[j];
    }
    /* out[l] = (sum_j e_j * v_j[l]) / Z */
    for (l = 0; l < d; ++l) {
        double acc = 0.0;
        for (j = 0; j < n; ++j) acc += scores[j] * (double)vbase[j * vstride + l];
        out[l] = acc / z;
    }
}

/* Full prefill.  q, k, v: [B, S, H*d] f32.  out: [B, S, H*d] f64.
 * causal != 0: query i sees keys 0..i; otherwise all S keys.
 * Returns 0, or -1 on a non-positive dimension / allocation failure. */
int oracle_prefill(const float *q, const float *k, const float *v, double *out,
                   int64_t B, int64_t S, int64_t H, int64_t d, float scale,
                   int causal)
{
    int64_t unit, n_units;
    int failed = 0;
    if (B <= 0 || S <= 0 || H <= 0 || d <= 0) return -1;
    n_units = B * H;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (unit = 0; unit < n_units; ++unit) {
        int64_t b = unit / H, h = unit % H, i;
        int64_t row = H * d; /* floats between consecutive tokens */
        double *scores = (double *)malloc(sizeof(double) * (size_t)S);
        if (!scores) { failed |= 1; continue; }
        for (i = 0; i < S; ++i) {
            const float *qi = q + (b * S + i) * row + h * d;
            int64_t n = causal ? i + 1 : S;
            attend_row(qi, k + b * S * row + h * d, row, v + b * S * row + h * d,
                       row, n, d, (double)scale, scores,
                       out + (b * S + i) * row + h * d);
        }
        free(scores);
    }
    return failed ? -1 : 0;
}

/* Selected prefill rows.  sel: n_sel triples (b, i, h).  out: n_sel x d f64,
 * row t holds O[b, i, h*d : (h+1)*d].  Same definition as oracle_prefill. */
int oracle_prefill_rows(const float *q, const float *k, const float *v,
                        const int64_t *sel, int64_t n_sel, double *out,
                        int64_t B, int64_t S, int64_t H, int64_t d, float scale,
                        int causal)
{
    int64_t t;
    int failed = 0;
    if (B <= 0 || S <= 0 || H <= 0 || d <= 0 || n_sel < 0) return -1;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (t = 0; t < n_sel; ++t) {
        int64_t b = sel[3 * t], i = sel[3 * t + 1], h = sel[3 * t + 2];
        int64_t row = H * d;
        double *scores;
        if (b < 0 || b >= B || i < 0 || i >= S || h < 0 || h >= H) { failed |= 1; continue; }
        scores = (double *)malloc(sizeof(double) * (size_t)S);
        if (!scores) { failed |= 1; continue; }
        attend_row(q + (b * S + i) * row + h * d, k + b * S * row + h * d, row,
                   v + b * S * row + h * d, row, causal ? i + 1 : S, d,
                   (double)scale, scores, out + t * d);
        free(scores);
    }
    return failed ? -1 : 0;
}

/* Batched GQA decode.  q: [M, H*d] (one token per sequence).  k_cache,
 * v_cache: [M, Hkv, max_len, d].  lens: M keys-attended counts, each in
 * [0, max_len].  out: [M, H*d] f64.  Only rows j < lens[m] are read. */
int oracle_decode(const float *q, const float *k_cache, const float *v_cache,
                  const int32_t *lens, double *out, int64_t M, int64_t H,
                  int64_t Hkv, int64_t d, int64_t max_len, float scale)
{
    int64_t unit, n_units, m;
    int failed = 0;
    if (M <= 0 || H <= 0 || Hkv <= 0 || d <= 0 || max_len <= 0) return -1;
    if (H % Hkv != 0) return -1;
    for (m = 0; m < M; ++m)
        if (lens[m] < 0 || lens[m] > max_len) return -1;
    n_units = M * H;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (unit = 0; unit < n_units; ++unit) {
        int64_t mm = unit / H, h = unit % H;
        int64_t group = H / Hkv;     /* query heads per KV head */
        int64_t kh = h / group;      /* contiguous-group GQA map */
        int64_t off = (mm * Hkv + kh) * max_len * d;
        double *scores = (double *)malloc(sizeof(double) * (size_t)max_len);
        if (!scores) { failed |= 1; continue; }
        attend_row(q + mm * H * d + h * d, k_cache + off, d, v_cache + off, d,
                   lens[mm], d, (double)scale, scores, out + mm * H * d + h * d);
        free(scores);
    }
    return failed ? -1 : 0;
}

/* Selected decode outputs.  sel: n_sel pairs (m, h); out: n_sel x d f64. */
int oracle_decode_rows(const float *q, const float *k_cache, const float *v_cache,
                       const int32_t *lens, const int64_t *sel, int64_t n_sel,
                       double *out, int64_t M, int64_t H, int64_t Hkv, int64_t d,
                       int64_t max_len, float scale)
{
    int64_t t;
    int failed = 0;
    if (M <= 0 || H <= 0 || Hkv <= 0 || d <= 0 || max_len <= 0 || n_sel < 0) return -1;
    if (H % Hkv != 0) return -1;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (t = 0; t < n_sel; ++t) {
        int64_t mm = sel[2 * t], h = sel[2 * t + 1];
        int64_t kh, off;
        double *scores;
        if (mm < 0 || mm >= M || h < 0 || h >= H) { failed |= 1; continue; }
        if (lens[mm] < 0 || lens[mm] > max_len) { failed |= 1; continue; }
        kh = h / (H / Hkv);
        off = (mm * Hkv + kh) * max_len * d;
        scores = (double *)malloc(sizeof(double) * (size_t)max_len);
        if (!scores) { failed |= 1; continue; }
        attend_row(q + mm * H * d + h * d, k_cache + off, d, v_cache + off, d,
                   lens[mm], d, (double)scale, scores, out + t * d);
        free(scores);
    }
    return failed ? -1 : 0;
}

/* KV-cache append.  k_new, v_new: [M, n_new, Hkv*d] interleaved rows.
 * k_cache, v_cache: [M, Hkv, max_len, d].  Row r of sequence m, KV head kh,
 * is copied bit for bit to cache position cache_lens[m] + r.  Every other
 * cache element is left as it was.  Returns -1 (and writes nothing) when a
 * write would fall outside [0, max_len). */
int oracle_scatter(const float *k_new, const float *v_new, float *k_cache,
                   float *v_cache, const int32_t *cache_lens, int64_t M,
                   int64_t n_new, int64_t Hkv, int64_t d, int64_t max_len)
{
    int64_t m, r, kh, l;
    if (M <= 0 || n_new <= 0 || Hkv <= 0 || d <= 0 || max_len <= 0) return -1;
    for (m = 0; m < M; ++m)
        if (cache_lens[m] < 0 || (int64_t)cache_lens[m] + n_new > max_len) return -1;
    for (m = 0; m < M; ++m)
        for (r = 0; r < n_new; ++r)
            for (kh = 0; kh < Hkv; ++kh) {
                int64_t src = (m * n_new + r) * Hkv * d + kh * d;
                int64_t dst = ((m * Hkv + kh) * max_len + cache_lens[m] + r) * d;
                for (l = 0; l < d; ++l) {
                    uint32_t bits;
                    memcpy(&bits, &k_new[src + l], 4);
                    memcpy(&k_cache[dst + l], &bits, 4);
                    memcpy(&bits, &v_new[src + l], 4);
                    memcpy(&v_cache[dst + l], &bits, 4);
                }
            }
    return 0;
}

/* Copy of a prefilled single-sequence cache into slot `slot` of the batched
 * cache (realizar 0.8.5 ..., `scatter_single_kv_to_batched`: once a prefill has
 * filled the single cache, its rows go to the batched cache at the slot's
 * offset slot * Hkv * max_len * d and the slot's length becomes seq_len; a
 * seq_len of 0 changes nothing).  The single cache is [Hkv, src_max_len, d]
 * (`init_kv_cache_gpu`), the batched one [M, Hkv, max_len, d]
 * (`init_batched_kv_cache_gpu`).  For every KV head kh, rows 0 .. seq_len-1 of
 * head kh are copied bit for bit to rows 0 .. seq_len-1 of head kh of the slot,
 * so that decoding the slot sees exactly what decoding the single cache saw.
 * Returns -1 (nothing written) on invalid sizes. */
int oracle_copy_to_slot(const float *src_k, const float *src_v, int64_t src_max_len,
                        int64_t seq_len, float *dst_k, float *dst_v, int64_t slot, int64_t M,
                        int64_t Hkv, int64_t d, int64_t max_len)
{
    int64_t kh, r, l;
    if (M <= 0 || Hkv <= 0 || d <= 0 || max_len <= 0 || src_max_len <= 0) return -1;
    if (slot < 0 || slot >= M || seq_len < 0 || seq_len > src_max_len || seq_len > max_len) return -1;
    for (kh = 0; kh < Hkv; ++kh)
        for (r = 0; r < seq_len; ++r) {
            int64_t s = (kh * src_max_len + r) * d;
            int64_t t = ((slot * Hkv + kh) * max_len + r) * d;
            for (l = 0; l < d; ++l) {
                uint32_t bits;
                memcpy(&bits, &src_k[s + l], 4);
                memcpy(&dst_k[t + l], &bits, 4);
                memcpy(&bits, &src_v[s + l], 4);
                memcpy(&dst_v[t + l], &bits, 4);
            }
        }
    return 0;
}

/* Chunked prefill behind an existing cache (the offset causal mask:
 * trustformers-core 0.2.0 ..., `attention_prefill_gpu_to_gpu` leaves a prefill
 * that follows cached tokens to the per-token decode path; this is that case in
 * one call).  Sequence m holds cache_lens[m] = P rows already; its n_new new
 * tokens sit at absolute positions P .. P+n_new-1.  Query r (position P + r)
 * of head h attends to keys 0 .. P + r of KV head h / (H/Hkv), where key j is
 * cache row j when j < P and new row j - P otherwise.
 *   q: [M, n_new, H*d]; k_new, v_new: [M, n_new, Hkv*d];
 *   k_cache, v_cache: [M, Hkv, max_len, d] (only rows < P are read);
 *   out: [M, n_new, H*d] f64.
 * The keys of one (m, kh) are gathered into a contiguous scratch first, so the
 * row function above applies unchanged. */
int oracle_prefill_cached(const float *q, const float *k_new, const float *v_new,
                          const float *k_cache, const float *v_cache,
                          const int32_t *cache_lens, double *out, int64_t M,
                          int64_t n_new, int64_t H, int64_t Hkv, int64_t d,
                          int64_t max_len, float scale)
{
    int64_t unit, n_units, m;
    int failed = 0;
    if (M <= 0 || n_new <= 0 || H <= 0 || Hkv <= 0 || d <= 0 || max_len <= 0) return -1;
    if (H % Hkv != 0) return -1;
    for (m = 0; m < M; ++m)
        if (cache_lens[m] < 0 || (int64_t)cache_lens[m] + n_new > max_len) return -1;
    n_units = M * H;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (unit = 0; unit < n_units; ++unit) {
        int64_t mm = unit / H, h = unit % H, kh = h / (H / Hkv), r, j, l;
        int64_t P = cache_lens[mm], total = P + n_new;
        float *keys = (float *)malloc(sizeof(float) * (size_t)(total * d));
        float *vals = (float *)malloc(sizeof(float) * (size_t)(total * d));
        double *scores = (double *)malloc(sizeof(double) * (size_t)total);
        if (!keys || !vals || !scores) {
            free(keys); free(vals); free(scores);
            failed |= 1;
            continue;
        }
        for (j = 0; j < total; ++j)
            for (l = 0; l < d; ++l) {
                if (j < P) {
                    int64_t c = ((mm * Hkv + kh) * max_len + j) * d + l;
                    keys[j * d + l] = k_cache[c];
                    vals[j * d + l] = v_cache[c];
                } else {
                    int64_t c = (mm * n_new + (j - P)) * Hkv * d + kh * d + l;
                    keys[j * d + l] = k_new[c];
                    vals[j * d + l] = v_new[c];
                }
            }
        for (r = 0; r < n_new; ++r)
            attend_row(q + (mm * n_new + r) * H * d + h * d, keys, d, vals, d, P + r + 1, d,
                       (double)scale, scores, out + (mm * n_new + r) * H * d + h * d);
        free(keys);
        free(vals);
        free(scores);
    }
    return failed ? -1 : 0;
}

/* Selected rows of oracle_prefill_cached.  sel: n_sel triples (m, r, h);
 * out: n_sel x d f64, row t = out[m, r, h*d : (h+1)*d] of the full call. */
int oracle_prefill_cached_rows(const float *q, const float *k_new, const float *v_new,
                               const float *k_cache, const float *v_cache,
                               const int32_t *cache_lens, const int64_t *sel, int64_t n_sel,
                               double *out, int64_t M, int64_t n_new, int64_t H, int64_t Hkv,
                               int64_t d, int64_t max_len, float scale)
{
    int64_t t, m;
    int failed = 0;
    if (M <= 0 || n_new <= 0 || H <= 0 || Hkv <= 0 || d <= 0 || max_len <= 0 || n_sel < 0) return -1;
    if (H % Hkv != 0) return -1;
    for (m = 0; m < M; ++m)
        if (cache_lens[m] < 0 || (int64_t)cache_lens[m] + n_new > max_len) return -1;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (t = 0; t < n_sel; ++t) {
        int64_t mm = sel[3 * t], r = sel[3 * t + 1], h = sel[3 * t + 2], kh, P, n, j, l;
        float *keys, *vals;
        double *scores;
        if (mm < 0 || mm >= M || r < 0 || r >= n_new || h < 0 || h >= H) { failed |= 1; continue; }
        kh = h / (H / Hkv);
        P = cache_lens[mm];
        n = P + r + 1; /* keys visible to this query */
        keys = (float *)malloc(sizeof(float) * (size_t)(n * d));
        vals = (float *)malloc(sizeof(float) * (size_t)(n * d));
        scores = (double *)malloc(sizeof(double) * (size_t)n);
        if (!keys || !vals || !scores) {
            free(keys); free(vals); free(scores);
            failed |= 1;
            continue;
        }
        for (j = 0; j < n; ++j)
            for (l = 0; l < d; ++l) {
                int64_t c = j < P ? ((mm * Hkv + kh) * max_len + j) * d + l
                                  : (mm * n_new + (j - P)) * Hkv * d + kh * d + l;
                keys[j * d + l] = j < P ? k_cache[c] : k_new[c];
                vals[j * d + l] = j < P ? v_cache[c] : v_new[c];
            }
        attend_row(q + (mm * n_new + r) * H * d + h * d, keys, d, vals, d, n, d, (double)scale, scores,
                   out + t * d);
        free(keys);
        free(vals);
        free(scores);
    }
    return failed ? -1 : 0;
}

/* Rotary position embedding, GPT-NeoX half-split convention (trustformers-core
 * 0.2.0 ..., `rope_neox_gpu_to_gpu`; realizar 0.8.5 ..., `apply_rope_to_buffer`,
 * the rotary_ndims = head_dim case with base = rope theta), written from what
 * the rotation is.  With half = rotary_ndims / 2, dims k and k + half of a head
 * form one complex number z_k = x_k + i x_{k+half}.  At position p the
 * embedding turns z_k through the angle p * base^(-2k / rotary_ndims), i.e.
 * multiplies it by the unit complex number of that angle, and leaves every
 * dim >= rotary_ndims as it is.  x: n_rows rows of H heads of d floats, row t
 * at absolute position pos[t].  out: same shape, f64. */
int oracle_rope(const float *x, const int32_t *pos, double *out, int64_t n_rows, int64_t H,
                int64_t d, int64_t rotary_ndims, double base)
{
    int64_t t;
    if (n_rows < 0 || H <= 0 || d <= 0 || rotary_ndims < 0 || rotary_ndims > d || rotary_ndims % 2) return -1;
    if (!(base > 0.0)) return -1;
#pragma omp parallel for schedule(static)
    for (t = 0; t < n_rows; ++t) {
        const int64_t half = rotary_ndims / 2;
        int64_t h, k, l;
        for (h = 0; h < H; ++h) {
            const float *src = x + (t * H + h) * d;
            double *dst = out + (t * H + h) * d;
            for (k = 0; k < half; ++k) {
                double a = (double)pos[t] * pow(base, -2.0 * (double)k / (double)rotary_ndims);
                double complex turn = cexp(I * a);
                double complex z = (double)src[k] + I * (double)src[k + half];
                z = z * turn;
                dst[k] = creal(z);
                dst[k + half] = cimag(z);
            }
            for (l = rotary_ndims; l < d; ++l) dst[l] = (double)src[l];
        }
    }
    return 0;
}

/* Rounding of an f32 value to a 16-bit floating-point format, round to
 * nearest, ties to even (IEEE 754 binary16, or bfloat16: the f32 exponent
 * range with 8 significant bits).  The reduced-precision prefill (trueno-gpu
 * 0.4.11 ..., `batched_gemm`: the GEMM operands go through fp16 tensor cores
 * when k >= 64) computes attention of the inputs rounded this way.
 * fmt 1 = binary16 (11 significant bits, normal exponents >= -14, largest
 * finite 65504), fmt 2 = bfloat16 (8 bits, >= -126, largest (2 - 2^-7) 2^127).
 * Written from the definition: find the spacing of representable numbers at
 * x (the subnormal spacing below the smallest normal), round x / spacing to
 * the nearest integer (ties to even: nearbyint in the default rounding mode),
 * and overflow to infinity past the largest finite value. */
static double round_sig(double x, int p, int emin, double maxv)
{
    int e;
    double q, r;
    if (x == 0.0 || !isfinite(x)) return x;
    frexp(x, &e); /* |x| = m 2^e, 1/2 <= m < 1: leading bit at 2^(e-1) */
    e -= 1;
    if (e < emin) e = emin;
    q = ldexp(1.0, e - (p - 1));
    r = nearbyint(x / q) * q;
    if (fabs(r) > maxv) return copysign(INFINITY, x);
    return r;
}

int oracle_round16(const float *x, float *y, int64_t n, int fmt)
{
    int64_t i;
    int p, emin;
    double maxv;
    if (fmt == 1) {
        p = 11; emin = -14; maxv = 65504.0;
    } else if (fmt == 2) {
        p = 8; emin = -126; maxv = ldexp(2.0 - ldexp(1.0, -7), 127);
    } else {
        return -1;
    }
    for (i = 0; i < n; ++i) y[i] = (float)round_sig((double)x[i], p, emin, maxv);
    return 0;
}

/* Reduced-precision prefill: oracle_prefill of q, k and v each rounded to the
 * 16-bit format `fmt` (the products of 16-bit operands are exact in the
 * wider accumulation; what the device's own rounding of the probabilities adds
 * is bounded in the tests, not modelled here). */
int oracle_prefill_lowp(const float *q, const float *k, const float *v, double *out, int64_t B,
                        int64_t S, int64_t H, int64_t d, float scale, int causal, int fmt)
{
    int64_t n = B * S * H * d;
    float *rq, *rk, *rv;
    int rc = -1;
    if (n <= 0) return -1;
    rq = (float *)malloc((size_t)n * sizeof(float));
    rk = (float *)malloc((size_t)n * sizeof(float));
    rv = (float *)malloc((size_t)n * sizeof(float));
    if (rq && rk && rv && oracle_round16(q, rq, n, fmt) == 0 && oracle_round16(k, rk, n, fmt) == 0 &&
        oracle_round16(v, rv, n, fmt) == 0)
        rc = oracle_prefill(rq, rk, rv, out, B, S, H, d, scale, causal);
    free(rq);
    free(rk);
    free(rv);
    return rc;
}

/* Threads for the following parallel regions (timing only: results do not
   depend on it, every output element is computed by one thread in the same
   order).  n <= 0 leaves the setting as it is. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/* A chunk behind a cache with a GPT-NeoX rotary embedding: the rotation of
 * trustformers-core 0.2.0 ..., `rope_neox_gpu_to_gpu` applied at the absolute
 * position of each new token, composed with the chunked prefill above.  Query
 * row r and new key row r of sequence m are rotated (oracle_rope) to position
 * cache_lens[m] + r and handed over as f32, the precision in which the cache
 * keeps rotated keys; values are not rotated; cached rows 0 .. cache_lens[m]-1
 * are taken as they are (already rotated when they were appended).  Then
 * oracle_prefill_cached.  out as there. */
int oracle_prefill_cached_rope(const float *q, const float *k_new, const float *v_new,
                               const float *k_cache, const float *v_cache,
                               const int32_t *cache_lens, double *out, int64_t M,
                               int64_t n_new, int64_t H, int64_t Hkv, int64_t d,
                               int64_t max_len, float scale, int64_t rotary_ndims,
                               double base)
{
    int64_t m, r, i;
    const int64_t nq = M * n_new * H * d, nk = M * n_new * Hkv * d;
    int rc = -1;
    int32_t *pos;
    double *qr, *kr;
    float *qf, *kf;
    if (M <= 0 || n_new <= 0 || H <= 0 || Hkv <= 0 || d <= 0) return -1;
    pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * n_new));
    qr = (double *)malloc(sizeof(double) * (size_t)nq);
    kr = (double *)malloc(sizeof(double) * (size_t)nk);
    qf = (float *)malloc(sizeof(float) * (size_t)nq);
    kf = (float *)malloc(sizeof(float) * (size_t)nk);
    if (!pos || !qr || !kr || !qf || !kf) goto done;
    for (m = 0; m < M; ++m)
        for (r = 0; r < n_new; ++r) pos[m * n_new + r] = cache_lens[m] + (int32_t)r;
    if (oracle_rope(q, pos, qr, M * n_new, H, d, rotary_ndims, base) != 0) goto done;
    if (oracle_rope(k_new, pos, kr, M * n_new, Hkv, d, rotary_ndims, base) != 0) goto done;
    for (i = 0; i < nq; ++i) qf[i] = (float)qr[i];
    for (i = 0; i < nk; ++i) kf[i] = (float)kr[i];
    rc = oracle_prefill_cached(qf, kf, v_new, k_cache, v_cache, cache_lens, out, M, n_new, H, Hkv, d,
                               max_len, scale);
done:
    free(pos);
    free(qr);
    free(kr);
    free(qf);
    free(kf);
    return rc;
}
