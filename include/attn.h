/*
 * attn.h -- C ABI of libattn.so: GPU-resident scaled-dot-product attention
 * for AMD Instinct MI355X (gfx950).
 *
 *   out = softmax(scale * Q K^T [+ causal mask]) V
 *
 * Four operations, each enqueued on a caller-supplied HIP stream:
 *   attn_prefill             full-sequence attention over interleaved
 *                            [batch, seq, n_heads * head_dim] activations,
 *                            optionally causal (attn_prefill_lowp: the same
 *                            on 16-bit fp16 / bf16 matrix-core operands);
 *   attn_decode_gqa_batched  one query token per sequence for up to 32
 *                            sequences against a preallocated GQA KV cache,
 *                            each sequence with its own length;
 *   kv_cache_scatter         append rows of new keys/values into that cache
 *                            at each sequence's current length;
 *   attn_prefill_cached      a chunk of new tokens behind an existing cache:
 *                            append, then attend with the causal mask offset
 *                            by each sequence's cached length.
 * The append, the decode and the chunked prefill also come with a rotary
 * position embedding fused in (kv_cache_scatter_rope,
 * attn_decode_gqa_batched_rope, attn_prefill_cached_rope); a prefilled
 * single-sequence cache can be copied into a batch slot
 * (kv_cache_copy_to_slot), and the host length arrays reset or rolled back.
 *
 * Conventions shared by every entry point
 *   - Tensors are f32, row-major, contiguous, in DEVICE memory owned by the
 *     caller.  The library allocates nothing, keeps no per-call state and is
 *     safe to call from several host threads (attn_decode_gqa_batched_noalloc
 *     alone uses memory of the library's own: see there).  Pointers marked HOST are read
 *     synchronously during the call and may be reused on return.
 *   - Device pointers must be 16-byte aligned (128-bit accesses).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued and
 *     the call returns without synchronising; the caller orders later work on
 *     the same stream.
 *   - Every argument is validated on the host before anything is enqueued.  A
 *     non-zero return therefore means nothing was queued and every output is
 *     untouched.  The only exception is ATTN_ERR_HIP, returned when the HIP
 *     runtime rejects a launch (work may then have been partly queued).
 *   - Outputs must not overlap inputs (ATTN_ERR_ALIAS).
 *
 * Sources (page title, then section): trueno-gpu 0.4.11
 * src/memory/resident/attention.rs (`batched_multihead_attention`, `batched_gemm`,
 * `incremental_attention_gpu_with_stream`, `kv_cache_scatter_gpu`);
 * trustformers-core 0.2.0 src/gpu_ops/cuda/oxicuda/attention.rs
 * (`attention_prefill_gpu_to_gpu`, `attention_decode_gpu_to_gpu`,
 * `checked_len`, `rope_neox_gpu_to_gpu`, `rope_reference`); realizar 0.8.5
 * src/cuda/executor/cache_from_cache_from_kv_cache.rs (`init_kv_cache_gpu`,
 * `init_batched_kv_cache_gpu`).
 */
#ifndef TRANSFORMER_ATTENTION_FLASH_AMD_ATTN_H
#define TRANSFORMER_ATTENTION_FLASH_AMD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbol visibility; exactly the functions
 * declared here are exported. */
#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility push(default)
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
    ATTN_ERR_INVALID_DIM = 2, /* a size, length or position is out of range */
    ATTN_ERR_UNSUPPORTED = 3, /* head_dim not in {32, 64, 128}, or a pointer not 16-byte aligned */
    ATTN_ERR_OVERFLOW = 4,    /* a size product does not fit the index types used */
    ATTN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than attn_decode_workspace_bytes() */
    ATTN_ERR_HIP = 6,         /* the HIP runtime reported an error for a launch */
    ATTN_ERR_ALIAS = 7        /* an output buffer overlaps an input buffer */
} attn_status;

/* Operand formats of attn_prefill_lowp. */
typedef enum {
    ATTN_PREC_FP16 = 1, /* IEEE binary16: 11 significant bits, largest finite 65504 */
    ATTN_PREC_BF16 = 2  /* bfloat16: 8 significant bits, the f32 exponent range */
} attn_precision;

/* Largest number of sequences a decode or scatter call takes (the batched
 * cache holds 1..32 sequences: realizar `init_batched_kv_cache_gpu`). */
#define ATTN_MAX_SEQS 32

/*
 * Full-sequence multi-head attention (prefill).
 *
 * Defines: trueno-gpu `batched_multihead_attention` (softmax(Q K^T/sqrt(d_k)) V
 * per head over interleaved [seq, n_heads * head_dim]) and trustformers-core
 * `attention_prefill_gpu_to_gpu` (caller-chosen scale; the causal mask assumes
 * nothing is cached yet, so query i sees keys 0..=i; masked probabilities are
 * exactly 0).
 * Batch elements are independent.
 *
 *   q, k, v  [batch, seq_len, n_heads * head_dim]  read
 *   out      [batch, seq_len, n_heads * head_dim]  written, every element
 *   out[b, i, h*d + l] = sum_j p_ij v[b, j, h*d + l],
 *   p_ij = exp(s_ij - max_j s_ij) / sum_j exp(...),
 *   s_ij = scale * sum_l q[b, i, h*d + l] k[b, j, h*d + l] over visible j.
 *   scale    usually 1/sqrtf(head_dim); any finite value is accepted.
 *   causal   0: every query sees all seq_len keys; 1: query i sees 0..i.
 *
 * Errors: NULL pointer; batch, seq_len, n_heads <= 0 or causal not 0/1
 * (INVALID_DIM); head_dim not in {32, 64, 128} or misaligned (UNSUPPORTED);
 * batch*seq_len*n_heads*head_dim >= 2^31 (OVERFLOW); scale not finite
 * (INVALID_DIM); out overlapping q, k or v (ALIAS).
 */
int attn_prefill(const float *q, const float *k, const float *v, float *out,
                 int32_t batch, int32_t seq_len, int32_t n_heads, int32_t head_dim,
                 float scale, int32_t causal, void *stream);

/*
 * Reduced-precision full-sequence attention: attn_prefill with both products
 * on 16-bit matrix-core operands.
 *
 * Defines: trueno-gpu `batched_gemm`, which runs the attention GEMMs on fp16
 * tensor-core operands once k >= 64 (WMMA, wider accumulation).  Here q, k and
 * v are rounded to `precision` (nearest, ties to even) as they are read; the
 * scores accumulate in f32 (the product of two 16-bit values is exact in f32);
 * the softmax runs in f32; the probabilities are rounded to `precision` as the
 * operand of the P.V product, which accumulates in f32; the running sums and
 * the final normalisation use the f32 probabilities.  Inputs and output stay
 * f32 in memory, with the layout, arguments and errors of attn_prefill.
 *   precision  ATTN_PREC_FP16 or ATTN_PREC_BF16 (anything else: UNSUPPORTED)
 * Accuracy: against the exact attention of the rounded inputs, an output
 * element is off by at most about u * max|v| (u = 2^-11 for fp16, 2^-8 for
 * bf16: the rounding of the probabilities) plus f32 rounding; inputs must fit
 * the format (|x| <= 65504 for fp16, else they round to infinity).
 */
int attn_prefill_lowp(const float *q, const float *k, const float *v, float *out,
                      int32_t batch, int32_t seq_len, int32_t n_heads, int32_t head_dim,
                      float scale, int32_t causal, int32_t precision, void *stream);

/*
 * Chunked prefill behind an existing KV cache: append the keys and values of a
 * chunk of n_new tokens to each sequence's cache and attend the chunk's queries
 * causally over everything cached so far.
 *
 * Defines: trustformers-core `attention_prefill_gpu_to_gpu` restricts its causal
 * mask to a prefill with nothing cached and sends a prefill that follows cached
 * tokens to the decode path one token at a time; this entry point covers that
 * case in one call.  Sequence m
 * holds P = cache_lens[m] rows; its new tokens sit at positions P .. P+n_new-1,
 * and query r (position P + r) of head h sees keys 0 .. P + r of KV head
 * h / (num_heads / num_kv_heads), laid out as realizar `init_batched_kv_cache_gpu`.
 *
 *   q                 [M, n_new, num_heads * head_dim]       read
 *   k_new, v_new      [M, n_new, num_kv_heads * head_dim]    read
 *   k_cache, v_cache  [M, num_kv_heads, max_len, head_dim]   rows P .. P+n_new-1
 *                     written exactly as kv_cache_scatter would; rows < P read
 *   cache_lens        HOST [M] int32, P per sequence (not updated: lengths are
 *                     caller state; the new length is P + n_new)
 *   out               [M, n_new, num_heads * head_dim]       written, every element
 *   With cache_lens all 0 and num_kv_heads == num_heads this equals
 *   kv_cache_scatter followed by attn_prefill(causal = 1); with n_new == 1 it
 *   equals kv_cache_scatter followed by attn_decode_gqa_batched with
 *   seq_lens = P + 1.
 *
 * Errors: NULL pointer; M not in [1, 32], n_new/num_heads/num_kv_heads/max_len
 * <= 0, num_heads % num_kv_heads != 0, num_kv_heads > num_heads, a cache_lens
 * value < 0 or cache_lens[m] + n_new > max_len, scale not finite
 * (INVALID_DIM); head_dim not in {32, 64, 128} or a misaligned pointer
 * (UNSUPPORTED); M*n_new*num_heads*head_dim >= 2^31 or a cache element count
 * >= 2^40 (OVERFLOW); out or a cache overlapping an input, or the caches
 * overlapping each other or out (ALIAS).  Two launches (append, attention)
 * are enqueued on `stream`.
 */
int attn_prefill_cached(const float *q, const float *k_new, const float *v_new, float *k_cache,
                        float *v_cache, const int32_t *cache_lens, float *out, int32_t num_seqs,
                        int32_t n_new, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t max_len, float scale, void *stream);

/*
 * attn_prefill_cached with a GPT-NeoX rotary position embedding fused in: the
 * chunk's keys are appended rotated to their cache rows P + r (exactly as
 * kv_cache_scatter_rope writes them), and query r is rotated to the same
 * position P + r before it is scored against the cache, whose rows < P are
 * taken as already rotated (written by earlier rotary appends).
 *
 * Defines: trustformers-core `rope_neox_gpu_to_gpu` (the rotation applied at
 * an absolute position offset: dim i < rotary_ndims / 2 paired with
 * i + rotary_ndims / 2, angle pos * rope_theta^(-2i / rotary_ndims), dims at or
 * past rotary_ndims unchanged) composed with `attention_prefill_gpu_to_gpu`'s
 * causal attention, for the prefill behind a cache that page leaves to the
 * decode path.
 *
 *   arguments as attn_prefill_cached, plus
 *   rotary_ndims      0 (no rotation: identical to attn_prefill_cached) or a
 *                     multiple of 8 up to head_dim
 *   rope_theta        rotary base, finite and > 0
 *   With n_new == 1 this equals kv_cache_scatter_rope followed by
 *   attn_decode_gqa_batched_rope with seq_lens = P + 1.
 *
 * Errors: those of attn_prefill_cached; rotary_ndims < 0 or > head_dim,
 * rope_theta not finite or <= 0 (INVALID_DIM); rotary_ndims not a multiple
 * of 8 (UNSUPPORTED).
 */
int attn_prefill_cached_rope(const float *q, const float *k_new, const float *v_new, float *k_cache,
                             float *v_cache, const int32_t *cache_lens, float *out, int32_t num_seqs,
                             int32_t n_new, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_len, float scale, int32_t rotary_ndims, float rope_theta,
                             void *stream);

/*
 * Bytes of device workspace attn_decode_gqa_batched needs for these sizes
 * (per-split partial maxima, sums and unnormalised outputs).  Returns 0 when
 * the sizes are invalid or max_len > 2^30.  Pure host arithmetic; no HIP call.
 */
size_t attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                   int32_t max_len);

/*
 * Batched grouped-query decode attention: one new query token per sequence.
 *
 * Defines: trueno-gpu `incremental_attention_gpu_with_stream` (one query per
 * head against a head-first cache, empty sequence -> zeros, caller's stream,
 * no sync) generalised to GQA and to M sequences as laid out by realizar
 * `init_kv_cache_gpu` / `init_batched_kv_cache_gpu`.  Query head h reads KV
 * head h / (num_heads / num_kv_heads) (contiguous groups).
 *
 *   q          [M, num_heads * head_dim]                       read
 *   k_cache    [M, num_kv_heads, max_len, head_dim]             read, rows < seq_lens[m] only
 *   v_cache    [M, num_kv_heads, max_len, head_dim]             read, rows < seq_lens[m] only
 *   seq_lens   HOST [M] int32, keys attended by sequence m, 0 <= L <= max_len;
 *              L = 0 gives zeros for that sequence
 *   out        [M, num_heads * head_dim]                        written, every element
 *   workspace  device scratch of >= attn_decode_workspace_bytes(M, num_heads,
 *              head_dim, max_len) bytes, 16-byte aligned, owned by the caller,
 *              contents on entry irrelevant; must not be used by other work
 *              that can run concurrently with this call.
 *
 * Errors: NULL pointer; M not in [1, 32], num_heads/num_kv_heads/max_len <= 0,
 * num_kv_heads > num_heads, num_heads % num_kv_heads != 0, a seq_lens value
 * outside [0, max_len], scale not finite (INVALID_DIM); head_dim not in
 * {32, 64, 128} or misaligned pointer (UNSUPPORTED); max_len > 2^30 or an
 * element count >= 2^40 (OVERFLOW); workspace too small (WORKSPACE); out
 * overlapping an input or the workspace (ALIAS).
 */
int attn_decode_gqa_batched(const float *q, const float *k_cache, const float *v_cache,
                            const int32_t *seq_lens, float *out, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_len, float scale, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Bytes of device scratch built into the library for
 * attn_decode_gqa_batched_noalloc (one such array per GPU it runs on). */
#define ATTN_DECODE_SCRATCH_BYTES (64u << 20)

/*
 * attn_decode_gqa_batched without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, results and
 * errors as attn_decode_gqa_batched otherwise, bit for bit (the same kernels).
 *
 * The per-split partials go to a scratch array of ATTN_DECODE_SCRATCH_BYTES
 * that the library holds on every GPU it runs on, from the first call on that
 * GPU until the process ends.  Sizes whose attn_decode_workspace_bytes()
 * exceeds it are refused with ATTN_ERR_WORKSPACE (64 MiB covers any
 * max_len with num_seqs * num_heads <= 2016 at head_dim 128; the long-context
 * M = 16, 64-head decode needs 34 MB).  Nothing is allocated or freed: the
 * first call on a GPU looks the array's address up (ATTN_ERR_HIP if that
 * fails); no call clears it, as every value the decode reads from it is
 * written earlier in the same call.  All calls on one GPU share the array:
 * calls that can overlap on one GPU (concurrent streams, several host threads)
 * race on it and must be ordered by the caller.  The array's GPU is the one
 * that runs `stream`.
 */
int attn_decode_gqa_batched_noalloc(const float *q, const float *k_cache, const float *v_cache,
                                    const int32_t *seq_lens, float *out, int32_t num_seqs,
                                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_len, float scale, void *stream);

/*
 * KV-cache append (scatter).
 *
 * Defines: trueno-gpu `kv_cache_scatter_gpu` (an interleaved [n_heads *
 * head_dim] row goes to cache[head, pos, :]; pos must be < max_seq_len)
 * generalised to n_new rows and M sequences of the batched cache (realizar
 * `init_batched_kv_cache_gpu`, per-sequence stride num_kv_heads * max_len *
 * head_dim).  Bytes are copied verbatim; nothing else in the caches changes.
 *
 *   k_new, v_new      [M, n_new, num_kv_heads * head_dim]   read
 *   k_cache, v_cache  [M, num_kv_heads, max_len, head_dim]   rows written:
 *       cache[m, kh, cache_lens[m] + r, :] = new[m, r, kh*d : (kh+1)*d]
 *   cache_lens        HOST [M] int32, write start position of sequence m
 *
 * Errors: NULL pointer; M not in [1, 32], n_new/num_kv_heads/max_len <= 0, a
 * cache_lens value < 0 or cache_lens[m] + n_new > max_len (INVALID_DIM);
 * head_dim not in {32, 64, 128} or misaligned (UNSUPPORTED); an element count
 * >= 2^40 (OVERFLOW); a cache overlapping a source or the other cache (ALIAS).
 */
int kv_cache_scatter(const float *k_new, const float *v_new, float *k_cache, float *v_cache,
                     const int32_t *cache_lens, int32_t num_seqs, int32_t n_new,
                     int32_t num_kv_heads, int32_t head_dim, int32_t max_len, void *stream);

/*
 * Copy a prefilled single-sequence cache into one slot of the batched cache.
 *
 * Defines: realizar `scatter_single_kv_to_batched` (after a prefill fills the
 * single cache of `init_kv_cache_gpu`, its rows go to the batched cache of
 * `init_batched_kv_cache_gpu` at offset slot * num_kv_heads * max_len *
 * head_dim, the slot's length becomes seq_len, and seq_len 0 does nothing).
 * The copy is per KV head: rows 0 .. seq_len-1 of head kh of the single cache
 * go to rows 0 .. seq_len-1 of head kh of the slot, bit for bit, so a decode of
 * the slot sees what a decode of the single cache saw.  (The page writes one
 * contiguous copy of num_kv_heads * seq_len * head_dim floats, which is the
 * same thing only when num_kv_heads == 1 or seq_len == max_len.)  One layer
 * per call; other rows and slots are untouched.
 *
 *   src_k, src_v      [num_kv_heads, src_max_len, head_dim]      read, rows < seq_len
 *   k_cache, v_cache  [num_seqs, num_kv_heads, max_len, head_dim]  slot's rows < seq_len written
 *   slot_lens         HOST [num_seqs] int32 or NULL; on success slot_lens[slot] = seq_len
 *
 * Errors: NULL cache or source pointer; num_seqs not in [1, 32], slot outside
 * [0, num_seqs), num_kv_heads/max_len/src_max_len <= 0, seq_len < 0 or larger
 * than src_max_len or max_len (INVALID_DIM); head_dim not in {32, 64, 128} or a
 * misaligned pointer (UNSUPPORTED); an element count >= 2^40 (OVERFLOW); a cache
 * overlapping a source or the other cache (ALIAS).  One launch (none for
 * seq_len 0).
 */
int kv_cache_copy_to_slot(const float *src_k, const float *src_v, int32_t src_max_len,
                          int32_t seq_len, float *k_cache, float *v_cache, int32_t slot,
                          int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                          int32_t max_len, int32_t *slot_lens, void *stream);

/*
 * Host bookkeeping of the per-sequence lengths (caller-owned HOST arrays of
 * num_seqs int32, the lengths every other entry point takes).  No HIP call.
 *   kv_lengths_reset     every length becomes 0 (realizar
 *                        `reset_batched_kv_cache_gpu`, `reset_kv_cache_gpu`:
 *                        a new generation; cache contents are left as they are
 *                        and are never read past a length).
 *   kv_lengths_rollback  every length above `position` becomes `position`
 *                        (realizar `rollback_kv_cache_gpu`: drop speculative
 *                        tokens, keep rows 0 .. position-1); shorter lengths stay.
 * Errors: lens NULL (NULL); num_seqs not in [1, 32] or position < 0
 * (INVALID_DIM), with lens untouched.
 */
int kv_lengths_reset(int32_t *lens, int32_t num_seqs);
int kv_lengths_rollback(int32_t *lens, int32_t num_seqs, int32_t position);

/*
 * Rotary position embedding (used by the *_rope entry points).
 *
 * Defines: trustformers-core `rope_neox_gpu_to_gpu` (GPT-NeoX half-split
 * partial rotation of [seq, heads, head_dim] rows at an absolute position
 * offset: 0 for a prefill, the cached length during decode) and its CPU
 * helper `rope_reference`; realizar `set_rope_theta` / `apply_rope_to_buffer`
 * (the same rotation over the whole head, base = rope theta, e.g. 10000 or
 * 1000000).  In every head of a row at position p, dim i < half =
 * rotary_ndims / 2 is paired with dim i + half and the pair is turned by
 * a = p * rope_theta^(-2 i / rotary_ndims) radians:
 *   y_i = x_i cos a - x_{i+half} sin a,   y_{i+half} = x_i sin a + x_{i+half} cos a;
 * dims >= rotary_ndims are unchanged.
 *   rotary_ndims  0 (no rotation) or a multiple of 8 up to head_dim
 *   rope_theta    the base; finite and > 0
 * Accuracy: angles are reduced to a fraction of a turn in double before the
 * single-precision sin/cos, so a rotated element is within a few f32 ulps of
 * the exact rotation at every int32 position (a single-precision angle
 * p * freq would be off by up to ~2e-3 rad near p = 32768).
 * Extra errors: rotary_ndims < 0 or > head_dim, rope_theta not finite or <= 0
 * (INVALID_DIM); rotary_ndims not a multiple of 8 (UNSUPPORTED).  They are
 * checked after the arguments the plain entry point checks.
 */

/*
 * kv_cache_scatter with the keys rotated to their cache positions: key row r
 * of sequence m is stored rotated to position cache_lens[m] + r.  Values are
 * copied verbatim, as are the key dims >= rotary_ndims.  Same arguments,
 * layout and errors as kv_cache_scatter, plus rotary_ndims and rope_theta.
 */
int kv_cache_scatter_rope(const float *k_new, const float *v_new, float *k_cache, float *v_cache,
                          const int32_t *cache_lens, int32_t num_seqs, int32_t n_new,
                          int32_t num_kv_heads, int32_t head_dim, int32_t max_len,
                          int32_t rotary_ndims, float rope_theta, void *stream);

/*
 * attn_decode_gqa_batched with the query rotated: sequence m's query is the
 * newest token, at position seq_lens[m] - 1, and is rotated to that position
 * before it is scored; the cached keys are used as stored (already rotated,
 * e.g. by kv_cache_scatter_rope).  Same arguments, layout, workspace and errors
 * as attn_decode_gqa_batched, plus rotary_ndims and rope_theta.
 */
int attn_decode_gqa_batched_rope(const float *q, const float *k_cache, const float *v_cache,
                                 const int32_t *seq_lens, float *out, int32_t num_seqs,
                                 int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_len, float scale, int32_t rotary_ndims,
                                 float rope_theta, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Static, NUL-terminated description of a status code. */
const char *attn_status_string(int status);

#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif /* TRANSFORMER_ATTENTION_FLASH_AMD_ATTN_H */
