// attn_api.hip -- the C ABI of libattn.so (declared in include/attn.h).
//
// Host-side validation comes first and is complete before anything is
// enqueued, so an error return leaves every buffer untouched (the pages'
// helpers likewise reject bad sizes before launching: trueno-gpu 0.4.11
// src/memory/resident/attention.rs, `incremental_attention_gpu` /
// `kv_cache_scatter_gpu`; trustformers-core 0.2.0
// src/gpu_ops/cuda/oxicuda/attention.rs, `checked_len`).  Then exactly the
// kernels of the operation are launched on the caller's stream; nothing is
// allocated, copied or synchronised.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "launch.h"
#include "rope.h"

// Scratch memory of attn_decode_gqa_batched_noalloc, for callers that cannot
// allocate: one array on every GPU the library runs on, held until the
// process ends.  In host code this name stands for a host-side placeholder,
// not for device memory: its device address is looked up once per device
// (decode_scratch below) and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

namespace {

using attn::SeqInts;

constexpr int64_t kMaxElems32 = (int64_t(1) << 31) - 1;  // prefill indexes tokens*H*D in int32-safe ranges
constexpr int64_t kMaxElems = int64_t(1) << 40;          // decode/scatter element-count bound
// Decode cache rows: key positions plus one chunk step stay inside int32.
constexpr int32_t kMaxDecodeLen = int32_t(1) << 30;

bool head_dim_ok(int32_t d) { return d == 32 || d == 64 || d == 128; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [p, p + n) and [q, q + m) (bytes) overlap?
bool overlaps(const void *p, int64_t n, const void *q, int64_t m) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(q);
    return a0 < b0 + (uintptr_t)m && b0 < a0 + (uintptr_t)n;
}

// a * b * ... with an overflow check against `limit`.
bool checked_mul(std::initializer_list<int64_t> xs, int64_t limit, int64_t *out) {
    int64_t acc = 1;
    for (int64_t x : xs) {
        if (x < 0) return false;
        if (x != 0 && acc > limit / x) return false;
        acc *= x;
    }
    if (acc > limit) return false;
    *out = acc;
    return true;
}

int from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Rotary embedding arguments: 0 <= rotary_ndims <= head_dim, a multiple of 8
// (so a 16-byte vector never straddles the rotated and unrotated dims), and a
// finite positive base.
int check_rope(int32_t rotary_ndims, int32_t head_dim, float rope_theta) {
    if (rotary_ndims < 0 || rotary_ndims > head_dim) return ATTN_ERR_INVALID_DIM;
    if (!isfinite(rope_theta) || !(rope_theta > 0.0f)) return ATTN_ERR_INVALID_DIM;
    if (rotary_ndims % 8 != 0) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

// Validation of a decode call's arguments other than its workspace.  On
// success *args is filled except for the workspace pointers, *need is the
// workspace size in bytes, and nothing has been enqueued.
int check_decode(const float *q, const float *k_cache, const float *v_cache, const int32_t *seq_lens, float *out,
                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_len,
                 float scale, attn::DecodeArgs *args, size_t *need) {
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return ATTN_ERR_NULL;
    if (num_seqs < 1 || num_seqs > ATTN_MAX_SEQS) return ATTN_ERR_INVALID_DIM;
    if (num_heads <= 0 || num_kv_heads <= 0 || max_len <= 0 || head_dim <= 0) return ATTN_ERR_INVALID_DIM;
    if (num_kv_heads > num_heads || num_heads % num_kv_heads != 0) return ATTN_ERR_INVALID_DIM;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_DIM;
    SeqInts lens{};
    for (int32_t m = 0; m < num_seqs; ++m) {
        if (seq_lens[m] < 0 || seq_lens[m] > max_len) return ATTN_ERR_INVALID_DIM;
        lens.v[m] = seq_lens[m];
    }
    if (!head_dim_ok(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return ATTN_ERR_UNSUPPORTED;
    if (max_len > kMaxDecodeLen) return ATTN_ERR_OVERFLOW;
    int64_t q_elems, cache_elems;
    if (!checked_mul({num_seqs, num_heads, head_dim}, kMaxElems, &q_elems) ||
        !checked_mul({num_seqs, num_kv_heads, max_len, head_dim}, kMaxElems, &cache_elems))
        return ATTN_ERR_OVERFLOW;
    int64_t units;  // upper bound on pass-1 work units and workspace slots
    if (!checked_mul({num_seqs, num_heads, attn::decode_max_splits(num_seqs, num_heads, max_len)}, kMaxElems32, &units))
        return ATTN_ERR_OVERFLOW;
    *need = attn_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_len);
    if (*need == 0) return ATTN_ERR_OVERFLOW;
    const int64_t qb = q_elems * 4, cb = cache_elems * 4;
    if (overlaps(out, qb, q, qb) || overlaps(out, qb, k_cache, cb) || overlaps(out, qb, v_cache, cb))
        return ATTN_ERR_ALIAS;
    *args = attn::DecodeArgs{q,    k_cache,  v_cache,   out,          nullptr,  nullptr,
                             lens, num_seqs, num_heads, num_kv_heads, head_dim, max_len,
                             attn::decode_max_splits(num_seqs, num_heads, max_len), scale};
    return ATTN_OK;
}

// Point the decode at its workspace: acc[M][H][max_splits][D], then ml.
void set_decode_workspace(attn::DecodeArgs *a, void *workspace) {
    float *ws = static_cast<float *>(workspace);
    a->ws_acc = ws;
    a->ws_ml = ws + (size_t)a->M * a->H * a->max_splits * a->D;
}

// Validation shared by the plain and rotary variants of the decode with a
// caller-owned workspace; on success *args is filled and nothing has been
// enqueued.
int prepare_decode(const float *q, const float *k_cache, const float *v_cache, const int32_t *seq_lens,
                   float *out, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t max_len, float scale, void *workspace, size_t workspace_bytes,
                   attn::DecodeArgs *args) {
    if (!workspace) return ATTN_ERR_NULL;
    size_t need = 0;
    const int st = check_decode(q, k_cache, v_cache, seq_lens, out, num_seqs, num_heads, num_kv_heads, head_dim,
                                max_len, scale, args, &need);
    if (st != ATTN_OK) return st;
    if (!aligned16(workspace)) return ATTN_ERR_UNSUPPORTED;
    if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    const int64_t qb = (int64_t)num_seqs * num_heads * head_dim * 4;
    const int64_t cb = (int64_t)num_seqs * num_kv_heads * max_len * head_dim * 4;
    if (overlaps(out, qb, workspace, (int64_t)need) || overlaps(workspace, (int64_t)need, q, qb) ||
        overlaps(workspace, (int64_t)need, k_cache, cb) || overlaps(workspace, (int64_t)need, v_cache, cb))
        return ATTN_ERR_ALIAS;
    set_decode_workspace(args, workspace);
    return ATTN_OK;
}

// Device address of `scratch` on the GPU that runs `stream`, looked up once
// per device with that device current and then reused.
constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];

int decode_scratch(hipStream_t stream, void **ptr) {
    int dev = -1, cur = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return ATTN_ERR_HIP;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_HIP;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) return ATTN_ERR_HIP;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return ATTN_OK;
}

int prepare_scatter(const float *k_new, const float *v_new, float *k_cache, float *v_cache,
                    const int32_t *cache_lens, int32_t num_seqs, int32_t n_new, int32_t num_kv_heads,
                    int32_t head_dim, int32_t max_len, attn::ScatterArgs *args) {
    if (!k_new || !v_new || !k_cache || !v_cache || !cache_lens) return ATTN_ERR_NULL;
    if (num_seqs < 1 || num_seqs > ATTN_MAX_SEQS) return ATTN_ERR_INVALID_DIM;
    if (n_new <= 0 || num_kv_heads <= 0 || max_len <= 0 || head_dim <= 0) return ATTN_ERR_INVALID_DIM;
    SeqInts pos{};
    for (int32_t m = 0; m < num_seqs; ++m) {
        if (cache_lens[m] < 0 || (int64_t)cache_lens[m] + n_new > max_len) return ATTN_ERR_INVALID_DIM;
        pos.v[m] = cache_lens[m];
    }
    if (!head_dim_ok(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
        return ATTN_ERR_UNSUPPORTED;
    int64_t src_elems, cache_elems, per_seq;
    if (!checked_mul({num_seqs, n_new, num_kv_heads, head_dim}, kMaxElems, &src_elems) ||
        !checked_mul({num_seqs, num_kv_heads, max_len, head_dim}, kMaxElems, &cache_elems) ||
        !checked_mul({n_new, num_kv_heads, head_dim}, kMaxElems32, &per_seq))
        return ATTN_ERR_OVERFLOW;
    const int64_t sb = src_elems * 4, cb = cache_elems * 4;
    if (overlaps(k_cache, cb, v_cache, cb) || overlaps(k_cache, cb, k_new, sb) ||
        overlaps(k_cache, cb, v_new, sb) || overlaps(v_cache, cb, k_new, sb) || overlaps(v_cache, cb, v_new, sb))
        return ATTN_ERR_ALIAS;

    *args = attn::ScatterArgs{k_new, v_new, k_cache, v_cache, pos, num_seqs, n_new, num_kv_heads, head_dim,
                              max_len};
    return ATTN_OK;
}

// Validation of a chunked prefill; on success *sa and *pa are filled (the
// prefill without a rotary embedding) and nothing has been enqueued.
int prepare_prefill_cached(const float *q, const float *k_new, const float *v_new, float *k_cache,
                           float *v_cache, const int32_t *cache_lens, float *out, int32_t num_seqs,
                           int32_t n_new, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t max_len, float scale, attn::ScatterArgs *sa, attn::PrefillArgs *pa) {
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !cache_lens || !out) return ATTN_ERR_NULL;
    if (num_seqs < 1 || num_seqs > ATTN_MAX_SEQS) return ATTN_ERR_INVALID_DIM;
    if (n_new <= 0 || num_heads <= 0 || num_kv_heads <= 0 || max_len <= 0 || head_dim <= 0)
        return ATTN_ERR_INVALID_DIM;
    if (num_kv_heads > num_heads || num_heads % num_kv_heads != 0) return ATTN_ERR_INVALID_DIM;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_DIM;
    SeqInts pos{};
    for (int32_t m = 0; m < num_seqs; ++m) {
        if (cache_lens[m] < 0 || (int64_t)cache_lens[m] + n_new > max_len) return ATTN_ERR_INVALID_DIM;
        pos.v[m] = cache_lens[m];
    }
    if (!head_dim_ok(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(out))
        return ATTN_ERR_UNSUPPORTED;
    int64_t q_elems, new_elems, cache_elems, per_seq;
    if (!checked_mul({num_seqs, n_new, num_heads, head_dim}, kMaxElems32, &q_elems) ||
        !checked_mul({num_seqs, n_new, num_kv_heads, head_dim}, kMaxElems32, &new_elems) ||
        !checked_mul({num_seqs, num_kv_heads, max_len, head_dim}, kMaxElems, &cache_elems) ||
        !checked_mul({n_new, num_kv_heads, head_dim}, kMaxElems32, &per_seq))
        return ATTN_ERR_OVERFLOW;
    const int64_t qb = q_elems * 4, nb = new_elems * 4, cb = cache_elems * 4;
    const void *ins[] = {q, k_new, v_new};
    const int64_t in_bytes[] = {qb, nb, nb};
    for (int i = 0; i < 3; ++i)
        if (overlaps(out, qb, ins[i], in_bytes[i]) || overlaps(k_cache, cb, ins[i], in_bytes[i]) ||
            overlaps(v_cache, cb, ins[i], in_bytes[i]))
            return ATTN_ERR_ALIAS;
    if (overlaps(out, qb, k_cache, cb) || overlaps(out, qb, v_cache, cb) || overlaps(k_cache, cb, v_cache, cb))
        return ATTN_ERR_ALIAS;

    *sa = attn::ScatterArgs{k_new, v_new, k_cache, v_cache, pos, num_seqs, n_new, num_kv_heads, head_dim, max_len};
    attn::PrefillArgs &a = *pa;
    a = attn::PrefillArgs{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.B = num_seqs;
    a.S = n_new;
    a.H = num_heads;
    a.D = head_dim;
    a.scale = scale;
    a.causal = 1;
    a.cached = 1;
    a.Hkv = num_kv_heads;
    a.max_len = max_len;
    a.pos = pos;
    return ATTN_OK;
}

}  // namespace

extern "C" {

const char *attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_INVALID_DIM: return "a size, length or position is out of range";
        case ATTN_ERR_UNSUPPORTED: return "unsupported head_dim (32, 64, 128) or pointer not 16-byte aligned";
        case ATTN_ERR_OVERFLOW: return "a size product overflows the supported range";
        case ATTN_ERR_WORKSPACE:
            return "decode workspace missing or too small (attn_decode_gqa_batched_noalloc: the sizes need more "
                   "than its ATTN_DECODE_SCRATCH_BYTES of built-in scratch)";
        case ATTN_ERR_HIP: return "the HIP runtime reported an error";
        case ATTN_ERR_ALIAS: return "an output buffer overlaps an input buffer";
        default: return "unknown status";
    }
}

int attn_prefill(const float *q, const float *k, const float *v, float *out, int32_t batch,
                 int32_t seq_len, int32_t n_heads, int32_t head_dim, float scale, int32_t causal,
                 void *stream) {
    if (!q || !k || !v || !out) return ATTN_ERR_NULL;
    if (batch <= 0 || seq_len <= 0 || n_heads <= 0 || head_dim <= 0) return ATTN_ERR_INVALID_DIM;
    if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_DIM;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_DIM;
    if (!head_dim_ok(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_ERR_UNSUPPORTED;
    int64_t elems;
    if (!checked_mul({batch, seq_len, n_heads, head_dim}, kMaxElems32, &elems)) return ATTN_ERR_OVERFLOW;
    const int64_t bytes = elems * 4;
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
        return ATTN_ERR_ALIAS;

    attn::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.B = batch;
    a.S = seq_len;
    a.H = n_heads;
    a.D = head_dim;
    a.scale = scale;
    a.causal = causal;
    a.cached = 0;
    a.Hkv = n_heads;
    a.max_len = seq_len;
    return from_hip(attn::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

int attn_prefill_lowp(const float *q, const float *k, const float *v, float *out, int32_t batch,
                      int32_t seq_len, int32_t n_heads, int32_t head_dim, float scale, int32_t causal,
                      int32_t precision, void *stream) {
    if (!q || !k || !v || !out) return ATTN_ERR_NULL;
    if (batch <= 0 || seq_len <= 0 || n_heads <= 0 || head_dim <= 0) return ATTN_ERR_INVALID_DIM;
    if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_DIM;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_DIM;
    if (!head_dim_ok(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (precision != ATTN_PREC_FP16 && precision != ATTN_PREC_BF16) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_ERR_UNSUPPORTED;
    int64_t elems;
    if (!checked_mul({batch, seq_len, n_heads, head_dim}, kMaxElems32, &elems)) return ATTN_ERR_OVERFLOW;
    const int64_t bytes = elems * 4;
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
        return ATTN_ERR_ALIAS;

    attn::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.B = batch;
    a.S = seq_len;
    a.H = n_heads;
    a.D = head_dim;
    a.scale = scale;
    a.causal = causal;
    a.cached = 0;
    a.Hkv = n_heads;
    a.max_len = seq_len;
    return from_hip(attn::launch_prefill_lowp(a, precision, static_cast<hipStream_t>(stream)));
}


int attn_prefill_cached(const float *q, const float *k_new, const float *v_new, float *k_cache,
                        float *v_cache, const int32_t *cache_lens, float *out, int32_t num_seqs,
                        int32_t n_new, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t max_len, float scale, void *stream) {
    attn::ScatterArgs sa;
    attn::PrefillArgs a;
    const int st = prepare_prefill_cached(q, k_new, v_new, k_cache, v_cache, cache_lens, out, num_seqs, n_new,
                                          num_heads, num_kv_heads, head_dim, max_len, scale, &sa, &a);
    if (st != ATTN_OK) return st;
    // Append the chunk's K/V rows at each sequence's length, then attend over
    // the cache; both launches go on the same stream, in that order.
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (attn::launch_kv_scatter(sa, hs) != hipSuccess) return ATTN_ERR_HIP;
    return from_hip(attn::launch_prefill(a, hs));
}

int attn_prefill_cached_rope(const float *q, const float *k_new, const float *v_new, float *k_cache,
                             float *v_cache, const int32_t *cache_lens, float *out, int32_t num_seqs,
                             int32_t n_new, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_len, float scale, int32_t rotary_ndims, float rope_theta,
                             void *stream) {
    attn::ScatterArgs sa;
    attn::PrefillArgs a;
    int st = prepare_prefill_cached(q, k_new, v_new, k_cache, v_cache, cache_lens, out, num_seqs, n_new, num_heads,
                                    num_kv_heads, head_dim, max_len, scale, &sa, &a);
    if (st != ATTN_OK) return st;
    if ((st = check_rope(rotary_ndims, head_dim, rope_theta)) != ATTN_OK) return st;
    // The chunk's keys go into the cache rotated to their rows P_m + r, and
    // query r is rotated to the same position inside the attention.
    const attn::RopeParams rp = attn::make_rope(rotary_ndims, rope_theta);
    a.rope = rp;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (attn::launch_kv_scatter(sa, hs, &rp) != hipSuccess) return ATTN_ERR_HIP;
    return from_hip(attn::launch_prefill(a, hs));
}

size_t attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                   int32_t max_len) {
    if (num_seqs < 1 || num_seqs > ATTN_MAX_SEQS || num_heads <= 0 || max_len <= 0) return 0;
    if (!head_dim_ok(head_dim) || max_len > kMaxDecodeLen) return 0;
    int64_t slots;
    if (!checked_mul({num_seqs, num_heads, attn::decode_max_splits(num_seqs, num_heads, max_len), head_dim + 2}, kMaxElems,
                     &slots))
        return 0;
    return attn::decode_workspace_bytes(num_seqs, num_heads, head_dim, max_len);
}

int attn_decode_gqa_batched(const float *q, const float *k_cache, const float *v_cache,
                            const int32_t *seq_lens, float *out, int32_t num_seqs, int32_t num_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t max_len, float scale,
                            void *workspace, size_t workspace_bytes, void *stream) {
    attn::DecodeArgs a;
    const int st = prepare_decode(q, k_cache, v_cache, seq_lens, out, num_seqs, num_heads, num_kv_heads,
                                  head_dim, max_len, scale, workspace, workspace_bytes, &a);
    if (st != ATTN_OK) return st;
    return from_hip(attn::launch_decode(a, static_cast<hipStream_t>(stream)));
}

int attn_decode_gqa_batched_noalloc(const float *q, const float *k_cache, const float *v_cache,
                                    const int32_t *seq_lens, float *out, int32_t num_seqs, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t max_len, float scale,
                                    void *stream) {
    attn::DecodeArgs a;
    size_t need = 0;
    int st = check_decode(q, k_cache, v_cache, seq_lens, out, num_seqs, num_heads, num_kv_heads, head_dim, max_len,
                          scale, &a, &need);
    if (st != ATTN_OK) return st;
    if (need > ATTN_DECODE_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if ((st = decode_scratch(hs, &ws)) != ATTN_OK) return st;
    set_decode_workspace(&a, ws);
    return from_hip(attn::launch_decode(a, hs));
}

int attn_decode_gqa_batched_rope(const float *q, const float *k_cache, const float *v_cache,
                                 const int32_t *seq_lens, float *out, int32_t num_seqs, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_len, float scale,
                                 int32_t rotary_ndims, float rope_theta, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    attn::DecodeArgs a;
    int st = prepare_decode(q, k_cache, v_cache, seq_lens, out, num_seqs, num_heads, num_kv_heads, head_dim,
                            max_len, scale, workspace, workspace_bytes, &a);
    if (st != ATTN_OK) return st;
    if ((st = check_rope(rotary_ndims, head_dim, rope_theta)) != ATTN_OK) return st;
    const attn::RopeParams rp = attn::make_rope(rotary_ndims, rope_theta);
    return from_hip(attn::launch_decode(a, static_cast<hipStream_t>(stream), &rp));
}

int kv_cache_scatter(const float *k_new, const float *v_new, float *k_cache, float *v_cache,
                     const int32_t *cache_lens, int32_t num_seqs, int32_t n_new, int32_t num_kv_heads,
                     int32_t head_dim, int32_t max_len, void *stream) {
    attn::ScatterArgs a;
    const int st = prepare_scatter(k_new, v_new, k_cache, v_cache, cache_lens, num_seqs, n_new, num_kv_heads,
                                   head_dim, max_len, &a);
    if (st != ATTN_OK) return st;
    return from_hip(attn::launch_kv_scatter(a, static_cast<hipStream_t>(stream)));
}

int kv_cache_scatter_rope(const float *k_new, const float *v_new, float *k_cache, float *v_cache,
                          const int32_t *cache_lens, int32_t num_seqs, int32_t n_new, int32_t num_kv_heads,
                          int32_t head_dim, int32_t max_len, int32_t rotary_ndims, float rope_theta,
                          void *stream) {
    attn::ScatterArgs a;
    int st = prepare_scatter(k_new, v_new, k_cache, v_cache, cache_lens, num_seqs, n_new, num_kv_heads,
                             head_dim, max_len, &a);
    if (st != ATTN_OK) return st;
    if ((st = check_rope(rotary_ndims, head_dim, rope_theta)) != ATTN_OK) return st;
    const attn::RopeParams rp = attn::make_rope(rotary_ndims, rope_theta);
    return from_hip(attn::launch_kv_scatter(a, static_cast<hipStream_t>(stream), &rp));
}

int kv_cache_copy_to_slot(const float *src_k, const float *src_v, int32_t src_max_len, int32_t seq_len,
                          float *k_cache, float *v_cache, int32_t slot, int32_t num_seqs, int32_t num_kv_heads,
                          int32_t head_dim, int32_t max_len, int32_t *slot_lens, void *stream) {
    if (!src_k || !src_v || !k_cache || !v_cache) return ATTN_ERR_NULL;
    if (num_seqs < 1 || num_seqs > ATTN_MAX_SEQS || slot < 0 || slot >= num_seqs) return ATTN_ERR_INVALID_DIM;
    if (num_kv_heads <= 0 || head_dim <= 0 || max_len <= 0 || src_max_len <= 0) return ATTN_ERR_INVALID_DIM;
    if (seq_len < 0 || seq_len > src_max_len || seq_len > max_len) return ATTN_ERR_INVALID_DIM;
    if (!head_dim_ok(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(k_cache) || !aligned16(v_cache))
        return ATTN_ERR_UNSUPPORTED;
    int64_t src_elems, cache_elems, per_head;
    if (!checked_mul({num_kv_heads, src_max_len, head_dim}, kMaxElems, &src_elems) ||
        !checked_mul({num_seqs, num_kv_heads, max_len, head_dim}, kMaxElems, &cache_elems) ||
        !checked_mul({seq_len, head_dim}, kMaxElems32, &per_head))
        return ATTN_ERR_OVERFLOW;
    const int64_t sb = src_elems * 4, cb = cache_elems * 4;
    if (overlaps(k_cache, cb, v_cache, cb) || overlaps(k_cache, cb, src_k, sb) || overlaps(k_cache, cb, src_v, sb) ||
        overlaps(v_cache, cb, src_k, sb) || overlaps(v_cache, cb, src_v, sb))
        return ATTN_ERR_ALIAS;
    attn::SlotCopyArgs a{src_k, src_v, k_cache, v_cache, src_max_len, seq_len, slot, num_kv_heads, head_dim, max_len};
    const int st = from_hip(attn::launch_slot_copy(a, static_cast<hipStream_t>(stream)));
    if (st == ATTN_OK && slot_lens) slot_lens[slot] = seq_len;
    return st;
}

int kv_lengths_reset(int32_t *lens, int32_t num_seqs) {
    if (!lens) return ATTN_ERR_NULL;
    if (num_seqs < 1 || num_seqs > ATTN_MAX_SEQS) return ATTN_ERR_INVALID_DIM;
    for (int32_t m = 0; m < num_seqs; ++m) lens[m] = 0;
    return ATTN_OK;
}

int kv_lengths_rollback(int32_t *lens, int32_t num_seqs, int32_t position) {
    if (!lens) return ATTN_ERR_NULL;
    if (num_seqs < 1 || num_seqs > ATTN_MAX_SEQS || position < 0) return ATTN_ERR_INVALID_DIM;
    for (int32_t m = 0; m < num_seqs; ++m)
        if (lens[m] > position) lens[m] = position;
    return ATTN_OK;
}

}  // extern "C"
