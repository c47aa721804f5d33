// launch.h -- internal interface between the C-ABI layer (attn_api.hip) and
// the kernel translation units.  Arguments reaching these launchers have been
// validated on the host already; each launcher only computes its grid and
// enqueues on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attn.h"
#include "rope.h"

namespace attn {

// Per-sequence host values travel in the kernel arguments (at most 32).
struct SeqInts {
    int32_t v[ATTN_MAX_SEQS];
};

struct ScatterArgs {
    const float *k_new;
    const float *v_new;
    float *k_cache;
    float *v_cache;
    SeqInts pos;  // write start position per sequence
    int32_t M, n_new, Hkv, D, max_len;
};
// With rope (rotary_ndims > 0) the keys are rotated to their cache positions.
hipError_t launch_kv_scatter(const ScatterArgs &a, hipStream_t stream, const RopeParams *rope = nullptr);

// Copy of rows 0 .. seq_len-1 of every KV head of a single cache
// [Hkv, src_max_len, D] into slot `slot` of the batched cache [M, Hkv, max_len, D].
struct SlotCopyArgs {
    const float *src_k;
    const float *src_v;
    float *k_cache;
    float *v_cache;
    int32_t src_max_len, seq_len, slot, Hkv, D, max_len;
};
hipError_t launch_slot_copy(const SlotCopyArgs &a, hipStream_t stream);

// Full-sequence attention.  q and out are [B, S, H * D] (S queries per batch
// element).  With cached == 0, k and v are [B, S, H * D] too (prefill from an
// empty cache).  With cached == 1, k and v are the caches [B, Hkv, max_len, D]:
// element b's queries sit at absolute positions pos[b] .. pos[b] + S - 1 and
// query i attends to cache rows 0 .. pos[b] + i (causal must be 1); with
// rope.rot > 0 (cached mode only) query i is first rotated to its position
// pos[b] + i.
struct PrefillArgs {
    const float *q;
    const float *k;
    const float *v;
    float *out;
    int32_t B, S, H, D;
    float scale;
    int32_t causal;
    int32_t cached;
    int32_t Hkv, max_len;
    SeqInts pos;
    RopeParams rope;  // rot == 0: queries not rotated
};
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);
// The prefill of a small problem (head_dim 32, 64 or 128) on 16-query waves
// whose workgroups split the keys four ways; `cus` = compute units of the
// device.
hipError_t launch_prefill_small(const PrefillArgs &a, int32_t cus, hipStream_t stream);
// Mean cached length over the batch (0 without a cache).
int32_t prefill_cached_rows(const PrefillArgs &a);
// The same attention (cached must be 0) on 16-bit MFMA operands:
// precision ATTN_PREC_FP16 or ATTN_PREC_BF16.
hipError_t launch_prefill_lowp(const PrefillArgs &a, int32_t precision, hipStream_t stream);

// Split-KV decode.  Workspace layout (floats):
//   acc[M][H][max_splits][D]  unnormalised per-split outputs
//   ml [M][H][max_splits][2]  per-split (running max in log2 units, sum)
struct DecodeArgs {
    const float *q;
    const float *k_cache;
    const float *v_cache;
    float *out;
    float *ws_acc;
    float *ws_ml;
    SeqInts lens;
    int32_t M, H, Hkv, D, max_len;
    int32_t max_splits;  // capacity of the workspace's split axis
    float scale;
};
// Number of split slots per (sequence, head) the workspace must hold.
int32_t decode_max_splits(int32_t M, int32_t H, int32_t max_len);
// Bytes of workspace for (M, H, D, max_len); 0 if it overflows.
size_t decode_workspace_bytes(int64_t M, int64_t H, int64_t D, int64_t max_len);
// With rope (rotary_ndims > 0) each sequence's query is rotated to position
// lens[m] - 1 (the newest cached token's) before scoring.
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream, const RopeParams *rope = nullptr);

}  // namespace attn
