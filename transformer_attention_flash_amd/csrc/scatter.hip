// scatter.hip -- KV-cache writes.  The append copies rows of new keys and values from the
// interleaved [M, n_new, Hkv * D] layout the projections produce into the
// head-first batched cache [M, Hkv, max_len, D] at each sequence's position.
//
// Semantics: trueno-gpu 0.4.11 src/memory/resident/attention.rs,
// `kv_cache_scatter_gpu` (position pos of an interleaved row goes to
// cache[head, pos, :]), generalised to n_new rows and to the batched cache of
// realizar 0.8.5 src/cuda/executor/cache_from_cache_from_kv_cache.rs,
// `init_batched_kv_cache_gpu` (per-sequence stride Hkv * max_len * D).
// The slot copy moves a prefilled single-sequence cache into one slot of the
// batched cache (realizar, `scatter_single_kv_to_batched`), head by head.
//
// The copy is HBM-bound: each 16-byte vector is read once and written once.
// Consecutive lanes take consecutive vectors of the source, so reads are fully
// coalesced and every cache row (D floats) is written by D/4 adjacent lanes.
// Each thread keeps kVecPerThread loads in flight before its stores, and both
// directions use non-temporal hints since no byte is touched twice.
//
// With a rotary embedding (rope.h) the keys are turned to their cache
// position on the way; the partner dims half a rotary width away come from
// the neighbouring lane that loaded them.  Values are always copied verbatim.
#include "device_common.h"
#include "launch.h"
#include "rope.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;

// Division by a runtime divisor via multiply-high (Granlund & Montgomery,
// "Division by invariant integers using multiplication", 1994): for
// 1 <= d < 2^31 and n < 2^31, n / d == (umulhi(n, magic) + n) >> shift with
// shift = ceil(log2 d) and magic = floor(2^32 * (2^shift - d) / d) + 1.
struct FastDiv {
    uint32_t d, magic, shift;
};

FastDiv make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while ((1u << s) < d) ++s;
    uint64_t magic = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
    return FastDiv{d, uint32_t(magic), s};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
    return (__umulhi(n, f.magic) + n) >> f.shift;
}

template <int D, bool ROPE>
__global__ __launch_bounds__(kThreads) void kv_scatter_kernel(ScatterArgs a, FastDiv by_hkv,
                                                              uint32_t per_seq_vec, RopeParams rp) {
    constexpr int Q = D / 4;  // 16-byte vectors per row
    static_assert(kWave % Q == 0 && kThreads % Q == 0, "a row must not straddle waves or steps");
    // Plain copy: grid (blocks, 1, 2M), z = 2m + (0: K, 1: V).  With a
    // rotation the K and V blocks of a sequence alternate along x instead,
    // so every CU mixes the ALU-heavy K blocks with the pure-copy V blocks.
    const int m = ROPE ? blockIdx.z : blockIdx.z >> 1;
    const bool is_v = ROPE ? (blockIdx.x & 1) : (blockIdx.z & 1);
    const uint32_t blk = ROPE ? blockIdx.x >> 1 : blockIdx.x;
    const f32x4 *__restrict__ src =
        reinterpret_cast<const f32x4 *>(is_v ? a.v_new : a.k_new) + (size_t)m * per_seq_vec;
    f32x4 *__restrict__ cache = reinterpret_cast<f32x4 *>(is_v ? a.v_cache : a.k_cache);
    const size_t seq_base = (size_t)m * a.Hkv * a.max_len;  // first cache row of sequence m
    const int32_t pos = a.pos.v[m];

    const uint32_t first = blk * (kThreads * kVecPerThread) + threadIdx.x;
    f32x4 buf[kVecPerThread];
    uint32_t rr[kVecPerThread];  // token row of each vector
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
        const uint32_t i = first + u * kThreads;
        if constexpr (ROPE) buf[u] = f32x4{0, 0, 0, 0};  // lanes past the end still take part in the exchange
        if (i < per_seq_vec) buf[u] = __builtin_nontemporal_load(src + i);
        rr[u] = fdiv(i / Q, by_hkv);
    }

    if constexpr (ROPE) {
        if (!is_v) {  // uniform over the block
            // A wave covers whole rows (64 % Q == 0) and a thread's vectors
            // are kThreads apart (a multiple of Q), so every vector of this
            // thread holds the same dims l0 .. l0+3 and the partner vector is
            // held by the lane hq away in the same wave: exchange, not reload.
            const int lane = threadIdx.x & (kWave - 1);
            const int l0 = 4 * (lane % Q);
            const bool in_rot = l0 < rp.rot;
            const bool low = l0 < rp.half;
            const int hq = rp.half / 4;
            const int src_lane = in_rot ? (low ? lane + hq : lane - hq) : lane;
            const int i0 = in_rot ? (low ? l0 : l0 - rp.half) : 0;
            double turns[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) turns[c] = in_rot ? rp.turns[i0 + c] : 0.0;
            // Consecutive vectors of a thread usually share a token row (the
            // rows of its heads), hence a position: sin/cos are recomputed only
            // when the position changes.
            int32_t last = -1;
            float sn[4], cs[4];
#pragma unroll
            for (int u = 0; u < kVecPerThread; ++u) {
                f32x4 part;
#pragma unroll
                for (int c = 0; c < 4; ++c) part[c] = __shfl(buf[u][c], src_lane);
                const uint32_t i = first + u * kThreads;
                if (in_rot && i < per_seq_vec) {
                    const int32_t p = pos + (int32_t)rr[u];
                    if (p != last) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) rope_sincos(p, turns[c], sn[c], cs[c]);
                        last = p;
                    }
                    buf[u] = rope_apply4(buf[u], part, low, sn, cs);
                }
            }
        }
    }

#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
        const uint32_t i = first + u * kThreads;
        if (i < per_seq_vec) {
            const uint32_t row = i / Q;  // r * Hkv + kh
            const uint32_t r = rr[u];
            const uint32_t kh = row - r * by_hkv.d;
            const size_t dst_row = seq_base + (size_t)kh * a.max_len + (size_t)(pos + (int32_t)r);
            __builtin_nontemporal_store(buf[u], cache + dst_row * Q + (i - row * Q));
        }
    }
}

template <bool ROPE>
hipError_t launch_typed(const ScatterArgs &a, const RopeParams &rp, hipStream_t stream) {
    const uint32_t per_seq_vec = (uint32_t)((int64_t)a.n_new * a.Hkv * a.D / 4);
    const uint32_t per_block = kThreads * kVecPerThread;
    const uint32_t blocks = (per_seq_vec + per_block - 1) / per_block;
    dim3 grid = ROPE ? dim3(2 * blocks, 1, a.M) : dim3(blocks, 1, 2 * a.M);
    dim3 block(kThreads);
    const FastDiv by_hkv = make_fastdiv((uint32_t)a.Hkv);
    switch (a.D) {
        case 32: kv_scatter_kernel<32, ROPE><<<grid, block, 0, stream>>>(a, by_hkv, per_seq_vec, rp); break;
        case 64: kv_scatter_kernel<64, ROPE><<<grid, block, 0, stream>>>(a, by_hkv, per_seq_vec, rp); break;
        case 128: kv_scatter_kernel<128, ROPE><<<grid, block, 0, stream>>>(a, by_hkv, per_seq_vec, rp); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Slot copy: grid (vector blocks of one head, Hkv, 2 = K/V).  A head's live
// rows are seq_len * D contiguous floats in both caches, so this is a straight
// streaming copy per head at two different base offsets.
constexpr int kSlotVec = 4;  // 16-byte vectors per thread

__global__ __launch_bounds__(kThreads) void slot_copy_kernel(SlotCopyArgs a, uint32_t per_head_vec) {
    const int kh = blockIdx.y;
    const bool is_v = blockIdx.z;
    const size_t q = (size_t)a.D / 4;
    const f32x4 *__restrict__ src =
        reinterpret_cast<const f32x4 *>(is_v ? a.src_v : a.src_k) + (size_t)kh * a.src_max_len * q;
    f32x4 *__restrict__ dst = reinterpret_cast<f32x4 *>(is_v ? a.v_cache : a.k_cache) +
                              ((size_t)a.slot * a.Hkv + kh) * a.max_len * q;
    const uint32_t first = blockIdx.x * (kThreads * kSlotVec) + threadIdx.x;
    f32x4 buf[kSlotVec];
#pragma unroll
    for (int u = 0; u < kSlotVec; ++u) {
        const uint32_t i = first + u * kThreads;
        if (i < per_head_vec) buf[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kSlotVec; ++u) {
        const uint32_t i = first + u * kThreads;
        if (i < per_head_vec) __builtin_nontemporal_store(buf[u], dst + i);
    }
}

}  // namespace

hipError_t launch_slot_copy(const SlotCopyArgs &a, hipStream_t stream) {
    if (a.seq_len == 0) return hipSuccess;
    const uint32_t per_head_vec = (uint32_t)((int64_t)a.seq_len * a.D / 4);
    const uint32_t per_block = kThreads * kSlotVec;
    dim3 grid((per_head_vec + per_block - 1) / per_block, a.Hkv, 2);
    slot_copy_kernel<<<grid, dim3(kThreads), 0, stream>>>(a, per_head_vec);
    return hipGetLastError();
}

hipError_t launch_kv_scatter(const ScatterArgs &a, hipStream_t stream, const RopeParams *rope) {
    if (rope && rope->rot > 0) return launch_typed<true>(a, *rope, stream);
    return launch_typed<false>(a, RopeParams{}, stream);
}

}  // namespace attn
