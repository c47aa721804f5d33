// scatter.hip -- KV-cache append: copy rows of new keys and values from the
// interleaved [M, n_new, Hkv * D] layout the projections produce into the
// head-first batched cache [M, Hkv, max_len, D] at each sequence's position.
//
// Semantics: trueno-gpu 0.4.11 src/memory/resident/attention.rs,
// `kv_cache_scatter_gpu` (position pos of an interleaved row goes to
// cache[head, pos, :]), generalised to n_new rows and to the batched cache of
// realizar 0.8.5 src/cuda/executor/cache_from_cache_from_kv_cache.rs,
// `init_batched_kv_cache_gpu` (per-sequence stride Hkv * max_len * D).
//
// The copy is HBM-bound: each 16-byte vector is read once and written once.
// Consecutive lanes take consecutive vectors of the source, so reads are fully
// coalesced and every cache row (D floats) is written by D/4 adjacent lanes.
// Each thread keeps kVecPerThread loads in flight before its stores, and both
// directions use non-temporal hints since no byte is touched twice.
#include "device_common.h"
#include "launch.h"

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

template <int D>
__global__ __launch_bounds__(kThreads) void kv_scatter_kernel(ScatterArgs a, FastDiv by_hkv,
                                                              uint32_t per_seq_vec) {
    constexpr int Q = D / 4;  // 16-byte vectors per row
    const int m = blockIdx.z >> 1;
    const bool is_v = blockIdx.z & 1;
    const f32x4 *__restrict__ src =
        reinterpret_cast<const f32x4 *>(is_v ? a.v_new : a.k_new) + (size_t)m * per_seq_vec;
    f32x4 *__restrict__ cache = reinterpret_cast<f32x4 *>(is_v ? a.v_cache : a.k_cache);
    const size_t seq_base = (size_t)m * a.Hkv * a.max_len;  // first cache row of sequence m
    const int32_t pos = a.pos.v[m];

    const uint32_t first = blockIdx.x * (kThreads * kVecPerThread) + threadIdx.x;
    f32x4 buf[kVecPerThread];
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
        const uint32_t i = first + u * kThreads;
        if (i < per_seq_vec) buf[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
        const uint32_t i = first + u * kThreads;
        if (i < per_seq_vec) {
            const uint32_t row = i / Q;  // r * Hkv + kh
            const uint32_t r = fdiv(row, by_hkv);
            const uint32_t kh = row - r * by_hkv.d;
            const size_t dst_row = seq_base + (size_t)kh * a.max_len + (size_t)(pos + (int32_t)r);
            __builtin_nontemporal_store(buf[u], cache + dst_row * Q + (i - row * Q));
        }
    }
}

}  // namespace

hipError_t launch_kv_scatter(const ScatterArgs &a, hipStream_t stream) {
    const uint32_t per_seq_vec = (uint32_t)((int64_t)a.n_new * a.Hkv * a.D / 4);
    const uint32_t per_block = kThreads * kVecPerThread;
    dim3 grid((per_seq_vec + per_block - 1) / per_block, 1, 2 * a.M);
    dim3 block(kThreads);
    const FastDiv by_hkv = make_fastdiv((uint32_t)a.Hkv);
    switch (a.D) {
        case 32: kv_scatter_kernel<32><<<grid, block, 0, stream>>>(a, by_hkv, per_seq_vec); break;
        case 64: kv_scatter_kernel<64><<<grid, block, 0, stream>>>(a, by_hkv, per_seq_vec); break;
        case 128: kv_scatter_kernel<128><<<grid, block, 0, stream>>>(a, by_hkv, per_seq_vec); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace attn
