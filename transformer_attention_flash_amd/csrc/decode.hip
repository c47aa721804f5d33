// decode.hip -- batched grouped-query decode attention, split over the key axis.
//
// Semantics: trueno-gpu 0.4.11 src/memory/resident/attention.rs,
// `incremental_attention_gpu` (one query per head against a head-first cache,
// empty sequence -> zeros), with the GQA / batched cache layout of realizar
// 0.8.5 src/cuda/executor/cache_from_cache_from_kv_cache.rs
// (`init_kv_cache_gpu`: [num_kv_heads, max_len, head_dim];
// `init_batched_kv_cache_gpu`: [M, num_kv_heads, max_len, head_dim]).
//
// Pass 1 (decode_split_kernel): one wavefront per work unit (sequence m, KV
// head kh, block of up to 16 query heads of that KV head's group, key split
// s).  The wave streams the split's K rows once and V rows once straight from
// HBM and serves every query head of the group from each load: the g query
// heads sharing a KV head make the scores a dense [16 x d] x [d x 16]
// contraction per 16 keys (heads padded to 16), which runs on
// v_mfma_f32_16x16x4_f32 and leaves the VALU free for the softmax.  The
// split's running max m_s (log2 units), sum l_s and unnormalised output
// acc_s are written to the workspace.
//
// Pass 2 (decode_combine_kernel): one wavefront per (m, h) merges the splits
// in index order: M* = max_s m_s, w_s = 2^(m_s - M*), out = sum_s w_s acc_s /
// sum_s w_s l_s, or zeros when the sequence is empty.
//
// Register layouts of v_mfma_f32_16x16x4_f32 (lane l, i = l % 16, k = l / 16):
// operand A supplies A[i][k], operand B supplies B[k][i], and output register
// r holds D[4k + r][i].  Scores are formed transposed, S^T = K q^T (rows =
// keys, columns = heads), so that output register r of a lane is exactly the
// operand-B value that lane supplies at key step r of the P.V contraction
// O^T = V^T P^T: no data moves between the two products.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kChunk = 32;  // keys per softmax step: two 16-key MFMA tiles

// Column of the head dimension that n-tile n, row i (0..15) of O^T stands for.
// Chosen so each lane's share of a V row is one or two contiguous 16-byte
// vectors and 16 lanes cover a row contiguously.
template <int D>
__host__ __device__ constexpr int ocol(int n, int i) {
    if constexpr (D >= 64) {
        return 64 * (n / 4) + 4 * i + (n % 4);
    } else {
        return 2 * i + n;
    }
}

struct UnitMap {
    int32_t start[ATTN_MAX_SEQS + 1];  // first unit of each sequence; start[M] = total
};

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a, UnitMap map,
                                                                int32_t T, int32_t n_hblk) {
    constexpr int NT = D / 16;     // 16-column tiles of O^T
    constexpr int KV4 = D / 16;    // 16-byte K vectors per lane per 16-key tile
    constexpr int VW = D >= 64 ? 4 : 2;  // floats per V vector
    constexpr int NVV = NT / VW;   // V vectors per lane per key
    typedef typename VecN<VW>::type vvec;

    const int lane = threadIdx.x & (kWave - 1);
    const int unit = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (unit >= map.start[a.M]) return;  // whole wave leaves; no block barrier below

    // unit -> (m, kh, head block hb, split s)
    int m = 0;
    while (unit >= map.start[m + 1]) ++m;
    const int L = a.lens.v[m];
    const int nsplit = (L + T - 1) / T;
    int rem = unit - map.start[m];
    const int s = rem % nsplit;
    rem /= nsplit;
    const int hb = rem % n_hblk;
    const int kh = rem / n_hblk;

    const int g = a.H / a.Hkv;
    const int hi = lane & 15;  // head column / key row within a tile
    const int kq = lane >> 4;  // k-slot of the MFMA operands
    const int head_in_group = hb * 16 + hi;
    const bool head_ok = head_in_group < g;
    const int h = kh * g + head_in_group;

    const int k0 = s * T;
    const int k1 = min(k0 + T, L);

    // q^T operand, pre-scaled so scores come out in log2 units.
    const float qs = a.scale * kLog2e;
    float qreg[KV4][4];
    {
        const float *qp = a.q + ((size_t)m * a.H + (head_ok ? h : 0)) * D + 4 * kq;
#pragma unroll
        for (int j = 0; j < KV4; ++j) {
            f32x4 v4 = head_ok ? *reinterpret_cast<const f32x4 *>(qp + 16 * j) : f32x4{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < 4; ++c) qreg[j][c] = v4[c] * qs;
        }
    }

    const size_t head_row0 = ((size_t)m * a.Hkv + kh) * (size_t)a.max_len;
    const float *__restrict__ kc = a.k_cache + head_row0 * D;
    const float *__restrict__ vc = a.v_cache + head_row0 * D;

    f32x4 o[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = f32x4{0, 0, 0, 0};
    float m_run = kNegBig;
    float l_run = 0.f;

    for (int kb = k0; kb < k1; kb += kChunk) {
        // Issue every load of the chunk first: K rows (lane = key row, k-slot
        // picks 16-byte columns) and V rows (16 lanes cover a row).
        f32x4 kf[2][KV4];
        vvec vf[2][4][NVV];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int krow = min(kb + 16 * t + hi, k1 - 1);
#pragma unroll
            for (int j = 0; j < KV4; ++j)
                kf[t][j] = *reinterpret_cast<const f32x4 *>(kc + (size_t)krow * D + 16 * j + 4 * kq);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int vrow = min(kb + 16 * t + 4 * kq + r, k1 - 1);
#pragma unroll
                for (int c = 0; c < NVV; ++c)
                    vf[t][r][c] = *reinterpret_cast<const vvec *>(vc + (size_t)vrow * D + 64 * c + VW * hi);
            }
        }

        // S^T tiles: rows = keys kb + 16t + 4kq + r, columns = heads.
        f32x4 sc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < KV4; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc = mfma16(kf[t][j][c], qreg[j][c], acc);
            sc[t] = acc;
        }

        // Online softmax over the chunk; keys >= k1 are masked.
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool live = kb + 16 * t + 4 * kq + r < k1;
                sc[t][r] = live ? sc[t][r] : -INFINITY;
                mx = fmaxf(mx, sc[t][r]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sc[t][r] = fast_exp2(sc[t][r] - m_new);
                psum += sc[t][r];
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int n = 0; n < NT; ++n) o[n] *= alpha;

        // O^T += V^T P^T; rows of V past the split end contribute zero.
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool live = kb + 16 * t + 4 * kq + r < k1;
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const float vv = live ? vget<VW>(vf[t][r][n / VW], n % VW) : 0.f;
                    o[n] = mfma16(vv, sc[t][r], o[n]);
                }
            }
    }

    // Each k-slot group summed its own keys; combine them.
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);

    if (head_ok) {
        const size_t slot = ((size_t)m * a.H + h) * a.max_splits + s;
        if (kq == 0) {
            *reinterpret_cast<f32x2 *>(a.ws_ml + 2 * slot) = f32x2{m_run, l_run};
        }
        float *dst = a.ws_acc + slot * D;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * kq + r;
#pragma unroll
            for (int c = 0; c < NVV; ++c) {
                vvec val;
#pragma unroll
                for (int e = 0; e < VW; ++e) vset<VW>(val, e, o[c * VW + e][r]);
                *reinterpret_cast<vvec *>(dst + ocol<D>(c * VW, i)) = val;
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeArgs a, int32_t T) {
    constexpr int PER = D >= 64 ? D / 64 : 1;  // floats per lane
    constexpr int LANES = D / PER;             // lanes holding output columns
    typedef typename VecN<PER>::type pvec;

    const int lane = threadIdx.x & (kWave - 1);
    const int w = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (w >= a.M * a.H) return;
    const int m = w / a.H;
    const int L = a.lens.v[m];
    const int nsplit = (L + T - 1) / T;
    float *dst = a.out + (size_t)w * D;

    if (nsplit == 0) {
        if (lane < LANES) *reinterpret_cast<pvec *>(dst + PER * lane) = pvec{};
        return;
    }
    const size_t slot0 = (size_t)w * a.max_splits;
    const float *ml = a.ws_ml + 2 * slot0;

    float mstar = -INFINITY;
    for (int s = lane; s < nsplit; s += kWave) mstar = fmaxf(mstar, ml[2 * s]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mstar = fmaxf(mstar, __shfl_xor(mstar, off));

    float lsum = 0.f;
    pvec acc{};
    const float *accp = a.ws_acc + slot0 * D + PER * lane;
    for (int s = 0; s < nsplit; ++s) {
        const float wgt = fast_exp2(ml[2 * s] - mstar);
        lsum += wgt * ml[2 * s + 1];
        if (lane < LANES) acc += wgt * *reinterpret_cast<const pvec *>(accp + (size_t)s * D);
    }
    if (lane < LANES) *reinterpret_cast<pvec *>(dst + PER * lane) = acc * (1.0f / lsum);
}

// Smallest split length (keys per work unit) for a cache of max_len rows: a
// multiple of the chunk that keeps the workspace's split axis at <= 256 slots.
int32_t min_split(int32_t max_len) {
    int32_t t = 64;
    while ((int64_t)t * 256 < max_len) t *= 2;
    return t;
}

}  // namespace

int32_t decode_max_splits(int32_t max_len) {
    const int32_t t = min_split(max_len);
    return (max_len + t - 1) / t;
}

size_t decode_workspace_bytes(int64_t M, int64_t H, int64_t D, int64_t max_len) {
    const int64_t slots = M * H * (int64_t)decode_max_splits((int32_t)max_len);
    return (size_t)(slots * (D + 2) * (int64_t)sizeof(float));
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    const int32_t g = a.H / a.Hkv;
    const int32_t n_hblk = (g + 15) / 16;
    // Split length: the smallest workspace-compatible power of two is doubled
    // while the grid would still have at least kMinUnits waves, so long
    // sequences get long splits (less partial traffic) and short batches still
    // fill the 256 compute units.
    constexpr int64_t kMinUnits = 4096;
    auto units_for = [&](int32_t t) {
        int64_t u = 0;
        for (int i = 0; i < a.M; ++i) u += (a.lens.v[i] + t - 1) / t;
        return u * a.Hkv * n_hblk;
    };
    int32_t T = min_split(a.max_len);
    while (T < a.max_len && units_for(2 * T) >= kMinUnits) T *= 2;

    UnitMap map;
    int32_t acc = 0;
    for (int i = 0; i < a.M; ++i) {
        map.start[i] = acc;
        acc += ((a.lens.v[i] + T - 1) / T) * a.Hkv * n_hblk;
    }
    for (int i = a.M; i <= ATTN_MAX_SEQS; ++i) map.start[i] = acc;

    dim3 block(kThreads);
    if (acc > 0) {
        dim3 grid((acc + kWavesPerBlock - 1) / kWavesPerBlock);
        switch (a.D) {
            case 32: decode_split_kernel<32><<<grid, block, 0, stream>>>(a, map, T, n_hblk); break;
            case 64: decode_split_kernel<64><<<grid, block, 0, stream>>>(a, map, T, n_hblk); break;
            case 128: decode_split_kernel<128><<<grid, block, 0, stream>>>(a, map, T, n_hblk); break;
            default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 grid2((a.M * a.H + kWavesPerBlock - 1) / kWavesPerBlock);
    switch (a.D) {
        case 32: decode_combine_kernel<32><<<grid2, block, 0, stream>>>(a, T); break;
        case 64: decode_combine_kernel<64><<<grid2, block, 0, stream>>>(a, T); break;
        case 128: decode_combine_kernel<128><<<grid2, block, 0, stream>>>(a, T); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace attn
