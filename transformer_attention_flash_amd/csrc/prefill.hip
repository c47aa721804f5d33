// prefill.hip -- fused full-sequence attention (optionally causal) over
// interleaved [B, S, H * D] f32 activations, on CDNA4 fp32 MFMA.
//
// Semantics: trueno-gpu 0.4.11 src/memory/resident/attention.rs,
// `batched_multihead_attention` (softmax(Q K^T / sqrt(d_k)) V per head, heads
// interleaved in the row) and trustformers-core 0.2.0
// src/gpu_ops/cuda/oxicuda/attention.rs, `attention_prefill_gpu_to_gpu`
// (caller-chosen scale, causal mask from an empty cache: query i sees keys
// 0..=i, masked probabilities exactly zero).  Instead of the pages' per-head
// extract / transpose / GEMM / softmax / GEMM chain, one kernel reads the
// head's columns straight out of the interleaved rows and never materialises
// scores: an online softmax (running row max and sum, output rescaled when
// the max grows) walks the key axis tile by tile.
//
// Work decomposition: a workgroup owns BM = 128 queries of one (b, h); each
// of its 4 wavefronts owns 32 of them and keeps its Q slice in VGPRs and its
// 32 x D output accumulator in registers.  K and V tiles of BN = 32 keys are
// staged through LDS, the next tile's global loads in flight (in registers)
// while the current tile is consumed.  Both products run on v_mfma_f32_32x32x2_f32.
//
// Register layouts of v_mfma_f32_32x32x2_f32 (lane l, i = l % 32, k = l / 32):
// operand A supplies A[i][k], operand B supplies B[k][i], and output register
// v holds D[8 (v / 4) + 4 k + (v % 4)][i].  Scores are formed transposed,
// S^T = K Q^T (rows = keys, columns = queries), and the output as O^T = V^T
// P^T, so output register v of the score product is exactly the operand-B
// value its lane supplies at key step v of the output product, and each lane
// holds one query column in both, which makes the row max/sum a reduction
// over 16 registers plus one exchange with the partner half-wave.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int BM = 32 * kWaves;  // queries per workgroup
constexpr int BN = 32;           // keys per LDS tile
constexpr int kPad = 4;          // floats of padding per K row in LDS (bank spread)

__device__ __forceinline__ f32x16 mfma32(float a, float b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Key row (within a 32-key sub-tile) / output row of register v in lane-half k.
__device__ __forceinline__ int mrow(int v, int k) { return 8 * (v >> 2) + 4 * k + (v & 3); }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a, int32_t n_qtiles,
                                                              int32_t xcd_remap) {
    constexpr int NT = D / 32;         // 32-row tiles of O^T; also floats per lane per V row
    constexpr int QV = D / 8;          // 16-byte Q/K vectors per lane
    constexpr int KROW = D + kPad;     // LDS row pitch of K (floats)
    constexpr int TILE_VEC = BN * D / 4;              // 16-byte vectors per K (or V) tile
    constexpr int LD_PER_THREAD = TILE_VEC / kThreads;  // per tensor
    typedef typename VecN<NT>::type vrow_t;

    __shared__ __attribute__((aligned(16))) float Ks[BN * KROW];
    __shared__ __attribute__((aligned(16))) float Vs[BN * D];

    // ---- block -> (b, h, query tile); heavy causal tiles first, and with
    // xcd_remap the query tiles of one (b, h) stay on one XCD (blocks are
    // dealt to the 8 XCDs round-robin), so its K/V stream shares an L2.
    const int BH = a.B * a.H;
    int bh, qt;
    {
        const int bid = blockIdx.x;
        int rank;
        if (xcd_remap) {
            const int per_xcd_bh = BH / 8;
            const int x = bid % 8, t = bid / 8;
            bh = 8 * (t % per_xcd_bh) + x;
            rank = t / per_xcd_bh;
        } else {
            bh = bid % BH;
            rank = bid / BH;
        }
        qt = CAUSAL ? n_qtiles - 1 - rank : rank;
    }
    const int b = bh / a.H;
    const int h = bh % a.H;
    const int S = a.S;
    const size_t row_stride = (size_t)a.H * D;  // floats between consecutive tokens
    const size_t head_base = (size_t)b * S * row_stride + (size_t)h * D;
    const float *__restrict__ qg = a.q + head_base;
    const float *__restrict__ kg = a.k + head_base;
    const float *__restrict__ vg = a.v + head_base;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = lane & 31;  // query column of this lane
    const int lk = lane >> 5;  // half-wave (MFMA k-slot)
    const int q0 = qt * BM;
    const int qw0 = q0 + 32 * wave;  // first query of this wave
    const int my_q = qw0 + li;

    // ---- Q^T operand, pre-scaled so scores are in log2 units.
    const float qs = a.scale * kLog2e;
    float qreg[QV][4];
    {
        const bool ok = my_q < S;
        const float *qp = qg + (size_t)(ok ? my_q : 0) * row_stride + 4 * lk;
#pragma unroll
        for (int j = 0; j < QV; ++j) {
            f32x4 v4 = ok ? *reinterpret_cast<const f32x4 *>(qp + 8 * j) : f32x4{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < 4; ++c) qreg[j][c] = v4[c] * qs;
        }
    }

    f32x16 o[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = f32x16{};
    float m_run = kNegBig;
    float l_run = 0.f;

    const int n_ktiles_all = (S + BN - 1) / BN;
    const int n_ktiles = CAUSAL ? min(n_ktiles_all, (min(q0 + BM, S) - 1) / BN + 1) : n_ktiles_all;

    // Cooperative global -> register loads of one K/V tile.
    f32x4 kbuf[LD_PER_THREAD], vbuf[LD_PER_THREAD];
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int u = 0; u < LD_PER_THREAD; ++u) {
            const int idx = tid + u * kThreads;
            const int r = idx / (D / 4), c4 = idx % (D / 4);
            const int key = kt * BN + r;
            if (key < S) {
                kbuf[u] = *reinterpret_cast<const f32x4 *>(kg + (size_t)key * row_stride + 4 * c4);
                vbuf[u] = *reinterpret_cast<const f32x4 *>(vg + (size_t)key * row_stride + 4 * c4);
            } else {
                kbuf[u] = f32x4{0, 0, 0, 0};
                vbuf[u] = f32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int u = 0; u < LD_PER_THREAD; ++u) {
            const int idx = tid + u * kThreads;
            const int r = idx / (D / 4), c4 = idx % (D / 4);
            *reinterpret_cast<f32x4 *>(&Ks[r * KROW + 4 * c4]) = kbuf[u];
            *reinterpret_cast<f32x4 *>(&Vs[r * D + 4 * c4]) = vbuf[u];
        }
    };

    load_tile(0);
    store_tile();
    __syncthreads();

    for (int kt = 0; kt < n_ktiles; ++kt) {
        if (kt + 1 < n_ktiles) load_tile(kt + 1);

#pragma unroll
        for (int st = 0; st < BN / 32; ++st) {
            const int ks0 = kt * BN + st * 32;  // first key of the sub-tile
            if (ks0 >= S) break;
            if (CAUSAL && ks0 > qw0 + 31) break;  // whole sub-tile above this wave's diagonal

            // S^T = K Q^T over D (k-slot lk of step (j, c) is column 8j + 4lk + c).
            f32x16 s = f32x16{};
            const float *krow = &Ks[(st * 32 + li) * KROW + 4 * lk];
#pragma unroll
            for (int j = 0; j < QV; ++j) {
                const f32x4 kv = *reinterpret_cast<const f32x4 *>(krow + 8 * j);
#pragma unroll
                for (int c = 0; c < 4; ++c) s = mfma32(kv[c], qreg[j][c], s);
            }

            // Mask: keys past S, and (causal) keys after the query.
            const bool need_mask = (ks0 + 32 > S) || (CAUSAL && ks0 + 31 > qw0);
            if (need_mask) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = ks0 + mrow(v, lk);
                    const bool dead = key >= S || (CAUSAL && key > my_q);
                    s[v] = dead ? -INFINITY : s[v];
                }
            }

            float mx = s[0];
#pragma unroll
            for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            float psum = 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                s[v] = fast_exp2(s[v] - m_new);
                psum += s[v];
            }
            l_run = l_run * alpha + psum;
            // Once the running maxima settle, alpha is 1 in every lane: skip the
            // 16*NT multiplies then (a wave-uniform branch).
#ifndef ATTN_PREFILL_SKIP_RESCALE
#define ATTN_PREFILL_SKIP_RESCALE 1
#endif
            if (!ATTN_PREFILL_SKIP_RESCALE || __any(alpha != 1.0f)) {
#pragma unroll
                for (int n = 0; n < NT; ++n) o[n] *= alpha;
            }

            // O^T += V^T P^T: at key step v this lane supplies V[key][NT*li + n]
            // for n-tile n and P^T[key][my_q] = s[v].
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const vrow_t vv = *reinterpret_cast<const vrow_t *>(&Vs[(st * 32 + mrow(v, lk)) * D + NT * li]);
#pragma unroll
                for (int n = 0; n < NT; ++n) o[n] = mfma32(vget<NT>(vv, n), s[v], o[n]);
            }
        }

        if (kt + 1 < n_ktiles) {
            __syncthreads();
            store_tile();
            __syncthreads();
        }
    }

    // ---- normalise and store: lane holds query my_q, columns NT*row + n.
    l_run += __shfl_xor(l_run, 32);
    if (my_q < S) {
        const float inv = 1.0f / l_run;
        float *op = a.out + head_base + (size_t)my_q * row_stride;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            vrow_t val;
#pragma unroll
            for (int n = 0; n < NT; ++n) vset<NT>(val, n, o[n][v] * inv);
            *reinterpret_cast<vrow_t *>(op + NT * mrow(v, lk)) = val;
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_typed(const PrefillArgs &a, hipStream_t stream) {
    const int32_t n_qtiles = (a.S + BM - 1) / BM;
    const int32_t BH = a.B * a.H;
    const int32_t xcd_remap = (BH % 8 == 0) ? 1 : 0;
    dim3 grid((unsigned)(BH * n_qtiles));
    prefill_kernel<D, CAUSAL><<<grid, dim3(kThreads), 0, stream>>>(a, n_qtiles, xcd_remap);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    switch (a.D) {
        case 32: return a.causal ? launch_typed<32, true>(a, stream) : launch_typed<32, false>(a, stream);
        case 64: return a.causal ? launch_typed<64, true>(a, stream) : launch_typed<64, false>(a, stream);
        case 128: return a.causal ? launch_typed<128, true>(a, stream) : launch_typed<128, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
