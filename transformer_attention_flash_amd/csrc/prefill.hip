// prefill.hip -- fused full-sequence attention (optionally causal) over
// interleaved [B, S, H * D] f32 activations, on CDNA4 fp32 MFMA.
//
// Semantics: trueno-gpu 0.4.11 src/memory/resident/attention.rs,
// `batched_multihead_attention` (softmax(Q K^T / sqrt(d_k)) V per head, heads
// interleaved in the row) and trustformers-core 0.2.0
// src/gpu_ops/cuda/oxicuda/attention.rs, `attention_prefill_gpu_to_gpu`
// (caller-chosen scale, causal mask from an empty cache: query i sees keys
// 0..=i, masked probabilities exactly zero).  The same kernel also runs a
// chunk of queries behind an existing KV cache (the case that page leaves to
// other paths): keys then come from the GQA cache slab [max_len, D] of the
// query head's KV head and query i of the chunk sees cache rows 0..P+i.
// Instead of the pages' per-head extract / transpose / GEMM / softmax / GEMM
// chain, one kernel reads the head's columns straight out of the interleaved
// rows and never materialises scores: an online softmax (running row sum
// against a reference maximum, output rescaled when that reference moves)
// walks the key axis tile by tile.
//
// Work decomposition: a workgroup owns BM = 32 NW queries of one (b, h) (NW =
// 8 waves, or 4 for smaller problems); each wavefront owns 32 of them and
// keeps its Q slice in VGPRs and its 32 x D output accumulator in registers.
// K and V tiles of BN keys (64 for the eight-wave kernels at head_dim 64 and
// 128, else 32) go from HBM straight into a double-buffered LDS tile
// (global_load_lds, no register staging); the next tile's transfer is in
// flight while the current one is consumed, with one workgroup barrier per
// tile.  Both products run on v_mfma_f32_32x32x2_f32.  A 64-key tile is two
// 32-key sub-tiles whose score products are two independent accumulation
// chains (B=4 S=2048 H=32 d=128: causal 1106 -> 1095 us, non-causal 2023 ->
// 2004 us against 32-key tiles with three chains; at d=64 1.5-3% on five
// shapes, B=2 S=4096 H=32 causal 1122 -> 1085 us).  In a causal wave's
// diagonal 64-key tile whose second sub-tile lies wholly above the wave's
// queries, only the first is computed (1096 -> 1090 us; the 2048-behind-2048
// chunk 3129 -> 3100 us).  (Problems too small to
// fill the CUs with these workgroups, and mid-size causal ones, run
// prefill_small.hip; see launch_typed.)
//
// Register layouts of v_mfma_f32_32x32x2_f32 (lane l, i = l % 32, k = l / 32):
// operand A supplies A[i][k], operand B supplies B[k][i], and output register
// v holds D[8 (v / 4) + 4 k + (v % 4)][i].  Scores are formed transposed,
// S^T = K Q^T (rows = keys, columns = queries), and the output as O^T = V^T
// P^T, so output register v of the score product is exactly the operand-B
// value its lane supplies at key step v of the output product, and each lane
// holds one query column in both, which makes the row max/sum a reduction
// over 16 registers plus one exchange with the partner half-wave.
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr float kLazy = 8.0f;  // log2 headroom of the lazily rescaled softmax

__device__ __forceinline__ f32x16 mfma32(float a, float b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Key row (within a 32-key sub-tile) / output row of register v in lane-half k.
__device__ __forceinline__ int mrow(int v, int k) { return 8 * (v >> 2) + 4 * k + (v & 3); }

typedef __attribute__((address_space(3))) void lds_void_t;

// One 16-byte global -> LDS transfer per lane (global_load_lds_dwordx4): lane l's
// 16 bytes land at lds_base + 16 l, lds_base being uniform over the wave.
__device__ __forceinline__ void dma16(const float *src, float *lds_base) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src), (lds_void_t *)lds_base, 16, 0, 0);
}

// Wait until this wave has no global loads (including LDS transfers) in flight.
__device__ __forceinline__ void wait_vmem_all() {
    // s_waitcnt vmcnt(0), expcnt/lgkmcnt unconstrained (7 and 15).
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

// NW waves of 32 queries each (BM = 32 NW queries per workgroup) walk all of
// their key tiles (BN keys: one or two 32-key MFMA sub-tiles) together.
template <int D, int NW, bool CAUSAL, int BN = 32>
__global__ __launch_bounds__(kWave * NW, 8 / NW) void prefill_kernel(PrefillArgs a, int32_t n_qtiles,
                                                                     int32_t xcd_remap) {
    constexpr int NSUB = BN / 32;  // 32-key sub-tiles per tile
    static_assert(NSUB == 1 || NSUB == 2, "tiles of 32 or 64 keys");
    constexpr int QW = NW;  // query waves per workgroup
    constexpr int BM = 32 * QW;
    constexpr int NT = D / 32;          // 32-row tiles of O^T; also floats per lane per V row
    constexpr int QV = D / 8;           // 16-byte Q/K vectors per lane
    constexpr int CPR = D / 4;          // 16-byte chunks per K/V row
    constexpr int RPI = kWave / CPR;    // rows moved by one wave-wide 1 KiB transfer
    constexpr int XPW = BN / RPI / QW;  // transfers per wave per tensor per tile
    constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;  // K chunk swizzle mask
    typedef typename VecN<NT>::type vrow_t;
    static_assert(XPW >= 1 && XPW * RPI * QW == BN, "tile must split evenly over the waves");

    // Double-buffered K/V tiles.  K chunk c of row r sits at chunk position
    // c ^ (r & SWZ), so the 16 rows of one half-wave operand read hit distinct
    // banks; V rows are read contiguously and are stored as they are.
    // Separate objects (not one [2][..] array) so the compiler can see that a
    // transfer into one buffer does not alias reads of the other and does not
    // make those reads wait for it.
    __shared__ __attribute__((aligned(16))) float Ks0[BN * D];
    __shared__ __attribute__((aligned(16))) float Vs0[BN * D];
    __shared__ __attribute__((aligned(16))) float Ks1[BN * D];
    __shared__ __attribute__((aligned(16))) float Vs1[BN * D];

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
    const int S = a.S;                           // queries of this batch element
    const size_t row_stride = (size_t)a.H * D;  // floats between consecutive tokens
    const size_t head_base = (size_t)b * S * row_stride + (size_t)h * D;
    const float *__restrict__ qg = a.q + head_base;
    // Keys: the interleaved activations (key j = token j), or the cache slab of
    // KV head h / (H / Hkv) (key j = cache row j, queries offset by P).
    const int P = a.cached ? a.pos.v[b] : 0;    // key index of query 0
    const int Sk = P + S;                        // keys a query can reach at most
    size_t kv_stride, kv_base;
    if (a.cached) {
        kv_stride = D;
        kv_base = ((size_t)b * a.Hkv + h / (a.H / a.Hkv)) * (size_t)a.max_len * D;
    } else {
        kv_stride = row_stride;
        kv_base = head_base;
    }
    const float *__restrict__ kg = a.k + kv_base;
    const float *__restrict__ vg = a.v + kv_base;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = lane & 31;  // query column of this lane
    const int lk = lane >> 5;  // half-wave (MFMA k-slot)
    const int qwave = wave;          // query slice of this wave
    const int q0 = qt * BM;
    const int qw0 = q0 + 32 * qwave;  // first query of this wave
    const int my_q = qw0 + li;

    // ---- Q^T operand, pre-scaled so scores are in log2 units (behind a cache
    // with a rotary embedding, first turned to the query's position P + my_q;
    // the partner dims half a rotary width away come from the same row).
    const float qs = a.scale * kLog2e;
    float qreg[QV][4];
    {
        const bool ok = my_q < S;
        const float *qrow = qg + (size_t)(ok ? my_q : 0) * row_stride;
        const float *qp = qrow + 4 * lk;
#pragma unroll
        for (int j = 0; j < QV; ++j) {
            f32x4 v4 = ok ? *reinterpret_cast<const f32x4 *>(qp + 8 * j) : f32x4{0, 0, 0, 0};
            if (a.rope.rot > 0) {
                const int l0 = 8 * j + 4 * lk;
                const int pl = l0 < a.rope.half ? l0 + a.rope.half : l0 - a.rope.half;
                const f32x4 part =
                    (ok && l0 < a.rope.rot) ? *reinterpret_cast<const f32x4 *>(qrow + pl) : f32x4{0, 0, 0, 0};
                v4 = rope_rotate4(v4, part, l0, P + my_q, a.rope);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) qreg[j][c] = v4[c] * qs;
        }
    }

    f32x16 o[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = f32x16{};
    float m_run = kNegBig;
    float l_run = 0.f;

    const int n_ktiles_all = (Sk + BN - 1) / BN;
    const int n_ktiles = CAUSAL ? min(n_ktiles_all, (P + min(q0 + BM, S) - 1) / BN + 1) : n_ktiles_all;
    const int T = n_ktiles;

    // Each wave moves XPW 1 KiB pieces of the K tile and of the V tile straight
    // into LDS.  Keys past Sk read row Sk - 1 (in bounds); their scores are
    // masked and their probabilities are exactly 0, so the values never matter.
    auto issue_tile = [&](int kt, float *kdst, float *vdst) {
#pragma unroll
        for (int u = 0; u < XPW; ++u) {
            const int piece = qwave * XPW + u;
            const int row = piece * RPI + lane / CPR;
            const int chunk = lane % CPR;
            const size_t key = (size_t)min(kt * BN + row, Sk - 1);
            dma16(kg + key * kv_stride + 4 * (chunk ^ (row & SWZ)), kdst + piece * 256);
            dma16(vg + key * kv_stride + 4 * chunk, vdst + piece * 256);
        }
    };

    // One tile: wait for it, barrier, start the next tile's transfer into the
    // other buffer, consume this one.
    auto step = [&](int kt, const float *Kt, const float *Vt, float *Kn, float *Vn) {
        wait_vmem_all();  // this wave's share of tile kt has landed
        __syncthreads();  // ... and every other wave's; all are done with tile kt-1
        if (kt + 1 < T) issue_tile(kt + 1, Kn, Vn);

        const int ks0 = kt * BN;  // first key of the tile
        if (CAUSAL && ks0 > P + qw0 + 31) return;  // whole tile above this wave's diagonal

        // The tile's work for NS computed 32-key sub-tiles: NS = 1 (causal)
        // when the second sub-tile of a 64-key tile lies wholly above this
        // wave's diagonal (its scores would all be masked).
        auto body = [&](auto ns_tag) {
            constexpr int NS = decltype(ns_tag)::value;
            // S^T = K Q^T over D (k-slot lk of step (j, c) is column 8j + 4lk + c).
            f32x16 s = f32x16{};
            const float *kbase = Kt + li * D;
            f32x16 sb = f32x16{};  // second sub-tile (keys 32 .. 63) of a 64-key tile
            // Raised wave priority while this wave issues matrix instructions:
            // the SIMD's other wave (in its softmax or waiting) does not delay
            // them.
            __builtin_amdgcn_s_setprio(1);
            // Independent accumulation chains, summed afterwards: back-to-back
            // dependent MFMAs issue more slowly (two chains gave +7%, four another
            // +5% on the causal d = 128 prefill, before the lazy softmax update
            // below).  The causal d = 128 kernels now use three: four leave no
            // registers for the lazy update, and three with it beat four without
            // it by 3-4%.  The non-causal d = 128 kernels keep two (three gave
            // nothing there, four spill).
            f32x16 s2 = f32x16{}, s3 = f32x16{}, s4 = f32x16{};
            if constexpr (NS == 2) {
                // Two sub-tiles: two independent chains, interleaved, no sums.
                const float *kbase2 = Kt + (32 + li) * D;
    #pragma unroll
                for (int j = 0; j < QV; ++j) {
                    const int cpos = 4 * ((2 * j + lk) ^ (li & SWZ));  // rows li and 32 + li share the swizzle
                    const f32x4 kv = *reinterpret_cast<const f32x4 *>(kbase + cpos);
                    const f32x4 kv2 = *reinterpret_cast<const f32x4 *>(kbase2 + cpos);
    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s = mfma32(kv[e], qreg[j][e], s);
                        sb = mfma32(kv2[e], qreg[j][e], sb);
                    }
                }
                __builtin_amdgcn_s_setprio(0);
            } else if constexpr (CAUSAL && D == 128) {
    #pragma unroll
                for (int j = 0; j < QV; ++j) {
                    const f32x4 kv = *reinterpret_cast<const f32x4 *>(kbase + 4 * ((2 * j + lk) ^ (li & SWZ)));
    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = (4 * j + e) % 3;  // compile-time after unrolling
                        if (c == 0)
                            s = mfma32(kv[e], qreg[j][e], s);
                        else if (c == 1)
                            s2 = mfma32(kv[e], qreg[j][e], s2);
                        else
                            s3 = mfma32(kv[e], qreg[j][e], s3);
                    }
                }
                __builtin_amdgcn_s_setprio(0);
                s += s2;
                s += s3;
            } else {
                constexpr bool kFourChains = CAUSAL || D < 128;
    #pragma unroll
                for (int j = 0; j < QV; ++j) {
                    const f32x4 kv = *reinterpret_cast<const f32x4 *>(kbase + 4 * ((2 * j + lk) ^ (li & SWZ)));
                    s = mfma32(kv[0], qreg[j][0], s);
                    s2 = mfma32(kv[1], qreg[j][1], s2);
                    if constexpr (kFourChains) {
                        s3 = mfma32(kv[2], qreg[j][2], s3);
                        s4 = mfma32(kv[3], qreg[j][3], s4);
                    } else {
                        s = mfma32(kv[2], qreg[j][2], s);
                        s2 = mfma32(kv[3], qreg[j][3], s2);
                    }
                }
                __builtin_amdgcn_s_setprio(0);
                s += s2;
                if constexpr (kFourChains) {
                    s3 += s4;
                    s += s3;
                }
            }

            // Mask: keys past Sk, and (causal) keys after the query's position.
            const bool need_mask = (ks0 + 32 * NS > Sk) || (CAUSAL && ks0 + 32 * NS - 1 > P + qw0);
            if (need_mask) {
    #pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = ks0 + mrow(v, lk);
                    const bool dead = key >= Sk || (CAUSAL && key > P + my_q);
                    s[v] = dead ? -INFINITY : s[v];
                    if constexpr (NS == 2) {
                        const bool dead2 = key + 32 >= Sk || (CAUSAL && key + 32 > P + my_q);
                        sb[v] = dead2 ? -INFINITY : sb[v];
                    }
                }
            }

            float mx = s[0];
    #pragma unroll
            for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
            if constexpr (NS == 2) {
    #pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sb[v]);
            }
            mx = max_xor32(mx);
            // Lazy rescaling: the reference maximum m_run moves (and O and l are
            // rescaled) only when a lane's scores would exceed it by more than
            // 2^kLazy; otherwise the probabilities are taken against the stale
            // reference (below 2^kLazy, exact enough in f32).  The decision is
            // wave-uniform, so most tiles skip the 16 * NT multiplies.
            if (__any(mx - m_run > kLazy)) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
    #pragma unroll
                for (int n = 0; n < NT; ++n) o[n] *= alpha;
            }
            float psum = 0.f, psum2 = 0.f;
    #pragma unroll
            for (int v = 0; v < 16; ++v) {
                s[v] = fast_exp2(s[v] - m_run);
                psum += s[v];
                if constexpr (NS == 2) {
                    sb[v] = fast_exp2(sb[v] - m_run);
                    psum2 += sb[v];
                }
            }
            l_run += psum + psum2;

            // O^T += V^T P^T: at key step v this lane supplies V[key][NT*li + n]
            // for n-tile n and P^T[key][my_q] = s[v].
            __builtin_amdgcn_s_setprio(1);
    #pragma unroll
            for (int v = 0; v < 16; ++v) {
                const vrow_t vv = *reinterpret_cast<const vrow_t *>(Vt + mrow(v, lk) * D + NT * li);
    #pragma unroll
                for (int n = 0; n < NT; ++n) o[n] = mfma32(vget<NT>(vv, n), s[v], o[n]);
            }
            if constexpr (NS == 2) {
    #pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const vrow_t vv = *reinterpret_cast<const vrow_t *>(Vt + (32 + mrow(v, lk)) * D + NT * li);
    #pragma unroll
                    for (int n = 0; n < NT; ++n) o[n] = mfma32(vget<NT>(vv, n), sb[v], o[n]);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        };
        if constexpr (NSUB == 2 && CAUSAL) {
            if (ks0 + 32 > P + qw0 + 31)
                body(std::integral_constant<int, 1>{});
            else
                body(std::integral_constant<int, 2>{});
        } else {
            body(std::integral_constant<int, NSUB>{});
        }
    };

    // Two-stage pipeline with one barrier per tile: after a tile's barrier every
    // wave has finished the previous tile, so the next tile can be transferred
    // into the buffer the previous one used while this one is consumed.
    issue_tile(0, Ks0, Vs0);
    for (int kt = 0; kt < T; kt += 2) {
        step(kt, Ks0, Vs0, Ks1, Vs1);
        if (kt + 1 < T) step(kt + 1, Ks1, Vs1, Ks0, Vs0);
    }

    // ---- normalise and store: lane holds query my_q, columns NT*row + n.
    l_run = sum_xor32(l_run);
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

// Compute units of the current device, queried once per device.
constexpr int kMaxDevices = 64;
std::atomic<int32_t> g_cus[kMaxDevices];
int32_t device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int32_t n = g_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
    g_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Eight waves (256 queries) per workgroup halve the K/V tile transfers per
// query; four waves keep small problems spread over the CUs.  One eight-wave
// workgroup fills a CU, so eight waves are used when that still gives at least
// two workgroups per CU (and D >= 64: a 32-key tile of D = 32 rows is too small
// to split over eight waves).  A problem too small to give every CU a
// four-wave workgroup runs on 16-query waves whose workgroups split the keys
// four ways (prefill_small.hip), and so does a causal one with fewer than
// four four-wave workgroups per CU unless a cache longer than the chunk makes
// its work nearly uniform: the heaviest query tiles then set the time, and
// splitting their keys shortens them (4096 tokens x 8 heads at d = 128:
// 549 -> 329 us; 2048 x 16 at d = 64: 159 -> 90 us).
template <int D, bool CAUSAL>
hipError_t launch_typed(const PrefillArgs &a, hipStream_t stream) {
    const int32_t BH = a.B * a.H;
    const int32_t xcd_remap = (BH % 8 == 0) ? 1 : 0;
    const int32_t tiles8 = (a.S + 255) / 256;
    const int32_t tiles4 = (a.S + 127) / 128;
    if constexpr (D >= 64) {
        if ((int64_t)BH * tiles8 >= 512) {
            dim3 grid((unsigned)(BH * tiles8));
            if constexpr (D >= 64)
                prefill_kernel<D, 8, CAUSAL, 64><<<grid, dim3(kWave * 8), 0, stream>>>(a, tiles8, xcd_remap);
            else
                prefill_kernel<D, 8, CAUSAL><<<grid, dim3(kWave * 8), 0, stream>>>(a, tiles8, xcd_remap);
            return hipGetLastError();
        }
    }
    const int64_t units4 = (int64_t)BH * tiles4;
    if (units4 < 256 || (CAUSAL && units4 < 1024 && prefill_cached_rows(a) < a.S))
        return launch_prefill_small(a, device_cus(), stream);
    dim3 grid((unsigned)(BH * tiles4));
    prefill_kernel<D, 4, CAUSAL><<<grid, dim3(kWave * 4), 0, stream>>>(a, tiles4, xcd_remap);
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
