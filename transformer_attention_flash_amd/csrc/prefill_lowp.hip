// prefill_lowp.hip -- reduced-precision fused prefill: the attention of
// [B, S, H * D] f32 activations with both products on 16-bit MFMA operands
// (binary16 or bfloat16) and everything else in f32.
//
// Semantics: the same attention as prefill.hip (trueno-gpu 0.4.11
// src/memory/resident/attention.rs, `batched_multihead_attention`;
// trustformers-core 0.2.0 src/gpu_ops/cuda/oxicuda/attention.rs,
// `attention_prefill_gpu_to_gpu`), computed the way trueno-gpu's
// `batched_gemm` does once k >= 64: GEMM operands rounded to fp16 for the
// tensor cores, products accumulated wider.  Here q, k and v are rounded to
// the 16-bit type (nearest, ties to even) as they are loaded; the scores
// S^T = K Q^T accumulate in f32 (a product of two 16-bit values is exact in
// f32); the online softmax runs in f32; the probabilities are rounded to the
// 16-bit type as the operand of O^T = V^T P^T, which accumulates in f32; the
// running sum and the final normalisation use the f32 probabilities.
//
// Layout of v_mfma_f32_32x32x16_{bf16,f16} (lane l, i = l % 32, h = l / 32):
// operand A supplies A[i][8h .. 8h+7], operand B supplies B[8h .. 8h+7][i],
// output register v holds D[8 (v / 4) + 4 h + (v % 4)][i].  The k order inside
// one instruction is free as long as both operands agree, which the P.V
// product uses: the score registers of a lane hold keys 4h .. 4h+3 and
// 8+4h .. 8+4h+3 of each 16-key half of a 32-key sub-tile, so those eight keys
// are that lane's k slots, the probabilities go from score registers to
// operand registers with a conversion only, and V^T is read at the same keys.
//
// Work decomposition as in prefill.hip: a workgroup owns 32 queries per
// query wave of one (b, h) (8 waves, or 4 for mid-size problems; small ones
// split 8 waves into key groups, see launch_typed), each wave with its Q slice
// (16-bit) and its 32 x D f32 output in registers.  K/V tiles
// of BN keys are loaded as f32 into registers one tile ahead, rounded, and
// written to a double-buffered LDS tile: K row-major (rows padded by 16 bytes:
// the 16-byte operand reads of 8 consecutive rows hit distinct banks), V
// transposed to [D][BN] with its 4-key groups paired and XOR-swizzled by
// dimension (one conflict-free 16-byte read per operand, see vswz).  One
// workgroup barrier per tile.  The softmax rescales lazily (see kLazy).
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr float kLazy = 8.0f;    // log2 headroom of the lazily rescaled softmax

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename T> struct Lp;
template <> struct Lp<__bf16> {
    typedef bf16x4 v4;
    typedef bf16x8 v8;
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, const f32x16 &c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Lp<_Float16> {
    typedef f16x4 v4;
    typedef f16x8 v8;
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, const f32x16 &c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// While a wave issues its matrix instructions it runs at a raised wave
// priority, so that the SIMD's other wave (in its softmax) does not delay
// them: the matrix pipe stays fed and the VALU work of the other wave fills
// the gaps.
__device__ __forceinline__ void mfma_priority(int p) {
    if (p)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// Key row (within a 32-key sub-tile) / output row of register v in lane-half h.
__device__ __forceinline__ int mrow(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

template <typename T, typename V4>
__device__ __forceinline__ V4 round4(f32x4 x) {
    return V4{(T)x[0], (T)x[1], (T)x[2], (T)x[3]};
}

// V^T layout in LDS: row dim holds the tile's BN keys in 4-key groups, group
// kq stored at position kq with bits 0 and 1 swapped, so the two groups one
// lane needs for a P.V step (4t + lh and 4t + 2 + lh of a 32-key sub-tile,
// see the layout note above) are adjacent; each such 16-byte pair p is
// stored at pair position p ^ vswz(dim % 32), which puts the 16-byte reads of
// any 8 or 16 consecutive dims (one LDS cycle) in distinct banks.  The
// swizzle repeats every 32 dims, so a lane's reads for its dims li + 32 n
// differ by constant offsets.
template <int BN>
__device__ __forceinline__ int vswz(int d) {
    return BN == 64 ? ((d ^ (d >> 3)) & 7) : (((d >> 1) ^ (d >> 3)) & 3);
}

// NW waves in KS groups: the NW / KS waves of a group own 32 queries each
// (BM = 32 NW / KS queries per workgroup) and group g walks the g-th of KS
// contiguous ranges of the key tiles of BN keys (KS > 1 only for small
// problems; the groups' softmax states are merged at the end).
// Two waves per SIMD either way.
//
// HM: head-major launch order (the query tiles of one (b, h) run next to each
// other, so they stream its K/V through the same L2 at about the same time);
// otherwise query-tile-major, heaviest causal tiles first.
template <int D, int NW, int KS, int BN, bool CAUSAL, typename T, bool HM = false, bool PAIR = false>
__global__ __launch_bounds__(kWave * NW, 8 / NW) void prefill_lowp_kernel(PrefillArgs a, int32_t n_qtiles,
                                                                          int32_t xcd_remap) {
    constexpr int QW = NW / KS;       // query waves per group
    constexpr int kThreads = kWave * QW;  // threads of one group (they stage its tiles)
    constexpr int BM = 32 * QW;
    typedef typename Lp<T>::v4 v4;
    typedef typename Lp<T>::v8 v8;
    constexpr int NT = D / 32;   // 32-row tiles of O^T
    constexpr int KK = D / 16;   // k steps of the score product
    constexpr int NSUB = BN / 32;  // 32-key sub-tiles per tile
    constexpr int KP = D + 8;    // LDS pitch of a K row (elements)
    // Staging: a thread moves blocks of 4 keys x 4 dims of K and of V.
    constexpr int NBLK = (BN / 4) * (D / 4);
    constexpr int BPT = (NBLK + kThreads - 1) / kThreads;  // blocks per thread
    static_assert(BN == 32 || BN == 64, "tile of 32 or 64 keys");
    static_assert(NW % KS == 0, "key groups of whole query waves");

    __shared__ __attribute__((aligned(16))) T Ks0[KS * BN * KP];
    __shared__ __attribute__((aligned(16))) T Vt0[KS * D * BN];
    __shared__ __attribute__((aligned(16))) T Ks1[KS * BN * KP];
    __shared__ __attribute__((aligned(16))) T Vt1[KS * D * BN];
    // Key-group merge: the parked wave states go to the K/V tile buffers
    // when they fit there, else to an array of their own.
    constexpr int SLOT = kWave * (16 * NT + 2);  // floats of one parked wave state
    constexpr int PK = (int)(KS * BN * KP * sizeof(T)) / (SLOT * 4);  // slots per K buffer
    constexpr int PV = (int)(KS * D * BN * sizeof(T)) / (SLOT * 4);   // slots per V buffer
    constexpr bool kParkInTiles = 2 * (PK + PV) >= (KS - 1) * QW;
    __shared__ float Red[KS > 1 && !kParkInTiles ? (KS - 1) * QW * SLOT : 1];

    // ---- block -> (b, h, query tile): heavy causal tiles first; with
    // xcd_remap the query tiles of one (b, h) share an XCD (and its L2).
    // PAIR (causal): the workgroup takes query tiles T-1-j and j of one (b, h)
    // (T = n_qtiles), so every workgroup has the same number of key tiles, and
    // the P = ceil(T/2) workgroups of a (b, h) run side by side on one XCD.
    // The first tile of the pair walks its keys upwards and the second
    // downwards from its diagonal: all P workgroups then read the same K/V
    // tile at about the same time in both phases, and it comes from HBM once.
    static_assert(!PAIR || (CAUSAL && KS == 1), "pairs: causal, one key group");
    const int BH = a.B * a.H;
    int bh, qt_first, qt_second = -1;
    {
        const int bid = blockIdx.x;
        if constexpr (PAIR) {
            const int P = (n_qtiles + 1) / 2;
            int j;
            if (xcd_remap) {
                const int x = bid % 8, t = bid / 8;
                bh = 8 * (t / P) + x;
                j = t % P;
            } else {
                bh = bid / P;
                j = bid % P;
            }
            qt_first = n_qtiles - 1 - j;
            if (j < qt_first) qt_second = j;
        } else {
            int rank;
            if (xcd_remap) {
                const int per_xcd_bh = BH / 8;
                const int x = bid % 8, t = bid / 8;
                bh = 8 * (HM ? t / n_qtiles : t % per_xcd_bh) + x;
                rank = HM ? t % n_qtiles : t / per_xcd_bh;
            } else {
                bh = HM ? bid / n_qtiles : bid % BH;
                rank = HM ? bid % n_qtiles : bid / BH;
            }
            qt_first = CAUSAL ? n_qtiles - 1 - rank : rank;
        }
    }
    const int b = bh / a.H;
    const int hd = bh % a.H;
    const int S = a.S;
    const size_t row_stride = (size_t)a.H * D;
    const size_t head_base = (size_t)b * S * row_stride + (size_t)hd * D;
    const float *__restrict__ qg = a.q + head_base;
    const float *__restrict__ kg = a.k + head_base;
    const float *__restrict__ vg = a.v + head_base;

    const int tid_all = threadIdx.x;
    const int grp = tid_all / kThreads;   // key group of this wave
    const int tid = tid_all % kThreads;   // thread index within the group
    const int wave = tid >> 6;            // query wave within the group
    const int lane = tid & 63;
    const int li = lane & 31;
    const int lh = lane >> 5;
    constexpr int NPH = PAIR ? 2 : 1;
#pragma unroll 1
    for (int ph = 0; ph < NPH; ++ph) {
        const int qt = ph == 0 ? qt_first : qt_second;
        if (qt < 0) break;
        const bool desc = PAIR && ph == 1;  // walk the key tiles from the last one down
        const int q0 = qt * BM;
        const int qw0 = q0 + 32 * wave;
        const int my_q = qw0 + li;

        // ---- Q^T operand: query my_q, dims 16 kk + 8 lh .. +7, rounded.  For a
        // negative scale the query is negated first (rounding is symmetric, so
        // the scores are exactly negated) and |scale| is used: the softmax then
        // always multiplies by a non-negative factor and can take its maximum on
        // the raw scores.
        const float qsign = a.scale < 0.f ? -1.f : 1.f;
        const float qsa = fabsf(a.scale) * kLog2e;  // raw scores to log2 units
        v8 qop[KK];  // filled below, once the first K/V tile's loads are in flight
        auto load_q = [&]() {
            const bool ok = my_q < S;
            const float *qp = qg + (size_t)(ok ? my_q : 0) * row_stride + 8 * lh;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const f32x4 x0 = ok ? *reinterpret_cast<const f32x4 *>(qp + 16 * kk) : f32x4{0, 0, 0, 0};
                const f32x4 x1 = ok ? *reinterpret_cast<const f32x4 *>(qp + 16 * kk + 4) : f32x4{0, 0, 0, 0};
                const v4 r0 = round4<T, v4>(x0 * qsign), r1 = round4<T, v4>(x1 * qsign);
                qop[kk] = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        };

        f32x16 o[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) o[n] = f32x16{};
        float m_run = kNegBig;
        float l_run = 0.f;

        const int n_ktiles_all = (S + BN - 1) / BN;
        const int n_ktiles = CAUSAL ? min(n_ktiles_all, (min(q0 + BM, S) - 1) / BN + 1) : n_ktiles_all;
        const int TG = (n_ktiles + KS - 1) / KS;  // key tiles per group; group grp owns tiles grp*TG ..
        const int gt0 = grp * TG;

        // ---- staging: block blk = (key quad kq, dim chunk c).  Element offsets
        // within a tile are fixed per thread; a tile adds a uniform base, so a
        // load is a 32-bit offset from a scalar base.  In the last, partial tile
        // rows past S read row S - 1 (in bounds; their scores are masked and their
        // probabilities are exactly 0).
        f32x4 kst[BPT][4], vst[BPT][4];
        uint32_t goff[BPT];  // element offset of row 4 kq, chunk c, within a tile (row 4 kq + j: + j row_stride)
        int rowq[BPT];       // 4 kq
        const uint32_t rs32 = (uint32_t)row_stride;
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int blk = tid + kThreads * u;
            const int c = blk % (D / 4), kq = blk / (D / 4);
            rowq[u] = 4 * kq;
            goff[u] = (uint32_t)((size_t)(4 * kq) * row_stride + 4 * c);
        }
        auto load_tile = [&](int kt) {
            kt += gt0;
            if (desc) kt = n_ktiles - 1 - kt;
            if (KS > 1 && kt >= n_ktiles) return;  // past this group's range (uniform per group)
            const size_t tbase = (size_t)kt * BN * row_stride;
            const float *kt_g = kg + tbase;
            const float *vt_g = vg + tbase;
            const bool partial = kt * BN + BN > S;  // uniform
#pragma unroll
            for (int u = 0; u < BPT; ++u) {
                const int blk = tid + kThreads * u;
                if (NBLK % kThreads == 0 || blk < NBLK) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        uint32_t off = goff[u] + (uint32_t)j * rs32;
                        if (partial) {
                            const int over = kt * BN + rowq[u] + j - (S - 1);
                            if (over > 0) off -= (uint32_t)((size_t)over * row_stride);
                        }
                        kst[u][j] = *reinterpret_cast<const f32x4 *>(kt_g + off);
                        vst[u][j] = *reinterpret_cast<const f32x4 *>(vt_g + off);
                    }
                }
            }
        };
        auto write_tile = [&](T *Ks, T *Vt) {
            Ks += grp * BN * KP;
            Vt += grp * D * BN;
#pragma unroll
            for (int u = 0; u < BPT; ++u) {
                const int blk = tid + kThreads * u;
                if (NBLK % kThreads == 0 || blk < NBLK) {
                    const int c = blk % (D / 4), kq = blk / (D / 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<v4 *>(Ks + (4 * kq + j) * KP + 4 * c) = round4<T, v4>(kst[u][j]);
                    const int pq = (kq & ~3) | ((kq & 1) << 1) | ((kq >> 1) & 1);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int dim = 4 * c + e;
                        const f32x4 col = {vst[u][0][e], vst[u][1][e], vst[u][2][e], vst[u][3][e]};
                        *reinterpret_cast<v4 *>(Vt + dim * BN + 8 * ((pq >> 1) ^ vswz<BN>(dim & 31)) + 4 * (pq & 1)) =
                            round4<T, v4>(col);
                    }
                }
            }
        };

        auto compute = [&](int kt, const T *Ks, const T *Vt) {
            kt += gt0;
            if (desc) kt = n_ktiles - 1 - kt;
            if (KS > 1 && kt >= n_ktiles) return;  // this group's range is done (uniform per group)
            Ks += grp * BN * KP;
            Vt += grp * D * BN;
            const int kt0 = kt * BN;  // first key of the tile
            if (CAUSAL && kt0 > qw0 + 31) return;  // wave-uniform: whole tile above this wave's diagonal
            // S^T = K Q^T for the NSUB 32-key sub-tiles of the tile; lane supplies
            // K[key 32 sub + li][16 kk + 8 lh .. +7].  One sub-tile: all its K
            // operands are read from LDS before the MFMA chain starts, so the chain
            // does not wait on an LDS round trip per step.  Two sub-tiles: their
            // chains are independent and interleaved instead.
            f32x16 s[NSUB];
            if constexpr (NSUB == 1) {
                v8 kop[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    kop[kk] = *reinterpret_cast<const v8 *>(Ks + li * KP + 8 * lh + 16 * kk);
                // Keep the reads ahead of the chain (the scheduler would otherwise
                // sink each read next to its MFMA to save registers).
                __builtin_amdgcn_sched_barrier(0);
                // Two independent accumulation chains (even and odd k steps).
                f32x16 s1 = f32x16{};
                s[0] = f32x16{};
                mfma_priority(1);
#pragma unroll
                for (int kk = 0; kk < KK; kk += 2) {
                    s[0] = Lp<T>::mfma(kop[kk], qop[kk], s[0]);
                    if (kk + 1 < KK) s1 = Lp<T>::mfma(kop[kk + 1], qop[kk + 1], s1);
                }
                mfma_priority(0);
                s[0] += s1;
            } else {
#pragma unroll
                for (int sub = 0; sub < NSUB; ++sub) s[sub] = f32x16{};
                mfma_priority(1);
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                    for (int sub = 0; sub < NSUB; ++sub)
                        s[sub] = Lp<T>::mfma(
                            *reinterpret_cast<const v8 *>(Ks + (32 * sub + li) * KP + 8 * lh + 16 * kk), qop[kk],
                            s[sub]);
                mfma_priority(0);
            }

            // Online softmax over the tile's BN keys in raw score units: the
            // scale (>= 0, see qsa) is folded into the exponent's FMA.
            const bool need_mask = (kt0 + BN > S) || (CAUSAL && kt0 + BN - 1 > qw0);
            if (need_mask) {
#pragma unroll
                for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int key = kt0 + 32 * sub + mrow(v, lh);
                        if (key >= S || (CAUSAL && key > my_q)) s[sub][v] = -INFINITY;
                    }
            }
            float mx = s[0][0];
#pragma unroll
            for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[sub][v]);
            mx = max_xor32(mx);
            // Lazy rescaling: the reference maximum m_run moves (and O and l are
            // rescaled) only when a lane's scores would exceed it by more than
            // 2^kLazy; otherwise the probabilities are taken against the stale
            // reference and stay below 2^kLazy, well inside f32 and both 16-bit
            // formats.  The decision is wave-uniform, so most tiles skip the
            // 16 * NT multiplies of the rescale.
            if (__any((mx - m_run) * qsa > kLazy)) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = fast_exp2((m_run - m_new) * qsa);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int n = 0; n < NT; ++n) o[n] *= alpha;
            }
            const float mb = m_run * qsa;
            float psum = 0.f;
            // Probabilities: summed in f32 and rounded at once to the P.V operands
            // (score registers 8t .. 8t + 7 of a sub-tile are the k slots of its
            // step t).  Masked scores give exact zeros (also for scale 0, where the
            // exponent alone would not); tiles without masked keys skip the test.
            v8 pop[NSUB][2];
            auto probabilities = [&](auto masked) {
#pragma unroll
                for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        f32x4 pr[2];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float sv = s[sub][8 * t + j];
                            float pv = fast_exp2(fmaf(sv, qsa, -mb));
                            if constexpr (decltype(masked)::value) pv = (sv == -INFINITY) ? 0.f : pv;
                            pr[j / 4][j % 4] = pv;
                            psum += pv;
                        }
                        pop[sub][t] = __builtin_shufflevector(round4<T, v4>(pr[0]), round4<T, v4>(pr[1]), 0, 1, 2, 3, 4,
                                                              5, 6, 7);
                    }
            };
            if (need_mask)
                probabilities(std::true_type{});
            else
                probabilities(std::false_type{});
            l_run += psum;

            // O^T += V^T P^T over the 16-key halves t of each sub-tile: this lane's
            // k slots are keys 16t + 4lh + (0..3) and 16t + 8 + 4lh + (0..3).  All
            // V operands of a sub-tile are read before its MFMAs, as for K.
#pragma unroll
            for (int sub = 0; sub < NSUB; ++sub) {
                __builtin_amdgcn_sched_barrier(0);  // not above the previous sub-tile's MFMAs (registers)
                v8 vop[2][NT];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int pair = 4 * sub + 2 * t + lh;  // key groups 4t + lh and 4t + 2 + lh of the sub-tile
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        const int dim = 32 * n + li;
                        vop[t][n] = *reinterpret_cast<const v8 *>(Vt + dim * BN + 8 * (pair ^ vswz<BN>(li)));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                mfma_priority(1);
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int n = 0; n < NT; ++n) o[n] = Lp<T>::mfma(vop[t][n], pop[sub][t], o[n]);
                mfma_priority(0);
            }
        };

        // ---- pipeline: tile kt+1 is in registers while tile kt is consumed from
        // LDS; after the barrier that ends tile kt, tile kt+2's loads go out.
        load_tile(0);
        load_q();  // the Q and first-tile loads overlap: one memory round trip, not two
        write_tile(Ks0, Vt0);
        __syncthreads();
        if (TG > 1) load_tile(1);
        for (int kt = 0; kt < TG; kt += 2) {
            compute(kt, Ks0, Vt0);
            if (kt + 1 < TG) write_tile(Ks1, Vt1);
            __syncthreads();
            if (kt + 2 < TG) load_tile(kt + 2);
            if (kt + 1 < TG) {
                compute(kt + 1, Ks1, Vt1);
                if (kt + 2 < TG) write_tile(Ks0, Vt0);
                __syncthreads();
                if (kt + 3 < TG) load_tile(kt + 3);
            }
        }

        // ---- merge the key groups: groups 1.. park (reference max, partial sum,
        // output) of each lane, group 0 folds them in.  Every group's softmax
        // state is relative to its own reference max m (probabilities
        // 2^((s - m) qsa)), so the usual rescaling applies.
        if constexpr (KS > 1) {
            // The tile buffers are free: the last tile step ended in a barrier.
            auto slot_ptr = [&](int sl) -> float * {
                if (!kParkInTiles) return Red + sl * SLOT;
                if (sl < PK) return reinterpret_cast<float *>(Ks0) + sl * SLOT;
                sl -= PK;
                if (sl < PV) return reinterpret_cast<float *>(Vt0) + sl * SLOT;
                sl -= PV;
                if (sl < PK) return reinterpret_cast<float *>(Ks1) + sl * SLOT;
                return reinterpret_cast<float *>(Vt1) + (sl - PK) * SLOT;
            };
            if (grp > 0) {
                float *dst = slot_ptr((grp - 1) * QW + wave) + lane;
#pragma unroll
                for (int n = 0; n < NT; ++n)
#pragma unroll
                    for (int v = 0; v < 16; ++v) dst[(16 * n + v) * kWave] = o[n][v];
                dst[16 * NT * kWave] = m_run;
                dst[(16 * NT + 1) * kWave] = l_run;
            }
            __syncthreads();
            if (grp > 0) return;
#pragma unroll
            for (int g = 1; g < KS; ++g) {
                const float *src = slot_ptr((g - 1) * QW + wave) + lane;
                const float m_g = src[16 * NT * kWave];
                const float m_new = fmaxf(m_run, m_g);
                const float keep = fast_exp2((m_run - m_new) * qsa), take = fast_exp2((m_g - m_new) * qsa);
                l_run = l_run * keep + src[(16 * NT + 1) * kWave] * take;
#pragma unroll
                for (int n = 0; n < NT; ++n)
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[n][v] = o[n][v] * keep + src[(16 * n + v) * kWave] * take;
                m_run = m_new;
            }
        }

        // ---- normalise and store: lane holds query my_q, dims 32 n + 8 g + 4 lh + (0..3).
        l_run = sum_xor32(l_run);
        if (my_q < S) {
            const float inv = 1.0f / l_run;
            float *op = a.out + head_base + (size_t)my_q * row_stride + 4 * lh;
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<f32x4 *>(op + 32 * n + 8 * g) =
                        f32x4{o[n][4 * g] * inv, o[n][4 * g + 1] * inv, o[n][4 * g + 2] * inv, o[n][4 * g + 3] * inv};
        }
    }
}

// Eight waves (256 queries) per workgroup halve the K/V reads and conversions
// per query; four waves keep smaller problems spread over the CUs.  One
// eight-wave workgroup fills a CU, so eight waves are used when that still
// gives at least two workgroups per CU.
// Workgroups of `threads` threads of `kernel` that the current device holds
// at once (CUs x resident workgroups per CU, at least 1 per CU), queried once
// per device and kernel: `cache` is that kernel's per-device slot.
constexpr int kMaxDevices = 64;

int64_t device_slots(const void *kernel, int threads, std::atomic<int64_t> (&cache)[kMaxDevices]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int64_t n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    n = (int64_t)cus * per_cu;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Causal prefill over BH (batch, head) rows of T query tiles, each tile with
// `p` tile-sized blocks of cached keys in front: whether workgroups that take
// query tiles T-1-j and j (the same 2p + T + 1 key blocks each, in
// ceil(BH ceil(T/2) / slots) rounds) finish no later than single tiles taken
// heaviest first (at best the heaviest tile, p + T blocks, or the mean load
// per slot).  Ties go to the pairs: their workgroups read a row's K/V about
// once between them.
bool pair_query_tiles(int64_t BH, int64_t T, int64_t p, int64_t slots) {
    if (T < 2 || slots < 1) return false;
    const int64_t paired = (BH * ((T + 1) / 2) + slots - 1) / slots * (2 * p + T + 1);
    const int64_t total = BH * (p * T + T * (T + 1) / 2);
    const int64_t single = total / slots + (total % slots != 0);
    return paired <= (single > p + T ? single : p + T);
}

template <int D, bool CAUSAL, typename T>
hipError_t launch_typed(const PrefillArgs &a, hipStream_t stream) {
    const int32_t BH = a.B * a.H;
    const int32_t xcd_remap = (BH % 8 == 0) ? 1 : 0;
    const int32_t tiles8 = (a.S + 255) / 256;
    if ((int64_t)BH * tiles8 >= 512) {
        // Non-causal: head-major order (a (b, h)'s query tiles share its K/V in
        // L2: B=4 S=2048 H=32 d=128 412 -> 363 us).  Causal: pairs of query
        // tiles when they fill the device as well as single tiles do (B=4
        // S=2048 H=32 d=128: HBM reads 1.00 -> 0.55 GB, about 2% faster), else
        // single tiles heaviest first (head-major single tiles would run the
        // heavy tiles of the last heads last).
        if constexpr (CAUSAL) {
            static std::atomic<int64_t> pair_slots[kMaxDevices];
            const int64_t slots = device_slots(
                (const void *)prefill_lowp_kernel<D, 8, 1, 64, true, T, false, true>, kWave * 8, pair_slots);
            if (pair_query_tiles(BH, tiles8, 0, slots)) {
                dim3 grid((unsigned)(BH * ((tiles8 + 1) / 2)));
                prefill_lowp_kernel<D, 8, 1, 64, true, T, false, true>
                    <<<grid, dim3(kWave * 8), 0, stream>>>(a, tiles8, xcd_remap);
            } else {
                dim3 grid((unsigned)(BH * tiles8));
                prefill_lowp_kernel<D, 8, 1, 64, true, T><<<grid, dim3(kWave * 8), 0, stream>>>(a, tiles8, xcd_remap);
            }
        } else {
            dim3 grid((unsigned)(BH * tiles8));
            prefill_lowp_kernel<D, 8, 1, 64, false, T, true><<<grid, dim3(kWave * 8), 0, stream>>>(a, tiles8,
                                                                                                 xcd_remap);
        }
        return hipGetLastError();
    }
    const int32_t tiles4 = (a.S + 127) / 128;
    if ((int64_t)BH * tiles4 < 256) {
        // Too small to give every CU a workgroup: split each workgroup's keys
        // over groups of query waves (causal: the groups split the tiles the
        // workgroup's queries see, heaviest workgroups first).  d <= 64: 4
        // groups of 2 waves (64 queries per workgroup); d = 128: 2 groups of 4
        // (128 queries; 4 groups would need twice the staging registers).
        if constexpr (D <= 64) {
            const int32_t tiles2 = (a.S + 63) / 64;
            dim3 grid((unsigned)(BH * tiles2));
            prefill_lowp_kernel<D, 8, 4, 32, CAUSAL, T><<<grid, dim3(kWave * 8), 0, stream>>>(a, tiles2, xcd_remap);
        } else {
            dim3 grid((unsigned)(BH * tiles4));
            prefill_lowp_kernel<D, 8, 2, 32, CAUSAL, T><<<grid, dim3(kWave * 8), 0, stream>>>(a, tiles4, xcd_remap);
        }
        return hipGetLastError();
    }
    dim3 grid((unsigned)(BH * tiles4));
    prefill_lowp_kernel<D, 4, 1, 32, CAUSAL, T><<<grid, dim3(kWave * 4), 0, stream>>>(a, tiles4, xcd_remap);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const PrefillArgs &a, hipStream_t stream) {
    switch (a.D) {
        case 32: return a.causal ? launch_typed<32, true, T>(a, stream) : launch_typed<32, false, T>(a, stream);
        case 64: return a.causal ? launch_typed<64, true, T>(a, stream) : launch_typed<64, false, T>(a, stream);
        case 128: return a.causal ? launch_typed<128, true, T>(a, stream) : launch_typed<128, false, T>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill_lowp(const PrefillArgs &a, int32_t precision, hipStream_t stream) {
    if (precision == ATTN_PREC_BF16) return launch_t<__bf16>(a, stream);
    if (precision == ATTN_PREC_FP16) return launch_t<_Float16>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
