// prefill_small.hip -- the prefill of problems too small to give every CU a
// workgroup of the main kernel, and of mid-size causal ones (head_dim 32, 64
// or 128; behind a KV cache too), on 16-query waves and v_mfma_f32_16x16x4_f32.
//
// Semantics: the attention of prefill.hip (trueno-gpu 0.4.11
// src/memory/resident/attention.rs, `batched_multihead_attention`: per head,
// softmax(scale Q K^T) V over the interleaved [B, S, H * D] rows; with the
// causal mask of trustformers-core 0.2.0 src/gpu_ops/cuda/oxicuda/attention.rs,
// `attention_prefill_gpu_to_gpu`: query i sees keys 0..=i; behind a cache of
// P rows, keys from the cache slab and query i sees rows 0..P+i); this file
// only changes how the work is cut.
//
// Why: the time of a small problem is that of its most loaded CU.  With
// 32-query waves a workgroup covers at least 32 queries of one head, so a
// head of S = 1500 queries gives units of 32 (47 per head) or 64 (24 per
// head): 8 heads make 376 or 192 units, i.e. two units on some of the 256
// CUs, or 192 CUs busy.  16-query waves allow units of 16, 32, 48 or 64
// queries; 48 gives 32 units per head, 256 in all, one per CU.
//
// Work decomposition: a workgroup owns BM = 16 QW queries of one (b, h) and
// has QW query waves in each of 4 key groups; group g walks the g-th quarter
// of the key tiles (32 keys each, 16 at head_dim 128) the workgroup's queries
// can see, its QW waves sharing every tile, and the groups' partial softmax
// states are merged through LDS at the end.  With the causal mask, a wave
// skips the tiles wholly above its diagonal, the diagonal tile is masked per
// element, and the workgroups with the most visible keys are dispatched
// first (for mid-size causal problems the key split also shortens the
// heaviest workgroups, which set the time there).  K and V
// tiles go from HBM straight into double-buffered LDS (global_load_lds), all
// four groups' tiles moved by all the workgroup's waves, one barrier per tile.
//
// Register layouts of v_mfma_f32_16x16x4_f32 (lane l, i = l % 16, k = l / 16):
// operand A supplies A[i][k], operand B supplies B[k][i], and output register
// r holds D[4 k + r][i].  Scores are formed transposed, S^T = K Q^T (rows =
// keys, columns = queries), with head dim (D / 4) k + j at step j, so each lane
// reads its K row and holds its Q row as contiguous dims.  Output register r
// of a 16-key score tile is then the operand-B value its lane supplies at step
// r of O^T = V^T P^T (key 4 k + r).  Row i of output tile n (NT = D / 16
// tiles) stands for dim NT i + n, or at head_dim 128 for dim
// 4 i + 64 (n / 4) + n % 4, so a lane's V operands for one step are NT
// contiguous floats of one V row, or two runs of 4.
#include <algorithm>
#include <map>
#include <mutex>
#include <queue>
#include <tuple>
#include <vector>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int SKS = 4;  // key groups per workgroup
constexpr float kLazySmall = 8.0f;  // log2 headroom of the lazily rescaled softmax

// Keys per LDS tile: two 16-key MFMA tiles at d <= 64, one at d = 128 (LDS:
// the four groups' double-buffered K and V tiles take 128 KiB either way).
template <int D>
constexpr int tile_keys() { return D == 128 ? 16 : 32; }

// Head dim that row i of 16-row output tile n stands for (NT = D / 16 tiles).
template <int D>
__device__ __forceinline__ constexpr int odim(int i, int n) {
    return D >= 64 ? 4 * i + 64 * (n / 4) + (n % 4) : 2 * i + n;
}

__device__ __forceinline__ f32x4 mfma16x4(float a, float b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One 16-byte global -> LDS transfer per lane (global_load_lds_dwordx4): lane l's
// 16 bytes land at lds_base + 16 l, lds_base being uniform over the wave.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void dma16_small(const float *src, float *lds_base) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src), (lds_void_t *)lds_base, 16, 0, 0);
}

// Wait until this wave has no global loads (including LDS transfers) in flight.
__device__ __forceinline__ void wait_vmem_all_small() {
    // s_waitcnt vmcnt(0), expcnt/lgkmcnt unconstrained (7 and 15).
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

template <int D, int QW, bool CAUSAL>
__global__ __launch_bounds__(kWave * QW * SKS, 1) void prefill_small_kernel(PrefillArgs a, int32_t n_qtiles,
                                                                          int32_t xcd_remap) {
    constexpr int SBN = tile_keys<D>();  // keys per LDS tile
    constexpr int TPT = SBN / 16;        // 16-key MFMA tiles per LDS tile
    constexpr int NWV = QW * SKS;         // waves per workgroup
    constexpr int BM = 16 * QW;           // queries per workgroup
    constexpr int KC = D / 4;             // 16-byte chunks per K/V row
    constexpr int RPI = kWave / KC;       // rows moved by one wave-wide 1 KiB transfer
    constexpr int PPT = SBN / RPI;        // transfers per tensor per group tile
    constexpr int NPIECE = SKS * 2 * PPT; // transfers per workgroup per tile step
    constexpr int SWZ = (KC < 16 ? KC : 16) - 1;  // K chunk swizzle mask
    constexpr int NT = D / 16;            // 16-row tiles of O^T; floats per lane per V row
    constexpr int QJ = D / 4;             // k steps of the score product
    constexpr int VW = NT < 4 ? NT : 4;   // floats per V / output vector
    constexpr int NVW = NT / VW;          // vectors per lane per V row
    typedef typename VecN<VW>::type vec_t;
    static_assert(D == 32 || D == 64 || D == 128, "head_dim 32, 64 or 128");
    static_assert(RPI * KC == kWave && PPT * RPI == SBN, "tile transfers");
    constexpr bool kPreloadK = !(D == 128 && QW == 4);
    static_assert(kPreloadK || TPT == 1, "chunk-by-chunk K reads use one 16-key tile");

    // Double-buffered K/V tiles: each buffer holds the four groups' K tiles
    // (SBN x D each), then their V tiles.  K chunk c of row r sits at chunk
    // position c ^ (r & SWZ), so the 16 rows of one score operand read fall
    // in distinct banks; V rows are read whole by 16 lanes and are stored as
    // they are.  The two buffers are separate objects, so the compiler sees
    // that a transfer into one does not alias reads of the other.
    __shared__ __attribute__((aligned(16))) float KV0[2 * SKS * SBN * D];
    __shared__ __attribute__((aligned(16))) float KV1[2 * SKS * SBN * D];

    // ---- block -> (b, h, query tile); heavy causal tiles first, and with
    // xcd_remap the query tiles of one (b, h) stay on one XCD (blocks are
    // dealt to the 8 XCDs round-robin).
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
    const size_t row_stride = (size_t)a.H * D;
    const size_t head_base = (size_t)b * S * row_stride + (size_t)h * D;
    const float *__restrict__ qg = a.q + head_base;
    // Keys: the interleaved activations (key j = token j), or the cache slab of
    // KV head h / (H / Hkv) (key j = cache row j, queries offset by P).
    const int P = a.cached ? a.pos.v[b] : 0;  // key index of query 0
    const int Sk = P + S;                      // keys a query can reach at most
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
    const int li = lane & 15;   // query column / key row within a 16 x 16 tile
    const int lk = lane >> 4;   // k-slot of the MFMA operands
    const int qwave = wave % QW;
    const int grp = wave / QW;
    const int q0 = qt * BM;               // the workgroup's first query
    const int qw0 = q0 + 16 * qwave;      // this wave's first query
    const int my_q = qw0 + li;

    // ---- Q operand, pre-scaled so scores are in log2 units: lane supplies
    // Q[my_q][(D / 4) lk + j] at step j (behind a cache with a rotary
    // embedding, first turned to the query's position P + my_q; the partner
    // dims half a rotary width away come from the same row).
    const float qs = a.scale * kLog2e;
    float qreg[QJ];
    {
        const bool ok = my_q < S;
        const float *qrow = qg + (size_t)(ok ? my_q : 0) * row_stride;
        const float *qp = qrow + QJ * lk;
#pragma unroll
        for (int jj = 0; jj < QJ / 4; ++jj) {
            f32x4 v4 = ok ? *reinterpret_cast<const f32x4 *>(qp + 4 * jj) : f32x4{0, 0, 0, 0};
            if (a.rope.rot > 0) {
                const int l0 = QJ * lk + 4 * jj;
                const int pl = l0 < a.rope.half ? l0 + a.rope.half : l0 - a.rope.half;
                const f32x4 part =
                    (ok && l0 < a.rope.rot) ? *reinterpret_cast<const f32x4 *>(qrow + pl) : f32x4{0, 0, 0, 0};
                v4 = rope_rotate4(v4, part, l0, P + my_q, a.rope);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) qreg[4 * jj + e] = v4[e] * qs;
        }
    }

    f32x4 o[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = f32x4{0, 0, 0, 0};
    float m_run = kNegBig;
    float l_run = 0.f;

    const int n_ktiles_all = (Sk + SBN - 1) / SBN;
    const int n_ktiles = CAUSAL ? min(n_ktiles_all, (P + min(q0 + BM, S) - 1) / SBN + 1) : n_ktiles_all;
    const int T = (n_ktiles + SKS - 1) / SKS;  // tile steps; group g owns tiles g T .. g T + T - 1
    const int gt0 = grp * T;

    // Tile step kt moves tile g T + kt of every group g that has one: the
    // workgroup's waves share the NPIECE 1 KiB transfers, wave w taking pieces
    // w, w + NWV, ...  A piece's lane addresses only move by whole tiles from
    // step to step, so they are set up once: the lane's source in tile 0, its
    // row within the tile, and the piece's group and LDS offset.  Keys past Sk
    // read row Sk - 1 (in bounds); their scores are masked and their
    // probabilities are exactly 0, so the values never matter.
    constexpr int MAXP = (NPIECE + NWV - 1) / NWV;  // pieces per wave at most
    const float *psrc[MAXP];
    int prow[MAXP];
    int pg[MAXP], pdst[MAXP];  // pg = SKS: no such piece
#pragma unroll
    for (int u = 0; u < MAXP; ++u) {
        const int p = wave + NWV * u;
        const int g = p / (2 * PPT);
        const int is_v = (p / PPT) % 2;
        const int pi = p % PPT;
        const int row = pi * RPI + lane / KC;
        const int chunk = lane % KC;
        prow[u] = row;
        pg[u] = p < NPIECE ? g : SKS;
        pdst[u] = (is_v ? SKS * SBN * D : 0) + g * SBN * D + pi * kWave * 4;
        psrc[u] = (is_v ? vg + 4 * chunk : kg + 4 * (chunk ^ (row & SWZ)));
    }
    auto issue_tile = [&](int kt, float *kv_dst) {
#pragma unroll
        for (int u = 0; u < MAXP; ++u) {
            if (pg[u] >= SKS) continue;
            const int tile = pg[u] * T + kt;
            if (tile >= n_ktiles) continue;
            const int key = min(tile * SBN + prow[u], Sk - 1);
            dma16_small(psrc[u] + (size_t)key * kv_stride, kv_dst + pdst[u]);
        }
    };

    // This lane's V operand offset within a buffer (group, k-slot and column
    // folded in once): the reads below are then one variable and one
    // constant step from the buffer itself, which keeps the compiler able to
    // see which buffer they read (and not wait for the other buffer's
    // transfers in flight).
    const int vlane = SKS * SBN * D + grp * SBN * D + 4 * lk * D + odim<D>(li, 0);
    auto compute = [&](int kt, const float *Kt, const float *KVb) {
        const int tile = gt0 + kt;
        if (tile >= n_ktiles) return;  // this group's range is done (wave-uniform)
        if (CAUSAL && tile * SBN > P + qw0 + 15) return;  // whole tile above this wave's diagonal
        Kt += grp * SBN * D;
        const int ks0 = tile * SBN;

        // S^T for the tile's 16-key MFMA tiles in two independent chains (the
        // two tiles, or with one tile its even and odd k steps).  The K
        // operands are read before the chains start, or at d = 128 with 16
        // waves (128 registers a lane) chunk by chunk.
        auto kchunk = [&](int t, int jj) -> f32x4 {
            const int row = 16 * t + li;
            const int chunk = (QJ / 4) * lk + jj;
            return *reinterpret_cast<const f32x4 *>(Kt + row * D + 4 * (chunk ^ (row & SWZ)));
        };
        f32x4 acc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
        if constexpr (kPreloadK) {
            f32x4 kv[TPT][QJ / 4];
#pragma unroll
            for (int jj = 0; jj < QJ / 4; ++jj)
#pragma unroll
                for (int t = 0; t < TPT; ++t) kv[t][jj] = kchunk(t, jj);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int jj = 0; jj < QJ / 4; ++jj)
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int t = 0; t < TPT; ++t) {
                        const int c = TPT == 2 ? t : (jj & 1);
                        acc[c] = mfma16x4(kv[t][jj][e], qreg[4 * jj + e], acc[c]);
                    }
        } else {
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int jj = 0; jj < QJ / 4; ++jj) {
                const f32x4 k4 = kchunk(0, jj);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[jj & 1] = mfma16x4(k4[e], qreg[4 * jj + e], acc[jj & 1]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        f32x4 s[TPT];
        if constexpr (TPT == 2) {
            s[0] = acc[0];
            s[1] = acc[1];
        } else {
            s[0] = acc[0] + acc[1];
        }

        // Keys past Sk (the last tile) and, causal, keys after the query's
        // position P + q are masked.  A lane whose keys are all masked keeps
        // its state: the running max stays put (finite) and the probabilities
        // are 0.
        if (ks0 + SBN > Sk || (CAUSAL && ks0 + SBN - 1 > P + qw0)) {
#pragma unroll
            for (int t = 0; t < TPT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = ks0 + 16 * t + 4 * lk + r;
                    if (key >= Sk || (CAUSAL && key > P + my_q)) s[t][r] = -INFINITY;
                }
        }
        float mx = s[0][0];
#pragma unroll
        for (int t = 0; t < TPT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[t][r]);
        mx = max4(mx);
        // Lazy rescaling: the reference maximum m_run moves (and O and l are
        // rescaled) only when a lane's scores would exceed it by more than
        // 2^kLazySmall; otherwise the probabilities are taken against the
        // stale reference (below 2^kLazySmall, exact enough in f32).  The
        // decision is wave-uniform, so most tiles skip the rescale.
        if (__any(mx - m_run > kLazySmall)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int n = 0; n < NT; ++n) o[n] *= alpha;
        }
        float psum = 0.f;
#pragma unroll
        for (int t = 0; t < TPT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s[t][r] = fast_exp2(s[t][r] - m_run);
                psum += s[t][r];
            }
        l_run += psum;

        // O^T += V^T P^T: step (t, r) is key 16 t + 4 lk + r for this lane,
        // which supplies V[key][odim(li, n)] for output tile n.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < TPT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float *vrow = KVb + vlane + (16 * t + r) * D;
                vec_t vv[NVW];
#pragma unroll
                for (int w = 0; w < NVW; ++w) vv[w] = *reinterpret_cast<const vec_t *>(vrow + 64 * w);
#pragma unroll
                for (int n = 0; n < NT; ++n) o[n] = mfma16x4(vget<VW>(vv[n / VW], n % VW), s[t][r], o[n]);
            }
        __builtin_amdgcn_s_setprio(0);
    };

    // One barrier per tile step: after it every wave's share of step kt has
    // landed and every wave is done with step kt - 1, whose buffer takes step
    // kt + 1 while step kt is consumed.
    auto step = [&](int kt, const float *KVt, float *KVn) {
        wait_vmem_all_small();
        __syncthreads();
        if (kt + 1 < T) issue_tile(kt + 1, KVn);
        compute(kt, KVt, KVt);
    };

    issue_tile(0, KV0);
    for (int kt = 0; kt < T; kt += 2) {
        step(kt, KV0, KV1);
        if (kt + 1 < T) step(kt + 1, KV1, KV0);
    }

    // ---- merge the key groups: groups 1.. park (max, partial sum, output) of
    // each lane in LDS, group 0 folds them in with the usual rescaling.  No
    // transfer is in flight: the last step issued none.
    {
        constexpr int SLOT = kWave * (4 * NT + 2);  // floats per parked wave
        constexpr int PER = (2 * SKS * SBN * D) / SLOT;  // parked waves per buffer
        static_assert(2 * PER >= (SKS - 1) * QW, "LDS too small to merge the key groups");
        auto slot_ptr = [&](int sl) -> float * { return (sl < PER ? KV0 : KV1) + (sl % PER) * SLOT; };
        __syncthreads();  // every wave is done with the K/V tiles
        if (grp > 0) {
            float *dst = slot_ptr((grp - 1) * QW + qwave) + lane;
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(4 * n + r) * kWave] = o[n][r];
            dst[4 * NT * kWave] = m_run;
            dst[(4 * NT + 1) * kWave] = l_run;
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int g = 1; g < SKS; ++g) {
            const float *src = slot_ptr((g - 1) * QW + qwave) + lane;
            const float m_g = src[4 * NT * kWave];
            const float m_new = fmaxf(m_run, m_g);
            const float keep = fast_exp2(m_run - m_new), take = fast_exp2(m_g - m_new);
            l_run = l_run * keep + src[(4 * NT + 1) * kWave] * take;
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[n][r] = o[n][r] * keep + src[(4 * n + r) * kWave] * take;
            m_run = m_new;
        }
    }

    // ---- normalise and store: lane holds query my_q, dims odim(4 lk + r, n).
    l_run = sum4(l_run);
    if (my_q < S) {
        const float inv = 1.0f / l_run;
        float *op = a.out + head_base + (size_t)my_q * row_stride;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int w = 0; w < NVW; ++w) {
                vec_t val;
#pragma unroll
                for (int e = 0; e < VW; ++e) vset<VW>(val, e, o[VW * w + e][r] * inv);
                *reinterpret_cast<vec_t *>(op + odim<D>(4 * lk + r, VW * w)) = val;
            }
    }
}

template <int D, int QW>
hipError_t launch_qw(const PrefillArgs &a, hipStream_t stream) {
    const int32_t BH = a.B * a.H;
    const int32_t tiles = (a.S + 16 * QW - 1) / (16 * QW);
    const int32_t xcd_remap = (BH % 8 == 0) ? 1 : 0;
    dim3 grid((unsigned)(BH * tiles)), block(kWave * QW * SKS);
    if (a.causal)
        prefill_small_kernel<D, QW, true><<<grid, block, 0, stream>>>(a, tiles, xcd_remap);
    else
        prefill_small_kernel<D, QW, false><<<grid, block, 0, stream>>>(a, tiles, xcd_remap);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs &a, int32_t qw, hipStream_t stream) {
    switch (qw) {
        case 1: return launch_qw<D, 1>(a, stream);
        case 2: return launch_qw<D, 2>(a, stream);
        case 3: return launch_qw<D, 3>(a, stream);
        default: return launch_qw<D, 4>(a, stream);
    }
}

}  // namespace

namespace {

// Causal: the work of a query tile grows with its position, so the cut is
// chosen by simulating the dispatch: workgroups in launch order (heaviest
// first) each go to the slot that frees first, at a speed set by the waves a
// SIMD holds (one workgroup of 4 QW waves per CU at d = 64 and 128, two at
// d = 32 for LDS), and the cut with the earliest end wins.  The speed factors
// per waves per SIMD (1: 0.3, 2: 0.6, 3: 0.8, 4: 1) pick the fastest cut, or
// one within 5% of it, on every shape timed (S 200..16384, 4..32 heads, d 32,
// 64 and 128).  Behind a cache of P rows every query tile has P more keys.
// Results are cached per shape.
int32_t causal_qw(int32_t BH, int32_t S, int32_t D, int32_t P, int32_t cus) {
    static const double kSpeed[5] = {0.0, 0.3, 0.6, 0.8, 1.0};
    const int32_t per_cu = D == 32 ? 2 : 1;
    int32_t best = 1;
    double best_end = -1.0;
    for (int32_t qw = 1; qw <= 4; ++qw) {
        const int64_t bm = 16 * qw;
        const int64_t n = (S + bm - 1) / bm;
        const double speed = kSpeed[std::min<int32_t>(4, qw * per_cu)] / per_cu;
        std::priority_queue<double, std::vector<double>, std::greater<double>> slots;
        for (int32_t i = 0; i < cus * per_cu; ++i) slots.push(0.0);
        double end = 0.0;
        for (int64_t qt = n - 1; qt >= 0; --qt) {
            const double work = (double)(bm * (P + std::min<int64_t>((qt + 1) * bm, S))) / speed;
            for (int32_t h = 0; h < BH; ++h) {
                const double t = slots.top() + work;
                slots.pop();
                slots.push(t);
                end = std::max(end, t);
            }
        }
        if (best_end < 0 || end < best_end) {
            best = qw;
            best_end = end;
        }
    }
    return best;
}

std::mutex g_causal_mu;
std::map<std::tuple<int32_t, int32_t, int32_t, int32_t, int32_t>, int32_t> g_causal_qw;

int32_t prefill_small_qw_causal(int32_t BH, int32_t S, int32_t D, int32_t P, int32_t cus) {
    const auto key = std::make_tuple(BH, S, D, P, cus);
    {
        std::lock_guard<std::mutex> lock(g_causal_mu);
        const auto it = g_causal_qw.find(key);
        if (it != g_causal_qw.end()) return it->second;
    }
    const int32_t qw = causal_qw(BH, S, D, P, cus);
    std::lock_guard<std::mutex> lock(g_causal_mu);
    if (g_causal_qw.size() < 4096) g_causal_qw[key] = qw;
    return qw;
}

int32_t prefill_small_qw(int32_t BH, int32_t S, int32_t cus) {
    // Non-causal: queries per workgroup 16 QW, the cut whose most loaded CU
    // (one workgroup per CU at a time) has the fewest queries; ties go to
    // fewer, larger workgroups.
    int32_t best = 4;
    int64_t best_cost = -1;
    for (int32_t qw = 4; qw >= 1; --qw) {
        const int64_t grid = (int64_t)BH * ((S + 16 * qw - 1) / (16 * qw));
        const int64_t cost = (grid + cus - 1) / cus * qw;
        if (best_cost < 0 || cost < best_cost) {
            best = qw;
            best_cost = cost;
        }
    }
    return best;
}

}  // namespace

int32_t prefill_cached_rows(const PrefillArgs &a) {
    if (!a.cached) return 0;
    int64_t sum = 0;
    for (int32_t b = 0; b < a.B; ++b) sum += a.pos.v[b];
    return (int32_t)(sum / a.B);
}

hipError_t launch_prefill_small(const PrefillArgs &a, int32_t cus, hipStream_t stream) {
    // The cut for a cache behind the chunk is chosen as if every sequence had
    // the mean cached length, rounded down to 64 rows (few distinct shapes).
    const int32_t qw = a.causal ? prefill_small_qw_causal(a.B * a.H, a.S, a.D, prefill_cached_rows(a) / 64 * 64, cus)
                                : prefill_small_qw(a.B * a.H, a.S, cus);
    switch (a.D) {
        case 32: return launch_d<32>(a, qw, stream);
        case 64: return launch_d<64>(a, qw, stream);
        case 128: return launch_d<128>(a, qw, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
