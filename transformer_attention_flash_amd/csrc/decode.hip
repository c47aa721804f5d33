// decode.hip -- batched grouped-query decode attention, split over the key axis.
//
// Semantics: trueno-gpu 0.4.11 src/memory/resident/attention.rs,
// `incremental_attention_gpu` (one query per head against a head-first cache,
// empty sequence -> zeros), with the GQA / batched cache layout of realizar
// 0.8.5 src/cuda/executor/cache_from_cache_from_kv_cache.rs
// (`init_kv_cache_gpu`: [num_kv_heads, max_len, head_dim];
// `init_batched_kv_cache_gpu`: [M, num_kv_heads, max_len, head_dim]).
//
// Pass 1 (decode_split_kernel): one workgroup per work unit (sequence m, KV
// head kh, block of up to 16 query heads of that KV head's group, key block).
// Its four waves stream adjacent 32-key chunks of the block side by side, each
// K row and V row read once straight from HBM, and every query head of the
// group is served from each load: the g query heads sharing a KV head make the
// scores a dense [16 x d] x [d x 16] contraction per 16 keys (heads padded to
// 16), which runs on v_mfma_f32_16x16x4_f32 and leaves the VALU free for the
// softmax.  Each wave keeps a running max (log2 units), sum and unnormalised
// output over its chunks; at the end the four waves merge theirs through LDS
// into one split per key block, (m_s, l_s, acc_s), written to the workspace.
//
// Pass 2 (decode_combine_kernel): one wave per (m, h) merges the splits:
// with M* = max_s m_s and w_s = 2^(m_s - M*), out = sum_s w_s acc_s /
// sum_s w_s l_s, or zeros when the sequence is empty, folded split by split in
// split order with a running max (the same identity applied incrementally),
// so the result is the same on every run.  When a sequence has more than 16
// splits (calls of one or a few sequences, up to 512 splits) and there are no
// more (m, h) than CUs, decode_combine_wide_kernel gives each (m, h) sixteen
// waves, each folding a contiguous range of the splits, and folds their
// states in range order.
//
// Register layouts of v_mfma_f32_16x16x4_f32 (lane l, i = l % 16, k = l / 16):
// operand A supplies A[i][k], operand B supplies B[k][i], and output register
// r holds D[4k + r][i].  Scores are formed transposed, S^T = K q^T (rows =
// keys, columns = heads), so that output register r of a lane is exactly the
// operand-B value that lane supplies at key step r of the P.V contraction
// O^T = V^T P^T: no data moves between the two products.
#include <atomic>
#include <climits>

#include "decode_plan.h"
#include "device_common.h"
#include "launch.h"
#include "rope.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

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

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Cache rows are read exactly once per call: stream them past the caches.
template <typename T>
__device__ __forceinline__ T load_stream(const T *p) {
    return __builtin_nontemporal_load(p);
}

template <int D, int CH, bool ROPE>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(DecodeArgs a, SegMap map,
                                                                int32_t n_hblk, RopeParams rp) {
    constexpr int NT = D / 16;     // 16-column tiles of O^T
    constexpr int KV4 = D / 16;    // 16-byte K vectors per lane per 16-key tile
    constexpr int VW = D >= 64 ? 4 : 2;  // floats per V vector
    constexpr int NVV = NT / VW;   // V vectors per lane per key
    constexpr int NTL = CH / 16;   // 16-key MFMA tiles per chunk
    typedef typename VecN<VW>::type vvec;
    static_assert(CH == 16 || CH == 32, "chunks of 16 or 32 keys");

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int wg = blockIdx.x;  // the grid has exactly map.start[map.nseg] blocks

    // workgroup -> (segment s, unit, block p of the segment) -> (m, kh, head
    // block hb, split slot kblk, keys [k0, k1)).  Wave w of the workgroup
    // takes chunks w, w + 4, w + 8, ... of the key block, so the four waves
    // stream adjacent 32-key chunks of K (and of V) side by side.  The
    // segment is the number of segment starts <= wg, less one (starts
    // increase, and the entries past the last segment hold the grid size).
    // The lanes load every start and every sequence length at once and the
    // values needed are read from their lanes, so that the lookup waits on
    // two loads (the starts, then the segment's fields), not on a search
    // whose every step waits on one.
    constexpr int kStartLoads = (kMaxSegs + kWave) / kWave;  // kMaxSegs + 1 starts
    static_assert(ATTN_MAX_SEQS <= kWave, "one sequence length per lane");
    int st[kStartLoads];
#pragma unroll
    for (int c = 0; c < kStartLoads; ++c) {
        const int i = c * kWave + lane;
        st[c] = i <= kMaxSegs ? map.start[i] : INT_MAX;
    }
    const int len_lane = lane < ATTN_MAX_SEQS ? a.lens.v[lane] : 0;
    int s = -1;
#pragma unroll
    for (int c = 0; c < kStartLoads; ++c) s += __popcll(__ballot(st[c] <= wg));
    // s < nseg <= kMaxSegs, so its start is held by lane s % 64 of load s / 64
    int st_s = st[0];
#pragma unroll
    for (int c = 1; c < kStartLoads; ++c) st_s = s >= c * kWave ? st[c] : st_s;
    const uint32_t info = map.info[s];
    const int m = seg_seq(info);
    const int L = __builtin_amdgcn_readlane(len_lane, m);
    const int npiece = seg_npiece(info);
    const int rem = wg - __builtin_amdgcn_readlane(st_s, s & (kWave - 1));
    const int p = rem % npiece;
    const int hb = (rem / npiece) % n_hblk;
    const int kh = (rem / npiece) / n_hblk;
    const int kblk = seg_piece0(info) + p;
    const int k0 = map.kbase[s] + p * map.span[s];  // the workgroup's keys are [k0, k1)
    const int k1 = min(k0 + map.span[s], L);

    const int g = a.H / a.Hkv;
    const int hi = lane & 15;  // head column / key row within a tile
    const int kq = lane >> 4;  // k-slot of the MFMA operands
    const int head_in_group = hb * 16 + hi;
    const bool head_ok = head_in_group < g;
    const int h = kh * g + head_in_group;

    const int kfirst = k0 + CH * wave;
    constexpr int kStep = CH * kWavesPerBlock;

    // q^T operand, pre-scaled so scores come out in log2 units.  With a
    // rotary embedding the query is first turned to the position of the
    // newest cached token, L - 1 (lane's dims 16j + 4kq .. +3; the partner
    // dims half a rotary width away are read from the same small q row).
    const float qs = a.scale * kLog2e;
    float qreg[KV4][4];
    f32x4 qraw[KV4], qpart[KV4];
    const float *qhead = a.q + ((size_t)m * a.H + (head_ok ? h : 0)) * D;
    auto load_q = [&]() {
#pragma unroll
        for (int j = 0; j < KV4; ++j) {
            const int l0 = 16 * j + 4 * kq;
            qraw[j] = head_ok ? *reinterpret_cast<const f32x4 *>(qhead + l0) : f32x4{0, 0, 0, 0};
            if constexpr (ROPE) {
                const int pl = l0 < rp.half ? l0 + rp.half : l0 - rp.half;
                qpart[j] = (head_ok && l0 < rp.rot) ? *reinterpret_cast<const f32x4 *>(qhead + pl)
                                                    : f32x4{0, 0, 0, 0};
            }
        }
    };
    auto finish_q = [&]() {
#pragma unroll
        for (int j = 0; j < KV4; ++j) {
            f32x4 v4 = qraw[j];
            if constexpr (ROPE) v4 = rope_rotate4(v4, qpart[j], 16 * j + 4 * kq, L > 0 ? L - 1 : 0, rp);
#pragma unroll
            for (int c = 0; c < 4; ++c) qreg[j][c] = v4[c] * qs;
        }
    };
    if constexpr (!ROPE) {
#pragma unroll
        for (int j = 0; j < KV4; ++j) {
            const f32x4 v4 = head_ok ? *reinterpret_cast<const f32x4 *>(qhead + 16 * j + 4 * kq) : f32x4{0, 0, 0, 0};
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

    // K goes global -> registers -> LDS -> MFMA operand registers.  The MFMA
    // operand layout puts only four lanes on a key row (64 bytes per row per
    // instruction), which would make the memory pipeline carry every K line
    // as two half-line requests; instead each global load instruction reads
    // two whole rows (1 KiB, fully coalesced) and the operand is gathered from
    // this wave's LDS tile.  Rows are padded by 4 floats so the 16 keys of an
    // operand read fall in distinct banks.  V is read straight into operand
    // registers: 16 lanes cover a row, 256 contiguous bytes per row.  Rows
    // past the key block's end are clamped to its last row (in bounds) and
    // masked below.
    constexpr int KROW = D + 4;                      // LDS pitch of a K row (floats)
    constexpr int KST = CH * D / 4 / kWave;          // 16-byte K vectors per lane per chunk
    __shared__ __attribute__((aligned(16))) float k_lds[kWavesPerBlock][CH * KROW];
    float *kl = k_lds[wave];
    f32x4 kst[KST];
    vvec vf[NTL][4][NVV];
    auto load_k = [&](int kb) {
#pragma unroll
        for (int u = 0; u < KST; ++u) {
            const int idx = lane + kWave * u;
            const int krow = min(kb + idx / (D / 4), k1 - 1);
            kst[u] = load_stream(reinterpret_cast<const f32x4 *>(kc + (size_t)krow * D + 4 * (idx % (D / 4))));
        }
    };
    auto stage_k = [&]() {
#pragma unroll
        for (int u = 0; u < KST; ++u) {
            const int idx = lane + kWave * u;
            *reinterpret_cast<f32x4 *>(kl + (idx / (D / 4)) * KROW + 4 * (idx % (D / 4))) = kst[u];
        }
    };
    auto load_v = [&](int kb) {
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int vrow = min(kb + 16 * t + 4 * kq + r, k1 - 1);
#pragma unroll
                for (int c = 0; c < NVV; ++c)
                    vf[t][r][c] = load_stream(reinterpret_cast<const vvec *>(vc + (size_t)vrow * D + 64 * c + VW * hi));
            }
        }
    };

    // Software pipeline: chunk c+1's K loads are issued as soon as chunk c's
    // K rows are staged in LDS, and its V loads as soon as the P.V products of
    // chunk c are issued, so every wave keeps about a chunk's worth of HBM
    // reads in flight while it computes.  The scheduling barriers stop
    // the compiler from sinking the loads next to their uses.  The loads are
    // unconditional (exact wait counts across the loop back-edge): after the
    // last chunk every lane's row clamps to k1 - 1, one row already in cache.
    load_k(kfirst);
    __builtin_amdgcn_sched_barrier(0);  // K before V, the order the loop keeps
    if constexpr (ROPE) {
        // The query's rotation (sin/cos per dim) overlaps the first chunk's
        // loads: its q loads go out between K and V, so waiting for them
        // leaves the V loads in flight.
        load_q();
        __builtin_amdgcn_sched_barrier(0);
    }
    load_v(kfirst);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (ROPE) finish_q();
    for (int kb = kfirst; kb < k1; kb += kStep) {

        // Chunk kb's K rows into this wave's LDS tile (a wave's LDS accesses
        // are processed in order, so the reads below see these writes and the
        // previous chunk's reads completed before they are overwritten).
        stage_k();
        __builtin_amdgcn_sched_barrier(0);
        // The staging registers are free again: chunk c+1's K loads go out now
        // and have this chunk's scores, softmax and P.V to arrive.
        load_k(kb + kStep);
        __builtin_amdgcn_sched_barrier(0);

        // S^T tiles: rows = keys kb + 16t + 4kq + r, columns = heads.
        f32x4 sc[NTL];
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            f32x4 acc = {0, 0, 0, 0};
            const float *krow = kl + (16 * t + hi) * KROW + 4 * kq;
#pragma unroll
            for (int j = 0; j < KV4; ++j) {
                const f32x4 kv = *reinterpret_cast<const f32x4 *>(krow + 16 * j);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc = mfma16(kv[c], qreg[j][c], acc);
            }
            sc[t] = acc;
        }

        // Online softmax over the chunk; keys >= k1 are masked.
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NTL; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool live = kb + 16 * t + 4 * kq + r < k1;
                sc[t][r] = live ? sc[t][r] : -INFINITY;
                mx = fmaxf(mx, sc[t][r]);
            }
        mx = max4(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int t = 0; t < NTL; ++t)
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
        for (int t = 0; t < NTL; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool live = kb + 16 * t + 4 * kq + r < k1;
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const float vv = live ? vget<VW>(vf[t][r][n / VW], n % VW) : 0.f;
                    o[n] = mfma16(vv, sc[t][r], o[n]);
                }
            }
        __builtin_amdgcn_sched_barrier(0);
        load_v(kb + kStep);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Each k-slot group summed its own keys; combine them.
    l_run = sum4(l_run);

    // Merge the four waves' states through LDS: each wave parks (m, l, O^T)
    // in its own K tile (its last reads of that tile are behind it: a wave's
    // LDS accesses complete in order), then wave w merges output register r = w
    // of every lane from all four, i.e. rows 4 kq + w of O^T, and writes them.
    // A wave that had no chunk of the key block parks max kNegBig, sum 0,
    // output 0, which the merge weighs by 2^(kNegBig - M*) = 0 (wave 0 always
    // has a chunk, so M* is a real maximum).
    static_assert(16 * D + 32 <= CH * KROW, "parked state fits the K tile");
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) kl[(4 * n + r) * kWave + lane] = o[n][r];
    if (kq == 0) {
        kl[16 * D + hi] = m_run;
        kl[16 * D + 16 + hi] = l_run;
    }
    __syncthreads();
    float mw[kWavesPerBlock], wt[kWavesPerBlock];
    float mstar = kNegBig;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        mw[w] = k_lds[w][16 * D + hi];
        mstar = fmaxf(mstar, mw[w]);
    }
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        wt[w] = fast_exp2(mw[w] - mstar);
        lsum += wt[w] * k_lds[w][16 * D + 16 + hi];
    }
    if (head_ok) {
        const size_t slot = ((size_t)m * a.H + h) * a.max_splits + kblk;
        if (wave == 0 && kq == 0) *reinterpret_cast<f32x2 *>(a.ws_ml + 2 * slot) = f32x2{mstar, lsum};
        float *dst = a.ws_acc + slot * D;
        const int r = wave;
#pragma unroll
        for (int c = 0; c < NVV; ++c) {
            vvec val;
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                const int n = c * VW + e;
                float acc = 0.f;
#pragma unroll
                for (int w = 0; w < kWavesPerBlock; ++w) acc += wt[w] * k_lds[w][(4 * n + r) * kWave + lane];
                vset<VW>(val, e, acc);
            }
            *reinterpret_cast<vvec *>(dst + ocol<D>(c * VW, 4 * kq + r)) = val;
        }
    }
}

// Folds splits [s_lo, s_hi) of one (m, h) into the running (m_run, l_run,
// acc) in split order, loads of BATCH splits in flight together (the merge
// waits on one memory latency per batch, about a microsecond).  Lane l holds
// output columns PER*l .. PER*l + PER - 1 (lanes >= LANES hold none).
template <int D>
struct Fold {
    static constexpr int PER = D >= 64 ? D / 64 : 1;  // floats per lane
    static constexpr int LANES = D / PER;             // lanes holding output columns
    static constexpr int BATCH = 16;
    typedef typename VecN<PER>::type pvec;

    __device__ static void run(const float *ml, const float *accp, int s_lo, int s_hi, int lane, float &m_run,
                               float &l_run, pvec &acc) {
        for (int s0 = s_lo; s0 < s_hi; s0 += BATCH) {
            f32x2 mlv[BATCH];
            pvec av[BATCH];
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                const int s = s0 + b;
                const bool ok = s < s_hi;
                mlv[b] = ok ? *reinterpret_cast<const f32x2 *>(ml + 2 * s) : f32x2{kNegBig, 0.f};
                av[b] = (ok && lane < LANES) ? *reinterpret_cast<const pvec *>(accp + (size_t)s * D) : pvec{};
            }
#pragma unroll
            for (int b = 0; b < BATCH; ++b) merge(m_run, l_run, acc, mlv[b][0], mlv[b][1], av[b]);
        }
    }

    // (m_run, l_run, acc) <- the fold of itself and one more state (m, l, a).
    __device__ static void merge(float &m_run, float &l_run, pvec &acc, float m, float l, const pvec &a) {
        const float m_new = fmaxf(m_run, m);
        const float keep = fast_exp2(m_run - m_new), take = fast_exp2(m - m_new);
        l_run = l_run * keep + l * take;
        acc = acc * keep + a * take;
        m_run = m_new;
    }
};

// One wave per (m, h): folds the nsplit[m] splits in split order with a
// running max and writes out[m][h] = acc / l, or zeros for an empty sequence.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeArgs a, SegMap map) {
    typedef Fold<D> F;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (w >= a.M * a.H) return;  // no barrier below
    const int nsplit = map.nsplit[w / a.H];
    const size_t slot0 = (size_t)w * a.max_splits;
    float m_run = kNegBig, l_run = 0.f;
    typename F::pvec acc{};
    F::run(a.ws_ml + 2 * slot0, a.ws_acc + slot0 * D + F::PER * lane, 0, nsplit, lane, m_run, l_run, acc);
    if (lane < F::LANES)
        *reinterpret_cast<typename F::pvec *>(a.out + (size_t)w * D + F::PER * lane) =
            nsplit > 0 ? acc * (1.0f / l_run) : typename F::pvec{};
}

// For calls whose sequences have many splits: one workgroup of kWideWaves
// waves per (m, h).  Wave v folds the v-th of kWideWaves contiguous ranges of
// the splits, then wave 0 folds the waves' states in wave order, so the
// splits are still combined in one fixed order on every run.
constexpr int kWideWaves = 16;
constexpr int kWideSplits = Fold<32>::BATCH;  // the wide merge runs when a sequence has more splits

template <int D>
__global__ __launch_bounds__(kWideWaves * kWave) void decode_combine_wide_kernel(DecodeArgs a, SegMap map) {
    typedef Fold<D> F;
    __shared__ float st_acc[kWideWaves][D];
    __shared__ float st_ml[kWideWaves][2];
    const int lane = threadIdx.x & (kWave - 1);
    const int v = threadIdx.x >> 6;
    const int w = blockIdx.x;  // (m, h); the grid is exactly M * H
    const int nsplit = map.nsplit[w / a.H];
    const int per = (nsplit + kWideWaves - 1) / kWideWaves;
    const int s_lo = min(v * per, nsplit), s_hi = min(s_lo + per, nsplit);
    const size_t slot0 = (size_t)w * a.max_splits;
    float m_run = kNegBig, l_run = 0.f;
    typename F::pvec acc{};
    F::run(a.ws_ml + 2 * slot0, a.ws_acc + slot0 * D + F::PER * lane, s_lo, s_hi, lane, m_run, l_run, acc);
    if (lane < F::LANES) *reinterpret_cast<typename F::pvec *>(&st_acc[v][F::PER * lane]) = acc;
    if (lane == 0) {
        st_ml[v][0] = m_run;
        st_ml[v][1] = l_run;
    }
    __syncthreads();
    if (v != 0) return;
    m_run = kNegBig;
    l_run = 0.f;
    acc = typename F::pvec{};
    for (int u = 0; u < kWideWaves; ++u) {
        const typename F::pvec au =
            lane < F::LANES ? *reinterpret_cast<const typename F::pvec *>(&st_acc[u][F::PER * lane])
                            : typename F::pvec{};
        F::merge(m_run, l_run, acc, st_ml[u][0], st_ml[u][1], au);
    }
    if (lane < F::LANES)
        *reinterpret_cast<typename F::pvec *>(a.out + (size_t)w * D + F::PER * lane) =
            nsplit > 0 ? acc * (1.0f / l_run) : typename F::pvec{};
}

// Workgroups of decode_split_kernel<D, CH, ROPE> that fit on the device at
// once (CUs x resident blocks per CU), queried once per device and kernel.
constexpr int kMaxDevices = 64;
std::atomic<int32_t> g_capacity[kMaxDevices][3][2][2];
std::atomic<int32_t> g_cus[kMaxDevices];

// Compute units of the current device, queried once per device.
int32_t decode_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int32_t n = g_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
    g_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

template <int D, int CH, bool ROPE>
int32_t query_capacity() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 512;
    const int slot = D == 32 ? 0 : D == 64 ? 1 : 2;
    int32_t cap = g_capacity[dev][slot][CH == 16][ROPE].load(std::memory_order_relaxed);
    if (cap > 0) return cap;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0 ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<D, CH, ROPE>, kThreads, 0) != hipSuccess ||
        per_cu <= 0)
        return 512;
    cap = cus * per_cu;
    g_capacity[dev][slot][CH == 16][ROPE].store(cap, std::memory_order_relaxed);
    return cap;
}

template <int D>
int32_t capacity_d(int32_t CH, bool rot) {
    if (CH == 16) return rot ? query_capacity<D, 16, true>() : query_capacity<D, 16, false>();
    return rot ? query_capacity<D, 32, true>() : query_capacity<D, 32, false>();
}

int32_t capacity_for(int32_t D, int32_t CH, bool rot) {
    switch (D) {
        case 32: return capacity_d<32>(CH, rot);
        case 64: return capacity_d<64>(CH, rot);
        default: return capacity_d<128>(CH, rot);
    }
}

template <int D, int CH>
void launch_split(bool rot, dim3 grid, hipStream_t stream, const DecodeArgs &a, const SegMap &map, int32_t n_hblk,
                  const RopeParams &rp) {
    if (rot)
        decode_split_kernel<D, CH, true><<<grid, dim3(kThreads), 0, stream>>>(a, map, n_hblk, rp);
    else
        decode_split_kernel<D, CH, false><<<grid, dim3(kThreads), 0, stream>>>(a, map, n_hblk, rp);
}

}  // namespace

int32_t decode_max_splits(int32_t M, int32_t H, int32_t max_len) { return max_splits_for(M, H, max_len); }

size_t decode_workspace_bytes(int64_t M, int64_t H, int64_t D, int64_t max_len) {
    const int64_t slots = M * H * (int64_t)max_splits_for(M, H, (int32_t)max_len);
    return (size_t)(slots * (D + 2) * (int64_t)sizeof(float));
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream, const RopeParams *rope) {
    const int32_t n_hblk = (a.H / a.Hkv + 15) / 16;
    const bool rot = rope && rope->rot > 0;
    DecodePlan plan;
    plan_decode(a.lens.v, a.M, a.H, a.Hkv, a.max_len, decode_cus(), capacity_for(a.D, 32, rot),
                capacity_for(a.D, 16, rot), &plan);
    const SegMap &map = plan.map;
    const int32_t ch = plan.ch, acc = plan.grid;

    dim3 block(kThreads);
    if (acc > 0) {
        dim3 grid(acc);
        const RopeParams none{};
        const RopeParams &rp = rot ? *rope : none;
        switch (a.D * 2 + (ch == 16)) {
            case 64: launch_split<32, 32>(rot, grid, stream, a, map, n_hblk, rp); break;
            case 65: launch_split<32, 16>(rot, grid, stream, a, map, n_hblk, rp); break;
            case 128: launch_split<64, 32>(rot, grid, stream, a, map, n_hblk, rp); break;
            case 129: launch_split<64, 16>(rot, grid, stream, a, map, n_hblk, rp); break;
            case 256: launch_split<128, 32>(rot, grid, stream, a, map, n_hblk, rp); break;
            case 257: launch_split<128, 16>(rot, grid, stream, a, map, n_hblk, rp); break;
            default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // The 16-wave merge when a sequence has more splits than one batch and
    // there are no more (m, h) than CUs (one workgroup each); with more, one
    // wave per (m, h) folding batch after batch keeps the device fuller.
    if (plan.most > kWideSplits && (int64_t)a.M * a.H <= decode_cus()) {
        dim3 grid2(a.M * a.H), block2(kWideWaves * kWave);
        switch (a.D) {
            case 32: decode_combine_wide_kernel<32><<<grid2, block2, 0, stream>>>(a, map); break;
            case 64: decode_combine_wide_kernel<64><<<grid2, block2, 0, stream>>>(a, map); break;
            case 128: decode_combine_wide_kernel<128><<<grid2, block2, 0, stream>>>(a, map); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    dim3 grid2((a.M * a.H + kWavesPerBlock - 1) / kWavesPerBlock);
    switch (a.D) {
        case 32: decode_combine_kernel<32><<<grid2, block, 0, stream>>>(a, map); break;
        case 64: decode_combine_kernel<64><<<grid2, block, 0, stream>>>(a, map); break;
        case 128: decode_combine_kernel<128><<<grid2, block, 0, stream>>>(a, map); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace attn
