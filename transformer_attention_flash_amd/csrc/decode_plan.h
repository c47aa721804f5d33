// decode_plan.h -- host-side work decomposition of the split decode.
//
// Pure host arithmetic (no HIP call), shared by the launcher in decode.hip
// and by a CPU test that checks, on random calls, that the key blocks tile
// every sequence exactly and stay within the workspace's split bound.
#pragma once

#include <stdint.h>

#include "../../include/attn.h"

namespace attn {

// Work decomposition of one call, computed on the host from the lengths.
// The keys of every unit (kh, head block) of sequence m are cut, in key
// order, into nsplit[m] key blocks.  A segment is a run of blocks of one
// sequence and one span: segment s holds npiece[s] blocks per unit, of
// span[s] keys each from key kbase[s] on (a block is clipped to the sequence
// length), and workgroup start[s] + u * npiece[s] + p runs block p of unit u,
// whose split slot is piece0[s] + p; sequence, npiece and piece0 share one
// word (seg_info), so that a workgroup reads its segment in one round trip.
// plan_decode orders the segments so
// that the blocks of the device's first round come first, sized for the slot
// each will occupy, and small tail blocks after them.
constexpr int kMaxSlotsPerCu = 3;  // first-round block kinds (workgroups per CU)
constexpr int kMaxSegs = (kMaxSlotsPerCu + 1) * ATTN_MAX_SEQS;
struct SegMap {
    int32_t start[kMaxSegs + 1];    // first workgroup of segment s; from nseg on, the grid size
    int32_t kbase[kMaxSegs];        // first key of its first block
    int32_t span[kMaxSegs];         // keys per block
    uint32_t info[kMaxSegs];        // seg_info(sequence, npiece, piece0)
    int32_t nsplit[ATTN_MAX_SEQS];  // key blocks per unit of each sequence
    int32_t nseg;
};

// Sequence (8 bits), blocks per unit and first split slot (12 bits each) of a
// segment; a sequence has at most kMaxKeyBlocksFew <= 4095 blocks.
constexpr uint32_t seg_info(int32_t seq, int32_t npiece, int32_t piece0) {
    return (uint32_t)seq | (uint32_t)npiece << 8 | (uint32_t)piece0 << 20;
}
constexpr int32_t seg_seq(uint32_t info) { return (int32_t)(info & 0xffu); }
constexpr int32_t seg_npiece(uint32_t info) { return (int32_t)((info >> 8) & 0xfffu); }
constexpr int32_t seg_piece0(uint32_t info) { return (int32_t)(info >> 20); }

constexpr int32_t kSpanQuantum = 128;  // keys: one 32-key chunk per wave
constexpr int32_t kMaxKeyBlocks = 64;       // per (sequence, head), calls with many units
constexpr int32_t kMaxKeyBlocksFew = 512;   // per (sequence, head), calls with few units
constexpr int64_t kKeyBlocksWanted = 1024;  // key blocks per call: about four per CU
static_assert(kMaxKeyBlocksFew < 4096 && ATTN_MAX_SEQS <= 256, "seg_info field widths");

// Key blocks a sequence may be cut into when a call has `units` work units
// (sequence, KV head, head block) over all its sequences: 64, doubled up to
// 512 while the call would have fewer than kKeyBlocksWanted blocks in all, so
// that a call of one or two sequences still fills the device.
inline int32_t key_block_limit(int64_t units) {
    int32_t n = kMaxKeyBlocks;
    while (n < kMaxKeyBlocksFew && units * n < kKeyBlocksWanted) n *= 2;
    return n;
}

// Smallest key-block span for a cache of max_len rows: a power-of-two multiple
// of the quantum that keeps a sequence at <= `limit` key blocks (64-bit
// arithmetic: max_len may be any positive int32).
inline int32_t span_floor(int32_t max_len, int32_t limit) {
    int64_t s = kSpanQuantum;
    while (((int64_t)max_len + s - 1) / s > limit) s *= 2;
    return (int32_t)s;
}

// Splits a call of M sequences and H query heads may write per (m, h).  A
// sequence's units number num_kv_heads * ceil(group / 16) >= ceil(H / 16),
// so the launch, which sizes its floor from its actual units, never uses a
// smaller floor (more blocks) than this bound allows.
inline int32_t max_splits_for(int64_t M, int64_t H, int32_t max_len) {
    const int64_t sf = span_floor(max_len, key_block_limit(M * ((H + 15) / 16)));
    return (int32_t)(((int64_t)max_len + sf - 1) / sf);
}

// The first round of the grid carries about kFirstRoundPct percent of the
// keys, the rest goes to tail blocks of kTailFloors x span_floor keys.
// Workgroups co-resident on one CU stream at unequal speeds: the one placed
// first wins issue arbitration on every SIMD.  Timed per workgroup on the
// device, the second-placed streams at 0.69-0.74 of the first's rate and a
// third at about a quarter, so the first round's block for the k-th
// workgroup of a CU is sized by kSlotWeight[k] (percent), and all of them
// finish at about the same time.
constexpr int64_t kFirstRoundPct = 95;
constexpr int32_t kTailFloors = 1;
constexpr int64_t kSlotWeight[kMaxSlotsPerCu] = {100, 72, 28};

// Below this many keys per workgroup slot (at 32-key chunks) a call streams
// 16-key chunks: half the loads in flight per wave and a third resident
// workgroup per CU, which shortens each key block's start and the queueing
// of a short call (M 32, up to 4096 keys: 92 -> 88 us); long contexts keep
// 32-key chunks (M 16, 16K-32K keys: 1-3% faster than 16).
constexpr int64_t kShortKeysPerSlot = 4096;

// Blocks per CU for a call of few units, all of one span: on such calls equal
// blocks ran faster than the slot-sized first round (M 1, 8 KV heads, 131072
// keys: split pass 164 against 178 us), and one per CU faster than two (one
// KV head, 65536 keys: 25.6 against 30.7 us, half as many splits to merge).
constexpr int64_t kFewBlocksPerCu = 1;

// The decomposition of one call.  ch: keys per chunk (16 or 32) of the
// split kernel; grid: its workgroups; most: the largest nsplit[m].
struct DecodePlan {
    SegMap map;
    int32_t ch, grid, most;
};

// lens: M sequence lengths (0 <= L <= max_len); cus: the device's compute
// units; cap32, cap16: workgroups of the split kernel (this head_dim and
// rotation) resident on the whole device at once with 32- and 16-key chunks.
inline void plan_decode(const int32_t *lens, int32_t M, int32_t H, int32_t Hkv, int32_t max_len, int64_t cus,
                        int64_t cap32, int64_t cap16, DecodePlan *out) {
    const int32_t g = H / Hkv;
    const int32_t n_hblk = (g + 15) / 16;
    const int64_t units_per_seq = (int64_t)Hkv * n_hblk;

    // First round: the k-th workgroup placed on a CU (k < the kernel's
    // workgroups per CU) gets a block of span[k] keys, span[k] proportional
    // to kSlotWeight[k], kFirstRoundPct percent of the keys over all of them.
    // Each kind holds one block per CU, counted in units of whole sequences
    // (all units of a sequence have the same blocks), and goes to the
    // sequences with the most keys left, in key order: a sequence's kind-0
    // blocks come first, then its kind-1 blocks, ...  The keys left after the
    // first round go to tail blocks of kTailFloors x span_floor keys, which
    // run last.  A call of few units (fewer than kKeyBlocksWanted /
    // kMaxKeyBlocks over all its sequences) has no first round: its
    // sequences are cut into equal blocks, about kFewBlocksPerCu per CU over
    // the call.  Every span is at least span_floor (the floor for the call's
    // own units, no smaller than the one the workspace was sized with), so a
    // sequence of L keys has at most ceil(L / span_floor) <= max_splits
    // blocks: all but its last block hold span_floor keys or more.
    int64_t lsum = 0;
    for (int i = 0; i < M; ++i) lsum += lens[i];
    const int64_t total = lsum * units_per_seq;
    const int32_t ch = total < kShortKeysPerSlot * cap32 ? 16 : 32;
    int64_t per_cu = (ch == 16 ? cap16 : cap32) / cus;
    per_cu = per_cu < 1 ? 1 : per_cu > kMaxSlotsPerCu ? kMaxSlotsPerCu : per_cu;
    const int64_t call_units = (int64_t)M * units_per_seq;
    const int64_t sf = span_floor(max_len, key_block_limit(call_units));
    const bool few = call_units * kMaxKeyBlocks < kKeyBlocksWanted;
    int64_t tspan = sf * kTailFloors;
    if (few) {
        const int64_t blocks = kFewBlocksPerCu * cus;
        int64_t even = ((total + blocks - 1) / blocks + kSpanQuantum - 1) / kSpanQuantum * kSpanQuantum;
        if (even > max_len) even = max_len;  // one block per sequence at most (few CUs)
        tspan = even > sf ? even : sf;
    }
    const int64_t nkind = few ? 0 : cus / units_per_seq;  // blocks of each kind, in sequences

    int64_t rem[ATTN_MAX_SEQS];
    int32_t nk[kMaxSlotsPerCu][ATTN_MAX_SEQS] = {};
    int64_t kspan[kMaxSlotsPerCu] = {};
    for (int i = 0; i < ATTN_MAX_SEQS; ++i) rem[i] = i < M ? lens[i] : 0;
    int64_t wsum = 0;
    for (int k = 0; k < per_cu; ++k) wsum += kSlotWeight[k];
    for (int k = 0; k < per_cu && nkind > 0; ++k) {
        int64_t span = kFirstRoundPct * lsum * kSlotWeight[k] / (100 * nkind * wsum);
        // no longer than the longest sequence left, or no sequence could take one
        int64_t longest = 0;
        for (int i = 0; i < M; ++i) longest = rem[i] > longest ? rem[i] : longest;
        if (span > longest) span = longest;
        span = span / sf * sf;
        if (span < sf) continue;
        kspan[k] = span;
        // Blocks in proportion to the keys left (largest remainders next),
        // never more than a sequence can hold.
        int64_t left = 0;
        for (int i = 0; i < M; ++i) left += rem[i];
        if (left == 0) break;
        int64_t given = 0;
        for (int i = 0; i < M; ++i) {
            const int64_t cap = rem[i] / span;
            const int64_t want = nkind * rem[i] / left;
            nk[k][i] = (int32_t)(want < cap ? want : cap);
            given += nk[k][i];
        }
        while (given < nkind) {
            int best = -1;
            int64_t best_left = 0;
            for (int i = 0; i < M; ++i) {
                const int64_t after = rem[i] - (int64_t)nk[k][i] * span;
                if (after >= span && after > best_left) {
                    best = i;
                    best_left = after;
                }
            }
            if (best < 0) break;
            ++nk[k][best];
            ++given;
        }
        for (int i = 0; i < M; ++i) rem[i] -= (int64_t)nk[k][i] * span;
    }

    SegMap &map = out->map;
    int nseg = 0;
    int32_t acc = 0;
    int32_t done[ATTN_MAX_SEQS] = {};    // blocks laid so far per sequence
    int64_t kdone[ATTN_MAX_SEQS] = {};   // keys covered so far per sequence
    auto add_segment = [&](int i, int32_t n, int64_t span) {
        map.start[nseg] = acc;
        map.kbase[nseg] = (int32_t)kdone[i];
        map.span[nseg] = (int32_t)span;
        map.info[nseg] = seg_info(i, n, done[i]);
        acc += n * (int32_t)units_per_seq;
        done[i] += n;
        ++nseg;
    };
    for (int k = 0; k < per_cu; ++k)
        for (int i = 0; i < M; ++i)
            if (nk[k][i] > 0) {
                add_segment(i, nk[k][i], kspan[k]);
                kdone[i] += (int64_t)nk[k][i] * kspan[k];
            }
    for (int i = 0; i < M; ++i)
        if (rem[i] > 0) add_segment(i, (int32_t)((rem[i] + tspan - 1) / tspan), (int32_t)tspan);
    map.nseg = nseg;
    for (int i = nseg; i <= kMaxSegs; ++i) map.start[i] = acc;
    for (int i = nseg; i < kMaxSegs; ++i) {
        map.kbase[i] = map.span[i] = 0;
        map.info[i] = 0;
    }
    for (int i = 0; i < ATTN_MAX_SEQS; ++i) map.nsplit[i] = done[i];

    int32_t most = 0;
    for (int i = 0; i < M; ++i) most = done[i] > most ? done[i] : most;
    out->ch = ch;
    out->grid = acc;
    out->most = most;
}

}  // namespace attn
