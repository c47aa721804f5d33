// Checks the split decode's host-side work decomposition (plan_decode in
// decode_plan.h) on seeded random calls: the key blocks of every sequence
// tile [0, L) exactly, in split-slot order (which the merge folds in), no
// sequence gets more splits than the workspace holds (max_splits_for), every
// block but a sequence's last holds at least the span floor, and the segment
// table and grid size agree.  Pure host code, built with g++.
//
//   decode_plan_check <seed> <calls> [corrupt]
//
// With "corrupt", one planned segment is altered before the checks, which
// must then fail (a check of the checker).  Exit status 0 when every call
// passes.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../transformer_attention_flash_amd/csrc/decode_plan.h"

using namespace attn;

namespace {

uint64_t g_state;

uint64_t next_u64() {  // splitmix64
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int64_t uniform(int64_t lo, int64_t hi) { return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1)); }

#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "check failed: %s: ", #cond);                 \
            fprintf(stderr, __VA_ARGS__);                                 \
            fprintf(stderr, "\n");                                        \
            return false;                                                 \
        }                                                                 \
    } while (0)

struct Block {
    int32_t slot;
    int64_t k0, k1;
};

bool check_call(const int32_t *lens, int32_t M, int32_t H, int32_t Hkv, int32_t max_len, int64_t cus, int64_t cap32,
                int64_t cap16, bool corrupt, int64_t *wide, int64_t *altered) {
    DecodePlan plan;
    plan_decode(lens, M, H, Hkv, max_len, cus, cap32, cap16, &plan);
    SegMap &m = plan.map;
    if (corrupt) {
        if (m.nseg == 0) return true;  // nothing to alter: not counted
        const int s = (int)(next_u64() % (uint64_t)m.nseg);
        switch (next_u64() % 3) {
            case 0: m.kbase[s] += 1; break;   // a gap of one key
            case 1: m.info[s] += 1u << 20; break;  // a split slot out of order
            default: m.info[s] += 1u << 8; break;  // one block too many
        }
        ++*altered;
    }
    const int64_t units = (int64_t)Hkv * ((H / Hkv + 15) / 16);
    const int32_t limit = key_block_limit((int64_t)M * units);
    const int64_t sf = span_floor(max_len, limit);
    const int32_t ms = max_splits_for(M, H, max_len);
    CHECK(limit <= key_block_limit((int64_t)M * ((H + 15) / 16)), "floor finer than the workspace bound");
    CHECK(plan.ch == 16 || plan.ch == 32, "ch %d", plan.ch);
    CHECK(m.nseg >= 0 && m.nseg <= kMaxSegs, "nseg %d", m.nseg);
    int64_t grid = 0;
    for (int s = 0; s < m.nseg; ++s) {
        CHECK(m.start[s] == grid, "segment %d starts at %d, expected %lld", s, m.start[s], (long long)grid);
        const int32_t np = seg_npiece(m.info[s]), sq = seg_seq(m.info[s]);
        CHECK(np >= 1 && m.span[s] >= 1, "segment %d: %d blocks of %d keys", s, np, m.span[s]);
        CHECK(sq < M, "segment %d: sequence %d", s, sq);
        CHECK(seg_info(sq, np, seg_piece0(m.info[s])) == m.info[s], "segment %d: fields overflow", s);
        grid += (int64_t)np * units;
    }
    CHECK(grid == plan.grid && grid < (1ll << 31), "grid %d, segments give %lld", plan.grid, (long long)grid);
    for (int s = m.nseg; s <= kMaxSegs; ++s) CHECK(m.start[s] == plan.grid, "start[%d] past the last segment", s);
    int32_t most = 0;
    for (int i = 0; i < M; ++i) {
        std::vector<Block> blocks;
        for (int s = 0; s < m.nseg; ++s) {
            if (seg_seq(m.info[s]) != i) continue;
            for (int p = 0; p < seg_npiece(m.info[s]); ++p) {
                const int64_t k0 = (int64_t)m.kbase[s] + (int64_t)p * m.span[s];
                const int64_t k1 = std::min<int64_t>(k0 + m.span[s], lens[i]);
                CHECK(k0 < k1, "sequence %d: empty block [%lld, %lld)", i, (long long)k0, (long long)k1);
                CHECK(k0 + m.span[s] < (1ll << 31), "sequence %d: key index overflows int32", i);
                blocks.push_back({seg_piece0(m.info[s]) + p, k0, k1});
            }
        }
        std::sort(blocks.begin(), blocks.end(), [](const Block &x, const Block &y) { return x.slot < y.slot; });
        const int32_t n = (int32_t)blocks.size();
        CHECK(n == m.nsplit[i], "sequence %d: %d blocks, nsplit %d", i, n, m.nsplit[i]);
        CHECK(n <= ms, "sequence %d: %d blocks, the workspace holds %d", i, n, ms);
        CHECK((lens[i] == 0) == (n == 0), "sequence %d of %d keys has %d blocks", i, lens[i], n);
        int64_t pos = 0;
        for (int32_t j = 0; j < n; ++j) {
            CHECK(blocks[j].slot == j, "sequence %d: split slot %d at rank %d", i, blocks[j].slot, j);
            CHECK(blocks[j].k0 == pos, "sequence %d: block %d starts at %lld, keys end at %lld", i, j,
                  (long long)blocks[j].k0, (long long)pos);
            CHECK(j == n - 1 || blocks[j].k1 - blocks[j].k0 >= sf, "sequence %d: block %d below the floor", i, j);
            pos = blocks[j].k1;
        }
        CHECK(pos == lens[i], "sequence %d: blocks end at %lld of %d keys", i, (long long)pos, lens[i]);
        most = std::max(most, n);
    }
    for (int i = M; i < ATTN_MAX_SEQS; ++i) CHECK(m.nsplit[i] == 0, "unused sequence %d has splits", i);
    CHECK(plan.most == most, "most %d, expected %d", plan.most, most);
    *wide += most > 16;
    return true;
}

}  // namespace

int main(int argc, char **argv) {
    if (argc < 3) {
        fprintf(stderr, "usage: %s <seed> <calls> [corrupt]\n", argv[0]);
        return 2;
    }
    g_state = strtoull(argv[1], nullptr, 10);
    const long calls = strtol(argv[2], nullptr, 10);
    const bool corrupt = argc > 3 && strcmp(argv[3], "corrupt") == 0;
    static const int32_t kv_choices[] = {1, 2, 3, 4, 8, 16, 64};
    static const int32_t g_choices[] = {1, 2, 3, 4, 7, 8, 16, 20, 32};
    static const int64_t cu_choices[] = {8, 32, 80, 104, 256, 304};
    int64_t wide = 0, failed = 0, altered = 0;
    for (long c = 0; c < calls; ++c) {
        const int32_t M = (int32_t)uniform(1, ATTN_MAX_SEQS);
        const int32_t Hkv = kv_choices[uniform(0, 6)];
        const int32_t H = Hkv * g_choices[uniform(0, 8)];
        // max_len log-uniform over [1, 2^30], then the lengths: all full, uniform,
        // or uniform in the top half, with an empty and a one-key sequence mixed in.
        const int32_t max_len = (int32_t)std::min<int64_t>(1ll << 30, uniform(1, 2) << uniform(0, 29));
        int32_t lens[ATTN_MAX_SEQS] = {};
        const int64_t mode = uniform(0, 3);
        for (int i = 0; i < M; ++i)
            lens[i] = (int32_t)(mode == 0 ? max_len : mode == 1 ? uniform(0, max_len) : uniform(max_len / 2, max_len));
        if (mode == 3 && M >= 3) {
            lens[uniform(0, M - 1)] = 0;
            lens[uniform(0, M - 1)] = 1;
        }
        const int64_t cus = cu_choices[uniform(0, 5)];
        const int64_t cap32 = cus * uniform(1, 2), cap16 = std::max(cap32, cus * uniform(1, 3));
        if (!check_call(lens, M, H, Hkv, max_len, cus, cap32, cap16, corrupt, &wide, &altered)) {
            fprintf(stderr, "call %ld: M %d H %d Hkv %d max_len %d CUs %lld capacities %lld / %lld\n", c, M, H, Hkv,
                    max_len, (long long)cus, (long long)cap32, (long long)cap16);
            ++failed;
            if (!corrupt) return 1;
        }
    }
    if (corrupt) {
        printf("altered plans rejected: %lld of %lld\n", (long long)failed, (long long)altered);
        return failed == altered && altered > calls / 2 ? 0 : 1;
    }
    printf("ok %ld calls (%lld with more than 16 splits in a sequence)\n", calls, (long long)wide);
    return 0;
}
