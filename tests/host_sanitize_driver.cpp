// Test driver for the host logic of libcpattn (host.cpp), built by
// tests/test_host_sanitized.py with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer (every finding aborts the run).
//
// It first runs a fixed battery of host calls -- the zigzag partition, ring
// order and chunk classes over many (S, R, rank, step, window) shapes, the tile
// shape, and argument errors -- checking the invariants it can check alone
// (exit 1 on a violation).  Then it reads problems from stdin, one per line:
//   hq hkv head_dim q_rows kv_rows n_q (row pos len)*n_q n_kv (row pos len)*n_kv
//   m00 m01 m10 m11 window kv_split n_docs cu[0..n_docs]   (n_docs 0: no documents)
// and prints one line per problem with the results of every host call on it:
//   status n_q_tiles n_k_tiles status_map map_hash status_pairs pairs split(1)
//   split(8) split(64) split(256) ws(1) .. ws(8)
// which the test compares with the regular build's results.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "cpattn.h"

namespace {

int g_fail = 0;

void check(bool ok, const char* what, long long a = 0, long long b = 0, long long c = 0) {
    if (!ok) {
        std::fprintf(stderr, "battery: %s (%lld %lld %lld)\n", what, a, b, c);
        g_fail = 1;
    }
}

void battery() {
    // partition: a permutation of [0, S) over the ranks, each 2c positions, chunks r and 2R-1-r
    for (int R = 1; R <= 16; ++R)
        for (int64_t S : {int64_t(2 * R), int64_t(4 * R), int64_t(6 * R), int64_t(64 * R), int64_t(2 * R * 37)}) {
            std::vector<int> seen(size_t(S), 0);
            const int64_t c = S / (2 * R);
            for (int r = 0; r < R; ++r) {
                std::vector<int64_t> pos(size_t(S / R), -1);
                check(cp_partition_zigzag(S, R, r, pos.data()) == CP_OK, "partition status", S, R, r);
                for (int64_t i = 0; i < S / R; ++i) {
                    const int64_t x = pos[size_t(i)];
                    check(x >= 0 && x < S, "partition range", S, R, x);
                    if (x >= 0 && x < S) seen[size_t(x)]++;
                    const int64_t chunk = (i < c) ? r : 2 * R - 1 - r;
                    check(x / c == chunk, "partition chunk", S, R, i);
                }
                for (int t = 0; t < R; ++t) {
                    int32_t src = -1;
                    check(cp_ring_source(R, r, t, &src) == CP_OK && src == ((r - t) % R + R) % R, "ring source", R,
                          r, t);
                    int32_t m[4], mw[4];
                    for (int packed = 0; packed < 2; ++packed) {
                        check(cp_step_masks(R, r, t, packed, m) == CP_OK, "step masks", R, r, t);
                        for (int64_t win : {int64_t(0), int64_t(1), c, 2 * c + 1, S}) {
                            check(cp_step_masks_window(S, R, r, t, packed, win, mw) == CP_OK, "window masks", S, r,
                                  win);
                            if (win == 0)
                                for (int e = 0; e < 4; ++e) check(mw[e] == m[e], "window 0 equals causal", R, r, t);
                        }
                    }
                }
            }
            for (int64_t x = 0; x < S; ++x) check(seen[size_t(x)] == 1, "partition permutation", S, R, x);
        }
    // argument errors
    int64_t pos[8];
    int32_t m[4], src;
    check(cp_partition_zigzag(10, 3, 0, pos) == CP_ERR_INVALID_ARG, "partition S % 2R");
    check(cp_partition_zigzag(8, 2, 2, pos) == CP_ERR_INVALID_ARG, "partition rank");
    check(cp_partition_zigzag(8, 2, 0, nullptr) == CP_ERR_INVALID_ARG, "partition NULL");
    check(cp_partition_zigzag(0, 2, 0, pos) == CP_ERR_INVALID_ARG, "partition S = 0");
    check(cp_ring_source(0, 0, 0, &src) == CP_ERR_INVALID_ARG, "ring cp 0");
    check(cp_ring_source(4, 0, 4, &src) == CP_ERR_INVALID_ARG, "ring step");
    check(cp_ring_source(4, 0, 0, nullptr) == CP_ERR_INVALID_ARG, "ring NULL");
    check(cp_step_masks(4, 4, 0, 0, m) == CP_ERR_INVALID_ARG, "masks rank");
    check(cp_step_masks(4, 0, 0, 0, nullptr) == CP_ERR_INVALID_ARG, "masks NULL");
    check(cp_step_masks_window(16, 4, 0, 0, 0, -1, m) == CP_ERR_INVALID_ARG, "masks window < 0");
    check(cp_step_masks_window(18, 4, 0, 0, 0, 3, m) == CP_ERR_INVALID_ARG, "masks window S");
    int32_t bm = 0, bn = 0;
    check(cp_tile_shape(32, 8, 128, &bm, &bn) == CP_OK && bm > 0 && bn > 0, "tile shape");
    check(cp_tile_shape(32, 8, 96, &bm, &bn) == CP_ERR_UNSUPPORTED, "tile shape head_dim");
    check(cp_tile_shape(32, 8, 128, nullptr, &bn) == CP_ERR_INVALID_ARG, "tile shape NULL");
    check(cp_block_map_size(nullptr, nullptr, nullptr) == CP_ERR_INVALID_ARG, "block map size NULL");
    check(cp_block_map(nullptr, nullptr) == CP_ERR_INVALID_ARG, "block map NULL");
    check(cp_count_pairs(nullptr, nullptr) == CP_ERR_INVALID_ARG, "pairs NULL");
    check(cp_bwd_kv_split(nullptr, 1, nullptr) == CP_ERR_INVALID_ARG, "split NULL");
    check(cp_bwd_workspace_size(nullptr, 2, nullptr) == CP_ERR_INVALID_ARG, "workspace NULL");
    for (int s : {-3, -2, -1, 0, 1, 2, 3, 7})
        check(cp_status_string(cp_status(s)) != nullptr && cp_last_error() != nullptr, "status string", s);
    check(cp_abi_version() == CPATTN_ABI_VERSION, "abi version");
}

uint64_t fnv(const std::vector<uint8_t>& v) {
    uint64_t h = 1469598103934665603ull;
    for (uint8_t b : v) {
        h ^= b;
        h *= 1099511628211ull;
    }
    return h;
}

}  // namespace

int main() {
    battery();
    std::string line;
    while (std::getline(std::cin, line)) {
        if (line.empty()) continue;
        std::istringstream in(line);
        cp_attn_problem p;
        std::memset(&p, 0, sizeof(p));
        in >> p.hq >> p.hkv >> p.head_dim >> p.q_rows >> p.kv_rows >> p.n_q_seg;
        for (int i = 0; i < p.n_q_seg && i < 2; ++i) in >> p.q_seg[i].row0 >> p.q_seg[i].pos0 >> p.q_seg[i].len;
        in >> p.n_kv_seg;
        for (int j = 0; j < p.n_kv_seg && j < 2; ++j) in >> p.kv_seg[j].row0 >> p.kv_seg[j].pos0 >> p.kv_seg[j].len;
        in >> p.mask[0][0] >> p.mask[0][1] >> p.mask[1][0] >> p.mask[1][1] >> p.window >> p.kv_split >> p.n_docs;
        // the document table lives in a buffer of exactly n_docs + 1 entries
        std::vector<int32_t> cu(size_t(p.n_docs > 0 ? p.n_docs + 1 : 0));
        for (auto& x : cu) in >> x;
        p.cu_seqlens = p.n_docs > 0 ? cu.data() : nullptr;
        p.scale = 0.125f;
        int64_t nq = -1, nk = -1, pairs = -1;
        const int st = cp_block_map_size(&p, &nq, &nk);
        int st_map = -100;
        uint64_t h = 0;
        if (st == CP_OK) {
            // the map of exactly n_q_tiles x n_k_tiles entries (a host document
            // table is checked here, not by the size query)
            std::vector<uint8_t> map(size_t(nq * nk));
            st_map = cp_block_map(&p, map.data());
            if (st_map == CP_OK) h = fnv(map);
        }
        const int st_pairs = cp_count_pairs(&p, &pairs);
        std::cout << st << ' ' << nq << ' ' << nk << ' ' << st_map << ' ' << h << ' ' << st_pairs << ' ' << pairs;
        for (int n_cu : {1, 8, 64, 256}) {
            int32_t split = -1;
            std::cout << ' ' << (cp_bwd_kv_split(&p, n_cu, &split) == CP_OK ? split : -1);
        }
        for (int s = 1; s <= 8; ++s) {
            int64_t b = -1;
            std::cout << ' ' << (cp_bwd_workspace_size(&p, s, &b) == CP_OK ? b : -1);
        }
        std::cout << '\n';
    }
    return g_fail;
}
