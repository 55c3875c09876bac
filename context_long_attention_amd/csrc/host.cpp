// Host-side logic of libcpattn: argument validation, the zigzag partition, the
// ring order, chunk-pair classes, the tile block map and pair counts.  Plain
// C++17 with no HIP calls, so it also builds with g++ under sanitizers.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <queue>
#include <string>
#include <vector>

#include "internal.h"

namespace cpattn {

namespace {
thread_local std::string g_last_error;
constexpr int64_t kPosLimit = int64_t(1) << 31;
constexpr int64_t kNoLowerBound = std::numeric_limits<int64_t>::min() / 4;
// Largest query head count (keeps the kernels' 32-bit tile byte offsets in range).
constexpr int kMaxHeads = 8192;
}  // namespace

void set_error(const std::string& msg) { g_last_error = msg; }

cp_status fail(cp_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

TileGeom fwd_geom(int hq, int hkv) {
    int g = hq / hkv;
    int hpw = (g % 4 == 0) ? 4 : (g % 2 == 0 ? 2 : 1);
    return TileGeom{32 * kFwdWaves / hpw, 64, hpw};
}

int64_t doc_start_host(const int32_t* cu, int32_t n_docs, int64_t pos) {
    // last index d in [0, n_docs) with cu[d] <= pos
    int32_t lo = 0, hi = n_docs - 1;
    while (lo < hi) {
        int32_t mid = (lo + hi + 1) / 2;
        if (cu[mid] <= pos)
            lo = mid;
        else
            hi = mid - 1;
    }
    return cu[lo];
}

cp_status validate_problem(const cp_attn_problem* p, bool device_docs) {
    if (!p) return fail(CP_ERR_INVALID_ARG, "problem is NULL");
    if (p->hq <= 0 || p->hkv <= 0) return fail(CP_ERR_INVALID_ARG, "head counts must be positive");
    if (p->hq % p->hkv) return fail(CP_ERR_INVALID_ARG, "hq must be a multiple of hkv");
    // tiles are addressed with 32-bit byte offsets: 64 rows of hq * head_dim bf16 stay far below 2^31
    if (p->hq > kMaxHeads) return fail(CP_ERR_UNSUPPORTED, "hq above " + std::to_string(kMaxHeads));
    if (p->head_dim != 64 && p->head_dim != 128) return fail(CP_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (!std::isfinite(p->scale)) return fail(CP_ERR_INVALID_ARG, "scale must be finite");
    if (p->q_rows < 0 || p->kv_rows < 0 || p->q_rows >= kPosLimit || p->kv_rows >= kPosLimit)
        return fail(CP_ERR_INVALID_ARG, "row counts must be in [0, 2^31)");
    if (p->n_q_seg < 1 || p->n_q_seg > 2 || p->n_kv_seg < 1 || p->n_kv_seg > 2)
        return fail(CP_ERR_INVALID_ARG, "segment counts must be 1 or 2");
    if (p->window < 0) return fail(CP_ERR_INVALID_ARG, "window must be >= 0");
    if (p->kv_split < 0 || p->kv_split > kMaxKvSplit)
        return fail(CP_ERR_INVALID_ARG, "kv_split must be in [0, " + std::to_string(kMaxKvSplit) + "]");
    bool any_doc = false;
    // Range checks written so that no sum of caller values can overflow.
    for (int i = 0; i < p->n_q_seg; ++i) {
        const cp_segment& s = p->q_seg[i];
        if (s.row0 < 0 || s.len < 0 || s.pos0 < 0 || s.len > p->q_rows - s.row0 || s.pos0 > kPosLimit - s.len)
            return fail(CP_ERR_INVALID_ARG, "query segment out of range");
        for (int j = 0; j < p->n_kv_seg; ++j) {
            int m = p->mask[i][j];
            if (m < CP_MASK_FULL || m > CP_MASK_SKIP) return fail(CP_ERR_INVALID_ARG, "bad mask value");
            if (m == CP_MASK_DOC) any_doc = true;
        }
    }
    if (p->n_q_seg == 2) {
        const cp_segment& a = p->q_seg[0];
        const cp_segment& b = p->q_seg[1];
        if (a.len > 0 && b.len > 0 && a.row0 < b.row0 + b.len && b.row0 < a.row0 + a.len)
            return fail(CP_ERR_INVALID_ARG, "query segments overlap");
    }
    for (int j = 0; j < p->n_kv_seg; ++j) {
        const cp_segment& s = p->kv_seg[j];
        if (s.row0 < 0 || s.len < 0 || s.pos0 < 0 || s.len > p->kv_rows - s.row0 || s.pos0 > kPosLimit - s.len)
            return fail(CP_ERR_INVALID_ARG, "KV segment out of range");
    }
    if (p->n_kv_seg == 2) {
        const cp_segment& a = p->kv_seg[0];
        const cp_segment& b = p->kv_seg[1];
        if (a.len > 0 && b.len > 0 && a.row0 < b.row0 + b.len && b.row0 < a.row0 + a.len)
            return fail(CP_ERR_INVALID_ARG, "KV segments overlap");
    }
    if (any_doc) {
        if (!p->cu_seqlens || p->n_docs < 1) return fail(CP_ERR_INVALID_ARG, "DOC mask needs cu_seqlens");
        if (!device_docs) {
            const int32_t* cu = p->cu_seqlens;
            if (cu[0] != 0) return fail(CP_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
            for (int32_t d = 0; d < p->n_docs; ++d)
                if (cu[d + 1] < cu[d]) return fail(CP_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing");
            int64_t maxpos = 0;
            for (int i = 0; i < p->n_q_seg; ++i) maxpos = std::max(maxpos, p->q_seg[i].pos0 + p->q_seg[i].len);
            for (int j = 0; j < p->n_kv_seg; ++j) maxpos = std::max(maxpos, p->kv_seg[j].pos0 + p->kv_seg[j].len);
            if (cu[p->n_docs] < maxpos) return fail(CP_ERR_INVALID_ARG, "cu_seqlens does not cover the positions");
        }
    }
    return CP_OK;
}

int64_t row_lower_bound(const cp_attn_problem* p, int mask, int64_t q) {
    int64_t lo = kNoLowerBound;
    if (mask == CP_MASK_DOC) lo = doc_start_host(p->cu_seqlens, p->n_docs, q);
    if (p->window > 0 && (mask == CP_MASK_DOC || mask == CP_MASK_DIAG_CAUSAL)) lo = std::max(lo, q - p->window + 1);
    return lo;
}

static bool any_doc_pair(const cp_attn_problem* p) {
    for (int i = 0; i < p->n_q_seg; ++i)
        for (int j = 0; j < p->n_kv_seg; ++j)
            if (p->mask[i][j] == CP_MASK_DOC) return true;
    return false;
}

bool heavier_last(const std::vector<int64_t>& work) {
    const int64_t n = int64_t(work.size());
    double total = 0.0, moment = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        total += double(work[size_t(i)]);
        moment += double(i) * double(work[size_t(i)]);
    }
    if (n < 2 || total <= 0.0) return false;
    return moment / total > 0.5 * double(n - 1) + 0.01 * double(n - 1);
}

std::vector<int64_t> query_tile_work(const cp_attn_problem* p, int bm, int bn) {
    std::vector<int64_t> work;
    if (any_doc_pair(p)) return work;
    for (int i = 0; i < p->n_q_seg; ++i) {
        const cp_segment& qs = p->q_seg[i];
        for (int64_t qt = 0; qt < ceil_div(qs.len, bm); ++qt) {
            const int64_t q0 = qs.pos0 + qt * bm;
            const int64_t q1 = std::min(qs.pos0 + qs.len, q0 + bm) - 1;
            int64_t n = 0;
            for (int j = 0; j < p->n_kv_seg; ++j) {
                const int m = p->mask[i][j];
                const TileRange r = tile_range(m, q0, q1, row_lower_bound(p, m, q0), p->kv_seg[j].pos0,
                                               p->kv_seg[j].len, bn);
                n += r.t_hi - r.t_lo;
            }
            work.push_back(n);
        }
    }
    return work;
}

std::vector<int64_t> key_block_items(const cp_attn_problem* p, const int32_t* host_cu) {
    // Per 128-key block: the query tiles (of kBwdQRows rows, per query head) that
    // see one of its keys, by the ranges the dK/dV kernel walks.
    std::vector<int64_t> items;
    if (any_doc_pair(p) && !host_cu) return items;
    constexpr int64_t kInf = std::numeric_limits<int64_t>::max();
    const int64_t group = p->hq / p->hkv;
    for (int j = 0; j < p->n_kv_seg; ++j) {
        const cp_segment& ks = p->kv_seg[j];
        for (int64_t kb = 0; kb < ceil_div(ks.len, kBwdKeysPerWG); ++kb) {
            const int64_t k0 = ks.pos0 + kb * kBwdKeysPerWG;
            const int64_t k1 = std::min(ks.pos0 + ks.len, k0 + kBwdKeysPerWG) - 1;
            int64_t n = 0;
            for (int i = 0; i < p->n_q_seg; ++i) {
                const cp_segment& qs = p->q_seg[i];
                const int m = p->mask[i][j];
                const int64_t nqt = ceil_div(qs.len, kBwdQRows);
                if (m == CP_MASK_SKIP || qs.len == 0) continue;
                if (m == CP_MASK_FULL) {
                    n += nqt;
                    continue;
                }
                if (k0 > qs.pos0 + qs.len - 1) continue;  // causal: rows q >= k0
                const int64_t lo = (k0 <= qs.pos0) ? 0 : (k0 - qs.pos0) / kBwdQRows;
                // rows q < end of the last key's document and q < k1 + window
                int64_t qe = kInf;
                if (m == CP_MASK_DOC) {
                    int32_t a = 0, b = p->n_docs - 1;  // last document starting at or before k1
                    while (a < b) {
                        const int32_t mid = (a + b + 1) / 2;
                        if (host_cu[mid] <= k1)
                            a = mid;
                        else
                            b = mid - 1;
                    }
                    qe = host_cu[a + 1];
                }
                if (p->window > 0) qe = std::min(qe, k1 + p->window);
                int64_t hi = nqt;
                if (qe != kInf) hi = (qe - 1 < qs.pos0) ? 0 : std::min(nqt, (qe - 1 - qs.pos0) / kBwdQRows + 1);
                n += std::max<int64_t>(0, hi - lo);
            }
            items.push_back(n * group);
        }
    }
    return items;
}

bool dkdv_latest_first(const cp_attn_problem* p) {
    return !any_doc_pair(p) && heavier_last(key_block_items(p, nullptr));
}

int32_t dkdv_split(const cp_attn_problem* p, const int32_t* host_cu, int64_t n_cu) {
    // With documents and no host cu_seqlens the blocks' ranges are unknown: no split.
    if (any_doc_pair(p) && !host_cu) return 1;
    const std::vector<int64_t> items = key_block_items(p, host_cu);  // per block, in key-tile index order
    // the launch's block order, as the kernel takes it (documents: earliest first)
    const bool latest_first = !any_doc_pair(p) && heavier_last(items);
    const int64_t n_kt = int64_t(items.size());
    // Makespan of the launch in item times when workgroup w starts on the first
    // free slot in id order (two dK/dV workgroups per CU): part w / n_blocks of
    // block w mod n_blocks, whose key blocks run KV-head-minor, with the items of
    // a block in runs of ceil(items / split) per part.  A workgroup also costs a
    // fixed overhead (its K/V rows, the ring's fill and drain, the output
    // writes: about kWgOverhead items) and an empty one half an item.  A split
    // adds the reduction pass, which reads every slot of a block with more than
    // one part (and the outputs once more): kReduceSlotCost item times each.
    const int64_t slots = 2 * std::max<int64_t>(1, n_cu);
    const int64_t n_blocks = int64_t(items.size()) * p->hkv;
    if (n_blocks == 0 || n_blocks * kMaxKvSplit > (int64_t(1) << 22)) return 1;
    auto makespan = [&](int64_t split) {
        std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
        double end = 0.0;
        for (int64_t w = 0; w < split * n_blocks; ++w) {
            const int64_t part = w / n_blocks, kt0 = (w % n_blocks) / p->hkv;
            const int64_t kt = latest_first ? n_kt - 1 - kt0 : kt0;
            const int64_t n = items[kt];
            const int64_t run = (n + split - 1) / split;
            const int64_t it0 = std::min(n, part * run);
            const int64_t mine = std::min(n, it0 + run) - it0;
            const double cost = mine ? double(mine) + kWgOverhead : 0.5;
            double start = 0.0;
            if (int64_t(free_at.size()) == slots) {
                start = free_at.top();
                free_at.pop();
            }
            free_at.push(start + cost);
            end = std::max(end, start + cost);
        }
        if (split > 1) {
            double reads = 0.0;
            for (int64_t n : items) {
                const int64_t run = (n + split - 1) / split;
                const int64_t parts = run ? (n + run - 1) / run : 0;
                if (parts > 1) reads += double(parts + 1) * double(p->hkv);
            }
            end += kReduceSlotCost * reads;
        }
        return end;
    };
    // No split can beat the even share of all items over the slots: stop if the
    // launch without one is within 3% of it.  Otherwise take the smallest of 2, 4
    // and 8 within 3% of the best, if that gains 3% over no split.
    const double one = makespan(1);
    double total = 0.0;
    for (int64_t n : items) total += double(n) * p->hkv;
    if (one <= 1.03 * (total / double(slots))) return 1;
    const int64_t cand[3] = {2, 4, kMaxKvSplit};
    double t[3], best = one;
    for (int c = 0; c < 3; ++c) best = std::min(best, t[c] = makespan(cand[c]));
    if (best > 0.97 * one) return 1;
    for (int c = 0; c < 3; ++c)
        if (t[c] <= 1.03 * best) return int32_t(cand[c]);
    return 1;
}

cp_attn_problem live_queries(const cp_attn_problem* p) {
    cp_attn_problem r = *p;
    int n = 0;
    for (int i = 0; i < p->n_q_seg; ++i) {
        bool live = false;
        for (int j = 0; j < p->n_kv_seg; ++j) live |= p->mask[i][j] != CP_MASK_SKIP && p->kv_seg[j].len > 0;
        if (!live || p->q_seg[i].len == 0) continue;
        r.q_seg[n] = p->q_seg[i];
        for (int j = 0; j < 2; ++j) r.mask[n][j] = p->mask[i][j];
        ++n;
    }
    for (int i = n; i < 2; ++i) {
        r.q_seg[i] = cp_segment{0, 0, 0};
        for (int j = 0; j < 2; ++j) r.mask[i][j] = CP_MASK_SKIP;
    }
    r.n_q_seg = n;
    return r;
}

TileRange tile_range(int mask, int64_t q0, int64_t q1, int64_t lo0, int64_t kpos0, int64_t klen, int bn) {
    int64_t nkt = ceil_div(klen, bn);
    if (mask == CP_MASK_SKIP || klen == 0 || q1 < q0) return {0, 0};
    if (mask == CP_MASK_FULL) return {0, nkt};
    // Visible keys of the tile's rows form [lo0, q1] (lo is non-decreasing in q
    // and lo(q) <= q, so the per-row ranges [lo(q), q] chain without gaps).
    int64_t t_hi = (q1 < kpos0) ? 0 : std::min(nkt, (q1 - kpos0) / bn + 1);
    int64_t t_lo = 0;
    if (lo0 > kpos0) {
        if (lo0 > kpos0 + klen - 1) return {0, 0};
        t_lo = (lo0 - kpos0) / bn;
    }
    if (t_lo >= t_hi) return {0, 0};
    return {t_lo, t_hi};
}

int tile_class(int mask, int64_t q0, int64_t q1, int64_t lo1, int64_t kpos0, int64_t klen, int bn, int64_t t) {
    if (mask == CP_MASK_FULL) return CP_TILE_FULL;
    int64_t k0 = kpos0 + t * bn;
    int64_t k1 = std::min(kpos0 + klen, k0 + bn) - 1;
    // every pair visible iff the last row's lower bound is <= k0 and k1 <= q0
    (void)q1;
    return (k1 <= q0 && k0 >= lo1) ? CP_TILE_FULL : CP_TILE_PARTIAL;
}

}  // namespace cpattn

using namespace cpattn;

extern "C" {

int32_t cp_abi_version(void) { return CPATTN_ABI_VERSION; }

const char* cp_status_string(cp_status s) {
    switch (s) {
        case CP_OK: return "ok";
        case CP_ERR_INVALID_ARG: return "invalid argument";
        case CP_ERR_UNSUPPORTED: return "unsupported";
        case CP_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* cp_last_error(void) { return g_last_error.c_str(); }

cp_status cp_partition_zigzag(int64_t seq_len, int32_t cp_size, int32_t rank, int64_t* pos_out) {
    if (!pos_out) return fail(CP_ERR_INVALID_ARG, "pos_out is NULL");
    if (cp_size < 1 || rank < 0 || rank >= cp_size) return fail(CP_ERR_INVALID_ARG, "rank out of range");
    if (seq_len <= 0 || seq_len % (2 * int64_t(cp_size)))
        return fail(CP_ERR_INVALID_ARG, "seq_len must be a positive multiple of 2*cp_size");
    const int64_t c = seq_len / (2 * int64_t(cp_size));
    const int64_t first = rank, second = 2 * int64_t(cp_size) - 1 - rank;
    for (int64_t i = 0; i < c; ++i) {
        pos_out[i] = first * c + i;
        pos_out[c + i] = second * c + i;
    }
    return CP_OK;
}

cp_status cp_ring_source(int32_t cp_size, int32_t rank, int32_t step, int32_t* src_out) {
    if (!src_out) return fail(CP_ERR_INVALID_ARG, "src_out is NULL");
    if (cp_size < 1 || rank < 0 || rank >= cp_size || step < 0 || step >= cp_size)
        return fail(CP_ERR_INVALID_ARG, "rank or step out of range");
    *src_out = ((rank - step) % cp_size + cp_size) % cp_size;
    return CP_OK;
}

cp_status cp_step_masks(int32_t cp_size, int32_t rank, int32_t step, int32_t packed, int32_t mask_out[4]) {
    int32_t src = 0;
    cp_status st = cp_ring_source(cp_size, rank, step, &src);
    if (st != CP_OK) return st;
    if (!mask_out) return fail(CP_ERR_INVALID_ARG, "mask_out is NULL");
    const int32_t qchunk[2] = {rank, 2 * cp_size - 1 - rank};
    const int32_t kchunk[2] = {src, 2 * cp_size - 1 - src};
    for (int i = 0; i < 2; ++i) {
        for (int j = 0; j < 2; ++j) {
            int32_t m;
            if (kchunk[j] > qchunk[i])
                m = CP_MASK_SKIP;
            else if (packed)
                m = CP_MASK_DOC;
            else
                m = (kchunk[j] < qchunk[i]) ? CP_MASK_FULL : CP_MASK_DIAG_CAUSAL;
            mask_out[2 * i + j] = m;
        }
    }
    return CP_OK;
}

cp_status cp_step_masks_window(int64_t seq_len, int32_t cp_size, int32_t rank, int32_t step, int32_t packed,
                               int64_t window, int32_t mask_out[4]) {
    int32_t src = 0;
    cp_status st = cp_ring_source(cp_size, rank, step, &src);
    if (st != CP_OK) return st;
    if (!mask_out) return fail(CP_ERR_INVALID_ARG, "mask_out is NULL");
    if (window < 0) return fail(CP_ERR_INVALID_ARG, "window must be >= 0");
    if (seq_len <= 0 || seq_len % (2 * int64_t(cp_size)))
        return fail(CP_ERR_INVALID_ARG, "seq_len must be a positive multiple of 2*cp_size");
    const int64_t c = seq_len / (2 * int64_t(cp_size));
    const int64_t qchunk[2] = {rank, 2 * int64_t(cp_size) - 1 - rank};
    const int64_t kchunk[2] = {src, 2 * int64_t(cp_size) - 1 - src};
    for (int i = 0; i < 2; ++i) {
        for (int j = 0; j < 2; ++j) {
            const int64_t gap = qchunk[i] - kchunk[j];
            int32_t m;
            if (gap < 0 || (window > 0 && (gap - 1) * c + 1 >= window))
                m = CP_MASK_SKIP;  // above the diagonal, or even the closest pair is out of the window
            else if (packed)
                m = CP_MASK_DOC;
            else if (gap > 0 && (window == 0 || (gap + 1) * c - 1 < window))
                m = CP_MASK_FULL;  // strictly below the diagonal and the farthest pair in the window
            else
                m = CP_MASK_DIAG_CAUSAL;
            mask_out[2 * i + j] = m;
        }
    }
    return CP_OK;
}

cp_status cp_tile_shape(int32_t hq, int32_t hkv, int32_t head_dim, int32_t* bm_out, int32_t* bn_out) {
    if (!bm_out || !bn_out) return fail(CP_ERR_INVALID_ARG, "output pointer is NULL");
    if (hq <= 0 || hkv <= 0 || hq % hkv) return fail(CP_ERR_INVALID_ARG, "bad head counts");
    if (head_dim != 64 && head_dim != 128) return fail(CP_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    TileGeom g = fwd_geom(hq, hkv);
    *bm_out = g.bm;
    *bn_out = g.bn;
    return CP_OK;
}

cp_status cp_block_map_size(const cp_attn_problem* p, int64_t* n_q_tiles, int64_t* n_k_tiles) {
    if (!n_q_tiles || !n_k_tiles) return fail(CP_ERR_INVALID_ARG, "output pointer is NULL");
    cp_status st = validate_problem(p, true);
    if (st != CP_OK) return st;
    TileGeom g = fwd_geom(p->hq, p->hkv);
    int64_t nq = 0, nk = 0;
    for (int i = 0; i < p->n_q_seg; ++i) nq += ceil_div(p->q_seg[i].len, g.bm);
    for (int j = 0; j < p->n_kv_seg; ++j) nk += ceil_div(p->kv_seg[j].len, g.bn);
    *n_q_tiles = nq;
    *n_k_tiles = nk;
    return CP_OK;
}

cp_status cp_block_map(const cp_attn_problem* p, uint8_t* map_out) {
    int64_t nq = 0, nk = 0;
    cp_status st = cp_block_map_size(p, &nq, &nk);
    if (st != CP_OK) return st;
    st = validate_problem(p, false);
    if (st != CP_OK) return st;
    if (!map_out && nq * nk > 0) return fail(CP_ERR_INVALID_ARG, "map_out is NULL");
    TileGeom g = fwd_geom(p->hq, p->hkv);
    int64_t row = 0;
    for (int i = 0; i < p->n_q_seg; ++i) {
        const cp_segment& qs = p->q_seg[i];
        for (int64_t qt = 0; qt < ceil_div(qs.len, g.bm); ++qt, ++row) {
            const int64_t q0 = qs.pos0 + qt * g.bm;
            const int64_t q1 = std::min(qs.pos0 + qs.len, q0 + g.bm) - 1;
            int64_t col = 0;
            for (int j = 0; j < p->n_kv_seg; ++j) {
                const cp_segment& ks = p->kv_seg[j];
                const int m = p->mask[i][j];
                const int64_t lo0 = row_lower_bound(p, m, q0);
                const int64_t lo1 = row_lower_bound(p, m, q1);
                const int64_t nkt = ceil_div(ks.len, g.bn);
                TileRange r = tile_range(m, q0, q1, lo0, ks.pos0, ks.len, g.bn);
                for (int64_t t = 0; t < nkt; ++t) {
                    uint8_t c = CP_TILE_SKIP;
                    if (t >= r.t_lo && t < r.t_hi)
                        c = uint8_t(tile_class(m, q0, q1, lo1, ks.pos0, ks.len, g.bn, t));
                    map_out[row * nk + col + t] = c;
                }
                col += nkt;
            }
        }
    }
    return CP_OK;
}

cp_status cp_bwd_kv_split(const cp_attn_problem* p, int32_t n_cu, int32_t* split_out) {
    if (!split_out) return fail(CP_ERR_INVALID_ARG, "split_out is NULL");
    if (n_cu < 1) return fail(CP_ERR_INVALID_ARG, "n_cu must be positive");
    cp_status st = validate_problem(p, false);
    if (st != CP_OK) return st;
    *split_out = dkdv_split(p, p->cu_seqlens, n_cu);
    return CP_OK;
}

cp_status cp_bwd_workspace_size(const cp_attn_problem* p, int32_t kv_split, int64_t* bytes_out) {
    if (!bytes_out) return fail(CP_ERR_INVALID_ARG, "bytes_out is NULL");
    if (kv_split < 1 || kv_split > kMaxKvSplit)
        return fail(CP_ERR_INVALID_ARG, "kv_split must be in [1, " + std::to_string(kMaxKvSplit) + "]");
    cp_status st = validate_problem(p, true);
    if (st != CP_OK) return st;
    *bytes_out = dkdv_workspace_bytes(p, kv_split);
    return CP_OK;
}

cp_status cp_count_pairs(const cp_attn_problem* p, int64_t* pairs_out) {
    if (!pairs_out) return fail(CP_ERR_INVALID_ARG, "pairs_out is NULL");
    cp_status st = validate_problem(p, false);
    if (st != CP_OK) return st;
    int64_t total = 0;
    for (int i = 0; i < p->n_q_seg; ++i) {
        const cp_segment& qs = p->q_seg[i];
        for (int j = 0; j < p->n_kv_seg; ++j) {
            const cp_segment& ks = p->kv_seg[j];
            const int m = p->mask[i][j];
            if (m == CP_MASK_SKIP || qs.len == 0 || ks.len == 0) continue;
            if (m == CP_MASK_FULL) {
                total += qs.len * ks.len;
                continue;
            }
            const int64_t kend = ks.pos0 + ks.len;  // exclusive
            for (int64_t r = 0; r < qs.len; ++r) {
                const int64_t q = qs.pos0 + r;
                const int64_t lo = std::max(ks.pos0, row_lower_bound(p, m, q));
                const int64_t hi = std::min(kend, q + 1);  // exclusive
                if (hi > lo) total += hi - lo;
            }
        }
    }
    *pairs_out = total;
    return CP_OK;
}

}  // extern "C"
