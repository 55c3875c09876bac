// Backward of one Pass-KV ring step on gfx950 ("Announcing Long-Context
// Training on TPUs with MaxText Context Parallelism", section "Built on a fast
// attention kernel": the ring calls the kernel once per step in the backward
// pass as well).  Given the final LSE and delta = rowsum(dO * O) of every local
// row, one step contributes
//   P = exp(scale q.k - LSE) on visible pairs,  dS = P (dO.v - delta),
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,  dQ_i += scale sum_j dS_ij k_j.
//
// Two kernels, no atomics in their loops (wave64, 32x32x16 bf16 MFMA, fp32 accumulation):
//  * bwd_dkdv_kernel: a 4-wave workgroup owns 128 keys (32 per wave) of one KV
//    head, holds their K and V rows in registers, and walks every (query head of
//    the group, 32-row query tile) that can see them.  Query and dO tiles, with
//    their LSE and delta rows, stream HBM -> LDS through a four-slot ring two
//    items ahead.  S = Q K^T and dP = dO V^T put the queries on the MFMA M axis,
//    so each lane holds one key and its P / dS registers are directly the B
//    operands of dV^T += dO^T P and dK^T += Q^T dS; dO^T and Q^T come from the
//    row-major LDS tiles through the transposing LDS read.  dK/dV stay in
//    registers and are written once.  When an unbalanced block's items are split
//    over several workgroups, the first part writes the outputs and the others
//    write their partial sums to a caller-supplied workspace, which a small
//    reduction kernel adds to the outputs in part order: no atomics, so the
//    result does not depend on timing.
//  * bwd_dq_kernel: the forward kernel's shape (8 waves, 32 query rows of one
//    head per wave, heads of a GQA group sharing K/V tiles, four-slot ring of
//    K/V tiles): S^T = K Q^T and dP^T = V dO^T put one query per lane, so the
//    row's LSE and delta are per-lane scalars, and dQ^T += K^T dS^T reads K
//    transposed from the same LDS tile.  Each wave owns its dQ rows and adds
//    its sum to the accumulator once.
// This recomputes S and dP in both kernels (7 products instead of 5) in
// exchange for no atomics anywhere and two clean streaming loops.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "internal.h"
#include "tiles.h"

namespace cpattn {
namespace {

using namespace dev;

constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* d_o;
    const float* lse;
    const float* delta;
    float* dq;
    float* dk;
    float* dv;
    float* ws;  // split parts 1 .. kv_split-1: [kv_split - 1][n_work_kv][2][BK][D] partial dK, dV
    const int32_t* cu;
    int32_t n_docs;
    int32_t window;  // sliding window (0: none)
    int32_t hq, hkv, group;
    int32_t q_rows;
    float scale, scale_log2;
    int32_t nq_seg, nkv_seg;
    int32_t qs_row0[2], qs_pos0[2], qs_len[2];
    int32_t ks_row0[2], ks_pos0[2], ks_len[2];
    int32_t mask[2][2];
    // dK/dV kernel: 128-key tiles, each spread over kv_split workgroups;
    // k_last: key tiles latest first instead of earliest first
    int32_t ktiles0, n_ktiles, n_work_kv, kv_split, k_last;
    // dQ kernel: query tiles of BMQ rows; q_first: earliest first instead of
    // latest first
    int32_t qtiles0, n_qtiles, n_work_q, n_hb, q_first;
};

// ============================================================================ dK / dV
constexpr int kKvWaves = 4;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int BK = kBwdKeysPerWG;  // 128 keys per workgroup
constexpr int BQ = kBwdQRows;      // 32 query rows per tile
constexpr int kAuxBytes = 256 * kKvWaves;  // per slot: LSE row, delta row, two dummy areas
constexpr int kNoEnd = 0x7fffffff;

// Rows q visible from key k satisfy k <= q < qend: qend is the end of k's
// document (DOC) and k + window (sliding window, DIAG and DOC), whichever is
// earlier; both are non-decreasing in k.
__device__ __forceinline__ int window_end(int win, int k) { return (win > 0 && k <= kNoEnd - win) ? k + win : kNoEnd; }
__device__ __forceinline__ int query_end(int m, int doc_end, int w_end) {
    return (m == CP_MASK_DOC) ? min(doc_end, w_end) : (m == CP_MASK_DIAG_CAUSAL ? w_end : kNoEnd);
}

// Key block b of a dK/dV launch (BK keys of KV head g, blocks KV-head-minor)
// and its items: the (query head of the group, BQ-row query tile) pairs that
// see one of its keys, n0 + (thi[1] - tlo[1]) tiles per head over the two
// query segments, n_all in all.  The dK/dV kernel walks these items and the
// reduction kernel recounts them.
struct KvBlock {
    int g, s, kt_in, key_row0, kpos0, kcount;
    bool any_doc;
    int kend_first, kend_last;  // document ends of the first and last key (DOC pairs)
    int tlo[2], thi[2];
    int n0, per_head, n_all;
};

__device__ __forceinline__ KvBlock kv_block(const BwdParams& p, int b) {
    KvBlock k;
    k.g = b % p.hkv;
    const int kt = p.k_last ? p.n_ktiles - 1 - b / p.hkv : b / p.hkv;
    k.s = (kt < p.ktiles0) ? 0 : 1;
    k.kt_in = k.s ? kt - p.ktiles0 : kt;
    k.key_row0 = p.ks_row0[k.s] + k.kt_in * BK;
    k.kpos0 = p.ks_pos0[k.s] + k.kt_in * BK;
    k.kcount = min(BK, p.ks_len[k.s] - k.kt_in * BK);
    const int k0p = k.kpos0, k1p = k.kpos0 + k.kcount - 1;
    k.any_doc = false;
    for (int qs = 0; qs < p.nq_seg; ++qs) k.any_doc |= (p.mask[qs][k.s] == CP_MASK_DOC);
    k.kend_first = k.kend_last = kNoEnd;
    if (k.any_doc) {
        k.kend_first = p.cu[doc_index(p.cu, p.n_docs, k0p) + 1];
        k.kend_last = p.cu[doc_index(p.cu, p.n_docs, k1p) + 1];
    }
    const int wend_last = window_end(p.window, k1p);
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        k.tlo[qs] = k.thi[qs] = 0;
        if (qs >= p.nq_seg) continue;
        const int m = p.mask[qs][k.s];
        const int plen = p.qs_len[qs], ppos = p.qs_pos0[qs];
        const int nqt = (plen + BQ - 1) / BQ;
        if (m == CP_MASK_SKIP || plen == 0 || k.kcount <= 0) continue;
        if (m == CP_MASK_FULL) {
            k.thi[qs] = nqt;
            continue;
        }
        if (k0p > ppos + plen - 1) continue;  // causal: rows q >= k0p
        const int lo = (k0p <= ppos) ? 0 : (k0p - ppos) / BQ;
        int hi = nqt;
        const int qe = query_end(m, k.kend_last, wend_last);  // and q < qend of the last key
        if (qe != kNoEnd) {
            const int qmax = qe - 1;
            hi = (qmax < ppos) ? 0 : min(nqt, (qmax - ppos) / BQ + 1);
        }
        if (lo < hi) {
            k.tlo[qs] = lo;
            k.thi[qs] = hi;
        }
    }
    k.n0 = k.thi[0] - k.tlo[0];
    k.per_head = k.n0 + (k.thi[1] - k.tlo[1]);
    k.n_all = k.per_head * p.group;
    return k;
}

// Items of part `part` when a block's n_all items are split over `split`
// workgroups: consecutive runs of ceil(n_all / split) items, so the parts that
// have items come first and number ceil(n_all / run).
__device__ __forceinline__ int split_run(int n_all, int split) { return (n_all + split - 1) / split; }
__device__ __forceinline__ void part_items(int n_all, int split, int part, int& it0, int& n_it) {
    const int run = split_run(n_all, split);
    it0 = min(n_all, part * run);
    n_it = min(n_all, it0 + run) - it0;
}


template <int D>
__global__ __launch_bounds__(kKvThreads, 2) void bwd_dkdv_kernel(const BwdParams p) {
    using L = TileLayout<D, BQ>;
    constexpr int DS = D / 16;
    constexpr int DB = D / 32;
    // four-slot ring: query tile, dO tile and (LSE, delta) rows of one item each
    __shared__ __attribute__((aligned(16))) char qt0[L::BYTES];
    __shared__ __attribute__((aligned(16))) char qt1[L::BYTES];
    __shared__ __attribute__((aligned(16))) char qt2[L::BYTES];
    __shared__ __attribute__((aligned(16))) char qt3[L::BYTES];
    __shared__ __attribute__((aligned(16))) char ot0[L::BYTES];
    __shared__ __attribute__((aligned(16))) char ot1[L::BYTES];
    __shared__ __attribute__((aligned(16))) char ot2[L::BYTES];
    __shared__ __attribute__((aligned(16))) char ot3[L::BYTES];
    __shared__ __attribute__((aligned(16))) char ax0[kAuxBytes];
    __shared__ __attribute__((aligned(16))) char ax1[kAuxBytes];
    __shared__ __attribute__((aligned(16))) char ax2[kAuxBytes];
    __shared__ __attribute__((aligned(16))) char ax3[kAuxBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int hl = lane >> 5;
    const int ql = lane & 31;

    // workgroup w takes part w / n_work_kv of key block b = w mod n_work_kv, which
    // runs on XCD b mod 8 when n_work_kv is a multiple of 8 (workgroups are dealt
    // round-robin): KV head b mod Hkv, key tiles earliest first (the most queries
    // under a causal mask; latest first when the host found those to see more)
    const int w = blockIdx.x;
    if (w >= p.n_work_kv * p.kv_split) return;
    const int part = w / p.n_work_kv;
    const int b = w - part * p.n_work_kv;
    const KvBlock kb = kv_block(p, b);
    const int g = kb.g, s = kb.s, key_row0 = kb.key_row0, kpos0 = kb.kpos0, kcount = kb.kcount;
    // query-segment parameters as opaque scalars, selected by value below (an
    // index into the parameter block would be a scalar memory load, whose wait
    // also drains the LDS counter, at every use)
    const int qlen_a = sreg(p.qs_len[0]), qlen_b = sreg(p.qs_len[1]);
    const int qrow_a = sreg(p.qs_row0[0]), qrow_b = sreg(p.qs_row0[1]);
    const int qpos_a = sreg(p.qs_pos0[0]), qpos_b = sreg(p.qs_pos0[1]);
    const int mq_a = sreg(s ? p.mask[0][1] : p.mask[0][0]), mq_b = sreg(s ? p.mask[1][1] : p.mask[1][0]);
    const int k1p = kpos0 + kcount - 1;
    const int kk = 32 * wave + ql;  // this lane's key within the tile
    const bool key_valid = kk < kcount;
    const int kp = kpos0 + kk;
    const int64_t kv_stride = (int64_t)p.hkv * D;

    // ---- this lane's key and value rows as MFMA B operands (k-slots = dims 16ds + 8hl + 0..7)
    bf16x8 kf[DS], vf[DS];
    {
        const int64_t base = (int64_t)(key_row0 + kk) * kv_stride + (int64_t)g * D + 8 * hl;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if (key_valid) {
                a = *reinterpret_cast<const u32x4*>(p.k + base + 16 * ds);
                b = *reinterpret_cast<const u32x4*>(p.v + base + 16 * ds);
            }
            kf[ds] = __builtin_bit_cast(bf16x8, a);
            vf[ds] = __builtin_bit_cast(bf16x8, b);
        }
    }

    // ---- this lane's query end (see query_end), and the block's first key's
    int kend_lane = kNoEnd;
    if (kb.any_doc) {
        int j = doc_index(p.cu, p.n_docs, kpos0);
        if (key_valid) {
            while (j + 1 < p.n_docs && p.cu[j + 1] <= kp) ++j;
        }
        kend_lane = p.cu[j + 1];
    }
    const int win = p.window;
    const int wend_lane = window_end(win, kp), wend_first = window_end(win, kpos0);
    const int kend_first = kb.kend_first;
    auto qend = [](int m, int doc_end, int w_end) { return query_end(m, doc_end, w_end); };

    // ---- this workgroup's part of the block's items: [it0, it0 + n_it)
    const int tlo[2] = {kb.tlo[0], kb.tlo[1]};
    const int n0 = kb.n0, per_head = kb.per_head;
    int it0, n_it;
    part_items(kb.n_all, p.kv_split, part, it0, n_it);
    const int qrow_bytes = p.hq * D * 2;

    struct Item {
        int head, qs, tq;
    };
    auto item_of = [&](int it) -> Item {
        const int gi = it0 + it;
        const int head = g * p.group + gi / max(per_head, 1);
        const int rem = gi - (head - g * p.group) * per_head;
        const int qs = (rem < n0) ? 0 : 1;
        return Item{head, qs, qs ? tlo[1] + (rem - n0) : tlo[0] + rem};
    };
    // loads of item `it` (empty descriptors past the end keep every step's load count equal)
    auto issue = [&](int it, char* qdst, char* odst, char* adst) {
        const Item x = item_of(it);
        const bool live = it < n_it;
        const int rows = live ? min(BQ, pick(x.qs != 0, qlen_b, qlen_a) - x.tq * BQ) : 0;
        const int row0 = pick(x.qs != 0, qrow_b, qrow_a) + x.tq * BQ;
        const int64_t off = ((int64_t)row0 * p.hq + x.head) * D;
        load_tile_lds<D, BQ, kKvWaves>(qdst, tile_rsrc(p.q + off, rows, qrow_bytes), qrow_bytes, wave, lane);
        load_tile_lds<D, BQ, kKvWaves>(odst, tile_rsrc(p.d_o + off, rows, qrow_bytes), qrow_bytes, wave, lane);
        const int64_t roff = (int64_t)x.head * p.q_rows + row0;
        const float* src = (wave == 0) ? p.lse + roff : p.delta + roff;
        load_dwords_lds(adst + 256 * wave, tile_rsrc(src, wave < 2 ? rows : 0, 4), lane * 4);
    };

    f32x16 dka[DB], dva[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dka[db] = f32x16{};
        dva[db] = f32x16{};
    }
    const float c2 = p.scale_log2;
    const int q_lane = TileLayout<D, BQ>::off(ql, 8 * hl);
    const int grp = lane >> 4, jl = lane & 15;
    const int t_lane = TileLayout<D, BQ>::off(4 * (grp >> 1) + (jl >> 2), 16 * (grp & 1) + 4 * (jl & 3));
    auto step = [&](auto bar, int it, const char* qsl, const char* osl, const char* asl, char* qfill, char* ofill,
                    char* afill) {
        const Item x = item_of(it);
        const int m = pick(x.qs != 0, mq_b, mq_a);
        const int qrows = min(BQ, pick(x.qs != 0, qlen_b, qlen_a) - x.tq * BQ);
        const int qpos0 = pick(x.qs != 0, qpos_b, qpos_a) + x.tq * BQ;

        // S = Q K^T and dP = dO V^T: 32 queries x this wave's 32 keys
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(qsl + q_lane + L::off(0, 16 * ds));
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[ds], sc, 0, 0, 0);
        }
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(osl + q_lane + L::off(0, 16 * ds));
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[ds], dp, 0, 0, 0);
            if (ds == 1) {
                order_memory();
                issue(it + 2, qfill, ofill, afill);
                order_memory();
            }
        }

        // P = exp2(c2 s - log2e LSE) and dS = P (dP - delta); rows past a ragged tile
        // have zero Q and dO and contribute nothing, so only visibility is masked
        const bool full = (m == CP_MASK_FULL) || (k1p <= qpos0 && qpos0 + qrows - 1 < qend(m, kend_first, wend_first));
        const int qk = qpos0 - kp + 4 * hl;                              // q - k without the register's offset
        const unsigned span = (unsigned)(qend(m, kend_lane, wend_lane) - kp);
        const float* lse_row = reinterpret_cast<const float*>(asl);
        const float* del_row = reinterpret_cast<const float*>(asl + 256);
        f32x16 pr, dsr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_row + 8 * i + 4 * hl);
#pragma unroll
            for (int j = 0; j < 4; ++j) pr[4 * i + j] = __builtin_amdgcn_exp2f(fmaf(sc[4 * i + j], c2, -l4[j] * kLog2e));
        }
        if (!full) {  // element mask on partial tiles only (a wave-uniform branch)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if ((unsigned)(qk + 8 * i + j) >= span) pr[4 * i + j] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(del_row + 8 * i + 4 * hl);
#pragma unroll
            for (int j = 0; j < 4; ++j) dsr[4 * i + j] = pr[4 * i + j] * (dp[4 * i + j] - d4[j]);
        }
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            f32x8 a, b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                a[e] = pr[8 * h2 + e];
                b[e] = dsr[8 * h2 + e];
            }
            pb[h2] = __builtin_convertvector(a, bf16x8);
            sb[h2] = __builtin_convertvector(b, bf16x8);
        }

        // dV^T += dO^T P and dK^T += Q^T dS (M = dims, N = keys, K = queries 16 s2 + 4hl + {0..3, 8..11});
        // MFMA m: pair e = m / 2 (s2 = e / DB, db = e % DB), dV for even m and dK for odd m, its A
        // operand read two MFMAs ahead
        auto t_operand = [&](int m) -> bf16x8 {
            const int e = m >> 1;
            const char* base = (m & 1) ? qsl : osl;
            const int o = t_lane + L::off(16 * (e / DB), 32 * (e % DB));
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + o));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + o + L::off(8, 0)));
            const s16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(bf16x8, a);
        };
        bf16x8 ta[3];
        ta[0] = t_operand(0);
        ta[1] = t_operand(1);
#pragma unroll
        for (int m = 0; m < 4 * DB; ++m) {
            if (m + 2 < 4 * DB) {
                ta[(m + 2) % 3] = t_operand(m + 2);
                order_memory();
            }
            const int e = m >> 1, s2 = e / DB, db = e % DB;
            if ((m & 1) == 0) {
                dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[m % 3], pb[s2], dva[db], 0, 0, 0);
                pin(dva[db]);
            } else {
                dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[m % 3], sb[s2], dka[db], 0, 0, 0);
                pin(dka[db]);
            }
        }
        if constexpr (decltype(bar)::value) ring_barrier<0>();
    };

    // Item s reads slot s mod 4 and fills slot (s+2) mod 4, last read by item
    // s-2, before the last barrier; a barrier after every odd item first waits
    // for all of the wave's loads, so the next two items have landed.
    if (n_it > 0) {
        issue(0, qt0, ot0, ax0);
        issue(1, qt1, ot1, ax1);
        ring_barrier<0>();  // items 0 and 1 have landed
        using NoBar = std::integral_constant<bool, false>;
        using Bar = std::integral_constant<bool, true>;
        for (int it = 0; it < n_it; it += 4) {
            step(NoBar{}, it, qt0, ot0, ax0, qt2, ot2, ax2);
            if (it + 1 < n_it) step(Bar{}, it + 1, qt1, ot1, ax1, qt3, ot3, ax3);
            if (it + 2 < n_it) step(NoBar{}, it + 2, qt2, ot2, ax2, qt0, ot0, ax0);
            if (it + 3 < n_it) step(Bar{}, it + 3, qt3, ot3, ax3, qt1, ot1, ax1);
        }
    }

    // ---- write this workgroup's dK (scaled) and dV rows: the outputs for part 0
    // (zeros if it has no items), the workspace slot of (part, block) for a later
    // part with items.  Lane-derived values of the epilogue are recomputed here
    // (from the lane count, not from registers kept through the loop).
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int ql_e = lane_e & 31, hl_e = lane_e >> 5, kk_e = 32 * wave + ql_e;
    if (part > 0 && n_it == 0) return;
    if (kk_e < kcount) {
        float* dk_row;
        float* dv_row;
        if (part == 0) {
            dk_row = p.dk + (int64_t)(key_row0 + kk_e) * kv_stride + (int64_t)g * D;
            dv_row = p.dv + (int64_t)(key_row0 + kk_e) * kv_stride + (int64_t)g * D;
        } else {
            float* slot = p.ws + ((int64_t)(part - 1) * p.n_work_kv + b) * (2 * BK * D);
            dk_row = slot + (int64_t)kk_e * D;
            dv_row = slot + (int64_t)(BK + kk_e) * D;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * hl_e;
                const f32x4 kv4 = {dka[db][4 * i] * p.scale, dka[db][4 * i + 1] * p.scale,
                                   dka[db][4 * i + 2] * p.scale, dka[db][4 * i + 3] * p.scale};
                const f32x4 vv4 = {dva[db][4 * i], dva[db][4 * i + 1], dva[db][4 * i + 2], dva[db][4 * i + 3]};
                *reinterpret_cast<f32x4*>(dk_row + d0) = kv4;
                *reinterpret_cast<f32x4*>(dv_row + d0) = vv4;
            }
    }
}

// Second pass of a split dK/dV step: for every key block whose items were
// spread over more than one workgroup, add the partial sums of parts 1, 2, ...
// (in that order) from the workspace to the outputs, which hold part 0's.
// One workgroup per key block; rows past the block's keys are not touched.
template <int D>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const BwdParams p) {
    const int b = blockIdx.x;
    if (b >= p.n_work_kv) return;
    const KvBlock kb = kv_block(p, b);
    const int run = split_run(kb.n_all, p.kv_split);
    const int n_parts = (run > 0) ? (kb.n_all + run - 1) / run : 0;
    if (n_parts <= 1) return;
    const int64_t kv_stride = (int64_t)p.hkv * D;
    constexpr int V4 = D / 4;
    for (int i = threadIdx.x; i < BK * V4; i += blockDim.x) {
        const int key = i / V4, d = 4 * (i % V4);
        if (key >= kb.kcount) break;
        const int64_t at = (int64_t)(kb.key_row0 + key) * kv_stride + (int64_t)kb.g * D + d;
        f32x4 sk = *reinterpret_cast<const f32x4*>(p.dk + at);
        f32x4 sv = *reinterpret_cast<const f32x4*>(p.dv + at);
        for (int part = 1; part < n_parts; ++part) {
            const float* slot = p.ws + ((int64_t)(part - 1) * p.n_work_kv + b) * (2 * BK * D);
            sk += *reinterpret_cast<const f32x4*>(slot + (int64_t)key * D + d);
            sv += *reinterpret_cast<const f32x4*>(slot + (int64_t)(BK + key) * D + d);
        }
        *reinterpret_cast<f32x4*>(p.dk + at) = sk;
        *reinterpret_cast<f32x4*>(p.dv + at) = sv;
    }
}

// ============================================================================ dQ
constexpr int kQWaves = kFwdWaves;  // 8 waves, the forward kernel's shape
constexpr int kQThreads = 64 * kQWaves;
constexpr int kBN = 64;

template <int D, int HPW>
__global__ __launch_bounds__(kQThreads, 2) void bwd_dq_kernel(const BwdParams p) {
    using L = TileLayout<D, kBN>;
    constexpr int WPH = kQWaves / HPW;
    constexpr int BMQ = 32 * WPH;
    constexpr int DS = D / 16;
    constexpr int DB = D / 32;
    __shared__ __attribute__((aligned(16))) char kb0[L::BYTES];
    __shared__ __attribute__((aligned(16))) char kb1[L::BYTES];
    __shared__ __attribute__((aligned(16))) char kb2[L::BYTES];
    __shared__ __attribute__((aligned(16))) char kb3[L::BYTES];
    __shared__ __attribute__((aligned(16))) char vb0[L::BYTES];
    __shared__ __attribute__((aligned(16))) char vb1[L::BYTES];
    __shared__ __attribute__((aligned(16))) char vb2[L::BYTES];
    __shared__ __attribute__((aligned(16))) char vb3[L::BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int hl = lane >> 5;
    const int ql = lane & 31;

    // as in the forward: head block w mod n_hb, query tiles latest first (or
    // earliest first where those see the most keys)
    const int w = blockIdx.x;
    if (w >= p.n_work_q) return;
    const int hb = w % p.n_hb;
    const int qt = p.q_first ? w / p.n_hb : p.n_qtiles - 1 - w / p.n_hb;
    const int qs = (qt < p.qtiles0) ? 0 : 1;
    const int qt_in = qs ? qt - p.qtiles0 : qt;
    const int tile_row0 = p.qs_row0[qs] + qt_in * BMQ;
    const int tile_pos0 = p.qs_pos0[qs] + qt_in * BMQ;
    const int tile_rows = min(BMQ, p.qs_len[qs] - qt_in * BMQ);
    const int q0 = tile_pos0, q1 = tile_pos0 + tile_rows - 1;
    const int head = hb * HPW + wave / WPH;
    const int kvh = (hb * HPW) / p.group;
    const int row_in_tile = (wave % WPH) * 32 + ql;
    const bool row_valid = row_in_tile < tile_rows;
    const int my_row = tile_row0 + row_in_tile;
    const int my_pos = tile_pos0 + row_in_tile;

    const bool any_doc = (p.mask[qs][0] == CP_MASK_DOC) || (p.nkv_seg > 1 && p.mask[qs][1] == CP_MASK_DOC);
    int lo0 = 0, lo1 = 0, my_lo = 0;
    if (any_doc) {
        const int d0 = doc_index(p.cu, p.n_docs, q0);
        lo0 = p.cu[d0];
        lo1 = p.cu[doc_index(p.cu, p.n_docs, q1)];
        int j = d0;
        if (row_valid) {
            while (j + 1 < p.n_docs && p.cu[j + 1] <= my_pos) ++j;
        }
        my_lo = p.cu[j];
    }
    const int mk0 = (p.nkv_seg > 0) ? p.mask[qs][0] : CP_MASK_SKIP;
    const int mk1 = (p.nkv_seg > 1) ? p.mask[qs][1] : CP_MASK_SKIP;
    const int len0 = p.ks_len[0], len1 = p.ks_len[1];
    const int pos0 = p.ks_pos0[0], pos1 = p.ks_pos0[1];
    // first visible key of a row (document start, window start), as in the forward kernel
    const int win = p.window;
    const int wlo0 = (win > 0) ? q0 - win + 1 : 0, wlo1 = (win > 0) ? q1 - win + 1 : 0;
    const int my_wlo = (win > 0) ? my_pos - win + 1 : 0;
    auto lower = [](int m, int doc_lo, int win_lo) {
        return (m == CP_MASK_DOC) ? max(doc_lo, win_lo) : (m == CP_MASK_DIAG_CAUSAL ? win_lo : 0);
    };
    const int my_lo_doc = max(my_lo, my_wlo);
    const SegRange r0 = key_tile_range<kBN>(mk0, q0, q1, lower(mk0, lo0, wlo0), pos0, len0);
    const SegRange r1 = (p.nkv_seg > 1) ? key_tile_range<kBN>(mk1, q0, q1, lower(mk1, lo0, wlo0), pos1, len1)
                                        : SegRange{0, 0};
    const int tlo0 = r0.t_lo, tlo1 = r1.t_lo;
    const int n0 = r0.t_hi - r0.t_lo;
    const int n_it = n0 + (r1.t_hi - r1.t_lo);

    // ---- Q and dO fragments (lane holds query ql, dims 16 ds + 8 hl + 0..7), LSE and delta
    bf16x8 qf[DS], of[DS];
    {
        const int64_t off = ((int64_t)my_row * p.hq + head) * D + 8 * hl;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if (row_valid && n_it > 0) {
                a = *reinterpret_cast<const u32x4*>(p.q + off + 16 * ds);
                b = *reinterpret_cast<const u32x4*>(p.d_o + off + 16 * ds);
            }
            qf[ds] = __builtin_bit_cast(bf16x8, a);
            of[ds] = __builtin_bit_cast(bf16x8, b);
        }
    }
    float nl = 0.f, dl = 0.f;
    if (row_valid && n_it > 0) {
        const float l = p.lse[(int64_t)head * p.q_rows + my_row];
        nl = (l == -INFINITY) ? 0.f : -l * kLog2e;  // a row with no visible key is fully masked
        dl = p.delta[(int64_t)head * p.q_rows + my_row];
    }

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    const float c2 = p.scale_log2;
    const int row_bytes = p.hkv * D * 2;
    const int64_t head_off = (int64_t)kvh * D;
    const uint16_t* const kseg0 = p.k + (int64_t)p.ks_row0[0] * p.hkv * D + head_off;
    const uint16_t* const kseg1 = p.k + (int64_t)p.ks_row0[1] * p.hkv * D + head_off;
    const uint16_t* const vseg0 = p.v + (int64_t)p.ks_row0[0] * p.hkv * D + head_off;
    const uint16_t* const vseg1 = p.v + (int64_t)p.ks_row0[1] * p.hkv * D + head_off;
    const int64_t tile_elems = (int64_t)kBN * p.hkv * D;

    struct TileRef {
        int t, len, pos, mask, seg;
    };
    // by-value capture: a select between captured references becomes a select of
    // addresses, which the compiler then keeps in (slow) private memory
    auto tile_of = [=](int it) -> TileRef {
        const bool second = it >= n0;
        const int t = second ? tlo1 + (it - n0) : tlo0 + it;
        return TileRef{t, second ? len1 : len0, second ? pos1 : pos0, second ? mk1 : mk0, second ? 1 : 0};
    };
    auto issue = [&](int it, char* kdst, char* vdst) {
        const TileRef tr = tile_of(it);
        const bool live = it < n_it;
        const int rows = live ? min(kBN, tr.len - tr.t * kBN) : 0;
        const int64_t toff = live ? tr.t * tile_elems : 0;
        load_tile_lds<D, kBN, kQWaves>(kdst, tile_rsrc((tr.seg ? kseg1 : kseg0) + toff, rows, row_bytes), row_bytes,
                                       wave, lane);
        load_tile_lds<D, kBN, kQWaves>(vdst, tile_rsrc((tr.seg ? vseg1 : vseg0) + toff, rows, row_bytes), row_bytes,
                                       wave, lane);
    };
    const int k_lane = L::off(ql, 8 * hl);
    const int grp = lane >> 4, jl = lane & 15;
    const int t_lane = L::off(4 * (grp >> 1) + (jl >> 2), 16 * (grp & 1) + 4 * (jl & 3));

    auto step = [&](auto bar, int it, const char* ksl, const char* vsl, char* kfill, char* vfill) {
        const TileRef tr = tile_of(it);
        // S^T = K Q^T and dP^T = V dO^T: 64 keys x this wave's 32 queries
        f32x16 sc[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sc[kb] = f32x16{};
            dp[kb] = f32x16{};
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(ksl + k_lane + L::off(32 * kb, 16 * ds));
                sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], sc[kb], 0, 0, 0);
                if (kb == 0 && ds == 3) {
                    // this step's loads, a few MFMAs in: their address arithmetic is
                    // off the path from the barrier to the first MFMA
                    order_memory();
                    issue(it + 2, kfill, vfill);
                    order_memory();
                }
            }
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(vsl + k_lane + L::off(32 * kb, 16 * ds));
                dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, of[ds], dp[kb], 0, 0, 0);
            }
        }
        // element mask on partial or ragged tiles, as in the forward kernel
        const int kcount = min(kBN, tr.len - tr.t * kBN);
        const int kp0 = tr.pos + tr.t * kBN;
        const int m = tr.mask;
        const bool full = key_tile_full<kBN>(m, q0, lower(m, lo1, wlo1), tr.pos, tr.len, tr.t);
        bool vis_all = true;
        int lo_l = 0;
        unsigned span = 0;
        bool none = false;
        if (!full || kcount < kBN) {
            vis_all = false;
            int hi_lim = kcount - 1;
            int lo_lim = 0;
            if (m != CP_MASK_FULL) {
                hi_lim = min(hi_lim, my_pos - kp0);
                lo_lim = max(0, ((m == CP_MASK_DOC) ? my_lo_doc : my_wlo) - kp0);
            }
            lo_l = lo_lim - 4 * hl;
            span = (unsigned)(hi_lim - lo_lim);
            none = hi_lim < lo_lim;
        }
        // P = exp2(c2 s - log2e LSE), dS = P (dP - delta), rounded to bf16 for dQ
        bf16x8 sb[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[kb][r] = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], c2, nl));
        if (!vis_all) {  // element mask on partial or ragged tiles only (a wave-uniform branch)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (none || (unsigned)(row_of_reg(kb, r, 0) - lo_l) > span) sc[kb][r] = 0.f;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x8 v8;
#pragma unroll
                for (int e = 0; e < 8; ++e) v8[e] = sc[kb][8 * half + e] * (dp[kb][8 * half + e] - dl);
                sb[2 * kb + half] = __builtin_convertvector(v8, bf16x8);
            }
        }
        // dQ^T += K^T dS^T: step s4 covers keys 16 s4 + 4hl + {0..3, 8..11}
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const char* a0 = ksl + t_lane + L::off(16 * s4, 32 * db);
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0 + L::off(8, 0)));
                const s16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), sb[s4], acc[db],
                                                                   0, 0, 0);
            }
        }
        if constexpr (decltype(bar)::value) ring_barrier<0>();
    };

    // Step s reads tile s (slot s mod 4) and fills slot (s+2) mod 4, last read at
    // step s-2, before the last barrier; a barrier after every odd step first
    // waits for all of the wave's loads, so the two tiles the next two steps
    // read have landed.
    if (n_it > 0) {
        issue(0, kb0, vb0);
        issue(1, kb1, vb1);
        ring_barrier<0>();  // tiles 0 and 1 have landed
        using NoBar = std::integral_constant<bool, false>;
        using Bar = std::integral_constant<bool, true>;
        for (int it = 0; it < n_it; it += 4) {
            step(NoBar{}, it, kb0, vb0, kb2, vb2);
            if (it + 1 < n_it) step(Bar{}, it + 1, kb1, vb1, kb3, vb3);
            if (it + 2 < n_it) step(NoBar{}, it + 2, kb2, vb2, kb0, vb0);
            if (it + 3 < n_it) step(Bar{}, it + 3, kb3, vb3, kb1, vb1);
        }
    }

    // ---- dQ[row, head, :] += scale * (dS K)[row, :]; each wave owns its rows
    if (row_valid && n_it > 0) {
        float* dqrow = p.dq + ((int64_t)my_row * p.hq + head) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4* ptr = reinterpret_cast<f32x4*>(dqrow + 32 * db + 8 * i + 4 * hl);
                f32x4 cur = *ptr;
                cur.x += p.scale * acc[db][4 * i];
                cur.y += p.scale * acc[db][4 * i + 1];
                cur.z += p.scale * acc[db][4 * i + 2];
                cur.w += p.scale * acc[db][4 * i + 3];
                *ptr = cur;
            }
    }
}

// CUs of the current device (2 dK/dV workgroups run on each); 256 if unknown.
int64_t device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        return 256;
    return n;
}

template <int D>
hipError_t launch_dkdv(const BwdParams& prm, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3(grid), dim3(kKvThreads), 0, stream, prm);
    return hipGetLastError();
}

template <int D>
hipError_t launch_reduce(const BwdParams& prm, hipStream_t stream) {
    hipLaunchKernelGGL((dkdv_reduce_kernel<D>), dim3(prm.n_work_kv), dim3(256), 0, stream, prm);
    return hipGetLastError();
}

template <int D, int HPW>
hipError_t launch_dq(const BwdParams& prm, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, HPW>), dim3(grid), dim3(kQThreads), 0, stream, prm);
    return hipGetLastError();
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

namespace cpattn {

cp_status bwd_step(const cp_attn_problem* p, const void* q, const void* k, const void* v, const void* d_o,
                   const float* lse, const float* delta, float* dq_acc, float* dk_out, float* dv_out, void* workspace,
                   int64_t workspace_bytes, hipStream_t stream) {
    cp_status st = validate_problem(p, true);
    if (st != CP_OK) return st;
    if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace))
        return fail(CP_ERR_INVALID_ARG, "workspace_bytes > 0 needs a workspace pointer (and must not be negative)");
    const TileGeom gq = fwd_geom(p->hq, p->hkv);
    BwdParams prm = {};
    prm.q = static_cast<const uint16_t*>(q);
    prm.k = static_cast<const uint16_t*>(k);
    prm.v = static_cast<const uint16_t*>(v);
    prm.d_o = static_cast<const uint16_t*>(d_o);
    prm.lse = lse;
    prm.delta = delta;
    prm.dq = dq_acc;
    prm.dk = dk_out;
    prm.dv = dv_out;
    prm.ws = static_cast<float*>(workspace);
    prm.cu = p->cu_seqlens;
    prm.n_docs = p->n_docs;
    prm.window = p->window;
    prm.hq = p->hq;
    prm.hkv = p->hkv;
    prm.group = p->hq / p->hkv;
    prm.q_rows = int32_t(p->q_rows);
    prm.scale = p->scale;
    prm.scale_log2 = p->scale * kLog2e;
    prm.nq_seg = p->n_q_seg;
    prm.nkv_seg = p->n_kv_seg;
    int64_t nk = 0;
    for (int i = 0; i < 2; ++i) {
        const bool on = i < p->n_q_seg;
        prm.qs_row0[i] = on ? int32_t(p->q_seg[i].row0) : 0;
        prm.qs_pos0[i] = on ? int32_t(p->q_seg[i].pos0) : 0;
        prm.qs_len[i] = on ? int32_t(p->q_seg[i].len) : 0;
        const bool kon = i < p->n_kv_seg;
        prm.ks_row0[i] = kon ? int32_t(p->kv_seg[i].row0) : 0;
        prm.ks_pos0[i] = kon ? int32_t(p->kv_seg[i].pos0) : 0;
        prm.ks_len[i] = kon ? int32_t(p->kv_seg[i].len) : 0;
        nk += ceil_div(prm.ks_len[i], BK);
    }
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j)
            prm.mask[i][j] = (i < p->n_q_seg && j < p->n_kv_seg) ? p->mask[i][j] : CP_MASK_SKIP;
    prm.ktiles0 = int32_t(ceil_div(prm.ks_len[0], BK));
    prm.n_ktiles = int32_t(nk);
    prm.k_last = dkdv_latest_first(p) ? 1 : 0;
    const int64_t work_kv = nk * p->hkv;
    // dQ: query segments that see no KV segment get nothing and stay out of the
    // launch (the dK/dV kernel still walks every segment)
    const cp_attn_problem lq = live_queries(p);
    BwdParams prm_q = prm;
    int64_t nq = 0;
    for (int i = 0; i < 2; ++i) {
        const bool on = i < lq.n_q_seg;
        prm_q.qs_row0[i] = on ? int32_t(lq.q_seg[i].row0) : 0;
        prm_q.qs_pos0[i] = on ? int32_t(lq.q_seg[i].pos0) : 0;
        prm_q.qs_len[i] = on ? int32_t(lq.q_seg[i].len) : 0;
        for (int j = 0; j < 2; ++j) prm_q.mask[i][j] = (on && j < p->n_kv_seg) ? lq.mask[i][j] : CP_MASK_SKIP;
        nq += ceil_div(prm_q.qs_len[i], gq.bm);
    }
    prm_q.nq_seg = lq.n_q_seg;
    prm_q.qtiles0 = int32_t(ceil_div(prm_q.qs_len[0], gq.bm));
    prm_q.n_qtiles = int32_t(nq);
    {
        // the heaviest query tiles first (their work listed in the default order)
        std::vector<int64_t> work = query_tile_work(&lq, gq.bm, kBN);
        std::reverse(work.begin(), work.end());
        prm_q.q_first = heavier_last(work) ? 1 : 0;
    }
    const int64_t work_q = nq * (p->hq / gq.hpw);
    if (work_kv == 0 && work_q == 0) return CP_OK;
    if (!q || !k || !v || !d_o || !lse || !delta || !dq_acc || !dk_out || !dv_out)
        return fail(CP_ERR_INVALID_ARG, "NULL tensor pointer");
    if (!all_aligned16({q, k, v, d_o, lse, delta, dq_acc, dk_out, dv_out, workspace}))
        return fail(CP_ERR_INVALID_ARG, "tensor or workspace pointer not 16-byte aligned");
    if (work_kv > (int64_t(1) << 30) || work_q > (int64_t(1) << 30))
        return fail(CP_ERR_UNSUPPORTED, "problem too large for one launch");
    prm.n_work_kv = int32_t(work_kv);
    prm.n_hb = p->hq / gq.hpw;
    // the dK/dV split: as asked (with room for it in the workspace), or chosen
    // here and reduced to 1 when the workspace cannot hold its parts
    int32_t split = p->kv_split;
    if (split > 0) {
        if (dkdv_workspace_bytes(p, split) > workspace_bytes)
            return fail(CP_ERR_INVALID_ARG, "kv_split " + std::to_string(split) + " needs " +
                                                std::to_string(dkdv_workspace_bytes(p, split)) +
                                                " workspace bytes (cp_bwd_workspace_size), got " +
                                                std::to_string(workspace_bytes));
    } else {
        split = dkdv_split(p, nullptr, device_cus());
        if (dkdv_workspace_bytes(p, split) > workspace_bytes) split = 1;
    }
    prm.kv_split = split;
    prm_q.n_work_kv = prm.n_work_kv;
    prm_q.n_hb = prm.n_hb;
    prm_q.kv_split = prm.kv_split;
    prm_q.n_work_q = int32_t(work_q);
    if (work_kv * prm.kv_split > (int64_t(1) << 30)) return fail(CP_ERR_UNSUPPORTED, "problem too large for one launch");
    hipError_t e = hipSuccess;
    if (work_kv > 0) {
        const int grid = int(work_kv * prm.kv_split);
        e = (p->head_dim == 128) ? launch_dkdv<128>(prm, grid, stream) : launch_dkdv<64>(prm, grid, stream);
        if (e != hipSuccess) return fail(CP_ERR_HIP, std::string("bwd dK/dV launch: ") + hipGetErrorString(e));
        if (prm.kv_split > 1) {
            e = (p->head_dim == 128) ? launch_reduce<128>(prm, stream) : launch_reduce<64>(prm, stream);
            if (e != hipSuccess) return fail(CP_ERR_HIP, std::string("dK/dV reduction launch: ") + hipGetErrorString(e));
        }
    }
    if (work_q > 0) {
        const int grid = int(work_q);
        if (p->head_dim == 128)
            e = (gq.hpw == 4) ? launch_dq<128, 4>(prm_q, grid, stream)
                              : (gq.hpw == 2 ? launch_dq<128, 2>(prm_q, grid, stream) : launch_dq<128, 1>(prm_q, grid, stream));
        else
            e = (gq.hpw == 4) ? launch_dq<64, 4>(prm_q, grid, stream)
                              : (gq.hpw == 2 ? launch_dq<64, 2>(prm_q, grid, stream) : launch_dq<64, 1>(prm_q, grid, stream));
        if (e != hipSuccess) return fail(CP_ERR_HIP, std::string("bwd dQ launch: ") + hipGetErrorString(e));
    }
    return CP_OK;
}

// ---------------------------------------------------------------- no-alloc variant
// The dK/dV split's workspace for callers that cannot allocate: a fixed array in
// the code object, one per device the library runs on, held until the process
// ends.  Host code never names it after set-up: its address on each device comes
// from hipGetSymbolAddress (the name itself is only a host-side stand-in).
constexpr int64_t kScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Address of the current device's scratch array, looked up on its first use.
cp_status scratch_of_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(CP_ERR_UNSUPPORTED, "device index beyond 63");
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !ptr)
                return fail(CP_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return CP_OK;
}

}  // namespace cpattn

extern "C" cp_status cp_attn_bwd_step_noalloc(const cp_attn_problem* p, const void* q, const void* k, const void* v,
                                              const void* d_o, const float* lse, const float* delta, float* dq_acc,
                                              float* dk_out, float* dv_out, hipStream_t stream) {
    cp_status st = validate_problem(p, true);
    if (st != CP_OK) return st;
    if (p->kv_split > 1 && dkdv_workspace_bytes(p, p->kv_split) > kScratchBytes)
        return fail(CP_ERR_INVALID_ARG, "kv_split " + std::to_string(p->kv_split) + " needs " +
                                            std::to_string(dkdv_workspace_bytes(p, p->kv_split)) +
                                            " workspace bytes; the no-alloc entry point has " +
                                            std::to_string(kScratchBytes));
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != CP_OK) return st;
    return bwd_step(p, q, k, v, d_o, lse, delta, dq_acc, dk_out, dv_out, ws, kScratchBytes, stream);
}

extern "C" cp_status cp_attn_bwd_step(const cp_attn_problem* p, const void* q, const void* k, const void* v,
                                      const void* d_o, const float* lse, const float* delta, float* dq_acc,
                                      float* dk_out, float* dv_out, void* workspace, int64_t workspace_bytes,
                                      hipStream_t stream) {
    return bwd_step(p, q, k, v, d_o, lse, delta, dq_acc, dk_out, dv_out, workspace, workspace_bytes, stream);
}
