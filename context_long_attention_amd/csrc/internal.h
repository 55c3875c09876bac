// Internal declarations shared by the host logic (host.cpp, plain C++) and the
// HIP launchers (*.hip).  Not part of the ABI.
#pragma once

#include <cstdint>
#include <initializer_list>
#include <string>
#include <vector>

#include "cpattn.h"

namespace cpattn {

// Forward tile geometry.  A workgroup is kFwdWaves wave64s; each wave owns 32
// query rows of one head.  hpw heads of one GQA group share a workgroup (and
// every K/V tile it stages), so a workgroup covers bm = 32 * kFwdWaves / hpw
// query rows.
constexpr int kFwdWaves = 8;
struct TileGeom {
    int bm;   // query rows per workgroup tile
    int bn;   // keys per K/V tile
    int hpw;  // query heads per workgroup (divides Hq / Hkv)
};
TileGeom fwd_geom(int hq, int hkv);

// Backward geometry: a workgroup owns bnk keys of one KV head (32 per wave)
// and walks query tiles of bmq rows.
constexpr int kBwdKeysPerWG = 128;
constexpr int kBwdQRows = 32;
// A key block's query items may be spread over up to kMaxKvSplit workgroups;
// the first writes dK/dV, the others a workspace slot each, summed into dK/dV
// in part order by a second pass.  kWgOverhead: the fixed cost of a dK/dV
// workgroup in item times; kReduceSlotCost: the chip-wide cost of the second
// pass per slot it reads (2 x 128 rows x head_dim floats), in item times (used
// to choose the split).
constexpr int kMaxKvSplit = 8;
constexpr double kWgOverhead = 3.0;
constexpr double kReduceSlotCost = 0.03;

void set_error(const std::string& msg);
cp_status fail(cp_status s, const std::string& msg);

// Validate a problem.  device_docs: cu_seqlens will be read by a kernel (only
// its presence is checked) rather than on the host (where it is also checked
// for monotonicity and range).
cp_status validate_problem(const cp_attn_problem* p, bool device_docs);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The kernels move every tensor in 16-byte vectors: each tensor pointer must be
// 16-byte aligned (a torch allocation, or a view of it starting at a row, is).
inline bool all_aligned16(std::initializer_list<const void*> ptrs) {
    for (const void* q : ptrs)
        if (reinterpret_cast<uintptr_t>(q) & 15u) return false;
    return true;
}

// The step kernels address a KV tile by a 32-bit byte offset into a buffer
// descriptor spanning one segment of one KV head, so every KV segment must
// stay below 1 GiB (len * Hkv * D * 2 bytes), leaving headroom for the offsets
// of tiles past the end.
inline bool kv_spans_fit(const cp_attn_problem* p) {
    for (int j = 0; j < p->n_kv_seg; ++j)
        if (p->kv_seg[j].len * int64_t(p->hkv) * p->head_dim * 2 >= (int64_t(1) << 30)) return false;
    return true;
}

// Tile-range rule shared by the host block map and (as a mirror in device
// code) the forward kernel.  For a query tile [q0, q1] (global positions, q1
// the last row) and a KV segment starting at kpos0 with klen keys in tiles of
// bn: visited tiles are [t_lo, t_hi).  lo0 / lo1 are the first visible key
// position of rows q0 / q1 (row_lower_bound).
struct TileRange {
    int64_t t_lo, t_hi;
};
TileRange tile_range(int mask, int64_t q0, int64_t q1, int64_t lo0, int64_t kpos0, int64_t klen, int bn);
// Class of tile t inside the visited range.
int tile_class(int mask, int64_t q0, int64_t q1, int64_t lo1, int64_t kpos0, int64_t klen, int bn, int64_t t);

// Document start of a global position (host cu_seqlens).
int64_t doc_start_host(const int32_t* cu, int32_t n_docs, int64_t pos);

// First visible key position of query position q under a pair's mask: the
// document start (DOC) and q - window + 1 (sliding window, DIAG_CAUSAL and DOC),
// whichever is later; unbounded below otherwise.  Non-decreasing in q and <= q.
int64_t row_lower_bound(const cp_attn_problem* p, int mask, int64_t q);

// Work-item order.  The forward and dQ kernels take query tiles latest first
// and the dK/dV kernel takes key blocks earliest first: under a causal mask
// those have the most pairs, so the longest items start first.  Where the work
// runs the other way (a sliding window's triangle at a chunk boundary, where
// the earliest queries and the latest keys see the most), a launch takes its
// items in the opposite order.  Decided on the host from every item's work;
// problems with a DOC pair keep the default order (their ranges need the
// documents, which a step call only has on the device).
//
// True when `work`, listed in a launch's default order, is heavier in its
// second half (its centre of mass lies more than 1% of the span past the
// middle), i.e. when the launch should take its items from the other end.
bool heavier_last(const std::vector<int64_t>& work);
// Visible key tiles (bn keys each) of every query tile (bm rows each) of the
// forward and dQ kernels, in tile index order (first query segment first).
// Empty when a pair is DOC.
std::vector<int64_t> query_tile_work(const cp_attn_problem* p, int bm, int bn);
// Query items (kBwdQRows rows of one query head) of every 128-key block of
// one KV head, in the dK/dV kernel's key-tile index order.  host_cu: host
// cu_seqlens for DOC pairs; empty with a DOC pair and no host_cu.
std::vector<int64_t> key_block_items(const cp_attn_problem* p, const int32_t* host_cu);
// The dK/dV launch order: key blocks latest first instead of earliest first.
bool dkdv_latest_first(const cp_attn_problem* p);

// Number of workgroups (1..kMaxKvSplit) over which the dK/dV kernel spreads
// each key block's query items: the one with the shortest simulated launch,
// from the items of every block (the ranges that kernel walks) and the CU
// count.  host_cu: host cu_seqlens for DOC masks; NULL with a DOC mask gives 1.
int32_t dkdv_split(const cp_attn_problem* p, const int32_t* host_cu, int64_t n_cu);

// Workspace bytes a backward step with dK/dV split `split` needs: one slot of
// 2 * kBwdKeysPerWG * head_dim floats (partial dK and dV) per key block of
// every KV head, for each part after the first.  0 for split <= 1.
inline int64_t dkdv_workspace_bytes(const cp_attn_problem* p, int32_t split) {
    if (split <= 1) return 0;
    int64_t blocks = 0;
    for (int j = 0; j < p->n_kv_seg; ++j) blocks += ceil_div(p->kv_seg[j].len, kBwdKeysPerWG);
    return int64_t(split - 1) * blocks * p->hkv * 2 * kBwdKeysPerWG * p->head_dim * int64_t(sizeof(float));
}

// The problem restricted to its query segments that pair with some KV rows
// (a mask other than SKIP against a non-empty KV segment), in their order;
// n_q_seg may become 0.  Rows of the other segments receive nothing in a
// merging forward step and nothing in dQ, so those launches leave them out.
cp_attn_problem live_queries(const cp_attn_problem* p);

}  // namespace cpattn
