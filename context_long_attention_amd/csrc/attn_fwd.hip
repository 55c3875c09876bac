// Forward of one Pass-KV ring step on gfx950: blockwise causal flash attention
// of the stationary local queries against the KV block held at this step
// ("Announcing Long-Context Training on TPUs with MaxText Context
// Parallelism", section "Built on a fast attention kernel"; the ring itself is
// "Context Parallelism for Scalable Million-Token Inference", section "Ring
// Attention Algorithms").
//
// Design (gfx950, wave64, 32x32x16 bf16 MFMA with fp32 accumulation):
//  * One 8-wave workgroup per CU (2 waves per SIMD).  Each wave owns 32 query
//    rows of one query head; HPW heads of one GQA group share the workgroup,
//    so every K/V tile staged in LDS serves 256 query-row-heads.
//  * Scores are computed transposed, S^T = K Q^T (keys on the MFMA M axis,
//    queries on N): each lane holds one query and 32 of its keys, so the row
//    max needs one exchange between the half-waves and the row sum none until
//    the epilogue.  The P registers, rounded to bf16, are directly the B
//    operand of O^T += V^T P^T; V stays row-major in LDS and its transposed
//    operand comes from the transposing LDS read (ds_read_tr16_b64).
//  * K/V tiles move HBM -> LDS with direct buffer loads (rows past a ragged
//    tile read as zero) into a ring of four K and four V buffers, two tiles
//    ahead of use, with one workgroup barrier every second tile.
//  * Rotated pipeline: one step alternates the MFMAs of the P V product of
//    tile i-1 and of the scores of tile i+1, with the exponentials, row sum and
//    bf16 convert of tile i spread over them.
//  * No running row maximum on the fast path: exponentials are taken against a
//    reference set by a row's first visible tile.  A row whose tile sum
//    exceeds 2^20 or is not finite (or that has no reference yet) takes a slow
//    path that raises the reference to the tile's true maximum, rescales and
//    recomputes the tile.  P then stays below 2^20, which fp32 accumulation
//    and bf16 rounding hold without loss of relative precision.
//  * Tiles with no visible pair are never visited (block-sparse skip); the
//    element mask runs only on partially visible or ragged tiles.
//  * Work items are dealt to the XCDs round-robin: each XCD keeps the same head
//    blocks (K/V shared in its L2; with Hkv a multiple of 8 all head blocks of
//    a KV head share one XCD), the query tiles with the most keys first (latest
//    positions, or earliest where a window's triangle makes those the longest),
//    and query tiles of a head block shared by several XCDs interleave across
//    them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "cpattn_diag.h"
#include "internal.h"
#include "tiles.h"

namespace cpattn {

namespace {

using namespace dev;

constexpr int kBN = 64;                    // keys per tile
constexpr int kWaves = kFwdWaves;          // 8 waves: 2 per SIMD, one workgroup per CU
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;                 // K/V tiles in flight (LDS ring)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct FwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    float* o;
    float* lse;
    const int32_t* cu;
    uint8_t* tile_map;
    int32_t n_docs;
    int32_t window;  // sliding window (0: none)
    int32_t hq, hkv, group;
    int32_t q_rows;
    float scale, scale_log2;
    int32_t nkv_seg;
    int32_t qs_row0[2], qs_pos0[2], qs_len[2];
    int32_t ks_row0[2], ks_pos0[2], ks_len[2];
    int32_t mask[2][2];
    int32_t qtiles0, n_qtiles;
    int32_t ktiles0, n_ktiles;
    int32_t n_work, n_hb;
    int32_t q_first;          // query tiles earliest first instead of latest first
    unsigned long long* clk;  // diagnostics: per-workgroup start/end counters, or null
    int32_t clk_wgs;
};

// MERGE: instead of writing this step's (O, LSE), merge it into the running
// accumulator held in p.o / p.lse (rows with no visible key are left as they are).
template <int D, int HPW, bool MERGE>
__global__ __launch_bounds__(kThreads, 2) void fwd_step_kernel(const FwdParams p) {
    using L = TileLayout<D, kBN>;
    constexpr int WPH = kWaves / HPW; // waves per head
    constexpr int BMQ = 32 * WPH;     // query rows per workgroup tile
    constexpr int DS = D / 16;        // MFMA k-steps over the head dim
    constexpr int DB = D / 32;        // 32-row blocks of O^T
    // A ring of kStages K tiles and kStages V tiles, each its own LDS object,
    // so the compiler can tell that loads in flight into one buffer do not
    // alias the operand reads of another.
    __shared__ __attribute__((aligned(16))) char kb0[L::BYTES];
    __shared__ __attribute__((aligned(16))) char kb1[L::BYTES];
    __shared__ __attribute__((aligned(16))) char kb2[L::BYTES];
    __shared__ __attribute__((aligned(16))) char kb3[L::BYTES];
    __shared__ __attribute__((aligned(16))) char vb0[L::BYTES];
    __shared__ __attribute__((aligned(16))) char vb1[L::BYTES];
    __shared__ __attribute__((aligned(16))) char vb2[L::BYTES];
    __shared__ __attribute__((aligned(16))) char vb3[L::BYTES];
    static_assert(kStages == 4, "the unrolled ring below assumes four stages");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int hl = lane >> 5;
    const int ql = lane & 31;

    // ---- work decode.  Workgroups are dealt to the 8 XCDs round-robin by id, so
    // item w goes to XCD w mod 8: head block u = w mod n_hb (every XCD keeps the
    // same head blocks, whose K/V then stay in its L2) and query tiles latest
    // first (the most keys under a causal mask; earliest first when the host
    // found those to see more), interleaved across the XCDs sharing a head block.
    const int w = blockIdx.x;
    if (w >= p.n_work) return;
    const bool probe = p.clk != nullptr && w < p.clk_wgs;
    unsigned long long t0_cycles = 0, t0_ticks = 0;
    if (probe) {
        t0_cycles = __builtin_readcyclecounter();
        t0_ticks = __builtin_readsteadycounter();
    }
    // With Hkv a multiple of 8 the head blocks of a KV head all go to one XCD
    // (u mod 8 picks the KV head), so each XCD streams the K/V of Hkv / 8 KV
    // heads rather than of several per round; the map is the identity when a
    // KV head has one head block.
    const int u = w % p.n_hb;
    int hb = u;
    if ((p.hkv & 7) == 0) {
        const int nb = p.n_hb / p.hkv;  // head blocks per KV head
        hb = ((u & 7) + 8 * ((u >> 3) / nb)) * nb + (u >> 3) % nb;
    }
    const int qt = p.q_first ? w / p.n_hb : p.n_qtiles - 1 - w / p.n_hb;
    const int qs = (qt < p.qtiles0) ? 0 : 1;
    const int qt_in = qs ? qt - p.qtiles0 : qt;
    // Segment parameters as opaque scalars; nothing below indexes the parameter
    // arrays with a runtime value (see sreg).
    const int qrow0_a = sreg(p.qs_row0[0]), qrow0_b = sreg(p.qs_row0[1]);
    const int qpos0_a = sreg(p.qs_pos0[0]), qpos0_b = sreg(p.qs_pos0[1]);
    const int qlen_a = sreg(p.qs_len[0]), qlen_b = sreg(p.qs_len[1]);
    const int m00 = sreg(p.mask[0][0]), m01 = sreg(p.mask[0][1]);
    const int m10 = sreg(p.mask[1][0]), m11 = sreg(p.mask[1][1]);
    const int len0 = sreg(p.ks_len[0]), len1 = sreg(p.ks_len[1]);
    const int pos0 = sreg(p.ks_pos0[0]), pos1 = sreg(p.ks_pos0[1]);
    const int krow0 = sreg(p.ks_row0[0]), krow1 = sreg(p.ks_row0[1]);
    const int qrow0 = qs ? qrow0_b : qrow0_a;
    const int qpos0 = qs ? qpos0_b : qpos0_a;
    const int qlen = qs ? qlen_b : qlen_a;
    const int mk0 = qs ? m10 : m00;  // the host marks absent KV segments SKIP
    const int mk1 = qs ? m11 : m01;
    const int tile_row0 = qrow0 + qt_in * BMQ;
    const int tile_pos0 = qpos0 + qt_in * BMQ;
    const int tile_rows = min(BMQ, qlen - qt_in * BMQ);
    const int q0 = tile_pos0, q1 = tile_pos0 + tile_rows - 1;

    const int head = hb * HPW + wave / WPH;
    const int kvh = (hb * HPW) / p.group;  // the workgroup's heads share one KV head (HPW divides G)
    const int row_in_tile = (wave % WPH) * 32 + ql;
    const bool row_valid = row_in_tile < tile_rows;
    const int my_row = tile_row0 + row_in_tile;
    const int my_pos = tile_pos0 + row_in_tile;

    // ---- tile ranges of the (up to) two KV segments
    const bool any_doc = (mk0 == CP_MASK_DOC) || (mk1 == CP_MASK_DOC);
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
    // First visible key of a row under a pair's mask: the document start (DOC)
    // and, with a sliding window, position - window + 1 (DIAG and DOC); 0 is no
    // bound (positions are >= 0).  Non-decreasing in the row and <= the row.
    const int win = sreg(p.window);
    const int wlo0 = (win > 0) ? q0 - win + 1 : 0, wlo1 = (win > 0) ? q1 - win + 1 : 0;
    const int my_wlo = (win > 0) ? my_pos - win + 1 : 0;
    auto lower = [](int m, int doc_lo, int win_lo) {
        return (m == CP_MASK_DOC) ? max(doc_lo, win_lo) : (m == CP_MASK_DIAG_CAUSAL ? win_lo : 0);
    };
    const SegRange r0 = key_tile_range<kBN>(mk0, q0, q1, lower(mk0, lo0, wlo0), pos0, len0);
    const SegRange r1 = key_tile_range<kBN>(mk1, q0, q1, lower(mk1, lo0, wlo0), pos1, len1);
    const int tlo0 = r0.t_lo, thi0 = r0.t_hi, tlo1 = r1.t_lo, thi1 = r1.t_hi;
    // tiles of each segment that need no element mask
    const SegRange f0r = full_tile_range<kBN>(mk0, q0, lower(mk0, lo1, wlo1), pos0, len0);
    const SegRange f1r = full_tile_range<kBN>(mk1, q0, lower(mk1, lo1, wlo1), pos1, len1);
    const int my_lo_doc = max(my_lo, my_wlo);  // this row's lower bound on DOC pairs
    const int flo0 = f0r.t_lo, fn0 = f0r.t_hi - f0r.t_lo;
    const int flo1 = f1r.t_lo, fn1 = f1r.t_hi - f1r.t_lo;

    if (p.tile_map) {
        for (int col = tid; col < p.n_ktiles; col += kThreads) {
            const bool sec = col >= p.ktiles0;
            const int t = sec ? col - p.ktiles0 : col;
            const int m = sec ? mk1 : mk0;
            uint8_t c = CP_TILE_SKIP;
            if (t >= (sec ? tlo1 : tlo0) && t < (sec ? thi1 : thi0))
                c = key_tile_full<kBN>(m, q0, lower(m, lo1, wlo1), sec ? pos1 : pos0, sec ? len1 : len0, t)
                        ? CP_TILE_FULL
                        : CP_TILE_PARTIAL;
            p.tile_map[(int64_t)qt * p.n_ktiles + col] = c;
        }
    }

    const int n0 = thi0 - tlo0;
    const int n_it = n0 + (thi1 - tlo1);

    // ---- Q fragment in registers: lane holds query ql, dims 16*ds + 8*hl + 0..7
    bf16x8 qf[DS];
    {
        const uint16_t* qrow = p.q + ((int64_t)my_row * p.hq + head) * D + 8 * hl;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            u32x4 val = {0u, 0u, 0u, 0u};
            if (row_valid && n_it > 0) val = *reinterpret_cast<const u32x4*>(qrow + 16 * ds);
            qf[ds] = __builtin_bit_cast(bf16x8, val);
        }
    }

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    float m2 = -INFINITY;  // reference maximum of the row, in the exp2 domain (scores * c2)
    float l_run = 0.f;     // this half-wave's share of sum_j exp2(c2 s_j - m2)
    const float c2 = p.scale_log2;
    const int row_bytes = p.hkv * D * 2;

    // One descriptor per segment over this KV head's rows of that segment; a
    // tile is addressed by its byte offset in the span (rows past the segment
    // read as zero, kDeadTile past the last tile loads nothing).
    const int64_t head_off = (int64_t)kvh * D;
    const int64_t kv_stride = (int64_t)p.hkv * D;
    const __amdgpu_buffer_rsrc_t rk0 = span_rsrc(p.k + krow0 * kv_stride + head_off, (uint32_t)(len0 * row_bytes));
    const __amdgpu_buffer_rsrc_t rk1 = span_rsrc(p.k + krow1 * kv_stride + head_off, (uint32_t)(len1 * row_bytes));
    const __amdgpu_buffer_rsrc_t rv0 = span_rsrc(p.v + krow0 * kv_stride + head_off, (uint32_t)(len0 * row_bytes));
    const __amdgpu_buffer_rsrc_t rv1 = span_rsrc(p.v + krow1 * kv_stride + head_off, (uint32_t)(len1 * row_bytes));
    const int tile_bytes = kBN * row_bytes;
    const int toff0 = tlo0 * tile_bytes, toff1 = (tlo1 - n0) * tile_bytes;
    const TileLanes<D, kBN, kWaves> lanes(row_bytes, wave, lane);
    // loads of K or V tile j of the step's visit order
    auto issue = [=](bool is_v, int j, char* dst) {
        const bool second = j >= n0;
        const uint32_t off = (j < n_it) ? (uint32_t)(j * tile_bytes + pick(second, toff1, toff0)) : kDeadTile;
        const __amdgpu_buffer_rsrc_t rs = is_v ? pick(second, rv1, rv0) : pick(second, rk1, rk0);
        load_tile_at<D, kBN, kWaves>(dst, rs, lanes, off, wave);
    };

    // Tile `it` of the visit order: whether it needs the element mask, its key
    // count, first key position and mask.  (By-value capture: a select between
    // captured references becomes a select between addresses, which the compiler
    // keeps in a stack table and loads with a full wait.)
    struct TileInfo {
        bool full;
        int kcount, kp0, mask;
    };
    auto tile_info = [=](int it) -> TileInfo {
        const bool second = it >= n0;
        const int t = it + pick(second, tlo1 - n0, tlo0);  // tile index within its segment
        const bool full = (unsigned)(t - pick(second, flo1, flo0)) < (unsigned)pick(second, fn1, fn0);
        return TileInfo{full, min(kBN, pick(second, len1, len0) - t * kBN), pick(second, pos1, pos0) + t * kBN,
                        pick(second, mk1, mk0)};
    };

    // per-lane parts of the operand addresses (see TileLayout and key_of_reg)
    const int k_lane = L::off(ql, 8 * hl);
    const int grp = lane >> 4, jl = lane & 15;
    const int v_lane = L::off(4 * (grp >> 1) + (jl >> 2), 16 * (grp & 1) + 4 * (jl & 3));

    // S^T of one tile: 64 keys x this wave's 32 queries (prologue only)
    auto scores = [&](const char* kt, f32x16* sc) {
        sc[0] = f32x16{};
        sc[1] = f32x16{};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + k_lane + L::off(32 * kb, 16 * ds));
                sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], sc[kb], 0, 0, 0);
            }
    };

    bf16x8 pa[4], pbb[4];  // P (bf16) of two consecutive tiles: one being made, one consumed by P V

    // Element mask of tile it's scores on partial or ragged tiles: key k of the
    // tile is visible iff lo_lim <= k <= hi_lim, tested as one unsigned range
    // compare with the lane's 4 hl folded into the limits.
    auto mask_tile = [&](int it, f32x16* cur) {
        const TileInfo ti = tile_info(it);
        if (ti.full) return;
        int hi_lim = ti.kcount - 1;
        int lo_lim = 0;
        if (ti.mask != CP_MASK_FULL) {
            hi_lim = min(hi_lim, my_pos - ti.kp0);
            lo_lim = max(0, pick(ti.mask == CP_MASK_DOC, my_lo_doc, my_wlo) - ti.kp0);
        }
        const int lo_l = lo_lim - 4 * hl;
        const unsigned span = (unsigned)(hi_lim - lo_lim);
        const bool none = hi_lim < lo_lim;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key0 = row_of_reg(kb, r, 0);
                if (none || (unsigned)(key0 - lo_l) > span) cur[kb][r] = -INFINITY;
            }
    };

    // O^T += V^T P^T over one V tile: MFMA i = s4 * DB + db covers keys
    // 16 s4 + 4hl + {0..3, 8..11} and output dims 32 db .. 32 db + 31.  Its A
    // operand is two transposing reads of the row-major V tile.
    auto v_operand = [&](lds_char* vbase, int i) -> bf16x8 {
        lds_char* a0 = vbase + L::off(16 * (i / DB), 32 * (i % DB));
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0 + L::off(8, 0)));
        const s16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, a);
    };
    constexpr int kPV = 4 * DB;  // MFMAs of one P V product
    constexpr int kS = 2 * DS;   // MFMAs of one tile's scores
    static_assert(kPV == kS, "the step alternates P V and score MFMAs");
    constexpr int kEPM = 32 / (kPV + kS);  // scores of this lane per MFMA of a step (1 at D = 128, 2 at D = 64)
    // MFMA i of a tile's scores: head-dim step i / 2, key block i % 2
    auto k_operand = [&](lds_char* kbase, int i) -> bf16x8 {
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            kbase + L::off(32 * (i & 1), 16 * (i >> 1)));
    };

    // Exponential of this lane's scores e, e + 1 against the reference maximum:
    // P = 2^(c2 s - m2) as two fp32 values (for the row sum) and one packed bf16 pair.
    auto exp_pair = [&](const f32x16* cur, int e, float nb, float& x0, float& x1) -> uint32_t {
        x0 = __builtin_amdgcn_exp2f(fmaf(cur[e >> 4][e & 15], c2, nb));
        x1 = __builtin_amdgcn_exp2f(fmaf(cur[e >> 4][(e & 15) + 1], c2, nb));
        const f32x2 two = {x0, x1};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(two, bf16x2));
    };
    auto pack_p = [&](const uint32_t* pbits, bf16x8* pout) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const u32x4 w = {pbits[4 * q4], pbits[4 * q4 + 1], pbits[4 * q4 + 2], pbits[4 * q4 + 3]};
            pout[q4] = __builtin_bit_cast(bf16x8, w);
            materialise(pout[q4]);
        }
    };
    // The row maximum of a tile's scores (both half-waves), in the exp2 domain.
    auto tile_max2 = [&](const f32x16* cur) -> float {
        float mloc = cur[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, cur[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, cur[1][r]);
        return max_halves(mloc) * c2;
    };
    // Move the reference maximum up to mt2 where it is larger, rescaling the row
    // sum and the accumulator (from -inf: both are still zero).
    auto raise_max = [&](float mt2) {
        const float m2n = fmaxf(m2, mt2);
        const float alpha = (m2n == m2) ? 1.f : __builtin_amdgcn_exp2f(m2 - m2n);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        m2 = m2n;
    };
    // P of a whole tile (no interleaving): its row sum, bf16 P into pout.
    auto tile_exp = [&](const f32x16* cur, bf16x8* pout) -> float {
        const float nb = (m2 == -INFINITY) ? 0.f : -m2;
        float sa = 0.f, sb = 0.f;
        uint32_t pbits[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x0, x1;
            pbits[i] = exp_pair(cur, 2 * i, nb, x0, x1);
            sa += x0;
            sb += x1;
        }
        pack_p(pbits, pout);
        return sa + sb;
    };

    // The reference maximum m2 is not tracked tile by tile.  Exponentials are
    // taken against the current m2 and a row whose tile sum exceeds kPMax (or is
    // not finite), or that has no reference yet, takes the slow path: the tile's
    // true maximum raises m2, the accumulator and row sum are rescaled and the
    // tile's P is recomputed.  P then never exceeds kPMax, which bf16 and fp32
    // hold exactly in range; the P of a tile is only consumed by the next step's
    // P V, after this check.
    constexpr float kPMax = 1048576.f;  // 2^20
    auto check_tile = [&](const f32x16* cur, bf16x8* pout, float tsum) -> float {
        const bool bad = (m2 == -INFINITY) || !(tsum <= kPMax);
        if (__any(bad)) {
            raise_max(tile_max2(cur));
            tsum = tile_exp(cur, pout);
        }
        return tsum;
    };

    // Scores of tile 1 (16 MFMAs, K read two ahead) with the exponentials, bf16
    // P and row sum of tile 0 spread over them (prologue; tile 0's maximum is
    // already the reference).
    auto scores_and_exp = [&](const char* k_read, const f32x16* cur, f32x16* nxt, bf16x8* pout) -> float {
        lds_char* kbase = lds_base(k_read, k_lane);
        const float nb = (m2 == -INFINITY) ? 0.f : -m2;
        bf16x8 ka[3];
        ka[0] = k_operand(kbase, 0);
        ka[1] = k_operand(kbase, 1);
        nxt[0] = f32x16{};
        nxt[1] = f32x16{};
        float sa = 0.f, sb = 0.f;
        uint32_t pbits[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + 2 < kS) {
                ka[(i + 2) % 3] = k_operand(kbase, i + 2);
                order_memory();
            }
            if (i < kS) {
                nxt[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % 3], qf[i >> 1], nxt[i & 1], 0, 0, 0);
                pin(nxt[i & 1]);
            }
            float x0, x1;
            pbits[i] = exp_pair(cur, 2 * i, nb, x0, x1);
            sa += x0;
            sb += x1;
            pin(pbits[i]);
            pin(sa);
            pin(sb);
        }
        pack_p(pbits, pout);
        return sa + sb;
    };

    // Pipeline step it (1 <= it < n_it):
    //   mask of tile it (partial tiles only);
    //   loads (issued after the fourth MFMA): K(it+3) and V(it+1);
    //   32 MFMAs alternating O^T += V(it-1)^T P(it-1) and the scores of tile it+1,
    //   with the exponential, bf16 convert and row sum of one score of tile it
    //   after each (P(it) into p_new);
    //   the slow-path check of tile it.
    //   a barrier after every second step (even it), when bar is true.
    // Slots: K(j) and V(j) live in slot j mod 4, so each unrolled copy below
    // touches statically known buffers.  Step s reads K(s+1) and V(s-1) and
    // fills the slots of K(s-1) and V(s-3), whose last reads were at steps s-2
    // and earlier, before the last barrier (after step s-1 or s-2).  Every
    // barrier first waits for all of the wave's loads, so the tiles the next two
    // steps read (issued in the two steps before the barrier) have landed.
    auto step = [&](auto bar, int it, f32x16* cur, f32x16* nxt, const bf16x8* p_old, bf16x8* p_new, char* k_fill,
                    const char* k_read, char* v_fill, const char* v_read) {
        mask_tile(it, cur);
        lds_char* vbase = lds_base(v_read, v_lane);
        lds_char* kbase = lds_base(k_read, k_lane);
        const float nb = (m2 == -INFINITY) ? 0.f : -m2;
        bf16x8 va[3], ka[3];
        va[0] = v_operand(vbase, 0);
        ka[0] = k_operand(kbase, 0);
        va[1] = v_operand(vbase, 1);
        ka[1] = k_operand(kbase, 1);
        nxt[0] = f32x16{};
        nxt[1] = f32x16{};
        float sa = 0.f, sb = 0.f, x_prev = 0.f;
        uint32_t pbits[16];
#pragma unroll
        for (int j = 0; j < kPV + kS; ++j) {
            const int i = j >> 1;
            if ((j & 1) == 0) {
                if (i + 2 < kPV) {
                    va[(i + 2) % 3] = v_operand(vbase, i + 2);
                    order_memory();
                }
                acc[i % DB] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % 3], p_old[i / DB], acc[i % DB], 0, 0, 0);
                pin(acc[i % DB]);
            } else {
                if (i + 2 < kS) {
                    ka[(i + 2) % 3] = k_operand(kbase, i + 2);
                    order_memory();
                }
                nxt[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % 3], qf[i >> 1], nxt[i & 1], 0, 0, 0);
                pin(nxt[i & 1]);
            }
            if (j == 3) {
                // this step's loads, issued a few MFMAs in so that their address
                // arithmetic is off the path from the barrier to the first MFMA
                issue(false, it + 3, k_fill);
                issue(true, it + 1, v_fill);
                order_memory();
            }
            // scores e of this lane (register e % 16 of block e / 16)
#pragma unroll
            for (int u = 0; u < kEPM; ++u) {
                const int e = j * kEPM + u;
                const float x = __builtin_amdgcn_exp2f(fmaf(cur[e >> 4][e & 15], c2, nb));
                if ((e & 1) == 0) {
                    sa += x;
                    x_prev = x;
                    pin(sa);
                } else {
                    sb += x;
                    const f32x2 two = {x_prev, x};
                    pbits[e >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(two, bf16x2));
                    pin(pbits[e >> 1]);
                    pin(sb);
                }
            }
        }
        pack_p(pbits, p_new);
        l_run += check_tile(cur, p_new, sa + sb);
        if constexpr (decltype(bar)::value) ring_barrier<0>();
    };

    f32x16 sa[2], sb[2];
    if (n_it > 0) {
        issue(false, 0, kb0);
        issue(false, 1, kb1);
        __syncthreads();
        scores(kb0, sa);
        issue(false, 2, kb2);
        issue(true, 0, vb0);
        // step 0: no P V yet; tile 0's maximum sets the reference
        issue(false, 3, kb3);
        issue(true, 1, vb1);
        mask_tile(0, sa);
        raise_max(tile_max2(sa));
        l_run += scores_and_exp(kb1, sa, sb, pa);
        ring_barrier<0>();
        using NoBar = std::integral_constant<bool, false>;
        using Bar = std::integral_constant<bool, true>;
        for (int it = 1; it < n_it; it += 4) {
            step(NoBar{}, it, sb, sa, pa, pbb, kb0, kb2, vb2, vb0);
            if (it + 1 < n_it) step(Bar{}, it + 1, sa, sb, pbb, pa, kb1, kb3, vb3, vb1);
            if (it + 2 < n_it) step(NoBar{}, it + 2, sb, sa, pa, pbb, kb2, kb0, vb0, vb2);
            if (it + 3 < n_it) step(Bar{}, it + 3, sa, sb, pbb, pa, kb3, kb1, vb1, vb3);
        }
        // the last P V: V(n_it - 1) landed at the last step's barrier; P(j)
        // lives in pa for even j and in pbb for odd j
        const int last = (n_it - 1) & 3;
        lds_char* v_last = lds_base((last == 0) ? vb0 : (last == 1) ? vb1 : (last == 2) ? vb2 : vb3, v_lane);
        auto last_pv = [&](const bf16x8* pl) {
#pragma unroll
            for (int i = 0; i < kPV; ++i)
                acc[i % DB] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(v_last, i), pl[i / DB], acc[i % DB], 0, 0, 0);
        };
        if (last & 1)
            last_pv(pbb);
        else
            last_pv(pa);
    }

    // ---- epilogue: normalise and write O (fp32) and LSE (natural log), or
    // merge them into the accumulator: with this step's Ls and the stored La
    // (base 2 below), L = log2(2^La + 2^Ls), O = 2^(La-L) O_acc + 2^(Ls-L) acc / l.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (row_valid) {
        float* orow = p.o + ((int64_t)my_row * p.hq + head) * D;
        float* lrow = p.lse + (int64_t)head * p.q_rows + my_row;
        if constexpr (!MERGE) {
            const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 val = {acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv, acc[db][4 * i + 2] * inv,
                                 acc[db][4 * i + 3] * inv};
                    *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * i + 4 * hl) = val;
                }
            if (hl == 0) *lrow = (l_tot > 0.f) ? (m2 + __log2f(l_tot)) * kLn2 : -INFINITY;
        } else if (l_tot > 0.f) {
            const float ls2 = m2 + __log2f(l_tot);
            const float la2 = *lrow * kLog2e;  // -inf stays -inf
            const float hi = fmaxf(la2, ls2);
            const float l2 = hi + __log2f(1.f + __builtin_amdgcn_exp2f(-fabsf(la2 - ls2)));
            const float wa = __builtin_amdgcn_exp2f(la2 - l2);
            const float ws = __builtin_amdgcn_exp2f(ls2 - l2) / l_tot;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4* ptr = reinterpret_cast<f32x4*>(orow + 32 * db + 8 * i + 4 * hl);
                    const f32x4 old = *ptr;
                    f32x4 val;
#pragma unroll
                    for (int j = 0; j < 4; ++j) val[j] = fmaf(wa, old[j], ws * acc[db][4 * i + j]);
                    *ptr = val;
                }
            if (hl == 0) *lrow = l2 * kLn2;
        }
    }
    if (probe && tid == 0) {
        unsigned long long* rec = p.clk + 4 * (int64_t)w;
        rec[0] = t0_cycles;
        rec[1] = t0_ticks;
        rec[2] = __builtin_readcyclecounter();
        rec[3] = __builtin_readsteadycounter();
    }
}

template <int D, int HPW>
hipError_t launch(const FwdParams& prm, int grid, bool merge, hipStream_t stream) {
    if (merge)
        hipLaunchKernelGGL((fwd_step_kernel<D, HPW, true>), dim3(grid), dim3(kThreads), 0, stream, prm);
    else
        hipLaunchKernelGGL((fwd_step_kernel<D, HPW, false>), dim3(grid), dim3(kThreads), 0, stream, prm);
    return hipGetLastError();
}

// diagnostics (cp_debug_clock_probe)
std::atomic<unsigned long long*> g_clock_buf{nullptr};
std::atomic<int64_t> g_clock_cap{0};

cp_status fwd_step(const cp_attn_problem* p, const void* q, const void* k, const void* v, float* o_step,
                           float* lse_step, uint8_t* tile_map_out, bool merge, hipStream_t stream) {
    cp_status st = validate_problem(p, true);
    if (st != CP_OK) return st;
    // A merging step leaves rows that see no KV segment untouched: their query
    // segments stay out of the launch (unless the tile map is asked for, which
    // covers every query tile).
    const cp_attn_problem live = (merge && !tile_map_out) ? live_queries(p) : *p;
    p = &live;
    const TileGeom g = fwd_geom(p->hq, p->hkv);
    FwdParams prm = {};
    prm.q = static_cast<const uint16_t*>(q);
    prm.k = static_cast<const uint16_t*>(k);
    prm.v = static_cast<const uint16_t*>(v);
    prm.o = o_step;
    prm.lse = lse_step;
    prm.cu = p->cu_seqlens;
    prm.tile_map = tile_map_out;
    prm.clk = g_clock_buf.load();
    prm.clk_wgs = int32_t(std::min<int64_t>(g_clock_cap.load() / 4, int64_t(1) << 30));
    prm.n_docs = p->n_docs;
    prm.window = p->window;
    prm.hq = p->hq;
    prm.hkv = p->hkv;
    prm.group = p->hq / p->hkv;
    prm.q_rows = int32_t(p->q_rows);
    prm.scale = p->scale;
    prm.scale_log2 = p->scale * 1.4426950408889634f;
    prm.nkv_seg = p->n_kv_seg;
    int64_t nq = 0, nk = 0;
    for (int i = 0; i < 2; ++i) {
        const bool on = i < p->n_q_seg;
        prm.qs_row0[i] = on ? int32_t(p->q_seg[i].row0) : 0;
        prm.qs_pos0[i] = on ? int32_t(p->q_seg[i].pos0) : 0;
        prm.qs_len[i] = on ? int32_t(p->q_seg[i].len) : 0;
        const bool kon = i < p->n_kv_seg;
        prm.ks_row0[i] = kon ? int32_t(p->kv_seg[i].row0) : 0;
        prm.ks_pos0[i] = kon ? int32_t(p->kv_seg[i].pos0) : 0;
        prm.ks_len[i] = kon ? int32_t(p->kv_seg[i].len) : 0;
        for (int j = 0; j < 2; ++j)
            prm.mask[i][j] = (on && j < p->n_kv_seg) ? p->mask[i][j] : CP_MASK_SKIP;
        nq += ceil_div(prm.qs_len[i], g.bm);
        nk += ceil_div(prm.ks_len[i], g.bn);
    }
    prm.qtiles0 = int32_t(ceil_div(prm.qs_len[0], g.bm));
    prm.n_qtiles = int32_t(nq);
    prm.ktiles0 = int32_t(ceil_div(prm.ks_len[0], g.bn));
    prm.n_ktiles = int32_t(nk);
    const int64_t n_work = nq * (p->hq / g.hpw);
    if (n_work == 0) return CP_OK;
    if (!q || !o_step || !lse_step) return fail(CP_ERR_INVALID_ARG, "NULL tensor pointer");
    if (nk > 0 && (!k || !v)) return fail(CP_ERR_INVALID_ARG, "NULL K/V pointer");
    if (!all_aligned16({q, k, v, o_step, lse_step})) return fail(CP_ERR_INVALID_ARG, "tensor pointer not 16-byte aligned");
    if (n_work > (int64_t(1) << 30)) return fail(CP_ERR_UNSUPPORTED, "problem too large for one launch");
    if (!kv_spans_fit(p)) return fail(CP_ERR_UNSUPPORTED, "a KV segment spans 1 GiB or more");
    prm.n_work = int32_t(n_work);
    prm.n_hb = p->hq / g.hpw;
    {
        // the heaviest query tiles first (their work listed in the default order)
        std::vector<int64_t> work = query_tile_work(p, g.bm, g.bn);
        std::reverse(work.begin(), work.end());
        prm.q_first = heavier_last(work) ? 1 : 0;
    }
    const int grid = int(n_work);
    hipError_t e;
    if (p->head_dim == 128) {
        e = (g.hpw == 4) ? launch<128, 4>(prm, grid, merge, stream)
                         : (g.hpw == 2 ? launch<128, 2>(prm, grid, merge, stream)
                                       : launch<128, 1>(prm, grid, merge, stream));
    } else {
        e = (g.hpw == 4) ? launch<64, 4>(prm, grid, merge, stream)
                         : (g.hpw == 2 ? launch<64, 2>(prm, grid, merge, stream)
                                       : launch<64, 1>(prm, grid, merge, stream));
    }
    if (e != hipSuccess) return fail(CP_ERR_HIP, std::string("fwd launch: ") + hipGetErrorString(e));
    return CP_OK;
}

}  // namespace

}  // namespace cpattn

using namespace cpattn;

extern "C" cp_status cp_attn_fwd_step(const cp_attn_problem* p, const void* q, const void* k, const void* v,
                                      float* o_step, float* lse_step, uint8_t* tile_map_out,
                                      hipStream_t stream) {
    return fwd_step(p, q, k, v, o_step, lse_step, tile_map_out, false, stream);
}

extern "C" cp_status cp_attn_fwd_step_merge(const cp_attn_problem* p, const void* q, const void* k, const void* v,
                                            float* o_acc, float* lse_acc, uint8_t* tile_map_out,
                                            hipStream_t stream) {
    return fwd_step(p, q, k, v, o_acc, lse_acc, tile_map_out, true, stream);
}

extern "C" cp_status cp_debug_clock_probe(uint64_t* dev_buf, int64_t capacity) {
    if (dev_buf && capacity < 4) return fail(CP_ERR_INVALID_ARG, "clock probe buffer holds fewer than 4 values");
    g_clock_cap.store(dev_buf ? capacity : 0);
    g_clock_buf.store(reinterpret_cast<unsigned long long*>(dev_buf));
    return CP_OK;
}
