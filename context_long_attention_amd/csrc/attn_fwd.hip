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
//    tile read as zero) into a ring of four K and four V buffers, three tiles
//    ahead of use; each step waits only for the tiles the next step reads.
//  * Rotated pipeline: the P V product of tile i-1 overlaps the mask and row
//    max of tile i; the scores of tile i+1 overlap the exponentials of tile i.
//  * The reference maximum is raised only when a row's maximum grows by more
//    than 2^8 in the exp2 domain, so the accumulator is rescaled rarely; P is
//    then bounded by 256, which fp32 accumulation and bf16 rounding absorb.
//  * Tiles with no visible pair are never visited (block-sparse skip); the
//    element mask runs only on partially visible or ragged tiles.
//  * Workgroup ids map each XCD (ids equal mod 8) to one range of head blocks
//    (K/V shared in its L2), latest query positions first.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "internal.h"
#include "tiles.h"

namespace cpattn {

namespace {

using namespace dev;

constexpr int kBN = 64;                    // keys per tile
constexpr int kWaves = kFwdWaves;          // 8 waves: 2 per SIMD, one workgroup per CU
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;                 // K/V tiles in flight (LDS ring)

struct FwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    float* o;
    float* lse;
    const int32_t* cu;
    uint8_t* tile_map;
    int32_t n_docs;
    int32_t hq, hkv, group;
    int32_t q_rows;
    float scale, scale_log2;
    int32_t nkv_seg;
    int32_t qs_row0[2], qs_pos0[2], qs_len[2];
    int32_t ks_row0[2], ks_pos0[2], ks_len[2];
    int32_t mask[2][2];
    int32_t qtiles0, n_qtiles;
    int32_t ktiles0, n_ktiles;
    int32_t n_work;
};

template <int D, int HPW>
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

    // ---- work decode: XCD-major ranges of head blocks, latest query tiles first
    const int per_xcd = gridDim.x >> 3;
    const int w = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (w >= p.n_work) return;
    const int hb = w / p.n_qtiles;
    const int qt = p.n_qtiles - 1 - (w % p.n_qtiles);
    const int qs = (qt < p.qtiles0) ? 0 : 1;
    const int qt_in = qs ? qt - p.qtiles0 : qt;
    const int tile_row0 = p.qs_row0[qs] + qt_in * BMQ;
    const int tile_pos0 = p.qs_pos0[qs] + qt_in * BMQ;
    const int tile_rows = min(BMQ, p.qs_len[qs] - qt_in * BMQ);
    const int q0 = tile_pos0, q1 = tile_pos0 + tile_rows - 1;

    const int head = hb * HPW + wave / WPH;
    const int kvh = (hb * HPW) / p.group;  // the workgroup's heads share one KV head (HPW divides G)
    const int row_in_tile = (wave % WPH) * 32 + ql;
    const bool row_valid = row_in_tile < tile_rows;
    const int my_row = tile_row0 + row_in_tile;
    const int my_pos = tile_pos0 + row_in_tile;

    // ---- tile ranges of the (up to) two KV segments
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
    SegRange rng[2];
    int mk[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        mk[s] = (s < p.nkv_seg) ? p.mask[qs][s] : CP_MASK_SKIP;
        const bool doc = (mk[s] == CP_MASK_DOC);
        rng[s] = (s < p.nkv_seg) ? key_tile_range<kBN>(mk[s], q0, q1, doc ? lo0 : 0, p.ks_pos0[s], p.ks_len[s])
                                 : SegRange{0, 0};
    }

    if (p.tile_map) {
        for (int col = tid; col < p.n_ktiles; col += kThreads) {
            const int s = (col < p.ktiles0) ? 0 : 1;
            const int t = s ? col - p.ktiles0 : col;
            uint8_t c = CP_TILE_SKIP;
            if (t >= rng[s].t_lo && t < rng[s].t_hi)
                c = key_tile_full<kBN>(mk[s], q0, mk[s] == CP_MASK_DOC ? lo1 : 0, p.ks_pos0[s], p.ks_len[s], t)
                        ? CP_TILE_FULL
                        : CP_TILE_PARTIAL;
            p.tile_map[(int64_t)qt * p.n_ktiles + col] = c;
        }
    }

    const int n0 = rng[0].t_hi - rng[0].t_lo;
    const int n_it = n0 + (rng[1].t_hi - rng[1].t_lo);

    // ---- Q fragment in registers: lane holds query ql, dims 16*ds + 8*hl + 0..7
    bf16x8 qf[DS];
    {
        const uint16_t* qrow = p.q + ((int64_t)my_row * p.hq + head) * D + 8 * hl;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            u32x4 val = {0u, 0u, 0u, 0u};
            if (row_valid) val = *reinterpret_cast<const u32x4*>(qrow + 16 * ds);
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

    // Per-segment values held in scalars for the whole tile loop (a runtime
    // index into the parameter block would reload it from memory every tile).
    const int len0 = p.ks_len[0], len1 = p.ks_len[1];
    const int pos0 = p.ks_pos0[0], pos1 = p.ks_pos0[1];
    const int mk0 = mk[0], mk1 = mk[1];
    const int tlo0 = rng[0].t_lo, tlo1 = rng[1].t_lo;
    const int64_t head_off = (int64_t)kvh * D;
    const uint16_t* const kseg0 = p.k + (int64_t)p.ks_row0[0] * p.hkv * D + head_off;
    const uint16_t* const kseg1 = p.k + (int64_t)p.ks_row0[1] * p.hkv * D + head_off;
    const uint16_t* const vseg0 = p.v + (int64_t)p.ks_row0[0] * p.hkv * D + head_off;
    const uint16_t* const vseg1 = p.v + (int64_t)p.ks_row0[1] * p.hkv * D + head_off;
    const int64_t tile_elems = (int64_t)kBN * p.hkv * D;

    struct TileRef {
        int t, len, pos, mask, seg;
    };
    auto tile_of = [&](int it) -> TileRef {
        const bool second = it >= n0;
        const int t = second ? tlo1 + (it - n0) : tlo0 + it;
        return TileRef{t, second ? len1 : len0, second ? pos1 : pos0, second ? mk1 : mk0, second ? 1 : 0};
    };
    // Descriptor of tile `it`; past the last tile an empty descriptor, whose
    // loads fetch nothing and write zeros (every step issues the same loads).
    auto rsrc_of = [&](bool is_v, int it) -> __amdgpu_buffer_rsrc_t {
        const TileRef tr = tile_of(it);
        const bool live = it < n_it;
        const uint16_t* base = is_v ? (tr.seg ? vseg1 : vseg0) : (tr.seg ? kseg1 : kseg0);
        return tile_rsrc(live ? base + tr.t * tile_elems : base, live ? min(kBN, tr.len - tr.t * kBN) : 0,
                         row_bytes);
    };

    // per-lane parts of the operand addresses (see TileLayout and key_of_reg)
    const int k_lane = L::off(ql, 8 * hl);
    const int grp = lane >> 4, jl = lane & 15;
    const int v_lane = L::off(4 * (grp >> 1) + (jl >> 2), 16 * (grp & 1) + 4 * (jl & 3));

    // S^T of one tile: 64 keys x this wave's 32 queries
    auto scores = [&](const char* kt, f32x16* sc) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sc[kb] = f32x16{};
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + k_lane + L::off(32 * kb, 16 * ds));
                sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], sc[kb], 0, 0, 0);
            }
        }
    };

    // At each step's barrier the loads of the last two steps may still be in
    // flight; everything older (the tiles the next step reads) has landed.
    constexpr int kPending = 2 * 2 * (L::NBLK / kWaves);

    bf16x8 pb[4];  // P of the previous tile (bf16), consumed by the next step's P V
    // Rotated pipeline step `it` (0 <= it <= n_it):
    //   loads:  K(it+4) into the K slot freed by K(it), V(it+2) into the V slot freed by V(it-2);
    //   PV:     O^T += V(it-1)^T P(it-1)                       (MFMA, overlaps the next part)
    //   mask, row max and rare rescale of tile it's scores  (VALU)
    //   scores of tile it+1 (MFMA) overlapping exp / sum / bf16 of tile it (VALU) -> P(it)
    // Slots: K(j) and V(j) live in slot j mod 4, so each unrolled copy below
    // touches statically known buffers.
    auto step = [&](int it, f32x16* cur, f32x16* nxt, char* k_fill, const char* k_read, char* v_fill,
                    const char* v_read) {
        load_tile_lds<D, kBN, kWaves>(k_fill, rsrc_of(false, it + 4), row_bytes, wave, lane);
        load_tile_lds<D, kBN, kWaves>(v_fill, rsrc_of(true, it + 2), row_bytes, wave, lane);

        if (it >= 1) {
            // O^T += V^T P^T: step s4 covers keys 16 s4 + 4hl + {0..3, 8..11}
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const char* a0 = v_read + v_lane + L::off(16 * s4, 32 * db);
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0 + L::off(8, 0)));
                    const s16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb[s4],
                                                                       acc[db], 0, 0, 0);
                }
            }
        }

        if (it < n_it) {
            const TileRef tr = tile_of(it);
            // element mask on partial or ragged tiles: key k of the tile is visible
            // iff lo_lim <= k <= hi_lim, tested as one unsigned range compare with the
            // lane's 4 hl folded into the limits
            const int kcount = min(kBN, tr.len - tr.t * kBN);
            const int kp0 = tr.pos + tr.t * kBN;
            const int m = tr.mask;
            const bool full = key_tile_full<kBN>(m, q0, m == CP_MASK_DOC ? lo1 : 0, tr.pos, tr.len, tr.t);
            if (!full || kcount < kBN) {
                int hi_lim = kcount - 1;
                int lo_lim = 0;
                if (m != CP_MASK_FULL) {
                    hi_lim = min(hi_lim, my_pos - kp0);
                    if (m == CP_MASK_DOC) lo_lim = max(0, my_lo - kp0);
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
            }

            // row maximum; the reference maximum is raised only when it grows by more than 2^8
            float mloc = cur[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, cur[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, cur[1][r]);
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
            const float mt2 = mloc * c2;
            const bool raise = mt2 > m2 + 8.f;
            if (__any(raise)) {
                const float m2n = raise ? mt2 : m2;
                const float alpha = (m2n == m2) ? 1.f : __builtin_amdgcn_exp2f(m2 - m2n);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db] *= alpha;
                m2 = m2n;
            }
            const float nb = (m2 == -INFINITY) ? 0.f : -m2;

            // scores of the next tile (its K tile is resident; unused after the last tile)
            scores(k_read, nxt);

            float part[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    f32x8 pv;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        pv[e] = __builtin_amdgcn_exp2f(fmaf(cur[kb][8 * half + e], c2, nb));
                    pb[2 * kb + half] = __builtin_convertvector(pv, bf16x8);
                    part[2 * kb + half] =
                        ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
                }
            }
            l_run += (part[0] + part[1]) + (part[2] + part[3]);
        }
        ring_barrier<kPending>();  // the tiles the next step reads have landed; this step's slots are free
    };

    f32x16 sa[2], sb[2];
    if (n_it > 0) {
        load_tile_lds<D, kBN, kWaves>(kb0, rsrc_of(false, 0), row_bytes, wave, lane);
        load_tile_lds<D, kBN, kWaves>(kb1, rsrc_of(false, 1), row_bytes, wave, lane);
        __syncthreads();
        scores(kb0, sa);
        // issue order matters for the wait counts: V0, K2, V1, K3, then two per step
        load_tile_lds<D, kBN, kWaves>(vb0, rsrc_of(true, 0), row_bytes, wave, lane);
        load_tile_lds<D, kBN, kWaves>(kb2, rsrc_of(false, 2), row_bytes, wave, lane);
        load_tile_lds<D, kBN, kWaves>(vb1, rsrc_of(true, 1), row_bytes, wave, lane);
        load_tile_lds<D, kBN, kWaves>(kb3, rsrc_of(false, 3), row_bytes, wave, lane);
        ring_barrier<kPending>();  // K(1) and V(0) have landed; every wave has read K(0)
        for (int it = 0; it <= n_it; it += 4) {
            step(it, sa, sb, kb0, kb1, vb2, vb3);
            if (it + 1 <= n_it) step(it + 1, sb, sa, kb1, kb2, vb3, vb0);
            if (it + 2 <= n_it) step(it + 2, sa, sb, kb2, kb3, vb0, vb1);
            if (it + 3 <= n_it) step(it + 3, sb, sa, kb3, kb0, vb1, vb2);
        }
    }

    // ---- epilogue: normalise, write O (fp32) and LSE (natural log)
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (row_valid) {
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        float* orow = p.o + ((int64_t)my_row * p.hq + head) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 val = {acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv, acc[db][4 * i + 2] * inv,
                             acc[db][4 * i + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * i + 4 * hl) = val;
            }
        if (hl == 0) {
            const float lse = (l_tot > 0.f) ? (m2 + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
            p.lse[(int64_t)head * p.q_rows + my_row] = lse;
        }
    }
}

template <int D, int HPW>
hipError_t launch(const FwdParams& prm, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((fwd_step_kernel<D, HPW>), dim3(grid), dim3(kThreads), 0, stream, prm);
    return hipGetLastError();
}

}  // namespace

}  // namespace cpattn

using namespace cpattn;

extern "C" cp_status cp_attn_fwd_step(const cp_attn_problem* p, const void* q, const void* k, const void* v,
                                      float* o_step, float* lse_step, uint8_t* tile_map_out,
                                      hipStream_t stream) {
    cp_status st = validate_problem(p, true);
    if (st != CP_OK) return st;
    const TileGeom g = fwd_geom(p->hq, p->hkv);
    FwdParams prm = {};
    prm.q = static_cast<const uint16_t*>(q);
    prm.k = static_cast<const uint16_t*>(k);
    prm.v = static_cast<const uint16_t*>(v);
    prm.o = o_step;
    prm.lse = lse_step;
    prm.cu = p->cu_seqlens;
    prm.tile_map = tile_map_out;
    prm.n_docs = p->n_docs;
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
    if (n_work > (int64_t(1) << 30)) return fail(CP_ERR_UNSUPPORTED, "problem too large for one launch");
    prm.n_work = int32_t(n_work);
    const int grid = int(ceil_div(n_work, 8) * 8);
    hipError_t e;
    if (p->head_dim == 128) {
        e = (g.hpw == 4) ? launch<128, 4>(prm, grid, stream)
                         : (g.hpw == 2 ? launch<128, 2>(prm, grid, stream) : launch<128, 1>(prm, grid, stream));
    } else {
        e = (g.hpw == 4) ? launch<64, 4>(prm, grid, stream)
                         : (g.hpw == 2 ? launch<64, 2>(prm, grid, stream) : launch<64, 1>(prm, grid, stream));
    }
    if (e != hipSuccess) return fail(CP_ERR_HIP, std::string("fwd launch: ") + hipGetErrorString(e));
    return CP_OK;
}
