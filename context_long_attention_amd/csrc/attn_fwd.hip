// Forward of one Pass-KV ring step on gfx950: blockwise causal flash attention
// of the stationary local queries against the KV block held at this step
// ("Announcing Long-Context Training on TPUs with MaxText Context
// Parallelism", section "Built on a fast attention kernel"; the ring itself is
// "Context Parallelism for Scalable Million-Token Inference", section "Ring
// Attention Algorithms").
//
// Design (gfx950, wave64, 32x32x16 bf16 MFMA with fp32 accumulation):
//  * A workgroup is 4 waves.  Each wave owns 32 query rows of one query head;
//    HPW heads of one GQA group share the workgroup, so every K/V tile staged
//    in LDS serves HPW heads (BMQ = 128 / HPW rows per workgroup tile).
//  * Scores are computed transposed, S^T = K Q^T (keys on the MFMA M axis,
//    queries on N): each lane then holds one query and 32 of its keys, so the
//    row max needs a single exchange between the two half-waves and the row
//    sum needs none until the epilogue.
//  * K rows are loaded into the MFMA in a permuted order chosen so that the
//    fp32 score registers, rounded to bf16, are directly the B operand of the
//    P V product (O^T = V^T P^T); V is stored transposed in LDS so the A
//    operand of that product is one 16-byte LDS read.
//  * K/V tiles are double-buffered in LDS with rows padded by 16 bytes (the
//    MFMA operand reads of 16 lanes then hit distinct banks and every read is
//    a base register plus an immediate offset); the global loads of tile i+1
//    are issued before the MFMAs of tile i.
//  * Tiles with no visible pair are never visited (block-sparse skip); the
//    element mask is applied only to partially visible or ragged tiles.
//  * Workgroup ids are mapped so each XCD (ids equal mod 8) works on one
//    range of head blocks (sharing K/V in its L2), latest positions first.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "internal.h"

namespace cpattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBN = 64;       // keys per tile
constexpr int kThreads = 256; // 4 waves

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

// Key (within a 64-key tile) held by score register r of key block kb in half
// hl of the wave.  MFMA output row m = 8i + 4hl + j (r = 4i + j) is fed by K
// row perm(m) = 16(i/2) + 8hl + 4(i%2) + j, so that registers 8(s%2)..8(s%2)+7
// of block s/2 hold keys 16s + 8hl + 0..7: the B operand of PV step s.
__device__ __forceinline__ int key_of_reg(int kb, int r, int hl) {
    const int i = r >> 2, j = r & 3;
    return 32 * kb + 16 * (i >> 1) + 8 * hl + 4 * (i & 1) + j;
}

__device__ __forceinline__ int perm_row(int m) {
    const int i = m >> 3, h = (m >> 2) & 1, j = m & 3;
    return 16 * (i >> 1) + 8 * h + 4 * (i & 1) + j;
}

// LDS row pitches (bytes): K tile [kBN][D], transposed V tile [D][kBN].
template <int D>
constexpr int k_pitch() { return D * 2 + 16; }
constexpr int kVtPitch = kBN * 2 + 16;

__device__ __forceinline__ int doc_index(const int32_t* cu, int n_docs, int pos) {
    int lo = 0, hi = n_docs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= pos)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

struct SegRange {
    int t_lo, t_hi;
};

// Mirror of the host tile_range rule (global positions, q1 = last row).
__device__ __forceinline__ SegRange seg_range(int mask, int q0, int q1, int lo0, int kpos0, int klen) {
    const int nkt = (klen + kBN - 1) / kBN;
    if (mask == CP_MASK_SKIP || klen == 0) return {0, 0};
    if (mask == CP_MASK_FULL) return {0, nkt};
    const int t_hi = (q1 < kpos0) ? 0 : min(nkt, (q1 - kpos0) / kBN + 1);
    int t_lo = 0;
    if (lo0 > kpos0) {
        if (lo0 > kpos0 + klen - 1) return {0, 0};
        t_lo = (lo0 - kpos0) / kBN;
    }
    if (t_lo >= t_hi) return {0, 0};
    return {t_lo, t_hi};
}

__device__ __forceinline__ bool tile_full(int mask, int q0, int lo1, int kpos0, int klen, int t) {
    if (mask == CP_MASK_FULL) return true;
    const int k0 = kpos0 + t * kBN;
    const int k1 = min(kpos0 + klen, k0 + kBN) - 1;
    return k1 <= q0 && k0 >= lo1;
}

template <int D>
struct Stage {
    u32x4 kreg[D / 32];  // K: BN*D/8 16-byte chunks over 256 threads
    u32x4 vreg[4];       // V: 4 keys x 8 dims per thread
};

template <int D>
__device__ __forceinline__ void load_tile(Stage<D>& st, const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, int64_t row_stride,
                                          int kcount, int tid) {
    constexpr int CPR = D / 8;  // 16-byte chunks per key row
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
        const int c = tid + kThreads * j;
        const int kr = c / CPR, dc = c % CPR;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (kr < kcount) val = *reinterpret_cast<const u32x4*>(kbase + kr * row_stride + dc * 8);
        st.kreg[j] = val;
    }
    constexpr int VBLOCKS = (kBN / 4) * (D / 8);
    if (VBLOCKS == kThreads || tid < VBLOCKS) {
        const int kq = tid / (D / 8), dg = tid % (D / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int kr = kq * 4 + r;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (kr < kcount) val = *reinterpret_cast<const u32x4*>(vbase + kr * row_stride + dg * 8);
            st.vreg[r] = val;
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const Stage<D>& st, char* klds, char* vlds, int tid) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
        const int c = tid + kThreads * j;
        const int kr = c / CPR, dc = c % CPR;
        *reinterpret_cast<u32x4*>(klds + kr * k_pitch<D>() + (dc << 4)) = st.kreg[j];
    }
    constexpr int VBLOCKS = (kBN / 4) * (D / 8);
    if (VBLOCKS == kThreads || tid < VBLOCKS) {
        const int kq = tid / (D / 8), dg = tid % (D / 8);
        // Transpose the 4 keys x 8 dims block: for each dim, the 4 keys are one 8-byte run of V^T.
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            u32x2 pk;
            pk.x = __builtin_amdgcn_perm(st.vreg[1][w], st.vreg[0][w], sel);
            pk.y = __builtin_amdgcn_perm(st.vreg[3][w], st.vreg[2][w], sel);
            const int d = dg * 8 + e;
            const int off = d * kVtPitch + (kq << 3);
            *reinterpret_cast<u32x2*>(vlds + off) = pk;
        }
    }
}

template <int D, int HPW>
__global__ __launch_bounds__(kThreads, 2) void fwd_step_kernel(const FwdParams p) {
    constexpr int WPH = 4 / HPW;      // waves per head
    constexpr int BMQ = 32 * WPH;     // query rows per workgroup tile
    constexpr int DS = D / 16;        // MFMA k-steps over the head dim
    constexpr int DB = D / 32;        // 32-row blocks of O^T
    constexpr int KBYTES = kBN * k_pitch<D>();
    constexpr int VBYTES = D * kVtPitch;
    __shared__ __attribute__((aligned(16))) char smem[2 * (KBYTES + VBYTES)];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
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
    const int kvh = head / p.group;
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
        rng[s] = (s < p.nkv_seg) ? seg_range(mk[s], q0, q1, doc ? lo0 : 0, p.ks_pos0[s], p.ks_len[s])
                                 : SegRange{0, 0};
    }

    if (p.tile_map) {
        for (int col = tid; col < p.n_ktiles; col += kThreads) {
            const int s = (col < p.ktiles0) ? 0 : 1;
            const int t = s ? col - p.ktiles0 : col;
            uint8_t c = CP_TILE_SKIP;
            if (t >= rng[s].t_lo && t < rng[s].t_hi)
                c = tile_full(mk[s], q0, mk[s] == CP_MASK_DOC ? lo1 : 0, p.ks_pos0[s], p.ks_len[s], t)
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
    float m_run = -INFINITY;
    float l_run = 0.f;
    const float c2 = p.scale_log2;
    const int64_t kv_stride = (int64_t)p.hkv * D;

    auto tile_of = [&](int it, int& s, int& t) {
        s = (it < n0) ? 0 : 1;
        t = s ? rng[1].t_lo + (it - n0) : rng[0].t_lo + it;
    };

    Stage<D> st;
    if (n_it > 0) {
        int s, t;
        tile_of(0, s, t);
        const int64_t r0 = p.ks_row0[s] + (int64_t)t * kBN;
        const uint16_t* kb = p.k + (r0 * p.hkv + kvh) * D;
        const uint16_t* vb = p.v + (r0 * p.hkv + kvh) * D;
        load_tile<D>(st, kb, vb, kv_stride, min(kBN, p.ks_len[s] - t * kBN), tid);
        store_tile<D>(st, smem, smem + KBYTES, tid);
    }
    __syncthreads();

    for (int it = 0; it < n_it; ++it) {
        char* klds = smem + (it & 1) * (KBYTES + VBYTES);
        char* vlds = klds + KBYTES;
        int s, t;
        tile_of(it, s, t);
        if (it + 1 < n_it) {
            int s2, t2;
            tile_of(it + 1, s2, t2);
            const int64_t r0 = p.ks_row0[s2] + (int64_t)t2 * kBN;
            const uint16_t* kb = p.k + (r0 * p.hkv + kvh) * D;
            const uint16_t* vb = p.v + (r0 * p.hkv + kvh) * D;
            load_tile<D>(st, kb, vb, kv_stride, min(kBN, p.ks_len[s2] - t2 * kBN), tid);
        }

        // ---- S^T = K Q^T for 64 keys x 32 queries
        f32x16 sc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sc[kb] = f32x16{};
            const int kr = 32 * kb + perm_row(ql);
            const char* krow = klds + kr * k_pitch<D>() + (hl << 4);
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (ds << 5));
                sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], sc[kb], 0, 0, 0);
            }
        }

        // ---- element mask on partial or ragged tiles
        const int kcount = min(kBN, p.ks_len[s] - t * kBN);
        const int kp0 = p.ks_pos0[s] + t * kBN;
        const int m = mk[s];
        const bool full = tile_full(m, q0, m == CP_MASK_DOC ? lo1 : 0, p.ks_pos0[s], p.ks_len[s], t);
        if (!full || kcount < kBN) {
            int hi_lim = kcount - 1;
            int lo_lim = -kBN;
            if (m != CP_MASK_FULL) {
                hi_lim = min(hi_lim, my_pos - kp0);
                if (m == CP_MASK_DOC) lo_lim = my_lo - kp0;
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key_of_reg(kb, r, hl);
                    if (key > hi_lim || key < lo_lim) sc[kb][r] = -INFINITY;
                }
        }

        // ---- online softmax (exp2 domain, scale folded into one FMA)
        float mloc = sc[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, sc[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sc[1][r]);
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_run, mloc);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
        const float nb = -m_use * c2;
        m_run = m_new;
        float lsum = 0.f;
        bf16x8 pb[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x8 pv;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pe = __builtin_amdgcn_exp2f(fmaf(sc[kb][8 * half + e], c2, nb));
                    pv[e] = pe;
                    lsum += pe;
                }
                pb[2 * kb + half] = __builtin_convertvector(pv, bf16x8);
            }
        }
        l_run = l_run * alpha + lsum;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = 32 * db + ql;
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(vlds + d * kVtPitch + (s4 << 5) + (hl << 4));
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s4], acc[db], 0, 0, 0);
            }
        }

        if (it + 1 < n_it) {
            char* knext = smem + ((it + 1) & 1) * (KBYTES + VBYTES);
            store_tile<D>(st, knext, knext + KBYTES, tid);
        }
        __syncthreads();
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
            const float lse = (l_tot > 0.f) ? m_run * p.scale + __logf(l_tot) : -INFINITY;
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
