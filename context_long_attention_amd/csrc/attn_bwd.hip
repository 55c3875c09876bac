// Backward of one Pass-KV ring step on gfx950 ("Announcing Long-Context
// Training on TPUs with MaxText Context Parallelism", section "Built on a fast
// attention kernel": the ring calls the kernel once per step in the backward
// pass as well).  Given the final LSE and delta = rowsum(dO * O) of every local
// row, one step contributes
//   P = exp(scale q.k - LSE) on visible pairs,  dS = P (dO.v - delta),
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,  dQ_i += scale sum_j dS_ij k_j.
//
// Design (wave64, 32x32x16 bf16 MFMA, fp32 accumulation):
//  * A workgroup owns 128 keys (32 per wave) of one KV head and walks every
//    (query head of the GQA group, 32-row query tile) that can see them, so
//    dK and dV accumulate in registers and are written once, without atomics.
//  * S = Q K^T and dP = dO V^T put queries on the MFMA M axis; the query rows
//    are fed in a permuted order so that the P and dS registers are directly
//    the B operands of dV^T = dO^T P and dK^T = Q^T dS.  The transposed dO and
//    Q operands come from row-major LDS tiles through the gfx950 transposing
//    LDS read (ds_read_tr16_b64): 16 lanes read a 4-row x 16-column block and
//    each lane receives 4 consecutive rows of one column.
//  * dS goes through LDS once per tile; each wave then computes one 32-column
//    block of dQ over all 128 keys and adds it to the fp32 accumulator with
//    hardware float atomics (one add per element per workgroup and tile).
//  * Query tiles and their LSE/delta rows are double-buffered in LDS; one
//    barrier per tile.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BK = kBwdKeysPerWG;  // 128 keys per workgroup
constexpr int BQ = kBwdQRows;      // 32 query rows per tile

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
    const int32_t* cu;
    int32_t n_docs;
    int32_t hq, hkv, group;
    int32_t q_rows;
    float scale, scale_log2;
    int32_t nq_seg;
    int32_t qs_row0[2], qs_pos0[2], qs_len[2];
    int32_t ks_row0[2], ks_pos0[2], ks_len[2];
    int32_t mask[2][2];
    int32_t ktiles0, n_ktiles;
    int32_t n_work;
};

// Query index (within the 32-row tile) of score register r in half hl: MFMA
// row m = 8i + 4hl + j is fed by query row perm(m) = 16(i/2) + 8hl + 4(i%2) + j,
// so registers 8s..8s+7 hold queries 16s + 8hl + 0..7.
__device__ __forceinline__ int q_of_reg(int r, int hl) {
    const int i = r >> 2, j = r & 3;
    return 16 * (i >> 1) + 8 * hl + 4 * (i & 1) + j;
}

__device__ __forceinline__ int perm_row(int m) {
    const int i = m >> 3, h = (m >> 2) & 1, j = m & 3;
    return 16 * (i >> 1) + 8 * h + 4 * (i & 1) + j;
}

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

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// A/B operand of a 32x32x16 MFMA whose 8 k-slots of half hl are rows
// rbase + 8hl + 0..7 of a row-major LDS matrix X at column cbase + (lane % 32):
// two transposing reads, each giving 4 consecutive rows of one column.
__device__ __forceinline__ bf16x8 tr_operand(const char* x, int pitch, int rbase, int cbase, int lane) {
    const int grp = lane >> 4, j = lane & 15;
    const int row = rbase + 8 * (grp >> 1) + (j >> 2);
    const int col = cbase + 16 * (grp & 1) + 4 * (j & 3);
    const char* a0 = x + row * pitch + col * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0 + 4 * pitch));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

template <int D>
constexpr int row_pitch() { return D * 2 + 16; }
constexpr int kDsPitch = BQ * 2 + 16;

template <int D>
struct QStage {
    u32x4 q[D / 64];   // 32 rows x D/8 chunks over 256 threads
    u32x4 o[D / 64];
    float aux;         // lse*log2e, delta or document start of one row
};

template <int D>
__device__ __forceinline__ void load_q(QStage<D>& st, const BwdParams& p, int head, int qs, int tq, int mode,
                                       int tid) {
    constexpr int CPR = D / 8;
    const int rows = min(BQ, p.qs_len[qs] - tq * BQ);
    const int row0 = p.qs_row0[qs] + tq * BQ;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
        const int c = tid + kThreads * j;
        const int r = c / CPR, dc = c % CPR;
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (r < rows) {
            const int64_t off = ((int64_t)(row0 + r) * p.hq + head) * D + dc * 8;
            a = *reinterpret_cast<const u32x4*>(p.q + off);
            b = *reinterpret_cast<const u32x4*>(p.d_o + off);
        }
        st.q[j] = a;
        st.o[j] = b;
    }
    st.aux = 0.f;
    if (tid < 3 * BQ) {
        const int which = tid / BQ, r = tid % BQ;
        if (which == 0) {
            float v = INFINITY;  // rows outside the segment: P = 0
            if (r < rows) {
                const float l = p.lse[(int64_t)head * p.q_rows + row0 + r];
                v = (l == -INFINITY) ? INFINITY : l * 1.4426950408889634f;
            }
            st.aux = v;
        } else if (which == 1) {
            st.aux = (r < rows) ? p.delta[(int64_t)head * p.q_rows + row0 + r] : 0.f;
        } else if (mode == CP_MASK_DOC && r < rows) {
            const int pos = p.qs_pos0[qs] + tq * BQ + r;
            st.aux = __int_as_float(p.cu[doc_index(p.cu, p.n_docs, pos)]);
        }
    }
}

template <int D>
__device__ __forceinline__ void store_q(const QStage<D>& st, char* qlds, char* olds, float* aux, int tid) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
        const int c = tid + kThreads * j;
        const int r = c / CPR, dc = c % CPR;
        *reinterpret_cast<u32x4*>(qlds + r * row_pitch<D>() + dc * 16) = st.q[j];
        *reinterpret_cast<u32x4*>(olds + r * row_pitch<D>() + dc * 16) = st.o[j];
    }
    if (tid < 3 * BQ) aux[tid] = st.aux;
}

struct TileList {
    int lo[2], hi[2];  // query-tile ranges per query segment
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_step_kernel(const BwdParams p) {
    constexpr int DS = D / 16;
    constexpr int DB = D / 32;
    constexpr int RP = row_pitch<D>();
    constexpr int KT_BYTES = BK * RP;
    constexpr int QT_BYTES = BQ * RP;
    constexpr int DS_BYTES = BK * kDsPitch;
    // [K tile][2 x (Q, dO)][2 x dS^T][2 x aux(3 x 32 floats)]
    __shared__ __attribute__((aligned(16))) char smem[KT_BYTES + 4 * QT_BYTES + 2 * DS_BYTES + 2 * 3 * BQ * 4];
    char* ktile = smem;
    char* qbuf = smem + KT_BYTES;
    char* dsbuf = qbuf + 4 * QT_BYTES;
    float* auxbuf = reinterpret_cast<float*>(dsbuf + 2 * DS_BYTES);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int hl = lane >> 5;
    const int ql = lane & 31;

    const int per_xcd = gridDim.x >> 3;
    const int w = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (w >= p.n_work) return;
    const int g = w / p.n_ktiles;
    const int kt = w % p.n_ktiles;
    const int s = (kt < p.ktiles0) ? 0 : 1;
    const int kt_in = s ? kt - p.ktiles0 : kt;
    const int key_row0 = p.ks_row0[s] + kt_in * BK;
    const int kpos0 = p.ks_pos0[s] + kt_in * BK;
    const int kcount = min(BK, p.ks_len[s] - kt_in * BK);
    const int k0p = kpos0, k1p = kpos0 + kcount - 1;
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
    // ---- the whole K tile, row-major in LDS, for the dQ product
    {
        constexpr int CPR = D / 8;
        for (int c = tid; c < BK * CPR; c += kThreads) {
            const int r = c / CPR, dc = c % CPR;
            u32x4 a = {0u, 0u, 0u, 0u};
            if (r < kcount) a = *reinterpret_cast<const u32x4*>(p.k + (int64_t)(key_row0 + r) * kv_stride +
                                                                (int64_t)g * D + dc * 8);
            *reinterpret_cast<u32x4*>(ktile + r * RP + dc * 16) = a;
        }
    }

    // ---- query tiles that see any key of [k0p, k1p], per query segment
    TileList tl;
    int docend = 0x7fffffff;
    bool any_doc = false;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        tl.lo[qs] = tl.hi[qs] = 0;
        if (qs >= p.nq_seg) continue;
        const int m = p.mask[qs][s];
        const int plen = p.qs_len[qs], ppos = p.qs_pos0[qs];
        const int nqt = (plen + BQ - 1) / BQ;
        if (m == CP_MASK_SKIP || plen == 0 || kcount <= 0) continue;
        if (m == CP_MASK_FULL) {
            tl.hi[qs] = nqt;
            continue;
        }
        // causal: rows q >= k0p
        if (k0p > ppos + plen - 1) continue;
        int lo = (k0p <= ppos) ? 0 : (k0p - ppos) / BQ;
        int hi = nqt;
        if (m == CP_MASK_DOC) {
            any_doc = true;
            // rows whose document starts at or before k1p: q < end of k1p's document
            const int d1 = doc_index(p.cu, p.n_docs, k1p);
            docend = p.cu[d1 + 1];
            const int qmax = docend - 1;
            hi = (qmax < ppos) ? 0 : min(nqt, (qmax - ppos) / BQ + 1);
        }
        if (lo < hi) {
            tl.lo[qs] = lo;
            tl.hi[qs] = hi;
        }
    }
    (void)any_doc;
    (void)docend;
    const int n0 = tl.hi[0] - tl.lo[0];
    const int per_head = n0 + (tl.hi[1] - tl.lo[1]);
    const int n_it = per_head * p.group;

    auto item = [&](int it, int& head, int& qs, int& tq) {
        head = g * p.group + it / per_head;
        const int rem = it % per_head;
        qs = (rem < n0) ? 0 : 1;
        tq = qs ? tl.lo[1] + (rem - n0) : tl.lo[0] + rem;
    };

    f32x16 dka[DB], dva[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dka[db] = f32x16{};
        dva[db] = f32x16{};
    }
    const float c2 = p.scale_log2;

    QStage<D> st;
    if (n_it > 0) {
        int head, qs, tq;
        item(0, head, qs, tq);
        load_q<D>(st, p, head, qs, tq, p.mask[qs][s], tid);
        store_q<D>(st, qbuf, qbuf + QT_BYTES, auxbuf, tid);
    }
    __syncthreads();

    // dQ work split: D/32 column blocks over 4 waves; waves sharing a block split the keys
    constexpr int WPB = 4 / DB;          // waves per dQ column block
    const int dq_blk = wave % DB;
    const int dq_part = wave / DB;
    constexpr int KSTEPS = (BK / 16) / WPB;

    for (int it = 0; it < n_it; ++it) {
        const int buf = it & 1;
        char* qlds = qbuf + buf * 2 * QT_BYTES;
        char* olds = qlds + QT_BYTES;
        const float* aux = auxbuf + buf * 3 * BQ;
        char* dst = dsbuf + buf * DS_BYTES;
        int head, qs, tq;
        item(it, head, qs, tq);
        const int m = p.mask[qs][s];
        const int qrows = min(BQ, p.qs_len[qs] - tq * BQ);
        const int qrow0 = p.qs_row0[qs] + tq * BQ;
        const int qpos0 = p.qs_pos0[qs] + tq * BQ;
        if (it + 1 < n_it) {
            int h2, qs2, tq2;
            item(it + 1, h2, qs2, tq2);
            load_q<D>(st, p, h2, qs2, tq2, p.mask[qs2][s], tid);
        }

        // ---- S = Q K^T and dP = dO V^T (32 queries x this wave's 32 keys)
        f32x16 sc = f32x16{}, dp = f32x16{};
        {
            const char* qrow = qlds + perm_row(ql) * RP + 16 * hl;
            const char* orow = olds + perm_row(ql) * RP + 16 * hl;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(qrow + 32 * ds);
                sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[ds], sc, 0, 0, 0);
            }
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(orow + 32 * ds);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[ds], dp, 0, 0, 0);
            }
        }

        // ---- P and dS (fp32), element mask on partially visible or ragged tiles
        const int q_last = qpos0 + qrows - 1;
        bool full = (m == CP_MASK_FULL);
        if (!full) {
            const int lo_last = (m == CP_MASK_DOC) ? __float_as_int(aux[2 * BQ + qrows - 1]) : 0;
            full = (k1p <= qpos0) && (lo_last <= k0p);
        }
        const bool need_mask = !full || kcount < BK;
        f32x16 pr, dsr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qi = 16 * (i >> 1) + 8 * hl + 4 * (i & 1);
            const f32x4 l2 = *reinterpret_cast<const f32x4*>(aux + qi);
            const f32x4 dl = *reinterpret_cast<const f32x4*>(aux + BQ + qi);
            f32x4 lo4 = {0.f, 0.f, 0.f, 0.f};
            if (need_mask && m == CP_MASK_DOC) lo4 = *reinterpret_cast<const f32x4*>(aux + 2 * BQ + qi);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * i + j;
                float pv = __builtin_amdgcn_exp2f(fmaf(sc[r], c2, -l2[j]));
                if (need_mask) {
                    bool vis = key_valid;
                    if (m != CP_MASK_FULL) {
                        vis = vis && (kp <= qpos0 + qi + j);
                        if (m == CP_MASK_DOC) vis = vis && (kp >= __float_as_int(lo4[j]));
                    }
                    if (!vis) pv = 0.f;
                }
                pr[r] = pv;
                dsr[r] = pv * (dp[r] - dl[j]);
            }
        }
        (void)q_last;
        bf16x8 pb[2], db8[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            f32x8 a, b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                a[e] = pr[8 * s2 + e];
                b[e] = dsr[8 * s2 + e];
            }
            pb[s2] = __builtin_convertvector(a, bf16x8);
            db8[s2] = __builtin_convertvector(b, bf16x8);
        }

        // ---- dV^T += dO^T P and dK^T += Q^T dS  (M = dims, N = keys, K = queries)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 ao = tr_operand(olds, RP, 16 * s2, 32 * db, lane);
                dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, pb[s2], dva[db], 0, 0, 0);
                const bf16x8 aq = tr_operand(qlds, RP, 16 * s2, 32 * db, lane);
                dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, db8[s2], dka[db], 0, 0, 0);
            }
        }

        // ---- dS^T (bf16) to LDS: row = key, 4 consecutive queries per write
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qi = 16 * (i >> 1) + 8 * hl + 4 * (i & 1);
            f32x4 v4 = {dsr[4 * i], dsr[4 * i + 1], dsr[4 * i + 2], dsr[4 * i + 3]};
            const bf16x4 b4 = __builtin_convertvector(v4, bf16x4);
            *reinterpret_cast<bf16x4*>(dst + kk * kDsPitch + qi * 2) = b4;
        }

        if (it + 1 < n_it) {
            char* qn = qbuf + (buf ^ 1) * 2 * QT_BYTES;
            store_q<D>(st, qn, qn + QT_BYTES, auxbuf + (buf ^ 1) * 3 * BQ, tid);
        }
        __syncthreads();

        // ---- dQ[:, block] += scale * dS K  (M = queries, N = dims, K = keys)
        f32x16 dqa = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const int kb = 16 * (dq_part * KSTEPS + ks);
            const bf16x8 a = tr_operand(dst, kDsPitch, kb, 0, lane);
            const bf16x8 b = tr_operand(ktile, RP, kb, 32 * dq_blk, lane);
            dqa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, dqa, 0, 0, 0);
        }
        float* dqh = p.dq + (int64_t)head * D + 32 * dq_blk + ql;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qi = 8 * (r >> 2) + 4 * hl + (r & 3);
            if (qi < qrows) unsafeAtomicAdd(dqh + (int64_t)(qrow0 + qi) * p.hq * D, p.scale * dqa[r]);
        }
    }

    // ---- write this workgroup's dK (scaled) and dV rows
    if (key_valid) {
        const int64_t base = (int64_t)(key_row0 + kk) * kv_stride + (int64_t)g * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * hl;
                const f32x4 kv4 = {dka[db][4 * i] * p.scale, dka[db][4 * i + 1] * p.scale,
                                   dka[db][4 * i + 2] * p.scale, dka[db][4 * i + 3] * p.scale};
                const f32x4 vv4 = {dva[db][4 * i], dva[db][4 * i + 1], dva[db][4 * i + 2], dva[db][4 * i + 3]};
                *reinterpret_cast<f32x4*>(p.dk + base + d0) = kv4;
                *reinterpret_cast<f32x4*>(p.dv + base + d0) = vv4;
            }
    }
}

template <int D>
hipError_t launch(const BwdParams& prm, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((bwd_step_kernel<D>), dim3(grid), dim3(kThreads), 0, stream, prm);
    return hipGetLastError();
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" cp_status cp_attn_bwd_step(const cp_attn_problem* p, const void* q, const void* k, const void* v,
                                      const void* d_o, const float* lse, const float* delta, float* dq_acc,
                                      float* dk_out, float* dv_out, hipStream_t stream) {
    cp_status st = validate_problem(p, true);
    if (st != CP_OK) return st;
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
    prm.cu = p->cu_seqlens;
    prm.n_docs = p->n_docs;
    prm.hq = p->hq;
    prm.hkv = p->hkv;
    prm.group = p->hq / p->hkv;
    prm.q_rows = int32_t(p->q_rows);
    prm.scale = p->scale;
    prm.scale_log2 = p->scale * 1.4426950408889634f;
    prm.nq_seg = p->n_q_seg;
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
    const int64_t n_work = nk * p->hkv;
    if (n_work == 0) return CP_OK;
    if (!q || !k || !v || !d_o || !lse || !delta || !dq_acc || !dk_out || !dv_out)
        return fail(CP_ERR_INVALID_ARG, "NULL tensor pointer");
    if (n_work > (int64_t(1) << 30)) return fail(CP_ERR_UNSUPPORTED, "problem too large for one launch");
    prm.n_work = int32_t(n_work);
    const int grid = int(ceil_div(n_work, 8) * 8);
    hipError_t e = (p->head_dim == 128) ? launch<128>(prm, grid, stream) : launch<64>(prm, grid, stream);
    if (e != hipSuccess) return fail(CP_ERR_HIP, std::string("bwd launch: ") + hipGetErrorString(e));
    return CP_OK;
}
