// HBM-bound elementwise kernels of the ring:
//  * merge of partial (O, LSE) pairs over disjoint key sets ("Context
//    Parallelism for Scalable Million-Token Inference", section "Ring
//    Attention Algorithms": the partial outputs of Pass KV are merged into
//    the full attention output);
//  * delta = rowsum(dO * O) for the backward pass.
// One group of D/4 lanes handles one (row, head): each lane moves one float4
// of the head dimension, so a wave reads and writes contiguous 512-byte rows.
// All lanes of a group sit in the same wave, so every lane reads the old LSE
// before the group's first lane overwrites it.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>

#include "internal.h"

namespace cpattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(float* __restrict__ o_acc, float* __restrict__ lse_acc,
                                                         const float* __restrict__ o_t,
                                                         const float* __restrict__ lse_t, int64_t rows,
                                                         int heads) {
    constexpr int LPG = D / 4;  // lanes per (row, head)
    const int64_t gidx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t pair = gidx / LPG;
    const int sub = int(gidx % LPG);
    if (pair >= rows * heads) return;
    const int64_t row = pair / heads;
    const int head = int(pair % heads);
    const int64_t li = (int64_t)head * rows + row;
    const float la = lse_acc[li];
    const float lb = lse_t[li];
    const float mx = fmaxf(la, lb);
    f32x4 out = {0.f, 0.f, 0.f, 0.f};
    float lnew = -INFINITY;
    if (mx != -INFINITY) {
        const float wa = __expf(la - mx);
        const float wb = __expf(lb - mx);
        const float inv = 1.f / (wa + wb);
        lnew = mx + __logf(wa + wb);
        const f32x4 a = *reinterpret_cast<const f32x4*>(o_acc + pair * D + sub * 4);
        const f32x4 b = *reinterpret_cast<const f32x4*>(o_t + pair * D + sub * 4);
        // with wa, wb in (0, 1] and max(wa, wb) == 1 the division is well conditioned
        out = a * (wa * inv) + b * (wb * inv);
    }
    *reinterpret_cast<f32x4*>(o_acc + pair * D + sub * 4) = out;
    if (sub == 0) lse_acc[li] = lnew;
}

// The N-way merge: the partials of one query row over n disjoint key sets (an
// owner merging what Pass Q's all-to-all delivers), read once each.
constexpr int kMaxParts = 64;
struct MergeNParams {
    const float* o[kMaxParts];
    const float* lse[kMaxParts];
    float* o_out;
    float* lse_out;
    int64_t rows;
    int32_t heads, n;
};

template <int D>
__global__ __launch_bounds__(kThreads) void merge_n_kernel(const MergeNParams p) {
    constexpr int LPG = D / 4;
    const int64_t gidx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t pair = gidx / LPG;
    const int sub = int(gidx % LPG);
    if (pair >= p.rows * p.heads) return;
    const int64_t row = pair / p.heads;
    const int head = int(pair % p.heads);
    const int64_t li = (int64_t)head * p.rows + row;
    const int64_t oi = pair * D + sub * 4;
    float mx = -INFINITY;
#pragma unroll 4
    for (int i = 0; i < p.n; ++i) mx = fmaxf(mx, p.lse[i][li]);
    f32x4 out = {0.f, 0.f, 0.f, 0.f};
    float lnew = -INFINITY;
    if (mx != -INFINITY) {
        // weights e^(L_i - max) in (0, 1], one of them 1: the sum is >= 1
        float sum = 0.f;
#pragma unroll 4
        for (int i = 0; i < p.n; ++i) {
            const float wgt = __expf(p.lse[i][li] - mx);
            sum += wgt;
            out += *reinterpret_cast<const f32x4*>(p.o[i] + oi) * wgt;
        }
        out *= 1.f / sum;
        lnew = mx + __logf(sum);
    }
    *reinterpret_cast<f32x4*>(p.o_out + oi) = out;
    if (sub == 0) p.lse_out[li] = lnew;
}

template <int D>
__global__ __launch_bounds__(kThreads) void delta_kernel(const uint16_t* __restrict__ d_o,
                                                         const float* __restrict__ o, float* __restrict__ delta,
                                                         int64_t rows, int heads) {
    constexpr int LPG = D / 4;
    const int64_t gidx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t pair = gidx / LPG;
    const int sub = int(gidx % LPG);
    const bool live = pair < rows * heads;
    float part = 0.f;
    if (live) {
        const f32x4 ov = *reinterpret_cast<const f32x4*>(o + pair * D + sub * 4);
        const u32x2 raw = *reinterpret_cast<const u32x2*>(d_o + pair * D + sub * 4);
        const float g0 = __uint_as_float(raw.x << 16), g1 = __uint_as_float(raw.x & 0xffff0000u);
        const float g2 = __uint_as_float(raw.y << 16), g3 = __uint_as_float(raw.y & 0xffff0000u);
        part = ov.x * g0 + ov.y * g1 + ov.z * g2 + ov.w * g3;
    }
    // reduce over the LPG lanes of the group (a power of two that divides 64)
#pragma unroll
    for (int off = LPG / 2; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (live && sub == 0) {
        const int64_t row = pair / heads;
        const int head = int(pair % heads);
        delta[(int64_t)head * rows + row] = part;
    }
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" cp_status cp_merge_partials(float* o_acc, float* lse_acc, const float* o_step, const float* lse_step,
                                       int64_t rows, int32_t heads, int32_t head_dim, hipStream_t stream) {
    if (rows < 0 || heads <= 0) return fail(CP_ERR_INVALID_ARG, "bad sizes");
    if (head_dim != 64 && head_dim != 128) return fail(CP_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (rows == 0) return CP_OK;
    if (!o_acc || !lse_acc || !o_step || !lse_step) return fail(CP_ERR_INVALID_ARG, "NULL pointer");
    if (!all_aligned16({o_acc, lse_acc, o_step, lse_step}))
        return fail(CP_ERR_INVALID_ARG, "tensor pointer not 16-byte aligned");
    if (rows > (int64_t(1) << 40) / heads) return fail(CP_ERR_UNSUPPORTED, "too large");  // keeps the product in range
    const int64_t threads = rows * heads * (head_dim / 4);
    const int64_t grid = ceil_div(threads, kThreads);
    if (grid > 0x7fffffff) return fail(CP_ERR_UNSUPPORTED, "too large");
    if (head_dim == 128)
        hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, o_acc, lse_acc, o_step,
                           lse_step, rows, heads);
    else
        hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, o_acc, lse_acc, o_step,
                           lse_step, rows, heads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CP_ERR_HIP, std::string("merge launch: ") + hipGetErrorString(e));
    return CP_OK;
}

extern "C" cp_status cp_merge_partials_n(float* o_out, float* lse_out, const float* const* o_parts,
                                         const float* const* lse_parts, int32_t n_parts, int64_t rows, int32_t heads,
                                         int32_t head_dim, hipStream_t stream) {
    if (rows < 0 || heads <= 0) return fail(CP_ERR_INVALID_ARG, "bad sizes");
    if (head_dim != 64 && head_dim != 128) return fail(CP_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (n_parts < 1 || n_parts > kMaxParts)
        return fail(CP_ERR_INVALID_ARG, "n_parts must be in [1, " + std::to_string(kMaxParts) + "]");
    if (rows == 0) return CP_OK;
    if (!o_out || !lse_out || !o_parts || !lse_parts) return fail(CP_ERR_INVALID_ARG, "NULL pointer");
    MergeNParams prm = {};
    for (int i = 0; i < n_parts; ++i) {
        if (!o_parts[i] || !lse_parts[i]) return fail(CP_ERR_INVALID_ARG, "NULL part pointer");
        if (!all_aligned16({o_parts[i], lse_parts[i]}))
            return fail(CP_ERR_INVALID_ARG, "tensor pointer not 16-byte aligned");
        prm.o[i] = o_parts[i];
        prm.lse[i] = lse_parts[i];
    }
    if (!all_aligned16({o_out, lse_out})) return fail(CP_ERR_INVALID_ARG, "tensor pointer not 16-byte aligned");
    prm.o_out = o_out;
    prm.lse_out = lse_out;
    prm.rows = rows;
    prm.heads = heads;
    prm.n = n_parts;
    if (rows > (int64_t(1) << 40) / heads) return fail(CP_ERR_UNSUPPORTED, "too large");  // keeps the product in range
    const int64_t threads = rows * heads * (head_dim / 4);
    const int64_t grid = ceil_div(threads, kThreads);
    if (grid > 0x7fffffff) return fail(CP_ERR_UNSUPPORTED, "too large");
    if (head_dim == 128)
        hipLaunchKernelGGL(merge_n_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, prm);
    else
        hipLaunchKernelGGL(merge_n_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, prm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CP_ERR_HIP, std::string("merge launch: ") + hipGetErrorString(e));
    return CP_OK;
}

extern "C" cp_status cp_attn_bwd_prep(const void* d_o, const float* o, float* delta, int64_t rows, int32_t heads,
                                      int32_t head_dim, hipStream_t stream) {
    if (rows < 0 || heads <= 0) return fail(CP_ERR_INVALID_ARG, "bad sizes");
    if (head_dim != 64 && head_dim != 128) return fail(CP_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (rows == 0) return CP_OK;
    if (!d_o || !o || !delta) return fail(CP_ERR_INVALID_ARG, "NULL pointer");
    if (!all_aligned16({d_o, o, delta})) return fail(CP_ERR_INVALID_ARG, "tensor pointer not 16-byte aligned");
    if (rows > (int64_t(1) << 40) / heads) return fail(CP_ERR_UNSUPPORTED, "too large");  // keeps the product in range
    const int64_t threads = rows * heads * (head_dim / 4);
    const int64_t grid = ceil_div(threads, kThreads);
    if (grid > 0x7fffffff) return fail(CP_ERR_UNSUPPORTED, "too large");
    if (head_dim == 128)
        hipLaunchKernelGGL(delta_kernel<128>, dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(d_o), o, delta, rows, heads);
    else
        hipLaunchKernelGGL(delta_kernel<64>, dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(d_o), o, delta, rows, heads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CP_ERR_HIP, std::string("delta launch: ") + hipGetErrorString(e));
    return CP_OK;
}
