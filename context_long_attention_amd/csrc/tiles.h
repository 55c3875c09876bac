// Device-side helpers shared by the attention step kernels (gfx950): vector
// types, the LDS tile layout filled by direct buffer-to-LDS loads, block-sparse
// tile ranges, and the document lookup.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace cpattn {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Index (within a 64-row block of two 32x32 MFMA tiles) of the row held by
// accumulator register r = 4i + j of block kb in half hl of the wave: the
// 32x32 MFMA output row 8i + 4hl + j.  Registers 8(s%2)..8(s%2)+7 of block s/2
// then hold rows 16s + 4hl + {0..3, 8..11}: as a B operand whose k-slots are
// those rows, they pair with two transposing reads of the same rows.
__device__ __forceinline__ int row_of_reg(int kb, int r, int hl) {
    return 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
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

// LDS tile layout of ROWS rows x D bf16 columns.  One direct buffer-to-LDS load
// per wave moves 1 KiB (64 lanes x 16 B, lane i landing at base + 16 i); that
// KiB holds RB = 1024 / (2D) consecutive rows, stored chunk-major: (row j,
// 16-byte chunk c) at 16 (RB c + j).  Blocks are BLK bytes apart; the padding
// makes 16-byte operand reads of 16 consecutive rows, and transposing reads of
// a 4 x 16 block, hit distinct banks.  Every operand address is a per-lane base
// plus an immediate.
template <int D, int ROWS>
struct TileLayout {
    static constexpr int RB = 1024 / (2 * D);
    static constexpr int BLK = 1024 + (D == 128 ? 64 : 128);
    static constexpr int NBLK = ROWS / RB;
    static constexpr int BYTES = NBLK * BLK;
    static __device__ __forceinline__ int off(int row, int col) {
        return (row / RB) * BLK + 16 * (RB * (col / 8) + row % RB) + 2 * (col % 8);
    }
};

// Buffer descriptor over rows [0, rows) of one head of a [rows, H, D] bf16
// tensor starting at `base`: reads of later rows return zero (rows = 0 gives a
// descriptor whose loads fetch nothing and write zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int rows, int row_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, rows * row_bytes, 0x00020000);
}

// Direct-to-LDS loads of one tile: this wave's NBLK / WAVES blocks.
template <int D, int ROWS, int WAVES>
__device__ __forceinline__ void load_tile_lds(char* dst, __amdgpu_buffer_rsrc_t rs, int row_bytes, int wave,
                                              int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
    using L = TileLayout<D, ROWS>;
    static_assert(L::NBLK % WAVES == 0, "every wave must issue the same number of loads");
    const int j = lane % L::RB, c = lane / L::RB;
#pragma unroll
    for (int b = 0; b < L::NBLK / WAVES; ++b) {
        const int blk = wave + WAVES * b;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + blk * L::BLK), 16,
                                                 (blk * L::RB + j) * row_bytes + c * 16, 0, 0, 0);
    }
#endif
}

// One 4-byte value per lane, straight into LDS (lane i at base + 4 i).
__device__ __forceinline__ void load_dwords_lds(char* dst, __amdgpu_buffer_rsrc_t rs, int byte_off) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 4, byte_off, 0, 0, 0);
#endif
}

// Wait until at most `pending` of this wave's vector memory operations are in
// flight and every LDS/scalar access has completed, then synchronise the
// workgroup (s_waitcnt: vmcnt bits 3:0 and 15:14, expcnt 6:4 = 7 (no wait),
// lgkmcnt 11:8 = 0).
template <int PENDING>
__device__ __forceinline__ void ring_barrier() {
    static_assert(PENDING < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((PENDING & 15) | ((PENDING >> 4) << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();
}

struct SegRange {
    int t_lo, t_hi;
};

// Key tiles of one KV segment [kpos0, kpos0 + klen) that a query tile [q0, q1]
// (global positions, q1 its last row) can see.  lo0 is the first visible key of
// row q0 (document start for DOC masks, 0 otherwise).  Visible keys of the
// tile's rows form [lo0, q1]: lo is non-decreasing in q and lo(q) <= q, so the
// per-row ranges [lo(q), q] chain without gaps.  Mirror of the host rule.
template <int BN>
__device__ __forceinline__ SegRange key_tile_range(int mask, int q0, int q1, int lo0, int kpos0, int klen) {
    const int nkt = (klen + BN - 1) / BN;
    if (mask == CP_MASK_SKIP || klen == 0) return {0, 0};
    if (mask == CP_MASK_FULL) return {0, nkt};
    const int t_hi = (q1 < kpos0) ? 0 : min(nkt, (q1 - kpos0) / BN + 1);
    int t_lo = 0;
    if (lo0 > kpos0) {
        if (lo0 > kpos0 + klen - 1) return {0, 0};
        t_lo = (lo0 - kpos0) / BN;
    }
    if (t_lo >= t_hi) return {0, 0};
    return {t_lo, t_hi};
}

// Every pair of the tile visible: the last row's document starts at or before
// the first key (lo1 <= k0) and the last key is at or before the first row.
template <int BN>
__device__ __forceinline__ bool key_tile_full(int mask, int q0, int lo1, int kpos0, int klen, int t) {
    if (mask == CP_MASK_FULL) return true;
    const int k0 = kpos0 + t * BN;
    const int k1 = min(kpos0 + klen, k0 + BN) - 1;
    return k1 <= q0 && k0 >= lo1;
}

}  // namespace dev
}  // namespace cpattn
