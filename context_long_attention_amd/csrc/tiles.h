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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;

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

// Pins a wave-uniform value in a scalar register as an opaque value.  Kernel
// parameters are read through it: a select between two fields of the
// parameter block can otherwise be turned into a select between their
// addresses, which forces a stack copy of the block and a memory load (with a
// full wait on the vector memory counter) at every use.
__device__ __forceinline__ int sreg(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+s"(x));
#endif
    return x;
}

// `tile + lane_off` with the lane offset opaque to the optimiser: the reads of
// one tile then share this base and carry their offsets in the 16-bit
// immediate field (folded with the buffer's absolute LDS address the constant
// can exceed 16 bits and cost one add per read).  The pointer still derives
// from the tile's own LDS object, so the compiler can tell that it does not
// alias the buffers that loads in flight are filling.
__device__ __forceinline__ lds_char* lds_base(const char* tile, int lane_off) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(lane_off));
#endif
    return (lds_char*)tile + lane_off;
}

// Marks a value as needed at this point, so that it is computed before it
// (the compiler otherwise sinks work past the step's barrier into the block
// that uses it, out of reach of the instruction interleaving).
template <typename T>
__device__ __forceinline__ void materialise(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" ::"v"(x));
#endif
}

// Pins a value to this point of the instruction stream: it is produced before
// and consumed after (the empty volatile statement is ordered with the
// others), which keeps a hand-interleaved schedule in the order written.
template <typename T>
__device__ __forceinline__ void pin(T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(x));
#endif
}

// Keeps the memory operations written before it ahead of those after it
// (loads issued early stay early), without waiting for any of them.
__device__ __forceinline__ void order_memory() {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" ::: "memory");
#endif
}

// c ? a : b on values.  A conditional between two lvalues (members of a
// lambda closure, fields of the parameter block) is emitted as a choice between
// their addresses followed by one load, which keeps both in stack memory.
template <typename T>
__device__ __forceinline__ T pick(bool c, T a, T b) {
    return c ? a : b;
}

// A half-open range [t_lo, t_hi) of tile indices.
struct SegRange {
    int t_lo, t_hi;
};

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

// Buffer descriptor over `bytes` bytes from `base` (bytes < 2^31): loads at
// byte offsets >= bytes return zero, so a descriptor over one KV segment of one
// head zero-fills the rows of a ragged last tile, and kDeadTile puts a whole
// tile out of range.
constexpr uint32_t kDeadTile = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Per-lane byte offsets, within one tile, of the rows this wave loads
// (NBLK / WAVES direct-to-LDS loads of 1 KiB each).
template <int D, int ROWS, int WAVES>
struct TileLanes {
    using L = TileLayout<D, ROWS>;
    static_assert(L::NBLK % WAVES == 0, "every wave must issue the same number of loads");
    static constexpr int N = L::NBLK / WAVES;
    uint32_t off[N];
    __device__ __forceinline__ TileLanes(int row_bytes, int wave, int lane) {
        const int j = lane % L::RB, c = lane / L::RB;
#pragma unroll
        for (int b = 0; b < N; ++b) off[b] = (uint32_t)(((wave + WAVES * b) * L::RB + j) * row_bytes + c * 16);
    }
};

// Direct-to-LDS loads of the tile that starts `tile_off` bytes into the span of `rs`.
template <int D, int ROWS, int WAVES>
__device__ __forceinline__ void load_tile_at(char* dst, __amdgpu_buffer_rsrc_t rs, const TileLanes<D, ROWS, WAVES>& tl,
                                             uint32_t tile_off, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
    using L = TileLayout<D, ROWS>;
#pragma unroll
    for (int b = 0; b < TileLanes<D, ROWS, WAVES>::N; ++b)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (wave + WAVES * b) * L::BLK), 16,
                                                 tl.off[b] + tile_off, 0, 0, 0);
#endif
}

// Maximum over the two half-waves (lanes l and l ^ 32), without LDS.
__device__ __forceinline__ float max_halves(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
#else
    return x;
#endif
}

// First and one-past-last tile (of BN keys, within a segment [kpos0, kpos0 + klen))
// whose every pair is visible to every row of the query tile [q0, ...]: keys at
// or before q0, at or after lo1 (the document start of the tile's last row, 0
// without documents), and not the ragged last tile.
template <int BN>
__device__ __forceinline__ SegRange full_tile_range(int mask, int q0, int lo1, int kpos0, int klen) {
    const int whole = klen / BN;
    if (mask == CP_MASK_SKIP) return {0, 0};
    if (mask == CP_MASK_FULL) return {0, whole};
    const int d = q0 - kpos0 - (BN - 1);
    const int hi = (d < 0) ? 0 : min(whole, d / BN + 1);
    const int lo = (lo1 > kpos0) ? (lo1 - kpos0 + BN - 1) / BN : 0;
    return {lo, max(lo, hi)};
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
