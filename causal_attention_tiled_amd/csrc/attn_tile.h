// attn_tile.h -- pieces shared by the tiled threshold-attention kernels
// (Threshold Rectified Attention and Threshold Differential Attention): the
// ReLU-power weight, the workgroup -> (head, query tile) order, the LDS tile
// swizzle and the HBM -> LDS staging.  Internal to the library.
#pragma once

#include "attn_internal.h"

namespace attn {

enum PowMode { kPowGeneral = 0, kPowOne = 1, kPowTwo = 2 };

template <int PM>
__device__ __forceinline__ float relu_pow(float x, float p) {
    if constexpr (PM == kPowOne) {
        return fmaxf(x, 0.0f);
    } else if constexpr (PM == kPowTwo) {
        const float r = fmaxf(x, 0.0f);
        return r * r;
    } else {
        // x^p = 2^(p log2 x) for x > 0 (v_log_f32 / v_exp_f32 are base 2).
        return x > 0.0f ? __builtin_amdgcn_exp2f(p * __builtin_amdgcn_logf(x)) : 0.0f;
    }
}

// Workgroup id -> (head slab, query tile).  Heavy tiles first; with BH % 8 == 0
// the heads are split into 8 contiguous ranges, one per XCD (workgroup ids are
// dealt to XCDs round-robin, so id % 8 names the XCD).
__device__ __forceinline__ void tile_order(int bid, int BH, int nqt, int &bh, int &qt) {
    if ((BH & 7) == 0) {
        const int xcd = bid & 7, s = bid >> 3, hpx = BH >> 3;
        bh = xcd * hpx + s % hpx;
        qt = nqt - 1 - s / hpx;
    } else {
        bh = bid % BH;
        qt = nqt - 1 - bid / BH;
    }
}

// LDS tile layout (K and V alike): row-major [key][dim], D*2 bytes per row, no
// padding; the 16-byte chunk c of row r sits in chunk slot c ^ tile_swz<D>(r).  The
// LDS has 64 four-byte banks (256 bytes per cycle).  With this swizzle the 16 rows
// that 16 consecutive lanes read for the K operand (ds_read_b128), and the 4 rows x
// 64 bytes that 32 lanes read for the V operand (ds_read_b64_tr_b16), each cover
// all 64 banks once.
template <int D>
__device__ __forceinline__ int tile_swz(int row) {
    if constexpr (D == 128)  // one row per bank line, 16 chunk slots
        return ((row & 3) << 2) | ((row >> 2) & 3);
    else                     // two 128-byte rows per bank line, 8 chunk slots
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;

// Raw buffer resource (gfx9 layout) over `bytes` bytes at `base`, held in scalar
// registers; loads past the end return 0.
__device__ __forceinline__ u32x4 make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    u32x4 r = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu), bytes,
               0x00020000u};
    return r;
}

// 16 bytes per lane from global memory (resource + voff + soff) straight into LDS at
// lds + 16 * lane.  Issued as inline assembly so that the compiler does not add its
// own (conservative) waits for it before unrelated LDS reads: completion is awaited
// explicitly, with s_waitcnt vmcnt, before the barrier that publishes the tile.
// M0 carries the LDS address and is set here for each transfer.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(u32x4 rsrc, void *lds, int voff, int soff) {
    const uint32_t m0v = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop


}  // namespace attn
