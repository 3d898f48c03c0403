// attn_tile.h -- pieces shared by the tiled threshold-attention kernels
// (Threshold Rectified Attention and Threshold Differential Attention): the
// ReLU-power weight, the workgroup -> (head, query tile) order, the LDS tile
// swizzle and the HBM -> LDS staging.  Internal to the library.
#pragma once

#include "attn_internal.h"

namespace attn {

// kPowThreeHalves: p = 1.5 exactly, max(x, 0)^1.5 = r * sqrt(r) with one square root
// instead of a log and an exp (the same value up to rounding).
enum PowMode { kPowGeneral = 0, kPowOne = 1, kPowTwo = 2, kPowThreeHalves = 3 };

// The kernel instantiation for a power p: exact forms for p = 1, 2 and 1.5, else exp2/log2.
inline int pow_mode(float p) {
    return p == 1.0f ? kPowOne : p == 2.0f ? kPowTwo : p == 1.5f ? kPowThreeHalves : kPowGeneral;
}

template <int PM>
__device__ __forceinline__ float relu_pow(float x, float p) {
    if constexpr (PM == kPowOne) {
        return fmaxf(x, 0.0f);
    } else if constexpr (PM == kPowTwo) {
        const float r = fmaxf(x, 0.0f);
        return r * r;
    } else if constexpr (PM == kPowThreeHalves) {
        const float r = fmaxf(x, 0.0f);
        return r * __builtin_amdgcn_sqrtf(r);
    } else {
        // x^p = 2^(p log2 x) for x > 0 (v_log_f32 / v_exp_f32 are base 2).  For x <= 0
        // (and the -inf of masked keys) max(x, 0) = 0, log2(0) = -inf and, as p > 0,
        // 2^(p * -inf) = 0 exactly: no compare and select.
        return __builtin_amdgcn_exp2f(p * __builtin_amdgcn_logf(fmaxf(x, 0.0f)));
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

// s_waitcnt with only vmcnt = n (expcnt and lgkmcnt at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

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

// The same for 4 bytes per lane, to lds + 4 * lane.
__device__ __forceinline__ void dma4(u32x4 rsrc, void *lds, int voff, int soff) {
    const uint32_t m0v = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

// Eight transposing LDS reads (ds_read_b64_tr_b16): r[2k] at LDS byte address
// addr[k], r[2k+1] at addr[k] + OFF, in one statement that first waits until at most
// VM of this wave's memory instructions are outstanding (s_waitcnt vmcnt(VM)) and
// ends with lgkmcnt(0).  For a tile that arrived by LDS DMA this awaits exactly that
// transfer (VM = the memory instructions issued after it), with nothing scheduled
// between the wait and the reads, and the results are complete when the statement
// ends.  The compiler sees no LDS read here, so it adds no wait of its own for the
// DMA (which would be vmcnt(0): it cannot tell the tiles apart, and that would also
// drain the loads of the next chunk).
template <int VM, int OFF>
__device__ __forceinline__ void tr_read4x2(bf16x4_t (&r)[8], const uint32_t (&addr)[4]) {
    static_assert(VM >= 0 && VM < 64 && OFF >= 0 && OFF < 65536, "immediates");
    asm volatile(
        "s_waitcnt vmcnt(%12)\n\t"
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %2, %9\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %11\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "n"(VM), "n"(OFF)
        : "memory");
}

// Eight 16-byte LDS reads (ds_read_b128): r[2k] at LDS byte address addr[k], r[2k+1]
// at addr[k] + OFF, after s_waitcnt vmcnt(VM) and ending with lgkmcnt(0), in one
// statement (as tr_read4x2, for row-major operand reads of a DMA'd tile).
template <int VM, int OFF>
__device__ __forceinline__ void row_read4x2(u32x4 (&r)[8], const uint32_t (&addr)[4]) {
    static_assert(VM >= 0 && VM < 64 && OFF >= 0 && OFF < 65536, "immediates");
    asm volatile(
        "s_waitcnt vmcnt(%12)\n\t"
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:%13\n\t"
        "ds_read_b128 %2, %9\n\t"
        "ds_read_b128 %3, %9 offset:%13\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %10 offset:%13\n\t"
        "ds_read_b128 %6, %11\n\t"
        "ds_read_b128 %7, %11 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "n"(VM), "n"(OFF)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}
#pragma clang diagnostic pop


}  // namespace attn
