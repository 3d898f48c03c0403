// attn_internal.h -- types and helpers shared by the gfx950 kernels of libattn.so.
// Internal to the library; the public C ABI is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand lanes: A[m = lane%32][k = 8*(lane/32)+t],
// B[k = 8*(lane/32)+t][n = lane%32], t = 0..7.  Accumulator: C[m][n] with n = lane%32,
// m = 8*(r/4) + 4*(lane/32) + r%4 for register r = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA, fp32 accumulate.  Operand lanes: A[m = lane%16][k = 8*(lane/16)+t],
// B[k = 8*(lane/16)+t][n = lane%16].  Accumulator: C[m][n] with n = lane%16,
// m = 4*(lane/16) + r for register r = 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Order LDS traffic between the lanes of one wavefront (a write by one lane
// that another lane of the same wave reads next).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Query rows per workgroup of the bf16 / fp32 Threshold Rectified Attention kernels
// (bf16: 32 rows per wavefront; 8 wavefronts at D = 128, 4 at D = 64).
constexpr int tra_bf16_waves(int D) { return D == 128 ? 8 : 4; }
constexpr int tra_bf16_rows(int D) { return 32 * tra_bf16_waves(D); }
constexpr int kTraF32Rows = 8;
// Query rows per workgroup of the Threshold Differential Attention kernel.
constexpr int kTdaRows = 256;
// Key rows per workgroup of the Threshold Rectified Attention backward's dk/dv kernels
// (64 keys per wave at D = 128, 32 at D = 64; four waves).  The dq kernel's workgroups
// take as many query rows, so this also sizes the larger of the two grids.
constexpr int tra_bwd_dkv_rows(int D) { return D == 128 ? 256 : 128; }

// Host-side launchers (one per kernel family); they pick the template
// instance and return the HIP launch status.
hipError_t launch_tra_fwd_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               uint16_t *out, int BH, int T, int D, float beta, float p,
                               hipStream_t stream);
hipError_t launch_tra_fwd_f32(const float *q, const float *k, const float *v, float *out,
                              int BH, int T, int D, float beta, float p, hipStream_t stream);
hipError_t launch_tra_bwd_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const uint16_t *dout, uint16_t *dq, uint16_t *dk, uint16_t *dv,
                               int BH, int T, int D, float beta, float p, hipStream_t stream);
hipError_t launch_nsa_sel_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *block_idx, const uint16_t *out, const float *lse,
                              const uint16_t *dout, uint16_t *dq, uint16_t *dk, uint16_t *dv,
                              void *workspace, int B, int Hq, int Hkv, int T, int D,
                              int block_size, int S, hipStream_t stream);
// Workspace bytes of the NSA selection backward (block lists, per-row delta).
size_t nsa_sel_bwd_workspace(int B, int Hq, int Hkv, int T, int D, int block_size, int S);

// Inverted NSA selection (nsa_index.hip): per list (group * nblk + block) the
// increasing positions of the queries attending the block, list offsets, per-word
// ranks, and segments of at most kNsaSegQ queries.  pairs bounds the total list length,
// max_segs the segments, max_part the segments of lists longer than kNsaSegQ.
size_t nsa_sel_fsa_workspace(int B, int Hq, int Hkv, int T, int D, int block_size, int S);
hipError_t launch_nsa_sel_fsa(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *block_idx, uint16_t *out, float *lse,
                              void *workspace, int B, int Hq, int Hkv, int T, int D,
                              int block_size, int S, hipStream_t stream);

constexpr int kNsaSegQ = 512;
struct NsaIndex {
    uint32_t *bits;
    int32_t *rank, *counts, *offsets, *list, *nseg, *npart, *seg_start, *part_start, *seg_list;
    int nblk, words;
    int64_t nlists, pairs, max_segs, max_part;
};
// Pointers into ws (256-byte aligned, ws may be null to size only); *bytes = bytes used.
NsaIndex nsa_index_carve(void *ws, int B, int Hkv, int T, int bs, int S, size_t *bytes);
hipError_t nsa_index_build(const NsaIndex &ix, const int32_t *block_idx, int B, int Hkv, int T,
                           int bs, int S, hipStream_t stream);
hipError_t launch_tda_fwd_bf16(const uint16_t *q1, const uint16_t *q2, const uint16_t *k1,
                               const uint16_t *k2, const uint16_t *v, uint16_t *out,
                               uint16_t *workspace, int BH, int T, int D, float beta,
                               float lam, float p, int normalize, hipStream_t stream);
hipError_t launch_nsa_sel_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *block_idx, uint16_t *out, float *lse, int B,
                              int Hq, int Hkv, int T, int D, int block_size, int S,
                              hipStream_t stream);

}  // namespace attn
