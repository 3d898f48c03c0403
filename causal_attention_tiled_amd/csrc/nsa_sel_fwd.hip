// nsa_sel_fwd.hip -- NSA selection-branch forward for gfx950 (query-outer gather).
//
// Definition (msb-msb/openbox-llm, page "nsa_selection_kernel.py": module docstring,
// `selection_forward_reference`, `_selection_fwd_kernel`): for query i of head h in
// GQA group kv = h / G, softmax attention with scale D^-0.5 over the union of the
// tokens j <= i of the blocks listed in block_idx[b, kv, i, :]; negative slots are
// padding, a repeated block counts once, an empty selection yields out = 0 and the
// lse sentinel -1e9.
//
// Design:
//  * One wavefront per (b, kv group, query i); a workgroup holds 4 consecutive
//    queries of one group.  The G query heads of the group are packed into the N
//    dimension of v_mfma_f32_16x16x32_bf16, so every gathered K/V tile is read once
//    per group, not once per head.
//  * The wave walks the S slots of its block_idx row (wave-uniform scalar loads),
//    skipping padding, blocks past T/bs, blocks entirely after i and repeats of an
//    earlier slot.  No scan over the KV sequence takes place.
//  * Scores are computed transposed, S^T = K Q^T: K streams straight from global
//    memory into the A operand (16 keys x 32 dims per MFMA), Q^T sits in registers.
//    Each lane then holds ONE head (lane % 16) and 16 keys, so the online-softmax
//    state (running max, partial sum, output rescale) is per-lane scalar work plus a
//    two-step cross-lane max.
//  * The exponentials (base 2, scale*log2e folded in) are rounded to bf16 and, in
//    accumulator register order, form the B operand of O^T += V^T P^T.  V^T comes
//    from a per-wave LDS tile written transposed from the gathered V rows; the key
//    order implied by the accumulator layout is folded into that LDS layout.
//  * Workgroup order keeps each XCD on a contiguous range of (group, query) work so a
//    group's K/V stays in one XCD's L2.
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// V^T chunk in LDS: row = head dim, column = key position within a chunk of KC keys.
// In every 32-key group the key offset o = 16a + 4g + j is stored at 8g + 4a + j, so
// that the 8 keys a lane feeds to one 16x16x32 MFMA are contiguous.  4-key units are
// XOR-swizzled by an even, row-dependent amount to spread the transposing writes.
__device__ __forceinline__ int nsa_vt_pos(int o) {
    return (o & ~31) | (((o >> 2) & 3) << 3) | (((o >> 4) & 1) << 2) | (o & 3);
}
template <int NU>
__device__ __forceinline__ int nsa_vt_offset(int row, int pos, int stride) {
    const int unit = (pos >> 2) ^ ((row >> 2) & (NU - 2));
    return row * stride + (unit << 2) + (pos & 3);
}

template <int D, int BS>
__global__ __launch_bounds__(kThreads) void nsa_sel_fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ IDX, uint16_t *__restrict__ O,
    float *__restrict__ LSE, int Hq, int Hkv, int G, int T, int S, int nq4, int ngroups,
    float score_scale) {
    constexpr int KC = BS < 64 ? BS : 64;  // keys per processed chunk
    constexpr int NCH = BS / KC;           // chunks per selected block
    constexpr int NKK = KC / 16;           // 16-key sub-tiles (S^T MFMA rows)
    constexpr int NPV = KC / 32;           // 32-key PV steps
    constexpr int NDS = D / 32;            // S^T MFMA k-steps
    constexpr int NDT = D / 16;            // 16-dim output tiles
    constexpr int VSTR = KC + 8;           // V^T row stride (elements)
    constexpr int NU = KC / 4;             // 4-key units per V^T row
    constexpr int DC = D / 8;              // 16-byte chunks per row
    constexpr int VPL = (KC / 4) * DC / 64;  // 4-key x 8-dim V blocks per lane
    static_assert(VPL >= 1 && (KC / 4) * DC % 64 == 0, "V blocks must tile the wave");

    __shared__ __attribute__((aligned(16))) uint16_t Vs[kWaves][D * VSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;

    // workgroup -> (group, query quad); each XCD takes one contiguous range
    const int W = ngroups * nq4;
    int f = blockIdx.x;
    if ((W & 7) == 0) f = (blockIdx.x & 7) * (W >> 3) + (blockIdx.x >> 3);
    const int group = f / nq4;
    const int i = (nq4 - 1 - f % nq4) * kWaves + wave;  // later (busier) queries first
    if (i >= T) return;  // no workgroup-wide barrier in this kernel
    const int b = group / Hkv, kv = group % Hkv;
    const size_t kvslab = (size_t)group * T * D;
    const int32_t *slots = IDX + ((size_t)group * T + i) * S;
    uint16_t *vts = Vs[wave];

    // Q^T operand: head kv*G + n16 (zero for n16 >= G), dims 32*ds + 8*g4 .. +7
    const bool head_ok = n16 < G;
    const size_t qrow = ((size_t)(b * Hq + kv * G + (head_ok ? n16 : 0)) * T + i) * D;
    bf16x8 qf[NDS];
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            u32x4 r = z;
            if (head_ok) r = *(const u32x4 *)(Q + qrow + ds * 32 + g4 * 8);
            qf[ds] = as_bf16x8(r);
        }
    }

    float m = -INFINITY;  // running max of the base-2 scores (this lane's head)
    float lsum = 0.0f;    // this lane's share of the running sum
    f32x4 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nblk = T / BS;
    for (int s = 0; s < S; ++s) {
        const int blk = slots[s];
        if (blk < 0 || blk >= nblk || blk * BS > i) continue;
        bool dup = false;
        for (int s2 = 0; s2 < s; ++s2) dup |= (slots[s2] == blk);
        if (dup) continue;

#pragma unroll 1
        for (int ch = 0; ch < NCH; ++ch) {
            const int k0 = blk * BS + ch * KC;
            if (k0 > i) break;
            const int nvalid = min(KC, i - k0 + 1);  // keys k0 .. k0+nvalid-1 are causal

            // gather K (MFMA A operand, straight from global) and V (rows, for LDS)
            u32x4 kf[NKK][NDS];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds)
                    kf[kk][ds] = *(const u32x4 *)(K + kvslab + (size_t)(k0 + kk * 16 + n16) * D +
                                                  ds * 32 + g4 * 8);
            u32x4 vr[VPL][4];
#pragma unroll
            for (int r = 0; r < VPL; ++r) {
                const int blkid = lane + 64 * r;
                const int kg = blkid / DC, dc = blkid % DC;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    vr[r][e] = *(const u32x4 *)(V + kvslab + (size_t)(k0 + kg * 4 + e) * D + dc * 8);
            }

            // S^T = K Q^T : register j of st[kk] is key k0 + 16*kk + 4*g4 + j, head n16
            f32x4 st[NKK];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                st[kk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds)
                    st[kk] = mfma_16x16x32(as_bf16x8(kf[kk][ds]), qf[ds], st[kk]);
            }
            float mloc = -INFINITY;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float t = st[kk][j] * score_scale;
                    if (kk * 16 + g4 * 4 + j >= nvalid) t = -INFINITY;
                    st[kk][j] = t;
                    mloc = fmaxf(mloc, t);
                }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
            const float mnew = fmaxf(m, mloc);  // finite: key k0 is always causal
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);
            m = mnew;
            float psum = 0.0f;
            bf16x8 pf[NPV];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float e = __builtin_amdgcn_exp2f(st[kk][j] - mnew);
                    psum += e;
                    pf[kk >> 1][(kk & 1) * 4 + j] = (__bf16)e;
                }
            lsum = lsum * alpha + psum;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;

            // V rows -> V^T in this wave's LDS tile (after every lane has finished
            // reading the previous chunk)
            wave_lds_sync();
#pragma unroll
            for (int r = 0; r < VPL; ++r) {
                const int blkid = lane + 64 * r;
                const int kg = blkid / DC, dc = blkid % DC;
                const int pos = nsa_vt_pos(kg * 4);
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    const int w = d >> 1;
                    uint32_t lo, hi2;
                    if (d & 1) {
                        lo = (vr[r][0][w] >> 16) | (vr[r][1][w] & 0xffff0000u);
                        hi2 = (vr[r][2][w] >> 16) | (vr[r][3][w] & 0xffff0000u);
                    } else {
                        lo = (vr[r][0][w] & 0xffffu) | (vr[r][1][w] << 16);
                        hi2 = (vr[r][2][w] & 0xffffu) | (vr[r][3][w] << 16);
                    }
                    const u32x2 pr = {lo, hi2};
                    *(u32x2 *)(&vts[nsa_vt_offset<NU>(dc * 8 + d, pos, VSTR)]) = pr;
                }
            }
            wave_lds_sync();

            // O^T += V^T P^T : register j of oacc[dt] is dim 16*dt + 4*g4 + j, head n16
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int c = 0; c < NPV; ++c) {
                    const bf16x8 a = *(const bf16x8 *)(&vts[nsa_vt_offset<NU>(
                        dt * 16 + n16, c * 32 + g4 * 8, VSTR)]);
                    oacc[dt] = mfma_16x16x32(a, pf[c], oacc[dt]);
                }
        }
    }

    // finalize: total sum of this head over its 4 lanes
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (head_ok) {
        const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
        uint16_t *orow = O + qrow;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const u32x2 pr = {pack_bf16x2(oacc[dt][0] * inv, oacc[dt][1] * inv),
                              pack_bf16x2(oacc[dt][2] * inv, oacc[dt][3] * inv)};
            *(u32x2 *)(orow + dt * 16 + g4 * 4) = pr;
        }
        if (LSE != nullptr && g4 == 0)
            LSE[(size_t)(b * Hq + kv * G + n16) * T + i] =
                lsum > 0.0f ? (m + __builtin_amdgcn_logf(lsum)) * kLn2 : -1e9f;
    }
}

template <int D, int BS>
hipError_t launch(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *idx,
                  uint16_t *out, float *lse, int B, int Hq, int Hkv, int T, int S,
                  hipStream_t stream) {
    int G = Hq / Hkv;
    int nq4 = (T + kWaves - 1) / kWaves;
    int ngroups = B * Hkv;
    float score_scale = kLog2e / sqrtf((float)D);
    void *args[] = {&q, &k, &v, &idx, &out, &lse, &Hq, &Hkv, &G, &T, &S, &nq4, &ngroups,
                    &score_scale};
    return hipLaunchKernel((const void *)nsa_sel_fwd_kernel<D, BS>,
                           dim3((unsigned)(ngroups * nq4)), dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_nsa_sel_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *block_idx, uint16_t *out, float *lse, int B,
                              int Hq, int Hkv, int T, int D, int block_size, int S,
                              hipStream_t stream) {
#define ATTN_NSA_CASE(DD, BB)                                                                \
    if (D == DD && block_size == BB)                                                        \
        return launch<DD, BB>(q, k, v, block_idx, out, lse, B, Hq, Hkv, T, S, stream);
    ATTN_NSA_CASE(128, 64)
    ATTN_NSA_CASE(128, 32)
    ATTN_NSA_CASE(128, 128)
    ATTN_NSA_CASE(64, 64)
    ATTN_NSA_CASE(64, 32)
    ATTN_NSA_CASE(64, 128)
#undef ATTN_NSA_CASE
    return hipErrorInvalidValue;
}

}  // namespace attn
