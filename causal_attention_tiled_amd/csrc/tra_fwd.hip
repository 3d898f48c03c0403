// tra_fwd.hip -- Threshold Rectified Attention forward for gfx950.
//
// Definition (snap-research/TDA, page "triton_threshold_attention.py", module
// docstring and `_threshold_rela_fwd_kernel`):
//     out_i = sum_{j <= i} max(q_i . k_j - tau_i, 0)^p v_j,   tau_i = beta*sqrt(2 ln(i+1) / D)
// with a 0-based query position i, natural log, no 1/sqrt(D) scale and no softmax.
//
// bf16 kernel design (one workgroup = 4 wavefronts = 128 query rows of one (b,h)):
//  * Each wave owns 32 query rows.  It computes the TRANSPOSED score tile
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16, K (A operand) from LDS, Q (B operand)
//    held in registers for the whole key loop.  In the accumulator every lane then
//    holds ONE query (lane % 32) and 16 keys, so tau_i is a per-lane scalar and the
//    causal test is a per-lane compare.
//  * The epilogue (threshold, ReLU, power, causal mask) runs on those registers and
//    rounds the weights to bf16; the register order of the accumulator directly forms
//    the B operand of O^T += V^T P^T (again 32x32x16), so P never touches LDS.  The
//    key order this implies is absorbed into the V^T layout in LDS.
//  * K and V tiles of 64 keys are double-buffered through LDS: the next tile's global
//    loads are issued before the current tile's MFMAs and written to the other buffer
//    afterwards (one barrier per tile).  V is transposed on its way into LDS.
//  * Causal tile skipping: key tiles past the workgroup's last query are never loaded;
//    32-key sub-tiles past a wave's last query are skipped by that wave; the mask is
//    evaluated only on sub-tiles that straddle the diagonal.
//  * Launch order: the heaviest query tiles (largest i) first, and the heads split
//    into 8 contiguous groups so that each XCD (dispatch is round-robin over the 8
//    XCDs) works on its own heads and keeps their K/V in its private L2.
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per LDS tile

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
__device__ __forceinline__ void tra_tile_of(int bid, int BH, int nqt, int &bh, int &qt) {
    if ((BH & 7) == 0) {
        const int xcd = bid & 7, s = bid >> 3, hpx = BH >> 3;
        bh = xcd * hpx + s % hpx;
        qt = nqt - 1 - s / hpx;
    } else {
        bh = bid % BH;
        qt = nqt - 1 - bid / BH;
    }
}

// V^T tile in LDS: row = head dim d (D rows), column = key position in the tile.
// Within each 16-key group the key offset o = 8a + 4b + c is stored at 8b + 4a + c
// (bits 2 and 3 swapped) so that a lane's 8 MFMA k-values are 16 contiguous bytes.
// The 4-key units of a row are XOR-swizzled by an even amount that depends on the
// row, which spreads the transposing writes over the banks and keeps 8-key reads
// contiguous.
__device__ __forceinline__ int vt_pos_of_key(int o) {
    return (o & ~15) | ((o & 4) << 1) | ((o & 8) >> 1) | (o & 3);
}
__device__ __forceinline__ int vt_offset(int row, int pos, int stride) {
    const int unit = (pos >> 2) ^ ((row >> 2) & 14);  // even XOR < 16 units per row
    return row * stride + (unit << 2) + (pos & 3);
}

template <int D, int PM>
__global__ __launch_bounds__(kThreads) void tra_fwd_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, int BH, int T, int nqt,
    float beta, float p) {
    constexpr int KSTR = D + 8;    // K row stride in LDS (elements): 16 B of padding
    constexpr int VSTR = kBN + 8;  // V^T row stride in LDS (elements)
    constexpr int DC = D / 8;      // 16-byte chunks per head-dim row
    constexpr int KLOADS = kBN * DC / kThreads;
    constexpr int VBLK = (kBN / 4) * DC;  // 4-key x 8-dim blocks per tile
    constexpr int NDS = D / 16;           // MFMA k-steps for S^T
    constexpr int NDT = D / 32;           // 32-dim output tiles
    static_assert(VBLK <= kThreads, "one V block per thread");

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][D * VSTR];

    int bh, qt;
    tra_tile_of(blockIdx.x, BH, nqt, bh, qt);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const size_t slab = (size_t)bh * T * D;
    const uint16_t *Kg = K + slab;
    const uint16_t *Vg = V + slab;

    const int q0 = qt * kBM;
    const int qw0 = q0 + wave * 32;
    const int my_q = qw0 + l32;
    const bool wave_active = qw0 < T;
    const int wave_last = min(qw0 + 31, T - 1);
    const int q_last = min(q0 + kBM, T) - 1;
    const int ntiles = q_last / kBN + 1;

    // Q^T operand: this lane's query, dims 16*ds + 8*hi .. +7.
    bf16x8 qf[NDS];
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            u32x4 r = z;
            if (my_q < T) r = *(const u32x4 *)(Q + slab + (size_t)my_q * D + ds * 16 + hi * 8);
            qf[ds] = as_bf16x8(r);
        }
    }
    const float tau = beta * sqrtf(2.0f * logf((float)(my_q + 1)) / (float)D);

    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;

    u32x4 kr[KLOADS];
    u32x4 vr[4];
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    auto gload = [&](int n) {
        const int k0 = n * kBN;
#pragma unroll
        for (int r = 0; r < KLOADS; ++r) {
            const int c = tid + r * kThreads;
            const int key = k0 + c / DC;
            kr[r] = key < T ? *(const u32x4 *)(Kg + (size_t)key * D + (c % DC) * 8) : zero4;
        }
        if (tid < VBLK) {
            const int kg = tid / DC, dc = tid % DC;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + kg * 4 + r;
                vr[r] = key < T ? *(const u32x4 *)(Vg + (size_t)key * D + dc * 8) : zero4;
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int r = 0; r < KLOADS; ++r) {
            const int c = tid + r * kThreads;
            *(u32x4 *)(&Ks[buf][(c / DC) * KSTR + (c % DC) * 8]) = kr[r];
        }
        if (tid < VBLK) {
            const int kg = tid / DC, dc = tid % DC;
            const int pos = vt_pos_of_key(kg * 4);
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const int w = d >> 1;
                uint32_t lo, hi2;
                if (d & 1) {
                    lo = (vr[0][w] >> 16) | (vr[1][w] & 0xffff0000u);
                    hi2 = (vr[2][w] >> 16) | (vr[3][w] & 0xffff0000u);
                } else {
                    lo = (vr[0][w] & 0xffffu) | (vr[1][w] << 16);
                    hi2 = (vr[2][w] & 0xffffu) | (vr[3][w] << 16);
                }
                const u32x2 pr = {lo, hi2};
                *(u32x2 *)(&Vs[buf][vt_offset(dc * 8 + d, pos, VSTR)]) = pr;
            }
        }
    };

    gload(0);
    sstore(0);
    __syncthreads();

    for (int n = 0; n < ntiles; ++n) {
        const int buf = n & 1;
        if (n + 1 < ntiles) gload(n + 1);
        if (wave_active) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int kbase = n * kBN + kb * 32;
                if (kbase <= wave_last) {
                    f32x16 s;
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
                    for (int ds = 0; ds < NDS; ++ds) {
                        const bf16x8 a = *(const bf16x8 *)(&Ks[buf][(kb * 32 + l32) * KSTR +
                                                                   ds * 16 + hi * 8]);
                        s = mfma_32x32x16(a, qf[ds], s);
                    }
                    // epilogue: S^T register r holds key kbase + 8*(r/4) + 4*hi + r%4
                    const bool diag = kbase + 31 > qw0;
                    bf16x8 pf[2];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float w = relu_pow<PM>(s[r] - tau, p);
                        if (diag) {
                            const int key = kbase + 8 * (r >> 2) + 4 * hi + (r & 3);
                            if (key > my_q) w = 0.0f;
                        }
                        pf[r >> 3][r & 7] = (__bf16)w;
                    }
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        const int row = dt * 32 + l32;
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            const int pos = kb * 32 + c * 16 + hi * 8;
                            const bf16x8 a =
                                *(const bf16x8 *)(&Vs[buf][vt_offset(row, pos, VSTR)]);
                            oacc[dt] = mfma_32x32x16(a, pf[c], oacc[dt]);
                        }
                    }
                }
            }
        }
        if (n + 1 < ntiles) sstore(buf ^ 1);
        __syncthreads();
    }

    // O^T accumulator: lane holds query my_q, dims 32*dt + 8*i + 4*hi + j.
    if (my_q < T) {
        uint16_t *orow = O + slab + (size_t)my_q * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x2 pr = {pack_bf16x2(oacc[dt][4 * i], oacc[dt][4 * i + 1]),
                                  pack_bf16x2(oacc[dt][4 * i + 2], oacc[dt][4 * i + 3])};
                *(u32x2 *)(orow + dt * 32 + 8 * i + 4 * hi) = pr;
            }
    }
}

// fp32 kernel: 64 query rows per workgroup, 4 lanes per row (each a quarter of the
// head dim), K/V tiles of 64 keys staged in LDS, all arithmetic in fp32.
template <int D, int PM>
__global__ __launch_bounds__(kThreads) void tra_fwd_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, int T, int nqt, float beta, float p) {
    constexpr int BQ = 64, BK = 64, DPT = D / 4;
    __shared__ float Ksh[BK][D];
    __shared__ float Vsh[BK][D];

    const int bh = blockIdx.x / nqt;
    const int qt = nqt - 1 - blockIdx.x % nqt;
    const int tid = threadIdx.x;
    const int part = tid & 3;
    const int my_q = qt * BQ + (tid >> 2);
    const size_t slab = (size_t)bh * T * D;

    float qv[DPT], acc[DPT];
#pragma unroll
    for (int d = 0; d < DPT; ++d) {
        qv[d] = my_q < T ? Q[slab + (size_t)my_q * D + part * DPT + d] : 0.0f;
        acc[d] = 0.0f;
    }
    const float tau = beta * sqrtf(2.0f * logf((float)(my_q + 1)) / (float)D);
    const int q_last = min(qt * BQ + BQ, T) - 1;

    for (int k0 = 0; k0 <= q_last; k0 += BK) {
        __syncthreads();
        for (int e = tid; e < BK * D; e += kThreads) {
            const int row = e / D, col = e % D, key = k0 + row;
            Ksh[row][col] = key < T ? K[slab + (size_t)key * D + col] : 0.0f;
            Vsh[row][col] = key < T ? V[slab + (size_t)key * D + col] : 0.0f;
        }
        __syncthreads();
        const int jn = min(BK, q_last - k0 + 1);
        for (int j = 0; j < jn; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int d = 0; d < DPT; ++d) s = fmaf(qv[d], Ksh[j][part * DPT + d], s);
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            float w = relu_pow<PM>(s - tau, p);
            if (k0 + j > my_q) w = 0.0f;
#pragma unroll
            for (int d = 0; d < DPT; ++d) acc[d] = fmaf(w, Vsh[j][part * DPT + d], acc[d]);
        }
    }
    if (my_q < T) {
#pragma unroll
        for (int d = 0; d < DPT; ++d) O[slab + (size_t)my_q * D + part * DPT + d] = acc[d];
    }
}

template <int D, int PM>
hipError_t launch_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *out,
                       int BH, int T, float beta, float p, hipStream_t stream) {
    int nqt = (T + kBM - 1) / kBM;
    void *args[] = {&q, &k, &v, &out, &BH, &T, &nqt, &beta, &p};
    return hipLaunchKernel((const void *)tra_fwd_bf16_kernel<D, PM>,
                           dim3((unsigned)(BH * nqt)), dim3(kThreads), args, 0, stream);
}

template <int D, int PM>
hipError_t launch_f32(const float *q, const float *k, const float *v, float *out, int BH,
                      int T, float beta, float p, hipStream_t stream) {
    int nqt = (T + 63) / 64;
    void *args[] = {&q, &k, &v, &out, &T, &nqt, &beta, &p};
    return hipLaunchKernel((const void *)tra_fwd_f32_kernel<D, PM>,
                           dim3((unsigned)(BH * nqt)), dim3(kThreads), args, 0, stream);
}

int pow_mode(float p) { return p == 1.0f ? kPowOne : (p == 2.0f ? kPowTwo : kPowGeneral); }

}  // namespace

hipError_t launch_tra_fwd_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               uint16_t *out, int BH, int T, int D, float beta, float p,
                               hipStream_t stream) {
    const int pm = pow_mode(p);
    if (D == 128) {
        if (pm == kPowTwo) return launch_bf16<128, kPowTwo>(q, k, v, out, BH, T, beta, p, stream);
        if (pm == kPowOne) return launch_bf16<128, kPowOne>(q, k, v, out, BH, T, beta, p, stream);
        return launch_bf16<128, kPowGeneral>(q, k, v, out, BH, T, beta, p, stream);
    }
    if (pm == kPowTwo) return launch_bf16<64, kPowTwo>(q, k, v, out, BH, T, beta, p, stream);
    if (pm == kPowOne) return launch_bf16<64, kPowOne>(q, k, v, out, BH, T, beta, p, stream);
    return launch_bf16<64, kPowGeneral>(q, k, v, out, BH, T, beta, p, stream);
}

hipError_t launch_tra_fwd_f32(const float *q, const float *k, const float *v, float *out,
                              int BH, int T, int D, float beta, float p, hipStream_t stream) {
    const int pm = pow_mode(p);
    if (D == 128) {
        if (pm == kPowTwo) return launch_f32<128, kPowTwo>(q, k, v, out, BH, T, beta, p, stream);
        if (pm == kPowOne) return launch_f32<128, kPowOne>(q, k, v, out, BH, T, beta, p, stream);
        return launch_f32<128, kPowGeneral>(q, k, v, out, BH, T, beta, p, stream);
    }
    if (pm == kPowTwo) return launch_f32<64, kPowTwo>(q, k, v, out, BH, T, beta, p, stream);
    if (pm == kPowOne) return launch_f32<64, kPowOne>(q, k, v, out, BH, T, beta, p, stream);
    return launch_f32<64, kPowGeneral>(q, k, v, out, BH, T, beta, p, stream);
}

}  // namespace attn
