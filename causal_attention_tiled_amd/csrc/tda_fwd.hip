// tda_fwd.hip -- Threshold Differential Attention forward for gfx950.
//
// Definition (snap-research/TDA, page "triton_threshold_attention.py",
// `differential_threshold_rela_triton`): when normalisation is on, every row of
// q1, k1, q2, k2 is first divided by max(||row||_2, 1e-12); then two Threshold
// Rectified Attention outputs over the same v are combined,
//     out_i = sum_{j<=i} [ max(q1_i.k1_j - tau_i, 0)^p - lam * max(q2_i.k2_j - tau_i, 0)^p ] v_j
// with lam = clamp(lambda, 0, 1) and tau_i = beta*sqrt(2 ln(i+1)/D).
//
// The page runs the two attention passes separately and combines their outputs.
// Both passes multiply the same V, so here one kernel streams K1, K2 and V once,
// combines the two weights of every key pair in registers and runs ONE weighted
// sum with V: three MFMA contractions per pair instead of four, and one read of V.
//
// Layout of the work is that of the Threshold Rectified Attention kernel: 256
// query rows of one (b,h) per workgroup, 8 wavefronts of 32 rows, transposed
// score tiles (one query per lane, so tau is a per-lane scalar), 64-key tiles of
// K1, K2 and V staged HBM -> LDS by buffer loads, double-buffered, V read
// transposed from LDS.  The score accumulators start at -tau, as in that kernel (so
// lambda = 0 reproduces it bit for bit).  At D = 128 the Q2^T operands are read from
// a copy of the workgroup's Q2 rows in LDS instead of being held in registers, which
// leaves room for the -tau registers without spilling.
//
// Normalisation, as torch.nn.functional.normalize does on the page's bf16 tensors:
// the row's 2-norm rounded to bf16 (at least 1e-12), then each element divided by
// it and rounded to bf16.  A query row is normalised in registers when the wave
// loads it.  Key rows are normalised once, by a row-normalisation pass that writes
// them to the caller's workspace, since every workgroup of a head re-reads the keys.
#include <type_traits>

#include "attn_tile.h"

namespace attn {
namespace {

constexpr int kWaves = 8;  // wavefronts per workgroup, 32 query rows each
static_assert(kWaves * 32 == kTdaRows, "workgroup rows");
constexpr int kBN = 64;    // keys per LDS tile

// torch.nn.functional.normalize on a bf16 tensor divides by a bf16 norm, clamped
// below at 1e-12 (also a bf16 value: 0x2b8d as bf16 bits).
constexpr float kNormEps = 1.0018652574217413e-12f;

// The bf16 value nearest (ties to even) to sqrt(ss), as a float.  ss is the sum of
// squares of a bf16 row accumulated in fp64, which is exact unless the row's
// magnitudes span about 2^30; the fp64 square root is then rounded straight to 8
// significant bits (no intermediate fp32 rounding), so the result is the exact
// norm rounded once, except where that lies within ~2^-50 of a bf16 midpoint.
__device__ __forceinline__ float bf16_norm(double ss) {
    uint64_t b = __builtin_bit_cast(uint64_t, __builtin_sqrt(ss));
    b += (((uint64_t)1 << 44) - 1) + ((b >> 45) & 1);  // nearest-even at bit 45
    b &= ~(((uint64_t)1 << 45) - 1);
    return fmaxf((float)__builtin_bit_cast(double, b), kNormEps);
}
// Each normalised element is bf16(x / n) for bf16 values x and n.  Such a quotient
// is never within 2^-17 (relative) of a bf16 rounding midpoint, so x * (1/n) in
// fp32 (relative error below 2^-22) rounds to the same bf16 value as the exact
// quotient does.

// Row L2 normalisation, bf16 -> bf16: y = bf16(x / bf16_norm(sum x^2)).  D/8 lanes
// per row, 16 bytes per lane; blockIdx.y picks one of two tensors.
template <int D>
__global__ __launch_bounds__(256) void l2norm_rows_kernel(const uint16_t *__restrict__ x0,
                                                          const uint16_t *__restrict__ x1,
                                                          uint16_t *__restrict__ y0,
                                                          uint16_t *__restrict__ y1,
                                                          int64_t rows) {
    constexpr int LPR = D / 8;
    const uint16_t *x = blockIdx.y ? x1 : x0;
    uint16_t *y = blockIdx.y ? y1 : y0;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / LPR;
    const int part = (int)(gid % LPR);
    // whole groups of LPR lanes leave together, so the shuffles below stay within
    // groups whose lanes are all active
    if (row >= rows) return;
    const u32x4 raw = *(const u32x4 *)(x + row * D + part * 8);
    const bf16x8 e = as_bf16x8(raw);
    float f[8];
    double ss = 0.0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        f[t] = (float)e[t];
        ss = __builtin_fma((double)f[t], (double)f[t], ss);
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
    const float r = 1.0f / bf16_norm(ss);
    const u32x4 o = {pack_bf16x2(f[0] * r, f[1] * r), pack_bf16x2(f[2] * r, f[3] * r),
                     pack_bf16x2(f[4] * r, f[5] * r), pack_bf16x2(f[6] * r, f[7] * r)};
    *(u32x4 *)(y + row * D + part * 8) = o;
}

template <int D, int PM>
__global__ __launch_bounds__(64 * kWaves) void tda_fwd_bf16_kernel(
    const uint16_t *__restrict__ Q1, const uint16_t *__restrict__ Q2,
    const uint16_t *__restrict__ K1, const uint16_t *__restrict__ K2,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, int BH, int T, int nqt,
    float beta, float lam, float p, int norm_q) {
    constexpr int BM = kWaves * 32;                  // query rows per workgroup
    constexpr int ROWB = D * 2;                      // bytes per key row
    constexpr int CH = D / 8;                        // 16-byte chunks per row
    constexpr int TILEB = kBN * ROWB;                // bytes of one tile of one tensor
    constexpr int BLKB = 32 * ROWB;                  // bytes of one 32-key block
    constexpr int LOADS = kBN * CH / (64 * kWaves);  // 16-byte chunks per lane per tensor
    constexpr int NDS = D / 16;                      // S^T MFMA k-steps
    constexpr int NDT = D / 32;                      // 32-dim output tiles
    // LDS: K1 tiles (buffers 0, 1), K2 tiles, V tiles
    constexpr int K1B = 0, K2B = 2 * TILEB, VB = 4 * TILEB;
    static_assert(LOADS >= 1 && kBN * CH % (64 * kWaves) == 0, "tile staging");
    static_assert(TILEB == kWaves * LOADS * 1024, "one 1 KB DMA block per wave and chunk");
    static_assert(K2B + TILEB + BLKB + 32 * ROWB <= 65536, "K immediate offsets");

    // At D = 128 the Q2^T operands live in LDS (the workgroup's Q2 rows, after the K/V
    // tiles: 160 KB in all), which frees the registers that let the scores start at -tau
    constexpr bool kQ2Lds = D == 128;
    constexpr int Q2B = 6 * TILEB;
    __shared__ __attribute__((aligned(16))) uint8_t lds[6 * TILEB + (kQ2Lds ? BM * ROWB : 0)];

    int bh, qt;
    tile_order(blockIdx.x, BH, nqt, bh, qt);
    bh = __builtin_amdgcn_readfirstlane(bh);
    qt = __builtin_amdgcn_readfirstlane(qt);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const size_t slab = (size_t)bh * T * D;

    const int q0 = qt * BM;
    const int qw0 = q0 + 32 * wave;
    const int q_last = min(q0 + BM, T) - 1;
    const int ntiles = q_last / kBN + 1;

    const u32x4 rk1 = make_rsrc(K1 + slab, (uint32_t)T * ROWB);
    const u32x4 rk2 = make_rsrc(K2 + slab, (uint32_t)T * ROWB);
    const u32x4 rv = make_rsrc(V + slab, (uint32_t)T * ROWB);
    int dma_src[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int pos = (wave * LOADS + j) * 1024 + lane * 16;
        const int row = pos / ROWB, slot = (pos % ROWB) >> 4;
        dma_src[j] = row * ROWB + ((slot ^ tile_swz<D>(row)) << 4);
    }
    auto gload = [&](int n, int buf) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int dst = buf * TILEB + (wave * LOADS + j) * 1024;
            dma16(rk1, &lds[K1B + dst], dma_src[j], n * TILEB);
            dma16(rk2, &lds[K2B + dst], dma_src[j], n * TILEB);
            dma16(rv, &lds[VB + dst], dma_src[j], n * TILEB);
        }
    };

    int koff[NDS];  // K row l32, chunk 2*ds + hi
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) koff[ds] = l32 * ROWB + (((2 * ds + hi) ^ tile_swz<D>(l32)) << 4);
    const int g16 = lane >> 4, s16 = lane & 15;
    const int vrow = 4 * (g16 >> 1) + (s16 >> 2);
    int voff[NDT][2];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = vrow + 8 * h;
            voff[dt][h] = VB + row * ROWB +
                          (((4 * dt + 2 * (g16 & 1) + ((s16 & 3) >> 1)) ^ tile_swz<D>(row)) << 4) +
                          8 * (s16 & 1);
        }
    auto k_frag = [&](int tensor_base, int buf, int kb, int ds) {
        return *(const bf16x8 *)(&lds[koff[ds] + tensor_base + buf * TILEB + kb * BLKB]);
    };
    auto v_frag = [&](int buf, int kb, int dt, int c) {
        const uint8_t *base = &lds[buf * TILEB + kb * BLKB + 16 * c * ROWB];
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + voff[dt][0]));
        const bf16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + voff[dt][1]));
        return (bf16x8)__builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;

    gload(0, 0);
    // Q^T operands of both paths, normalised in registers when asked: a lane holds
    // half of its row (the other half is in lane ^ 32).
    const int myq = qw0 + l32;
    bf16x8 qf1[NDS], qf2[NDS];
    {
        const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            u32x4 r1 = zero4, r2 = zero4;
            if (myq < T) {
                r1 = *(const u32x4 *)(Q1 + slab + (size_t)myq * D + ds * 16 + hi * 8);
                r2 = *(const u32x4 *)(Q2 + slab + (size_t)myq * D + ds * 16 + hi * 8);
            }
            qf1[ds] = as_bf16x8(r1);
            qf2[ds] = as_bf16x8(r2);
        }
    }
    if (norm_q) {
        auto qnorm = [&](bf16x8 (&qf)[NDS]) {
            double ss = 0.0;
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const double x = (double)(float)qf[ds][t];
                    ss = __builtin_fma(x, x, ss);
                }
            ss += __shfl_xor(ss, 32, 64);
            const float r = 1.0f / bf16_norm(ss);
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
                for (int t = 0; t < 8; ++t) qf[ds][t] = (__bf16)((float)qf[ds][t] * r);
        };
        qnorm(qf1);
        qnorm(qf2);
    }
    // Q2^T operands: this wave's 32 rows at rows 32*wave + l32 of the LDS copy, in the
    // K tiles' chunk order
    int q2off[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) q2off[ds] = Q2B + wave * 32 * ROWB + koff[ds];
    if constexpr (kQ2Lds) {
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) *(bf16x8 *)(&lds[q2off[ds]]) = qf2[ds];
    }
    auto q2_frag = [&](int ds) {
        if constexpr (kQ2Lds)
            return *(const bf16x8 *)(&lds[q2off[ds]]);
        else
            return qf2[ds];
    };
    const float tau = beta * sqrtf(2.0f * logf((float)(myq + 1)) / (float)D);
    // -tau as the score accumulators' starting value (sixteen registers feeding the
    // first MFMA of each chain as its C operand): no subtraction per score
    f32x16 cinit;
#pragma unroll
    for (int r = 0; r < 16; ++r) cinit[r] = -tau;

    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();

    auto mask_block = [&](f32x16 &sv, int kbase) {
        const int lim = qw0 + l32 - kbase - 4 * hi;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) > lim) sv[r] = -INFINITY;
    };
    auto tile_sync = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
    };

    // Per 32-key block, in order: S1 = K1 Q1^T, S2 = K2 Q2^T, the mask,
    // P = bf16(relu(S1 - tau)^p - lam * relu(S2 - tau)^p), O += V P; each operand is
    // read from LDS just before its product and the compiler interleaves the rest
    // (the other wave on the SIMD covers each wave's vector-only stretch).
    auto tile = [&](int n, auto masked, int buf) {
        constexpr bool kMasked = decltype(masked)::value;
        if (n + 1 < ntiles) gload(n + 1, buf ^ 1);
        if constexpr (kMasked) {
            // every key of the tile lies after every row of this wave
            if (n * kBN > qw0 + 31) {
                tile_sync();
                return;
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 s1 = cinit, s2 = cinit;
            bf16x8 pf[2];
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) s1 = mfma_32x32x16(k_frag(K1B, buf, kb, ds), qf1[ds], s1);
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) s2 = mfma_32x32x16(k_frag(K2B, buf, kb, ds), q2_frag(ds), s2);
            if constexpr (kMasked) {
                mask_block(s1, n * kBN + 32 * kb);
                mask_block(s2, n * kBN + 32 * kb);
            }
            {
#pragma clang fp contract(off)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float w1 = relu_pow<PM>(s1[r], p);
                    const float w2 = relu_pow<PM>(s2[r], p);
                    pf[r >> 3][r & 7] = (__bf16)__builtin_fmaf(-lam, w2, w1);
                }
            }
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    oacc[dt] = mfma_32x32x16(v_frag(buf, kb, dt, c), pf[c], oacc[dt]);
        }
        tile_sync();
    };

    const int n_interior = min(ntiles, (qw0 + 1) / kBN);
    const std::false_type plain{};
    const std::true_type masked{};
    int n = 0;
    for (; n + 1 < n_interior; n += 2) {
        tile(n, plain, 0);
        tile(n + 1, plain, 1);
    }
    if (n < n_interior) tile(n++, plain, 0);
    if (n < ntiles && (n & 1)) tile(n++, masked, 1);
    for (; n + 1 < ntiles; n += 2) {
        tile(n, masked, 0);
        tile(n + 1, masked, 1);
    }
    if (n < ntiles) tile(n++, masked, 0);

    if (myq < T) {
        uint16_t *orow = O + slab + (size_t)myq * D;
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

template <int D, int PM>
hipError_t launch_main(const uint16_t *q1, const uint16_t *q2, const uint16_t *k1,
                       const uint16_t *k2, const uint16_t *v, uint16_t *out, int BH, int T,
                       float beta, float lam, float p, int norm_q, hipStream_t stream) {
    int nqt = (T + kTdaRows - 1) / kTdaRows;
    void *args[] = {&q1, &q2, &k1, &k2, &v, &out, &BH, &T, &nqt, &beta, &lam, &p, &norm_q};
    return hipLaunchKernel((const void *)tda_fwd_bf16_kernel<D, PM>, dim3((unsigned)(BH * nqt)),
                           dim3(64 * kWaves), args, 0, stream);
}

template <int D>
hipError_t launch_d(const uint16_t *q1, const uint16_t *q2, const uint16_t *k1,
                    const uint16_t *k2, const uint16_t *v, uint16_t *out, uint16_t *ws, int BH,
                    int T, float beta, float lam, float p, int normalize, hipStream_t stream) {
    if (normalize) {
        int64_t rows = (int64_t)BH * T;
        const uint16_t *x0 = k1, *x1 = k2;
        uint16_t *y0 = ws, *y1 = ws + rows * D;
        void *args[] = {&x0, &x1, &y0, &y1, &rows};
        const int64_t blocks = (rows * (D / 8) + 255) / 256;
        const hipError_t e = hipLaunchKernel((const void *)l2norm_rows_kernel<D>,
                                             dim3((unsigned)blocks, 2), dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
        k1 = y0;
        k2 = y1;
    }
    const int pm = pow_mode(p);
    if (pm == kPowTwo) return launch_main<D, kPowTwo>(q1, q2, k1, k2, v, out, BH, T, beta, lam, p, normalize, stream);
    if (pm == kPowOne) return launch_main<D, kPowOne>(q1, q2, k1, k2, v, out, BH, T, beta, lam, p, normalize, stream);
    if (pm == kPowThreeHalves)
        return launch_main<D, kPowThreeHalves>(q1, q2, k1, k2, v, out, BH, T, beta, lam, p, normalize, stream);
    return launch_main<D, kPowGeneral>(q1, q2, k1, k2, v, out, BH, T, beta, lam, p, normalize, stream);
}

}  // namespace

hipError_t launch_tda_fwd_bf16(const uint16_t *q1, const uint16_t *q2, const uint16_t *k1,
                               const uint16_t *k2, const uint16_t *v, uint16_t *out,
                               uint16_t *workspace, int BH, int T, int D, float beta,
                               float lam, float p, int normalize, hipStream_t stream) {
    const float lc = fminf(fmaxf(lam, 0.0f), 1.0f);
    if (D == 128)
        return launch_d<128>(q1, q2, k1, k2, v, out, workspace, BH, T, beta, lc, p, normalize, stream);
    return launch_d<64>(q1, q2, k1, k2, v, out, workspace, BH, T, beta, lc, p, normalize, stream);
}

}  // namespace attn
