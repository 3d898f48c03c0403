// tra_bwd.hip -- Threshold Rectified Attention backward for gfx950.
//
// Definition (snap-research/TDA, page "triton_threshold_attention.py",
// `_threshold_rela_bwd_kernel_dq`, `_threshold_rela_bwd_kernel_dkv` and
// `ThresholdRelaFunction.backward`): with x_ij = q_i.k_j - tau_i over the causal
// pairs j <= i, w_ij = max(x_ij, 0)^p and g_ij = p * max(x_ij, 0)^(p-1) (0 for
// x_ij <= 0), and a_ij = (dout_i . v_j) * g_ij,
//     dq_i = sum_{j<=i} a_ij k_j,   dk_j = sum_{i>=j} a_ij q_i,   dv_j = sum_{i>=j} w_ij dout_i.
// Gradients of q, k and v only (beta and p get none), in the input dtype.
//
// Two kernels, as on the page, so that every gradient row is written by exactly
// one wavefront (no atomics; the result does not depend on scheduling):
//  * tra_bwd_dq_kernel: the forward's layout, 32 query rows per wavefront, 8
//    wavefronts (256 rows, two per SIMD) per workgroup at D = 128 and 4 at D = 64,
//    transposed score tiles so tau and the mask are per lane.  Per 32-key block:
//    S^T = K Q^T, dP^T = V dO^T, then A^T = dP^T * g (rounded to bf16, in the
//    accumulator's register order) and dQ^T += K^T A^T with K^T read transposed
//    from LDS, each operand read just before its product so that the Q and dO
//    operands and the dQ accumulator leave room for two waves per SIMD; the
//    other wave of the SIMD covers the read latency.  At D = 64 the S and dP
//    chains are interleaved instead, with each step's K and V rows read one step
//    ahead.  K and V tiles stream HBM -> LDS by DMA, double-buffered, as in the
//    forward.
//  * tra_bwd_dkv_kernel (D = 64): 128 key rows per workgroup, 4 wavefronts of 32
//    keys, one per SIMD.  A wave keeps its K and V rows in registers; Q and dO
//    tiles of 64 queries stream through LDS.  Per 32-query block: S = -tau + Q K^T
//    and dP = dO V^T (one key per lane, so the query thresholds come from a small
//    LDS table), W and A rounded to bf16, then dV^T += dO^T W and dK^T += Q^T A
//    with dO^T and Q^T read transposed from LDS.
//  * tra_bwd_dkv_wide_kernel (D = 128): the same products for 64 keys per
//    wavefront (256 per workgroup, one wave per SIMD), as two 32-key groups that
//    share every Q, dO, Q^T and dO^T operand read (half the LDS reads per MFMA,
//    and two independent chains in each phase).  The dK and dV accumulators (256
//    registers per lane) live in the accumulation registers, the K rows in vector
//    registers and the workgroup's V rows in LDS.
// The constant factor p of g is applied once to dq and dk at the end.
#include <type_traits>

#include "attn_tile.h"

namespace attn {
namespace {

// dq kernel waves per workgroup (32 query rows each): at D = 128 eight, two per SIMD
// (256 registers each); at D = 64 four, with two or three workgroups per compute unit
template <int D>
constexpr int dq_waves() { return D == 128 ? 8 : 4; }
constexpr int kDkvWaves = 4;  // dk/dv kernel: 32 key rows per wave
static_assert(kDkvWaves * 32 == tra_bwd_dkv_rows(64), "dk/dv workgroup rows");
constexpr int kBN = 64;       // keys (dq kernel) or queries (dk/dv kernel) per LDS tile

// max(x, 0)^(p-1) for x > 0, else 0 (the factor p is applied to the sums).
template <int PM>
__device__ __forceinline__ float relu_pow_m1(float x, float p) {
    if constexpr (PM == kPowOne) {
        return x > 0.0f ? 1.0f : 0.0f;
    } else if constexpr (PM == kPowTwo) {
        return fmaxf(x, 0.0f);
    } else if constexpr (PM == kPowThreeHalves) {
        return __builtin_amdgcn_sqrtf(fmaxf(x, 0.0f));
    } else {
        return x > 0.0f ? __builtin_amdgcn_exp2f((p - 1.0f) * __builtin_amdgcn_logf(x)) : 0.0f;
    }
}

// The weight max(x, 0)^p and max(x, 0)^(p-1) (0 for x <= 0) of one score, as
// relu_pow and relu_pow_m1 give them; the general power takes log2 max(x, 0) once
// for both.
template <int PM>
__device__ __forceinline__ void relu_pow_both(float x, float p, float &w, float &g) {
    if constexpr (PM == kPowGeneral) {
        const float l = __builtin_amdgcn_logf(fmaxf(x, 0.0f));
        w = __builtin_amdgcn_exp2f(p * l);
        g = x > 0.0f ? __builtin_amdgcn_exp2f((p - 1.0f) * l) : 0.0f;
    } else if constexpr (PM == kPowThreeHalves) {
        const float r = fmaxf(x, 0.0f);
        g = __builtin_amdgcn_sqrtf(r);
        w = r * g;
    } else {
        w = relu_pow<PM>(x, p);
        g = relu_pow_m1<PM>(x, p);
    }
}

// Workgroup id -> (head slab, key tile) for the dk/dv kernel: key tiles with the
// most queries after them (small index) first; heads split over the 8 XCDs as in
// tile_order.
__device__ __forceinline__ void key_tile_order(int bid, int BH, int &bh, int &kt) {
    if ((BH & 7) == 0) {
        const int xcd = bid & 7, s = bid >> 3, hpx = BH >> 3;
        bh = xcd * hpx + s % hpx;
        kt = s / hpx;
    } else {
        bh = bid % BH;
        kt = bid / BH;
    }
}

template <int D, int PM, int kDqWaves = dq_waves<D>()>
__global__ __launch_bounds__(64 * kDqWaves) void tra_bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO, uint16_t *__restrict__ dQ,
    int BH, int T, int nqt, float beta, float p) {
    constexpr int BM = kDqWaves * 32;
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    constexpr int TILEB = kBN * ROWB;
    constexpr int BLKB = 32 * ROWB;
    constexpr int LOADS = kBN * CH / (64 * kDqWaves);
    constexpr int NDS = D / 16;
    constexpr int NDT = D / 32;
    constexpr int KB = 0, VB = 2 * TILEB;  // K tiles (2 buffers), then V tiles
    static_assert(LOADS >= 1 && kBN * CH % (64 * kDqWaves) == 0, "tile staging");
    static_assert(TILEB == kDqWaves * LOADS * 1024, "one 1 KB DMA block per wave and chunk");

    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * TILEB];

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

    const u32x4 rk = make_rsrc(K + slab, (uint32_t)T * ROWB);
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
            dma16(rk, &lds[KB + dst], dma_src[j], n * TILEB);
            dma16(rv, &lds[VB + dst], dma_src[j], n * TILEB);
        }
    };

    // row-operand reads (K or V rows l32, chunk 2*ds + hi) and transposed K reads
    int koff[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) koff[ds] = l32 * ROWB + (((2 * ds + hi) ^ tile_swz<D>(l32)) << 4);
    const int g16 = lane >> 4, s16 = lane & 15;
    const int trow = 4 * (g16 >> 1) + (s16 >> 2);
    int toff[NDT][2];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = trow + 8 * h;
            toff[dt][h] = row * ROWB +
                          (((4 * dt + 2 * (g16 & 1) + ((s16 & 3) >> 1)) ^ tile_swz<D>(row)) << 4) +
                          8 * (s16 & 1);
        }
    auto row_frag = [&](int base, int buf, int kb, int ds) {
        return *(const bf16x8 *)(&lds[koff[ds] + base + buf * TILEB + kb * BLKB]);
    };
    // K^T operand for keys 16c + {4hi..4hi+3, 8+4hi..8+4hi+3} of the block, dims 32dt + lane%32
    auto kt_frag = [&](int buf, int kb, int dt, int c) {
        const uint8_t *base = &lds[KB + buf * TILEB + kb * BLKB + 16 * c * ROWB];
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + toff[dt][0]));
        const bf16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + toff[dt][1]));
        return (bf16x8)__builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    f32x16 dqacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqacc[dt][r] = 0.0f;

    gload(0, 0);
    const int myq = qw0 + l32;
    bf16x8 qf[NDS], df[NDS];
    {
        const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            u32x4 a = zero4, b = zero4;
            if (myq < T) {
                a = *(const u32x4 *)(Q + slab + (size_t)myq * D + ds * 16 + hi * 8);
                b = *(const u32x4 *)(dO + slab + (size_t)myq * D + ds * 16 + hi * 8);
            }
            qf[ds] = as_bf16x8(a);
            df[ds] = as_bf16x8(b);
        }
    }
    const float tau = beta * sqrtf(2.0f * logf((float)(myq + 1)) / (float)D);
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

    // Per 32-key block: S^T = K Q^T, dP^T = V dO^T, S^T <- max(S^T - tau, 0)^(p-1),
    // A^T = bf16(dP^T * S^T), dQ^T += K^T A^T.
    auto tile = [&](int n, auto masked, int buf) {
        constexpr bool kMasked = decltype(masked)::value;
        if (n + 1 < ntiles) gload(n + 1, buf ^ 1);
        if constexpr (kMasked) {
            if (n * kBN > qw0 + 31) {
                tile_sync();
                return;
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 s = {}, dp = {};
            bf16x8 af[2];
            if constexpr (D == 64) {
                // the S and dP chains interleaved, each step's K and V rows read one step
                // ahead of its products (fenced so the compiler keeps the order); at
                // D = 64 this also leaves room for three waves per SIMD
                bf16x8 kr = row_frag(KB, buf, kb, 0), vr = row_frag(VB, buf, kb, 0);
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) {
                    bf16x8 kn = kr, vn = vr;
                    if (ds + 1 < NDS) {
                        kn = row_frag(KB, buf, kb, ds + 1);
                        vn = row_frag(VB, buf, kb, ds + 1);
                    }
                    s = mfma_32x32x16(kr, qf[ds], s);
                    dp = mfma_32x32x16(vr, df[ds], dp);
                    __builtin_amdgcn_sched_barrier(0);
                    kr = kn;
                    vr = vn;
                }
                if constexpr (kMasked) mask_block(s, n * kBN + 32 * kb);
            } else {
                // at D = 128 each operand is read just before its product: the registers
                // a read-ahead needs make the kernel spill
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) s = mfma_32x32x16(row_frag(KB, buf, kb, ds), qf[ds], s);
                if constexpr (kMasked) mask_block(s, n * kBN + 32 * kb);
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) dp = mfma_32x32x16(row_frag(VB, buf, kb, ds), df[ds], dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = relu_pow_m1<PM>(s[r] - tau, p);
#pragma unroll
            for (int r = 0; r < 16; ++r) af[r >> 3][r & 7] = (__bf16)(dp[r] * s[r]);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    dqacc[dt] = mfma_32x32x16(kt_frag(buf, kb, dt, c), af[c], dqacc[dt]);
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

    // dQ^T accumulator: lane holds row qw0 + l32, dims 32*dt + 8*i + 4*hi + j.
    if (myq < T) {
        uint16_t *row = dQ + slab + (size_t)myq * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x2 pr = {pack_bf16x2(p * dqacc[dt][4 * i], p * dqacc[dt][4 * i + 1]),
                                  pack_bf16x2(p * dqacc[dt][4 * i + 2], p * dqacc[dt][4 * i + 3])};
                *(u32x2 *)(row + dt * 32 + 8 * i + 4 * hi) = pr;
            }
    }
}

template <int D, int PM>
__global__ __launch_bounds__(64 * kDkvWaves) void tra_bwd_dkv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, int BH, int T, float beta, float p) {
    constexpr int BK = kDkvWaves * 32;               // key rows per workgroup
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    constexpr int TILEB = kBN * ROWB;                // one tile of 64 query rows
    constexpr int BLKB = 32 * ROWB;
    constexpr int LOADS = kBN * CH / (64 * kDkvWaves);
    constexpr int NDS = D / 16;
    constexpr int NDT = D / 32;
    constexpr int QB = 0, OB = 2 * TILEB;            // Q tiles (2 buffers), then dO tiles
    static_assert(LOADS >= 1 && kBN * CH % (64 * kDkvWaves) == 0, "tile staging");
    static_assert(TILEB == kDkvWaves * LOADS * 1024, "one 1 KB DMA block per wave and chunk");

    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * TILEB];
    __shared__ __attribute__((aligned(16))) float ntau[2][kBN];  // -tau of each query of a tile

    int bh, kt;
    key_tile_order(blockIdx.x, BH, bh, kt);
    bh = __builtin_amdgcn_readfirstlane(bh);
    kt = __builtin_amdgcn_readfirstlane(kt);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const size_t slab = (size_t)bh * T * D;
    const int k0 = kt * BK;
    const int kw0 = k0 + 32 * wave;                  // this wave's keys kw0 .. kw0+31
    const int mykey = kw0 + l32;
    const int n0 = k0 / kBN;                         // first query tile with a query >= k0
    const int ntiles = (T - 1) / kBN + 1;
    const int jd = kw0 / 32;                         // this wave's diagonal 32-query block

    const u32x4 rq = make_rsrc(Q + slab, (uint32_t)T * ROWB);
    const u32x4 ro = make_rsrc(dO + slab, (uint32_t)T * ROWB);
    int dma_src[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int pos = (wave * LOADS + j) * 1024 + lane * 16;
        const int row = pos / ROWB, slot = (pos % ROWB) >> 4;
        dma_src[j] = row * ROWB + ((slot ^ tile_swz<D>(row)) << 4);
    }
    const float tscale = 2.0f / (float)D;
    auto gload = [&](int n, int buf) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int dst = buf * TILEB + (wave * LOADS + j) * 1024;
            dma16(rq, &lds[QB + dst], dma_src[j], n * TILEB);
            dma16(ro, &lds[OB + dst], dma_src[j], n * TILEB);
        }
        if (wave == 0) ntau[buf][lane] = -beta * sqrtf(tscale * logf((float)(n * kBN + lane + 1)));
    };

    int roff[NDS];  // Q or dO rows l32, chunk 2*ds + hi
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) roff[ds] = l32 * ROWB + (((2 * ds + hi) ^ tile_swz<D>(l32)) << 4);
    const int g16 = lane >> 4, s16 = lane & 15;
    const int trow = 4 * (g16 >> 1) + (s16 >> 2);
    int toff[NDT][2];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = trow + 8 * h;
            toff[dt][h] = row * ROWB +
                          (((4 * dt + 2 * (g16 & 1) + ((s16 & 3) >> 1)) ^ tile_swz<D>(row)) << 4) +
                          8 * (s16 & 1);
        }
    auto row_frag = [&](int base, int buf, int qb, int ds) {
        return *(const bf16x8 *)(&lds[roff[ds] + base + buf * TILEB + qb * BLKB]);
    };
    // transposed operand (dO^T or Q^T) for queries 16c + {4hi..4hi+3, 8+4hi..8+4hi+3}
    // of the block, dims 32dt + lane%32
    auto t_frag = [&](int base, int buf, int qb, int dt, int c) {
        const uint8_t *b = &lds[base + buf * TILEB + qb * BLKB + 16 * c * ROWB];
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(b + toff[dt][0]));
        const bf16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(b + toff[dt][1]));
        return (bf16x8)__builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    f32x16 dkacc[NDT], dvacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkacc[dt][r] = dvacc[dt][r] = 0.0f;

    gload(n0, 0);
    // this wave's key and value rows as the B operands (lane = key, 8 dims per k-step)
    bf16x8 kf[NDS], vf[NDS];
    {
        const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            u32x4 a = zero4, b = zero4;
            if (mykey < T) {
                a = *(const u32x4 *)(K + slab + (size_t)mykey * D + ds * 16 + hi * 8);
                b = *(const u32x4 *)(V + slab + (size_t)mykey * D + ds * 16 + hi * 8);
            }
            kf[ds] = as_bf16x8(a);
            vf[ds] = as_bf16x8(b);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();

    f32x16 zero16;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero16[r] = 0.0f;
    // diagonal block: key kw0 + l32 against query kw0 + 8*(r/4) + 4*hi + r%4
    auto mask_diag = [&](f32x16 &sv) {
        const int lim = l32 - 4 * hi;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (lim > 8 * (r >> 2) + (r & 3)) sv[r] = -INFINITY;
    };

    // Per 32-query block, four phases, each with the operands of the next one read
    // alongside its MFMAs:
    //   1: S = -tau + Q K^T            (dO rows read)
    //   2: dP = dO V^T || W, G from S  (dO^T read)
    //   3: dV^T += dO^T W || A = dP G  (Q^T read)
    //   4: dK^T += Q^T A               (the next block's Q rows and -tau read)
    bf16x8 qrow[NDS], orow[NDS], tf[NDT][2];
    f32x16 sinit;
    auto read_q = [&](int buf, int qb) {
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qrow[ds] = row_frag(QB, buf, qb, ds);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 t4 = *(const f32x4 *)(&ntau[buf][32 * qb + 8 * g + 4 * hi]);
#pragma unroll
            for (int j = 0; j < 4; ++j) sinit[4 * g + j] = t4[j];
        }
    };
    // One tile of 64 queries (two blocks).  Only the workgroup's first two tiles hold
    // blocks before or at a wave's diagonal block (the masked form); the rest run
    // mask-free, two tiles at a time so that every LDS buffer offset is a constant.
    auto tile = [&](int n, auto masked, int buf) {
        constexpr bool kMasked = decltype(masked)::value;
        if (n + 1 < ntiles) gload(n + 1, buf ^ 1);
        bool have_q = false;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int jb = 2 * n + qb;  // global 32-query block
            if constexpr (kMasked) {
                if (jb < jd) continue;  // every query of the block precedes every key of the wave
            }
            if (!have_q) read_q(buf, qb);
            // 1
            f32x16 s = sinit;
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) orow[ds] = row_frag(OB, buf, qb, ds);
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) s = mfma_32x32x16(qrow[ds], kf[ds], s);
#pragma unroll
            for (int i = 0; i < NDS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kMasked) {
                if (jb == jd) mask_diag(s);
            }
            // 2
            f32x16 dp = zero16;
            bf16x8 wf[2];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) tf[dt][c] = t_frag(OB, buf, qb, dt, c);
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) dp = mfma_32x32x16(orow[ds], vf[ds], dp);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float w, g;
                relu_pow_both<PM>(s[r], p, w, g);
                wf[r >> 3][r & 7] = (__bf16)w;
                s[r] = g;
            }
#pragma unroll
            for (int i = 0; i < NDS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            // 3
            bf16x8 af[2];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) dvacc[dt] = mfma_32x32x16(tf[dt][c], wf[c], dvacc[dt]);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) tf[dt][c] = t_frag(QB, buf, qb, dt, c);
#pragma unroll
            for (int r = 0; r < 16; ++r) af[r >> 3][r & 7] = (__bf16)(dp[r] * s[r]);
#pragma unroll
            for (int i = 0; i < 2 * NDT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            // 4
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) dkacc[dt] = mfma_32x32x16(tf[dt][c], af[c], dkacc[dt]);
            have_q = false;
            if (qb == 0) {
                read_q(buf, 1);
                have_q = true;
#pragma unroll
                for (int i = 0; i < 2 * NDT; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
    };
    const std::true_type masked{};
    const std::false_type plain{};
    tile(n0, masked, 0);
    if (n0 + 1 < ntiles) tile(n0 + 1, masked, 1);
    int n = n0 + 2;
    for (; n + 1 < ntiles; n += 2) {
        tile(n, plain, 0);
        tile(n + 1, plain, 1);
    }
    if (n < ntiles) tile(n, plain, 0);

    // dK^T, dV^T accumulators: lane holds key kw0 + l32, dims 32*dt + 8*i + 4*hi + j.
    if (mykey < T) {
        uint16_t *krow = dK + slab + (size_t)mykey * D;
        uint16_t *vrow = dV + slab + (size_t)mykey * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x2 kp = {pack_bf16x2(p * dkacc[dt][4 * i], p * dkacc[dt][4 * i + 1]),
                                  pack_bf16x2(p * dkacc[dt][4 * i + 2], p * dkacc[dt][4 * i + 3])};
                const u32x2 vp = {pack_bf16x2(dvacc[dt][4 * i], dvacc[dt][4 * i + 1]),
                                  pack_bf16x2(dvacc[dt][4 * i + 2], dvacc[dt][4 * i + 3])};
                *(u32x2 *)(krow + dt * 32 + 8 * i + 4 * hi) = kp;
                *(u32x2 *)(vrow + dt * 32 + 8 * i + 4 * hi) = vp;
            }
    }
}

// dK/dV accumulation into an accumulator held in the accumulation registers: the
// MFMA is written out so that its C/D operand can be an AGPR tuple while the score
// products keep the vector-register form.  The compiler does not see an MFMA here,
// so the hazards it would otherwise cover are handled in place: the B operand (W or
// A, just written by VALU instructions) needs two wait states before the MFMA
// reads it (s_nop 1); back-to-back accumulation into the same tuple needs none.  These
// are the distances the compiler keeps between its own MFMAs and their producers on
// this target (two wait states after v_cvt_pk_bf16_f32; dependent accumulations issued
// back to back).
__device__ __forceinline__ void mfma_acc(f32x16 &acc, bf16x8 a, bf16x8 b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

constexpr int kDkvWideWaves = 4;  // 64 keys per wave, one wave per SIMD
static_assert(kDkvWideWaves * 64 == tra_bwd_dkv_rows(128), "dk/dv workgroup rows");

// dK/dV for D = 128 with 64 keys per wave.  The accumulators of 64 keys x 128 dims
// (dK and dV: 256 fp32 registers per lane) fill the accumulation registers, so
// those products go through mfma_acc; the score products S and dP keep the
// vector-register form the epilogue reads.  Every phase step issues its two MFMAs
// (one per 32-key group) before its VALU work and the LDS reads for the next phase,
// with a scheduling fence per step holding that order.

template <int D, int PM>
__global__ __launch_bounds__(64 * kDkvWideWaves) void tra_bwd_dkv_wide_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, int BH, int T, float beta, float p) {
    constexpr int BK = kDkvWideWaves * 64;           // key rows per workgroup
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    constexpr int TILEB = kBN * ROWB;                // one tile of 64 query rows
    constexpr int BLKB = 32 * ROWB;
    constexpr int LOADS = kBN * CH / (64 * kDkvWideWaves);
    constexpr int NDS = D / 16;
    constexpr int NDT = D / 32;
    constexpr int QB = 0, OB = 2 * TILEB, VB = 4 * TILEB;  // Q tiles, dO tiles, V rows
    constexpr int VLOADS = BK * ROWB / (1024 * kDkvWideWaves);
    static_assert(LOADS >= 1 && kBN * CH % (64 * kDkvWideWaves) == 0, "tile staging");
    static_assert(TILEB == kDkvWideWaves * LOADS * 1024, "one 1 KB DMA block per wave and chunk");

    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * TILEB + BK * ROWB];
    __shared__ __attribute__((aligned(16))) float ntau[2][kBN];

    int bh, kt;
    key_tile_order(blockIdx.x, BH, bh, kt);
    bh = __builtin_amdgcn_readfirstlane(bh);
    kt = __builtin_amdgcn_readfirstlane(kt);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const size_t slab = (size_t)bh * T * D;
    const int k0 = kt * BK;
    const int kw0 = k0 + 64 * wave;                  // this wave's keys kw0 .. kw0+63
    const int n0 = k0 / kBN;
    const int ntiles = (T - 1) / kBN + 1;
    const int jd = kw0 / 32;                         // diagonal block of the first 32 keys

    const u32x4 rq = make_rsrc(Q + slab, (uint32_t)T * ROWB);
    const u32x4 ro = make_rsrc(dO + slab, (uint32_t)T * ROWB);
    int dma_src[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int pos = (wave * LOADS + j) * 1024 + lane * 16;
        const int row = pos / ROWB, slot = (pos % ROWB) >> 4;
        dma_src[j] = row * ROWB + ((slot ^ tile_swz<D>(row)) << 4);
    }
    const float tscale = 2.0f / (float)D;
    auto gload = [&](int n, int buf) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int dst = buf * TILEB + (wave * LOADS + j) * 1024;
            dma16(rq, &lds[QB + dst], dma_src[j], n * TILEB);
            dma16(ro, &lds[OB + dst], dma_src[j], n * TILEB);
        }
        if (wave == 0) ntau[buf][lane] = -beta * sqrtf(tscale * logf((float)(n * kBN + lane + 1)));
    };
    {
        // the workgroup's value rows, swizzled like the query tiles
        const u32x4 rv = make_rsrc(V + slab, (uint32_t)T * ROWB);
#pragma unroll
        for (int j = 0; j < VLOADS; ++j) {
            const int pos = (wave * VLOADS + j) * 1024 + lane * 16;
            const int row = pos / ROWB, slot = (pos % ROWB) >> 4;
            dma16(rv, &lds[VB + (wave * VLOADS + j) * 1024], row * ROWB + ((slot ^ tile_swz<D>(row)) << 4),
                  k0 * ROWB);
        }
    }

    int roff[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) roff[ds] = l32 * ROWB + (((2 * ds + hi) ^ tile_swz<D>(l32)) << 4);
    const int g16 = lane >> 4, s16 = lane & 15;
    const int trow = 4 * (g16 >> 1) + (s16 >> 2);
    int toff[NDT][2];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = trow + 8 * h;
            toff[dt][h] = row * ROWB +
                          (((4 * dt + 2 * (g16 & 1) + ((s16 & 3) >> 1)) ^ tile_swz<D>(row)) << 4) +
                          8 * (s16 & 1);
        }
    auto row_frag = [&](int base, int buf, int qb, int ds) {
        return *(const bf16x8 *)(&lds[roff[ds] + base + buf * TILEB + qb * BLKB]);
    };
    auto v_frag = [&](int g, int ds) {
        return *(const bf16x8 *)(&lds[roff[ds] + VB + (64 * wave + 32 * g) * ROWB]);
    };
    auto t_frag = [&](int base, int buf, int qb, int dt, int c) {
        const uint8_t *b = &lds[base + buf * TILEB + qb * BLKB + 16 * c * ROWB];
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(b + toff[dt][0]));
        const bf16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(b + toff[dt][1]));
        return (bf16x8)__builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    f32x16 dkacc[2][NDT], dvacc[2][NDT];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) dkacc[g][dt][r] = dvacc[g][dt][r] = 0.0f;
    // the zeros reach the accumulation registers before any MFMA reads them
    asm volatile("s_nop 4" : "+a"(dkacc[0][0]), "+a"(dkacc[0][1]), "+a"(dkacc[0][2]), "+a"(dkacc[0][3]),
                 "+a"(dkacc[1][0]), "+a"(dkacc[1][1]), "+a"(dkacc[1][2]), "+a"(dkacc[1][3]));
    asm volatile("s_nop 4" : "+a"(dvacc[0][0]), "+a"(dvacc[0][1]), "+a"(dvacc[0][2]), "+a"(dvacc[0][3]),
                 "+a"(dvacc[1][0]), "+a"(dvacc[1][1]), "+a"(dvacc[1][2]), "+a"(dvacc[1][3]));

    gload(n0, 0);
    // this wave's key rows as the B operands (lane = key, 8 dims per k-step)
    bf16x8 kf[2][NDS];
    {
        const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int key = kw0 + 32 * g + l32;
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                u32x4 a = zero4;
                if (key < T) a = *(const u32x4 *)(K + slab + (size_t)key * D + ds * 16 + hi * 8);
                kf[g][ds] = as_bf16x8(a);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();

    f32x16 zero16;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero16[r] = 0.0f;
    auto mask_diag = [&](f32x16 &sv) {
        const int lim = l32 - 4 * hi;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (lim > 8 * (r >> 2) + (r & 3)) sv[r] = -INFINITY;
    };

    f32x16 sinit;
    auto read_tau = [&](int buf, int qb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 t4 = *(const f32x4 *)(&ntau[buf][32 * qb + 8 * g + 4 * hi]);
#pragma unroll
            for (int j = 0; j < 4; ++j) sinit[4 * g + j] = t4[j];
        }
    };
    // Per 32-query block, four phases of eight fenced steps; each step issues its two
    // MFMAs (one per 32-key group, sharing the LDS operand) first, then its share of
    // the VALU work and the LDS reads for the next phase:
    //   A: S_g = -tau + Q K_g^T         reads dO rows (and the first V rows of B)
    //   B: dP_g = dO V_g^T  || W, G     reads V rows two steps ahead, dO^T
    //   C: dV_g^T += dO^T W_g || A = dP G   reads Q^T
    //   D: dK_g^T += Q^T A_g            reads the next block's Q rows
    bf16x8 qrow[NDS], orow[NDS], tfo[NDT][2], tq[NDT][2], vfa[3][2];
    bool have_q = false;
    auto tile = [&](int n, auto masked, int buf) {
        constexpr bool kMasked = decltype(masked)::value;
        if (n + 1 < ntiles) gload(n + 1, buf ^ 1);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int jb = 2 * n + qb;
            if constexpr (kMasked) {
                if (jb < jd) continue;
            }
            if (!have_q) {
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) qrow[ds] = row_frag(QB, buf, qb, ds);
                read_tau(buf, qb);
            }
            __builtin_amdgcn_sched_barrier(0);
            // A
            f32x16 s0, s1;
#pragma unroll
            for (int i = 0; i < NDS; ++i) {
                s0 = mfma_32x32x16(qrow[i], kf[0][i], i == 0 ? sinit : s0);
                s1 = mfma_32x32x16(qrow[i], kf[1][i], i == 0 ? sinit : s1);
                orow[i] = row_frag(OB, buf, qb, i);
                if (i >= NDS - 2) {
                    vfa[i - (NDS - 2)][0] = v_frag(0, i - (NDS - 2));
                    vfa[i - (NDS - 2)][1] = v_frag(1, i - (NDS - 2));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (kMasked) {
                if (jb == jd) {
                    mask_diag(s0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) s1[r] = -INFINITY;
                } else if (jb == jd + 1) {
                    mask_diag(s1);
                }
            }
            // B
            f32x16 dp0, dp1;
            bf16x8 wf[2][2];
#pragma unroll
            for (int i = 0; i < NDS; ++i) {
                dp0 = mfma_32x32x16(orow[i], vfa[i % 3][0], i == 0 ? zero16 : dp0);
                dp1 = mfma_32x32x16(orow[i], vfa[i % 3][1], i == 0 ? zero16 : dp1);
                if (i + 2 < NDS) {
                    vfa[(i + 2) % 3][0] = v_frag(0, i + 2);
                    vfa[(i + 2) % 3][1] = v_frag(1, i + 2);
                }
#pragma unroll
                for (int r = 2 * i; r < 2 * i + 2; ++r) {
                    float w, g;
                    relu_pow_both<PM>(s0[r], p, w, g);
                    wf[0][r >> 3][r & 7] = (__bf16)w;
                    s0[r] = g;
                    relu_pow_both<PM>(s1[r], p, w, g);
                    wf[1][r >> 3][r & 7] = (__bf16)w;
                    s1[r] = g;
                }
                tfo[i & 3][i >> 2] = t_frag(OB, buf, qb, i & 3, i >> 2);
                __builtin_amdgcn_sched_barrier(0);
            }
            // C
            bf16x8 af[2][2];
#pragma unroll
            for (int j = 0; j < 2 * NDT; ++j) {
                const int c = j / NDT, dt = j % NDT;
                mfma_acc(dvacc[0][dt], tfo[dt][c], wf[0][c]);
                mfma_acc(dvacc[1][dt], tfo[dt][c], wf[1][c]);
#pragma unroll
                for (int r = 2 * j; r < 2 * j + 2; ++r) {
                    af[0][r >> 3][r & 7] = (__bf16)(dp0[r] * s0[r]);
                    af[1][r >> 3][r & 7] = (__bf16)(dp1[r] * s1[r]);
                }
                tq[dt][c] = t_frag(QB, buf, qb, dt, c);
                __builtin_amdgcn_sched_barrier(0);
            }
            // D
            have_q = false;
#pragma unroll
            for (int j = 0; j < 2 * NDT; ++j) {
                const int c = j / NDT, dt = j % NDT;
                mfma_acc(dkacc[0][dt], tq[dt][c], af[0][c]);
                mfma_acc(dkacc[1][dt], tq[dt][c], af[1][c]);
                if (qb == 0) qrow[j] = row_frag(QB, buf, 1, j);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (qb == 0) {
                read_tau(buf, 1);
                have_q = true;
            }
        }
        have_q = false;
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
    };
    const std::true_type masked{};
    const std::false_type plain{};
    int n = n0;
    for (; n < n0 + 4 && n < ntiles; ++n) tile(n, masked, (n - n0) & 1);
    for (; n + 1 < ntiles; n += 2) {
        tile(n, plain, 0);
        tile(n + 1, plain, 1);
    }
    if (n < ntiles) tile(n, plain, 0);

    // the last accumulations have left the matrix unit before the reads below
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(dkacc[0][0]), "+a"(dkacc[0][1]), "+a"(dkacc[0][2]),
                 "+a"(dkacc[0][3]), "+a"(dkacc[1][0]), "+a"(dkacc[1][1]), "+a"(dkacc[1][2]), "+a"(dkacc[1][3]));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(dvacc[0][0]), "+a"(dvacc[0][1]), "+a"(dvacc[0][2]),
                 "+a"(dvacc[0][3]), "+a"(dvacc[1][0]), "+a"(dvacc[1][1]), "+a"(dvacc[1][2]), "+a"(dvacc[1][3]));
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int key = kw0 + 32 * g + l32;
        if (key < T) {
            uint16_t *krow = dK + slab + (size_t)key * D;
            uint16_t *vrow = dV + slab + (size_t)key * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x2 kp = {pack_bf16x2(p * dkacc[g][dt][4 * i], p * dkacc[g][dt][4 * i + 1]),
                                      pack_bf16x2(p * dkacc[g][dt][4 * i + 2], p * dkacc[g][dt][4 * i + 3])};
                    const u32x2 vp = {pack_bf16x2(dvacc[g][dt][4 * i], dvacc[g][dt][4 * i + 1]),
                                      pack_bf16x2(dvacc[g][dt][4 * i + 2], dvacc[g][dt][4 * i + 3])};
                    *(u32x2 *)(krow + dt * 32 + 8 * i + 4 * hi) = kp;
                    *(u32x2 *)(vrow + dt * 32 + 8 * i + 4 * hi) = vp;
                }
        }
    }
}

template <int D, int PM>
hipError_t launch(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                  uint16_t *dq, uint16_t *dk, uint16_t *dv, int BH, int T, float beta, float p,
                  hipStream_t stream) {
    constexpr int W = dq_waves<D>();
    int nqt = (T + 32 * W - 1) / (32 * W);
    void *a1[] = {&q, &k, &v, &dout, &dq, &BH, &T, &nqt, &beta, &p};
    hipError_t e = hipLaunchKernel((const void *)tra_bwd_dq_kernel<D, PM>,
                                   dim3((unsigned)(BH * nqt)), dim3(64 * W), a1, 0, stream);
    if (e != hipSuccess) return e;
    void *a2[] = {&q, &k, &v, &dout, &dk, &dv, &BH, &T, &beta, &p};
    if constexpr (D == 128) {
        int nkt = (T + tra_bwd_dkv_rows(D) - 1) / tra_bwd_dkv_rows(D);
        return hipLaunchKernel((const void *)tra_bwd_dkv_wide_kernel<D, PM>,
                               dim3((unsigned)(BH * nkt)), dim3(64 * kDkvWideWaves), a2, 0, stream);
    } else {
        int nkt = (T + tra_bwd_dkv_rows(D) - 1) / tra_bwd_dkv_rows(D);
        return hipLaunchKernel((const void *)tra_bwd_dkv_kernel<D, PM>, dim3((unsigned)(BH * nkt)),
                               dim3(64 * kDkvWaves), a2, 0, stream);
    }
}

}  // namespace

hipError_t launch_tra_bwd_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const uint16_t *dout, uint16_t *dq, uint16_t *dk, uint16_t *dv,
                               int BH, int T, int D, float beta, float p, hipStream_t stream) {
    const int pm = pow_mode(p);
    if (D == 128) {
        if (pm == kPowTwo) return launch<128, kPowTwo>(q, k, v, dout, dq, dk, dv, BH, T, beta, p, stream);
        if (pm == kPowOne) return launch<128, kPowOne>(q, k, v, dout, dq, dk, dv, BH, T, beta, p, stream);
        if (pm == kPowThreeHalves)
            return launch<128, kPowThreeHalves>(q, k, v, dout, dq, dk, dv, BH, T, beta, p, stream);
        return launch<128, kPowGeneral>(q, k, v, dout, dq, dk, dv, BH, T, beta, p, stream);
    }
    if (pm == kPowTwo) return launch<64, kPowTwo>(q, k, v, dout, dq, dk, dv, BH, T, beta, p, stream);
    if (pm == kPowOne) return launch<64, kPowOne>(q, k, v, dout, dq, dk, dv, BH, T, beta, p, stream);
    if (pm == kPowThreeHalves)
        return launch<64, kPowThreeHalves>(q, k, v, dout, dq, dk, dv, BH, T, beta, p, stream);
    return launch<64, kPowGeneral>(q, k, v, dout, dq, dk, dv, BH, T, beta, p, stream);
}

}  // namespace attn
