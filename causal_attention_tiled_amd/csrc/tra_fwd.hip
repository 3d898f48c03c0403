// tra_fwd.hip -- Threshold Rectified Attention forward for gfx950.
//
// Definition (snap-research/TDA, page "triton_threshold_attention.py", module
// docstring and `_threshold_rela_fwd_kernel`):
//     out_i = sum_{j <= i} max(q_i . k_j - tau_i, 0)^p v_j,   tau_i = beta*sqrt(2 ln(i+1) / D)
// with a 0-based query position i, natural log, no 1/sqrt(D) scale and no softmax.
//
// bf16 kernel design (one workgroup = 8 wavefronts = 256 query rows of one (b,h) at
// D = 128, two wavefronts per SIMD; 4 wavefronts = 128 rows at D = 64, where two or
// three workgroups share a compute unit):
//  * Each wave owns 32 query rows.  It computes the TRANSPOSED score tile
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16, K (A operand) from LDS, Q (B operand)
//    held in registers for the whole key loop.  In the accumulator every lane then
//    holds ONE query (lane % 32) and 16 keys, so tau_i is a per-lane scalar (folded
//    into the accumulator's initial value) and the causal test is a per-lane compare.
//  * The epilogue (ReLU, power, causal mask) runs on those registers and rounds the
//    weights to bf16; the register order of the accumulator directly forms the B
//    operand of O^T += V^T P^T (again 32x32x16), so P never touches LDS.  V stays
//    row-major in LDS and is read as the V^T operand with transposing LDS reads.
//  * K and V tiles of 64 keys go from HBM straight into LDS (buffer loads with the
//    LDS as destination), double-buffered: the next tile's loads are issued at the
//    start of the current tile and awaited, with one barrier, at its end.
//  * Causal tile skipping: key tiles past the workgroup's last query are never loaded;
//    tiles wholly after a wave's rows are skipped by that wave; the mask is evaluated
//    only on tiles that reach past a wave's first row.
//  * The wave issuing the second score block and the first epilogue runs at raised
//    issue priority, so that of two waves on a SIMD the one with the mixed MFMA and
//    VALU phase goes first.
//  * For the general power at D = 64 the phases are dropped: each 32-key block runs
//    scores, weights and P V in order and the compiler interleaves them, since the
//    weights (a log and an exp each) are more vector work than the phase pattern
//    leaves room for.
//  * Launch order: the heaviest query tiles (largest i) first, and the heads split
//    into 8 contiguous groups so that each XCD (dispatch is round-robin over the 8
//    XCDs) works on its own heads and keeps their K/V in its private L2.
#include <type_traits>

#include "attn_tile.h"

namespace attn {
namespace {

constexpr int kThreads = 512;    // fp32 kernel: 16 key slices of 32 lanes
constexpr int kQueryBlocks = 1;  // bf16 kernel: 32-row query blocks per wave
constexpr int kBN = 64;   // keys per LDS tile

template <int D, int PM, int QB, int NW>
__global__ __launch_bounds__(64 * NW) void tra_fwd_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, int BH, int T, int nqt,
    float beta, float p) {
    constexpr int BM = NW * 32 * QB;            // query rows per workgroup
    constexpr int ROWB = D * 2;                 // bytes per key row
    constexpr int CH = D / 8;                   // 16-byte chunks per row
    constexpr int TILEB = kBN * ROWB;           // bytes of one K (or V) tile
    constexpr int LOADS = kBN * CH / (64 * NW); // 16-byte chunks per thread per tensor
    constexpr int NDS = D / 16;                 // S^T MFMA k-steps
    constexpr int NDT = D / 32;                 // 32-dim output tiles
    constexpr bool kPlainOrder = D == 64 && PM == kPowGeneral;  // see the tile body
    static_assert(LOADS >= 1 && kBN * CH % (64 * NW) == 0, "tile staging");
    static_assert(TILEB == NW * LOADS * 1024, "one 1 KB DMA block per wave and chunk");

    // Two LDS buffers, each holding the K and V tiles of one 64-key tile: tile n
    // lives in lds_a when n is even and in lds_b when n is odd, and is fetched one
    // tile ahead, while the previous tile is being consumed.
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][TILEB];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][TILEB];
    typedef uint8_t TileBuf[2][TILEB];

    int bh, qt;
    tile_order(blockIdx.x, BH, nqt, bh, qt);
    // workgroup-uniform: keep them (and the buffer resources built from them) scalar
    bh = __builtin_amdgcn_readfirstlane(bh);
    qt = __builtin_amdgcn_readfirstlane(qt);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const size_t slab = (size_t)bh * T * D;

    // this wave's rows: qw0 + 32*qb + l32, qb < QB
    const int q0 = qt * BM;
    const int qw0 = q0 + wave * 32 * QB;
    const int q_last = min(q0 + BM, T) - 1;
    const int ntiles = q_last / kBN + 1;

    // Causal mask of one 32-key block starting at kbase (only for blocks that reach
    // past this wave's first row): register r holds key kbase + 8*(r/4) + 4*hi + r%4.
    auto mask_block = [&](f32x16 (&sv)[QB], int kbase) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int lim = qw0 + 32 * qb + l32 - kbase - 4 * hi;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + (r & 3) > lim) sv[qb][r] = -INFINITY;
        }
    };

    f32x16 oacc[QB][NDT];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][dt][r] = 0.0f;

    // Staging: K and V tiles go from HBM straight into LDS (buffer_load ... lds).
    // Instruction j of wave w fills LDS bytes [(w*LOADS + j)*1024, +1024) of a tile,
    // lane i the 16 bytes at +16*i; the lane loads the global chunk that the
    // swizzle puts there.  Rows at or past T read as zero (buffer range check).
    const u32x4 rk = make_rsrc(K + slab, (uint32_t)T * ROWB);
    const u32x4 rv = make_rsrc(V + slab, (uint32_t)T * ROWB);
    int dma_src[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int pos = (wave * LOADS + j) * 1024 + lane * 16;
        const int row = pos / ROWB, slot = (pos % ROWB) >> 4;
        dma_src[j] = row * ROWB + ((slot ^ tile_swz<D>(row)) << 4);
    }
    auto gload = [&](int n, TileBuf &dst) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            dma16(rk, &dst[0][(wave * LOADS + j) * 1024], dma_src[j], n * TILEB);
            dma16(rv, &dst[1][(wave * LOADS + j) * 1024], dma_src[j], n * TILEB);
        }
    };

    // operand read offsets (bytes within a tile)
    int koff[NDS];  // K row kb*32 + l32, chunk 2*ds + hi
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) koff[ds] = l32 * ROWB + (((2 * ds + hi) ^ tile_swz<D>(l32)) << 4);
    const int g16 = lane >> 4, s16 = lane & 15;
    const int vrow = 4 * (g16 >> 1) + (s16 >> 2);  // + kb*32 + 16c, + 8 for the upper keys
    int voff[NDT][2];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = vrow + 8 * h;
            voff[dt][h] = row * ROWB +
                          (((4 * dt + 2 * (g16 & 1) + ((s16 & 3) >> 1)) ^ tile_swz<D>(row)) << 4) +
                          8 * (s16 & 1);
        }

    auto k_frag = [&](const TileBuf &t, int kb, int ds) {
        return *(const bf16x8 *)(&t[0][koff[ds] + kb * 32 * ROWB]);
    };
    // V^T operand for keys kb*32 + 16c + {4hi..4hi+3, 8+4hi..8+4hi+3}, dims 32dt + lane%32
    auto v_frag = [&](const TileBuf &t, int kb, int dt, int c) {
        const uint8_t *base = &t[1][(kb * 32 + 16 * c) * ROWB];
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + voff[dt][0]));
        const bf16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + voff[dt][1]));
        return (bf16x8)__builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // weights of one S^T block (threshold and mask already applied), rounded to bf16
    // in the register order of the two P^T operands
    auto epilogue = [&](const f32x16 &sv, bf16x8 (&pf)[2]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (__bf16)relu_pow<PM>(sv[r], p);
    };

    // End-of-tile synchronisation: each wave waits for its own DMAs (the next tile)
    // and its own LDS reads (of this tile), then all waves meet.  After the barrier
    // the next tile is complete in LDS and nobody reads the buffer that the next
    // DMA overwrites.
    auto tile_sync = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) expcnt(7) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
    };

    gload(0, lds_a);
    // Q^T operands and thresholds (loaded while the first tile streams in)
    bf16x8 qf[QB][NDS];
    float tau[QB];
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int myq = qw0 + 32 * qb + l32;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            u32x4 r = zero4;
            if (myq < T) r = *(const u32x4 *)(Q + slab + (size_t)myq * D + ds * 16 + hi * 8);
            qf[qb][ds] = as_bf16x8(r);
        }
        tau[qb] = beta * sqrtf(2.0f * logf((float)(myq + 1)) / (float)D);
    }

    // S^T accumulators start from -tau of the lane's row, so the epilogue never
    // subtracts the threshold.
    f32x16 cinit[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) cinit[qb][r] = -tau[qb];
    // Drain everything once: the first tiles have landed and the Q operands are in
    // registers, so nothing issued before the loop is waited on inside it.
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();

    // One 64-key tile = two 32-key blocks, in four phases:
    //   A: S0 = -tau + K0 Q^T               (DMA of the next tile issued)
    //   B: S1 = -tau + K1 Q^T || epilogue(S0)
    //   C: O += V0 P0         || epilogue(S1)
    //   D: O += V1 P1
    auto tile = [&](int n, auto masked, const TileBuf &buf, TileBuf &next) {
        constexpr bool kMasked = decltype(masked)::value;
        if constexpr (kPlainOrder) {
            // general power at D = 64: the weights cost a log and an exp each, more
            // vector work than the phase interleave below leaves room for; each 32-key
            // block is done in order and the compiler interleaves freely
            if (n + 1 < ntiles) gload(n + 1, next);
            if constexpr (kMasked) {
                if (n * kBN > qw0 + 32 * QB - 1) {
                    tile_sync();
                    return;
                }
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 sv[QB];
                bf16x8 pf[QB][2];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sv[qb] = cinit[qb];
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) {
                    const bf16x8 kf = k_frag(buf, kb, ds);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) sv[qb] = mfma_32x32x16(kf, qf[qb][ds], sv[qb]);
                }
                if constexpr (kMasked) mask_block(sv, n * kBN + 32 * kb);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) epilogue(sv[qb], pf[qb]);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const bf16x8 vfr = v_frag(buf, kb, dt, c);
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb)
                            oacc[qb][dt] = mfma_32x32x16(vfr, pf[qb][c], oacc[qb][dt]);
                    }
            }
            tile_sync();
            return;
        }
        bf16x8 ka[NDS], kb1[NDS], va[NDT][2], vb[NDT][2];
        f32x16 s0[QB], s1[QB];
        bf16x8 p0[QB][2], p1[QB][2];
        // A
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) ka[ds] = k_frag(buf, 0, ds);
        if (n + 1 < ntiles) gload(n + 1, next);
        if constexpr (kMasked) {
            // every key of the tile lies after every row of this wave: nothing to add
            if (n * kBN > qw0 + 32 * QB - 1) {
                tile_sync();
                return;
            }
        }
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) kb1[ds] = k_frag(buf, 1, ds);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s0[qb] = cinit[qb];
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s0[qb] = mfma_32x32x16(ka[ds], qf[qb][ds], s0[qb]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kMasked) mask_block(s0, n * kBN);
        // B (raised issue priority until C; at D = 128 only from the S1 products on,
        // since raising it before the V operand reads makes the compiler spill)
        if constexpr (D != 128) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int c = 0; c < 2; ++c) va[dt][c] = v_frag(buf, 0, dt, c);
        if constexpr (D == 128) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s1[qb] = cinit[qb];
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s1[qb] = mfma_32x32x16(kb1[ds], qf[qb][ds], s1[qb]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) epilogue(s0[qb], p0[qb]);
#pragma unroll
        for (int i = 0; i < NDS * QB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // then VALU
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // then an LDS read
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kMasked) mask_block(s1, n * kBN + 32);
        // C
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int c = 0; c < 2; ++c) vb[dt][c] = v_frag(buf, 1, dt, c);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    oacc[qb][dt] = mfma_32x32x16(va[dt][c], p0[qb][c], oacc[qb][dt]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) epilogue(s1[qb], p1[qb]);
#pragma unroll
        for (int i = 0; i < NDT * 2 * QB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // D
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    oacc[qb][dt] = mfma_32x32x16(vb[dt][c], p1[qb][c], oacc[qb][dt]);
        tile_sync();
    };
    // Tiles entirely at or below this wave's first row need no mask; the rest
    // (diagonal, past the wave's rows, or past T) take the masked body.  Every wave
    // runs ntiles iterations, so the barriers stay matched.
    const int n_interior = min(ntiles, (qw0 + 1) / kBN);
    const std::false_type plain{};
    const std::true_type masked{};
    int n = 0;
    for (; n + 1 < n_interior; n += 2) {
        tile(n, plain, lds_a, lds_b);
        tile(n + 1, plain, lds_b, lds_a);
    }
    if (n < n_interior) tile(n++, plain, lds_a, lds_b);
    if (n < ntiles && (n & 1)) tile(n++, masked, lds_b, lds_a);
    for (; n + 1 < ntiles; n += 2) {
        tile(n, masked, lds_a, lds_b);
        tile(n + 1, masked, lds_b, lds_a);
    }
    if (n < ntiles) tile(n++, masked, lds_a, lds_b);

    // O^T accumulator: lane holds row qw0 + 32*qb + l32, dims 32*dt + 8*i + 4*hi + j.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int myq = qw0 + 32 * qb + l32;
        if (myq < T) {
            uint16_t *orow = O + slab + (size_t)myq * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x2 pr = {pack_bf16x2(oacc[qb][dt][4 * i], oacc[qb][dt][4 * i + 1]),
                                      pack_bf16x2(oacc[qb][dt][4 * i + 2], oacc[qb][dt][4 * i + 3])};
                    *(u32x2 *)(orow + dt * 32 + 8 * i + 4 * hi) = pr;
                }
        }
    }
}

// fp32 kernel: 8 query rows per workgroup of 512 threads; each group of 32 lanes (a
// key slice, two per wave) takes one sixteenth of every 64-key tile for all 8 rows
// (4 lanes per row, each a quarter of the head dim), and the sixteen partial outputs
// are summed through LDS at the end, in slice order.  K/V tiles of 64 keys are staged
// in LDS; all arithmetic is fp32.
template <int D, int PM>
__global__ __launch_bounds__(kThreads) void tra_fwd_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, int T, int nqt, float beta, float p) {
    constexpr int BQ = kTraF32Rows, BK = 64, DPT = D / 4;
    constexpr int NSL = kThreads / (BQ * 4);     // key slices per workgroup
    constexpr int KS = BK / NSL;                 // keys of a tile per slice
    static_assert(NSL * BQ * 4 == kThreads && KS % 4 == 0, "slices");
    static_assert(NSL * BQ * D <= 2 * BK * D, "the reduction reuses the K and V tiles");
    __shared__ __attribute__((aligned(16))) float KVsh[2][BK][D];
    float (&Ksh)[BK][D] = KVsh[0];
    float (&Vsh)[BK][D] = KVsh[1];

    const int bh = blockIdx.x / nqt;
    const int qt = nqt - 1 - blockIdx.x % nqt;
    const int tid = threadIdx.x;
    const int part = tid & 3;
    const int row = (tid >> 2) % BQ;
    const int slice = tid / (BQ * 4);
    const int my_q = qt * BQ + row;
    const size_t slab = (size_t)bh * T * D;

    float qv[DPT], acc[DPT];
#pragma unroll
    for (int d = 0; d < DPT; ++d) {
        qv[d] = my_q < T ? Q[slab + (size_t)my_q * D + part * DPT + d] : 0.0f;
        acc[d] = 0.0f;
    }
    const float tau = beta * sqrtf(2.0f * logf((float)(my_q + 1)) / (float)D);
    const int q_last = min(qt * BQ + BQ, T) - 1;

    // K/V tile staging: 16-byte pieces, all of a thread's loads issued before its LDS
    // stores, and the next tile's loads issued before the current tile is computed
    constexpr int PER = BK * D / 4 / kThreads;  // 4-float pieces per thread per tensor
    static_assert(BK * D % (4 * kThreads) == 0, "tile staging");
    // native 4-float vectors: with HIP's float4 struct the prefetched pieces went
    // through private memory
    f32x4 kr[PER], vr[PER];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = (tid + i * kThreads) * 4;
            const int key = k0 + e / D;
            const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            kr[i] = key < T ? *(const f32x4 *)(K + slab + (size_t)key * D + e % D) : z;
            vr[i] = key < T ? *(const f32x4 *)(V + slab + (size_t)key * D + e % D) : z;
        }
    };
    fetch(0);
    for (int k0 = 0; k0 <= q_last; k0 += BK) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = (tid + i * kThreads) * 4;
            *(f32x4 *)(&Ksh[e / D][e % D]) = kr[i];
            *(f32x4 *)(&Vsh[e / D][e % D]) = vr[i];
        }
        __syncthreads();
        if (k0 + BK <= q_last) fetch(k0 + BK);
        // this slice's keys, four per step: four independent dot-product chains, then
        // the weighted rows added in key order; keys past the row get weight 0
        const int j0 = slice * KS;
        if (k0 + j0 <= q_last) {
            for (int j = j0; j < j0 + KS; j += 4) {
                float sc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int d = 0; d < DPT; ++d)
#pragma unroll
                    for (int u = 0; u < 4; ++u) sc[u] = fmaf(qv[d], Ksh[j + u][part * DPT + d], sc[u]);
                float w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float x = sc[u] + __shfl_xor(sc[u], 1);
                    x += __shfl_xor(x, 2);
                    w[u] = k0 + j + u > my_q ? 0.0f : relu_pow<PM>(x - tau, p);
                }
#pragma unroll
                for (int d = 0; d < DPT; ++d)
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc[d] = fmaf(w[u], Vsh[j + u][part * DPT + d], acc[d]);
            }
        }
    }
    // sum the slices' partial outputs (in slice order) through the K tile's LDS
    __syncthreads();
    float *red = &KVsh[0][0][0];  // [slice][row][D]
#pragma unroll
    for (int d = 0; d < DPT; ++d) red[(slice * BQ + row) * D + part * DPT + d] = acc[d];
    __syncthreads();
    if (slice == 0 && my_q < T) {
#pragma unroll
        for (int d = 0; d < DPT; ++d) {
            float o = red[row * D + part * DPT + d];
#pragma unroll
            for (int sl = 1; sl < NSL; ++sl) o += red[(sl * BQ + row) * D + part * DPT + d];
            O[slab + (size_t)my_q * D + part * DPT + d] = o;
        }
    }
}

template <int D, int PM>
hipError_t launch_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *out,
                       int BH, int T, float beta, float p, hipStream_t stream) {
    constexpr int NW = tra_bf16_waves(D), ROWS = tra_bf16_rows(D);
    static_assert(NW * 32 * kQueryBlocks == ROWS, "workgroup rows");
    int nqt = (T + ROWS - 1) / ROWS;
    void *args[] = {&q, &k, &v, &out, &BH, &T, &nqt, &beta, &p};
    return hipLaunchKernel((const void *)tra_fwd_bf16_kernel<D, PM, kQueryBlocks, NW>,
                           dim3((unsigned)(BH * nqt)), dim3(64 * NW), args, 0, stream);
}

template <int D, int PM>
hipError_t launch_f32(const float *q, const float *k, const float *v, float *out, int BH,
                      int T, float beta, float p, hipStream_t stream) {
    int nqt = (T + kTraF32Rows - 1) / kTraF32Rows;
    void *args[] = {&q, &k, &v, &out, &T, &nqt, &beta, &p};
    return hipLaunchKernel((const void *)tra_fwd_f32_kernel<D, PM>,
                           dim3((unsigned)(BH * nqt)), dim3(kThreads), args, 0, stream);
}


}  // namespace

hipError_t launch_tra_fwd_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               uint16_t *out, int BH, int T, int D, float beta, float p,
                               hipStream_t stream) {
    const int pm = pow_mode(p);
    if (D == 128) {
        if (pm == kPowTwo) return launch_bf16<128, kPowTwo>(q, k, v, out, BH, T, beta, p, stream);
        if (pm == kPowOne) return launch_bf16<128, kPowOne>(q, k, v, out, BH, T, beta, p, stream);
        if (pm == kPowThreeHalves) return launch_bf16<128, kPowThreeHalves>(q, k, v, out, BH, T, beta, p, stream);
        return launch_bf16<128, kPowGeneral>(q, k, v, out, BH, T, beta, p, stream);
    }
    if (pm == kPowTwo) return launch_bf16<64, kPowTwo>(q, k, v, out, BH, T, beta, p, stream);
    if (pm == kPowOne) return launch_bf16<64, kPowOne>(q, k, v, out, BH, T, beta, p, stream);
    if (pm == kPowThreeHalves) return launch_bf16<64, kPowThreeHalves>(q, k, v, out, BH, T, beta, p, stream);
    return launch_bf16<64, kPowGeneral>(q, k, v, out, BH, T, beta, p, stream);
}

hipError_t launch_tra_fwd_f32(const float *q, const float *k, const float *v, float *out,
                              int BH, int T, int D, float beta, float p, hipStream_t stream) {
    const int pm = pow_mode(p);
    if (D == 128) {
        if (pm == kPowTwo) return launch_f32<128, kPowTwo>(q, k, v, out, BH, T, beta, p, stream);
        if (pm == kPowOne) return launch_f32<128, kPowOne>(q, k, v, out, BH, T, beta, p, stream);
        if (pm == kPowThreeHalves) return launch_f32<128, kPowThreeHalves>(q, k, v, out, BH, T, beta, p, stream);
        return launch_f32<128, kPowGeneral>(q, k, v, out, BH, T, beta, p, stream);
    }
    if (pm == kPowTwo) return launch_f32<64, kPowTwo>(q, k, v, out, BH, T, beta, p, stream);
    if (pm == kPowOne) return launch_f32<64, kPowOne>(q, k, v, out, BH, T, beta, p, stream);
    if (pm == kPowThreeHalves) return launch_f32<64, kPowThreeHalves>(q, k, v, out, BH, T, beta, p, stream);
    return launch_f32<64, kPowGeneral>(q, k, v, out, BH, T, beta, p, stream);
}

}  // namespace attn
