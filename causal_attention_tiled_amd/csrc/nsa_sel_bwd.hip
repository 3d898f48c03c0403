// nsa_sel_bwd.hip -- NSA selection-branch backward for gfx950.
//
// The gradients of the selection forward (msb-msb/openbox-llm, page
// "nsa_selection_kernel.py": module docstring, `selection_forward_reference`,
// `_selection_fwd_kernel`) with respect to q, k and v; the page keeps the lse
// output for such a backward but does not show one.  With A_i the attended set of
// query i (its selected blocks' tokens j <= i, duplicates once), s_ij = scale
// q_i.k_j, P_ij = exp(s_ij - lse_i), dP_ij = dout_i.v_j, delta_i = sum_j P_ij dP_ij
// and dS_ij = P_ij (dP_ij - delta_i), for every head h of kv
// group kv = h / G:
//     dq_i = scale sum_{j in A_i} dS_ij k_j
//     dk_j = scale sum_{h, i : j in A_i} dS_ij q_i,   dv_j = sum_{h, i : j in A_i} P_ij dout_i
//
// Kernels (all on the caller's stream, workspace from the caller):
//  * The selection inverted (nsa_index.hip): for each (group, block) the increasing
//    list of queries that attend it, cut into segments of at most kNsaSegQ queries.
//  * dq: one wavefront per (group, query), as the forward (kept blocks walked in
//    decreasing block order): the G heads fill the N
//    dimension of 16x16x32 MFMAs, S^T = K Q^T and dP^T = V dO^T per 32-key chunk,
//    P = exp2(S' - lse') from the forward's lse, dS^T rounded to bf16 in register
//    order, and dQ^T += K^T (.)^T.  K and V rows go by DMA, whole rows per
//    instruction, into one K and one V tile of LDS per wave; the K tile serves both
//    the K operand (row reads) and K^T (transposing reads).  Each chunk's operands
//    are all read into registers first, so the next chunk's transfers go into the
//    same tiles right away (16 KB of LDS per wave: 8 waves per compute unit).  delta is needed before the first dS and is only known after the
//    last key, and dout . out from the forward's bf16 output is too coarse a value for
//    dP - delta, which cancels.  So one pass accumulates, against the estimate
//    m = dout . out, X = sum_j bf16(P_j (dP_j - m)) k_j, Y = sum_j bf16(P_j) k_j and
//    delta = sum_j P_j dP_j in fp32, and ends with dq = scale (X - (delta - m) Y): the
//    correction term is small, so its bf16 operand costs nothing, and the rounding
//    of the main term is the rounding of dS itself.  The kernel writes delta per
//    (head, query) for the next kernel.
//  * dk/dv: one workgroup per segment of a (group, block) list, one wavefront per 32
//    keys of the block holding its K and V rows in registers, the segment's queries
//    walked in chunks of 32 rows (query, head): their Q and dO rows are gathered into
//    LDS by the memory unit, up to three chunks ahead, with lse, delta and position in
//    a small table.  S = Q K^T and dP = dO V^T (one key per lane), then dV^T += dO^T P
//    and dK^T += Q^T dS with dO^T and Q^T read transposed from LDS; the chunk loop is
//    software-pipelined (S and dP of the next chunk are issued before this chunk's
//    products, its weights after them).  A list of one
//    segment writes its key rows; a longer list writes fp32 partials that a reduce
//    kernel sums in segment order.  Each key row has one writer: deterministic.
#include <algorithm>
#include <type_traits>

#include "attn_tile.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunk = 32;  // keys per processed chunk in the dq kernel
constexpr int kDqWaves = 4;

typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t bwd_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ void bwd_dma16(__amdgpu_buffer_rsrc_t r, void *lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, soff, 0, 0);
}

// LDS K chunk (32 rows x D*2 bytes): 16-byte piece c of row r at slot c ^ swz(r).  At
// D = 128 (one row per 256-byte bank line) the 16 rows x 16 bytes that 16 lanes read
// for the K operand, and the 8 rows x 32 bytes that 32 lanes read transposed for the
// K^T operand, each cover all 64 banks once.
template <int D>
__host__ __device__ constexpr int chunk_swz(int row) {
    if constexpr (D == 128)
        return ((row & 7) << 1) | ((row >> 3) & 1);
    else
        return ((row >> 1) & 3) << 1;
}

// ---------------------------------------------------------------------------
// dq (query-outer) and delta
// ---------------------------------------------------------------------------

template <int D, int BS>
__global__ __launch_bounds__(64 * kDqWaves) void nsa_bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ IDX,
    const uint16_t *__restrict__ O, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, uint16_t *__restrict__ dQ, float *__restrict__ DELTA,
    int Hq, int Hkv, int G, int T, int S, int nq4, int ngroups, float score_scale, float scale) {
    constexpr int ROWB = D * 2;
    constexpr int NCH = BS / kChunk;
    constexpr int NDS = D / 32;              // k-steps of S^T and dP^T
    constexpr int NDT = D / 16;              // 16-dim tiles of dQ^T
    constexpr int KTILE = kChunk * ROWB;
    constexpr int KDMA = KTILE / 1024;
    static_assert(BS % kChunk == 0 && KTILE % 1024 == 0, "chunking");

    __shared__ __attribute__((aligned(16))) uint8_t kbuf[kDqWaves][KTILE];
    __shared__ __attribute__((aligned(16))) uint8_t vbuf[kDqWaves][KTILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    const int W = ngroups * nq4;
    int f = blockIdx.x;
    if ((W & 7) == 0) f = (blockIdx.x & 7) * (W >> 3) + (blockIdx.x >> 3);
    const int group = __builtin_amdgcn_readfirstlane(f / nq4);
    const int i = __builtin_amdgcn_readfirstlane((nq4 - 1 - f % nq4) * kDqWaves + wave);
    if (i >= T) return;  // no workgroup-wide barrier in this kernel
    const int b = group / Hkv, kv = group % Hkv;
    const size_t kvslab = (size_t)group * T * D;
    const __amdgpu_buffer_rsrc_t rk = bwd_rsrc(K + kvslab, (uint32_t)T * ROWB);
    const __amdgpu_buffer_rsrc_t rv = bwd_rsrc(V + kvslab, (uint32_t)T * ROWB);

    const int nblk = T / BS;
    const int32_t *slots = IDX + ((size_t)group * T + i) * S;
    const int myblk = lane < S ? slots[lane] : -1;
    bool keep = myblk >= 0 && myblk < nblk && myblk * BS <= i;
    for (int s2 = 0; s2 < S; ++s2) {
        const int other = __builtin_amdgcn_readlane(myblk, s2);
        keep = keep && !(s2 < lane && other == myblk);
    }
    // The kept blocks are visited in decreasing block order, as in the forward (lane s's
    // rank = the number of kept blocks above its own): the waves of neighbouring queries
    // then read nearby blocks at the same time, which keeps more of them in L2.
    const uint64_t kept = __builtin_amdgcn_ballot_w64(keep);
    const int nkept = __builtin_popcountll(kept);
    int rank = 0;
    for (int s2 = 0; s2 < S; ++s2) {
        const int other = __builtin_amdgcn_readlane(myblk, s2);
        rank += (int)(((kept >> s2) & 1) != 0 && other > myblk);
    }
    int taken = 0;

    // Q^T and dO^T operands: head kv*G + n16 (zero for n16 >= G), dims 32*ds + 8*g4 .. +7
    const bool head_ok = n16 < G;
    const int head = kv * G + (head_ok ? n16 : 0);
    const size_t qrow = ((size_t)(b * Hq + head) * T + i) * D;
    bf16x8 qf[NDS], df[NDS];
    float m = 0.0f;  // dout . out of head n16, the estimate of delta
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            u32x4 a = z, c = z, o = z;
            if (head_ok) {
                a = *(const u32x4 *)(Q + qrow + ds * 32 + g4 * 8);
                c = *(const u32x4 *)(dO + qrow + ds * 32 + g4 * 8);
                o = *(const u32x4 *)(O + qrow + ds * 32 + g4 * 8);
            }
            qf[ds] = as_bf16x8(a);
            df[ds] = as_bf16x8(c);
            const bf16x8 of = as_bf16x8(o);
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaf((float)df[ds][e], (float)of[e], m);
        }
        m += __shfl_xor(m, 16);
        m += __shfl_xor(m, 32);
    }
    const float lse2 = head_ok ? LSE[(size_t)(b * Hq + head) * T + i] * kLog2e : 0.0f;

    int kdma_off[KDMA];  // K and V tiles alike
#pragma unroll
    for (int j = 0; j < KDMA; ++j) {
        const int pos = j * 1024 + lane * 16;
        const int row = pos / ROWB, slot = (pos % ROWB) >> 4;
        kdma_off[j] = row * ROWB + ((slot ^ chunk_swz<D>(row)) << 4);
    }
    // K^T operand reads: rows 4*g4 + s/4 (and 16 rows further, same swizzle), dims
    // 16*dt + 4*(s%4)
    static_assert(chunk_swz<D>(16) == chunk_swz<D>(0), "upper keys: same swizzle");
    int krd_off[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        const int row = 4 * g4 + (n16 >> 2);
        const int col = 16 * dt + 4 * (n16 & 3);
        krd_off[dt] = row * ROWB + (((col >> 3) ^ chunk_swz<D>(row)) << 4) + (col & 7) * 2;
    }

    // K rows as A operands of S^T, read from the LDS copy: row 16*kk + n16, dims
    // 32*ds + 8*g4 (the kk = 1 rows 16 rows further, same swizzle)
    int krow_off[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
        krow_off[ds] = n16 * ROWB + (((4 * ds + g4) ^ chunk_swz<D>(n16)) << 4);

    // V rows (A operands of dP^T) through an LDS tile of the same layout as K's: each
    // DMA instruction moves whole rows, where loads in the operand layout would touch
    // 16 rows at 64 bytes each
    auto load_chunk = [&](int k0) {
#pragma unroll
        for (int j = 0; j < KDMA; ++j) bwd_dma16(rv, &vbuf[wave][j * 1024], kdma_off[j], k0 * ROWB);
#pragma unroll
        for (int j = 0; j < KDMA; ++j) bwd_dma16(rk, &kbuf[wave][j * 1024], kdma_off[j], k0 * ROWB);
    };
    // S^T and dP^T of one chunk: register j of st[kk] / dp[kk] is key k0 + 16*kk + 4*g4 + j,
    // head n16; returns the probabilities (0 for keys after i) in pr
    auto scores = [&](int k0, const bf16x8 (&kf)[2][NDS], const bf16x8 (&vf)[2][NDS],
                      f32x4 (&pr)[2], f32x4 (&dp)[2]) {
        f32x4 st[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            st[kk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            dp[kk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                st[kk] = mfma_16x16x32(kf[kk][ds], qf[ds], st[kk]);
                dp[kk] = mfma_16x16x32(vf[kk][ds], df[ds], dp[kk]);
            }
        }
        const int lim = i - k0 - 4 * g4;  // key offset 16*kk + j is attended iff <= lim
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float e = __builtin_amdgcn_exp2f(st[kk][j] * score_scale - lse2);
                pr[kk][j] = 16 * kk + j > lim ? 0.0f : e;
            }
    };

    // register j of xacc[dt] / yacc[dt] is dim 16*dt + 4*g4 + j, head n16
    f32x4 xacc[NDT], yacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        xacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        yacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    float dl = 0.0f;  // this lane's part of delta
    int cur_blk = -1, cur_c = 0;
    auto next_chunk = [&]() -> int {
        if (cur_blk >= 0 && cur_c + 1 < NCH && cur_blk * BS + (cur_c + 1) * kChunk <= i) {
            ++cur_c;
            return cur_blk * BS + cur_c * kChunk;
        }
        if (taken == nkept) return -1;
        const int s = __builtin_ctzll(__builtin_amdgcn_ballot_w64(keep && rank == taken));
        ++taken;
        cur_blk = __builtin_amdgcn_readlane(myblk, s);
        cur_c = 0;
        return cur_blk * BS;
    };

    // One stage per chunk: every operand of the chunk (V and K rows, K^T) is read from
    // its LDS tiles first -- after all of this wave's transfers, which are then exactly
    // this chunk's -- and the next chunk's transfers go into the same tiles right after,
    // with the whole stage to land.
    auto compute_chunk = [&](int k0, int &nxt) {
        const uint32_t base = lds_addr(&kbuf[wave][0]);
        bf16x8 kf[2][NDS], vf[2][NDS], ktf[NDT];
        {
            const uint32_t vbase = lds_addr(&vbuf[wave][0]);
            uint32_t ad[4];
            u32x4 rd[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) ad[e] = vbase + krow_off[e % NDS];
            row_read4x2<0, 16 * ROWB>(rd, ad);
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                vf[0][ds] = as_bf16x8(rd[2 * ds]);
                vf[1][ds] = as_bf16x8(rd[2 * ds + 1]);
            }
        }
        {
            static_assert(NDS == 4 || NDS == 2, "K row reads");
            uint32_t ad[4];
            u32x4 rd[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) ad[e] = base + krow_off[e % NDS];
            row_read4x2<63, 16 * ROWB>(rd, ad);
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                kf[0][ds] = as_bf16x8(rd[2 * ds]);
                kf[1][ds] = as_bf16x8(rd[2 * ds + 1]);
            }
        }
        // K^T operands of X^T and Y^T: dims 16*dt + 4*g4 .. , keys 4*(n16%4) + .. (both halves)
#pragma unroll
        for (int d4 = 0; d4 < NDT; d4 += 4) {
            uint32_t ad[4];
            bf16x4_t rd[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) ad[e] = base + krd_off[d4 + e];
            tr_read4x2<63, 16 * ROWB>(rd, ad);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ktf[d4 + e] = __builtin_shufflevector(rd[2 * e], rd[2 * e + 1], 0, 1, 2, 3, 4, 5,
                                                      6, 7);
        }
        nxt = next_chunk();
        if (nxt >= 0) load_chunk(nxt);
        f32x4 pr[2], dp[2];
        scores(k0, kf, vf, pr, dp);
        bf16x8 xf, yf;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dl = fmaf(pr[kk][j], dp[kk][j], dl);
                xf[kk * 4 + j] = (__bf16)(pr[kk][j] * (dp[kk][j] - m));
                yf[kk * 4 + j] = (__bf16)pr[kk][j];
            }
        // X^T += K^T xf^T, Y^T += K^T yf^T
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            xacc[dt] = mfma_16x16x32(ktf[dt], xf, xacc[dt]);
            yacc[dt] = mfma_16x16x32(ktf[dt], yf, yacc[dt]);
        }
    };

    int cur = next_chunk();
    if (cur >= 0) {
        load_chunk(cur);
        while (cur >= 0) {
            int nxt;
            compute_chunk(cur, nxt);
            cur = nxt;
        }
    }

    dl += __shfl_xor(dl, 16);
    dl += __shfl_xor(dl, 32);
    const float corr = dl - m;
    if (head_ok) {
        if (g4 == 0) DELTA[(size_t)(b * Hq + head) * T + i] = dl;
        uint16_t *row = dQ + qrow;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            f32x4 r;
#pragma unroll
            for (int j = 0; j < 4; ++j) r[j] = scale * fmaf(-corr, yacc[dt][j], xacc[dt][j]);
            const u32x2 pk = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
            *(u32x2 *)(row + dt * 16 + g4 * 4) = pk;
        }
    }
}

// ---------------------------------------------------------------------------
// dk / dv (block-outer over the inverted CSR)
// ---------------------------------------------------------------------------


template <int D, int BS>
__global__ __launch_bounds__(64 * (BS / 32)) void nsa_bwd_dkv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ DELTA,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ list,
    const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_list,
    const int32_t *__restrict__ part_start, float *__restrict__ part, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, int Hq, int Hkv, int G, int T, int nblk, int nlists,
    float score_scale, float scale) {
    constexpr int NW = BS / 32;                  // one wave per 32 keys of the block
    constexpr int NBUF = BS == 32 ? 3 : 4;       // staged chunks (ring)
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    constexpr int TILEB = 32 * ROWB;             // 32 gathered rows of one tensor
    constexpr int LOADS = 32 * CH / (64 * NW);   // 16-byte chunks per lane per tensor
    constexpr int OPS = 2 * LOADS + 2;           // memory instructions per wave per chunk
    constexpr int NDS = D / 16;
    constexpr int NDT = D / 32;
    static_assert(LOADS >= 1 && 32 * CH % (64 * NW) == 0, "row staging");
    static_assert((NBUF - 2) * OPS < 64, "vmcnt range");

    // buffer u: Q rows at tile 2u, dO rows at tile 2u+1
    __shared__ __attribute__((aligned(16))) uint8_t lds[NBUF * 2 * TILEB];
    // per staged row: lse (natural), delta, query position (-1: no row)
    __shared__ __attribute__((aligned(16))) float rlse[NBUF][32];
    __shared__ __attribute__((aligned(16))) float rdelta[NBUF][32];
    __shared__ __attribute__((aligned(16))) int rpos[NBUF][32];
    __shared__ int qpos[kNsaSegQ];

    // workgroup -> segment in list order (group, then block): the workgroups in flight
    // work on one kv group at a time, whose gathered q rows (G*T rows per group) are
    // then the working set of the memory-side cache, and the heavily attended early
    // blocks of each group come first
    const int seg_total = seg_start[nlists];
    const int sidx = blockIdx.x;
    if (sidx >= seg_total) return;  // whole workgroup, before any barrier
    const int l = __builtin_amdgcn_readfirstlane(seg_list[sidx]);
    const int seg = sidx - seg_start[l];
    const bool multi = seg_start[l + 1] - seg_start[l] > 1;
    const int group = l / nblk, blk = l % nblk;
    const int b = group / Hkv, kv = group % Hkv;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const size_t kvslab = (size_t)group * T * D;
    const int kw0 = blk * BS + 32 * wave;        // this wave's keys
    const int mykey = kw0 + l32;

    const int lbeg = offsets[l] + seg * kNsaSegQ;
    const int nq = min(kNsaSegQ, offsets[l + 1] - lbeg);
    const int qc = 32 / G;                       // queries per chunk of rows
    const int rows_used = qc * G;
    const int nchunks = (nq + qc - 1) / qc;

    // K and V rows of this wave's keys as B operands (before any DMA: in-order waits)
    bf16x8 kf[NDS], vf[NDS];
    {
        const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            u32x4 a = zero4, c = zero4;
            if (mykey < T) {
                a = *(const u32x4 *)(K + kvslab + (size_t)mykey * D + ds * 16 + hi * 8);
                c = *(const u32x4 *)(V + kvslab + (size_t)mykey * D + ds * 16 + hi * 8);
            }
            kf[ds] = as_bf16x8(a);
            vf[ds] = as_bf16x8(c);
        }
    }
    for (int t = tid; t < nq; t += 64 * NW) qpos[t] = list[lbeg + t];

    // Q, dO, lse and delta of batch b: row (h, i) at (h*T + i)
    const size_t bslab = (size_t)b * Hq * T;
    const uint32_t bbytes = (uint32_t)((size_t)Hq * T * ROWB);
    const uint32_t tbytes = (uint32_t)((size_t)Hq * T * 4);
    const u32x4 rq = make_rsrc(Q + bslab * D, bbytes);
    const u32x4 ro = make_rsrc(dO + bslab * D, bbytes);
    const u32x4 rl = make_rsrc(LSE + bslab, tbytes);
    const u32x4 rd = make_rsrc(DELTA + bslab, tbytes);

    // staging positions: DMA instruction j of wave w fills tile bytes
    // [(w*LOADS + j)*1024, +1024); lane l the 16 bytes at +16*l, i.e. row r = pos / ROWB
    // and chunk slot; it fetches chunk slot ^ swz(r) of that row's source
    int srow[LOADS], sslot[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int pos = (wave * LOADS + j) * 1024 + lane * 16;
        srow[j] = pos / ROWB;
        sslot[j] = ((pos % ROWB) >> 4) ^ tile_swz<D>(pos / ROWB);
    }
    // OPS memory instructions per wave: LOADS for Q, LOADS for dO, lse, delta.  Row r of
    // chunk c is query qpos[c*qc + r/G], head kv*G + r%G; absent rows read as zero.
    auto stage = [&](int c, int u) {
        int off[LOADS];  // all query positions read first (one LDS wait), then the DMAs
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int r = srow[j];
            const int qi = c * qc + r / G;
            const bool ok = r < rows_used && qi < nq;
            const int pos = qpos[ok ? qi : 0];  // c < nchunks, so nq > 0
            off[j] = ok ? ((kv * G + r % G) * T + pos) * ROWB + (sslot[j] << 4) : (int)bbytes;
        }
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int dst = (wave * LOADS + j) * 1024;
            dma16(rq, &lds[(2 * u) * TILEB + dst], off[j], 0);
            dma16(ro, &lds[(2 * u + 1) * TILEB + dst], off[j], 0);
        }
        if (lane < 32) {  // every wave writes the same table entries
            const int qi = c * qc + lane / G;
            int toff = (int)tbytes, pos = -1;
            if (lane < rows_used && qi < nq) {
                pos = qpos[qi];
                toff = ((kv * G + lane % G) * T + pos) * 4;
            }
            dma4(rl, &rlse[u][0], toff, 0);
            dma4(rd, &rdelta[u][0], toff, 0);
            rpos[u][lane] = pos;
        }
    };

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
    // LDS operand reads are issued in groups of eight per statement (tr_read4x2,
    // row_read4x2), so one wait covers eight reads and the products of a group run while
    // the next group is read.  Chunk tiles are complete before any of them (waited and
    // published by the barrier), hence vmcnt(63): no memory wait inside.
    const uint32_t lds0 = lds_addr(&lds[0]);
    static_assert(NDS % 4 == 0 && NDT % 2 == 0, "operand read groups");

    f32x16 dkacc[NDT], dvacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkacc[dt][r] = dvacc[dt][r] = 0.0f;
    f32x16 zero16;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero16[r] = 0.0f;

    // K and V rows and the query list are in: waited here once, so that no wait for
    // them (which would also drain the staged chunks) lands inside the loop
    wait_vm<0>();
    __syncthreads();  // qpos
    for (int c = 0; c < NBUF - 1 && c < nchunks; ++c) stage(c, c);

    // S = Q K^T and dP = dO V^T of chunk c (register r: row m = 8*(r/4) + 4*hi + r%4 of
    // the chunk, key mykey), then P and dS rounded to bf16 in the register order of the
    // B operands of dV^T += dO^T P and dK^T += Q^T dS
    auto scores = [&](int u, f32x16 &s, f32x16 &dp) {
        s = zero16;
        dp = zero16;
#pragma unroll
        for (int d4 = 0; d4 < NDS; d4 += 4) {
            uint32_t ad[4];
            u32x4 rd[8];  // rd[2e]: Q row piece d4+e, rd[2e+1]: the dO row piece
#pragma unroll
            for (int e = 0; e < 4; ++e) ad[e] = lds0 + 2 * u * TILEB + roff[d4 + e];
            row_read4x2<63, TILEB>(rd, ad);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s = mfma_32x32x16(as_bf16x8(rd[2 * e]), kf[d4 + e], s);
                dp = mfma_32x32x16(as_bf16x8(rd[2 * e + 1]), vf[d4 + e], dp);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // dV^T += dO^T P and dK^T += Q^T dS for chunk tile u
    auto products = [&](int u, const bf16x8 (&pb)[2], const bf16x8 (&sb)[2]) {
#pragma unroll
        for (int d2 = 0; d2 < NDT; d2 += 2)
#pragma unroll
            for (int t = 1; t >= 0; --t) {  // dO^T (dV) then Q^T (dK)
                uint32_t ad[4];
                bf16x4_t rd[8];  // rd[4e + 2h + c]: dim tile d2+e, half h, key group c
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int h = 0; h < 2; ++h) ad[2 * e + h] = lds0 + (2 * u + t) * TILEB + toff[d2 + e][h];
                tr_read4x2<63, 16 * ROWB>(rd, ad);
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const bf16x8 a = __builtin_shufflevector(rd[4 * e + c], rd[4 * e + 2 + c], 0, 1,
                                                                 2, 3, 4, 5, 6, 7);
                        if (t == 1) dvacc[d2 + e] = mfma_32x32x16(a, pb[c], dvacc[d2 + e]);
                        else dkacc[d2 + e] = mfma_32x32x16(a, sb[c], dkacc[d2 + e]);
                    }
                __builtin_amdgcn_sched_barrier(0);
            }
    };
    auto weights = [&](int u, const f32x16 &s, const f32x16 &dp, bf16x8 (&pb)[2],
                       bf16x8 (&sb)[2]) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 ls = *(const f32x4 *)(&rlse[u][8 * g + 4 * hi]);
            const f32x4 de = *(const f32x4 *)(&rdelta[u][8 * g + 4 * hi]);
            const i32x4 ps = *(const i32x4 *)(&rpos[u][8 * g + 4 * hi]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * g + j;
                float pr = __builtin_amdgcn_exp2f(s[r] * score_scale - ls[j] * kLog2e);
                if (mykey > ps[j]) pr = 0.0f;  // after the query (or no row: ps = -1)
                pb[r >> 3][r & 7] = (__bf16)pr;
                sb[r >> 3][r & 7] = (__bf16)(pr * (dp[r] - de[j]));
            }
        }
    };
    // wait until chunk c's transfers are in; the chunks staged after it may still be
    // outstanding, OPS instructions each: before the loop (c = 0) chunks 1 .. NBUF-2, and
    // when iteration c-1 waits for chunk c, chunks c+1 .. c+NBUF-3
    auto wait_chunk = [&](int c) {
        const int after = c > 0 ? min(NBUF - 3, nchunks - 1 - c) : min(NBUF - 2, nchunks - 1);
        if constexpr (NBUF >= 4) {
            if (after >= 2) wait_vm<2 * OPS>();
            else if (after == 1) wait_vm<OPS>();
            else wait_vm<0>();
        } else {
            if (after >= 1) wait_vm<OPS>();
            else wait_vm<0>();
        }
    };

    // Software pipeline over chunks: iteration c issues S and dP of chunk c+1, then the
    // dV/dK products of chunk c, then the weights of chunk c+1 (VALU work that runs while
    // chunk c's products occupy the matrix unit).
    bf16x8 pb[2], sb[2];
    if (nchunks > 0) {
        wait_chunk(0);
        __syncthreads();
        f32x16 s, dp;
        scores(0, s, dp);
        weights(0, s, dp, pb, sb);
    }
    for (int c = 0; c < nchunks; ++c) {
        const int u = c % NBUF, un = (c + 1) % NBUF;
        const bool more = c + 1 < nchunks;
        if (more) wait_chunk(c + 1);
        __syncthreads();  // chunk c+1 is in for every wave; chunk c-1 is consumed
        f32x16 s, dp;
        if (more) scores(un, s, dp);
        products(u, pb, sb);
        // staged behind the products, so its LDS reads and address work overlap them
        if (c + NBUF - 1 < nchunks) stage(c + NBUF - 1, (c + NBUF - 1) % NBUF);
        if (more) weights(un, s, dp, pb, sb);
    }

    if (mykey >= T) return;
    if (!multi) {
        uint16_t *krow = dK + kvslab + (size_t)mykey * D;
        uint16_t *vrow = dV + kvslab + (size_t)mykey * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const u32x2 kp = {pack_bf16x2(scale * dkacc[dt][4 * i4], scale * dkacc[dt][4 * i4 + 1]),
                                  pack_bf16x2(scale * dkacc[dt][4 * i4 + 2], scale * dkacc[dt][4 * i4 + 3])};
                const u32x2 vp = {pack_bf16x2(dvacc[dt][4 * i4], dvacc[dt][4 * i4 + 1]),
                                  pack_bf16x2(dvacc[dt][4 * i4 + 2], dvacc[dt][4 * i4 + 3])};
                *(u32x2 *)(krow + dt * 32 + 8 * i4 + 4 * hi) = kp;
                *(u32x2 *)(vrow + dt * 32 + 8 * i4 + 4 * hi) = vp;
            }
    } else {
        // fp32 partial of this segment: [2][BS][D], dK unscaled
        float *pk = part + (size_t)(part_start[l] + seg) * 2 * BS * D + (size_t)(32 * wave + l32) * D;
        float *pv = pk + BS * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = dt * 32 + 8 * i4 + 4 * hi;
                *(f32x4 *)(pk + d0) = f32x4{dkacc[dt][4 * i4], dkacc[dt][4 * i4 + 1],
                                            dkacc[dt][4 * i4 + 2], dkacc[dt][4 * i4 + 3]};
                *(f32x4 *)(pv + d0) = f32x4{dvacc[dt][4 * i4], dvacc[dt][4 * i4 + 1],
                                            dvacc[dt][4 * i4 + 2], dvacc[dt][4 * i4 + 3]};
            }
    }
}

// Lists split over several segments: dK = scale * (sum of the partials), dV = sum, in
// segment order.  (BS*D/1024) workgroups per list, 4 consecutive values per thread.
template <int D, int BS>
__global__ __launch_bounds__(256) void dkv_reduce_kernel(
    const float *__restrict__ part, const int32_t *__restrict__ seg_start,
    const int32_t *__restrict__ part_start, uint16_t *__restrict__ dK, uint16_t *__restrict__ dV,
    int T, int nblk, float scale) {
    constexpr int WPL = BS * D / 1024;
    const int l = blockIdx.x / WPL;
    const int ns = seg_start[l + 1] - seg_start[l];
    if (ns <= 1) return;
    const int e = ((blockIdx.x % WPL) * 256 + threadIdx.x) * 4;  // < BS*D
    const float *p = part + (size_t)part_start[l] * 2 * BS * D + e;
    f32x4 sk = {0.0f, 0.0f, 0.0f, 0.0f}, sv = sk;
    for (int s = 0; s < ns; ++s) {
        sk += *(const f32x4 *)(p + (size_t)s * 2 * BS * D);
        sv += *(const f32x4 *)(p + (size_t)s * 2 * BS * D + BS * D);
    }
    const int group = l / nblk, blk = l % nblk;
    const size_t o = ((size_t)group * T + blk * BS) * D + e;
    *(u32x2 *)(dK + o) = u32x2{pack_bf16x2(scale * sk[0], scale * sk[1]),
                               pack_bf16x2(scale * sk[2], scale * sk[3])};
    *(u32x2 *)(dV + o) = u32x2{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3])};
}

// Workspace: the inverted index, then delta [B*Hq*T] fp32, then the fp32 dk/dv partials
// of split lists ([max_part][2][BS][D]).
struct BwdLayout {
    NsaIndex ix;
    float *delta, *part;
    size_t total;
};

BwdLayout layout(void *ws, int B, int Hq, int Hkv, int T, int D, int bs, int S) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    BwdLayout L;
    size_t o;
    L.ix = nsa_index_carve(ws, B, Hkv, T, bs, S, &o);
    const size_t o_delta = o;
    o = al(o + (size_t)B * Hq * T * 4);
    const size_t o_part = o;
    o = al(o + (size_t)L.ix.max_part * 2 * bs * D * 4);
    L.total = o;
    uint8_t *w = static_cast<uint8_t *>(ws);
    L.delta = (float *)(w + o_delta);
    L.part = (float *)(w + o_part);
    return L;
}

template <int D, int BS>
hipError_t launch(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *idx,
                  const uint16_t *out, const float *lse, const uint16_t *dout, uint16_t *dq,
                  uint16_t *dk, uint16_t *dv, uint8_t *ws, int B, int Hq, int Hkv, int T, int S,
                  hipStream_t stream) {
    const BwdLayout L = layout(ws, B, Hq, Hkv, T, D, BS, S);
    const int32_t *offsets = L.ix.offsets, *list = L.ix.list, *seg_start = L.ix.seg_start;
    const int32_t *seg_list = L.ix.seg_list, *part_start = L.ix.part_start;
    float *delta = L.delta, *part = L.part;
    int nblk = T / BS;
    int64_t nlists = L.ix.nlists;
    int nl = (int)nlists;
    int G = Hq / Hkv;
    float score_scale = kLog2e / sqrtf((float)D);
    float scale = 1.0f / sqrtf((float)D);
    hipError_t e = nsa_index_build(L.ix, idx, B, Hkv, T, BS, S, stream);
    if (e != hipSuccess) return e;
    {
        int nq4 = (T + kDqWaves - 1) / kDqWaves;
        int ngroups = B * Hkv;
        void *a[] = {&q, &k, &v, &idx, &out, &lse, &dout, &dq, &delta, &Hq, &Hkv, &G, &T, &S,
                     &nq4, &ngroups, &score_scale, &scale};
        e = hipLaunchKernel((const void *)nsa_bwd_dq_kernel<D, BS>,
                            dim3((unsigned)(ngroups * nq4)), dim3(64 * kDqWaves), a, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        const unsigned grid = (unsigned)(8 * ((L.ix.max_segs + 7) / 8));
        void *a[] = {&q, &k, &v, &lse, &dout, &delta, &offsets, &list, &seg_start, &seg_list,
                     &part_start, &part, &dk, &dv, &Hq, &Hkv, &G, &T, &nblk, &nl,
                     &score_scale, &scale};
        e = hipLaunchKernel((const void *)nsa_bwd_dkv_kernel<D, BS>, dim3(grid),
                            dim3(64 * (BS / 32)), a, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        void *a[] = {&part, &seg_start, &part_start, &dk, &dv, &T, &nblk, &scale};
        return hipLaunchKernel((const void *)dkv_reduce_kernel<D, BS>,
                               dim3((unsigned)(nlists * (BS * D / 1024))), dim3(256), a, 0,
                               stream);
    }
}

}  // namespace

size_t nsa_sel_bwd_workspace(int B, int Hq, int Hkv, int T, int D, int block_size, int S) {
    return layout(nullptr, B, Hq, Hkv, T, D, block_size, S).total;
}

hipError_t launch_nsa_sel_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *block_idx, const uint16_t *out, const float *lse,
                              const uint16_t *dout, uint16_t *dq, uint16_t *dk, uint16_t *dv,
                              void *workspace, int B, int Hq, int Hkv, int T, int D,
                              int block_size, int S, hipStream_t stream) {
    uint8_t *ws = static_cast<uint8_t *>(workspace);
#define ATTN_NSA_BWD_CASE(DD, BB)                                                            \
    if (D == DD && block_size == BB)                                                        \
        return launch<DD, BB>(q, k, v, block_idx, out, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, T, \
                              S, stream);
    ATTN_NSA_BWD_CASE(128, 64)
    ATTN_NSA_BWD_CASE(128, 32)
    ATTN_NSA_BWD_CASE(128, 128)
    ATTN_NSA_BWD_CASE(64, 64)
    ATTN_NSA_BWD_CASE(64, 32)
    ATTN_NSA_BWD_CASE(64, 128)
#undef ATTN_NSA_BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace attn
