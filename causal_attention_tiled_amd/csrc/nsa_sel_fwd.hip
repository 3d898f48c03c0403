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
//  * The S slots of the query's block_idx row are validated lane-parallel (lane s
//    holds slot s): padding, ids past T/bs, blocks after i and repeats of an earlier
//    slot are dropped, and the wave walks the survivors in decreasing block order.
//    No scan over the KV sequence takes place.  The order only changes the rounding
//    order of the online softmax; it makes the waves that run together on an XCD read
//    nearby blocks at the same time (their k-th largest), which at T = 32768 G = 16
//    keeps enough of the gathers in L2 to cut the time by a fifth against slot order.
//  * Keys are processed in chunks of 32, with one K tile and one V tile of LDS per
//    wave.  Both go from HBM straight into LDS (buffer loads with the LDS as
//    destination), each 1 KB instruction moving whole rows (4 rows at D = 128): K
//    rows loaded into registers in the MFMA operand layout would touch 16 rows at 64
//    bytes per instruction, and that gather pattern, not the bytes, was the limit.
//  * Software pipeline, one stage per chunk t: read K(t)'s operands from LDS, issue
//    K(t+1) into the K tile, S^T(t) = K Q^T, then the deferred O^T += V^T P^T of
//    chunk t-1 from the V tile, then issue V(t) into it, then chunk t's softmax.  So
//    each transfer has about one stage to land, with single-buffered tiles (16 KB of
//    LDS per wave at D = 128: two workgroups, 8 waves, per compute unit).
//  * Scores are computed transposed, S^T = K Q^T, so each lane holds ONE head (lane %
//    16): the online-softmax state (running max in base-2 units, per-lane partial
//    sum, output rescale) is per-lane work plus a two-step cross-lane max.  Only the
//    chunk that holds position i is masked.  The rescale of O by chunk t's max moves
//    into the accumulator input of chunk t's own P V product in the next stage.
//  * The exponentials, rounded to bf16, form in accumulator register order the B
//    operand of O^T += V^T P^T; the V^T operand is read from the row-major LDS tile
//    with ds_read_b64_tr_b16 (in each 16-lane group, output lane i, value t is
//    element i % 4 of the 8 bytes that source lane 4t + i/4 addresses).  K and V
//    operand reads sit in one statement with an s_waitcnt vmcnt that awaits exactly
//    their own tile's transfer (the younger transfer stays in flight); the compiler's
//    own wait for DMA'd LDS data would be vmcnt(0).
//  * Workgroup order keeps each XCD on a contiguous range of (group, query) work so a
//    group's K/V stays in one XCD's L2.
#include <type_traits>

#include "attn_tile.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kChunk = 32;  // keys per processed chunk
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over `bytes` bytes at `base` (gfx9 layout, range-checked).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t nsa_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16 bytes per lane from (resource, voff + soff) into LDS at lds + 16 * lane.
__device__ __forceinline__ void nsa_dma16(__amdgpu_buffer_rsrc_t r, void *lds, int voff,
                                          int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, soff, 0, 0);
}

// V chunk in LDS: 32 rows (keys) x D*2 bytes, row-major; the 16-byte chunk c of row r
// sits at chunk slot c ^ nsa_swz<D>(r).  A 16-lane group of the transposing read
// takes 4 consecutive rows x 32 bytes; with this swizzle the 32 lanes served per
// cycle (8 rows) cover all 64 banks once.
template <int D>
__host__ __device__ constexpr int nsa_swz(int row) {
    if constexpr (D == 128)
        return (row & 7) << 1;          // one row per 256-byte bank line
    else
        return ((row >> 1) & 3) << 1;   // two rows per bank line
}

// K chunk in LDS: 32 rows x D*2 bytes, row-major, chunk c of row r at slot
// c ^ nsa_kswz<D>(r): the 16 rows that 16 consecutive lanes read for one MFMA
// A operand (ds_read_b128, the same 16-byte chunk of each row) cover all 64 banks.
template <int D>
__host__ __device__ constexpr int nsa_kswz(int row) {
    if constexpr (D == 128)
        return row & 15;                // one row per bank line, 16 chunk slots
    else
        return (row >> 1) & 7;          // two rows per bank line, 8 chunk slots
}

template <int D, int BS>
__global__ __launch_bounds__(kThreads, 2) void nsa_sel_fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ IDX, uint16_t *__restrict__ O,
    float *__restrict__ LSE, int Hq, int Hkv, int G, int T, int S, int nq4, int ngroups,
    float score_scale) {
    constexpr int ROWB = D * 2;              // bytes per key row
    constexpr int NCH = BS / kChunk;         // chunks per selected block
    constexpr int NDS = D / 32;              // S^T MFMA k-steps
    constexpr int NDT = D / 16;              // 16-dim output tiles
    constexpr int VTILE = kChunk * ROWB;     // bytes of one K (or V) chunk
    constexpr int VDMA = VTILE / 1024;       // 1 KB DMA instructions per chunk and tensor
    static_assert(BS % kChunk == 0 && VTILE % 1024 == 0, "chunking");

    __shared__ __attribute__((aligned(16))) uint8_t kbuf[kWaves][VTILE];
    __shared__ __attribute__((aligned(16))) uint8_t vbuf[kWaves][VTILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;

    // workgroup -> (group, query quad); each XCD takes one contiguous range
    const int W = ngroups * nq4;
    int f = blockIdx.x;
    if ((W & 7) == 0) f = (blockIdx.x & 7) * (W >> 3) + (blockIdx.x >> 3);
    const int group = __builtin_amdgcn_readfirstlane(f / nq4);
    const int i = __builtin_amdgcn_readfirstlane((nq4 - 1 - f % nq4) * kWaves + wave);
    if (i >= T) return;  // no workgroup-wide barrier in this kernel
    const int b = group / Hkv, kv = group % Hkv;
    const size_t kvslab = (size_t)group * T * D;
    const __amdgpu_buffer_rsrc_t rk = nsa_rsrc(K + kvslab, (uint32_t)T * ROWB);
    const __amdgpu_buffer_rsrc_t rv = nsa_rsrc(V + kvslab, (uint32_t)T * ROWB);

    // ---- the selected blocks: lane s holds slot s (S <= 64) ----
    const int nblk = T / BS;
    const int32_t *slots = IDX + ((size_t)group * T + i) * S;
    const int myblk = lane < S ? slots[lane] : -1;
    bool keep = myblk >= 0 && myblk < nblk && myblk * BS <= i;
    for (int s2 = 0; s2 < S; ++s2) {  // drop repeats of an earlier slot
        const int other = __builtin_amdgcn_readlane(myblk, s2);
        keep = keep && !(s2 < lane && other == myblk);
    }
    // The kept blocks are visited in decreasing block order: lane s's rank is the
    // number of kept blocks above its own (the kept blocks are distinct, so the ranks
    // are 0 .. nkept-1).  Waves of neighbouring queries run at the same time and reach
    // their k-th largest blocks together, so the blocks read across an XCD at any
    // moment lie close together and more of them are still in its L2; in slot order
    // (random) the whole causal prefix is in use at once.
    const uint64_t kept = __builtin_amdgcn_ballot_w64(keep);
    const int nkept = __builtin_popcountll(kept);
    int rank = 0;
    for (int s2 = 0; s2 < S; ++s2) {
        const int other = __builtin_amdgcn_readlane(myblk, s2);
        rank += (int)(((kept >> s2) & 1) != 0 && other > myblk);
    }
    int taken = 0;

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

    // ---- per-lane load offsets (bytes within a chunk) ----
    int vdma_off[VDMA], kdma_off[VDMA];     // rows written by DMA instruction j
#pragma unroll
    for (int j = 0; j < VDMA; ++j) {
        const int pos = j * 1024 + lane * 16;
        const int row = pos / ROWB, slot = (pos % ROWB) >> 4;
        vdma_off[j] = row * ROWB + ((slot ^ nsa_swz<D>(row)) << 4);
        kdma_off[j] = row * ROWB + ((slot ^ nsa_kswz<D>(row)) << 4);
    }
    // K operand reads: row n16 (+16 for the upper keys, same swizzle), chunk 4*ds + g4
    // (at D = 64, NDS = 2: the last two addresses repeat the first two, reads unused)
    static_assert(nsa_kswz<D>(16) == nsa_kswz<D>(0), "upper keys: same swizzle");
    uint32_t krd_off[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        krd_off[e] = n16 * ROWB + ((((4 * (e % NDS) + g4)) ^ nsa_kswz<D>(n16)) << 4);
    // V^T operand reads: rows 4*g4 + s/4 (and 16 rows further for the upper keys,
    // same swizzle), dims 16*dt + 4*(s%4)
    const int s16 = n16;
    static_assert(nsa_swz<D>(16) == nsa_swz<D>(0), "upper keys: same swizzle");
    int vrd_off[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        const int row = 4 * g4 + (s16 >> 2);
        const int col = 16 * dt + 4 * (s16 & 3);  // element
        vrd_off[dt] = row * ROWB + (((col >> 3) ^ nsa_swz<D>(row)) << 4) + (col & 7) * 2;
    }

    auto dma_k = [&](int k0) {
#pragma unroll
        for (int j = 0; j < VDMA; ++j) nsa_dma16(rk, &kbuf[wave][j * 1024], kdma_off[j], k0 * ROWB);
    };
    auto dma_v = [&](int k0) {
#pragma unroll
        for (int j = 0; j < VDMA; ++j) nsa_dma16(rv, &vbuf[wave][j * 1024], vdma_off[j], k0 * ROWB);
    };

    float m = -INFINITY;  // running max of the base-2 scores (this lane's head)
    float lsum = 0.0f;    // this lane's share of the running sum
    f32x4 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8 pprev;              // probabilities of the previous chunk (B operand order;
                               // set by every stage before the P V that reads it)
    float alpha_prev = 0.0f;   // rescale of O that precedes the previous chunk's P V

    // O^T = alpha_prev O^T + V^T P^T of the previous chunk, its V read from the LDS tile
    // after exactly its own transfer (VM = memory instructions issued after it)
    auto pv = [&](auto vm) {
        constexpr int VM = decltype(vm)::value;
        const uint32_t base = lds_addr(&vbuf[wave][0]);
#pragma unroll
        for (int d4 = 0; d4 < NDT; d4 += 4) {
            uint32_t ad[4];
            bf16x4_t rd[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) ad[e] = base + vrd_off[d4 + e];
            if (d4 == 0)
                tr_read4x2<VM, 16 * ROWB>(rd, ad);
            else
                tr_read4x2<63, 16 * ROWB>(rd, ad);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x8 a = __builtin_shufflevector(rd[2 * e], rd[2 * e + 1], 0, 1, 2, 3, 4,
                                                         5, 6, 7);
                oacc[d4 + e] = mfma_16x16x32(a, pprev, oacc[d4 + e] * alpha_prev);
            }
        }
    };
    using vdma_ops = std::integral_constant<int, VDMA>;
    using no_ops = std::integral_constant<int, 0>;

    // Walk the chunks of the kept blocks in decreasing block order: chunk (blk, c) starts at key
    // blk*BS + 32*c and exists while it starts at or before i.
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

    // One stage per chunk, with one K tile and one V tile per wave.  Issue order of the
    // transfers: K(t+1) during stage t, then V(t) once the previous chunk's P V has
    // read V(t-1); so stage t+1 finds K(t+1) complete when only V(t) is younger, and
    // the P V of chunk t (in stage t+1) finds V(t) complete when only K(t+2) is.
    auto stage = [&](int k0, auto first, int &nxt) {
        constexpr bool kFirst = decltype(first)::value;
        // K operands: register j of kf[kk] is row 16*kk + n16, dims 32*ds + 8*g4 .. +7
        bf16x8 kf[2][NDS];
        {
            const uint32_t kbase = lds_addr(&kbuf[wave][0]);
            uint32_t ad[4];
            u32x4 rd[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) ad[e] = kbase + krd_off[e];
            row_read4x2<kFirst ? 0 : VDMA, 16 * ROWB>(rd, ad);
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                kf[0][ds] = as_bf16x8(rd[2 * ds]);
                kf[1][ds] = as_bf16x8(rd[2 * ds + 1]);
            }
        }
        nxt = next_chunk();
        if (nxt >= 0) dma_k(nxt);
        // S^T = K Q^T : register j of st[kk] is key k0 + 16*kk + 4*g4 + j, head n16
        f32x4 st[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            st[kk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) st[kk] = mfma_16x16x32(kf[kk][ds], qf[ds], st[kk]);
        }
        // the previous chunk's P V (its V landed while this chunk's K was in flight)
        if constexpr (!kFirst) {
            if (nxt >= 0)
                pv(vdma_ops{});
            else
                pv(no_ops{});
        }
        dma_v(k0);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) st[kk] *= score_scale;
        if (k0 + kChunk - 1 > i) {  // the chunk holding position i: mask later keys
            const int lim = i - k0 - 4 * g4;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (16 * kk + j > lim) st[kk][j] = -INFINITY;
        }
        float mloc = fmaxf(fmaxf(fmaxf(st[0][0], st[0][1]), fmaxf(st[0][2], st[0][3])),
                           fmaxf(fmaxf(st[1][0], st[1][1]), fmaxf(st[1][2], st[1][3])));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float mnew = fmaxf(m, mloc);  // finite: key k0 <= i is never masked
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        float psum = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e = __builtin_amdgcn_exp2f(st[kk][j] - mnew);
                psum += e;
                pprev[kk * 4 + j] = (__bf16)e;
            }
        lsum = lsum * alpha + psum;
        alpha_prev = alpha;
    };

    int cur = next_chunk();
    if (cur >= 0) {
        dma_k(cur);
        int nxt;
        stage(cur, std::true_type{}, nxt);
        while (nxt >= 0) {
            cur = nxt;
            stage(cur, std::false_type{}, nxt);
        }
        pv(no_ops{});  // the last chunk's P V: nothing was issued after its V
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
