// nsa_sel_fsa.hip -- NSA selection forward in block-outer form, for gfx950.
//
// The same outputs as nsa_sel_fwd (msb-msb/openbox-llm, page "nsa_selection_kernel.py":
// module docstring, `selection_forward_reference`, `_selection_fwd_kernel`), computed the
// way the page's `_selection_fwd_blockouter_kernel` and `selection_forward_fsa` arrange it:
// each selected key block is loaded once and every query that selects it is processed
// against it, leaving a partial softmax state per (query, block); a combine pass merges
// the partials of each query with the log-sum-exp rule, which gives one softmax over the
// union of the selected causal tokens.
//
//  * Index (nsa_index.hip): per (group, block) the increasing list of queries that select
//    it, cut into segments of at most kNsaSegQ queries, and per 32-bit word the list
//    position of its first query (so a query finds its place in a list in O(1)).
//  * Partial kernel: one workgroup (two waves) per segment.  The block's K rows sit in
//    every wave's registers as the A operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16),
//    its V rows in LDS (one DMA per workgroup).  The segment's (query, head) rows are
//    walked in chunks of 32; each wave gathers its chunks' Q rows into its own LDS ring
//    (two buffers, DMA, explicit vmcnt waits).  Per chunk: S^T, the causal mask (keys
//    after the query, own block only), the block-local row max m and sum l, P in bf16 in
//    accumulator order as the B operand of O^T += V^T P^T (V^T by transposing LDS reads),
//    and a store of (O / l in bf16, m, l) for each row at its list position.
//  * Combine kernel: one wave per (group, query), or per 2, 4 or 8 consecutive ones when
//    the G heads' outputs fill fewer than 33 lanes.  Lane s holds slot s (kept as in
//    the forward: valid, causal, first occurrence) and finds the query's list position
//    in its block's list; the kept partials are merged in slot order, their loads
//    issued several at a time:
//    M = max m_s, L = sum l_s 2^(m_s - M), out = sum l_s 2^(m_s - M) (O_s / l_s) / L,
//    lse = (M + log2 L) ln 2; no kept slot gives out = 0 and lse = -1e9.
#include <type_traits>

#include "attn_tile.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kFsaWaves = 2;  // waves per partial-kernel workgroup

__device__ __forceinline__ __amdgpu_buffer_rsrc_t fsa_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

template <int D, int BS>
__global__ __launch_bounds__(64 * kFsaWaves) void nsa_fsa_partial_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ list, const int32_t *__restrict__ seg_start,
    const int32_t *__restrict__ seg_list, uint16_t *__restrict__ PA, float *__restrict__ PM,
    float *__restrict__ PL, int Hq, int Hkv, int G, int T, int nblk, int nlists,
    float score_scale) {
    constexpr int ROWB = D * 2;
    constexpr int NKT = BS / 32;             // 32-key tiles of the block
    constexpr int NDS = D / 16;              // k-steps of S^T
    constexpr int NDT = D / 32;              // 32-dim tiles of O^T
    constexpr int QTILE = 32 * ROWB;         // 32 gathered Q rows
    constexpr int QLOADS = QTILE / 1024;     // DMA instructions per chunk (one wave)
    constexpr int VBYTES = BS * ROWB;
    constexpr int VLOADS = VBYTES / 1024 / kFsaWaves;
    constexpr int NST = 4 * NDT + 2;         // buffer stores per chunk
    static_assert(VBYTES % (1024 * kFsaWaves) == 0 && QTILE % 1024 == 0, "staging");
    static_assert(NST + QLOADS < 64, "vmcnt range");

    __shared__ __attribute__((aligned(16))) uint8_t vt[VBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t qt[kFsaWaves][2][QTILE];
    __shared__ int rpos[kFsaWaves][2][32];   // query position of each staged row (-1: none)
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
    const int lbeg = offsets[l] + seg * kNsaSegQ;
    const int nq = min(kNsaSegQ, offsets[l + 1] - lbeg);
    if (nq <= 0) return;                          // a block nobody selects: nothing to write
    const int group = l / nblk, blk = l % nblk;
    const int b = group / Hkv, kv = group % Hkv;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int qc = 32 / G;                        // queries per chunk of 32 rows
    const int rows_used = qc * G;
    const int nchunks = (nq + qc - 1) / qc;
    const int key0 = blk * BS;

    // K rows as A operands: tile t, key key0 + 32t + l32, dims 16ds + 8hi .. +7
    const size_t kvslab = (size_t)group * T * D;
    bf16x8 kf[NKT][NDS];
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
            kf[t][ds] = as_bf16x8(
                *(const u32x4 *)(K + kvslab + (size_t)(key0 + 32 * t + l32) * D + ds * 16 + hi * 8));
    // V rows into LDS, row-major with the tile swizzle
    {
        const u32x4 rv = make_rsrc(V + kvslab + (size_t)key0 * D, VBYTES);
#pragma unroll
        for (int j = 0; j < VLOADS; ++j) {
            const int pos = (wave * VLOADS + j) * 1024 + lane * 16;
            const int row = pos / ROWB, slot = (pos % ROWB) >> 4;
            dma16(rv, &vt[(wave * VLOADS + j) * 1024], row * ROWB + ((slot ^ tile_swz<D>(row)) << 4),
                  0);
        }
    }
    for (int t = tid; t < nq; t += 64 * kFsaWaves) qpos[t] = list[lbeg + t];
    wait_vm<0>();     // K rows, V tile and the query list are in: no wait for them in the loop
    __syncthreads();

    // Q rows of batch b: row (h, i) at (h*T + i); row r of chunk c is query
    // qpos[c*qc + r/G], head kv*G + r%G; absent rows read as zero
    const uint32_t qbytes = (uint32_t)((size_t)Hq * T * ROWB);
    const u32x4 rq = make_rsrc(Q + (size_t)b * Hq * T * D, qbytes);
    int srow[QLOADS], sslot[QLOADS];
#pragma unroll
    for (int j = 0; j < QLOADS; ++j) {
        const int pos = j * 1024 + lane * 16;
        srow[j] = pos / ROWB;
        sslot[j] = ((pos % ROWB) >> 4) ^ tile_swz<D>(pos / ROWB);
    }
    auto stage = [&](int c, int u) {  // QLOADS memory instructions
        int off[QLOADS];  // all query positions read first (one LDS wait), then the DMAs
#pragma unroll
        for (int j = 0; j < QLOADS; ++j) {
            const int r = srow[j];
            const int qi = c * qc + r / G;
            const bool ok = r < rows_used && qi < nq;
            const int pos = qpos[ok ? qi : 0];  // c < nchunks, so nq > 0
            off[j] = ok ? ((kv * G + r % G) * T + pos) * ROWB + (sslot[j] << 4) : (int)qbytes;
        }
#pragma unroll
        for (int j = 0; j < QLOADS; ++j) dma16(rq, &qt[wave][u][j * 1024], off[j], 0);
        if (lane < 32) {
            const int qi = c * qc + lane / G;
            rpos[wave][u][lane] = (lane < rows_used && qi < nq) ? qpos[qi] : -1;
        }
    };

    int roff[NDS];  // Q row l32, dims 16ds + 8hi
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) roff[ds] = l32 * ROWB + (((2 * ds + hi) ^ tile_swz<D>(l32)) << 4);
    const int g16 = lane >> 4, s16 = lane & 15;
    const int vrow = 4 * (g16 >> 1) + (s16 >> 2);  // + 32t + 16c, + 8 for the upper keys
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
    // V^T operand for keys 32t + 16c + {4hi..4hi+3, 8+4hi..8+4hi+3}, dims 32dt + lane%32
    auto v_frag = [&](int t, int dt, int c) {
        const uint8_t *base = &vt[(t * 32 + 16 * c) * ROWB];
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + voff[dt][0]));
        const bf16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + voff[dt][1]));
        return (bf16x8)__builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    // partial rows of this segment: (query index in the segment) * G + head
    const uint32_t abytes = (uint32_t)(nq * G * ROWB), sbytes = (uint32_t)(nq * G * 4);
    const __amdgpu_buffer_rsrc_t ra = fsa_rsrc(PA + (size_t)lbeg * G * D, abytes);
    const __amdgpu_buffer_rsrc_t rm = fsa_rsrc(PM + (size_t)lbeg * G, sbytes);
    const __amdgpu_buffer_rsrc_t rl = fsa_rsrc(PL + (size_t)lbeg * G, sbytes);

    f32x16 zero16;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero16[r] = 0.0f;

    // this wave's chunks: wave, wave + kFsaWaves, ...
    const int nmine = nchunks > wave ? (nchunks - wave + kFsaWaves - 1) / kFsaWaves : 0;
    if (nmine > 0) stage(wave, 0);
    if (nmine > 1) stage(wave + kFsaWaves, 1);
    for (int k = 0; k < nmine; ++k) {
        const int c = wave + kFsaWaves * k, u = k & 1;
        // chunk k's transfer is done once at most these remain: the stores of chunk k-1
        // and the staging of chunk k+1, each if it happened
        const bool nxt = k + 1 < nmine;
        if (k >= 1) {
            if (nxt) wait_vm<NST + QLOADS>();
            else wait_vm<NST>();
        } else {
            if (nxt) wait_vm<QLOADS>();
            else wait_vm<0>();
        }

        // S^T: register r of s[t] is key key0 + 32t + 8(r/4) + 4hi + r%4, row l32
        f32x16 s[NKT];
#pragma unroll
        for (int t = 0; t < NKT; ++t) s[t] = zero16;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            const bf16x8 qf = *(const bf16x8 *)(&qt[wave][u][roff[ds]]);
#pragma unroll
            for (int t = 0; t < NKT; ++t) s[t] = mfma_32x32x16(kf[t][ds], qf, s[t]);
        }
        const int pos = rpos[wave][u][l32];
        float m = -INFINITY;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
                const float x = key > pos ? -INFINITY : s[t][r] * score_scale;
                s[t][r] = x;
                m = fmaxf(m, x);
            }
        m = fmaxf(m, __shfl_xor(m, 32));
        if (m == -INFINITY) m = 0.0f;  // no row here (never stored)
        float lsum = 0.0f;
        bf16x8 pf[NKT][2];
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(s[t][r] - m);
                lsum += e;
                pf[t][r >> 3][r & 7] = (__bf16)e;
            }
        lsum += __shfl_xor(lsum, 32);

        // O^T: register r of o[dt] is dim 32dt + 8(r/4) + 4hi + r%4, row l32
        f32x16 o[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = zero16;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) o[dt] = mfma_32x32x16(v_frag(t, dt, c2), pf[t][c2], o[dt]);

        // NST stores, always issued (absent rows go past the buffer end and are dropped)
        const int qi = c * qc + l32 / G;
        const bool ok = l32 < rows_used && qi < nq;
        const int prow = qi * G + l32 % G;
        const int aoff = ok ? prow * ROWB : (int)abytes;
        const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const u32x2 pk = {pack_bf16x2(o[dt][4 * i4] * inv, o[dt][4 * i4 + 1] * inv),
                                  pack_bf16x2(o[dt][4 * i4 + 2] * inv, o[dt][4 * i4 + 3] * inv)};
                __builtin_amdgcn_raw_buffer_store_b64(pk, ra, aoff + (32 * dt + 8 * i4 + 4 * hi) * 2, 0,
                                                      0);
            }
        const int soff = (ok && hi == 0) ? prow * 4 : (int)sbytes;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, m), rm, soff, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lsum), rl, soff, 0, 0);

        if (k + 2 < nmine) {
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this buffer's reads are done
            stage(c + 2 * kFsaWaves, u);
        }
    }
}

// One wave per QPW consecutive (group, query) rows; the G heads' outputs of a row are cut
// into 8-dim pieces, spread over the row's 64 / QPW lanes (CPL pieces per lane).  Small
// groups put several rows in a wave so that every lane merges; KPR partials are loaded
// per round before any is merged.
template <int D, int QPW, int CPL, int KPR>
__global__ __launch_bounds__(256) void nsa_fsa_combine_kernel(
    const int32_t *__restrict__ IDX, const uint32_t *__restrict__ bits,
    const int32_t *__restrict__ rank, const uint16_t *__restrict__ PA,
    const float *__restrict__ PM, const float *__restrict__ PL, uint16_t *__restrict__ O,
    float *__restrict__ LSE, int Hq, int Hkv, int G, int T, int S, int nblk, int words,
    int64_t nrows) {
    constexpr int DC = D / 8;       // 8-dim pieces per head
    constexpr int LPQ = 64 / QPW;   // lanes per row
    static_assert(QPW == 1 || CPL == 1, "several rows per wave only with one piece per lane");
    __shared__ int kpos[4][QPW][64];  // per wave and row: list positions of the kept slots
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * QPW;
    if (row0 >= nrows) return;      // no barrier in this kernel
    const int qsub = lane / LPQ, cl = lane % LPQ;
    const int nch = G * DC;

    // slot pass, one row at a time, lane s holding slot s: kept slots (valid, not after
    // the query's block, first occurrence) leave their list positions in slot order
    int nk_mine = 0, maxnk = 0;
#pragma unroll
    for (int r = 0; r < QPW; ++r) {
        const int64_t row = row0 + r;
        if (row >= nrows) break;
        const int64_t group = row / T;
        const int i = (int)(row % T);
        const int32_t *slots = IDX + row * S;
        const int myblk = lane < S ? slots[lane] : -1;
        bool keep = myblk >= 0 && myblk < nblk && myblk * (T / nblk) <= i;
        for (int s2 = 0; s2 < S; ++s2) {
            const int other = __builtin_amdgcn_readlane(myblk, s2);
            keep = keep && !(s2 < lane && other == myblk);
        }
        const uint64_t kept = __builtin_amdgcn_ballot_w64(keep);
        if (keep) {
            const int64_t lst = group * nblk + myblk;
            const int w = i >> 5;
            const uint32_t word = bits[lst * words + w];
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(kept >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)kept, 0u));
            kpos[wave][r][below] =
                rank[lst * words + w] + __builtin_popcount(word & ((1u << (i & 31)) - 1u));
        }
        const int n = __builtin_popcountll(kept);
        if (qsub == r) nk_mine = n;
        maxnk = max(maxnk, n);
    }
    // the positions were written by other lanes of this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float M[CPL], L[CPL], acc[CPL][8];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        M[j] = -INFINITY;
        L[j] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
    }
    for (int base = 0; base < maxnk; base += KPR) {
        int ps[KPR];
#pragma unroll
        for (int t = 0; t < KPR; ++t) ps[t] = base + t < nk_mine ? kpos[wave][qsub][base + t] : -1;
        float pm[KPR][CPL], pl[KPR][CPL];
        bf16x8 pa[KPR][CPL];
#pragma unroll
        for (int t = 0; t < KPR; ++t)
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = cl + LPQ * j;
                pm[t][j] = -INFINITY;
                pl[t][j] = 0.0f;
                pa[t][j] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
                if (ps[t] >= 0 && c < nch) {
                    const size_t pr = (size_t)ps[t] * G + c / DC;
                    pm[t][j] = PM[pr];
                    pl[t][j] = PL[pr];
                    pa[t][j] = as_bf16x8(*(const u32x4 *)(PA + pr * D + (c % DC) * 8));
                }
            }
#pragma unroll
        for (int t = 0; t < KPR; ++t) {
            if (ps[t] < 0) continue;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const float mn = fmaxf(M[j], pm[t][j]);
                const float sc = __builtin_amdgcn_exp2f(M[j] - mn);
                const float w = pl[t][j] * __builtin_amdgcn_exp2f(pm[t][j] - mn);
                L[j] = L[j] * sc + w;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[j][e] = acc[j][e] * sc + w * (float)pa[t][j][e];
                M[j] = mn;
            }
        }
    }
    const int64_t row = row0 + qsub;
    if (row >= nrows) return;
    const int64_t group = row / T;
    const int i = (int)(row % T);
    const int b = (int)(group / Hkv), kv = (int)(group % Hkv);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = cl + LPQ * j;
        if (c >= nch) continue;
        const int h = kv * G + c / DC;
        const size_t orow = ((size_t)b * Hq + h) * T + i;
        const float inv = L[j] > 0.0f ? 1.0f / L[j] : 0.0f;
        const u32x4 pk = {pack_bf16x2(acc[j][0] * inv, acc[j][1] * inv),
                          pack_bf16x2(acc[j][2] * inv, acc[j][3] * inv),
                          pack_bf16x2(acc[j][4] * inv, acc[j][5] * inv),
                          pack_bf16x2(acc[j][6] * inv, acc[j][7] * inv)};
        *(u32x4 *)(O + orow * D + (c % DC) * 8) = pk;
        if (LSE != nullptr && c % DC == 0)
            LSE[orow] = L[j] > 0.0f ? (M[j] + __builtin_amdgcn_logf(L[j])) * kLn2 : -1e9f;
    }
}

// Rows per wave and pieces per lane for G heads of D dims: nch = G * D / 8 pieces per
// row; up to 32 pieces put 64 / nch (rounded down to a power of two) rows in a wave.
template <int D, int QPW, int CPL, int KPR>
hipError_t launch_combine(void **args, int64_t nrows, hipStream_t stream) {
    const int64_t waves = (nrows + QPW - 1) / QPW;
    return hipLaunchKernel((const void *)nsa_fsa_combine_kernel<D, QPW, CPL, KPR>,
                           dim3((unsigned)((waves + 3) / 4)), dim3(256), args, 0, stream);
}

template <int D>
hipError_t combine(void **args, int G, int64_t nrows, hipStream_t stream) {
    const int nch = G * (D / 8);
    if (nch <= 8) return launch_combine<D, 8, 1, 8>(args, nrows, stream);
    if (nch <= 16) return launch_combine<D, 4, 1, 8>(args, nrows, stream);
    if (nch <= 32) return launch_combine<D, 2, 1, 8>(args, nrows, stream);
    if (nch <= 64) return launch_combine<D, 1, 1, 8>(args, nrows, stream);
    if (nch <= 128) return launch_combine<D, 1, 2, 8>(args, nrows, stream);
    return launch_combine<D, 1, 4, 4>(args, nrows, stream);
}

// Workspace: the inverted index, then the partials: O / l bf16 [pairs][G][D], m and l
// fp32 [pairs][G] (pairs = the index's bound on list entries).
struct FsaLayout {
    NsaIndex ix;
    uint16_t *pa;
    float *pm, *pl;
    size_t total;
};

FsaLayout fsa_layout(void *ws, int B, int Hq, int Hkv, int T, int D, int bs, int S) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    FsaLayout L;
    size_t o;
    L.ix = nsa_index_carve(ws, B, Hkv, T, bs, S, &o);
    const size_t rows = (size_t)L.ix.pairs * (size_t)(Hq / Hkv);
    const size_t o_pa = o;
    o = al(o + rows * D * 2);
    const size_t o_pm = o;
    o = al(o + rows * 4);
    const size_t o_pl = o;
    o = al(o + rows * 4);
    L.total = o;
    uint8_t *w = static_cast<uint8_t *>(ws);
    L.pa = (uint16_t *)(w + o_pa);
    L.pm = (float *)(w + o_pm);
    L.pl = (float *)(w + o_pl);
    return L;
}

template <int D, int BS>
hipError_t launch(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *idx,
                  uint16_t *out, float *lse, void *ws, int B, int Hq, int Hkv, int T, int S,
                  hipStream_t stream) {
    const FsaLayout L = fsa_layout(ws, B, Hq, Hkv, T, D, BS, S);
    hipError_t e = nsa_index_build(L.ix, idx, B, Hkv, T, BS, S, stream);
    if (e != hipSuccess) return e;
    const int32_t *offsets = L.ix.offsets, *list = L.ix.list, *seg_start = L.ix.seg_start;
    const int32_t *seg_list = L.ix.seg_list, *rank = L.ix.rank;
    const uint32_t *bits = L.ix.bits;
    uint16_t *pa = L.pa;
    float *pm = L.pm, *pl = L.pl;
    int nblk = L.ix.nblk, words = L.ix.words, nl = (int)L.ix.nlists;
    int G = Hq / Hkv;
    float score_scale = kLog2e / sqrtf((float)D);
    {
        const unsigned grid = (unsigned)(8 * ((L.ix.max_segs + 7) / 8));
        void *a[] = {&q, &k, &v, &offsets, &list, &seg_start, &seg_list, &pa, &pm, &pl,
                     &Hq, &Hkv, &G, &T, &nblk, &nl, &score_scale};
        e = hipLaunchKernel((const void *)nsa_fsa_partial_kernel<D, BS>, dim3(grid),
                            dim3(64 * kFsaWaves), a, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        int64_t nrows = (int64_t)B * Hkv * T;
        void *a[] = {&idx, &bits, &rank, &pa, &pm, &pl, &out, &lse, &Hq, &Hkv, &G, &T, &S,
                     &nblk, &words, &nrows};
        return combine<D>(a, G, nrows, stream);
    }
}

}  // namespace

size_t nsa_sel_fsa_workspace(int B, int Hq, int Hkv, int T, int D, int block_size, int S) {
    return fsa_layout(nullptr, B, Hq, Hkv, T, D, block_size, S).total;
}

hipError_t launch_nsa_sel_fsa(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *block_idx, uint16_t *out, float *lse,
                              void *workspace, int B, int Hq, int Hkv, int T, int D,
                              int block_size, int S, hipStream_t stream) {
#define ATTN_NSA_FSA_CASE(DD, BB)                                                            \
    if (D == DD && block_size == BB)                                                        \
        return launch<DD, BB>(q, k, v, block_idx, out, lse, workspace, B, Hq, Hkv, T, S, stream);
    ATTN_NSA_FSA_CASE(128, 64)
    ATTN_NSA_FSA_CASE(128, 32)
    ATTN_NSA_FSA_CASE(128, 128)
    ATTN_NSA_FSA_CASE(64, 64)
    ATTN_NSA_FSA_CASE(64, 32)
    ATTN_NSA_FSA_CASE(64, 128)
#undef ATTN_NSA_FSA_CASE
    return hipErrorInvalidValue;
}

}  // namespace attn
