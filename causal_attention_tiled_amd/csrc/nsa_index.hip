// nsa_index.hip -- the selection inverted on the GPU, for the block-outer NSA kernels.
//
// The selection (msb-msb/openbox-llm, page "nsa_selection_kernel.py": module docstring,
// `selection_forward_reference`) lists, per (batch, kv head, query), the blocks the
// query attends.  The block-outer forward and the backward's dk/dv need the inverse:
// per (group = batch*Hkv + kv head, block) the increasing list of queries that attend
// the block (a listed block that is valid, not after the query's own block; a repeat
// counts once).  Built each call from block_idx, with no host round trip:
//  1. a bitmap per (group, block) over the query positions, built per 32-query word in
//     an LDS hash table keyed by block (a repeated slot sets the same bit again, so
//     duplicates vanish) and stored word by word;
//  2. popcount per list; 3. one workgroup scans the counts into list offsets;
//  4. one wave per list writes the positions of its set bits in order, and for each
//     32-bit word the list position of its first set bit;
//  5. lists are cut into segments of at most kNsaSegQ queries (one workgroup each in
//     the block-outer kernels): counts, scans and a segment -> list table.
// Every step's result is independent of scheduling.
#include "attn_internal.h"

namespace attn {
namespace {

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *__restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// one workgroup per (group, 32-query word w): the listed blocks of the word's queries go
// into an LDS hash table (open addressing on the block id, at least twice as many entries
// as the word has slots, so a probe always ends), each entry ORing in its queries' bits;
// then every entry is stored as word w of its block's bitmap.  Word w of a group's lists
// has this one writer, so plain stores suffice (the words no query lists stay zero).
constexpr int kHashMax = 4096;  // entries for S = 64: 2 * 32 * 64

__global__ __launch_bounds__(256) void csr_bitmap_kernel(const int32_t *__restrict__ idx,
                                                         uint32_t *__restrict__ bits, int T,
                                                         int S, int nblk, int bs, int words,
                                                         int tbits) {
    __shared__ int key[kHashMax];
    __shared__ uint32_t val[kHashMax];
    const int tsize = 1 << tbits;
    const int64_t group = blockIdx.x / words;
    const int w = (int)(blockIdx.x % words);
    for (int k = threadIdx.x; k < tsize; k += 256) {
        key[k] = -1;
        val[k] = 0u;
    }
    __syncthreads();
    const int i0 = w * 32;
    const int n = min(32, T - i0) * S;
    const int32_t *src = idx + (group * T + i0) * S;
    for (int e = threadIdx.x; e < n; e += 256) {
        const int blk = src[e];
        const int i = i0 + e / S;
        if (blk < 0 || blk >= nblk || blk * bs > i) continue;
        int h = (int)(((uint32_t)blk * 2654435761u) >> (32 - tbits));
        while (true) {
            const int prev = atomicCAS(&key[h], -1, blk);
            if (prev == -1 || prev == blk) {
                atomicOr(&val[h], 1u << (i & 31));
                break;
            }
            h = (h + 1) & (tsize - 1);
        }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < tsize; k += 256) {
        const int blk = key[k];
        if (blk >= 0) bits[(group * nblk + blk) * words + w] = val[k];
    }
}

// one wave per (group, block): number of attending queries
__global__ __launch_bounds__(256) void csr_count_kernel(const uint32_t *__restrict__ bits,
                                                        int32_t *__restrict__ counts, int words,
                                                        int64_t nlists) {
    const int64_t list = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (list >= nlists) return;
    const uint32_t *w = bits + list * words;
    int c = 0;
    for (int k = lane; k < words; k += 64) c += __builtin_popcount(w[k]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, 64);
    if (lane == 0) counts[list] = c;
}

// one workgroup: offsets[0] = 0, offsets[k+1] = offsets[k] + counts[k]
__global__ __launch_bounds__(1024) void csr_scan_kernel(const int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ offsets,
                                                        int nlists) {
    __shared__ int32_t part[1024];
    const int t = threadIdx.x;
    const int per = (nlists + 1023) / 1024;
    const int lo = min(t * per, nlists), hi = min(lo + per, nlists);
    int s = 0;
    for (int k = lo; k < hi; ++k) s += counts[k];
    part[t] = s;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan of the per-thread sums
        const int v = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int run = t > 0 ? part[t - 1] : 0;
    if (t == 0) offsets[0] = 0;
    for (int k = lo; k < hi; ++k) {
        run += counts[k];
        offsets[k + 1] = run;
    }
}

// one wave per (group, block): positions of the set bits, increasing, and for every
// 32-bit word the list position of its first set bit (rank[w] + popcount of the bits
// below position i in word w = where query i sits in the list)
__global__ __launch_bounds__(256) void csr_fill_kernel(const uint32_t *__restrict__ bits,
                                                       const int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ list,
                                                       int32_t *__restrict__ rank, int words,
                                                       int64_t nlists) {
    const int64_t l = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (l >= nlists) return;
    const uint32_t *w = bits + l * words;
    int base = offsets[l];
    for (int k0 = 0; k0 < words; k0 += 64) {
        const int k = k0 + lane;
        uint32_t x = k < words ? w[k] : 0u;
        const int c = __builtin_popcount(x);
        int incl = c;  // inclusive prefix over the wave
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const int y = __shfl_up(incl, m, 64);
            if (lane >= m) incl += y;
        }
        int pos = base + incl - c;
        if (k < words) rank[l * words + k] = pos;
        while (x) {
            const int bit = __builtin_ctz(x);
            x &= x - 1;
            list[pos++] = k * 32 + bit;
        }
        base += __shfl(incl, 63, 64);
    }
}


// one thread per (group, block) list: its segments of at most kNsaSegQ queries (at least
// one, so that a block nothing attends is still visited: the backward writes its zero
// gradients there) and the partial results a split list leaves (none for one segment)
__global__ __launch_bounds__(256) void seg_count_kernel(const int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ nseg,
                                                        int32_t *__restrict__ npart,
                                                        int64_t nlists) {
    const int64_t l = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (l >= nlists) return;
    const int nq = offsets[l + 1] - offsets[l];
    const int s = nq > kNsaSegQ ? (nq + kNsaSegQ - 1) / kNsaSegQ : 1;
    nseg[l] = s;
    npart[l] = s > 1 ? s : 0;
}

// one thread per list: seg_list[k] = list of segment k
__global__ __launch_bounds__(256) void seg_fill_kernel(const int32_t *__restrict__ seg_start,
                                                       int32_t *__restrict__ seg_list,
                                                       int64_t nlists) {
    const int64_t l = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (l >= nlists) return;
    for (int k = seg_start[l]; k < seg_start[l + 1]; ++k) seg_list[k] = (int)l;
}


}  // namespace

NsaIndex nsa_index_carve(void *ws, int B, int Hkv, int T, int bs, int S, size_t *bytes) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int nblk = T / bs;
    NsaIndex ix;
    ix.nblk = nblk;
    ix.words = (T + 31) / 32;
    ix.nlists = (int64_t)B * Hkv * nblk;
    ix.pairs = (int64_t)B * Hkv * T * (int64_t)(S < nblk ? S : nblk);
    ix.max_segs = ix.nlists + ix.pairs / kNsaSegQ;
    ix.max_part = 2 * ix.pairs / kNsaSegQ + 1;
    const size_t nl = (size_t)ix.nlists;
    size_t o = 0;
    const size_t o_bits = o;       o = al(o + nl * ix.words * 4);
    const size_t o_rank = o;       o = al(o + nl * ix.words * 4);
    const size_t o_counts = o;     o = al(o + nl * 4);
    const size_t o_offsets = o;    o = al(o + (nl + 1) * 4);
    const size_t o_list = o;       o = al(o + (size_t)ix.pairs * 4);
    const size_t o_nseg = o;       o = al(o + nl * 4);
    const size_t o_npart = o;      o = al(o + nl * 4);
    const size_t o_seg_start = o;  o = al(o + (nl + 1) * 4);
    const size_t o_part_start = o; o = al(o + (nl + 1) * 4);
    const size_t o_seg_list = o;   o = al(o + (size_t)ix.max_segs * 4);
    *bytes = o;
    uint8_t *w = static_cast<uint8_t *>(ws);
    ix.bits = (uint32_t *)(w + o_bits);
    ix.rank = (int32_t *)(w + o_rank);
    ix.counts = (int32_t *)(w + o_counts);
    ix.offsets = (int32_t *)(w + o_offsets);
    ix.list = (int32_t *)(w + o_list);
    ix.nseg = (int32_t *)(w + o_nseg);
    ix.npart = (int32_t *)(w + o_npart);
    ix.seg_start = (int32_t *)(w + o_seg_start);
    ix.part_start = (int32_t *)(w + o_part_start);
    ix.seg_list = (int32_t *)(w + o_seg_list);
    return ix;
}

hipError_t nsa_index_build(const NsaIndex &ix, const int32_t *idx, int B, int Hkv, int T, int bs,
                           int S, hipStream_t stream) {
    uint32_t *bits = ix.bits;
    int32_t *counts = ix.counts, *offsets = ix.offsets, *list = ix.list, *rank = ix.rank;
    int32_t *nseg = ix.nseg, *npart = ix.npart, *seg_start = ix.seg_start;
    int32_t *part_start = ix.part_start, *seg_list = ix.seg_list;
    int nblk = ix.nblk, words = ix.words;
    int64_t nlists = ix.nlists;
    int nl = (int)nlists;
    const unsigned lgrid = (unsigned)((nlists + 255) / 256);
    hipError_t e;
    {
        int64_t n = nlists * words;
        void *a[] = {&bits, &n};
        e = hipLaunchKernel((const void *)fill_u32_kernel, dim3((unsigned)((n + 255) / 256)),
                            dim3(256), a, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        int tbits = 8;  // table entries: a power of two >= 2 * 32 * S
        while ((1 << tbits) < 64 * S) ++tbits;
        void *a[] = {&idx, &bits, &T, &S, &nblk, &bs, &words, &tbits};
        e = hipLaunchKernel((const void *)csr_bitmap_kernel, dim3((unsigned)((int64_t)B * Hkv * words)),
                            dim3(256), a, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        void *a[] = {&bits, &counts, &words, &nlists};
        e = hipLaunchKernel((const void *)csr_count_kernel, dim3((unsigned)((nlists + 3) / 4)),
                            dim3(256), a, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        void *a[] = {&counts, &offsets, &nl};
        e = hipLaunchKernel((const void *)csr_scan_kernel, dim3(1), dim3(1024), a, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        void *a[] = {&bits, &offsets, &list, &rank, &words, &nlists};
        e = hipLaunchKernel((const void *)csr_fill_kernel, dim3((unsigned)((nlists + 3) / 4)),
                            dim3(256), a, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        void *a[] = {&offsets, &nseg, &npart, &nlists};
        e = hipLaunchKernel((const void *)seg_count_kernel, dim3(lgrid), dim3(256), a, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        void *a[] = {&nseg, &seg_start, &nl};
        e = hipLaunchKernel((const void *)csr_scan_kernel, dim3(1), dim3(1024), a, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        void *a[] = {&npart, &part_start, &nl};
        e = hipLaunchKernel((const void *)csr_scan_kernel, dim3(1), dim3(1024), a, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        void *a[] = {&seg_start, &seg_list, &nlists};
        return hipLaunchKernel((const void *)seg_fill_kernel, dim3(lgrid), dim3(256), a, 0,
                               stream);
    }
}

}  // namespace attn
