// attn_api.hip -- the C ABI of libattn.so (declared in include/attn.h).
//
// Every argument is validated on the host before any HIP call; then the kernel is
// launched asynchronously on the caller's stream.  Nothing is allocated and nothing is
// synchronised; the only state kept between calls is tda_fwd_noalloc's static scratch
// array and its address on each device.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "attn.h"
#include "attn_internal.h"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// The grid is one dimension of at most 2^31-1 workgroups.
bool grid_fits(int64_t n) { return n > 0 && n <= 0x7fffffffLL; }

// The bf16 kernels read a (batch, head) slab of T x D elements through a buffer
// resource with 32-bit byte offsets (rows past the slab read as zero), so a slab
// must stay below 2^31 bytes.
bool bf16_slab_fits(int T, int D) { return (int64_t)T * D * 2 < ((int64_t)1 << 31); }

int tra_validate(const void *q, const void *k, const void *v, const void *out, int B, int H,
                 int T, int D, float beta, float p, int rows_per_wg, bool *noop) {
    *noop = false;
    if (B < 0 || H < 0 || T < 0 || D < 0) return ATTN_ERR_SHAPE;
    if (!isfinite(beta) || !isfinite(p) || !(p > 0.0f)) return ATTN_ERR_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || T == 0) {
        *noop = true;
        return ATTN_OK;
    }
    if (!q || !k || !v || !out) return ATTN_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out)) return ATTN_ERR_ALIGN;
    if (!grid_fits((int64_t)B * H * ((T + rows_per_wg - 1) / rows_per_wg))) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

// Shared checks of the NSA selection forward and backward (shapes, sizes, the
// pointers both read); *noop is set for an empty problem.
int nsa_validate(const void *q, const void *k, const void *v, const int32_t *block_idx,
                 int B, int Hq, int Hkv, int T, int D, int block_size, int S, bool *noop) {
    *noop = false;
    if (B < 0 || Hq < 0 || Hkv <= 0 || T < 0 || D < 0 || S < 1 || block_size <= 0)
        return ATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (block_size != 32 && block_size != 64 && block_size != 128) return ATTN_ERR_UNSUPPORTED;
    if (Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
    if (S > 64) return ATTN_ERR_UNSUPPORTED;
    if (T % block_size != 0) return ATTN_ERR_SHAPE;
    if (B == 0 || Hq == 0 || T == 0) {
        *noop = true;
        return ATTN_OK;
    }
    if (!q || !k || !v || !block_idx) return ATTN_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v)) return ATTN_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(block_idx) & 3u) != 0) return ATTN_ERR_ALIGN;
    if (!grid_fits((int64_t)B * Hkv * ((T + 3) / 4))) return ATTN_ERR_SHAPE;
    if (!bf16_slab_fits(T, D)) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

// The inverted selection (block-outer NSA kernels) keeps list positions in int32: the
// number of (group, query, block) entries it may hold must stay below 2^31.
bool nsa_index_fits(int B, int Hkv, int T, int block_size, int S) {
    const int64_t nblk = T / block_size;
    return (int64_t)B * Hkv * T * (S < nblk ? S : nblk) < ((int64_t)1 << 31);
}

}  // namespace

ATTN_EXPORT int tra_fwd(const void *q, const void *k, const void *v, void *out, int B, int H,
                        int T, int D, float beta, float p, void *stream) {
    bool noop;
    const int st = tra_validate(q, k, v, out, B, H, T, D, beta, p, attn::tra_bf16_rows(D), &noop);
    if (st != ATTN_OK || noop) return st;
    if (!bf16_slab_fits(T, D)) return ATTN_ERR_UNSUPPORTED;
    const hipError_t e = attn::launch_tra_fwd_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), static_cast<uint16_t *>(out), B * H, T, D, beta, p,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_EXPORT int tra_fwd_f32(const float *q, const float *k, const float *v, float *out, int B,
                            int H, int T, int D, float beta, float p, void *stream) {
    bool noop;
    const int st = tra_validate(q, k, v, out, B, H, T, D, beta, p, attn::kTraF32Rows, &noop);
    if (st != ATTN_OK || noop) return st;
    const hipError_t e = attn::launch_tra_fwd_f32(q, k, v, out, B * H, T, D, beta, p,
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_EXPORT int tra_bwd(const void *q, const void *k, const void *v, const void *dout, void *dq,
                        void *dk, void *dv, int B, int H, int T, int D, float beta, float p,
                        void *stream) {
    bool noop;
    const int st = tra_validate(q, k, v, dq, B, H, T, D, beta, p, attn::tra_bwd_dkv_rows(D), &noop);
    if (st != ATTN_OK || noop) return st;
    if (!bf16_slab_fits(T, D)) return ATTN_ERR_UNSUPPORTED;
    if (!dout || !dk || !dv) return ATTN_ERR_NULL;
    if (misaligned(dout) || misaligned(dk) || misaligned(dv)) return ATTN_ERR_ALIGN;
    const hipError_t e = attn::launch_tra_bwd_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), static_cast<const uint16_t *>(dout),
        static_cast<uint16_t *>(dq), static_cast<uint16_t *>(dk), static_cast<uint16_t *>(dv),
        B * H, T, D, beta, p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_EXPORT size_t tda_workspace_bytes(int B, int H, int T, int D, int normalize) {
    if (!normalize || B <= 0 || H <= 0 || T <= 0 || D <= 0) return 0;
    return (size_t)2 * (size_t)B * (size_t)H * (size_t)T * (size_t)D * 2;
}

namespace {

// Checks of tda_fwd's arguments other than the workspace; *noop for an empty problem.
int tda_validate(const void *q1, const void *q2, const void *k1, const void *k2, const void *v,
                 const void *out, int B, int H, int T, int D, float beta, float lambda, float p,
                 bool *noop) {
    *noop = false;
    if (!isfinite(lambda)) return ATTN_ERR_SHAPE;
    const int st = tra_validate(q1, k1, v, out, B, H, T, D, beta, p, attn::kTdaRows, noop);
    if (st != ATTN_OK || *noop) return st;
    if (!bf16_slab_fits(T, D)) return ATTN_ERR_UNSUPPORTED;
    if (!q2 || !k2) return ATTN_ERR_NULL;
    if (misaligned(q2) || misaligned(k2)) return ATTN_ERR_ALIGN;
    return ATTN_OK;
}

int tda_launch(const void *q1, const void *q2, const void *k1, const void *k2, const void *v,
               void *out, void *workspace, int B, int H, int T, int D, float beta,
               float lambda, float p, int normalize, void *stream) {
    const hipError_t e = attn::launch_tda_fwd_bf16(
        static_cast<const uint16_t *>(q1), static_cast<const uint16_t *>(q2),
        static_cast<const uint16_t *>(k1), static_cast<const uint16_t *>(k2),
        static_cast<const uint16_t *>(v), static_cast<uint16_t *>(out),
        static_cast<uint16_t *>(workspace), B * H, T, D, beta, lambda, p, normalize ? 1 : 0,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Scratch memory of tda_fwd_noalloc: the normalised k1 and k2 rows.  Every GPU the
// library runs on holds its own copy of this array, at its own address, until the
// process ends.  In host code `scratch` names a host-side stand-in, never the device
// memory: kernels take the address that hipGetSymbolAddress returns for the current
// device, kept per device in scratch_dev.
constexpr size_t kTdaScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kTdaScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_dev[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per device,
// on the first call made with that device current.
int scratch_ptr(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_dev[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return ATTN_ERR_LAUNCH;
        scratch_dev[dev] = p;
    }
    *ptr = scratch_dev[dev];
    return ATTN_OK;
}

}  // namespace

ATTN_EXPORT int tda_fwd(const void *q1, const void *q2, const void *k1, const void *k2,
                        const void *v, void *out, void *workspace, size_t workspace_bytes,
                        int B, int H, int T, int D, float beta, float lambda, float p,
                        int normalize, void *stream) {
    bool noop;
    const int st = tda_validate(q1, q2, k1, k2, v, out, B, H, T, D, beta, lambda, p, &noop);
    if (st != ATTN_OK || noop) return st;
    const size_t need = tda_workspace_bytes(B, H, T, D, normalize);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
        if (misaligned(workspace)) return ATTN_ERR_ALIGN;
    }
    return tda_launch(q1, q2, k1, k2, v, out, workspace, B, H, T, D, beta, lambda, p, normalize,
                      stream);
}

ATTN_EXPORT size_t tda_noalloc_scratch_bytes(void) { return kTdaScratchBytes; }

ATTN_EXPORT int tda_fwd_noalloc(const void *q1, const void *q2, const void *k1, const void *k2,
                                const void *v, void *out, int B, int H, int T, int D,
                                float beta, float lambda, float p, int normalize, void *stream) {
    bool noop;
    const int st = tda_validate(q1, q2, k1, k2, v, out, B, H, T, D, beta, lambda, p, &noop);
    if (st != ATTN_OK || noop) return st;
    const size_t need = tda_workspace_bytes(B, H, T, D, normalize);
    if (need > kTdaScratchBytes) return ATTN_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        const int sst = scratch_ptr(&ws);
        if (sst != ATTN_OK) return sst;
    }
    return tda_launch(q1, q2, k1, k2, v, out, ws, B, H, T, D, beta, lambda, p, normalize, stream);
}

ATTN_EXPORT int nsa_sel_fwd(const void *q, const void *k, const void *v,
                            const int32_t *block_idx, void *out, float *lse, int B, int Hq,
                            int Hkv, int T, int D, int block_size, int S, void *stream) {
    bool noop;
    const int st = nsa_validate(q, k, v, block_idx, B, Hq, Hkv, T, D, block_size, S, &noop);
    if (st != ATTN_OK || noop) return st;
    if (!out) return ATTN_ERR_NULL;
    if (misaligned(out)) return ATTN_ERR_ALIGN;
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_ERR_ALIGN;
    const hipError_t e = attn::launch_nsa_sel_fwd(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), block_idx, static_cast<uint16_t *>(out), lse, B, Hq,
        Hkv, T, D, block_size, S, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}


ATTN_EXPORT size_t nsa_sel_bwd_workspace_bytes(int B, int Hq, int Hkv, int T, int D,
                                               int block_size, int S) {
    if (B <= 0 || Hq <= 0 || T <= 0 || D <= 0 || block_size <= 0 || T % block_size != 0 || S < 1 ||
        Hkv <= 0 || Hq % Hkv != 0)
        return 0;
    return attn::nsa_sel_bwd_workspace(B, Hq, Hkv, T, D, block_size, S);
}

ATTN_EXPORT int nsa_sel_bwd(const void *q, const void *k, const void *v,
                            const int32_t *block_idx, const void *out, const float *lse,
                            const void *dout, void *dq, void *dk, void *dv, void *workspace,
                            size_t workspace_bytes, int B, int Hq, int Hkv, int T, int D,
                            int block_size, int S, void *stream) {
    bool noop;
    const int st = nsa_validate(q, k, v, block_idx, B, Hq, Hkv, T, D, block_size, S, &noop);
    if (st != ATTN_OK || noop) return st;
    if (!out || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
    if (misaligned(out) || misaligned(dout) || misaligned(dq) || misaligned(dk) || misaligned(dv))
        return ATTN_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_ERR_ALIGN;
    // per-batch byte offsets of q / dout rows must fit the 32-bit buffer addressing
    if ((int64_t)Hq * T * D * 2 >= (int64_t)1 << 31) return ATTN_ERR_UNSUPPORTED;
    if (!nsa_index_fits(B, Hkv, T, block_size, S)) return ATTN_ERR_UNSUPPORTED;
    const size_t need = attn::nsa_sel_bwd_workspace(B, Hq, Hkv, T, D, block_size, S);
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_ERR_ALIGN;
    const hipError_t e = attn::launch_nsa_sel_bwd(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), block_idx, static_cast<const uint16_t *>(out), lse,
        static_cast<const uint16_t *>(dout), static_cast<uint16_t *>(dq),
        static_cast<uint16_t *>(dk), static_cast<uint16_t *>(dv), workspace, B, Hq, Hkv, T, D,
        block_size, S, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_EXPORT size_t nsa_sel_fsa_workspace_bytes(int B, int Hq, int Hkv, int T, int D,
                                               int block_size, int S) {
    if (B <= 0 || Hq <= 0 || T <= 0 || D <= 0 || block_size <= 0 || T % block_size != 0 || S < 1 ||
        Hkv <= 0 || Hq % Hkv != 0)
        return 0;
    return attn::nsa_sel_fsa_workspace(B, Hq, Hkv, T, D, block_size, S);
}

ATTN_EXPORT int nsa_sel_fwd_fsa(const void *q, const void *k, const void *v,
                                const int32_t *block_idx, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, int B, int Hq, int Hkv, int T, int D,
                                int block_size, int S, void *stream) {
    bool noop;
    const int st = nsa_validate(q, k, v, block_idx, B, Hq, Hkv, T, D, block_size, S, &noop);
    if (st != ATTN_OK || noop) return st;
    if (!out) return ATTN_ERR_NULL;
    if (misaligned(out)) return ATTN_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_ERR_ALIGN;
    // per-batch byte offsets of q rows must fit the 32-bit buffer addressing
    if ((int64_t)Hq * T * D * 2 >= (int64_t)1 << 31) return ATTN_ERR_UNSUPPORTED;
    if (!nsa_index_fits(B, Hkv, T, block_size, S)) return ATTN_ERR_UNSUPPORTED;
    const size_t need = attn::nsa_sel_fsa_workspace(B, Hq, Hkv, T, D, block_size, S);
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_ERR_ALIGN;
    const hipError_t e = attn::launch_nsa_sel_fsa(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), block_idx, static_cast<uint16_t *>(out), lse,
        workspace, B, Hq, Hkv, T, D, block_size, S, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_EXPORT const char *attn_status_str(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "null pointer argument";
        case ATTN_ERR_SHAPE: return "invalid shape or scalar argument";
        case ATTN_ERR_UNSUPPORTED: return "unsupported head dim, block size or group size";
        case ATTN_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case ATTN_ERR_LAUNCH: return "HIP kernel launch failed";
        case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case ATTN_ERR_SCRATCH: return "problem needs more than the library's static scratch holds";
        default: return "unknown status";
    }
}
