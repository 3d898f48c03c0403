/*
 * attn.h -- C ABI of libattn.so: fused, tiled causal-attention forwards for
 * AMD Instinct MI355X (gfx950), hand-written HIP.
 *
 * Common rules for every entry point
 * ----------------------------------
 *  - Every tensor pointer is a DEVICE pointer to memory the caller owns and
 *    keeps alive until the work on `stream` has finished.  The library never
 *    allocates, frees, or keeps a pointer after returning (tda_fwd_noalloc
 *    uses a static device array that the library itself carries).
 *  - Tensors are dense and row-major (contiguous) in the shapes given below;
 *    "bf16" means IEEE bfloat16 stored as 16-bit words.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *    enqueued asynchronously; no call synchronises the device or the host.
 *  - Output buffers are fully overwritten (every element is written).
 *  - All arguments are validated on the host before any HIP call.  On a
 *    validation error nothing is enqueued.  Offsets between (batch, head)
 *    slabs are computed in 64-bit, so tensors may exceed 2^31 elements; the
 *    bf16 kernels address within one slab of T x D elements with 32-bit byte
 *    offsets, so every bf16 entry point requires T * D * 2 < 2^31 (T < 2^23
 *    at D = 128, T < 2^24 at D = 64), else ATTN_ERR_UNSUPPORTED.
 *  - The library is stateless (apart from tda_fwd_noalloc's scratch) and may
 *    be called from several host threads.
 *  - A size of zero in B, H/Hq or T is a successful no-op once the other
 *    arguments have been validated; the tensor pointers may then be NULL.
 *
 * Return value: ATTN_OK (0) on success, otherwise one of the negative
 * ATTN_ERR_* codes below; attn_status_str() names each.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
#define ATTN_ERR_NULL (-1)        /* a required pointer is NULL */
#define ATTN_ERR_SHAPE (-2)       /* negative size, inconsistent shape, bad scalar */
#define ATTN_ERR_UNSUPPORTED (-3) /* valid but not built: head dim, block size, group size */
#define ATTN_ERR_ALIGN (-4)       /* a tensor pointer is not 16-byte aligned */
#define ATTN_ERR_LAUNCH (-5)      /* the HIP launch reported an error */
#define ATTN_ERR_WORKSPACE (-6)   /* workspace missing or smaller than required */
#define ATTN_ERR_SCRATCH (-7)     /* needs more than the library's static scratch holds */

/*
 * Threshold Rectified Attention forward, bf16 in / bf16 out.
 *
 * Source: snap-research/TDA, page "triton_threshold_attention.py" -- module
 * docstring (out = ReLU(Q K^T - tau)^p V, tau(i) = beta*sqrt(2 log(i+1)/d))
 * and `_threshold_rela_fwd_kernel` (0-based query position i, natural log,
 * d = head dim, only keys j <= i contribute, fp32 accumulation).
 *
 *   out[b,h,i,:] = sum_{j<=i} max(q_i . k_j - tau_i, 0)^p * v_j
 *   tau_i        = beta * sqrt(2 * ln(i + 1) / D)
 *
 * There is no 1/sqrt(D) scale, no softmax and no normalisation.  A masked
 * pair (j > i) contributes exactly 0 for every beta.
 *
 *   q, k, v : bf16 [B, H, T, D]      (read only)
 *   out     : bf16 [B, H, T, D]      (written; may not alias q, k or v)
 *   D       : 64 or 128 (else ATTN_ERR_UNSUPPORTED)
 *   beta    : finite (else ATTN_ERR_SHAPE)
 *   p       : finite and > 0 (else ATTN_ERR_SHAPE); p == 1 and p == 2 take
 *             exact fast paths, any other p uses exp2(p * log2(x)).
 *
 * Numerics: q.k in bf16 x bf16 products with fp32 accumulation; the weight
 * ReLU(.)^p is computed in fp32 and rounded to bf16 (nearest-even) before
 * it multiplies V; the output accumulates in fp32 and is rounded to bf16.
 */
int tra_fwd(const void *q, const void *k, const void *v, void *out,
            int B, int H, int T, int D, float beta, float p, void *stream);

/*
 * Threshold Rectified Attention forward, fp32 in / fp32 out.
 * Same definition, arguments and errors as tra_fwd; every value (scores,
 * weights, accumulation) is fp32.  Source: as for tra_fwd (the page's
 * forward runs its kernel on fp32 copies of the inputs).
 */
int tra_fwd_f32(const float *q, const float *k, const float *v, float *out,
                int B, int H, int T, int D, float beta, float p, void *stream);

/*
 * Threshold Rectified Attention backward, bf16 in / bf16 out.
 *
 * Source: snap-research/TDA, page "triton_threshold_attention.py" --
 * `_threshold_rela_bwd_kernel_dq`, `_threshold_rela_bwd_kernel_dkv` and
 * `ThresholdRelaFunction.backward` (gradients of q, k and v of the forward
 * above; none for beta or p; returned in the input dtype).
 *
 * With x_ij = q_i . k_j - tau_i over the causal pairs j <= i (masked pairs
 * contribute nothing), w_ij = max(x_ij, 0)^p, g_ij = p * x_ij^(p-1) for
 * x_ij > 0 (else 0) and a_ij = (dout_i . v_j) * g_ij:
 *   dq_i = sum_{j<=i} a_ij k_j,  dk_j = sum_{i>=j} a_ij q_i,  dv_j = sum_{i>=j} w_ij dout_i
 *
 *   q, k, v, dout : bf16 [B, H, T, D]      (read only)
 *   dq, dk, dv    : bf16 [B, H, T, D]      (written; may not alias the inputs or
 *                                            each other)
 *   D, beta, p    : as tra_fwd
 *
 * Numerics: scores and dout.v in fp32 from bf16 products; w and a rounded to
 * bf16 before the products that consume them; fp32 accumulation; gradients
 * rounded to bf16.  Every gradient row is written by one wavefront (no
 * atomics): results are deterministic.
 */
int tra_bwd(const void *q, const void *k, const void *v, const void *dout,
            void *dq, void *dk, void *dv,
            int B, int H, int T, int D, float beta, float p, void *stream);

/*
 * Threshold Differential Attention forward, bf16 in / bf16 out.
 *
 * Source: snap-research/TDA, page "triton_threshold_attention.py" --
 * `differential_threshold_rela_triton` (optional L2 normalisation of q1, k1,
 * q2, k2 along the head dimension, two Threshold Rectified Attention outputs
 * over the same v, beta and p, combined as out1 - clamp(lambda, 0, 1) * out2),
 * with torch.nn.functional.normalize's x / max(||x||_2, 1e-12).
 *
 *   out[b,h,i,:] = sum_{j<=i} ( max(a1_ij - tau_i, 0)^p
 *                               - lam * max(a2_ij - tau_i, 0)^p ) * v_j
 *   a_ij = q_i . k_j (normalize == 0) or the cosine of q_i and k_j (normalize != 0)
 *   lam  = min(max(lambda, 0), 1),   tau_i = beta * sqrt(2 * ln(i + 1) / D)
 *
 *   q1, q2, k1, k2, v : bf16 [B, H, T, D]      (read only)
 *   out               : bf16 [B, H, T, D]      (written; may not alias an input)
 *   workspace         : device memory the call may overwrite, at least
 *                       tda_workspace_bytes(B, H, T, D, normalize) bytes, 16-byte
 *                       aligned; it holds the normalised k1 and k2 rows.  May be
 *                       NULL when that size is 0 (normalize == 0).  Smaller or
 *                       NULL when needed: ATTN_ERR_WORKSPACE.  Calls that share
 *                       one workspace must not overlap in time.
 *   D                 : 64 or 128 (else ATTN_ERR_UNSUPPORTED)
 *   beta, lambda      : finite (else ATTN_ERR_SHAPE)
 *   p                 : finite and > 0 (else ATTN_ERR_SHAPE)
 *
 * Normalisation follows torch.nn.functional.normalize on bf16 tensors: the
 * row's 2-norm is itself rounded to bf16 (nearest-even, at least the bf16 value
 * of 1e-12) and each element x / norm is rounded to bf16.
 *
 * Numerics: as tra_fwd; normalised rows are rounded to bf16; the two
 * weights of a pair are combined in fp32 and rounded to bf16 once, and one
 * fp32 accumulation over v gives the output (rounded to bf16 once).
 */
int tda_fwd(const void *q1, const void *q2, const void *k1, const void *k2, const void *v,
            void *out, void *workspace, size_t workspace_bytes,
            int B, int H, int T, int D, float beta, float lambda, float p, int normalize,
            void *stream);

/* Workspace bytes tda_fwd needs for these sizes (0 when normalize == 0, or
 * when a size is negative or zero). */
size_t tda_workspace_bytes(int B, int H, int T, int D, int normalize);

/*
 * tda_fwd without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same definition, arguments (minus the workspace), numerics
 * and errors as tda_fwd, and the same kernels.
 *
 * The normalised k1 and k2 rows go to a static scratch array inside the library
 * (tda_noalloc_scratch_bytes() = 64 MiB), which every GPU the library runs on
 * holds until the process ends; its address on the current device is looked up
 * on the first call made with that device current (a HIP runtime query, no
 * allocation).  Nothing is allocated or freed by any call.
 *
 *   limit   : tda_workspace_bytes(B, H, T, D, normalize) <= 64 MiB, i.e.
 *             B*H*T*D <= 2^24 elements when normalising (else ATTN_ERR_SCRATCH);
 *             without normalisation no scratch is used and there is no limit.
 *   device  : the current HIP device; `stream` must belong to it.
 *   sharing : all calls on one GPU share that GPU's scratch, which keeps the last
 *             call's contents (each call overwrites every byte it reads), so calls
 *             whose work may overlap in time on one GPU -- on different streams, or
 *             from several host threads -- race and must be serialised by the
 *             caller.  Calls on one stream are ordered and safe.
 *   errors  : as tda_fwd; ATTN_ERR_SCRATCH as above; ATTN_ERR_LAUNCH also when
 *             the scratch address cannot be looked up.
 */
int tda_fwd_noalloc(const void *q1, const void *q2, const void *k1, const void *k2, const void *v,
                    void *out, int B, int H, int T, int D, float beta, float lambda, float p,
                    int normalize, void *stream);

/* Bytes of the static scratch tda_fwd_noalloc uses (its size limit). */
size_t tda_noalloc_scratch_bytes(void);

/*
 * NSA selection-branch forward, bf16 in / bf16 out, fp32 lse.
 *
 * Source: msb-msb/openbox-llm, page "nsa_selection_kernel.py" -- module
 * docstring (GQA layout, Hq = Hkv * G, kv head of query head h is h / G, the
 * S selected blocks per (batch, kv head, query) are shared by the G heads of
 * the group, -1 slots are padding, causal j <= i, softmax with scale D^-0.5,
 * a query with no valid block outputs 0), `selection_forward_reference`
 * (the selection is a set: a block listed twice is attended once) and
 * `_selection_fwd_kernel` (lse = max + log(sum) of the scaled scores, natural
 * log, finite sentinel -1e9 for an empty row).
 *
 * For query i of head h (kv = h / G), A = the union over slots s of the
 * tokens j of block blk = block_idx[b,kv,i,s] (blk*block_size <= j <
 * (blk+1)*block_size) with j <= i.  A negative slot, or a block id >=
 * T/block_size, adds nothing.  With s_j = (q_i . k_j) / sqrt(D):
 *   out[b,h,i,:] = sum_{j in A} softmax_j(s) v_j,   lse[b,h,i] = ln sum_{j in A} exp(s_j)
 * and an empty A gives out = 0 (exactly) and lse = -1e9 (exactly).
 *
 *   q          : bf16  [B, Hq, T, D]
 *   k, v       : bf16  [B, Hkv, T, D]
 *   block_idx  : int32 [B, Hkv, T, S]
 *   out        : bf16  [B, Hq, T, D]  (written)
 *   lse        : fp32  [B, Hq, T]     (written; may be NULL to skip it)
 *   D          : 64 or 128                     (else ATTN_ERR_UNSUPPORTED)
 *   block_size : 32, 64 or 128                 (else ATTN_ERR_UNSUPPORTED)
 *   Hq % Hkv   : must be 0                     (else ATTN_ERR_SHAPE)
 *   G = Hq/Hkv : 1 .. 16                       (else ATTN_ERR_UNSUPPORTED)
 *   T          : a multiple of block_size      (else ATTN_ERR_SHAPE), and
 *                T * D * 2 < 2^31               (else ATTN_ERR_UNSUPPORTED)
 *   S          : 1 .. 64                       (< 1: ATTN_ERR_SHAPE, > 64: ATTN_ERR_UNSUPPORTED)
 *
 * Numerics: scores in fp32 from bf16 products; softmax state (running max,
 * sum, accumulator) in fp32; probabilities rounded to bf16 before they
 * multiply V; out rounded to bf16.
 */
int nsa_sel_fwd(const void *q, const void *k, const void *v, const int32_t *block_idx,
                void *out, float *lse,
                int B, int Hq, int Hkv, int T, int D, int block_size, int S, void *stream);

/*
 * NSA selection-branch backward, bf16 in / bf16 out.
 *
 * Source: msb-msb/openbox-llm, page "nsa_selection_kernel.py" -- the forward
 * above defines the function; the page keeps its lse output for a backward
 * pass that it does not show.  These are the gradients of that forward with
 * respect to q, k and v (block_idx is an integer index and gets none).
 *
 * With A_i the attended set of query i (as in the forward), s_ij = (q_i . k_j)
 * / sqrt(D), P_ij = exp(s_ij - lse_i), dP_ij = dout_i . v_j, delta_i =
 * sum_{j in A_i} P_ij dP_ij (= dout_i . out_i) and dS_ij = P_ij (dP_ij - delta_i),
 * for each head h of kv group kv:
 *   dq_i = sum_{j in A_i} dS_ij k_j / sqrt(D)
 *   dk_j = sum_{h in group, i : j in A_i} dS_ij q_i / sqrt(D)
 *   dv_j = sum_{h in group, i : j in A_i} P_ij dout_i
 *
 *   q, dout, out : bf16 [B, Hq, T, D]   (out and lse as returned by nsa_sel_fwd)
 *   k, v         : bf16 [B, Hkv, T, D]
 *   block_idx    : int32 [B, Hkv, T, S]
 *   lse          : fp32 [B, Hq, T]
 *   dq           : bf16 [B, Hq, T, D]   (written)
 *   dk, dv       : bf16 [B, Hkv, T, D]  (written; a key row no query attends gets 0)
 *   workspace    : device memory the call overwrites, at least
 *                  nsa_sel_bwd_workspace_bytes(...) bytes, 256-byte aligned (else
 *                  ATTN_ERR_WORKSPACE / ATTN_ERR_ALIGN).  Calls that share one
 *                  workspace must not overlap in time.
 *   sizes        : as nsa_sel_fwd; in addition Hq*T*D*2 < 2^31 and
 *                  B*Hkv*T*min(S, T/block_size) < 2^31 (else ATTN_ERR_UNSUPPORTED).
 *
 * Numerics: scores, dP and delta in fp32 from bf16 products.  delta is summed
 * from the recomputed probabilities; dout . out (out is bf16) serves only as an
 * estimate m of it, with dq = scale (sum_j P_ij (dP_ij - m) k_j - (delta_i - m)
 * sum_j P_ij k_j).  P and dS rounded to bf16 before the products that consume
 * them; fp32 accumulation; every gradient row has one writer (no atomics on
 * values): deterministic.
 */
int nsa_sel_bwd(const void *q, const void *k, const void *v, const int32_t *block_idx,
                const void *out, const float *lse, const void *dout,
                void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
                int B, int Hq, int Hkv, int T, int D, int block_size, int S, void *stream);

/* Workspace bytes nsa_sel_bwd needs for these sizes (0 if a size is invalid or
 * the problem is empty). */
size_t nsa_sel_bwd_workspace_bytes(int B, int Hq, int Hkv, int T, int D, int block_size, int S);

/*
 * NSA selection-branch forward in block-outer form: the same outputs as
 * nsa_sel_fwd, computed block by block.
 *
 * Source: msb-msb/openbox-llm, page "nsa_selection_kernel.py" --
 * `_selection_fwd_blockouter_kernel` (each selected key block loaded once, the
 * queries that select it processed against it, a partial (max, sum, weighted
 * sum) left per (query, block)) and `selection_forward_fsa` (the partials of a
 * query merged with the log-sum-exp rule: one softmax over the union of its
 * selected causal tokens).  Same arguments, semantics and limits as
 * nsa_sel_fwd, plus:
 *   workspace : device memory the call overwrites, at least
 *               nsa_sel_fsa_workspace_bytes(...) bytes, 256-byte aligned (else
 *               ATTN_ERR_WORKSPACE / ATTN_ERR_ALIGN); it holds the inverted
 *               selection and one partial per (query, selected block, head).
 *               Calls that share one workspace must not overlap in time.
 *   sizes     : in addition Hq*T*D*2 < 2^31 and B*Hkv*T*min(S, T/block_size)
 *               < 2^31 (else ATTN_ERR_UNSUPPORTED).
 *
 * Numerics: scores fp32 from bf16 products; per block the row max, sum and
 * weighted sum in fp32, probabilities rounded to bf16 before they multiply V,
 * the block's normalised output stored in bf16; the merge in fp32; out bf16.
 *
 * Which form to call: nsa_sel_fwd gathers the selected K/V rows once per (kv
 * group, query), this form once per (kv group, block segment) but writes and
 * reads a partial per (query, block, head).  Measured on MI355X at Hq=16,
 * T=8192, D=128, block 64, S=16: this form is faster for G = Hq/Hkv <= 4
 * (about 5.5x at G=1, 3x at G=2, 1.6x at G=4), nsa_sel_fwd for G >= 8
 * (0.8x at G=8, 0.4x at G=16).
 */
int nsa_sel_fwd_fsa(const void *q, const void *k, const void *v, const int32_t *block_idx,
                    void *out, float *lse, void *workspace, size_t workspace_bytes,
                    int B, int Hq, int Hkv, int T, int D, int block_size, int S, void *stream);

/* Workspace bytes nsa_sel_fwd_fsa needs for these sizes (0 if a size is invalid
 * or the problem is empty). */
size_t nsa_sel_fsa_workspace_bytes(int B, int Hq, int Hkv, int T, int D, int block_size, int S);

/* Human-readable name of a status code (static string, never NULL). */
const char *attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
