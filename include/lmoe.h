/*
 * lmoe.h — C ABI of the Stable LatentMoE layer forward pass on AMD gfx950 (MI355X).
 *
 * Pages cited (site and section):
 *   [vxz]   vxz.us, "苏神复盘 Kimi K3：896 个专家背后，藏着哪些关键技术取舍？", sections 01 and 02.
 *   [tahou] tahou.com K3 architecture write-up, sections SiTU激活优化, 归一化策略调整, 负载均衡优化.
 *   [slm]   lukebest.github.io "Stable Latent MoE", sections 路由机制, Quantile Balancing,
 *           Latent-Space MoE, SiTU 激活, 训练基础设施.
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is caller-owned DEVICE memory (hipMalloc / PyTorch), row-major, and
 *     16-byte aligned. The library never allocates or frees device memory; scratch space is the
 *     caller's `workspace` (size from lmoe_workspace_bytes).
 *   - Calls only enqueue kernels on `stream` (a hipStream_t; NULL = the null stream) and never
 *     synchronise with the host. Ragged expert sizes stay on the device.
 *   - Arguments are validated before anything is enqueued; on an error the call returns a status
 *     and enqueues nothing, so outputs are untouched. A failed launch returns LMOE_ERR_HIP. Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - Storage types: `act_dtype` selects float32 or bfloat16 (bit pattern in uint16) for
 *     activations and layer weights. Router weights, bias, scores, thresholds, gamma and combine
 *     weights are always float32. Accumulation is float32.
 *   - Concurrent calls that share output or workspace buffers race; distinct buffers are safe.
 */
#ifndef LMOE_H
#define LMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMOE_OK = 0,
  LMOE_ERR_INVALID_ARGUMENT = 1, /* NULL or misaligned pointer, inconsistent shape */
  LMOE_ERR_UNSUPPORTED = 2,      /* valid but outside what the kernels handle (see each call) */
  LMOE_ERR_WORKSPACE = 3,        /* workspace NULL or smaller than lmoe_workspace_bytes() */
  LMOE_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} lmoe_status;

typedef enum { LMOE_F32 = 0, LMOE_BF16 = 1 } lmoe_dtype;

/* Layer shape. T tokens; D = d_model; L = d_latent; E routed experts; top_k = k; inter = routed
 * expert inner size I; n_shared = S; inter_shared = I_s; n_bins = NB; beta1 / beta2 = SiTU gate
 * bound and up-branch soft cap ([tahou] SiTU激活优化: 4 and 25); rms_eps for RMSNorm. */
typedef struct {
  int32_t T, d_model, d_latent, n_experts, top_k, inter, n_shared, inter_shared, n_bins;
  float beta1, beta2, rms_eps;
  int32_t act_dtype; /* lmoe_dtype */
} lmoe_shape;

/* Shape limits common to the calls: 0 < top_k < n_experts and T >= 0 (T = 0 enqueues nothing but
 * the zero offsets of lmoe_permute), else LMOE_ERR_INVALID_ARGUMENT; d_model, d_latent, inter and
 * inter_shared multiples of 64, n_experts <= 2048, top_k <= 64, n_bins in [2, 32768] and a latent
 * row of at most 16 KiB (d_latent <= 8192 in bf16, 4096 in f32), else LMOE_ERR_UNSUPPORTED. */

enum {
  LMOE_CALL_ROUTE = 0, LMOE_CALL_PERMUTE = 1, LMOE_CALL_GROUPED_GLU = 2, LMOE_CALL_COMBINE_NORM_UP = 3,
  /* backward calls */
  LMOE_CALL_BWD_UP = 16, LMOE_CALL_BWD_COMBINE_NORM = 17, LMOE_CALL_BWD_EXPERTS = 18, LMOE_CALL_BWD_DOWN = 19,
  LMOE_CALL_BWD_SHARED = 20, LMOE_CALL_GROUPED_GLU_MX = 32
};

/* Bytes of workspace `which_call` needs for this shape (0 when none). For LMOE_CALL_GROUPED_GLU
 * the value covers any group count up to max(n_experts, 1) and the shared-expert call.
 * Small batches (whose dense GEMMs would occupy fewer than half the CUs) split the contraction
 * dimension and sum f32 partial products in the workspace; the returned size includes that space.
 * A call given less than the returned size but at least its own minimum (the tile list, the router
 * weight split, the permutation counts) runs its dense GEMMs unsplit: same results up to f32
 * summation order, slower on small batches. */
size_t lmoe_workspace_bytes(const lmoe_shape* shape, int which_call);

/* Human-readable name of a status. */
const char* lmoe_status_string(lmoe_status status);

/* One-time preparation of the router weights for bf16 layers (A1 at f32 accuracy on bf16 MFMA):
 * w_router [E, D] f32 -> w_router_split [E, 3D] bf16 bits, row e = [hi | mid | lo] with
 * hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid) (each step one f32 operation), so that
 * every product x . hi + x . mid + x . lo is exact in f32. Re-run after every weight change.
 * LMOE_ERR_UNSUPPORTED for f32 layers (their router multiplies the f32 weights directly). */
lmoe_status lmoe_split_router(const lmoe_shape* shape, const float* w_router, void* w_router_split, void* stream);

/* A1 + A2: router scores, biased top-k selection and combine weights.
 * [slm] 路由机制 (router over x, then top-K); [vxz] 02 (per-expert selection bias, no aux loss).
 *   x            [T, D] act_dtype         token activations
 *   w_router     [E, D] f32               router weights (unused when w_router_split is given)
 *   w_router_split [E, 3D] bf16 or NULL   the split written by lmoe_split_router (bf16 layers only;
 *                                         NULL: the call splits w_router itself, in the workspace;
 *                                         LMOE_ERR_INVALID_ARGUMENT if given for an f32 layer)
 *   bias         [E] f32                  quantile-balancing selection bias b
 *   logit_offset [E] f32 or NULL          added to the logits before the sigmoid
 *   scores       [T, E] f32   (out)       s = sigmoid(x . w_router^T + logit_offset)
 *   topk_idx     [T, k] i32   (out)       experts in rank order of s + b (descending; ties go to the
 *                                         lower expert index)
 *   topk_w       [T, k] f32   (out)       s of the selected experts divided by their sum
 *   thresh       [T, 2] f32   (out)       k-th and (k+1)-th largest s + b of the row
 *   workspace    LMOE_CALL_ROUTE bytes    (the per-call split when w_router_split is NULL, and
 *                                         split-K partial logits of small or half-chip batches)  */
lmoe_status lmoe_route(const lmoe_shape* shape, const void* x, const float* w_router, const void* w_router_split,
                       const float* bias, const float* logit_offset, float* scores, int32_t* topk_idx,
                       float* topk_w, float* thresh, void* workspace, size_t workspace_bytes, void* stream);

/* A3: quantile-balancing histogram ([vxz] 02; [tahou] 负载均衡优化: bin the scores after mapping
 * them to 0..1, and add histograms across micro-batches).
 * For every (t, e): s_hat = scores + bias (f32 add); theta = thresh[t,1] if e is among the top-k of
 * t, else thresh[t,0]; m = s_hat - theta; u = clamp((m + 1) * 0.5, 0, 1);
 * bin = min(NB - 1, floor(u * NB)); hist[e, bin] += 1. Each step is one f32 operation.
 *   scores [T,E] f32, bias [E] f32, topk_idx [T,k] i32, thresh [T,2] f32: as written by lmoe_route
 *   hist   [E, NB] u32 (in/out)           incremented (never cleared here)                       */
lmoe_status lmoe_qb_histogram(const lmoe_shape* shape, const float* scores, const float* bias,
                              const int32_t* topk_idx, const float* thresh, uint32_t* hist, void* stream);

/* A4: quantile-balancing bias update at a step boundary ([vxz] 02; [slm] Quantile Balancing).
 * Per expert, in f64: c* = (E - k) * n_acc / E; j* = first bin with cumulative count >= c*;
 * u_hat = (j* + (c* - cum(j* - 1)) / hist[e, j*]) / NB; m_hat = 2 u_hat - 1;
 * bias[e] = (float)((double)bias[e] - m_hat). Then hist is zeroed. n_acc = tokens counted into
 * hist since the last update; n_acc <= 0 leaves bias unchanged (hist is still zeroed).
 *   hist [E, NB] u32 (in/out), bias [E] f32 (in/out)                                             */
lmoe_status lmoe_qb_update(const lmoe_shape* shape, uint32_t* hist, int64_t n_acc, float* bias, void* stream);

/* A5 + A6: down-projection to the latent space and permutation of (token, slot) pairs by expert
 * ([vxz] 01: tokens are compressed to d_latent before being dispatched to the routed experts;
 * [slm] 训练基础设施: static shapes, no host synchronisation).
 *   x              [T, D] act_dtype
 *   w_down         [L, D] act_dtype
 *   topk_idx       [T, k] i32               expert ids; an id outside [0, E), or one a row lists a
 *                                           second time, drops that pair (slot -1, no sorted row)
 *   x_lat          [T, L] act_dtype (out)   x . w_down^T
 *   expert_offsets [E + 1] i32 (out)        first sorted row of each expert; [E] = pairs kept (T*k
 *                                           when every row holds k distinct ids in [0, E), as
 *                                           lmoe_route writes them)
 *   sorted_token   [T*k] i32 (out)          token of each sorted row (tokens ascending per expert)
 *   slot_of_pair   [T*k] i32 (out)          sorted row of pair t*k + j (-1 for a dropped pair)
 *   x_perm         [T*k, L] act_dtype (out) x_lat[sorted_token[r]], or NULL to skip the copy (the
 *                                           routed GEMM can read x_lat through sorted_token)
 *   workspace      LMOE_CALL_PERMUTE bytes                                                         */
lmoe_status lmoe_permute(const lmoe_shape* shape, const void* x, const void* w_down, const int32_t* topk_idx,
                         void* x_lat, int32_t* expert_offsets, int32_t* sorted_token, int32_t* slot_of_pair,
                         void* x_perm, void* workspace, size_t workspace_bytes, void* stream);

/* A7 + A8 (and A10 with one group): grouped SiTU-GLU FFN over ragged row groups.
 * [tahou] SiTU激活优化 and [slm] SiTU 激活: gate = first half of the first projection, up = second
 * half; h = beta1*tanh(g/beta1)*sigmoid(g) * beta2*tanh(u/beta2) in f32, fused in the epilogue.
 * For group g with rows [off[g], off[g+1]):
 *   [g | u] = A[rows] . w1[g]^T ;  h[rows] = SiTU-GLU ;  y[rows] = h[rows] . w2[g]^T
 * where row r of A is a[a_row_index[r]] (dispatch by gather: a = x_lat, a_row_index = sorted_token
 * from lmoe_permute), or a[r] when a_row_index is NULL. A gathered index outside [0, a_rows) reads
 * as a zero row.
 *   n_groups      G >= 1
 *   rows          total rows of h and y (= group_offsets[G])
 *   K             input width (multiple of 64), inter: inner size (multiple of 64),
 *   n_out         output width
 *   a             [a_rows, K] act_dtype; a_rows must equal rows when a_row_index is NULL
 *   a_row_index   [rows] i32 device, or NULL
 *   group_offsets [G + 1] i32 device, non-decreasing, [0] = 0; NULL means one group of all rows
 *   w1            [G, 2*inter, K] act_dtype (gate rows 0..inter-1, up rows inter..2*inter-1)
 *   w2            [G, n_out, inter] act_dtype, or NULL to stop after h (y is then unused)
 *   h             [rows, inter] act_dtype (out)
 *   y             [rows, n_out] y_dtype (out; y_dtype is LMOE_F32 or act_dtype)
 *   workspace     LMOE_CALL_GROUPED_GLU bytes (device tile list; split-K partials for one group)
 * With a_row_index, a must be under 2 GiB (31-bit byte offsets; LMOE_ERR_UNSUPPORTED otherwise). */
lmoe_status lmoe_grouped_situ_glu(const lmoe_shape* shape, int32_t n_groups, int32_t rows, int32_t K,
                                  int32_t inter, int32_t n_out, const void* a, int32_t a_rows,
                                  const int32_t* a_row_index, const int32_t* group_offsets, const void* w1,
                                  const void* w2, void* h, void* y, int32_t y_dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* lmoe_grouped_situ_glu without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation). Same arguments
 * and results, except that:
 *   - the grouped m-tile list lives in a 16 KiB array of the library's own device memory, one per
 *     device, held until the process ends: n_groups + 1 <= 4096, else LMOE_ERR_UNSUPPORTED;
 *   - dense calls (group_offsets NULL) run without split-K partials (same results up to f32
 *     summation order; slower on small batches).
 * Every call on one device shares that device's array: calls that overlap on one device (other
 * streams, other host threads) race and must be ordered by the caller. The array's contents are
 * rewritten in full by each call, nothing needs clearing. Allocates nothing (no hipMalloc, no
 * library allocation); the first call on a device looks the array's address up once. */
lmoe_status lmoe_grouped_situ_glu_noalloc(const lmoe_shape* shape, int32_t n_groups, int32_t rows, int32_t K,
                                          int32_t inter, int32_t n_out, const void* a, int32_t a_rows,
                                          const int32_t* a_row_index, const int32_t* group_offsets,
                                          const void* w1, const void* w2, void* h, void* y, int32_t y_dtype,
                                          void* stream);

/* Shared experts as one FFN ([vxz] 01: always-on shared experts; by linearity S SiTU-GLU experts
 * equal one of inner size S*I_s with the gate blocks, up blocks and down blocks concatenated).
 * One-time weight repack, not part of the per-batch pass:
 *   w1s [S, 2*I_s, D] -> w1s_packed [2*S*I_s, D] = gates of experts 0..S-1, then their up rows
 *   w2s [S, D, I_s]   -> w2s_packed [D, S*I_s]   = [w2s[0] | w2s[1] | ...]                        */
lmoe_status lmoe_pack_shared(const lmoe_shape* shape, const void* w1s, const void* w2s, void* w1s_packed,
                             void* w2s_packed, void* stream);

/* A9 + A11: router-weighted combine, RMSNorm, up-projection and shared-expert add
 * ([vxz] 02 and [tahou] 归一化策略调整: the norm sits after the aggregation and before the
 * up-projection; no extra scaling factor).
 *   y_perm       [T*k, L] act_dtype       routed expert outputs in sorted-row order
 *   slot_of_pair [T*k] i32
 *   topk_w       [T, k] f32
 *   gamma        [L] f32 or NULL (= ones)
 *   w_up         [D, L] act_dtype
 *   shared part, at most one of:
 *     y_shared   [T, D] f32               the shared experts' output, added before the final rounding
 *     h_shared + w2_shared                their inner activations [T, S*I_s] and packed down weights
 *                                         [D, S*I_s] (lmoe_pack_shared): out = [n | h_s] . [w_up |
 *                                         w2_shared]^T accumulates both products in one f32 sum
 *   n_out        [T, L] act_dtype (out)   n = gamma * z / sqrt(mean(z^2) + eps), z = sum_j w_tj y(t,j)
 *   out          [T, D] out_dtype (out)   n . w_up^T + shared part, rounded once from the f32
 *                                         accumulator; out_dtype is LMOE_F32 or act_dtype
 *   workspace    LMOE_CALL_COMBINE_NORM_UP bytes, or NULL (no split-K for small batches)          */
lmoe_status lmoe_combine_norm_up(const lmoe_shape* shape, const void* y_perm, const int32_t* slot_of_pair,
                                 const float* topk_w, const float* gamma, const void* w_up,
                                 const float* y_shared, const void* h_shared, const void* w2_shared,
                                 void* n_out, void* out, int32_t out_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* A9 alone: the combine and RMSNorm of lmoe_combine_norm_up (same arguments, same n_out). Its
 * kernel holds few registers and no LDS to speak of, so it can run on one stream while another
 * stream runs a GEMM that does not read n (the shared experts' GEMM1): its waves fit beside a
 * GEMM workgroup on each CU. No workspace.                                                        */
lmoe_status lmoe_combine_norm(const lmoe_shape* shape, const void* y_perm, const int32_t* slot_of_pair,
                              const float* topk_w, const float* gamma, void* n_out, void* stream);

/* A11 alone: the up-projection and shared-expert add of lmoe_combine_norm_up, from an n written
 * by lmoe_combine_norm (same arguments, same out; workspace as for LMOE_CALL_COMBINE_NORM_UP).
 * lmoe_combine_norm followed by lmoe_up_project on one stream equals lmoe_combine_norm_up bit for
 * bit.                                                                                              */
lmoe_status lmoe_up_project(const lmoe_shape* shape, const void* n, const void* w_up, const float* y_shared,
                            const void* h_shared, const void* w2_shared, void* out, int32_t out_dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ================================================================================================
 * Backward pass (training). The pages train this layer ([vxz] 01-02, [slm] 训练基础设施) but
 * print no backward pass; these calls apply the chain rule to the forward above, step by step in
 * reverse. The quantile-balancing bias selects experts only and has no gradient; the top-k set is
 * held fixed and the combine weights are differentiated through the unbiased scores.
 * Storage: the incoming dout and every activation gradient are act_dtype; weight gradients, dgamma,
 * the router-logit gradients and dx are f32. Each output is written in full (no accumulation into
 * caller data except dx where stated). Gradients of unselected experts are zero. The forward
 * tensors are those the forward calls produced for the same batch.
 * Workspace: lmoe_workspace_bytes(shape, LMOE_CALL_BWD_*); transposed activations live there.
 * ============================================================================================== */

/* B0: transposed copies of the dense weights (their backward products contract over the forward's
 * output dimension and run on the 256x256 MFMA pipeline). Re-run after every weight change. The
 * routed experts' weights need no copy: their products read them in place.
 *   w_up [D, L] -> w_up_t [L, D];  w_down [L, D] -> w_down_t [D, L];
 *   w2s_packed [D, S*I_s] -> w2s_t [S*I_s, D];  w1s_packed [2*S*I_s, D] -> w1s_t [D, 2*S*I_s]
 *   (the shared pair may both be NULL)                                                           */
lmoe_status lmoe_bwd_transpose_weights(const lmoe_shape* shape, const void* w_up, const void* w2s_packed,
                                       const void* w1s_packed, const void* w_down, void* w_up_t, void* w2s_t,
                                       void* w1s_t, void* w_down_t, void* stream);

/* B1 (A11 reversed): out = [n | h_s] . [w_up | w2s_packed]^T.
 *   dout [T, D], n [T, L], h_shared [T, S*I_s] or NULL (then no shared part), w_up_t, w2s_t from B0
 *   dn [T, L] (out) = dout . w_up;  dh_shared [T, S*I_s] (out) = dout . w2s_packed
 *   dw_up [D, L] f32 (out) = dout^T n;  dw2_shared [D, S*I_s] f32 (out) = dout^T h_s (packed)   */
lmoe_status lmoe_bwd_up(const lmoe_shape* shape, const void* dout, const void* n, const void* h_shared,
                        const void* w_up_t, const void* w2s_t, void* dn, void* dh_shared, float* dw_up,
                        float* dw2_shared, void* workspace, size_t workspace_bytes, void* stream);

/* B2 (A9 and the combine weights reversed), per token t with z = sum_j w_tj y(t,j) recomputed:
 *   dz = r gamma dn - (r^3 / L) sum(gamma dn z) z,  r = (mean(z^2) + eps)^-1/2;  dgamma = sum_t dn z r
 *   dy_perm[slot(t,j)] = w_tj dz;  dw_tj = <dz, y(t,j)>;  S = sum_j s_tj (selected scores);
 *   dlogit[t,j] = (dw_tj - sum_i w_ti dw_ti) / S * s_tj (1 - s_tj);  dlogit_sorted[slot(t,j)] = the same
 *   dn [T, L], y_perm [T*k, L], slot_of_pair, topk_idx, scores [T, E], topk_w, gamma: forward tensors
 *   dy_perm [T*k, L] (out), dlogit [T, k] f32 (out), dlogit_sorted [T*k] f32 (out), dgamma [L] f32 (out) */
lmoe_status lmoe_bwd_combine_norm(const lmoe_shape* shape, const void* dn, const void* y_perm,
                                  const int32_t* slot_of_pair, const int32_t* topk_idx, const float* scores,
                                  const float* topk_w, const float* gamma, void* dy_perm, float* dlogit,
                                  float* dlogit_sorted, float* dgamma, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* B3 (A1 reversed): logits = x . w_router^T (+ offset).
 *   dw_router [E, D] f32 (out): row e = sum over expert e's sorted rows r of dlogit_sorted[r] x[sorted_token[r]]
 *   dx [T, D] f32 (out, overwritten) = sum_j dlogit[t, j] w_router[topk_idx[t, j]]                   */
lmoe_status lmoe_bwd_router(const lmoe_shape* shape, const void* x, const float* w_router, const float* dlogit,
                            const float* dlogit_sorted, const int32_t* topk_idx, const int32_t* expert_offsets,
                            const int32_t* sorted_token, float* dw_router, float* dx, void* stream);

/* B4 (A7 + A8 reversed), rows in expert-sorted order, expert e on rows [off_e, off_{e+1}):
 *   dh = dy . w2_e (out, [T*k, I]);  dw2_e = dy_e^T h_e (f32 [E, L, I], out)
 *   [g | u] = x_lat[sorted_token] . w1_e^T recomputed; dgu (out, [T*k, 2I]) = [dg | du] of SiTU-GLU
 *   dx_perm = dgu . w1_e (out, [T*k, L]);  dw1_e = dgu_e^T x_lat[sorted_token]_e (f32 [E, 2I, L], out)
 *   x_lat [T, L], sorted_token, expert_offsets, w1 [E, 2I, L], w2 [E, L, I], h [T*k, I], dy_perm:
 *   forward tensors and weights / B2                                                              */
lmoe_status lmoe_bwd_experts(const lmoe_shape* shape, const void* x_lat, const int32_t* sorted_token,
                             const int32_t* expert_offsets, const void* w1, const void* w2, const void* h,
                             const void* dy_perm, void* dh, void* dgu, void* dx_perm, float* dw1, float* dw2,
                             void* workspace, size_t workspace_bytes, void* stream);

/* B5 (A6 + A5 reversed): dx_lat[t] = sum_j dx_perm[slot(t,j)] (out, [T, L]);
 *   dw_down [L, D] f32 (out) = dx_lat^T x;  dx [T, D] f32 (in/out) += dx_lat . w_down            */
lmoe_status lmoe_bwd_down(const lmoe_shape* shape, const void* x, const void* dx_perm, const int32_t* slot_of_pair,
                          const void* w_down_t, void* dx_lat, float* dw_down, float* dx, void* workspace,
                          size_t workspace_bytes, void* stream);

/* B6 (A10 reversed, packed shared experts): [g_s | u_s] = x . w1s_packed^T recomputed;
 *   dgu_shared [T, 2*S*I_s] (out) = [dg_s | du_s] of SiTU-GLU for dh_shared (B1);
 *   dw1s_packed [2*S*I_s, D] f32 (out) = dgu_shared^T x;  dx [T, D] f32 (in/out) += dgu_shared . w1s_packed */
lmoe_status lmoe_bwd_shared(const lmoe_shape* shape, const void* x, const void* w1s_packed, const void* w1s_t,
                            const void* dh_shared, void* dgu_shared, float* dw1s_packed, float* dx, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ================================================================================================
 * MX formats for the routed experts ([slm] 训练基础设施: MXFP4 weights with MXFP8 activations).
 * The pages name the formats only; these calls follow the OCP Microscaling definitions: blocks of
 * 32 consecutive elements along the contraction dimension share an E8M0 scale byte e (value
 * 2^(e - 127)); the shared exponent is floor(log2(block max)) - emax (emax 2 for FP4 E2M1, 8 for
 * FP8 E4M3), clamped to [-127, 127], 0 for an all-zero block; each element is v / 2^(e - 127)
 * rounded to nearest, ties to the even significand, saturated at the largest normal (6, 448).
 * ============================================================================================== */
enum { LMOE_MX_FP4 = 4, LMOE_MX_FP8 = 8 };

/* MX quantisation of the rows of x [rows, K] (act_dtype, K a multiple of 32) along K.
 *   fmt LMOE_MX_FP4: codes [rows, K/2] u8, two E2M1 codes per byte, element 2i in the low nibble
 *   fmt LMOE_MX_FP8: codes [rows, K] u8, one E4M3 code per byte (NaN codes never produced)
 *   scales [rows, K/32] u8 E8M0 bytes. x and codes 16-byte aligned.
 * Routed weights: w1 as rows = E*2I, K = L; w2 as rows = E*L, K = I (one-time, per weight change). */
lmoe_status lmoe_mx_quantize(const lmoe_shape* shape, int32_t fmt, int64_t rows, int32_t K, const void* x,
                             void* codes, void* scales, void* stream);

/* A7 + A8 with MX operands: the routed experts of lmoe_grouped_situ_glu on MXFP8 activations and
 * MXFP4 weights (bf16 act_dtype only). Per group g:
 *   [g | u] = deq(A[rows]) . deq(w1[g])^T ;  h = SiTU-GLU (f32, stored bf16) ;
 *   h is MX-quantised to FP8 along inter ;  y[rows] = deq(hq[rows]) . deq(w2[g])^T (stored bf16)
 * The products run on the scaled MFMA with f32 accumulation.
 *   K, inter      multiples of 128
 *   a_codes       [a_rows, K] FP8 codes, a_scales [a_rows, K/32] (lmoe_mx_quantize of x_lat, fmt FP8)
 *   a_row_index, group_offsets, a_rows, rows, n_groups, n_out: as lmoe_grouped_situ_glu
 *   w1_codes      [G, 2*inter, K/2] FP4 (packed), w1_scales [G, 2*inter, K/32]
 *   w2_codes      [G, n_out, inter/2] FP4 (packed), w2_scales [G, n_out, inter/32]
 *   h             [rows, inter] bf16 (out), y [rows, n_out] bf16 (out)
 *   workspace     at least lmoe_workspace_bytes(shape, LMOE_CALL_GROUPED_GLU_MX) for rows = T*k,
 *                 inter = shape inter: the tile list and the FP8 copy of h with its scales
 * a_codes must be under 2 GiB (31-bit byte offsets). Codes 16-byte and scales 4-byte aligned.   */
lmoe_status lmoe_grouped_situ_glu_mx(const lmoe_shape* shape, int32_t n_groups, int32_t rows, int32_t K,
                                     int32_t inter, int32_t n_out, const void* a_codes, const void* a_scales,
                                     int32_t a_rows, const int32_t* a_row_index, const int32_t* group_offsets,
                                     const void* w1_codes, const void* w1_scales, const void* w2_codes,
                                     const void* w2_scales, void* h, void* y, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Kernel timing for measurement. When enabled, every kernel the library enqueues is bracketed by
 * HIP events on its stream. lmoe_profile_collect() synchronises those events and folds them into
 * per-kernel totals; lmoe_profile_get() reads the totals of kernel `name` (count of launches and
 * summed milliseconds). lmoe_profile_only(name) restricts the timing to the kernels named `name`
 * (NULL: every kernel again), so that a timed region carries only the events it needs; `name` is
 * copied. A measurement aid: with timing off (the default) a launch reads one atomic flag and no
 * other state; with timing on, the process-wide event lists are guarded by a lock, so calls from
 * several host threads stay safe (their launches are then timed together). */
void lmoe_profile_enable(int on);
void lmoe_profile_only(const char* name);
void lmoe_profile_reset(void);
lmoe_status lmoe_profile_collect(void);
int lmoe_profile_get(const char* name, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* LMOE_H */
