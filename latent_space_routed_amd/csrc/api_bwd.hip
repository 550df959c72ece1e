// C ABI of the backward pass: argument validation, workspace sizing and the kernels behind each call.
// The calls follow the forward in reverse ([vxz] 01-02, [slm] Latent-Space MoE): up-projection,
// combine + RMSNorm + routing weights, router, routed experts, un-permutation + down-projection,
// shared experts. Products that contract over an output dimension use transposed copies (weights:
// lmoe_bwd_transpose_weights; activations: transposed inside the calls, with every expert's rows
// padded to a multiple of 64 so that each expert's weight gradient is one K-range of a K-grouped
// GEMM).
#include "common.h"

using namespace lmoe;

namespace {

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
int esize(int dtype) { return dtype == LMOE_BF16 ? 2 : 4; }
lmoe_status hip_status(hipError_t e) { return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP; }

lmoe_status check_bwd_shape(const lmoe_shape* sh) {
  const lmoe_status st = validate_shape(sh);  // the forward's limits
  if (st != LMOE_OK) return st;
  // the combine backward keeps a latent row of at most 512 16-byte chunks per wave
  if ((int64_t)sh->d_latent * esize(sh->act_dtype) / 16 > 512) return LMOE_ERR_UNSUPPORTED;
  if ((int64_t)sh->T * sh->top_k + 64LL * sh->n_experts > 0x3fffffffLL) return LMOE_ERR_UNSUPPORTED;
  return LMOE_OK;
}

int64_t tpad(const lmoe_shape* sh) { return ((int64_t)(sh->T > 0 ? sh->T : 1) + 63) / 64 * 64; }
// columns of an expert-padded transposed activation: sum_e round_up(n_e, 64) <= T*k + 63 E
int64_t kpad(const lmoe_shape* sh) { return ((int64_t)sh->T * sh->top_k + 64LL * sh->n_experts + 63) / 64 * 64; }
int64_t shared_inner(const lmoe_shape* sh) { return (int64_t)sh->n_shared * sh->inter_shared; }

size_t ws_up(const lmoe_shape* sh) {
  return round_up((size_t)(sh->d_model + sh->d_latent + shared_inner(sh)) * tpad(sh) * esize(sh->act_dtype));
}
size_t ws_combine(const lmoe_shape* sh) {  // block partials of dgamma and their first fold
  const size_t blocks = (size_t)combine_bwd_blocks(sh->T);
  return round_up((blocks + (blocks + 63) / 64) * sh->d_latent * sizeof(float));
}
size_t ws_experts(const lmoe_shape* sh) {
  const size_t idx = 3 * round_up((size_t)(sh->n_experts + 1) * 4);
  const size_t rows = (size_t)(sh->d_latent + sh->inter + 2 * sh->inter + sh->d_latent);
  return idx + round_up(rows * kpad(sh) * esize(sh->act_dtype));
}
size_t ws_down(const lmoe_shape* sh) {
  return round_up((size_t)(sh->d_latent + sh->d_model) * tpad(sh) * esize(sh->act_dtype));
}
size_t ws_shared(const lmoe_shape* sh) {
  return round_up((size_t)(2 * shared_inner(sh) + sh->d_model) * tpad(sh) * esize(sh->act_dtype));
}

GemmArgs gargs(const lmoe_shape* sh) {
  GemmArgs a{};
  a.beta1 = sh->beta1;
  a.beta2 = sh->beta2;
  a.G = 1;
  return a;
}

GemmShape dense_shape(int64_t M, int64_t N) {
  return ceil_div(M, 256) * ceil_div(N, 256) >= 256 ? GemmShape::Big : GemmShape::Small;
}

// C[M, N] (out_dtype) = A[M, K] . B[N, K]^T, both K-contiguous; residual: C = acc + residual (f32).
hipError_t dense(const lmoe_shape* sh, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                 int out_dtype, int M, int N, int K, const float* residual, const char* tag, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  GemmArgs a = gargs(sh);
  a.A = A;
  a.lda = lda;
  a.a_kwrap = K;
  a.B = B;
  a.ldb = ldb;
  a.C = C;
  a.ldc = ldc;
  a.c_dtype = out_dtype;
  a.M = M;
  a.N = N;
  a.K = K;
  a.residual = residual;
  a.ldr = ldc;
  a.tag = tag;
  return launch_gemm(a, sh->act_dtype, residual ? Epi::AddF32 : Epi::Store, dense_shape(M, N), s);
}

// Transposed copy of a [rows, C] activation into [C, tpad] with zero columns past rows.
hipError_t transpose_act(const lmoe_shape* sh, const void* in, int64_t ld_in, int C, int rows, void* out,
                         hipStream_t s) {
  return launch_transpose_cols(in, ld_in, C, nullptr, nullptr, 0, rows, nullptr, out, tpad(sh), (int)tpad(sh),
                               esize(sh->act_dtype), s);
}

}  // namespace

namespace lmoe {
size_t bwd_workspace_bytes(const lmoe_shape* sh, int which) {
  if (check_bwd_shape(sh) != LMOE_OK) return 0;
  switch (which) {
    case LMOE_CALL_BWD_UP: return ws_up(sh);
    case LMOE_CALL_BWD_COMBINE_NORM: return ws_combine(sh);
    case LMOE_CALL_BWD_EXPERTS: return ws_experts(sh);
    case LMOE_CALL_BWD_DOWN: return ws_down(sh);
    case LMOE_CALL_BWD_SHARED: return ws_shared(sh);
  }
  return 0;
}
}  // namespace lmoe

extern "C" {

lmoe_status lmoe_bwd_transpose_weights(const lmoe_shape* sh, const void* w_up, const void* w2s_packed,
                                       const void* w1s_packed, const void* w_down, void* w_up_t, void* w2s_t,
                                       void* w1s_t, void* w_down_t, void* stream) {
  lmoe_status st = check_bwd_shape(sh);
  if (st != LMOE_OK) return st;
  if (!aligned16(w_up) || !aligned16(w_down) || !aligned16(w_up_t) || !aligned16(w_down_t))
    return LMOE_ERR_INVALID_ARGUMENT;
  const int64_t Ss = shared_inner(sh);
  const bool shared = w2s_packed || w1s_packed;
  if (shared && (Ss < 64 || !aligned16(w2s_packed) || !aligned16(w1s_packed) || !aligned16(w2s_t) ||
                 !aligned16(w1s_t)))
    return LMOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = sh->d_model, L = sh->d_latent, esz = esize(sh->act_dtype);
  st = hip_status(launch_transpose(w_up, w_up_t, 1, D, L, 0, 0, esz, s));
  if (st == LMOE_OK) st = hip_status(launch_transpose(w_down, w_down_t, 1, L, D, 0, 0, esz, s));
  if (st == LMOE_OK && shared) st = hip_status(launch_transpose(w2s_packed, w2s_t, 1, D, (int)Ss, 0, 0, esz, s));
  if (st == LMOE_OK && shared) st = hip_status(launch_transpose(w1s_packed, w1s_t, 1, (int)(2 * Ss), D, 0, 0, esz, s));
  return st;
}

lmoe_status lmoe_bwd_up(const lmoe_shape* sh, const void* dout, const void* n, const void* h_shared,
                        const void* w_up_t, const void* w2s_t, void* dn, void* dh_shared, float* dw_up,
                        float* dw2_shared, void* workspace, size_t workspace_bytes, void* stream) {
  lmoe_status st = check_bwd_shape(sh);
  if (st != LMOE_OK) return st;
  const int64_t Ss = shared_inner(sh);
  const bool shared = h_shared != nullptr;
  if (!aligned16(dout) || !aligned16(n) || !aligned16(w_up_t) || !aligned16(dn) || !aligned16(dw_up))
    return LMOE_ERR_INVALID_ARGUMENT;
  if (shared && (Ss < 64 || !aligned16(h_shared) || !aligned16(w2s_t) || !aligned16(dh_shared) ||
                 !aligned16(dw2_shared)))
    return LMOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace) || workspace_bytes < ws_up(sh)) return LMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = sh->T, D = sh->d_model, L = sh->d_latent, dt = sh->act_dtype, esz = esize(dt);
  const int64_t Tp = tpad(sh);
  char* ws = static_cast<char*>(workspace);
  void* dout_t = ws;                               // [D, Tp]
  void* n_t = ws + (size_t)D * Tp * esz;           // [L, Tp]
  void* hs_t = ws + (size_t)(D + L) * Tp * esz;    // [Ss, Tp]
  // dn = dout . w_up, dh_s = dout . w2s (through the transposed weights)
  st = hip_status(dense(sh, dout, D, w_up_t, D, dn, L, dt, T, L, D, nullptr, "bwd_gemm_dn", s));
  if (st == LMOE_OK && shared)
    st = hip_status(dense(sh, dout, D, w2s_t, D, dh_shared, Ss, dt, T, (int)Ss, D, nullptr, "bwd_gemm_dn", s));
  // dW_up = dout^T n, dW2s = dout^T h_s (contraction over tokens)
  if (st == LMOE_OK) st = hip_status(transpose_act(sh, dout, D, D, T, dout_t, s));
  if (st == LMOE_OK) st = hip_status(transpose_act(sh, n, L, L, T, n_t, s));
  if (st == LMOE_OK)
    st = hip_status(dense(sh, dout_t, Tp, n_t, Tp, dw_up, L, LMOE_F32, D, L, (int)Tp, nullptr, "bwd_gemm_dw", s));
  if (st == LMOE_OK && shared) st = hip_status(transpose_act(sh, h_shared, Ss, (int)Ss, T, hs_t, s));
  if (st == LMOE_OK && shared)
    st = hip_status(
        dense(sh, dout_t, Tp, hs_t, Tp, dw2_shared, Ss, LMOE_F32, D, (int)Ss, (int)Tp, nullptr, "bwd_gemm_dw", s));
  return st;
}

lmoe_status lmoe_bwd_combine_norm(const lmoe_shape* sh, const void* dn, const void* y_perm,
                                  const int32_t* slot_of_pair, const int32_t* topk_idx, const float* scores,
                                  const float* topk_w, const float* gamma, void* dy_perm, float* dlogit,
                                  float* dlogit_sorted, float* dgamma, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  lmoe_status st = check_bwd_shape(sh);
  if (st != LMOE_OK) return st;
  if (!aligned16(dn) || !aligned16(y_perm) || !aligned4(slot_of_pair) || !aligned4(topk_idx) || !aligned4(scores) ||
      !aligned4(topk_w) || (gamma && !aligned4(gamma)) || !aligned16(dy_perm) || !aligned4(dlogit) ||
      !aligned4(dlogit_sorted) || !aligned4(dgamma))
    return LMOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace) || workspace_bytes < ws_combine(sh)) return LMOE_ERR_WORKSPACE;
  return hip_status(launch_combine_bwd(dn, y_perm, slot_of_pair, topk_idx, scores, topk_w, gamma, sh->T, sh->top_k,
                                       sh->n_experts, sh->d_latent, sh->rms_eps, sh->act_dtype, dy_perm, dlogit,
                                       dlogit_sorted, static_cast<float*>(workspace), dgamma,
                                       static_cast<hipStream_t>(stream)));
}

lmoe_status lmoe_bwd_router(const lmoe_shape* sh, const void* x, const float* w_router, const float* dlogit,
                            const float* dlogit_sorted, const int32_t* topk_idx, const int32_t* expert_offsets,
                            const int32_t* sorted_token, float* dw_router, float* dx, void* stream) {
  lmoe_status st = check_bwd_shape(sh);
  if (st != LMOE_OK) return st;
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(dlogit) || !aligned4(dlogit_sorted) ||
      !aligned4(topk_idx) || !aligned4(expert_offsets) || !aligned4(sorted_token) || !aligned16(dw_router) ||
      !aligned16(dx))
    return LMOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_router_bwd(x, w_router, dlogit, dlogit_sorted, topk_idx, expert_offsets, sorted_token,
                                      sh->T, sh->d_model, sh->n_experts, sh->top_k, sh->act_dtype, dw_router, dx,
                                      static_cast<hipStream_t>(stream)));
}

lmoe_status lmoe_bwd_experts(const lmoe_shape* sh, const void* x_lat, const int32_t* sorted_token,
                             const int32_t* expert_offsets, const void* w1, const void* w2, const void* h,
                             const void* dy_perm, void* dh, void* dgu, void* dx_perm, float* dw1, float* dw2,
                             void* workspace, size_t workspace_bytes, void* stream) {
  lmoe_status st = check_bwd_shape(sh);
  if (st != LMOE_OK) return st;
  if (!aligned16(x_lat) || !aligned4(sorted_token) || !aligned4(expert_offsets) || !aligned16(w1) ||
      !aligned16(w2) || !aligned16(h) || !aligned16(dy_perm) || !aligned16(dh) ||
      !aligned16(dgu) || !aligned16(dx_perm) || !aligned16(dw1) || !aligned16(dw2))
    return LMOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace) || workspace_bytes < ws_experts(sh)) return LMOE_ERR_WORKSPACE;
  if ((int64_t)sh->T * sh->d_latent * esize(sh->act_dtype) > 0x7fff0000LL) return LMOE_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = sh->T, L = sh->d_latent, E = sh->n_experts, I = sh->inter, dt = sh->act_dtype, esz = esize(dt);
  const int rows = T * sh->top_k;
  const int64_t Kp = kpad(sh);
  char* ws = static_cast<char*>(workspace);
  const size_t ia = round_up((size_t)(E + 1) * 4);
  int32_t* mts = reinterpret_cast<int32_t*>(ws);                // m-tile prefix of the grouped GEMMs
  int32_t* ptile = reinterpret_cast<int32_t*>(ws + ia);         // 64-row tile prefix (padded K ranges)
  int32_t* mts_kn = reinterpret_cast<int32_t*>(ws + 2 * ia);    // m-tile prefix of the [K, N]-B GEMMs
  char* tb = ws + 3 * ia;
  void* dy_t = tb;                                       // [L, Kp]
  void* h_t = tb + (size_t)L * Kp * esz;                 // [I, Kp]
  void* dgu_t = tb + (size_t)(L + I) * Kp * esz;         // [2I, Kp]
  void* xp_t = tb + (size_t)(L + 3 * I) * Kp * esz;      // [L, Kp]
  // with no rows every K-range is empty and the K-grouped GEMMs write zero gradients
  const GemmShape gshape = (int64_t)rows >= (int64_t)E * 64 ? GemmShape::Big : GemmShape::Small;
  // The products that read W2_e and W1_e in place as [K, N] run on the 256-row DMA pipeline for bf16
  // only; f32 takes 128-row register tiles, and the m-tile numbering must follow the tile launched.
  const GemmShape kn_shape = dt == LMOE_BF16 ? gshape : GemmShape::Small;
  st = hip_status(launch_mtile_prefix(expert_offsets, E, gemm_block_m(gshape), mts, s));
  if (st == LMOE_OK) st = hip_status(launch_mtile_prefix(expert_offsets, E, 64, ptile, s));
  if (st == LMOE_OK && kn_shape != gshape)
    st = hip_status(launch_mtile_prefix(expert_offsets, E, gemm_block_m(kn_shape), mts_kn, s));
  if (st != LMOE_OK) return st;
  const int32_t* kn_mts = kn_shape != gshape ? mts_kn : mts;
  auto grouped = [&](const void* A, int64_t lda, const void* B, int64_t ldb, int64_t bstride, void* C, int64_t ldc,
                     int N, int K, const char* tag) {
    GemmArgs a = gargs(sh);
    a.A = A;
    a.lda = lda;
    a.a_kwrap = K;
    a.B = B;
    a.ldb = ldb;
    a.b_gstride = bstride;
    a.C = C;
    a.ldc = ldc;
    a.c_dtype = dt;
    a.goff = expert_offsets;
    a.mtile_start = mts;
    a.G = E;
    a.M = rows;
    a.N = N;
    a.K = K;
    a.tag = tag;
    return a;
  };
  auto kgrouped = [&](const void* A, const void* B, float* C, int M, int N, const char* tag) {
    GemmArgs a = gargs(sh);
    a.A = A;
    a.lda = Kp;
    a.a_kwrap = (int)Kp;
    a.B = B;
    a.ldb = Kp;
    a.C = C;
    a.ldc = N;
    a.c_dtype = LMOE_F32;
    a.koff = ptile;
    a.koff_scale = 64;
    a.c_gstride = (int64_t)M * N;
    a.G = E;
    a.M = M;
    a.N = N;
    a.K = 0;
    a.tag = tag;
    return launch_gemm(a, dt, Epi::Store, (int64_t)M * N >= 256 * 256 ? GemmShape::Big : GemmShape::Small, s);
  };
  // dh = dy . W2_e, W2_e read as [K = L, N = I]
  if (rows > 0) {
    GemmArgs a = grouped(dy_perm, L, w2, I, (int64_t)L * I, dh, I, I, L, "bwd_gemm_dh");
    a.b_kn = true;
    a.mtile_start = kn_mts;
    st = hip_status(launch_gemm(a, dt, Epi::Store, kn_shape, s));
  }
  // dW2_e = dy_e^T h_e
  if (st == LMOE_OK)
    st = hip_status(launch_transpose_cols(dy_perm, L, L, expert_offsets, ptile, E, rows, nullptr, dy_t, Kp, (int)Kp,
                                          esz, s));
  if (st == LMOE_OK)
    st = hip_status(
        launch_transpose_cols(h, I, I, expert_offsets, ptile, E, rows, nullptr, h_t, Kp, (int)Kp, esz, s));
  if (st == LMOE_OK) st = hip_status(kgrouped(dy_t, h_t, dw2, L, I, "bwd_gemm_dw_experts"));
  // d[g | u]: the gate/up projections recomputed with the SiTU-GLU derivative in the epilogue
  if (st == LMOE_OK && rows > 0) {
    GemmArgs a = grouped(x_lat, L, w1, L, (int64_t)2 * I * L, dgu, 2 * I, I, L, "bwd_gemm_dgu");
    a.a_rows = sorted_token;
    a.a_nrows = T;
    a.glu_up_off = I;
    a.aux = dh;
    a.ld_aux = I;
    st = hip_status(launch_gemm(a, dt, Epi::GluBwd, gshape, s));
  }
  // dx_perm = d[g | u] . W1_e, W1_e read as [K = 2I, N = L]
  if (st == LMOE_OK && rows > 0) {
    GemmArgs a = grouped(dgu, 2 * I, w1, L, (int64_t)2 * I * L, dx_perm, L, L, 2 * I, "bwd_gemm_dx_experts");
    a.b_kn = true;
    a.mtile_start = kn_mts;
    st = hip_status(launch_gemm(a, dt, Epi::Store, kn_shape, s));
  }
  // dW1_e = d[g | u]_e^T x_perm_e (x_perm gathered from x_lat through sorted_token)
  if (st == LMOE_OK)
    st = hip_status(launch_transpose_cols(dgu, 2 * I, 2 * I, expert_offsets, ptile, E, rows, nullptr, dgu_t, Kp,
                                          (int)Kp, esz, s));
  if (st == LMOE_OK)
    st = hip_status(launch_transpose_cols(x_lat, L, L, expert_offsets, ptile, E, rows, sorted_token, xp_t, Kp,
                                          (int)Kp, esz, s));
  if (st == LMOE_OK) st = hip_status(kgrouped(dgu_t, xp_t, dw1, 2 * I, L, "bwd_gemm_dw_experts"));
  return st;
}

lmoe_status lmoe_bwd_down(const lmoe_shape* sh, const void* x, const void* dx_perm, const int32_t* slot_of_pair,
                          const void* w_down_t, void* dx_lat, float* dw_down, float* dx, void* workspace,
                          size_t workspace_bytes, void* stream) {
  lmoe_status st = check_bwd_shape(sh);
  if (st != LMOE_OK) return st;
  if (!aligned16(x) || !aligned16(dx_perm) || !aligned4(slot_of_pair) || !aligned16(w_down_t) || !aligned16(dx_lat) ||
      !aligned16(dw_down) || !aligned16(dx))
    return LMOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace) || workspace_bytes < ws_down(sh)) return LMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = sh->T, D = sh->d_model, L = sh->d_latent, dt = sh->act_dtype, esz = esize(dt);
  const int64_t Tp = tpad(sh);
  char* ws = static_cast<char*>(workspace);
  void* dxl_t = ws;                            // [L, Tp]
  void* x_t = ws + (size_t)L * Tp * esz;       // [D, Tp]
  if (T > 0) st = hip_status(launch_unpermute(dx_perm, slot_of_pair, T, sh->top_k, L, dt, dx_lat, s));
  if (st == LMOE_OK) st = hip_status(transpose_act(sh, dx_lat, L, L, T, dxl_t, s));
  if (st == LMOE_OK) st = hip_status(transpose_act(sh, x, D, D, T, x_t, s));
  if (st == LMOE_OK)
    st = hip_status(dense(sh, dxl_t, Tp, x_t, Tp, dw_down, D, LMOE_F32, L, D, (int)Tp, nullptr, "bwd_gemm_dw", s));
  if (st == LMOE_OK && T > 0)
    st = hip_status(dense(sh, dx_lat, L, w_down_t, L, dx, D, LMOE_F32, T, D, L, dx, "bwd_gemm_dx", s));
  return st;
}

lmoe_status lmoe_bwd_shared(const lmoe_shape* sh, const void* x, const void* w1s_packed, const void* w1s_t,
                            const void* dh_shared, void* dgu_shared, float* dw1s_packed, float* dx, void* workspace,
                            size_t workspace_bytes, void* stream) {
  lmoe_status st = check_bwd_shape(sh);
  if (st != LMOE_OK) return st;
  const int64_t Ss = shared_inner(sh);
  if (Ss < 64) return LMOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w1s_packed) || !aligned16(w1s_t) || !aligned16(dh_shared) ||
      !aligned16(dgu_shared) || !aligned16(dw1s_packed) || !aligned16(dx))
    return LMOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace) || workspace_bytes < ws_shared(sh)) return LMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = sh->T, D = sh->d_model, dt = sh->act_dtype, esz = esize(dt);
  const int64_t Tp = tpad(sh);
  char* ws = static_cast<char*>(workspace);
  void* dgu_t = ws;                                 // [2 Ss, Tp]
  void* x_t = ws + (size_t)2 * Ss * Tp * esz;       // [D, Tp]
  if (T > 0) {  // d[g_s | u_s] from the recomputed shared projections
    GemmArgs a = gargs(sh);
    a.A = x;
    a.lda = D;
    a.a_kwrap = D;
    a.B = w1s_packed;
    a.ldb = D;
    a.C = dgu_shared;
    a.ldc = 2 * Ss;
    a.c_dtype = dt;
    a.M = T;
    a.N = (int)Ss;
    a.K = D;
    a.glu_up_off = (int)Ss;
    a.aux = dh_shared;
    a.ld_aux = Ss;
    a.tag = "bwd_gemm_dgu";
    st = hip_status(launch_gemm(a, dt, Epi::GluBwd, dense_shape(T, 2 * Ss), s));
  }
  if (st == LMOE_OK) st = hip_status(transpose_act(sh, dgu_shared, 2 * Ss, (int)(2 * Ss), T, dgu_t, s));
  if (st == LMOE_OK) st = hip_status(transpose_act(sh, x, D, D, T, x_t, s));
  if (st == LMOE_OK)
    st = hip_status(
        dense(sh, dgu_t, Tp, x_t, Tp, dw1s_packed, D, LMOE_F32, (int)(2 * Ss), D, (int)Tp, nullptr, "bwd_gemm_dw", s));
  if (st == LMOE_OK && T > 0)
    st = hip_status(dense(sh, dgu_shared, 2 * Ss, w1s_t, 2 * Ss, dx, D, LMOE_F32, T, D, (int)(2 * Ss), dx,
                          "bwd_gemm_dx", s));
  return st;
}

}  // extern "C"
