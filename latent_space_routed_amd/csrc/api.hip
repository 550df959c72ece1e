// C ABI of the library: argument validation (before anything is enqueued), workspace sizing and the
// composition of kernels behind each call.
#include <mutex>

#include "common.h"

using namespace lmoe;

namespace {

constexpr int kMaxExperts = 2048;  // top-k keeps 32 scores per lane; the permutation keeps 4 x E masks in LDS
constexpr int kMaxTopK = 64;
constexpr int kMaxBins = 32768;
constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int esize(int dtype) { return dtype == LMOE_BF16 ? 2 : 4; }

lmoe_status check_shape(const lmoe_shape* sh) {
  if (!sh) return LMOE_ERR_INVALID_ARGUMENT;
  if (sh->act_dtype != LMOE_F32 && sh->act_dtype != LMOE_BF16) return LMOE_ERR_INVALID_ARGUMENT;
  if (sh->T < 0 || sh->d_model <= 0 || sh->d_latent <= 0 || sh->n_experts <= 0 || sh->top_k <= 0 ||
      sh->inter <= 0 || sh->n_shared < 0 || sh->inter_shared < 0 || sh->n_bins <= 0)
    return LMOE_ERR_INVALID_ARGUMENT;
  if (sh->top_k >= sh->n_experts) return LMOE_ERR_INVALID_ARGUMENT;  // the (k+1)-th score must exist
  if (!(sh->beta1 > 0.0f) || !(sh->beta2 > 0.0f) || !(sh->rms_eps >= 0.0f)) return LMOE_ERR_INVALID_ARGUMENT;
  if (sh->n_experts > kMaxExperts || sh->top_k > kMaxTopK || sh->n_bins < 2 || sh->n_bins > kMaxBins)
    return LMOE_ERR_UNSUPPORTED;
  if (sh->d_model % 64 || sh->d_latent % 64 || sh->inter % 64 || sh->inter_shared % 64) return LMOE_ERR_UNSUPPORTED;
  if ((int64_t)sh->d_latent * esize(sh->act_dtype) / 16 > 1024) return LMOE_ERR_UNSUPPORTED;  // combine row in registers
  if ((int64_t)sh->T * sh->top_k > 0x7fffffffLL) return LMOE_ERR_UNSUPPORTED;
  return LMOE_OK;
}

lmoe_status hip_status(hipError_t e) { return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP; }

GemmArgs gemm_args() {
  GemmArgs a{};
  a.beta1 = 4.0f;
  a.beta2 = 25.0f;
  a.G = 1;
  return a;
}

// Tile shape: 256x256 blocks when they still give every CU work, else 128x128.
GemmShape dense_shape(int64_t M, int64_t N_tile_cols_big) {
  const int64_t tiles = ceil_div(M, 256) * N_tile_cols_big;
  return tiles >= 256 ? GemmShape::Big : GemmShape::Small;
}

size_t route_ws(const lmoe_shape* sh) {
  return sh->act_dtype == LMOE_BF16 ? round_up((size_t)3 * sh->n_experts * sh->d_model * 2) : 0;
}
size_t permute_ws(const lmoe_shape* sh) {
  return round_up((size_t)ceil_div(sh->T > 0 ? sh->T : 1, kPermChunk) * sh->n_experts * 4);
}
size_t glu_ws(int groups) { return round_up((size_t)(groups + 1) * 4); }
// tile list, then the FP8 codes and the scales of h
size_t mx_glu_ws(int groups, int64_t rows, int inter) {
  return glu_ws(groups) + round_up((size_t)rows * inter) + round_up((size_t)rows * (inter / 32));
}

// Split-K plans of the dense GEMMs behind each call (no split once the batch fills the chip).
SplitPlan router_plan(const lmoe_shape* sh) {
  const int D = sh->d_model, K = sh->act_dtype == LMOE_BF16 ? 3 * D : D;
  const SplitPlan small = plan_split_k(sh->T, sh->n_experts, K, 0, D, esize(sh->act_dtype));
  if (small.splits > 1) return small;
  return plan_split_k_big(sh->T, sh->n_experts, K, 0, esize(sh->act_dtype));
}
SplitPlan down_plan(const lmoe_shape* sh) {
  return plan_split_k(sh->T, sh->d_latent, sh->d_model, 0, sh->d_model, esize(sh->act_dtype));
}
SplitPlan up_plan(const lmoe_shape* sh, bool shared_folded) {
  const int Ss = sh->n_shared * sh->inter_shared;
  return plan_split_k(sh->T, sh->d_model, sh->d_latent, shared_folded ? Ss : 0, sh->d_latent, esize(sh->act_dtype));
}
size_t split_bytes(const SplitPlan& sp, int64_t M, int64_t n_cols) { return round_up(split_k_bytes(sp, M, n_cols)); }
size_t shared_split_bytes(const lmoe_shape* sh) {
  const int Ss = sh->n_shared * sh->inter_shared;
  if (Ss < 64) return 0;
  const int esz = esize(sh->act_dtype);
  const size_t g1 = split_bytes(plan_split_k(sh->T, 2 * (int64_t)Ss, sh->d_model, 0, sh->d_model, esz), sh->T, 2 * (int64_t)Ss);
  const size_t g2 = split_bytes(plan_split_k(sh->T, sh->d_model, Ss, 0, Ss, esz), sh->T, sh->d_model);
  return g1 > g2 ? g1 : g2;
}
size_t combine_split_bytes(const lmoe_shape* sh) {
  const size_t a = split_bytes(up_plan(sh, false), sh->T, sh->d_model);
  const size_t b = sh->n_shared * sh->inter_shared >= 64 ? split_bytes(up_plan(sh, true), sh->T, sh->d_model) : 0;
  return a > b ? a : b;
}

// The partial-product region after the call's own workspace (at offset `base`), or nullptr when the
// plan has no split or the caller's workspace does not hold it (the GEMM then runs unsplit).
float* split_region(const SplitPlan& sp, int64_t M, int64_t n_cols, void* workspace, size_t workspace_bytes,
                    size_t base) {
  if (sp.splits < 2 || !workspace || !aligned16(workspace)) return nullptr;
  if (workspace_bytes < base + split_k_bytes(sp, M, n_cols)) return nullptr;
  return reinterpret_cast<float*>(static_cast<char*>(workspace) + base);
}

hipError_t run_gemm(const GemmArgs& a, int dtype, Epi epi, GemmShape shape, const SplitPlan& sp, float* part,
                    hipStream_t s) {
  return part ? launch_gemm_split(a, dtype, epi, sp, part, s) : launch_gemm(a, dtype, epi, shape, s);
}

}  // namespace

lmoe_status lmoe::validate_shape(const lmoe_shape* sh) { return check_shape(sh); }

extern "C" {

const char* lmoe_status_string(lmoe_status s) {
  switch (s) {
    case LMOE_OK: return "LMOE_OK";
    case LMOE_ERR_INVALID_ARGUMENT: return "LMOE_ERR_INVALID_ARGUMENT";
    case LMOE_ERR_UNSUPPORTED: return "LMOE_ERR_UNSUPPORTED";
    case LMOE_ERR_WORKSPACE: return "LMOE_ERR_WORKSPACE";
    case LMOE_ERR_HIP: return "LMOE_ERR_HIP";
  }
  return "LMOE_UNKNOWN_STATUS";
}

size_t lmoe_workspace_bytes(const lmoe_shape* sh, int which) {
  if (check_shape(sh) != LMOE_OK) return 0;
  switch (which) {
    case LMOE_CALL_ROUTE: return route_ws(sh) + split_bytes(router_plan(sh), sh->T, sh->n_experts);
    case LMOE_CALL_PERMUTE: return permute_ws(sh) + split_bytes(down_plan(sh), sh->T, sh->d_latent);
    case LMOE_CALL_GROUPED_GLU: return glu_ws(sh->n_experts > 1 ? sh->n_experts : 1) + shared_split_bytes(sh);
    case LMOE_CALL_COMBINE_NORM_UP: return combine_split_bytes(sh);
    case LMOE_CALL_GROUPED_GLU_MX:
      return mx_glu_ws(sh->n_experts > 1 ? sh->n_experts : 1, (int64_t)sh->T * sh->top_k, sh->inter);
    default: return bwd_workspace_bytes(sh, which);
  }
}

lmoe_status lmoe_split_router(const lmoe_shape* sh, const float* w_router, void* w_router_split, void* stream) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if (sh->act_dtype != LMOE_BF16) return LMOE_ERR_UNSUPPORTED;
  if (!aligned16(w_router) || !aligned16(w_router_split)) return LMOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_split3(w_router, static_cast<uint16_t*>(w_router_split), sh->n_experts, sh->d_model,
                                  static_cast<hipStream_t>(stream)));
}

lmoe_status lmoe_route(const lmoe_shape* sh, const void* x, const float* w_router, const void* w_router_split,
                       const float* bias, const float* logit_offset, float* scores, int32_t* topk_idx, float* topk_w,
                       float* thresh, void* workspace, size_t workspace_bytes, void* stream) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if (sh->T == 0) return LMOE_OK;
  const bool presplit = sh->act_dtype == LMOE_BF16 && w_router_split != nullptr;
  if (!aligned16(x) || !(presplit ? aligned16(w_router_split) : aligned16(w_router)) || !aligned4(bias) ||
      !aligned16(scores) || !aligned4(topk_idx) || !aligned4(topk_w) || !aligned4(thresh) ||
      (logit_offset && !aligned4(logit_offset)))
    return LMOE_ERR_INVALID_ARGUMENT;
  if (sh->act_dtype != LMOE_BF16 && w_router_split) return LMOE_ERR_INVALID_ARGUMENT;
  const size_t need = presplit ? 0 : route_ws(sh);
  if (need && (!workspace || workspace_bytes < need || !aligned16(workspace))) return LMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = sh->T, D = sh->d_model, E = sh->n_experts;
  GemmArgs a = gemm_args();
  a.A = x;
  a.lda = D;
  a.a_kwrap = D;
  a.C = scores;
  a.ldc = E;
  a.c_dtype = LMOE_F32;
  a.M = T;
  a.N = E;
  a.col_bias = logit_offset;
  a.tag = "gemm_router";
  if (sh->act_dtype == LMOE_BF16) {
    const uint16_t* wsplit = static_cast<const uint16_t*>(w_router_split);
    if (!presplit) {  // the three-part split of this call's weights, in the workspace
      uint16_t* tmp = static_cast<uint16_t*>(workspace);
      st = hip_status(launch_split3(w_router, tmp, E, D, s));
      if (st != LMOE_OK) return st;
      wsplit = tmp;
    }
    a.B = wsplit;
    a.ldb = 3 * (int64_t)D;
    a.K = 3 * D;
  } else {
    a.B = w_router;
    a.ldb = D;
    a.K = D;
  }
  const SplitPlan sp = router_plan(sh);
  float* part = split_region(sp, T, E, workspace, workspace_bytes, need);
  if (part && sp.big) {  // a few halves of K on the DMA pipeline: the top-k sums them itself
    st = hip_status(launch_gemm_split(a, sh->act_dtype, Epi::Sigmoid, sp, part, s, false));
    if (st != LMOE_OK) return st;
    return hip_status(launch_topk_partials(part, sp.splits, logit_offset, scores, bias, T, E, sh->top_k, topk_idx,
                                           topk_w, thresh, s));
  }
  st = hip_status(run_gemm(a, sh->act_dtype, Epi::Sigmoid, dense_shape(T, ceil_div(E, 256)), sp, part, s));
  if (st != LMOE_OK) return st;
  return hip_status(launch_topk(scores, bias, T, E, sh->top_k, topk_idx, topk_w, thresh, s));
}

lmoe_status lmoe_qb_histogram(const lmoe_shape* sh, const float* scores, const float* bias, const int32_t* topk_idx,
                              const float* thresh, uint32_t* hist, void* stream) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if (sh->T == 0) return LMOE_OK;
  if (!aligned4(scores) || !aligned4(bias) || !aligned4(topk_idx) || !aligned4(thresh) || !aligned4(hist))
    return LMOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_qb_hist(scores, bias, topk_idx, thresh, sh->T, sh->n_experts, sh->top_k, sh->n_bins, hist,
                                   static_cast<hipStream_t>(stream)));
}

lmoe_status lmoe_qb_update(const lmoe_shape* sh, uint32_t* hist, int64_t n_acc, float* bias, void* stream) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if (!aligned4(hist) || !aligned4(bias)) return LMOE_ERR_INVALID_ARGUMENT;
  if (n_acc > (int64_t(1) << 52) / (sh->n_experts > 0 ? sh->n_experts : 1)) return LMOE_ERR_UNSUPPORTED;
  return hip_status(launch_qb_update(hist, sh->n_experts, sh->top_k, sh->n_bins, n_acc, bias,
                                     static_cast<hipStream_t>(stream)));
}

lmoe_status lmoe_permute(const lmoe_shape* sh, const void* x, const void* w_down, const int32_t* topk_idx,
                         void* x_lat, int32_t* expert_offsets, int32_t* sorted_token, int32_t* slot_of_pair,
                         void* x_perm, void* workspace, size_t workspace_bytes, void* stream) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if (sh->T == 0) {
    // no tokens: every expert is empty (a fill kernel, not a memset node, so the call can be captured)
    if (!aligned4(expert_offsets)) return LMOE_ERR_INVALID_ARGUMENT;
    return hip_status(launch_fill_i32(expert_offsets, sh->n_experts + 1, 0, static_cast<hipStream_t>(stream)));
  }
  if (!aligned16(x) || !aligned16(w_down) || !aligned4(topk_idx) || !aligned16(x_lat) || !aligned4(expert_offsets) ||
      !aligned4(sorted_token) || !aligned4(slot_of_pair) || (x_perm && !aligned16(x_perm)))
    return LMOE_ERR_INVALID_ARGUMENT;
  const size_t need = permute_ws(sh);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return LMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = sh->T, D = sh->d_model, L = sh->d_latent, E = sh->n_experts, k = sh->top_k;
  GemmArgs a = gemm_args();
  a.A = x;
  a.lda = D;
  a.a_kwrap = D;
  a.B = w_down;
  a.ldb = D;
  a.C = x_lat;
  a.ldc = L;
  a.c_dtype = sh->act_dtype;
  a.M = T;
  a.N = L;
  a.K = D;
  a.tag = "gemm_down";
  const SplitPlan sp = down_plan(sh);
  float* part = split_region(sp, T, L, workspace, workspace_bytes, need);
  st = hip_status(run_gemm(a, sh->act_dtype, Epi::Store, dense_shape(T, ceil_div(L, 256)), sp, part, s));
  if (st != LMOE_OK) return st;
  st = hip_status(launch_permute(topk_idx, T, E, k, expert_offsets, sorted_token, slot_of_pair,
                                 static_cast<int32_t*>(workspace), s));
  if (st != LMOE_OK) return st;
  if (!x_perm) return LMOE_OK;  // the routed GEMM gathers latent rows itself
  return hip_status(launch_gather_rows(x_lat, slot_of_pair, T, k, (int64_t)L * esize(sh->act_dtype), x_perm, s));
}

}  // extern "C"

namespace {

// Validation of lmoe_grouped_situ_glu's arguments other than the workspace.
lmoe_status check_grouped(const lmoe_shape* sh, int32_t G, int32_t rows, int32_t K, int32_t inter, int32_t n_out,
                          const void* a_in, int32_t a_rows, const int32_t* a_row_index,
                          const int32_t* group_offsets, const void* w1, const void* w2, void* h, void* y,
                          int32_t y_dtype) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if (G < 1 || rows < 0 || a_rows < 0 || K <= 0 || inter <= 0 || (w2 && n_out <= 0)) return LMOE_ERR_INVALID_ARGUMENT;
  if (w2 && y_dtype != LMOE_F32 && y_dtype != sh->act_dtype) return LMOE_ERR_INVALID_ARGUMENT;
  if (K % 64 || inter % 64) return LMOE_ERR_UNSUPPORTED;
  if (!group_offsets && G != 1) return LMOE_ERR_INVALID_ARGUMENT;
  if (!a_row_index && a_rows != rows) return LMOE_ERR_INVALID_ARGUMENT;
  if (a_row_index && (int64_t)a_rows * K * esize(sh->act_dtype) > 0x7fff0000LL)
    return LMOE_ERR_UNSUPPORTED;  // a gathered A is addressed with 31-bit byte offsets
  if (rows == 0) return LMOE_OK;
  if (!aligned16(a_in) || !aligned16(w1) || !aligned16(h) || (a_row_index && !aligned4(a_row_index)) ||
      (group_offsets && !aligned4(group_offsets)) || (w2 && (!aligned16(w2) || !aligned16(y))))
    return LMOE_ERR_INVALID_ARGUMENT;
  return LMOE_OK;
}

// The grouped GEMMs with the m-tile list in `mts` (G + 1 ints, grouped calls only) and optional
// split-K partials (dense calls: `split_ws`, nullptr = run unsplit).
lmoe_status grouped_glu(const lmoe_shape* sh, int32_t G, int32_t rows, int32_t K, int32_t inter, int32_t n_out,
                        const void* a_in, int32_t a_rows, const int32_t* a_row_index, const int32_t* group_offsets,
                        const void* w1, const void* w2, void* h, void* y, int32_t y_dtype, int32_t* mts_buf,
                        void* split_ws, size_t split_ws_bytes, hipStream_t s) {
  lmoe_status st = LMOE_OK;
  const int dt = sh->act_dtype;
  GemmShape shape;
  if (group_offsets) {
    // 256-row tiles when the groups average 64 rows or more, and for bf16 groups whose weights are
    // wide enough to stream (K >= 1024, inter >= 256) whatever their rows: the persistent pipeline
    // DMAs the weight slices straight into LDS, and with a few rows per expert (decode: 64 tokens
    // over 896 experts) the GEMMs are that stream (measured at K3 decode: GEMM1 0.76 -> 0.71 ms,
    // GEMM2 0.42 -> 0.38 ms against 128-row tiles on the register pipeline).
    const bool stream_w = dt == LMOE_BF16 && K >= 1024 && inter >= 256;
    shape = ((int64_t)rows >= (int64_t)G * 64 || stream_w) ? GemmShape::Big : GemmShape::Small;
    st = hip_status(launch_mtile_prefix(group_offsets, G, gemm_block_m(shape), mts_buf, s));
    if (st != LMOE_OK) return st;
  } else {
    shape = dense_shape(rows, ceil_div(inter, 128));
  }
  const int32_t* mts = group_offsets ? mts_buf : nullptr;

  GemmArgs g1 = gemm_args();
  g1.A = a_in;
  g1.lda = K;
  g1.a_kwrap = K;
  g1.a_rows = a_row_index;
  g1.a_nrows = a_rows;
  g1.B = w1;
  g1.ldb = K;
  g1.b_gstride = (int64_t)2 * inter * K;
  g1.C = h;
  g1.ldc = inter;
  g1.c_dtype = dt;
  g1.goff = group_offsets;
  g1.mtile_start = mts;
  g1.G = G;
  g1.M = rows;
  g1.N = inter;
  g1.K = K;
  g1.glu_up_off = inter;
  g1.beta1 = sh->beta1;
  g1.beta2 = sh->beta2;
  g1.tag = group_offsets ? "gemm_glu_grouped" : "gemm_glu_dense";
  SplitPlan sp1, sp2;
  float *part1 = nullptr, *part2 = nullptr;
  if (!group_offsets && !a_row_index && split_ws) {
    sp1 = plan_split_k(rows, 2 * (int64_t)inter, K, 0, K, esize(dt));
    part1 = split_region(sp1, rows, 2 * (int64_t)inter, split_ws, split_ws_bytes, 0);
    if (w2) {
      sp2 = plan_split_k(rows, n_out, inter, 0, inter, esize(dt));
      part2 = split_region(sp2, rows, n_out, split_ws, split_ws_bytes, 0);
    }
  }
  st = hip_status(run_gemm(g1, dt, Epi::Glu, shape, sp1, part1, s));
  if (st != LMOE_OK || !w2) return st;

  GemmArgs g2 = g1;
  g2.A = h;
  g2.lda = inter;
  g2.a_kwrap = inter;
  g2.a_rows = nullptr;
  g2.a_nrows = rows;
  g2.B = w2;
  g2.ldb = inter;
  g2.b_gstride = (int64_t)n_out * inter;
  g2.C = y;
  g2.ldc = n_out;
  g2.c_dtype = y_dtype;
  g2.N = n_out;
  g2.K = inter;
  g2.tag = group_offsets ? "gemm_down_grouped" : "gemm_out_dense";
  if (!group_offsets) shape = dense_shape(rows, ceil_div(n_out, 256));
  return hip_status(run_gemm(g2, dt, Epi::Store, shape, sp2, part2, s));
}

// Scratch of lmoe_grouped_situ_glu_noalloc: the m-tile list (G + 1 ints), on every device.
constexpr size_t kNoAllocScratchBytes = 16384;
__device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per device.
lmoe_status noalloc_scratch(int32_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LMOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LMOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LMOE_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return LMOE_OK;
}

}  // namespace

extern "C" {

lmoe_status lmoe_grouped_situ_glu(const lmoe_shape* sh, int32_t G, int32_t rows, int32_t K, int32_t inter,
                                  int32_t n_out, const void* a_in, int32_t a_rows, const int32_t* a_row_index,
                                  const int32_t* group_offsets, const void* w1, const void* w2, void* h, void* y,
                                  int32_t y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  lmoe_status st = check_grouped(sh, G, rows, K, inter, n_out, a_in, a_rows, a_row_index, group_offsets, w1, w2, h, y,
                                 y_dtype);
  if (st != LMOE_OK || rows == 0) return st;
  const size_t need = group_offsets ? glu_ws(G) : 0;
  if (need && (!workspace || workspace_bytes < need || !aligned16(workspace))) return LMOE_ERR_WORKSPACE;
  const size_t base = round_up(need);
  void* split_ws = workspace && aligned16(workspace) && workspace_bytes > base ? static_cast<char*>(workspace) + base
                                                                               : nullptr;
  return grouped_glu(sh, G, rows, K, inter, n_out, a_in, a_rows, a_row_index, group_offsets, w1, w2, h, y, y_dtype,
                     static_cast<int32_t*>(workspace), split_ws, split_ws ? workspace_bytes - base : 0,
                     static_cast<hipStream_t>(stream));
}

lmoe_status lmoe_grouped_situ_glu_noalloc(const lmoe_shape* sh, int32_t G, int32_t rows, int32_t K, int32_t inter,
                                          int32_t n_out, const void* a_in, int32_t a_rows,
                                          const int32_t* a_row_index, const int32_t* group_offsets, const void* w1,
                                          const void* w2, void* h, void* y, int32_t y_dtype, void* stream) {
  lmoe_status st = check_grouped(sh, G, rows, K, inter, n_out, a_in, a_rows, a_row_index, group_offsets, w1, w2, h, y,
                                 y_dtype);
  if (st != LMOE_OK || rows == 0) return st;
  if ((size_t)(G + 1) * sizeof(int32_t) > kNoAllocScratchBytes) return LMOE_ERR_UNSUPPORTED;
  int32_t* mts = nullptr;
  if (group_offsets) {
    st = noalloc_scratch(&mts);
    if (st != LMOE_OK) return st;
  }
  return grouped_glu(sh, G, rows, K, inter, n_out, a_in, a_rows, a_row_index, group_offsets, w1, w2, h, y, y_dtype,
                     mts, nullptr, 0, static_cast<hipStream_t>(stream));
}

}  // extern "C"

extern "C" {

lmoe_status lmoe_pack_shared(const lmoe_shape* sh, const void* w1s, const void* w2s, void* w1s_packed,
                             void* w2s_packed, void* stream) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if (sh->n_shared < 1 || sh->inter_shared < 64) return LMOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(w1s) || !aligned16(w2s) || !aligned16(w1s_packed) || !aligned16(w2s_packed))
    return LMOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_pack_shared(w1s, w2s, sh->n_shared, sh->inter_shared, sh->d_model, esize(sh->act_dtype),
                                       w1s_packed, w2s_packed, static_cast<hipStream_t>(stream)));
}

lmoe_status lmoe_combine_norm(const lmoe_shape* sh, const void* y_perm, const int32_t* slot_of_pair,
                              const float* topk_w, const float* gamma, void* n_out, void* stream) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if (sh->T == 0) return LMOE_OK;
  if (!aligned16(y_perm) || !aligned4(slot_of_pair) || !aligned4(topk_w) || (gamma && !aligned4(gamma)) ||
      !aligned16(n_out))
    return LMOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_combine_norm(y_perm, slot_of_pair, topk_w, gamma, sh->T, sh->top_k, sh->d_latent,
                                        sh->rms_eps, sh->act_dtype, n_out, static_cast<hipStream_t>(stream)));
}

lmoe_status lmoe_up_project(const lmoe_shape* sh, const void* n, const void* w_up, const float* y_shared,
                            const void* h_shared, const void* w2_shared, void* out, int32_t out_dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if (out_dtype != LMOE_F32 && out_dtype != sh->act_dtype) return LMOE_ERR_INVALID_ARGUMENT;
  if (sh->T == 0) return LMOE_OK;
  if ((h_shared != nullptr) != (w2_shared != nullptr) || (h_shared && y_shared)) return LMOE_ERR_INVALID_ARGUMENT;
  const int Ss = sh->n_shared * sh->inter_shared;
  if (h_shared && Ss < 64) return LMOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(n) || !aligned16(w_up) || (y_shared && !aligned4(y_shared)) || (h_shared && !aligned16(h_shared)) ||
      (w2_shared && !aligned16(w2_shared)) || !aligned16(out))
    return LMOE_ERR_INVALID_ARGUMENT;
  const int T = sh->T, D = sh->d_model, L = sh->d_latent;
  GemmArgs a = gemm_args();
  a.A = n;
  a.lda = L;
  a.a_kwrap = L;
  a.a_nrows = T;
  a.B = w_up;
  a.ldb = L;
  a.C = out;
  a.ldc = D;
  a.c_dtype = out_dtype;
  a.M = T;
  a.N = D;
  a.K = L;
  a.residual = y_shared;
  a.ldr = D;
  a.tag = "gemm_up";
  if (h_shared) {  // out = [n | h_s] . [w_up | w2_shared]^T: one accumulator for both products
    a.A2 = h_shared;
    a.lda2 = Ss;
    a.B2 = w2_shared;
    a.ldb2 = Ss;
    a.K1 = L;
    a.K = L + Ss;
  }
  const SplitPlan sp = up_plan(sh, h_shared != nullptr);
  float* part = split_region(sp, T, D, workspace, workspace_bytes, 0);
  return hip_status(run_gemm(a, sh->act_dtype, y_shared ? Epi::AddF32 : Epi::Store, dense_shape(T, ceil_div(D, 256)),
                             sp, part, static_cast<hipStream_t>(stream)));
}

lmoe_status lmoe_combine_norm_up(const lmoe_shape* sh, const void* y_perm, const int32_t* slot_of_pair,
                                 const float* topk_w, const float* gamma, const void* w_up, const float* y_shared,
                                 const void* h_shared, const void* w2_shared, void* n_out, void* out,
                                 int32_t out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if (out_dtype != LMOE_F32 && out_dtype != sh->act_dtype) return LMOE_ERR_INVALID_ARGUMENT;
  if (sh->T == 0) return LMOE_OK;
  if ((h_shared != nullptr) != (w2_shared != nullptr) || (h_shared && y_shared)) return LMOE_ERR_INVALID_ARGUMENT;
  const int Ss = sh->n_shared * sh->inter_shared;
  if (h_shared && Ss < 64) return LMOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y_perm) || !aligned4(slot_of_pair) || !aligned4(topk_w) || (gamma && !aligned4(gamma)) ||
      !aligned16(w_up) || (y_shared && !aligned4(y_shared)) || (h_shared && !aligned16(h_shared)) ||
      (w2_shared && !aligned16(w2_shared)) || !aligned16(n_out) || !aligned16(out))
    return LMOE_ERR_INVALID_ARGUMENT;
  st = lmoe_combine_norm(sh, y_perm, slot_of_pair, topk_w, gamma, n_out, stream);
  if (st != LMOE_OK) return st;
  return lmoe_up_project(sh, n_out, w_up, y_shared, h_shared, w2_shared, out, out_dtype, workspace, workspace_bytes,
                         stream);
}

lmoe_status lmoe_mx_quantize(const lmoe_shape* sh, int32_t fmt, int64_t rows, int32_t K, const void* x, void* codes,
                             void* scales, void* stream) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if ((fmt != LMOE_MX_FP4 && fmt != LMOE_MX_FP8) || rows < 0 || K <= 0) return LMOE_ERR_INVALID_ARGUMENT;
  if (K % 32) return LMOE_ERR_UNSUPPORTED;
  if (rows == 0) return LMOE_OK;
  if (!aligned16(x) || !aligned16(codes) || !scales) return LMOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_mx_quantize(x, sh->act_dtype, rows * (int64_t)(K / 32), fmt == LMOE_MX_FP4, codes, scales,
                                       static_cast<hipStream_t>(stream)));
}

lmoe_status lmoe_grouped_situ_glu_mx(const lmoe_shape* sh, int32_t G, int32_t rows, int32_t K, int32_t inter,
                                     int32_t n_out, const void* a_codes, const void* a_scales, int32_t a_rows,
                                     const int32_t* a_row_index, const int32_t* group_offsets, const void* w1_codes,
                                     const void* w1_scales, const void* w2_codes, const void* w2_scales, void* h,
                                     void* y, void* workspace, size_t workspace_bytes, void* stream) {
  lmoe_status st = check_shape(sh);
  if (st != LMOE_OK) return st;
  if (sh->act_dtype != LMOE_BF16) return LMOE_ERR_UNSUPPORTED;
  if (G < 1 || rows < 0 || a_rows < 0 || K <= 0 || inter <= 0 || n_out <= 0) return LMOE_ERR_INVALID_ARGUMENT;
  if (K % 128 || inter % 128 || n_out % 8) return LMOE_ERR_UNSUPPORTED;
  if (!group_offsets && G != 1) return LMOE_ERR_INVALID_ARGUMENT;
  if (!a_row_index && a_rows != rows) return LMOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)a_rows * K > 0x7fff0000LL || (int64_t)rows * inter > 0x7fff0000LL) return LMOE_ERR_UNSUPPORTED;
  if (rows == 0) return LMOE_OK;
  if (!aligned16(a_codes) || !aligned4(a_scales) || !aligned16(w1_codes) || !aligned4(w1_scales) ||
      !aligned16(w2_codes) || !aligned4(w2_scales) || !aligned16(h) || !aligned16(y) ||
      (a_row_index && !aligned4(a_row_index)) || (group_offsets && !aligned4(group_offsets)))
    return LMOE_ERR_INVALID_ARGUMENT;
  const size_t need = mx_glu_ws(G, rows, inter);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return LMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* mts = reinterpret_cast<int32_t*>(ws);
  uint8_t* h_codes = reinterpret_cast<uint8_t*>(ws + glu_ws(G));
  uint8_t* h_scales = h_codes + round_up((size_t)rows * inter);
  if (group_offsets) {
    st = hip_status(launch_mtile_prefix(group_offsets, G, gemm_block_m(GemmShape::Big), mts, s));
    if (st != LMOE_OK) return st;
  }
  GemmArgs g1 = gemm_args();
  g1.A = a_codes;
  g1.lda = K;  // bytes of FP8 codes
  g1.a_kwrap = K;
  g1.a_scale = static_cast<const uint8_t*>(a_scales);
  g1.a_rows = a_row_index;
  g1.a_nrows = a_rows;
  g1.B = w1_codes;
  g1.ldb = K / 2;  // bytes of packed FP4 codes
  g1.b_gstride = (int64_t)2 * inter * (K / 2);
  g1.b_scale = static_cast<const uint8_t*>(w1_scales);
  g1.b_scale_gstride = (int64_t)2 * inter * (K / 32);
  g1.C = h;
  g1.ldc = inter;
  g1.c_dtype = LMOE_BF16;
  g1.goff = group_offsets;
  g1.mtile_start = group_offsets ? mts : nullptr;
  g1.G = G;
  g1.M = rows;
  g1.N = inter;
  g1.K = K;
  g1.glu_up_off = inter;
  g1.beta1 = sh->beta1;
  g1.beta2 = sh->beta2;
  g1.tag = "gemm_glu_mx";
  st = hip_status(launch_gemm_mx(g1, Epi::Glu, s));
  if (st != LMOE_OK) return st;
  st = hip_status(launch_mx_quantize(h, LMOE_BF16, (int64_t)rows * (inter / 32), false, h_codes, h_scales, s));
  if (st != LMOE_OK) return st;
  GemmArgs g2 = g1;
  g2.A = h_codes;
  g2.lda = inter;
  g2.a_kwrap = inter;
  g2.a_scale = h_scales;
  g2.a_rows = nullptr;
  g2.a_nrows = rows;
  g2.B = w2_codes;
  g2.ldb = inter / 2;
  g2.b_gstride = (int64_t)n_out * (inter / 2);
  g2.b_scale = static_cast<const uint8_t*>(w2_scales);
  g2.b_scale_gstride = (int64_t)n_out * (inter / 32);
  g2.C = y;
  g2.ldc = n_out;
  g2.N = n_out;
  g2.K = inter;
  g2.tag = "gemm_down_mx";
  return hip_status(launch_gemm_mx(g2, Epi::Store, s));
}

}  // extern "C"
