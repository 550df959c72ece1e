// Shared device helpers and internal launcher declarations for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lmoe.h"

namespace lmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: workgroups are dispatched round-robin over 8 XCDs

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t hmin(int64_t a, int64_t b) { return a < b ? a : b; }
inline int64_t hmax(int64_t a, int64_t b) { return a > b ? a : b; }

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round to nearest even (gfx950 converts in hardware; NaN stays NaN).
__device__ inline uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

template <typename T>
__device__ inline float load_as_f32(const T* p, int64_t i);
template <>
__device__ inline float load_as_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ inline float load_as_f32<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename T>
__device__ inline void store_f32_as(T* p, int64_t i, float v);
template <>
__device__ inline void store_f32_as<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ inline void store_f32_as<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

// 1/x through the hardware reciprocal (about 1 ulp): rcp(inf) = 0, rcp(1) = 1.
__device__ inline float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// sigmoid through one exponential: 1 / (1 + e^-x); e^-x -> inf gives 0 and -> 0 gives 1.
__device__ inline float sigmoid_fast(float x) { return fast_rcp(1.0f + __expf(-x)); }

// tanh(y) = 1 - 2 / (e^{2y} + 1): saturates to +-1 without overflow (e^{2y} -> inf or 0).
__device__ inline float tanh_fast(float y) { return 1.0f - 2.0f * fast_rcp(__expf(2.0f * y) + 1.0f); }

// SiTU-GLU of one gate/up pair ([tahou] SiTU激活优化, [slm] SiTU 激活):
//   beta1*tanh(g/beta1)*sigmoid(g) * beta2*tanh(u/beta2)
// with 1/beta passed in, and each factor clamped to its bound so rounding cannot step outside it.
// The f32 storage path (ACCURATE) uses the full-precision tanhf/expf and IEEE division instead.
template <bool ACCURATE>
__device__ inline float situ_glu(float g, float u, float beta1, float inv_beta1, float beta2, float inv_beta2) {
  float act, cap;
  if constexpr (ACCURATE) {
    act = beta1 * tanhf(g / beta1) * (1.0f / (1.0f + expf(-g)));
    cap = beta2 * tanhf(u / beta2);
  } else {
    act = beta1 * tanh_fast(g * inv_beta1) * sigmoid_fast(g);
    cap = beta2 * tanh_fast(u * inv_beta2);
  }
  act = fminf(act, beta1);
  cap = fminf(fmaxf(cap, -beta2), beta2);
  return act * cap;
}

// ------------------------------------------------------------------------------------------------
// kernel timing (profile.cpp)
// ------------------------------------------------------------------------------------------------
struct KernelTimer {
  KernelTimer(const char* name, hipStream_t s);
  ~KernelTimer();
  const char* name;
  hipStream_t stream;
  void* ev0;
};

// ------------------------------------------------------------------------------------------------
// launchers (return hipSuccess or the launch error)
// ------------------------------------------------------------------------------------------------
// Store: C = acc; Glu: C = SiTU-GLU(gate acc, up acc); Sigmoid: C = sigmoid(acc + col_bias) (f32);
// AddF32: C = acc + residual (f32); GluBwd: from the recomputed gate/up accumulators and the
// incoming dh (aux), C[:, c] = dg and C[:, N + c] = du (the SiTU-GLU derivative).
enum class Epi : int { Store = 0, Glu = 1, Sigmoid = 2, AddF32 = 3, GluBwd = 4 };

// Derivative of h = SiTU(g) * cap(u): returns dg and du for the incoming dh, in f32 with the
// full-precision tanhf/expf.
__device__ inline void situ_glu_bwd(float g, float u, float dh, float beta1, float beta2, float& dg, float& du) {
  const float t1 = tanhf(g / beta1), sg = 1.0f / (1.0f + expf(-g)), t2 = tanhf(u / beta2);
  const float act = beta1 * t1 * sg, cap = beta2 * t2;
  const float dact = (1.0f - t1 * t1) * sg + beta1 * t1 * sg * (1.0f - sg);
  dg = dh * cap * dact;
  du = dh * act * (1.0f - t2 * t2);
}

struct GemmArgs {
  const void* A;
  int64_t lda;        // elements
  int a_kwrap;        // A is read at column (k mod a_kwrap); = K when no wrap
  const void* B;
  int64_t ldb;        // elements
  int64_t b_gstride;  // elements between groups of B
  void* C;
  int64_t ldc;        // elements
  int c_dtype;        // lmoe_dtype of C
  const int32_t* goff;         // [G+1] device row offsets, or nullptr for one group of M rows
  const int32_t* mtile_start;  // [G+1] device m-tile prefix (grouped only)
  int G, M, N, K;              // N = output columns (GLU: inner size)
  int glu_up_off;              // GLU: first up row of B inside a group
  float beta1, beta2;
  const float* col_bias;       // Sigmoid: per-column logit offset or nullptr
  const float* residual;       // AddF32: [M, N] f32
  int64_t ldr;
  const char* tag;             // kernel name for timing
  // Row gather of A: GEMM row r reads A row a_rows[r] (a_nrows rows in A); nullptr = row r.
  const int32_t* a_rows;
  int a_nrows;
  // Second K segment: k >= K1 reads A2 [M, K - K1] and B2 [N, K - K1] (nullptr = none, K1 = K).
  const void* A2;
  int64_t lda2;
  const void* B2;
  int64_t ldb2;
  int K1;
  // Split-K (register pipeline, dense): workgroup row blockIdx.y = s multiplies K-chunk s (K
  // elements) of the concatenated range [0, K1) of A/B then [K1, ...) of A2/B2, and stores its f32
  // partial product at C + s * c_split. splits <= 1: no split.
  int splits;
  int64_t c_split;
  // GluBwd: dh [M, N] in the input type, row stride ld_aux.
  const void* aux;
  int64_t ld_aux;
  // K-grouped (weight gradients): koff [G+1] device, group g contracts K in
  // [koff[g] * koff_scale, koff[g+1] * koff_scale) of A and B (both [*, K_total]) into its own
  // output C + g * c_gstride of M x N. Mutually exclusive with goff.
  const int32_t* koff;
  int koff_scale;
  int64_t c_gstride;
  // B stored [K, N] (row k holds every output column; ldb = row stride) instead of [N, K]: the
  // register pipeline transposes it on its way into LDS. Store / AddF32 epilogues, no second K
  // segment, no split.
  bool b_kn;
  // MX operands (launch_gemm_mx): E8M0 scale bytes [rows, K/32] of A and [N, K/32] of each B group
  // (b_scale_gstride bytes apart); A, B, lda, ldb and b_gstride then count bytes of element codes.
  const uint8_t* a_scale;
  const uint8_t* b_scale;
  int64_t b_scale_gstride;
};

// K-split of a dense GEMM on few rows (decode-size batches), so that its register-pipeline tiles
// occupy every CU; the partial products are then summed by a reduction that applies the epilogue.
struct SplitPlan {
  int splits = 1;    // 1 = no split
  int chunk = 0;     // K elements per split
  bool big = false;  // splits run on the 256x256 DMA pipeline (else the 128x128 register pipeline)
};
SplitPlan plan_split_k(int64_t M, int64_t n_cols, int K1, int K2, int a_kwrap, int esz);
// Split for a bf16 GEMM whose 256x256 tiles fill between a quarter and all of the CUs: the fewest
// splits (at most 4) that give every CU a tile, each a whole number of DMA K-tiles of one segment.
SplitPlan plan_split_k_big(int64_t M, int64_t n_cols, int K1, int K2, int esz);
size_t split_k_bytes(const SplitPlan& sp, int64_t M, int64_t n_cols);
// Runs a (dense, non-gathered) GEMM as the planned split plus the reducing epilogue; partials holds
// split_k_bytes() bytes, split s of output row m at partials + (s * M + m) * n_cols. With reduce =
// false only the partial products are written (the caller's next kernel sums them).
hipError_t launch_gemm_split(const GemmArgs& a, int in_dtype, Epi epi, const SplitPlan& sp, float* partials,
                             hipStream_t s, bool reduce = true);

enum class GemmShape : int { Big = 0, Small = 1 };

hipError_t launch_gemm(const GemmArgs& a, int in_dtype, Epi epi, GemmShape shape, hipStream_t s);
int gemm_block_m(GemmShape shape);
hipError_t launch_mtile_prefix(const int32_t* goff, int G, int bm, int32_t* mtile_start, hipStream_t s);

// shape validation shared by the forward and backward calls (api.hip); backward workspace sizes
lmoe_status validate_shape(const lmoe_shape* sh);
size_t bwd_workspace_bytes(const lmoe_shape* sh, int which);

hipError_t launch_gemm_mx(const GemmArgs& a, Epi epi, hipStream_t s);

// MX quantisation (mx.hip): nblocks blocks of 32 elements of x (act dtype) -> FP4 (packed) or FP8
// codes and E8M0 scale bytes
hipError_t launch_mx_quantize(const void* x, int dtype, int64_t nblocks, bool fp4, void* codes, void* scales,
                              hipStream_t s);

// backward (backward.hip)
hipError_t launch_transpose(const void* in, void* out, int batch, int R, int C, int64_t in_bstride,
                            int64_t out_bstride, int esz, hipStream_t s);
hipError_t launch_transpose_cols(const void* in, int64_t ld_in, int C, const int32_t* goff, const int32_t* ptile,
                                 int G, int rows, const int32_t* row_map, void* out, int64_t ld_out, int Q, int esz,
                                 hipStream_t s);
int combine_bwd_blocks(int T);
hipError_t launch_combine_bwd(const void* dn, const void* y, const int32_t* slot, const int32_t* idx,
                              const float* scores, const float* w, const float* gamma, int T, int k, int E, int L,
                              float eps, int dtype, void* dy, float* dl, float* dl_sorted, float* part,
                              float* dgamma, hipStream_t s);
hipError_t launch_router_bwd(const void* x, const float* w_router, const float* dl, const float* dl_sorted,
                             const int32_t* topk_idx, const int32_t* goff, const int32_t* sorted_token, int T, int D,
                             int E, int k, int dtype, float* dw_router, float* dx, hipStream_t s);
hipError_t launch_unpermute(const void* src, const int32_t* slot_of_pair, int T, int k, int L, int dtype, void* out,
                            hipStream_t s);

hipError_t launch_split3(const float* w, uint16_t* out, int rows, int cols, hipStream_t s);
hipError_t launch_topk(const float* scores, const float* bias, int T, int E, int k, int32_t* idx, float* w,
                       float* thresh, hipStream_t s);
// The router's split-K reduction fused with the top-k: scores = sigmoid(sum of the `splits` partial
// logits in split order + logit_offset), written to `scores` and selected from registers.
hipError_t launch_topk_partials(const float* partials, int splits, const float* logit_offset, float* scores,
                                const float* bias, int T, int E, int k, int32_t* idx, float* w, float* thresh,
                                hipStream_t s);
hipError_t launch_qb_hist(const float* scores, const float* bias, const int32_t* idx, const float* thresh, int T,
                          int E, int k, int nb, uint32_t* hist, hipStream_t s);
hipError_t launch_qb_update(uint32_t* hist, int E, int k, int nb, int64_t n_acc, float* bias, hipStream_t s);

hipError_t launch_permute(const int32_t* idx, int T, int E, int k, int32_t* offsets, int32_t* sorted_token,
                          int32_t* slot_of_pair, int32_t* chunk_count, hipStream_t s);
hipError_t launch_gather_rows(const void* x_lat, const int32_t* slot_of_pair, int T, int k, int64_t row_bytes,
                              void* x_perm, hipStream_t s);
hipError_t launch_combine_norm(const void* y, const int32_t* slot_of_pair, const float* w, const float* gamma,
                               int T, int k, int L, float eps, int dtype, void* n_out, hipStream_t s);
hipError_t launch_pack_shared(const void* w1s, const void* w2s, int S, int Is, int D, int esz, void* w1p,
                              void* w2p, hipStream_t s);

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

constexpr int kPermChunk = 256;  // tokens per permutation chunk

}  // namespace lmoe
