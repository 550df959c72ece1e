// Backward-pass kernels that are not GEMMs: transposes that feed the weight-gradient GEMMs, the
// combine + RMSNorm + routing-weight backward, the router gradients, the un-permutation of the
// expert-input gradients, and the reduction of the RMSNorm gain gradient.
//
// The layer is [vxz] 01-02 / [slm] Latent-Space MoE; its gradients are the chain rule of the
// forward (the pages print no backward pass). Every sum runs in a fixed order, so results are
// deterministic run to run.
#include "common.h"

namespace lmoe {
namespace {

// ------------------------------------------------------------------------------------------------
// transposes: 64 x 64 tiles through LDS, 16-byte loads along the input rows and 16-byte stores
// along the output rows (V = 16 / sizeof(T) elements per access)
// ------------------------------------------------------------------------------------------------
template <typename T>
struct Pack16 {
  static constexpr int V = 16 / (int)sizeof(T);
};

template <typename T>
__device__ inline void tile_to_out(const T (*tile)[64 + 16 / sizeof(T)], T* __restrict__ out, int64_t ld_out,
                                   int c0, int q0, int C, int Q) {
  constexpr int V = Pack16<T>::V;
  constexpr int SEGS = 64 / V;  // 16-byte chunks per output row of the tile
  for (int ch = threadIdx.x; ch < 64 * SEGS; ch += 256) {
    const int oc = ch / SEGS, seg = ch % SEGS;
    const int c = c0 + oc, q = q0 + seg * V;
    if (c >= C || q >= Q) continue;
    T v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = tile[seg * V + i][oc];
    *reinterpret_cast<uint4*>(out + (int64_t)c * ld_out + q) = *reinterpret_cast<const uint4*>(v);
  }
}

// out[b][c][r] = in[b][r][c] for in [B][R][C] row-major; R and C multiples of 16 / sizeof(T).
template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(const T* __restrict__ in, T* __restrict__ out, int R, int C,
                                                        int64_t in_bstride, int64_t out_bstride) {
  constexpr int V = Pack16<T>::V;
  constexpr int SEGS = 64 / V;
  __shared__ __attribute__((aligned(16))) T tile[64][64 + V];
  const int64_t b = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const T* src = in + b * in_bstride;
  for (int ch = threadIdx.x; ch < 64 * SEGS; ch += 256) {
    const int i = ch / SEGS, seg = ch % SEGS;
    const int r = r0 + i, c = c0 + seg * V;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < R && c < C) v = *reinterpret_cast<const uint4*>(src + (int64_t)r * C + c);
    *reinterpret_cast<uint4*>(&tile[i][seg * V]) = v;
  }
  __syncthreads();
  tile_to_out<T>(tile, out + b * out_bstride, R, c0, r0, C, R);
}

// out[c][q] (ld_out columns) for q in [0, Q): column q takes input row src(q), or zero.
//   grouped (goff != nullptr): rows of group g occupy columns [64 * ptile[g], 64 * ptile[g] + n_g),
//     n_g = goff[g+1] - goff[g], and the rest of the group's 64-padded range is zero; ptile is the
//     prefix of ceil(n_g / 64);
//   plain: column q < rows takes row q, the rest is zero.
// With row_map the source row r is read at in[row_map[r]] (a gather). C and Q are multiples of
// 16 / sizeof(T).
template <typename T>
__global__ void __launch_bounds__(256) transpose_cols_kernel(const T* __restrict__ in, int64_t ld_in, int C,
                                                             const int32_t* __restrict__ goff,
                                                             const int32_t* __restrict__ ptile, int G, int rows,
                                                             const int32_t* __restrict__ row_map, T* __restrict__ out,
                                                             int64_t ld_out, int Q) {
  constexpr int V = Pack16<T>::V;
  constexpr int SEGS = 64 / V;
  __shared__ __attribute__((aligned(16))) T tile[64][64 + V];
  __shared__ int src[64];
  const int q0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (threadIdx.x < 64) {
    const int q = q0 + threadIdx.x;
    int sr = -1;
    if (q < Q) {
      if (goff != nullptr) {
        if (q < ptile[G] * 64) {
          int lo = 0, hi = G;  // 64 * ptile[lo] <= q < 64 * ptile[hi]
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (ptile[mid] * 64 <= q) lo = mid; else hi = mid;
          }
          const int local = q - ptile[lo] * 64;
          if (local < goff[lo + 1] - goff[lo]) sr = goff[lo] + local;
        }
      } else if (q < rows) {
        sr = q;
      }
      if (sr >= 0 && row_map != nullptr) sr = row_map[sr];
    }
    src[threadIdx.x] = sr;
  }
  __syncthreads();
  for (int ch = threadIdx.x; ch < 64 * SEGS; ch += 256) {
    const int i = ch / SEGS, seg = ch % SEGS;
    const int sr = src[i], c = c0 + seg * V;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (sr >= 0 && c < C) v = *reinterpret_cast<const uint4*>(in + (int64_t)sr * ld_in + c);
    *reinterpret_cast<uint4*>(&tile[i][seg * V]) = v;
  }
  __syncthreads();
  tile_to_out<T>(tile, out, ld_out, c0, q0, C, Q);
}

// ------------------------------------------------------------------------------------------------
// 16-byte vectors of activations
// ------------------------------------------------------------------------------------------------
template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ static inline void unpack(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static inline uint4 pack(const float* f) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static inline void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static inline uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// ------------------------------------------------------------------------------------------------
// combine + RMSNorm + routing-weight backward: one wave per token, kTokPerWave tokens per wave
// ------------------------------------------------------------------------------------------------
constexpr int kTokPerWave = 1;
constexpr int kTokPerBlock = 4 * kTokPerWave;

// Per token t (lane owns chunks c = lane + 64 i of the latent row):
//   z = sum_j w_j y_j (f32, j in rank order: the forward's value), r = 1 / sqrt(mean(z^2) + eps)
//   dz = r * gamma * dn - (r^3 / L) * sum(gamma dn z) * z;   dgamma += dn * z * r
//   dw_j = <dz, y_j>; dy[slot_j] = w_j dz;
//   S = sum_j s_j, ds_j = (dw_j - sum_i w_i dw_i) / S, dl_j = ds_j s_j (1 - s_j)
// The block's dgamma partial (its tokens summed in order) goes to part[blockIdx.x].
template <typename T, int CPL>
__global__ void __launch_bounds__(256) combine_bwd_kernel(const T* __restrict__ dn, const T* __restrict__ y,
                                                          const int32_t* __restrict__ slot_of_pair,
                                                          const int32_t* __restrict__ topk_idx,
                                                          const float* __restrict__ scores,
                                                          const float* __restrict__ topk_w,
                                                          const float* __restrict__ gamma, int T_, int k, int E,
                                                          int L, float eps, T* __restrict__ dy, float* __restrict__ dl,
                                                          float* __restrict__ dl_sorted, float* __restrict__ part) {
  constexpr int V = Vec<T>::N;
  __shared__ float red[3][1024 * 4];  // dgamma partials of waves 1..3 (up to 4096 floats each)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunks = L / V;
  float gacc[CPL][V];
#pragma unroll
  for (int i = 0; i < CPL; ++i)
#pragma unroll
    for (int v = 0; v < V; ++v) gacc[i][v] = 0.0f;

  for (int tw = 0; tw < kTokPerWave; ++tw) {
    const int64_t t = (int64_t)blockIdx.x * kTokPerBlock + wave * kTokPerWave + tw;
    if (t >= T_) break;
    float z[CPL][V];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int v = 0; v < V; ++v) z[i][v] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int32_t slot = slot_of_pair[t * k + j];
      if (slot < 0) continue;  // a pair the permutation dropped
      const float wj = topk_w[t * k + j];
      const T* row = y + (int64_t)slot * L;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < chunks) {
          float f[V];
          Vec<T>::unpack(*reinterpret_cast<const uint4*>(row + (int64_t)c * V), f);
#pragma unroll
          for (int v = 0; v < V; ++v) z[i][v] += wj * f[v];
        }
      }
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int v = 0; v < V; ++v) ss += z[i][v] * z[i][v];
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)L + eps);
    // sum(gamma dn z) and the dgamma contribution
    float saz = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) {
        float f[V];
        Vec<T>::unpack(*reinterpret_cast<const uint4*>(dn + t * L + (int64_t)c * V), f);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const float g = gamma ? gamma[c * V + v] : 1.0f;
          saz += g * f[v] * z[i][v];
          gacc[i][v] += f[v] * z[i][v] * r;
        }
      }
    }
    saz = wave_sum(saz);
    const float cz = r * r * r * saz / (float)L;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) {
        float f[V];
        Vec<T>::unpack(*reinterpret_cast<const uint4*>(dn + t * L + (int64_t)c * V), f);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const float g = gamma ? gamma[c * V + v] : 1.0f;
          z[i][v] = r * (g * f[v]) - cz * z[i][v];  // z now holds dz
        }
      }
    }
    // dw_j and dy rows
    float my_dw = 0.0f, my_w = 0.0f, my_s = 0.0f;
    int my_slot = -1;
    for (int j = 0; j < k; ++j) {
      const int32_t slot = slot_of_pair[t * k + j];
      const float wj = topk_w[t * k + j];
      const T* row = y + (int64_t)slot * L;
      T* drow = dy + (int64_t)slot * L;
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < chunks && slot >= 0) {
          float f[V], o[V];
          Vec<T>::unpack(*reinterpret_cast<const uint4*>(row + (int64_t)c * V), f);
#pragma unroll
          for (int v = 0; v < V; ++v) {
            dot += z[i][v] * f[v];
            o[v] = wj * z[i][v];
          }
          *reinterpret_cast<uint4*>(drow + (int64_t)c * V) = Vec<T>::pack(o);
        }
      }
      dot = wave_sum(dot);
      if (lane == j && slot >= 0) {
        my_dw = dot;
        my_w = wj;
        my_slot = slot;
        my_s = scores[t * E + topk_idx[t * k + j]];
      }
    }
    const float S = wave_sum(my_s);            // lanes >= k hold zeros
    const float wdw = wave_sum(my_w * my_dw);
    if (lane < k) {
      const float ds = (my_dw - wdw) / S;
      const float g = ds * my_s * (1.0f - my_s);
      dl[t * k + lane] = g;
      if (my_slot >= 0) dl_sorted[my_slot] = g;
    }
  }
  // dgamma: block partial = wave 0 + wave 1 + wave 2 + wave 3, in that order
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int v = 0; v < V; ++v) red[wave - 1][(i * V + v) * 64 + lane] = gacc[i][v];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float a = gacc[i][v];
        for (int w = 0; w < 3; ++w) a += red[w][(i * V + v) * 64 + lane];
        if (c < chunks) part[(int64_t)blockIdx.x * L + c * V + v] = a;
      }
    }
  }
}

// out[g][l] = sum over rows b in [64 g, 64 g + 64) of part[b][l], in row order.
__global__ void __launch_bounds__(256) sum_rows_kernel(const float* __restrict__ part, int nrows, int L,
                                                       float* __restrict__ out) {
  const int l = blockIdx.x * 256 + threadIdx.x;
  const int g = blockIdx.y;
  if (l >= L) return;
  const int b1 = min(nrows, 64 * (g + 1));
  float a = 0.0f;
  for (int b = 64 * g; b < b1; ++b) a += part[(int64_t)b * L + l];
  out[(int64_t)g * L + l] = a;
}

// ------------------------------------------------------------------------------------------------
// router gradients
// ------------------------------------------------------------------------------------------------
// dW_r[e, cols] = sum over expert e's sorted rows r (ascending) of dl_sorted[r] * x[sorted_token[r], cols].
// One wave per (column chunk, expert); each lane owns one 16-byte chunk of x.
template <typename T>
__global__ void __launch_bounds__(64) router_dw_kernel(const T* __restrict__ x, int D,
                                                       const int32_t* __restrict__ goff,
                                                       const int32_t* __restrict__ sorted_token,
                                                       const float* __restrict__ dl_sorted, float* __restrict__ dw) {
  constexpr int V = Vec<T>::N;
  const int e = blockIdx.y;
  const int c = blockIdx.x * 64 + threadIdx.x;  // chunk of V columns
  const bool ok = c * V < D;
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.0f;
  const int r0 = goff[e], r1 = goff[e + 1];
  for (int r = r0; r < r1; ++r) {
    const float g = dl_sorted[r];
    const int64_t t = sorted_token[r];
    if (ok) {
      float f[V];
      Vec<T>::unpack(*reinterpret_cast<const uint4*>(x + t * D + (int64_t)c * V), f);
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] += g * f[v];
    }
  }
  if (ok) {
#pragma unroll
    for (int v = 0; v < V; ++v) dw[(int64_t)e * D + c * V + v] = acc[v];
  }
}

// dx[t, cols] = sum_j dl[t, j] * W_r[idx[t, j], cols] (f32, j in rank order); overwrites dx.
__global__ void __launch_bounds__(64) router_dx_kernel(const float* __restrict__ w_router, int D,
                                                       const int32_t* __restrict__ topk_idx,
                                                       const float* __restrict__ dl, int k, float* __restrict__ dx) {
  const int64_t t = blockIdx.y;
  const int c = blockIdx.x * 64 + threadIdx.x;  // chunk of 4 columns
  if (c * 4 >= D) return;
  float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j = 0; j < k; ++j) {
    const float g = dl[t * k + j];
    const float4 w = *reinterpret_cast<const float4*>(w_router + (int64_t)topk_idx[t * k + j] * D + c * 4);
    a.x += g * w.x;
    a.y += g * w.y;
    a.z += g * w.z;
    a.w += g * w.w;
  }
  *reinterpret_cast<float4*>(dx + t * D + c * 4) = a;
}

// ------------------------------------------------------------------------------------------------
// un-permutation: dx_lat[t] = sum_j dx_perm[slot(t, j)] (f32 in rank order, stored)
// ------------------------------------------------------------------------------------------------
template <typename T, int CPL>
__global__ void __launch_bounds__(256) unpermute_kernel(const T* __restrict__ src, const int32_t* __restrict__ slot_of_pair,
                                                        int T_, int k, int L, T* __restrict__ out) {
  constexpr int V = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const int chunks = L / V;
  float a[CPL][V];
#pragma unroll
  for (int i = 0; i < CPL; ++i)
#pragma unroll
    for (int v = 0; v < V; ++v) a[i][v] = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int32_t slot = slot_of_pair[t * k + j];
    if (slot < 0) continue;  // a pair the permutation dropped
    const T* row = src + (int64_t)slot * L;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) {
        float f[V];
        Vec<T>::unpack(*reinterpret_cast<const uint4*>(row + (int64_t)c * V), f);
#pragma unroll
        for (int v = 0; v < V; ++v) a[i][v] += f[v];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (c < chunks) *reinterpret_cast<uint4*>(out + t * L + (int64_t)c * V) = Vec<T>::pack(a[i]);
  }
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------
hipError_t launch_transpose(const void* in, void* out, int batch, int R, int C, int64_t in_bstride,
                            int64_t out_bstride, int esz, hipStream_t s) {
  KernelTimer timer("bwd_transpose", s);
  if (batch <= 0 || R <= 0 || C <= 0) return hipSuccess;
  if (ceil_div(R, 64) > 65535 || batch > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)ceil_div(C, 64), (unsigned)ceil_div(R, 64), (unsigned)batch), block(256);
  if (esz == 2)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, block, 0, s, static_cast<const uint16_t*>(in),
                       static_cast<uint16_t*>(out), R, C, in_bstride, out_bstride);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, s, static_cast<const float*>(in),
                       static_cast<float*>(out), R, C, in_bstride, out_bstride);
  return hipGetLastError();
}

hipError_t launch_transpose_cols(const void* in, int64_t ld_in, int C, const int32_t* goff, const int32_t* ptile,
                                 int G, int rows, const int32_t* row_map, void* out, int64_t ld_out, int Q, int esz,
                                 hipStream_t s) {
  KernelTimer timer("bwd_transpose", s);
  if (C <= 0 || Q <= 0) return hipSuccess;
  if (ceil_div(Q, 64) > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)ceil_div(C, 64), (unsigned)ceil_div(Q, 64)), block(256);
  if (esz == 2)
    hipLaunchKernelGGL(transpose_cols_kernel<uint16_t>, grid, block, 0, s, static_cast<const uint16_t*>(in), ld_in, C,
                       goff, ptile, G, rows, row_map, static_cast<uint16_t*>(out), ld_out, Q);
  else
    hipLaunchKernelGGL(transpose_cols_kernel<float>, grid, block, 0, s, static_cast<const float*>(in), ld_in, C, goff,
                       ptile, G, rows, row_map, static_cast<float*>(out), ld_out, Q);
  return hipGetLastError();
}

int combine_bwd_blocks(int T) { return (int)ceil_div(T > 0 ? T : 1, kTokPerBlock); }

template <typename T>
static hipError_t combine_bwd_t(const void* dn, const void* y, const int32_t* slot, const int32_t* idx,
                                const float* scores, const float* w, const float* gamma, int T_, int k, int E, int L,
                                float eps, void* dy, float* dl, float* dl_sorted, float* part, hipStream_t s) {
  const int cpl = (int)ceil_div(L / Vec<T>::N, 64);
  const dim3 grid((unsigned)combine_bwd_blocks(T_)), block(256);
  const T* a = static_cast<const T*>(dn);
  const T* b = static_cast<const T*>(y);
  T* o = static_cast<T*>(dy);
#define LMOE_CB(C)                                                                                               \
  hipLaunchKernelGGL((combine_bwd_kernel<T, C>), grid, block, 0, s, a, b, slot, idx, scores, w, gamma, T_, k, E, \
                     L, eps, o, dl, dl_sorted, part)
  if (cpl <= 1) LMOE_CB(1);
  else if (cpl <= 2) LMOE_CB(2);
  else if (cpl <= 4) LMOE_CB(4);
  else if (cpl <= 8) LMOE_CB(8);
  else return hipErrorInvalidValue;
#undef LMOE_CB
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dn, const void* y, const int32_t* slot, const int32_t* idx,
                              const float* scores, const float* w, const float* gamma, int T, int k, int E, int L,
                              float eps, int dtype, void* dy, float* dl, float* dl_sorted, float* part,
                              float* dgamma, hipStream_t s) {
  {
    KernelTimer timer("bwd_combine_norm", s);
    const hipError_t e =
        dtype == LMOE_BF16
            ? combine_bwd_t<uint16_t>(dn, y, slot, idx, scores, w, gamma, T, k, E, L, eps, dy, dl, dl_sorted, part, s)
            : combine_bwd_t<float>(dn, y, slot, idx, scores, w, gamma, T, k, E, L, eps, dy, dl, dl_sorted, part, s);
    if (e != hipSuccess) return e;
  }
  // dgamma = sum of the block partials, folding 64 rows at a time in row order; the levels alternate
  // between the partial rows and the region after them (part holds blocks + ceil(blocks / 64) rows)
  KernelTimer timer("bwd_dgamma", s);
  const int blocks = combine_bwd_blocks(T);
  float* bufs[2] = {part, part + (size_t)blocks * L};
  int cur = 0, nrows = blocks;
  for (;;) {
    const int groups = (int)ceil_div(nrows, 64);
    float* dst = groups == 1 ? dgamma : bufs[cur ^ 1];
    hipLaunchKernelGGL(sum_rows_kernel, dim3((unsigned)ceil_div(L, 256), (unsigned)groups), dim3(256), 0, s, bufs[cur],
                       nrows, L, dst);
    if (groups == 1) break;
    nrows = groups;
    cur ^= 1;
  }
  return hipGetLastError();
}

hipError_t launch_router_bwd(const void* x, const float* w_router, const float* dl, const float* dl_sorted,
                             const int32_t* topk_idx, const int32_t* goff, const int32_t* sorted_token, int T, int D,
                             int E, int k, int dtype, float* dw_router, float* dx, hipStream_t s) {
  {
    KernelTimer timer("bwd_router_dw", s);
    const int V = dtype == LMOE_BF16 ? 8 : 4;
    const dim3 grid((unsigned)ceil_div(D / V, 64), (unsigned)E), block(64);
    if (dtype == LMOE_BF16)
      hipLaunchKernelGGL(router_dw_kernel<uint16_t>, grid, block, 0, s, static_cast<const uint16_t*>(x), D, goff,
                         sorted_token, dl_sorted, dw_router);
    else
      hipLaunchKernelGGL(router_dw_kernel<float>, grid, block, 0, s, static_cast<const float*>(x), D, goff,
                         sorted_token, dl_sorted, dw_router);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  KernelTimer timer("bwd_router_dx", s);
  if (T <= 0) return hipSuccess;
  if (T > 65535) {  // one grid row per token: split long batches
    for (int t0 = 0; t0 < T; t0 += 65535) {
      const int n = T - t0 < 65535 ? T - t0 : 65535;
      hipLaunchKernelGGL(router_dx_kernel, dim3((unsigned)ceil_div(D / 4, 64), (unsigned)n), dim3(64), 0, s, w_router,
                         D, topk_idx + (int64_t)t0 * k, dl + (int64_t)t0 * k, k, dx + (int64_t)t0 * D);
    }
  } else {
    hipLaunchKernelGGL(router_dx_kernel, dim3((unsigned)ceil_div(D / 4, 64), (unsigned)T), dim3(64), 0, s, w_router, D,
                       topk_idx, dl, k, dx);
  }
  return hipGetLastError();
}

hipError_t launch_unpermute(const void* src, const int32_t* slot_of_pair, int T, int k, int L, int dtype, void* out,
                            hipStream_t s) {
  KernelTimer timer("bwd_unpermute", s);
  const dim3 grid((unsigned)ceil_div(T, 4)), block(256);
  const int V = dtype == LMOE_BF16 ? 8 : 4;
  const int cpl = (int)ceil_div(L / V, 64);
#define LMOE_UP(TT, C)                                                                                           \
  hipLaunchKernelGGL((unpermute_kernel<TT, C>), grid, block, 0, s, static_cast<const TT*>(src), slot_of_pair, T, k, L, \
                     static_cast<TT*>(out))
  if (dtype == LMOE_BF16) {
    if (cpl <= 1) LMOE_UP(uint16_t, 1);
    else if (cpl <= 2) LMOE_UP(uint16_t, 2);
    else if (cpl <= 4) LMOE_UP(uint16_t, 4);
    else if (cpl <= 8) LMOE_UP(uint16_t, 8);
    else if (cpl <= 16) LMOE_UP(uint16_t, 16);
    else return hipErrorInvalidValue;
  } else {
    if (cpl <= 1) LMOE_UP(float, 1);
    else if (cpl <= 2) LMOE_UP(float, 2);
    else if (cpl <= 4) LMOE_UP(float, 4);
    else if (cpl <= 8) LMOE_UP(float, 8);
    else if (cpl <= 16) LMOE_UP(float, 16);
    else return hipErrorInvalidValue;
  }
#undef LMOE_UP
  return hipGetLastError();
}

}  // namespace lmoe
