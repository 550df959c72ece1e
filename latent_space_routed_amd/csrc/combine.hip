// Router-weighted combine and RMSNorm, one wave per token ([vxz] 02; [tahou] 归一化策略调整: the
// norm sits after the aggregation of the routed experts and before the up-projection).
//   z = sum_j w[t, j] * y[slot(t, j)]   (f32, in rank order j = 0..k-1)
//   n = gamma * z / sqrt(mean(z^2) + eps)
// A lane owns CPL 16-byte chunks of the latent row (chunk c = lane + 64 i), so every y row is read
// with fully coalesced 16-byte loads and z never leaves registers.
#include "common.h"

namespace lmoe {
namespace {

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

// 16-byte load with the non-temporal hint: every y row is read once, here, so it is streamed past
// the caches (measured at K3 prefill: 0.219 -> 0.196 ms).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ inline uint4 load16_nt(const void* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T, int CPL>
__global__ void __launch_bounds__(256) combine_norm_kernel(const T* __restrict__ y, const int32_t* __restrict__ slot_of_pair,
                                                           const float* __restrict__ w, const float* __restrict__ gamma,
                                                           int T_, int k, int L, float eps, T* __restrict__ n_out) {
  constexpr int V = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const int chunks = L / V;
  float z[CPL][V];
#pragma unroll
  for (int i = 0; i < CPL; ++i)
#pragma unroll
    for (int v = 0; v < V; ++v) z[i][v] = 0.0f;
  // the token's slots and weights are loaded once, lane j holding pair j (k <= 64), and read back
  // as wave-uniform values, so no load of a y row waits on a load of its slot
  const int32_t my_slot = lane < k ? slot_of_pair[t * k + lane] : -1;
  const float my_w = lane < k ? w[t * k + lane] : 0.0f;
  // two rows in flight per step; the sum still runs in rank order j = 0, 1, 2, ...
  for (int j = 0; j < k; j += 2) {
    const bool two = j + 1 < k;
    const int32_t s0 = __builtin_amdgcn_readlane(my_slot, j);
    const int32_t s1 = two ? __builtin_amdgcn_readlane(my_slot, j + 1) : -1;
    const float w0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j));
    const float w1 = two ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j + 1))
                         : 0.0f;
    uint4 r0[CPL], r1[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      r0[i] = (c < chunks && s0 >= 0) ? load16_nt(y + (int64_t)s0 * L + (int64_t)c * V) : make_uint4(0, 0, 0, 0);
      r1[i] = (c < chunks && s1 >= 0) ? load16_nt(y + (int64_t)s1 * L + (int64_t)c * V) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      float f[V];
      if (s0 >= 0) {
        Vec<T>::unpack(r0[i], f);
#pragma unroll
        for (int v = 0; v < V; ++v) z[i][v] += w0 * f[v];
      }
      if (s1 >= 0) {
        Vec<T>::unpack(r1[i], f);
#pragma unroll
        for (int v = 0; v < V; ++v) z[i][v] += w1 * f[v];
      }
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < CPL; ++i)
#pragma unroll
    for (int v = 0; v < V; ++v) ss += z[i][v] * z[i][v];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d);
  const float r = 1.0f / sqrtf(ss / (float)L + eps);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (c < chunks) {
      float f[V];
#pragma unroll
      for (int v = 0; v < V; ++v) f[v] = (gamma ? gamma[c * V + v] : 1.0f) * (z[i][v] * r);
      *reinterpret_cast<uint4*>(n_out + t * L + (int64_t)c * V) = Vec<T>::pack(f);
    }
  }
}

template <typename T>
hipError_t launch_t(const void* y, const int32_t* sp, const float* w, const float* gamma, int T_, int k, int L,
                    float eps, void* n, hipStream_t s) {
  const int cpl = (int)ceil_div(L / Vec<T>::N, 64);
  const dim3 grid((unsigned)ceil_div(T_, 4)), block(256);
  const T* yy = static_cast<const T*>(y);
  T* nn = static_cast<T*>(n);
#define LMOE_COMBINE_CASE(C) \
  case C: hipLaunchKernelGGL((combine_norm_kernel<T, C>), grid, block, 0, s, yy, sp, w, gamma, T_, k, L, eps, nn); break;
  switch (cpl) {  // one instance per chunk count, so no lane carries a dead chunk's registers
    LMOE_COMBINE_CASE(1) LMOE_COMBINE_CASE(2) LMOE_COMBINE_CASE(3) LMOE_COMBINE_CASE(4)
    LMOE_COMBINE_CASE(5) LMOE_COMBINE_CASE(6) LMOE_COMBINE_CASE(7) LMOE_COMBINE_CASE(8)
    LMOE_COMBINE_CASE(9) LMOE_COMBINE_CASE(10) LMOE_COMBINE_CASE(11) LMOE_COMBINE_CASE(12)
    LMOE_COMBINE_CASE(13) LMOE_COMBINE_CASE(14) LMOE_COMBINE_CASE(15) LMOE_COMBINE_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef LMOE_COMBINE_CASE
  return hipGetLastError();
}

// Lean variant: four waves per token (a workgroup of 256 lanes), lane g owning the 16-byte chunks
// g + 256 i of the latent row, R rows in flight per step. Few registers per wave (about 60 at K3
// shape against 129 for one wave per token), so its waves fit beside a resident GEMM workgroup
// (which leaves 80 VGPRs and 32 KB of LDS per SIMD) when a caller runs the combine beside a dense
// GEMM on another stream. The four waves' partial sums of squares meet in LDS.
template <typename T, int CPW, int R>
__global__ void __launch_bounds__(256) combine_norm_lean_kernel(const T* __restrict__ y,
                                                                const int32_t* __restrict__ slot_of_pair,
                                                                const float* __restrict__ w,
                                                                const float* __restrict__ gamma, int T_, int k, int L,
                                                                float eps, T* __restrict__ n_out) {
  constexpr int V = Vec<T>::N;
  __shared__ float ssw[4];
  const int g = threadIdx.x, lane = g & 63, wv = g >> 6;
  const int64_t t = blockIdx.x;
  if (t >= T_) return;
  const int chunks = L / V;
  float z[CPW][V];
#pragma unroll
  for (int i = 0; i < CPW; ++i)
#pragma unroll
    for (int v = 0; v < V; ++v) z[i][v] = 0.0f;
  const int32_t my_slot = lane < k ? slot_of_pair[t * k + lane] : -1;
  const float my_w = lane < k ? w[t * k + lane] : 0.0f;
  for (int j0 = 0; j0 < k; j0 += R) {
    int32_t s[R];
    float wt[R];
    uint4 r[R][CPW];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int j = j0 + q;
      s[q] = j < k ? __builtin_amdgcn_readlane(my_slot, j) : -1;
      wt[q] = j < k ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j)) : 0.0f;
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int c = g + 256 * i;
        r[q][i] = (c < chunks && s[q] >= 0) ? load16_nt(y + (int64_t)s[q] * L + (int64_t)c * V) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {  // rank order j = j0, j0 + 1, ...
      if (s[q] < 0) continue;
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        float f[V];
        Vec<T>::unpack(r[q][i], f);
#pragma unroll
        for (int v = 0; v < V; ++v) z[i][v] += wt[q] * f[v];
      }
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < CPW; ++i)
#pragma unroll
    for (int v = 0; v < V; ++v) ss += z[i][v] * z[i][v];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d);
  if (lane == 0) ssw[wv] = ss;
  __syncthreads();
  const float tot = (ssw[0] + ssw[1]) + (ssw[2] + ssw[3]);
  const float rn = 1.0f / sqrtf(tot / (float)L + eps);
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = g + 256 * i;
    if (c < chunks) {
      float f[V];
#pragma unroll
      for (int v = 0; v < V; ++v) f[v] = (gamma ? gamma[c * V + v] : 1.0f) * (z[i][v] * rn);
      *reinterpret_cast<uint4*>(n_out + t * L + (int64_t)c * V) = Vec<T>::pack(f);
    }
  }
}

template <typename T, int R>
hipError_t launch_lean(const void* y, const int32_t* sp, const float* w, const float* gamma, int T_, int k, int L,
                       float eps, void* n, hipStream_t s) {
  const int cpw = (int)ceil_div(L / Vec<T>::N, 256);
  const dim3 grid((unsigned)T_), block(256);
  const T* yy = static_cast<const T*>(y);
  T* nn = static_cast<T*>(n);
  switch (cpw) {
    case 1: hipLaunchKernelGGL((combine_norm_lean_kernel<T, 1, R>), grid, block, 0, s, yy, sp, w, gamma, T_, k, L, eps, nn); break;
    case 2: hipLaunchKernelGGL((combine_norm_lean_kernel<T, 2, R>), grid, block, 0, s, yy, sp, w, gamma, T_, k, L, eps, nn); break;
    case 3: hipLaunchKernelGGL((combine_norm_lean_kernel<T, 3, R>), grid, block, 0, s, yy, sp, w, gamma, T_, k, L, eps, nn); break;
    case 4: hipLaunchKernelGGL((combine_norm_lean_kernel<T, 4, R>), grid, block, 0, s, yy, sp, w, gamma, T_, k, L, eps, nn); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_norm(const void* y, const int32_t* slot_of_pair, const float* w, const float* gamma, int T,
                               int k, int L, float eps, int dtype, void* n_out, hipStream_t s) {
  KernelTimer timer("combine_norm", s);
  // The four-wave form whenever a row fits four chunks per lane (L <= 8192 bf16, 4096 f32); it times
  // the same as one wave per token when it runs alone (k3_prefill: 0.191 vs 0.192 ms).
  const int vec = dtype == LMOE_BF16 ? 8 : 4;
  if (ceil_div(L / vec, 256) <= 4) {
    if (dtype == LMOE_BF16) return launch_lean<uint16_t, 4>(y, slot_of_pair, w, gamma, T, k, L, eps, n_out, s);
    return launch_lean<float, 4>(y, slot_of_pair, w, gamma, T, k, L, eps, n_out, s);
  }
  if (dtype == LMOE_BF16) return launch_t<uint16_t>(y, slot_of_pair, w, gamma, T, k, L, eps, n_out, s);
  return launch_t<float>(y, slot_of_pair, w, gamma, T, k, L, eps, n_out, s);
}

}  // namespace lmoe
