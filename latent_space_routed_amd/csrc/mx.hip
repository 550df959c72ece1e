// MX quantisation (MXFP4 weights, MXFP8 activations) of the routed experts ([slm] 训练基础设施:
// MXFP4 weights with MXFP8 activations). Formats: OCP Microscaling — blocks of 32 elements along
// the contraction dimension share an E8M0 scale 2^(e - 127); elements are E2M1 (FP4) or E4M3
// (FP8). The shared exponent is floor(log2(block max)) - emax (emax 2 for E2M1, 8 for E4M3),
// clamped to [-127, 127] (an all-zero block takes e = 0); each element is v / 2^se rounded to the
// nearest value, ties to the even significand, saturated at the largest normal (6, 448).
//
// One thread per block: the division by the power of two is exact, and the rounding is done on the
// element's own exponent and significand with rintf (ties to even), so the codes are bit-exact.
#include "common.h"

namespace lmoe {
namespace {

// |x| of an E2M1 / E4M3 element after scaling (a < 2^(emax + 1)) to its magnitude code.
__device__ inline uint32_t fp4_mag_code(float a) {
  if (a >= 6.0f) return 7u;                      // [6, 8): 6, or saturated
  if (a < 1.0f) return (uint32_t)rintf(a * 2.0f);  // subnormal step 0.5: codes 0, 1 (0.5), 2 (1.0)
  int e;
  const float f = frexpf(a, &e);                 // a = f 2^e, f in [0.5, 1): floor(log2 a) = e - 1
  const int ex = e - 1;                          // 0, 1 or 2
  const uint32_t m = (uint32_t)rintf((ldexpf(f, 1) - 1.0f) * 2.0f);  // 0, 1 or 2
  return (uint32_t)((ex + 1) * 2) + m;           // m = 2 carries into the next exponent
}

__device__ inline uint32_t fp8_mag_code(float a) {
  if (a >= 448.0f) return 126u;                   // largest normal, or saturated
  if (a < 0.015625f) return (uint32_t)rintf(a * 512.0f);  // subnormal step 2^-9: codes 0..8
  int e;
  const float f = frexpf(a, &e);
  const int ex = e - 1;                           // -6 .. 8
  const uint32_t m = (uint32_t)rintf((ldexpf(f, 1) - 1.0f) * 8.0f);  // 0..8
  return (uint32_t)((ex + 7) * 8) + m;
}

// The 32 elements of block b (16-byte loads).
template <typename T>
__device__ inline void load_block(const T* p, int64_t b, float (&v)[32]);
template <>
__device__ inline void load_block<uint16_t>(const uint16_t* p, int64_t b, float (&v)[32]) {
  const uint4* q = reinterpret_cast<const uint4*>(p + b * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = q[i];
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(u[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
    }
  }
}
template <>
__device__ inline void load_block<float>(const float* p, int64_t b, float (&v)[32]) {
  const float4* q = reinterpret_cast<const float4*>(p + b * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 w = q[i];
    v[4 * i] = w.x;
    v[4 * i + 1] = w.y;
    v[4 * i + 2] = w.z;
    v[4 * i + 3] = w.w;
  }
}

template <typename T, bool FP4>
__global__ void __launch_bounds__(256) mx_quantize_kernel(const T* __restrict__ x, int64_t nblocks,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  float v[32];
  load_block<T>(x, b, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  constexpr int kEmax = FP4 ? 2 : 8;
  int se = 0;
  uint32_t sbyte = 0;
  if (amax > 0.0f) {
    int e;
    frexpf(amax, &e);
    se = min(127, max(-127, e - 1 - kEmax));
    sbyte = (uint32_t)(se + 127);
  } else {
    se = -127;  // every element is zero: codes 0 whatever the scale
  }
  uint32_t out[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float a = ldexpf(fabsf(v[i]), -se);
    uint32_t c = FP4 ? fp4_mag_code(a) : fp8_mag_code(a);
    if (v[i] < 0.0f && c != 0u) c |= FP4 ? 8u : 128u;
    if constexpr (FP4)
      out[i / 8] |= c << (4 * (i % 8));
    else
      out[i / 4] |= c << (8 * (i % 4));
  }
  if constexpr (FP4) {
    *reinterpret_cast<uint4*>(codes + b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  } else {
    *reinterpret_cast<uint4*>(codes + b * 32) = make_uint4(out[0], out[1], out[2], out[3]);
    *reinterpret_cast<uint4*>(codes + b * 32 + 16) = make_uint4(out[4], out[5], out[6], out[7]);
  }
  scales[b] = (uint8_t)sbyte;
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, int dtype, int64_t nblocks, bool fp4, void* codes, void* scales,
                              hipStream_t s) {
  KernelTimer timer("mx_quantize", s);
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(nblocks, 256)), block(256);
  uint8_t* c = static_cast<uint8_t*>(codes);
  uint8_t* sc = static_cast<uint8_t*>(scales);
  if (dtype == LMOE_BF16) {
    const uint16_t* xx = static_cast<const uint16_t*>(x);
    if (fp4) hipLaunchKernelGGL((mx_quantize_kernel<uint16_t, true>), grid, block, 0, s, xx, nblocks, c, sc);
    else hipLaunchKernelGGL((mx_quantize_kernel<uint16_t, false>), grid, block, 0, s, xx, nblocks, c, sc);
  } else {
    const float* xx = static_cast<const float*>(x);
    if (fp4) hipLaunchKernelGGL((mx_quantize_kernel<float, true>), grid, block, 0, s, xx, nblocks, c, sc);
    else hipLaunchKernelGGL((mx_quantize_kernel<float, false>), grid, block, 0, s, xx, nblocks, c, sc);
  }
  return hipGetLastError();
}

}  // namespace lmoe
