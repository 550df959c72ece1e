// Routing and quantile balancing kernels: router-weight split, biased top-k, QB histogram, QB
// bias update. All integer results (indices, bins, counts) are exact and order-independent.
#include <math.h>

#include <mutex>

#include "common.h"

namespace lmoe {
namespace {

// ------------------------------------------------------------------------------------------------
// Router weight split for exact products on bf16 MFMA: w = hi + mid + lo, each bf16, every
// remainder exact in f32 (the error of rounding to a narrower format is representable in the
// wider one). x (bf16) times a bf16 part has a 16-bit significand, so each product is exact in
// f32 and the router logits accumulate in f32 like an f32 GEMM. Output row e = [hi | mid | lo].
// ------------------------------------------------------------------------------------------------
__device__ inline void split3(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(hi);
  mid = f32_to_bf16(r1);
  lo = f32_to_bf16(r1 - bf16_to_f32(mid));
}

// Eight consecutive weights per thread: two 16-byte loads, one 16-byte store per part (cols a
// multiple of 8, both matrices 16-byte aligned).
__global__ void split3_vec_kernel(const float* __restrict__ w, uint16_t* __restrict__ out, int rows, int cols) {
  const int64_t n8 = (int64_t)rows * cols / 8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i * 8 / cols, c = i * 8 % cols;
    const float4 a = reinterpret_cast<const float4*>(w)[2 * i], b = reinterpret_cast<const float4*>(w)[2 * i + 1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint16_t h[8], m[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) split3(v[j], h[j], m[j], l[j]);
    uint16_t* o = out + r * 3 * cols + c;
    *reinterpret_cast<uint4*>(o) = *reinterpret_cast<const uint4*>(h);
    *reinterpret_cast<uint4*>(o + cols) = *reinterpret_cast<const uint4*>(m);
    *reinterpret_cast<uint4*>(o + 2 * (int64_t)cols) = *reinterpret_cast<const uint4*>(l);
  }
}

__global__ void split3_kernel(const float* __restrict__ w, uint16_t* __restrict__ out, int rows, int cols) {
  const int64_t n = (int64_t)rows * cols;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, c = i % cols;
    uint16_t hi, mid, lo;
    split3(w[i], hi, mid, lo);
    uint16_t* o = out + r * 3 * cols + c;
    o[0] = hi;
    o[cols] = mid;
    o[2 * (int64_t)cols] = lo;
  }
}

// ------------------------------------------------------------------------------------------------
// Biased top-k, one wave per token row ([vxz] 02 selection bias; order: descending s + b, equal
// values to the lower expert index). Lane l holds experts l, l+64, ... in registers as
// order-preserving integer keys.
//
// Candidate pass: the (k+1)-th largest of the 64 lane maxima is a lower bound t0 of the (k+1)-th
// largest key (k+1 distinct keys, one per lane, reach it), so the k+1 winners are among the keys
// >= t0. For scores without mass ties these are a few dozen; when at most 64 they are compacted
// one per lane through LDS and each one's place in the order is counted directly against the
// others (keys compared, then indices). Radix select on the lane maxima costs one compare per bit
// instead of one per key.
//
// Exact pass (more than 64 candidates, e.g. many equal scores): the (k+1)-th largest key K is found
// MSB-first, one bit per step, from wave-wide counts (ballots: no cross-lane data movement); the
// selection is every key above K plus the keys equal to K with the lowest indices; each selected
// element's place in the order is the count of selected elements ahead of it.
//
// Either way the winners meet in LDS so that lane r holds the r-th, and the routing weights are
// normalised by a fixed-order tree over lanes 0..k-1.
//
// PART: the scores are first made from the router GEMM's split-K partial logits (summed in split
// order, plus the logit offset, then the sigmoid: the reduction's own arithmetic), stored, and
// selected from the same registers.
// ------------------------------------------------------------------------------------------------
__device__ inline uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0;  // -0 and +0 compare equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

template <int NPL, bool PART>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ scores, const float* __restrict__ part,
                                                   int splits, const float* __restrict__ offset,
                                                   float* __restrict__ scores_out, const float* __restrict__ bias,
                                                   int T, int E, int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ w, float* __restrict__ thresh) {
  __shared__ int win_e[4][65];  // ranks 0..k, k <= 64
  __shared__ uint32_t win_key[4][65];
  __shared__ float win_s[4][65];
  __shared__ int cand_e[4][65];  // candidates of the candidate pass (<= 64) or the k+1 winners of the exact pass
  __shared__ uint32_t cand_key[4][65];
  __shared__ float cand_s[4][65];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wv;
  if (t >= T) return;  // the whole wave leaves together
  uint32_t key[NPL];
  float sv[NPL];  // the unbiased scores, for the routing weights
  uint32_t present = 0;
  if constexpr (PART) {  // split by split, all of the lane's loads of one split in flight together
#pragma unroll
    for (int i = 0; i < NPL; ++i) sv[i] = 0.0f;
    for (int sp = 0; sp < splits; ++sp) {
      const float* prow = part + ((int64_t)sp * T + t) * E;
      float pv[NPL];
#pragma unroll
      for (int i = 0; i < NPL; ++i) pv[i] = lane + 64 * i < E ? prow[lane + 64 * i] : 0.0f;
#pragma unroll
      for (int i = 0; i < NPL; ++i) sv[i] += pv[i];
    }
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = 0;
    if (e < E) {
      float sc;
      if constexpr (PART) {
        const float x = sv[i] + (offset ? offset[e] : 0.0f);
        sc = 1.0f / (1.0f + expf(-x));
        scores_out[t * E + e] = sc;
      } else {
        sc = scores[t * E + e];
      }
      sv[i] = sc;
      key[i] = order_key(sc + bias[e]);
      present |= 1u << i;
    } else {
      sv[i] = 0.0f;
    }
  }
  const int kk = k + 1;
  const uint64_t lower_lanes = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  // Wave-wide sum of per-lane counts (each below 2^CB): the lane counts are summed bit-slice by
  // bit-slice with ballots, log2(NPL) + 1 scalar popcounts rather than NPL.
  constexpr int CB = NPL <= 2 ? 2 : NPL <= 4 ? 3 : NPL <= 8 ? 4 : NPL <= 16 ? 5 : 6;
  auto wave_sum = [&](int own) __attribute__((always_inline)) {
    int total = 0;
#pragma unroll
    for (int b = 0; b < CB; ++b) total += __popcll(__ballot((own >> b) & 1)) << b;
    return total;
  };
  auto count_ge = [&](uint32_t c) __attribute__((always_inline)) {
    int own = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) own += (((present >> i) & 1u) && key[i] >= c) ? 1 : 0;
    return wave_sum(own);
  };

  // candidate pass
  uint32_t lmax = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i)
    if ((present >> i) & 1u) lmax = key[i] > lmax ? key[i] : lmax;
  const bool voter = present != 0;
  uint32_t t0 = 0;  // the kk-th largest lane maximum (0 when fewer than kk lanes hold experts)
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = t0 | (1u << b);
    if (__popcll(__ballot(voter && lmax >= cand)) >= kk) t0 = cand;
  }
  int own = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) own += (((present >> i) & 1u) && key[i] >= t0) ? 1 : 0;
  const int n_cand = wave_sum(own);
  if (n_cand <= 64) {
    int pos = 0;  // exclusive prefix of the lane counts
#pragma unroll
    for (int b = 0; b < CB; ++b) pos += __popcll(__ballot((own >> b) & 1) & lower_lanes) << b;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (((present >> i) & 1u) && key[i] >= t0) {
        cand_key[wv][pos] = key[i];
        cand_e[wv][pos] = lane + 64 * i;
        cand_s[wv][pos] = sv[i];
        ++pos;
      }
    __builtin_amdgcn_wave_barrier();  // a wave's LDS accesses complete in issue order
    const bool have = lane < n_cand;
    const uint32_t ck = have ? cand_key[wv][lane] : 0u;
    const int ce = have ? cand_e[wv][lane] : 0;
    const float cs = have ? cand_s[wv][lane] : 0.0f;
    int place = 0;
    for (int j = 0; j < n_cand; ++j) {
      const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)ck, j);
      const int ej = __builtin_amdgcn_readlane(ce, j);
      place += (kj > ck || (kj == ck && ej < ce)) ? 1 : 0;
    }
    if (have && place < kk) {
      win_e[wv][place] = ce;
      win_key[wv][place] = ck;
      win_s[wv][place] = cs;
    }
  } else {
    // exact pass
    uint32_t kth = 0;  // the largest key with at least kk keys >= it: the kk-th largest
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = kth | (1u << b);
      if (count_ge(cand) >= kk) kth = cand;
    }
    const int above = kth == 0xffffffffu ? 0 : count_ge(kth + 1);
    const int need_eq = kk - above;  // >= 1 keys equal to kth, lowest indices first (index = lane + 64 i)
    uint32_t sel = 0;
    int eq_before = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const bool p = (present >> i) & 1u;
      const bool eq = p && key[i] == kth;
      const uint64_t m = __ballot(eq);
      if ((p && key[i] > kth) || (eq && eq_before + __popcll(m & lower_lanes) < need_eq)) sel |= 1u << i;
      eq_before += __popcll(m);
    }
    // The kk winners go to LDS in lane order, then each is ranked against all of them (key, then
    // index): one LDS pass instead of a rank counter per key in registers, which keeps the kernel's
    // registers at the candidate pass's count (eight waves per SIMD).
    int own_sel = __popc(sel);
    int pos = 0;
#pragma unroll
    for (int b = 0; b < CB; ++b) pos += __popcll(__ballot((own_sel >> b) & 1) & lower_lanes) << b;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if ((sel >> i) & 1u) {
        cand_key[wv][pos] = key[i];
        cand_e[wv][pos] = lane + 64 * i;
        cand_s[wv][pos] = sv[i];
        ++pos;
      }
    __builtin_amdgcn_wave_barrier();  // a wave's LDS accesses complete in issue order
    for (int c = lane; c < kk; c += 64) {
      const uint32_t ck = cand_key[wv][c];
      const int ce = cand_e[wv][c];
      const float cs = cand_s[wv][c];
      int place = 0;
      for (int j = 0; j < kk; ++j) {
        const uint32_t kj = cand_key[wv][j];
        const int ej = cand_e[wv][j];
        place += (kj > ck || (kj == ck && ej < ce)) ? 1 : 0;
      }
      win_e[wv][place] = ce;
      win_key[wv][place] = ck;
      win_s[wv][place] = cs;
    }
  }
  __builtin_amdgcn_wave_barrier();
  const int my_idx = lane < k ? win_e[wv][lane] : 0;
  const float my_s = lane < k ? win_s[wv][lane] : 0.0f;
  float sum = my_s;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d);
  if (lane < k) {
    idx[t * k + lane] = my_idx;
    w[t * k + lane] = my_s / sum;
  }
  if (lane == 0) {
    thresh[2 * t] = key_value(win_key[wv][k - 1]);
    thresh[2 * t + 1] = key_value(win_key[wv][k]);
  }
}

// ------------------------------------------------------------------------------------------------
// QB histogram ([tahou] 负载均衡优化: map to 0..1 and bin). A workgroup owns a slice of EB
// experts for every token: its [EB, NB] counters live in LDS and are added to the caller's
// histogram with plain read-add-writes (no other workgroup touches those bins), so the result is
// exact and independent of scheduling. Lane l of a wave takes expert e0 + l % EB of token
// sub-row l / EB, so one load instruction reads 64 / EB tokens' slices as runs of 4 EB contiguous
// bytes (a run per cache line, where a lane per token would touch a line per lane). The kernel is
// bound by loads in flight (each workgroup walks all T rows), so every lane issues U = 16 tokens'
// loads before it uses any, and the slice width leaves at least 192 workgroups. The row's k-th
// expert index only breaks exact ties with v_k and is loaded only then. Slices are numbered so
// that the slices on one XCD (workgroup w runs on XCD w % 8) are contiguous experts, and the score
// lines they share are fetched into that XCD's L2 once.
// Selection of e by t is decided from the row's k-th value v_k and the k-th expert index e_k (the
// order is value desc, index asc): e is selected iff s_hat > v_k, or s_hat == v_k and e <= e_k.
// ------------------------------------------------------------------------------------------------
constexpr int kHistThreads = 1024;
constexpr int kHistLdsBytes = 128 * 1024;
constexpr int kHistUnroll = 16;

__device__ inline int xcd_contiguous(int w, int n) {  // bijection on [0, n): XCD x gets a contiguous run
  const int x = w % kXcds, m = w / kXcds, q = n / kXcds, r = n % kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + m;
}

template <int EB>
__global__ void __launch_bounds__(kHistThreads)
    qb_hist_kernel(const float* __restrict__ scores, const float* __restrict__ bias, const int32_t* __restrict__ idx,
                   const float* __restrict__ thresh, int T, int E, int k, int nb, uint32_t* __restrict__ hist) {
  extern __shared__ uint32_t cnt[];  // [EB][nb]
  constexpr int TPW = kWave / EB;                      // tokens per wave per load
  constexpr int TPB = TPW * (kHistThreads / kWave);    // tokens per workgroup per load
  const int e0 = xcd_contiguous(blockIdx.x, gridDim.x) * EB;
  for (int i = threadIdx.x; i < EB * nb; i += kHistThreads) cnt[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane % EB;
  const int e = e0 + j;
  const bool has_e = e < E;
  const float be = has_e ? bias[e] : 0.0f;
  const float fnb = (float)nb;
  const int t_lane = wave * TPW + lane / EB;
  for (int tb = 0; tb < T; tb += TPB * kHistUnroll) {
    float s[kHistUnroll], vk[kHistUnroll], vk1[kHistUnroll];
#pragma unroll
    for (int u = 0; u < kHistUnroll; ++u) {
      const int t = tb + u * TPB + t_lane;
      const int64_t tc = t < T ? t : 0;
      s[u] = has_e ? scores[tc * E + e] : 0.0f;
      vk[u] = thresh[2 * tc];
      vk1[u] = thresh[2 * tc + 1];
    }
#pragma unroll
    for (int u = 0; u < kHistUnroll; ++u) {
      const int t = tb + u * TPB + t_lane;
      if (!has_e || t >= T) continue;
      const float sh = __fadd_rn(s[u], be);
      bool sel = sh > vk[u];
      if (sh == vk[u]) sel = e <= idx[(int64_t)t * k + k - 1];
      const float m = __fsub_rn(sh, sel ? vk1[u] : vk[u]);
      float uu = __fmul_rn(__fadd_rn(m, 1.0f), 0.5f);
      uu = fminf(fmaxf(uu, 0.0f), 1.0f);
      const int b = min(nb - 1, (int)floorf(__fmul_rn(uu, fnb)));
      atomicAdd(&cnt[j * nb + b], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < EB * nb; i += kHistThreads) {
    const uint32_t c = cnt[i];
    const int ee = e0 + i / nb;
    if (c != 0 && ee < E) hist[(int64_t)ee * nb + i % nb] += c;
  }
}

// ------------------------------------------------------------------------------------------------
// QB bias update, one wave per expert ([vxz] 02; [slm] Quantile Balancing). Lane l sums bins
// [l*bpl, (l+1)*bpl); a wave scan gives each lane its cumulative base; the one lane whose range
// crosses c* walks its bins to j*, interpolates in f64 and moves the bias; then the row is zeroed.
// ------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) qb_update_kernel(uint32_t* __restrict__ hist, int E, int k, int nb,
                                                        int64_t n_acc, float* __restrict__ bias, bool al16) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  uint32_t* h = hist + (int64_t)e * nb;
  const int bpl = (nb + 63) / 64;
  const int j0 = min(nb, lane * bpl), j1 = min(nb, j0 + bpl);
  // the lane's bins are read once, 16 at a time (all loads in flight together), and kept for the
  // walk to j*
  constexpr int R = 16;
  uint32_t hv[R];
  uint64_t lsum = 0;
  const bool cached = j1 - j0 <= R;
  // whole 16-byte groups when every lane's run starts on 16 bytes (nb = 1000: 4 loads of 4 bins
  // instead of 16 of one); a lane's run is then a whole number of groups
  const bool vec = al16 && bpl <= R && bpl % 4 == 0 && nb % 4 == 0;
  if (vec) {
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      const uint4 v = j0 + 4 * q < j1 ? *reinterpret_cast<const uint4*>(h + j0 + 4 * q) : make_uint4(0, 0, 0, 0);
      hv[4 * q] = v.x;
      hv[4 * q + 1] = v.y;
      hv[4 * q + 2] = v.z;
      hv[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) hv[i] = (cached && j0 + i < j1) ? h[j0 + i] : 0u;
  }
  if (cached) {
#pragma unroll
    for (int i = 0; i < R; ++i) lsum += hv[i];
  } else {
    for (int j = j0; j < j1; ++j) lsum += h[j];
  }
  uint64_t incl = lsum;  // inclusive wave scan
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  const uint64_t base = incl - lsum;
  if (n_acc > 0) {
    const double c_star = (double)((int64_t)(E - k) * n_acc) / (double)E;
    if ((double)base < c_star && (double)incl >= c_star) {
      uint64_t cum = base;
      bool done = false;
      // bin j holds hj counts: the first bin whose cumulative count reaches c* is j*
      auto visit = [&](int j, uint64_t hj) __attribute__((always_inline)) {
        if (done) return;
        if ((double)(cum + hj) >= c_star) {
          const double frac = (c_star - (double)cum) / (double)hj;
          const double u_hat = ((double)j + frac) / (double)nb;
          const double m_hat = 2.0 * u_hat - 1.0;
          bias[e] = (float)((double)bias[e] - m_hat);
          done = true;
        }
        cum += hj;
      };
      if (cached) {
#pragma unroll
        for (int i = 0; i < R; ++i)
          if (j0 + i < j1) visit(j0 + i, hv[i]);
      } else {
        for (int j = j0; j < j1 && !done; ++j) visit(j, h[j]);
      }
    }
  }
  if (vec) {
#pragma unroll
    for (int q = 0; q < R / 4; ++q)
      if (j0 + 4 * q < j1) *reinterpret_cast<uint4*>(h + j0 + 4 * q) = make_uint4(0, 0, 0, 0);
  } else {
    for (int j = j0; j < j1; ++j) h[j] = 0;
  }
}

template <int NPL, bool PART>
void launch_topk_t(const float* s, const float* part, int splits, const float* off, float* s_out, const float* b, int T,
                   int E, int k, int32_t* idx, float* w, float* th, hipStream_t st) {
  hipLaunchKernelGGL((topk_kernel<NPL, PART>), dim3((unsigned)ceil_div(T, 4)), dim3(256), 0, st, s, part, splits, off,
                     s_out, b, T, E, k, idx, w, th);
}

template <bool PART>
hipError_t launch_topk_any(const float* s, const float* part, int splits, const float* off, float* s_out,
                           const float* b, int T, int E, int k, int32_t* idx, float* w, float* th, hipStream_t st) {
  const int npl = (int)ceil_div(E, 64);
  if (npl <= 2) launch_topk_t<2, PART>(s, part, splits, off, s_out, b, T, E, k, idx, w, th, st);
  else if (npl <= 4) launch_topk_t<4, PART>(s, part, splits, off, s_out, b, T, E, k, idx, w, th, st);
  else if (npl <= 8) launch_topk_t<8, PART>(s, part, splits, off, s_out, b, T, E, k, idx, w, th, st);
  else if (npl <= 16) launch_topk_t<16, PART>(s, part, splits, off, s_out, b, T, E, k, idx, w, th, st);
  else if (npl <= 32) launch_topk_t<32, PART>(s, part, splits, off, s_out, b, T, E, k, idx, w, th, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split3(const float* w, uint16_t* out, int rows, int cols, hipStream_t s) {
  KernelTimer timer("router_split", s);
  const int64_t n = (int64_t)rows * cols;
  if (cols % 8 == 0 && reinterpret_cast<uintptr_t>(w) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0) {
    const unsigned blocks = (unsigned)hmin(ceil_div(n / 8, 256), 8192);
    hipLaunchKernelGGL(split3_vec_kernel, dim3(blocks), dim3(256), 0, s, w, out, rows, cols);
    return hipGetLastError();
  }
  const unsigned blocks = (unsigned)hmin(ceil_div(n, 256), 8192);
  hipLaunchKernelGGL(split3_kernel, dim3(blocks), dim3(256), 0, s, w, out, rows, cols);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, const float* bias, int T, int E, int k, int32_t* idx, float* w,
                       float* thresh, hipStream_t s) {
  KernelTimer timer("route_topk", s);
  return launch_topk_any<false>(scores, nullptr, 0, nullptr, nullptr, bias, T, E, k, idx, w, thresh, s);
}

hipError_t launch_topk_partials(const float* partials, int splits, const float* logit_offset, float* scores,
                                const float* bias, int T, int E, int k, int32_t* idx, float* w, float* thresh,
                                hipStream_t s) {
  KernelTimer timer("route_topk", s);
  return launch_topk_any<true>(nullptr, partials, splits, logit_offset, scores, bias, T, E, k, idx, w, thresh, s);
}

template <int EB>
hipError_t launch_qb_hist_t(const float* scores, const float* bias, const int32_t* idx, const float* thresh, int T,
                            int E, int k, int nb, uint32_t* hist, hipStream_t s) {
  // the LDS limit is a property of the function: set once per process (thread-safe), before any
  // launch, so the launch itself is all a graph capture records
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute((const void*)qb_hist_kernel<EB>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               kHistLdsBytes);
  });
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((qb_hist_kernel<EB>), dim3((unsigned)ceil_div(E, EB)), dim3(kHistThreads), (size_t)EB * nb * 4,
                     s, scores, bias, idx, thresh, T, E, k, nb, hist);
  return hipGetLastError();
}

hipError_t launch_qb_hist(const float* scores, const float* bias, const int32_t* idx, const float* thresh, int T,
                          int E, int k, int nb, uint32_t* hist, hipStream_t s) {
  KernelTimer timer("qb_hist", s);
  // experts per workgroup: the most that still give 192 workgroups, within the LDS budget
  auto ok = [&](int eb) { return (int64_t)eb * nb * 4 <= kHistLdsBytes && ceil_div(E, eb) >= 192; };
  const int eb = ok(8) ? 8 : ok(4) ? 4 : ok(2) ? 2 : 1;
  if ((int64_t)eb * nb * 4 > kHistLdsBytes) return hipErrorInvalidValue;
  if (eb == 8) return launch_qb_hist_t<8>(scores, bias, idx, thresh, T, E, k, nb, hist, s);
  if (eb == 4) return launch_qb_hist_t<4>(scores, bias, idx, thresh, T, E, k, nb, hist, s);
  if (eb == 2) return launch_qb_hist_t<2>(scores, bias, idx, thresh, T, E, k, nb, hist, s);
  return launch_qb_hist_t<1>(scores, bias, idx, thresh, T, E, k, nb, hist, s);
}

hipError_t launch_qb_update(uint32_t* hist, int E, int k, int nb, int64_t n_acc, float* bias, hipStream_t s) {
  KernelTimer timer("qb_update", s);
  const bool al16 = reinterpret_cast<uintptr_t>(hist) % 16 == 0;
  hipLaunchKernelGGL(qb_update_kernel, dim3((unsigned)ceil_div(E, 4)), dim3(256), 0, s, hist, E, k, nb, n_acc, bias,
                     al16);
  return hipGetLastError();
}

}  // namespace lmoe
