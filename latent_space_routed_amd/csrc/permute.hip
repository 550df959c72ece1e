// Dispatch of (token, slot) pairs to experts: a stable counting sort by expert computed on the
// device (no host synchronisation, static shapes: [slm] 训练基础设施), then a gather of latent rows.
//
//   count   : per 256-token chunk, how many of its tokens chose each expert      -> cc[chunk][e]
//             (the chunk's 64-token blocks mark their tokens' experts in an LDS bitmask per
//             expert, four lanes per token; the count is the masks' popcount, so a token that lists
//             an expert twice counts once)
//   scan    : exclusive prefix over chunks (in place) and over experts          -> offsets[E+1]
//   scatter : per chunk, one lane per token marks the masks in pair order (a pair whose bit is
//             already set repeats an expert and is dropped) and leaves each pair's expert in LDS;
//             then four lanes per token rank and store: the rank of token t inside expert e is
//             offsets[e] + cc[chunk][e] + (tokens of earlier 64-token blocks) + popcount(mask_e &
//             lanes below t). Tokens therefore ascend inside an expert.
//   gather  : one wave per token loads its latent row once and writes it to its k sorted rows.
// An expert index outside [0, E), or one that a token lists a second time, drops the pair: its slot is
// -1, it takes no sorted row, and later kernels skip it. expert_offsets[E] is then the number of
// pairs kept.
#include <mutex>

#include "common.h"

namespace lmoe {
namespace {

constexpr int kMaxExpertsLds = 2048;  // the library's largest expert count
constexpr int kMaxTopKLds = 64;       // and its largest k

constexpr int kPermLanes = 4;                           // lanes per token in the count and the ranking
constexpr int kPermThreads = kPermChunk * kPermLanes;  // threads of a count or scatter workgroup

__global__ void __launch_bounds__(kPermThreads) perm_count_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                                   int32_t* __restrict__ cc) {
  extern __shared__ unsigned long long marks[];  // [4][E]: bit l of marks[b][e] = token 64 b + l chose e
  constexpr int W = kPermChunk / 64;
  for (int i = threadIdx.x; i < W * E; i += kPermThreads) marks[i] = 0ull;
  __syncthreads();
  // lane group g takes pairs g, g + 4, ... of token ti (a wave holds 64 consecutive tokens)
  const int ti = threadIdx.x % kPermChunk, g = threadIdx.x / kPermChunk;
  const int lane = ti & 63, tb = ti >> 6;
  const int64_t t = (int64_t)blockIdx.x * kPermChunk + ti;
  if (t < T) {
    for (int j = g; j < k; j += kPermLanes) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E) atomicOr(&marks[tb * E + e], 1ull << lane);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) n += __popcll(marks[w * E + e]);
    cc[(int64_t)blockIdx.x * E + e] = n;
  }
}

__global__ void __launch_bounds__(1024) perm_scan_kernel(int32_t* __restrict__ cc, int chunks, int E,
                                                          int32_t* __restrict__ offsets) {
  extern __shared__ int32_t tot[];  // [E]
  __shared__ int32_t wsum[16];
  constexpr int B = 16;  // chunk counts loaded together, so that their latencies overlap
  for (int e = threadIdx.x; e < E; e += 1024) {
    int32_t run = 0;
    for (int c0 = 0; c0 < chunks; c0 += B) {
      int32_t v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) v[i] = c0 + i < chunks ? cc[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < B; ++i) {
        if (c0 + i < chunks) cc[(int64_t)(c0 + i) * E + e] = run;
        run += v[i];
      }
    }
    tot[e] = run;
  }
  __syncthreads();
  // exclusive scan of tot over experts: thread i owns a contiguous run of `per` experts
  const int per = (E + 1023) / 1024;
  const int e0 = min(E, threadIdx.x * per), e1 = min(E, e0 + per);
  int32_t local = 0;
  for (int e = e0; e < e1; ++e) local += tot[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int32_t wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += wsum[w];
  int32_t run = wbase + incl - local;
  for (int e = e0; e < e1; ++e) {
    const int32_t v = tot[e];
    offsets[e] = run;
    run += v;
  }
  if (threadIdx.x == 1023) offsets[E] = run;
}

__global__ void __launch_bounds__(kPermThreads) perm_scatter_kernel(const int32_t* __restrict__ idx, int T, int E,
                                                                     int k, const int32_t* __restrict__ cc,
                                                                     const int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ sorted_token,
                                                                     int32_t* __restrict__ slot_of_pair) {
  // [4][E] masks, then [E] i32 bases of this chunk, then [256][k] i32: each pair's expert, -1 if dropped
  extern __shared__ unsigned long long bits[];
  constexpr int W = kPermChunk / 64;
  int32_t* base_e = reinterpret_cast<int32_t*>(bits + W * E);
  int32_t* pair_e = base_e + E;
  for (int i = threadIdx.x; i < W * E; i += kPermThreads) bits[i] = 0ull;
  // the chunk's first slot in every expert, read once with coalesced loads
  for (int e = threadIdx.x; e < E; e += kPermThreads) base_e[e] = offsets[e] + cc[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  if (threadIdx.x < kPermChunk) {
    // One lane per token sets the token's bits in pair order, so a pair whose bit is already set
    // repeats an earlier pair's expert and is dropped. The pairs' expert indices are loaded KB at a
    // time, so that a pair's loads do not wait on the previous pair's atomics.
    const int lane = threadIdx.x & 63, tb = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * kPermChunk + threadIdx.x;
    const bool live = t < T;
    constexpr int KB = 8;
    for (int j0 = 0; j0 < k; j0 += KB) {
      int e[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) e[i] = (live && j0 + i < k) ? idx[t * k + j0 + i] : -1;
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        if (j0 + i >= k) break;
        int v = -1;
        if (e[i] >= 0 && e[i] < E && !(atomicOr(&bits[tb * E + e[i]], 1ull << lane) >> lane & 1ull)) v = e[i];
        pair_e[threadIdx.x * k + j0 + i] = v;
      }
    }
  }
  __syncthreads();
  // four lanes per token rank and store its pairs (lane group g: pairs g, g + 4, ...)
  const int ti = threadIdx.x % kPermChunk, g = threadIdx.x / kPermChunk;
  const int lane = ti & 63, tb = ti >> 6;
  const int64_t t = (int64_t)blockIdx.x * kPermChunk + ti;
  if (t >= T) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int j = g; j < k; j += kPermLanes) {
    const int e = pair_e[ti * k + j];
    int32_t slot = -1;
    if (e >= 0) {
      int r = base_e[e];
      for (int b = 0; b < tb; ++b) r += __popcll(bits[b * E + e]);
      r += __popcll(bits[tb * E + e] & below);
      slot = r;
      sorted_token[r] = (int32_t)t;
    }
    slot_of_pair[t * k + j] = slot;
  }
}

// One wave per token: 16-byte chunks of the row are loaded once and stored to each sorted row.
__global__ void __launch_bounds__(256) gather_rows_kernel(const char* __restrict__ x_lat,
                                                          const int32_t* __restrict__ slot_of_pair, int T, int k,
                                                          int64_t row_bytes, char* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t chunks = row_bytes / 16;
  const char* src = x_lat + t * row_bytes;
  for (int64_t c = lane; c < chunks; c += 64) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + c * 16);
    for (int j = 0; j < k; ++j) {
      const int32_t slot = slot_of_pair[t * k + j];
      if (slot >= 0) *reinterpret_cast<uint4*>(x_perm + (int64_t)slot * row_bytes + c * 16) = v;
    }
  }
}

// Shared-expert repack: gates of all experts, then their up rows; down blocks side by side.
__global__ void pack_w1_kernel(const char* __restrict__ w1s, char* __restrict__ w1p, int S, int Is, int64_t row_bytes) {
  const int64_t chunks = row_bytes / 16;
  const int64_t n = (int64_t)S * 2 * Is * chunks;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t src_row = i / chunks, c = i % chunks;
    const int64_t j = src_row / (2 * Is), r = src_row % (2 * Is);
    const int64_t dst_row = r < Is ? j * Is + r : (int64_t)S * Is + j * Is + (r - Is);
    *reinterpret_cast<uint4*>(w1p + dst_row * row_bytes + c * 16) =
        *reinterpret_cast<const uint4*>(w1s + src_row * row_bytes + c * 16);
  }
}

__global__ void pack_w2_kernel(const char* __restrict__ w2s, char* __restrict__ w2p, int S, int D, int64_t blk_bytes) {
  // w2s [S][D][Is] -> w2p [D][S*Is]; blk_bytes = Is * esz
  const int64_t chunks = blk_bytes / 16;
  const int64_t n = (int64_t)S * D * chunks;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = i % chunks, d = (i / chunks) % D, j = i / (chunks * D);
    *reinterpret_cast<uint4*>(w2p + d * S * blk_bytes + j * blk_bytes + c * 16) =
        *reinterpret_cast<const uint4*>(w2s + (j * D + d) * blk_bytes + c * 16);
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)hmin(1024, ceil_div(n, 256))), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int T, int E, int k, int32_t* offsets, int32_t* sorted_token,
                          int32_t* slot_of_pair, int32_t* cc, hipStream_t s) {
  const int chunks = (int)ceil_div(T, kPermChunk);
  {
    KernelTimer timer("perm_count", s);
    static std::once_flag once;  // the masks pass the default 64 KB of dynamic LDS at the largest expert counts
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
      attr = hipFuncSetAttribute((const void*)perm_count_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 kMaxExpertsLds * 8 * (kPermChunk / 64));
    });
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(perm_count_kernel, dim3(chunks), dim3(kPermThreads), (size_t)E * 8 * (kPermChunk / 64), s,
                       idx, T, E, k, cc);
  }
  {
    KernelTimer timer("perm_scan", s);
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), (size_t)E * 4, s, cc, chunks, E, offsets);
  }
  {
    KernelTimer timer("perm_scatter", s);
    // the masks, bases and pair experts pass the default 64 KB of dynamic LDS at the largest expert
    // counts and k
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
      attr = hipFuncSetAttribute((const void*)perm_scatter_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 kMaxExpertsLds * (8 * (kPermChunk / 64) + 4) + kPermChunk * kMaxTopKLds * 4);
    });
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(chunks), dim3(kPermThreads),
                       (size_t)E * (8 * (kPermChunk / 64) + 4) + (size_t)kPermChunk * k * 4, s, idx, T, E, k, cc,
                       offsets, sorted_token, slot_of_pair);
  }
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x_lat, const int32_t* slot_of_pair, int T, int k, int64_t row_bytes,
                              void* x_perm, hipStream_t s) {
  KernelTimer timer("gather_rows", s);
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)ceil_div(T, 4)), dim3(256), 0, s,
                     static_cast<const char*>(x_lat), slot_of_pair, T, k, row_bytes, static_cast<char*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_pack_shared(const void* w1s, const void* w2s, int S, int Is, int D, int esz, void* w1p, void* w2p,
                              hipStream_t s) {
  KernelTimer timer("pack_shared", s);
  hipLaunchKernelGGL(pack_w1_kernel, dim3(2048), dim3(256), 0, s, static_cast<const char*>(w1s),
                     static_cast<char*>(w1p), S, Is, (int64_t)D * esz);
  hipLaunchKernelGGL(pack_w2_kernel, dim3(2048), dim3(256), 0, s, static_cast<const char*>(w2s),
                     static_cast<char*>(w2p), S, D, (int64_t)Is * esz);
  return hipGetLastError();
}

}  // namespace lmoe
