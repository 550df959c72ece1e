// MFMA GEMM for gfx950: C[rows, N] = A[rows, K] . B[N, K]^T with fused epilogues, over one dense
// matrix or ragged row groups (one B per group, rows of a group contiguous in A and C).
//
// Layout and schedule:
//  * A and B are K-contiguous ("[out, in]" weights), so both MFMA operands are read as 16-byte
//    chunks along K. A K-tile is 128 bytes of every row (64 bf16 or 32 f32), staged in LDS with a
//    144-byte row pitch: eight lanes reading 16 bytes of eight consecutive rows then cover all 32
//    banks, which keeps the ds_read_b128 fragment loads conflict-free.
//  * Two LDS stages: global loads of K-tile t+1 are issued into registers before the MFMAs of
//    K-tile t and written to the other stage afterwards, so one barrier per K-tile suffices.
//  * Waves tile the block as WAVES_M x WAVES_N; a wave owns WM row-blocks and WN column-blocks of
//    32x32 (v_mfma_f32_32x32x16_bf16, or four v_mfma_f32_32x32x2f32 for f32 data). Row-blocks are
//    interleaved across the M-waves so a ragged tail spreads evenly, and row-blocks past the end of
//    a group are skipped entirely (no loads, no MFMAs).
//  * The GLU epilogue needs gate column c and up column c in the same lane: a wave's first WN/2
//    column-blocks read gate rows of B and its last WN/2 the matching up rows, so the MFMA result
//    layouts coincide and SiTU-GLU is applied in registers (unfused it costs an extra pass over
//    the 2*inter wide projection, [slm] SiTU 激活).
//  * Tiles are numbered group by group (n-tile major, m-tile minor inside a group) and the
//    numbering is split into 8 contiguous ranges, one per XCD (workgroup i runs on XCD i mod 8):
//    the m-tiles sharing an expert's weight slice, and the n-tiles sharing its rows, run together
//    on one XCD and meet in its L2.
#include <type_traits>

#include "common.h"

namespace lmoe {
namespace {

constexpr int kRowPitch = 144;

template <typename TI>
struct Mfma;

template <>
struct Mfma<uint16_t> {
  __device__ static inline void run(f32x16& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                  0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  // The four k-values of a lane's chunk pair up with the same four k-values of B in the same lane;
  // every k of the 32-byte step is covered once across the two lane halves.
  __device__ static inline void run(f32x16& acc, const uint4& a, const uint4& b) {
    const float4 fa = __builtin_bit_cast(float4, a), fb = __builtin_bit_cast(float4, b);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.x, fb.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.y, fb.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.z, fb.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.w, fb.w, acc, 0, 0, 0);
  }
};

// Raw buffer resource over [base, base + bytes): dword 3 = 0x00020000 is the gfx9-family raw
// buffer format (32-bit data, no swizzle, offset-checked against num_records).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ inline uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline void store_out(const GemmArgs& p, int64_t off, float v) {
  if (p.c_dtype == LMOE_F32)
    static_cast<float*>(p.C)[off] = v;
  else
    static_cast<uint16_t*>(p.C)[off] = f32_to_bf16(v);
}

template <typename TI, int WAVES_M, int WAVES_N, int WM, int WN, Epi EPI>
__global__ void __launch_bounds__(WAVES_M* WAVES_N* kWave) gemm_kernel(GemmArgs p) {
  constexpr int NT = WAVES_M * WAVES_N * kWave;
  constexpr int BM = WAVES_M * WM * 32;
  constexpr int BNB = WAVES_N * WN * 32;  // rows of B per tile
  constexpr bool GLU = EPI == Epi::Glu;
  static_assert(!GLU || WN % 2 == 0, "GLU needs gate/up column-block pairs");
  constexpr int BNO = GLU ? BNB / 2 : BNB;  // output columns per tile
  constexpr int WNO = GLU ? WN / 2 : WN;    // output column-blocks per wave
  constexpr int A_PER = BM * 8 / NT;
  constexpr int B_PER = BNB * 8 / NT;
  static_assert(A_PER * NT == BM * 8 && B_PER * NT == BNB * 8, "chunk split");
  constexpr int A_BYTES = BM * kRowPitch;
  constexpr int STAGE = (BM + BNB) * kRowPitch;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  // ---------------------------------------------------------------- tile assignment
  const bool grouped = p.goff != nullptr;
  const int n_tiles = (int)ceil_div(p.N, BNO);
  const int mt_total = grouped ? p.mtile_start[p.G] : (int)ceil_div(p.M, BM);
  const int total = mt_total * n_tiles;
  const int per = (total + kXcds - 1) / kXcds;
  const int loc = blockIdx.x / kXcds;
  if (loc >= per) return;
  const int lt = (blockIdx.x % kXcds) * per + loc;
  if (lt >= total) return;

  int g = 0, n_tile, row0, rows;
  if (grouped) {
    const int q = lt / n_tiles;
    int lo = 0, hi = p.G;  // mtile_start[lo] <= q < mtile_start[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.mtile_start[mid] <= q) lo = mid; else hi = mid;
    }
    g = lo;
    const int ms0 = p.mtile_start[g];
    const int mtg = p.mtile_start[g + 1] - ms0;
    const int r = lt - n_tiles * ms0;
    n_tile = r / mtg;
    const int m_tile = r % mtg;
    row0 = p.goff[g] + m_tile * BM;
    rows = min(BM, p.goff[g + 1] - row0);
  } else {
    constexpr int GM = 8;  // raster: 8 m-tiles x all n-tiles, m fastest
    const int MT = (int)ceil_div(p.M, BM);
    const int gsz = GM * n_tiles;
    const int grp = lt / gsz, first = grp * GM, gm = min(MT - first, GM), r = lt % gsz;
    n_tile = r / gm;
    row0 = (first + r % gm) * BM;
    rows = min(BM, p.M - row0);
  }
  const int n0 = n_tile * BNO;
  const int act_rb = (rows + 31) >> 5;
  const int act_cb = (min(BNO, p.N - n0) + 31) >> 5;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // ---------------------------------------------------------------- global -> LDS staging
  // Buffer resources span exactly the tile's valid rows of A and of B (one each for the gate and
  // up halves of a GLU tile): a chunk past the end reads as zero in hardware, so ragged row and
  // column tails need neither predication nor clamping. The K offset is the uniform soffset, so
  // a lane's 32-bit voffsets stay fixed for the whole K loop.
  const int64_t a_ld = p.lda * (int64_t)sizeof(TI), b_ld = p.ldb * (int64_t)sizeof(TI);
  const char* Ab = static_cast<const char*>(p.A) + (int64_t)row0 * a_ld;
  const char* Bb = static_cast<const char*>(p.B) + (int64_t)g * p.b_gstride * (int64_t)sizeof(TI);
  const int ncols = min(BNO, p.N - n0);
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(Ab, (int)(rows * a_ld));
  const __amdgpu_buffer_rsrc_t b_rsrc0 = make_rsrc(Bb + (int64_t)n0 * b_ld, (int)(ncols * b_ld));
  const __amdgpu_buffer_rsrc_t b_rsrc1 =
      GLU ? make_rsrc(Bb + (int64_t)(p.glu_up_off + n0) * b_ld, (int)(ncols * b_ld)) : b_rsrc0;
  const int a_wrap = p.a_kwrap * (int)sizeof(TI);
  const int KT = p.K * (int)sizeof(TI) / 128;
  static_assert(!GLU || BNO % (NT / 8) == 0, "a B chunk index must stay in one GLU half");

  int a_voff[A_PER], b_voff[B_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int c = tid + i * NT;
    a_voff[i] = (c >> 3) * (int)a_ld + (c & 7) * 16;
  }
#pragma unroll
  for (int i = 0; i < B_PER; ++i) {
    const int c = tid + i * NT;
    b_voff[i] = ((c >> 3) % BNO) * (int)b_ld + (c & 7) * 16;
  }

  uint4 ra[A_PER], rb[B_PER];
  int ka = 0;  // byte offset of the next K-tile inside A's (possibly wrapped) row
  auto gload = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) ra[i] = buffer_load16(a_rsrc, a_voff[i], ka);
#pragma unroll
    for (int i = 0; i < B_PER; ++i)
      rb[i] = buffer_load16((GLU && (i * NT / 8) >= BNO) ? b_rsrc1 : b_rsrc0, b_voff[i], kt * 128);
    ka += 128;
    if (ka == a_wrap) ka = 0;
  };
  auto lstore = [&](int stage) __attribute__((always_inline)) {
    char* base = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(base + (c >> 3) * kRowPitch + (c & 7) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(base + A_BYTES + (c >> 3) * kRowPitch + (c & 7) * 16) = rb[i];
    }
  };

  // ---------------------------------------------------------------- MFMA main loop
  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // The wave's row-blocks i * WAVES_M + wm that hold rows of the tile form a prefix i < na, so the
  // K loop is instantiated per na, so no branch sits between the LDS reads and the MFMAs. Every
  // column-block is computed; column tails are masked at the store.
  const int na = min(WM, max(0, (act_rb - wm + WAVES_M - 1) / WAVES_M));
  const int frag_off = (lane & 31) * kRowPitch + (lane >> 5) * 16;

  auto main_loop = [&](auto na_c) __attribute__((always_inline)) {
    constexpr int NA = decltype(na_c)::value;
    auto compute = [&](int stage) __attribute__((always_inline)) {
      const char* base = smem + stage * STAGE;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 af[NA > 0 ? NA : 1], bf[WN];
#pragma unroll
        for (int i = 0; i < NA; ++i)
          af[i] = *reinterpret_cast<const uint4*>(base + (i * WAVES_M + wm) * 32 * kRowPitch + frag_off + s * 32);
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const int ocb = (j % WNO) * WAVES_N + wn;
          const int bblk = (GLU && j >= WNO) ? BNO / 32 + ocb : ocb;
          bf[j] = *reinterpret_cast<const uint4*>(base + A_BYTES + bblk * 32 * kRowPitch + frag_off + s * 32);
        }
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j) Mfma<TI>::run(acc[i][j], af[i], bf[j]);
      }
    };
    // K-tile t sits in LDS stage t % 2; one barrier per K-tile.
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) gload(kt + 1);
      if (NA > 0) compute(kt & 1);
      if (kt + 1 < KT) lstore((kt + 1) & 1);
      __syncthreads();
    }
  };
  static_assert(WM <= 4, "main-loop specialisations cover up to four row-blocks per wave");
  switch (na) {
    case 0: main_loop(std::integral_constant<int, 0>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (WM >= 2) main_loop(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (WM >= 3) main_loop(std::integral_constant<int, 3>{}); break;
    default: if constexpr (WM >= 4) main_loop(std::integral_constant<int, 4>{}); break;
  }

  // ---------------------------------------------------------------- epilogue
  const float inv_b1 = 1.0f / p.beta1, inv_b2 = 1.0f / p.beta2;
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int rbk = i * WAVES_M + wm;
    if (rbk >= act_rb) continue;
#pragma unroll
    for (int j = 0; j < WNO; ++j) {
      const int ocb = j * WAVES_N + wn;
      if (ocb >= act_cb) continue;
      const int col = n0 + ocb * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = rbk * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (r >= rows) continue;
        const int64_t grow = row0 + r;
        const int64_t off = grow * p.ldc + col;
        if constexpr (EPI == Epi::Store) {
          store_out(p, off, acc[i][j][q]);
        } else if constexpr (EPI == Epi::Glu) {
          store_out(p, off, situ_glu<sizeof(TI) == 4>(acc[i][j][q], acc[i][j + WNO][q], p.beta1, inv_b1, p.beta2, inv_b2));
        } else if constexpr (EPI == Epi::Sigmoid) {
          const float v = acc[i][j][q] + (p.col_bias ? p.col_bias[col] : 0.0f);
          static_cast<float*>(p.C)[off] = 1.0f / (1.0f + expf(-v));
        } else {
          store_out(p, off, acc[i][j][q] + p.residual[grow * p.ldr + col]);
        }
      }
    }
  }
}

template <typename TI, int WAVES_M, int WAVES_N, int WM, int WN>
hipError_t launch_shape(const GemmArgs& a, Epi epi, hipStream_t s) {
  constexpr int BM = WAVES_M * WM * 32, BNB = WAVES_N * WN * 32;
  const int bno = epi == Epi::Glu ? BNB / 2 : BNB;
  const int64_t n_tiles = ceil_div(a.N, bno);
  const int64_t m_tiles = a.goff ? (int64_t)a.M / BM + a.G : ceil_div(a.M, BM);  // upper bound if grouped
  const int64_t blocks = ceil_div(m_tiles * n_tiles, kXcds) * kXcds;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(WAVES_M * WAVES_N * kWave);
  switch (epi) {
    case Epi::Store: hipLaunchKernelGGL((gemm_kernel<TI, WAVES_M, WAVES_N, WM, WN, Epi::Store>), grid, block, 0, s, a); break;
    case Epi::Glu: hipLaunchKernelGGL((gemm_kernel<TI, WAVES_M, WAVES_N, WM, WN, Epi::Glu>), grid, block, 0, s, a); break;
    case Epi::Sigmoid: hipLaunchKernelGGL((gemm_kernel<TI, WAVES_M, WAVES_N, WM, WN, Epi::Sigmoid>), grid, block, 0, s, a); break;
    case Epi::AddF32: hipLaunchKernelGGL((gemm_kernel<TI, WAVES_M, WAVES_N, WM, WN, Epi::AddF32>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

// Exclusive prefix of ceil(n_g / bm) over groups: m-tile numbering of a grouped GEMM.
__global__ void __launch_bounds__(1024) mtile_prefix_kernel(const int32_t* goff, int G, int bm, int32_t* ms) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < G; base += 1024) {
    const int g = base + threadIdx.x;
    const int v = g < G ? (goff[g + 1] - goff[g] + bm - 1) / bm : 0;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // Hillis-Steele inclusive scan
      const int t = threadIdx.x >= d ? part[threadIdx.x - d] : 0;
      __syncthreads();
      part[threadIdx.x] += t;
      __syncthreads();
    }
    if (g < G) ms[g] = carry + part[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) ms[G] = carry;
}

}  // namespace

int gemm_block_m(GemmShape shape) { return shape == GemmShape::Big ? 256 : 128; }

hipError_t launch_gemm(const GemmArgs& a, int in_dtype, Epi epi, GemmShape shape, hipStream_t s) {
  KernelTimer timer(a.tag ? a.tag : "gemm", s);
  if (in_dtype == LMOE_BF16) {
    if (shape == GemmShape::Big) return launch_shape<uint16_t, 2, 4, 4, 2>(a, epi, s);
    return launch_shape<uint16_t, 2, 2, 2, 2>(a, epi, s);
  }
  if (shape == GemmShape::Big) return launch_shape<float, 2, 4, 4, 2>(a, epi, s);
  return launch_shape<float, 2, 2, 2, 2>(a, epi, s);
}

hipError_t launch_mtile_prefix(const int32_t* goff, int G, int bm, int32_t* mtile_start, hipStream_t s) {
  KernelTimer timer("mtile_prefix", s);
  hipLaunchKernelGGL(mtile_prefix_kernel, dim3(1), dim3(1024), 0, s, goff, G, bm, mtile_start);
  return hipGetLastError();
}

}  // namespace lmoe
