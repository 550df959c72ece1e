// MFMA GEMM for gfx950: C[rows, N] = A[rows, K] . B[N, K]^T with fused epilogues, over one dense
// matrix or ragged row groups (one B per group, rows of a group contiguous in A and C).
//
// Layout and schedule:
//  * A and B are K-contiguous ("[out, in]" weights), so both MFMA operands are read as 16-byte
//    chunks along K: lane l of a 32x32x16 MFMA takes 8 k-values of row l % 32 (A) or column l % 32
//    (B), the two lane halves covering the 16 k of the step.
//  * Waves tile the block as WAVES_M x WAVES_N; a wave owns WM row-blocks and WN column-blocks of
//    32x32 (v_mfma_f32_32x32x16_bf16, or four v_mfma_f32_32x32x2f32 for f32 data). Row-blocks are
//    interleaved across the M-waves so a ragged tail spreads evenly; a wave's row-blocks holding
//    rows of the tile form a prefix, and the K loop is instantiated per prefix length, so no
//    branch sits between the LDS reads and the MFMAs and empty row-blocks cost nothing.
//  * Two pipelines:
//    - DMA (256x256 tiles): K-tiles go straight from HBM into LDS with buffer_load ... lds, without
//      register staging, into a ring of NS stages (measured best: two stages of 64 bf16 per row,
//      64 KB each; the next K-tile streams in while the MFMAs consume the current one, and the
//      wider K-tile halves the barriers against four stages of 32). A DMA instruction writes 64
//      lanes x 16 bytes contiguously (1 KB of consecutive rows); each lane fetches the chunk that
//      belongs at its slot under an XOR swizzle. A ds_read_b128 is served 16 lanes (256 bytes of
//      banks) at a time, and the swizzle places the 16 rows one pass reads in 16 distinct 16-byte
//      bank groups.
//      The DMA is issued from inline assembly with its own vmcnt waits, because the compiler's
//      waitcnt pass would otherwise drain every outstanding DMA before each LDS read.
//    - Registers (128x128 tiles): K-tiles of 128 bytes per row are loaded into registers one
//      K-tile ahead and written to one of two padded LDS stages (144-byte pitch, conflict-free).
//  * Global loads use buffer resources that span exactly the tile's valid rows of A and of B (one
//    each for the gate and up halves of a GLU tile): past the end a load returns zero, so ragged
//    row and column tails need no predication. The K offset rides in the uniform soffset.
//  * Optional row gather of A (row r of the GEMM reads A row a_rows[r]): the routed experts read
//    their tokens' latent rows in place, so the permuted copy is never written. Optional second K
//    segment (A2, B2): the up-projection and the shared experts' down-projection share one
//    output and one accumulator, [n | h_s] . [W_up | W2_s]^T.
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// Raw buffer descriptor over [base, base + bytes): word 3 = 0x00020000 is the gfx9-family raw
// buffer format (32-bit data, no swizzle); reads past num_records return zero.
constexpr unsigned kBufWord3 = 0x00020000u;
constexpr int kOutOfRange = 0x7fff0000;  // a voffset past any buffer this library builds: reads zero

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufWord3);
}

__device__ inline u32x4 make_desc(const void* base, int bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  u32x4 d;
  d.x = __builtin_amdgcn_readfirstlane((unsigned)a);
  d.y = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);  // stride 0
  d.z = __builtin_amdgcn_readfirstlane((unsigned)bytes);
  d.w = kBufWord3;
  return d;
}

__device__ inline uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// One wave-wide DMA: lane i's 16 bytes from desc + voff + soff land at LDS lds_addr + 16 i.
__device__ inline void dma16(const u32x4& desc, int voff, int soff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(desc), "s"(soff)
               : "memory", "m0");
}

// The same with the non-temporal hint: for operands streamed through once (the routed experts' W1
// and W2 slices), so that they do not displace the rows that the other n-tiles of the same expert
// read again (measured at K3 prefill: routed GEMM1 1.54 -> 1.42 ms; GEMM2, on the three-stage B
// ring, 0.92 -> 0.91 ms; the dense GEMMs and the MX pipeline gain nothing or lose). A template
// instance of its own, so that the other GEMMs keep their code.
__device__ inline void dma16_nt(const u32x4& desc, int voff, int soff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(desc), "s"(soff)
               : "memory", "m0");
}

// XOR key of the DMA pipeline's LDS layout (rows of KB bytes): the 16-byte slot of chunk c in row r
// is c ^ swz<KB>(r). A ds_read_b128 is served 16 lanes (256 bytes of banks) at a time, and the 16
// rows one pass reads then land in 16 distinct 16-byte bank groups.
template <int KB>
__device__ constexpr int swz(int r) { return (r / (256 / KB)) % (KB / 16); }

template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ inline void store_out(const GemmArgs& p, int64_t off, float v) {
  if (p.c_dtype == LMOE_F32)
    static_cast<float*>(p.C)[off] = v;
  else
    static_cast<uint16_t*>(p.C)[off] = f32_to_bf16(v);
}

// ------------------------------------------------------------------------------------------------
// tile assignment and epilogue shared by both pipelines
// ------------------------------------------------------------------------------------------------
struct TileInfo {
  int g, n0, row0, rows;
  int mtg = 1;    // m-tiles of the tile's group (grouped GEMMs)
  int k0, klen;   // contraction range of the tile (elements)
  int64_t coff;   // element offset of the tile's output block (K-grouped GEMMs)
};

// Tile of (virtual) workgroup vb: workgroup vb runs on XCD vb % 8, and each XCD takes a contiguous
// run of tile numbers, so that the n-tiles of one m-tile share that XCD's L2.
template <int BM, int BNO>
__device__ inline bool assign_tile(const GemmArgs& p, TileInfo& t, int vb) {
  const bool grouped = p.goff != nullptr;
  const int n_tiles = (int)ceil_div(p.N, BNO);
  const int mt_total = p.koff ? p.G * (int)ceil_div(p.M, BM) : grouped ? p.mtile_start[p.G] : (int)ceil_div(p.M, BM);
  const int total = mt_total * n_tiles;
  const int per = (total + kXcds - 1) / kXcds;
  const int loc = vb / kXcds;
  if (loc >= per) return false;
  const int lt = (vb % kXcds) * per + loc;
  if (lt >= total) return false;
  int n_tile;
  t.g = 0;
  t.k0 = 0;
  t.klen = p.K;
  t.coff = 0;
  if (p.koff) {  // K-grouped: group-major; inside a group n-tile major, m-tile minor
    const int MT = (int)ceil_div(p.M, BM);
    const int tpg = MT * n_tiles;
    t.g = lt / tpg;
    const int r = lt - t.g * tpg;
    n_tile = r / MT;
    t.row0 = (r % MT) * BM;
    t.rows = min(BM, p.M - t.row0);
    t.k0 = p.koff[t.g] * p.koff_scale;
    t.klen = (p.koff[t.g + 1] - p.koff[t.g]) * p.koff_scale;
    t.coff = (int64_t)t.g * p.c_gstride;
  } else if (grouped) {
    const int q = lt / n_tiles;
    int lo = 0, hi = p.G;  // mtile_start[lo] <= q < mtile_start[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.mtile_start[mid] <= q) lo = mid; else hi = mid;
    }
    t.g = lo;
    const int ms0 = p.mtile_start[lo];
    const int mtg = p.mtile_start[lo + 1] - ms0;
    t.mtg = mtg;
    const int r = lt - n_tiles * ms0;
    n_tile = r / mtg;
    t.row0 = p.goff[lo] + (r % mtg) * BM;
    t.rows = min(BM, p.goff[lo + 1] - t.row0);
  } else {
    constexpr int GM = 8;  // raster: 8 m-tiles x all n-tiles, m fastest
    const int MT = (int)ceil_div(p.M, BM);
    const int gsz = GM * n_tiles;
    const int grp = lt / gsz, first = grp * GM, gm = min(MT - first, GM), r = lt % gsz;
    n_tile = r / gm;
    t.row0 = (first + r % gm) * BM;
    t.rows = min(BM, p.M - t.row0);
  }
  t.n0 = n_tile * BNO;
  return true;
}

// assign_tile for a grouped GEMM (no K groups) when this workgroup's previous tile was in group
// g_hint: tile numbers only grow along a workgroup's walk, so the group is searched forward from
// g_hint through a window of W entries of mtile_start read at once (one load round trip instead of
// a binary search's chain of log2(G)), with the binary search as the fallback past the window.
// mt_total is mtile_start[G]. On success g_hint holds the tile's group.
template <int BM, int BNO>
__device__ inline bool assign_tile_after(const GemmArgs& p, TileInfo& t, int vb, int mt_total, int& g_hint) {
  constexpr int W = 16;
  const int n_tiles = (int)ceil_div(p.N, BNO);
  const int total = mt_total * n_tiles;
  const int per = (total + kXcds - 1) / kXcds;
  const int loc = vb / kXcds;
  if (loc >= per) return false;
  const int lt = (vb % kXcds) * per + loc;
  if (lt >= total) return false;
  const int q = lt / n_tiles;
  int v[W];
#pragma unroll
  for (int j = 0; j < W; ++j) v[j] = p.mtile_start[min(g_hint + 1 + j, p.G)];
  int g = g_hint;  // mtile_start[g] <= q; the group is the last such g (mtile_start[G] > q)
#pragma unroll
  for (int j = 0; j < W; ++j) g += (g_hint + 1 + j < p.G && v[j] <= q) ? 1 : 0;
  if (g == g_hint + W) {  // past the window
    int lo = g, hi = p.G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.mtile_start[mid] <= q) lo = mid; else hi = mid;
    }
    g = lo;
  }
  g_hint = g;
  t.g = g;
  t.k0 = 0;
  t.klen = p.K;
  t.coff = 0;
  const int ms0 = p.mtile_start[g];
  const int mtg = p.mtile_start[g + 1] - ms0;
  t.mtg = mtg;
  const int r = lt - n_tiles * ms0;
  t.row0 = p.goff[g] + (r % mtg) * BM;
  t.rows = min(BM, p.goff[g + 1] - t.row0);
  t.n0 = (r / mtg) * BNO;
  return true;
}

template <typename TI, int WAVES_M, int WAVES_N, int WM, int WN, Epi EPI>
__device__ inline void epilogue(const GemmArgs& p, const TileInfo& t, f32x16 (&acc)[WM][WN], int wm, int wn,
                                int lane, int na) {
  constexpr bool GLU = EPI == Epi::Glu || EPI == Epi::GluBwd;
  constexpr int WNO = GLU ? WN / 2 : WN;
  const float inv_b1 = 1.0f / p.beta1, inv_b2 = 1.0f / p.beta2;
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    if (i >= na) continue;
    const int rbk = i * WAVES_M + wm;
#pragma unroll
    for (int j = 0; j < WNO; ++j) {
      const int col = t.n0 + (j * WAVES_N + wn) * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = rbk * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (r >= t.rows) continue;
        const int64_t grow = t.row0 + r;
        const int64_t off = grow * p.ldc + col + t.coff;
        if constexpr (EPI == Epi::Store) {
          store_out(p, off, acc[i][j][q]);
        } else if constexpr (EPI == Epi::GluBwd) {
          const int64_t ai = grow * p.ld_aux + col;
          const float dh = sizeof(TI) == 2 ? bf16_to_f32(static_cast<const uint16_t*>(p.aux)[ai])
                                           : static_cast<const float*>(p.aux)[ai];
          float dg, du;
          situ_glu_bwd(acc[i][j][q], acc[i][j + WNO][q], dh, p.beta1, p.beta2, dg, du);
          store_out(p, off, dg);
          store_out(p, off + p.N, du);
        } else if constexpr (EPI == Epi::Glu) {
          store_out(p, off, situ_glu<sizeof(TI) == 4>(acc[i][j][q], acc[i][j + WNO][q], p.beta1, inv_b1, p.beta2,
                                                      inv_b2));
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

// Epilogue through LDS for Store/Glu into TO (bf16 or f32): the wave writes its outputs into its own
// LDS region in row-major order, then every lane stores whole 16-byte chunks (one instruction per
// 8 bf16 or 4 f32) instead of one scalar per element. Needs N and ldc multiples of 16 / sizeof(TO)
// and a 16-byte aligned C. Row-blocks are staged RBP at a time to fit the region.
template <typename TI, typename TO, int WAVES_M, int WAVES_N, int WM, int WN, Epi EPI, int REGION, bool NTC = false>
__device__ inline void epilogue_staged(const GemmArgs& p, const TileInfo& t, f32x16 (&acc)[WM][WN], int wm, int wn,
                                       int lane, int na, char* region) {
  constexpr bool GLU = EPI == Epi::Glu;
  static_assert(EPI == Epi::Store || GLU, "staged epilogue covers plain and GLU stores");
  constexpr int WNO = GLU ? WN / 2 : WN;
  constexpr int COLS = WNO * 32;
  constexpr int ROWB = COLS * (int)sizeof(TO);
  constexpr int VEC = 16 / (int)sizeof(TO);
  constexpr int CPB = 32 / VEC;   // chunks per row of one 32-column block
  constexpr int CPR = WNO * CPB;  // chunks per staged row
  constexpr int RBP = REGION / (32 * ROWB) < WM ? REGION / (32 * ROWB) : WM;
  static_assert(RBP >= 1, "region holds at least one row-block");
  const float inv_b1 = 1.0f / p.beta1, inv_b2 = 1.0f / p.beta2;
  TO* st = reinterpret_cast<TO*>(region);
#pragma unroll
  for (int i0 = 0; i0 < WM; i0 += RBP) {
    if (i0 >= na) break;
#pragma unroll
    for (int ii = 0; ii < RBP; ++ii) {
      const int i = i0 + ii;
      if (i >= WM || i >= na) break;
#pragma unroll
      for (int j = 0; j < WNO; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int lr = ii * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
          float v = acc[i][j][q];
          if constexpr (GLU) v = situ_glu<sizeof(TI) == 4>(v, acc[i][j + WNO][q], p.beta1, inv_b1, p.beta2, inv_b2);
          if constexpr (sizeof(TO) == 2)
            st[lr * COLS + j * 32 + (lane & 31)] = f32_to_bf16(v);
          else
            st[lr * COLS + j * 32 + (lane & 31)] = v;
        }
    }
    __builtin_amdgcn_wave_barrier();
    const int nrb = min(RBP, na - i0);
    for (int c = lane; c < nrb * 32 * CPR; c += kWave) {
      const int lr = c / CPR, cc = c % CPR;
      const int j = cc / CPB, cv = (cc % CPB) * VEC;
      const int r = ((i0 + lr / 32) * WAVES_M + wm) * 32 + (lr % 32);
      const int col = t.n0 + (j * WAVES_N + wn) * 32 + cv;
      if (r < t.rows && col < p.N) {
        uint4* dst = reinterpret_cast<uint4*>(static_cast<TO*>(p.C) + (int64_t)(t.row0 + r) * p.ldc + col + t.coff);
        const uint4 v = *reinterpret_cast<const uint4*>(region + lr * ROWB + (j * 32 + cv) * (int)sizeof(TO));
        if constexpr (NTC) {
          __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
        } else {
          *dst = v;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int WM, int WN>
__device__ inline void zero_acc(f32x16 (&acc)[WM][WN]) {
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
}

// Calls f(integral_constant<NA>) for the wave's active row-block count na (0..WM).
template <int WM, typename F>
__device__ inline void dispatch_na(int na, F&& f) {
  static_assert(WM <= 4, "specialisations cover up to four row-blocks per wave");
  switch (na) {
    case 0: f(std::integral_constant<int, 0>{}); break;
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (WM >= 2) f(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (WM >= 3) f(std::integral_constant<int, 3>{}); break;
    default: if constexpr (WM >= 4) f(std::integral_constant<int, 4>{}); break;
  }
}

// MFMAs of one K-tile of the DMA pipeline: A's stage at `base` (BM rows of KB bytes), B's at `bbase`
// (BNB rows of KB bytes, or KB/sizeof(TI) k-rows of BNB columns when BKN), both swizzled by swz<KB>.
// The fragments of k-step s + 1 are read from LDS while the MFMAs of k-step s run.
template <typename TI, int WAVES_M, int WAVES_N, int WM, int WN, int KB, bool GLU, bool BKN, int NA>
__device__ inline void dma_ktile(const char* base, const char* bbase, const int (&fo)[KB / 32], int wm, int wn,
                                 int lane, f32x16 (&acc)[WM][WN]) {
  constexpr int KS = KB / 32;
  constexpr int BNB = WAVES_N * WN * 32;
  constexpr int BNO = GLU ? BNB / 2 : BNB;
  constexpr int WNO = GLU ? WN / 2 : WN;
  constexpr int BROW = BNB * (int)sizeof(TI);  // bytes of one k-row of a [K, N] B tile
  uint4 af[2][NA > 0 ? NA : 1], bf[2][WN];
  auto load = [&](int s, uint4 (&a)[NA > 0 ? NA : 1], uint4 (&b)[WN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      a[i] = *reinterpret_cast<const uint4*>(base + (i * WAVES_M + wm) * 32 * KB + fo[s]);
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int ocb = (j % WNO) * WAVES_N + wn;
      const int bblk = (GLU && j >= WNO) ? BNO / 32 + ocb : ocb;
      if constexpr (BKN) {
        const int n = bblk * 32 + (lane & 31), c = n >> 3, e = n & 7;
        const int k0 = s * 16 + 8 * (lane >> 5);
        uint16_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          v[i] = *reinterpret_cast<const uint16_t*>(bbase + (k0 + i) * BROW + ((c ^ ((k0 + i) & 15)) << 4) + e * 2);
        b[j] = *reinterpret_cast<const uint4*>(v);
      } else {
        b[j] = *reinterpret_cast<const uint4*>(bbase + bblk * 32 * KB + fo[s]);
      }
    }
  };
  load(0, af[0], bf[0]);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (s + 1 < KS) load(s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) Mfma<TI>::run(acc[i][j], af[s & 1][i], bf[s & 1][j]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ------------------------------------------------------------------------------------------------
// DMA pipeline: 256x256 tiles, LDS fed straight from HBM, three K-tiles in flight
// ------------------------------------------------------------------------------------------------
// BKN: B is stored [K, N] (bf16): a K-tile of B is 64 rows of BNB columns, DMA'd row by row into
// LDS with the 16-byte chunk c of row k at slot c ^ (k % 16); a B fragment (8 consecutive k of one
// column) is gathered with 16-bit LDS reads, which the swizzle spreads over distinct banks.
// NTB: B is streamed through once (the routed experts' W1): its DMA carries the non-temporal hint.
// NTC: C is written once and read once later (the routed experts' y): stored with the non-temporal
// hint (measured at K3 prefill: the combine that reads y 0.196 -> 0.189 ms, GEMM2 unchanged).
// XB: B's ring holds XB more stages than A's, and B's K-tiles are issued XB tiles further ahead
// (two A stages and three B stages of 64-element K-tiles fill the 160 KB of LDS).
template <typename TI, int WAVES_M, int WAVES_N, int WM, int WN, int NS, int KB, Epi EPI, bool BKN = false,
          bool NTB = false, int XB = 0, bool NTC = false>
__global__ void __launch_bounds__(WAVES_M* WAVES_N* kWave)
    __attribute__((amdgpu_waves_per_eu(WAVES_M* WAVES_N / 4, WAVES_M* WAVES_N / 4)))  // one workgroup per CU
    gemm_dma_kernel(GemmArgs p_in) {
  GemmArgs p = p_in;
  int ka0 = 0;  // byte offset inside A's wrapped row where this workgroup's K range starts
  if (p.splits > 1) {  // split-K (one K segment, no groups): K-chunk blockIdx.y into its own f32 partial
    const int sp = blockIdx.y;
    ka0 = (int)(((int64_t)sp * p.K) % p.a_kwrap) * (int)sizeof(TI);
    p.B = static_cast<const char*>(p.B) + (int64_t)sp * p.K * (int64_t)sizeof(TI);
    p.K1 = p.K;
    p.C = static_cast<float*>(p.C) + sp * p.c_split;
  }
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int BM = WAVES_M * WM * 32;
  constexpr int BNB = WAVES_N * WN * 32;  // rows of B per tile
  constexpr bool GLU = EPI == Epi::Glu || EPI == Epi::GluBwd;
  static_assert(!GLU || WN % 2 == 0, "GLU needs gate/up column-block pairs");
  constexpr int BNO = GLU ? BNB / 2 : BNB;
  constexpr int WNO = GLU ? WN / 2 : WN;
  // NS LDS stages of KB bytes of every row per K-tile
  static_assert(NS >= 2 && NS <= 5 && (KB == 64 || KB == 128), "pipeline shape");
  static_assert(XB == 0 || (XB == 1 && NS == 2), "B runs one K-tile further ahead only on a two-stage A ring");
  constexpr int NSB = NS + XB;  // stages of B
  constexpr int RPD = 1024 / KB;           // rows per 1 KB DMA block
  constexpr int A_PW = BM / RPD / NW;      // DMA blocks per wave per K-tile
  constexpr int B_PW = BNB / RPD / NW;
  static_assert(A_PW * RPD * NW == BM && B_PW * RPD * NW == BNB, "DMA split");
  // On the two-stage ring with [N, K] B, the upper half of the waves issues every DMA of a K-tile
  // while the lower half goes straight to its MFMAs: a K-tile's 64 DMA instructions keep the
  // address unit busy for about 1400 cycles, and with all eight waves issuing, every wave of a SIMD
  // sat in that queue at once with the matrix pipe idle (measured at K3 prefill: 750-990 of
  // 3300-3650 cycles per K-tile; shared GEMM1 0.917 -> 0.862 ms, down-projection 0.416 -> 0.388,
  // up-projection 0.924 -> 0.853, outputs bit-identical).
  constexpr bool DS = XB == 0 && !BKN && NW % 2 == 0;
  constexpr int A_PWI = DS ? 2 * A_PW : A_PW;  // DMA blocks per issuing wave per K-tile
  constexpr int B_PWI = DS ? 2 * B_PW : B_PW;
  static_assert(!GLU || BNO % RPD == 0, "a DMA block stays in one GLU half");
  constexpr int A_BYTES = BM * KB;  // one stage of A; the NS stages of A come first, then the NSB of B
  constexpr int B_BYTES = BNB * KB;
  constexpr int B_BASE = NS * A_BYTES;
  constexpr int LDS_BYTES = B_BASE + NSB * B_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  TileInfo t;
  if (!assign_tile<BM, BNO>(p, t, blockIdx.x)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int na = min(WM, max(0, (((t.rows + 31) >> 5) - wm + WAVES_M - 1) / WAVES_M));

  const int64_t a_ld = p.lda * (int64_t)sizeof(TI), b_ld = p.ldb * (int64_t)sizeof(TI);
  const int64_t a_ld2 = p.lda2 * (int64_t)sizeof(TI), b_ld2 = p.ldb2 * (int64_t)sizeof(TI);
  const char* Bb = static_cast<const char*>(p.B) + (int64_t)t.g * p.b_gstride * (int64_t)sizeof(TI) +
                   (int64_t)t.k0 * (int64_t)sizeof(TI);
  const int ncols = min(BNO, p.N - t.n0);
  const bool gather = p.a_rows != nullptr;
  const bool seg2 = !GLU && p.A2 != nullptr;
  const u32x4 a_desc = gather ? make_desc(p.A, (int)(p.a_nrows * a_ld))
                              : make_desc(static_cast<const char*>(p.A) + (int64_t)t.row0 * a_ld +
                                              (int64_t)t.k0 * (int64_t)sizeof(TI), (int)(t.rows * a_ld));
  static_assert(!BKN || (sizeof(TI) == 2 && KB == 128 && !GLU && EPI == Epi::Store), "[K, N] B: bf16 store");
  const u32x4 b_desc0 = BKN ? make_desc(Bb + (int64_t)t.n0 * (int64_t)sizeof(TI),
                                        (int)((int64_t)p.K * b_ld - (int64_t)t.n0 * (int64_t)sizeof(TI)))
                            : make_desc(Bb + (int64_t)t.n0 * b_ld, (int)(ncols * b_ld));
  const u32x4 b_desc1 = GLU ? make_desc(Bb + (int64_t)(p.glu_up_off + t.n0) * b_ld, (int)(ncols * b_ld)) : b_desc0;
  const u32x4 a2_desc =
      seg2 ? make_desc(static_cast<const char*>(p.A2) + (int64_t)t.row0 * a_ld2, (int)(t.rows * a_ld2)) : a_desc;
  const u32x4 b2_desc =
      seg2 ? make_desc(static_cast<const char*>(p.B2) + (int64_t)t.n0 * b_ld2, (int)(ncols * b_ld2)) : b_desc0;
  const int a_wrap = p.a_kwrap * (int)sizeof(TI);
  const int KT = t.klen * (int)sizeof(TI) / KB;
  const int KT1 = p.K1 * (int)sizeof(TI) / KB;

  // The lane's source chunk for each DMA block of this wave (swizzled so that LDS slot s of row r
  // holds chunk s ^ swz<KB>(r)). A gathered row outside A gets an offset past the buffer end.
  const int lr = lane / (KB / 16), slot = lane % (KB / 16);
  const bool issuer = !DS || wave >= NW / 2;
  const int wi = DS ? (issuer ? wave - NW / 2 : 0) : wave;  // index among the issuing waves
  int a_voff[A_PWI], b_voff[B_PWI], a2_voff[A_PWI], b2_voff[B_PWI];
#pragma unroll
  for (int i = 0; i < A_PWI; ++i) {
    const int r = (wi * A_PWI + i) * RPD + lr;
    const int ch = (slot ^ swz<KB>(r)) * 16;
    if (gather) {
      const int src = r < t.rows ? p.a_rows[t.row0 + r] : -1;
      a_voff[i] = (src >= 0 && src < p.a_nrows) ? src * (int)a_ld + ch : kOutOfRange;
    } else {
      a_voff[i] = r * (int)a_ld + ch;
    }
    a2_voff[i] = r * (int)a_ld2 + ch;
  }
#pragma unroll
  for (int i = 0; i < B_PWI; ++i) {
    if constexpr (BKN) {  // block j holds k-rows 2j and 2j + 1; lane l fills slot l % 32 of row 2j + l / 32
      const int k = 2 * (wave * B_PW + i) + lane / 32;
      b_voff[i] = k * (int)b_ld + (((lane % 32) ^ (k % 16)) * 16);
      b2_voff[i] = b_voff[i];
    } else {
      const int r = (wi * B_PWI + i) * RPD + lr;
      const int ch = (slot ^ swz<KB>(r)) * 16;
      b_voff[i] = (r % BNO) * (int)b_ld + ch;
      b2_voff[i] = (r % BNO) * (int)b_ld2 + ch;
    }
  }
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(
      (unsigned)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));

  int ka = ka0;  // byte offset of the next issued K-tile inside A's (possibly wrapped) row
  auto issue_a = [&](int kt, int stage) __attribute__((always_inline)) {
    if (!issuer) return;
    const unsigned base = lds0 + stage * A_BYTES;
    if (!seg2 || kt < KT1) {
#pragma unroll
      for (int i = 0; i < A_PWI; ++i) dma16(a_desc, a_voff[i], ka, base + (wi * A_PWI + i) * 1024);
      ka += KB;
      if (ka == a_wrap) ka = 0;
    } else {
      const int kk = (kt - KT1) * KB;
#pragma unroll
      for (int i = 0; i < A_PWI; ++i) dma16(a2_desc, a2_voff[i], kk, base + (wi * A_PWI + i) * 1024);
    }
  };
  auto issue_b = [&](int kt, int stage) __attribute__((always_inline)) {
    if (!issuer) return;
    const unsigned base = lds0 + B_BASE + stage * B_BYTES;
    if (!seg2 || kt < KT1) {
#pragma unroll
      for (int i = 0; i < B_PWI; ++i) {
        const bool up = GLU && (wi * B_PWI + i) * RPD >= BNO;
        const int soff = BKN ? kt * (KB / (int)sizeof(TI)) * (int)b_ld : kt * KB;
        if constexpr (NTB)
          dma16_nt(up ? b_desc1 : b_desc0, b_voff[i], soff, base + (wi * B_PWI + i) * 1024);
        else
          dma16(up ? b_desc1 : b_desc0, b_voff[i], soff, base + (wi * B_PWI + i) * 1024);
      }
    } else {
      const int kk = (kt - KT1) * KB;
#pragma unroll
      for (int i = 0; i < B_PWI; ++i) dma16(b2_desc, b2_voff[i], kk, base + (wi * B_PWI + i) * 1024);
    }
  };
  constexpr int PER_TILE = A_PWI + B_PWI;  // DMA instructions per issuing wave per K-tile
  auto wait_tiles_after = [&](int n) __attribute__((always_inline)) {
    if (NS > 4 && n >= 3) wait_vmcnt<3 * PER_TILE>();
    else if (NS > 3 && n == 2) wait_vmcnt<2 * PER_TILE>();
    else if (NS > 2 && n == 1) wait_vmcnt<PER_TILE>();
    else wait_vmcnt<0>();
  };

  f32x16 acc[WM][WN];
  zero_acc(acc);
  // fragment offset of each 32-byte k-step of a K-tile (row-block bases, multiples of 32 rows, keep
  // the swizzle key of row lane & 31)
  constexpr int KS = KB / 32;
  int fo[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) fo[s] = (lane & 31) * KB + (((2 * s + (lane >> 5)) ^ swz<KB>(lane & 31)) * 16);

  dispatch_na<WM>(na, [&](auto na_c) __attribute__((always_inline)) {
    constexpr int NA = decltype(na_c)::value;
    auto compute = [&](int sa, int sb) __attribute__((always_inline)) {
      dma_ktile<TI, WAVES_M, WAVES_N, WM, WN, KB, GLU, BKN, NA>(smem + sa * A_BYTES, smem + B_BASE + sb * B_BYTES, fo,
                                                              wm, wn, lane, acc);
    };
    if constexpr (XB == 0) {
      const int pre = min(KT, NS - 1);
      for (int kt = 0; kt < pre; ++kt) {
        issue_a(kt, kt);
        issue_b(kt, kt);
      }
      for (int kt = 0; kt < KT; ++kt) {
        wait_tiles_after(min(KT - kt - 1, NS - 2));  // K-tile kt has landed in LDS (this wave's part)
        __syncthreads();                             // ... and every wave's; stage kt-1 is free again
        if (kt + NS - 1 < KT) {
          issue_a(kt + NS - 1, (kt + NS - 1) % NS);
          issue_b(kt + NS - 1, (kt + NS - 1) % NS);
        }
        if (NA > 0) compute(kt % NS, kt % NS);
      }
    } else {
      // Issue order A0 B0 B1 | A1 B2 | A2 B3 | ...: when A(kt) and B(kt) have landed, only B(kt+1)
      // can still be in flight (loads complete in issue order).
      issue_a(0, 0);
      issue_b(0, 0);
      if (KT > 1) issue_b(1, 1);
      for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) wait_vmcnt<B_PW>();
        else wait_vmcnt<0>();
        __syncthreads();  // every wave's part has landed; A stage (kt+1)%2 and B stage (kt+2)%3 are free
        if (kt + 1 < KT) issue_a(kt + 1, (kt + 1) & 1);
        if (kt + 2 < KT) issue_b(kt + 2, (kt + 2) % 3);
        if (NA > 0) compute(kt & 1, kt % 3);
      }
    }
  });
  if constexpr (EPI == Epi::Store || EPI == Epi::Glu) {
    constexpr int REGION = LDS_BYTES / NW;  // each wave's slice of the pipeline LDS
    const bool bf = p.c_dtype == LMOE_BF16;
    const int vec = bf ? 8 : 4;
    if (p.N % vec == 0 && p.ldc % vec == 0) {
      __syncthreads();  // every wave is done reading the pipeline stages
      char* region = smem + wave * REGION;
      if (bf)
        epilogue_staged<TI, uint16_t, WAVES_M, WAVES_N, WM, WN, EPI, REGION, NTC>(p, t, acc, wm, wn, lane, na,
                                                                                 region);
      else
        epilogue_staged<TI, float, WAVES_M, WAVES_N, WM, WN, EPI, REGION, NTC>(p, t, acc, wm, wn, lane, na, region);
      return;
    }
  }
  epilogue<TI, WAVES_M, WAVES_N, WM, WN, EPI>(p, t, acc, wm, wn, lane, na);
}

// ------------------------------------------------------------------------------------------------
// Persistent DMA pipeline for the routed experts' GEMMs
// ------------------------------------------------------------------------------------------------
// The grouped GEMMs of the routed experts (GEMM1 with the SiTU-GLU epilogue, GEMM2 with a plain
// store) stream each expert's weights (B) from HBM once. With one workgroup per tile, every tile
// pays its set-up (tile lookup, row indices), the first DMA round trip and its epilogue with no B
// bytes in flight: measured at K3 prefill, 11 % of GEMM1's and 42 % of GEMM2's cycles. Here one
// workgroup per CU walks its XCD's share of the tile numbers (the same numbering as the one-shot
// launch), and the next tile's first two B K-tiles are in flight while the current tile's epilogue
// runs. The epilogue is staged through the two A stages only (8 KB per wave), so the B stages can
// take the next tile's data; the next tile's lookup and row indices are read while the current
// tile's first K-tile is in flight. Same 256x256 tiles, swizzle, two A and three B stages as the
// one-shot kernel (B one K-tile further ahead, with the non-temporal hint).
template <typename TI, int WAVES_M, int WAVES_N, int WM, int WN, int KB, Epi EPI, bool NTC, bool IS = true>
__global__ void __launch_bounds__(WAVES_M* WAVES_N* kWave)
    __attribute__((amdgpu_waves_per_eu(WAVES_M* WAVES_N / 4, WAVES_M* WAVES_N / 4)))  // one workgroup per CU
    gemm_routed_kernel(GemmArgs p) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int BM = WAVES_M * WM * 32;
  constexpr int BNB = WAVES_N * WN * 32;
  constexpr bool GLU = EPI == Epi::Glu;
  static_assert(GLU || EPI == Epi::Store, "routed GEMM1 (GLU) or GEMM2 (plain store)");
  static_assert(!GLU || WN % 2 == 0, "GLU needs gate/up column-block pairs");
  constexpr int BNO = GLU ? BNB / 2 : BNB;
  constexpr int RPD = 1024 / KB;
  constexpr int A_PW = BM / RPD / NW;
  constexpr int B_PW = BNB / RPD / NW;
  static_assert(A_PW * RPD * NW == BM && B_PW * RPD * NW == BNB, "DMA split");
  static_assert(!GLU || BNO % RPD == 0, "a DMA block stays in one GLU half");
  // IS: the upper half of the waves issues every DMA (as in the dense kernel), so that the lower
  // half starts its MFMAs at once and never waits for the epilogue's stores to complete.
  static_assert(!IS || NW % 2 == 0, "issue split needs an even wave count");
  constexpr int A_PWI = IS ? 2 * A_PW : A_PW;  // DMA blocks per issuing wave per K-tile
  constexpr int B_PWI = IS ? 2 * B_PW : B_PW;
  constexpr int A_BYTES = BM * KB;
  constexpr int B_BYTES = BNB * KB;
  constexpr int B_BASE = 2 * A_BYTES;
  constexpr int LDS_BYTES = B_BASE + 3 * B_BYTES;
  constexpr int REGION = B_BASE / NW;  // epilogue staging: each wave's slice of the A stages
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  int vb = blockIdx.x;
  TileInfo t;
  if (!assign_tile<BM, BNO>(p, t, vb)) return;
  const int mt_total = p.mtile_start[p.G];
  int g_hint = t.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int64_t a_ld = p.lda * (int64_t)sizeof(TI), b_ld = p.ldb * (int64_t)sizeof(TI);
  const bool gather = p.a_rows != nullptr;
  const int KT = p.K * (int)sizeof(TI) / KB;
  const int lr = lane / (KB / 16), slot = lane % (KB / 16);
  const bool issuer = !IS || wave >= NW / 2;
  const int wi = IS ? (issuer ? wave - NW / 2 : 0) : wave;  // index among the issuing waves
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(
      (unsigned)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));

  // Source row of each of the lane's A DMA blocks (gather: the row of A, -1 past the tile's rows).
  auto load_src = [&](const TileInfo& tt, int (&src)[A_PWI]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_PWI; ++i) {
      const int r = (wi * A_PWI + i) * RPD + lr;
      src[i] = gather ? (issuer && r < tt.rows ? p.a_rows[tt.row0 + r] : -1) : r;
    }
  };
  u32x4 a_desc, b_desc0, b_desc1;
  int a_voff[A_PWI], b_voff[B_PWI];
#pragma unroll
  for (int i = 0; i < B_PWI; ++i) {
    const int r = (wi * B_PWI + i) * RPD + lr;
    b_voff[i] = (r % BNO) * (int)b_ld + ((slot ^ swz<KB>(r)) * 16);
  }
  auto set_a = [&](const TileInfo& tt, const int (&src)[A_PWI]) __attribute__((always_inline)) {
    a_desc = gather ? make_desc(p.A, (int)(p.a_nrows * a_ld))
                    : make_desc(static_cast<const char*>(p.A) + (int64_t)tt.row0 * a_ld, (int)(tt.rows * a_ld));
#pragma unroll
    for (int i = 0; i < A_PWI; ++i) {
      const int r = (wi * A_PWI + i) * RPD + lr;
      const int ch = (slot ^ swz<KB>(r)) * 16;
      if (gather)
        a_voff[i] = (src[i] >= 0 && src[i] < p.a_nrows) ? src[i] * (int)a_ld + ch : kOutOfRange;
      else
        a_voff[i] = r * (int)a_ld + ch;
    }
  };
  // B streams with the non-temporal hint when its group has one m-tile (read once); a group of
  // several m-tiles reads the same weight slices once per m-tile, and those tiles run close together
  // on one XCD, so there B is loaded plainly and the later m-tiles find it cached (measured on
  // batches of 32768 tokens, about three m-tiles per expert: GEMM2 2.93 -> 2.75 ms, GEMM1 within
  // 1 %; at 8192 tokens, one m-tile per expert, unchanged).
  bool b_nt = true;
  auto set_b = [&](const TileInfo& tt) __attribute__((always_inline)) {
    b_nt = tt.mtg == 1;
    const char* Bb = static_cast<const char*>(p.B) + (int64_t)tt.g * p.b_gstride * (int64_t)sizeof(TI);
    const int ncols = min(BNO, p.N - tt.n0);
    b_desc0 = make_desc(Bb + (int64_t)tt.n0 * b_ld, (int)(ncols * b_ld));
    b_desc1 = GLU ? make_desc(Bb + (int64_t)(p.glu_up_off + tt.n0) * b_ld, (int)(ncols * b_ld)) : b_desc0;
  };
  auto issue_a = [&](int kt, int stage) __attribute__((always_inline)) {
    if (!issuer) return;
    const unsigned base = lds0 + stage * A_BYTES;
#pragma unroll
    for (int i = 0; i < A_PWI; ++i) dma16(a_desc, a_voff[i], kt * KB, base + (wi * A_PWI + i) * 1024);
  };
  auto issue_b = [&](int kt, int stage) __attribute__((always_inline)) {
    if (!issuer) return;
    const unsigned base = lds0 + B_BASE + stage * B_BYTES;
#pragma unroll
    for (int i = 0; i < B_PWI; ++i) {
      const bool up = GLU && (wi * B_PWI + i) * RPD >= BNO;
      if (b_nt)
        dma16_nt(up ? b_desc1 : b_desc0, b_voff[i], kt * KB, base + (wi * B_PWI + i) * 1024);
      else
        dma16(up ? b_desc1 : b_desc0, b_voff[i], kt * KB, base + (wi * B_PWI + i) * 1024);
    }
  };
  constexpr int KS = KB / 32;
  int fo[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) fo[s] = (lane & 31) * KB + (((2 * s + (lane >> 5)) ^ swz<KB>(lane & 31)) * 16);

  {
    int src[A_PWI];
    load_src(t, src);
    set_a(t, src);
  }
  set_b(t);
  issue_a(0, 0);
  issue_b(0, 0);
  if (KT > 1) issue_b(1, 1);
  for (;;) {
    // The next tile's lookup and row indices, read while this tile's first K-tile is in flight
    // (the wait at K-tile 0 covers them).
    TileInfo tn;
    const bool has_next = assign_tile_after<BM, BNO>(p, tn, vb + (int)gridDim.x, mt_total, g_hint);
    int src_n[A_PWI];
    if (has_next) load_src(tn, src_n);
    const int na = min(WM, max(0, (((t.rows + 31) >> 5) - wm + WAVES_M - 1) / WAVES_M));
    f32x16 acc[WM][WN];
    zero_acc(acc);
    dispatch_na<WM>(na, [&](auto na_c) __attribute__((always_inline)) {
      constexpr int NA = decltype(na_c)::value;
      // Issue order per K-tile kt: A(kt+1), then B(kt+2); when A(kt) has landed only B(kt+1) can
      // still be in flight (loads complete in issue order).
      for (int kt = 0; kt < KT; ++kt) {
        if (issuer) {  // the other waves issue no loads
          if (kt == 0 || kt + 1 >= KT) wait_vmcnt<0>();
          else wait_vmcnt<B_PWI>();
        }
        __syncthreads();  // every wave's part has landed; A stage (kt+1)%2 and B stage (kt+2)%3 are free
        if (kt + 1 < KT) issue_a(kt + 1, (kt + 1) & 1);
        if (kt + 2 < KT) issue_b(kt + 2, (kt + 2) % 3);
        if (NA > 0)
          dma_ktile<TI, WAVES_M, WAVES_N, WM, WN, KB, GLU, false, NA>(smem + (kt & 1) * A_BYTES,
                                                                     smem + B_BASE + (kt % 3) * B_BYTES, fo, wm, wn,
                                                                     lane, acc);
      }
    });
    __syncthreads();  // every wave is done reading the pipeline stages
    if (has_next) {
      set_b(tn);
      issue_b(0, 0);
      if (KT > 1) issue_b(1, 1);
    }
    char* region = smem + wave * REGION;
    if (p.c_dtype == LMOE_BF16)
      epilogue_staged<TI, uint16_t, WAVES_M, WAVES_N, WM, WN, EPI, REGION, NTC>(p, t, acc, wm, wn, lane, na, region);
    else
      epilogue_staged<TI, float, WAVES_M, WAVES_N, WM, WN, EPI, REGION, NTC>(p, t, acc, wm, wn, lane, na, region);
    if (!has_next) break;
    __syncthreads();  // every wave is done with its staging region: the A stages take the next tile
    set_a(tn, src_n);
    issue_a(0, 0);
    t = tn;
    vb += (int)gridDim.x;
  }
}

// ------------------------------------------------------------------------------------------------
// MX pipeline: FP8 (E4M3) A x FP4 (E2M1) B with E8M0 scales per 32 k, on
// v_mfma_scale_f32_32x32x64_f8f6f4 (the block scales are applied inside the MFMA)
// ------------------------------------------------------------------------------------------------
// Same 256x256 tiles, DMA ring and XCD-contiguous numbering as the bf16 DMA pipeline, with a K-tile
// of 128 k: 128 bytes of every A row, 64 bytes of every B row and one dword of four scale bytes per
// row of each, so a K-tile is 7 DMA instructions per wave and 50 KB of LDS. A K-tile carries half
// the bytes of a bf16 one for the same MFMA time, so the ring holds three (measured: 4 % faster than
// two). Operand layout of the 32x32x64 step
// (lane l: row or column l % 32, half h = l / 32):
//   A fp8: bytes 0..15 hold k in [16h, 16h + 16), bytes 16..31 k in [32 + 16h, 48 + 16h) -- two
//          16-byte LDS reads, chunks h and h + 2 of the step's 64 bytes;
//   B fp4: 16 bytes, 32 nibbles (low nibble first) of k in [32h, 32h + 32) -- chunk h of the
//          step's 32 bytes;
//   scales: lane (r, h) supplies the scale of 32-k block h of the step for row (column) r.
// A and B rows carry the same swizzle as the bf16 pipeline (key r/2 % 8 for 128-byte rows, r/4 % 4
// for 64-byte rows), which keeps both fragment reads free of bank conflicts.
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ inline void dma4(const u32x4& desc, int voff, int soff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(desc), "s"(soff)
               : "memory", "m0");
}

constexpr int kMxK = 128;     // k per K-tile of the MX pipeline
constexpr int kMxStages = 3;  // 150 KB of LDS: two K-tiles in flight while a third is consumed

template <int WAVES_M, int WAVES_N, int WM, int WN, int NS, Epi EPI, bool DS = true>
__global__ void __launch_bounds__(WAVES_M* WAVES_N* kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_mx_kernel(GemmArgs p) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int BM = WAVES_M * WM * 32;
  constexpr int BNB = WAVES_N * WN * 32;
  constexpr bool GLU = EPI == Epi::Glu;
  static_assert(EPI == Epi::Store || GLU, "MX pipeline: plain or GLU stores");
  static_assert(!GLU || WN % 2 == 0, "GLU needs gate/up column-block pairs");
  constexpr int BNO = GLU ? BNB / 2 : BNB;
  constexpr int KA = kMxK, KBB = kMxK / 2;   // bytes per row per K-tile: A (fp8), B (fp4)
  constexpr int RPA = 1024 / KA, RPB = 1024 / KBB;
  constexpr int A_PW = BM / RPA / NW, B_PW = BNB / RPB / NW;
  static_assert(A_PW * RPA * NW == BM && B_PW * RPB * NW == BNB, "DMA split");
  static_assert(!GLU || BNO % RPB == 0, "a DMA block stays in one GLU half");
  constexpr int SA_N = BM / 64, SB_N = BNB / 64;  // scale dword DMAs per K-tile (64 rows each)
  static_assert(SA_N + SB_N == NW, "one scale DMA per wave");
  // DS: as in the bf16 pipeline, the upper half of the waves issues every DMA of a K-tile (twice
  // the blocks and two scale DMAs each) while the lower half goes straight to its MFMAs (the MX
  // GEMM1 only: measured at K3 prefill, 4-5 % faster there and 6 % slower on GEMM2).
  static_assert(!DS || NW % 2 == 0, "issue split needs an even wave count");
  constexpr int NI = DS ? 2 : 1;  // share of the K-tile's DMA blocks per issuing wave
  static_assert(!GLU || BNO % 64 == 0, "a scale DMA stays in one GLU half");
  constexpr int A_BYTES = BM * KA, B_BYTES = BNB * KBB;
  constexpr int STAGE = A_BYTES + B_BYTES + (BM + BNB) * 4;
  static_assert(STAGE % 1024 == 0, "stage alignment");
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];

  TileInfo t;
  if (!assign_tile<BM, BNO>(p, t, blockIdx.x)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int na = min(WM, max(0, (((t.rows + 31) >> 5) - wm + WAVES_M - 1) / WAVES_M));

  // byte strides: codes (A fp8: K bytes a row, B fp4: K/2), scales K/32 bytes a row
  const int64_t a_ld = p.lda, b_ld = p.ldb, s_ld = p.K / 32;
  const char* Bb = static_cast<const char*>(p.B) + (int64_t)t.g * p.b_gstride;
  const char* Sb = reinterpret_cast<const char*>(p.b_scale) + (int64_t)t.g * p.b_scale_gstride;
  const int ncols = min(BNO, p.N - t.n0);
  const bool gather = p.a_rows != nullptr;
  const u32x4 a_desc = gather ? make_desc(p.A, (int)(p.a_nrows * a_ld))
                              : make_desc(static_cast<const char*>(p.A) + (int64_t)t.row0 * a_ld, (int)(t.rows * a_ld));
  const u32x4 as_desc = gather ? make_desc(p.a_scale, (int)(p.a_nrows * s_ld))
                               : make_desc(p.a_scale + (int64_t)t.row0 * s_ld, (int)(t.rows * s_ld));
  const u32x4 b_desc0 = make_desc(Bb + (int64_t)t.n0 * b_ld, (int)(ncols * b_ld));
  const u32x4 b_desc1 = GLU ? make_desc(Bb + (int64_t)(p.glu_up_off + t.n0) * b_ld, (int)(ncols * b_ld)) : b_desc0;
  const u32x4 bs_desc0 = make_desc(Sb + (int64_t)t.n0 * s_ld, (int)(ncols * s_ld));
  const u32x4 bs_desc1 =
      GLU ? make_desc(Sb + (int64_t)(p.glu_up_off + t.n0) * s_ld, (int)(ncols * s_ld)) : bs_desc0;
  const int KT = p.K / kMxK;

  auto a_src = [&](int r) __attribute__((always_inline)) {  // source row of tile row r, or -1
    if (!gather) return r;
    const int src = r < t.rows ? p.a_rows[t.row0 + r] : -1;
    return (src >= 0 && src < p.a_nrows) ? src : -1;
  };
  const bool issuer = !DS || wave >= NW / 2;
  const int wi = DS ? (issuer ? wave - NW / 2 : 0) : wave;  // index among the issuing waves
  int a_voff[NI * A_PW], b_voff[NI * B_PW];
  {
    const int lr = lane / (KA / 16), slot = lane % (KA / 16);
#pragma unroll
    for (int i = 0; i < NI * A_PW; ++i) {
      const int r = (wi * NI * A_PW + i) * RPA + lr;
      const int src = a_src(r);
      a_voff[i] = src >= 0 ? src * (int)a_ld + ((slot ^ swz<KA>(r)) * 16) : kOutOfRange;
    }
  }
  {
    const int lr = lane / (KBB / 16), slot = lane % (KBB / 16);
#pragma unroll
    for (int i = 0; i < NI * B_PW; ++i) {
      const int r = (wi * NI * B_PW + i) * RPB + lr;
      b_voff[i] = (r % BNO) * (int)b_ld + ((slot ^ swz<KBB>(r)) * 16);
    }
  }
  // scale DMAs of this wave: scale block sw covers A rows [64 sw, 64 sw + 64) for sw < SA_N, else
  // B rows [64 (sw - SA_N), ...); an issuing wave takes blocks NI wi .. NI wi + NI - 1
  u32x4 s_desc[NI];
  int s_voff[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int sw = NI * wi + q;
    if (sw < SA_N) {
      const int src = a_src(sw * 64 + lane);
      s_desc[q] = as_desc;
      s_voff[q] = src >= 0 ? src * (int)s_ld : kOutOfRange;
    } else {
      const int r = (sw - SA_N) * 64 + lane;
      s_desc[q] = (GLU && (sw - SA_N) * 64 >= BNO) ? bs_desc1 : bs_desc0;
      s_voff[q] = (r % BNO) * (int)s_ld;
    }
  }
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(
      (unsigned)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));

  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    if (!issuer) return;
    const unsigned base = lds0 + stage * STAGE;
#pragma unroll
    for (int i = 0; i < NI * A_PW; ++i) dma16(a_desc, a_voff[i], kt * KA, base + (wi * NI * A_PW + i) * 1024);
#pragma unroll
    for (int i = 0; i < NI * B_PW; ++i) {
      const bool up = GLU && (wi * NI * B_PW + i) * RPB >= BNO;
      dma16(up ? b_desc1 : b_desc0, b_voff[i], kt * KBB, base + A_BYTES + (wi * NI * B_PW + i) * 1024);
    }
#pragma unroll
    for (int q = 0; q < NI; ++q) dma4(s_desc[q], s_voff[q], kt * 4, base + A_BYTES + B_BYTES + (NI * wi + q) * 256);
  };
  constexpr int PER_TILE = NI * (A_PW + B_PW + 1);  // DMA instructions per issuing wave per K-tile
  auto wait_tiles_after = [&](int n) __attribute__((always_inline)) {
    if (NS > 3 && n >= 2) wait_vmcnt<2 * PER_TILE>();
    else if (NS > 2 && n == 1) wait_vmcnt<PER_TILE>();
    else wait_vmcnt<0>();
  };

  f32x16 acc[WM][WN];
  zero_acc(acc);
  const int h = lane >> 5, r32 = lane & 31;
  int foa[2][2], fob[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    foa[s][0] = r32 * KA + (((4 * s + h) ^ swz<KA>(r32)) * 16);
    foa[s][1] = r32 * KA + (((4 * s + 2 + h) ^ swz<KA>(r32)) * 16);
    fob[s] = r32 * KBB + (((2 * s + h) ^ swz<KBB>(r32)) * 16);
  }

  dispatch_na<WM>(na, [&](auto na_c) __attribute__((always_inline)) {
    constexpr int NA = decltype(na_c)::value;
    constexpr int NAR = NA > 0 ? NA : 1;
    auto compute = [&](int stage) __attribute__((always_inline)) {
      const char* base = smem + stage * STAGE;
      const uint32_t* sA = reinterpret_cast<const uint32_t*>(base + A_BYTES + B_BYTES);
      const uint32_t* sB = sA + BM;
      uint32_t sa[NAR], sb[WN];  // the four block scales of this K-tile, lane half's block in byte 0
#pragma unroll
      for (int i = 0; i < NA; ++i) sa[i] = sA[(i * WAVES_M + wm) * 32 + r32] >> (8 * h);
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int ocb = (j % (GLU ? WN / 2 : WN)) * WAVES_N + wn;
        const int bblk = (GLU && j >= WN / 2) ? BNO / 32 + ocb : ocb;
        sb[j] = sB[bblk * 32 + r32] >> (8 * h);
      }
      uint4 af[2][NAR][2], bf[2][WN];
      auto load = [&](int s, uint4 (&a)[NAR][2], uint4 (&b)[WN]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          const char* ab = base + (i * WAVES_M + wm) * 32 * KA;
          a[i][0] = *reinterpret_cast<const uint4*>(ab + foa[s][0]);
          a[i][1] = *reinterpret_cast<const uint4*>(ab + foa[s][1]);
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const int ocb = (j % (GLU ? WN / 2 : WN)) * WAVES_N + wn;
          const int bblk = (GLU && j >= WN / 2) ? BNO / 32 + ocb : ocb;
          b[j] = *reinterpret_cast<const uint4*>(base + A_BYTES + bblk * 32 * KBB + fob[s]);
        }
      };
      load(0, af[0], bf[0]);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s == 0) load(1, af[1], bf[1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          const uint4 lo = af[s][i][0], hi = af[s][i][1];
          const i32x8 av = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          const int sca = (int)((sa[i] >> (16 * s)) & 0xffu);
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            const uint4 bq = bf[s][j];
            const i32x8 bv = {(int)bq.x, (int)bq.y, (int)bq.z, (int)bq.w, 0, 0, 0, 0};
            const int scb = (int)((sb[j] >> (16 * s)) & 0xffu);
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 0, 4, 0, sca, 0, scb);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    const int pre = min(KT, NS - 1);
    for (int kt = 0; kt < pre; ++kt) issue(kt, kt);
    for (int kt = 0; kt < KT; ++kt) {
      wait_tiles_after(min(KT - kt - 1, NS - 2));
      __syncthreads();
      if (kt + NS - 1 < KT) issue(kt + NS - 1, (kt + NS - 1) % NS);
      if (NA > 0) compute(kt % NS);
    }
  });
  constexpr int REGION = NS * STAGE / NW;
  if (p.N % 8 == 0 && p.ldc % 8 == 0) {
    __syncthreads();
    epilogue_staged<uint16_t, uint16_t, WAVES_M, WAVES_N, WM, WN, EPI, REGION>(p, t, acc, wm, wn, lane, na,
                                                                             smem + wave * REGION);
    return;
  }
  epilogue<uint16_t, WAVES_M, WAVES_N, WM, WN, EPI>(p, t, acc, wm, wn, lane, na);
}

// ------------------------------------------------------------------------------------------------
// register pipeline: 128x128 tiles, one K-tile of loads in flight, two padded LDS stages
// ------------------------------------------------------------------------------------------------
constexpr int kRowPitch = 144;

template <typename TI, int WAVES_M, int WAVES_N, int WM, int WN, Epi EPI>
__global__ void __launch_bounds__(WAVES_M* WAVES_N* kWave) gemm_reg_kernel(GemmArgs p_in) {
  GemmArgs p = p_in;
  if (p.splits > 1) {  // this workgroup's K-chunk, as a plain GEMM over K = chunk into its own partial
    const int s = blockIdx.y, s1 = p.K1 / p.K;
    if (s < s1) {
      p.A = static_cast<const char*>(p.A) + (int64_t)((s * p.K) % p.a_kwrap) * (int64_t)sizeof(TI);
      p.B = static_cast<const char*>(p.B) + (int64_t)s * p.K * (int64_t)sizeof(TI);
    } else {
      p.A = static_cast<const char*>(p.A2) + (int64_t)(s - s1) * p.K * (int64_t)sizeof(TI);
      p.lda = p.lda2;
      p.B = static_cast<const char*>(p.B2) + (int64_t)(s - s1) * p.K * (int64_t)sizeof(TI);
      p.ldb = p.ldb2;
    }
    p.A2 = nullptr;
    p.K1 = p.K;
    p.a_kwrap = p.K;
    p.C = static_cast<float*>(p.C) + s * p.c_split;
  }
  constexpr int NT = WAVES_M * WAVES_N * kWave;
  constexpr int BM = WAVES_M * WM * 32;
  constexpr int BNB = WAVES_N * WN * 32;
  constexpr bool GLU = EPI == Epi::Glu || EPI == Epi::GluBwd;
  static_assert(!GLU || WN % 2 == 0, "GLU needs gate/up column-block pairs");
  constexpr int BNO = GLU ? BNB / 2 : BNB;
  constexpr int WNO = GLU ? WN / 2 : WN;
  constexpr int A_PER = BM * 8 / NT;
  constexpr int B_PER = BNB * 8 / NT;
  static_assert(A_PER * NT == BM * 8 && B_PER * NT == BNB * 8, "chunk split");
  static_assert(!GLU || BNO % (NT / 8) == 0, "a B chunk index must stay in one GLU half");
  constexpr int A_BYTES = BM * kRowPitch;
  constexpr int STAGE = (BM + BNB) * kRowPitch;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  TileInfo t;
  if (!assign_tile<BM, BNO>(p, t, blockIdx.x)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int na = min(WM, max(0, (((t.rows + 31) >> 5) - wm + WAVES_M - 1) / WAVES_M));

  const int64_t a_ld = p.lda * (int64_t)sizeof(TI), b_ld = p.ldb * (int64_t)sizeof(TI);
  const int64_t a_ld2 = p.lda2 * (int64_t)sizeof(TI), b_ld2 = p.ldb2 * (int64_t)sizeof(TI);
  const char* Bb = static_cast<const char*>(p.B) + (int64_t)t.g * p.b_gstride * (int64_t)sizeof(TI) +
                   (int64_t)t.k0 * (int64_t)sizeof(TI);
  const int ncols = min(BNO, p.N - t.n0);
  const bool gather = p.a_rows != nullptr;
  const bool seg2 = !GLU && p.A2 != nullptr;
  const __amdgpu_buffer_rsrc_t a_rsrc =
      gather ? make_rsrc(p.A, (int)(p.a_nrows * a_ld))
             : make_rsrc(static_cast<const char*>(p.A) + (int64_t)t.row0 * a_ld + (int64_t)t.k0 * (int64_t)sizeof(TI),
                         (int)(t.rows * a_ld));
  const __amdgpu_buffer_rsrc_t b_rsrc0 = make_rsrc(Bb + (int64_t)t.n0 * b_ld, (int)(ncols * b_ld));
  const __amdgpu_buffer_rsrc_t b_rsrc1 =
      GLU ? make_rsrc(Bb + (int64_t)(p.glu_up_off + t.n0) * b_ld, (int)(ncols * b_ld)) : b_rsrc0;
  const __amdgpu_buffer_rsrc_t a2_rsrc =
      seg2 ? make_rsrc(static_cast<const char*>(p.A2) + (int64_t)t.row0 * a_ld2, (int)(t.rows * a_ld2)) : a_rsrc;
  const __amdgpu_buffer_rsrc_t b2_rsrc =
      seg2 ? make_rsrc(static_cast<const char*>(p.B2) + (int64_t)t.n0 * b_ld2, (int)(ncols * b_ld2)) : b_rsrc0;
  const int a_wrap = p.a_kwrap * (int)sizeof(TI);
  const int KT = t.klen * (int)sizeof(TI) / 128;
  const int KT1 = p.K1 * (int)sizeof(TI) / 128;

  int a_voff[A_PER], b_voff[B_PER], a2_voff[A_PER], b2_voff[B_PER];
  // B stored [K, N]: each thread loads pairs of rows (2 kap, 2 kap + 1) of one 16-byte column chunk
  // nc and writes them transposed into the [n][k] LDS layout, two k per 32-bit word (bf16) or as a
  // k pair (f32). Pair p of this thread: kap = p % 8 + 8 * (p / (8 * CPR)), nc = (p / 8) % CPR.
  constexpr int KE = 128 / (int)sizeof(TI);          // k per K-tile
  constexpr int CPR = BNB * (int)sizeof(TI) / 16;    // 16-byte chunks per row of the B tile
  constexpr int NPAIR = KE / 2 * CPR / NT;           // pairs per thread
  static_assert(!(KE / 2 * CPR % NT) && 2 * NPAIR <= B_PER, "B pair split");
  const bool bkn = p.b_kn;
  const __amdgpu_buffer_rsrc_t b_rsrc_kn =
      make_rsrc(Bb + (int64_t)t.n0 * (int64_t)sizeof(TI),
                (int)((int64_t)p.K * b_ld - (int64_t)t.n0 * (int64_t)sizeof(TI)));
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int c = tid + i * NT, r = c >> 3;
    if (gather) {
      const int src = r < t.rows ? p.a_rows[t.row0 + r] : -1;
      a_voff[i] = (src >= 0 && src < p.a_nrows) ? src * (int)a_ld + (c & 7) * 16 : kOutOfRange;
    } else {
      a_voff[i] = r * (int)a_ld + (c & 7) * 16;
    }
    a2_voff[i] = r * (int)a_ld2 + (c & 7) * 16;
  }
#pragma unroll
  for (int i = 0; i < B_PER; ++i) {
    const int c = tid + i * NT;
    b_voff[i] = ((c >> 3) % BNO) * (int)b_ld + (c & 7) * 16;
    b2_voff[i] = ((c >> 3) % BNO) * (int)b_ld2 + (c & 7) * 16;
  }

  uint4 ra[A_PER], rb[B_PER];
  int ka = 0;  // byte offset of the next K-tile inside A's (possibly wrapped) row
  auto gload = [&](int kt) __attribute__((always_inline)) {
    if (bkn) {
#pragma unroll
      for (int i = 0; i < A_PER; ++i) ra[i] = buffer_load16(a_rsrc, a_voff[i], ka);
#pragma unroll
      for (int q = 0; q < NPAIR; ++q) {
        const int pp = tid + q * NT;
        const int kap = pp % 8 + 8 * (pp / (8 * CPR)), nc = (pp / 8) % CPR;
        const int voff = 2 * kap * (int)b_ld + nc * 16;
        const int soff = kt * KE * (int)b_ld;
        rb[2 * q] = buffer_load16(b_rsrc_kn, voff, soff);
        rb[2 * q + 1] = buffer_load16(b_rsrc_kn, voff + (int)b_ld, soff);
      }
      ka += 128;
      if (ka == a_wrap) ka = 0;
    } else if (!seg2 || kt < KT1) {
#pragma unroll
      for (int i = 0; i < A_PER; ++i) ra[i] = buffer_load16(a_rsrc, a_voff[i], ka);
#pragma unroll
      for (int i = 0; i < B_PER; ++i)
        rb[i] = buffer_load16((GLU && (i * NT / 8) >= BNO) ? b_rsrc1 : b_rsrc0, b_voff[i], kt * 128);
      ka += 128;
      if (ka == a_wrap) ka = 0;
    } else {
      const int kk = (kt - KT1) * 128;
#pragma unroll
      for (int i = 0; i < A_PER; ++i) ra[i] = buffer_load16(a2_rsrc, a2_voff[i], kk);
#pragma unroll
      for (int i = 0; i < B_PER; ++i) rb[i] = buffer_load16(b2_rsrc, b2_voff[i], kk);
    }
  };
  auto lstore = [&](int stage) __attribute__((always_inline)) {
    char* base = smem + stage * STAGE;
    if (bkn) {
#pragma unroll
      for (int i = 0; i < A_PER; ++i) {
        const int c = tid + i * NT;
        *reinterpret_cast<uint4*>(base + (c >> 3) * kRowPitch + (c & 7) * 16) = ra[i];
      }
#pragma unroll
      for (int q = 0; q < NPAIR; ++q) {
        const int pp = tid + q * NT;
        const int kap = pp % 8 + 8 * (pp / (8 * CPR)), nc = (pp / 8) % CPR;
        const uint32_t* lo = reinterpret_cast<const uint32_t*>(&rb[2 * q]);
        const uint32_t* hi = reinterpret_cast<const uint32_t*>(&rb[2 * q + 1]);
        if constexpr (sizeof(TI) == 2) {  // 8 columns per chunk; word = (k even, k odd) of one column
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t a = (lo[j >> 1] >> (16 * (j & 1))) & 0xffffu, b = (hi[j >> 1] >> (16 * (j & 1))) & 0xffffu;
            *reinterpret_cast<uint32_t*>(base + A_BYTES + (nc * 8 + j) * kRowPitch + kap * 4) = a | (b << 16);
          }
        } else {  // 4 columns per chunk; (k even, k odd) of one column as 8 bytes
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<uint2*>(base + A_BYTES + (nc * 4 + j) * kRowPitch + kap * 8) = make_uint2(lo[j], hi[j]);
        }
      }
      return;
    }
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

  f32x16 acc[WM][WN];
  zero_acc(acc);
  const int frag_off = (lane & 31) * kRowPitch + (lane >> 5) * 16;
  dispatch_na<WM>(na, [&](auto na_c) __attribute__((always_inline)) {
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
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) gload(kt + 1);
      if (NA > 0) compute(kt & 1);
      if (kt + 1 < KT) lstore((kt + 1) & 1);
      __syncthreads();
    }
  });
  epilogue<TI, WAVES_M, WAVES_N, WM, WN, EPI>(p, t, acc, wm, wn, lane, na);
}

// Sums the split-K partials (in split order) and applies the epilogue of the unsplit GEMM; four
// consecutive outputs of one row per thread. GLU partials hold the gate columns, then the up columns.
template <Epi EPI, bool ACCURATE>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmArgs p, const float* __restrict__ part, int splits,
                                                            int64_t stride, int n_cols) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (int64_t)p.M * p.N) return;
  const int64_t m = i / p.N;
  const int c = (int)(i - m * p.N);
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f}, u[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const float* pr = part + m * n_cols + c;
  for (int s = 0; s < splits; ++s) {
    const float4 a = *reinterpret_cast<const float4*>(pr + s * stride);
    v[0] += a.x;
    v[1] += a.y;
    v[2] += a.z;
    v[3] += a.w;
    if constexpr (EPI == Epi::Glu) {
      const float4 b = *reinterpret_cast<const float4*>(pr + s * stride + p.N);
      u[0] += b.x;
      u[1] += b.y;
      u[2] += b.z;
      u[3] += b.w;
    }
  }
  const float inv_b1 = 1.0f / p.beta1, inv_b2 = 1.0f / p.beta2;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t off = m * p.ldc + c + q;
    if constexpr (EPI == Epi::Store) {
      store_out(p, off, v[q]);
    } else if constexpr (EPI == Epi::Glu) {
      store_out(p, off, situ_glu<ACCURATE>(v[q], u[q], p.beta1, inv_b1, p.beta2, inv_b2));
    } else if constexpr (EPI == Epi::Sigmoid) {
      const float x = v[q] + (p.col_bias ? p.col_bias[c + q] : 0.0f);
      static_cast<float*>(p.C)[off] = 1.0f / (1.0f + expf(-x));
    } else {
      store_out(p, off, v[q] + p.residual[m * p.ldr + c + q]);
    }
  }
}

template <Epi EPI, bool ACCURATE>
void launch_reduce(dim3 grid, hipStream_t s, const GemmArgs& a, const float* part, int splits, int64_t stride,
                   int n_cols) {
  hipLaunchKernelGGL((splitk_reduce_kernel<EPI, ACCURATE>), grid, dim3(256), 0, s, a, part, splits, stride, n_cols);
}

int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// ------------------------------------------------------------------------------------------------
// launch
// ------------------------------------------------------------------------------------------------
template <int BM, int BNB>
int64_t grid_blocks(const GemmArgs& a, Epi epi) {
  const int bno = (epi == Epi::Glu || epi == Epi::GluBwd) ? BNB / 2 : BNB;
  const int64_t n_tiles = ceil_div(a.N, bno);
  const int64_t m_tiles = a.koff   ? (int64_t)a.G * ceil_div(a.M, BM)
                          : a.goff ? (int64_t)a.M / BM + a.G  // upper bound if grouped
                                   : ceil_div(a.M, BM);
  return ceil_div(m_tiles * n_tiles, kXcds) * kXcds;
}

#define LMOE_LAUNCH_EPI(KERNEL, ...)                                                                              \
  switch (epi) {                                                                                                  \
    case Epi::Store: hipLaunchKernelGGL((KERNEL<__VA_ARGS__, Epi::Store>), grid, block, 0, s, a); break;         \
    case Epi::Glu: hipLaunchKernelGGL((KERNEL<__VA_ARGS__, Epi::Glu>), grid, block, 0, s, a); break;             \
    case Epi::Sigmoid: hipLaunchKernelGGL((KERNEL<__VA_ARGS__, Epi::Sigmoid>), grid, block, 0, s, a); break;     \
    case Epi::AddF32: hipLaunchKernelGGL((KERNEL<__VA_ARGS__, Epi::AddF32>), grid, block, 0, s, a); break;       \
    case Epi::GluBwd: hipLaunchKernelGGL((KERNEL<__VA_ARGS__, Epi::GluBwd>), grid, block, 0, s, a); break;       \
  }

constexpr int kDmaStages = 2;    // LDS stages of the DMA pipeline
constexpr int kDmaKBytes = 128;  // bytes of every row per K-tile (64 bf16)

// The persistent routed kernel covers grouped GEMMs over whole K (no K groups, splits or second
// segment, A not wrapped) whose outputs take the staged epilogue.
bool routed_persistent(const GemmArgs& a) {
  const int vec = a.c_dtype == LMOE_BF16 ? 8 : 4;
  return a.goff && !a.koff && !a.A2 && !a.b_kn && a.splits <= 1 && a.a_kwrap == a.K && a.N % vec == 0 &&
         a.ldc % vec == 0;
}

// One workgroup per CU (a multiple of the XCD count), at most one per tile.
template <typename TI, Epi EPI, bool NTC>
hipError_t launch_routed(const GemmArgs& a, int64_t blocks, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t per_chip = cus >= kXcds ? cus / kXcds * kXcds : kXcds;
  const dim3 grid((unsigned)(blocks < per_chip ? blocks : per_chip)), block(8 * kWave);
  hipLaunchKernelGGL((gemm_routed_kernel<TI, 2, 4, 4, 2, kDmaKBytes, EPI, NTC>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <typename TI>
hipError_t launch_big(const GemmArgs& a, Epi epi, hipStream_t s) {
  const int64_t blocks = grid_blocks<256, 256>(a, epi);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(8 * kWave);
  if (a.b_kn) {
    if constexpr (sizeof(TI) == 2)
      hipLaunchKernelGGL((gemm_dma_kernel<TI, 2, 4, 4, 2, kDmaStages, kDmaKBytes, Epi::Store, true>), grid, block, 0, s,
                         a);
    return hipGetLastError();
  }
  // The routed experts' GEMMs stream their weights (B) from HBM once: B runs a three-stage ring
  // one K-tile further ahead than A (measured at K3 prefill: GEMM1 1.43 -> 1.29 ms, GEMM2 0.92 ->
  // 0.90 ms; the backward's recomputed GEMM1 2.69 -> 2.58 ms; the dense GEMMs, whose B comes from
  // L2, the router's split-K halves and the [K, N]-B products lose 1-5 % with it and keep two stages).
  if (epi == Epi::Glu && a.goff) {  // routed GEMM1: W1 slices streamed with the non-temporal hint
    if (routed_persistent(a)) return launch_routed<TI, Epi::Glu, false>(a, blocks, s);
    hipLaunchKernelGGL((gemm_dma_kernel<TI, 2, 4, 4, 2, kDmaStages, kDmaKBytes, Epi::Glu, false, true, 1>), grid,
                       block, 0, s, a);
    return hipGetLastError();
  }
  if (epi == Epi::GluBwd && a.goff && !a.koff) {  // backward: routed GEMM1 recomputed, W1 streamed
    hipLaunchKernelGGL((gemm_dma_kernel<TI, 2, 4, 4, 2, kDmaStages, kDmaKBytes, Epi::GluBwd, false, false, 1>), grid,
                       block, 0, s, a);
    return hipGetLastError();
  }
  if (epi == Epi::Store && a.goff && !a.koff && !a.A2 && a.splits <= 1) {  // routed GEMM2: W2 in, y out, non-temporal
    if (routed_persistent(a)) return launch_routed<TI, Epi::Store, true>(a, blocks, s);
    hipLaunchKernelGGL((gemm_dma_kernel<TI, 2, 4, 4, 2, kDmaStages, kDmaKBytes, Epi::Store, false, true, 1, true>),
                       grid, block, 0, s, a);
    return hipGetLastError();
  }
  LMOE_LAUNCH_EPI(gemm_dma_kernel, TI, 2, 4, 4, 2, kDmaStages, kDmaKBytes)
  return hipGetLastError();
}

template <typename TI>
hipError_t launch_small(const GemmArgs& a, Epi epi, hipStream_t s) {
  const int64_t blocks = grid_blocks<128, 128>(a, epi);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(4 * kWave);
  LMOE_LAUNCH_EPI(gemm_reg_kernel, TI, 2, 2, 2, 2)
  return hipGetLastError();
}
#undef LMOE_LAUNCH_EPI

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

// Split only when the 128x128 tiles cover less than half the CUs: the largest K-chunk (whole
// register K-tiles, at least four, dividing both K segments and the A wrap period) that gives about
// 256 workgroups, at most 64 splits.
SplitPlan plan_split_k(int64_t M, int64_t n_cols, int K1, int K2, int a_kwrap, int esz) {
  SplitPlan none;
  if (M <= 0 || n_cols <= 0 || n_cols % 4 != 0 || K1 <= 0 || K2 < 0 || a_kwrap <= 0) return none;
  const int64_t tiles = ceil_div(M, 128) * ceil_div(n_cols, 128);
  if (tiles >= 128) return none;
  const int gran = 128 / esz;  // elements of one register K-tile
  int g = gcd_int(K1, a_kwrap);
  if (K2 > 0) g = gcd_int(g, K2);
  if (g % gran) return none;
  const int want = (int)ceil_div(256, tiles);
  SplitPlan best;
  for (int c = g; c >= 4 * gran; c -= gran) {
    if (g % c) continue;
    const int n = (K1 + K2) / c;
    if (n > 64) break;
    best.splits = n;
    best.chunk = c;
    if (n >= want) break;
  }
  return best.splits >= 2 ? best : none;
}

SplitPlan plan_split_k_big(int64_t M, int64_t n_cols, int K1, int K2, int esz) {
  SplitPlan none;
  if (esz != 2 || M <= 0 || n_cols <= 0 || n_cols % 4 != 0 || K1 <= 0 || K2 != 0) return none;
  const int64_t tiles = ceil_div(M, 256) * ceil_div(n_cols, 256);
  if (tiles >= 256 || tiles < 64) return none;
  const int gran = kDmaKBytes / esz;  // elements of one DMA K-tile
  for (int n = (int)ceil_div(256, tiles); n <= 4; ++n) {
    if (K1 % n || (K1 / n) % gran || K1 / n < 4 * gran) continue;
    SplitPlan sp;
    sp.splits = n;
    sp.chunk = K1 / n;
    sp.big = true;
    return sp;
  }
  return none;
}

size_t split_k_bytes(const SplitPlan& sp, int64_t M, int64_t n_cols) {
  return sp.splits > 1 ? (size_t)sp.splits * (size_t)M * (size_t)n_cols * sizeof(float) : 0;
}

hipError_t launch_gemm_split(const GemmArgs& a, int in_dtype, Epi epi, const SplitPlan& sp, float* partials,
                             hipStream_t s, bool reduce) {
  const bool glu = epi == Epi::Glu;
  const int n_cols = glu ? 2 * a.N : a.N;
  if (sp.splits < 2 || a.goff || a.koff || a.a_rows || epi == Epi::GluBwd || (glu && a.glu_up_off != a.N))
    return hipErrorInvalidValue;
  GemmArgs q = a;
  q.K1 = a.A2 ? a.K1 : a.K;  // end of the first K segment
  q.K = sp.chunk;
  q.splits = sp.splits;
  q.c_split = (int64_t)a.M * n_cols;
  q.C = partials;
  q.ldc = n_cols;
  q.c_dtype = LMOE_F32;
  q.N = n_cols;
  q.col_bias = nullptr;
  q.residual = nullptr;
  if (sp.big) {  // the DMA pipeline starts each split at its own offset inside A's wrapped row
    if (in_dtype != LMOE_BF16 || a.A2 || sp.chunk % (kDmaKBytes / 2)) return hipErrorInvalidValue;
    KernelTimer timer(a.tag ? a.tag : "gemm", s);
    const int64_t blocks = grid_blocks<256, 256>(q, Epi::Store);
    if (blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)blocks, (unsigned)sp.splits), block(8 * kWave);
    hipLaunchKernelGGL((gemm_dma_kernel<uint16_t, 2, 4, 4, 2, kDmaStages, kDmaKBytes, Epi::Store>), grid, block, 0, s,
                       q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    KernelTimer timer(a.tag ? a.tag : "gemm", s);
    const int64_t blocks = grid_blocks<128, 128>(q, Epi::Store);
    if (blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)blocks, (unsigned)sp.splits), block(4 * kWave);
    if (in_dtype == LMOE_BF16)
      hipLaunchKernelGGL((gemm_reg_kernel<uint16_t, 2, 2, 2, 2, Epi::Store>), grid, block, 0, s, q);
    else
      hipLaunchKernelGGL((gemm_reg_kernel<float, 2, 2, 2, 2, Epi::Store>), grid, block, 0, s, q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!reduce) return hipSuccess;
  KernelTimer timer("splitk_reduce", s);
  const int64_t quads = (int64_t)a.M * a.N / 4;
  const dim3 grid((unsigned)ceil_div(quads, 256));
  const int64_t stride = q.c_split;
  if (in_dtype == LMOE_F32) {
    switch (epi) {
      case Epi::Store: launch_reduce<Epi::Store, true>(grid, s, a, partials, sp.splits, stride, n_cols); break;
      case Epi::Glu: launch_reduce<Epi::Glu, true>(grid, s, a, partials, sp.splits, stride, n_cols); break;
      case Epi::Sigmoid: launch_reduce<Epi::Sigmoid, true>(grid, s, a, partials, sp.splits, stride, n_cols); break;
      case Epi::AddF32: launch_reduce<Epi::AddF32, true>(grid, s, a, partials, sp.splits, stride, n_cols); break;
    }
  } else {
    switch (epi) {
      case Epi::Store: launch_reduce<Epi::Store, false>(grid, s, a, partials, sp.splits, stride, n_cols); break;
      case Epi::Glu: launch_reduce<Epi::Glu, false>(grid, s, a, partials, sp.splits, stride, n_cols); break;
      case Epi::Sigmoid: launch_reduce<Epi::Sigmoid, false>(grid, s, a, partials, sp.splits, stride, n_cols); break;
      case Epi::AddF32: launch_reduce<Epi::AddF32, false>(grid, s, a, partials, sp.splits, stride, n_cols); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int in_dtype, Epi epi, GemmShape shape, hipStream_t s) {
  KernelTimer timer(a.tag ? a.tag : "gemm", s);
  if (a.b_kn) {  // B stored [K, N]: plain epilogues; the DMA pipeline takes bf16 stores only
    if ((epi != Epi::Store && epi != Epi::AddF32) || a.A2 || a.koff || a.splits > 1) return hipErrorInvalidValue;
    if (in_dtype != LMOE_BF16 || epi != Epi::Store) shape = GemmShape::Small;
  }
  if (in_dtype == LMOE_BF16)
    return shape == GemmShape::Big ? launch_big<uint16_t>(a, epi, s) : launch_small<uint16_t>(a, epi, s);
  return shape == GemmShape::Big ? launch_big<float>(a, epi, s) : launch_small<float>(a, epi, s);
}

// MX GEMM (bf16 output): A fp8 codes [rows, K] + scales [rows, K/32], B fp4 codes [N, K/2] + scales
// [N, K/32] per group; lda / ldb / b_gstride / b_scale_gstride in bytes; K a multiple of 128.
hipError_t launch_gemm_mx(const GemmArgs& a, Epi epi, hipStream_t s) {
  KernelTimer timer(a.tag ? a.tag : "gemm_mx", s);
  if ((epi != Epi::Store && epi != Epi::Glu) || a.K % kMxK || a.c_dtype != LMOE_BF16 || a.koff || a.A2 ||
      a.splits > 1 || a.b_kn || !a.a_scale || !a.b_scale)
    return hipErrorInvalidValue;
  const int64_t blocks = grid_blocks<256, 256>(a, epi);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(8 * kWave);
  if (epi == Epi::Glu)
    hipLaunchKernelGGL((gemm_mx_kernel<2, 4, 4, 2, kMxStages, Epi::Glu>), grid, block, 0, s, a);
  else
    // GEMM2's short K loop (4 K-tiles at K3 shape) loses with the issue split: 0.55-0.58 ms with
    // every wave issuing against 0.59-0.61 with the split; GEMM1 gains (0.66-0.69 vs 0.68-0.72)
    hipLaunchKernelGGL((gemm_mx_kernel<2, 4, 4, 2, kMxStages, Epi::Store, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mtile_prefix(const int32_t* goff, int G, int bm, int32_t* mtile_start, hipStream_t s) {
  KernelTimer timer("mtile_prefix", s);
  hipLaunchKernelGGL(mtile_prefix_kernel, dim3(1), dim3(1024), 0, s, goff, G, bm, mtile_start);
  return hipGetLastError();
}

}  // namespace lmoe
