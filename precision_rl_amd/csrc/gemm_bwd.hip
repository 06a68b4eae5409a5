// Steps b2-b6: the straight-through BF16 backward GEMMs on gfx950 (AI summary,
// "Methodology in Plain English": straight-through estimator on the saved
// original BF16 operands; miniTE Technical Report, section 4.3: BF16 backward
// through the layer bypass, no backward quantisation).
//
//   dgrad (M = dispatched rows of expert e, ragged):
//     b2: dA  = dO_e . W2[e]     K = H,  N = I, epilogue = SwiGLU backward (b4)
//     b5: dXp = dH_e . W1[e]     K = 2I, N = H
//   wgrad (K = dispatched rows of expert e, ragged, possibly empty):
//     b3: dW2[e] = dO_e^T . a_e            M = H,  N = I
//     b6: dW1[e] = dH_e^T . x[src_row]     M = 2I, N = H
//
// 256 x 256 output tile per workgroup of 8 waves (4 x 2, 64 x 128 per wave, two
// waves per SIMD), MFMA 32x32x16 bf16, FP32 accumulation.  K advances 64 per
// stage through double-buffered LDS holding both operands K-contiguous (row
// stride 144 B, conflict-free b128 fragment reads).  Waves 0-3 stage one
// operand and waves 4-7 the other, one stage ahead of the MFMAs.  Operands
// stored K-contiguous in HBM (dO, dH rows of the dgrad) are copied in 16 B
// chunks; operands stored the other way round (weights in the dgrad, both
// operands of the wgrad) are read as 8 x 8 bf16 micro-blocks, transposed in
// registers with v_perm_b32 and written as 16 B rows.  B's LDS rows are
// permuted so that each lane ends up owning 4 consecutive output columns
// (8 B stores in the epilogue).

#include "gemm_common.h"
#include "internal.h"

namespace w4a4 {
namespace {

constexpr int kBK = 64;
constexpr int kRowElems = kBK + 8;         // 72 bf16 = 144 B per LDS row
constexpr int kOpElems = kTileM * kRowElems;
constexpr int kStageElems = 2 * kOpElems;
constexpr int kLdsBytes = 2 * kStageElems * 2;  // 2 stages, bf16
constexpr int kLoaders = kGemmThreads / 2;      // threads staging one operand

// Global column of B staged into LDS row p: lane j of wave column wn owns
// columns n0 + wn*128 + 4j + {0,1,2,3} (one per MFMA tile ni).
__device__ __forceinline__ int b_lds_row_of_col(int c) {  // c = column offset in tile
  const int wn = c >> 7, rem = c & 127, j = rem >> 2, ni = rem & 3;
  return wn * 128 + ni * 32 + j;
}

struct Regs8 {
  u32x4_t v[8];
};

// 8 x 8 bf16 transpose: in.v[i] holds columns c..c+7 of k-row i; out.v[r]
// holds k-rows 0..7 of column c+r.
__device__ __forceinline__ void transpose8x8(const Regs8& in, Regs8& out) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t sel = (r & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      out.v[r][d] = __builtin_amdgcn_perm(in.v[2 * d + 1][r >> 1], in.v[2 * d][r >> 1], sel);
  }
}

// K-contiguous operand staged by 256 threads: chunk q = lt + 256 i (i < 8) is
// row q / 8, 16 B column q % 8 of the stage.
__device__ __forceinline__ void store_krows(uint16_t* s, int lt, const Regs8& r) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = lt + i * kLoaders;
    *reinterpret_cast<u32x4_t*>(s + (q >> 3) * kRowElems + (q & 7) * 8) = r.v[i];
  }
}

// Transposed operand staged by 256 threads: element (tile row p, k) lives at
// krow(k)[col0 + p].  Thread lt owns k-rows 8 (lt % 8) .. +7 and the 8 tile
// rows 8 cb .. +7, with cb = lt / 8 for A and cb = lt / 8 with bits 0 and 2
// swapped for B (whose LDS rows are permuted).  Either way the 16 lanes of one
// LDS write cycle hit 16 distinct 16-byte bank groups, and a wave's global
// loads cover 8 k-rows x 128 contiguous bytes.
template <bool PERMUTE_ROWS>
__device__ __forceinline__ int t_col_block(int lt) {
  const int g8 = lt >> 3;
  if constexpr (PERMUTE_ROWS) return (g8 & ~5) | ((g8 & 1) << 2) | ((g8 >> 2) & 1);
  return g8;
}
__device__ __forceinline__ int t_k_block(int lt) { return lt & 7; }

template <bool PERMUTE_ROWS>
__device__ __forceinline__ void store_transposed(uint16_t* s, int lt, const Regs8& in) {
  Regs8 out;
  transpose8x8(in, out);
  const int c0 = 8 * t_col_block<PERMUTE_ROWS>(lt), kb = 8 * t_k_block(lt);
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int p = PERMUTE_ROWS ? b_lds_row_of_col(c0 + r) : c0 + r;
    *reinterpret_cast<u32x4_t*>(s + p * kRowElems + kb) = out.v[r];
  }
}

__device__ __forceinline__ void mma_stage(const uint16_t* sa, const uint16_t* sb, int a_row0,
                                          int b_row0, int hl, floatx16_t (&acc)[2][4]) {
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    bf16x8_t af[2], bf[4];
#pragma unroll
    for (int f = 0; f < 2; ++f)
      af[f] = *reinterpret_cast<const bf16x8_t*>(sa + (a_row0 + f * 32) * kRowElems + ks * 16 + hl * 8);
#pragma unroll
    for (int f = 0; f < 4; ++f)
      bf[f] = *reinterpret_cast<const bf16x8_t*>(sb + (b_row0 + f * 32) * kRowElems + ks * 16 + hl * 8);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
  }
}

__device__ __forceinline__ void zero_acc(floatx16_t (&acc)[2][4]) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;
}

// ------------------------------------------------------------------ dgrad
enum class DgradMode { FC2_SWIGLU, FC1 };

struct DgradArgs {
  int64_t rows_alloc;
  int K, N, I, E;
  const int32_t* offsets;
  const uint16_t* g;   // [rows, K]   dO or dH
  const uint16_t* w;   // [E, K, N]   W2[e] ([H, I]) or W1[e] ([2I, H])
  const uint16_t* h;   // [rows, 2I]  saved FC1 output (FC2_SWIGLU)
  uint16_t* out;       // dH [rows, 2I] or dXp [rows, H]
};

template <DgradMode MODE>
__global__ void __launch_bounds__(kGemmThreads, 1)
dgrad_kernel(DgradArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  uint16_t* lds = reinterpret_cast<uint16_t*>(lds_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2, r32 = lane & 31, hl = lane >> 5;
  const int n_tiles = (args.N + kTileN - 1) / kTileN;
  TileCoord tc = grouped_m_tile(args.offsets, args.E, n_tiles, reinterpret_cast<int*>(lds_raw));
  if (!tc.valid) return;
  __syncthreads();
  const int n0 = tc.n_tile * kTileN;

  // waves 0-3: B = W[e] viewed as [K][N] (transposed staging);
  // waves 4-7: A = rows of dO / dH (K-contiguous staging)
  const bool loads_a = tid >= kLoaders;
  const int lt = tid & (kLoaders - 1);
  const uint16_t* src[8];
  bool live = true;
  if (loads_a) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = lt + i * kLoaders;
      int64_t r = tc.m0 + (q >> 3);
      if (r >= args.rows_alloc) r = args.rows_alloc - 1;   // in bounds; never stored
      src[i] = args.g + r * args.K + (q & 7) * 8;
    }
  } else {
    const int bcol = 8 * t_col_block<true>(lt);
    const int kb = 8 * t_k_block(lt);
    live = n0 + bcol < args.N;   // N % 8 == 0: whole group in or out
    const uint16_t* wb = args.w + static_cast<int64_t>(tc.e) * args.K * args.N + n0 + bcol;
#pragma unroll
    for (int i = 0; i < 8; ++i) src[i] = wb + static_cast<int64_t>(kb + i) * args.N;
  }
  const int64_t kstep = loads_a ? kBK : static_cast<int64_t>(kBK) * args.N;  // elements per stage
  Regs8 pf;
  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pf.v[i] = live ? *reinterpret_cast<const u32x4_t*>(src[i] + kt * kstep) : u32x4_t{0u, 0u, 0u, 0u};
  };
  auto store = [&](int buf) {
    uint16_t* s = lds + buf * kStageElems;
    if (loads_a) store_krows(s, lt, pf);
    else store_transposed<true>(s + kOpElems, lt, pf);
  };

  floatx16_t acc[2][4];
  zero_acc(acc);
  const int a_row0 = wm * kWaveM + r32, b_row0 = wn * kWaveN + r32;
  const int nk = args.K / kBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(kt + 1);
    const uint16_t* sa = lds + (kt & 1) * kStageElems;
    mma_stage(sa, sa + kOpElems, a_row0, b_row0, hl, acc);
    if (kt + 1 < nk) store((kt + 1) & 1);
    __syncthreads();
  }

  const int n = n0 + wn * kWaveN + 4 * r32;
  if (n >= args.N) return;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    if (tc.m0 + wm * kWaveM + mi * 32 >= tc.m_end) continue;
    if constexpr (MODE == DgradMode::FC1) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = tc.m0 + acc_row(wm * kWaveM, mi, v, hl);
        if (row >= tc.m_end) continue;
        u32x2_t pk;
        pk[0] = pack_bf16x2(acc[mi][0][v], acc[mi][1][v]);
        pk[1] = pack_bf16x2(acc[mi][2][v], acc[mi][3][v]);
        *reinterpret_cast<u32x2_t*>(args.out + row * args.N + n) = pk;
      }
    } else {
      // SwiGLU backward: issue the 16 rows' h loads together, then compute
      const int I = args.I;
      u32x2_t hg[16], hu[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        int64_t row = tc.m0 + acc_row(wm * kWaveM, mi, v, hl);
        if (row >= tc.m_end) row = tc.m_end - 1;   // clamped: value unused
        hg[v] = *reinterpret_cast<const u32x2_t*>(args.h + row * (2 * I) + n);
        hu[v] = *reinterpret_cast<const u32x2_t*>(args.h + row * (2 * I) + I + n);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = tc.m0 + acc_row(wm * kWaveM, mi, v, hl);
        if (row >= tc.m_end) continue;
        float dg[4], du[4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          // dA is stored as bf16 before the SwiGLU backward
          const float da = bf16_to_f32(f32_to_bf16(acc[mi][ni][v]));
          const float gt = bf16_to_f32(static_cast<uint16_t>(hg[v][ni >> 1] >> (16 * (ni & 1))));
          const float up = bf16_to_f32(static_cast<uint16_t>(hu[v][ni >> 1] >> (16 * (ni & 1))));
          const float sg = 1.0f / (1.0f + expf(-gt));
          dg[ni] = da * up * sg * (1.0f + gt * (1.0f - sg));
          du[ni] = da * gt * sg;
        }
        u32x2_t pg, pu;
        pg[0] = pack_bf16x2(dg[0], dg[1]);
        pg[1] = pack_bf16x2(dg[2], dg[3]);
        pu[0] = pack_bf16x2(du[0], du[1]);
        pu[1] = pack_bf16x2(du[2], du[3]);
        *reinterpret_cast<u32x2_t*>(args.out + row * (2 * I) + n) = pg;
        *reinterpret_cast<u32x2_t*>(args.out + row * (2 * I) + I + n) = pu;
      }
    }
  }
}

// ------------------------------------------------------------------ wgrad
struct WgradArgs {
  int M, N, E;             // dW[e] is [M, N]
  int64_t g_stride;        // row stride of G (= M)
  int64_t s_stride;        // row stride of S (= N)
  const int32_t* offsets;
  const uint16_t* g;       // G [rows, M]:  A(m, r) = G[r][m]
  const uint16_t* s;       // S [*, N]:     B(r, n) = S[src(r)][n]
  const int32_t* src_row;  // gather variant: src(r) = src_row[r] (-1 = zero row)
  uint16_t* out;           // [E, M, N]
};

// GATHER: B rows are S[src_row[r]] (x gathered by token), else S[r].
template <bool GATHER>
__global__ void __launch_bounds__(kGemmThreads, 1)
wgrad_kernel(WgradArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  uint16_t* lds = reinterpret_cast<uint16_t*>(lds_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2, r32 = lane & 31, hl = lane >> 5;
  const int m_tiles = args.M / kTileM, n_tiles = (args.N + kTileN - 1) / kTileN;
  const int64_t total = static_cast<int64_t>(args.E) * m_tiles * n_tiles;
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t y = blockIdx.x / kXcds, x = blockIdx.x % kXcds;
  if (y >= per_xcd) return;
  const int64_t L = x * per_xcd + y;
  if (L >= total) return;
  const int e = static_cast<int>(L / (m_tiles * n_tiles));
  const int mt = static_cast<int>((L / n_tiles) % m_tiles);
  const int nt = static_cast<int>(L % n_tiles);
  const int m0 = mt * kTileM, n0 = nt * kTileN;
  const int64_t r_begin = args.offsets[e], r_end = args.offsets[e + 1];

  // waves 0-3 stage A (rows of G), waves 4-7 stage B (rows of S); both transposed
  const bool loads_b = tid >= kLoaders;
  const int lt = tid & (kLoaders - 1);
  const int kb = 8 * t_k_block(lt);
  const uint16_t* base;
  int64_t stride;
  bool live;
  if (loads_b) {
    const int bcol = 8 * t_col_block<true>(lt);
    base = args.s + n0 + bcol;
    stride = args.s_stride;
    live = n0 + bcol < args.N;
  } else {
    base = args.g + m0 + 8 * t_col_block<false>(lt);
    stride = args.g_stride;
    live = true;
  }
  // Source rows, one stage ahead of the data loads (the gather's index loads
  // would otherwise sit on the critical path).
  int32_t src[8];
  auto load_src = [&](int64_t r0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = r0 + kb + i;
      if (GATHER && loads_b) src[i] = r < r_end ? args.src_row[r] : -1;
      else src[i] = r < r_end ? static_cast<int32_t>(r) : -1;
    }
  };
  Regs8 pf;
  auto load = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pf.v[i] = (src[i] >= 0 && live)
                    ? *reinterpret_cast<const u32x4_t*>(base + static_cast<int64_t>(src[i]) * stride)
                    : u32x4_t{0u, 0u, 0u, 0u};
  };
  auto store = [&](int buf) {
    uint16_t* s = lds + buf * kStageElems;
    if (loads_b) store_transposed<true>(s + kOpElems, lt, pf);
    else store_transposed<false>(s, lt, pf);
  };

  floatx16_t acc[2][4];
  zero_acc(acc);
  const int a_row0 = wm * kWaveM + r32, b_row0 = wn * kWaveN + r32;
  const int64_t nk = (r_end - r_begin + kBK - 1) / kBK;
  if (nk > 0) {
    load_src(r_begin);
    load();
    load_src(r_begin + kBK);
    store(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) {
        load();
        load_src(r_begin + (kt + 2) * kBK);
      }
      const uint16_t* sa = lds + (kt & 1) * kStageElems;
      mma_stage(sa, sa + kOpElems, a_row0, b_row0, hl, acc);
      if (kt + 1 < nk) store((kt + 1) & 1);
      __syncthreads();
    }
  }
  uint16_t* out = args.out + static_cast<int64_t>(e) * args.M * args.N;
  const int n = n0 + wn * kWaveN + 4 * r32;
  if (n >= args.N) return;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t m = m0 + acc_row(wm * kWaveM, mi, v, hl);
      u32x2_t pk;
      pk[0] = pack_bf16x2(acc[mi][0][v], acc[mi][1][v]);
      pk[1] = pack_bf16x2(acc[mi][2][v], acc[mi][3][v]);
      *reinterpret_cast<u32x2_t*>(out + m * args.N + n) = pk;
    }
  }
}

template <typename Kern>
hipError_t set_lds(Kern k) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
}

template <DgradMode MODE>
bool launch_dgrad(const DgradArgs& a, const char* name, hipStream_t s) {
  static const hipError_t attr = set_lds(&dgrad_kernel<MODE>);
  if (attr != hipSuccess) return launch_ok(name) && false;
  const int64_t tiles = grouped_m_tiles_bound(a.rows_alloc, a.E) * ((a.N + kTileN - 1) / kTileN);
  if (tiles == 0) return true;
  {
    ProfScope p(name, s);
    dgrad_kernel<MODE><<<dim3(xcd_grid(tiles)), dim3(kGemmThreads), kLdsBytes, s>>>(a);
  }
  return launch_ok(name);
}

template <bool GATHER>
bool launch_wgrad(const WgradArgs& a, const char* name, hipStream_t s) {
  static const hipError_t attr = set_lds(&wgrad_kernel<GATHER>);
  if (attr != hipSuccess) return launch_ok(name) && false;
  const int64_t tiles = static_cast<int64_t>(a.E) * (a.M / kTileM) * ((a.N + kTileN - 1) / kTileN);
  if (tiles == 0) return true;
  {
    ProfScope p(name, s);
    wgrad_kernel<GATHER><<<dim3(xcd_grid(tiles)), dim3(kGemmThreads), kLdsBytes, s>>>(a);
  }
  return launch_ok(name);
}

}  // namespace

bool launch_dgrad_fc2(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets,
                      const uint16_t* dO, const uint16_t* w2, const uint16_t* h, uint16_t* dH,
                      hipStream_t s) {
  DgradArgs a{rows_alloc, H, I, I, E, offsets, dO, w2, h, dH};
  return launch_dgrad<DgradMode::FC2_SWIGLU>(a, "gemm_dgrad_fc2", s);
}

bool launch_dgrad_fc1(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets,
                      const uint16_t* dH, const uint16_t* w1, uint16_t* dXp, hipStream_t s) {
  DgradArgs a{rows_alloc, 2 * I, H, I, E, offsets, dH, w1, nullptr, dXp};
  return launch_dgrad<DgradMode::FC1>(a, "gemm_dgrad_fc1", s);
}

bool launch_wgrad_fc2(int H, int I, int E, const int32_t* offsets, const uint16_t* dO,
                      const uint16_t* a, uint16_t* dW2, hipStream_t s) {
  WgradArgs w{H, I, E, H, I, offsets, dO, a, nullptr, dW2};
  return launch_wgrad<false>(w, "gemm_wgrad_fc2", s);
}

bool launch_wgrad_fc1(int H, int I, int E, const int32_t* offsets, const uint16_t* dH,
                      const uint16_t* x, const int32_t* src_row, uint16_t* dW1, hipStream_t s) {
  WgradArgs w{2 * I, H, E, 2 * I, H, offsets, dH, x, src_row, dW1};
  return launch_wgrad<true>(w, "gemm_wgrad_fc1", s);
}

}  // namespace w4a4
