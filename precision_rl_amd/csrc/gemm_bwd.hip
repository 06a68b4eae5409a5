// The straight-through BF16 backward GEMMs on gfx950 (AI summary,
// "Methodology in Plain English": straight-through estimator on the saved
// original BF16 operands; miniTE Technical Report, section 4.3: BF16 backward
// through the layer bypass, no backward quantisation).
//
//   dgrad (M = dispatched rows of expert e, ragged):
//     FC2 dgrad: dA  = dO_e . W2[e]     K = H,  N = I, epilogue = SwiGLU backward
//     FC1 dgrad: dXp = dH_e . W1[e]     K = 2I, N = H
//   wgrad (K = dispatched rows of expert e, ragged, possibly empty):
//     FC2 wgrad: dW2[e] = dO_e^T . a_e            M = H,  N = I
//     FC1 wgrad: dW1[e] = dH_e^T . xp_e           M = 2I, N = H   (xp = x gathered by row)
//
// 256 x 256 output tile per workgroup, MFMA 32x32x16 bf16, FP32 accumulation.
// K advances 32 per stage through a 4-deep LDS ring filled by the hardware's
// global -> LDS copies three stages ahead of the MFMAs (no register staging).
// Tiles that are K-contiguous in HBM (dO, dH rows in the dgrad) keep rows of
// 64 B with their 16-byte chunks XOR-swizzled by (row / 4) % 4; tiles that are
// contiguous along M or N in HBM (the weights in the dgrad, both wgrad
// operands) are kept as [k][256] rows of 512 B, chunks swizzled by 4 (k % 4),
// and read with ds_read_b64_tr_b16, which hands each lane four consecutive k
// of its column.  Both layouts make every read cycle conflict-free.

#include "gemm_common.h"
#include "internal.h"

namespace w4a4 {
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 32;
constexpr int kStages = 4;
constexpr int kAhead = kStages - 1;
constexpr int kTileBytes = kTileM * kBK * 2;       // 16 KB: one operand, one stage
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kRingBytes = kStages * kStageBytes;  // 128 KB
constexpr int kSlotOffset = kRingBytes;
constexpr int kLdsBytes = kSlotOffset + 16;
constexpr int kCopiesPerStage = 2 * kTileBytes / 1024;  // 1 KB per wave-wide copy

// Wave grid of a workgroup: WAVES_M x WAVES_N waves over the 256 x 256 tile.
template <int WAVES_M, int WAVES_N>
struct Grid {
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRows = kTileM / WAVES_M;   // per wave
  static constexpr int kCols = kTileN / WAVES_N;
  static constexpr int kMI = kRows / 32;
  static constexpr int kNI = kCols / 32;
  static constexpr int kCopies = kCopiesPerStage / kWaves;  // copies per wave per stage
};

__device__ __forceinline__ bf16x8_t join_bf16(short4_t lo, short4_t hi) {
  typedef short short8_t __attribute__((ext_vector_type(8)));
  const short8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ short4_t ds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(p));
}

// ---- K-contiguous tile: 256 rows x 32 k, 64 B per row, chunk c of row r at
// slot c ^ ((r >> 2) & 3).  Copy q (16 rows): lane i fills row 16 q + i / 4,
// slot i % 4.
__device__ __forceinline__ int krow_src_chunk(int row, int lane) {
  return (lane & 3) ^ ((row >> 2) & 3);
}
__device__ __forceinline__ int krow_frag_offset(int row, int ks, int hl) {
  return row * 64 + (((ks * 2 + hl) ^ ((row >> 2) & 3)) * 16);
}

// ---- [k][256] tile: 32 k-rows of 512 B, 16-byte chunk c of k-row k at slot
// c ^ (4 (k & 3)).  Copy q (2 k-rows): lane i fills k-row 2 q + i / 32, slot
// i % 32.
__device__ __forceinline__ int kcol_src_chunk(int k, int lane) {
  return (lane & 31) ^ (4 * (k & 3));
}
// Byte offset of the 8-byte piece lane l reads with ds_read_tr for the 32 x 16
// MFMA operand block whose columns start at col0 (multiple of 32), for k block
// ks (16 k) and half r (k +0..3 or +4..7).
__device__ __forceinline__ int kcol_frag_offset(int col0, int ks, int r, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int k = ks * 16 + 8 * (g >> 1) + 4 * r + (j >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (j & 3);
  return k * 512 + (((col >> 3) ^ (4 * (k & 3))) * 16) + (col & 7) * 2;
}

template <int MI, int NI>
__device__ __forceinline__ void zero_acc(floatx16_t (&acc)[MI][NI]) {
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;
}

template <int N>
__device__ __forceinline__ void wait_stage(int later) {
  // later = stages issued after the one being waited for (0 .. kAhead-1)
  if (later >= 2) wait_vm_barrier<2 * N>();
  else if (later == 1) wait_vm_barrier<N>();
  else wait_vm_barrier<0>();
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

template <DgradMode MODE, class G>
__global__ void __launch_bounds__(G::kThreads, 1)
dgrad_kernel(DgradArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wrow = (wave % (kTileM / G::kRows)) * G::kRows;
  const int wcol = (wave / (kTileM / G::kRows)) * G::kCols;
  const int r32 = lane & 31, hl = lane >> 5;
  const int n_tiles = (args.N + kTileN - 1) / kTileN;
  TileCoord tc = grouped_m_tile(args.offsets, args.E, n_tiles, reinterpret_cast<int*>(lds + kSlotOffset));
  if (!tc.valid) return;
  const int n0 = tc.n_tile * kTileN;
  const int64_t last_row = args.rows_alloc - 1;

  // ---- copy sources: A = rows of dO / dH (K-contiguous), B = W[e] as [K][N]
  const uint8_t* a_src[G::kCopies / 2];
  const uint8_t* b_src[G::kCopies / 2];
  const uint16_t* we = args.w + static_cast<int64_t>(tc.e) * args.K * args.N;
#pragma unroll
  for (int c = 0; c < G::kCopies / 2; ++c) {
    const int q = wave * (G::kCopies / 2) + c;
    const int row = 16 * q + (lane >> 2);
    a_src[c] = reinterpret_cast<const uint8_t*>(args.g + min(tc.m0 + row, last_row) * args.K) +
               krow_src_chunk(row, lane) * 16;
    const int k = 2 * q + (lane >> 5);
    int col = n0 + kcol_src_chunk(k, lane) * 8;
    col = min(col, args.N - 8);   // columns past N only feed outputs never stored
    b_src[c] = reinterpret_cast<const uint8_t*>(we + static_cast<int64_t>(k) * args.N + col);
  }
  const int64_t a_step = kBK * 2, b_step = static_cast<int64_t>(kBK) * args.N * 2;  // bytes per stage
  auto issue = [&](int kt) {
    uint8_t* st = lds + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int c = 0; c < G::kCopies / 2; ++c) {
      const int q = wave * (G::kCopies / 2) + c;
      dma16(a_src[c] + kt * a_step, st + q * 1024);
      dma16(b_src[c] + kt * b_step, st + kTileBytes + q * 1024);
    }
  };

  // ---- fragment addresses (within a stage)
  int a_off[G::kMI][2], b_off[G::kNI][2][2];
#pragma unroll
  for (int f = 0; f < G::kMI; ++f)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) a_off[f][ks] = krow_frag_offset(wrow + f * 32 + r32, ks, hl);
#pragma unroll
  for (int f = 0; f < G::kNI; ++f)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 2; ++r) b_off[f][ks][r] = kTileBytes + kcol_frag_offset(wcol + f * 32, ks, r, lane);

  floatx16_t acc[G::kMI][G::kNI];
  zero_acc(acc);
  const int nk = args.K / kBK;
  for (int s = 0; s < kAhead && s < nk; ++s) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    wait_stage<G::kCopies>(min(kAhead - 1, nk - 1 - kt));
    if (kt + kAhead < nk) issue(kt + kAhead);
    const uint8_t* st = lds + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[G::kMI], bf[G::kNI];
#pragma unroll
      for (int f = 0; f < G::kMI; ++f) af[f] = *reinterpret_cast<const bf16x8_t*>(st + a_off[f][ks]);
#pragma unroll
      for (int f = 0; f < G::kNI; ++f)
        bf[f] = join_bf16(ds_read_tr(st + b_off[f][ks][0]), ds_read_tr(st + b_off[f][ks][1]));
#pragma unroll
      for (int mi = 0; mi < G::kMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < G::kNI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    }
  }

  // ---- epilogue: lane (r32, hl) holds column wcol + 32 ni + r32 of 16 rows per mi
#pragma unroll
  for (int mi = 0; mi < G::kMI; ++mi) {
    if (tc.m0 + wrow + mi * 32 >= tc.m_end) continue;
#pragma unroll
    for (int ni = 0; ni < G::kNI; ++ni) {
      const int n = n0 + wcol + ni * 32 + r32;
      if (n >= args.N) continue;
      if constexpr (MODE == DgradMode::FC1) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = tc.m0 + acc_row(wrow, mi, v, hl);
          if (row < tc.m_end) args.out[row * args.N + n] = f32_to_bf16(acc[mi][ni][v]);
        }
      } else {
        // SwiGLU backward on bf16 dA, gate / up from the saved bf16 h
        const int I = args.I;
        uint16_t hg[16], hu[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          int64_t row = tc.m0 + acc_row(wrow, mi, v, hl);
          if (row >= tc.m_end) row = tc.m_end - 1;   // clamped: value unused
          hg[v] = args.h[row * (2 * I) + n];
          hu[v] = args.h[row * (2 * I) + I + n];
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = tc.m0 + acc_row(wrow, mi, v, hl);
          if (row >= tc.m_end) continue;
          const float da = bf16_to_f32(f32_to_bf16(acc[mi][ni][v]));
          const float gt = bf16_to_f32(hg[v]), up = bf16_to_f32(hu[v]);
          const float sg = 1.0f / (1.0f + expf(-gt));
          args.out[row * (2 * I) + n] = f32_to_bf16(da * up * sg * (1.0f + gt * (1.0f - sg)));
          args.out[row * (2 * I) + I + n] = f32_to_bf16(da * gt * sg);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ wgrad
struct WgradArgs {
  int M, N, E;             // dW[e] is [M, N]
  const int32_t* offsets;
  const uint16_t* g;       // G [rows, M]:  A(m, r) = G[r][m]
  const uint16_t* s;       // S [rows, N]:  B(r, n) = S[r][n]
  uint16_t* out;           // [E, M, N]
};

template <class G>
__global__ void __launch_bounds__(G::kThreads, 1)
wgrad_kernel(WgradArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wrow = (wave % (kTileM / G::kRows)) * G::kRows;
  const int wcol = (wave / (kTileM / G::kRows)) * G::kCols;
  const int r32 = lane & 31, hl = lane >> 5;
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
  const int64_t nrows = r_end - r_begin;
  const int nk = static_cast<int>((nrows + kBK - 1) / kBK);

  // ---- copy sources: both operands [k = row][256 columns]
  int a_col[G::kCopies / 2], b_col[G::kCopies / 2], kk[G::kCopies / 2];
#pragma unroll
  for (int c = 0; c < G::kCopies / 2; ++c) {
    const int q = wave * (G::kCopies / 2) + c;
    kk[c] = 2 * q + (lane >> 5);
    a_col[c] = m0 + kcol_src_chunk(kk[c], lane) * 8;
    b_col[c] = min(n0 + kcol_src_chunk(kk[c], lane) * 8, args.N - 8);  // past N: never stored
  }
  auto issue = [&](int kt) {
    uint8_t* st = lds + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int c = 0; c < G::kCopies / 2; ++c) {
      const int q = wave * (G::kCopies / 2) + c;
      // rows past the expert's end are re-read from its last row and zeroed in LDS
      const int64_t r = min(r_begin + static_cast<int64_t>(kt) * kBK + kk[c], r_end - 1);
      dma16(args.g + r * args.M + a_col[c], st + q * 1024);
      dma16(args.s + r * args.N + b_col[c], st + kTileBytes + q * 1024);
    }
  };

  int a_off[G::kMI][2][2], b_off[G::kNI][2][2];
#pragma unroll
  for (int f = 0; f < G::kMI; ++f)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 2; ++r) a_off[f][ks][r] = kcol_frag_offset(wrow + f * 32, ks, r, lane);
#pragma unroll
  for (int f = 0; f < G::kNI; ++f)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 2; ++r) b_off[f][ks][r] = kTileBytes + kcol_frag_offset(wcol + f * 32, ks, r, lane);

  floatx16_t acc[G::kMI][G::kNI];
  zero_acc(acc);
  const int tail = static_cast<int>(nrows - static_cast<int64_t>(nk - 1) * kBK);  // valid k of the last stage
  for (int s = 0; s < kAhead && s < nk; ++s) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    wait_stage<G::kCopies>(min(kAhead - 1, nk - 1 - kt));
    uint8_t* st = lds + (kt % kStages) * kStageBytes;
    if (kt == nk - 1 && tail < kBK) {
      // every copy of the workgroup has landed (vmcnt 0 + barrier above): zero
      // the k-rows past the expert's end in both operands, then sync again
      for (int i = tid; i < (kBK - tail) * 64; i += G::kThreads) {
        const int op = i / ((kBK - tail) * 32), rem = i % ((kBK - tail) * 32);
        *reinterpret_cast<u32x4_t*>(st + op * kTileBytes + (tail + rem / 32) * 512 + (rem % 32) * 16) =
            u32x4_t{0u, 0u, 0u, 0u};
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (kt + kAhead < nk) issue(kt + kAhead);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[G::kMI], bf[G::kNI];
#pragma unroll
      for (int f = 0; f < G::kMI; ++f)
        af[f] = join_bf16(ds_read_tr(st + a_off[f][ks][0]), ds_read_tr(st + a_off[f][ks][1]));
#pragma unroll
      for (int f = 0; f < G::kNI; ++f)
        bf[f] = join_bf16(ds_read_tr(st + b_off[f][ks][0]), ds_read_tr(st + b_off[f][ks][1]));
#pragma unroll
      for (int mi = 0; mi < G::kMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < G::kNI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    }
  }
  uint16_t* out = args.out + static_cast<int64_t>(e) * args.M * args.N;
#pragma unroll
  for (int ni = 0; ni < G::kNI; ++ni) {
    const int n = n0 + wcol + ni * 32 + r32;
    if (n >= args.N) continue;
#pragma unroll
    for (int mi = 0; mi < G::kMI; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        out[static_cast<int64_t>(m0 + acc_row(wrow, mi, v, hl)) * args.N + n] = f32_to_bf16(acc[mi][ni][v]);
  }
}

using BwdGrid = Grid<4, 2>;   // 8 waves, 64 x 128 per wave

template <typename Kern>
hipError_t set_lds(Kern k) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
}

template <DgradMode MODE>
bool launch_dgrad(const DgradArgs& a, const char* name, hipStream_t s) {
  static const hipError_t attr = set_lds(&dgrad_kernel<MODE, BwdGrid>);
  if (attr != hipSuccess) return launch_ok(name) && false;
  const int64_t tiles = grouped_m_tiles_bound(a.rows_alloc, a.E) * ((a.N + kTileN - 1) / kTileN);
  if (tiles == 0) return true;
  {
    ProfScope p(name, s);
    dgrad_kernel<MODE, BwdGrid><<<dim3(xcd_grid(tiles)), dim3(BwdGrid::kThreads), kLdsBytes, s>>>(a);
  }
  return launch_ok(name);
}

bool launch_wgrad(const WgradArgs& a, const char* name, hipStream_t s) {
  static const hipError_t attr = set_lds(&wgrad_kernel<BwdGrid>);
  if (attr != hipSuccess) return launch_ok(name) && false;
  const int64_t tiles = static_cast<int64_t>(a.E) * (a.M / kTileM) * ((a.N + kTileN - 1) / kTileN);
  if (tiles == 0) return true;
  {
    ProfScope p(name, s);
    wgrad_kernel<BwdGrid><<<dim3(xcd_grid(tiles)), dim3(BwdGrid::kThreads), kLdsBytes, s>>>(a);
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
  WgradArgs w{H, I, E, offsets, dO, a, dW2};
  return launch_wgrad(w, "gemm_wgrad_fc2", s);
}

bool launch_wgrad_fc1(int H, int I, int E, const int32_t* offsets, const uint16_t* dH,
                      const uint16_t* xp, uint16_t* dW1, hipStream_t s) {
  WgradArgs w{2 * I, H, E, offsets, dH, xp, dW1};
  return launch_wgrad(w, "gemm_wgrad_fc1", s);
}

}  // namespace w4a4
