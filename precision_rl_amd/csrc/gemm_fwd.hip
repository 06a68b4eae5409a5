// FC1 (with the SwiGLU in its epilogue) and FC2: grouped block-scaled GEMMs on gfx950.
//
// The pages' recipe (rainbus review, "core method"; AI summary, "Methodology in
// Plain English") accumulates the block-scaled product U_e = MMA(X_e, W_e^T)
// natively and applies the outer factors g_x g_w in FP32 in the epilogue.
// gfx950's scaled FP4 MFMA takes E8M0 (power-of-two) scales per 32 elements,
// which cannot carry NVFP4's E4M3 scale per 16.  Instead each operand element
// is decoded exactly to f16: d * c has at most 6 significant bits and lies in
// [2^-10, 2688], so the f16 value is exact, f16 x f16 products are exact in
// FP32, and only the MFMA's FP32 accumulation rounds.  Decoding happens in
// registers right before the MFMA (hardware fp4 -> f16 conversion, which
// applies only the exponent of its scale operand, then one v_pk_mul_f16 by the
// E4M3 block scale); decoded operands never touch memory.
//
// Tiling: 128 x 256 output tile per workgroup of 4 waves (2 x 2, 64 x 128 per
// wave), MFMA 32x32x16 f16, and two workgroups per CU (56.5 / 64.5 KB of LDS
// and at most 256 registers per wave each), so that one workgroup's
// epilogue, tile set-up and barrier waits overlap the other's MFMAs, and each
// SIMD holds two waves whose operand decode interleaves with the other's
// matrix work.  The 128-row tile also bounds the padding work of an expert's
// last, partial M tile.  Each pipeline stage covers 64 of K (32 B of packed
// codes and 4 B of block scales per row of both operands); the codes are
// copied global -> LDS by the hardware (no register staging) two stages at a
// time, 64 B per row and copy, into one of two pair buffers (one-stage
// copies of 32 B per row took as many L1-to-L2 requests for half the bytes);
// a pair's copies go out in two parts after consecutive stage waits, so that
// no stage issues them all.  Code rows keep their four 16-byte chunks
// permuted by (row / 4) % 4, so fragment reads of 16 consecutive rows hit 16
// distinct bank groups.  Inside a stage, lane half h (lanes 32-63) owns the
// stage's second 32 k of its row; A and B use the same assignment, so every
// MFMA k slot pairs equal k indices (the reduction runs in a permuted K
// order; FP32 rounding of the sum is covered by the tolerance, and sums that
// are exact in FP32 are order independent).  The epilogue writes the bf16 tile through
// the idle ring so that global stores are whole 16-byte row chunks
// (non-temporal: the outputs are read once, by a later kernel).

#include "gemm_common.h"
#include "internal.h"

namespace w4a4 {
namespace {

constexpr int kThreads = 256;                // 4 waves, 2 (M) x 2 (N)
constexpr int kBM = 128, kBN = 256;          // workgroup tile
constexpr int kWM = 64, kWN = 128;           // wave tile
constexpr int kBK = 64;                      // K per stage
constexpr int kCodeRow = kBK / 2;            // 32 B of codes per row per stage
constexpr int kScaleRow = kBK / 16;          // 4 scale bytes per row per stage
// Scale rows of a stage, 4 B each: A rows 0..127, B rows 128..383, and 128
// filler rows so that every wave issues the same two copies.
constexpr int kScaleRows = 512;
constexpr int kBScaleRow0 = kBM;

// Codes arrive two stages at a time (64 B per row and copy, 16-byte chunk c
// of row r at slot c ^ ((r >> 2) & 3)) into one of two pair buffers; without
// grouped scales a pair buffer also holds its two stages' scale dwords.
constexpr int kPairRow = 2 * kCodeRow;                  // 64 B
constexpr int kPairACodes = kBM * kPairRow;             // 8 KB
constexpr int kPairCodes = (kBM + kBN) * kPairRow;      // 24 KB
constexpr int kPairScales = 2 * kScaleRows * 4;         // 4 KB

// Grouped scales (K a multiple of 256): the scales of four stages, 16 B per
// row, arrive in one copy issued with the codes of every other pair, into one
// of two 8 KB buffers after the pair buffers (same 512-row numbering as
// above).
constexpr int kGroup = 4;
constexpr int kScaleBufBytes = kScaleRows * 16;                // 8 KB
constexpr int kGsScaleOffset = 2 * kPairCodes;                 // 48 KB

// Epilogue staging in the pair buffers: 64 rows of 512 B of bf16 per round,
// rows padded by 16 B so that the two lane halves' writes (4 rows apart) fall
// on different banks.
constexpr int kOutRows = 64;
constexpr int kOutPitch = 528;
static_assert(kOutRows * kOutPitch <= 2 * kPairCodes, "staging fits in the pair buffers");

template <bool GS>
struct FwdLds {
  static constexpr int kPair = GS ? kPairCodes : kPairCodes + kPairScales;
  static constexpr int kGx = GS ? kGsScaleOffset + 2 * kScaleBufBytes : 2 * kPair;
  static constexpr int kSlot = kGx + kBM * 4;
  static constexpr int kBytes = kSlot + 16;      // 56.5 / 64.5 KB: two workgroups per CU
  static_assert(2 * kBytes <= 160 * 1024, "two workgroups per CU must fit in LDS");
};

__device__ __forceinline__ int pair_slot(int r, int c) { return c ^ ((r >> 2) & 3); }

enum class FwdMode { FC1, FC2 };

struct FwdArgs {
  int64_t rows_alloc;
  int K;             // reduction length (H for FC1, I for FC2)
  int N;             // output features (2I for FC1, H for FC2)
  int I;             // SwiGLU width (FC1)
  int E;
  const int32_t* offsets;
  Fp4Operand a;      // [rows, K]
  Fp4Operand w;      // [E, N, K]
  uint16_t* out;     // FC1: h [rows, 2I] (may be null); FC2: o [rows, N]
  uint16_t* act;     // FC1: a [rows, I]
  float* dbg;        // FC1: pre-cast [rows, 2I] (may be null)
};

// Global row of B (weights) staged into LDS row p of the tile: lane j of wave
// column wn ends up owning 4 consecutive outputs (FC2: columns; FC1: the gate
// and up halves of two consecutive SwiGLU features).
template <FwdMode MODE>
__device__ __forceinline__ int b_row_of(int p, int n_tile, int I) {
  const int wn = p >> 7, ni = (p >> 5) & 3, j = p & 31;
  if constexpr (MODE == FwdMode::FC2) {
    return n_tile * kBN + wn * 128 + 4 * j + ni;
  } else {
    const int half = ni >> 1;
    const int i = n_tile * 128 + wn * 64 + 2 * j + (ni & 1);
    return half * I + i;
  }
}


__device__ __forceinline__ half8_t decode8(uint32_t codes8, half2_t d2) {
  half2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, 1.0f, 0) * d2;
  half2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, 1.0f, 1) * d2;
  half2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, 1.0f, 2) * d2;
  half2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes8, 1.0f, 3) * d2;
  half8_t r;
  r[0] = v0[0]; r[1] = v0[1]; r[2] = v1[0]; r[3] = v1[1];
  r[4] = v2[0]; r[5] = v2[1]; r[6] = v3[0]; r[7] = v3[1];
  return r;
}

// The lane's two E4M3 block scales of a stage (blocks 2h, 2h+1 of the row's
// four, the low 16 bits of `pair`) as f16 pairs (d, d).
__device__ __forceinline__ void scale_pairs(uint32_t pair, half2_t& d0, half2_t& d1) {
  const half2_t v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pair, 1.0f, false);
  d0 = half2_t{v[0], v[0]};
  d1 = half2_t{v[1], v[1]};
}

// Epilogue of the forward GEMMs: out = bf16(acc * (g_x[row] * g_w[n])) (FP32
// products; 1.0 factors where the recipe has no outer scales), FC1 with the
// SwiGLU.  s_gx: the tile's row outer scales in LDS; gw: this lane's four
// weight outer scales; lds: the idle ring, used as staging.
template <FwdMode MODE>
__device__ __forceinline__ void fwd_epilogue(const FwdArgs& args, floatx16_t (&acc)[2][4], const TileCoord& tc,
                                             const float* s_gx, const float (&gw)[4], uint8_t* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r32 = lane & 31, hl = lane >> 5;
  // ---------------------------------------------------------------- epilogue
  // The tile leaves in two rounds of 64 rows (MFMA row block mi = q of both
  // wave rows) staged as bf16 in the idle ring, so that every global store is
  // a 16-byte chunk of a row and a wave writes whole rows.  Staging row s holds
  // tile row (s / 32) * 64 + 32 q + s % 32.  FC1 stages h (gate half, then up
  // half, 128 features each) and computes the SwiGLU on the staged bf16 values
  // while storing.
  uint8_t* so = lds;
  auto tile_row = [&](int s, int q) { return (s >> 5) * kWM + 32 * q + (s & 31); };
  if constexpr (MODE == FwdMode::FC2) {
    const int n_loc = wn * kWN + 4 * r32;
    uint16_t* out = args.out + tc.n_tile * kBN;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q > 0) __syncthreads();   // previous round's reads done
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int s = wm * 32 + acc_row(0, 0, v, hl);
        const float gx = s_gx[tile_row(s, q)];
        u32x2_t pk;
        pk[0] = pack_bf16x2(acc[q][0][v] * (gx * gw[0]), acc[q][1][v] * (gx * gw[1]));
        pk[1] = pack_bf16x2(acc[q][2][v] * (gx * gw[2]), acc[q][3][v] * (gx * gw[3]));
        *reinterpret_cast<u32x2_t*>(so + s * kOutPitch + n_loc * 2) = pk;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kOutRows * 32 / kThreads; ++j) {
        const int c = tid + j * kThreads;
        const int s = c >> 5, ch = c & 31;
        const int64_t row = tc.m0 + tile_row(s, q);
        if (row < tc.m_end)
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(so + s * kOutPitch + ch * 16),
                                      reinterpret_cast<u32x4_t*>(out + row * args.N + ch * 8));
      }
    }
  } else {
    const int I = args.I;
    const int i_loc = wn * 64 + 2 * r32;
    const int i = tc.n_tile * 128 + i_loc;
    const float gw_g0 = gw[0], gw_g1 = gw[1], gw_u0 = gw[2], gw_u1 = gw[3];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q > 0) __syncthreads();   // previous round's reads done
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int s = wm * 32 + acc_row(0, 0, v, hl);
        const float gx = s_gx[tile_row(s, q)];
        const float g0 = acc[q][0][v] * (gx * gw_g0);
        const float g1 = acc[q][1][v] * (gx * gw_g1);
        const float u0 = acc[q][2][v] * (gx * gw_u0);
        const float u1 = acc[q][3][v] * (gx * gw_u1);
        if (args.dbg != nullptr) {
          const int64_t row = tc.m0 + tile_row(s, q);
          if (row < tc.m_end) {
            float* d = args.dbg + row * (2 * I);
            *reinterpret_cast<float2*>(d + i) = make_float2(g0, g1);
            *reinterpret_cast<float2*>(d + I + i) = make_float2(u0, u1);
          }
        }
        *reinterpret_cast<uint32_t*>(so + s * kOutPitch + i_loc * 2) = pack_bf16x2(g0, g1);
        *reinterpret_cast<uint32_t*>(so + s * kOutPitch + 256 + i_loc * 2) = pack_bf16x2(u0, u1);
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kOutRows * 16 / kThreads; ++j) {
        const int c = tid + j * kThreads;
        const int s = c >> 4, ch = c & 15;
        const int64_t row = tc.m0 + tile_row(s, q);
        if (row >= tc.m_end) continue;
        const u32x4_t hg = *reinterpret_cast<const u32x4_t*>(so + s * kOutPitch + ch * 16);
        const u32x4_t hu = *reinterpret_cast<const u32x4_t*>(so + s * kOutPitch + 256 + ch * 16);
        const int64_t col = tc.n_tile * 128 + ch * 8;
        if (args.out != nullptr) {
          uint16_t* h = args.out + row * (2 * I) + col;
          __builtin_nontemporal_store(hg, reinterpret_cast<u32x4_t*>(h));
          __builtin_nontemporal_store(hu, reinterpret_cast<u32x4_t*>(h + I));
        }
        // SwiGLU on the bf16-rounded h, FP32 arithmetic (hardware exp2 / rcp)
        u32x4_t a;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float bg0 = bf16_to_f32(static_cast<uint16_t>(hg[w] & 0xFFFFu));
          const float bg1 = bf16_to_f32(static_cast<uint16_t>(hg[w] >> 16));
          const float bu0 = bf16_to_f32(static_cast<uint16_t>(hu[w] & 0xFFFFu));
          const float bu1 = bf16_to_f32(static_cast<uint16_t>(hu[w] >> 16));
          a[w] = pack_bf16x2(bg0 * sigmoid_fast(bg0) * bu0, bg1 * sigmoid_fast(bg1) * bu1);
        }
        __builtin_nontemporal_store(a, reinterpret_cast<u32x4_t*>(args.act + row * I + col));
      }
    }
  }
}

template <FwdMode MODE, bool GS>
__global__ void __launch_bounds__(kThreads, 2)
fwd_gemm_kernel(FwdArgs args) {
  using L = FwdLds<GS>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r32 = lane & 31, hl = lane >> 5;

  const int n_tiles = MODE == FwdMode::FC1 ? args.I / 128 : args.N / kBN;
  TileCoord tc = grouped_m_tile<kBM>(args.offsets, args.E, n_tiles,
                                     reinterpret_cast<int*>(lds + L::kSlot));
  if (!tc.valid) return;

  const int64_t K2 = args.K / 2, K16 = args.K / 16;
  const int64_t last_row = args.rows_alloc - 1;
  // ---- this wave's copies.  Codes: a wave-uniform base (the tile's first
  // row, resp. the expert's weights, advanced per stage) plus a small per-lane
  // offset.  Rows past the allocation are clamped: they only feed accumulator
  // rows that are never stored.
  const uint8_t* a_codes = args.a.codes + tc.m0 * K2;
  const uint8_t* w_codes = args.w.codes + static_cast<int64_t>(tc.e) * args.N * K2;
  const uint8_t* w_scales = args.w.scales + static_cast<int64_t>(tc.e) * args.N * K16;
  const int a_rows = static_cast<int>(min<int64_t>(kBM, last_row + 1 - tc.m0));   // >= 1
  // Code copies per pair: copy q fills 16 staged rows (1 KB), lane i row
  // 16 q' + i / 4 at slot i % 4; A: q' = 2 wave + q, B: q' = 4 wave + q.
  uint32_t a_code_off[2], b_code_off[4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * (2 * wave + q) + (lane >> 2);
    a_code_off[q] = static_cast<uint32_t>(min(row, a_rows - 1) * K2 + pair_slot(row, lane & 3) * 16);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 16 * (4 * wave + q) + (lane >> 2);
    b_code_off[q] = static_cast<uint32_t>(b_row_of<MODE>(row, tc.n_tile, args.I) * K2 +
                                          pair_slot(row, lane & 3) * 16);
  }
  // Scales: one dword per scale row per stage, from A or B (per-lane pointer).
  const uint8_t* scale_src[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int q = 128 * wave + 64 * c + lane;
    if (q < kBScaleRow0) {
      scale_src[c] = args.a.scales + (tc.m0 + min(q, a_rows - 1)) * K16;
    } else if (q < kBScaleRow0 + kBN) {
      scale_src[c] = w_scales + static_cast<int64_t>(b_row_of<MODE>(q - kBScaleRow0, tc.n_tile, args.I)) * K16;
    } else {
      scale_src[c] = args.a.scales + tc.m0 * K16;            // filler: a valid row, never read
    }
  }
  // Grouped scales: copy q = 2 wave + c moves scale rows 64 q .. 64 q + 63,
  // 16 B each (A rows, then B rows, then filler).
  const uint8_t* gscale_src[2];
  if constexpr (GS) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int q = 64 * (2 * wave + c) + lane;
      if (q < kBScaleRow0) {
        gscale_src[c] = args.a.scales + (tc.m0 + min(q, a_rows - 1)) * K16;
      } else if (q < kBScaleRow0 + kBN) {
        gscale_src[c] = w_scales + static_cast<int64_t>(b_row_of<MODE>(q - kBScaleRow0, tc.n_tile, args.I)) * K16;
      } else {
        gscale_src[c] = args.a.scales + tc.m0 * K16;          // filler: a valid row, never read
      }
    }
  }
  const uint32_t lds0 = lds_addr(lds);
  // Pair p (stages 2p, 2p+1): grouped scales of group p / 2 first (even p),
  // then the A codes; then the B codes and (ungrouped) the two stages' scale
  // dwords.  Pairs 0 and 1 go out whole before the loop; later pairs in two
  // parts, after consecutive waits, so that no stage issues them all.
  auto issue_a = [&](int p) {
    const uint32_t st = lds0 + (p & 1) * L::kPair;
    if constexpr (GS) {
      if (p % 2 == 0) {
        const int g = p / 2;
        const uint32_t sb = lds0 + kGsScaleOffset + (g % 2) * kScaleBufBytes;
#pragma unroll
        for (int c = 0; c < 2; ++c) dma16(gscale_src[c] + g * 16, sb + (2 * wave + c) * 1024);
      }
    }
    const int cb = p * kPairRow;
#pragma unroll
    for (int q = 0; q < 2; ++q) dma16_off(a_codes + cb, a_code_off[q], st + (2 * wave + q) * 1024);
  };
  auto issue_b = [&](int p) {
    const uint32_t st = lds0 + (p & 1) * L::kPair;
    const int cb = p * kPairRow;
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16_off(w_codes + cb, b_code_off[q], st + kPairACodes + (4 * wave + q) * 1024);
    if constexpr (!GS) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          dma4(scale_src[c] + (2 * p + h) * kScaleRow, st + kPairCodes + h * (kScaleRows * 4) + (2 * wave + c) * 256);
    }
  };
  // Waits until stage kt (its pair's codes and its scales) has landed in every
  // wave.  Pair kt/2 + 1's first part goes out after the wait of each even
  // kt >= 2 and its second part after the next wait (each part's buffer
  // region is then done with); loads return in order, so the wait allows the
  // copies issued after stage kt's last one: at kt <= 1 pair 1's, at odd
  // kt >= 3 the first part of pair (kt+1)/2, at even kt >= 2 none (checked
  // against a simulation of this order).
  auto stage_ready = [&](int kt, int nk) {
    const int np = nk / 2;
    int after = 0;
    if (kt <= 1) {
      after = np > 1 ? (GS ? 6 : 10) : 0;
    } else if (kt & 1) {
      const int q = (kt + 1) / 2;
      after = q < np ? 2 + (GS && q % 2 == 0 ? 2 : 0) : 0;
    }
    switch (after) {
      case 10: wait_vm_barrier<10>(); break;
      case 6: wait_vm_barrier<6>(); break;
      case 4: wait_vm_barrier<4>(); break;
      case 2: wait_vm_barrier<2>(); break;
      default: wait_vm_barrier<0>(); break;
    }
  };

  // outer scales of the tile's rows, read by the epilogue
  // outer scales of the tile's rows (written to LDS after the main loop, for
  // the epilogue: loading them now and waiting then keeps the load's latency
  // out of the tile's start)
  const float gx_row = args.a.outer[tc.m0 + min(tid % kBM, a_rows - 1)];
  // and this lane's four weight outer scales (its output columns: FC2 four
  // consecutive n; FC1 the gate and up halves of two features), loaded here
  // so that the epilogue does not wait for them
  float gw[4];
  {
    const float* wouter = args.w.outer + static_cast<int64_t>(tc.e) * args.N;
    if constexpr (MODE == FwdMode::FC2) {
      const int n = tc.n_tile * kBN + wn * kWN + 4 * r32;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) gw[ni] = wouter[n + ni];
    } else {
      const int i = tc.n_tile * 128 + wn * 64 + 2 * r32;
      gw[0] = wouter[i];
      gw[1] = wouter[i + 1];
      gw[2] = wouter[args.I + i];
      gw[3] = wouter[args.I + i + 1];
    }
  }

  floatx16_t acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  const int a_row0 = wm * kWM + r32, b_row0 = wn * kWN + r32;
  // This lane's LDS offsets within a stage: its code chunk (k half hl) of the
  // first A / B row block, and its half (2 of the row's 4 block scales) of the
  // scale dword of the same rows.
  constexpr int kSStride = GS ? 16 : 4;   // bytes per scale row
  uint32_t a_code_lane[2], b_code_lane[2];   // by the stage's half of its pair
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    a_code_lane[h] = a_row0 * kPairRow + pair_slot(a_row0, 2 * h + hl) * 16;
    b_code_lane[h] = kPairACodes + b_row0 * kPairRow + pair_slot(b_row0, 2 * h + hl) * 16;
  }
  const uint32_t a_scale_lane = a_row0 * kSStride + 2 * hl;
  const uint32_t b_scale_lane = (kBScaleRow0 + b_row0) * kSStride + 2 * hl;
  const int nk = args.K / kBK;   // even: K % 128 == 0
  const int np = nk / 2;
  issue_a(0);
  issue_b(0);
  if (np > 1) {
    issue_a(1);
    issue_b(1);
  }

  // A wave whose 64 rows all lie past the expert's end (the padding half of
  // a ragged last tile) only copies and waits: its SIMD's matrix core goes to
  // the other workgroup on the CU.
  const bool rows_live = tc.m0 + wm * kWM < tc.m_end;
  for (int kt = 0; kt < nk; ++kt) {
    stage_ready(kt, nk);
    // refills the buffer of pair kt/2 - 1, read in iterations kt-2 and kt-1
    // (grouped scales: the buffer of group kt/4 - 1, done)
    if (kt >= 2 && (kt & 1) == 0 && kt / 2 + 1 < np) issue_a(kt / 2 + 1);
    if (kt >= 3 && (kt & 1) && (kt + 1) / 2 < np) issue_b((kt + 1) / 2);
    if (!rows_live) continue;
    // LDS addresses: the pair buffer's base (a scalar) plus this lane's
    // offsets for the stage's half; the other fragments are immediates (+2048
    // per 32 code rows, +32 scale rows)
    const uint32_t st = opaque_sgpr(lds0 + ((kt >> 1) & 1) * L::kPair);
    const uint32_t sb = opaque_sgpr(GS ? lds0 + kGsScaleOffset + ((kt / kGroup) % 2) * kScaleBufBytes + (kt % kGroup) * 4
                                       : st + kPairCodes + (kt & 1) * (kScaleRows * 4));
    uint32_t la0 = a_code_lane[0], la1 = a_code_lane[1], lb0 = b_code_lane[0], lb1 = b_code_lane[1];
    asm volatile("" : "+v"(la0), "+v"(la1), "+v"(lb0), "+v"(lb1));   // a select, not an indexed load
    const bool h = kt & 1;
    const uint32_t pa = st + (h ? la1 : la0), pb = st + (h ? lb1 : lb0);
    const uint32_t qa = sb + a_scale_lane, qb = sb + b_scale_lane;
    u32x4_t ac[2], bc[4];
    uint32_t as[2], bs[4];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      ac[f] = *lds_ptr<u32x4_t>(pa + f * 32 * kPairRow);
      as[f] = *lds_ptr<uint16_t>(qa + f * 32 * kSStride);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      bc[f] = *lds_ptr<u32x4_t>(pb + f * 32 * kPairRow);
      bs[f] = *lds_ptr<uint16_t>(qb + f * 32 * kSStride);
    }
    half2_t ad[2][2], bd[4][2];
#pragma unroll
    for (int f = 0; f < 2; ++f) scale_pairs(as[f], ad[f][0], ad[f][1]);
#pragma unroll
    for (int f = 0; f < 4; ++f) scale_pairs(bs[f], bd[f][0], bd[f][1]);
    // Software-pipelined issue order: decode task t (k slice t / 6; fragments
    // A0, B0, B1, B2, B3, A1) is issued right after MFMA t - 2, so a wave's
    // own decode runs under its MFMAs (one 8-instruction decode lasts about
    // one MFMA); the fences keep the compiler from regrouping them.
    half8_t da[4][2], db[4][4];
    auto decode_task = [&](int t) {
      const int s4 = t / 6, i = t % 6;
      if (i == 0) da[s4][0] = decode8(ac[0][s4], ad[0][s4 >> 1]);
      else if (i == 5) da[s4][1] = decode8(ac[1][s4], ad[1][s4 >> 1]);
      else db[s4][i - 1] = decode8(bc[i - 1][s4], bd[i - 1][s4 >> 1]);
    };
    decode_task(0);
    decode_task(1);
    __builtin_amdgcn_sched_barrier(0);
    // The stage's MFMAs at raised wave priority: the SIMD's arbiter then
    // prefers this wave's next MFMA (and the decode between them) to the
    // other workgroup's wave while it copies, waits or stores (FC1 -3%).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int s4 = m >> 3, mi = (m >> 2) & 1, ni = m & 3;
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[s4][mi], db[s4][ni], acc[mi][ni], 0, 0, 0);
      if (m + 2 < 24) decode_task(m + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  float* s_gx = reinterpret_cast<float*>(lds + L::kGx);
  if (tid < kBM) s_gx[tid] = gx_row;
  __syncthreads();   // s_gx visible; every wave is past its last read of the ring

  fwd_epilogue<MODE>(args, acc, tc, s_gx, gw, lds);
}

// ------------------------------------------------------------ MXFP4 recipe
// The same grouped GEMMs for MXFP4 operands (E2M1 codes, one E8M0 scale per
// 32 elements along K, no outer scales): gfx950's scaled FP4 MFMA
// (32x32x64, f32 accumulate) consumes the packed codes and the scale bytes
// as they are, so nothing is decoded.  Lane l of a 32x32x64 operand holds
// row l % 32, elements 32 (l / 32) .. +31 of the 64 (16 bytes, element 2j in
// the low nibble of byte j) and that run's E8M0 byte, which is exactly the
// 16-byte chunk and block scale the NVFP4 kernel's lanes read.
// A stage covers 128 of K: 64 B of codes per row (four 16-byte chunks,
// stored at chunk slot c ^ ((r >> 2) & 3), so that the 16 rows one
// ds_read_b128 phase touches fill all 64 banks) and 4 scale bytes per row
// (one dword, same 512-row numbering as the NVFP4 stage); three stages ring,
// two in flight, 78.5 KB: two workgroups per CU.  K % 128 == 0.
constexpr int kMxBK = 128;
constexpr int kMxStages = 3;
constexpr int kMxAhead = kMxStages - 1;
constexpr int kMxCodeRow = kMxBK / 2;                          // 64 B
constexpr int kMxACodes = kBM * kMxCodeRow;                    // 8 KB
constexpr int kMxBCodes = kBN * kMxCodeRow;                    // 16 KB
constexpr int kMxScalesOffset = kMxACodes + kMxBCodes;
constexpr int kMxStageBytes = kMxScalesOffset + kScaleRows * 4;   // 26 KB
constexpr int kMxDmaPerStage = 8;            // per wave: 2 A-code, 4 B-code, 2 scale copies
constexpr int kMxGx = kMxStages * kMxStageBytes;
constexpr int kMxSlot = kMxGx + kBM * 4;
constexpr int kMxLdsBytes = kMxSlot + 16;
static_assert(2 * kMxLdsBytes <= 160 * 1024, "two workgroups per CU must fit in LDS");
static_assert(kOutRows * kOutPitch <= kMxStages * kMxStageBytes, "staging fits in the ring");

__device__ __forceinline__ int mx_code_slot(int r, int c) { return c ^ ((r >> 2) & 3); }

template <FwdMode MODE>
__global__ void __launch_bounds__(kThreads, 2)
fwd_mx_kernel(FwdArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r32 = lane & 31, hl = lane >> 5;

  const int n_tiles = MODE == FwdMode::FC1 ? args.I / 128 : args.N / kBN;
  TileCoord tc = grouped_m_tile<kBM>(args.offsets, args.E, n_tiles, reinterpret_cast<int*>(lds + kMxSlot));
  if (!tc.valid) return;

  const int64_t K2 = args.K / 2, K32 = args.K / 32;
  const int64_t last_row = args.rows_alloc - 1;
  const uint8_t* a_codes = args.a.codes + tc.m0 * K2;
  const uint8_t* w_codes = args.w.codes + static_cast<int64_t>(tc.e) * args.N * K2;
  const uint8_t* w_scales = args.w.scales + static_cast<int64_t>(tc.e) * args.N * K32;
  const int a_rows = static_cast<int>(min<int64_t>(kBM, last_row + 1 - tc.m0));   // >= 1
  // Code copies: copy q of this wave fills 16 staged rows (1 KB), lane i
  // row 16 q' + i / 4 at slot i % 4; A: q' = 2 wave + q, B: q' = 4 wave + q.
  // Rows past the allocation are clamped (they feed only rows never stored).
  uint32_t a_code_off[2], b_code_off[4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * (2 * wave + q) + (lane >> 2);
    a_code_off[q] = static_cast<uint32_t>(min(row, a_rows - 1) * K2 + mx_code_slot(row, lane & 3) * 16);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 16 * (4 * wave + q) + (lane >> 2);
    b_code_off[q] = static_cast<uint32_t>(b_row_of<MODE>(row, tc.n_tile, args.I) * K2 +
                                          mx_code_slot(row, lane & 3) * 16);
  }
  // Scale copies: one dword (the stage's 4 blocks) per staged row.
  const uint8_t* scale_src[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int q = 128 * wave + 64 * c + lane;
    if (q < kBScaleRow0)
      scale_src[c] = args.a.scales + (tc.m0 + min(q, a_rows - 1)) * K32;
    else if (q < kBScaleRow0 + kBN)
      scale_src[c] = w_scales + static_cast<int64_t>(b_row_of<MODE>(q - kBScaleRow0, tc.n_tile, args.I)) * K32;
    else
      scale_src[c] = args.a.scales + tc.m0 * K32;            // filler: a valid row, never read
  }
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int kt) {
    const uint32_t st = lds0 + (kt % kMxStages) * kMxStageBytes;
    const int cb = kt * kMxCodeRow;
#pragma unroll
    for (int q = 0; q < 2; ++q) dma16_off(a_codes + cb, a_code_off[q], st + (2 * wave + q) * 1024);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16_off(w_codes + cb, b_code_off[q], st + kMxACodes + (4 * wave + q) * 1024);
#pragma unroll
    for (int c = 0; c < 2; ++c) dma4(scale_src[c] + kt * 4, st + kMxScalesOffset + (2 * wave + c) * 256);
  };

  floatx16_t acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  const int a_row0 = wm * kWM + r32, b_row0 = wn * kWN + r32;
  // This lane's LDS offsets within a stage: its chunk (K-step s, half hl) of
  // the first A / B row block (the slot is the same for every row block:
  // they are 32 rows apart), and its rows' scale dwords.
  const int sw = (r32 >> 2) & 3;
  uint32_t a_lane[2], b_lane[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    a_lane[s2] = a_row0 * kMxCodeRow + ((2 * s2 + hl) ^ sw) * 16;
    b_lane[s2] = kMxACodes + b_row0 * kMxCodeRow + ((2 * s2 + hl) ^ sw) * 16;
  }
  const uint32_t a_scale_lane = kMxScalesOffset + a_row0 * 4;
  const uint32_t b_scale_lane = kMxScalesOffset + (kBScaleRow0 + b_row0) * 4;
  const int nk = args.K / kMxBK;
  for (int s0 = 0; s0 < kMxAhead && s0 < nk; ++s0) issue(s0);

  const bool rows_live = tc.m0 + wm * kWM < tc.m_end;
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed in every wave: at most the copies issued after it
    // (stage kt + 1, if any) are pending
    if (kt + 1 < nk) wait_vm_barrier<kMxDmaPerStage>();
    else wait_vm_barrier<0>();
    if (kt + kMxAhead < nk) issue(kt + kMxAhead);   // refills the slot read in iteration kt-1
    if (!rows_live) continue;
    const uint32_t st = opaque_sgpr(lds0 + (kt % kMxStages) * kMxStageBytes);
    uint32_t as[2], bs[4];
#pragma unroll
    for (int f = 0; f < 2; ++f) as[f] = *lds_ptr<uint32_t>(st + a_scale_lane + f * 32 * 4);
#pragma unroll
    for (int f = 0; f < 4; ++f) bs[f] = *lds_ptr<uint32_t>(st + b_scale_lane + f * 32 * 4);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4_t ac[2], bc[4];
#pragma unroll
      for (int f = 0; f < 2; ++f) ac[f] = *lds_ptr<u32x4_t>(st + a_lane[s2] + f * 32 * kMxCodeRow);
#pragma unroll
      for (int f = 0; f < 4; ++f) bc[f] = *lds_ptr<u32x4_t>(st + b_lane[s2] + f * 32 * kMxCodeRow);
      const int sh = 8 * (2 * s2 + hl);   // this lane's block within the stage's four
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const i32x8_t av = {static_cast<int>(ac[mi][0]), static_cast<int>(ac[mi][1]),
                            static_cast<int>(ac[mi][2]), static_cast<int>(ac[mi][3]), 0, 0, 0, 0};
        const int sa = static_cast<int>((as[mi] >> sh) & 0xFFu);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const i32x8_t bv = {static_cast<int>(bc[ni][0]), static_cast<int>(bc[ni][1]),
                              static_cast<int>(bc[ni][2]), static_cast<int>(bc[ni][3]), 0, 0, 0, 0};
          const int sb = static_cast<int>((bs[ni] >> sh) & 0xFFu);
          // formats 4 = FP4 E2M1 for both operands; scale bytes in bits 7:0
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[mi][ni], 4, 4, 0, sa, 0, sb);
        }
      }
    }
  }
  float* s_gx = reinterpret_cast<float*>(lds + kMxGx);
  if (tid < kBM) s_gx[tid] = 1.0f;   // no outer scales: the epilogue's factors are 1
  __syncthreads();   // s_gx visible; every wave is past its last read of the ring
  const float gw[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  fwd_epilogue<MODE>(args, acc, tc, s_gx, gw, lds);
}

template <FwdMode MODE>
bool launch_fwd_mx(const FwdArgs& args, int n_tiles, const char* name, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_mx_kernel<MODE>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kMxLdsBytes);
  if (attr != hipSuccess) return launch_ok(name) && false;
  const int64_t tiles = grouped_m_tiles_bound(args.rows_alloc, args.E, kBM) * n_tiles;
  if (tiles == 0) return true;
  launch_kernel(name, fwd_mx_kernel<MODE>, dim3(xcd_grid(tiles)), dim3(kThreads), kMxLdsBytes, s, args);
  return launch_ok(name);
}

// ---------------------------------------------------- MXFP8 backward GEMMs
// C = A B^T with MXFP8 operands (E4M3 bytes, one E8M0 scale per 32 along K,
// both operands K-contiguous) on the scaled FP8 MFMA (32x32x64), bf16 out.
//   dgrad (WGRAD = false): A rows grouped by expert (offsets), B = the
//     expert's [N, K] slab; the reduction runs over K.
//   wgrad (WGRAD = true): per expert e, A [M1, pitch] and B [N, pitch] are
//     transposed operands whose columns are dispatched rows; the reduction
//     runs over the expert's rows [offsets[e], offsets[e+1]) (a multiple of
//     128: row_align 128), out = dW[e] [M1, N]; an empty expert writes zeros.
// Lane layout of the FP8 operand (checked on the box with one-hot inputs):
// lane l holds row l % 32; its 32 bytes are K [16 h, 16 h + 16) and
// [32 + 16 h, 32 + 16 h + 16) for h = l / 32, bytes 0-15 scaled by lane half
// 0's scale byte of the row and 16-31 by lane half 1's; so lane half h
// supplies the scale of 32-block h.  A stage covers 64 of K (64 B per row,
// the four 16-byte chunks swizzled as in the MXFP4 kernel); the scales of two
// stages (one dword per row) arrive with every other stage in one of two
// buffers.  Three-stage ring, 77.5 KB: two workgroups per CU.
constexpr int kM8BK = 64;
constexpr int kM8Stages = 3;
constexpr int kM8Ahead = kM8Stages - 1;
constexpr int kM8Row = kM8BK;                                  // 64 B of codes per row per stage
constexpr int kM8A = kBM * kM8Row;                             // 8 KB
constexpr int kM8Stage = kM8A + kBN * kM8Row;                  // 24 KB
constexpr int kM8ScaleBuf = kM8Stages * kM8Stage;              // two buffers of 512 rows x 4 B
constexpr int kM8Gx = kM8ScaleBuf + 2 * kScaleRows * 4;
constexpr int kM8Slot = kM8Gx + kBM * 4;
constexpr int kM8LdsBytes = kM8Slot + 16;
static_assert(2 * kM8LdsBytes <= 160 * 1024, "two workgroups per CU must fit in LDS");
static_assert(kOutRows * kOutPitch <= kM8Stages * kM8Stage, "staging fits in the ring");

struct Mx8Args {
  int64_t rows_alloc;       // dgrad: rows of A
  int K;                    // dgrad: reduction length
  int N;                    // columns of C (rows of B)
  int M1;                   // wgrad: rows of C (rows of A)
  int E;
  const int32_t* offsets;
  const uint8_t* a;         // codes
  const uint8_t* as;        // scales
  const uint8_t* b;
  const uint8_t* bs;
  int64_t pitch;            // wgrad: bytes per row of A and B (a multiple of 128)
  uint16_t* out;
};

template <bool WGRAD>
__global__ void __launch_bounds__(kThreads, 2)
mx8_gemm_kernel(Mx8Args args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r32 = lane & 31, hl = lane >> 5;
  const int n_tiles = args.N / kBN;

  TileCoord tc;
  int64_t kofs = 0;        // wgrad: first K column (the expert's first row)
  int kext;                // reduction length of this tile
  const uint8_t* a_base;
  const uint8_t* b_base;
  const uint8_t* as_base;
  const uint8_t* bs_base;
  int64_t a_pitch, b_pitch;
  int a_rows;
  uint16_t* out = args.out;
  if constexpr (!WGRAD) {
    tc = grouped_m_tile<kBM>(args.offsets, args.E, n_tiles, reinterpret_cast<int*>(lds + kM8Slot));
    if (!tc.valid) return;
    kext = args.K;
    a_pitch = b_pitch = args.K;
    a_rows = static_cast<int>(min<int64_t>(kBM, args.rows_alloc - tc.m0));
    a_base = args.a + tc.m0 * a_pitch;
    as_base = args.as + tc.m0 * (a_pitch / 32);
    b_base = args.b + static_cast<int64_t>(tc.e) * args.N * b_pitch;
    bs_base = args.bs + static_cast<int64_t>(tc.e) * args.N * (b_pitch / 32);
  } else {
    // expert-major tiles, dealt in contiguous runs per XCD
    const int m_tiles = args.M1 / kBM;
    const int64_t total = static_cast<int64_t>(args.E) * m_tiles * n_tiles;
    const int64_t per_xcd = (total + kXcds - 1) / kXcds;
    const int64_t bid = blockIdx.x;
    const int64_t L = (bid % kXcds) * per_xcd + bid / kXcds;
    if (bid / kXcds >= per_xcd || L >= total) return;
    const int e = static_cast<int>(L / (m_tiles * n_tiles));
    const int rem = static_cast<int>(L % (m_tiles * n_tiles));
    tc.e = e;
    tc.m0 = static_cast<int64_t>(rem / n_tiles) * kBM;
    tc.m_end = args.M1;
    tc.n_tile = rem % n_tiles;
    tc.valid = true;
    kofs = args.offsets[e];
    kext = args.offsets[e + 1] - static_cast<int>(kofs);
    a_pitch = b_pitch = args.pitch;
    a_rows = kBM;
    a_base = args.a + tc.m0 * a_pitch + kofs;
    as_base = args.as + tc.m0 * (a_pitch / 32) + kofs / 32;
    b_base = args.b + kofs;
    bs_base = args.bs + kofs / 32;
    out += static_cast<int64_t>(e) * args.M1 * args.N;
  }

  // code copies: copy q of this wave fills 16 staged rows (1 KB), lane i row
  // 16 q' + i / 4 at slot i % 4 (A: q' = 2 wave + q; B: q' = 4 wave + q)
  uint32_t a_off[2], b_off[4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * (2 * wave + q) + (lane >> 2);
    a_off[q] = static_cast<uint32_t>(min(row, a_rows - 1) * a_pitch + mx_code_slot(row, lane & 3) * 16);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 16 * (4 * wave + q) + (lane >> 2);
    b_off[q] = static_cast<uint32_t>(b_row_of<FwdMode::FC2>(row, tc.n_tile, 0) * b_pitch +
                                     mx_code_slot(row, lane & 3) * 16);
  }
  // scale copies: one dword (two stages' blocks) per staged row
  const uint8_t* scale_src[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int q = 128 * wave + 64 * c + lane;
    if (q < kBScaleRow0)
      scale_src[c] = as_base + static_cast<int64_t>(min(q, a_rows - 1)) * (a_pitch / 32);
    else if (q < kBScaleRow0 + kBN)
      scale_src[c] = bs_base + static_cast<int64_t>(b_row_of<FwdMode::FC2>(q - kBScaleRow0, tc.n_tile, 0)) *
                                   (b_pitch / 32);
    else
      scale_src[c] = as_base;                                  // filler: a valid row, never read
  }
  // The copies' global offsets are 32-bit: bound checked by the host.
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int kt) {
    if (kt % 2 == 0) {   // the pair's scales go out first: they land before the stage's codes
      const uint32_t sb = lds0 + kM8ScaleBuf + ((kt / 2) % 2) * (kScaleRows * 4);
#pragma unroll
      for (int c = 0; c < 2; ++c) dma4(scale_src[c] + (kt / 2) * 4, sb + (2 * wave + c) * 256);
    }
    const uint32_t st = lds0 + (kt % kM8Stages) * kM8Stage;
    const int cb = kt * kM8Row;
#pragma unroll
    for (int q = 0; q < 2; ++q) dma16_off(a_base + cb, a_off[q], st + (2 * wave + q) * 1024);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16_off(b_base + cb, b_off[q], st + kM8A + (4 * wave + q) * 1024);
  };

  floatx16_t acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  const int a_row0 = wm * kWM + r32, b_row0 = wn * kWN + r32;
  const int sw = (r32 >> 2) & 3;
  const uint32_t a_lane0 = a_row0 * kM8Row + (hl ^ sw) * 16, a_lane1 = a_row0 * kM8Row + ((2 + hl) ^ sw) * 16;
  const uint32_t b_lane0 = kM8A + b_row0 * kM8Row + (hl ^ sw) * 16;
  const uint32_t b_lane1 = kM8A + b_row0 * kM8Row + ((2 + hl) ^ sw) * 16;
  const uint32_t a_scale_lane = a_row0 * 4, b_scale_lane = (kBScaleRow0 + b_row0) * 4;
  const int nk = kext / kM8BK;
  for (int s0 = 0; s0 < kM8Ahead && s0 < nk; ++s0) issue(s0);

  const bool rows_live = tc.m0 + wm * kWM < tc.m_end;
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt (and its pair's scales) has landed in every wave: at most the
    // copies of stage kt + 1, if issued, are pending
    if (kt + 1 < nk) {
      if ((kt + 1) % 2 == 0) wait_vm_barrier<8>();
      else wait_vm_barrier<6>();
    } else {
      wait_vm_barrier<0>();
    }
    if (kt + kM8Ahead < nk) issue(kt + kM8Ahead);
    if (!rows_live) continue;
    const uint32_t st = opaque_sgpr(lds0 + (kt % kM8Stages) * kM8Stage);
    const uint32_t sb = opaque_sgpr(lds0 + kM8ScaleBuf + ((kt / 2) % 2) * (kScaleRows * 4));
    const int sh = 8 * (2 * (kt % 2) + hl);   // this lane's block among the dword's four
    int sa[2], sbv[4];
    i32x8_t av[2], bv[4];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const u32x4_t lo = *lds_ptr<u32x4_t>(st + a_lane0 + f * 32 * kM8Row);
      const u32x4_t hi = *lds_ptr<u32x4_t>(st + a_lane1 + f * 32 * kM8Row);
      av[f] = i32x8_t{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                      static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                      static_cast<int>(hi[2]), static_cast<int>(hi[3])};
      sa[f] = static_cast<int>((*lds_ptr<uint32_t>(sb + a_scale_lane + f * 32 * 4) >> sh) & 0xFFu);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const u32x4_t lo = *lds_ptr<u32x4_t>(st + b_lane0 + f * 32 * kM8Row);
      const u32x4_t hi = *lds_ptr<u32x4_t>(st + b_lane1 + f * 32 * kM8Row);
      bv[f] = i32x8_t{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                      static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                      static_cast<int>(hi[2]), static_cast<int>(hi[3])};
      sbv[f] = static_cast<int>((*lds_ptr<uint32_t>(sb + b_scale_lane + f * 32 * 4) >> sh) & 0xFFu);
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        // formats 0 = FP8 E4M3 for both operands; scale bytes in bits 7:0
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[mi], bv[ni], acc[mi][ni], 0, 0, 0,
                                                                      sa[mi], 0, sbv[ni]);
  }
  float* s_gx = reinterpret_cast<float*>(lds + kM8Gx);
  if (tid < kBM) s_gx[tid] = 1.0f;
  __syncthreads();   // s_gx visible; every wave is past its last read of the ring
  const float gw[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  FwdArgs fa{};
  fa.N = args.N;
  fa.out = out;
  fwd_epilogue<FwdMode::FC2>(fa, acc, tc, s_gx, gw, lds);
}

template <bool WGRAD>
bool launch_mx8(const Mx8Args& args, int64_t tiles, const char* name, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&mx8_gemm_kernel<WGRAD>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kM8LdsBytes);
  if (attr != hipSuccess) return launch_ok(name) && false;
  if (tiles == 0) return true;
  launch_kernel(name, mx8_gemm_kernel<WGRAD>, dim3(xcd_grid(tiles)), dim3(kThreads), kM8LdsBytes, s, args);
  return launch_ok(name);
}

template <FwdMode MODE, bool GS>
bool launch_fwd_variant(const FwdArgs& args, int64_t tiles, const char* name, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fwd_gemm_kernel<MODE, GS>),
      hipFuncAttributeMaxDynamicSharedMemorySize, FwdLds<GS>::kBytes);
  if (attr != hipSuccess) return launch_ok(name) && false;
  launch_kernel(name, fwd_gemm_kernel<MODE, GS>, dim3(xcd_grid(tiles)), dim3(kThreads), FwdLds<GS>::kBytes, s,
                args);
  return launch_ok(name);
}

template <FwdMode MODE>
bool launch_fwd(const FwdArgs& args, int n_tiles, const char* name, hipStream_t s) {
  const int64_t tiles = grouped_m_tiles_bound(args.rows_alloc, args.E, kBM) * n_tiles;
  if (tiles == 0) return true;
  // codes arrive in pairs of 64-k stages: every caller's K (H, I, the dense
  // layer's K) is a multiple of 128, which the shape checks enforce
  if (args.K % (2 * kBK) != 0) return false;
  if (args.K % (kGroup * kBK) == 0) return launch_fwd_variant<MODE, true>(args, tiles, name, s);
  return launch_fwd_variant<MODE, false>(args, tiles, name, s);
}

}  // namespace

bool launch_fc1(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets, Fp4Operand x,
                Fp4Operand w1, uint16_t* h_out, uint16_t* a_out, float* dbg_f32, hipStream_t s) {
  FwdArgs args{rows_alloc, H, 2 * I, I, E, offsets, x, w1, h_out, a_out, dbg_f32};
  return launch_fwd<FwdMode::FC1>(args, I / 128, "gemm_fc1", s);
}

bool launch_fc2(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets, Fp4Operand a,
                Fp4Operand w2, uint16_t* o_out, hipStream_t s) {
  FwdArgs args{rows_alloc, I, H, I, E, offsets, a, w2, o_out, nullptr, nullptr};
  return launch_fwd<FwdMode::FC2>(args, H / kBN, "gemm_fc2", s);
}

bool launch_linear_fwd(int64_t T, int K, int N, const int32_t* offsets, Fp4Operand x, Fp4Operand w,
                       uint16_t* y, hipStream_t s) {
  FwdArgs args{T, K, N, K, 1, offsets, x, w, y, nullptr, nullptr};
  return launch_fwd<FwdMode::FC2>(args, N / kBN, "gemm_linear", s);
}

bool launch_fc1_mx(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets, Fp4Operand x,
                   Fp4Operand w1, uint16_t* h_out, uint16_t* a_out, float* dbg_f32, hipStream_t s) {
  if (H % kMxBK) return false;
  FwdArgs args{rows_alloc, H, 2 * I, I, E, offsets, x, w1, h_out, a_out, dbg_f32};
  return launch_fwd_mx<FwdMode::FC1>(args, I / 128, "mx_gemm_fc1", s);
}

bool launch_fc2_mx(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets, Fp4Operand a,
                   Fp4Operand w2, uint16_t* o_out, hipStream_t s) {
  if (I % kMxBK) return false;
  FwdArgs args{rows_alloc, I, H, I, E, offsets, a, w2, o_out, nullptr, nullptr};
  return launch_fwd_mx<FwdMode::FC2>(args, H / kBN, "mx_gemm_fc2", s);
}

bool launch_mx8_dgrad(int64_t rows_alloc, int K, int N, int E, const int32_t* offsets, const uint8_t* a,
                      const uint8_t* as, const uint8_t* b, const uint8_t* bs, uint16_t* out, const char* name,
                      hipStream_t s) {
  if (K % 128 || N % kBN) return false;
  if (static_cast<int64_t>(kBM) * K > (int64_t{1} << 31) || static_cast<int64_t>(N) * K > (int64_t{1} << 31))
    return false;   // 32-bit per-lane copy offsets
  Mx8Args args{rows_alloc, K, N, 0, E, offsets, a, as, b, bs, 0, out};
  return launch_mx8<false>(args, grouped_m_tiles_bound(rows_alloc, E, kBM) * (N / kBN), name, s);
}

bool launch_mx8_wgrad(int M1, int N, int E, const int32_t* offsets, const uint8_t* a, const uint8_t* as,
                      const uint8_t* b, const uint8_t* bs, int64_t pitch, uint16_t* out, const char* name,
                      hipStream_t s) {
  if (M1 % kBM || N % kBN || pitch % 128) return false;
  if (static_cast<int64_t>(N) * pitch > (int64_t{1} << 31) || static_cast<int64_t>(kBM) * pitch > (int64_t{1} << 31))
    return false;   // 32-bit per-lane copy offsets
  Mx8Args args{0, 0, N, M1, E, offsets, a, as, b, bs, pitch, out};
  return launch_mx8<true>(args, static_cast<int64_t>(E) * (M1 / kBM) * (N / kBN), name, s);
}

}  // namespace w4a4
