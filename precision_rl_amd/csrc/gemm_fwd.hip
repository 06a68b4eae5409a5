// Steps a5 (+a6) and a8: grouped block-scaled GEMMs FC1 and FC2 on gfx950.
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
// Tiling: 256 x 256 output tile per workgroup of 8 waves (4 x 2, 64 x 128 per
// wave, two waves per SIMD), MFMA 32x32x16 f16.  Each pipeline stage covers 128
// of K: packed codes (64 B per row) and block scales (8 B per row) of both
// operands go through LDS, double buffered; waves 0-3 fetch the activation tile
// and waves 4-7 the weight tile, one stage ahead of the MFMAs.  Inside a stage,
// lane half h (lanes 32-63) owns the stage's second 64 k of its row; A and B
// use the same assignment, so every MFMA k slot pairs equal k indices (the
// reduction runs in a permuted K order; FP32 rounding of the sum is covered by
// the tolerance, and sums that are exact in FP32 are order independent).

#include "gemm_common.h"
#include "internal.h"

namespace w4a4 {
namespace {

constexpr int kBK = 128;                    // K per stage
constexpr int kCodeRow = kBK / 2;           // 64 B of codes per row per stage
constexpr int kCodeStride = kCodeRow + 16;  // 80 B: conflict-free b128 reads
constexpr int kScaleRow = kBK / 16;         // 8 scale bytes per row per stage
constexpr int kOpCodes = kTileM * kCodeStride;
constexpr int kOpScales = kTileM * kScaleRow;
constexpr int kOpBytes = kOpCodes + kOpScales;
constexpr int kStageBytes = 2 * kOpBytes;
constexpr int kGxOffset = 2 * kStageBytes;  // 2 stages, then the tile's g_x
constexpr int kLdsBytes = kGxOffset + kTileM * 4;
constexpr int kLoaders = kGemmThreads / 2;  // threads fetching one operand

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
    return n_tile * kTileN + wn * 128 + 4 * j + ni;
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

// Two of the four E4M3 scale bytes in `sc` (selected by HI) as f16 pairs.
template <bool HI>
__device__ __forceinline__ void scale_pairs(uint32_t sc, half2_t& d0, half2_t& d1) {
  const half2_t v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, HI);
  d0 = half2_t{v[0], v[0]};
  d1 = half2_t{v[1], v[1]};
}

template <FwdMode MODE>
__global__ void __launch_bounds__(kGemmThreads, 1)
fwd_gemm_kernel(FwdArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 3, wn = wave >> 2;
  const int r32 = lane & 31, hl = lane >> 5;

  const int n_tiles = MODE == FwdMode::FC1 ? args.I / 128 : args.N / kTileN;
  TileCoord tc = grouped_m_tile(args.offsets, args.E, n_tiles, reinterpret_cast<int*>(lds));
  if (!tc.valid) return;
  __syncthreads();  // the scan scratch aliases the stage buffers

  const int64_t K2 = args.K / 2, K16 = args.K / 16;
  // ---- this thread's loads: waves 0-3 fetch A (activations), 4-7 fetch B (weights)
  const bool loads_b = tid >= kLoaders;
  const int lt = tid & (kLoaders - 1);
  const uint8_t* code_src[4];
  const uint8_t* scale_src;
  {
    const uint8_t* wcodes = args.w.codes + static_cast<int64_t>(tc.e) * args.N * K2;
    const uint8_t* wscales = args.w.scales + static_cast<int64_t>(tc.e) * args.N * K16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = lt + i * kLoaders;
      const int row = q >> 2, col = q & 3;
      if (loads_b) {
        code_src[i] = wcodes + static_cast<int64_t>(b_row_of<MODE>(row, tc.n_tile, args.I)) * K2 + col * 16;
      } else {
        int64_t ar = tc.m0 + row;
        if (ar >= args.rows_alloc) ar = args.rows_alloc - 1;   // in bounds; never stored
        code_src[i] = args.a.codes + ar * K2 + col * 16;
      }
    }
    if (loads_b) {
      scale_src = wscales + static_cast<int64_t>(b_row_of<MODE>(lt, tc.n_tile, args.I)) * K16;
    } else {
      int64_t ar = tc.m0 + lt;
      if (ar >= args.rows_alloc) ar = args.rows_alloc - 1;
      scale_src = args.a.scales + ar * K16;
      // outer scales of the tile's rows, read by the epilogue from LDS
      reinterpret_cast<float*>(lds + kGxOffset)[lt] = args.a.outer[ar];
    }
  }
  const float* s_gx = reinterpret_cast<const float*>(lds + kGxOffset);
  const int op_off = loads_b ? kOpBytes : 0;

  u32x4_t pf_code[4];
  u32x2_t pf_scale;
  auto load_stage = [&](int kt) {
    const int64_t cb = static_cast<int64_t>(kt) * kCodeRow;
#pragma unroll
    for (int i = 0; i < 4; ++i) pf_code[i] = *reinterpret_cast<const u32x4_t*>(code_src[i] + cb);
    pf_scale = *reinterpret_cast<const u32x2_t*>(scale_src + static_cast<int64_t>(kt) * kScaleRow);
  };
  auto store_stage = [&](int buf) {
    uint8_t* base = lds + buf * kStageBytes + op_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = lt + i * kLoaders;
      *reinterpret_cast<u32x4_t*>(base + (q >> 2) * kCodeStride + (q & 3) * 16) = pf_code[i];
    }
    *reinterpret_cast<u32x2_t*>(base + kOpCodes + lt * kScaleRow) = pf_scale;
  };

  floatx16_t acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;
  bool mi_live[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) mi_live[mi] = tc.m0 + wm * kWaveM + mi * 32 < tc.m_end;

  const int a_row0 = wm * kWaveM + r32, b_row0 = wn * kWaveN + r32;
  const int nk = args.K / kBK;
  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_stage(kt + 1);
    const uint8_t* sa = lds + (kt & 1) * kStageBytes;
    const uint8_t* sb = sa + kOpBytes;
    uint32_t a_sc[2], b_sc[4];
#pragma unroll
    for (int f = 0; f < 2; ++f)
      a_sc[f] = *reinterpret_cast<const uint32_t*>(sa + kOpCodes + (a_row0 + f * 32) * kScaleRow + hl * 4);
#pragma unroll
    for (int f = 0; f < 4; ++f)
      b_sc[f] = *reinterpret_cast<const uint32_t*>(sb + kOpCodes + (b_row0 + f * 32) * kScaleRow + hl * 4);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      u32x4_t ac[2], bc[4];
#pragma unroll
      for (int f = 0; f < 2; ++f)
        ac[f] = *reinterpret_cast<const u32x4_t*>(sa + (a_row0 + f * 32) * kCodeStride + hl * 32 + hh * 16);
#pragma unroll
      for (int f = 0; f < 4; ++f)
        bc[f] = *reinterpret_cast<const u32x4_t*>(sb + (b_row0 + f * 32) * kCodeStride + hl * 32 + hh * 16);
      half2_t ad[2][2], bd[4][2];   // block scales of blocks 2hh, 2hh+1 as f16 pairs
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (hh == 0) scale_pairs<false>(a_sc[f], ad[f][0], ad[f][1]);
        else scale_pairs<true>(a_sc[f], ad[f][0], ad[f][1]);
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if (hh == 0) scale_pairs<false>(b_sc[f], bd[f][0], bd[f][1]);
        else scale_pairs<true>(b_sc[f], bd[f][0], bd[f][1]);
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        half8_t af[2], bf[4];
#pragma unroll
        for (int f = 0; f < 2; ++f) af[f] = decode8(ac[f][s4], ad[f][s4 >> 1]);
#pragma unroll
        for (int f = 0; f < 4; ++f) bf[f] = decode8(bc[f][s4], bd[f][s4 >> 1]);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          if (!mi_live[mi]) continue;   // all 32 rows past the expert's end
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) store_stage((kt + 1) & 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  const float* wouter = args.w.outer + static_cast<int64_t>(tc.e) * args.N;
  if constexpr (MODE == FwdMode::FC2) {
    const int n = tc.n_tile * kTileN + wn * kWaveN + 4 * r32;
    float gw[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) gw[ni] = wouter[n + ni];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lrow = acc_row(wm * kWaveM, mi, v, hl);
        const int64_t row = tc.m0 + lrow;
        if (row >= tc.m_end) continue;
        const float gx = s_gx[lrow];
        float o[4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) o[ni] = acc[mi][ni][v] * (gx * gw[ni]);
        u32x2_t pk;
        pk[0] = pack_bf16x2(o[0], o[1]);
        pk[1] = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<u32x2_t*>(args.out + row * args.N + n) = pk;
      }
    }
  } else {
    const int I = args.I;
    const int i = tc.n_tile * 128 + wn * 64 + 2 * r32;
    const float gw_g0 = wouter[i], gw_g1 = wouter[i + 1];
    const float gw_u0 = wouter[I + i], gw_u1 = wouter[I + i + 1];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lrow = acc_row(wm * kWaveM, mi, v, hl);
        const int64_t row = tc.m0 + lrow;
        if (row >= tc.m_end) continue;
        const float gx = s_gx[lrow];
        const float g0 = acc[mi][0][v] * (gx * gw_g0);
        const float g1 = acc[mi][1][v] * (gx * gw_g1);
        const float u0 = acc[mi][2][v] * (gx * gw_u0);
        const float u1 = acc[mi][3][v] * (gx * gw_u1);
        if (args.dbg != nullptr) {
          float* d = args.dbg + row * (2 * I);
          *reinterpret_cast<float2*>(d + i) = make_float2(g0, g1);
          *reinterpret_cast<float2*>(d + I + i) = make_float2(u0, u1);
        }
        const uint32_t hg = pack_bf16x2(g0, g1), hu = pack_bf16x2(u0, u1);
        if (args.out != nullptr) {
          uint16_t* h = args.out + row * (2 * I);
          *reinterpret_cast<uint32_t*>(h + i) = hg;
          *reinterpret_cast<uint32_t*>(h + I + i) = hu;
        }
        // SwiGLU on the bf16-rounded h, FP32 arithmetic
        const float bg0 = bf16_to_f32(static_cast<uint16_t>(hg & 0xFFFFu));
        const float bg1 = bf16_to_f32(static_cast<uint16_t>(hg >> 16));
        const float bu0 = bf16_to_f32(static_cast<uint16_t>(hu & 0xFFFFu));
        const float bu1 = bf16_to_f32(static_cast<uint16_t>(hu >> 16));
        const float a0 = bg0 / (1.0f + expf(-bg0)) * bu0;
        const float a1 = bg1 / (1.0f + expf(-bg1)) * bu1;
        *reinterpret_cast<uint32_t*>(args.act + row * I + i) = pack_bf16x2(a0, a1);
      }
    }
  }
}

template <FwdMode MODE>
bool launch_fwd(const FwdArgs& args, int n_tiles, const char* name, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fwd_gemm_kernel<MODE>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (attr != hipSuccess) return launch_ok(name) && false;
  const int64_t tiles = grouped_m_tiles_bound(args.rows_alloc, args.E) * n_tiles;
  if (tiles == 0) return true;
  {
    ProfScope p(name, s);
    fwd_gemm_kernel<MODE><<<dim3(xcd_grid(tiles)), dim3(kGemmThreads), kLdsBytes, s>>>(args);
  }
  return launch_ok(name);
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
  return launch_fwd<FwdMode::FC2>(args, H / kTileN, "gemm_fc2", s);
}

}  // namespace w4a4
