// MXFP8 operand preparation for the MXFP8 variant of the straight-through
// backward on gfx950: quantisers along rows and along columns (transposing),
// and the SwiGLU backward as a pass of its own.
//
// Format (OCP Microscaling Formats v1.0, section 6.3, with E4M3 elements;
// the backward the pages compare against their BF16 one, AI summary, key
// findings): per block of 32 consecutive elements along the GEMM's reduction
// axis, X = floor(log2 amax) - 8 clamped to [-127, 127], an E8M0 scale byte
// X + 127, and elements Q_E4M3(x / 2^X) -- round to nearest, ties to even,
// subnormals kept, saturating at 448 (amax / 2^X lies in [256, 512)).  From
// the bf16 exponent field eb of the block amax the byte is max(eb - 8, 0).
// x / 2^X is exact in FP32 (a bf16 value scaled by a power of two; results
// below FP32's subnormal range lie far below E4M3's smallest midpoint), so the
// rounding acts on the exact quotient.

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace w4a4 {
namespace {

constexpr int kQ8Threads = 256;

// E4M3FN byte of v >= 0 (finite), RNE, subnormals kept, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_of(float v) {
  if (v >= 448.0f) return 0x7Eu;
  if (v < 0.015625f)                                             // below 2^-6: spacing 2^-9
    return static_cast<uint32_t>(__builtin_rintf(v * 512.0f));   // 0..8; 8 is 2^-6 = 0x08
  const uint32_t b = __float_as_uint(v);
  const uint32_t m3 = (b >> 20) & 7u, rem = b & 0xFFFFFu;
  uint32_t r = ((((b >> 23) & 0xFFu) - 120u) << 3) | m3;         // biased exponent e + 7
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++r;    // carries into the exponent
  return r < 0x7Eu ? r : 0x7Eu;
}

// Scale byte and 2^-X of a block from its amax (bf16 magnitude bits).
__device__ __forceinline__ uint32_t mx8_scale_byte(uint32_t amax16) {
  const uint32_t eb = amax16 >> 7;
  return eb > 8u ? eb - 8u : 0u;
}
__device__ __forceinline__ float mx8_inv_scale(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);   // 2^(127 - byte) = 2^-X, X in [-127, 119]
}

__device__ __forceinline__ uint32_t e4m3_of_bf16(uint32_t x16, float inv) {
  const float v = bf16_to_f32(static_cast<uint16_t>(x16 & 0x7FFFu)) * inv;
  return e4m3_of(v) | ((x16 >> 8) & 0x80u);
}

// ------------------------------------------------------------- along rows
// One thread per block of 32 elements of a row: 64 B read, 32 B of E4M3 and
// one scale byte written.  Rows [0, offsets[E]) when offsets is given (the
// dispatched rows; pad rows are zeros and encode as zeros), else all rows.
__global__ void __launch_bounds__(kQ8Threads)
q8_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int K, const int32_t* __restrict__ offsets, int E,
               uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int nb = K / 32;
  int64_t n = rows;
  if (offsets != nullptr) n = min<int64_t>(n, offsets[E]);
  const int64_t total = n * nb;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kQ8Threads + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * kQ8Threads) {
    const int64_t r = i / nb;
    const int b = static_cast<int>(i % nb);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + r * K + b * 32);
    u32x4_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = __builtin_nontemporal_load(src + j);
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int d = 0; d < 4; ++d) amax = max(amax, max(w[j][d] & 0x7FFFu, (w[j][d] >> 16) & 0x7FFFu));
    const uint32_t byte = mx8_scale_byte(amax);
    const float inv = mx8_inv_scale(byte);
    u32x4_t o[2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = e4m3_of_bf16(w[j][d] & 0xFFFFu, inv), hi = e4m3_of_bf16(w[j][d] >> 16, inv);
        const int e = 8 * j + 2 * d;   // element index within the block
        const uint32_t pair = lo | (hi << 8);
        if ((e & 3) == 0) o[e >> 4][(e >> 2) & 3] = pair;
        else o[e >> 4][(e >> 2) & 3] |= pair << 16;
      }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(q + r * K + b * 32);
    __builtin_nontemporal_store(o[0], dst);
    __builtin_nontemporal_store(o[1], dst + 1);
    s[r * nb + b] = static_cast<uint8_t>(byte);
  }
}

// ---------------------------------------------------------- along columns
// x: `batch` matrices [R, C] bf16 (batch stride R*C).  Output per matrix:
// q [C, pitch] E4M3 (row c holds column c of x, quantised in blocks of 32
// consecutive rows), s [C, pitch/32].  A workgroup takes 128 rows x 64
// columns through LDS (each input row segment is one 128-byte line); four
// consecutive threads encode the four 32-row blocks of one column, so that
// together they write the column's 128 output bytes as one line.  Row tiles
// at or past offsets[E] (when given) are skipped: the rows encoded must come
// in whole tiles of 128 (row_align 128 for dispatched rows; R % 128 == 0
// for weights).
constexpr int kColTileRows = 128, kColTileCols = 64;
constexpr int kColPitch = kColTileCols + 2;   // elements; 2-way LDS conflicts at most on the column reads
__global__ void __launch_bounds__(kQ8Threads)
q8_cols_kernel(const uint16_t* __restrict__ x, int64_t R, int C, const int32_t* __restrict__ offsets, int E,
               int64_t pitch, uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  __shared__ uint16_t tile[kColTileRows * kColPitch];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kColTileRows;
  const int c0 = blockIdx.y * kColTileCols;
  const int mat = blockIdx.z;
  const int64_t rlim = offsets != nullptr ? min<int64_t>(R, offsets[E]) : R;
  if (r0 >= rlim) return;
  const uint16_t* xm = x + static_cast<int64_t>(mat) * R * C;
  const int t = threadIdx.x;
  // load: thread t moves the 16-byte chunk t % 8 of rows t / 8 + 32 i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = t / 8 + 32 * i, ch = t % 8;
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(xm + (r0 + lr) * C + c0 + ch * 8));
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + lr * kColPitch + ch * 8);
#pragma unroll
    for (int d = 0; d < 4; ++d) dst[d] = v[d];
  }
  __syncthreads();
  const int c = t / 4, blk = t % 4;
  const uint16_t* col = tile + (32 * blk) * kColPitch + c;
  uint32_t amax = 0;
#pragma unroll
  for (int r = 0; r < 32; ++r) amax = max(amax, static_cast<uint32_t>(col[r * kColPitch] & 0x7FFFu));
  const uint32_t byte = mx8_scale_byte(amax);
  const float inv = mx8_inv_scale(byte);
  u32x4_t o[2];
#pragma unroll
  for (int r = 0; r < 32; r += 4) {
    uint32_t wd = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) wd |= e4m3_of_bf16(col[(r + j) * kColPitch], inv) << (8 * j);
    o[r >> 4][(r >> 2) & 3] = wd;
  }
  const int64_t cc = c0 + c;
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(q + static_cast<int64_t>(mat) * C * pitch + cc * pitch + r0 + 32 * blk);
  __builtin_nontemporal_store(o[0], dst);
  __builtin_nontemporal_store(o[1], dst + 1);
  s[(static_cast<int64_t>(mat) * C + cc) * (pitch / 32) + r0 / 32 + blk] = static_cast<uint8_t>(byte);
}

// ------------------------------------------------------- SwiGLU backward
// dH = [dA u s (1 + g (1 - s)), dA g s] with g, u the bf16 gate / up halves
// of h and s = sigmoid(g), FP32 arithmetic, bf16 results (the formula and
// arithmetic of the BF16 backward's fused epilogue).  One thread per 8
// features of a row; rows [0, offsets[E]).
__global__ void __launch_bounds__(kQ8Threads)
swiglu_bwd_kernel(const uint16_t* __restrict__ dA, const uint16_t* __restrict__ h, int64_t rows, int I,
                  const int32_t* __restrict__ offsets, int E, uint16_t* __restrict__ dH) {
  const int64_t n = min<int64_t>(rows, offsets[E]);
  const int per_row = I / 8;
  const int64_t total = n * per_row;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kQ8Threads + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * kQ8Threads) {
    const int64_t r = i / per_row;
    const int c = static_cast<int>(i % per_row) * 8;
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(dA + r * I + c));
    const u32x4_t hg = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(h + r * (2 * I) + c));
    const u32x4_t hu = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(h + r * (2 * I) + I + c));
    u32x4_t dg, du;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float rg[2], ru[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const float da = bf16_to_f32(static_cast<uint16_t>(v[d] >> (16 * p)));
        const float gt = bf16_to_f32(static_cast<uint16_t>(hg[d] >> (16 * p)));
        const float up = bf16_to_f32(static_cast<uint16_t>(hu[d] >> (16 * p)));
        const float sg = sigmoid_fast(gt);
        rg[p] = da * up * sg * (1.0f + gt * (1.0f - sg));
        ru[p] = da * gt * sg;
      }
      dg[d] = pack_bf16x2(rg[0], rg[1]);
      du[d] = pack_bf16x2(ru[0], ru[1]);
    }
    __builtin_nontemporal_store(dg, reinterpret_cast<u32x4_t*>(dH + r * (2 * I) + c));
    __builtin_nontemporal_store(du, reinterpret_cast<u32x4_t*>(dH + r * (2 * I) + I + c));
  }
}

unsigned grid_for(int64_t work) {
  const int64_t blocks = (work + kQ8Threads - 1) / kQ8Threads;
  return static_cast<unsigned>(std::min<int64_t>(std::max<int64_t>(blocks, 1),
                                                 static_cast<int64_t>(device_cu_count()) * 16));
}

}  // namespace

bool launch_q8_rows(const uint16_t* x, int64_t rows, int K, const int32_t* offsets, int E, uint8_t* q,
                    uint8_t* s, const char* name, hipStream_t st) {
  if (rows == 0) return true;
  launch_kernel(name, q8_rows_kernel, dim3(grid_for(rows * (K / 32))), dim3(kQ8Threads), 0, st, x, rows, K,
                offsets, E, q, s);
  return launch_ok(name);
}

bool launch_q8_cols(const uint16_t* x, int64_t R, int C, int batch, const int32_t* offsets, int E,
                    int64_t pitch, uint8_t* q, uint8_t* s, const char* name, hipStream_t st) {
  if (R == 0 || batch == 0) return true;
  if (C % kColTileCols || pitch % 128) return false;
  if (offsets == nullptr && R % kColTileRows) return false;
  const dim3 grid(static_cast<unsigned>(R / kColTileRows), static_cast<unsigned>(C / kColTileCols),
                  static_cast<unsigned>(batch));
  launch_kernel(name, q8_cols_kernel, grid, dim3(kQ8Threads), 0, st, x, R, C, offsets, E, pitch, q, s);
  return launch_ok(name);
}

bool launch_swiglu_bwd(const uint16_t* dA, const uint16_t* h, int64_t rows, int I, const int32_t* offsets, int E,
                       uint16_t* dH, hipStream_t st) {
  if (rows == 0) return true;
  launch_kernel("swiglu_bwd", swiglu_bwd_kernel, dim3(grid_for(rows * (I / 8))), dim3(kQ8Threads), 0, st, dA, h,
                rows, I, offsets, E, dH);
  return launch_ok("swiglu_bwd");
}

}  // namespace w4a4
