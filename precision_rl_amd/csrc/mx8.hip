// MXFP8 operand preparation for the MXFP8 variant of the straight-through
// backward on gfx950: a quantiser along columns (transposing; the weights),
// and one that writes both forms of a matrix from a single read (dO; and dH,
// formed from dA and h by the SwiGLU backward inside the pass).
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
// rounding acts on the exact quotient.  The rounding itself is the
// hardware's FP8 conversion (checked byte for byte against the oracle).

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace w4a4 {
namespace {

constexpr int kQ8Threads = 256;

typedef short short2_t __attribute__((ext_vector_type(2)));

// Scale byte and 2^-X of a block from its amax (bf16 magnitude bits).
__device__ __forceinline__ uint32_t mx8_scale_byte(uint32_t amax16) {
  const uint32_t eb = amax16 >> 7;
  return eb > 8u ? eb - 8u : 0u;
}
__device__ __forceinline__ float mx8_inv_scale(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);   // 2^(127 - byte) = 2^-X, X in [-127, 119]
}

// E4M3FN bytes of two bf16 values x0, x1 scaled by inv (a power of two):
// byte 0 from x0, byte 1 from x1.  The magnitudes |x| * inv are exact in FP32;
// clamped to 448 they go through the hardware's OCP FP8 conversion (round to
// nearest even, subnormals kept), which then never overflows: saturating
// RNE of anything at or above 448 is 448.  The sign bits are copied from x
// (-0 encodes as 0x80).
__device__ __forceinline__ uint32_t e4m3_pair_of_bf16(uint32_t x0, uint32_t x1, float inv) {
  const float v0 = fminf(bf16_to_f32(static_cast<uint16_t>(x0 & 0x7FFFu)) * inv, 448.0f);
  const float v1 = fminf(bf16_to_f32(static_cast<uint16_t>(x1 & 0x7FFFu)) * inv, 448.0f);
  const short2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(short2_t{0, 0}, v0, v1, 1.0f, false);
  const uint32_t m = static_cast<uint32_t>(static_cast<uint16_t>(r[0]));
  return m | ((x0 >> 8) & 0x80u) | (x1 & 0x8000u);
}

// ------------------------------------------------------ column / row passes
// Tiles of 128 rows x 128 columns go through LDS (each input row segment is
// two 128-byte lines).  Along columns, four consecutive threads encode the
// four 32-row blocks of one column, so that together they write its 128
// output bytes as one line and its four scale bytes as one dword; along rows
// (the dual pass), four consecutive threads encode the four 32-column blocks
// of one row, likewise one line and one dword.
constexpr int kColTileRows = 128, kColTileCols = 128;
constexpr int kColPitch = kColTileCols + 2;   // elements; 2-way LDS conflicts at most on the column reads

// The four scale bytes of lanes 4j .. 4j+3 (byte of lane 4j + b in bits 8b) in every one of them.
__device__ __forceinline__ uint32_t gather4(uint32_t byte, int blk) {
  uint32_t v = byte << (8 * blk);
  v |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 1, kWave));
  v |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 2, kWave));
  return v;
}

// Encodes 32 values of the tile, `stride` elements apart from `p`: the E4M3
// bytes into o[0..1], returns the scale byte.
__device__ __forceinline__ uint32_t encode32(const uint16_t* p, int stride, u32x4_t (&o)[2]) {
  uint32_t amax = 0;
#pragma unroll
  for (int r = 0; r < 32; ++r) amax = max(amax, static_cast<uint32_t>(p[r * stride] & 0x7FFFu));
  const uint32_t byte = mx8_scale_byte(amax);
  const float inv = mx8_inv_scale(byte);
#pragma unroll
  for (int r = 0; r < 32; r += 4) {
    const uint32_t lo = e4m3_pair_of_bf16(p[r * stride], p[(r + 1) * stride], inv);
    const uint32_t hi = e4m3_pair_of_bf16(p[(r + 2) * stride], p[(r + 3) * stride], inv);
    o[r >> 4][(r >> 2) & 3] = lo | (hi << 16);
  }
  return byte;
}

// Along columns of the staged tile into q_c [C, pitch], s_c [C, pitch/32].
__device__ __forceinline__ void tile_columns(const uint16_t* tile, int64_t r0, int c0, int64_t pitch, uint8_t* q_c,
                                             uint8_t* s_c) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int task = t + 256 * i, c = task / 4, blk = task % 4;
    u32x4_t o[2];
    const uint32_t byte = encode32(tile + (32 * blk) * kColPitch + c, kColPitch, o);
    const int64_t cc = c0 + c;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(q_c + cc * pitch + r0 + 32 * blk);
    __builtin_nontemporal_store(o[0], dst);
    __builtin_nontemporal_store(o[1], dst + 1);
    const uint32_t four = gather4(byte, blk);
    if (blk == 0) *reinterpret_cast<uint32_t*>(s_c + cc * (pitch / 32) + r0 / 32) = four;
  }
}

// x: `batch` matrices [R, C] bf16 (batch stride R*C).  Output per matrix:
// q [C, pitch] E4M3 (row c holds column c of x, quantised in blocks of 32
// consecutive rows), s [C, pitch/32].  Row tiles at or past offsets[E] (when
// given) are skipped: the rows encoded must come in whole tiles of 128
// (row_align 128 for dispatched rows; R % 128 == 0 for weights).
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
  // load: thread t moves the 16-byte chunk t % 16 of rows t / 16 + 16 i
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int lr = t / 16 + 16 * i, ch = t % 16;
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(xm + (r0 + lr) * C + c0 + ch * 8));
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + lr * kColPitch + ch * 8);
#pragma unroll
    for (int d = 0; d < 4; ++d) dst[d] = v[d];
  }
  __syncthreads();
  tile_columns(tile, r0, c0, pitch, q + static_cast<int64_t>(mat) * C * pitch,
               s + static_cast<int64_t>(mat) * C * (pitch / 32));
}

// ------------------------------------------------- both axes in one pass
// Both MXFP8 forms of the staged tile (columns [c0, c0 + 128) of an [R, C]
// matrix): along columns, and along rows (four consecutive threads: one
// row's four 32-column blocks, one 128-byte line and one 4-byte scale store).
__device__ __forceinline__ void tile_both(const uint16_t* tile, int64_t r0, int c0, int C, int64_t pitch,
                                          uint8_t* q_r, uint8_t* s_r, uint8_t* q_c, uint8_t* s_c) {
  tile_columns(tile, r0, c0, pitch, q_c, s_c);
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int task = t + 256 * i, lr = task / 4, blk = task % 4;
    u32x4_t o[2];
    const uint32_t byte = encode32(tile + lr * kColPitch + 32 * blk, 1, o);
    const int64_t r = r0 + lr;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(q_r + r * C + c0 + 32 * blk);
    __builtin_nontemporal_store(o[0], dst);
    __builtin_nontemporal_store(o[1], dst + 1);
    const uint32_t four = gather4(byte, blk);
    if (blk == 0) *reinterpret_cast<uint32_t*>(s_r + r * (C / 32) + c0 / 32) = four;
  }
}

__device__ __forceinline__ void tile_store(uint16_t* tile, int lr, int ch, const u32x4_t& v) {
  uint32_t* dst = reinterpret_cast<uint32_t*>(tile + lr * kColPitch + ch * 8);
#pragma unroll
  for (int d = 0; d < 4; ++d) dst[d] = v[d];
}

// The two MXFP8 forms of one [R, C] bf16 matrix from a single read: along
// rows (q_r [R, C], s_r [R, C/32], the dgrad operand) and along columns
// (q_c [C, pitch], s_c [C, pitch/32], the wgrad operand).  SWIGLU: the
// matrix is dH [R, 2I] = [dgate | dup], computed in the load from dA [R, I]
// and the saved h [R, 2I] (the SwiGLU backward's formula and FP32
// arithmetic, bf16-rounded as the BF16 path stores dH), so dH itself is never
// written; a workgroup takes the gate-half tile at c0 and the up-half tile at
// I + c0, which read the same dA and h columns, from one read (two LDS tiles,
// 66.5 KB: two workgroups per CU).  Row tiles at
// or past offsets[E] (when given; else R, a multiple of 128) are skipped.
constexpr int kTileElems = kColTileRows * kColPitch;
template <bool SWIGLU>
constexpr uint32_t dual_lds_bytes() { return (SWIGLU ? 2 : 1) * kTileElems * sizeof(uint16_t); }

template <bool SWIGLU>
__global__ void __launch_bounds__(kQ8Threads)
q8_dual_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ h, int64_t R, int C, int I,
               const int32_t* __restrict__ offsets, int E, int64_t pitch, uint8_t* __restrict__ q_r,
               uint8_t* __restrict__ s_r, uint8_t* __restrict__ q_c, uint8_t* __restrict__ s_c) {
  extern __shared__ __attribute__((aligned(16))) uint16_t tile[];   // SWIGLU: gate tile, then up tile
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kColTileRows;
  const int c0 = blockIdx.y * kColTileCols;
  if (r0 >= (offsets != nullptr ? min<int64_t>(R, offsets[E]) : R)) return;
  const int t = threadIdx.x;
  if constexpr (!SWIGLU) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int lr = t / 16 + 16 * i, ch = t % 16;
      tile_store(tile, lr, ch,
                 __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + (r0 + lr) * C + c0 + ch * 8)));
    }
    __syncthreads();
    tile_both(tile, r0, c0, C, pitch, q_r, s_r, q_c, s_c);
  } else {
    uint16_t* tile_u = tile + kTileElems;
#pragma unroll 2
    for (int i = 0; i < 8; ++i) {
      const int lr = t / 16 + 16 * i, ch = t % 16;
      const int64_t r = r0 + lr;
      const int i0 = c0 + ch * 8;   // feature index in [0, I)
      const u32x4_t da = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + r * I + i0));
      const u32x4_t hg = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(h + r * (2 * I) + i0));
      const u32x4_t hu = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(h + r * (2 * I) + I + i0));
      u32x4_t vg, vu;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        float g2[2], u2[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const float a = bf16_to_f32(static_cast<uint16_t>(da[d] >> (16 * p)));
          const float gt = bf16_to_f32(static_cast<uint16_t>(hg[d] >> (16 * p)));
          const float up = bf16_to_f32(static_cast<uint16_t>(hu[d] >> (16 * p)));
          const float sg = sigmoid_fast(gt);
          g2[p] = a * up * sg * (1.0f + gt * (1.0f - sg));
          u2[p] = a * gt * sg;
        }
        vg[d] = pack_bf16x2(g2[0], g2[1]);
        vu[d] = pack_bf16x2(u2[0], u2[1]);
      }
      tile_store(tile, lr, ch, vg);
      tile_store(tile_u, lr, ch, vu);
    }
    __syncthreads();
    tile_both(tile, r0, c0, C, pitch, q_r, s_r, q_c, s_c);
    tile_both(tile_u, r0, I + c0, C, pitch, q_r, s_r, q_c, s_c);
  }
}

unsigned grid_for(int64_t work) {
  const int64_t blocks = (work + kQ8Threads - 1) / kQ8Threads;
  return static_cast<unsigned>(std::min<int64_t>(std::max<int64_t>(blocks, 1),
                                                 static_cast<int64_t>(device_cu_count()) * 16));
}

}  // namespace

bool launch_q8_cols(const uint16_t* x, int64_t R, int C, int batch, const int32_t* offsets, int E,
                    int64_t pitch, uint8_t* q, uint8_t* s, const char* name, hipStream_t st) {
  if (R == 0 || batch == 0) return true;
  if (C % kColTileCols || pitch % 128) return false;
  if (offsets == nullptr && R % kColTileRows) return false;
  const dim3 grid(static_cast<unsigned>((R + kColTileRows - 1) / kColTileRows),
                  static_cast<unsigned>(C / kColTileCols), static_cast<unsigned>(batch));
  launch_kernel(name, q8_cols_kernel, grid, dim3(kQ8Threads), 0, st, x, R, C, offsets, E, pitch, q, s);
  return launch_ok(name);
}

bool launch_q8_dual(const uint16_t* x, const uint16_t* h, int64_t R, int C, int I, const int32_t* offsets, int E,
                    int64_t pitch, uint8_t* q_r, uint8_t* s_r, uint8_t* q_c, uint8_t* s_c, const char* name,
                    hipStream_t st) {
  if (R == 0) return true;
  if (C % kColTileCols || pitch % 128 || (h != nullptr && (C != 2 * I || I % kColTileCols))) return false;   // C % 128
  if (offsets == nullptr && R % kColTileRows) return false;
  // SWIGLU: one workgroup per gate-half tile (it also writes the up-half tile)
  const dim3 grid(static_cast<unsigned>((R + kColTileRows - 1) / kColTileRows),
                  static_cast<unsigned>((h == nullptr ? C : I) / kColTileCols));
  if (h == nullptr) {
    launch_kernel(name, q8_dual_kernel<false>, grid, dim3(kQ8Threads), dual_lds_bytes<false>(), st, x, h, R, C, I,
                  offsets, E, pitch, q_r, s_r, q_c, s_c);
  } else {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&q8_dual_kernel<true>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       dual_lds_bytes<true>());
    if (attr != hipSuccess) return launch_ok(name) && false;
    launch_kernel(name, q8_dual_kernel<true>, grid, dim3(kQ8Threads), dual_lds_bytes<true>(), st, x, h, R, C, I,
                  offsets, E, pitch, q_r, s_r, q_c, s_c);
  }
  return launch_ok(name);
}

}  // namespace w4a4
