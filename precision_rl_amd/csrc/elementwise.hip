// HBM-bound gathers of the expert path (gfx950):
//   unpermute:     y[t]  = bf16( sum_j p[t,j] * o[row_map[t,j]] )
//   gather-sum:    dX[t] = bf16( sum_j dXp[row_map[t,j]] )
//   scatter:       dO[row_map[t,j]] = bf16( p[t,j] * dY[t] );  xp[row_map[t,j]] = x[t]
// The router coefficients enter in the unpermute, on the bf16 expert outputs,
// summed in FP32 in ascending j (a reading of the pages, which name the
// router-coefficient position as a choice the execution specification must fix:
// AI summary, "Methodology in Plain English").  All loads and stores are 16 B
// and non-temporal (every row is touched once).

#include "device_common.h"
#include "internal.h"

namespace w4a4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void acc_bf16x8(float (&acc)[8], u32x4_t v, float w) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    acc[2 * d] += w * bf16_to_f32(static_cast<uint16_t>(v[d] & 0xFFFFu));
    acc[2 * d + 1] += w * bf16_to_f32(static_cast<uint16_t>(v[d] >> 16));
  }
}

// A workgroup per token (workgroups stride over the tokens when the grid is
// smaller than T); thread c handles 16 B chunks c, c+256, ...
__global__ void __launch_bounds__(kThreads)
gather_sum_kernel(int64_t T, int H, int k, const uint16_t* __restrict__ src, const int32_t* __restrict__ row_map,
                  const float* __restrict__ w, uint16_t* __restrict__ out) {
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
  const int chunks = H / 8;
  int32_t rows[16];
  float ws[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k) {
      rows[j] = row_map[t * k + j];
      ws[j] = w ? w[t * k + j] : 1.0f;
    }
  }
  for (int c = threadIdx.x; c < chunks; c += kThreads) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < k) {
        const u32x4_t v = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(src + static_cast<int64_t>(rows[j]) * H + c * 8));
        acc_bf16x8(acc, v, ws[j]);
      }
    }
    u32x4_t o;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(acc[2 * d], acc[2 * d + 1]);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(out + t * H + c * 8));
  }
  }
}

// One workgroup per token t.  DY: dY[t] is read once and written, scaled by
// the router weight, to each of the token's k dispatched rows of dO.  X: x[t]
// is read once and copied to the token's k rows of xp.  Token order keeps the
// reads sequential; the writes are whole rows.  The two run as separate
// kernels: dO is needed first, xp only by the last GEMM.
template <bool DY>
__global__ void __launch_bounds__(kThreads)
scatter_kernel(int64_t T, int H, int k, const uint16_t* __restrict__ src, const int32_t* __restrict__ row_map,
               const float* __restrict__ w, uint16_t* __restrict__ dst) {
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
  int32_t rows[16];
  float ps[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k) {
      rows[j] = row_map[t * k + j];
      if constexpr (DY) ps[j] = w[t * k + j];
    }
  }
  for (int c = threadIdx.x; c < H / 8; c += kThreads) {
    const u32x4_t g = *reinterpret_cast<const u32x4_t*>(src + t * H + c * 8);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < k) {
        u32x4_t o = g;
        if constexpr (DY) {
#pragma unroll
          for (int d = 0; d < 4; ++d)
            o[d] = pack_bf16x2(ps[j] * bf16_to_f32(static_cast<uint16_t>(g[d] & 0xFFFFu)),
                               ps[j] * bf16_to_f32(static_cast<uint16_t>(g[d] >> 16)));
        }
        const int64_t r = rows[j];
        // non-temporal: the next kernel reads dO / xp from HBM anyway, and
        // dirty lines left in L2 cost the FC2 dgrad more than they save here
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(dst + r * H + c * 8));
      }
    }
  }
  }
}

// Pad rows (src_row < 0, rows [0, offsets[E])) of a [rows, H] bf16 buffer: zeros.
__global__ void __launch_bounds__(kThreads)
zero_pad_rows_kernel(int H, const int32_t* __restrict__ src_row, const int32_t* __restrict__ offsets,
                     int E, uint16_t* __restrict__ dst) {
  const int64_t r = blockIdx.x;
  if (r >= offsets[E] || src_row[r] >= 0) return;
  for (int c = threadIdx.x; c < H / 8; c += kThreads)
    *reinterpret_cast<u32x4_t*>(dst + r * H + c * 8) = u32x4_t{0u, 0u, 0u, 0u};
}

}  // namespace

bool launch_unpermute(int64_t T, int H, int k, const uint16_t* o, const int32_t* row_map,
                      const float* topk_w, uint16_t* y, hipStream_t s) {
  if (T == 0) return true;
  launch_kernel("unpermute", gather_sum_kernel, dim3(static_cast<unsigned>(T)), dim3(kThreads), 0, s, T, H, k, o,
                row_map, topk_w, y);
  return launch_ok("unpermute");
}

bool launch_gather_sum(int64_t T, int H, int k, const uint16_t* dXp, const int32_t* row_map,
                       uint16_t* dx, hipStream_t s) {
  if (T == 0) return true;
  launch_kernel("dx_gather_sum", gather_sum_kernel, dim3(static_cast<unsigned>(T)), dim3(kThreads), 0, s, T, H, k,
                dXp, row_map, static_cast<const float*>(nullptr), dx);
  return launch_ok("dx_gather_sum");
}

bool launch_scatter_dy(int64_t T, int H, int k, const uint16_t* dy, const int32_t* row_map,
                       const float* topk_w, uint16_t* dO, hipStream_t s) {
  if (T == 0) return true;
  launch_kernel("dy_scatter", scatter_kernel<true>, dim3(static_cast<unsigned>(T)), dim3(kThreads), 0, s, T, H, k,
                dy, row_map, topk_w, dO);
  return launch_ok("dy_scatter");
}

bool launch_scatter_x(int64_t T, int H, int k, const uint16_t* x, const int32_t* row_map, uint16_t* xp,
                      hipStream_t s) {
  if (T == 0) return true;
  launch_kernel("x_scatter", scatter_kernel<false>, dim3(static_cast<unsigned>(T)), dim3(kThreads), 0, s, T, H, k,
                x, row_map, static_cast<const float*>(nullptr), xp);
  return launch_ok("x_scatter");
}

bool launch_zero_pad_rows(int64_t rows_alloc, int H, const int32_t* src_row, const int32_t* offsets,
                          int E, uint16_t* dst, hipStream_t s) {
  if (rows_alloc == 0) return true;
  launch_kernel("zero_pad_rows", zero_pad_rows_kernel, dim3(static_cast<unsigned>(rows_alloc)), dim3(kThreads), 0,
                s, H, src_row, offsets, E, dst);
  return launch_ok("zero_pad_rows");
}

}  // namespace w4a4
