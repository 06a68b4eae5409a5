// HBM-bound gathers of the expert path (gfx950):
//   unpermute:     y[t]  = bf16( sum_j p[t,j] * o[row_map[t,j]] )
//   gather-sum:    dX[t] = bf16( sum_j dXp[row_map[t,j]] )
//   gather-scale:  dO[r] = bf16( p[t,j] * dY[t] ),  t = src_row[r], pad rows 0
// The router coefficients enter in the unpermute, on the bf16 expert outputs,
// summed in FP32 in ascending j (a reading of the pages, which name the
// router-coefficient position as a choice the execution specification must fix:
// AI summary, "Methodology in Plain English").  All loads and stores are 16 B.

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

// One workgroup per token; thread c handles 16 B chunks c, c+256, ...
__global__ void __launch_bounds__(kThreads)
gather_sum_kernel(int H, int k, const uint16_t* __restrict__ src, const int32_t* __restrict__ row_map,
                  const float* __restrict__ w, uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
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
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + static_cast<int64_t>(rows[j]) * H + c * 8);
        acc_bf16x8(acc, v, ws[j]);
      }
    }
    u32x4_t o;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(acc[2 * d], acc[2 * d + 1]);
    *reinterpret_cast<u32x4_t*>(out + t * H + c * 8) = o;
  }
}

// One wave per dispatched row.
__global__ void __launch_bounds__(kThreads)
gather_scale_kernel(int64_t rows_alloc, int H, int k, const uint16_t* __restrict__ dy,
                    const int32_t* __restrict__ row_map, const int32_t* __restrict__ src_row,
                    const float* __restrict__ w, const int32_t* __restrict__ offsets, int E,
                    uint16_t* __restrict__ dO) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + (threadIdx.x >> 6);
  if (r >= rows_alloc || r >= offsets[E]) return;
  const int32_t t = src_row[r];
  float p = 0.0f;
  if (t >= 0) {
    for (int j = 0; j < k; ++j)
      if (row_map[static_cast<int64_t>(t) * k + j] == r) p = w[static_cast<int64_t>(t) * k + j];
  }
  const int chunks = H / 8;
  for (int c = lane; c < chunks; c += kWave) {
    u32x4_t o = {0u, 0u, 0u, 0u};
    if (t >= 0) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(dy + static_cast<int64_t>(t) * H + c * 8);
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o[d] = pack_bf16x2(p * bf16_to_f32(static_cast<uint16_t>(v[d] & 0xFFFFu)),
                           p * bf16_to_f32(static_cast<uint16_t>(v[d] >> 16)));
    }
    *reinterpret_cast<u32x4_t*>(dO + r * H + c * 8) = o;
  }
}

// One workgroup per dispatched row: xp[r] = x[src_row[r]], zeros for pad rows.
__global__ void __launch_bounds__(kThreads)
gather_rows_kernel(int H, const uint16_t* __restrict__ x, const int32_t* __restrict__ src_row,
                   const int32_t* __restrict__ offsets, int E, uint16_t* __restrict__ xp) {
  const int64_t r = blockIdx.x;
  if (r >= offsets[E]) return;
  const int32_t t = src_row[r];
  for (int c = threadIdx.x; c < H / 8; c += kThreads) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (t >= 0) v = *reinterpret_cast<const u32x4_t*>(x + static_cast<int64_t>(t) * H + c * 8);
    *reinterpret_cast<u32x4_t*>(xp + r * H + c * 8) = v;
  }
}

}  // namespace

bool launch_gather_rows(int64_t rows_alloc, int H, const uint16_t* x, const int32_t* src_row,
                        const int32_t* offsets, int E, uint16_t* xp, hipStream_t s) {
  if (rows_alloc == 0) return true;
  {
    ProfScope p("x_gather_rows", s);
    gather_rows_kernel<<<dim3(static_cast<unsigned>(rows_alloc)), dim3(kThreads), 0, s>>>(
        H, x, src_row, offsets, E, xp);
  }
  return launch_ok("x_gather_rows");
}

bool launch_unpermute(int64_t T, int H, int k, const uint16_t* o, const int32_t* row_map,
                      const float* topk_w, uint16_t* y, hipStream_t s) {
  if (T == 0) return true;
  {
    ProfScope p("unpermute", s);
    gather_sum_kernel<<<dim3(static_cast<unsigned>(T)), dim3(kThreads), 0, s>>>(H, k, o, row_map,
                                                                                topk_w, y);
  }
  return launch_ok("unpermute");
}

bool launch_gather_sum(int64_t T, int H, int k, const uint16_t* dXp, const int32_t* row_map,
                       uint16_t* dx, hipStream_t s) {
  if (T == 0) return true;
  {
    ProfScope p("dx_gather_sum", s);
    gather_sum_kernel<<<dim3(static_cast<unsigned>(T)), dim3(kThreads), 0, s>>>(H, k, dXp, row_map,
                                                                                nullptr, dx);
  }
  return launch_ok("dx_gather_sum");
}

bool launch_gather_scale(int64_t rows_alloc, int H, int k, const uint16_t* dy,
                         const int32_t* row_map, const int32_t* src_row, const float* topk_w,
                         const int32_t* offsets, int E, uint16_t* dO, hipStream_t s) {
  const int64_t blocks = (rows_alloc + kThreads / kWave - 1) / (kThreads / kWave);
  if (blocks == 0) return true;
  {
    ProfScope p("do_gather_scale", s);
    gather_scale_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s>>>(
        rows_alloc, H, k, dy, row_map, src_row, topk_w, offsets, E, dO);
  }
  return launch_ok("do_gather_scale");
}

}  // namespace w4a4
