// Routing and NVFP4 encoding kernels of the W4A4 MoE expert path on gfx950:
//   route_count / route_scan  -- stable counting sort of (token, slot) entries
//                                into expert-contiguous rows, offsets on device;
//   quantize_scatter          -- per-token amax, two-level NVFP4 encoding and
//                                the scatter of the encoded row to its k rows;
//   requant                   -- the same encoder on the FC2 input rows.
//
// Encoding (miniTE Technical Report, section 5.1, block-scale equation; rainbus
// review of the miniTE paper, method step 4):
//   g   = RN_f32(max|x| / (6*448))
//   d_b = Q_E4M3(amax(block b) / (6 g))          one E4M3 scale per 16 elements
//   c   = Q_E2M1(x / (g d_b))                    round to nearest, ties to even
// Every Q(.) rounds the exact quotient.  The E4M3 quotient is formed as one
// correctly rounded float64 division, which keeps the side of every rounding
// midpoint (operands have <= 8 and <= 26 significant bits).  For the E2M1 codes
// the seven midpoints mu * g * d_b (mu in .25 .75 1.25 1.75 2.5 3.5 5) are
// exact float64 products; each is turned into the smallest bf16 value that a
// bf16 |x| must reach to cross it (ties resolved towards the even code), so
// the per-element work is seven integer compares on the bf16 bit pattern.

#include "device_common.h"
#include "internal.h"

namespace w4a4 {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWavesPerBlock * kWave;

// ------------------------------------------------------------------ E4M3 RNE
// Round q >= 0 to the nearest E4M3FN value (ties to even, subnormals kept,
// saturating at 448).  Returns the byte; *val receives the value.
__device__ __forceinline__ uint32_t e4m3_rne(double q, double* val) {
  if (!(q > 0.0)) {
    *val = 0.0;
    return 0u;
  }
  if (q >= 448.0) {
    *val = 448.0;
    return 0x7Eu;
  }
  int ex;
  frexp(q, &ex);
  int e = ex - 1;                    // floor(log2 q)
  if (e < -6) e = -6;                // subnormal binade spacing 2^-9
  double r = rint(ldexp(q, 3 - e));  // exact scaling, round half to even
  double v = ldexp(r, e - 3);
  *val = v;
  if (v == 0.0) return 0u;
  frexp(v, &ex);
  int e2 = ex - 1;
  if (e2 < -6) return static_cast<uint32_t>(ldexp(v, 9));                  // m * 2^-9
  return static_cast<uint32_t>(((e2 + 7) << 3) | (static_cast<int>(ldexp(v, 3 - e2)) - 8));
}

__device__ __forceinline__ float next_up(float f) {  // f >= 0, finite
  return __uint_as_float(__float_as_uint(f) + 1u);
}

// Smallest bf16 bit pattern b (as a magnitude) with value(b) >= t, resp. > t.
__device__ __forceinline__ uint32_t bf16_ceil_bits(float f) {
  return (__float_as_uint(f) + 0xFFFFu) >> 16;
}
__device__ __forceinline__ uint32_t thr_ge(double t) {
  float f = static_cast<float>(t);
  if (static_cast<double>(f) < t) f = next_up(f);
  return bf16_ceil_bits(f);
}
__device__ __forceinline__ uint32_t thr_gt(double t) {
  float f = static_cast<float>(t);
  if (static_cast<double>(f) <= t) f = next_up(f);
  return bf16_ceil_bits(f);
}

struct BlockThresholds {
  uint32_t t[7];
};

// Crossing thresholds of the seven E2M1 midpoints for one block.  Midpoint j
// (1-based) separates magnitude codes j-1 and j; an exact tie goes to the even
// code, i.e. down for odd j and up for even j.
__device__ __forceinline__ BlockThresholds make_thresholds(double gd) {
  BlockThresholds th;
  if (gd > 0.0) {
    th.t[0] = thr_gt(0.25 * gd);
    th.t[1] = thr_ge(0.75 * gd);
    th.t[2] = thr_gt(1.25 * gd);
    th.t[3] = thr_ge(1.75 * gd);
    th.t[4] = thr_gt(2.5 * gd);
    th.t[5] = thr_ge(3.5 * gd);
    th.t[6] = thr_gt(5.0 * gd);
  } else {
#pragma unroll
    for (int j = 0; j < 7; ++j) th.t[j] = 0xFFFFu;  // never crossed: zero codes
  }
  return th;
}

__device__ __forceinline__ uint32_t e2m1_code(uint32_t xbits16, const BlockThresholds& th) {
  uint32_t mag = xbits16 & 0x7FFFu;
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) c += mag >= th.t[j] ? 1u : 0u;
  return c | ((xbits16 >> 12) & 8u);
}

// One block of 16 bf16 values held as 8 packed dwords.
struct Block16 {
  uint32_t w[8];
};

__device__ __forceinline__ uint32_t block_amax_bits(const Block16& b) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t lo = b.w[i] & 0x7FFFu, hi = (b.w[i] >> 16) & 0x7FFFu;
    m = lo > m ? lo : m;
    m = hi > m ? hi : m;
  }
  return m;
}

// Encodes one block: returns the two code dwords; *scale receives the byte.
__device__ __forceinline__ u32x2_t encode_block(const Block16& b, uint32_t amax16, double g,
                                                uint32_t* scale) {
  double ab = static_cast<double>(bf16_to_f32(static_cast<uint16_t>(amax16)));
  double dval = 0.0;
  uint32_t dbits = 0;
  if (g > 0.0) dbits = e4m3_rne(ab / (6.0 * g), &dval);
  *scale = dbits;
  BlockThresholds th = make_thresholds(g * dval);
  u32x2_t out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w = b.w[h * 4 + i];
      v |= e2m1_code(w & 0xFFFFu, th) << (8 * i);
      v |= e2m1_code(w >> 16, th) << (8 * i + 4);
    }
    out[h] = v;
  }
  return out;
}

__device__ __forceinline__ Block16 load_block(const uint16_t* p) {
  const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
  u32x4_t a = q[0], b = q[1];
  Block16 r;
  r.w[0] = a[0]; r.w[1] = a[1]; r.w[2] = a[2]; r.w[3] = a[3];
  r.w[4] = b[0]; r.w[5] = b[1]; r.w[6] = b[2]; r.w[7] = b[3];
  return r;
}

// g = RN_f32(a / 2688) from the bf16 magnitude bits of the row amax.
__device__ __forceinline__ float outer_scale(uint32_t amax16) {
  double a = static_cast<double>(bf16_to_f32(static_cast<uint16_t>(amax16)));
  return static_cast<float>(a / 2688.0);
}

// ------------------------------------------------------------------ routing
// One workgroup per chunk of kRouteChunk tokens: a bit mask per expert marks
// the chunk's tokens routed to it; a token's rank inside the chunk is the
// popcount of the mask below it (stable: ascending token order).  The local
// rank is parked in row_map and the per-chunk counts in `counts`.
__global__ void __launch_bounds__(kRouteChunk)
route_count_kernel(const int32_t* __restrict__ topk_idx, int64_t T, int k, int E,
                   int32_t* __restrict__ row_map, int32_t* __restrict__ counts) {
  extern __shared__ uint32_t masks[];  // [E][kRouteChunk / 32]
  constexpr int W = kRouteChunk / 32;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  for (int i = tid; i < E * W; i += kRouteChunk) masks[i] = 0u;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(c) * kRouteChunk + tid;
  const bool live = t < T;
  if (live) {
    for (int j = 0; j < k; ++j) {
      int e = topk_idx[t * k + j];
      atomicOr(&masks[e * W + tid / 32], 1u << (tid % 32));
    }
  }
  __syncthreads();
  if (live) {
    for (int j = 0; j < k; ++j) {
      int e = topk_idx[t * k + j];
      const uint32_t* m = masks + e * W;
      int rank = __popc(m[tid / 32] & ((1u << (tid % 32)) - 1u));
      for (int w = 0; w < tid / 32; ++w) rank += __popc(m[w]);
      row_map[t * k + j] = rank;
    }
  }
  for (int e = tid; e < E; e += kRouteChunk) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) n += __popc(masks[e * W + w]);
    counts[static_cast<int64_t>(c) * E + e] = n;
  }
}

// Single workgroup: per expert, exclusive prefix of the chunk counts (in
// place, giving each chunk's first rank), the expert totals, and the padded
// expert offsets.
constexpr int kScanThreads = 1024;
constexpr int kScanTile = 8192;  // ints of the count matrix staged per pass

__global__ void __launch_bounds__(kScanThreads)
route_scan_kernel(int32_t* __restrict__ counts, int n_chunks, int E, int row_align,
                  int32_t* __restrict__ offsets, int32_t* __restrict__ expert_count) {
  __shared__ int32_t buf[kScanTile];
  __shared__ int32_t carry[1024];
  __shared__ int32_t scan[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kScanThreads) carry[e] = 0;
  const int rows_per_tile = kScanTile / E > 0 ? kScanTile / E : 1;
  __syncthreads();
  for (int c0 = 0; c0 < n_chunks; c0 += rows_per_tile) {
    const int rows = min(rows_per_tile, n_chunks - c0);
    const int64_t base = static_cast<int64_t>(c0) * E;
    for (int i = tid; i < rows * E; i += kScanThreads) buf[i] = counts[base + i];
    __syncthreads();
    for (int e = tid; e < E; e += kScanThreads) {
      int run = carry[e];
      for (int r = 0; r < rows; ++r) {
        int v = buf[r * E + e];
        buf[r * E + e] = run;
        run += v;
      }
      carry[e] = run;
    }
    __syncthreads();
    for (int i = tid; i < rows * E; i += kScanThreads) counts[base + i] = buf[i];
    __syncthreads();
  }
  // Exclusive scan of the padded group sizes over experts (E <= 1024).
  int padded = 0;
  if (tid < E) {
    int n = carry[tid];
    expert_count[tid] = n;
    padded = (n + row_align - 1) / row_align * row_align;
  }
  scan[tid] = padded;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  if (tid < E) offsets[tid + 1] = scan[tid];
  if (tid == 0) offsets[0] = 0;
}

// ---------------------------------------------------------- quantize + scatter
// One wave per token (identity mode: one wave per row).  MAXB = blocks of 16
// per lane, K <= 1024 * MAXB.
template <int MAXB>
__global__ void __launch_bounds__(kThreads)
quantize_scatter_kernel(const uint16_t* __restrict__ x, int64_t T, int K,
                        const int32_t* __restrict__ topk_idx, int k, int E, int row_align,
                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                        float* __restrict__ outer, int32_t* __restrict__ offsets,
                        int32_t* __restrict__ row_map, int32_t* __restrict__ src_row,
                        const int32_t* __restrict__ chunk_base,
                        const int32_t* __restrict__ expert_count, int64_t token_blocks) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int nb = K / 16;
  const int64_t K2 = K / 2, K16 = K / 16;

  if (static_cast<int64_t>(blockIdx.x) >= token_blocks) {
    // Pad-row writer: one wave per expert.
    if (topk_idx == nullptr) return;
    const int e = static_cast<int>((blockIdx.x - token_blocks) * kWavesPerBlock + wave);
    if (e >= E) return;
    const int64_t r0 = offsets[e] + expert_count[e], r1 = offsets[e + 1];
    for (int64_t r = r0; r < r1; ++r) {
      for (int b = lane; b < nb; b += kWave) {
        *reinterpret_cast<u32x2_t*>(codes + r * K2 + b * 8) = u32x2_t{0u, 0u};
        scales[r * K16 + b] = 0;
      }
      if (lane == 0) {
        outer[r] = 0.0f;
        src_row[r] = -1;
      }
    }
    return;
  }

  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (t >= T) return;

  Block16 blk[MAXB];
  uint32_t bmax[MAXB];
  uint32_t amax = 0;
  const uint16_t* xr = x + t * K;
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int b = lane + i * kWave;
    if (b < nb) {
      blk[i] = load_block(xr + b * 16);
      bmax[i] = block_amax_bits(blk[i]);
      amax = bmax[i] > amax ? bmax[i] : amax;
    }
  }
  amax = wave_max_u32(amax);
  const float g = outer_scale(amax);

  // Destination rows of this token.
  int64_t rows[8];
  int nrows;
  if (topk_idx == nullptr) {
    rows[0] = t;
    nrows = 1;
    if (lane == 0) {
      row_map[t] = static_cast<int32_t>(t);
      src_row[t] = static_cast<int32_t>(t);
      if (t == 0) {
        offsets[0] = 0;
        offsets[1] = static_cast<int32_t>(T);
      }
    }
  } else {
    const int64_t c = t / kRouteChunk;
    int32_t myrow = 0;
    if (lane < k) {
      const int e = topk_idx[t * k + lane];
      myrow = offsets[e] + chunk_base[c * E + e] + row_map[t * k + lane];
      row_map[t * k + lane] = myrow;
      src_row[myrow] = static_cast<int32_t>(t);
    }
    nrows = k;
#pragma unroll
    for (int j = 0; j < 8; ++j) rows[j] = __shfl(myrow, j, kWave);
  }

#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int b = lane + i * kWave;
    if (b < nb) {
      uint32_t sc;
      u32x2_t cw = encode_block(blk[i], bmax[i], static_cast<double>(g), &sc);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < nrows) {
          *reinterpret_cast<u32x2_t*>(codes + rows[j] * K2 + b * 8) = cw;
          scales[rows[j] * K16 + b] = static_cast<uint8_t>(sc);
        }
      }
    }
  }
  if (lane < nrows) {
    int64_t r = rows[0];
#pragma unroll
    for (int j = 1; j < 8; ++j)
      if (lane == j) r = rows[j];
    outer[r] = g;
  }
}

// Requantise rows [0, offsets[E]) of a [rows_alloc, K] bf16 matrix in place.
template <int MAXB>
__global__ void __launch_bounds__(kThreads)
requant_kernel(const uint16_t* __restrict__ a, int64_t rows_alloc, int K,
               const int32_t* __restrict__ offsets, int E, uint8_t* __restrict__ codes,
               uint8_t* __restrict__ scales, float* __restrict__ outer) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (r >= rows_alloc || r >= offsets[E]) return;
  const int nb = K / 16;
  Block16 blk[MAXB];
  uint32_t bmax[MAXB];
  uint32_t amax = 0;
  const uint16_t* ar = a + r * K;
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int b = lane + i * kWave;
    if (b < nb) {
      blk[i] = load_block(ar + b * 16);
      bmax[i] = block_amax_bits(blk[i]);
      amax = bmax[i] > amax ? bmax[i] : amax;
    }
  }
  amax = wave_max_u32(amax);
  const float g = outer_scale(amax);
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int b = lane + i * kWave;
    if (b < nb) {
      uint32_t sc;
      u32x2_t cw = encode_block(blk[i], bmax[i], static_cast<double>(g), &sc);
      *reinterpret_cast<u32x2_t*>(codes + r * (K / 2) + b * 8) = cw;
      scales[r * (K / 16) + b] = static_cast<uint8_t>(sc);
    }
  }
  if (lane == 0) outer[r] = g;
}

__global__ void zero_offsets_kernel(int32_t* offsets, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) offsets[i] = 0;
}

template <typename F>
bool dispatch_maxb(int K, F&& f) {
  if (K <= 1024) return f(std::integral_constant<int, 1>{});
  if (K <= 2048) return f(std::integral_constant<int, 2>{});
  if (K <= 4096) return f(std::integral_constant<int, 4>{});
  if (K <= 8192) return f(std::integral_constant<int, 8>{});
  return false;
}

}  // namespace

size_t route_workspace_bytes(int64_t T, int E) {
  const int64_t n_chunks = (T + kRouteChunk - 1) / kRouteChunk;
  return static_cast<size_t>(n_chunks * E + E) * sizeof(int32_t);
}

bool launch_quantize_permute(const uint16_t* x, int64_t T, int K, const int32_t* topk_idx,
                             int k, int E, int row_align, uint8_t* codes, uint8_t* scales,
                             float* outer, int32_t* offsets, int32_t* row_map, int32_t* src_row,
                             void* ws, hipStream_t s) {
  const int64_t n_chunks = (T + kRouteChunk - 1) / kRouteChunk;
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* expert_count = counts + n_chunks * E;
  if (T == 0) {  // nothing routed: every group is empty
    {
      ProfScope p("route_scan", s);
      zero_offsets_kernel<<<1, 256, 0, s>>>(offsets, E + 1);
    }
    return launch_ok("zero_offsets");
  }
  if (topk_idx != nullptr) {
    {
      ProfScope p("route_count", s);
      size_t lds = static_cast<size_t>(E) * (kRouteChunk / 32) * sizeof(uint32_t);
      route_count_kernel<<<dim3(static_cast<unsigned>(n_chunks)), dim3(kRouteChunk), lds, s>>>(
          topk_idx, T, k, E, row_map, counts);
    }
    if (!launch_ok("route_count")) return false;
  }
  if (topk_idx != nullptr) {
    {
      ProfScope p("route_scan", s);
      route_scan_kernel<<<1, kScanThreads, 0, s>>>(counts, static_cast<int>(n_chunks), E, row_align,
                                                    offsets, expert_count);
    }
    if (!launch_ok("route_scan")) return false;
  }
  const int64_t token_blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t pad_blocks = (topk_idx != nullptr && row_align > 1)
                                 ? (E + kWavesPerBlock - 1) / kWavesPerBlock : 0;
  const int64_t blocks = token_blocks + pad_blocks;
  if (blocks == 0) return true;
  return dispatch_maxb(K, [&](auto mb) {
    {
      ProfScope p("quantize_scatter", s);
      quantize_scatter_kernel<decltype(mb)::value>
          <<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s>>>(
              x, T, K, topk_idx, k, E, row_align, codes, scales, outer, offsets, row_map,
              src_row, counts, expert_count, token_blocks);
    }
    return launch_ok("quantize_scatter");
  });
}

bool launch_requant(const uint16_t* a, int64_t rows_alloc, int K, const int32_t* offsets, int E,
                    const int32_t* /*src_row*/, uint8_t* codes, uint8_t* scales, float* outer,
                    hipStream_t s) {
  const int64_t blocks = (rows_alloc + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return true;
  return dispatch_maxb(K, [&](auto mb) {
    {
      ProfScope p("requant", s);
      requant_kernel<decltype(mb)::value><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s>>>(
          a, rows_alloc, K, offsets, E, codes, scales, outer);
    }
    return launch_ok("requant");
  });
}

}  // namespace w4a4
