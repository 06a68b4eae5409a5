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
// Every Q(.) rounds the exact quotient.  Directly, the E4M3 quotient is one
// correctly rounded float64 division, which keeps the side of every rounding
// midpoint (operands have <= 8 and <= 26 significant bits), and for the E2M1
// codes the seven midpoints mu * g * d_b (mu in .25 .75 1.25 1.75 2.5 3.5 5)
// are exact float64 products, each turned into the smallest bf16 value that a
// bf16 |x| must reach to cross it (ties resolved towards the even code); the
// per-element work is then a three-step search over those thresholds on the
// bf16 bit patterns.  The row encoder takes a cheaper route to the same bytes
// for outer scales in [2^-100, 2^100]: the E4M3 code from a per-row reciprocal
// of 6 g with an exact check at E4M3 midpoints (checked against the direct
// route over every pair of row and block maxima), and the E2M1 codes from the
// hardware FP4 conversion of the quotient bracketed from below and above,
// which decides every element but those next to an E2M1 midpoint; blocks
// holding such an element take the exact thresholds.

#include <algorithm>
#include <mutex>
#include <type_traits>

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

// Value of an E4M3FN code (no NaN codes occur here): subnormal m * 2^-9,
// normal (8 + m) * 2^(e - 10).
__device__ __forceinline__ double e4m3_value(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  return e == 0u ? static_cast<double>(m) * 0x1p-9 : ldexp(static_cast<double>(8u + m), static_cast<int>(e) - 10);
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
// number of set bits below it (stable: ascending token order), from a per
// expert prefix of the mask words' popcounts and the popcount of its own
// word below its bit.  The local rank is parked in row_map and the
// per-chunk counts in `counts`.  A token's ids are read once and kept in
// registers (k <= kMaxRouteK).
__global__ void __launch_bounds__(kRouteChunk)
route_count_kernel(const int32_t* __restrict__ topk_idx, int64_t T, int k, int E,
                   int32_t* __restrict__ row_map, int32_t* __restrict__ counts) {
  constexpr int W = kRouteChunk / 32;
  extern __shared__ uint32_t masks[];      // [W][E] masks, then [W][E] popcount prefixes
  uint32_t* const prefix = masks + E * W;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  for (int i = tid; i < E * W; i += kRouteChunk) masks[i] = 0u;
  const int64_t t = static_cast<int64_t>(c) * kRouteChunk + tid;
  const bool live = t < T;
  int ids[kMaxRouteK];
#pragma unroll
  for (int j = 0; j < kMaxRouteK; ++j) ids[j] = (live && j < k) ? topk_idx[t * k + j] : 0;
  __syncthreads();
  const int word = tid / 32;
  const uint32_t bit = 1u << (tid % 32);
#pragma unroll
  for (int j = 0; j < kMaxRouteK; ++j)
    if (live && j < k) atomicOr(&masks[word * E + ids[j]], bit);
  __syncthreads();
  for (int e = tid; e < E; e += kRouteChunk) {
    uint32_t run = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      prefix[w * E + e] = run;
      run += __popc(masks[w * E + e]);
    }
    counts[static_cast<int64_t>(c) * E + e] = static_cast<int32_t>(run);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kMaxRouteK; ++j) {
    if (live && j < k) {
      const int m = word * E + ids[j];
      row_map[t * k + j] = static_cast<int32_t>(prefix[m] + __popc(masks[m] & (bit - 1u)));
    }
  }
}

// Dynamic LDS of route_count_kernel for E experts.
inline uint32_t route_count_lds(int E) {
  return 2u * static_cast<uint32_t>(E) * (kRouteChunk / 32) * sizeof(uint32_t);
}

// Single workgroup: per expert, exclusive prefix of the chunk counts (in
// place, giving each chunk's first rank), the expert totals, and the padded
// expert offsets.  Thread (e, s) owns expert e and a contiguous segment s of
// the chunks (S = 1024 / E segments): it sums its segment (keeping the first
// kKeep counts in registers), the segment sums meet in LDS, and it then
// writes its chunks' running prefix.  Wave 0 then forms the expert totals and
// scans the padded group sizes (each lane q = E / 64 consecutive experts in
// turn, the lanes by a wave prefix sum).
constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(kScanThreads)
route_scan_kernel(int32_t* __restrict__ counts, int n_chunks, int E, int row_align,
                  int32_t* __restrict__ offsets, int32_t* __restrict__ expert_count) {
  constexpr int kKeep = 16;
  __shared__ int32_t seg[kScanThreads];
  const int tid = threadIdx.x;
  const int S = max(1, kScanThreads / E);
  const int e = tid % E, sgi = tid / E;
  const bool owner = sgi < S && tid < E * S;
  const int per = (n_chunks + S - 1) / S;
  const int c0 = min(n_chunks, sgi * per), c1 = min(n_chunks, c0 + per);
  int keep[kKeep];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kKeep; ++i) {
    keep[i] = (owner && c0 + i < c1) ? counts[static_cast<int64_t>(c0 + i) * E + e] : 0;
    sum += keep[i];
  }
  if (owner)
    for (int c = c0 + kKeep; c < c1; ++c) sum += counts[static_cast<int64_t>(c) * E + e];
  seg[tid] = sum;
  __syncthreads();
  if (owner) {
    int run = 0;
    for (int j = 0; j < sgi; ++j) run += seg[j * E + e];   // segments before mine
#pragma unroll
    for (int i = 0; i < kKeep; ++i) {
      if (c0 + i < c1) {
        counts[static_cast<int64_t>(c0 + i) * E + e] = run;
        run += keep[i];
      }
    }
    for (int c = c0 + kKeep; c < c1; ++c) {
      const int64_t i = static_cast<int64_t>(c) * E + e;
      const int v = counts[i];
      counts[i] = run;
      run += v;
    }
  }
  if (tid >= kWave) return;
  // wave 0: expert totals and the exclusive scan of the padded group sizes
  // (E <= 1024: at most 16 experts per lane)
  const int q = (E + kWave - 1) / kWave;
  int tot = 0;
  for (int i = 0; i < q; ++i) {
    const int ee = tid * q + i;
    if (ee < E) {
      int n = 0;
      for (int j = 0; j < S; ++j) n += seg[j * E + ee];
      expert_count[ee] = n;
      tot += (n + row_align - 1) / row_align * row_align;
    }
  }
  int incl = tot;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(incl, d, kWave);
    if (tid >= d) incl += v;
  }
  int run = incl - tot;
  for (int i = 0; i < q; ++i) {
    const int ee = tid * q + i;
    if (ee < E) {
      int n = 0;
      for (int j = 0; j < S; ++j) n += seg[j * E + ee];
      run += (n + row_align - 1) / row_align * row_align;
      offsets[ee + 1] = run;
    }
  }
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

// ------------------------------------------------ row encoder, K % 32 == 0
// The E2M1 magnitude code of a bf16 magnitude m is the number of the block's
// seven crossing thresholds t_0 < ... < t_6 that m reaches.  It is found by
// a three-step binary search, two elements at a time in packed 16-bit
// integer arithmetic: with t' = t - 1, m reaches t exactly when t' - m is
// negative (no overflow: both lie in [-1, 0x7FFF]).  The never-crossed
// sentinel becomes t' = 0x7FFF.
struct PackedThr {
  uint32_t t[7];   // t - 1 in both 16-bit halves
};

__device__ __forceinline__ PackedThr pack_thresholds(const BlockThresholds& th) {
  PackedThr p;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const uint32_t v = th.t[j] >= 0x8000u ? 0x7FFFu : ((th.t[j] - 1u) & 0xFFFFu);
    p.t[j] = v * 0x00010001u;
  }
  return p;
}

// A constant the compiler cannot see through (an empty asm statement, which
// it may still hoist and merge): the patterns below stay the instructions they
// are written as instead of being rewritten for the known value.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm("" : "+s"(v));
  return v;
}

typedef int16_t i16x2_t __attribute__((ext_vector_type(2)));

// 0xFFFF in each 16-bit half whose magnitude reaches the threshold: the sign
// of t' - m, spread over the half (v_pk_sub_i16 and v_pk_ashrrev_i16; with a
// visible shift count of 15 the compiler turns the shift into compares on
// unpacked halves).
__device__ __forceinline__ uint32_t reach(uint32_t tp, uint32_t m) {
  const i16x2_t d = __builtin_bit_cast(i16x2_t, tp) - __builtin_bit_cast(i16x2_t, m);
  return __builtin_bit_cast(uint32_t, d >> __builtin_bit_cast(i16x2_t, opaque(0x000F000Fu)));
}

__device__ __forceinline__ uint32_t select_bits(uint32_t mask, uint32_t a, uint32_t b) {
  return (a & mask) | (b & ~mask);   // v_bfi_b32
}

// (a & mask) | (b & ~mask) as one v_bfi_b32 (with a visible constant mask the
// compiler splits nested inserts into ands and ors)
__device__ __forceinline__ uint32_t bit_insert(uint32_t mask, uint32_t a, uint32_t b) {
  return select_bits(opaque(mask), a, b);
}

// Two bf16 (one dword, element 2j low) -> two 4-bit codes in the low nibble
// of each 16-bit half.
__device__ __forceinline__ uint32_t code_pair(uint32_t w, const PackedThr& p) {
  const uint32_t m = w & 0x7FFF7FFFu;
  const uint32_t s4 = reach(p.t[3], m);
  const uint32_t s2 = reach(select_bits(s4, p.t[5], p.t[1]), m);
  const uint32_t t1 = select_bits(s4, select_bits(s2, p.t[6], p.t[4]), select_bits(s2, p.t[2], p.t[0]));
  const uint32_t s1 = reach(t1, m);
  // magnitude bits 2..0 of both halves from the masks, bit 3 the element's
  // sign (w >> 12 moves bits 15 and 31 to 3 and 19 and leaves 20..31 clear)
  const uint32_t y = bit_insert(0x00070007u, bit_insert(0x00040004u, s4, bit_insert(0x00020002u, s2, s1)),
                                w >> 12);
  // the high element's nibble (bits 16..19) next to the low one's: bits 8..31
  // of the result come from y >> 12, whose bits 8..31 are clear.  Kept opaque
  // so that the byte shifts of the caller are not folded back into the inserts.
  uint32_t b = bit_insert(0x0000000Fu, y, y >> 12);
  asm("" : "+v"(b));
  return b;
}

// 16 bf16 (8 dwords) -> 8 code bytes (2 dwords), element 2j in the low nibble of byte j.
__device__ __forceinline__ u32x2_t encode16(const uint32_t (&w)[8], const PackedThr& p) {
  u32x2_t out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t v = code_pair(w[4 * h], p);
#pragma unroll
    for (int i = 1; i < 4; ++i) v |= code_pair(w[4 * h + i], p) << (8 * i);
    out[h] = v;
  }
  return out;
}

typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                __builtin_bit_cast(u16x2_t, b)));
}

// Largest bf16 magnitude of 16 elements (magnitudes compare as integers),
// two at a time in packed 16-bit maxima.
__device__ __forceinline__ uint32_t amax16_of(const uint32_t (&w)[8]) {
  uint32_t m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = w[i] & 0x7FFF7FFFu;
  const uint32_t a = pk_max_u16(pk_max_u16(pk_max_u16(m[0], m[1]), pk_max_u16(m[2], m[3])),
                                pk_max_u16(pk_max_u16(m[4], m[5]), pk_max_u16(m[6], m[7])));
  return max(a & 0xFFFFu, a >> 16);
}

// E4M3 code of q = amax / (6 g), rounded to nearest even and saturated at 448,
// from q' = amax * RN64(1 / (6 g)).  q' is within 2^-51 of q (relative); when
// q is not itself a rounding midpoint it differs from every E4M3 midpoint M
// by more than 2^-31 of M (M has <= 5 significant bits, amax <= 8, 6 g <= 26),
// so q' and its float rounding lie on the same side of M as q.  Only when the
// float lands exactly on a midpoint is the side decided by the exact product
// 6 g M (<= 31 significant bits, exact in FP64) against amax.
__device__ __forceinline__ uint32_t e4m3_code_fast(uint32_t amax16, double inv6g, double g6) {
  const double ab = static_cast<double>(bf16_to_f32(static_cast<uint16_t>(amax16)));
  const float q = static_cast<float>(ab * inv6g);
  const uint32_t qb = __float_as_uint(q);
  const float qs = q * 512.0f;          // subnormal E4M3 values are multiples of 2^-9
  const bool sub = q < 0x1p-6f;
  // normal range: keep 3 mantissa bits, round half to even on the float's bits
  // (a carry moves to the next binade); the code is the shifted pattern
  // rebased from float exponent bias 127 to E4M3 bias 7
  uint32_t c = sub ? static_cast<uint32_t>(rintf(qs)) : ((qb + 0x7FFFFu + ((qb >> 20) & 1u)) >> 20) - 960u;
  const bool mid = sub ? (qs - floorf(qs)) == 0.5f : (qb & 0xFFFFFu) == 0x80000u;
  if (mid) {
    const double m = g6 * static_cast<double>(q);
    const uint32_t lo = sub ? static_cast<uint32_t>(floorf(qs)) : (qb >> 20) - 960u;
    if (ab > m) c = lo + 1u;
    else if (ab < m) c = lo;
  }
  return min(c, 0x7Eu);
}

// Value of E4M3 code c (0 < c <= 0x7E) as a float: normal codes are the
// float with exponent field e + 120 and mantissa m << 20, subnormal ones m 2^-9.
__device__ __forceinline__ float e4m3_float(uint32_t c) {
  return c >= 8u ? __uint_as_float((c << 20) + (120u << 23)) : static_cast<float>(c) * 0x1p-9f;
}

// E2M1 codes of 16 bf16 elements (8 dwords, element 2j low; 8 code bytes,
// element 2j in the low nibble of byte j) of a block with effective scale
// D = d g, by the hardware conversion v_cvt_scalef32_pk_fp4_f32 (round to
// nearest even onto E2M1, saturating at 6, the sign in bit 3), applied to x / D
// bracketed from both sides.  With ilo = RN(inv (1 - 2^-19)) and
// ihi = RN(inv (1 + 2^-19)), inv = rcp(RN(D)) within one float ulp, every
// product |RN(x ilo)| lies below |x| / D and |RN(x ihi)| above it (by more
// than 2^-20 of it: the four roundings add at most 2^-21.4); products that
// underflow only meet code 0, with the sign of x.  The conversion is monotone,
// so where the codes of the two products agree (`lo` = `hi`) they are the code
// of x / D itself; where they differ, by one, an E2M1 midpoint lies between
// the two products and the element is left to the exact check below.  D = 0 (a
// zero block scale): ilo = ihi = 0 gives the zero codes with the elements'
// signs.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Codes of the bf16 pair v, the quotients scaled by `inv`, into byte B of `acc`.
template <int B>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t acc, uint32_t v, float inv) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, bf16_lo(v) * inv, bf16_hi(v) * inv, 1.0f, B);
}

__device__ __forceinline__ void encode16_hw(const uint32_t (&w)[8], float ilo, float ihi, u32x2_t& lo, u32x2_t& hi) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t* p = w + 4 * h;
    lo[h] = fp4_pair<3>(fp4_pair<2>(fp4_pair<1>(fp4_pair<0>(0u, p[0], ilo), p[1], ilo), p[2], ilo), p[3], ilo);
    hi[h] = fp4_pair<3>(fp4_pair<2>(fp4_pair<1>(fp4_pair<0>(0u, p[0], ihi), p[1], ihi), p[2], ihi), p[3], ihi);
  }
}

// E2M1 codes of the 8 bf16 elements of v (element 2j low in dword j) times
// 2^sh (one code dword, element 2j in the low nibble of byte j).
__device__ __forceinline__ uint32_t fp4x8_ldexp(const u32x4_t& v, int sh) {
  auto pair = [&](uint32_t acc, uint32_t w, auto byte) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, __builtin_amdgcn_ldexpf(bf16_lo(w), sh),
                                                    __builtin_amdgcn_ldexpf(bf16_hi(w), sh), 1.0f,
                                                    decltype(byte)::value);
  };
  uint32_t r = pair(0u, v[0], std::integral_constant<int, 0>{});
  r = pair(r, v[1], std::integral_constant<int, 1>{});
  r = pair(r, v[2], std::integral_constant<int, 2>{});
  return pair(r, v[3], std::integral_constant<int, 3>{});
}

// The exact codes of the elements the bracket left open.  The 32 elements of
// a block pair: code dword k holds elements 8k .. 8k+7 (nibble n: element
// 8k + n), whose bf16 values are the four dwords of x[k]; nonzero nibbles of
// `open` mark the undecided elements, whose nibble in `cw` holds the lower of
// the two candidate codes c and c + 1.  The element takes c + 1 when its
// magnitude exceeds mu d g, mu the E2M1 midpoint between c and c + 1, or equals
// it and c is odd (the tie goes to the even code); mu d g has at most 31
// significant bits (mu at most 3, d 4, g 24), so the FP64 product and the
// comparison are exact.  One element per lane and iteration; the wave loops
// while any lane has one left (usually once: about one element in 500 is open
// for continuous data, mostly where rounding g to float32 put x / D within 2^-24
// of a midpoint).
__device__ __forceinline__ void settle_open(u32x4_t& cw, u32x4_t open, const u32x4_t (&x)[4], uint32_t sc2, float g) {
  // 4 mu for c = 0 .. 6 (0.25 0.75 1.25 1.75 2.5 3.5 5), 5 bits each
  constexpr uint64_t kMid4 = 1ull | 3ull << 5 | 5ull << 10 | 7ull << 15 | 10ull << 20 | 14ull << 25 | 20ull << 30;
  // the element values as plain registers: selecting among them must stay
  // v_cndmask (a select between array elements may become a dynamic index,
  // which would move the row buffer to scratch memory)
  uint32_t xs[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    xs[j] = x[j >> 2][j & 3];
    asm("" : "+v"(xs[j]));
  }
  while ((open[0] | open[1] | open[2] | open[3]) != 0u) {
    const bool k0 = open[0] != 0u, k1 = !k0 && open[1] != 0u, k2 = !k0 && !k1 && open[2] != 0u;
    const bool k3 = !k0 && !k1 && !k2;
    const uint32_t f = k0 ? open[0] : k1 ? open[1] : k2 ? open[2] : open[3];
    const uint32_t c = k0 ? cw[0] : k1 ? cw[1] : k2 ? cw[2] : cw[3];
    const uint32_t sh = static_cast<uint32_t>(__builtin_ctz(f)) & ~3u;   // 4 n
    const uint32_t n = sh >> 2;
    uint32_t xq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xq[q] = k0 ? xs[q] : k1 ? xs[4 + q] : k2 ? xs[8 + q] : xs[12 + q];
    const uint32_t wd = n < 2u ? xq[0] : n < 4u ? xq[1] : n < 6u ? xq[2] : xq[3];
    const uint32_t mag = ((n & 1u) ? (wd >> 16) : wd) & 0x7FFFu;
    const uint32_t clo = (c >> sh) & 7u;
    const uint32_t dbits = (sc2 >> ((k2 || k3) ? 8 : 0)) & 0xFFu;
    const double mu = static_cast<double>(static_cast<uint32_t>(kMid4 >> (5u * clo)) & 31u) * 0.25;
    const double t = mu * (e4m3_value(dbits) * static_cast<double>(g));
    const double xm = static_cast<double>(bf16_to_f32(static_cast<uint16_t>(mag)));
    const uint32_t up = (xm > t || (xm == t && (clo & 1u) != 0u)) ? 1u : 0u;
    const uint32_t nc = c + (up << sh);       // c + 1 <= 7: no carry into the sign bit
    const uint32_t clear = ~(0xFu << sh);
    cw[0] = k0 ? nc : cw[0];
    cw[1] = k1 ? nc : cw[1];
    cw[2] = k2 ? nc : cw[2];
    cw[3] = k3 ? nc : cw[3];
    open[0] = k0 ? (open[0] & clear) : open[0];
    open[1] = k1 ? (open[1] & clear) : open[1];
    open[2] = k2 ? (open[2] & clear) : open[2];
    open[3] = k3 ? (open[3] & clear) : open[3];
  }
}

enum class RowMode { Scatter, Identity, Requant };

// One team of TEAM lanes per row; lane l of a team owns block pairs
// l, l + TEAM, ... (PB of them), i.e. 32 consecutive elements each: 64 B
// loaded, 16 B of codes and 2 B of scales stored per destination row.  The
// workgroups stride over the rows and each wave loads its next row before
// encoding the current one.
//   Scatter:  rows are tokens, written to their k expert rows (routing done);
//   Identity: row r -> row r (weights), also writes row_map / src_row / offsets;
//   Requant:  row r -> row r for the rows [0, offsets[E]).
// MX: the MXFP4 recipe instead of NVFP4 -- each lane's 32 elements are one
// block with an E8M0 scale 2^X, X = floor(log2 amax) - 2 clamped to
// [-127, 127] (OCP Microscaling v1.0, section 6.3), codes Q_E2M1(x / 2^X);
// one scale byte per 32 elements, no outer scale.
// PF: load the wave's next row group while encoding the current one.  Worth
// it only when the waves stride over several row groups; without it the
// second row buffer's registers are free and more waves fit on a SIMD.
template <int TEAM, int PB, RowMode MODE, bool MX = false, bool PF = true>
__global__ void __launch_bounds__(kThreads)
quant_rows_kernel(const uint16_t* __restrict__ x, int64_t n_rows, int K,
                  const int32_t* __restrict__ topk_idx, int k, int E,
                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ outer,
                  int32_t* __restrict__ offsets, int32_t* __restrict__ row_map,
                  int32_t* __restrict__ src_row, const int32_t* __restrict__ chunk_base,
                  const uint32_t* __restrict__ group_amax, int64_t group_rows) {
  constexpr int kRowsPerWave = kWave / TEAM;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int team = lane / TEAM, tl = lane % TEAM;
  const int pairs = K / 32;
  const int64_t K2 = K / 2, K16 = K / 16, K32 = K / 32;
  int64_t n = n_rows;
  if constexpr (MODE == RowMode::Requant) n = min<int64_t>(n, offsets[E]);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWavesPerBlock * kRowsPerWave;
  int64_t r = (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave) * kRowsPerWave + team;

  u32x4_t cur[PB][4], nxt[PB][4];
  auto load = [&](int64_t row, u32x4_t (&buf)[PB][4]) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + row * K);
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int p = tl + i * TEAM;
      if (p < pairs) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // the activations are read once, from HBM: non-temporal (encoder
          // -8% flushed); the requantised a was just written by FC1 and may
          // still sit in the MALL: plain loads
          if constexpr (MODE == RowMode::Requant) buf[i][q] = src[p * 4 + q];
          else buf[i][q] = __builtin_nontemporal_load(src + p * 4 + q);
        }
      }
    }
  };
  if (r < n) load(r, cur);
  for (; r < n; r += stride) {
    if constexpr (PF)
      if (r + stride < n) load(r + stride, nxt);

    // block amaxes; row amax over the team (NVFP4 only)
    uint32_t bm[PB][2];
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int p = tl + i * TEAM;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w[8] = {cur[i][2 * h][0], cur[i][2 * h][1], cur[i][2 * h][2], cur[i][2 * h][3],
                               cur[i][2 * h + 1][0], cur[i][2 * h + 1][1], cur[i][2 * h + 1][2], cur[i][2 * h + 1][3]};
        bm[i][h] = p < pairs ? amax16_of(w) : 0u;
        amax = max(amax, bm[i][h]);
      }
    }
    float g = 0.0f;
    bool fast = false;
    double g6 = 0.0, inv6g = 0.0;
    if constexpr (!MX) {
#pragma unroll
      for (int off = TEAM / 2; off > 0; off >>= 1) amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), off, kWave)));
      // a wider outer-scale domain: the group's max instead of the row's
      if (group_amax != nullptr) amax = group_amax[r / group_rows];
      g = outer_scale(amax);
      fast = g == 0.0f || (g >= 0x1p-100f && g <= 0x1p100f);
      g6 = 6.0 * static_cast<double>(g);
      inv6g = g > 0.0f ? 1.0 / g6 : 0.0;
    }

    // destination rows
    int64_t dst[8];
    int ndst = 1;
    dst[0] = r;
    if constexpr (MODE == RowMode::Scatter) {
      int32_t myrow = 0;
      if (tl < k) {
        const int e = topk_idx[r * k + tl];
        myrow = offsets[e] + chunk_base[(r / kRouteChunk) * E + e] + row_map[r * k + tl];
        row_map[r * k + tl] = myrow;
        src_row[myrow] = static_cast<int32_t>(r);
      }
      ndst = k;
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j] = __shfl(myrow, team * TEAM + j, kWave);
    } else if constexpr (MODE == RowMode::Identity) {
      if (tl == 0) {
        row_map[r] = static_cast<int32_t>(r);
        src_row[r] = static_cast<int32_t>(r);
        if (r == 0) {
          offsets[0] = 0;
          offsets[1] = static_cast<int32_t>(n_rows);
        }
      }
    }

#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int p = tl + i * TEAM;
      if (p >= pairs) continue;
      u32x4_t cw;
      uint32_t sc2 = 0;
      if constexpr (MX) {
        // E8M0 byte X + 127 from the bf16 exponent field eb of the block max:
        // floor(log2 amax) = eb - 127 for a normal amax, so the byte is
        // eb - 2; zero and subnormal maxima (and eb <= 2) clamp to byte 0
        const uint32_t eb = max(bm[i][0], bm[i][1]) >> 7;
        sc2 = eb > 2u ? eb - 2u : 0u;
        // the codes of x 2^-X (|x 2^-X| < 8): a bf16 times a power of two is
        // exact down to 2^-126, and anything smaller meets a zero code (with
        // the sign of x) either way; the hardware conversion rounds it to
        // nearest even onto E2M1, saturating at 6
        const int sh = 127 - static_cast<int>(sc2);
#pragma unroll
        for (int q = 0; q < 4; ++q) cw[q] = fp4x8_ldexp(cur[i][q], sh);
      } else {
      u32x4_t open = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w[8] = {cur[i][2 * h][0], cur[i][2 * h][1], cur[i][2 * h][2], cur[i][2 * h][3],
                               cur[i][2 * h + 1][0], cur[i][2 * h + 1][1], cur[i][2 * h + 1][2], cur[i][2 * h + 1][3]};
        uint32_t dbits = 0;
        if (fast) {
          dbits = e4m3_code_fast(bm[i][h], inv6g, g6);
        } else if (g > 0.0f) {
          double dval;
          dbits = e4m3_rne(static_cast<double>(bf16_to_f32(static_cast<uint16_t>(bm[i][h]))) / g6, &dval);
        }
        // in-range rows: the hardware conversion of the bracketed quotient
        // (its open elements are settled below); out-of-range rows: the
        // exact thresholds
        if (fast) {
          const float inv = dbits != 0u ? __builtin_amdgcn_rcpf(e4m3_float(dbits) * g) : 0.0f;
          u32x2_t lo, hi;
          encode16_hw(w, inv * (1.0f - 0x1p-19f), inv * (1.0f + 0x1p-19f), lo, hi);
          cw[2 * h] = lo[0];
          cw[2 * h + 1] = lo[1];
          open[2 * h] = lo[0] ^ hi[0];
          open[2 * h + 1] = lo[1] ^ hi[1];
        } else {
          const u32x2_t c2 = encode16(w, pack_thresholds(make_thresholds(static_cast<double>(g) * e4m3_value(dbits))));
          cw[2 * h] = c2[0];
          cw[2 * h + 1] = c2[1];
        }
        sc2 |= dbits << (8 * h);
      }
      if (fast) settle_open(cw, open, cur[i], sc2, g);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < ndst) {
          *reinterpret_cast<u32x4_t*>(codes + dst[j] * K2 + p * 16) = cw;
          if constexpr (MX)
            scales[dst[j] * K32 + p] = static_cast<uint8_t>(sc2);
          else
            *reinterpret_cast<uint16_t*>(scales + dst[j] * K16 + p * 2) = static_cast<uint16_t>(sc2);
        }
      }
    }
    if (!MX && tl < ndst) {
      int64_t d = dst[0];
#pragma unroll
      for (int j = 1; j < 8; ++j)
        if (tl == j) d = dst[j];
      outer[d] = g;
    }
    if constexpr (PF) {
#pragma unroll
      for (int i = 0; i < PB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) cur[i][q] = nxt[i][q];
    } else if (r + stride < n) {
      load(r + stride, cur);
    }
  }
}

// Pad rows of the expert groups (rows [offsets[e] + count[e], offsets[e+1])):
// zero codes, scales and g (MX: no g; one scale per 32); src_row = -1.  One
// wave per expert.
template <bool MX = false>
__global__ void __launch_bounds__(kThreads)
pad_rows_kernel(int K, int E, const int32_t* __restrict__ offsets, const int32_t* __restrict__ expert_count,
                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ outer,
                int32_t* __restrict__ src_row) {
  const int lane = threadIdx.x % kWave;
  const int e = static_cast<int>(blockIdx.x) * kWavesPerBlock + static_cast<int>(threadIdx.x / kWave);
  if (e >= E) return;
  const int64_t K2 = K / 2, K16 = K / 16;
  const int64_t r0 = offsets[e] + expert_count[e], r1 = offsets[e + 1];
  for (int64_t r = r0; r < r1; ++r) {
    for (int b = lane; b < K / 16; b += kWave) {
      *reinterpret_cast<u32x2_t*>(codes + r * K2 + b * 8) = u32x2_t{0u, 0u};
      if (!MX) scales[r * K16 + b] = 0;
      else if (b < K / 32) scales[r * (K / 32) + b] = 0;
    }
    if (lane == 0) {
      if (!MX) outer[r] = 0.0f;
      src_row[r] = -1;
    }
  }
}

// Launches quant_rows_kernel with the team shape for K (K % 32 == 0, K <= 4096).
template <RowMode MODE, bool MX = false>
bool launch_rows(const char* name, const uint16_t* x, int64_t n_rows, int K, const int32_t* topk_idx, int k,
                 int E, uint8_t* codes, uint8_t* scales, float* outer, int32_t* offsets,
                 int32_t* row_map, int32_t* src_row, const int32_t* chunk_base, hipStream_t s,
                 const uint32_t* group_amax = nullptr, int64_t group_rows = 1) {
  const int pairs = K / 32;
  auto go = [&](auto team, auto pb) {
    constexpr int TEAM = decltype(team)::value, PB = decltype(pb)::value;
    constexpr int rows_per_block = kWavesPerBlock * (kWave / TEAM);
    // Up to 16 workgroups per CU: at the workloads' sizes every wave takes one
    // row group, and the waves that wait on memory are many (a grid sized to
    // the resident waves, each striding over several row groups, measured
    // slower); larger inputs make the waves stride.
    const int64_t need = (n_rows + rows_per_block - 1) / rows_per_block;
    const int64_t blocks = std::min<int64_t>(need, static_cast<int64_t>(device_cu_count()) * 16);
    if (blocks == 0) return true;
    // Requant bounds its rows by offsets[E] on the device: n_rows is the
    // allocation, an upper bound, so the choice is made on that bound.
    auto kernel = need > blocks ? quant_rows_kernel<TEAM, PB, MODE, MX, true>
                                : quant_rows_kernel<TEAM, PB, MODE, MX, false>;
    launch_kernel(name, kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                  s, x, n_rows, K, topk_idx, k, E, codes, scales, outer, offsets, row_map, src_row, chunk_base,
                  group_amax, group_rows);
    return launch_ok(name);
  };
  // One block pair per lane in a team that covers the row (a wave then
  // writes whole rows, which the 8-way scatter needs); rows of 24, 48 or 96
  // pairs, which would leave a quarter of a 32/64/128-lane team idle, take
  // three pairs per lane in a team of 8/16/32 instead.
  using I1 = std::integral_constant<int, 1>;
  using I3 = std::integral_constant<int, 3>;
  if (pairs == 24) return go(std::integral_constant<int, 8>{}, I3{});
  if (pairs == 48) return go(std::integral_constant<int, 16>{}, I3{});
  if (pairs == 96) return go(std::integral_constant<int, 32>{}, I3{});
  if (pairs <= 8) return go(std::integral_constant<int, 8>{}, I1{});
  if (pairs <= 16) return go(std::integral_constant<int, 16>{}, I1{});
  if (pairs <= 32) return go(std::integral_constant<int, 32>{}, I1{});
  if (pairs <= 64) return go(std::integral_constant<int, 64>{}, I1{});
  return go(std::integral_constant<int, 64>{}, std::integral_constant<int, 2>{});
}

bool rows_path(int K) { return K % 32 == 0 && K <= 4096; }

__global__ void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// Max |x| (bf16 magnitude bits) of each group of group_rows consecutive rows
// into amax[group] (zeroed before).  Workgroup b covers rows [b R, b R + R);
// the segment of each group in it is reduced over the workgroup and merged
// with one atomic max (exact and order-independent: bf16 magnitudes compare
// as integers).
constexpr int kAmaxThreads = 256;
__global__ void __launch_bounds__(kAmaxThreads)
group_amax_kernel(const uint16_t* __restrict__ x, int64_t n_rows, int K, int64_t group_rows,
                  int64_t rows_per_block, uint32_t* __restrict__ amax) {
  __shared__ uint32_t s_wave[kAmaxThreads / kWave];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rows_per_block;
  const int64_t r1 = min(n_rows, r0 + rows_per_block);
  for (int64_t a = r0; a < r1;) {
    const int64_t grp = a / group_rows;
    const int64_t b = min(r1, (grp + 1) * group_rows);
    const int64_t chunks = (b - a) * K / 8;   // 16-byte chunks (K % 32 == 0)
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(x + a * K);
    uint32_t m = 0;
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < chunks; i += kAmaxThreads) {
      const u32x4_t v = __builtin_nontemporal_load(p + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = v[j] & 0x7FFF7FFFu;
        m = max(m, max(w & 0xFFFFu, w >> 16));
      }
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
      m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off, kWave)));
    if (threadIdx.x % kWave == 0) s_wave[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < kAmaxThreads / kWave; ++w) t = max(t, s_wave[w]);
      if (t > 0) atomicMax(amax + grp, t);
    }
    __syncthreads();
    a = b;
  }
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
    launch_kernel("route_scan", zero_offsets_kernel, dim3(1), dim3(256), 0, s, offsets, E + 1);
    return launch_ok("zero_offsets");
  }
  if (topk_idx != nullptr) {
    launch_kernel("route_count", route_count_kernel, dim3(static_cast<unsigned>(n_chunks)), dim3(kRouteChunk),
                  route_count_lds(E),
                  s, topk_idx, T, k, E, row_map, counts);
    if (!launch_ok("route_count")) return false;
  }
  if (topk_idx != nullptr) {
    launch_kernel("route_scan", route_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts,
                  static_cast<int>(n_chunks), E, row_align, offsets, expert_count);
    if (!launch_ok("route_scan")) return false;
  }
  if (rows_path(K)) {
    const bool ok = topk_idx != nullptr
        ? launch_rows<RowMode::Scatter>("quantize_scatter", x, T, K, topk_idx, k, E, codes, scales, outer,
                                        offsets, row_map, src_row, counts, s)
        : launch_rows<RowMode::Identity>("quantize_scatter", x, T, K, nullptr, 1, 1, codes, scales, outer,
                                         offsets, row_map, src_row, nullptr, s);
    if (!ok) return false;
    if (topk_idx != nullptr && row_align > 1) {
      launch_kernel("pad_rows", pad_rows_kernel<false>, dim3(static_cast<unsigned>((E + kWavesPerBlock - 1) / kWavesPerBlock)),
                    dim3(kThreads), 0, s, K, E, offsets, expert_count, codes, scales, outer, src_row);
      return launch_ok("pad_rows");
    }
    return true;
  }
  const int64_t token_blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t pad_blocks = (topk_idx != nullptr && row_align > 1)
                                 ? (E + kWavesPerBlock - 1) / kWavesPerBlock : 0;
  const int64_t blocks = token_blocks + pad_blocks;
  if (blocks == 0) return true;
  return dispatch_maxb(K, [&](auto mb) {
    launch_kernel("quantize_scatter", quantize_scatter_kernel<decltype(mb)::value>,
                  dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, x, T, K, topk_idx, k, E, row_align,
                  codes, scales, outer, offsets, row_map, src_row, counts, expert_count, token_blocks);
    return launch_ok("quantize_scatter");
  });
}

size_t grouped_amax_bytes(int64_t T, int64_t group_rows) {
  const int64_t groups = group_rows > 0 ? (T + group_rows - 1) / group_rows : 0;
  return static_cast<size_t>(groups) * sizeof(uint32_t);
}

bool launch_quantize_permute_grouped(const uint16_t* x, int64_t T, int K, const int32_t* topk_idx,
                                     int k, int E, int row_align, int64_t group_rows, uint8_t* codes,
                                     uint8_t* scales, float* outer, int32_t* offsets, int32_t* row_map,
                                     int32_t* src_row, void* ws, uint32_t* amax, hipStream_t s) {
  if (!rows_path(K) || group_rows < 1) return false;
  if (T == 0) return launch_quantize_permute(x, T, K, topk_idx, k, E, row_align, codes, scales, outer,
                                             offsets, row_map, src_row, ws, s);
  const int64_t groups = (T + group_rows - 1) / group_rows;
  launch_kernel("zero_amax", zero_u32_kernel,
                dim3(static_cast<unsigned>(std::min<int64_t>((groups + 255) / 256, 1024))), dim3(256), 0, s,
                amax, groups);
  if (!launch_ok("zero_amax")) return false;
  const int64_t want_blocks = static_cast<int64_t>(device_cu_count()) * 4;
  const int64_t rows_per_block = std::max<int64_t>(1, (T + want_blocks - 1) / want_blocks);
  launch_kernel("group_amax", group_amax_kernel,
                dim3(static_cast<unsigned>((T + rows_per_block - 1) / rows_per_block)), dim3(kAmaxThreads), 0,
                s, x, T, K, group_rows, rows_per_block, amax);
  if (!launch_ok("group_amax")) return false;

  const int64_t n_chunks = (T + kRouteChunk - 1) / kRouteChunk;
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* expert_count = counts + n_chunks * E;
  if (topk_idx != nullptr) {
    launch_kernel("route_count", route_count_kernel, dim3(static_cast<unsigned>(n_chunks)), dim3(kRouteChunk),
                  route_count_lds(E),
                  s, topk_idx, T, k, E, row_map, counts);
    if (!launch_ok("route_count")) return false;
    launch_kernel("route_scan", route_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts,
                  static_cast<int>(n_chunks), E, row_align, offsets, expert_count);
    if (!launch_ok("route_scan")) return false;
  }
  const bool ok = topk_idx != nullptr
      ? launch_rows<RowMode::Scatter>("quantize_scatter", x, T, K, topk_idx, k, E, codes, scales, outer,
                                      offsets, row_map, src_row, counts, s, amax, group_rows)
      : launch_rows<RowMode::Identity>("quantize_scatter", x, T, K, nullptr, 1, 1, codes, scales, outer,
                                       offsets, row_map, src_row, nullptr, s, amax, group_rows);
  if (!ok) return false;
  if (topk_idx != nullptr && row_align > 1) {
    launch_kernel("pad_rows", pad_rows_kernel<false>, dim3(static_cast<unsigned>((E + kWavesPerBlock - 1) / kWavesPerBlock)),
                  dim3(kThreads), 0, s, K, E, offsets, expert_count, codes, scales, outer, src_row);
    return launch_ok("pad_rows");
  }
  return true;
}

bool launch_requant(const uint16_t* a, int64_t rows_alloc, int K, const int32_t* offsets, int E,
                    const int32_t* /*src_row*/, uint8_t* codes, uint8_t* scales, float* outer,
                    hipStream_t s) {
  if (rows_path(K))
    return launch_rows<RowMode::Requant>("requant", a, rows_alloc, K, nullptr, 1, E, codes, scales, outer,
                                         const_cast<int32_t*>(offsets), nullptr, nullptr, nullptr, s);
  const int64_t blocks = (rows_alloc + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return true;
  return dispatch_maxb(K, [&](auto mb) {
    launch_kernel("requant", requant_kernel<decltype(mb)::value>, dim3(static_cast<unsigned>(blocks)),
                  dim3(kThreads), 0, s, a, rows_alloc, K, offsets, E, codes, scales, outer);
    return launch_ok("requant");
  });
}

// MXFP4: route (as above), then the MX row encoder; K % 32 == 0, K <= 4096.
bool launch_quantize_permute_mx(const uint16_t* x, int64_t T, int K, const int32_t* topk_idx, int k, int E,
                                int row_align, uint8_t* codes, uint8_t* scales, int32_t* offsets,
                                int32_t* row_map, int32_t* src_row, void* ws, hipStream_t s) {
  if (!rows_path(K)) return false;
  const int64_t n_chunks = (T + kRouteChunk - 1) / kRouteChunk;
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* expert_count = counts + n_chunks * E;
  if (T == 0) {   // every group empty; all E + 1 offsets (an empty routing tensor may arrive as NULL)
    launch_kernel("route_scan", zero_offsets_kernel, dim3(1), dim3(256), 0, s, offsets, E + 1);
    return launch_ok("zero_offsets");
  }
  if (topk_idx != nullptr) {
    launch_kernel("route_count", route_count_kernel, dim3(static_cast<unsigned>(n_chunks)), dim3(kRouteChunk),
                  route_count_lds(E),
                  s, topk_idx, T, k, E, row_map, counts);
    if (!launch_ok("route_count")) return false;
    launch_kernel("route_scan", route_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts,
                  static_cast<int>(n_chunks), E, row_align, offsets, expert_count);
    if (!launch_ok("route_scan")) return false;
  }
  const bool ok = topk_idx != nullptr
      ? launch_rows<RowMode::Scatter, true>("mx_quantize_scatter", x, T, K, topk_idx, k, E, codes, scales,
                                            nullptr, offsets, row_map, src_row, counts, s)
      : launch_rows<RowMode::Identity, true>("mx_quantize_scatter", x, T, K, nullptr, 1, 1, codes, scales,
                                             nullptr, offsets, row_map, src_row, nullptr, s);
  if (!ok) return false;
  if (topk_idx != nullptr && row_align > 1) {
    launch_kernel("pad_rows", pad_rows_kernel<true>, dim3(static_cast<unsigned>((E + kWavesPerBlock - 1) / kWavesPerBlock)),
                  dim3(kThreads), 0, s, K, E, offsets, expert_count, codes, scales, nullptr, src_row);
    return launch_ok("pad_rows");
  }
  return true;
}

bool launch_requant_mx(const uint16_t* a, int64_t rows_alloc, int K, const int32_t* offsets, int E,
                       uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (!rows_path(K)) return false;
  return launch_rows<RowMode::Requant, true>("mx_requant", a, rows_alloc, K, nullptr, 1, E, codes, scales,
                                             nullptr, const_cast<int32_t*>(offsets), nullptr, nullptr, nullptr, s);
}

// ---------------------------------------------------------- routing validity
// err[0] = number of invalid entries of topk_idx [T, k] (an id outside
// [0, E), or equal to an earlier id of the same token), err[1] = the
// smallest flat index t*k + j of an invalid entry (INT32_MAX when none).
// err is set by routing_check_init_kernel and merged with vector atomics.
__global__ void routing_check_init_kernel(int32_t* __restrict__ err) {
  if (threadIdx.x == 0) {
    err[0] = 0;
    err[1] = 0x7FFFFFFF;
  }
}

__global__ void __launch_bounds__(256)
routing_check_kernel(const int32_t* __restrict__ topk_idx, int64_t T, int k, int E, int32_t* __restrict__ err) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  int bad = 0;
  int first = 0x7FFFFFFF;
  if (t < T) {
    int ids[kMaxRouteK];
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[t * k + j];
      ids[j] = e;
      bool ok = e >= 0 && e < E;
      for (int i = 0; i < j; ++i) ok = ok && ids[i] != e;
      if (!ok) {
        ++bad;
        first = min(first, static_cast<int>(t * k + j));
      }
    }
  }
  // wave totals, then one lane per wave merges them
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    bad += __shfl_xor(bad, off, kWave);
    first = min(first, __shfl_xor(first, off, kWave));
  }
  // a zero offset in a vector register keeps the atomics on the vector path
  uint32_t vzero = 0;
  asm volatile("" : "+v"(vzero));
  if ((threadIdx.x & 63) == 0 && bad > 0) {
    atomicAdd(err + vzero, bad);
    atomicMin(err + 1 + vzero, first);
  }
}

bool launch_check_routing(const int32_t* topk_idx, int64_t T, int k, int E, int32_t* err, hipStream_t s) {
  launch_kernel("routing_check_init", routing_check_init_kernel, dim3(1), dim3(64), 0, s, err);
  if (!launch_ok("routing_check_init")) return false;
  if (T == 0) return true;
  launch_kernel("routing_check", routing_check_kernel, dim3(static_cast<unsigned>((T + 255) / 256)), dim3(256), 0, s,
                topk_idx, T, k, E, err);
  return launch_ok("routing_check");
}

// ------------------------------------------------- allocation-free scratch
// The routing scratch (per-chunk expert counts and expert totals) of the
// allocation-free quantize+permute entry point lives in this file-scope
// array: each GPU the library runs on holds its own copy until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol); it looks up each device's address once,
// with that device current, and passes that.  Every call on one GPU shares
// the array, so calls that overlap on one GPU race.  Nothing in it has to
// start at zero: the count kernel writes every chunk's counts and the scan
// writes every expert total before they are read.
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

void* noalloc_scratch() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace w4a4
