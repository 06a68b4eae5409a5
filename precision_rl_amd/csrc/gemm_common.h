// Tile scheduling shared by the grouped GEMM kernels (gfx950).
#pragma once

#include "device_common.h"

namespace w4a4 {

// 8 waves per workgroup, two per SIMD: while one wave waits on memory or
// decodes operands, the other keeps the SIMD's matrix core busy.  Waves are
// laid out 4 (M) x 2 (N); each owns a 64 x 128 sub-tile of the 256 x 256 tile.
constexpr int kGemmThreads = 512;
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kWaveM = 64;
constexpr int kWaveN = 128;
constexpr int kXcds = 8;           // MI355X: workgroups are dealt round-robin over 8 XCDs

struct TileCoord {
  int e;         // expert
  int64_t m0;    // first row of the tile
  int64_t m_end; // end of the expert's rows
  int n_tile;
  bool valid;
};

// Maps blockIdx.x onto (expert, M tile, N tile) for a GEMM whose M dimension
// is the concatenation of the expert row groups [offsets[e], offsets[e+1]).
// The number of tiles exists only on the device; every workgroup recomputes
// it from the offsets (a scan over E in LDS).  Logical tiles are ordered
// expert-major, N fastest, and dealt out in contiguous runs per XCD so that an
// expert's weight tiles and an M tile's activations stay in one XCD's L2.
// `scratch` must hold kGemmThreads + E ints of LDS.
__device__ inline TileCoord grouped_m_tile(const int32_t* __restrict__ offsets, int E, int n_tiles,
                                           int* scratch) {
  const int tid = threadIdx.x;
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += kGemmThreads) {
    const int e = e0 + tid;
    int v = 0;
    if (e < E) {
      const int rows = offsets[e + 1] - offsets[e];
      v = (rows + kTileM - 1) / kTileM;
    }
    scratch[tid] = v;
    __syncthreads();
    for (int off = 1; off < kGemmThreads; off <<= 1) {
      int add = tid >= off ? scratch[tid - off] : 0;
      __syncthreads();
      scratch[tid] += add;
      __syncthreads();
    }
    const int incl = scratch[tid] + carry;
    const int chunk_total = scratch[kGemmThreads - 1];
    __syncthreads();
    if (e < E) scratch[kGemmThreads + e] = incl;  // parked above the scan window
    carry += chunk_total;
    __syncthreads();
  }
  const int total_m = carry;
  TileCoord tc;
  tc.valid = false;
  const int64_t total = static_cast<int64_t>(total_m) * n_tiles;
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t b = blockIdx.x;
  const int64_t y = b / kXcds, x = b % kXcds;
  if (y >= per_xcd) return tc;
  const int64_t L = x * per_xcd + y;
  if (L >= total) return tc;
  const int mt = static_cast<int>(L / n_tiles);
  tc.n_tile = static_cast<int>(L % n_tiles);
  // find expert e with incl[e-1] <= mt < incl[e]
  const int* incl = scratch + kGemmThreads;
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if (incl[mid] > mt) hi = mid; else lo = mid + 1;
  }
  const int e = lo;
  const int first = e ? incl[e - 1] : 0;
  tc.e = e;
  tc.m0 = offsets[e] + static_cast<int64_t>(mt - first) * kTileM;
  tc.m_end = offsets[e + 1];
  tc.valid = true;
  return tc;
}

// Upper bound of the M-tile count for a grouped GEMM: every expert adds at
// most one partial tile.
inline int64_t grouped_m_tiles_bound(int64_t rows_alloc, int E) {
  return (rows_alloc + kTileM - 1) / kTileM + E;
}

inline unsigned xcd_grid(int64_t tiles) {
  return static_cast<unsigned>((tiles + kXcds - 1) / kXcds * kXcds);
}

// Row of the output tile held in accumulator element v of lane (r32, hl) for
// MFMA 32x32 tile mi of a wave whose rows start at wave_row0.
__device__ __forceinline__ int acc_row(int wave_row0, int mi, int v, int hl) {
  return wave_row0 + mi * 32 + (v & 3) + 4 * hl + 8 * (v >> 2);
}

}  // namespace w4a4
