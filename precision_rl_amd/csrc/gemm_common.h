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

// Maps blockIdx.x onto (expert, M tile of TM rows, N tile) for a GEMM whose M
// dimension is the concatenation of the expert row groups
// [offsets[e], offsets[e+1]).
// The number of tiles exists only on the device; wave 0 of every workgroup
// recomputes it from the offsets (lane-local sums and a wave prefix scan) and
// publishes the result through `slot` (LDS, 4 ints).  Logical tiles are
// ordered expert-major and dealt out in contiguous runs per XCD, so that an
// expert's operands stay in one XCD's L2; within an expert N runs fastest
// (tiles that run together share activation rows), or with M_FAST the M
// tiles run fastest (tiles that run together share a weight slab, for a
// weight operand larger than the L2).  Contains one __syncthreads().
template <int TM = kTileM, bool M_FAST = false>
__device__ inline TileCoord grouped_m_tile(const int32_t* __restrict__ offsets, int E, int n_tiles,
                                           int* slot) {
  const int tid = threadIdx.x;
  if (tid < kWave) {
    const int lane = tid;
    const int per = (E + kWave - 1) / kWave;
    const int e0 = lane * per, e1 = min(E, e0 + per);
    int cnt = 0;
    for (int e = e0; e < e1; ++e) cnt += (offsets[e + 1] - offsets[e] + TM - 1) / TM;
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int t = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += t;
    }
    const int total_m = __shfl(incl, kWave - 1, kWave);
    const int64_t total = static_cast<int64_t>(total_m) * n_tiles;
    const int64_t per_xcd = (total + kXcds - 1) / kXcds;
    const int64_t b = blockIdx.x;
    const int64_t y = b / kXcds, x = b % kXcds;
    const int64_t L = x * per_xcd + y;
    const bool valid = y < per_xcd && L < total;
    if (!valid) {
      if (lane == 0) slot[0] = -1;
    } else {
      const int mt = static_cast<int>(L / n_tiles);
      if (mt >= incl - cnt && mt < incl) {   // exactly one lane owns tile mt
        int first = incl - cnt;
        for (int e = e0; e < e1; ++e) {
          const int t = (offsets[e + 1] - offsets[e] + TM - 1) / TM;
          if (mt < first + t) {
            slot[0] = e;
            slot[2] = offsets[e + 1];
            if constexpr (M_FAST) {
              const int64_t le = L - static_cast<int64_t>(first) * n_tiles;   // tile within the expert
              slot[1] = offsets[e] + static_cast<int>(le % t) * TM;
              slot[3] = static_cast<int>(le / t);
            } else {
              slot[1] = offsets[e] + (mt - first) * TM;
              slot[3] = static_cast<int>(L % n_tiles);
            }
            break;
          }
          first += t;
        }
      }
    }
  }
  __syncthreads();
  // the values are the same in every lane: keep them in scalar registers
  TileCoord tc;
  tc.e = __builtin_amdgcn_readfirstlane(slot[0]);
  tc.valid = tc.e >= 0;
  tc.m0 = __builtin_amdgcn_readfirstlane(slot[1]);
  tc.m_end = __builtin_amdgcn_readfirstlane(slot[2]);
  tc.n_tile = __builtin_amdgcn_readfirstlane(slot[3]);
  return tc;
}

// Upper bound of the M-tile count for a grouped GEMM: every expert adds at
// most one partial tile.
inline int64_t grouped_m_tiles_bound(int64_t rows_alloc, int E, int tm = kTileM) {
  return (rows_alloc + tm - 1) / tm + E;
}

inline unsigned xcd_grid(int64_t tiles) {
  return static_cast<unsigned>((tiles + kXcds - 1) / kXcds * kXcds);
}

// Row of the output tile held in accumulator element v of lane (r32, hl) for
// MFMA 32x32 tile mi of a wave whose rows start at wave_row0.
__device__ __forceinline__ int acc_row(int wave_row0, int mi, int v, int hl) {
  return wave_row0 + mi * 32 + (v & 3) + 4 * hl + 8 * (v >> 2);
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most `vm`
// vector-memory operations of this wave are outstanding; LDS and export
// counters are left alone.
constexpr int waitcnt_vm(int vm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// Asynchronous copy global -> LDS (global_load_lds_dwordx4 / _dword): lane
// i's 16 bytes (4 bytes) land at LDS byte address lds + 16 i (4 i); `lds` is
// wave-uniform (it is moved to M0).  The copy counts on this wave's
// vector-memory counter and has landed once wait_vm_barrier<> allows fewer
// outstanding operations than were issued after it.  Issued from inline
// assembly so that the compiler's dependency tracking does not treat every
// later LDS read as aliasing the in-flight copies (it would wait for all of
// them); the kernels order LDS reads after copies explicitly.  M0 (the copy's
// LDS base) is not used for anything else in these kernels.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));   // low half of the flat address
}
// LDS pointer from a 32-bit LDS byte address (reads through it are ds_read
// with the constant part of the address as an immediate offset).
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(3))) T* lds_ptr(uint32_t a) {
  return reinterpret_cast<const __attribute__((address_space(3))) T*>(static_cast<uintptr_t>(a));
}
// Keeps a wave-uniform value in a scalar register and opaque to the compiler,
// so that addresses derived from it stay "per-lane offset + this value"
// instead of being re-derived per lane.
__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}
// A pointer that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved; nothing else here uses it
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               ::"v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
// Same copies addressed as a wave-uniform base (SGPR pair) plus a 32-bit
// per-lane byte offset, which saves the per-lane 64-bit address registers.
__device__ __forceinline__ void dma16_off(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               ::"v"(off), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_off(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               ::"v"(off), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Pipeline step: wait until at most VM vector-memory operations of this wave
// are outstanding (older global->LDS copies have landed), then a workgroup
// barrier.  No memory fence: later LDS reads are ordered by the asm's memory
// clobber, and the copies' completion by the counter.
template <int VM>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(VM) : "memory");
}

}  // namespace w4a4
