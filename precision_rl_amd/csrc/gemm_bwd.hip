// The straight-through BF16 backward GEMMs on gfx950 (AI summary,
// "Methodology in Plain English": straight-through estimator on the saved
// original BF16 operands; miniTE Technical Report, section 4.3: BF16 backward
// through the layer bypass, no backward quantisation).
//
//   dgrad (M = dispatched rows of expert e, ragged):
//     FC2 dgrad: dA  = dO_e . W2[e]     K = H,  N = I, epilogue = SwiGLU backward
//     FC1 dgrad: dXp = dH_e . W1[e]     K = 2I, N = H
//   wgrad (K = dispatched rows of expert e, ragged, possibly empty):
//     FC2 wgrad: dW2[e] = dO_e^T . a_e            M = H,  N = I
//     FC1 wgrad: dW1[e] = dH_e^T . xp_e           M = 2I, N = H   (xp = x gathered by row)
//
// MFMA 32x32x16 bf16, FP32 accumulation, waves of 64 x 128 (two per SIMD).
// The MFMAs take the N-side fragment as their first operand and the M-side
// fragment as their second (except on the K pieces of a split wgrad, whose
// FP32 sums leave straight from the registers), which computes the
// transposed 32 x 32 block: each lane then holds four consecutive columns of
// one output row per register group, so the epilogue converts them to bf16
// in pairs and writes them to LDS 8 bytes at a time (a quarter of the LDS
// writes of the other layout; the products and sums are the same, and so are
// the results, bit for bit).
// Operands go global -> LDS through the hardware's copies (no register
// staging) into a ring a few stages ahead of the MFMAs.  Tiles that are
// K-contiguous in HBM (dO, dH rows in the dgrad) arrive two stages at a time,
// so that each row's copy is one whole 128-byte line (half-line copies took
// as many L1-to-L2 requests for half the bytes), kept as rows of 128 B with
// their 16-byte chunks XOR-swizzled by (row / 2) % 8; tiles that are contiguous
// along M or N in HBM (the weights in the dgrad, both wgrad operands) are kept
// as [k][columns] rows, chunks swizzled by 4 (k % 4), and read with
// ds_read_b64_tr_b16, which hands each lane four consecutive k of its column.
// Both layouts make every read cycle conflict-free.
//
// dgrad: 128 x 256 tiles, 4 waves, two workgroups per CU (80 KB of LDS each),
// so that one workgroup's epilogue and waits overlap the other's MFMAs, and
// an expert's partial last M tile costs at most 128 padded rows.  K advances
// 32 per stage: B through a 3-deep ring, A in two buffers of two stages.
// The epilogue stages the bf16 tile in the (then idle) ring and writes it,
// and reads the saved h of the SwiGLU backward, with 16-byte row-contiguous
// accesses.
//
// wgrad: 256 x 256 tiles, 8 waves, one persistent workgroup per CU with a
// 3-deep ring of 32 KB stages (a fourth stage in flight measured no faster);
// at the end of a tile the copies of the next tile's first stages are issued
// before the epilogue, which moves the bf16 tile in two 128-row rounds
// through a 64 KB staging area with 16-byte stores.
// Both operands are streamed (K = the expert's rows), and the larger tile
// halves the copy traffic per flop.

#include <algorithm>

#include "gemm_common.h"
#include "internal.h"

namespace w4a4 {
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t join_bf16(short4_t lo, short4_t hi) {
  typedef short short8_t __attribute__((ext_vector_type(8)));
  const short8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ short4_t ds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(p));
}
__device__ __forceinline__ short4_t ds_read_tr(const __attribute__((address_space(3))) uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(p));
}

// ---- [k][256] tile: 32 k-rows of 512 B, 16-byte chunk c of k-row k at slot
// c ^ (4 (k & 3)).  Copy q (2 k-rows): lane i fills k-row 2 q + i / 32, slot
// i % 32.
__device__ __forceinline__ int kcol_copy_k(int q, int lane) { return 2 * q + (lane >> 5); }
__device__ __forceinline__ int kcol_src_chunk(int k, int lane) { return (lane & 31) ^ (4 * (k & 3)); }
// Byte offset of the 8-byte piece lane l reads with ds_read_tr for the 32 x 16
// MFMA operand block whose columns start at col0 (multiple of 32), for k block
// ks (16 k) and half r (k +0..3 or +4..7).
__device__ __forceinline__ int kcol_frag_offset(int col0, int ks, int r, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int k = ks * 16 + 8 * (g >> 1) + 4 * r + (j >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (j & 3);
  return k * 512 + (((col >> 3) ^ (4 * (k & 3))) * 16) + (col & 7) * 2;
}


// ======================================================================= dgrad
namespace dg {

constexpr int kThreads = 256;                       // 4 waves, 2 (M) x 2 (N)
constexpr int kBM = 128, kBN = 256;                 // workgroup tile
constexpr int kWM = 64, kWN = 128;                  // wave tile
constexpr int kMI = kWM / 32, kNI = kWN / 32;
constexpr int kBK = 32;
constexpr int kStages = 3;                          // B ring slots
constexpr int kAPairBytes = kBM * 2 * kBK * 2;      // 16 KB: A, two stages (128 B per row)
constexpr int kBBytes = kBN * kBK * 2;              // 16 KB: B, one stage
constexpr int kBOffset = 2 * kAPairBytes;           // two A pair buffers, then the B ring
constexpr int kRingBytes = kBOffset + kStages * kBBytes;   // 80 KB
constexpr int kACopies = kAPairBytes / 1024 / 4;    // 1 KB copies per wave per pair
constexpr int kBCopies = kBBytes / 1024 / 4;        // 1 KB copies per wave per stage
static_assert(kACopies == kBCopies, "the waits count 4 copies per issue");
// Epilogue staging of the bf16 tile: rows of 512 B padded to 528 B.  An
// 8-byte accumulator write covers rows r32 = 0..31 of one column group: with
// the 132-dword pitch, rows r and r + 16 share banks and nothing else does,
// the two cycles that 128 dwords over 64 banks take anyway.
constexpr int kOutPitch = kBN * 2 + 16;
// The tile map is published through B ring slot 2, which no copy fills
// before every wave has read it (its first copy follows the first barrier).
constexpr int kSlotOffset = kBOffset + 2 * kBBytes;
constexpr int kLdsBytes = kRingBytes;

static_assert(kBM * kOutPitch <= kRingBytes, "output staging must fit in the ring");
static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per CU must fit in LDS");



// ---- [k][COLS] tile: 32 k-rows of 2 COLS bytes, 16-byte chunk c of k-row k
// at slot c ^ (4 (k & 3)).  Copy q (1 KB): lane i fills k-row
// (64 / chunks) q + i / chunks, slot i % chunks, with chunks = COLS / 8.
template <int COLS>
struct KCol {
  static constexpr int kChunks = COLS / 8;     // 16-byte chunks per k-row
  static constexpr int kRowBytes = COLS * 2;
  static constexpr int kRowsPerCopy = 64 / kChunks;
  __device__ static int copy_k(int q, int lane) { return kRowsPerCopy * q + lane / kChunks; }
  __device__ static int src_chunk(int k, int lane) { return (lane % kChunks) ^ (4 * (k & 3)); }
  // Byte offset of the 8-byte piece lane l reads with ds_read_tr for the
  // 32 x 16 MFMA operand block whose columns start at col0 (multiple of 32),
  // for k block ks (16 k) and half r (k +0..3 or +4..7).
  __device__ static int frag_offset(int col0, int ks, int r, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int k = ks * 16 + 8 * (g >> 1) + 4 * r + (j >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (j & 3);
    return k * kRowBytes + (((col >> 3) ^ (4 * (k & 3))) * 16) + (col & 7) * 2;
  }
};

__device__ __forceinline__ void zero_acc(floatx16_t (&acc)[kMI][kNI]) {
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;
}

// Waits for stage s of nk (its A pair and B slot) in every wave.  The copies
// go out in the order A(0), A(1), B(0), B(1); after the first wait B(2);
// after the wait for stage kt+1, B(kt+3) and, for odd kt, A((kt+3)/2), four
// per wave each (pairs and stages that exist).  Loads return in order, so
// the wait allows the copies issued after stage s's last one: none for the
// last stage, eight for odd s >= 3, else four (checked against a
// simulation of this order for every nk < 200).
__device__ __forceinline__ int copies_after(int s, int nk) {
  return s == nk - 1 ? 0 : (s >= 3 && (s & 1)) ? 8 : 4;
}
__device__ __forceinline__ void wait_stage(int s, int nk) {
  const int n = copies_after(s, nk);
  if (n == 8) wait_vm_barrier<8>();
  else if (n == 4) wait_vm_barrier<4>();
  else wait_vm_barrier<0>();
}
// Same, and this wave's LDS reads have completed (lgkmcnt 0) before the barrier.
__device__ __forceinline__ void wait_stage_lds(int s, int nk) {
  const int n = copies_after(s, nk);
  if (n == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if (n == 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Writes the wave's accumulators as bf16 into the staging tile (row-major,
// kOutPitch bytes per row); the caller synchronises around it.  acc[mi][ni]
// register 4 g + j of lane (r32, hl) is row 32 mi + r32, column
// 32 ni + 8 g + 4 hl + j of the wave's block.
__device__ __forceinline__ void stage_out(uint8_t* out_lds, const floatx16_t (&acc)[kMI][kNI],
                                          int wrow, int wcol, int r32, int hl) {
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int row = wrow + mi * 32 + r32, col = wcol + ni * 32 + 8 * vg + 4 * hl;
        const u32x2_t v{pack_bf16x2(acc[mi][ni][4 * vg], acc[mi][ni][4 * vg + 1]),
                        pack_bf16x2(acc[mi][ni][4 * vg + 2], acc[mi][ni][4 * vg + 3])};
        *reinterpret_cast<u32x2_t*>(out_lds + row * kOutPitch + col * 2) = v;
      }
}

// All waves are past their last LDS read of the ring and every copy has
// landed (the last stage waits for vmcnt 0): the ring may be overwritten.
__device__ __forceinline__ void ring_idle_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ------------------------------------------------------------------ dgrad
enum class DgradMode { FC2_SWIGLU, FC1 };

struct DgradArgs {
  int64_t rows_alloc;
  int K, N, I, E;
  const int32_t* offsets;
  const uint16_t* g;   // [rows, K]   dO or dH
  const uint16_t* w;   // [E, K, N]   W2[e] ([H, I]) or W1[e] ([2I, H])
  const uint16_t* h;   // [rows, 2I]  saved FC1 output (FC2_SWIGLU)
  uint16_t* out;       // dH [rows, 2I] or dXp [rows, H]
};

using BCol = KCol<kBN>;

template <DgradMode MODE>
__global__ void __launch_bounds__(kThreads, 2)
dgrad_kernel(DgradArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wrow = (wave & 1) * kWM, wcol = (wave >> 1) * kWN;
  const int r32 = lane & 31, hl = lane >> 5;
  const int n_tiles = (args.N + kBN - 1) / kBN;
  // FC1 dgrad: an expert's 6 MiB weight slab exceeds the XCD's L2 and its
  // dH rows (3 MiB at 1024 rows) do not, so M tiles run fastest.
  TileCoord tc = grouped_m_tile<kBM, MODE == DgradMode::FC1>(args.offsets, args.E, n_tiles,
                                                             reinterpret_cast<int*>(lds + kSlotOffset));
  if (!tc.valid) return;
  const int n0 = tc.n_tile * kBN;
  const int a_rows = static_cast<int>(min<int64_t>(kBM, args.rows_alloc - tc.m0));   // >= 1

  // ---- copies.  A = rows of dO / dH (K-contiguous), fetched two stages at
  // a time so that every row's copy is a whole 128-byte line: pair p (k
  // 64 p .. 64 p + 63) into buffer p % 2, copy q filling rows 8 q .. 8 q + 7
  // (lane i: row 8 q + i / 8, slot i % 8, 16-byte chunk c of a row at slot
  // c ^ ((row / 2) % 8)); rows past the allocation are clamped (they only
  // feed accumulator rows that are never stored).  B = W[e] as [K][N], one
  // stage per ring slot: columns past N are clamped (never stored either).
  const uint8_t* a_base = reinterpret_cast<const uint8_t*>(args.g + tc.m0 * args.K);
  const uint8_t* b_base = reinterpret_cast<const uint8_t*>(args.w + static_cast<int64_t>(tc.e) * args.K * args.N);
  uint32_t a_off_src[kACopies], b_off_src[kBCopies];
#pragma unroll
  for (int c = 0; c < kACopies; ++c) {
    const int row = 8 * (kACopies * wave + c) + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    a_off_src[c] = static_cast<uint32_t>((min(row, a_rows - 1) * args.K + chunk * 8) * 2);
  }
#pragma unroll
  for (int c = 0; c < kBCopies; ++c) {
    const int k = BCol::copy_k(kBCopies * wave + c, lane);
    const int col = min(n0 + BCol::src_chunk(k, lane) * 8, args.N - 8);
    b_off_src[c] = static_cast<uint32_t>((k * args.N + col) * 2);
  }
  const int b_step = kBK * args.N * 2;   // bytes per stage
  const uint32_t lds0 = lds_addr(lds);
  auto issue_a = [&](int p) {
    const uint32_t st = lds0 + (p & 1) * kAPairBytes;
#pragma unroll
    for (int c = 0; c < kACopies; ++c)
      dma16_off(a_base + static_cast<int64_t>(p) * 128, a_off_src[c], st + (kACopies * wave + c) * 1024);
  };
  auto issue_b = [&](int kt) {
    const uint32_t st = lds0 + kBOffset + (kt % kStages) * kBBytes;
#pragma unroll
    for (int c = 0; c < kBCopies; ++c)
      dma16_off(b_base + static_cast<int64_t>(kt) * b_step, b_off_src[c], st + (kBCopies * wave + c) * 1024);
  };

  // ---- fragment addresses: a per-lane offset for the first 32-row (A) /
  // 32-column (B) block; the rest are immediates: +4096 per 32 A rows, +8192
  // per 16-k slice of B, +2048 for the second 4-k half of B.  A's offset
  // depends on the stage's half of its pair and on the slice.
  uint32_t a_lane[2][2], b_lane[kNI];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int row = wrow + r32;
      a_lane[h][ks] = row * 128 + (((4 * h + 2 * ks + hl) ^ ((row >> 1) & 7)) * 16);
    }
#pragma unroll
  for (int f = 0; f < kNI; ++f) b_lane[f] = BCol::frag_offset(wcol + f * 32, 0, 0, lane);
  floatx16_t acc[kMI][kNI];
  zero_acc(acc);
  struct Slice {
    bf16x8_t a[kMI], b[kNI];
  };
  // LDS byte addresses of this lane's fragments in one ring slot (one add
  // each per stage; everything else is an immediate offset of the reads).
  struct Bases {
    uint32_t a[2], b[kNI];
  };
  auto stage_bases = [&](int kt, Bases& bs) {
    uint32_t sa = lds0 + ((kt >> 1) & 1) * kAPairBytes;
    uint32_t sb = lds0 + kBOffset + (kt % kStages) * kBBytes;
    asm volatile("" : "+s"(sa), "+s"(sb));   // wave-uniform values: keep the compiler from re-deriving them per lane
    // the stage's half of its pair picks the lane offsets (a select, not an
    // indexed load: the four offsets stay in registers)
    const bool h = kt & 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint32_t lo = a_lane[0][ks], hi = a_lane[1][ks];
      asm volatile("" : "+v"(lo), "+v"(hi));
      bs.a[ks] = sa + (h ? hi : lo);
    }
#pragma unroll
    for (int f = 0; f < kNI; ++f) bs.b[f] = sb + b_lane[f];
  };
  auto load_frag = [&](const Bases& bs, int ks, Slice& sl, int f) {
    if (f < kMI) {
      sl.a[f] = *lds_ptr<bf16x8_t>(bs.a[ks] + f * 4096);
    } else {
      const uint32_t p = bs.b[f - kMI] + ks * 8192;
      sl.b[f - kMI] = join_bf16(ds_read_tr(lds_ptr<uint8_t>(p)), ds_read_tr(lds_ptr<uint8_t>(p + 2048)));
    }
  };
  auto load_slice = [&](const Bases& bs, int ks, Slice& sl) {
#pragma unroll
    for (int f = 0; f < kMI + kNI; ++f) load_frag(bs, ks, sl, f);
  };
  // The slice's MFMAs, with the next slice's fragments loaded one at a time
  // in the order the next slice uses them (A0 B0 after MFMA 0, B1..B3 after
  // MFMAs 1..3, A1 after MFMA 4): each read has seven MFMAs of cover, and the
  // LDS requests of the waves spread over the slice instead of arriving in
  // one burst (FC1 dgrad -1%, both wgrads -2%).
  auto mfma_slice = [&](const Slice& sl, const Bases& bs, int ks, Slice& nx, bool have_next, int pair_mid = -1) {
#pragma unroll
    for (int m = 0; m < kMI * kNI; ++m) {
      const int mi = m / kNI, ni = m % kNI;
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sl.b[ni], sl.a[mi], acc[mi][ni], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (have_next) {
        if (m == 0) {
          load_frag(bs, ks, nx, 0);
          load_frag(bs, ks, nx, kMI);
        } else if (m < kNI) {
          load_frag(bs, ks, nx, kMI + m);
        } else if (m == kNI) {
          load_frag(bs, ks, nx, 1);
        }
      }
      if (m == kNI && pair_mid >= 0) issue_a(pair_mid);   // apart from the stage's B copies
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = args.K / kBK;   // >= 1, even (K % 64 == 0)
  const int np = nk / 2;
  issue_a(0);
  if (np > 1) issue_a(1);
  issue_b(0);
  if (nk > 1) issue_b(1);
  // Pipeline (two A pair buffers, a 3-slot B ring, two 16-k slices per
  // stage): the wait for stage kt+1 sits between the two slices of stage kt,
  // so the first slice of kt+1 is read from LDS under the MFMAs of the
  // second slice of kt.  After that barrier every wave has finished reading
  // stage kt (lgkmcnt 0): the copy of stage kt+3 refills its B slot, and
  // after an odd kt (the pair's second stage) pair (kt+3)/2 refills its A
  // buffer, issued after the fifth MFMA of the next slice so that its copies
  // do not queue behind the B copies (FC1 / FC2 dgrad -2%).
  wait_stage(0, nk);
  if (2 < nk) issue_b(2);
  Slice s0, s1;
  Bases bc;
  stage_bases(0, bc);
  load_slice(bc, 0, s0);
  int kt = 0;
  for (; kt + 1 < nk; ++kt) {
    mfma_slice(s0, bc, 1, s1, true);
    wait_stage_lds(kt + 1, nk);
    if (kt + 3 < nk) issue_b(kt + 3);
    stage_bases(kt + 1, bc);
    mfma_slice(s1, bc, 0, s0, true, ((kt & 1) && (kt + 3) / 2 < np) ? (kt + 3) / 2 : -1);
  }
  mfma_slice(s0, bc, 1, s1, true);
  mfma_slice(s1, bc, 0, s0, false);

  const int rows = static_cast<int>(min<int64_t>(kBM, tc.m_end - tc.m0));
  constexpr int kChunksPerRow = kBN / 8;
  constexpr int kIters = kBM * kChunksPerRow / kThreads;   // 16-byte chunks per thread
  static_assert(kBM * kChunksPerRow % kThreads == 0, "whole chunks per thread");
  if constexpr (MODE == DgradMode::FC1) {
    ring_idle_barrier();
    stage_out(lds, acc, wrow, wcol, r32, hl);
    __syncthreads();
#pragma unroll 4
    for (int it = 0; it < kIters; ++it) {
      const int c = tid + it * kThreads;
      const int lrow = c / kChunksPerRow, n = n0 + (c % kChunksPerRow) * 8;
      if (lrow >= rows || n >= args.N) continue;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + lrow * kOutPitch + (n - n0) * 2);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(args.out + (tc.m0 + lrow) * args.N + n));
    }
  } else {
    // SwiGLU backward on bf16 dA, gate / up from the saved bf16 h, in two
    // batches of chunks: the first batch's h loads go out before the
    // accumulators are staged (their HBM latency runs under the staging),
    // the second's before the first batch is computed.
    const int I = args.I;
    constexpr int kBatch = kIters / 2;
    static_assert(kIters % 2 == 0, "two whole batches");
    u32x4_t hg0[kBatch], hu0[kBatch], hg1[kBatch], hu1[kBatch];
    auto load_h = [&](int b0, u32x4_t (&hg)[kBatch], u32x4_t (&hu)[kBatch]) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        // unconditional (clamped to the tile's last row and the last column
        // chunk, both valid) so that no lane mask splits the batch
        const int c = tid + (b0 + i) * kThreads;
        const int lrow = min(c / kChunksPerRow, rows - 1);
        const int n = min(n0 + (c % kChunksPerRow) * 8, args.N - 8);
        const uint16_t* hr = args.h + (tc.m0 + lrow) * (2 * I) + n;
        hg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(hr));
        hu[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(hr + I));
      }
    };
    auto swiglu_store = [&](int b0, const u32x4_t (&hg)[kBatch], const u32x4_t (&hu)[kBatch]) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int c = tid + (b0 + i) * kThreads;
        const int lrow = c / kChunksPerRow, n = n0 + (c % kChunksPerRow) * 8;
        if (lrow >= rows || n >= args.N) continue;
        const int64_t row = tc.m0 + lrow;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + lrow * kOutPitch + (n - n0) * 2);
        u32x4_t dg, du;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          float rg[2], ru[2];
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float da = bf16_to_f32(static_cast<uint16_t>(v[d] >> (16 * p)));
            const float gt = bf16_to_f32(static_cast<uint16_t>(hg[i][d] >> (16 * p)));
            const float up = bf16_to_f32(static_cast<uint16_t>(hu[i][d] >> (16 * p)));
            const float sg = sigmoid_fast(gt);
            rg[p] = da * up * sg * (1.0f + gt * (1.0f - sg));
            ru[p] = da * gt * sg;
          }
          dg[d] = pack_bf16x2(rg[0], rg[1]);
          du[d] = pack_bf16x2(ru[0], ru[1]);
        }
        __builtin_nontemporal_store(dg, reinterpret_cast<u32x4_t*>(args.out + row * (2 * I) + n));
        __builtin_nontemporal_store(du, reinterpret_cast<u32x4_t*>(args.out + row * (2 * I) + I + n));
      }
    };
    load_h(0, hg0, hu0);
    ring_idle_barrier();
    stage_out(lds, acc, wrow, wcol, r32, hl);
    __syncthreads();
    load_h(kBatch, hg1, hu1);
    swiglu_store(0, hg0, hu0);
    swiglu_store(kBatch, hg1, hu1);
  }
}

}  // namespace dg

// ======================================================================= wgrad
namespace wg {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;                       // 8 waves, 4 (M) x 2 (N)
constexpr int kBM = 256, kBN = 256;                 // workgroup tile
constexpr int kWM = 64, kWN = 128;                  // wave tile
constexpr int kMI = kWM / 32, kNI = kWN / 32;
constexpr int kBK = 32;
constexpr int kStages = 3;
constexpr int kAhead = kStages - 1;
constexpr int kABytes = kBM * kBK * 2;              // 16 KB: A, one stage
constexpr int kBBytes = kBN * kBK * 2;              // 16 KB: B, one stage
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kRingBytes = kStages * kStageBytes;   // 96 KB
constexpr int kACopies = kABytes / 1024 / 8;        // 1 KB copies per wave per stage
constexpr int kBCopies = kBBytes / 1024 / 8;
constexpr int kDmaPerStage = kACopies + kBCopies;
// Epilogue staging: 128 rows of 512 B, the 16-byte chunk c of row s at slot
// c ^ (s % 32), so that an 8-byte accumulator write (32 rows, one column
// group) spreads over all banks and a row's 16-byte reads stay a permutation
// of its chunks.
constexpr int kRoundRows = 128;
constexpr int kRowBytes = kBN * 2;
constexpr int kOutOffset = kRingBytes;
constexpr int kLdsBytes = kOutOffset + kRoundRows * kRowBytes;   // 160 KB: one workgroup per CU
// The next tile's table entry is published through the last ring slot, which
// holds no data between the end of a tile's last stage and the first copy of
// the next tile's stage kStages - 1.
constexpr int kSlotOffset = (kStages - 1) * kStageBytes;

static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");

__device__ __forceinline__ void zero_acc(floatx16_t (&acc)[kMI][kNI]) {
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;
}

// Waits for stage kt: later = stages issued after it (0 .. kAhead-1).
__device__ __forceinline__ void wait_stage(int later) {
  if (later >= 2) wait_vm_barrier<2 * kDmaPerStage>();
  else if (later == 1) wait_vm_barrier<kDmaPerStage>();
  else wait_vm_barrier<0>();
}
// Same, and this wave's LDS reads have completed (lgkmcnt 0) before the barrier.
__device__ __forceinline__ void wait_stage_lds(int later) {
  if (later >= 2) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * kDmaPerStage) : "memory");
  else if (later == 1) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kDmaPerStage) : "memory");
  else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// All waves are past their last LDS read of the ring and every copy has
// landed (the last stage waits for vmcnt 0): the ring may be overwritten.
__device__ __forceinline__ void ring_idle_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Byte offset in the staging area of column col of staging row s.
__device__ __forceinline__ int stage_offset(int s, int col) {
  return s * kRowBytes + (((col >> 3) ^ (s & 31)) * 16) + (col & 7) * 2;
}

// Round Q of the epilogue, first half: every wave writes its accumulator rows
// [32 Q, 32 Q + 32) (wave-local, MFMA row block Q) as bf16 into staging rows
// wm * 32 + 0..31, four consecutive columns per 8-byte write.
template <int Q>
__device__ __forceinline__ void stage_round(uint8_t* so, const floatx16_t (&acc)[kMI][kNI], int wm,
                                            int wcol, int r32, int hl) {
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) {
      const int sr = wm * 32 + r32, col = wcol + ni * 32 + 8 * vg + 4 * hl;
      const u32x2_t v{pack_bf16x2(acc[Q][ni][4 * vg], acc[Q][ni][4 * vg + 1]),
                      pack_bf16x2(acc[Q][ni][4 * vg + 2], acc[Q][ni][4 * vg + 3])};
      *reinterpret_cast<u32x2_t*>(so + stage_offset(sr, col)) = v;
    }
}

// Tile row held by staging row s in round q.
__device__ __forceinline__ int round_tile_row(int s, int q) { return (s >> 5) * kWM + 32 * q + (s & 31); }

// ------------------------------------------------------------------ wgrad
// Tile schedule of the two wgrad GEMMs, computed on the device from the
// expert offsets before they run (one workgroup of 1024 threads, E <= 1024).
// The tiles are listed expert by expert in descending order of the expert's
// row count (an expert's tiles N fastest), each costing its K stages plus a
// constant for the epilogue.  An expert's tiles form one chunk, or, when
// they are so costly that an XCD running them in rounds of its workgroups
// would take longer than the ideal share of one workgroup, chunks of at
// most one tile per workgroup of an XCD.  The chunks are dealt to the XCDs
// in list order, each to the XCD with the least work so far, and an XCD's
// workgroups take the tiles of its chunks in order from an atomic counter.
// An expert's operands stay in one XCD's L2 (two or more for the few large
// experts), and a skewed routing no longer leaves one XCD with most of the
// work.
constexpr int kTileCostEpilogue = 2;   // stage-equivalents of a tile's epilogue
constexpr int kMaxChunks = 2048;
// Per GEMM: the first entry of each XCD's tiles in the tile table, their
// count, and the XCDs' tile counters; then the tile table: per XCD, in
// order, {L, expert, first row, end row} for the tile at list position L.
constexpr int kSchedBegin = 0, kSchedCount = 8, kSchedCounters = 16, kSchedTable = 32;

struct SchedGemm {
  int tpe;       // tiles per expert
  int per_xcd;   // workgroups per XCD of the GEMM's grid
  int split;     // K splits per tile (1: none)
  int32_t* out;  // kSchedTable + 4 E tpe split ints (nullptr: no GEMM)
};

// Inclusive prefix sum over the workgroup (1024 threads); `total` gets the
// sum of all values.  s_wave: 16 entries of scratch.
__device__ int64_t block_scan(int64_t v, int64_t& total, int64_t* s_wave) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  if (lane == 63) s_wave[w] = v;
  __syncthreads();
  int64_t add = 0, all = 0;
  for (int i = 0; i < 16; ++i) {
    const int64_t x = s_wave[i];
    add += i < w ? x : 0;
    all += x;
  }
  __syncthreads();
  total = all;
  return v + add;
}

__global__ void __launch_bounds__(1024)
schedule_kernel(const int32_t* __restrict__ offsets, int E, SchedGemm g0, SchedGemm g1) {
  __shared__ int s_rows[1024];
  __shared__ int s_nk[1024];     // K stages of the expert at each sorted position
  __shared__ int s_e[1024], s_rb[1024], s_re[1024];
  __shared__ int s_base[1024];   // first chunk of the expert
  __shared__ int s_csize[1024];  // tiles per chunk of the expert
  __shared__ uint32_t s_csum[kMaxChunks];
  __shared__ uint16_t s_ctiles[kMaxChunks];
  __shared__ uint8_t s_xcd[kMaxChunks];
  __shared__ int s_off[kMaxChunks];
  __shared__ int s_begin[kXcds];
  __shared__ int64_t s_wave[16];
  const int t = threadIdx.x;
  const int n = t < E ? offsets[t + 1] - offsets[t] : -1;
  s_rows[t] = n;
  __syncthreads();
  if (t < E) {
    int rank = 0;
    for (int i = 0; i < E; ++i) {
      const int m = s_rows[i];
      rank += (m > n) || (m == n && i < t);
    }
    s_e[rank] = t;
    s_rb[rank] = offsets[t];
    s_re[rank] = offsets[t + 1];
    s_nk[rank] = (n + kBK - 1) / kBK;
  }
  __syncthreads();
  for (int g = 0; g < 2; ++g) {
    const SchedGemm p = g ? g1 : g0;
    if (p.out == nullptr) continue;   // (the same in every thread)
    // A tile split over K in p.split pieces: pieces of span stages each (the
    // last one shorter), each listed as a tile of its own.
    const int nkt = t < E ? s_nk[t] : 0;   // thread t: sorted position t
    const int span = (nkt + p.split - 1) / p.split;
    const int c = t < E ? span + kTileCostEpilogue : 0;
    int64_t cost_sum;
    block_scan(c, cost_sum, s_wave);
    const int64_t tpe = static_cast<int64_t>(p.tpe) * p.split, tiles = tpe * E, total = tpe * cost_sum;
    // split an expert whose tiles, run whole on one XCD, would take longer
    // than the ideal share of one workgroup
    const int64_t ideal = total / (static_cast<int64_t>(kXcds) * p.per_xcd);
    const int kc = static_cast<int>((tpe + p.per_xcd - 1) / p.per_xcd);
    int nc = t < E ? (kc > 1 && static_cast<int64_t>(c) * kc > ideal ? kc : 1) : 0;
    int64_t nch;
    int64_t incl = block_scan(nc, nch, s_wave);
    if (nch > kMaxChunks) {   // too many chunks: whole experts
      nc = t < E ? 1 : 0;
      incl = t + 1;
      nch = E;
    }
    const int csize = nc > 0 ? static_cast<int>((tpe + nc - 1) / nc) : 0;
    // chunk costs, scaled to fit 31 bits
    int shift = 0;
    while ((total >> shift) >= (int64_t{1} << 31)) ++shift;
    if (t < E) {
      const int base = static_cast<int>(incl) - nc;
      s_base[t] = base;
      s_csize[t] = csize;
      for (int i = 0; i < nc; ++i) {
        const int size = static_cast<int>(min<int64_t>(csize, tpe - static_cast<int64_t>(i) * csize));
        s_ctiles[base + i] = static_cast<uint16_t>(size);
        s_csum[base + i] = static_cast<uint32_t>((static_cast<int64_t>(size) * c) >> shift);
      }
    }
    __syncthreads();
    // Chunks, in list order, each to the XCD with the least work so far.
    // Wave 0 runs the loop in step (every value is the same in all lanes,
    // so it runs on the scalar unit); lane i keeps the result of chunk
    // c0 + i of the batch.
    if (t < kWave) {
      uint32_t load[kXcds], ntiles[kXcds];
#pragma unroll
      for (int x = 0; x < kXcds; ++x) load[x] = ntiles[x] = 0;
      for (int c0 = 0; c0 < nch; c0 += kWave) {
        const bool mine = c0 + t < nch;
        const uint32_t v_sum = mine ? s_csum[c0 + t] : 0u;
        const uint32_t v_tiles = mine ? s_ctiles[c0 + t] : 0u;
        uint32_t v_xcd = 0, v_off = 0;
        const int m = static_cast<int>(min<int64_t>(kWave, nch - c0));
        for (int i = 0; i < m; ++i) {
          const uint32_t sum = __builtin_amdgcn_readlane(v_sum, i);
          const uint32_t size = __builtin_amdgcn_readlane(v_tiles, i);
          int x = 0;
          uint32_t lo = load[0];
#pragma unroll
          for (int y = 1; y < kXcds; ++y)
            if (load[y] < lo) {
              lo = load[y];
              x = y;
            }
          uint32_t off = 0;
#pragma unroll
          for (int y = 0; y < kXcds; ++y)
            if (y == x) {
              off = ntiles[y];
              load[y] += sum;
              ntiles[y] += size;
            }
          if (t == i) {
            v_xcd = static_cast<uint32_t>(x);
            v_off = off;
          }
        }
        if (mine) {
          s_xcd[c0 + t] = static_cast<uint8_t>(v_xcd);
          s_off[c0 + t] = static_cast<int>(v_off);
        }
      }
      if (t == 0) {
        uint32_t acc = 0;
#pragma unroll
        for (int x = 0; x < kXcds; ++x) {
          s_begin[x] = static_cast<int>(acc);
          p.out[kSchedBegin + x] = static_cast<int32_t>(acc);
          p.out[kSchedCount + x] = static_cast<int32_t>(ntiles[x]);
          p.out[kSchedCounters + x] = 2 * p.per_xcd;   // tickets below it are dealt statically
          acc += ntiles[x];
        }
      }
    }
    __syncthreads();
    // (list entry L = piece li of expert j: tile li / split, K piece
    // li % split; stepped by 1024 without divisions)
    u32x4_t* table = reinterpret_cast<u32x4_t*>(p.out + kSchedTable);
    const int tp = static_cast<int>(tpe), jstep = 1024 / tp, lstep = 1024 % tp;
    int j = t / tp, li = t % tp;
    for (int L = t; L < static_cast<int>(tiles); L += 1024) {
      const int cs = s_csize[j], i = li / cs;
      const int ch = s_base[j] + i;
      const int at = s_begin[s_xcd[ch]] + s_off[ch] + (li - i * cs);
      const int tile = li / p.split, piece = li % p.split;
      const int rb = s_rb[j], rows = s_re[j] - rb;
      const int pspan = ((s_nk[j] + p.split - 1) / p.split) * kBK;
      table[at] = u32x4_t{static_cast<uint32_t>(tile | (piece << 24)), static_cast<uint32_t>(s_e[j]),
                          static_cast<uint32_t>(rb + min(rows, piece * pspan)),
                          static_cast<uint32_t>(rb + min(rows, (piece + 1) * pspan))};
      j += jstep;
      li += lstep;
      if (li >= tp) {
        li -= tp;
        ++j;
      }
    }
    __syncthreads();
  }
}

struct WgradArgs {
  int M, N, E;             // dW[e] is [M, N]
  const uint16_t* g;       // G [rows, M]:  A(m, r) = G[r][m]
  const uint16_t* s;       // S [rows, N]:  B(r, n) = S[r][n]
  uint16_t* out;           // [E, M, N]
  int32_t* sched;          // this GEMM's schedule (its tile counters are updated)
  float* partial;          // K split (E = 1): [split, M, N] FP32 sums of the pieces; else nullptr
};

struct WTile {
  int e, m0, n0, piece;
  int64_t r_begin, r_end;
  int nk;
};

// SPLIT: the tiles are K pieces whose FP32 sums go to args.partial.  Their
// MFMAs keep the M-side fragment first, so that a lane holds one column and
// the 32 lanes of a row write 128 contiguous bytes per store; the transposed
// order (four columns per lane, for the 8-byte bf16 staging writes) would
// break those rows into 32-byte pieces (measured 25% slower on split tiles).
template <bool SPLIT>
__global__ void __launch_bounds__(kThreads, 1)
wgrad_kernel(WgradArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3;
  const int wrow = wm * kWM, wcol = (wave >> 2) * kWN;
  const int r32 = lane & 31, hl = lane >> 5;
  const int n_tiles = (args.N + kBN - 1) / kBN;
  // Tiles come from this workgroup's XCD's part of the tile table.  The
  // first two tickets of each workgroup are dealt statically (blockIdx /
  // kXcds and that plus the workgroups per XCD; the counters start past
  // them), later ones come from the XCD's counter.  Only thread 0 draws
  // tickets and loads table entries, two tiles ahead: the ticket of the
  // tile after next is drawn as the current tile's copies start, and its
  // entry is loaded when the current tile ends, so that both have landed
  // long before they are used (when a tile ends, every copy has landed and
  // waiting costs nothing).
  const int xcd = static_cast<int>(blockIdx.x % kXcds);
  const int per_xcd = static_cast<int>(gridDim.x / kXcds);
  int32_t* counter = args.sched + kSchedCounters + xcd;
  const u32x4_t* table = reinterpret_cast<const u32x4_t*>(args.sched + kSchedTable);
  const u32x4_t none{static_cast<uint32_t>(-1), 0u, 0u, 0u};
  // A zero offset hidden in a vector register: with an address it sees as
  // uniform, the compiler combines a wave's atomics and reads the result at
  // once, which would wait for every copy in flight.
  uint32_t vzero = 0;
  asm volatile("" : "+v"(vzero));
  // thread 0: this XCD's part of the table; `done` once a ticket past its
  // end was seen (no more are drawn)
  int32_t begin = 0, count = 0;
  bool done = false;
  // Thread 0: {L, expert, first row, end row} of ticket q (L = -1: past the
  // end of the XCD's tiles).
  auto entry = [&](int32_t q) -> u32x4_t {
    if (q < count) return table[begin + q];
    done = true;
    return none;
  };
  // The next tile passes from thread 0 to all waves through the last ring slot
  // (written only while no wave reads the ring, read by all waves before the
  // slot is refilled).
  u32x4_t* slot = reinterpret_cast<u32x4_t*>(lds + kSlotOffset);
  auto tile = [&](WTile& t) -> bool {
    const u32x4_t p = *slot;
    const int L = static_cast<int>(__builtin_amdgcn_readfirstlane(p[0]));
    if (L < 0) return false;
    const int local = L & 0xFFFFFF;   // the tile of the expert; the K piece above
    t.piece = L >> 24;
    t.e = static_cast<int>(__builtin_amdgcn_readfirstlane(p[1]));
    t.m0 = (local / n_tiles) * kBM;
    t.n0 = (local % n_tiles) * kBN;
    t.r_begin = static_cast<int32_t>(__builtin_amdgcn_readfirstlane(p[2]));
    t.r_end = static_cast<int32_t>(__builtin_amdgcn_readfirstlane(p[3]));
    t.nk = static_cast<int>((t.r_end - t.r_begin + kBK - 1) / kBK);
    return true;
  };
  // Thread 0: ticket of the tile after next (not reset per tile: a write to
  // a register that an atomic or load may still fill waits for it, and with
  // it for every copy in flight) and the entry of the next tile.
  int32_t q_ahead = 0;
  u32x4_t e_next = none;
  auto draw = [&] {
    if (tid == 0 && !done) q_ahead = atomicAdd(counter + vzero, 1);
  };
  if (tid == 0) {
    begin = args.sched[kSchedBegin + xcd];
    count = args.sched[kSchedCount + xcd];
    const int32_t q0 = static_cast<int32_t>(blockIdx.x / kXcds);
    const u32x4_t e0 = entry(q0);
    e_next = entry(q0 + per_xcd);
    *slot = e0;
  }
  __syncthreads();
  WTile tc;
  if (!tile(tc)) return;
  draw();

  // ---- copies: both operands [k = row][256 columns]; rows past the expert's
  // end are re-read from its last row and zeroed in LDS; columns past N are
  // clamped (never stored)
  // A stage's copies are addressed as a wave-uniform base (the stage's first
  // row, computed on the scalar unit) plus 32-bit lane offsets fixed per
  // tile; only an expert's last, partial stage clamps its rows per lane.
  int kk[kACopies], a_col[kACopies], b_col[kBCopies];
  uint32_t a_off[kACopies], b_off[kBCopies];
  auto setup = [&](const WTile& t) {
#pragma unroll
    for (int c = 0; c < kACopies; ++c) {
      kk[c] = kcol_copy_k(kACopies * wave + c, lane);
      a_col[c] = t.m0 + kcol_src_chunk(kk[c], lane) * 8;
      b_col[c] = min(t.n0 + kcol_src_chunk(kk[c], lane) * 8, args.N - 8);
      a_off[c] = static_cast<uint32_t>((kk[c] * args.M + a_col[c]) * 2);
      b_off[c] = static_cast<uint32_t>((kk[c] * args.N + b_col[c]) * 2);
    }
  };
  static_assert(kACopies == kBCopies, "A and B copies share their k rows");
  const uint32_t lds0 = lds_addr(lds);
  // part: 1 = the A copies, 2 = the B copies (an expert's last, partial
  // stage issues all of them with part 2), 3 = both.
  auto issue = [&](const WTile& t, int kt, int part = 3) {
    const uint32_t st = lds0 + (kt % kStages) * kStageBytes;
    const int64_t r0 = t.r_begin + static_cast<int64_t>(kt) * kBK;
    const uint16_t* ga = args.g + r0 * args.M;
    const uint16_t* gb = args.s + r0 * args.N;
    if (r0 + kBK <= t.r_end) {
#pragma unroll
      for (int c = 0; c < kACopies; ++c)
        if (part & 1) dma16_off(ga, a_off[c], st + (kACopies * wave + c) * 1024);
#pragma unroll
      for (int c = 0; c < kBCopies; ++c)
        if (part & 2) dma16_off(gb, b_off[c], st + kABytes + (kBCopies * wave + c) * 1024);
    } else if (part & 2) {
      // rows past the expert's end re-read its last row (zeroed in LDS later)
      const int last = static_cast<int>(t.r_end - 1 - r0);
#pragma unroll
      for (int c = 0; c < kACopies; ++c) {
        const int kr = min(kk[c], last);
        dma16_off(ga, static_cast<uint32_t>((kr * args.M + a_col[c]) * 2), st + (kACopies * wave + c) * 1024);
        dma16_off(gb, static_cast<uint32_t>((kr * args.N + b_col[c]) * 2),
                  st + kABytes + (kBCopies * wave + c) * 1024);
      }
    }
  };

  // ---- fragment addresses within a stage: a per-lane offset for each
  // 32-column block (A: M, B: N); +8192 per 16-k slice and +2048 for the
  // second 4-k half are immediates of the reads.
  uint32_t a_lane[kMI], b_lane[kNI];
#pragma unroll
  for (int f = 0; f < kMI; ++f) a_lane[f] = kcol_frag_offset(wrow + f * 32, 0, 0, lane);
#pragma unroll
  for (int f = 0; f < kNI; ++f) b_lane[f] = kABytes + kcol_frag_offset(wcol + f * 32, 0, 0, lane);
  struct Slice {
    bf16x8_t a[kMI], b[kNI];
  };
  struct Bases {
    uint32_t a[kMI], b[kNI];
  };
  auto stage_bases = [&](int kt, Bases& bs) {
    uint32_t st = lds0 + (kt % kStages) * kStageBytes;
    asm volatile("" : "+s"(st));   // a wave-uniform value: keep the compiler from re-deriving it per lane
#pragma unroll
    for (int f = 0; f < kMI; ++f) bs.a[f] = st + a_lane[f];
#pragma unroll
    for (int f = 0; f < kNI; ++f) bs.b[f] = st + b_lane[f];
  };
  auto load_frag = [&](const Bases& bs, int ks, Slice& sl, int f) {
    const uint32_t p = (f < kMI ? bs.a[f] : bs.b[f - kMI]) + ks * 8192;
    const bf16x8_t v = join_bf16(ds_read_tr(lds_ptr<uint8_t>(p)), ds_read_tr(lds_ptr<uint8_t>(p + 2048)));
    if (f < kMI) sl.a[f] = v;
    else sl.b[f - kMI] = v;
  };
  auto load_slice = [&](const Bases& bs, int ks, Slice& sl) {
#pragma unroll
    for (int f = 0; f < kMI + kNI; ++f) load_frag(bs, ks, sl, f);
  };

  setup(tc);
  for (int s = 0; s < kAhead && s < tc.nk; ++s) issue(tc, s);
  uint8_t* so = lds + kOutOffset;
  for (;;) {
    floatx16_t acc[kMI][kNI];
    zero_acc(acc);
    // The slice's MFMAs, the next slice's fragments loaded one at a time in
    // the order the next slice uses them (as in the dgrad).
    auto mfma_slice = [&](const Slice& sl, const Bases& bs, int ks, Slice& nx, bool have_next,
                          int issue_kt = -1) {
#pragma unroll
      for (int m = 0; m < kMI * kNI; ++m) {
        const int mi = m / kNI, ni = m % kNI;
        if constexpr (SPLIT)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sl.a[mi], sl.b[ni], acc[mi][ni], 0, 0, 0);
        else
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sl.b[ni], sl.a[mi], acc[mi][ni], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (have_next) {
          if (m == 0) {
            load_frag(bs, ks, nx, 0);
            load_frag(bs, ks, nx, kMI);
          } else if (m < kNI) {
            load_frag(bs, ks, nx, kMI + m);
          } else if (m == kNI) {
            load_frag(bs, ks, nx, 1);
          }
        }
        if (m == 2 && issue_kt >= 0) issue(tc, issue_kt, 1);
        if (m == 6 && issue_kt >= 0) issue(tc, issue_kt, 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    const int nk = tc.nk;   // 0 for an empty expert: its dW tile is zero
    const int tail = static_cast<int>(tc.r_end - tc.r_begin - static_cast<int64_t>(nk - 1) * kBK);
    // Once every copy of the last stage has landed in all waves (vmcnt 0 and
    // a barrier): zero its k-rows past the expert's end in both operands,
    // then synchronise again.
    auto zero_tail = [&](int kt) {
      if (kt == nk - 1 && tail < kBK) {
        uint8_t* st = lds + (kt % kStages) * kStageBytes;
        for (int i = tid; i < (kBK - tail) * 64; i += kThreads) {
          const int op = i / ((kBK - tail) * 32), rem = i % ((kBK - tail) * 32);
          *reinterpret_cast<u32x4_t*>(st + op * kABytes + (tail + rem / 32) * 512 + (rem % 32) * 16) =
              u32x4_t{0u, 0u, 0u, 0u};
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    };
    // Pipeline (3-slot ring, two 16-k slices per stage): the wait for stage
    // kt+1 sits between the two slices of stage kt, so the first slice of
    // kt+1 is read from LDS under the MFMAs of the second slice of kt.  After
    // that barrier every wave has finished reading stage kt (lgkmcnt 0), so
    // the copy of stage kt+3 refills its slot; its A and B halves go out
    // after the third and seventh MFMAs of that second slice rather than
    // right at the barrier, where every wave's copies and first fragment
    // reads would arrive together (both wgrads -5%).
    if (nk > 0) {
      wait_stage(min(kAhead - 1, nk - 1));
      zero_tail(0);
      if (kAhead < nk) issue(tc, kAhead);
      Slice s0, s1;
      Bases bc;
      stage_bases(0, bc);
      load_slice(bc, 0, s0);
      int kt = 0;
      for (; kt + 1 < nk; ++kt) {
        mfma_slice(s0, bc, 1, s1, true);
        wait_stage_lds(min(kAhead - 1, nk - 2 - kt));
        zero_tail(kt + 1);
        stage_bases(kt + 1, bc);
        mfma_slice(s1, bc, 0, s0, true, kt + 1 + kAhead < nk ? kt + 1 + kAhead : -1);
      }
      mfma_slice(s0, bc, 1, s1, true);
      mfma_slice(s1, bc, 0, s0, false);
    }

    // ---- next tile's first stages, then the epilogue of this one
    ring_idle_barrier();
    if (tid == 0) {
      *slot = e_next;
      e_next = done ? none : entry(q_ahead);
    }
    __syncthreads();
    WTile tn;
    const bool more = tile(tn);
    if (more) {
      draw();
      setup(tn);
      for (int s = 0; s < kAhead && s < tn.nk; ++s) issue(tn, s);
    }
    if constexpr (SPLIT) {
      // a K piece: its FP32 sums, stored straight from the accumulators (a
      // row's 32 columns of an MFMA block are 128 contiguous bytes)
      float* po = args.partial + static_cast<int64_t>(tc.piece) * args.M * args.N;
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni) {
          const int n = tc.n0 + wcol + ni * 32 + r32;
          if (n >= args.N) continue;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int m = tc.m0 + acc_row(wrow, mi, v, hl);
            __builtin_nontemporal_store(acc[mi][ni][v], po + static_cast<int64_t>(m) * args.N + n);
          }
        }
    } else {
      uint16_t* out = args.out + static_cast<int64_t>(tc.e) * args.M * args.N;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q == 0) stage_round<0>(so, acc, wm, wcol, r32, hl);
        else stage_round<1>(so, acc, wm, wcol, r32, hl);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kRoundRows * 32 / kThreads; ++j) {
          const int c = tid + j * kThreads;
          const int s = c >> 5, n = tc.n0 + (c & 31) * 8;
          if (n >= args.N) continue;
          __builtin_nontemporal_store(
              *reinterpret_cast<const u32x4_t*>(so + stage_offset(s, n - tc.n0)),
              reinterpret_cast<u32x4_t*>(out + static_cast<int64_t>(tc.m0 + round_tile_row(s, q)) * args.N + n));
        }
        if (q < 1) __syncthreads();   // staging free for the next round
      }
    }
    if (!more) break;
    tc = tn;
  }
}

// out = bf16(sum_s partial[s]) over the K pieces, in piece order (a fixed
// order: the result is reproducible).  8 elements per thread.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ partial, int split, int64_t n, uint16_t* __restrict__ out) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  for (int sp = 0; sp < split; ++sp) {
    const float* p = partial + sp * n + i;
    const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += a[j];
      acc[4 + j] += b[j];
    }
  }
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = static_cast<uint32_t>(f32_to_bf16(acc[2 * j])) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * j + 1])) << 16);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(out + i));
}

}  // namespace wg

// Persistent grid: one workgroup per CU (a multiple of the XCD count), or
// fewer when there are fewer tiles.
unsigned persistent_grid(int64_t tiles) {
  const int64_t cap = std::max<int64_t>(kXcds, device_cu_count() / kXcds * kXcds);
  return xcd_grid(std::min<int64_t>(tiles, cap));
}

template <typename Kern>
hipError_t set_lds(Kern k, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <dg::DgradMode MODE>
bool launch_dgrad(const dg::DgradArgs& a, const char* name, hipStream_t s) {
  static const hipError_t attr = set_lds(&dg::dgrad_kernel<MODE>, dg::kLdsBytes);
  if (attr != hipSuccess) return launch_ok(name) && false;
  // The A operand arrives 64 k at a time: every caller's K (H, 2I, the dense
  // layer's N) is a multiple of 256, which the shape checks enforce.
  if (a.K % 64 != 0) return false;
  const int64_t tiles = grouped_m_tiles_bound(a.rows_alloc, a.E, dg::kBM) * ((a.N + dg::kBN - 1) / dg::kBN);
  if (tiles == 0) return true;
  launch_kernel(name, dg::dgrad_kernel<MODE>, dim3(xcd_grid(tiles)), dim3(dg::kThreads), dg::kLdsBytes, s, a);
  return launch_ok(name);
}

// Grid of a wgrad GEMM of E experts' [M, N] tiles: one workgroup per CU,
// at most one per tile.
struct WgradPlan {
  int64_t tiles;   // list entries: tiles times K pieces
  unsigned grid;
  int tpe, per_xcd, split;
};
WgradPlan wgrad_plan(int M, int N, int E, int split = 1) {
  WgradPlan p;
  p.tpe = (M / wg::kBM) * ((N + wg::kBN - 1) / wg::kBN);
  p.split = split;
  p.tiles = static_cast<int64_t>(E) * p.tpe * split;
  p.grid = persistent_grid(p.tiles);
  p.per_xcd = std::max(1, static_cast<int>(p.grid / kXcds));
  return p;
}
// K pieces per tile of a one-group wgrad whose tiles do not fill the chip:
// enough for one list entry per CU, at most 8.
int wgrad_split_max(int M, int N) {
  const int64_t tiles = static_cast<int64_t>(M / wg::kBM) * ((N + wg::kBN - 1) / wg::kBN);
  const int64_t cus = device_cu_count();
  if (tiles >= cus) return 1;
  return static_cast<int>(std::min<int64_t>(8, (cus + tiles - 1) / tiles));
}
size_t wgrad_sched_ints(const WgradPlan& p) { return wg::kSchedTable + 4 * static_cast<size_t>(p.tiles); }

bool launch_wgrad(const wg::WgradArgs& a, const char* name, hipStream_t s, int split = 1) {
  static const hipError_t attr = set_lds(&wg::wgrad_kernel<false>, wg::kLdsBytes);
  static const hipError_t attr_split = set_lds(&wg::wgrad_kernel<true>, wg::kLdsBytes);
  if (attr != hipSuccess || attr_split != hipSuccess) return launch_ok(name) && false;
  const WgradPlan p = wgrad_plan(a.M, a.N, a.E, split);
  if (p.tiles == 0) return true;
  if (a.partial != nullptr)
    launch_kernel(name, wg::wgrad_kernel<true>, dim3(p.grid), dim3(wg::kThreads), wg::kLdsBytes, s, a);
  else
    launch_kernel(name, wg::wgrad_kernel<false>, dim3(p.grid), dim3(wg::kThreads), wg::kLdsBytes, s, a);
  return launch_ok(name);
}

}  // namespace

bool launch_dgrad_fc2(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets,
                      const uint16_t* dO, const uint16_t* w2, const uint16_t* h, uint16_t* dH,
                      hipStream_t s) {
  dg::DgradArgs a{rows_alloc, H, I, I, E, offsets, dO, w2, h, dH};
  return launch_dgrad<dg::DgradMode::FC2_SWIGLU>(a, "gemm_dgrad_fc2", s);
}

bool launch_dgrad_fc1(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets,
                      const uint16_t* dH, const uint16_t* w1, uint16_t* dXp, hipStream_t s) {
  dg::DgradArgs a{rows_alloc, 2 * I, H, I, E, offsets, dH, w1, nullptr, dXp};
  return launch_dgrad<dg::DgradMode::FC1>(a, "gemm_dgrad_fc1", s);
}

size_t wgrad_schedule_ints(int H, int I, int E) {
  if (E < 1 || H < wg::kBM || I < wg::kBM / 2) return 2 * wg::kSchedTable;
  return wgrad_sched_ints(wgrad_plan(H, I, E)) + wgrad_sched_ints(wgrad_plan(2 * I, H, E));
}

bool launch_wgrad_schedule(int H, int I, int E, const int32_t* offsets, int32_t* sched, hipStream_t s) {
  if (E < 1 || E > 1024) return false;
  const WgradPlan p2 = wgrad_plan(H, I, E), p1 = wgrad_plan(2 * I, H, E);
  launch_kernel("wgrad_schedule", wg::schedule_kernel, dim3(1), dim3(1024), 0, s, offsets, E,
                wg::SchedGemm{p2.tpe, p2.per_xcd, 1, sched},
                wg::SchedGemm{p1.tpe, p1.per_xcd, 1, sched + wgrad_sched_ints(p2)});
  return launch_ok("wgrad_schedule");
}

bool launch_wgrad_fc2(int H, int I, int E, const uint16_t* dO, const uint16_t* a, uint16_t* dW2,
                      int32_t* sched, hipStream_t s) {
  wg::WgradArgs w{H, I, E, dO, a, dW2, sched, nullptr};
  return launch_wgrad(w, "gemm_wgrad_fc2", s);
}

bool launch_wgrad_fc1(int H, int I, int E, const uint16_t* dH, const uint16_t* xp, uint16_t* dW1,
                      int32_t* sched, hipStream_t s) {
  wg::WgradArgs w{2 * I, H, E, dH, xp, dW1, sched + wgrad_sched_ints(wgrad_plan(H, I, E)), nullptr};
  return launch_wgrad(w, "gemm_wgrad_fc1", s);
}

// Linear wgrad workspace: the schedule (room for the largest K split), then
// the FP32 sums of the K pieces when the tiles are split.
size_t linear_wgrad_schedule_ints(int K, int N) {
  const int split = wgrad_split_max(N, K);
  const size_t sched = (wgrad_sched_ints(wgrad_plan(N, K, 1, split)) + 63) / 64 * 64;
  return sched + (split > 1 ? static_cast<size_t>(split) * N * K : 0);
}

bool launch_linear_dgrad(int64_t T, int K, int N, const int32_t* offsets, const uint16_t* dy,
                         const uint16_t* w, uint16_t* dx, hipStream_t s) {
  dg::DgradArgs a{T, N, K, N / 2, 1, offsets, dy, w, nullptr, dx};
  return launch_dgrad<dg::DgradMode::FC1>(a, "gemm_linear_dgrad", s);
}

bool launch_linear_wgrad(int64_t T, int K, int N, const int32_t* offsets, const uint16_t* dy,
                         const uint16_t* x, uint16_t* dw, int32_t* sched, hipStream_t s) {
  // split K only while each piece keeps at least 32 stages
  const int64_t nk = (T + wg::kBK - 1) / wg::kBK;
  int split = wgrad_split_max(N, K);
  while (split > 1 && nk / split < 32) --split;
  const WgradPlan p = wgrad_plan(N, K, 1, split);
  launch_kernel("wgrad_schedule", wg::schedule_kernel, dim3(1), dim3(1024), 0, s, offsets, 1,
                wg::SchedGemm{p.tpe, p.per_xcd, split, sched}, wg::SchedGemm{0, 1, 1, nullptr});
  if (!launch_ok("wgrad_schedule")) return false;
  const size_t sched_ints = (wgrad_sched_ints(wgrad_plan(N, K, 1, wgrad_split_max(N, K))) + 63) / 64 * 64;
  float* partial = split > 1 ? reinterpret_cast<float*>(sched + sched_ints) : nullptr;
  wg::WgradArgs w{N, K, 1, dy, x, dw, sched, partial};
  if (!launch_wgrad(w, "gemm_linear_wgrad", s, split)) return false;
  if (split == 1) return true;
  const int64_t n = static_cast<int64_t>(N) * K;   // a multiple of 8 (K % 256 == 0)
  launch_kernel("splitk_reduce", wg::splitk_reduce_kernel, dim3(static_cast<unsigned>((n / 8 + 255) / 256)),
                dim3(256), 0, s, partial, split, n, dw);
  return launch_ok("splitk_reduce");
}

}  // namespace w4a4
