// Internal declarations shared by the HIP sources of libw4a4moe (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/w4a4_moe.h"

namespace w4a4 {

// ---------------------------------------------------------------- profiling
// Timing events of one launch while kernel timing is enabled (both null when
// it is off).
struct ProfEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfEvents prof_events(const char* name);

// Every kernel of the library is launched through here.  While timing is on,
// the dispatch itself timestamps the launch's start and stop events, which
// adds no packets to the queue (separate event records cost about 2% of a
// learner step).
template <typename... Params, typename... Args>
inline void launch_kernel(const char* name, void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t lds,
                          hipStream_t s, Args... args) {
  const ProfEvents ev = prof_events(name);
  hipExtLaunchKernelGGL(kernel, grid, block, lds, s, ev.start, ev.stop, 0u, args...);
}

// Records the HIP error of the last launch; returns false on failure.
bool launch_ok(const char* what);

// Compute units of the current device (queried once).
int device_cu_count();

// ------------------------------------------------------------ routing / quant
constexpr int kRouteChunk = 256;      // tokens per routing chunk (one workgroup)
constexpr int kMaxRouteK = 8;         // largest k the routing kernels take

// Routing validity of topk_idx [T, k] (k <= kMaxRouteK): err[0] = invalid
// entries (id outside [0, E) or repeated within a token), err[1] = smallest
// flat index of one (INT32_MAX when none).
bool launch_check_routing(const int32_t* topk_idx, int64_t T, int k, int E, int32_t* err, hipStream_t s);

size_t route_workspace_bytes(int64_t T, int E);

// Scratch of the allocation-free quantize+permute: a file-scope device array
// of kNoAllocScratchBytes per GPU; noalloc_scratch() returns the current
// device's address of it (looked up once per device; nullptr on failure).
constexpr size_t kNoAllocScratchBytes = size_t{1} << 20;
void* noalloc_scratch();

// Route, per-token amax, two-level NVFP4, scatter to k rows.
bool launch_quantize_permute(const uint16_t* x, int64_t T, int K, const int32_t* topk_idx,
                             int k, int E, int row_align, uint8_t* codes, uint8_t* scales,
                             float* outer, int32_t* offsets, int32_t* row_map, int32_t* src_row,
                             void* ws, hipStream_t s);

// Requantise: per-row NVFP4 of the bf16 rows of `a` ([rows_alloc, K]) for the rows
// [0, offsets[E]) (device bound); pad rows (src_row < 0) get zeros.
// Quantize + permute with one outer scale per group of group_rows consecutive
// input rows (group_rows = T: per tensor; the rows of one expert's weight:
// per expert).  amax: grouped_amax_bytes(T, group_rows) bytes of scratch.
// Only for K % 32 == 0, K <= 4096 (returns false otherwise).
size_t grouped_amax_bytes(int64_t T, int64_t group_rows);
bool launch_quantize_permute_grouped(const uint16_t* x, int64_t T, int K, const int32_t* topk_idx,
                                     int k, int E, int row_align, int64_t group_rows, uint8_t* codes,
                                     uint8_t* scales, float* outer, int32_t* offsets, int32_t* row_map,
                                     int32_t* src_row, void* ws, uint32_t* amax, hipStream_t s);

bool launch_requant(const uint16_t* a, int64_t rows_alloc, int K, const int32_t* offsets, int E,
                    const int32_t* src_row, uint8_t* codes, uint8_t* scales, float* outer,
                    hipStream_t s);

// MXFP4 recipe (E2M1 codes, one E8M0 scale per 32 along the row, no outer
// scale): the same routing and scatter, the MX row encoder.  K % 32 == 0,
// K <= 4096 (returns false otherwise).  topk_idx = NULL: identity (weights).
bool launch_quantize_permute_mx(const uint16_t* x, int64_t T, int K, const int32_t* topk_idx, int k, int E,
                                int row_align, uint8_t* codes, uint8_t* scales, int32_t* offsets,
                                int32_t* row_map, int32_t* src_row, void* ws, hipStream_t s);
bool launch_requant_mx(const uint16_t* a, int64_t rows_alloc, int K, const int32_t* offsets, int E,
                       uint8_t* codes, uint8_t* scales, hipStream_t s);

// --------------------------------------------------------------- grouped GEMMs
struct Fp4Operand {
  const uint8_t* codes;   // [rows, K/2]
  const uint8_t* scales;  // [rows, K/16]
  const float* outer;     // [rows]
};

// FC1 (SwiGLU fused into the epilogue): over expert groups, SwiGLU in the epilogue.
bool launch_fc1(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets, Fp4Operand x,
                Fp4Operand w1, uint16_t* h_out, uint16_t* a_out, float* dbg_f32, hipStream_t s);

// FC2 over expert groups.
bool launch_fc2(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets, Fp4Operand a,
                Fp4Operand w2, uint16_t* o_out, hipStream_t s);

// MXFP4 FC1 / FC2 (scaled FP4 MFMA; operands' outer pointers unused).  The
// reduction length (H for FC1, I for FC2) must be a multiple of 128.
bool launch_fc1_mx(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets, Fp4Operand x,
                   Fp4Operand w1, uint16_t* h_out, uint16_t* a_out, float* dbg_f32, hipStream_t s);
bool launch_fc2_mx(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets, Fp4Operand a,
                   Fp4Operand w2, uint16_t* o_out, hipStream_t s);

// MXFP8 backward pieces.  Quantiser (E4M3 + E8M0 per 32) along columns of
// `batch` [R, C] matrices into q [batch][C, pitch], s [batch][C, pitch/32]
// (row blocks [0, offsets[E]) when given, in whole tiles of 128 rows;
// C % 128 == 0, pitch % 128 == 0).
bool launch_q8_cols(const uint16_t* x, int64_t R, int C, int batch, const int32_t* offsets, int E,
                    int64_t pitch, uint8_t* q, uint8_t* s, const char* name, hipStream_t st);
// Both forms of one [R, C] matrix from one read (rows [0, offsets[E]), whole
// tiles of 128): along rows into q_r [R, C], s_r [R, C/32]; along columns into
// q_c [C, pitch], s_c [C, pitch/32].  h != NULL: the matrix is the SwiGLU
// backward dH [R, 2I] of x = dA [R, I] on the saved h (C = 2I), never stored.
bool launch_q8_dual(const uint16_t* x, const uint16_t* h, int64_t R, int C, int I, const int32_t* offsets, int E,
                    int64_t pitch, uint8_t* q_r, uint8_t* s_r, uint8_t* q_c, uint8_t* s_c, const char* name,
                    hipStream_t st);
// C = A B^T on the scaled FP8 MFMA, bf16 out.  dgrad: A [rows_alloc, K] grouped
// by offsets, B [E][N, K]; wgrad: per expert, A [M1, pitch] and B [N, pitch]
// over the columns [offsets[e], offsets[e+1]) (multiples of 128), out [E][M1, N].
bool launch_mx8_dgrad(int64_t rows_alloc, int K, int N, int E, const int32_t* offsets, const uint8_t* a,
                      const uint8_t* as, const uint8_t* b, const uint8_t* bs, uint16_t* out, const char* name,
                      hipStream_t s);
bool launch_mx8_wgrad(int M1, int N, int E, const int32_t* offsets, const uint8_t* a, const uint8_t* as,
                      const uint8_t* b, const uint8_t* bs, int64_t pitch, uint16_t* out, const char* name,
                      hipStream_t s);

// Dense linear layer y = x W^T (one group of T rows; offsets = {0, T}).
bool launch_linear_fwd(int64_t T, int K, int N, const int32_t* offsets, Fp4Operand x, Fp4Operand w,
                       uint16_t* y, hipStream_t s);

// Unpermute: y[t] = bf16(sum_j p[t,j] o[row_map[t,j]]).
bool launch_unpermute(int64_t T, int H, int k, const uint16_t* o, const int32_t* row_map,
                      const float* topk_w, uint16_t* y, hipStream_t s);

// Token-order scatters of the backward's row operands: for each token t and
// slot j, dO[row_map[t,j]] = bf16(p[t,j] dY[t]), resp. xp[row_map[t,j]] = x[t].
bool launch_scatter_dy(int64_t T, int H, int k, const uint16_t* dy, const int32_t* row_map,
                       const float* topk_w, uint16_t* dO, hipStream_t s);
bool launch_scatter_x(int64_t T, int H, int k, const uint16_t* x, const int32_t* row_map, uint16_t* xp,
                      hipStream_t s);
// Zeros in the pad rows (src_row < 0) of a [rows, H] bf16 buffer (dO or xp).
bool launch_zero_pad_rows(int64_t rows_alloc, int H, const int32_t* src_row, const int32_t* offsets,
                          int E, uint16_t* dst, hipStream_t s);

// FC2 dgrad with the SwiGLU backward fused: dA = bf16(dO_e W2[e]) then the SwiGLU backward -> dH.
bool launch_dgrad_fc2(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets,
                      const uint16_t* dO, const uint16_t* w2, const uint16_t* h, uint16_t* dH,
                      hipStream_t s);

// FC1 dgrad: dXp = bf16(dH_e W1[e]).
bool launch_dgrad_fc1(int64_t rows_alloc, int H, int I, int E, const int32_t* offsets,
                      const uint16_t* dH, const uint16_t* w1, uint16_t* dXp, hipStream_t s);

// Tile schedule of the two wgrad GEMMs (experts by row count, blocks of
// tiles dealt to the XCDs longest first, tile counters), computed on the
// device from the offsets; `sched` holds wgrad_schedule_ints(H, I, E) ints
// and is read and updated by the two wgrad launches that follow on the same
// stream (each launch consumes its counters: the schedule is written again
// before the next pair).  1 <= E <= 1024.
size_t wgrad_schedule_ints(int H, int I, int E);
bool launch_wgrad_schedule(int H, int I, int E, const int32_t* offsets, int32_t* sched, hipStream_t s);

// FC2 wgrad: dW2[e] = bf16(dO_e^T a_e).   FC1 wgrad: dW1[e] = bf16(dH_e^T x[src_row]).
bool launch_wgrad_fc2(int H, int I, int E, const uint16_t* dO, const uint16_t* a, uint16_t* dW2,
                      int32_t* sched, hipStream_t s);
bool launch_wgrad_fc1(int H, int I, int E, const uint16_t* dH, const uint16_t* xp, uint16_t* dW1,
                      int32_t* sched, hipStream_t s);

// Dense linear backward: dx = bf16(dy W) [T, K]; dw = bf16(dy^T x) [N, K]
// (the wgrad launch computes its tile schedule first, into `sched` of
// linear_wgrad_schedule_ints(K, N) ints).
size_t linear_wgrad_schedule_ints(int K, int N);
bool launch_linear_dgrad(int64_t T, int K, int N, const int32_t* offsets, const uint16_t* dy,
                         const uint16_t* w, uint16_t* dx, hipStream_t s);
bool launch_linear_wgrad(int64_t T, int K, int N, const int32_t* offsets, const uint16_t* dy,
                         const uint16_t* x, uint16_t* dw, int32_t* sched, hipStream_t s);

// dX gather-sum: dX[t] = bf16(sum_j dXp[row_map[t,j]]).
bool launch_gather_sum(int64_t T, int H, int k, const uint16_t* dXp, const int32_t* row_map,
                       uint16_t* dx, hipStream_t s);

}  // namespace w4a4
