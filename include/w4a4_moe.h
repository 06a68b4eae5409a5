/*
 * w4a4_moe.h -- C ABI of the MI355X (gfx950) per-token NVFP4 W4A4 MoE expert
 * path: quantize+permute, grouped expert forward, straight-through backward.
 *
 * Conventions for every call
 * --------------------------
 *  - Pointers are DEVICE pointers unless marked (host).  Tensors are dense and
 *    row-major with the shapes given.  bf16 tensors are passed as void*.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  The library never synchronises, never reads device data on the
 *    host and never allocates or frees memory: the caller owns every buffer,
 *    including the workspace, whose size w4a4_workspace_size() returns.
 *  - Host-checkable arguments are validated before anything is launched; an
 *    invalid call returns a negative status and launches nothing.  No C++
 *    exception crosses this interface.  w4a4_last_error() gives detail.
 *  - Routing validity (0 <= topk_idx < E, k distinct experts per token) is the
 *    caller's contract: the path's calls do not check it.  A caller that
 *    cannot vouch for its router checks a batch with w4a4_check_routing,
 *    which sets a device error word.
 *  - Shapes: H and I (and a quantised row length K) must be multiples of 32
 *    (16 for K), else W4A4_ERR_INVALID_ARG.  The kernels take H % 256 == 0
 *    and I % 128 == 0, else W4A4_ERR_UNSUPPORTED: the forward GEMMs' output
 *    tiles are 256 columns of H (FC2) and 128 SwiGLU features = 256 columns
 *    of h (FC1) with reduction stages of 64, the backward GEMMs' weight tiles
 *    256 columns with stages of 32, and none of them masks a partial tile
 *    along N or K.  Qwen3-30B-A3B's expert layer (H = 2048, I = 768) and
 *    every layer width that is a multiple of 256 / 128 fit.
 *  - Results are bitwise reproducible from run to run, and a token's results
 *    do not depend on the other tokens of the batch (per-token scale domain).
 *  - Calls are thread-safe; concurrent calls on different streams need
 *    different workspaces.
 *  - w4a4_expert_bwd runs two of its kernels (the wgrad tile schedule and the
 *    copy of x to the expert rows) on a second stream of the current device
 *    (one per device, created on first use, default priority), forked from
 *    `stream` and joined back into it before the call's last kernels: work
 *    enqueued on `stream` after the call sees every output.  Each host
 *    thread forks and joins with events of its own, so concurrent calls from
 *    several threads enqueue without a common lock; their side-stream
 *    kernels share that stream in enqueue order.
 *
 * Data formats (miniTE Technical Report, sections 2.2 and 5.1; rainbus review
 * of the miniTE paper, "prerequisites: the NVFP4 format" and method step 4):
 *  - E2M1 codes: 4 bits per element (sign in bit 3, magnitudes
 *    {0,.5,1,1.5,2,3,4,6}), two per byte, element 2j in the low nibble of
 *    byte j of the row.
 *  - E4M3FN block scales: one byte per 16 consecutive elements of a row,
 *    d = Q_E4M3(amax(block) / (6 g)).
 *  - FP32 outer scale g per row: g = RN_f32(max|row| / (6*448)).
 *    Activations: one per dispatched token row.  Weights: one per output row.
 *  - Rounding is round-to-nearest-even of the exact quotient, ties to the
 *    even code, E2M1 saturating at 6; a zero row or an underflowed block
 *    encodes zero codes that keep the sign bit of x.
 *
 * Expert-contiguous layout (AI summary, "Methodology in Plain English"; rainbus
 * review, method step 6): dispatched rows are grouped by expert, expert e
 * owning rows [expert_offsets[e], expert_offsets[e+1]), its tokens in
 * ascending token order, each group padded up to a multiple of row_align with
 * pad rows whose codes, scales and g are zero.  The offsets live on the device
 * only.  cap = w4a4_rows_capacity(T, k, E, row_align) bounds the padded row
 * count; rows in [expert_offsets[E], cap) are never written.
 */
#ifndef W4A4_MOE_H
#define W4A4_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A4_OK = 0,
  W4A4_ERR_INVALID_ARG = -1,  /* null / misaligned pointer, bad size or shape */
  W4A4_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels support   */
  W4A4_ERR_WORKSPACE = -3,    /* workspace pointer null or too small          */
  W4A4_ERR_LAUNCH = -4        /* a kernel launch failed (HIP error)           */
} w4a4_status;

/* Which call a workspace is sized for. */
typedef enum {
  W4A4_WS_QUANTIZE_PERMUTE = 0,
  W4A4_WS_FORWARD = 1,
  W4A4_WS_BACKWARD = 2,
  W4A4_WS_LINEAR_BACKWARD = 3,  /* w4a4_linear_bwd: H = K, I = N; T, E, k, row_align unused */
  W4A4_WS_QUANTIZE_PERMUTE_DOMAIN = 4,  /* w4a4_quantize_permute_domain, any group_rows; H = K */
  W4A4_WS_MX8_BACKWARD = 5              /* w4a4_mx8_expert_bwd */
} w4a4_workspace_kind;

/* Padded dispatched-row capacity: T*k + E*(row_align-1).  Returns -1 on bad
 * arguments.  Host only, no device work. */
int64_t w4a4_rows_capacity(int64_t T, int k, int E, int row_align);

/* Workspace bytes needed by one call of the given kind.  For
 * W4A4_WS_QUANTIZE_PERMUTE, K is the row length and I is ignored.  Returns 0
 * on bad arguments.  Host only. */
size_t w4a4_workspace_size(int kind, int64_t T, int H, int I, int E, int k, int row_align);

/*
 * w4a4_quantize_permute -- route the tokens to their experts and
 * write each token's two-level NVFP4 encoding into every one of its k
 * expert-contiguous destination rows.  The per-token amax is gathered in the
 * same pass that reads the token (no separate amax scan).
 *   Defined by: rainbus review, method steps 4 and 6 (per-token g, fused sort
 *   and amax, padding that carries the statistics); miniTE Technical Report,
 *   section 5.1 (block-scale equation); AI summary, "Methodology in Plain
 *   English" (packed codes, block scales and outer scales written straight
 *   into contiguous GEMM-consumed buffers, device-side expert offsets).
 *
 *   x          [T, K] bf16, K % 16 == 0, K >= 16.
 *   topk_idx   [T, k] int32 expert ids, or NULL for identity routing (then
 *              k must be 1, E must be 1 and row r is token r: this is how
 *              weight rows are quantised, one outer scale per row).
 *   row_align  1, 16, 32, 64 or 128.
 *   codes      [cap, K/2] uint8 out.   scales [cap, K/16] uint8 out.
 *   outer      [cap] float out.
 *   expert_offsets [E+1] int32 out.    row_map [T, k] int32 out (dispatched
 *              row of token t's j-th expert).  src_row [cap] int32 out (token
 *              of each row, -1 for pad rows).
 *   workspace  >= w4a4_workspace_size(W4A4_WS_QUANTIZE_PERMUTE, ...) bytes.
 */
w4a4_status w4a4_quantize_permute(
    const void* x, int64_t T, int K,
    const int32_t* topk_idx, int k, int E, int row_align,
    uint8_t* codes, uint8_t* scales, float* outer,
    int32_t* expert_offsets, int32_t* row_map, int32_t* src_row,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4a4_quantize_permute_noalloc -- w4a4_quantize_permute for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid device allocation): the same arguments, results and
 * kernels without the workspace.  Its routing scratch is a 1 MiB array held
 * by the library on each GPU it runs on (until the process ends); the call
 * itself allocates nothing.
 *   Limit: the routing scratch, 4 * (E * ceil(T / 256) + E) bytes rounded up
 *   to 256, must fit in 1 MiB (T <= 524,032 tokens at E = 128); larger
 *   calls return W4A4_ERR_UNSUPPORTED and launch nothing.  Identity routing
 *   (topk_idx = NULL) uses no scratch.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap on
 *   one GPU (different streams, or host threads on one stream without
 *   ordering) race and must not be issued.
 */
w4a4_status w4a4_quantize_permute_noalloc(
    const void* x, int64_t T, int K,
    const int32_t* topk_idx, int k, int E, int row_align,
    uint8_t* codes, uint8_t* scales, float* outer,
    int32_t* expert_offsets, int32_t* row_map, int32_t* src_row,
    void* stream);

/*
 * w4a4_check_routing -- checks a router's output before the path uses it.
 *   Defined by: rainbus review, prerequisites "MoE and grouped GEMM" (each
 *   token goes to k distinct experts of E; an expert may receive none).
 *
 *   topk_idx   [T, k] int32 expert ids (k <= 8); may be NULL when T == 0.
 *   error_word [2] int32 out (device, 8-byte aligned): error_word[0] = the
 *              number of invalid entries (an id outside [0, E), or an id
 *              equal to an earlier id of the same token), error_word[1] = the
 *              smallest flat index t*k + j of an invalid entry, INT32_MAX
 *              when there is none.  Both are written on `stream` (the caller
 *              reads them after the stream's work).
 *   Reads topk_idx only; every id is bounds-checked before it is used.
 */
w4a4_status w4a4_check_routing(const int32_t* topk_idx, int64_t T, int k, int E, int32_t* error_word,
                               void* stream);

/*
 * w4a4_quantize_permute_domain -- w4a4_quantize_permute with an outer-scale
 * domain wider than a row: one FP32 outer scale per group of `group_rows`
 * consecutive input rows (the last group may be shorter).
 *   Defined by: miniTE Technical Report, section 2.2 (the recipe decides
 *   whether the outer scale is per tensor, per expert or per row) and the
 *   section 4.3 table (miniTE CUTLASS: one outer scale per expert weight
 *   tensor); AI summary, "Methodology in Plain English" (the per-tensor
 *   reference breaks the context-swap invariance that per-token scales keep).
 *
 *   g = RN_f32(max |x| over the group / (6*448)); every row of the group is
 *   then encoded as in w4a4_quantize_permute against that g (block scales
 *   and codes per row), and every destination row stores the group's g in
 *   `outer`, so the GEMM entry points consume the result unchanged.
 *   group_rows = 1: per token (the same result as w4a4_quantize_permute);
 *   group_rows = T: per tensor; identity routing over the E*N rows of stacked
 *   expert weights [E, N, K] with group_rows = N: per expert weight tensor.
 *
 *   Arguments and outputs as w4a4_quantize_permute.  Requirements: also
 *   K % 32 == 0 and K <= 4096 (else W4A4_ERR_UNSUPPORTED); group_rows >= 1.
 *   workspace: w4a4_workspace_size(W4A4_WS_QUANTIZE_PERMUTE_DOMAIN, T, K,
 *   0, E, k, row_align) bytes (also for identity routing).  Adds one pass
 *   over x (the group maxima) before the encoding.
 */
w4a4_status w4a4_quantize_permute_domain(
    const void* x, int64_t T, int K,
    const int32_t* topk_idx, int k, int E, int row_align, int64_t group_rows,
    uint8_t* codes, uint8_t* scales, float* outer,
    int32_t* expert_offsets, int32_t* row_map, int32_t* src_row,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4a4_grouped_expert_fwd -- FC1 -> SwiGLU -> requantise -> FC2
 * over ragged, possibly empty expert groups, then the router-weighted
 * unpermute.
 *   Defined by: rainbus review, "core method" and method steps 5-6 (block-
 *   scaled accumulate U_e = MMA(X_e, W_e^T), then g_x g_w applied in FP32 in
 *   the epilogue, BF16 cast at the end; FC1 and FC2 with their own tile
 *   configurations); AI summary, "Methodology in Plain English" (each
 *   dispatched row its own outer scale, decoded operands never materialised).
 *
 *   FC1: h[r, n] = bf16( (g_x[r] * g_w1[e,n]) * sum_k (d c)_x (d c)_w1 )
 *        over n in [0, 2I); the first I rows of W1[e] are the SwiGLU gate,
 *        the next I the up projection.
 *   a   = bf16( silu(h_gate) * h_up ), FP32 arithmetic on the bf16 h.
 *   a is requantised per dispatched row exactly as the activations are.
 *   FC2: o[r, n] = bf16( (g_a[r] * g_w2[e,n]) * sum_i (d c)_a (d c)_w2 ).
 *   y[t] = bf16( sum_{j=0..k-1} topk_w[t,j] * o[row_map[t,j]] ), FP32 sum
 *        in ascending j.
 *
 *   x_codes/x_scales/x_outer, expert_offsets, row_map, src_row: as written by
 *              w4a4_quantize_permute with K = H.
 *   topk_w     [T, k] float router weights.
 *   w1_codes [E, 2I, H/2], w1_scales [E, 2I, H/16], w1_outer [E, 2I];
 *   w2_codes [E, H, I/2],  w2_scales [E, H, I/16],  w2_outer [E, H]
 *              (weights quantised per row, e.g. by w4a4_quantize_permute
 *              with identity routing on the [E*N, K] weight matrix).
 *   y          [T, H] bf16 out.
 *   save_h     optional [cap, 2I] bf16 out (FC1 output, for the backward).
 *   save_a     optional [cap, I] bf16 out (SwiGLU output, for the backward).
 *   dbg_fc1_f32 optional [cap, 2I] float out: FC1 epilogue values before the
 *              bf16 cast.
 *   dbg_a_codes [cap, I/2], dbg_a_scales [cap, I/16], dbg_a_outer [cap]:
 *              optional copies of the FC2-input quantisation (all three or
 *              none).
 *   Optional outputs are skipped when NULL.  Rows of pad rows hold zeros.
 *   Requirements: H % 256 == 0, I % 128 == 0 (else W4A4_ERR_UNSUPPORTED).
 */
w4a4_status w4a4_grouped_expert_fwd(
    int64_t T, int H, int I, int E, int k, int row_align,
    const uint8_t* x_codes, const uint8_t* x_scales, const float* x_outer,
    const int32_t* expert_offsets, const int32_t* row_map, const int32_t* src_row,
    const float* topk_w,
    const uint8_t* w1_codes, const uint8_t* w1_scales, const float* w1_outer,
    const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_outer,
    void* y,
    void* save_h, void* save_a,
    float* dbg_fc1_f32,
    uint8_t* dbg_a_codes, uint8_t* dbg_a_scales, float* dbg_a_outer,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4a4_expert_bwd -- the straight-through BF16 backward on the
 * saved high-precision operands (no backward quantisation).
 *   Defined by: AI summary, "Methodology in Plain English" (the quantisers'
 *   gradient taken as the identity, computed from the bf16 activations and
 *   weights the forward saved); miniTE
 *   Technical Report, section 4.3 (BF16 backward through the layer bypass on
 *   the saved original operands).
 *
 *   dO[r]  = bf16(topk_w[t,j] * dy[t])                     (r = row_map[t,j])
 *   dA     = bf16(dO_e W2[e]);        dW2[e] = bf16(dO_e^T a_e)
 *   dgate  = bf16(dA * up * s * (1 + gate * (1 - s))),  s = sigmoid(gate)
 *   dup    = bf16(dA * gate * s)      (gate, up = halves of the saved h)
 *   dXp    = bf16(dH_e W1[e]);        dW1[e] = bf16(dH_e^T x[src_row])
 *   dx[t]  = bf16(sum_j dXp[row_map[t,j]])
 *   All products accumulate in FP32.
 *
 *   dy, x      [T, H] bf16.   w1 [E, 2I, H] bf16.   w2 [E, H, I] bf16.
 *   save_h     [cap, 2I] bf16, save_a [cap, I] bf16 from the forward.
 *   topk_w, expert_offsets, row_map, src_row as in the forward.
 *   dx [T, H], dw1 [E, 2I, H], dw2 [E, H, I] bf16 out, fully overwritten
 *   (zeros for an expert with no rows).
 *   The workspace (W4A4_WS_BACKWARD) holds dO, dH, dXp, the expert-row copy
 *   of x and the wgrad tile schedule, all written by the call before use.
 *   Requirements: H % 256 == 0, I % 128 == 0 (else W4A4_ERR_UNSUPPORTED).
 */
w4a4_status w4a4_expert_bwd(
    int64_t T, int H, int I, int E, int k, int row_align,
    const void* dy, const void* x,
    const void* w1, const void* w2,
    const void* save_h, const void* save_a, const float* topk_w,
    const int32_t* expert_offsets, const int32_t* row_map, const int32_t* src_row,
    void* dx, void* dw1, void* dw2,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4a4_linear_fwd -- dense per-token NVFP4 linear layer, y = x W^T: the
 * MoE path's quantisation and GEMM with a single group and no permutation.
 *   Defined by: miniTE Technical Report, section 4.1 (ordinary linear layers
 *   beside the MoE GroupedLinear, behind the same quantisation interface) and
 *   section 4.3 (the nvfp4_per_token recipe: one activation outer scale per
 *   token, one weight outer scale per output row).
 *
 *   y[t, n] = bf16(g_x[t] * g_w[n] * sum_k (d c)_x[t, k] (d c)_w[n, k]),
 *   the sum and the outer factors in FP32.
 *
 *   x_codes [T, K/2], x_scales [T, K/16], x_outer [T], offsets [2] = {0, T}:
 *   the outputs of w4a4_quantize_permute(x, T, K, NULL, ...) (identity
 *   routing).  w_codes [N, K/2], w_scales [N, K/16], w_outer [N]: the same
 *   call on the weight W [N, K].  y [T, N] bf16 out (device).
 *   Requirements: K % 256 == 0, N % 256 == 0, K, N <= 8192 (else
 *   W4A4_ERR_UNSUPPORTED).  No workspace.
 */
w4a4_status w4a4_linear_fwd(
    int64_t T, int K, int N,
    const uint8_t* x_codes, const uint8_t* x_scales, const float* x_outer,
    const int32_t* offsets,
    const uint8_t* w_codes, const uint8_t* w_scales, const float* w_outer,
    void* y, void* stream);

/*
 * w4a4_linear_bwd -- straight-through BF16 backward of w4a4_linear_fwd on the
 * saved bf16 x and W (Technical Report, section 4.3: the layer bypass).
 *
 *   dx = bf16(dy W)        [T, K]      dw = bf16(dy^T x)      [N, K]
 *   both accumulated in FP32.
 *
 *   dy [T, N], x [T, K], w [N, K] bf16 (device); offsets: the {0, T} of the
 *   forward's quantisation (device).  dx [T, K] and dw [N, K] bf16 out
 *   (dw is zeros when T = 0).  workspace: w4a4_workspace_size(
 *   W4A4_WS_LINEAR_BACKWARD, 0, K, N, 1, 1, 1) bytes (the weight-gradient
 *   tile schedule, written by the call).  Requirements as the forward.
 */
w4a4_status w4a4_linear_bwd(
    int64_t T, int K, int N,
    const void* dy, const void* x, const void* w, const int32_t* offsets,
    void* dx, void* dw,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * MXFP4 recipe -- E2M1 codes with one E8M0 (power-of-two) scale per 32
 * consecutive elements of a row and no FP32 outer scale.  The miniTE
 * Technical Report's appendix D1 format sweep measures this "E2M1 + E8M0"
 * scale format beside NVFP4's E4M3 block scales (2-3 dB lower SNR); the
 * format itself is the OCP Microscaling (MX) v1.0 FP4 format (section 6.3:
 * shared exponent X = floor(log2(block amax)) - 2 clamped to [-127, 127],
 * scale byte X + 127, codes Q_E2M1(x / 2^X) round-to-nearest-even saturating
 * at 6; an all-zero block takes byte 0).  gfx950's scaled FP4 matrix
 * instructions take these operands as stored.  It is a different recipe
 * from NVFP4: its results are not those of the NVFP4 calls.
 *
 * w4a4_mx_quantize_permute -- w4a4_quantize_permute for the MXFP4 recipe.
 *   x [T, K] bf16 with K % 32 == 0 and K <= 4096.  codes [cap, K/2] uint8
 *   out, scales [cap, K/32] uint8 (E8M0) out; no outer scales.  Routing
 *   arguments, row_align, the maps, the workspace (same size as
 *   W4A4_WS_QUANTIZE_PERMUTE) and topk_idx = NULL (identity routing, for
 *   weight rows) as in w4a4_quantize_permute.  Pad rows get codes 0 and
 *   scale bytes 0.
 */
w4a4_status w4a4_mx_quantize_permute(
    const void* x, int64_t T, int K,
    const int32_t* topk_idx, int k, int E, int row_align,
    uint8_t* codes, uint8_t* scales,
    int32_t* expert_offsets, int32_t* row_map, int32_t* src_row,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4a4_mx_grouped_expert_fwd -- w4a4_grouped_expert_fwd for the MXFP4
 * recipe: FC1 = sum_k (c 2^X)_x (c 2^X)_w1 accumulated in FP32 on the scaled
 * FP4 MFMA, h = bf16(FC1), a = bf16(SwiGLU(h)), a requantised to MXFP4,
 * o = bf16(FC2), y[t] = bf16(sum_j p[t,j] o[row_map[t,j]]).  Same routing,
 * cast points and router-coefficient position as the NVFP4 forward.
 *   x_codes [cap, H/2], x_scales [cap, H/32] from w4a4_mx_quantize_permute.
 *   w1_codes [E, 2I, H/2], w1_scales [E, 2I, H/32]; w2_codes [E, H, I/2],
 *   w2_scales [E, H, I/32] (MXFP4 of the weight rows along the reduction
 *   axis: w4a4_mx_quantize_permute with identity routing).
 *   H % 256 == 0, I % 128 == 0.  y, save_h, save_a, dbg_fc1_f32 as in
 *   w4a4_grouped_expert_fwd; dbg_a_codes [cap, I/2] and dbg_a_scales
 *   [cap, I/32]: both or neither.  workspace >= w4a4_workspace_size(
 *   W4A4_WS_FORWARD, ...) bytes.  The saved h and a feed w4a4_expert_bwd
 *   unchanged (its straight-through backward does not see the recipe).
 */
w4a4_status w4a4_mx_grouped_expert_fwd(
    int64_t T, int H, int I, int E, int k, int row_align,
    const uint8_t* x_codes, const uint8_t* x_scales,
    const int32_t* expert_offsets, const int32_t* row_map, const int32_t* src_row,
    const float* topk_w,
    const uint8_t* w1_codes, const uint8_t* w1_scales,
    const uint8_t* w2_codes, const uint8_t* w2_scales,
    void* y, void* save_h, void* save_a, float* dbg_fc1_f32,
    uint8_t* dbg_a_codes, uint8_t* dbg_a_scales,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4a4_mx8_expert_bwd -- the straight-through backward with every GEMM
 * operand in MXFP8 instead of BF16: the variant the pages measure against
 * their BF16 backward (AI summary, key findings: BF16 backward about 1.21x
 * faster, gradient rel-L2 0.001663 against 0.037653 for MXFP8; Technical
 * Report, section 4.3: backward precision is set apart from the forward).
 * Each operand is quantised from the same bf16 tensors the BF16 backward
 * uses, along that GEMM's reduction axis (E4M3 elements, one E8M0 scale per
 * 32, OCP Microscaling v1.0 section 6.3: X = floor(log2 amax) - 8, elements
 * Q_E4M3(x / 2^X) round-to-nearest-even, saturating at 448):
 *   dA = bf16(Q_H(dO) Q_H(W2[e])), dW2[e] = bf16(Q_r(dO_e)^T Q_r(a_e)),
 *   dH = SwiGLU backward (bf16, as w4a4_expert_bwd),
 *   dXp = bf16(Q_2I(dH) Q_2I(W1[e])), dW1[e] = bf16(Q_r(dH_e)^T Q_r(xp_e)),
 *   dX[t] = bf16(sum_j dXp[row_map[t,j]]),
 * where Q_r quantises along the expert's dispatched rows; the GEMMs run on
 * gfx950's scaled FP8 MFMA with FP32 accumulation.  Arguments as in
 * w4a4_expert_bwd, with row_align == 128 (the row blocks of 32 never
 * straddle two experts and each expert's rows are whole K stages), I % 256
 * == 0, and a workspace of w4a4_workspace_size(W4A4_WS_MX8_BACKWARD, ...)
 * bytes.  Runs on `stream` alone.  dW of an empty expert is zeros.
 */
w4a4_status w4a4_mx8_expert_bwd(
    int64_t T, int H, int I, int E, int k, int row_align,
    const void* dy, const void* x, const void* w1, const void* w2,
    const void* save_h, const void* save_a, const float* topk_w,
    const int32_t* expert_offsets, const int32_t* row_map, const int32_t* src_row,
    void* dx, void* dw1, void* dw2,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4a4_mx8_quantize -- the MXFP8 operand quantiser of w4a4_mx8_expert_bwd as
 * a call of its own: both forms of a bf16 matrix from one read.
 *   x       [R, C] bf16, R % 128 == 0, C % 128 == 0.
 *   q_rows  [R, C] E4M3 bytes, s_rows [R, C/32] E8M0: blocks of 32 along rows.
 *   q_cols  [C, pitch] E4M3 bytes, s_cols [C, pitch/32] E8M0: column c of x
 *           in row c, blocks of 32 consecutive rows; pitch >= R, a multiple
 *           of 128; bytes [R, pitch) of each row are not written.
 * Format and rounding as in w4a4_mx8_expert_bwd (E4M3FN bytes, sign in bit 7,
 * -0 encodes as 0x80).
 */
w4a4_status w4a4_mx8_quantize(
    const void* x, int64_t R, int C,
    uint8_t* q_rows, uint8_t* s_rows, uint8_t* q_cols, uint8_t* s_cols, int64_t pitch,
    void* stream);

/* Static description of a status code. */
const char* w4a4_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* w4a4_last_error(void);

/*
 * Kernel timing (diagnostics; not a step of the method).  While enabled, every
 * kernel the library launches is bracketed by HIP events on its stream.
 * w4a4_profiler_report() synchronises those events and writes a JSON object
 * {"kernel": {"count": n, "total_ms": t}, ...} into `buf` (host, `len`
 * bytes, NUL-terminated); it returns the full length needed, or -1.
 * Enabling, disabling or resetting drops the recorded events.  Not
 * thread-safe; meant for single-threaded benchmarks.
 */
int w4a4_profiler_enable(int on);
int w4a4_profiler_report(char* buf, size_t len);

#ifdef __cplusplus
}
#endif
#endif /* W4A4_MOE_H */
