// Host side of the C ABI declared in include/w4a4_moe.h: argument validation,
// workspace carving and the launch sequence of each call.  No device-memory
// allocation, no synchronisation, no device reads on the host.  The backward
// runs two of its kernels on a second stream of the same device (default
// priority, created once per device; fork / join events per host thread),
// forked from and joined back into the caller's stream.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace w4a4 {
namespace {

thread_local std::string g_last_error;

w4a4_status fail(w4a4_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
w4a4_status fail(w4a4_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The side stream of the current device (one per device, created once under
// a lock) and this host thread's fork / join events for it (created on the
// thread's first backward on the device, held until the process ends).
// Calls from different threads record and wait on their own events, so their
// enqueues share no lock; their side-stream kernels run on the one stream in
// enqueue order, each behind the fork event of its own call.
struct SideStream {
  hipStream_t stream = nullptr;
  static constexpr int kEvents = 3;
  hipEvent_t fork[kEvents] = {}, join[kEvents] = {};
};
bool side_stream(SideStream& out) {
  static std::mutex mu;
  static std::map<int, hipStream_t> streams;
  thread_local std::map<int, SideStream> mine;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  auto it = mine.find(dev);
  if (it == mine.end()) {
    SideStream ss;
    {
      std::lock_guard<std::mutex> lock(mu);
      auto st = streams.find(dev);
      if (st == streams.end()) {
        hipStream_t created = nullptr;
        if (hipStreamCreateWithFlags(&created, hipStreamNonBlocking) != hipSuccess) return false;
        st = streams.emplace(dev, created).first;
      }
      ss.stream = st->second;
    }
    for (int i = 0; i < SideStream::kEvents; ++i)
      if (hipEventCreateWithFlags(&ss.fork[i], hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&ss.join[i], hipEventDisableTiming) != hipSuccess)
        return false;
    it = mine.emplace(dev, ss).first;
  }
  out = it->second;
  return true;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool valid_align(int a) { return a == 1 || a == 16 || a == 32 || a == 64 || a == 128; }

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 8;
constexpr int kMaxRowLen = 8192;

// ------------------------------------------------------------------ profiler
struct ProfEntry {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfEntry> g_prof_entries;
std::vector<hipEvent_t> g_prof_pool;
size_t g_prof_pool_used = 0;

hipEvent_t prof_event() {
  if (g_prof_pool_used == g_prof_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_prof_pool.push_back(e);
  }
  return g_prof_pool[g_prof_pool_used++];
}

void prof_clear() {
  g_prof_entries.clear();
  g_prof_pool_used = 0;
}

// Workspace layouts ---------------------------------------------------------
struct FwdWs {
  size_t a, a_codes, a_scales, a_outer, o, total;
};
FwdWs fwd_ws(int64_t cap, int H, int I) {
  FwdWs w;
  size_t off = 0;
  w.a = off; off += round_up(static_cast<size_t>(cap) * I * 2);
  w.a_codes = off; off += round_up(static_cast<size_t>(cap) * I / 2);
  w.a_scales = off; off += round_up(static_cast<size_t>(cap) * I / 16);
  w.a_outer = off; off += round_up(static_cast<size_t>(cap) * 4);
  w.o = off; off += round_up(static_cast<size_t>(cap) * H * 2);
  w.total = off;
  return w;
}
struct BwdWs {
  size_t sched, dO, dH, dXp, xp, total;
};
BwdWs bwd_ws(int64_t cap, int H, int I, int E) {
  BwdWs w;
  size_t off = 0;
  w.sched = off; off += round_up(wgrad_schedule_ints(H, I, E) * 4);
  w.dO = off; off += round_up(static_cast<size_t>(cap) * H * 2);
  w.dH = off; off += round_up(static_cast<size_t>(cap) * 2 * I * 2);
  w.dXp = off; off += round_up(static_cast<size_t>(cap) * H * 2);
  w.xp = off; off += round_up(static_cast<size_t>(cap) * H * 2);
  w.total = off;
  return w;
}

// MXFP8 backward: the BF16 backward's buffers plus the MXFP8 operands, each
// GEMM operand quantised along that GEMM's reduction axis; transposed
// operands (columns = dispatched rows) have P = roundup(cap, 128) columns.
struct Mx8Ws {
  size_t dO, xp, dA, dXp, dOq, dOqs, dOt, dOts, at, ats, w2t, w2ts, dHq, dHqs, dHt, dHts, w1t, w1ts, xpt,
      xpts, total;
  int64_t P;
};
Mx8Ws mx8_ws(int64_t cap, int H, int I, int E) {
  Mx8Ws w;
  w.P = (cap + 127) / 128 * 128;
  const size_t c = static_cast<size_t>(cap), P = static_cast<size_t>(w.P), e = static_cast<size_t>(E);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += round_up(bytes); return o; };
  w.dO = take(c * H * 2);
  w.xp = take(c * H * 2);
  w.dA = take(c * I * 2);
  w.dXp = take(c * H * 2);
  w.dOq = take(c * H);          w.dOqs = take(c * H / 32);
  w.dOt = take(H * P);          w.dOts = take(H * P / 32);
  w.at = take(I * P);           w.ats = take(I * P / 32);
  w.w2t = take(e * I * H);      w.w2ts = take(e * I * H / 32);
  w.dHq = take(c * 2 * I);      w.dHqs = take(c * 2 * I / 32);
  w.dHt = take(2 * I * P);      w.dHts = take(2 * I * P / 32);
  w.w1t = take(e * H * 2 * I);  w.w1ts = take(e * H * 2 * I / 32);
  w.xpt = take(H * P);          w.xpts = take(H * P / 32);
  w.total = off;
  return w;
}

w4a4_status check_moe_shape(int64_t T, int H, int I, int E, int k, int row_align) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0)
    return fail(W4A4_ERR_INVALID_ARG, "non-positive size (T=%lld H=%d I=%d E=%d k=%d)",
                static_cast<long long>(T), H, I, E, k);
  if (H % 32 || I % 32) return fail(W4A4_ERR_INVALID_ARG, "H and I must be multiples of 32");
  if (k > E) return fail(W4A4_ERR_INVALID_ARG, "k=%d > E=%d", k, E);
  if (!valid_align(row_align)) return fail(W4A4_ERR_INVALID_ARG, "row_align %d not in {1,16,32,64,128}", row_align);
  if (H % 256 || I % 128)
    return fail(W4A4_ERR_UNSUPPORTED, "kernels need H %% 256 == 0 and I %% 128 == 0 (H=%d I=%d)", H, I);
  if (H > kMaxRowLen || 2 * I > kMaxRowLen * 2 || I > kMaxRowLen)
    return fail(W4A4_ERR_UNSUPPORTED, "H and I must be <= %d", kMaxRowLen);
  if (E > kMaxExperts || k > kMaxTopK)
    return fail(W4A4_ERR_UNSUPPORTED, "E <= %d and k <= %d supported", kMaxExperts, kMaxTopK);
  if (T * static_cast<int64_t>(k) + static_cast<int64_t>(E) * (row_align - 1) > (int64_t{1} << 31) - 1)
    return fail(W4A4_ERR_UNSUPPORTED, "T*k + E*(row_align-1) rows exceed int32 row indices");
  return W4A4_OK;
}

#define REQUIRE_PTR(p)                                                                   \
  do {                                                                                   \
    if ((p) == nullptr) return fail(W4A4_ERR_INVALID_ARG, "%s is NULL", #p);             \
    if (!aligned16(p)) return fail(W4A4_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)
#define OPTIONAL_PTR(p)                                                                  \
  do {                                                                                   \
    if ((p) != nullptr && !aligned16(p))                                                 \
      return fail(W4A4_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p);                 \
  } while (0)

}  // namespace

ProfEvents prof_events(const char* name) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfEvents ev;
  if (!g_prof_on) return ev;
  ProfEntry e{name, prof_event(), prof_event()};
  if (!e.start || !e.stop) return ev;
  g_prof_entries.push_back(e);
  ev.start = e.start;
  ev.stop = e.stop;
  return ev;
}

int device_cu_count() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    return cus;
  }();
  return n;
}

bool launch_ok(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    fail(W4A4_ERR_LAUNCH, "launch of %s failed: %s", what, hipGetErrorString(e));
    return false;
  }
  return true;
}

}  // namespace w4a4

using namespace w4a4;

extern "C" {

int64_t w4a4_rows_capacity(int64_t T, int k, int E, int row_align) {
  if (T < 0 || k <= 0 || E <= 0 || !valid_align(row_align)) return -1;
  return T * k + static_cast<int64_t>(E) * (row_align - 1);
}

size_t w4a4_workspace_size(int kind, int64_t T, int H, int I, int E, int k, int row_align) {
  if (kind == W4A4_WS_LINEAR_BACKWARD) {   // H = K (in features), I = N (out features)
    if (H <= 0 || I <= 0 || H % 256 || I % 256) return 0;
    return round_up(linear_wgrad_schedule_ints(H, I) * 4);
  }
  const int64_t cap = w4a4_rows_capacity(T, k, E, row_align);
  if (cap < 0 || H <= 0) return 0;
  switch (kind) {
    case W4A4_WS_QUANTIZE_PERMUTE:
      return round_up(route_workspace_bytes(T, E));
    case W4A4_WS_QUANTIZE_PERMUTE_DOMAIN:   // any group_rows >= 1
      return round_up(route_workspace_bytes(T, E)) + round_up(grouped_amax_bytes(T, 1));
    case W4A4_WS_FORWARD:
      if (I <= 0) return 0;
      return fwd_ws(cap, H, I).total;
    case W4A4_WS_BACKWARD:
      if (I <= 0) return 0;
      return bwd_ws(cap, H, I, E).total;
    case W4A4_WS_MX8_BACKWARD:
      if (I <= 0) return 0;
      return mx8_ws(cap, H, I, E).total;
    default:
      return 0;
  }
}

namespace {
// Argument checks shared by the two quantize+permute entry points.
// `outer` is checked only when need_outer (the MXFP4 recipe has no outer scales).
w4a4_status check_quantize_permute(const void* x, int64_t T, int K, const int32_t* topk_idx, int k,
                                   int E, int row_align, uint8_t* codes, uint8_t* scales,
                                   float* outer, int32_t* expert_offsets, int32_t* row_map,
                                   int32_t* src_row, bool need_outer = true) {
  if (T < 0) return fail(W4A4_ERR_INVALID_ARG, "T < 0");
  if (K < 16 || K % 16) return fail(W4A4_ERR_INVALID_ARG, "K=%d must be a positive multiple of 16", K);
  if (K > kMaxRowLen) return fail(W4A4_ERR_UNSUPPORTED, "K=%d > %d", K, kMaxRowLen);
  if (!valid_align(row_align)) return fail(W4A4_ERR_INVALID_ARG, "row_align %d not in {1,16,32,64,128}", row_align);
  if (topk_idx == nullptr && T > 0) {
    if (k != 1 || E != 1 || row_align != 1)
      return fail(W4A4_ERR_INVALID_ARG, "identity routing needs k=1, E=1, row_align=1");
  } else {
    if (k <= 0 || E <= 0 || k > E) return fail(W4A4_ERR_INVALID_ARG, "bad k=%d / E=%d", k, E);
    if (k > kMaxTopK || E > kMaxExperts)
      return fail(W4A4_ERR_UNSUPPORTED, "E <= %d and k <= %d supported", kMaxExperts, kMaxTopK);
    if (!aligned16(topk_idx)) return fail(W4A4_ERR_INVALID_ARG, "topk_idx is not 16-byte aligned");
  }
  REQUIRE_PTR(expert_offsets);
  if (T > 0) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(codes);
    REQUIRE_PTR(scales);
    if (need_outer) REQUIRE_PTR(outer);
    REQUIRE_PTR(row_map);
    REQUIRE_PTR(src_row);
  }
  if (T * static_cast<int64_t>(k) + static_cast<int64_t>(E) * (row_align - 1) > (int64_t{1} << 31) - 1)
    return fail(W4A4_ERR_UNSUPPORTED, "T*k + E*(row_align-1) rows exceed int32 row indices");
  return W4A4_OK;
}
}  // namespace

w4a4_status w4a4_quantize_permute_noalloc(const void* x, int64_t T, int K, const int32_t* topk_idx, int k,
                                          int E, int row_align, uint8_t* codes, uint8_t* scales, float* outer,
                                          int32_t* expert_offsets, int32_t* row_map, int32_t* src_row,
                                          void* stream) {
  g_last_error.clear();
  w4a4_status st = check_quantize_permute(x, T, K, topk_idx, k, E, row_align, codes, scales, outer,
                                          expert_offsets, row_map, src_row);
  if (st != W4A4_OK) return st;
  const size_t need = topk_idx != nullptr ? round_up(route_workspace_bytes(T, E)) : 0;
  if (need > kNoAllocScratchBytes)
    return fail(W4A4_ERR_UNSUPPORTED,
                "routing scratch of %zu bytes exceeds the library's %zu-byte scratch "
                "(fewer tokens or experts, or w4a4_quantize_permute with a workspace)",
                need, kNoAllocScratchBytes);
  void* scratch_ptr = noalloc_scratch();
  if (scratch_ptr == nullptr) return fail(W4A4_ERR_LAUNCH, "the scratch address of the current device was not found");
  if (!launch_quantize_permute(static_cast<const uint16_t*>(x), T, K, topk_idx, k, E, row_align, codes, scales,
                               outer, expert_offsets, row_map, src_row, scratch_ptr,
                               static_cast<hipStream_t>(stream)))
    return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

w4a4_status w4a4_check_routing(const int32_t* topk_idx, int64_t T, int k, int E, int32_t* error_word,
                               void* stream) {
  g_last_error.clear();
  if (T < 0) return fail(W4A4_ERR_INVALID_ARG, "T < 0");
  if (k <= 0 || E <= 0) return fail(W4A4_ERR_INVALID_ARG, "bad k=%d / E=%d", k, E);
  if (k > kMaxTopK) return fail(W4A4_ERR_UNSUPPORTED, "k <= %d supported", kMaxTopK);
  if (T * static_cast<int64_t>(k) > (int64_t{1} << 31) - 1)
    return fail(W4A4_ERR_UNSUPPORTED, "T*k exceeds int32 indices");
  if (error_word == nullptr) return fail(W4A4_ERR_INVALID_ARG, "error_word is NULL");
  if (reinterpret_cast<uintptr_t>(error_word) % 8) return fail(W4A4_ERR_INVALID_ARG, "error_word is not 8-byte aligned");
  if (T > 0) REQUIRE_PTR(topk_idx);
  if (!launch_check_routing(topk_idx, T, k, E, error_word, static_cast<hipStream_t>(stream)))
    return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

w4a4_status w4a4_quantize_permute_domain(const void* x, int64_t T, int K, const int32_t* topk_idx,
                                         int k, int E, int row_align, int64_t group_rows,
                                         uint8_t* codes, uint8_t* scales, float* outer,
                                         int32_t* expert_offsets, int32_t* row_map, int32_t* src_row,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  w4a4_status st = check_quantize_permute(x, T, K, topk_idx, k, E, row_align, codes, scales, outer,
                                          expert_offsets, row_map, src_row);
  if (st != W4A4_OK) return st;
  if (group_rows < 1) return fail(W4A4_ERR_INVALID_ARG, "group_rows=%lld < 1", static_cast<long long>(group_rows));
  if (K % 32 || K > 4096)
    return fail(W4A4_ERR_UNSUPPORTED, "grouped outer scales need K %% 32 == 0 and K <= 4096 (K=%d)", K);
  const size_t route = round_up(route_workspace_bytes(T, topk_idx ? E : 1));
  const size_t need = route + round_up(grouped_amax_bytes(T, group_rows));
  if (T > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(W4A4_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  OPTIONAL_PTR(workspace);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (!launch_quantize_permute_grouped(static_cast<const uint16_t*>(x), T, K, topk_idx, k, E, row_align,
                                       group_rows, codes, scales, outer, expert_offsets, row_map, src_row,
                                       ws, T > 0 ? reinterpret_cast<uint32_t*>(ws + route) : nullptr,
                                       static_cast<hipStream_t>(stream)))
    return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

w4a4_status w4a4_quantize_permute(const void* x, int64_t T, int K, const int32_t* topk_idx, int k,
                                  int E, int row_align, uint8_t* codes, uint8_t* scales,
                                  float* outer, int32_t* expert_offsets, int32_t* row_map,
                                  int32_t* src_row, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  g_last_error.clear();
  w4a4_status st = check_quantize_permute(x, T, K, topk_idx, k, E, row_align, codes, scales, outer,
                                          expert_offsets, row_map, src_row);
  if (st != W4A4_OK) return st;
  const size_t need = w4a4_workspace_size(W4A4_WS_QUANTIZE_PERMUTE, T, K, 0, E, k, row_align);
  if (topk_idx != nullptr && T > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(W4A4_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  OPTIONAL_PTR(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!launch_quantize_permute(static_cast<const uint16_t*>(x), T, K, topk_idx, k, E, row_align,
                               codes, scales, outer, expert_offsets, row_map, src_row, workspace, s))
    return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

w4a4_status w4a4_grouped_expert_fwd(
    int64_t T, int H, int I, int E, int k, int row_align, const uint8_t* x_codes,
    const uint8_t* x_scales, const float* x_outer, const int32_t* expert_offsets,
    const int32_t* row_map, const int32_t* src_row, const float* topk_w, const uint8_t* w1_codes,
    const uint8_t* w1_scales, const float* w1_outer, const uint8_t* w2_codes,
    const uint8_t* w2_scales, const float* w2_outer, void* y, void* save_h, void* save_a,
    float* dbg_fc1_f32, uint8_t* dbg_a_codes, uint8_t* dbg_a_scales, float* dbg_a_outer,
    void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  w4a4_status st = check_moe_shape(T, H, I, E, k, row_align);
  if (st != W4A4_OK) return st;
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(w1_codes); REQUIRE_PTR(w1_scales); REQUIRE_PTR(w1_outer);
  REQUIRE_PTR(w2_codes); REQUIRE_PTR(w2_scales); REQUIRE_PTR(w2_outer);
  if (T > 0) {
    REQUIRE_PTR(x_codes); REQUIRE_PTR(x_scales); REQUIRE_PTR(x_outer);
    REQUIRE_PTR(row_map); REQUIRE_PTR(src_row); REQUIRE_PTR(topk_w); REQUIRE_PTR(y);
  }
  OPTIONAL_PTR(save_h); OPTIONAL_PTR(save_a); OPTIONAL_PTR(dbg_fc1_f32);
  OPTIONAL_PTR(dbg_a_codes); OPTIONAL_PTR(dbg_a_scales); OPTIONAL_PTR(dbg_a_outer);
  const int nd = (dbg_a_codes != nullptr) + (dbg_a_scales != nullptr) + (dbg_a_outer != nullptr);
  if (nd != 0 && nd != 3)
    return fail(W4A4_ERR_INVALID_ARG, "dbg_a_codes, dbg_a_scales, dbg_a_outer: all or none");
  const int64_t cap = w4a4_rows_capacity(T, k, E, row_align);
  const FwdWs L = fwd_ws(cap, H, I);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(W4A4_ERR_WORKSPACE, "workspace needs %zu bytes", L.total);
  OPTIONAL_PTR(workspace);
  if (cap == 0) return W4A4_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* a_buf = save_a ? static_cast<uint16_t*>(save_a) : reinterpret_cast<uint16_t*>(ws + L.a);
  uint8_t* a_codes = nd ? dbg_a_codes : ws + L.a_codes;
  uint8_t* a_scales = nd ? dbg_a_scales : ws + L.a_scales;
  float* a_outer = nd ? dbg_a_outer : reinterpret_cast<float*>(ws + L.a_outer);
  uint16_t* o_buf = reinterpret_cast<uint16_t*>(ws + L.o);

  if (!launch_fc1(cap, H, I, E, expert_offsets, Fp4Operand{x_codes, x_scales, x_outer},
                  Fp4Operand{w1_codes, w1_scales, w1_outer}, static_cast<uint16_t*>(save_h), a_buf,
                  dbg_fc1_f32, s))
    return W4A4_ERR_LAUNCH;
  if (!launch_requant(a_buf, cap, I, expert_offsets, E, src_row, a_codes, a_scales, a_outer, s))
    return W4A4_ERR_LAUNCH;
  if (!launch_fc2(cap, H, I, E, expert_offsets, Fp4Operand{a_codes, a_scales, a_outer},
                  Fp4Operand{w2_codes, w2_scales, w2_outer}, o_buf, s))
    return W4A4_ERR_LAUNCH;
  if (!launch_unpermute(T, H, k, o_buf, row_map, topk_w, static_cast<uint16_t*>(y), s))
    return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

w4a4_status w4a4_expert_bwd(int64_t T, int H, int I, int E, int k, int row_align, const void* dy,
                            const void* x, const void* w1, const void* w2, const void* save_h,
                            const void* save_a, const float* topk_w,
                            const int32_t* expert_offsets, const int32_t* row_map,
                            const int32_t* src_row, void* dx, void* dw1, void* dw2,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  w4a4_status st = check_moe_shape(T, H, I, E, k, row_align);
  if (st != W4A4_OK) return st;
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(w1); REQUIRE_PTR(w2); REQUIRE_PTR(dw1); REQUIRE_PTR(dw2);
  if (T > 0) {
    REQUIRE_PTR(dy); REQUIRE_PTR(x); REQUIRE_PTR(save_h); REQUIRE_PTR(save_a);
    REQUIRE_PTR(topk_w); REQUIRE_PTR(row_map); REQUIRE_PTR(src_row); REQUIRE_PTR(dx);
  }
  const int64_t cap = w4a4_rows_capacity(T, k, E, row_align);
  const BwdWs L = bwd_ws(cap, H, I, E);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(W4A4_ERR_WORKSPACE, "workspace needs %zu bytes", L.total);
  OPTIONAL_PTR(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* sched = reinterpret_cast<int32_t*>(ws + L.sched);
  uint16_t* dO = reinterpret_cast<uint16_t*>(ws + L.dO);
  uint16_t* dH = reinterpret_cast<uint16_t*>(ws + L.dH);
  uint16_t* dXp = reinterpret_cast<uint16_t*>(ws + L.dXp);
  uint16_t* xp = reinterpret_cast<uint16_t*>(ws + L.xp);
  const uint16_t* h = static_cast<const uint16_t*>(save_h);
  const uint16_t* a = static_cast<const uint16_t*>(save_a);
  const uint16_t* W1 = static_cast<const uint16_t*>(w1);
  const uint16_t* W2 = static_cast<const uint16_t*>(w2);

  // Side stream: the copy of x to the expert rows (xp, read only by the last
  // GEMM) runs beside the FC2 wgrad and the FC1 dgrad: HBM-bound with few
  // registers and no LDS, beside MFMA-bound GEMMs.  The caller's stream
  // waits for it before the FC1 wgrad.
  SideStream side;
  if (!side_stream(side)) return fail(W4A4_ERR_LAUNCH, "side stream / events could not be created");
  auto fork = [&](int i) {
    return hipEventRecord(side.fork[i], s) == hipSuccess &&
           hipStreamWaitEvent(side.stream, side.fork[i], 0) == hipSuccess;
  };
  auto join = [&](int i) {
    return hipEventRecord(side.join[i], side.stream) == hipSuccess &&
           hipStreamWaitEvent(s, side.join[i], 0) == hipSuccess;
  };
  // The wgrad tile schedule (one workgroup) is computed on the side stream
  // beside the dY scatter and the FC2 dgrad; the FC2 wgrad waits for it.
  if (!fork(2)) return fail(W4A4_ERR_LAUNCH, "fork to the side stream failed");
  if (!launch_wgrad_schedule(H, I, E, expert_offsets, sched, side.stream)) return W4A4_ERR_LAUNCH;
  if (hipEventRecord(side.join[2], side.stream) != hipSuccess)
    return fail(W4A4_ERR_LAUNCH, "event record on the side stream failed");
  if (!launch_scatter_dy(T, H, k, static_cast<const uint16_t*>(dy), row_map, topk_w, dO, s))
    return W4A4_ERR_LAUNCH;
  if (row_align > 1 && !launch_zero_pad_rows(cap, H, src_row, expert_offsets, E, dO, s))
    return W4A4_ERR_LAUNCH;
  if (cap > 0 && !launch_dgrad_fc2(cap, H, I, E, expert_offsets, dO, W2, h, dH, s)) return W4A4_ERR_LAUNCH;
  // (forked after the FC2 dgrad: beside the persistent FC2 wgrad the copy
  // costs the GEMM little; beside the FC2 dgrad it took that kernel's slots.
  // The wait for the schedule comes before the fork, so that the FC2 wgrad
  // is dispatched first and takes its CUs before the copy does.)
  if (hipStreamWaitEvent(s, side.join[2], 0) != hipSuccess)
    return fail(W4A4_ERR_LAUNCH, "wait for the side stream failed");
  if (!fork(0)) return fail(W4A4_ERR_LAUNCH, "fork to the side stream failed");
  if (!launch_scatter_x(T, H, k, static_cast<const uint16_t*>(x), row_map, xp, side.stream))
    return W4A4_ERR_LAUNCH;
  if (row_align > 1 && !launch_zero_pad_rows(cap, H, src_row, expert_offsets, E, xp, side.stream))
    return W4A4_ERR_LAUNCH;
  if (!launch_wgrad_fc2(H, I, E, dO, a, static_cast<uint16_t*>(dw2), sched, s))
    return W4A4_ERR_LAUNCH;
  if (cap > 0 && !launch_dgrad_fc1(cap, H, I, E, expert_offsets, dH, W1, dXp, s))
    return W4A4_ERR_LAUNCH;
  // The dX gather-sum runs after the FC1 wgrad on the caller's stream: beside
  // it on the second stream it saved nothing (the step took as long) and
  // blurred the GEMM's own time.
  if (!join(0)) return fail(W4A4_ERR_LAUNCH, "join from the side stream failed");
  if (!launch_wgrad_fc1(H, I, E, dH, xp, static_cast<uint16_t*>(dw1), sched, s))
    return W4A4_ERR_LAUNCH;
  if (!launch_gather_sum(T, H, k, dXp, row_map, static_cast<uint16_t*>(dx), s))
    return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

namespace {
w4a4_status check_linear_shape(int64_t T, int K, int N) {
  if (T < 0 || K <= 0 || N <= 0)
    return fail(W4A4_ERR_INVALID_ARG, "non-positive size (T=%lld K=%d N=%d)", static_cast<long long>(T), K, N);
  if (K % 256 || N % 256)
    return fail(W4A4_ERR_UNSUPPORTED, "kernels need K %% 256 == 0 and N %% 256 == 0 (K=%d N=%d)", K, N);
  if (K > kMaxRowLen || N > kMaxRowLen)
    return fail(W4A4_ERR_UNSUPPORTED, "K and N must be <= %d", kMaxRowLen);
  if (T > (int64_t{1} << 31) - 1) return fail(W4A4_ERR_UNSUPPORTED, "T must be < 2^31");
  return W4A4_OK;
}
}  // namespace

w4a4_status w4a4_linear_fwd(int64_t T, int K, int N, const uint8_t* x_codes, const uint8_t* x_scales,
                            const float* x_outer, const int32_t* offsets, const uint8_t* w_codes,
                            const uint8_t* w_scales, const float* w_outer, void* y, void* stream) {
  g_last_error.clear();
  w4a4_status st = check_linear_shape(T, K, N);
  if (st != W4A4_OK) return st;
  REQUIRE_PTR(w_codes); REQUIRE_PTR(w_scales); REQUIRE_PTR(w_outer);
  if (T == 0) return W4A4_OK;
  REQUIRE_PTR(x_codes); REQUIRE_PTR(x_scales); REQUIRE_PTR(x_outer); REQUIRE_PTR(offsets);
  REQUIRE_PTR(y);
  if (!launch_linear_fwd(T, K, N, offsets, Fp4Operand{x_codes, x_scales, x_outer},
                         Fp4Operand{w_codes, w_scales, w_outer}, static_cast<uint16_t*>(y),
                         static_cast<hipStream_t>(stream)))
    return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

w4a4_status w4a4_linear_bwd(int64_t T, int K, int N, const void* dy, const void* x, const void* w,
                            const int32_t* offsets, void* dx, void* dw, void* workspace,
                            size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  w4a4_status st = check_linear_shape(T, K, N);
  if (st != W4A4_OK) return st;
  REQUIRE_PTR(w); REQUIRE_PTR(dw); REQUIRE_PTR(offsets);
  if (T > 0) {
    REQUIRE_PTR(dy); REQUIRE_PTR(x); REQUIRE_PTR(dx);
  }
  const size_t need = round_up(linear_wgrad_schedule_ints(K, N) * 4);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(W4A4_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  OPTIONAL_PTR(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* DY = static_cast<const uint16_t*>(dy);
  if (T > 0 && !launch_linear_dgrad(T, K, N, offsets, DY, static_cast<const uint16_t*>(w),
                                    static_cast<uint16_t*>(dx), s))
    return W4A4_ERR_LAUNCH;
  if (!launch_linear_wgrad(T, K, N, offsets, DY, static_cast<const uint16_t*>(x),
                           static_cast<uint16_t*>(dw), static_cast<int32_t*>(workspace), s))
    return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

w4a4_status w4a4_mx_quantize_permute(const void* x, int64_t T, int K, const int32_t* topk_idx, int k, int E,
                                     int row_align, uint8_t* codes, uint8_t* scales, int32_t* expert_offsets,
                                     int32_t* row_map, int32_t* src_row, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  w4a4_status st = check_quantize_permute(x, T, K, topk_idx, k, E, row_align, codes, scales, nullptr,
                                          expert_offsets, row_map, src_row, /*need_outer=*/false);
  if (st != W4A4_OK) return st;
  if (K % 32 || K > 4096)
    return fail(W4A4_ERR_UNSUPPORTED, "MXFP4 rows need K %% 32 == 0 and K <= 4096 (K=%d)", K);
  const size_t need = w4a4_workspace_size(W4A4_WS_QUANTIZE_PERMUTE, T, K, 0, E, k, row_align);
  if (topk_idx != nullptr && T > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(W4A4_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  OPTIONAL_PTR(workspace);
  if (!launch_quantize_permute_mx(static_cast<const uint16_t*>(x), T, K, topk_idx, k, E, row_align, codes,
                                  scales, expert_offsets, row_map, src_row, workspace,
                                  static_cast<hipStream_t>(stream)))
    return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

w4a4_status w4a4_mx_grouped_expert_fwd(
    int64_t T, int H, int I, int E, int k, int row_align, const uint8_t* x_codes,
    const uint8_t* x_scales, const int32_t* expert_offsets, const int32_t* row_map,
    const int32_t* src_row, const float* topk_w, const uint8_t* w1_codes, const uint8_t* w1_scales,
    const uint8_t* w2_codes, const uint8_t* w2_scales, void* y, void* save_h, void* save_a,
    float* dbg_fc1_f32, uint8_t* dbg_a_codes, uint8_t* dbg_a_scales, void* workspace,
    size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  w4a4_status st = check_moe_shape(T, H, I, E, k, row_align);
  if (st != W4A4_OK) return st;
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(w1_codes); REQUIRE_PTR(w1_scales);
  REQUIRE_PTR(w2_codes); REQUIRE_PTR(w2_scales);
  if (T > 0) {
    REQUIRE_PTR(x_codes); REQUIRE_PTR(x_scales);
    REQUIRE_PTR(row_map); REQUIRE_PTR(src_row); REQUIRE_PTR(topk_w); REQUIRE_PTR(y);
  }
  OPTIONAL_PTR(save_h); OPTIONAL_PTR(save_a); OPTIONAL_PTR(dbg_fc1_f32);
  OPTIONAL_PTR(dbg_a_codes); OPTIONAL_PTR(dbg_a_scales);
  const int nd = (dbg_a_codes != nullptr) + (dbg_a_scales != nullptr);
  if (nd == 1) return fail(W4A4_ERR_INVALID_ARG, "dbg_a_codes, dbg_a_scales: both or neither");
  // the MX row encoder of the FC2 input takes rows of at most 4096
  if (I > 4096) return fail(W4A4_ERR_UNSUPPORTED, "the MXFP4 forward needs I <= 4096 (I=%d)", I);
  const int64_t cap = w4a4_rows_capacity(T, k, E, row_align);
  const FwdWs L = fwd_ws(cap, H, I);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(W4A4_ERR_WORKSPACE, "workspace needs %zu bytes", L.total);
  OPTIONAL_PTR(workspace);
  if (cap == 0) return W4A4_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* a_buf = save_a ? static_cast<uint16_t*>(save_a) : reinterpret_cast<uint16_t*>(ws + L.a);
  // the NVFP4 layout's code and scale areas hold the MXFP4 ones (fewer scale bytes)
  uint8_t* a_codes = nd ? dbg_a_codes : ws + L.a_codes;
  uint8_t* a_scales = nd ? dbg_a_scales : ws + L.a_scales;
  uint16_t* o_buf = reinterpret_cast<uint16_t*>(ws + L.o);

  if (!launch_fc1_mx(cap, H, I, E, expert_offsets, Fp4Operand{x_codes, x_scales, nullptr},
                     Fp4Operand{w1_codes, w1_scales, nullptr}, static_cast<uint16_t*>(save_h), a_buf,
                     dbg_fc1_f32, s))
    return W4A4_ERR_LAUNCH;
  if (!launch_requant_mx(a_buf, cap, I, expert_offsets, E, a_codes, a_scales, s)) return W4A4_ERR_LAUNCH;
  if (!launch_fc2_mx(cap, H, I, E, expert_offsets, Fp4Operand{a_codes, a_scales, nullptr},
                     Fp4Operand{w2_codes, w2_scales, nullptr}, o_buf, s))
    return W4A4_ERR_LAUNCH;
  if (!launch_unpermute(T, H, k, o_buf, row_map, topk_w, static_cast<uint16_t*>(y), s))
    return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

w4a4_status w4a4_mx8_expert_bwd(int64_t T, int H, int I, int E, int k, int row_align, const void* dy,
                                const void* x, const void* w1, const void* w2, const void* save_h,
                                const void* save_a, const float* topk_w, const int32_t* expert_offsets,
                                const int32_t* row_map, const int32_t* src_row, void* dx, void* dw1, void* dw2,
                                void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  w4a4_status st = check_moe_shape(T, H, I, E, k, row_align);
  if (st != W4A4_OK) return st;
  if (row_align != 128)
    return fail(W4A4_ERR_UNSUPPORTED, "the MXFP8 backward needs row_align 128 (row_align=%d)", row_align);
  if (I % 256) return fail(W4A4_ERR_UNSUPPORTED, "the MXFP8 backward needs I %% 256 == 0 (I=%d)", I);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(w1); REQUIRE_PTR(w2); REQUIRE_PTR(dw1); REQUIRE_PTR(dw2);
  if (T > 0) {
    REQUIRE_PTR(dy); REQUIRE_PTR(x); REQUIRE_PTR(save_h); REQUIRE_PTR(save_a);
    REQUIRE_PTR(topk_w); REQUIRE_PTR(row_map); REQUIRE_PTR(src_row); REQUIRE_PTR(dx);
  }
  const int64_t cap = w4a4_rows_capacity(T, k, E, row_align);
  const Mx8Ws L = mx8_ws(cap, H, I, E);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(W4A4_ERR_WORKSPACE, "workspace needs %zu bytes", L.total);
  OPTIONAL_PTR(workspace);
  // the transposed operands ([H | I | 2I, P] bytes) are addressed with 32-bit offsets
  if (L.P * static_cast<int64_t>(std::max(H, 2 * I)) > (int64_t{1} << 31))
    return fail(W4A4_ERR_UNSUPPORTED, "too many dispatched rows for the MXFP8 backward's 32-bit offsets");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  auto bf = [&](size_t o) { return reinterpret_cast<uint16_t*>(ws + o); };
  uint16_t *dO = bf(L.dO), *xp = bf(L.xp), *dA = bf(L.dA), *dXp = bf(L.dXp);
  const uint16_t* h = static_cast<const uint16_t*>(save_h);
  const uint16_t* a = static_cast<const uint16_t*>(save_a);
  const uint16_t* W1 = static_cast<const uint16_t*>(w1);
  const uint16_t* W2 = static_cast<const uint16_t*>(w2);
  const int32_t* off = expert_offsets;
  const int64_t P = L.P;

  // the row operands in expert order (as the BF16 backward), pad rows zero
  if (!launch_scatter_dy(T, H, k, static_cast<const uint16_t*>(dy), row_map, topk_w, dO, s) ||
      !launch_zero_pad_rows(cap, H, src_row, off, E, dO, s) ||
      !launch_scatter_x(T, H, k, static_cast<const uint16_t*>(x), row_map, xp, s) ||
      !launch_zero_pad_rows(cap, H, src_row, off, E, xp, s))
    return W4A4_ERR_LAUNCH;
  // FC2: dA = Q_H(dO) Q_H(W2[e]);  dW2[e] = Q_r(dO_e)^T Q_r(a_e)
  if (!launch_q8_dual(dO, nullptr, cap, H, 0, off, E, P, ws + L.dOq, ws + L.dOqs, ws + L.dOt, ws + L.dOts,
                      "mx8_quant_dual_dO", s) ||
      !launch_q8_cols(a, cap, I, 1, off, E, P, ws + L.at, ws + L.ats, "mx8_quant_cols_a", s) ||
      !launch_q8_cols(W2, H, I, E, nullptr, 0, H, ws + L.w2t, ws + L.w2ts, "mx8_quant_cols_w2", s))
    return W4A4_ERR_LAUNCH;
  if (cap > 0 && !launch_mx8_dgrad(cap, H, I, E, off, ws + L.dOq, ws + L.dOqs, ws + L.w2t, ws + L.w2ts, dA,
                                   "mx8_dgrad_fc2", s))
    return W4A4_ERR_LAUNCH;
  if (!launch_mx8_wgrad(H, I, E, off, ws + L.dOt, ws + L.dOts, ws + L.at, ws + L.ats, P,
                        static_cast<uint16_t*>(dw2), "mx8_wgrad_fc2", s))
    return W4A4_ERR_LAUNCH;
  // FC1: dXp = Q_2I(dH) Q_2I(W1[e]);  dW1[e] = Q_r(dH_e)^T Q_r(xp_e), with dH the SwiGLU
  // backward of dA, formed tile by tile inside its quantiser
  if (!launch_q8_dual(dA, h, cap, 2 * I, I, off, E, P, ws + L.dHq, ws + L.dHqs, ws + L.dHt, ws + L.dHts,
                      "mx8_swiglu_quant_dual_dH", s) ||
      !launch_q8_cols(W1, 2 * I, H, E, nullptr, 0, 2 * I, ws + L.w1t, ws + L.w1ts, "mx8_quant_cols_w1", s) ||
      !launch_q8_cols(xp, cap, H, 1, off, E, P, ws + L.xpt, ws + L.xpts, "mx8_quant_cols_xp", s))
    return W4A4_ERR_LAUNCH;
  if (cap > 0 && !launch_mx8_dgrad(cap, 2 * I, H, E, off, ws + L.dHq, ws + L.dHqs, ws + L.w1t, ws + L.w1ts, dXp,
                                   "mx8_dgrad_fc1", s))
    return W4A4_ERR_LAUNCH;
  if (!launch_mx8_wgrad(2 * I, H, E, off, ws + L.dHt, ws + L.dHts, ws + L.xpt, ws + L.xpts, P,
                        static_cast<uint16_t*>(dw1), "mx8_wgrad_fc1", s))
    return W4A4_ERR_LAUNCH;
  if (!launch_gather_sum(T, H, k, dXp, row_map, static_cast<uint16_t*>(dx), s)) return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

w4a4_status w4a4_mx8_quantize(const void* x, int64_t R, int C, uint8_t* q_rows, uint8_t* s_rows, uint8_t* q_cols,
                              uint8_t* s_cols, int64_t pitch, void* stream) {
  g_last_error.clear();
  if (R < 0 || C <= 0) return fail(W4A4_ERR_INVALID_ARG, "bad size (R=%lld C=%d)", static_cast<long long>(R), C);
  if (R % 128 || C % 128)
    return fail(W4A4_ERR_UNSUPPORTED, "needs R %% 128 == 0 and C %% 128 == 0 (R=%lld C=%d)",
                static_cast<long long>(R), C);
  if (pitch < R || pitch % 128) return fail(W4A4_ERR_INVALID_ARG, "pitch must be >= R and a multiple of 128");
  if (R == 0) return W4A4_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(q_rows); REQUIRE_PTR(s_rows); REQUIRE_PTR(q_cols); REQUIRE_PTR(s_cols);
  if (!launch_q8_dual(static_cast<const uint16_t*>(x), nullptr, R, C, 0, nullptr, 0, pitch, q_rows, s_rows, q_cols,
                      s_cols, "mx8_quant_dual", static_cast<hipStream_t>(stream)))
    return W4A4_ERR_LAUNCH;
  return W4A4_OK;
}

const char* w4a4_status_string(int status) {
  switch (status) {
    case W4A4_OK: return "ok";
    case W4A4_ERR_INVALID_ARG: return "invalid argument";
    case W4A4_ERR_UNSUPPORTED: return "unsupported configuration";
    case W4A4_ERR_WORKSPACE: return "workspace missing or too small";
    case W4A4_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* w4a4_last_error(void) { return g_last_error.c_str(); }

int w4a4_profiler_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_clear();
  g_prof_on = on != 0;
  return 0;
}

int w4a4_profiler_report(char* buf, size_t len) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  struct Agg {
    int count = 0;
    double ms = 0.0;
  };
  std::map<std::string, Agg> agg;
  for (const ProfEntry& e : g_prof_entries) {
    if (hipEventSynchronize(e.stop) != hipSuccess) return -1;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, e.start, e.stop) != hipSuccess) return -1;
    Agg& a = agg[e.name];
    a.count += 1;
    a.ms += ms;
  }
  std::string out = "{";
  bool first = true;
  for (const auto& kv : agg) {
    char item[256];
    snprintf(item, sizeof item, "%s\"%s\": {\"count\": %d, \"total_ms\": %.6f}", first ? "" : ", ",
             kv.first.c_str(), kv.second.count, kv.second.ms);
    out += item;
    first = false;
  }
  out += "}";
  if (buf != nullptr && len > 0) {
    const size_t n = out.size() < len - 1 ? out.size() : len - 1;
    memcpy(buf, out.data(), n);
    buf[n] = '\0';
  }
  return static_cast<int>(out.size());
}

}  // extern "C"
