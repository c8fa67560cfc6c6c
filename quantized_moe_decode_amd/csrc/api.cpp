// C ABI of libhfq4moe.so (declared in include/hfq4moe.h).
//
// Every entry point validates its arguments on the host before touching the
// device, and refuses loudly with a detail string that names the argument
// and, for sizes, both the required and the given amount (the refusal style
// of the hipfire expert-offload explainer, section "放置算法": say what is
// short and by how much instead of failing later).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/hfq4moe.h"
#include "host_cpu.h"
#include "launch.h"
#include "placement.h"
#include "turbo.h"

namespace {

thread_local std::string g_err;
char g_arch_override[64] = {0};
std::mutex g_arch_mu;
int g_arch_ok[64] = {0};  // per device: 0 unknown, 1 gfx950, -1 other

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return HFQ4_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) overlap?
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

size_t packed(int64_t rows, int64_t K) { return (size_t)rows * (size_t)((K + 255) / 256) * 136u; }

int check_device() {
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (g_arch_override[0] && std::strncmp(g_arch_override, "gfx950", 6) != 0)
    return fail(HFQ4_E_DEVICE, "device is %s, this library is built for gfx950 only",
                g_arch_override);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HFQ4_E_DEVICE, "no usable HIP device: %s", hipGetErrorString(e));
  if (g_arch_override[0]) return HFQ4_OK;
  if (dev >= 0 && dev < 64 && g_arch_ok[dev] == 1) return HFQ4_OK;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess)
    return fail(HFQ4_E_DEVICE, "hipGetDeviceProperties(%d): %s", dev, hipGetErrorString(e));
  const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) g_arch_ok[dev] = is950 ? 1 : -1;
  if (!is950)
    return fail(HFQ4_E_DEVICE, "device %d is %s, this library is built for gfx950 only", dev,
                prop.gcnArchName);
  return HFQ4_OK;
}

int hip_status(int e, const char* what) {
  if (e != hipSuccess)
    return fail(HFQ4_E_HIP, "%s: %s", what, hipGetErrorString((hipError_t)e));
  return ok();
}

int check_layer(const moe_layer* L) {
  if (!L) return fail(HFQ4_E_INVALID, "layer descriptor is NULL");
  if (!L->gate || !L->up || !L->down) return fail(HFQ4_E_INVALID, "layer gate/up/down pointer is NULL");
  if (L->E < 1 || L->E > HFQ4_MAX_EXPERTS)
    return fail(HFQ4_E_INVALID, "E = %lld outside [1, %d]", (long long)L->E, HFQ4_MAX_EXPERTS);
  if (L->d < 4 || L->d > 2048 || (L->d & 3))
    return fail(HFQ4_E_UNSUPPORTED, "d = %lld: need 4 <= d <= 2048 and d %% 4 == 0", (long long)L->d);
  if (L->F < 4 || L->F > 2048 || (L->F & 3))
    return fail(HFQ4_E_UNSUPPORTED, "F = %lld: need 4 <= F <= 2048 and F %% 4 == 0", (long long)L->F);
  const size_t gb = packed(L->F, L->d), db = packed(L->d, L->F);
  if (L->stride_gate < (int64_t)gb || L->stride_up < (int64_t)gb)
    return fail(HFQ4_E_INVALID, "gate/up stride must be >= %zu bytes (one F x d HFQ4 matrix), got %lld / %lld",
                gb, (long long)L->stride_gate, (long long)L->stride_up);
  if (L->stride_down < (int64_t)db)
    return fail(HFQ4_E_INVALID, "down stride must be >= %zu bytes (one d x F HFQ4 matrix), got %lld", db,
                (long long)L->stride_down);
  if (!aligned16(L->gate) || !aligned16(L->up) || !aligned16(L->down) || (L->stride_gate & 15) ||
      (L->stride_up & 15) || (L->stride_down & 15))
    return fail(HFQ4_E_ALIGN, "expert weight pointers and strides must be 16-byte aligned");
  if (L->flags & ~HFQ4_LAYER_HOST_MAPPED) return fail(HFQ4_E_INVALID, "unknown layer flags 0x%x", L->flags);
  const int64_t lim = ((int64_t)1 << 32) - 256;
  if (L->E * L->stride_gate > lim || L->E * L->stride_up > lim || L->E * L->stride_down > lim)
    return fail(HFQ4_E_UNSUPPORTED, "E * stride must stay below 4 GiB per tensor (%lld / %lld / %lld bytes)",
                (long long)(L->E * L->stride_gate), (long long)(L->E * L->stride_up),
                (long long)(L->E * L->stride_down));
  return HFQ4_OK;
}

size_t ws_bytes_for(int64_t E, int B, int k, int64_t d, int64_t F, uint32_t flags) {
  return hq::ws_layout(E, B, k, d, F, flags).total;
}

int check_expert_io(const moe_layer* L, const float* x, int64_t ldx, int batch, const int32_t* idx,
                    const float* wts, int k, const float* residual, float* y, int64_t ldy) {
  if (!x || !y) return fail(HFQ4_E_INVALID, "x and y must be non-NULL");
  if (!idx || !wts) return fail(HFQ4_E_INVALID, "idx and wts must be non-NULL");
  if (batch < 1 || batch > HFQ4_MAX_BATCH)
    return fail(HFQ4_E_INVALID, "batch = %d outside [1, %d]", batch, HFQ4_MAX_BATCH);
  if (k < 1 || k > HFQ4_MAX_TOPK || k > L->E)
    return fail(HFQ4_E_INVALID, "k = %d: need 1 <= k <= min(E = %lld, %d)", k, (long long)L->E,
                HFQ4_MAX_TOPK);
  if (batch * k > 128)
    return fail(HFQ4_E_UNSUPPORTED, "batch * k = %d exceeds 128 (token, slot) pairs", batch * k);
  if (ldx < L->d || (ldx & 3)) return fail(HFQ4_E_ALIGN, "ldx = %lld: need ldx >= d and ldx %% 4 == 0", (long long)ldx);
  if (ldy < L->d) return fail(HFQ4_E_INVALID, "ldy = %lld < d = %lld", (long long)ldy, (long long)L->d);
  if (!aligned16(x)) return fail(HFQ4_E_ALIGN, "x must be 16-byte aligned");
  const size_t xb = sizeof(float) * ((size_t)(batch - 1) * ldx + L->d);
  const size_t yb = sizeof(float) * ((size_t)(batch - 1) * ldy + L->d);
  if (overlap(x, xb, y, yb)) return fail(HFQ4_E_INVALID, "y overlaps x");
  if (residual && residual != y && overlap(residual, yb, y, yb))
    return fail(HFQ4_E_INVALID, "residual partially overlaps y (it may equal y or be disjoint)");
  return HFQ4_OK;
}

}  // namespace

extern "C" {

const char* hfq4_last_error(void) { return g_err.c_str(); }

int hfq4_version(void) { return 100; }

// Testing hook: pretend the current device reports `arch` ("" restores the
// real query).  Used to exercise the device check without such a device.
int hfq4_debug_set_arch(const char* arch) {
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (!arch) arch = "";
  std::snprintf(g_arch_override, sizeof g_arch_override, "%s", arch);
  return ok();
}

// Diagnostics: register (or with NULL, clear) a device buffer of at least
// 4 * 1024 * 8 * 8 bytes that the decode kernels fill with per-workgroup
// phase timestamps.  Not for production use: it adds stores to every launch.
int hfq4_debug_set_trace(void* dev, size_t bytes) {
  if (dev && bytes < (size_t)4 * 1024 * 8 * 8)
    return fail(HFQ4_E_INVALID, "trace buffer needs %zu bytes, got %zu", (size_t)4 * 1024 * 8 * 8, bytes);
  hq::set_trace(static_cast<uint64_t*>(dev));
  return ok();
}

// Diagnostics: hipEvent_t handles recorded at the start and the end of every
// later launch of the expert gate/up kernel (NULL, NULL turns it off).
int hfq4_debug_set_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr))
    return fail(HFQ4_E_INVALID, "give both events or neither");
  hq::set_timing_events(start, stop);
  return ok();
}

// Diagnostics: one-token layers of the tuned shape as the three-launch
// chain (0, the default) or as one launch (1); results are the same bits.
int hfq4_debug_set_single_launch(int on) {
  hq::set_single_launch(on == 2 ? 2 : on != 0 ? 1 : 0);
  return ok();
}

int hfq4_debug_set_route_exchange(int min_batch) {
  if (min_batch < 2 || min_batch > HFQ4_MAX_BATCH + 1)
    return fail(HFQ4_E_INVALID, "min_batch = %d outside [2, %d]", min_batch, HFQ4_MAX_BATCH + 1);
  hq::set_route_exchange_min_batch(min_batch);
  return ok();
}

// Diagnostics: the TurboQuant encoder's nearest-level search by its bucket
// table (binary = 0, the default) or by binary search over the thresholds.
static std::atomic<int> g_turbo_binary_search{0};
int hfq4_debug_set_turbo_search(int binary) {
  g_turbo_binary_search.store(binary != 0 ? 1 : 0);
  return ok();
}

int hfq4_packed_bytes(int64_t rows, int64_t K, size_t* out) {
  if (!out) return fail(HFQ4_E_INVALID, "out is NULL");
  if (rows < 0) return fail(HFQ4_E_INVALID, "rows = %lld < 0", (long long)rows);
  if (K < 1) return fail(HFQ4_E_INVALID, "K = %lld < 1", (long long)K);
  *out = packed(rows, K);
  return ok();
}

int hfq4_pack(const float* w, int64_t rows, int64_t K, int64_t ldw, void* out, size_t out_bytes,
              int32_t* bad, hipStream_t stream) {
  if (rows < 0) return fail(HFQ4_E_INVALID, "rows = %lld < 0", (long long)rows);
  if (K < 1) return fail(HFQ4_E_INVALID, "K = %lld < 1", (long long)K);
  if (ldw < K) return fail(HFQ4_E_INVALID, "ldw = %lld < K = %lld", (long long)ldw, (long long)K);
  if (rows > 0 && (!w || !out)) return fail(HFQ4_E_INVALID, "w and out must be non-NULL");
  const size_t need = packed(rows, K);
  if (out_bytes < need)
    return fail(HFQ4_E_INVALID, "output needs %zu bytes, got %zu", need, out_bytes);
  if (rows > 0 && ((reinterpret_cast<uintptr_t>(out) & 7u) || (reinterpret_cast<uintptr_t>(w) & 3u)))
    return fail(HFQ4_E_ALIGN, "out must be 8-byte aligned and w 4-byte aligned");
  if (rows > 0 && overlap(w, sizeof(float) * ((size_t)(rows - 1) * ldw + K), out, need))
    return fail(HFQ4_E_INVALID, "out overlaps w");
  if (rows == 0) return ok();
  int r = check_device();
  if (r) return r;
  return hip_status(hq::launch_pack(w, rows, K, ldw, out, bad, stream), "hfq4_pack launch");
}

int hfq4_gemv(const void* W, int64_t rows, int64_t K, const float* x, int64_t ldx, int batch,
              const float* residual, int64_t ldr, float* y, int64_t ldy, hipStream_t stream) {
  if (rows < 0) return fail(HFQ4_E_INVALID, "rows = %lld < 0", (long long)rows);
  if (K < 1 || K > 16384) return fail(HFQ4_E_UNSUPPORTED, "K = %lld outside [1, 16384]", (long long)K);
  if (batch < 1 || batch > HFQ4_MAX_BATCH)
    return fail(HFQ4_E_INVALID, "batch = %d outside [1, %d]", batch, HFQ4_MAX_BATCH);
  if ((int64_t)batch * K > 32768)
    return fail(HFQ4_E_UNSUPPORTED, "batch * K = %lld exceeds 32768", (long long)batch * K);
  if (rows == 0) return ok();
  if (!W || !x || !y) return fail(HFQ4_E_INVALID, "W, x and y must be non-NULL");
  if (ldx < K || (ldx & 3)) return fail(HFQ4_E_ALIGN, "ldx = %lld: need ldx >= K and ldx %% 4 == 0", (long long)ldx);
  if (ldy < rows) return fail(HFQ4_E_INVALID, "ldy = %lld < rows = %lld", (long long)ldy, (long long)rows);
  if (residual && ldr < rows) return fail(HFQ4_E_INVALID, "ldr = %lld < rows = %lld", (long long)ldr, (long long)rows);
  if (!aligned16(W) || !aligned16(x)) return fail(HFQ4_E_ALIGN, "W and x must be 16-byte aligned");
  const size_t yb = sizeof(float) * ((size_t)(batch - 1) * ldy + rows);
  if (overlap(x, sizeof(float) * ((size_t)(batch - 1) * ldx + K), y, yb))
    return fail(HFQ4_E_INVALID, "y overlaps x");
  if (overlap(W, packed(rows, K), y, yb)) return fail(HFQ4_E_INVALID, "y overlaps W");
  if (residual && residual != y && overlap(residual, sizeof(float) * ((size_t)(batch - 1) * ldr + rows), y, yb))
    return fail(HFQ4_E_INVALID, "residual partially overlaps y");
  int r = check_device();
  if (r) return r;
  return hip_status(hq::launch_gemv(W, rows, K, x, ldx, batch, residual, ldr, y, ldy, stream),
                    "hfq4_gemv launch");
}

int moe_route_workspace_bytes(int64_t E, int batch, size_t* out) {
  if (!out) return fail(HFQ4_E_INVALID, "out is NULL");
  if (E < 1 || E > HFQ4_MAX_EXPERTS) return fail(HFQ4_E_INVALID, "E = %lld outside [1, %d]", (long long)E, HFQ4_MAX_EXPERTS);
  if (batch < 1 || batch > HFQ4_MAX_BATCH) return fail(HFQ4_E_INVALID, "batch = %d outside [1, %d]", batch, HFQ4_MAX_BATCH);
  *out = ws_bytes_for(E, batch, 0, 0, 0, 0);
  return ok();
}

int moe_route_topk(const float* Wr, const float* bias, int64_t E, int64_t d, const float* x,
                   int64_t ldx, int batch, int k, int32_t* idx, float* wts, float* logits_out,
                   void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!Wr || !x || !idx || !wts || !ws)
    return fail(HFQ4_E_INVALID, "Wr, x, idx, wts and ws must be non-NULL");
  if (E < 1 || E > HFQ4_MAX_EXPERTS) return fail(HFQ4_E_INVALID, "E = %lld outside [1, %d]", (long long)E, HFQ4_MAX_EXPERTS);
  if (d < 4 || d > 65536 || (d & 3)) return fail(HFQ4_E_UNSUPPORTED, "d = %lld: need 4 <= d <= 65536, d %% 4 == 0", (long long)d);
  if (batch < 1 || batch > HFQ4_MAX_BATCH) return fail(HFQ4_E_INVALID, "batch = %d outside [1, %d]", batch, HFQ4_MAX_BATCH);
  if (k < 1 || k > E || k > HFQ4_MAX_TOPK)
    return fail(HFQ4_E_INVALID, "k = %d: need 1 <= k <= min(E = %lld, %d)", k, (long long)E, HFQ4_MAX_TOPK);
  if (ldx < d || (ldx & 3)) return fail(HFQ4_E_ALIGN, "ldx = %lld: need ldx >= d and ldx %% 4 == 0", (long long)ldx);
  if (!aligned16(Wr) || !aligned16(x)) return fail(HFQ4_E_ALIGN, "Wr and x must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u)) return fail(HFQ4_E_ALIGN, "ws must be 256-byte aligned");
  const size_t need = ws_bytes_for(E, batch, 0, 0, 0, 0);
  if (ws_bytes < need) return fail(HFQ4_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  int r = check_device();
  if (r) return r;
  hq::Ws w = hq::ws_carve(ws, E, batch, 0, 0, 0, 0);
  return hip_status(hq::launch_route(Wr, bias, (int)E, (int)d, x, ldx, batch, k, idx, wts, logits_out, w, stream),
                    "moe_route_topk launch");
}

int moe_workspace_bytes(const moe_layer* L, int batch, int k, size_t* out) {
  if (!out) return fail(HFQ4_E_INVALID, "out is NULL");
  int r = check_layer(L);
  if (r) return r;
  if (batch < 1 || batch > HFQ4_MAX_BATCH) return fail(HFQ4_E_INVALID, "batch = %d outside [1, %d]", batch, HFQ4_MAX_BATCH);
  if (k < 1 || k > HFQ4_MAX_TOPK || k > L->E) return fail(HFQ4_E_INVALID, "k = %d outside [1, min(E, %d)]", k, HFQ4_MAX_TOPK);
  *out = ws_bytes_for(L->E, batch, k, L->d, L->F, L->flags);
  return ok();
}

int moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws) return fail(HFQ4_E_INVALID, "ws is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u)) return fail(HFQ4_E_ALIGN, "ws must be 256-byte aligned");
  int r = check_device();
  if (r) return r;
  return hip_status(hq::launch_fill_zero(ws, ws_bytes, stream), "moe_workspace_init launch");
}

static hq::LayerDev to_dev(const moe_layer* L) {
  hq::LayerDev D;
  D.gate = static_cast<const uint8_t*>(L->gate);
  D.up = static_cast<const uint8_t*>(L->up);
  D.down = static_cast<const uint8_t*>(L->down);
  D.sg = L->stride_gate;
  D.su = L->stride_up;
  D.sd = L->stride_down;
  D.E = (int)L->E;
  D.d = (int)L->d;
  D.F = (int)L->F;
  D.flags = L->flags;
  D.gate_bytes = (uint32_t)(L->E * L->stride_gate);
  D.up_bytes = (uint32_t)(L->E * L->stride_up);
  D.down_bytes = (uint32_t)(L->E * L->stride_down);
  return D;
}

int moe_expert_decode(const moe_layer* L, const float* x, int64_t ldx, int batch,
                      const int32_t* idx, const float* wts, int k, const float* residual, float* y,
                      int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream) {
  int r = check_layer(L);
  if (r) return r;
  r = check_expert_io(L, x, ldx, batch, idx, wts, k, residual, y, ldy);
  if (r) return r;
  if (!ws) return fail(HFQ4_E_INVALID, "ws is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u)) return fail(HFQ4_E_ALIGN, "ws must be 256-byte aligned");
  const size_t need = ws_bytes_for(L->E, batch, k, L->d, L->F, L->flags);
  if (ws_bytes < need) return fail(HFQ4_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  r = check_device();
  if (r) return r;
  hq::Ws w = hq::ws_carve(ws, L->E, batch, k, L->d, L->F, L->flags);
  return hip_status(hq::launch_experts(to_dev(L), x, ldx, batch, idx, wts, k, residual, y, ldy, w, stream),
                    "moe_expert_decode launch");
}

int moe_layer_decode(const moe_layer* L, const float* Wr, const float* bias, const float* x,
                     int64_t ldx, int batch, int k, int32_t* idx, float* wts, const float* residual,
                     float* y, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream) {
  int r = check_layer(L);
  if (r) return r;
  if (!Wr) return fail(HFQ4_E_INVALID, "Wr is NULL");
  if (!aligned16(Wr)) return fail(HFQ4_E_ALIGN, "Wr must be 16-byte aligned");
  r = check_expert_io(L, x, ldx, batch, idx, wts, k, residual, y, ldy);
  if (r) return r;
  if (!ws) return fail(HFQ4_E_INVALID, "ws is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u)) return fail(HFQ4_E_ALIGN, "ws must be 256-byte aligned");
  const size_t need = ws_bytes_for(L->E, batch, k, L->d, L->F, L->flags);
  if (ws_bytes < need) return fail(HFQ4_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  r = check_device();
  if (r) return r;
  hq::Ws w = hq::ws_carve(ws, L->E, batch, k, L->d, L->F, L->flags);
  return hip_status(hq::launch_layer(to_dev(L), Wr, bias, x, ldx, batch, k, idx, wts, residual, y, ldy, w, stream),
                    "moe_layer_decode launch");
}

// ---------------------------------------------------------------- no-alloc variant
//
// moe_layer_decode for callers that cannot allocate: the scratch memory the
// kernels need (logits, routing copy, h, token groups, staged down
// matrices) lives in a fixed device array of this library instead of a
// caller workspace.  Each GPU holds its own copy of the array, at its own
// address; host code never passes the array's name to a kernel (on the host
// it is only a stand-in for the symbol) but the address looked up per device.

}  // extern "C"

static __device__ __align__(256) uint8_t scratch[HFQ4_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {nullptr};   // per device: address of `scratch`

// The array's device address on the current device, looked up once per
// device with that device current.
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HFQ4_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(HFQ4_E_UNSUPPORTED, "device ordinal %d above 63", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(HFQ4_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return HFQ4_OK;
}
}  // namespace

extern "C" {

int moe_layer_decode_noalloc(const moe_layer* L, const float* Wr, const float* bias,
                             const float* x, int64_t ldx, int batch, int k, int32_t* idx,
                             float* wts, const float* residual, float* y, int64_t ldy,
                             uint32_t* err, hipStream_t stream) {
  int r = check_layer(L);
  if (r) return r;
  if (!Wr) return fail(HFQ4_E_INVALID, "Wr is NULL");
  if (!aligned16(Wr)) return fail(HFQ4_E_ALIGN, "Wr must be 16-byte aligned");
  r = check_expert_io(L, x, ldx, batch, idx, wts, k, residual, y, ldy);
  if (r) return r;
  if (err && (reinterpret_cast<uintptr_t>(err) & 3u)) return fail(HFQ4_E_ALIGN, "err must be 4-byte aligned");
  const size_t need = ws_bytes_for(L->E, batch, k, L->d, L->F, L->flags);
  if (need > HFQ4_NOALLOC_SCRATCH_BYTES)
    return fail(HFQ4_E_WORKSPACE,
                "this call needs %zu bytes of scratch, the fixed no-alloc scratch holds %zu "
                "(use moe_layer_decode with a caller workspace)",
                need, (size_t)HFQ4_NOALLOC_SCRATCH_BYTES);
  r = check_device();
  if (r) return r;
  void* base = nullptr;
  r = scratch_for_current_device(&base);
  if (r) return r;
  hq::Ws w = hq::ws_carve(base, L->E, batch, k, L->d, L->F, L->flags);
  // Device errors go to the caller's word when given; otherwise to the
  // array's own header word, which nothing reads.  Every other part of the
  // scratch is written before it is read within a call, so no part of it
  // needs clearing between calls.
  if (err) w.err = err;
  return hip_status(hq::launch_layer(to_dev(L), Wr, bias, x, ldx, batch, k, idx, wts, residual, y, ldy, w, stream),
                    "moe_layer_decode_noalloc launch");
}

int hfq4_gemv_host(const void* W, int64_t rows, int64_t K, const float* x, int64_t ldx, int batch,
                   const float* residual, int64_t ldr, float* y, int64_t ldy, int nthreads) {
  if (rows < 0) return fail(HFQ4_E_INVALID, "rows = %lld < 0", (long long)rows);
  if (K < 1) return fail(HFQ4_E_INVALID, "K = %lld < 1", (long long)K);
  if (batch < 1 || batch > HFQ4_MAX_BATCH)
    return fail(HFQ4_E_INVALID, "batch = %d outside [1, %d]", batch, HFQ4_MAX_BATCH);
  if (nthreads < 0) return fail(HFQ4_E_INVALID, "nthreads = %d < 0", nthreads);
  if (rows == 0) return ok();
  if (!W || !x || !y) return fail(HFQ4_E_INVALID, "W, x and y must be non-NULL");
  if (ldx < K) return fail(HFQ4_E_INVALID, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (ldy < rows) return fail(HFQ4_E_INVALID, "ldy = %lld < rows = %lld", (long long)ldy, (long long)rows);
  if (residual && ldr < rows) return fail(HFQ4_E_INVALID, "ldr = %lld < rows = %lld", (long long)ldr, (long long)rows);
  const size_t yb = sizeof(float) * ((size_t)(batch - 1) * ldy + rows);
  if (overlap(x, sizeof(float) * ((size_t)(batch - 1) * ldx + K), y, yb))
    return fail(HFQ4_E_INVALID, "y overlaps x");
  if (overlap(W, packed(rows, K), y, yb)) return fail(HFQ4_E_INVALID, "y overlaps W");
  if (residual && residual != y && overlap(residual, sizeof(float) * ((size_t)(batch - 1) * ldr + rows), y, yb))
    return fail(HFQ4_E_INVALID, "residual partially overlaps y");
  hq::gemv_host(static_cast<const uint8_t*>(W), rows, K, x, ldx, batch, residual, ldr, y, ldy,
                nthreads ? nthreads : hq::host_threads_default());
  return ok();
}

int moe_expert_decode_host(const moe_layer* L, const float* x, int64_t ldx, int batch,
                           const int32_t* idx, const float* wts, int k, const float* residual,
                           float* y, int64_t ldy, int nthreads, uint32_t* err) {
  int r = check_layer(L);
  if (r) return r;
  r = check_expert_io(L, x, ldx, batch, idx, wts, k, residual, y, ldy);
  if (r) return r;
  if (nthreads < 0) return fail(HFQ4_E_INVALID, "nthreads = %d < 0", nthreads);
  hq::HostLayer H{static_cast<const uint8_t*>(L->gate), static_cast<const uint8_t*>(L->up),
                  static_cast<const uint8_t*>(L->down), L->E, L->d, L->F,
                  L->stride_gate, L->stride_up, L->stride_down};
  hq::expert_decode_host(H, x, ldx, batch, idx, wts, k, residual, y, ldy,
                         nthreads ? nthreads : hq::host_threads_default(), err);
  return ok();
}

int hfq4_debug_set_host_kernel(int kernel, int* in_use) {
  if (kernel < 0 || kernel > 3)
    return fail(HFQ4_E_INVALID, "host kernel %d outside [0, 3]", kernel);
  if (!hq::set_host_kernel(kernel))
    return fail(HFQ4_E_UNSUPPORTED, "this CPU lacks the instructions of host kernel %d", kernel);
  if (in_use) *in_use = hq::host_kernel_in_use();
  return ok();
}

int moe_place_experts(int mode, int64_t layers, int64_t E, const uint64_t* heat,
                      uint64_t expert_bytes, uint64_t fixed_bytes, uint64_t budget_bytes,
                      uint8_t* resident, uint64_t* placed_bytes) {
  if (mode != HFQ4_PLACE_LAYERS && mode != HFQ4_PLACE_HOTSET)
    return fail(HFQ4_E_INVALID, "placement mode %d is neither HFQ4_PLACE_LAYERS nor HFQ4_PLACE_HOTSET", mode);
  if (layers < 1 || E < 1) return fail(HFQ4_E_INVALID, "layers = %lld, E = %lld: need >= 1", (long long)layers, (long long)E);
  if (!resident) return fail(HFQ4_E_INVALID, "resident is NULL");
  if (mode == HFQ4_PLACE_HOTSET && !heat) return fail(HFQ4_E_INVALID, "hot-set placement needs the heat counts");
  if (expert_bytes == 0) return fail(HFQ4_E_INVALID, "expert_bytes is 0");
  uint64_t placed = 0, shortb = 0;
  const int nofit = hq::place_experts(mode, layers, E, heat, expert_bytes, fixed_bytes, budget_bytes,
                                      resident, &placed, &shortb);
  if (placed_bytes) *placed_bytes = placed;
  if (nofit)
    return fail(HFQ4_E_NOFIT,
                "DOES NOT FIT: the fixed weights need %llu bytes, the HBM budget is %llu: short by "
                "%llu bytes (raise the budget by at least that)",
                (unsigned long long)fixed_bytes, (unsigned long long)budget_bytes,
                (unsigned long long)shortb);
  return ok();
}

int moe_layer_decode_table(const moe_layer_table* T, const float* Wr, const float* bias,
                           const float* x, int batch, int k, int32_t* idx, float* wts,
                           const float* residual, float* y, uint64_t* hits, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (!T) return fail(HFQ4_E_INVALID, "table layer descriptor is NULL");
  if (!T->ptr) return fail(HFQ4_E_INVALID, "table layer ptr is NULL");
  if (reinterpret_cast<uintptr_t>(T->ptr) & 7u) return fail(HFQ4_E_ALIGN, "ptr must be 8-byte aligned");
  if (hits && (reinterpret_cast<uintptr_t>(hits) & 7u)) return fail(HFQ4_E_ALIGN, "hits must be 8-byte aligned");
  if (T->E < 1 || T->E > HFQ4_MAX_EXPERTS)
    return fail(HFQ4_E_INVALID, "E = %lld outside [1, %d]", (long long)T->E, HFQ4_MAX_EXPERTS);
  if (batch != 1) return fail(HFQ4_E_UNSUPPORTED, "table layers take one token per call, got batch = %d", batch);
  if (k < 1 || k > HFQ4_MAX_TOPK || k > T->E)
    return fail(HFQ4_E_INVALID, "k = %d: need 1 <= k <= min(E = %lld, %d)", k, (long long)T->E, HFQ4_MAX_TOPK);
  if (!(T->d > 1792 && T->d <= 2048 && (T->d & 3) == 0 && T->F == 512 && (k == 2 || k == 4 || k == 8) &&
        T->E <= hq::XL_MAX))
    return fail(HFQ4_E_UNSUPPORTED, "table layers need 1792 < d <= 2048 (d %% 4 == 0), F = 512, "
                "k in {2, 4, 8}, E <= %d; got E = %lld, d = %lld, F = %lld, k = %d", hq::XL_MAX,
                (long long)T->E, (long long)T->d, (long long)T->F, k);
  if (!Wr || !aligned16(Wr)) return fail(HFQ4_E_ALIGN, "Wr must be non-NULL and 16-byte aligned");
  // reuse the HBM-layer checks for the activations and workspace
  moe_layer L{reinterpret_cast<const void*>(16), reinterpret_cast<const void*>(16),
              reinterpret_cast<const void*>(16), T->E, T->d, T->F,
              (int64_t)packed(T->F, T->d), (int64_t)packed(T->F, T->d), (int64_t)packed(T->d, T->F), 0u, 0u};
  int r = check_expert_io(&L, x, T->d, 1, idx, wts, k, residual, y, T->d);
  if (r) return r;
  if (!ws) return fail(HFQ4_E_INVALID, "ws is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u)) return fail(HFQ4_E_ALIGN, "ws must be 256-byte aligned");
  const size_t need = ws_bytes_for(T->E, 1, k, T->d, T->F, 0);
  if (ws_bytes < need) return fail(HFQ4_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  r = check_device();
  if (r) return r;
  if (!hq::single_launch_shape((int)T->E, (int)T->d, (int)T->F, k))
    return fail(HFQ4_E_UNSUPPORTED, "table layers run one workgroup per compute unit on a "
                "256-compute-unit device; this one has %d", hq::num_cus());
  hq::LayerDev D{};
  D.E = (int)T->E;
  D.d = (int)T->d;
  D.F = (int)T->F;
  hq::Ws w = hq::ws_carve(ws, T->E, 1, k, T->d, T->F, 0);
  return hip_status(hq::launch_layer_table(D, T->ptr, T->resident, reinterpret_cast<unsigned long long*>(hits),
                                           Wr, bias, x, k, idx, wts, residual, y, w, stream),
                    "moe_layer_decode_table launch");
}

static int check_turbo(int n, int bits) {
  if (n != 64 && n != 128 && n != 256) return fail(HFQ4_E_UNSUPPORTED, "n = %d: need 64, 128 or 256", n);
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(HFQ4_E_UNSUPPORTED, "bits = %d: need 2, 3, 4 or 8", bits);
  return HFQ4_OK;
}

// Level tables, computed on first use per (n, bits) and kept.
static const hq::TurboTable& turbo_table_for(int n, int bits) {
  static std::mutex mu;
  static hq::TurboTable* tabs[3][9] = {{nullptr}};
  const int ni = n == 64 ? 0 : n == 128 ? 1 : 2;
  std::lock_guard<std::mutex> lk(mu);
  if (!tabs[ni][bits]) {
    tabs[ni][bits] = new hq::TurboTable();
    hq::turbo_table(n, bits, tabs[ni][bits]);
  }
  return *tabs[ni][bits];
}

int turbo_record_bytes(int n, int bits, size_t* out) {
  if (!out) return fail(HFQ4_E_INVALID, "out is NULL");
  int r = check_turbo(n, bits);
  if (r) return r;
  *out = (size_t)n * bits / 8 + 4;
  return ok();
}

int turbo_levels(int n, int bits, float* levels) {
  if (!levels) return fail(HFQ4_E_INVALID, "levels is NULL");
  int r = check_turbo(n, bits);
  if (r) return r;
  const hq::TurboTable& t = turbo_table_for(n, bits);
  for (int j = 0; j < (1 << bits); ++j) levels[j] = t.cent[j];
  return ok();
}

int turbo_encode(const float* v, int64_t count, int n, int64_t ldv, int bits, void* out,
                 size_t out_bytes, hipStream_t stream) {
  int r = check_turbo(n, bits);
  if (r) return r;
  if (count < 0) return fail(HFQ4_E_INVALID, "count = %lld < 0", (long long)count);
  if (count == 0) return ok();
  if (!v || !out) return fail(HFQ4_E_INVALID, "v and out must be non-NULL");
  if (ldv < n) return fail(HFQ4_E_INVALID, "ldv = %lld < n = %d", (long long)ldv, n);
  const size_t rec = (size_t)n * bits / 8 + 4;
  if (out_bytes < rec * (size_t)count)
    return fail(HFQ4_E_INVALID, "out needs %zu bytes, got %zu", rec * (size_t)count, out_bytes);
  if ((reinterpret_cast<uintptr_t>(out) & 3u) || (reinterpret_cast<uintptr_t>(v) & 3u))
    return fail(HFQ4_E_ALIGN, "v and out must be 4-byte aligned");
  if (overlap(v, sizeof(float) * ((size_t)(count - 1) * ldv + n), out, rec * (size_t)count))
    return fail(HFQ4_E_INVALID, "out overlaps v");
  r = check_device();
  if (r) return r;
  return hip_status(hq::launch_turbo(true, v, count, n, ldv, out, bits, turbo_table_for(n, bits),
                                     g_turbo_binary_search.load() == 0, stream),
                    "turbo_encode launch");
}

int turbo_decode(const void* in, size_t in_bytes, int64_t count, int n, int bits, float* v,
                 int64_t ldv, hipStream_t stream) {
  int r = check_turbo(n, bits);
  if (r) return r;
  if (count < 0) return fail(HFQ4_E_INVALID, "count = %lld < 0", (long long)count);
  if (count == 0) return ok();
  if (!v || !in) return fail(HFQ4_E_INVALID, "in and v must be non-NULL");
  if (ldv < n) return fail(HFQ4_E_INVALID, "ldv = %lld < n = %d", (long long)ldv, n);
  const size_t rec = (size_t)n * bits / 8 + 4;
  if (in_bytes < rec * (size_t)count)
    return fail(HFQ4_E_INVALID, "in holds %zu bytes, %lld records need %zu", in_bytes, (long long)count,
                rec * (size_t)count);
  if ((reinterpret_cast<uintptr_t>(in) & 3u) || (reinterpret_cast<uintptr_t>(v) & 3u))
    return fail(HFQ4_E_ALIGN, "in and v must be 4-byte aligned");
  if (overlap(v, sizeof(float) * ((size_t)(count - 1) * ldv + n), in, rec * (size_t)count))
    return fail(HFQ4_E_INVALID, "v overlaps in");
  r = check_device();
  if (r) return r;
  return hip_status(hq::launch_turbo(false, in, count, n, ldv, v, bits, turbo_table_for(n, bits), true, stream),
                    "turbo_decode launch");
}

int hfq4_offload_choice(double pcie_seconds, double cpu_seconds, int* use_cpu) {
  if (!use_cpu) return fail(HFQ4_E_INVALID, "use_cpu is NULL");
  if (!(pcie_seconds > 0.0) || !(cpu_seconds > 0.0) || pcie_seconds == HUGE_VAL ||
      cpu_seconds == HUGE_VAL)
    return fail(HFQ4_E_INVALID, "times must be positive and finite (pcie %g s, cpu %g s)",
                pcie_seconds, cpu_seconds);
  *use_cpu = cpu_seconds * 1.15 <= pcie_seconds ? 1 : 0;
  return ok();
}

int hfq4_host_device_pointer(void* host, void** dev) {
  if (!host || !dev) return fail(HFQ4_E_INVALID, "host and dev must be non-NULL");
  int r = check_device();
  if (r) return r;
  return hip_status(hipHostGetDevicePointer(dev, host, 0), "hipHostGetDevicePointer");
}

}  // extern "C"
