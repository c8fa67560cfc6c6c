// Internal launch entry points (host side) behind the C ABI in hfq4moe.h.
// Every launcher assumes its arguments were validated by api.cpp and
// returns a hipError_t value (0 = success).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>


namespace hq {

// Kernel-side view of one MoE layer's expert weights.
struct LayerDev {
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  int64_t sg, su, sd;   // bytes between consecutive experts
  int E, d, F;
  uint32_t flags;
  // extent of each tensor (E * stride, < 2^32): one buffer descriptor per
  // tensor, with expert and row in the per-lane offset
  uint32_t gate_bytes, up_bytes, down_bytes;
};

// Token groups of a batched call: the pairs (token, slot) that selected the
// same expert.  Group ids follow the first pair of each group; members are
// in token order.
constexpr int GT_MAXU = 128;   // max groups (= max pairs B*k)
constexpr int GT_MAXM = 16;    // max members (= max tokens)
struct GroupTab {
  int U;
  int gexp[GT_MAXU];
  int gcnt[GT_MAXU];
  uint8_t gmem[GT_MAXU][GT_MAXM];   // member m of group u: pair id
};

// Workspace carve-up shared by the routing and expert kernels.
struct Ws {
  uint32_t* err;      // sticky HFQ4_DEV_ERR_* word
  uint32_t* ctr;      // inter-workgroup counters [WS_COUNTERS], zero between calls
  float* logits;      // [B][E]
  int32_t* idx;       // [B][k]  routing (internal copy)
  float* wts;         // [B][k]
  float* h;           // [B*k][F] SiLU(gate)*up per (token, slot)
  uint8_t* dstage;    // one token, host-mapped layer: [k][dslot] HBM copies of the
                      // selected experts' down matrices; null otherwise
  uint32_t dslot;     // bytes per staged down matrix
  GroupTab* gtab;     // batched: the token groups, published by the gate/up kernel
  uint64_t* trace;    // optional phase timestamps (null unless tracing is on)
  // one token, single-launch layer: words exchanged between its workgroups,
  // each (generation << 32 | value bits), and the call counter.  They sit
  // at the same place in every layout, right after the header, and no other
  // kernel writes there, so a workspace used for calls of other shapes in
  // between never leaves data that looks like a current word.
  uint64_t* xlog;     // [XL_MAX] router logits
  uint64_t* xh;       // [XH_MAX] SiLU(gate) * up, [k][F]
  uint32_t* xflag;    // [XG_MAX] generation of the last h a workgroup published
  uint32_t* gen;      // [1] single-launch calls run on this workspace
  uint64_t* xs;       // [XS_MAX] slot sums of the down rows, [slot][2048]
};
constexpr int XG_MAX = 1024;       // workgroups of the single-launch layer
constexpr int XL_MAX = 1024;       // experts (HFQ4_MAX_EXPERTS)
constexpr int XH_MAX = 8 * 512;    // k * F of the tuned shape
constexpr int XS_MAX = 8 * 2048;   // k * d of the tuned shape
constexpr int XREG_BYTES = 8 * XL_MAX + 8 * XH_MAX + 4 * XG_MAX + 256 + 8 * XS_MAX;
constexpr int WS_HEADER = 1024;    // err word at 0, counters from byte 64
constexpr int WS_COUNTERS = 240;

// Phase tracing: when a trace buffer is registered, thread 0 of every
// workgroup stamps s_memrealtime (100 MHz) at fixed points.  Slot layout:
// trace[(kernel * 1024 + workgroup) * 8 + point].
enum TraceKernel { TK_LOGITS = 0, TK_GATEUP = 1, TK_DOWN = 2, TK_TOPK = 3 };
void set_trace(uint64_t* p);
uint64_t* get_trace();
void set_timing_events(void* start, void* stop);
// Diagnostics: whether one-token layers of the tuned shape run as one
// launch (the default) or as the three-launch chain.
void set_single_launch(int mode);   // 0: three launches, 1: one, 2: two
// Diagnostics: batches of at least b tokens route by exchange (one router
// workgroup per token); smaller ones route in every gate/up workgroup.
void set_route_exchange_min_batch(int b);
// Shapes the single-launch layer (and so the pointer-table layers) serve.
bool single_launch_shape(int E, int d, int F, int k);

// Byte layout of a workspace for (E, B, k, d, F, layer flags) (k = 0:
// routing only).
constexpr uint32_t LAYER_HOST_MAPPED = 1u;
struct WsLayout {
  size_t logits, idx, wts, h, gtab, dstage, dslot, xlog, xh, xflag, gen, xs, total;
};
WsLayout ws_layout(int64_t E, int B, int k, int64_t d, int64_t F, uint32_t flags);
Ws ws_carve(void* base, int64_t E, int B, int k, int64_t d, int64_t F, uint32_t flags);

int launch_pack(const float* w, int64_t rows, int64_t K, int64_t ldw, void* out, int32_t* bad,
                hipStream_t s);
int launch_gemv(const void* W, int64_t rows, int64_t K, const float* x, int64_t ldx, int batch,
                const float* residual, int64_t ldr, float* y, int64_t ldy, hipStream_t s);
int launch_route(const float* Wr, const float* bias, int E, int d, const float* x, int64_t ldx,
                 int B, int k, int32_t* idx, float* wts, float* logits_out, Ws ws, hipStream_t s);
int launch_experts(const LayerDev& L, const float* x, int64_t ldx, int B, const int32_t* idx,
                   const float* wts, int k, const float* residual, float* y, int64_t ldy, Ws ws,
                   hipStream_t s);
int launch_layer(const LayerDev& L, const float* Wr, const float* bias, const float* x,
                 int64_t ldx, int B, int k, int32_t* idx, float* wts, const float* residual,
                 float* y, int64_t ldy, Ws ws, hipStream_t s);
int launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// TurboQuant: encode (f32 [count][ld] -> records) or decode (records -> f32);
// lut = false makes the encoder search the thresholds instead of using its
// bucket table.
struct TurboTable;   // turbo.h
int launch_turbo(bool encode, const void* src, int64_t count, int n, int64_t ld, void* dst,
                 int bits, const TurboTable& tab, bool lut, hipStream_t s);
// One token of the tuned shape with expert weights through a pointer table
// (ptr [E][3] device addresses of gate, up, down), hit counts into hits[2].
int launch_layer_table(const LayerDev& L, const uint64_t* ptr, const uint8_t* resident,
                       unsigned long long* hits, const float* Wr, const float* bias,
                       const float* x, int k, int32_t* idx, float* wts, const float* residual,
                       float* y, Ws ws, hipStream_t s);
// Compute units of the current device (cached per device).
int num_cus();

// Raise a kernel's dynamic LDS limit when its static plus dynamic use may
// pass the 64 KiB default (gfx950 has 160 KiB per CU).
template <typename K>
inline int allow_lds(K kernel, size_t bytes) {
  if (bytes <= 32768) return 0;
  return (int)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace hq
