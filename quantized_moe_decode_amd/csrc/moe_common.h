// Argument blocks and shape constants shared by the MoE decode kernels.
#pragma once
#include "hfq4_device.h"
#include "launch.h"

namespace hq {

constexpr int MAXP = 128;                      // max (token, slot) pairs: 16 x 8... up to B*k
constexpr int MAXK = 16;

struct RouteArgs {
  const float* Wr;
  const float* bias;
  int E, d;
  const float* x;
  int64_t ldx;
  int B, k;
  int32_t* idx_out;
  float* wts_out;
  float* logits_out;
};

struct ExpertArgs {
  LayerDev L;
  const float* x;
  int64_t ldx;
  int B, k;
  const int32_t* idx;   // [B][k]
  const float* wts;     // [B][k]
  const float* res;     // [B][ldy] or null
  float* y;
  int64_t ldy;
};

// Shapes of the workloads this build is tuned for: a gate/up row is 8 blocks
// = 64 segments (one per lane), a down row is 2 blocks = 16 segments (16
// lanes), up to 8 experts per token.
constexpr int FAST_SEGS_D = 64;
constexpr int FAST_SEGS_F = 16;
constexpr int FAST_F = 512;       // expert width of the tuned shape
constexpr int FAST_RP = 4;        // gate/up row pairs per wave item
constexpr int FAST_ROWS = 2;      // down output rows per wave

__host__ __device__ inline bool fast_shape(int d, int F, int k) {
  return d > 1792 && d <= 2048 && F == FAST_F && k <= 8;
}

// Batched path (2 <= B <= 16) on MFMA matrix cores.
constexpr int LG_KS = 4;   // K splits of the batched router GEMV (partial logit sets)
// Row stride of a partial logit set: E rounded up to 4 experts.
__host__ __device__ inline int lg_stride(int E) { return (E + 3) & ~3; }
// Up to LG_VALU_MAXB tokens the router is the VALU one-row-per-wave kernel,
// which writes whole sums (without the bias) into set 0: the routing then
// reads one set and adds the bias as it does to LG_KS partial sets.
constexpr int LG_VALU_MAXB = 4;
__host__ __device__ inline int lg_sets(int B) { return B <= LG_VALU_MAXB ? 1 : LG_KS; }
// The VALU router for 1..LG_VALU_MAXB tokens: logits of token b at
// out[b * ldl + e] (ldl = E for one token, lg_stride(E) for partial set 0).
int launch_logits_valu(const RouteArgs& ra, float* out, int ldl, hipStream_t s);
// gen (or null): the router also advances the workspace's call counter,
// whose new value the following gate/up kernel's routing exchange uses as
// this call's generation.
int launch_logits_batched(const RouteArgs& ra, float* part, uint32_t* gen, hipStream_t s);
// Whether a fused batched call of B tokens on the fast shape routes by
// exchange (one router workgroup per token) on this device.
bool batched_route_exchange(int B);
// Top-k and weights from the partial logits, one wave per token (routing
// only).
int launch_route_batched(const RouteArgs& ra, const float* part, uint32_t* err, hipStream_t s);
// gate/up then down for the fast shape (token groups built in-kernel); with
// ra set, the gate/up kernel also routes the tokens from the partial logits
// in ws.logits and publishes idx / wts to ra's outputs.
int launch_experts_batched(const ExpertArgs& a, Ws ws, int nwg, const RouteArgs* ra, hipStream_t s);

}  // namespace hq
