// Top-k routed MoE layer decode over HFQ4 experts (gfx950).
//
// Problem statement: each token is routed to the top 8 of a layer's experts
// (hipfire expert-offload explainer, section "125GB 的 MoE 模型，为什么 32GB
// 显卡也有得跑？"); every expert has gate, up and down tensors (Strata user
// report, section "3. 模型与引擎"); the expert weights are HFQ4 blocks (page
// "hipfire：为AMD RDNA GPU打造的Rust原生LLM推理引擎", section "2. HFQ量化格式
// 与GEMV优化"); host-resident experts are read by the kernel itself over PCIe
// (explainer, section "PCIe 直通") -- here that is just another pointer.
//
// Readings: softmax over all logits, top-k by logit with ties to the lower
// index, renormalised over the k selected (computed as the k-term softmax,
// which is the same quantity); expert = down(SiLU(gate x) * (up x)); layer
// output = sum_j w_j y_{e_j} (+ optional residual).
//
// Kernels
//   route_kernel   router GEMV (one wave per expert row) + top-k by the last
//                  workgroup to finish (atomic ticket).
//   gateup_kernel  grouped gate/up dequant-GEMV: tokens that picked the same
//                  expert share one read of its rows; writes h = SiLU(g)*u.
//   down_kernel    down dequant-GEMV for every (token, slot), weighted by the
//                  routing weight and summed per lane before one cross-lane
//                  reduction per output row (fixed order, no atomics).
//   layer_kernel   all of the above in one launch: one workgroup per CU,
//                  phases separated by counters in the workspace.
#include "hfq4_device.h"
#include "launch.h"

namespace hq {

constexpr uint64_t WAIT_TICKS = 20000000ull;   // 200 ms of s_memrealtime (100 MHz)
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

// ====================================================================== routing

// Logits of rows e = gw, gw + nw, ... for every token; one wave per row.
__device__ void router_rows(const RouteArgs& a, const Ws& ws, int gw, int nw) {
  const int lane = threadIdx.x & 63;
  const int nq = a.d >> 2;
  for (int e = gw; e < a.E; e += nw) {
    const f32x4* wr = reinterpret_cast<const f32x4*>(a.Wr + (int64_t)e * a.d);
    float acc[HFQ4_MAXB_DEV];
#pragma unroll
    for (int b = 0; b < HFQ4_MAXB_DEV; ++b) acc[b] = 0.f;
    for (int q0 = 0; q0 < nq; q0 += 64 * 8) {
      f32x4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + u * 64 + lane;
        w[u] = q < nq ? wr[q] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int b = 0; b < HFQ4_MAXB_DEV; ++b) {
        if (b < a.B) {
          const f32x4* xb = reinterpret_cast<const f32x4*>(a.x + b * a.ldx);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int q = q0 + u * 64 + lane;
            const f32x4 xv = q < nq ? xb[q] : f32x4{0.f, 0.f, 0.f, 0.f};
            acc[b] = __builtin_fmaf(w[u].x, xv.x, acc[b]);
            acc[b] = __builtin_fmaf(w[u].y, xv.y, acc[b]);
            acc[b] = __builtin_fmaf(w[u].z, xv.z, acc[b]);
            acc[b] = __builtin_fmaf(w[u].w, xv.w, acc[b]);
          }
        }
      }
    }
    const float bias = a.bias ? a.bias[e] : 0.f;
#pragma unroll
    for (int b = 0; b < HFQ4_MAXB_DEV; ++b) {
      if (b < a.B) {
        const float l = group_sum<64>(acc[b]) + bias;
        if (lane == 0) {
          ws.logits[b * a.E + e] = l;
          if (a.logits_out) a.logits_out[b * a.E + e] = l;
        }
      }
    }
  }
}

// (value, index) order for top-k: larger value first, equal values -> lower index.
__device__ __forceinline__ bool better(float av, int ae, float bv, int be) {
  if (ae < 0) return false;
  if (be < 0) return true;
  return av > bv || (av == bv && ae < be);
}

// Top-k of one token by one wave.  Logits are read from the workspace at
// agent scope (they were written by other workgroups).  On return lanes
// j < k hold (sel_e, sel_w); all lanes see the same selection.
__device__ void topk_wave(const float* logits, int E, int k, uint32_t* err, int& sel_e,
                          float& sel_w) {
  const int lane = threadIdx.x & 63;
  constexpr int PER = HFQ4_MAXE_DEV / 64;
  float v[PER];
  int nonfinite = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    float t = -INFINITY;
    if (e < E) {
      t = ld_agent(logits + e);
      if (__builtin_isnan(t)) {
        nonfinite = 1;
        t = -INFINITY;
      }
    }
    v[i] = t;
  }
  if (__any(nonfinite) && lane == 0)
    __hip_atomic_fetch_or(err, 4u /*HFQ4_DEV_ERR_NONFINITE*/, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  uint32_t taken = 0;
  sel_e = -1;
  float my_v = -INFINITY;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = -1;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (be < 0 || v[i] > bv)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oe = __shfl_xor(be, m, 64);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      sel_e = be;
      my_v = bv;
    }
  }
  // weights: k-term softmax in selection order (max is the first selected)
  const float v0 = __shfl(my_v, 0, 64);
  float ex = 0.f;
  if (lane < k) ex = (v0 == -INFINITY) ? 1.f : expf(my_v - v0);
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += __shfl(ex, j, 64);
  sel_w = ex / sum;
}

__global__ void __launch_bounds__(256) route_kernel(RouteArgs a, Ws ws) {
  const int nw = gridDim.x * (blockDim.x >> 6);
  const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  router_rows(a, ws, gw, nw);
  // last workgroup to finish selects the experts
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  __shared__ uint32_t ticket;
  if (threadIdx.x == 0)
    ticket = __hip_atomic_fetch_add(&ws.ctr[0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (ticket != gridDim.x - 1) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int b = wv; b < a.B; b += (blockDim.x >> 6)) {
    int e;
    float w;
    topk_wave(ws.logits + b * a.E, a.E, a.k, ws.err, e, w);
    if (lane < a.k) {
      a.idx_out[b * a.k + lane] = e;
      a.wts_out[b * a.k + lane] = w;
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(&ws.ctr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ====================================================================== grouping

// Tokens that routed to the same expert form a group, so its weights are
// read once for all of them.  Built in LDS by every workgroup that needs it
// (P = B*k <= 128 pairs, pair p = token*k + slot):
//   gexp[u]  expert of group u (groups in order of first appearance)
//   gcnt[u], gstart[u]; gmem[gstart[u] + r] = r-th pair of group u.
struct Groups {
  int U;
  int gexp[MAXP];
  int gcnt[MAXP];
  int gstart[MAXP];
  int gmem[MAXP];
  int pexp[MAXP];   // expert of pair p, -1 if out of range
  int first[MAXP];  // first pair with the same expert
};

__device__ void build_groups(const int32_t* idx, int P, int E, Groups& G, uint32_t* err,
                             bool idx_agent) {
  const int t = threadIdx.x;
  if (t < P) {
    int e = idx_agent ? ld_agent(idx + t) : idx[t];
    if (e < 0 || e >= E) {
      __hip_atomic_fetch_or(err, 1u /*HFQ4_DEV_ERR_INDEX*/, __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
      e = -1;
    }
    G.pexp[t] = e;
  }
  __syncthreads();
  if (t < P) {
    const int e = G.pexp[t];
    int f = t;
    if (e >= 0)
      for (int q = 0; q < t; ++q)
        if (G.pexp[q] == e) {
          f = q;
          break;
        }
    G.first[t] = (e >= 0) ? f : -1;
  }
  __syncthreads();
  if (t < P && G.first[t] == t) {
    int u = 0, cnt = 0;
    for (int q = 0; q < t; ++q) u += (G.first[q] == q);
    for (int q = t; q < P; ++q) cnt += (G.first[q] == t);
    G.gexp[u] = G.pexp[t];
    G.gcnt[u] = cnt;
  }
  if (t == 0) {
    int U = 0;
    for (int q = 0; q < P; ++q) U += (G.first[q] == q);
    G.U = U;
  }
  __syncthreads();
  if (t < G.U) {
    int s = 0;
    for (int u = 0; u < t; ++u) s += G.gcnt[u];
    G.gstart[t] = s;
  }
  __syncthreads();
  if (t < P && G.first[t] >= 0) {
    const int f = G.first[t];
    int u = 0, r = 0;
    for (int q = 0; q < f; ++q) u += (G.first[q] == q);
    for (int q = f; q < t; ++q) r += (G.first[q] == f);
    G.gmem[G.gstart[u] + r] = t;
  }
  __syncthreads();
}

// ====================================================================== gate / up

// Work item = (group u, chunk of gate/up rows).  Rows of NBD blocks; SEGS =
// 8*NBD lanes per row, GR = 64/SEGS rows per load, RPW loads per wave for
// each of gate and up.  x fragments for all B tokens are staged in LDS.
template <int NBD, int RPW>
__device__ void gateup_item(const ExpertArgs& a, const Ws& ws, const Groups& G,
                            const uint8_t* xfr, int item) {
  constexpr int SEGS = 8 * NBD, GR = 64 / SEGS, ROWS = GR * RPW;
  const int lane = threadIdx.x & 63;
  const int g = lane / SEGS, s = lane % SEGS;
  const int F = a.L.F, d = a.L.d;
  const int nchunk = (F + ROWS - 1) / ROWS;
  const int u = item / nchunk, chunk = item - u * nchunk;
  const int e = G.gexp[u];
  const int nb = (d + BLK - 1) / BLK;
  const int64_t rowb = (int64_t)nb * BLK_BYTES;
  const int f0 = chunk * ROWS;
  int nrows = F - f0;
  if (nrows > ROWS) nrows = ROWS;
  const uint32_t span = (uint32_t)(nrows * rowb);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.L.gate + e * a.L.sg + f0 * rowb, span);
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.L.up + e * a.L.su + f0 * rowb, span);
  const bool live = (s >> 3) < nb;
  u32x4 cg[RPW], cu[RPW];
  u32x2 hg[RPW], hu[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const uint32_t off = (uint32_t)((i * GR + g) * rowb + (s >> 3) * BLK_BYTES);
    const uint32_t coff = off + 8 + 16 * (s & 7);
    hg[i] = live ? bload8(rg, off) : u32x2{0u, 0u};
    cg[i] = live ? bload16(rg, coff) : u32x4{0u, 0u, 0u, 0u};
    hu[i] = live ? bload8(ru, off) : u32x2{0u, 0u};
    cu[i] = live ? bload16(ru, coff) : u32x4{0u, 0u, 0u, 0u};
  }
  const int fb = frag_bytes(SEGS);
  const int n = G.gcnt[u], st = G.gstart[u];
  for (int m = 0; m < n; ++m) {
    const int p = G.gmem[st + m];
    const int b = p / a.k;
    Frag f;
    frag_load(xfr + b * fb, SEGS, s, f);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const float gs = group_sum<SEGS>(dot_seg(cg[i], hg[i], f));
      const float us = group_sum<SEGS>(dot_seg(cu[i], hu[i], f));
      const int row = i * GR + g;
      if (s == 0 && row < nrows) ws.h[(int64_t)p * F + f0 + row] = silu_mul(gs, us);
    }
  }
}

// ====================================================================== down + combine

// Each wave produces ROUT output rows for one token: for every slot j the
// expert's down row is dotted with h(token, j); lane groups (SEGS = 8*NBF
// lanes each, GF = 64/SEGS groups) take slots g, g+GF, ...; each lane sums
// w_j * partial over its slots, then one 64-lane reduction gives the row.
template <int NBF, int ROUT>
__device__ void down_rows(const ExpertArgs& a, const Ws& ws, const uint8_t* hfr, int b, int r0,
                          const int* pexp) {
  constexpr int SEGS = 8 * NBF, GF = 64 / SEGS;
  const int lane = threadIdx.x & 63;
  const int g = lane / SEGS, s = lane % SEGS;
  const int F = a.L.F, d = a.L.d, k = a.k;
  const int nb = (F + BLK - 1) / BLK;
  const int64_t rowb = (int64_t)nb * BLK_BYTES;
  const bool live = (s >> 3) < nb;
  const int fb = frag_bytes(SEGS);
  float acc[ROUT];
#pragma unroll
  for (int r = 0; r < ROUT; ++r) acc[r] = 0.f;
  for (int j0 = 0; j0 < k; j0 += GF) {
    const int j = j0 + g;
    const int p = b * k + j;
    const int e = (j < k) ? pexp[p] : -1;
    const bool use = live && e >= 0;
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(a.L.down + (e >= 0 ? e : 0) * a.L.sd, (uint32_t)(d * rowb));
    u32x4 c[ROUT];
    u32x2 hd[ROUT];
#pragma unroll
    for (int r = 0; r < ROUT; ++r) {
      const int row = r0 + r;
      const uint32_t off = (uint32_t)(row * rowb + (s >> 3) * BLK_BYTES);
      hd[r] = (use && row < d) ? bload8(rd, off) : u32x2{0u, 0u};
      c[r] = (use && row < d) ? bload16(rd, off + 8 + 16 * (s & 7)) : u32x4{0u, 0u, 0u, 0u};
    }
    const float w = (j < k && e >= 0) ? a.wts[p] : 0.f;
    Frag f;
    frag_load(hfr + (j < k ? j : 0) * fb, SEGS, s, f);
#pragma unroll
    for (int r = 0; r < ROUT; ++r) acc[r] = __builtin_fmaf(w, dot_seg(c[r], hd[r], f), acc[r]);
  }
#pragma unroll
  for (int r = 0; r < ROUT; ++r) {
    const float v = group_sum<64>(acc[r]);
    const int row = r0 + r;
    if (lane == 0 && row < d)
      a.y[b * a.ldy + row] = (a.res ? a.res[b * a.ldy + row] : 0.f) + v;
  }
}

// Stage h(token b, slot j) for j < k into LDS fragments (F values each).
template <int NBF>
__device__ void stage_h(const ExpertArgs& a, const Ws& ws, int b, uint8_t* hfr, bool agent) {
  constexpr int SEGS = 8 * NBF;
  const int F = a.L.F, k = a.k;
  const int fb = frag_bytes(SEGS);
  for (int t = threadIdx.x; t < k * SEGS; t += blockDim.x) {
    const int j = t / SEGS, s = t - j * SEGS;
    const float* src = ws.h + (int64_t)(b * k + j) * F;
    float buf[32];
    const int base = s * SEG;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int f = base + i;
      buf[i] = (f < F) ? (agent ? ld_agent(src + f) : src[f]) : 0.f;
    }
    Frag fr;
    make_frag(buf, fr);
    frag_store(hfr + j * fb, SEGS, s, fr);
  }
}

// ====================================================================== standalone kernels

template <int NBD, int RPW>
__global__ void __launch_bounds__(256) gateup_kernel(ExpertArgs a, Ws ws) {
  constexpr int SEGS = 8 * NBD, ROWS = (64 / SEGS) * RPW;
  extern __shared__ __align__(16) uint8_t xfr[];
  __shared__ Groups G;
  build_groups(a.idx, a.B * a.k, a.L.E, G, ws.err, false);
  const int fb = frag_bytes(SEGS);
  for (int b = 0; b < a.B; ++b)
    stage_vector(a.x + b * a.ldx, a.L.d, SEGS, xfr + b * fb, threadIdx.x, blockDim.x);
  __syncthreads();
  const int nchunk = (a.L.F + ROWS - 1) / ROWS;
  const int items = G.U * nchunk;
  const int nw = gridDim.x * (blockDim.x >> 6);
  for (int it = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); it < items; it += nw)
    gateup_item<NBD, RPW>(a, ws, G, xfr, it);
}

template <int NBF, int ROUT>
__global__ void __launch_bounds__(256) down_kernel(ExpertArgs a, Ws ws) {
  extern __shared__ __align__(16) uint8_t hfr[];
  __shared__ int pexp[MAXP];
  const int P = a.B * a.k;
  for (int t = threadIdx.x; t < P; t += blockDim.x) {
    const int e = a.idx[t];
    pexp[t] = (e >= 0 && e < a.L.E) ? e : -1;
  }
  const int nw = gridDim.x * (blockDim.x >> 6);
  const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  for (int b = 0; b < a.B; ++b) {
    __syncthreads();
    stage_h<NBF>(a, ws, b, hfr, false);
    __syncthreads();
    for (int r0 = gw * ROUT; r0 < a.L.d; r0 += nw * ROUT) down_rows<NBF, ROUT>(a, ws, hfr, b, r0, pexp);
  }
}

// ====================================================================== fused layer

// One launch per layer, one workgroup per CU.  Phases:
//  0  stage x (LDS); router rows of this workgroup -> workspace logits
//  1  wait for all logits; top-k for every token (redundantly per WG, so no
//     second hop); WG 0 writes idx/wts; build groups
//  2  gate/up items -> h in workspace; signal
//  3  wait for all h; stage h (LDS); down rows + combine -> y
//  4  last workgroup out resets the counters.
template <int NBD, int NBF, int RPW, int ROUT>
__global__ void __launch_bounds__(256) layer_kernel(RouteArgs ra, ExpertArgs a, Ws ws) {
  constexpr int SEGS_D = 8 * NBD;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ Groups G;
  __shared__ int sel_idx[HFQ4_MAXB_DEV * MAXK];
  __shared__ float sel_w[HFQ4_MAXB_DEV * MAXK];
  const int nwg = gridDim.x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = nwg * (blockDim.x >> 6);
  const int gw = blockIdx.x * (blockDim.x >> 6) + wv;
  const int B = a.B, k = a.k, P = B * k;
  uint8_t* xfr = lds;
  uint8_t* hfr = lds + B * frag_bytes(SEGS_D);

  // phase 0
  router_rows(ra, ws, gw, nw);
  for (int b = 0; b < B; ++b)
    stage_vector(a.x + b * a.ldx, a.L.d, SEGS_D, xfr + b * frag_bytes(SEGS_D), threadIdx.x,
                 blockDim.x);
  wg_signal(&ws.ctr[0]);
  // phase 1
  if (!wg_wait(&ws.ctr[0], (uint32_t)nwg, ws.err, WAIT_TICKS)) goto done;
  for (int b = wv; b < B; b += (blockDim.x >> 6)) {
    int e;
    float w;
    topk_wave(ws.logits + b * ra.E, ra.E, k, ws.err, e, w);
    if (lane < k) {
      sel_idx[b * k + lane] = e;
      sel_w[b * k + lane] = w;
      if (blockIdx.x == 0) {
        ra.idx_out[b * k + lane] = e;
        ra.wts_out[b * k + lane] = w;
      }
    }
  }
  __syncthreads();
  build_groups(sel_idx, P, a.L.E, G, ws.err, false);
  {
    // phase 2
    constexpr int ROWS = (64 / SEGS_D) * RPW;
    const int nchunk = (a.L.F + ROWS - 1) / ROWS;
    const int items = G.U * nchunk;
    for (int it = gw; it < items; it += nw) gateup_item<NBD, RPW>(a, ws, G, xfr, it);
  }
  wg_signal(&ws.ctr[1]);
  if (!wg_wait(&ws.ctr[1], (uint32_t)nwg, ws.err, WAIT_TICKS)) goto done;
  {
    // phase 3: routing weights for the down pass come from LDS
    ExpertArgs ad = a;
    ad.wts = sel_w;
    for (int b = 0; b < B; ++b) {
      stage_h<NBF>(ad, ws, b, hfr, true);
      __syncthreads();
      for (int r0 = gw * ROUT; r0 < a.L.d; r0 += nw * ROUT)
        down_rows<NBF, ROUT>(ad, ws, hfr, b, r0, G.pexp);
      __syncthreads();
    }
  }
done:
  // phase 4: the last workgroup out clears the counters for the next call
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t =
        __hip_atomic_fetch_add(&ws.ctr[2], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (t == (uint32_t)nwg - 1) {
      __hip_atomic_store(&ws.ctr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ws.ctr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ws.ctr[2], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ====================================================================== host side

static inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t ws_layout(int64_t E, int B, int k, int64_t F, size_t* off_logits, size_t* off_idx,
                 size_t* off_wts, size_t* off_h) {
  size_t o = 256;  // err word + 16 counters + padding
  *off_logits = o;
  o = al256(o + sizeof(float) * (size_t)B * E);
  *off_idx = o;
  o = al256(o + sizeof(int32_t) * (size_t)B * k);
  *off_wts = o;
  o = al256(o + sizeof(float) * (size_t)B * k);
  *off_h = o;
  o = al256(o + sizeof(float) * (size_t)B * k * F);
  return o;
}

Ws ws_carve(void* base, int64_t E, int B, int k, int64_t F) {
  size_t ol, oi, ow, oh;
  ws_layout(E, B, k, F, &ol, &oi, &ow, &oh);
  uint8_t* p = static_cast<uint8_t*>(base);
  Ws w;
  w.err = reinterpret_cast<uint32_t*>(p);
  w.ctr = reinterpret_cast<uint32_t*>(p + 64);
  w.logits = reinterpret_cast<float*>(p + ol);
  w.idx = reinterpret_cast<int32_t*>(p + oi);
  w.wts = reinterpret_cast<float*>(p + ow);
  w.h = reinterpret_cast<float*>(p + oh);
  return w;
}

static int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && cached[dev]) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  return n;
}

int launch_route(const float* Wr, const float* bias, int E, int d, const float* x, int64_t ldx,
                 int B, int k, int32_t* idx, float* wts, float* logits_out, Ws ws, hipStream_t s) {
  RouteArgs a{Wr, bias, E, d, x, ldx, B, k, idx, wts, logits_out};
  const int waves = E;
  int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(256), 0, s, a, ws);
  return (int)hipGetLastError();
}

template <int NBD, int NBF>
static int launch_experts_t(const ExpertArgs& a, Ws ws, hipStream_t s) {
  constexpr int RPW = (NBD >= 8) ? 2 : 1;
  constexpr int ROUT = 2;
  constexpr int SEGS_D = 8 * NBD, ROWS = (64 / SEGS_D) * RPW;
  const int P = a.B * a.k;
  const int Umax = P < a.L.E ? P : a.L.E;
  const int items = Umax * ((a.L.F + ROWS - 1) / ROWS);
  int blocks = (items + 3) / 4;
  const size_t shm = (size_t)a.B * frag_bytes(SEGS_D);
  if (int e = allow_lds(gateup_kernel<NBD, RPW>, shm)) return e;
  hipLaunchKernelGGL((gateup_kernel<NBD, RPW>), dim3(blocks), dim3(256), shm, s, a, ws);
  int err = (int)hipGetLastError();
  if (err) return err;
  const int dwaves = (a.L.d + ROUT - 1) / ROUT;
  int dblocks = (dwaves + 3) / 4;
  hipLaunchKernelGGL((down_kernel<NBF, ROUT>), dim3(dblocks), dim3(256),
                     (size_t)a.k * frag_bytes(8 * NBF), s, a, ws);
  return (int)hipGetLastError();
}

static int nb_class(int64_t K) {
  const int64_t nb = (K + BLK - 1) / BLK;
  return nb <= 1 ? 1 : nb <= 2 ? 2 : nb <= 4 ? 4 : 8;
}

int launch_experts(const LayerDev& L, const float* x, int64_t ldx, int B, const int32_t* idx,
                   const float* wts, int k, const float* residual, float* y, int64_t ldy, Ws ws,
                   hipStream_t s) {
  ExpertArgs a{L, x, ldx, B, k, idx, wts, residual, y, ldy};
  const int cd = nb_class(L.d), cf = nb_class(L.F);
#define HQ_CASE(D, FF) \
  if (cd == D && cf == FF) return launch_experts_t<D, FF>(a, ws, s);
  HQ_CASE(1, 1) HQ_CASE(1, 2) HQ_CASE(1, 4) HQ_CASE(1, 8)
  HQ_CASE(2, 1) HQ_CASE(2, 2) HQ_CASE(2, 4) HQ_CASE(2, 8)
  HQ_CASE(4, 1) HQ_CASE(4, 2) HQ_CASE(4, 4) HQ_CASE(4, 8)
  HQ_CASE(8, 1) HQ_CASE(8, 2) HQ_CASE(8, 4) HQ_CASE(8, 8)
#undef HQ_CASE
  return (int)hipErrorInvalidValue;
}

template <int NBD, int NBF>
static int launch_layer_t(const RouteArgs& ra, const ExpertArgs& a, Ws ws, hipStream_t s) {
  constexpr int RPW = (NBD >= 8) ? 2 : 1;
  constexpr int ROUT = 2;
  const int nwg = num_cus();
  const size_t shm = (size_t)a.B * frag_bytes(8 * NBD) + (size_t)a.k * frag_bytes(8 * NBF);
  if (int e = allow_lds(layer_kernel<NBD, NBF, RPW, ROUT>, shm)) return e;
  hipLaunchKernelGGL((layer_kernel<NBD, NBF, RPW, ROUT>), dim3(nwg), dim3(256), shm, s, ra, a, ws);
  return (int)hipGetLastError();
}

int launch_layer(const LayerDev& L, const float* Wr, const float* bias, const float* x,
                 int64_t ldx, int B, int k, int32_t* idx, float* wts, const float* residual,
                 float* y, int64_t ldy, Ws ws, hipStream_t s) {
  RouteArgs ra{Wr, bias, L.E, L.d, x, ldx, B, k, idx, wts, nullptr};
  ExpertArgs a{L, x, ldx, B, k, idx, wts, residual, y, ldy};
  const int cd = nb_class(L.d), cf = nb_class(L.F);
#define HQ_CASE(D, FF) \
  if (cd == D && cf == FF) return launch_layer_t<D, FF>(ra, a, ws, s);
  HQ_CASE(1, 1) HQ_CASE(1, 2) HQ_CASE(1, 4) HQ_CASE(1, 8)
  HQ_CASE(2, 1) HQ_CASE(2, 2) HQ_CASE(2, 4) HQ_CASE(2, 8)
  HQ_CASE(4, 1) HQ_CASE(4, 2) HQ_CASE(4, 4) HQ_CASE(4, 8)
  HQ_CASE(8, 1) HQ_CASE(8, 2) HQ_CASE(8, 4) HQ_CASE(8, 8)
#undef HQ_CASE
  return (int)hipErrorInvalidValue;
}

int launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return 0;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<uint32_t*>(p), n);
  return (int)hipGetLastError();
}

}  // namespace hq
