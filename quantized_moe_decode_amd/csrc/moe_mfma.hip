// Batched decode (2..16 tokens) of the d = 2048, F = 512 layer shape on
// MFMA matrix cores (gfx950 v_mfma_f32_16x16x32_f16).
//
// With several tokens, an expert picked by n tokens is a small GEMM: its
// rows times an n-column activation matrix.  On the VALU path every extra
// token repeats the nibble decode and four v_dot2 per code dword, so the
// cost per weight grows with n; here each code dword is decoded once into
// an f16 operand and the matrix core multiplies it against all n tokens.
//
// Operands.  A = activations (16 rows = tokens or (token, slot) pairs of
// one expert group, 32 K per step), B = weights (16 rows of the matrix, the
// same 32 K).  Lane l of the wave carries row l%16 and K chunk l/16 of both
// (8 values each), so a lane decodes exactly the code dword it loaded, and
// the output lane (g = l/16, n = l%16) holds pairs 4g..4g+3 of row n --
// the row whose block headers it loaded itself.  Inside a block the K order
// is a permutation of the block's elements (the nibble order the decode
// produces, with the odd nibbles' activations pre-divided by 16) applied to
// both operands alike.  Weights enter as 1024 + q (1024 + 16q for odd
// nibbles) straight from the bit trick of the VALU path; per block and
// column the 1024 terms and the zero point are folded back in the epilogue:
//   sum_i w_i x_i = scale * xs * (C + off) + (zero + 8 scale) * sum_i x_i
// with off = -(1024 * sum of the stored halves + 8 * sum of the f16 values
// they stand for) and xs the column's power-of-two scale.  Each block's
// product starts from a zero accumulator, so scale and zero apply exactly.
//
// Kernels (one HIP graph node each; kernel boundaries are the only
// grid-wide synchronisation, so no workgroup ever waits on another):
//   logits_mfma_kernel   router GEMV as f32 MFMA (v_mfma_f32_16x16x4_f32):
//                        16 experts x 16 tokens per tile, K split over 4
//                        workgroups x 4 waves; writes 4 partial logit sets.
//   route_topk_kernel    one wave per token (each on its own CU): partial
//                        sums + bias, top-k and weights, and the token's
//                        activations staged once in the MFMA operand format.
//                        The expert kernels group the (token, slot) pairs by
//                        expert themselves.
//   gateup_mfma_kernel   items of (group, 16 rows) in contiguous runs per
//                        workgroup; a quad of waves computes gate and up over
//                        both K halves, reduces through LDS and writes
//                        h = SiLU(g) * u.  The workgroup copies in only the
//                        staged activations of the tokens its groups need.
//   down_mfma_kernel     work items of (group, 256 output rows): stages
//                        h of the group's pairs, writes
//                        w_p * (down h_p) per pair.
//   combine_kernel       y[b] = residual[b] + sum over the k slots of token b,
//                        in slot order.
#include "hfq4_device.h"
#include "launch.h"
#include "moe_common.h"
#include "topk_device.h"

namespace hq {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int XT_STRIDE = 4096 + 16;   // bytes per staged token (256 entries of 16 B + pad)
constexpr int HT_STRIDE = 1024 + 16;   // bytes per staged h vector (64 entries + pad)
constexpr int MM_ROWS = 16;            // rows per item
constexpr int DOWN_TILES = 2;          // 16-row tiles per wave in the down kernel
constexpr int DOWN_WAVES = 8;          // waves per down workgroup
constexpr int DOWN_CHUNK = 16 * DOWN_TILES * DOWN_WAVES;   // output rows per down work item

// Code dword -> B operand: 1024+q0, 1024+q4, 1024+16q1, 1024+16q5,
// 1024+q2, 1024+q6, 1024+16q3, 1024+16q7.
__device__ __forceinline__ h8 dec8(uint32_t d) {
  const uint32_t d8 = d >> 8;
  const u32x4 v = {(d & LO4) | MAGIC, (d & HI4) | MAGIC, (d8 & LO4) | MAGIC, (d8 & HI4) | MAGIC};
  return __builtin_bit_cast(h8, v);
}

__device__ __forceinline__ f32x4 mfma16(h8 a, h8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x128>(v));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float lane_bcast(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// Max over each 16-lane row (result in every lane of the row).
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x128>(v));
  return v;
}

// Power-of-two scale putting the largest magnitude in [2, 4) (1 for 0 or
// non-finite maxima); returns 2^-e, sets xs = 2^e.
__device__ __forceinline__ float pow2_scale(float amax, float& xs) {
  int e = 0;
  if (amax > 0.f && amax < INFINITY) {
    int ex;
    frexpf(amax, &ex);
    e = ex - 2;
  }
  xs = ldexpf(1.f, e);
  return ldexpf(1.f, -e);
}

// Write the 8 elements of one code dword's entry (scaled by inv) as 16 B at
// dst in the order dec8 produces -- pair q holds elements q and q+4, odd
// pairs divided by 16 -- and add to (sum of the stored halves, sum of the
// f16 values they stand for).
__device__ __forceinline__ void put_entry(const float* v, float inv, uint8_t* dst, float& sh,
                                          float& s16) {
  h2 p[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool hi = q & 1;
    const float s = hi ? 0.0625f : 1.0f;
    const _Float16 a = (_Float16)(v[q] * inv * s), b = (_Float16)(v[q + 4] * inv * s);
    p[q] = h2{a, b};
    const float fa = (float)a, fb = (float)b;
    sh += fa + fb;
    s16 += hi ? 16.f * (fa + fb) : (fa + fb);
  }
  const u32x4 e = {as_u32(p[0]), as_u32(p[1]), as_u32(p[2]), as_u32(p[3])};
  *reinterpret_cast<u32x4*>(dst) = e;
}

// Deterministic token groups from the k selections of B tokens (in LDS):
// group ids in order of each group's first pair, members in token order, at
// most one pair per token in a group (so <= 16 members, one MFMA column
// each).  A slot repeating an expert already chosen earlier by the same
// token (possible only with caller-supplied indices) forms a group of its
// own.  Pairs with an index outside [0, E) join no group (and set `err`
// when report is true).  P <= 128 <= blockDim.x.
struct GroupScratch {
  int first[HFQ4_MAXE_DEV];
  uint32_t tokmask[GT_MAXU];
  uint64_t lead[2];
};

__device__ void build_groups_mm(const int* s_idx, int P, int k, int E, GroupTab& G,
                                GroupScratch& S, uint32_t* err, bool report) {
  const int t = threadIdx.x;
  for (int i = t; i < E; i += blockDim.x) S.first[i] = 0x7FFFFFFF;
  if (t < GT_MAXU) S.tokmask[t] = 0u;
  __syncthreads();
  int e = -1;
  bool repeat = false;
  if (t < P) {
    e = s_idx[t];
    if (e < 0 || e >= E) {
      if (report)
        __hip_atomic_fetch_or(err, 1u /*HFQ4_DEV_ERR_INDEX*/, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      e = -1;
    } else {
      for (int q = t - t % k; q < t; ++q) repeat |= (s_idx[q] == e);
      if (!repeat) atomicMin(&S.first[e], t);
    }
  }
  __syncthreads();
  const bool lead = t < P && e >= 0 && (repeat || S.first[e] == t);
  if (t < 128) {
    const uint64_t m = __ballot(lead);
    if ((t & 63) == 0) S.lead[t >> 6] = m;
  }
  __syncthreads();
  auto rank = [&](int f) {   // number of group leaders before pair f
    const uint64_t m0 = S.lead[0], m1 = S.lead[1];
    if (f < 64) return __builtin_popcountll(m0 & ((1ull << f) - 1ull));
    return __builtin_popcountll(m0) + __builtin_popcountll(m1 & ((1ull << (f - 64)) - 1ull));
  };
  int u = -1;
  if (t < P && e >= 0) {
    u = rank(repeat ? t : S.first[e]);
    atomicOr(&S.tokmask[u], 1u << (t / k));
    if (lead) G.gexp[u] = e;
  }
  if (t == 0) G.U = __builtin_popcountll(S.lead[0]) + __builtin_popcountll(S.lead[1]);
  __syncthreads();
  if (u >= 0) {
    const uint32_t tm = S.tokmask[u];
    const int b = t / k;
    G.gmem[u][__builtin_popcount(tm & ((1u << b) - 1u))] = (uint8_t)t;
    if (lead) G.gcnt[u] = __builtin_popcount(tm);
  }
  __syncthreads();
}

// ====================================================================== router

// Partial router logits: part[ks][b][e] = sum over K split ks of
// Wr[e][i] * x[b][i].  A = x (16 tokens; rows past B read zeros), B = Wr
// (16 experts), 4 K per MFMA: lane (n, c) loads a float4 at K offset 4c of
// every 16-wide K step and feeds element j to the j-th MFMA, so both
// operands use the same K assignment.  The four waves of a workgroup take
// consecutive quarters of the split and meet in LDS in a fixed order.
__global__ void __launch_bounds__(256) logits_mfma_kernel(RouteArgs a, float* __restrict__ part,
                                                          uint64_t* trace) {
  __shared__ f32x4 red[4][64];
  const int wg = blockIdx.x + gridDim.x * blockIdx.y;
  trace_point_at(trace, TK_LOGITS, wg, 0);
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n16 = lane & 15, c = lane >> 4;
  const int rt = blockIdx.x, ks = blockIdx.y;
  const int Kq = ((a.d + LG_KS * 64 - 1) / (LG_KS * 64)) * 64;   // per split, multiple of 64
  const int Kw = Kq / 4;                                          // per wave, multiple of 16
  const int k_lo = ks * Kq + wv * Kw;
  const int row = rt * 16 + n16;
  const uint32_t xbytes = (uint32_t)(((int64_t)(a.B - 1) * a.ldx + a.d) * 4);
  const uint32_t wbytes = (uint32_t)((int64_t)a.E * a.d * 4);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, xbytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.Wr, wbytes);
  const bool tok_ok = n16 < a.B, row_ok = row < a.E;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = k_lo; k0 < k_lo + Kw; k0 += 8 * 16) {
    u32x4 xv[8], wv4[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int ki = k0 + 16 * s + 4 * c;
      const bool kin = ki < a.d && ki < k_lo + Kw;
      xv[s] = bload16(rx, (tok_ok && kin) ? (uint32_t)(((int64_t)n16 * a.ldx + ki) * 4) : xbytes);
      wv4[s] = bload16(rw, (row_ok && kin) ? (uint32_t)(((int64_t)row * a.d + ki) * 4) : wbytes);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(xv[s].x), as_f32(wv4[s].x), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(xv[s].y), as_f32(wv4[s].y), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(xv[s].z), as_f32(wv4[s].z), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(xv[s].w), as_f32(wv4[s].w), acc, 0, 0, 0);
    }
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0) {
    const f32x4 t = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    const float tv[4] = {t.x, t.y, t.z, t.w};
    // lane (c, n16) holds tokens 4c..4c+3 of expert row
    if (row_ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 4 * c + i;
        if (b < a.B) part[((int64_t)ks * a.B + b) * a.E + row] = tv[i];
      }
    }
  }
  trace_point_at(trace, TK_LOGITS, wg, 1);
}

struct BatchRouteArgs {
  const float* part;      // [LG_KS][B][E] partial logits
  const float* bias;      // [E] or null
  int E, B, k;
  int32_t* idx_out;       // [B][k]
  float* wts_out;         // [B][k]
  float* logits_out;      // [B][E] or null
  int32_t* idx_copy;      // workspace copies or null
  float* wts_copy;
  uint32_t* err;
  uint64_t* trace;
  const float* x;         // [B][ldx] activations to stage, or null
  int64_t ldx;
  int d;
  uint8_t* xg;            // [B][XG_STRIDE] staged activations (see stage_token)
};

template <int PER>
struct RouteLoads {
  uint32_t raw[LG_KS][PER];
  uint32_t rb[PER];
};

// Issue every load of one token's routing: the LG_KS partial logits and the
// bias of expert 64c + lane (coalesced).
template <int PER>
__device__ __forceinline__ void route_load(const BatchRouteArgs& r, int b, RouteLoads<PER>& L) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(r.part, (uint32_t)((int64_t)LG_KS * r.B * r.E * 4));
  const __amdgpu_buffer_rsrc_t rbias = make_rsrc(r.bias, r.bias ? (uint32_t)r.E * 4u : 0u);
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int e = 64 * c + lane;
#pragma unroll
    for (int p = 0; p < LG_KS; ++p)
      L.raw[p][c] = bload4(rp, e < r.E ? (uint32_t)((((int64_t)p * r.B + b) * r.E + e) * 4)
                                       : 0xFFFFFFF0u);
    L.rb[c] = bload4(rbias, (uint32_t)e * 4u);   // zero without a bias or past E
  }
}

// Sum, top-k and weights of one token from its loads.
template <int PER>
__device__ void route_token(const BatchRouteArgs& r, int b, const RouteLoads<PER>& L, float* lg) {
  const int lane = threadIdx.x & 63;
  // lane l sums expert 64c + l over the partial sets (+ bias) into LDS; the
  // top-k then reads its own PER consecutive experts
  int nan_seen = 0;
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int e = 64 * c + lane;
    if (e < r.E) {
      float l = 0.f;
#pragma unroll
      for (int p = 0; p < LG_KS; ++p) l += as_f32(L.raw[p][c]);
      if (r.bias) l += as_f32(L.rb[c]);
      if (r.logits_out) r.logits_out[(int64_t)b * r.E + e] = l;
      lg[e] = l;
      nan_seen |= __builtin_isnan(l);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  trace_point(r.trace, TK_TOPK, 2);
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane * PER + i;
    key[i] = e < r.E ? okey(lg[e]) : 0u;
  }
  int e;
  float w;
  topk_keys<PER>(key, r.E, r.k, e, w, nullptr, nullptr);
  trace_point(r.trace, TK_TOPK, 3);
  if (lane < r.k) {
    const int p = b * r.k + lane;
    r.idx_out[p] = e;
    r.wts_out[p] = w;
    if (r.idx_copy) {
      r.idx_copy[p] = e;
      r.wts_copy[p] = w;
    }
  }
  if (__any(nan_seen) && lane == 0)
    __hip_atomic_fetch_or(r.err, 4u /*HFQ4_DEV_ERR_NONFINITE*/, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
}

// Stage one token's activations (one wave) into the MFMA A-operand format
// at dst: 256 entries of 16 B (entry o = elements 8o..8o+7 scaled by 2^-e,
// in dec8 order), then per block (off, sx) as 8 float2, then xs = 2^e.
// Lane l takes entries o = l + 64m, so one load instruction covers 2 KB of
// x; entry o belongs to block o / 32 (2m for lanes 0-31, 2m+1 above).
constexpr int XG_ENTRIES = 4096, XG_BLK = 4096, XG_XS = 4096 + 64;
static_assert(XG_STRIDE >= XG_XS + 4, "staged token layout");

__device__ void stage_token(const float* __restrict__ xb, int d, uint8_t* dst) {
  const int lane = threadIdx.x & 63;
  float v[4][8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e0 = 8 * (lane + 64 * m);
    f32x4 t0 = f32x4{0.f, 0.f, 0.f, 0.f}, t1 = t0;
    if (e0 < d) t0 = *reinterpret_cast<const f32x4*>(xb + e0);
    if (e0 + 4 < d) t1 = *reinterpret_cast<const f32x4*>(xb + e0 + 4);
    v[m][0] = t0.x; v[m][1] = t0.y; v[m][2] = t0.z; v[m][3] = t0.w;
    v[m][4] = t1.x; v[m][5] = t1.y; v[m][6] = t1.z; v[m][7] = t1.w;
  }
  float am = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[m][i]));
  float xs;
  const float inv = pow2_scale(wave_max_f(am), xs);
  float2* blk = reinterpret_cast<float2*>(dst + XG_BLK);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float sh = 0.f, s16 = 0.f, sx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) sx += v[m][i];
    put_entry(v[m], inv, dst + XG_ENTRIES * 0 + 16 * (lane + 64 * m), sh, s16);
    // block sums over 32 lanes, fixed order
    sh = row_sum16(sh);
    s16 = row_sum16(s16);
    sx = row_sum16(sx);
    const float lo_sh = lane_bcast(sh, 0) + lane_bcast(sh, 16);
    const float hi_sh = lane_bcast(sh, 32) + lane_bcast(sh, 48);
    const float lo_16 = lane_bcast(s16, 0) + lane_bcast(s16, 16);
    const float hi_16 = lane_bcast(s16, 32) + lane_bcast(s16, 48);
    const float lo_sx = lane_bcast(sx, 0) + lane_bcast(sx, 16);
    const float hi_sx = lane_bcast(sx, 32) + lane_bcast(sx, 48);
    if (lane == 0) {
      blk[2 * m] = make_float2(-(1024.f * lo_sh + 8.f * lo_16), lo_sx);
      blk[2 * m + 1] = make_float2(-(1024.f * hi_sh + 8.f * hi_16), hi_sx);
    }
  }
  if (lane == 0) *reinterpret_cast<float*>(dst + XG_XS) = xs;
}

// One single-wave workgroup per token: partial sums + bias, top-k, weights
// (WITH_TOPK), and the token's activations staged for the expert kernels
// (when r.xg is set).  Tokens run on different CUs in parallel; the expert
// kernels build the token groups themselves from the indices
// (deterministically, so every workgroup sees the same groups).
template <bool WITH_TOPK>
__global__ void __launch_bounds__(64) route_topk_kernel(BatchRouteArgs r) {
  __shared__ float lg[HFQ4_MAXE_DEV];
  trace_point(r.trace, TK_TOPK, 0);
  const int b = blockIdx.x;
  // the routing loads go out first, the activation staging overlaps them
  if (!WITH_TOPK) {
    if (r.xg) stage_token(r.x + (int64_t)b * r.ldx, r.d, r.xg + (int64_t)b * XG_STRIDE);
  } else if (r.E <= 256) {
    RouteLoads<4> L;
    route_load<4>(r, b, L);
    if (r.xg) stage_token(r.x + (int64_t)b * r.ldx, r.d, r.xg + (int64_t)b * XG_STRIDE);
    route_token<4>(r, b, L, lg);
  } else if (r.E <= 512) {
    RouteLoads<8> L;
    route_load<8>(r, b, L);
    if (r.xg) stage_token(r.x + (int64_t)b * r.ldx, r.d, r.xg + (int64_t)b * XG_STRIDE);
    route_token<8>(r, b, L, lg);
  } else {
    RouteLoads<16> L;
    route_load<16>(r, b, L);
    if (r.xg) stage_token(r.x + (int64_t)b * r.ldx, r.d, r.xg + (int64_t)b * XG_STRIDE);
    route_token<16>(r, b, L, lg);
  }
  trace_point(r.trace, TK_TOPK, 1);
}

// ====================================================================== gate / up

// A workgroup of 16 waves = 4 quads; a quad takes one (group, 16-row tile)
// item at a time: its waves compute gate K-half 0, gate K-half 1, up K-half
// 0 and up K-half 1 (4 blocks each, all loads in flight at once), the
// partial tiles meet in LDS, and the first wave writes h = SiLU(g) * u.
__global__ void __launch_bounds__(1024) gateup_mfma_kernel(ExpertArgs a, Ws ws) {
  extern __shared__ __align__(16) uint8_t xt[];      // [B][XT_STRIDE]
  __shared__ GroupTab G;
  __shared__ GroupScratch GS;
  __shared__ int s_idx[MAXP];
  __shared__ float2 s_blk[HFQ4_MAXB_DEV][8];         // per token, block: (off, sx)
  __shared__ float s_xs[HFQ4_MAXB_DEV];
  __shared__ uint32_t s_need;
  __shared__ f32x4 red[4][3][64];                    // partial tiles of roles 1..3
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int quad = wv >> 2, role = wv & 3;
  const int B = a.B, k = a.k, P = B * k, F = a.L.F;
  trace_point(ws.trace, TK_GATEUP, 0);
  if ((int)threadIdx.x < P) s_idx[threadIdx.x] = a.idx[threadIdx.x];
  __syncthreads();
  build_groups_mm(s_idx, P, k, a.L.E, G, GS, ws.err, blockIdx.x == 0);
  trace_point(ws.trace, TK_GATEUP, 1);

  // 1. this workgroup's items: a contiguous run of (group, 16-row tile)
  const int tiles = F / MM_ROWS;                 // 32
  const int items = G.U * tiles;
  const int per = (items + gridDim.x - 1) / gridDim.x;
  const int i0 = blockIdx.x * per;
  const int i1 = min(items, i0 + per);
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    if (i0 < i1)
      for (int u = i0 / tiles; u <= (i1 - 1) / tiles; ++u) {
        for (int q = 0; q < G.gcnt[u]; ++q) m |= 1u << (G.gmem[u][q] / k);
      }
    s_need = m;
  }
  __syncthreads();

  // 2. the wave's first item: its role's 4 blocks, every load in flight
  constexpr int64_t ROWB = 8 * BLK_BYTES;
  const int n16 = lane & 15, c = lane >> 4;
  const int mat = role >> 1, kh = role & 1;
  const uint8_t* base = mat ? a.L.up : a.L.gate;
  const int64_t stride = mat ? a.L.su : a.L.sg;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, mat ? a.L.up_bytes : a.L.gate_bytes);
  u32x4 cd[4][2];
  u32x2 hd[4];
  auto issue = [&](int it) {
    const int u = it / tiles, tile = it - u * tiles;
    const uint32_t rowoff = (uint32_t)(G.gexp[u] * stride +
                                       (int64_t)(tile * MM_ROWS + n16) * ROWB + kh * 4 * BLK_BYTES);
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) {
      hd[bk] = bload8(rs, rowoff + bk * BLK_BYTES);
      cd[bk][0] = bload16(rs, rowoff + bk * BLK_BYTES + 8 + 16 * c);
      cd[bk][1] = bload16(rs, rowoff + bk * BLK_BYTES + 8 + 64 + 16 * c);
    }
  };
  // 3. the needed tokens' staged activations: every 16-byte chunk load in
  //    flight first (ahead of the weights in the memory queue), then the
  //    first item's weight loads, then the chunks go to LDS
  constexpr int XG_CHUNKS = (XG_XS + 4 + 15) / 16;   // 261 chunks of a staged token
  constexpr int XG_ITERS = (HFQ4_MAXB_DEV * XG_CHUNKS + 1023) / 1024;
  u32x4 xc[XG_ITERS];
  const uint32_t need = s_need;
#pragma unroll
  for (int j = 0; j < XG_ITERS; ++j) {
    const int ci = threadIdx.x + 1024 * j;
    const int tb = ci / XG_CHUNKS, ch = ci - tb * XG_CHUNKS;
    xc[j] = u32x4{0u, 0u, 0u, 0u};
    if (tb < B && ((need >> tb) & 1u))
      xc[j] = *reinterpret_cast<const u32x4*>(ws.xg + (int64_t)tb * XG_STRIDE + 16 * ch);
  }
  int it = i0 + quad;
  if (it < i1) issue(it);
#pragma unroll
  for (int j = 0; j < XG_ITERS; ++j) {
    const int ci = threadIdx.x + 1024 * j;
    const int tb = ci / XG_CHUNKS, ch = ci - tb * XG_CHUNKS;
    if (tb < B && ((need >> tb) & 1u)) {
      if (ch < 256) {
        *reinterpret_cast<u32x4*>(xt + tb * XT_STRIDE + 16 * ch) = xc[j];
      } else if (ch < 260) {   // (off, sx) of blocks 2(ch-256), 2(ch-256)+1
        s_blk[tb][2 * (ch - 256)] = make_float2(as_f32(xc[j].x), as_f32(xc[j].y));
        s_blk[tb][2 * (ch - 256) + 1] = make_float2(as_f32(xc[j].z), as_f32(xc[j].w));
      } else {
        s_xs[tb] = as_f32(xc[j].x);
      }
    }
  }
  __syncthreads();
  trace_point(ws.trace, TK_GATEUP, 3);

  // 4. rounds of one item per quad (uniform trip count: every wave meets
  //    every barrier)
  const int rounds = (i1 - i0 + 3) / 4;
  for (int rd = 0; rd < rounds; ++rd) {
    const bool live = it < i1;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int n = 0, u = 0, tile = 0;
    if (live) {
      u = it / tiles;
      tile = it - u * tiles;
      n = G.gcnt[u];
      // A operand source: member n16 of the group (zeros past the group)
      const int tok_a = n16 < n ? G.gmem[u][n16] / k : -1;
      const uint8_t* arow = xt + (tok_a >= 0 ? tok_a : 0) * XT_STRIDE + 16 * (4 * c) + kh * 4 * 512;
      int tok_c[4];
      float xs_c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * c + i;
        tok_c[i] = m < n ? G.gmem[u][m] / k : -1;
        xs_c[i] = tok_c[i] >= 0 ? s_xs[tok_c[i]] : 0.f;
      }
#pragma unroll
      for (int bk = 0; bk < 4; ++bk) {
        // the block's 8 A operands first, then two independent MFMA chains
        h8 av[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // entry 32 (4 kh + bk) + 16t + 4c + i of the token; rows past the
            // group read token 0's slot: their output rows are never used
            av[t][i] = *reinterpret_cast<const h8*>(arow + 16 * (32 * bk + 16 * t + i));
          }
        f32x4 c2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t q0[4] = {cd[bk][0].x, cd[bk][0].y, cd[bk][0].z, cd[bk][0].w};
          const uint32_t q1[4] = {cd[bk][1].x, cd[bk][1].y, cd[bk][1].z, cd[bk][1].w};
          c2[0] = mfma16(av[0][i], dec8(q0[i]), c2[0]);
          c2[1] = mfma16(av[1][i], dec8(q1[i]), c2[1]);
        }
        const f32x4 cb = c2[0] + c2[1];
        const float scale = as_f32(hd[bk].x), zero = as_f32(hd[bk].y);
        const float zp8 = __builtin_fmaf(8.f, scale, zero);
        const float cbv[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (tok_c[i] >= 0) {
            const float2 ob = s_blk[tok_c[i]][4 * kh + bk];
            acc[i] += __builtin_fmaf(scale * xs_c[i], cbv[i] + ob.x, zp8 * ob.y);
          }
        }
      }
    }
    // next item's loads go out before the exchange
    const int next = it + 4;
    if (next < i1) issue(next);
    if (role > 0) red[quad][role - 1][lane] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    __syncthreads();
    if (role == 0 && live) {
      const f32x4 g1 = red[quad][0][lane], u0 = red[quad][1][lane], u1 = red[quad][2][lane];
      const float gv[4] = {acc[0] + g1.x, acc[1] + g1.y, acc[2] + g1.z, acc[3] + g1.w};
      const float uv[4] = {u0.x + u1.x, u0.y + u1.y, u0.z + u1.z, u0.w + u1.w};
      const int row = tile * MM_ROWS + n16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * c + i;
        if (m < n) ws.h[(int64_t)G.gmem[u][m] * F + row] = silu_mul(gv[i], uv[i]);
      }
    }
    __syncthreads();   // red is reused by the next round
    it = next;
  }
  trace_point(ws.trace, TK_GATEUP, 5);
}

// ====================================================================== down + combine

__global__ void __launch_bounds__(64 * DOWN_WAVES) down_mfma_kernel(ExpertArgs a, Ws ws) {
  __shared__ __align__(16) uint8_t ht[GT_MAXM * HT_STRIDE];   // [member][HT_STRIDE]
  __shared__ float2 s_blk[GT_MAXM][2];
  __shared__ float s_xs[GT_MAXM];
  __shared__ GroupTab G;
  __shared__ GroupScratch GS;
  __shared__ int s_idx[MAXP];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int B = a.B, k = a.k, d = a.L.d, F = a.L.F;
  if ((int)threadIdx.x < B * k) s_idx[threadIdx.x] = a.idx[threadIdx.x];
  __syncthreads();
  build_groups_mm(s_idx, B * k, k, a.L.E, G, GS, ws.err, false);
  const int nch = (d + DOWN_CHUNK - 1) / DOWN_CHUNK;
  const int U = G.U;
  const int items = U * nch;
  constexpr int64_t ROWB = 2 * BLK_BYTES;
  const int n16 = lane & 15, c = lane >> 4;
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.L.down, a.L.down_bytes);
  trace_point(ws.trace, TK_DOWN, 0);
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int u = it / nch, ch = it - u * nch;
    const int n = G.gcnt[u], e = G.gexp[u];

    // 1. weight loads: wave wv owns rows ch*DOWN_CHUNK + 16*DOWN_TILES*wv .. (DOWN_TILES tiles)
    u32x4 cd[DOWN_TILES][2][2];
    u32x2 hd[DOWN_TILES][2];
#pragma unroll
    for (int tl = 0; tl < DOWN_TILES; ++tl) {
      const int row = ch * DOWN_CHUNK + 16 * (DOWN_TILES * wv + tl) + n16;
      const uint32_t ro = row < d ? (uint32_t)(e * a.L.sd + (int64_t)row * ROWB) : a.L.down_bytes;
#pragma unroll
      for (int bk = 0; bk < 2; ++bk) {
        hd[tl][bk] = bload8(rd, ro + bk * BLK_BYTES);
        cd[tl][bk][0] = bload16(rd, ro + bk * BLK_BYTES + 8 + 16 * c);
        cd[tl][bk][1] = bload16(rd, ro + bk * BLK_BYTES + 8 + 64 + 16 * c);
      }
    }

    // 2. stage h of the members: 32 threads per member (half a wave), thread
    //    s takes entries o = s + 32q (q < 2, block q), so the 32 threads read
    //    1 KB contiguously; scale per member over its F values
    {
      const int m = threadIdx.x >> 5, s = threadIdx.x & 31;
      const bool live = m < n;
      const int p = live ? G.gmem[u][m] : 0;
      float v[2][8];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int64_t e0 = (int64_t)p * F + 8 * (s + 32 * q);
        f32x4 h0 = f32x4{0.f, 0.f, 0.f, 0.f}, h1 = h0;
        if (live) {
          h0 = *reinterpret_cast<const f32x4*>(ws.h + e0);
          h1 = *reinterpret_cast<const f32x4*>(ws.h + e0 + 4);
        }
        v[q][0] = h0.x; v[q][1] = h0.y; v[q][2] = h0.z; v[q][3] = h0.w;
        v[q][4] = h1.x; v[q][5] = h1.y; v[q][6] = h1.z; v[q][7] = h1.w;
      }
      float am = 0.f;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[q][i]));
      am = row_max16(am);
      am = fmaxf(am, __shfl_xor(am, 16, 64));   // the member's 32 lanes
      float xs;
      const float inv = pow2_scale(am, xs);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float sh = 0.f, s16 = 0.f, sx = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sx += v[q][i];
        put_entry(v[q], inv, ht + m * HT_STRIDE + 16 * (s + 32 * q), sh, s16);
        sh = row_sum16(sh);
        s16 = row_sum16(s16);
        sx = row_sum16(sx);
        sh += __shfl_xor(sh, 16, 64);
        s16 += __shfl_xor(s16, 16, 64);
        sx += __shfl_xor(sx, 16, 64);
        if (s == 0) s_blk[m][q] = make_float2(-(1024.f * sh + 8.f * s16), sx);
      }
      if (s == 0) s_xs[m] = xs;
    }
    __syncthreads();
    if (it == (int)blockIdx.x) trace_point(ws.trace, TK_DOWN, 1);

    // 3. MFMA per tile, epilogue per block, weighted partial per member
    const bool a_live = n16 < n;
    const uint8_t* arow = ht + (a_live ? n16 : 0) * HT_STRIDE + 16 * (4 * c);
    if (it == (int)blockIdx.x) trace_point(ws.trace, TK_DOWN, 3);
    int pc[4];
    float wc[4], xsc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * c + i;
      pc[i] = m < n ? G.gmem[u][m] : -1;
      wc[i] = pc[i] >= 0 ? a.wts[pc[i]] : 0.f;
      xsc[i] = pc[i] >= 0 ? s_xs[m] : 0.f;
    }
#pragma unroll
    for (int tl = 0; tl < DOWN_TILES; ++tl) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bk = 0; bk < 2; ++bk) {
        h8 av[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            av[t][i] = *reinterpret_cast<const h8*>(arow + 16 * (32 * bk + 16 * t + i));
          }
        f32x4 c2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t q0[4] = {cd[tl][bk][0].x, cd[tl][bk][0].y, cd[tl][bk][0].z, cd[tl][bk][0].w};
          const uint32_t q1[4] = {cd[tl][bk][1].x, cd[tl][bk][1].y, cd[tl][bk][1].z, cd[tl][bk][1].w};
          c2[0] = mfma16(av[0][i], dec8(q0[i]), c2[0]);
          c2[1] = mfma16(av[1][i], dec8(q1[i]), c2[1]);
        }
        const f32x4 cb = c2[0] + c2[1];
        const float scale = as_f32(hd[tl][bk].x), zero = as_f32(hd[tl][bk].y);
        const float zp8 = __builtin_fmaf(8.f, scale, zero);
        const float cbv[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (pc[i] >= 0) {
            const float2 ob = s_blk[4 * c + i][bk];
            acc[i] += __builtin_fmaf(scale * xsc[i], cbv[i] + ob.x, zp8 * ob.y);
          }
        }
      }
      const int row = ch * DOWN_CHUNK + 16 * (DOWN_TILES * wv + tl) + n16;
      if (row < d) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (pc[i] >= 0) ws.ypart[(int64_t)pc[i] * d + row] = wc[i] * acc[i];
      }
    }
    if (it == (int)blockIdx.x) trace_point(ws.trace, TK_DOWN, 4);
    __syncthreads();   // ht is restaged by the next item
  }
  trace_point(ws.trace, TK_DOWN, 2);
}

// y[b][r] = residual[b][r] + sum_j w_j y_{e_j}[r] over the valid slots, in
// slot order (the weights are already in ypart).
__global__ void __launch_bounds__(256) combine_kernel(ExpertArgs a, Ws ws) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x, b = blockIdx.y;
  const int d = a.L.d, k = a.k;
  const int wg = blockIdx.x + gridDim.x * blockIdx.y;
  trace_point_at(ws.trace, TK_DOWN, wg, 5);
  if (r >= d) return;
  // every load at once: ypart rows of invalid slots are read but not added
  float part[MAXK];
  int ej[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    const int p = b * k + (j < k ? j : 0);
    ej[j] = a.idx[p];
    part[j] = ws.ypart[(int64_t)p * d + r];
  }
  float y = a.res ? a.res[b * a.ldy + r] : 0.f;
#pragma unroll
  for (int j = 0; j < MAXK; ++j)
    if (j < k && ej[j] >= 0 && ej[j] < a.L.E) y += part[j];
  a.y[b * a.ldy + r] = y;
  trace_point_at(ws.trace, TK_DOWN, wg, 6);
}

// ====================================================================== host

int launch_logits_batched(const RouteArgs& ra, float* part, hipStream_t s) {
  hipLaunchKernelGGL(logits_mfma_kernel, dim3((ra.E + 15) / 16, LG_KS), dim3(256), 0, s, ra, part,
                     get_trace());
  return (int)hipGetLastError();
}

int launch_route_batched(const RouteArgs& ra, const float* part, int32_t* idx_copy,
                         float* wts_copy, uint8_t* xg, uint32_t* err, hipStream_t s) {
  BatchRouteArgs r{part, ra.bias, ra.E, ra.B, ra.k, ra.idx_out, ra.wts_out, ra.logits_out,
                   idx_copy, wts_copy, err, get_trace(), ra.x, ra.ldx, ra.d, xg};
  hipLaunchKernelGGL(route_topk_kernel<true>, dim3(ra.B), dim3(64), 0, s, r);
  return (int)hipGetLastError();
}

int launch_stage_batched(const float* x, int64_t ldx, int B, int d, uint8_t* xg, hipStream_t s) {
  BatchRouteArgs r{};
  r.B = B;
  r.x = x;
  r.ldx = ldx;
  r.d = d;
  r.xg = xg;
  r.trace = get_trace();
  hipLaunchKernelGGL(route_topk_kernel<false>, dim3(B), dim3(64), 0, s, r);
  return (int)hipGetLastError();
}

int launch_experts_batched(const ExpertArgs& a, Ws ws, int nwg, hipStream_t s) {
  const size_t shm = (size_t)a.B * XT_STRIDE;
  if (int e = allow_lds(gateup_mfma_kernel, shm)) return e;
  hipLaunchKernelGGL(gateup_mfma_kernel, dim3(nwg), dim3(1024), shm, s, a, ws);
  int err = (int)hipGetLastError();
  if (err) return err;
  const int P = a.B * a.k;
  const int umax = P < a.L.E ? P : a.L.E;
  const int nch = (a.L.d + DOWN_CHUNK - 1) / DOWN_CHUNK;
  const int grid = umax * nch < 2 * nwg ? umax * nch : 2 * nwg;
  hipLaunchKernelGGL(down_mfma_kernel, dim3(grid), dim3(64 * DOWN_WAVES), 0, s, a, ws);
  err = (int)hipGetLastError();
  if (err) return err;
  hipLaunchKernelGGL(combine_kernel, dim3((a.L.d + 255) / 256, a.B), dim3(256), 0, s, a, ws);
  return (int)hipGetLastError();
}

}  // namespace hq
