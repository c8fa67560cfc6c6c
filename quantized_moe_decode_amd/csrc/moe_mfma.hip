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
//   sum_i w_i x_i = scale * xs * (C + off) + (zero + 8 scale) * sx
// with Sa = sum of the stored halves, S16 = sum of the values they stand
// for (odd pairs x16), off = -(1024 Sa + 8 S16), sx = xs * S16 and xs the
// column's power-of-two scale.  Sa and S16 come from one more MFMA chain
// per block against constant B rows, once per staged column.  Each block's
// product starts from a zero accumulator, so scale and zero apply exactly.
//
// Kernels (one HIP graph node each; apart from the routing exchange inside
// the gate/up kernel, kernel boundaries are the grid-wide synchronisation):
//   logits_mfma_kernel   router GEMV as f32 MFMA (v_mfma_f32_16x16x4_f32)
//                        for more than LG_VALU_MAXB tokens: 8 experts x 16
//                        tokens per tile, K split over 4 workgroups x 4
//                        waves; writes 4 partial logit sets.  Fewer tokens
//                        take the VALU router of moe.hip, which writes whole
//                        logits into set 0 (lg_sets).
//   gateup_mfma_kernel   workgroup b < B routes token b from the partial
//                        logits (sums + bias, top-k, weights) and publishes
//                        the selection, which every workgroup gathers
//                        (tagged words, xchg_device.h) while staging every
//                        token's activations in LDS in the MFMA operand
//                        format; the (token, slot) pairs are grouped by
//                        expert; items of
//                        (group, 16 rows) in contiguous runs per workgroup,
//                        a quad of waves computes gate and up over both K
//                        halves, reduces through LDS and writes
//                        h = SiLU(g) * u as f16 operand entries with one
//                        power-of-two exponent per (pair, 16-row tile).
//   route_topk_kernel    routing only (moe_route_topk): the same routing
//                        functions, one single-wave workgroup per token.
//   down_rows_kernel     8 output rows of every token per workgroup: stages
//                        h of all pairs, runs every group's down tile and
//                        sums w_p * (down h_p) over the slots onto the
//                        residual (no per-slot buffer, no combine kernel).
#include "hfq4_device.h"
#include "launch.h"
#include "moe_common.h"
#include "topk_device.h"
#include "xchg_device.h"

namespace hq {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int XT_STRIDE = 4096 + 16;   // bytes per staged token (256 entries of 16 B + pad)
constexpr int HT_STRIDE = 1024 + 16;   // bytes per staged h vector (64 entries + pad)
constexpr int MM_ROWS = 16;            // rows per item

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

// Exponent e with amax * 2^-e in [2, 4); H_EMPTY for a zero maximum (so it
// never wins a maximum over tiles), 0 for a non-finite one.
constexpr int H_EMPTY = -128;
__device__ __forceinline__ int pow2_exp(float amax) {
  if (!(amax > 0.f)) return H_EMPTY;
  if (!(amax < INFINITY)) return 0;
  int ex;
  frexpf(amax, &ex);
  return ex - 2;
}
// 2^d as a pair of f16 (d <= 0; 0 below the smallest subnormal).
__device__ __forceinline__ h2 f16_pow2_pair(int dlt) {
  uint32_t b = 0u;
  if (dlt >= -14) b = (uint32_t)(dlt + 15) << 10;
  else if (dlt >= -24) b = 1u << (dlt + 24);
  return as_h2(b | (b << 16));
}

// Write the 8 elements of one code dword's entry (scaled by inv) as 16 B at
// dst in the order dec8 produces: pair q holds elements q and q+4, odd pairs
// divided by 16.
__device__ __forceinline__ void put_entry(const float* v, float inv, uint8_t* dst) {
  const float i16 = inv * 0.0625f;
  const h2 p0 = {(_Float16)(v[0] * inv), (_Float16)(v[4] * inv)};
  const h2 p1 = {(_Float16)(v[1] * i16), (_Float16)(v[5] * i16)};
  const h2 p2 = {(_Float16)(v[2] * inv), (_Float16)(v[6] * inv)};
  const h2 p3 = {(_Float16)(v[3] * i16), (_Float16)(v[7] * i16)};
  *reinterpret_cast<u32x4*>(dst) = u32x4{as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)};
}

// Per-block sums of staged operand rows on the matrix cores.  For up to 16
// rows (row n16 of the A operand at base + n16 * stride, in the layout
// put_entry writes; rows >= nrows repeat row 0 and their sums are
// meaningless) and block bk (32 entries), a chain of 8 MFMAs against a
// constant B -- row 0 all ones, row 1 the pattern 1, 1, 16, 16 (the values
// the stored halves stand for), other rows zero -- gives Sa = sum of the
// stored halves and S16 = sum of the values they stand for.  Lanes (c, 1)
// end with (Sa, S16) of rows 4c..4c+3 in sa[i], s16[i].  With them,
// sum_i w_i v_i = xs (scale (C - 1024 Sa) + zero S16) for the block's
// dequantized weights w and the row's values v = xs * (stored halves).
__device__ __forceinline__ void block_sums_mfma(const uint8_t* base, int stride, int nrows, int bk,
                                                float* sa, float* s16) {
  const int lane = threadIdx.x & 63, n16 = lane & 15, c = lane >> 4;
  const _Float16 o1 = n16 < 2 ? (_Float16)1.f : (_Float16)0.f;
  const _Float16 o16 = n16 == 0 ? (_Float16)1.f : n16 == 1 ? (_Float16)16.f : (_Float16)0.f;
  const h8 bpat = {o1, o1, o16, o16, o1, o1, o16, o16};
  const uint8_t* arow = base + (n16 < nrows ? n16 : 0) * stride + 16 * (4 * c);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = mfma16(*reinterpret_cast<const h8*>(arow + 16 * (32 * bk + 16 * t + i)), bpat, acc);
  const int src = lane & ~15;   // lane (c, 0) holds Sa
  sa[0] = __shfl(acc.x, src, 64);
  sa[1] = __shfl(acc.y, src, 64);
  sa[2] = __shfl(acc.z, src, 64);
  sa[3] = __shfl(acc.w, src, 64);
  s16[0] = acc.x;
  s16[1] = acc.y;
  s16[2] = acc.z;
  s16[3] = acc.w;
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
                                GroupScratch& S, uint32_t* err, bool report, bool may_repeat) {
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
      if (may_repeat)
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

// Partial router logits: part[ks][b][e] (rows padded to a multiple of 4
// experts, so that a lane can read 4 consecutive experts at once) = sum over K split ks of
// Wr[e][i] * x[b][i].  A = x (16 tokens; rows past B read zeros), B = Wr
// (8 experts in the tile's first 8 rows, the other 8 load nothing), 4 K per
// MFMA: lane (n, c) loads a float4 at K offset 4c of every 16-wide K step
// and feeds element j to the j-th MFMA, so both operands use the same K
// assignment.  The four waves of a workgroup take consecutive quarters of
// the split and meet in LDS in a fixed order.  Every workgroup reads x of
// all tokens over its quarter (32 KB at 16 tokens) besides its rows of Wr;
// 8-expert tiles put 256 workgroups on the 512 experts of the skewed layer
// instead of 128 (0.25 - 0.3 us faster per step at 5 - 16 tokens than
// 16-expert tiles, same bits).
__global__ void __launch_bounds__(256) logits_mfma_kernel(RouteArgs a, float* __restrict__ part,
                                                          uint64_t* trace, uint32_t* gen) {
  __shared__ f32x4 red[4][64];
  const int wg = blockIdx.x + gridDim.x * blockIdx.y;
  trace_point_at(trace, TK_LOGITS, wg, 0);
  // the call counter for the gate/up kernel's routing exchange: one writer,
  // read after this launch ends
  if (gen && wg == 0 && threadIdx.x == 0) gen[0] = gen[0] + 1u;
  const int wv = wave_id(), lane = threadIdx.x & 63;
  const int n16 = lane & 15, c = lane >> 4;
  const int rt = blockIdx.x, ks = blockIdx.y;
  constexpr int LG_ROWS = 8;   // expert rows per workgroup (the tile's other 8 load nothing)
  const int Kq = ((a.d + LG_KS * 64 - 1) / (LG_KS * 64)) * 64;   // per split, multiple of 64
  const int Kw = Kq / 4;                                          // per wave, multiple of 16
  const int k_lo = ks * Kq + wv * Kw;
  const int row = rt * LG_ROWS + n16;
  const uint32_t xbytes = (uint32_t)(((int64_t)(a.B - 1) * a.ldx + a.d) * 4);
  const uint32_t wbytes = (uint32_t)((int64_t)a.E * a.d * 4);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, xbytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.Wr, wbytes);
  const bool tok_ok = n16 < a.B, row_ok = n16 < LG_ROWS && row < a.E;
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
    __builtin_amdgcn_sched_barrier(0);   // every load issued before the first product
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
        if (b < a.B) part[((int64_t)ks * a.B + b) * lg_stride(a.E) + row] = tv[i];
      }
    }
  }
  trace_point_at(trace, TK_LOGITS, wg, 1);
}

struct BatchRouteArgs {
  const float* part;      // [LG_KS][B][lg_stride(E)] partial logits
  const float* bias;      // [E] or null
  int E, B, k;
  int32_t* idx_out;       // [B][k]
  float* wts_out;         // [B][k]
  float* logits_out;      // [B][E] or null
  int32_t* idx_copy;      // workspace copies or null
  float* wts_copy;
  uint32_t* err;
  uint64_t* trace;
};

template <int PER>
struct RouteLoads {
  u32x4 raw[LG_KS][PER / 4];
  uint32_t rb[PER];
};

// Issue every load of one token's routing: lane l holds experts
// PER l .. PER l + PER - 1 -- the layout the top-k takes -- read 4 at a
// time from each of the LG_KS partial sets (rows padded to 4 experts), and
// their bias.
template <int PER>
__device__ __forceinline__ void route_load(const BatchRouteArgs& r, int b, RouteLoads<PER>& L) {
  const int lane = threadIdx.x & 63;
  const int stride = lg_stride(r.E);
  const int nsets = lg_sets(r.B);
  const uint32_t pbytes = (uint32_t)((int64_t)LG_KS * r.B * stride * 4);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(r.part, pbytes);
  const __amdgpu_buffer_rsrc_t rbias = make_rsrc(r.bias, r.bias ? (uint32_t)r.E * 4u : 0u);
#pragma unroll
  for (int c = 0; c < PER / 4; ++c) {
    const int e0 = lane * PER + 4 * c;
#pragma unroll
    for (int p = 0; p < LG_KS; ++p)   // sets past lg_sets(B) read zeros
      L.raw[p][c] = bload16(rp, (e0 < r.E && p < nsets)
                                    ? (uint32_t)((((int64_t)p * r.B + b) * stride + e0) * 4)
                                    : pbytes);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i)   // zero without a bias or past E
    L.rb[i] = bload4(rbias, (uint32_t)(lane * PER + i) * 4u);
}

// Sum, top-k and weights of one token from its loads.  The selection goes
// to s_idx / s_w (LDS, when given); the global outputs, the logits and the
// error bit are written only when `write` is set.
template <int PER>
__device__ void route_token(const BatchRouteArgs& r, int b, const RouteLoads<PER>& L,
                            int* s_idx, float* s_w, bool write) {
  const int lane = threadIdx.x & 63;
  // expert PER lane + i: the partial sets in order, then the bias
  int nan_seen = 0;
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane * PER + i;
    float l = 0.f;
#pragma unroll
    for (int p = 0; p < LG_KS; ++p) {
      const u32x4 q = L.raw[p][i / 4];
      const uint32_t qv[4] = {q.x, q.y, q.z, q.w};
      l += as_f32(qv[i % 4]);
    }
    if (r.bias) l += as_f32(L.rb[i]);
    const bool valid = e < r.E;
    if (valid && write && r.logits_out) r.logits_out[(int64_t)b * r.E + e] = l;
    nan_seen |= valid & __builtin_isnan(l);
    key[i] = valid ? okey(l) : 0u;
  }
  trace_point(r.trace, TK_TOPK, 2);
  int e;
  float w;
  topk_keys<PER>(key, r.E, r.k, r.k, e, w, nullptr);
  trace_point(r.trace, TK_TOPK, 3);
  if (lane < r.k) {
    const int p = b * r.k + lane;
    if (s_idx) {
      s_idx[p] = e;
      s_w[p] = w;
    }
    if (write) {
      r.idx_out[p] = e;
      r.wts_out[p] = w;
      if (r.idx_copy) {
        r.idx_copy[p] = e;
        r.wts_copy[p] = w;
      }
    }
  }
  if (write && __any(nan_seen) && lane == 0)
    __hip_atomic_fetch_or(r.err, 4u /*HFQ4_DEV_ERR_NONFINITE*/, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
}

// Stage one token's activations (one wave) in the MFMA A-operand format:
// 256 entries of 16 B at ent (entry o = elements 8o..8o+7 scaled by 2^-e,
// in dec8 order) and xs = 2^e (the per-block sums come from
// block_sums_mfma).  Lane l takes entries o = l + 64m, so one load
// instruction covers 2 KB of x and one LDS store 1 KB.
__device__ void stage_token(const float* __restrict__ xb, int d, uint8_t* ent, float* xs_out) {
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
#pragma unroll
  for (int m = 0; m < 4; ++m) put_entry(v[m], inv, ent + 16 * (lane + 64 * m));
  if (lane == 0) *xs_out = xs;
}

// Routing only (the two-call form): one single-wave workgroup per token,
// partial sums + bias, top-k and weights.  The fused layer runs the same
// two functions inside the gate/up kernel, so both forms give the same bits.
__global__ void __launch_bounds__(64) route_topk_kernel(BatchRouteArgs r) {
  trace_point(r.trace, TK_TOPK, 0);
  const int b = blockIdx.x;
  if (r.E <= 256) {
    RouteLoads<4> L;
    route_load<4>(r, b, L);
    route_token<4>(r, b, L, nullptr, nullptr, true);
  } else if (r.E <= 512) {
    RouteLoads<8> L;
    route_load<8>(r, b, L);
    route_token<8>(r, b, L, nullptr, nullptr, true);
  } else {
    RouteLoads<16> L;
    route_load<16>(r, b, L);
    route_token<16>(r, b, L, nullptr, nullptr, true);
  }
  trace_point(r.trace, TK_TOPK, 1);
}

// ====================================================================== gate / up

// A workgroup of 16 waves = 4 quads; a quad takes one (group, 16-row tile)
// item at a time: its waves compute gate K-half 0, gate K-half 1, up K-half
// 0 and up K-half 1 (4 blocks each, all loads in flight at once), the
// partial tiles meet in LDS, and the first wave writes h = SiLU(g) * u.
// Before that, the tokens' activations are staged in LDS and, with
// FROM_LOGITS, the tokens are routed from the router's partial logits by
// one workgroup each and the selections exchanged (no launch sits between
// the router and the experts; the routing workgroups publish idx and wts).
// The grid is one workgroup per compute unit.
template <bool FROM_LOGITS, bool XCH>
__global__ void __launch_bounds__(1024) gateup_mfma_kernel(ExpertArgs a, Ws ws, BatchRouteArgs r) {
  extern __shared__ __align__(16) uint8_t dyn[];
  uint8_t* xt = dyn;                                                     // [B][XT_STRIDE]
  __shared__ GroupTab G;
  __shared__ GroupScratch GS;
  __shared__ int s_idx[MAXP];
  __shared__ float s_wt[MAXP];
  __shared__ float2 s_blk[HFQ4_MAXB_DEV][8];         // per token, block: (off, sx)
  __shared__ float s_xs[HFQ4_MAXB_DEV];
  __shared__ f32x4 red[4][3][64];                    // partial tiles of roles 1..3
  const int wv = wave_id(), lane = threadIdx.x & 63;   // role and its gate/up descriptor: uniform
  const int quad = wv >> 2, role = wv & 3;
  const int B = a.B, k = a.k, P = B * k, F = a.L.F, E = a.L.E;
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws.h);   // [P][F] f16 operand entries
  int8_t* he = reinterpret_cast<int8_t*>(hq + (size_t)P * F * 2);   // [P][F / 16] exponents
  trace_point(ws.trace, TK_GATEUP, 0);

  // 1. Routing from the router's partial logits (FROM_LOGITS).
  //    XCH (more tokens): workgroup b < B routes token b with its wave 0
  //    and publishes the selection as tagged words (xchg_device.h), which
  //    every workgroup then gathers -- one top-k per token in the whole
  //    grid; meanwhile every workgroup stages every token's activations in
  //    LDS (wave (b + 1) % 16 takes token b, so a router workgroup's wave 0
  //    stages only after its routing).  The generation of the words is the
  //    call counter the router launch has just advanced, so no workgroup
  //    waits for another to start: every wait is for the router
  //    workgroups, the lowest-numbered ones.
  //    Otherwise every workgroup routes every token itself, wave b token b;
  //    the activations are staged by the idle waves B..2B-1 when there are
  //    enough of them (B <= 8), else by the routing wave, its loads
  //    overlapping the routing loads.  Routing given: wave b stages token b.
  __shared__ float s_rt[2 * MAXP];                   // gathered routing words
  // this call's generation: the router launch just advanced the counter
  const uint32_t g0 = XCH ? __builtin_amdgcn_readfirstlane(ws.gen[0]) : 0u;
  const bool split_stage = FROM_LOGITS && !XCH && 2 * B <= (int)(blockDim.x >> 6);
  // routing waves: wave 0 of workgroup b < B (XCH), or wave b of every workgroup
  const int rb = XCH ? (wv == 0 && (int)blockIdx.x < B ? (int)blockIdx.x : -1) : (wv < B ? wv : -1);
  if (FROM_LOGITS && rb >= 0) {
    const bool pub = XCH || blockIdx.x == 0;
    const bool stage_here = !XCH && !split_stage;
    const float* xb = a.x + (int64_t)rb * a.ldx;
    uint8_t* xe = xt + rb * XT_STRIDE;
    if (E <= 256) {
      RouteLoads<4> L;
      route_load<4>(r, rb, L);
      if (stage_here) stage_token(xb, a.L.d, xe, &s_xs[rb]);
      route_token<4>(r, rb, L, s_idx, s_wt, pub);
    } else if (E <= 512) {
      RouteLoads<8> L;
      route_load<8>(r, rb, L);
      if (stage_here) stage_token(xb, a.L.d, xe, &s_xs[rb]);
      route_token<8>(r, rb, L, s_idx, s_wt, pub);
    } else {   // 16 loads per lane: route first, then stage
      RouteLoads<16> L;
      route_load<16>(r, rb, L);
      route_token<16>(r, rb, L, s_idx, s_wt, pub);
      if (stage_here) stage_token(xb, a.L.d, xe, &s_xs[rb]);
    }
    if (XCH && lane < k) {
      const int p = rb * k + lane;
      put_word(ws.xlog + p, (uint32_t)s_idx[p], g0);
      put_word(ws.xlog + P + p, __float_as_uint(s_wt[p]), g0);
    }
  }
  {
    // the token this wave stages: (wv + 15) % 16 (XCH), wave B + b (split),
    // wave b (routing given)
    const int b = XCH ? (wv + 15) & 15 : split_stage ? wv - B : wv;
    if ((XCH || split_stage || !FROM_LOGITS) && b >= 0 && b < B)
      stage_token(a.x + (int64_t)b * a.ldx, a.L.d, xt + b * XT_STRIDE, &s_xs[b]);
  }
  if (!FROM_LOGITS && (int)threadIdx.x < P) s_idx[threadIdx.x] = a.idx[threadIdx.x];
  __syncthreads();
  trace_point(ws.trace, TK_GATEUP, 2);
  // per-block sums of the staged tokens: wave w < 8 takes block w
  if (wv < 8) {
    float sa[4], sv[4];
    block_sums_mfma(xt, XT_STRIDE, B, wv, sa, sv);
    if ((lane & 15) == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 4 * (lane >> 4) + i;
        if (b < B) s_blk[b][wv] = make_float2(-(1024.f * sa[i] + 8.f * sv[i]), s_xs[b] * sv[i]);
      }
    }
  }
  if (XCH) {
    const bool late = gather_words<1>(ws.xlog, 2 * P, g0, s_rt);
    if (late && threadIdx.x == 0)
      __hip_atomic_fetch_or(ws.err, 2u /*HFQ4_DEV_ERR_TIMEOUT*/, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int)threadIdx.x < P) s_idx[threadIdx.x] = __float_as_int(s_rt[threadIdx.x]);
  }
  // routing from top-k holds k distinct experts per token
  build_groups_mm(s_idx, P, k, E, G, GS, ws.err, !FROM_LOGITS && blockIdx.x == 0, !FROM_LOGITS);
  // workgroup 0 publishes the table for the down kernel
  if (blockIdx.x == 0) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&G);
    uint32_t* dst = reinterpret_cast<uint32_t*>(ws.gtab);
    for (int i = threadIdx.x; i < (int)(sizeof(GroupTab) / 4); i += blockDim.x) dst[i] = src[i];
  }
  trace_point(ws.trace, TK_GATEUP, 1);

  // 2. this workgroup's items: a contiguous run of (group, 16-row tile)
  constexpr int tiles = FAST_F / MM_ROWS;        // 32 (F == FAST_F on this path)
  const int items = G.U * tiles;
  const int per = (items + gridDim.x - 1) / gridDim.x;
  const int i0 = blockIdx.x * per;
  const int i1 = min(items, i0 + per);

  // 3. the wave's first item: its role's 4 blocks, every load in flight
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
  int it = i0 + quad;
  if (it < i1) issue(it);
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
      // h leaves as f16 in the down kernel's operand order with one
      // power-of-two exponent per (pair, 16-row tile): element q = row % 8
      // of entry row / 8 sits at half 2 (q % 4) + q / 4, odd q divided by 16
      const int row = tile * MM_ROWS + n16;
      const int q8 = row & 7;
      const int hoff = (row >> 3) * 16 + 2 * (2 * (q8 & 3) + (q8 >> 2));
      const float odd = (q8 & 1) ? 0.0625f : 1.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * c + i;
        const float hv = m < n ? silu_mul(gv[i], uv[i]) : 0.f;
        const int e = pow2_exp(row_max16(fabsf(hv)));
        if (m < n) {
          const int p = G.gmem[u][m];
          const float inv = e == H_EMPTY ? 0.f : ldexpf(odd, -e);
          *reinterpret_cast<_Float16*>(hq + (int64_t)p * (2 * F) + hoff) = (_Float16)(hv * inv);
          if (n16 == 0) he[(int64_t)p * (F / MM_ROWS) + tile] = (int8_t)e;
        }
      }
    }
    __syncthreads();   // red is reused by the next round
    it = next;
  }
  trace_point(ws.trace, TK_GATEUP, 5);
}

// ====================================================================== down + combine

// A workgroup owns DR_ROWS = 8 output rows of every token (d = 2048: 256
// workgroups, one per compute unit).  It stages h of all (token, slot)
// pairs once: the gate/up kernel wrote h as f16 in the MFMA operand order
// with one power-of-two exponent per 16-row tile; here each entry is
// brought to its block's exponent (the largest of the block's 16 tiles) and
// stored in LDS.  Then its 16 waves take the expert groups in turn (wave w:
// groups w, w + 16, ...): per group one MFMA tile over K = F, A = the
// group's pairs, B = the block's 8 rows of the expert's down matrix (the
// tile's other 8 rows load nothing), with the next group's weights in
// flight while the current one computes.  Each wave adds w_p * (down h_p)
// into its own [token][row] slice of LDS; at the end the slices are summed
// in wave order onto the residual.  The per-slot sum therefore needs no
// second kernel and no per-slot buffer.
//
// Every workgroup brings in all of h (B k F f16 values: 128 KB at 16
// tokens) besides its rows' weights, and a compute unit pulls a bounded
// number of bytes per unit of time (about 25 - 40 GB/s at these
// latencies), so the bytes per compute unit weigh on the time: half of
// the MFMA tile's rows left empty buys 256 workgroups instead of 128,
// half the weight bytes per unit (0.4 - 0.6 us faster per step at 2 - 16
// tokens than 16-row blocks).
constexpr int DR_ROWS = 8;    // output rows per workgroup (<= 16, the MFMA tile's rows)
constexpr int DR_WAVES = 16;
constexpr int DR_ENT_ITERS = MAXP * 64 / (64 * DR_WAVES);   // h entries per thread (F = 512)

__global__ void __launch_bounds__(64 * DR_WAVES) down_rows_kernel(ExpertArgs a, Ws ws) {
  extern __shared__ __align__(16) uint8_t ht[];            // [P][HT_STRIDE]
  __shared__ float ys[DR_WAVES][GT_MAXM][DR_ROWS];
  __shared__ float2 s_blk[MAXP][2];                        // per pair, block: (off, sx)
  __shared__ float s_xs[MAXP][2];                          // per pair, block: 2^e
  __shared__ int s_eb[MAXP][2];                            // per pair, block: e
  __shared__ uint32_t s_he[MAXP * 8];                      // per pair: 32 tile exponents
  __shared__ float s_w[MAXP];
  __shared__ GroupTab G;
  const int wv = wave_id(), lane = threadIdx.x & 63;
  const int B = a.B, k = a.k, P = B * k, d = a.L.d, F = a.L.F;
  const int r0 = blockIdx.x * DR_ROWS;
  const int n16 = lane & 15, c = lane >> 4;
  const uint8_t* hq = reinterpret_cast<const uint8_t*>(ws.h);   // [P][F] f16 operand entries
  const int8_t* he = reinterpret_cast<const int8_t*>(hq + (size_t)P * F * 2);
  trace_point(ws.trace, TK_DOWN, 0);

  // 1. the group table the gate/up kernel published, the routing weights
  //    and the tile exponents first, then every h entry (16 B, entry
  //    threadIdx.x + 1024 j), in flight while the table is stored and the
  //    first weights are requested
  constexpr int GT_WORDS = (int)(sizeof(GroupTab) / 4);
  static_assert(GT_WORDS <= 64 * DR_WAVES, "one table word per thread");
  const uint32_t gword =
      (int)threadIdx.x < GT_WORDS ? reinterpret_cast<const uint32_t*>(ws.gtab)[threadIdx.x] : 0u;
  const float wword = (int)threadIdx.x < P ? a.wts[threadIdx.x] : 0.f;
  const int EW = P * 8;   // exponent words (32 tiles per pair)
  const uint32_t eword = (int)threadIdx.x < EW ? reinterpret_cast<const uint32_t*>(he)[threadIdx.x] : 0u;
  // no branches around the loads (entries past the end read past the
  // descriptor and get zeros), so the stores below wait for their own loads
  const int NENT = P * 64;
  const uint32_t hbytes = (uint32_t)NENT * 16u;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(hq, hbytes);
  u32x4 hv[DR_ENT_ITERS];
#pragma unroll
  for (int j = 0; j < DR_ENT_ITERS; ++j) {
    const int el = threadIdx.x + 64 * DR_WAVES * j;
    hv[j] = bload16(rh, el < NENT ? (uint32_t)el * 16u : hbytes);
  }
  // the residual of output (token b, row r) for thread b * DR_ROWS + r,
  // needed only at the end, goes out now (a null residual reads 0)
  const int b_out = threadIdx.x / DR_ROWS, rr_out = r0 + (int)threadIdx.x - b_out * DR_ROWS;
  const bool y_out = b_out < B && rr_out < d;
  const uint32_t resb = a.res ? 4u * (uint32_t)((int64_t)(B - 1) * a.ldy + d) : 0u;
  const float res_out = as_f32(bload4(make_rsrc(a.res, resb),
                                      y_out ? 4u * (uint32_t)((int64_t)b_out * a.ldy + rr_out) : resb));
  if ((int)threadIdx.x < GT_WORDS) reinterpret_cast<uint32_t*>(&G)[threadIdx.x] = gword;
  if ((int)threadIdx.x < P) s_w[threadIdx.x] = wword;
  if ((int)threadIdx.x < EW) s_he[threadIdx.x] = eword;
#pragma unroll
  for (int i = threadIdx.x; i < DR_WAVES * GT_MAXM * DR_ROWS; i += 64 * DR_WAVES)
    (&ys[0][0][0])[i] = 0.f;
  __syncthreads();
  trace_point(ws.trace, TK_DOWN, 4);
  const int U = G.U;
  const int8_t* he_l = reinterpret_cast<const int8_t*>(s_he);
  // a block's exponent is the largest of its 16 tiles'
  if ((int)threadIdx.x < 2 * P) {
    const int p = threadIdx.x >> 1, bk = threadIdx.x & 1;
    int m = H_EMPTY;
#pragma unroll
    for (int t = 0; t < 16; ++t) m = max(m, (int)he_l[p * 32 + 16 * bk + t]);
    s_eb[p][bk] = m;
    s_xs[p][bk] = m == H_EMPTY ? 0.f : ldexpf(1.f, m);
  }

  // 2. the wave's first group: the block's DR_ROWS rows x 2 blocks, every
  //    load in flight
  constexpr int64_t ROWB = 2 * BLK_BYTES;
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.L.down, a.L.down_bytes);
  const int row = r0 + n16;
  const bool row_live = n16 < DR_ROWS && row < d;   // tile rows past the block load nothing
  u32x4 cdA[2][2], cdB[2][2];   // [block][half], two buffers
  u32x2 hdA[2], hdB[2];
  auto issue = [&](int u, u32x4 (&cd)[2][2], u32x2 (&hd)[2]) {
    const uint32_t ro = row_live ? (uint32_t)(G.gexp[u] * a.L.sd + (int64_t)row * ROWB) : a.L.down_bytes;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      hd[bk] = bload8(rd, ro + bk * BLK_BYTES);
      cd[bk][0] = bload16(rd, ro + bk * BLK_BYTES + 8 + 16 * c);
      cd[bk][1] = bload16(rd, ro + bk * BLK_BYTES + 8 + 64 + 16 * c);
    }
  };
  if (wv < U) issue(wv, cdA, hdA);
  trace_point(ws.trace, TK_DOWN, 5);
  __syncthreads();   // block exponents

  // 3. every entry brought from its tile's exponent to its block's (an
  //    exact power-of-two product in f16, barring values that fall below
  //    the f16 normal range), then stored in LDS; the per-block sums follow
#pragma unroll
  for (int j = 0; j < DR_ENT_ITERS; ++j) {
    const int el = threadIdx.x + 64 * DR_WAVES * j;
    if (el < NENT) {
      const int p = el >> 6, o = el & 63;
      const h2 f = f16_pow2_pair((int)he_l[p * 32 + (o >> 1)] - s_eb[p][o >> 5]);
      const u32x4 v = hv[j];
      *reinterpret_cast<u32x4*>(ht + p * HT_STRIDE + 16 * o) =
          u32x4{as_u32(as_h2(v.x) * f), as_u32(as_h2(v.y) * f), as_u32(as_h2(v.z) * f),
                as_u32(as_h2(v.w) * f)};
    }
  }
  if (wv + DR_WAVES < U) issue(wv + DR_WAVES, cdB, hdB);   // second group in flight too
  __syncthreads();
  trace_point(ws.trace, TK_DOWN, 6);
  // per-block sums of the staged pairs: job (16 pairs, block) per wave
  {
    const int jobs = 2 * ((P + 15) / 16);
    for (int job = wv; job < jobs; job += DR_WAVES) {   // wave-uniform
      const int j = job >> 1, bk = job & 1;
      float sa[4], sv[4];
      block_sums_mfma(ht + 16 * j * HT_STRIDE, HT_STRIDE, P - 16 * j, bk, sa, sv);
      if (n16 == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = 16 * j + 4 * c + i;
          if (p < P) s_blk[p][bk] = make_float2(-(1024.f * sa[i] + 8.f * sv[i]), s_xs[p][bk] * sv[i]);
        }
      }
    }
  }
  __syncthreads();
  trace_point(ws.trace, TK_DOWN, 1);

  // 4. the wave's groups, the next ones' weights in flight during each
  auto compute = [&](int u, const u32x4 (&cd)[2][2], const u32x2 (&hd)[2]) {
    const int n = G.gcnt[u];
    const int pa = n16 < n ? G.gmem[u][n16] : G.gmem[u][0];   // A row source
    const uint8_t* arow = ht + pa * HT_STRIDE + 16 * (4 * c);
    int pc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * c + i;
      pc[i] = m < n ? G.gmem[u][m] : -1;
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      h8 av[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) av[t][i] = *reinterpret_cast<const h8*>(arow + 16 * (32 * bk + 16 * t + i));
      const uint32_t q0[4] = {cd[bk][0].x, cd[bk][0].y, cd[bk][0].z, cd[bk][0].w};
      const uint32_t q1[4] = {cd[bk][1].x, cd[bk][1].y, cd[bk][1].z, cd[bk][1].w};
      f32x4 c2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c2[0] = mfma16(av[0][i], dec8(q0[i]), c2[0]);
        c2[1] = mfma16(av[1][i], dec8(q1[i]), c2[1]);
      }
      const f32x4 cb = c2[0] + c2[1];
      const float scale = as_f32(hd[bk].x), zero = as_f32(hd[bk].y);
      const float zp8 = __builtin_fmaf(8.f, scale, zero);
      const float cbv[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (pc[i] >= 0) {
          const float2 ob = s_blk[pc[i]][bk];
          acc[i] += __builtin_fmaf(scale * s_xs[pc[i]][bk], cbv[i] + ob.x, zp8 * ob.y);
        }
      }
    }
    // the pairs of a group belong to distinct tokens: the lanes of one
    // update touch distinct slots
    if (n16 < DR_ROWS) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (pc[i] >= 0) ys[wv][pc[i] / k][n16] += s_w[pc[i]] * acc[i];
    }
  };
  // buffers A and B hold groups u and u + 16; each is refilled with the
  // group two steps ahead as soon as it has been used
  for (int u = wv; u < U; u += 2 * DR_WAVES) {   // wave-uniform
    compute(u, cdA, hdA);
    if (u + 2 * DR_WAVES < U) issue(u + 2 * DR_WAVES, cdA, hdA);
    if (u + DR_WAVES >= U) break;
    compute(u + DR_WAVES, cdB, hdB);
    if (u + 3 * DR_WAVES < U) issue(u + 3 * DR_WAVES, cdB, hdB);
  }
  trace_point(ws.trace, TK_DOWN, 3);
  __syncthreads();

  // 5. y = residual + the waves' slices, in wave order
  if (y_out) {
    const int r = rr_out - r0;
    float y = res_out;
#pragma unroll
    for (int w = 0; w < DR_WAVES; ++w) y += ys[w][b_out][r];
    a.y[(int64_t)b_out * a.ldy + rr_out] = y;
  }
  trace_point(ws.trace, TK_DOWN, 2);
}

// ====================================================================== host

int launch_logits_batched(const RouteArgs& ra, float* part, uint32_t* gen, hipStream_t s) {
  if (lg_sets(ra.B) == 1) {
    if (gen) return (int)hipErrorInvalidValue;   // the exchange comes with the matrix-core router
    return launch_logits_valu(ra, part, lg_stride(ra.E), s);
  }
  hipLaunchKernelGGL(logits_mfma_kernel, dim3((ra.E + 7) / 8, LG_KS), dim3(256), 0, s, ra, part,
                     get_trace(), gen);
  return (int)hipGetLastError();
}

int launch_route_batched(const RouteArgs& ra, const float* part, uint32_t* err, hipStream_t s) {
  BatchRouteArgs r{part, ra.bias, ra.E, ra.B, ra.k, ra.idx_out, ra.wts_out, ra.logits_out,
                   nullptr, nullptr, err, get_trace()};
  hipLaunchKernelGGL(route_topk_kernel, dim3(ra.B), dim3(64), 0, s, r);
  return (int)hipGetLastError();
}

// Batches of at least this many tokens route by exchange (one router
// workgroup per token) instead of in every workgroup.
static int g_xch_min_batch = 9;
void set_route_exchange_min_batch(int b) { g_xch_min_batch = b; }
bool batched_route_exchange(int B) {
  return B >= g_xch_min_batch && lg_sets(B) > 1 && num_cus() <= XG_MAX;
}

int launch_experts_batched(const ExpertArgs& a, Ws ws, int nwg, const RouteArgs* ra, hipStream_t s) {
  const size_t shx = (size_t)a.B * XT_STRIDE;
  if (ra && batched_route_exchange(a.B) && nwg == num_cus()) {
    const BatchRouteArgs r{ws.logits, ra->bias, ra->E, ra->B, ra->k, ra->idx_out, ra->wts_out,
                           ra->logits_out, nullptr, nullptr, ws.err, get_trace()};
    if (int e = allow_lds(gateup_mfma_kernel<true, true>, shx)) return e;
    hipLaunchKernelGGL((gateup_mfma_kernel<true, true>), dim3(nwg), dim3(1024), shx, s, a, ws, r);
  } else if (ra) {
    const BatchRouteArgs r{ws.logits, ra->bias, ra->E, ra->B, ra->k, ra->idx_out, ra->wts_out,
                           ra->logits_out, nullptr, nullptr, ws.err, get_trace()};
    if (int e = allow_lds(gateup_mfma_kernel<true, false>, shx)) return e;
    hipLaunchKernelGGL((gateup_mfma_kernel<true, false>), dim3(nwg), dim3(1024), shx, s, a, ws, r);
  } else {
    const BatchRouteArgs r{};
    if (int e = allow_lds(gateup_mfma_kernel<false, false>, shx)) return e;
    hipLaunchKernelGGL((gateup_mfma_kernel<false, false>), dim3(nwg), dim3(1024), shx, s, a, ws, r);
  }
  int err = (int)hipGetLastError();
  if (err) return err;
  const size_t shd = (size_t)a.B * a.k * HT_STRIDE;
  if (int e = allow_lds(down_rows_kernel, shd)) return e;
  hipLaunchKernelGGL(down_rows_kernel, dim3((a.L.d + DR_ROWS - 1) / DR_ROWS), dim3(64 * DR_WAVES),
                     shd, s, a, ws);
  return (int)hipGetLastError();
}

}  // namespace hq
