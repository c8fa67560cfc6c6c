// Device-side building blocks shared by the HFQ4 kernels (gfx950, wave64).
//
// HFQ4 block (page "hipfire：为AMD RDNA GPU打造的Rust原生LLM推理引擎",
// section "2. HFQ量化格式与GEMV优化"): 256 weights in 136 bytes =
// f32 scale | f32 zero | 128 code bytes.  Byte j of the codes holds element
// 2j in its low nibble and 2j+1 in its high nibble; w = zero + scale*q.
//
// Dot-product scheme.  A row is read as "segments": 16 code bytes = 32
// weights; a block has 8 segments at byte offsets 8 + 16c.  One lane owns
// one segment position for every row it visits ("column-stationary"), so
// the activation values it needs stay in registers across rows.  A code
// dword is turned into four f16 pairs with no conversion instructions:
// OR-ing a nibble into the mantissa of 1024.0h gives 1024 + q exactly, and
// OR-ing the next nibble (4 bits higher) gives 1024 + 16q.  The matching
// activation pairs are pre-arranged (and pre-scaled by 1/16 where needed)
// once per vector, so each dword costs 4 bit-ops + 1 shift + 4 v_dot2
// (f16 x f16 products, f32 accumulate).  The constant 1024 terms and the
// zero point are folded back per segment with pre-computed sums:
//   sum_i w_i x_i = scale * sum_i (q_i - 8) x_i + (zero + 8 scale) * sum_i x_i
// where the first sum uses f16-rounded x and the second the exact f32 x.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BLK = 256;          // weights per block
constexpr int BLK_BYTES = 136;    // bytes per block
constexpr int SEG = 32;           // weights per segment (16 code bytes)
constexpr int SEGS_PER_BLK = 8;

#define HFQ4_MAXB_DEV 16      // max tokens per call (matches HFQ4_MAX_BATCH)
#define HFQ4_MAXE_DEV 1024    // max experts per layer (matches HFQ4_MAX_EXPERTS)

constexpr uint32_t MAGIC = 0x64006400u;   // two f16 1024.0
constexpr uint32_t LO4 = 0x000F000Fu;
constexpr uint32_t HI4 = 0x00F000F0u;

// Bit reinterpretation through by-value scalars.  (clang's __builtin_bit_cast
// applied directly to an ext-vector element such as v.y reads element 0, so
// vector elements always pass through one of these first.)
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// ---------------------------------------------------------------- loads

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // gfx9 family buffer descriptor word 3 (raw dword access, no swizzle)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// ---------------------------------------------------------------- fragments

// Activation fragment for one 32-element segment, in the order dot_seg uses.
// The segment is first scaled by a power of two, xs, chosen so that its
// largest magnitude lies in [2, 4): the f16 pairs then keep the same relative
// precision whatever the activations' range (a 40-layer residual stack grows
// them far beyond f16's maximum), and the f32 sums that cancel the 1024
// offsets stay small.  Scaling by a power of two is exact.
struct Frag {
  h2 p[16];
  float off;   // -(1024 * sum of all 32 stored halves + 8 * sum of the f16 values they stand for)
  float sx;    // f32 sum of the 32 (unscaled) activations
  float xs;    // the power-of-two scale: activation = xs * (stored value)
};

// Build a fragment from 32 f32 activations v[0..31] (element order).
// Dword w of a segment covers elements 8w..8w+7 (element 8w+n at nibble n).
__device__ __forceinline__ void make_frag(const float* v, Frag& f) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int e = 0;
  if (amax > 0.f && amax < INFINITY) {
    int ex;
    frexpf(amax, &ex);           // amax = m * 2^ex, m in [0.5, 1)
    e = ex - 2;                  // amax * 2^-e in [2, 4)
  }
  const float inv = ldexpf(1.0f, -e);
  float sum_half = 0.f, sum_x16 = 0.f, sx = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bool hi = (p & 1);                 // nibbles 1,3 (and 5,7) carry 16q
      const int n = p;                         // pair p = elements (8w+p, 8w+p+4)
      const float a = v[8 * w + n], b = v[8 * w + n + 4];
      const float s = hi ? 0.0625f : 1.0f;
      _Float16 ha = (_Float16)(a * inv * s), hb = (_Float16)(b * inv * s);
      f.p[4 * w + p] = h2{ha, hb};
      const float fa = (float)ha, fb = (float)hb;
      sum_half += fa + fb;
      sum_x16 += hi ? 16.f * (fa + fb) : (fa + fb);
      sx += a + b;
    }
  }
  f.off = -(1024.f * sum_half + 8.f * sum_x16);
  f.sx = sx;
  f.xs = ldexpf(1.0f, e);
}

// One code dword (8 weights) against 4 fragment pairs.
__device__ __forceinline__ float dot_dword(uint32_t d, const h2* x, float acc) {
  const uint32_t p0 = (d & LO4) | MAGIC;
  const uint32_t p1 = (d & HI4) | MAGIC;
  const uint32_t d8 = d >> 8;
  const uint32_t p2 = (d8 & LO4) | MAGIC;
  const uint32_t p3 = (d8 & HI4) | MAGIC;
  acc = __builtin_amdgcn_fdot2(as_h2(p0), x[0], acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(p1), x[1], acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(p2), x[2], acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(p3), x[3], acc, false);
  return acc;
}

// Contribution of one segment (16 code bytes + its block header) to a row dot.
__device__ __forceinline__ float dot_seg(u32x4 codes, u32x2 hdr, const Frag& f) {
  float acc = f.off;
  acc = dot_dword(codes.x, &f.p[0], acc);
  acc = dot_dword(codes.y, &f.p[4], acc);
  acc = dot_dword(codes.z, &f.p[8], acc);
  acc = dot_dword(codes.w, &f.p[12], acc);
  const float scale = as_f32(hdr.x);
  const float zero = as_f32(hdr.y);
  const float zp8 = __builtin_fmaf(8.f, scale, zero);
  return __builtin_fmaf(scale * f.xs, acc, zp8 * f.sx);
}

// ---------------------------------------------------------------- LDS fragment store
// Fragments of a vector with S segments live in LDS as 4 planes of S x 16 B
// (plane w = pairs 4w..4w+3 of every segment; consecutive segments are
// consecutive 16-byte slots, so a wave reading consecutive segments is
// conflict-free) followed by S x 16 B of (off, sx, xs, 0).
__device__ __forceinline__ void frag_store(uint8_t* lds, int S, int s, const Frag& f) {
  u32x4* planes = reinterpret_cast<u32x4*>(lds);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    u32x4 v;
    v.x = as_u32(f.p[4 * w + 0]);
    v.y = as_u32(f.p[4 * w + 1]);
    v.z = as_u32(f.p[4 * w + 2]);
    v.w = as_u32(f.p[4 * w + 3]);
    planes[w * S + s] = v;
  }
  f32x4* os = reinterpret_cast<f32x4*>(lds + 64 * S);
  os[s] = f32x4{f.off, f.sx, f.xs, 0.f};
}
__device__ __forceinline__ void frag_load(const uint8_t* lds, int S, int s, Frag& f) {
  const u32x4* planes = reinterpret_cast<const u32x4*>(lds);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const u32x4 v = planes[w * S + s];
    f.p[4 * w + 0] = as_h2(v.x);
    f.p[4 * w + 1] = as_h2(v.y);
    f.p[4 * w + 2] = as_h2(v.z);
    f.p[4 * w + 3] = as_h2(v.w);
  }
  const f32x4 os = reinterpret_cast<const f32x4*>(lds + 64 * S)[s];
  f.off = os.x;
  f.sx = os.y;
  f.xs = os.z;
}
__host__ __device__ constexpr int frag_bytes(int S) { return 80 * S; }

// Stage n f32 values (n <= 32*S; the rest read as 0) into LDS fragments,
// one segment per thread of the block (threads beyond S idle).
__device__ __forceinline__ void stage_vector(const float* __restrict__ v, int n, int S,
                                             uint8_t* lds, int tid, int nthreads) {
  for (int s = tid; s < S; s += nthreads) {
    float buf[32];
    const int base = s * SEG;
    if (base + SEG <= n) {
      const f32x4* v4 = reinterpret_cast<const f32x4*>(v + base);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4 t = v4[i];
        buf[4 * i + 0] = t.x; buf[4 * i + 1] = t.y; buf[4 * i + 2] = t.z; buf[4 * i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) buf[i] = (base + i < n) ? v[base + i] : 0.f;
    }
    Frag f;
    make_frag(buf, f);
    frag_store(lds, S, s, f);
  }
}

// ---------------------------------------------------------------- reductions


// Index of the calling wave in its workgroup, through readfirstlane: the
// compiler then knows it to be wave-uniform, so what follows from it (rows,
// items, buffer descriptors, offsets) is computed once per wave in scalar
// registers, and loads through a descriptor chosen by it need no per-lane
// waterfall loop.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---- DPP / permlane reductions (VALU only, fixed order, no LDS traffic)
template <int CTL>
__device__ __forceinline__ float dpp(float v) {
  return as_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__builtin_bit_cast(uint32_t, v), CTL,
                                                      0xf, 0xf, false));
}
// All-reduce over each 16-lane row: xor 1, xor 2, rotate 4, rotate 8.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  return v;
}
// gfx950 cross-row swaps.  a, b must be distinct values.
// swap32: returns {a.lo32 | b.lo32, a.hi32 | b.hi32} summed -> lanes 0-31 hold
// a reduced over xor 32, lanes 32-63 hold b reduced over xor 32.
__device__ __forceinline__ float fold32(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                            __builtin_bit_cast(uint32_t, b), false, false);
  return as_f32(r[0]) + as_f32(r[1]);
}
// swap16: rows {a.r0, b.r0, a.r2, b.r2} + {a.r1, b.r1, a.r3, b.r3}: rows 0 and 2
// hold a reduced over xor 16, rows 1 and 3 hold b.
__device__ __forceinline__ float fold16(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                            __builtin_bit_cast(uint32_t, b), false, false);
  return as_f32(r[0]) + as_f32(r[1]);
}
// Sum over aligned groups of WIDTH = 8, 16, 32 or 64 lanes (all active);
// every lane of a group gets the group sum, in a fixed order: DPP within a
// row, then the gfx950 row swaps.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(WIDTH == 8 || WIDTH == 16 || WIDTH == 32 || WIDTH == 64, "group width");
  if (WIDTH == 8) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    return v + dpp<0x141>(v);
  }
  v = row_sum16(v);
  if (WIDTH >= 32) {   // rows 0+1 and 2+3
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                                    __builtin_bit_cast(uint32_t, v), false, false);
    v = as_f32(r[0]) + as_f32(r[1]);
  }
  if (WIDTH == 64) {   // halves
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                                    __builtin_bit_cast(uint32_t, v), false, false);
    v = as_f32(r[0]) + as_f32(r[1]);
  }
  return v;
}
// Full 64-lane sum, result uniform (fixed order: rows, then row 0+1+2+3).
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// ---------------------------------------------------------------- eight-lane fragment builder
// Eight lanes (an aligned lane group, all active) build one segment's
// fragment with the same arithmetic as make_frag, up to the order of the
// three sums: lane j holds elements 4j..4j+3 of the segment, so one load
// instruction of a wave covers 1 KB of contiguous input.  Lanes 2w and
// 2w+1 swap values to form the four f16 pairs of plane dword w (two pairs
// each); the segment maximum and sums are 8-lane DPP reductions.  The
// result goes to dst in the frag_store layout.
//
// Loads go through a buffer descriptor over the vector's 4n bytes with n a
// multiple of 4 (a 16-byte load is wholly inside or wholly outside it), so
// segments past the end, and segment -1, read zeros without a branch.
__device__ __forceinline__ f32x4 load_seg8(__amdgpu_buffer_rsrc_t rv, int s, int j) {
  const uint32_t off = s >= 0 ? (uint32_t)(4 * (s * SEG + 4 * j)) : 0xfffffff0u;
  const u32x4 t = bload16(rv, off);
  return f32x4{as_f32(t.x), as_f32(t.y), as_f32(t.z), as_f32(t.w)};
}
__device__ __forceinline__ float sum8(float v) {   // mirror, xor 1, xor 2
  v += dpp<0x141>(v);
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  return v;
}
__device__ __forceinline__ void build_seg8(f32x4 xv, int S, int s, int j, uint8_t* dst) {
  const int w = j >> 1, hf = j & 1;
  float amax = fmaxf(fmaxf(fabsf(xv.x), fabsf(xv.y)), fmaxf(fabsf(xv.z), fabsf(xv.w)));
  amax = fmaxf(amax, dpp<0x141>(amax));
  amax = fmaxf(amax, dpp<0xB1>(amax));
  amax = fmaxf(amax, dpp<0x4E>(amax));
  int e = 0;
  if (amax > 0.f && amax < INFINITY) {
    int ex;
    frexpf(amax, &ex);           // amax = m * 2^ex, m in [0.5, 1)
    e = ex - 2;                  // amax * 2^-e in [2, 4)
  }
  const float inv = ldexpf(1.0f, -e);
  // Lane hf = 0 holds elements 8w..8w+3 (the first of each pair), hf = 1
  // holds 8w+4..8w+7 (the second).  This lane forms pairs p = 2hf + t
  // (t = 0, 1), elements (8w+p, 8w+p+4): it keeps its values t (hf = 0) or
  // 2+t (hf = 1) and receives the partner's values of the same index.
  const float keep0 = hf ? xv.z : xv.x, keep1 = hf ? xv.w : xv.y;
  const float send0 = hf ? xv.x : xv.z, send1 = hf ? xv.y : xv.w;
  const float got0 = dpp<0xB1>(send0), got1 = dpp<0xB1>(send1);
  float sum_half = 0.f, sum_x16 = 0.f, sx = 0.f;
  uint32_t out[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float kv = t ? keep1 : keep0, gv = t ? got1 : got0;
    const float av = hf ? gv : kv, bv = hf ? kv : gv;
    const float sc = t ? 0.0625f : 1.0f;   // p is odd exactly when t is: pairs 1, 3 meet 16q
    const _Float16 ha = (_Float16)(av * inv * sc), hb = (_Float16)(bv * inv * sc);
    out[t] = as_u32(h2{ha, hb});
    const float fa = (float)ha, fb = (float)hb;
    sum_half += fa + fb;
    sum_x16 += t ? 16.f * (fa + fb) : (fa + fb);
    sx += av + bv;
  }
  *reinterpret_cast<u32x2*>(dst + 16 * (w * S + s) + 8 * hf) = u32x2{out[0], out[1]};
  sum_half = sum8(sum_half);
  sum_x16 = sum8(sum_x16);
  sx = sum8(sx);
  if (j == 0)
    *reinterpret_cast<f32x4*>(dst + 64 * S + 16 * s) =
        f32x4{-(1024.f * sum_half + 8.f * sum_x16), sx, ldexpf(1.0f, e), 0.f};
}
// All S segments of v (n values, n a multiple of 4, the rest 0) into
// fragments at dst, eight lanes per segment, with the loads of up to four
// segments per lane in flight before any is used.  nthreads is a multiple
// of 64, tid & 63 is the lane.
__device__ __forceinline__ void stage_vector8(const float* __restrict__ v, int n, int S,
                                              uint8_t* dst, int tid, int nthreads) {
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v, 4u * (uint32_t)n);
  const int j = tid & 7;
  const int G = nthreads >> 3;   // segments per pass
  for (int s0 = tid >> 3; s0 < S; s0 += 4 * G) {
    const f32x4 x0 = load_seg8(rv, s0 < S ? s0 : -1, j);
    const f32x4 x1 = load_seg8(rv, s0 + G < S ? s0 + G : -1, j);
    const f32x4 x2 = load_seg8(rv, s0 + 2 * G < S ? s0 + 2 * G : -1, j);
    const f32x4 x3 = load_seg8(rv, s0 + 3 * G < S ? s0 + 3 * G : -1, j);
    build_seg8(x0, S, s0, j, dst);                   // conditions uniform per group
    if (s0 + G < S) build_seg8(x1, S, s0 + G, j, dst);
    if (s0 + 2 * G < S) build_seg8(x2, S, s0 + 2 * G, j, dst);
    if (s0 + 3 * G < S) build_seg8(x3, S, s0 + 3 * G, j, dst);
  }
}

__device__ __forceinline__ void trace_point_at(uint64_t* trace, int kernel, int wg, int point) {
  if (trace && threadIdx.x == 0 && wg < 1024)
    trace[((size_t)kernel * 1024 + wg) * 8 + point] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void trace_point(uint64_t* trace, int kernel, int point) {
  trace_point_at(trace, kernel, (int)blockIdx.x, point);
}

// SiLU(g) * u with the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

}  // namespace hq
