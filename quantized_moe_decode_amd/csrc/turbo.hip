// TurboQuant KV-vector codec on gfx950: encode f32 vectors of n = 64, 128 or
// 256 values into b-bit codes (b = 2, 3, 4 or 8) plus one f32 norm ratio,
// and decode them back.
//
// Page "hipfire：为AMD RDNA GPU打造的Rust原生LLM推理引擎", section "3.
// TurboQuant KV缓存压缩": each vector is normalised to unit L2 norm, rotated
// by a fast Walsh-Hadamard transform done with register-level lane swaps
// (no LDS and no barriers), quantised to Lloyd-Max centroids, and stored
// with the ratio of its norm to the norm of its reconstruction.  Readings
// (stated once, used by both kernels): the orthonormal Hadamard matrix in
// natural order, no random signs; the Lloyd-Max levels of the standard
// normal scaled by 1/sqrt(n), nearest level with ties to the lower one; the
// record is the codes packed LSB-first (code j at bits [j b, j b + b)) and
// then s = |v| / |c| as an f32.
//
// n / 8 lanes per vector, eight values per lane in two runs of four, so a
// wave holds 8, 4 or 2 vectors at once and the per-vector reductions are
// short lane-group sums: the butterflies of spans 1, 2 and n/2 stay in a
// lane, the others pair lane j with lane j ^ M through DPP (quad permutes,
// row rotations) or the gfx950 row swap; every output is the same sequence
// of exactly rounded adds and subtracts.  A wave takes two such sets per
// iteration with all their loads in flight together.  The level table is
// copied into LDS once per workgroup.  Both kernels are HBM streams: 4n
// bytes of f32 on one side, n b / 8 + 4 on the other.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hfq4_device.h"
#include "launch.h"
#include "turbo.h"

namespace hq {
namespace {

// The value of lane l ^ M in every lane: quad permutes (M = 1, 2) and row
// rotations (M = 4, 8) by DPP, the gfx950 row swap for 16 -- VALU only,
// no LDS crossbar.
template <int M>
__device__ __forceinline__ float partner(float v, int lane) {
  if (M == 16) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    return (lane & 16) ? as_f32(r[0]) : as_f32(r[1]);   // r[0]: bit 4 clear, r[1]: set
  }
  if (M == 1) return dpp<0xB1>(v);     // quad_perm [1,0,3,2]
  if (M == 2) return dpp<0x4E>(v);     // quad_perm [2,3,0,1]
  if (M == 8) return dpp<0x128>(v);    // row_ror:8
  // M = 4: row_ror:N reads lane l - N (mod 16).  Both moves run in every
  // lane (a DPP move reading a lane that is switched off would read the
  // fallback value), then each lane keeps its partner's.
  const float down4 = dpp<0x124>(v), up4 = dpp<0x12C>(v);
  return (lane & 4) ? down4 : up4;
}

// Register layout of one vector of n = 8 G values in an aligned group of G
// lanes: lane j holds the four values 4j .. 4j + 3 in x[0..3] and the four
// values n/2 + 4j .. n/2 + 4j + 3 in x[4..7], so each 16-byte load or store
// instruction of a wave covers contiguous memory.
//
// In-place orthonormal Walsh-Hadamard transform in that layout, stages in
// order of increasing span: spans 1 and 2 inside each run of four, spans
// 4 M (M = 1 .. G/2) between lane j and lane j ^ M, span n/2 between the
// two runs of a lane.  Every butterfly is (a, b) -> (a + b, a - b) with a
// the lower index, exactly rounded (a lane's new value is fma(+-1, own,
// partner), the same single rounding); then the 1/sqrt(n) scaling.
template <int G>
__device__ __forceinline__ void fwht8(float (&x)[8], int lane) {
#pragma unroll
  for (int h = 1; h < 4; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (!(e & h)) {
        const float a = x[e], b = x[e + h];
        x[e] = a + b;
        x[e + h] = a - b;
      }
  }
#define HQ_STAGE(M)                                            \
  if (M < G) {                                                 \
    const float sg = (lane & (M)) ? -1.f : 1.f;                \
    _Pragma("unroll") for (int e = 0; e < 8; ++e)              \
      x[e] = __builtin_fmaf(sg, x[e], partner<M>(x[e], lane)); \
  }
  HQ_STAGE(1) HQ_STAGE(2) HQ_STAGE(4) HQ_STAGE(8) HQ_STAGE(16)
#undef HQ_STAGE
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = x[e], b = x[e + 4];
    x[e] = a + b;
    x[e + 4] = a - b;
  }
  const float inv = G == 8 ? 0.125f : G == 16 ? 0.08838834764831845f : 0.0625f;   // 1/sqrt(8 G)
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= inv;
}

// A lane's two runs of four f32 values (16-byte loads and stores when the
// vector start is 16-byte aligned).
template <bool VEC>
__device__ __forceinline__ void load8(const float* a, const float* b, float (&x)[8]) {
  if constexpr (VEC) {
    const f32x4 p = *reinterpret_cast<const f32x4*>(a);
    const f32x4 q = *reinterpret_cast<const f32x4*>(b);
    x[0] = p.x; x[1] = p.y; x[2] = p.z; x[3] = p.w;
    x[4] = q.x; x[5] = q.y; x[6] = q.z; x[7] = q.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[e + 4] = b[e];
    }
  }
}
template <bool VEC>
__device__ __forceinline__ void store8(float* a, float* b, const float (&x)[8]) {
  if constexpr (VEC) {
    *reinterpret_cast<f32x4*>(a) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(b) = f32x4{x[4], x[5], x[6], x[7]};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = x[e];
      b[e] = x[e + 4];
    }
  }
}

// Encode.  The nearest level is the number of thresholds below the rotated
// value: a binary search over the thresholds in LDS, or for 8-bit codes a
// bucket table built in LDS per workgroup (3 LDS reads instead of 8).
// A wave holds 64 / G vectors at once (G = n / 8 lanes each) and
// takes U such sets per iteration, every load of the iteration issued before
// the first is used (a vector index past the end reads the last vector
// again and writes nothing).  Norms are G-lane sums; each lane's two runs of
// four codes go into the wave's records in LDS (value i's code at bits
// [i b, i b + b) of its vector's code stream), and the iteration's records,
// contiguous in memory, leave as whole words.
template <int G, int BITS, int U, bool VEC>
__global__ void __launch_bounds__(256) turbo_encode_kernel(const float* __restrict__ v, int64_t count,
                                                           int64_t ldv, uint8_t* __restrict__ out,
                                                           TurboTable tab) {
  constexpr int N = 8 * G, L = 1 << BITS, VW = 64 / G;
  constexpr int CW = N * BITS / 32, RW = CW + 1;   // code words, record words
  constexpr int WW = U * VW * RW;                  // record words of one wave iteration
  constexpr bool LUT = BITS == 8;                  // bucketed search (8 bits)
  constexpr int NBK = LUT ? TURBO_LUT_BUCKETS : 1;
  __shared__ uint32_t pk[4][WW];
  __shared__ float thr[L + 1], cent[L];
  __shared__ uint8_t bcnt[NBK];                    // thresholds in the buckets before bucket k
  __shared__ int tbk[LUT ? L : 1];                 // bucket of threshold t
  for (int i = threadIdx.x; i < L + 1; i += blockDim.x) {
    if (i < L) cent[i] = tab.cent[i];
    thr[i] = i < L - 1 ? tab.thr[i] : INFINITY;
  }
  auto bucket = [&](float r) {
    const float f = fminf(fmaxf(floorf((r - tab.lut_lo) * tab.lut_inv_w), 0.f), (float)(NBK - 1));
    return (int)f;   // NaN -> 0 (fmaxf returns the number)
  };
  bool lut = false;
  if (LUT && tab.lut_ok) {
    __syncthreads();
    for (int t = threadIdx.x; t < L; t += blockDim.x) tbk[t] = t < L - 1 ? bucket(thr[t]) : NBK;
    __syncthreads();
    // bcnt[k] = the number of thresholds whose bucket is below k (buckets
    // are monotone in the value, so those are exactly the ones below any
    // value of bucket k); a bucket holding three would break the search
    // below, so it turns the table off
    for (int kb = threadIdx.x; kb < NBK; kb += blockDim.x) {
      int lo = 0;
      for (int step = L / 2; step >= 1; step >>= 1)
        if (tbk[lo + step - 1] < kb) lo += step;
      bcnt[kb] = (uint8_t)lo;
    }
    int bad = 0;
    for (int t = threadIdx.x; t + 2 < L - 1; t += blockDim.x) bad |= tbk[t] == tbk[t + 2];
    lut = !__syncthreads_or(bad);
  }
  __syncthreads();
  const int wv = wave_id(), lane = threadIdx.x & 63;
  const int gi = lane / G, li = lane % G;          // vector of the set, lane within the vector
  constexpr int PER = U * VW;                      // vectors per wave iteration
  const int64_t stride = (int64_t)gridDim.x * 4 * PER;
  const uint32_t pa = (uint32_t)(4 * li) * BITS, pb = (uint32_t)(4 * li + N / 2) * BITS;   // run bits
  for (int64_t v0 = ((int64_t)blockIdx.x * 4 + wv) * PER; v0 < count; v0 += stride) {
    float x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* src = v + min(v0 + u * VW + gi, count - 1) * ldv + 4 * li;
      load8<VEC>(src, src + N / 2, x[u]);
    }
    for (int t = lane; t < WW; t += 64) pk[wv][t] = 0u;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[u][e], x[u][e], ss);
      const float norm = __builtin_sqrtf(group_sum<G>(ss));
      const float inv = norm > 0.f ? 1.f / norm : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[u][e] *= inv;
      fwht8<G>(x[u], lane);
      // nearest level: the number of thresholds strictly below r (binary search)
      float cc = 0.f;
      uint32_t run[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int lo = 0;
        if (LUT && lut) {
          // the count below the value's bucket, plus the (at most two)
          // thresholds of that bucket that lie below the value
          const int c = bcnt[bucket(x[u][e])];
          lo = c + (thr[c] < x[u][e]) + (thr[c + 1] < x[u][e]);
        } else {
#pragma unroll
          for (int step = L / 2; step >= 1; step >>= 1)
            if (thr[lo + step - 1] < x[u][e]) lo += step;
        }
        const uint32_t code = norm > 0.f ? (uint32_t)lo : 0u;
        const float c = cent[code];
        cc = __builtin_fmaf(c, c, cc);
        run[e >> 2] |= code << ((e & 3) * BITS);
      }
      const float cn = __builtin_sqrtf(group_sum<G>(cc));
      const float s = norm > 0.f ? norm / cn : 0.f;
      // the vector's record: code words, then s (the code stream ends on a
      // word boundary, so no run spills into the s word)
      uint32_t* rec = &pk[wv][(u * VW + gi) * RW];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint32_t p = r ? pb : pa;
        const uint64_t placed = (uint64_t)run[r] << (p & 31);
        atomicOr(rec + (p >> 5), (uint32_t)placed);
        if ((placed >> 32) != 0) atomicOr(rec + (p >> 5) + 1, (uint32_t)(placed >> 32));
      }
      if (li == 0) rec[CW] = __float_as_uint(s);
    }
    __builtin_amdgcn_wave_barrier();
    const int words = (int)min((int64_t)PER, count - v0) * RW;
    uint32_t* dst = reinterpret_cast<uint32_t*>(out + v0 * (4 * RW));
    for (int t = lane; t < words; t += 64) dst[t] = pk[wv][t];
    __builtin_amdgcn_wave_barrier();
  }
}

// Decode: the same vector layout; each lane reads the code words holding its
// two runs (one word each, two for 3-bit codes) and the s word, every load
// of the iteration in flight together.
template <int G, int BITS, int U, bool VEC>
__global__ void __launch_bounds__(256) turbo_decode_kernel(const uint8_t* __restrict__ in,
                                                           int64_t count, float* __restrict__ v,
                                                           int64_t ldv, TurboTable tab) {
  constexpr int N = 8 * G, L = 1 << BITS, VW = 64 / G;
  constexpr int CW = N * BITS / 32, REC = 4 * (CW + 1);
  constexpr bool TWO = (32 % (4 * BITS)) != 0;   // a run may straddle two words
  __shared__ float cent[L];
  for (int i = threadIdx.x; i < L; i += blockDim.x) cent[i] = tab.cent[i];
  __syncthreads();
  const int wv = wave_id(), lane = threadIdx.x & 63;
  const int gi = lane / G, li = lane % G;
  constexpr int PER = U * VW;
  const int64_t stride = (int64_t)gridDim.x * 4 * PER;
  const uint32_t pa = (uint32_t)(4 * li) * BITS, pb = (uint32_t)(4 * li + N / 2) * BITS;
  for (int64_t v0 = ((int64_t)blockIdx.x * 4 + wv) * PER; v0 < count; v0 += stride) {
    const int nrec = (int)min((int64_t)PER, count - v0);
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + v0 * REC, (uint32_t)(nrec * REC));
    uint32_t wa[U][2], wb[U][2], sw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t base = (uint32_t)(min(u * VW + gi, nrec - 1) * REC);
      wa[u][0] = bload4(rin, base + 4u * (pa >> 5));
      wb[u][0] = bload4(rin, base + 4u * (pb >> 5));
      if (TWO) {   // the next word: at most the s word
        wa[u][1] = bload4(rin, base + 4u * ((pa >> 5) + 1));
        wb[u][1] = bload4(rin, base + 4u * ((pb >> 5) + 1));
      } else {
        wa[u][1] = wb[u][1] = 0u;
      }
      sw[u] = bload4(rin, base + 4u * CW);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t ra = (uint32_t)(((((uint64_t)wa[u][1]) << 32) | wa[u][0]) >> (pa & 31));
      const uint32_t rb = (uint32_t)(((((uint64_t)wb[u][1]) << 32) | wb[u][0]) >> (pb & 31));
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = cent[(ra >> (e * BITS)) & (L - 1)];
        x[e + 4] = cent[(rb >> (e * BITS)) & (L - 1)];
      }
      fwht8<G>(x, lane);
      const float s = __uint_as_float(sw[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= s;
      if (u * VW + gi < nrec) {
        float* dst = v + (v0 + u * VW + gi) * ldv + 4 * li;
        store8<VEC>(dst, dst + N / 2, x);
      }
    }
  }
}

template <int G>
int launch_turbo_g(bool enc, const void* src, int64_t count, int64_t ld, void* dst, int bits,
                   const TurboTable& tab, hipStream_t s) {
  constexpr int U = 2;   // vector sets per wave and iteration
  constexpr int PER = U * (64 / G);
  int64_t blocks = (count + 4 * PER - 1) / (4 * PER);
  if (blocks > 4096) blocks = 4096;
  const void* fp = enc ? src : dst;   // the f32 side
  const bool vec = (ld % 4) == 0 && (reinterpret_cast<uintptr_t>(fp) % 16) == 0;
#define HQ_T(B, V)                                                                                  \
  if (enc)                                                                                          \
    hipLaunchKernelGGL((turbo_encode_kernel<G, B, U, V>), dim3((unsigned)blocks), dim3(256), 0, s, \
                       static_cast<const float*>(src), count, ld, static_cast<uint8_t*>(dst), tab);  \
  else                                                                                              \
    hipLaunchKernelGGL((turbo_decode_kernel<G, B, U, V>), dim3((unsigned)blocks), dim3(256), 0, s, \
                       static_cast<const uint8_t*>(src), count, static_cast<float*>(dst), ld, tab);  \
  return (int)hipGetLastError();
#define HQ_TB(B)          \
  if (bits == B) {        \
    if (vec) {            \
      HQ_T(B, true)       \
    } else {              \
      HQ_T(B, false)      \
    }                     \
  }
  HQ_TB(2) HQ_TB(3) HQ_TB(4) HQ_TB(8)
#undef HQ_TB
#undef HQ_T
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_turbo(bool encode, const void* src, int64_t count, int n, int64_t ld, void* dst,
                 int bits, const TurboTable& tab, hipStream_t s) {
  if (count == 0) return 0;
  if (n == 64) return launch_turbo_g<8>(encode, src, count, ld, dst, bits, tab, s);
  if (n == 128) return launch_turbo_g<16>(encode, src, count, ld, dst, bits, tab, s);
  if (n == 256) return launch_turbo_g<32>(encode, src, count, ld, dst, bits, tab, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace hq
