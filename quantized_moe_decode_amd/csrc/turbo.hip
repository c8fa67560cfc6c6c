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
// Both kernels are HBM streams (4n bytes of f32 on one side, n b / 8 + 4 on
// the other) whose per-vector arithmetic must stay under the stream:
//  - encode puts a vector on G = n / 32 lanes, 32 values per lane, so most
//    of the transform stays inside a lane (butterflies of spans 1, 2, 4,
//    n/4 and n/2) and the per-vector work (norm, square root, division) is
//    shared by 32 values; only spans 8 .. 4 G pair lane j with lane j ^ M
//    (M < G <= 8: DPP quad permutes, and for n = 256 a pair of row
//    rotations).
//  - decode, bound by its f32 stores, puts a vector on 8 lanes (16 at
//    n = 256; runs of four values) so that each store instruction writes
//    128 or 256 contiguous bytes per vector, and stores with the
//    non-temporal hint (the output is not read back by the kernel).
// Every butterfly is exactly rounded; the 1/sqrt(n) factor is folded into
// the normalisation (encode) or the norm ratio (decode).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hfq4_device.h"
#include "launch.h"
#include "turbo.h"

namespace hq {
namespace {

// The value of lane l ^ M in every lane, M = 1, 2, 4 or 8.  M = 1, 2: quad
// permutes.  M = 8: row_ror:8.  M = 4: row_ror:12 gives every lane lane
// l + 4 (mod 16), then row_ror:4, written only in banks 1 and 3 (the lanes
// with bit 2 set, whose partner is lane l - 4), replaces it there.  Every
// lane's result is written by one of the moves, so their old values are
// never read.
template <int M>
__device__ __forceinline__ float xlane(float v) {
  const int b = __builtin_bit_cast(int, v);
  if (M == 1) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0xB1, 0xf, 0xf, true));
  if (M == 2) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0x4E, 0xf, 0xf, true));
  if (M == 8) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0x128, 0xf, 0xf, true));
  const int up = __builtin_amdgcn_mov_dpp(b, 0x12C, 0xf, 0xf, true);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(up, b, 0x124, 0xf, 0xA, false));
}

// Sum over the G lanes of a vector (aligned groups of 2, 4 or 8 lanes):
// xor 1, xor 2, then the other quad of the eight (row_half_mirror).
template <int G>
__device__ __forceinline__ float lanes_sum(float v) {
  v += dpp<0xB1>(v);
  if (G >= 4) v += dpp<0x4E>(v);
  if (G >= 8) v += dpp<0x141>(v);
  return v;
}

// Register layout: a vector of n = G V values on an aligned group of G
// lanes, V values per lane in runs of RL contiguous values: lane j holds
// x[RL q + i] = value RL j + RL G q + i (q < V / RL, i < RL), each run one
// or two 16-byte accesses.  In index bits: the low log2 RL bits are i, the
// next log2 G bits the lane, the top bits q -- so all index bits but the
// lane's are bits of the register index e = RL q + i.
//
// Walsh-Hadamard transform in place, unscaled (H with entries +-1): the
// butterflies (a, b) -> (a + b, a - b), a the lower index, over the bits of
// e, then one stage per lane bit, where the lane holding a keeps own +
// partner and the one holding b partner - own (a single fma with a +-1
// factor, exactly rounded).
template <int G, int V>
__device__ __forceinline__ void fwht(float (&x)[V], int lane) {
#pragma unroll
  for (int h = 1; h < V; h <<= 1) {
#pragma unroll
    for (int e = 0; e < V; ++e)
      if (!(e & h)) {
        const float a = x[e], b = x[e + h];
        x[e] = a + b;
        x[e + h] = a - b;
      }
  }
#define HQ_XSTAGE(M)                                         \
  if (M < G) {                                               \
    const float sg = (lane & (M)) ? -1.f : 1.f;              \
    _Pragma("unroll") for (int e = 0; e < V; ++e)            \
      x[e] = __builtin_fmaf(sg, x[e], xlane<M>(x[e]));       \
  }
  HQ_XSTAGE(1) HQ_XSTAGE(2) HQ_XSTAGE(4) HQ_XSTAGE(8)
#undef HQ_XSTAGE
}

// A lane's runs: V / RL runs of RL f32 values starting at p, run q at
// p + RL G q.
template <int G, int V, int RL, bool VEC>
__device__ __forceinline__ void load_runs(const float* p, float (&x)[V]) {
#pragma unroll
  for (int q = 0; q < V / RL; ++q) {
    const float* r = p + RL * G * q;
    if constexpr (VEC) {
#pragma unroll
      for (int h = 0; h < RL / 4; ++h) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(r + 4 * h);
        x[RL * q + 4 * h + 0] = a.x;
        x[RL * q + 4 * h + 1] = a.y;
        x[RL * q + 4 * h + 2] = a.z;
        x[RL * q + 4 * h + 3] = a.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < RL; ++i) x[RL * q + i] = r[i];
    }
  }
}
// Stores with the non-temporal hint.
template <int G, int V, int RL, bool VEC>
__device__ __forceinline__ void store_runs(float* p, const float (&x)[V]) {
#pragma unroll
  for (int q = 0; q < V / RL; ++q) {
    float* r = p + RL * G * q;
    if constexpr (VEC) {
#pragma unroll
      for (int h = 0; h < RL / 4; ++h) {
        const f32x4 o{x[RL * q + 4 * h + 0], x[RL * q + 4 * h + 1], x[RL * q + 4 * h + 2],
                      x[RL * q + 4 * h + 3]};
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(r + 4 * h));
      }
    } else {
#pragma unroll
      for (int i = 0; i < RL; ++i) __builtin_nontemporal_store(x[RL * q + i], r + i);
    }
  }
}

template <int N>
constexpr float inv_sqrt_n() {
  return N == 64 ? 0.125f : N == 128 ? 0.08838834764831845f : 0.0625f;
}

// Encode.  The nearest level is the number of thresholds below the rotated
// value r.  With the bucket table (lut): bucket(r) = clamp(fma(r, a, b), 0,
// NBK - 1) truncated, the buckets narrower than half the smallest gap
// between two thresholds, so at most one threshold m (the count of those in
// lower buckets) can share r's bucket and one compare with it decides; the
// entry {threshold m, level m, level m + 1} is one 16-byte LDS read.  The
// workgroup builds the table in LDS and checks that no bucket holds two
// thresholds; otherwise (or when asked) it searches the thresholds (binary
// search, log2 L dependent LDS reads).
// Layout: G = n / 32 lanes per vector, V = 32, runs of RL = 8.
// A wave takes VW = 64 / G vectors per iteration (a vector index past the
// end reads the last vector again and writes nothing).  Each lane's runs of
// eight codes go into the wave's records in LDS (code i of the vector at
// bits [i b, i b + b) of its code stream: whole words for b = 4 and 8, for
// b = 3 (n >= 128) whole words assembled from a quad of lanes' runs, and
// otherwise runs or-ed into zeroed words), and the iteration's records,
// contiguous in memory, leave as whole words with the non-temporal hint.
template <int G, int BITS, bool VEC>
__global__ void __launch_bounds__(256) turbo_encode_kernel(const float* __restrict__ v, int64_t count,
                                                           int64_t ldv, uint8_t* __restrict__ out,
                                                           TurboTable tab, int use_lut) {
  constexpr int N = 32 * G, L = 1 << BITS, VW = 64 / G;
  constexpr int CW = N * BITS / 32, RW = CW + 1;   // code words, record words
  constexpr int WW = VW * RW;                      // record words of one wave iteration
  constexpr int NBK = turbo_lut_buckets(BITS);
  constexpr bool WHOLE = BITS == 4 || BITS == 8;   // a run of eight codes fills whole words
  // 3 bits with G >= 4: a quad of lanes holds four consecutive 24-bit runs,
  // which fill three whole words together
  constexpr bool QUADS = BITS == 3 && G >= 4;
  constexpr bool ZERO = !(WHOLE || QUADS);   // runs or-ed into zeroed words
  constexpr int RUNW = BITS == 8 ? 2 : 1;          // words of a run's codes
  __shared__ uint32_t pk[4][WW];
  __shared__ f32x4 qt[L];                          // {threshold m (inf for m = L - 1), level m, level m + 1, 0}
  __shared__ int tbk[L];                           // bucket of threshold m (NBK for m = L - 1)
  __shared__ uint8_t tb[NBK];                      // thresholds in the buckets below bucket k
  const float la = tab.lut_a, lb = tab.lut_b;
  auto bucket = [&](float r) -> uint32_t {
    // NaN -> 0 (fmaxf returns the number); truncation of the clamped value
    return (uint32_t)fminf(fmaxf(__builtin_fmaf(r, la, lb), 0.f), (float)(NBK - 1));
  };
  for (int i = threadIdx.x; i < L; i += blockDim.x) {
    const float t = i < L - 1 ? tab.thr[i] : INFINITY;
    qt[i] = f32x4{t, tab.cent[i], tab.cent[i < L - 1 ? i + 1 : i], 0.f};
    tbk[i] = i < L - 1 ? (int)bucket(t) : NBK;
  }
  __syncthreads();
  bool lut = false;
  if (use_lut) {
    // each thread fills KPT consecutive buckets: a binary search for the
    // first, then a walk (tbk is sorted, and tbk[L - 1] = NBK ends it)
    constexpr int KPT = NBK >= 2048 ? NBK / 256 : 1;
    for (int k0 = threadIdx.x * KPT; k0 < NBK; k0 += blockDim.x * KPT) {
      int lo = 0;
#pragma unroll
      for (int step = L / 2; step >= 1; step >>= 1)
        if (tbk[lo + step - 1] < k0) lo += step;
      tb[k0] = (uint8_t)lo;
      for (int k = k0 + 1; k < k0 + KPT; ++k) {
        while (tbk[lo] < k) ++lo;
        tb[k] = (uint8_t)lo;
      }
    }
    int bad = 0;
    for (int t = threadIdx.x; t + 1 < L - 1; t += blockDim.x) bad |= tbk[t] == tbk[t + 1];
    lut = __builtin_amdgcn_readfirstlane(__syncthreads_or(bad)) == 0;   // uniform: one branch per iteration
  }
  const int wv = wave_id(), lane = threadIdx.x & 63;
  const int gi = lane / G, li = lane % G;          // vector of the wave, lane within the vector
  const int64_t stride = (int64_t)gridDim.x * 4 * VW;
  for (int64_t v0 = ((int64_t)blockIdx.x * 4 + wv) * VW; v0 < count; v0 += stride) {
    float x[32];
    load_runs<G, 32, 8, VEC>(v + min(v0 + gi, count - 1) * ldv + 8 * li, x);
    if (ZERO) {
      for (int t = lane; t < WW; t += 64) pk[wv][t] = 0u;
    }
    float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 32; ++e) p4[e & 3] = __builtin_fmaf(x[e], x[e], p4[e & 3]);
    const float norm = __builtin_sqrtf(lanes_sum<G>((p4[0] + p4[1]) + (p4[2] + p4[3])));
    const bool live = norm > 0.f;
    const float inv = live ? inv_sqrt_n<N>() / norm : 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] *= inv;
    fwht<G, 32>(x, lane);
    float c4[4] = {0.f, 0.f, 0.f, 0.f};
    uint32_t run[4][RUNW] = {};
    auto put = [&](int e, uint32_t code, float cv) {
      c4[e & 3] = __builtin_fmaf(cv, cv, c4[e & 3]);
      const int bit = (e & 7) * BITS;
      run[e >> 3][bit >> 5] |= code << (bit & 31);
    };
    if (lut) {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const uint32_t c = tb[bucket(x[e])];
        const f32x4 qv = qt[c];
        const bool up = qv.x < x[e];
        put(e, c + (up ? 1u : 0u), up ? qv.z : qv.y);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        int lo = 0;
#pragma unroll
        for (int step = L / 2; step >= 1; step >>= 1)
          if (qt[lo + step - 1].x < x[e]) lo += step;
        put(e, (uint32_t)lo, qt[lo].y);
      }
    }
    const float cn = __builtin_sqrtf(lanes_sum<G>((c4[0] + c4[1]) + (c4[2] + c4[3])));
    const float s = live ? norm / cn : 0.f;
    // the vector's record: code words, then s (the code stream ends on a
    // word boundary, so no run spills into the s word)
    uint32_t* rec = &pk[wv][gi * RW];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t p = (uint32_t)(8 * li + 8 * G * q) * BITS;   // bit position of run q
      if (WHOLE) {
#pragma unroll
        for (int w = 0; w < RUNW; ++w) rec[(p >> 5) + w] = live ? run[q][w] : 0u;
      } else if (QUADS) {
        // runs m = 4 i + t (lane t of a quad) make words 3 i .. 3 i + 2: lane
        // t < 3 writes word 3 i + t from its run and the next lane's
        // (quad_perm [1, 2, 3, 3])
        const int own = (int)(live ? run[q][0] : 0u);
        const uint32_t nxt = (uint32_t)__builtin_amdgcn_mov_dpp(own, 0xF9, 0xf, 0xf, true);
        const int t = li & 3, m = li + G * q;
        if (t < 3) rec[3 * (m >> 2) + t] = ((uint32_t)own >> (8 * t)) | (nxt << (24 - 8 * t));
      } else {
        const uint64_t placed = (uint64_t)(live ? run[q][0] : 0u) << (p & 31);
        atomicOr(rec + (p >> 5), (uint32_t)placed);
        if ((placed >> 32) != 0) atomicOr(rec + (p >> 5) + 1, (uint32_t)(placed >> 32));
      }
    }
    if (li == 0) rec[CW] = __float_as_uint(s);
    __builtin_amdgcn_wave_barrier();
    const int words = (int)min((int64_t)VW, count - v0) * RW;
    uint32_t* dst = reinterpret_cast<uint32_t*>(out + v0 * (4 * RW));
    for (int t = lane; t < words; t += 64) __builtin_nontemporal_store(pk[wv][t], dst + t);
    __builtin_amdgcn_wave_barrier();
  }
}

// Decode.  Layout: G lanes per vector (8, or 16 at n = 256), V = n / G
// values per lane in runs of RL = 4, so that each 16-byte store instruction
// writes 16 G contiguous bytes per vector; the stores carry the
// non-temporal hint (the kernel never reads its output).  Each lane reads
// the code words holding its runs (the next word too where a run may span
// two) and the s word.  The launch gives every wave one set of 64 / G
// vectors; the loop covers any other grid.
template <int N, int BITS, bool VEC>
__global__ void __launch_bounds__(256) turbo_decode_kernel(const uint8_t* __restrict__ in,
                                                           int64_t count, float* __restrict__ v,
                                                           int64_t ldv, TurboTable tab) {
  constexpr int G = N == 256 ? 16 : 8, V = N / G, RL = 4, NR = V / RL;
  constexpr int L = 1 << BITS, VW = 64 / G;
  constexpr int CW = N * BITS / 32, REC = 4 * (CW + 1);
  constexpr bool TWO = BITS == 3;                  // a run of four 3-bit codes may span two words
  __shared__ float cent[L];
  for (int i = threadIdx.x; i < L; i += blockDim.x) cent[i] = tab.cent[i];
  __syncthreads();
  const int wv = wave_id(), lane = threadIdx.x & 63;
  const int gi = lane / G, li = lane % G;
  const int64_t stride = (int64_t)gridDim.x * 4 * VW;
  for (int64_t v0 = ((int64_t)blockIdx.x * 4 + wv) * VW; v0 < count; v0 += stride) {
    const int nrec = (int)min((int64_t)VW, count - v0);
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + v0 * REC, (uint32_t)(nrec * REC));
    const uint32_t base = (uint32_t)(min(gi, nrec - 1) * REC);
    uint32_t w0[NR], w1[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const uint32_t p = (uint32_t)(RL * li + RL * G * q) * BITS;   // bit position of run q
      w0[q] = bload4(rin, base + 4u * (p >> 5));
      w1[q] = TWO ? bload4(rin, base + 4u * ((p >> 5) + 1)) : 0u;   // at most the s word
    }
    const float s = __uint_as_float(bload4(rin, base + 4u * CW));
    float x[V];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const uint32_t p = (uint32_t)(RL * li + RL * G * q) * BITS;
      const uint64_t r = ((((uint64_t)w1[q]) << 32) | w0[q]) >> (p & 31);
#pragma unroll
      for (int i = 0; i < RL; ++i) x[RL * q + i] = cent[(uint32_t)(r >> (i * BITS)) & (L - 1)];
    }
    fwht<G, V>(x, lane);
    const float sc = s * inv_sqrt_n<N>();
#pragma unroll
    for (int e = 0; e < V; ++e) x[e] *= sc;
    if (gi < nrec) store_runs<G, V, RL, VEC>(v + (v0 + gi) * ldv + RL * li, x);
  }
}

template <int N>
int launch_turbo_n(bool enc, const void* src, int64_t count, int64_t ld, void* dst, int bits,
                   const TurboTable& tab, bool lut, hipStream_t s) {
  // vectors per workgroup and iteration: 4 waves of 64 / G, G = n / 32
  // (encode) or 8, 16 at n = 256 (decode)
  const int per = enc ? 4 * (64 / (N / 32)) : 4 * (64 / (N == 256 ? 16 : 8));
  // Grid: the decoder one iteration per wave; the encoder, which builds its
  // level tables once per workgroup, two (four at n = 256).  A queue of
  // short-lived workgroups keeps the chip's active loads on a narrow
  // stretch of memory; on 1 GiB streams it measured 5-10 % faster than a
  // capped grid whose waves stride through the whole range.
  int64_t blocks = (count + per - 1) / per;
  if (enc) {
    const int iters = N == 256 ? 4 : 2;
    blocks = (blocks + iters - 1) / iters;
  }
  const void* fp = enc ? src : dst;   // the f32 side
  const bool vec = (ld % 4) == 0 && (reinterpret_cast<uintptr_t>(fp) % 16) == 0;
  const int use_lut = lut && tab.lut_ok;
#define HQ_T(B, V)                                                                                  \
  if (enc)                                                                                          \
    hipLaunchKernelGGL((turbo_encode_kernel<N / 32, B, V>), dim3((unsigned)blocks), dim3(256), 0, s, \
                       static_cast<const float*>(src), count, ld, static_cast<uint8_t*>(dst), tab,  \
                       use_lut);                                                                    \
  else                                                                                              \
    hipLaunchKernelGGL((turbo_decode_kernel<N, B, V>), dim3((unsigned)blocks), dim3(256), 0, s,    \
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
                 int bits, const TurboTable& tab, bool lut, hipStream_t s) {
  if (count == 0) return 0;
  if (n == 64) return launch_turbo_n<64>(encode, src, count, ld, dst, bits, tab, lut, s);
  if (n == 128) return launch_turbo_n<128>(encode, src, count, ld, dst, bits, tab, lut, s);
  if (n == 256) return launch_turbo_n<256>(encode, src, count, ld, dst, bits, tab, lut, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace hq
