// hfq4_gemv: y = residual + W x for HFQ4 rows, batch 1..16.
//
// The dequantizing GEMV is the hot kernel the HFQ4 format was designed for
// (page "hipfire：为AMD RDNA GPU打造的Rust原生LLM推理引擎", section
// "2. HFQ量化格式与GEMV优化": few registers per lane so that many waves are
// in flight to hide memory latency).  On gfx950 the same goal is met by
// issuing every weight load of a wave before the first use, keeping the
// activation fragment of the lane's fixed segment in registers, and
// decoding nibbles straight into f16 pairs for v_dot2 (hfq4_device.h).
#include "hfq4_device.h"
#include "launch.h"

namespace hq {

constexpr int GEMV_WG_PER_CU = 4;   // workgroups per CU in the grid of a GEMV below 512 MiB
constexpr int GEMV_RPW_LONG = 4;    // row loads per wave and group of a long GEMV
// workgroups per CU in a long GEMV's grid: 3 fit at once (137 VGPRs), the
// others queue; a queue of workgroups that each take a short stretch of the
// matrix kept the chip's loads on fewer DRAM pages than 3 per CU striding
// through all of it (1-4 GiB: 5.5-5.7 against 5.3 TB/s; 6: 5.4, 12: 5.5,
// 48: 5.1-5.6, uncapped 3.4-3.6, where each workgroup's staging of x
// dominates)
constexpr int GEMV_WG_PER_CU_LONG = 24;

// Rows of nb <= NB blocks (K <= 256*NB); SEGS = 8*NB lanes per row, G =
// 64/SEGS rows per load instruction, RPW load instructions per wave: a
// wave's group is RPW*G rows.  Lanes whose block index is >= nb load
// nothing and contribute zero.  The grid is capped (4 or 24 workgroups per
// CU), so a wave walks groups wave, wave + (waves in the grid), ... with the
// next group's loads in flight while it computes the current one; x is
// staged once per workgroup.
template <int NB, int RPW>
__global__ void __launch_bounds__(256) gemv_narrow_kernel(const uint8_t* __restrict__ W,
                                                          int64_t rows, int K,
                                                          const float* __restrict__ x, int64_t ldx,
                                                          int batch, const float* __restrict__ res,
                                                          int64_t ldr, float* __restrict__ y,
                                                          int64_t ldy) {
  constexpr int SEGS = 8 * NB, G = 64 / SEGS, GROUP = RPW * G;
  const int nb = (K + BLK - 1) / BLK;
  const int64_t ROWB = (int64_t)nb * BLK_BYTES;
  extern __shared__ __align__(16) uint8_t lds[];
  // the wave index stays a per-lane value here: through wave_id() the
  // streaming loop measured slower
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane / SEGS, s = lane % SEGS;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + wv;
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x >> 6) * GROUP;
  int64_t row0 = wave * GROUP;

  // Token 0's activations go out first (eight lanes per segment, one pass:
  // SEGS <= 64 = 2 x 32 segment groups of the 256 threads), then this
  // wave's first weight loads, so that x is converted while the weights are
  // in flight.  With K not a multiple of 4 the staging below reads x itself.
  const bool k4 = (K & 3) == 0;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, 4u * (uint32_t)K);
  const int j8 = threadIdx.x & 7, s8 = threadIdx.x >> 3, G8 = blockDim.x >> 3;
  const f32x4 xa = load_seg8(rx, k4 && s8 < SEGS ? s8 : -1, j8);
  const f32x4 xb = load_seg8(rx, k4 && s8 + G8 < SEGS ? s8 + G8 : -1, j8);

  // One wave-uniform descriptor covers the matrix (rows * ROWB < 2^31,
  // split by the launcher); rows past the end and dead lanes read zeros,
  // so the loads need no branch.
  const uint32_t wbytes = (uint32_t)(rows * ROWB);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(W, wbytes);
  // token 0's residual travels with the weights (a null residual reads 0)
  const uint32_t rbytes = res ? (uint32_t)(4 * rows) : 0u;
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(res, rbytes);
  const bool live = (s >> 3) < nb;
  auto issue = [&](int64_t r0, u32x4 (&codes)[RPW], u32x2 (&hdr)[RPW], uint32_t (&r)[RPW]) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int64_t row = r0 + i * G + g;
      const uint32_t off = (live && row < rows) ? (uint32_t)(row * ROWB + (s >> 3) * BLK_BYTES) : wbytes;
      hdr[i] = bload8(rs, off);
      codes[i] = bload16(rs, off + 8 + 16 * (s & 7));
      r[i] = bload4(rr, row < rows ? (uint32_t)(4 * row) : rbytes);
    }
  };
  u32x4 codes[RPW];
  u32x2 hdr[RPW];
  uint32_t r0v[RPW];
  issue(row0, codes, hdr, r0v);

  const int fb = frag_bytes(SEGS);
  if (k4) {
    if (s8 < SEGS) build_seg8(xa, SEGS, s8, j8, lds);            // uniform per lane group
    if (s8 + G8 < SEGS) build_seg8(xb, SEGS, s8 + G8, j8, lds);
    for (int b = 1; b < batch; ++b)
      stage_vector8(x + b * ldx, K, SEGS, lds + b * fb, threadIdx.x, blockDim.x);
  } else {
    for (int b = 0; b < batch; ++b)
      stage_vector(x + b * ldx, K, SEGS, lds + b * fb, threadIdx.x, blockDim.x);
  }
  __syncthreads();

  auto compute = [&](int64_t r0, const u32x4 (&codes)[RPW], const u32x2 (&hdr)[RPW],
                     const uint32_t (&r)[RPW]) {
    for (int b = 0; b < batch; ++b) {
      Frag f;
      frag_load(lds + b * fb, SEGS, s, f);
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        float p = dot_seg(codes[i], hdr[i], f);
        p = group_sum<SEGS>(p);
        const int64_t row = r0 + i * G + g;
        if (s == 0 && row < rows) {
          const float rv = b == 0 ? as_f32(r[i]) : (res ? res[b * ldr + row] : 0.f);
          y[b * ldy + row] = rv + p;
        }
      }
    }
  };
  // two register sets in turn: the next group's loads go out before the
  // current group is computed, and no loaded value is copied
  u32x4 codes2[RPW];
  u32x2 hdr2[RPW];
  uint32_t r2v[RPW];
  while (row0 < rows) {
    issue(row0 + stride, codes2, hdr2, r2v);
    compute(row0, codes, hdr, r0v);
    row0 += stride;
    if (row0 >= rows) break;
    issue(row0 + stride, codes, hdr, r0v);
    compute(row0, codes2, hdr2, r2v);
    row0 += stride;
  }
}

// Rows wider than 2048: lanes stride over the segments of one row at a time.
__global__ void __launch_bounds__(256) gemv_wide_kernel(const uint8_t* __restrict__ W, int64_t rows,
                                                        int K, const float* __restrict__ x,
                                                        int64_t ldx, int batch,
                                                        const float* __restrict__ res, int64_t ldr,
                                                        float* __restrict__ y, int64_t ldy) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int NB = (K + BLK - 1) / BLK;
  const int S = NB * SEGS_PER_BLK;
  const int64_t ROWB = (int64_t)NB * BLK_BYTES;
  const int fb = frag_bytes(S);
  for (int b = 0; b < batch; ++b)
    stage_vector(x + b * ldx, K, S, lds + b * fb, threadIdx.x, blockDim.x);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(W, (uint32_t)(rows * ROWB));
  const uint32_t rbase = (uint32_t)(row * ROWB);
  float acc[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) acc[b] = 0.f;
  for (int s = lane; s < S; s += 64) {
    const uint32_t off = rbase + (uint32_t)((s >> 3) * BLK_BYTES);
    const u32x2 hdr = bload8(rs, off);
    const u32x4 codes = bload16(rs, off + 8 + 16 * (s & 7));
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      if (b < batch) {
        Frag f;
        frag_load(lds + b * fb, S, s, f);
        acc[b] += dot_seg(codes, hdr, f);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    if (b < batch) {
      const float p = group_sum<64>(acc[b]);
      if (lane == 0) y[b * ldy + row] = (res ? res[b * ldr + row] : 0.f) + p;
    }
  }
}

template <int NB, int RPW>
static int launch_narrow_rpw(const void* W, int64_t rows, int K, const float* x, int64_t ldx,
                             int batch, const float* res, int64_t ldr, float* y, int64_t ldy,
                             hipStream_t s) {
  constexpr int G = 64 / (8 * NB);
  const int64_t waves = (rows + RPW * G - 1) / (RPW * G);
  int64_t blocks = (waves + 3) / 4;
  // larger matrices loop (each wave strides over row groups)
  const int64_t cap = (int64_t)num_cus() * (RPW == 2 ? GEMV_WG_PER_CU : GEMV_WG_PER_CU_LONG);
  if (blocks > cap) blocks = cap;
  const size_t shm = (size_t)batch * frag_bytes(8 * NB);
  if (int e = allow_lds(gemv_narrow_kernel<NB, RPW>, shm)) return e;
  hipLaunchKernelGGL((gemv_narrow_kernel<NB, RPW>), dim3((unsigned)blocks), dim3(256), shm, s,
                     static_cast<const uint8_t*>(W), rows, K, x, ldx, batch, res, ldr, y, ldy);
  return (int)hipGetLastError();
}

// Two row loads per wave and group (more waves, shorter latency); from
// 512 MiB of weights on, GEMV_RPW_LONG (more bytes in flight per wave:
// measured 5.5 against 5.2 TB/s at 2-4 GiB, and slower below 512 MiB).
template <int NB>
static int launch_narrow(const void* W, int64_t rows, int K, const float* x, int64_t ldx,
                         int batch, const float* res, int64_t ldr, float* y, int64_t ldy,
                         hipStream_t s) {
  if (rows * (int64_t)(((K + BLK - 1) / BLK) * BLK_BYTES) < ((int64_t)1 << 29))
    return launch_narrow_rpw<NB, 2>(W, rows, K, x, ldx, batch, res, ldr, y, ldy, s);
  return launch_narrow_rpw<NB, GEMV_RPW_LONG>(W, rows, K, x, ldx, batch, res, ldr, y, ldy, s);
}

static int launch_gemv_rows(const void* W, int64_t rows, int64_t K, const float* x, int64_t ldx,
                            int batch, const float* residual, int64_t ldr, float* y, int64_t ldy,
                            hipStream_t s);

// Rows are processed in chunks whose packed size stays below 2^31 bytes, the
// reach of one buffer descriptor.
int launch_gemv(const void* W, int64_t rows, int64_t K, const float* x, int64_t ldx, int batch,
                const float* residual, int64_t ldr, float* y, int64_t ldy, hipStream_t s) {
  const int64_t rowb = ((K + BLK - 1) / BLK) * BLK_BYTES;
  const int64_t chunk = ((int64_t)1 << 31) / rowb;
  for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
    const int64_t n = rows - r0 < chunk ? rows - r0 : chunk;
    const int e = launch_gemv_rows(static_cast<const uint8_t*>(W) + r0 * rowb, n, K, x, ldx, batch,
                                   residual ? residual + r0 : nullptr, ldr, y + r0, ldy, s);
    if (e) return e;
  }
  return 0;
}

static int launch_gemv_rows(const void* W, int64_t rows, int64_t K, const float* x, int64_t ldx,
                            int batch, const float* residual, int64_t ldr, float* y, int64_t ldy,
                            hipStream_t s) {
  if (rows == 0) return 0;
  const int NB = (int)((K + BLK - 1) / BLK);
  const int k = (int)K;
  switch (NB) {
    case 1: return launch_narrow<1>(W, rows, k, x, ldx, batch, residual, ldr, y, ldy, s);
    case 2: return launch_narrow<2>(W, rows, k, x, ldx, batch, residual, ldr, y, ldy, s);
    case 3:
    case 4: return launch_narrow<4>(W, rows, k, x, ldx, batch, residual, ldr, y, ldy, s);
    case 5: case 6: case 7:
    case 8: return launch_narrow<8>(W, rows, k, x, ldx, batch, residual, ldr, y, ldy, s);
    default: {
      const int64_t blocks = (rows + 3) / 4;
      const size_t shm = (size_t)batch * frag_bytes(NB * SEGS_PER_BLK);
      if (int e = allow_lds(gemv_wide_kernel, shm)) return e;
      hipLaunchKernelGGL(gemv_wide_kernel, dim3((unsigned)blocks), dim3(256), shm, s,
                         static_cast<const uint8_t*>(W), rows, k, x, ldx, batch, residual, ldr, y,
                         ldy);
      return (int)hipGetLastError();
    }
  }
}

}  // namespace hq
