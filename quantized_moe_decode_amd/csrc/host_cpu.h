// Host (CPU) execution of HFQ4 experts: declarations shared by host_cpu.cpp
// and the C ABI.  Every pointer here is host memory.
#pragma once
#include <stdint.h>

namespace hq {

struct HostLayer {
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  int64_t E, d, F;
  int64_t stride_gate, stride_up, stride_down;
};

// Threads a call uses when the caller passes 0.
int host_threads_default();

// y[b] = residual[b] + W x[b] for b < batch (W: HFQ4 rows of K).
void gemv_host(const uint8_t* W, int64_t rows, int64_t K, const float* x, int64_t ldx, int batch,
               const float* residual, int64_t ldr, float* y, int64_t ldy, int nthreads);

// The expert half of a layer for a token batch, on the host: for each
// token, y = residual + sum_j wts_j * down_e(SiLU(gate_e x) * (up_e x)), e =
// idx_j; an index outside [0, E) adds nothing and sets bit 1 of *err.
void expert_decode_host(const HostLayer& L, const float* x, int64_t ldx, int batch,
                        const int32_t* idx, const float* wts, int k, const float* residual,
                        float* y, int64_t ldy, int nthreads, uint32_t* err);

}  // namespace hq
