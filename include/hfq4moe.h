/*
 * hfq4moe.h -- C ABI of libhfq4moe.so: HFQ4 4-bit block-quantized top-k MoE
 * decode on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *  [HFQ]     "hipfire：为AMD RDNA GPU打造的Rust原生LLM推理引擎", section
 *            "2. HFQ量化格式与GEMV优化": an HFQ4 block is 256 weights in 136
 *            bytes -- f32 scale, f32 zero point, 128 bytes of packed codes;
 *            the hot kernel is a dequantizing GEMV kept light on registers.
 *  [TOPK]    hipfire expert-offload explainer (m.lqnn.cn/news/267029),
 *            section "125GB 的 MoE 模型，为什么 32GB 显卡也有得跑？": each
 *            token activates 8 of a layer's routed experts (top-8).
 *  [PCIE]    same page, section "PCIe 直通": host-resident experts are read
 *            by the GPU kernel itself over PCIe from pinned, mapped memory.
 *  [REFUSE]  same page, section "放置算法": a configuration that does not
 *            fit is refused loudly, naming what is short and by how much.
 *  [EXPERTS] Strata user report (lcz.me), section "3. 模型与引擎": each
 *            expert of a layer has its own gate, up and down tensors.
 *
 * Readings taken where the pages are silent (stated once here, used by
 * every entry point): w = zero + scale*q; scale at byte 0 and zero at byte
 * 4 of a block (little-endian f32), codes at bytes 8..135 with element 2j
 * in the low nibble of byte j; blocks run along K inside one row and a
 * short row ends in a padded block (rows are never split across blocks);
 * routing = softmax over all E logits, top-k by logit (ties to the lower
 * expert index), selected probabilities renormalised to sum 1; expert FFN
 * = down( SiLU(gate x) * (up x) ); layer output = sum_j w_j * y_{e_j}.
 *
 * Conventions for every call:
 *  - Return value: HFQ4_OK (0) or a negative HFQ4_E_* code.  On error a
 *    detail string (e.g. "workspace needs N bytes, got M") is available
 *    from hfq4_last_error() in the calling thread.  Arguments are
 *    validated before anything is enqueued; a rejected call enqueues
 *    nothing.  No C++ exception ever crosses this interface.
 *  - Memory: every buffer belongs to the caller.  Device pointers may be
 *    device memory or pinned host memory mapped into the device address
 *    space (hipHostMalloc).  The library allocates nothing, frees nothing,
 *    keeps no pointer after a call returns and never synchronises: work is
 *    enqueued on `stream` (NULL = the null stream) and results are valid
 *    once the stream reaches that point.  Device faults surface as HIP
 *    errors at the caller's next synchronisation.
 *  - Outputs are overwritten, never accumulated into (a `residual` input,
 *    where offered, is added explicitly).  Results are bitwise
 *    reproducible for identical inputs and launch configuration.
 *  - Calls are safe from several host threads as long as calls that share
 *    a workspace are ordered on one stream.
 *  - Alignment: weight pointers and expert strides 16 bytes; f32 vectors
 *    16 bytes with leading dimensions a multiple of 4 elements.
 */
#ifndef HFQ4MOE_H
#define HFQ4MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status */
#define HFQ4_OK            0
#define HFQ4_E_INVALID    (-1)  /* bad argument: null, size, k > E, aliasing ... */
#define HFQ4_E_ALIGN      (-2)  /* pointer / stride / leading dimension misaligned */
#define HFQ4_E_WORKSPACE  (-3)  /* workspace too small (detail gives both sizes) */
#define HFQ4_E_DEVICE     (-4)  /* current device is not gfx950 */
#define HFQ4_E_HIP        (-5)  /* a HIP runtime call or kernel launch failed */
#define HFQ4_E_UNSUPPORTED (-6) /* valid request outside the sizes built here */

/* Sticky device-side error bits, OR-ed into the first 4 bytes of a MoE
 * workspace (see moe_workspace_bytes) or into hfq4_pack's `bad` counter. */
#define HFQ4_DEV_ERR_INDEX     1u  /* an expert index outside [0, E); its slot is skipped */
#define HFQ4_DEV_ERR_TIMEOUT   2u  /* reserved: no kernel of this build waits on another */
#define HFQ4_DEV_ERR_NONFINITE 4u  /* a non-finite router logit was seen */

/* Layer flags */
#define HFQ4_LAYER_HOST_MAPPED 1u  /* expert weights live in pinned host memory [PCIE].
                                      Results are bit-identical to the same layer in
                                      HBM.  With one token the gate/up kernel also copies
                                      the k selected down matrices into the workspace
                                      while the link is busy, so the down pass reads HBM
                                      (moe_workspace_bytes accounts for it). */

/* Limits of this build */
#define HFQ4_MAX_BATCH   16
#define HFQ4_MAX_EXPERTS 1024
#define HFQ4_MAX_TOPK    16

/* Thread-local detail of the last error in this thread ("" if none). */
const char* hfq4_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int hfq4_version(void);

/* ------------------------------------------------------------ HFQ4 format */

/* Bytes of an HFQ4 matrix of `rows` rows of length K [HFQ]:
 * rows * ceil(K/256) * 136.  K >= 1, rows >= 0.  Host only. */
int hfq4_packed_bytes(int64_t rows, int64_t K, size_t* out);

/* Quantize a row-major f32 matrix w[rows][ldw] (device) into HFQ4 rows
 * [HFQ].  Per 256-element block along K (the last one padded with code 0):
 * zero = min, scale = f32(f32(max - min) / 15), q = clamp(rint(f32(f32(w -
 * zero) / scale)), 0, 15) with round-half-to-even; scale 0 (all codes 0)
 * when max == min.  Output `out` (device, out_bytes >= hfq4_packed_bytes)
 * is written in canonical HFQ4 byte order, bit-exact with that definition.
 * A block holding a non-finite value, or whose f32 range overflows, is
 * written as all-zero bytes and counted: `bad` (device int32, may be NULL)
 * is incremented once per such block -- the caller zeroes it and reads it
 * back after synchronising.  Requires ldw >= K. */
int hfq4_pack(const float* w, int64_t rows, int64_t K, int64_t ldw,
              void* out, size_t out_bytes, int32_t* bad, hipStream_t stream);

/* Dequantizing GEMV [HFQ]:
 *   y[b][r] = residual[b][r] + sum_{i<K} (zero + scale*q)[r][i] * x[b][i]
 * for b < batch (1..HFQ4_MAX_BATCH), r < rows.  W: HFQ4 rows (device or
 * mapped host), x: f32 [batch][ldx], residual: f32 [batch][ldr] or NULL,
 * y: f32 [batch][ldy].  y must not overlap x or W; residual may be y itself
 * (in place) but must not partially overlap it.  Products are taken
 * with x scaled by a power of two per 32-element segment and rounded to
 * f16, accumulated in f32 (error well inside 1e-3 relative L2 for K <=
 * 16384, at any activation scale).  K <= 16384; batch*K <= 32768. */
int hfq4_gemv(const void* W, int64_t rows, int64_t K,
              const float* x, int64_t ldx, int batch,
              const float* residual, int64_t ldr,
              float* y, int64_t ldy, hipStream_t stream);

/* ------------------------------------------------------------ routing */

/* Workspace for moe_route_topk (bytes, device memory, zeroed once before
 * first use -- moe_workspace_init does it; the library leaves it zeroed
 * after every call that completes). */
int moe_route_workspace_bytes(int64_t E, int batch, size_t* out);

/* Router + top-k [TOPK]:
 *   logits[b][e] = sum_i Wr[e][i] * x[b][i] + bias[e]     (f32)
 *   idx[b][0..k)  = the k largest logits, ordered by (logit desc, index asc)
 *   wts[b][j]     = exp(l_j - l_0) / sum_{m<k} exp(l_m - l_0)
 * (identical to a full softmax over the E experts renormalised over the k
 * selected).  Wr: f32 [E][d] row-major; bias: f32 [E] or NULL; x: f32
 * [batch][ldx]; idx: int32 [batch][k]; wts: f32 [batch][k]; logits_out:
 * f32 [batch][E] or NULL.  1 <= k <= min(E, HFQ4_MAX_TOPK),
 * E <= HFQ4_MAX_EXPERTS, d % 4 == 0.  NaN logits are never selected
 * before finite ones and set HFQ4_DEV_ERR_NONFINITE in the workspace. */
int moe_route_topk(const float* Wr, const float* bias, int64_t E, int64_t d,
                   const float* x, int64_t ldx, int batch, int k,
                   int32_t* idx, float* wts, float* logits_out,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ experts */

/* One MoE layer's expert weights [EXPERTS]: for expert e,
 *   gate = (const uint8_t*)gate + e*stride_gate : HFQ4 [F rows][K = d]
 *   up   = (const uint8_t*)up   + e*stride_up   : HFQ4 [F rows][K = d]
 *   down = (const uint8_t*)down + e*stride_down : HFQ4 [d rows][K = F]
 * Strides >= the matrix size (so gate and up may be interleaved).
 * flags: HFQ4_LAYER_HOST_MAPPED when the pointers are pinned host memory
 * [PCIE] (same results; the reads cross PCIe, see the flag above). */
typedef struct moe_layer {
    const void* gate;
    const void* up;
    const void* down;
    int64_t E, d, F;
    int64_t stride_gate, stride_up, stride_down;
    uint32_t flags;
    uint32_t reserved;
} moe_layer;

/* Workspace for moe_expert_decode / moe_layer_decode (device bytes; first
 * 4 bytes = sticky HFQ4_DEV_ERR_* word; zero it once before first use). */
int moe_workspace_bytes(const moe_layer* L, int batch, int k, size_t* out);

/* Zero a workspace with a fill kernel (safe inside HIP graph capture). */
int moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/* Expert half of the layer, given the routing:
 *   y[b] = residual[b] + sum_{j<k} wts[b][j] * down_e( SiLU(gate_e x[b]) * (up_e x[b]) ),
 *   e = idx[b][j].
 * Tokens that share an expert read its weights once (grouping); an index
 * repeated within one token counts once per slot.  An index outside
 * [0, E) sets HFQ4_DEV_ERR_INDEX and contributes nothing.
 * x: f32 [batch][ldx]; idx: int32 [batch][k]; wts: f32 [batch][k];
 * residual: f32 [batch][ldy] or NULL; y: f32 [batch][ldy], must not
 * overlap x.  d <= 2048, F <= 2048, d % 4 == 0, F % 4 == 0.
 * For 1792 < d <= 2048, F = 512, k <= 8 the work runs on tuned kernels:
 * one token on the VALU (f16 dot products), 2..16 tokens on MFMA matrix
 * cores (each expert a small GEMM over the tokens that chose it).  The two
 * agree within the stated error, not bit for bit. */
int moe_expert_decode(const moe_layer* L, const float* x, int64_t ldx, int batch,
                      const int32_t* idx, const float* wts, int k,
                      const float* residual, float* y, int64_t ldy,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* Whole layer in one enqueue: moe_route_topk followed by
 * moe_expert_decode, same results bit for bit (idx, wts, y). */
int moe_layer_decode(const moe_layer* L, const float* Wr, const float* bias,
                     const float* x, int64_t ldx, int batch, int k,
                     int32_t* idx, float* wts, const float* residual,
                     float* y, int64_t ldy,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Testing hook: make the device check see `arch` instead of the real
 * device ("" or NULL restores the real query).  Lets the refusal on a
 * non-gfx950 device be exercised without such a device. */
int hfq4_debug_set_arch(const char* arch);

/* Diagnostics: register a device buffer (>= 256 KiB) that later decode
 * launches fill with per-workgroup phase timestamps (s_memrealtime, 100
 * MHz), slot [(kernel*1024 + workgroup)*8 + point]; NULL turns it off. */
int hfq4_debug_set_trace(void* dev, size_t bytes);

/* Diagnostics: hipEvent_t handles (cast to void*) recorded when each
 * later launch of the expert gate/up kernel starts and ends, so a caller
 * can time that kernel alone with hipEventElapsedTime; NULL, NULL turns it
 * off.  Not for use under HIP graph capture. */
int hfq4_debug_set_events(void* start, void* stop);

/* Device address of pinned host memory allocated with hipHostMalloc
 * (mapped), for use in moe_layer with HFQ4_LAYER_HOST_MAPPED [PCIE]. */
int hfq4_host_device_pointer(void* host, void** dev);

#ifdef __cplusplus
}
#endif
#endif /* HFQ4MOE_H */
