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
 *  [PLACE]   same page, section "放置算法：auto 自动放置…": fixed weights
 *            first, then routed experts fill the device budget layer by
 *            layer; a decode-heat ranking (hot set) lets the device keep
 *            the most often selected experts; a configuration that does
 *            not fit is refused, naming the bytes short.  Strata user
 *            report, sections "1. Strata 是什么" and "5. 实测速度": the most
 *            routed experts cached on the device, the cache's hit rate.
 *  [TURBO]   page "hipfire：为AMD RDNA GPU打造的Rust原生LLM推理引擎", section
 *            "3. TurboQuant KV缓存压缩": KV vectors normalised to unit norm,
 *            rotated by a fast Walsh-Hadamard transform, quantised to
 *            Lloyd-Max centroids, stored with the ratio of the original to
 *            the reconstructed norm (exact norm on decode); 3.88x / 7.5x /
 *            9.85x / 14.2x against f32 for 8 / 4 / 3 / 2 bits.
 *  [CPUEXEC] hipfire explainer, section "PCIe 直通": host-resident experts
 *            can instead be computed by a CPU GEMV; at load the PCIe path
 *            and the CPU path are timed and the CPU is used only when it
 *            is at least 15% faster.  Strata user report, sections "1.
 *            Strata 是什么" and "2. 硬件配置": experts that miss the VRAM
 *            cache run on the CPU (AVX-2 kernels).
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
#define HFQ4_E_NOFIT      (-7)  /* a placement does not fit its budget (detail: bytes short) */

/* Sticky device-side error bits, OR-ed into the first 4 bytes of a MoE
 * workspace (see moe_workspace_bytes) or into hfq4_pack's `bad` counter. */
#define HFQ4_DEV_ERR_INDEX     1u  /* an expert index outside [0, E); its slot is skipped */
#define HFQ4_DEV_ERR_TIMEOUT   2u  /* a workgroup of a launch whose workgroups exchange data
                                      (pointer-table layers, the one- and two-launch one-token
                                      forms, the routing exchange of larger batches) waited more
                                      than 2 ms for another: the call's outputs are undefined and
                                      the workspace must be zeroed again before its next use */
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

/* Expert half of the layer, given the routing [EXPERTS] [TOPK] [HFQ]: each
 * token runs the k experts its router chose (top-8 in [TOPK]), each expert
 * its own gate, up and down HFQ4 tensors ([EXPERTS]: the per-expert
 * ffn_gate / ffn_up / ffn_down weights of an MoE layer), and the outputs are
 * mixed by the routing weights:
 *   y[b] = residual[b] + sum_{j<k} wts[b][j] * down_e( SiLU(gate_e x[b]) * (up_e x[b]) ),
 *   e = idx[b][j].
 * Tokens that share an expert read its weights once (grouping); an index
 * repeated within one token counts once per slot.  An index outside
 * [0, E) sets HFQ4_DEV_ERR_INDEX and contributes nothing.
 * x: f32 [batch][ldx]; idx: int32 [batch][k]; wts: f32 [batch][k];
 * residual: f32 [batch][ldy] or NULL; y: f32 [batch][ldy], must not
 * overlap x.  d <= 2048, F <= 2048, d % 4 == 0, F % 4 == 0, and
 * batch * k <= 128 (token, slot) pairs (HFQ4_E_UNSUPPORTED otherwise).
 * For 1792 < d <= 2048, F = 512, k <= 8 the work runs on tuned kernels:
 * one token on the VALU (f16 dot products), 2..16 tokens on MFMA matrix
 * cores (each expert a small GEMM over the tokens that chose it).  The two
 * agree within the stated error, not bit for bit. */
int moe_expert_decode(const moe_layer* L, const float* x, int64_t ldx, int batch,
                      const int32_t* idx, const float* wts, int k,
                      const float* residual, float* y, int64_t ldy,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* Whole layer in one enqueue [TOPK] [EXPERTS]: the decode step of one
 * routed-expert layer -- router logits, top-k selection of that layer's
 * experts for each token (top-8 in [TOPK]) and the selected experts' gate /
 * up / down computation and weighted mix ([EXPERTS]) -- equal to
 * moe_route_topk followed by moe_expert_decode, same results bit for bit
 * (idx, wts, y).  Arguments as in those two calls; Wr: f32 [E][d], bias:
 * f32 [E] or NULL.  Errors: as the two calls (nothing is enqueued on a
 * refusal). */
int moe_layer_decode(const moe_layer* L, const float* Wr, const float* bias,
                     const float* x, int64_t ldx, int batch, int k,
                     int32_t* idx, float* wts, const float* residual,
                     float* y, int64_t ldy,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: moe_layer_decode without
 * a caller workspace.  The scratch it needs (the workspace's contents) is a
 * fixed device array of this library, HFQ4_NOALLOC_SCRATCH_BYTES per GPU,
 * held by each GPU the library runs on until the process ends; the call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * Arguments and results are those of moe_layer_decode, bit for bit, except:
 *  - no ws / ws_bytes; a call whose workspace (moe_workspace_bytes) would
 *    exceed HFQ4_NOALLOC_SCRATCH_BYTES is refused with HFQ4_E_WORKSPACE
 *    (every shape of d <= 2048, F = 512, E <= 1024, k <= 8 fits, host-mapped
 *    one-token layers included);
 *  - err: device uint32 that receives the sticky HFQ4_DEV_ERR_* bits (OR-ed;
 *    the caller zeroes it), or NULL to drop them.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or host threads without ordering) race and give
 * undefined results; order them on one stream.  No part of the array needs
 * to be zero at the start of a call. */
#define HFQ4_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_layer_decode_noalloc(const moe_layer* L, const float* Wr, const float* bias,
                             const float* x, int64_t ldx, int batch, int k,
                             int32_t* idx, float* wts, const float* residual,
                             float* y, int64_t ldy, uint32_t* err, hipStream_t stream);

/* ------------------------------------------------------------ expert cache [PLACE] */

#define HFQ4_PLACE_LAYERS 0   /* whole layers, first to last, while the budget lasts */
#define HFQ4_PLACE_HOTSET 1   /* single experts by decode heat, hottest first */

/* Placement of `layers` x E routed experts (expert_bytes each) into an HBM
 * budget [PLACE].  The fixed weights (router, dense, everything that is
 * not a routed expert: fixed_bytes) are placed first; if they alone exceed
 * budget_bytes the call fails with HFQ4_E_NOFIT and a detail naming the
 * bytes short.  Then experts are placed while they fit:
 *  HFQ4_PLACE_LAYERS  whole layers in order (heat may be NULL);
 *  HFQ4_PLACE_HOTSET  single experts by heat[l*E + e] (selection counts of
 *                     a calibration decode), the hottest first, equal heat
 *                     to the lower (layer, expert) index.
 * resident[l*E + e] (host, layers*E bytes) receives 1 for experts placed
 * in HBM, 0 for the rest (pinned host memory); *placed_bytes (may be NULL)
 * the expert bytes placed.  Host only, deterministic. */
int moe_place_experts(int mode, int64_t layers, int64_t E, const uint64_t* heat,
                      uint64_t expert_bytes, uint64_t fixed_bytes, uint64_t budget_bytes,
                      uint8_t* resident, uint64_t* placed_bytes);

/* A layer whose experts are reached through a pointer table [PLACE]
 * [PCIE]: ptr[3e + 0/1/2] (device memory, E*3 entries) hold device-visible
 * addresses of expert e's gate [F][d], up [F][d] and down [d][F] HFQ4
 * matrices -- an HBM slot of an expert cache, or pinned host memory mapped
 * for the device (hfq4_host_device_pointer) -- each 16-byte aligned and
 * valid for the whole call.  resident (device, E bytes, or NULL) marks the
 * experts whose matrices are in HBM. */
typedef struct moe_layer_table {
    const uint64_t* ptr;
    const uint8_t* resident;
    int64_t E, d, F;
} moe_layer_table;

/* moe_layer_decode for one token of a table layer: the same results, bit
 * for bit, as a layer holding the same bytes in one tensor each.  hits
 * (device uint64 [2], or NULL) accumulates the selections of experts
 * marked resident ([0]) and of the others ([1]) -- the cache's hit count.
 * It runs as the single-launch layer (one workgroup per compute unit).
 * Supported: batch 1, the tuned shape (1792 < d <= 2048, F = 512,
 * k in {2, 4, 8}, E <= 1024) and a device of 256 compute units; other
 * requests fail with HFQ4_E_UNSUPPORTED.  ws as for moe_layer_decode with
 * an HBM layer of the same E, d, F, batch 1. */
int moe_layer_decode_table(const moe_layer_table* L, const float* Wr, const float* bias,
                           const float* x, int batch, int k, int32_t* idx, float* wts,
                           const float* residual, float* y, uint64_t* hits,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ TurboQuant KV codec [TURBO] */

/* Readings (the page gives the steps, not these details): rotation by the
 * orthonormal Walsh-Hadamard matrix H_n / sqrt(n) in natural order, no
 * random signs; levels = the Lloyd-Max quantiser of the standard normal
 * with 2^bits levels scaled by 1/sqrt(n), each rotated coordinate taking
 * the nearest level (ties to the lower); record of one vector = the n codes
 * packed LSB-first (code j at bits [j*bits, j*bits + bits) of a
 * little-endian bit stream), then s = |v| / |c| as an f32 (c the chosen
 * levels), n*bits/8 + 4 bytes; a zero vector stores codes 0 and s = 0.
 * Decode: v' = s * H c / sqrt(n), whose norm is |v| up to the f32 of s.
 * Supported: n in {64, 128, 256}, bits in {2, 3, 4, 8}. */

/* Bytes of one encoded vector. */
int turbo_record_bytes(int n, int bits, size_t* out);

/* The level table the kernels use (host floats, 2^bits entries,
 * ascending), for inspection. */
int turbo_levels(int n, int bits, float* levels);

/* Encode count vectors v[i][0..n) (device f32, row stride ldv >= n
 * elements) into out (device, count * turbo_record_bytes bytes, 4-byte
 * aligned).  One wave per vector; enqueued on stream. */
int turbo_encode(const float* v, int64_t count, int n, int64_t ldv, int bits, void* out,
                 size_t out_bytes, hipStream_t stream);

/* Decode count records (device) into v[i][0..n) (device f32, row stride
 * ldv >= n). */
int turbo_decode(const void* in, size_t in_bytes, int64_t count, int n, int bits, float* v,
                 int64_t ldv, hipStream_t stream);

/* ------------------------------------------------------------ host CPU execution */

/* Dequantizing GEMV on the host CPU [CPUEXEC] [HFQ]: the same result as
 * hfq4_gemv (y[b] = residual[b] + W x[b]), computed in f32 with FMA
 * (AVX-512 or AVX2 where the CPU has it) on `nthreads` host threads (0 =
 * one per CPU in the calling process's affinity mask, at most
 * OMP_NUM_THREADS when that is set and at most 64; a pool created on first
 * use serves every later call).  Every
 * pointer is host memory (pinned or pageable); nothing touches a GPU and
 * the call returns when y is written.  Each output is summed by one thread
 * in a fixed order, so results do not depend on nthreads.  batch 1..16,
 * K >= 1; y must not overlap x or W, residual may be y. */
int hfq4_gemv_host(const void* W, int64_t rows, int64_t K, const float* x, int64_t ldx,
                   int batch, const float* residual, int64_t ldr, float* y, int64_t ldy,
                   int nthreads);

/* The expert half of a layer on the host CPU [CPUEXEC] [EXPERTS]: the same
 * result as moe_expert_decode, with L's gate/up/down pointers, x, idx, wts,
 * residual and y all host memory.  An index outside [0, E) adds nothing and
 * sets HFQ4_DEV_ERR_INDEX in *err (host uint32, may be NULL).  Layer limits
 * as for moe_expert_decode. */
int moe_expert_decode_host(const moe_layer* L, const float* x, int64_t ldx, int batch,
                           const int32_t* idx, const float* wts, int k,
                           const float* residual, float* y, int64_t ldy, int nthreads,
                           uint32_t* err);

/* The measured route choice for host-resident experts [CPUEXEC]: given the
 * time one decode step of such a layer takes when the GPU reads the experts
 * over PCIe and when the CPU computes them (both measured by the caller on
 * this machine), *use_cpu = 1 only if the CPU is at least 15% faster
 * (cpu_seconds * 1.15 <= pcie_seconds), else 0: the decision leans to the
 * PCIe path.  Times must be positive and finite. */
int hfq4_offload_choice(double pcie_seconds, double cpu_seconds, int* use_cpu);

/* Diagnostics: the row kernel of hfq4_gemv_host and moe_expert_decode_host
 * for later calls (process-wide): kernel = 0 the best this CPU has (the
 * default), 1 AVX-512, 2 AVX2 + FMA, 3 portable C++.  HFQ4_E_UNSUPPORTED
 * if the CPU lacks the instructions.  *in_use (may be NULL) receives the
 * kernel calls now use (1..3).  Results agree to f32 rounding across
 * kernels; each kernel alone is independent of the thread count. */
int hfq4_debug_set_host_kernel(int kernel, int* in_use);

/* Testing hook: make the device check see `arch` instead of the real
 * device ("" or NULL restores the real query).  Lets the refusal on a
 * non-gfx950 device be exercised without such a device. */
int hfq4_debug_set_arch(const char* arch);

/* Diagnostics: register a device buffer (>= 256 KiB) that later decode
 * launches fill with per-workgroup phase timestamps (s_memrealtime, 100
 * MHz), slot [(kernel*1024 + workgroup)*8 + point]; NULL turns it off. */
int hfq4_debug_set_trace(void* dev, size_t bytes);

/* Diagnostics: one-token layers of the tuned shape with k in {2, 4, 8}
 * (moe_layer_decode, moe_expert_decode) run as the three-launch chain
 * router -> gate/up -> down (on = 0, the default) or as one launch of one
 * workgroup per compute unit whose workgroups exchange the logits, each
 * slot's h and the per-slot down sums through tagged words (on != 0;
 * 256-compute-unit devices only).  Both give the same bits; the switch
 * exists to compare them and is process-wide. */
int hfq4_debug_set_single_launch(int on);

/* Diagnostics: batched calls (moe_layer_decode) of at least
 * max(min_batch, 5) tokens (2 <= min_batch <= HFQ4_MAX_BATCH + 1; default
 * 9) route by exchange -- one workgroup per token runs the top-k and the
 * gate/up workgroups gather the selections through tagged words, whose
 * generation the router launch advances -- and smaller ones route every
 * token in every gate/up workgroup.  Same bits either way; process-wide. */
int hfq4_debug_set_route_exchange(int min_batch);

/* Diagnostics: the TurboQuant encoder (turbo_encode) finds each nearest
 * level through its bucket table (binary = 0, the default) or by binary
 * search over the thresholds (binary != 0).  Same codes either way; the
 * switch exists to test the search the encoder falls back to, and is
 * process-wide. */
int hfq4_debug_set_turbo_search(int binary);

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
