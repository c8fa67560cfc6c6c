"""CPU oracle for HFQ4 top-k MoE decode -- TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The
product path (``quantized_moe_decode_amd``) never imports it, and this
package imports nothing from the product path: the two share no code.

What it is: a plain, slow, obviously correct restatement of what the
decode path computes, in numpy float64 (float32 only where the HFQ4 format
itself fixes f32 fields, i.e. the quantizer's scale/zero/code decisions).

Sources (web pages; cited by title and section):

* "hipfire：为AMD RDNA GPU打造的Rust原生LLM推理引擎" (zingnex.cn forum
  thread), section "2. HFQ量化格式与GEMV优化": the HFQ4 block -- 256
  weights stored in 136 bytes as an f32 scale, an f32 zero point and 128
  bytes of packed 4-bit data.
* hipfire expert-offload explainer (m.lqnn.cn/news/267029), section
  "125GB 的 MoE 模型，为什么 32GB 显卡也有得跑？": each token activates 8
  routed experts per MoE layer (top-8); section "PCIe 直通": the GPU kernel
  reads host-resident experts zero-copy (placement never changes results).
* Strata user report (lcz.me), section "3. 模型与引擎": every expert of a
  layer has its own gate, up and down tensors.

Everything the pages leave open (quantizer, dequant formula, nibble order,
router normalisation, activation, tie-break, padding of short rows) is a
stated reading; each function names the reading it takes.

Parity status per function:
* hfq4.quantize_rows / dequantize / matvec / packed_bytes -- pinned
  (hand-worked blocks, size identity against the page's per-layer figure,
  error bound, closed forms).
* moe.topk_lower_index / softmax_renorm -- pinned (closed forms, identity
  with the k-term softmax, brute force).
* moe.expert_forward / moe_layer -- pinned (constructed closed-form
  experts, brute-force enumeration on the tiny layer, permutation
  invariance).
* moe.zipf-biased routing, stack_step and host-mapped composition --
  "parity unpinned" against the pages: they follow readings, not passages;
  they are pinned only to their own stated definitions.
"""

from . import hfq4, moe  # noqa: F401
