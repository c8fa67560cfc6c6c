"""HFQ4 block format: quantize, dequantize, matvec (oracle; test infrastructure).

Format (page "hipfire：为AMD RDNA GPU打造的Rust原生LLM推理引擎", section
"2. HFQ量化格式与GEMV优化"): a block holds 256 weights in 136 bytes -- an f32
scale, an f32 zero point and 128 bytes of packed 4-bit codes.

Readings taken where the page is silent:

* byte order inside a block: scale at byte 0, zero at byte 4 (both
  little-endian IEEE f32), codes at bytes 8..135;
* nibble order: element 2j sits in the low nibble of code byte j, element
  2j+1 in its high nibble;
* dequantization: w = zero + scale * q, q in 0..15;
* quantizer: min/max affine -- zero = min, scale = (max - min) / 15 (f32
  subtract, then f32 divide), q = clamp(rint((w - zero) / scale), 0, 15)
  with f32 subtract and f32 divide and round-half-to-even; a block with
  max == min stores scale 0 and all codes 0;
* signed zeros: -0.0 and +0.0 compare equal, so a block whose minimum is a
  zero has no single "smallest" element; the zero field then holds +0.0
  (the minimum plus +0.0 in f32, which maps -0.0 to +0.0 and leaves every
  other value unchanged), so the stored bytes never depend on which of the
  equal zeros a min() happens to return;
* blocks run along K inside one row; a row whose K is not a multiple of 256
  ends in a padded block (min/max over the valid elements only, padded codes
  0, padded positions contribute nothing);
* non-finite weights, and blocks whose f32 range (max - min) overflows,
  are rejected.
"""

import numpy as np

BLOCK = 256          # weights per block
BLOCK_BYTES = 136    # 4 (scale) + 4 (zero) + 128 (codes)
CODE_BYTES = 128


def blocks_per_row(K):
    """Number of 256-weight blocks in one row of length K (last one padded)."""
    if K < 1:
        raise ValueError("K must be >= 1")
    return (K + BLOCK - 1) // BLOCK


def packed_bytes(rows, K):
    """Bytes of an HFQ4 matrix: rows * ceil(K/256) * 136 (no padding between
    blocks or rows)."""
    if rows < 0:
        raise ValueError("rows must be >= 0")
    return rows * blocks_per_row(K) * BLOCK_BYTES


def quantize_block(w):
    """Quantize <= 256 f32 values (one block) -> (scale f32, zero f32, codes u8[256]).

    Decisions are taken in f32, the precision of the stored fields.
    """
    w = np.asarray(w, dtype=np.float32)
    n = w.shape[0]
    if not 1 <= n <= BLOCK:
        raise ValueError("a block holds 1..256 valid weights")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    mn = np.float32(w.min())
    mx = np.float32(w.max())
    rng = np.float32(mx - mn)                      # f32 subtract
    if not np.isfinite(rng):
        raise ValueError("block range overflows f32")
    scale = np.float32(rng / np.float32(15.0))     # f32 divide
    zero = np.float32(mn + np.float32(0.0))        # -0.0 -> +0.0 (signed-zero reading)
    codes = np.zeros(BLOCK, dtype=np.uint8)
    if scale != 0:
        t = np.float32(w - zero) / scale           # f32 subtract, f32 divide
        t = t.astype(np.float32)
        q = np.rint(t)                             # round half to even
        q = np.clip(q, 0, 15)
        codes[:n] = q.astype(np.uint8)
    return scale, zero, codes


def encode_block(scale, zero, codes):
    """Serialise one block: [scale f32 LE][zero f32 LE][code byte j = q[2j] | q[2j+1] << 4]."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape == (BLOCK,)
    out = bytearray()
    out += np.array([scale], dtype="<f4").tobytes()
    out += np.array([zero], dtype="<f4").tobytes()
    lo = codes[0::2]
    hi = codes[1::2]
    out += (lo | (hi << 4)).astype(np.uint8).tobytes()
    assert len(out) == BLOCK_BYTES
    return bytes(out)


def quantize_rows(W):
    """Quantize a row-major f32 matrix [rows, K] -> packed uint8 array of
    packed_bytes(rows, K) bytes (rows concatenated, each row its blocks)."""
    W = np.asarray(W, dtype=np.float32)
    if W.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    rows, K = W.shape
    nb = blocks_per_row(K)
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    # Vectorised over blocks; identical decisions to quantize_block.
    pad = nb * BLOCK - K
    valid = np.ones((rows, nb * BLOCK), dtype=bool)
    if pad:
        valid[:, K:] = False
    Wp = np.zeros((rows, nb * BLOCK), dtype=np.float32)
    Wp[:, :K] = W
    Wb = Wp.reshape(rows, nb, BLOCK)
    Vb = valid.reshape(rows, nb, BLOCK)
    mn = np.where(Vb, Wb, np.float32(np.inf)).min(axis=2).astype(np.float32)
    mx = np.where(Vb, Wb, np.float32(-np.inf)).max(axis=2).astype(np.float32)
    with np.errstate(over="ignore"):
        rng = (mx - mn).astype(np.float32)
    if not np.all(np.isfinite(rng)):
        raise ValueError("block range overflows f32")
    scale = (rng / np.float32(15.0)).astype(np.float32)
    zero = (mn + np.float32(0.0)).astype(np.float32)   # -0.0 -> +0.0 (signed-zero reading)
    safe = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    t = ((Wb - zero[:, :, None]).astype(np.float32) / safe[:, :, None]).astype(np.float32)
    q = np.clip(np.rint(t), 0, 15).astype(np.uint8)
    q = np.where((scale == 0)[:, :, None] | ~Vb, np.uint8(0), q)
    out = np.empty((rows, nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:4] = scale.astype("<f4").view(np.uint8).reshape(rows, nb, 4)
    out[:, :, 4:8] = zero.astype("<f4").view(np.uint8).reshape(rows, nb, 4)
    out[:, :, 8:] = q[:, :, 0::2] | (q[:, :, 1::2] << 4)
    return out.reshape(-1)


def decode_fields(packed, rows, K):
    """Split packed bytes into (scale f32 [rows,nb], zero f32 [rows,nb], q u8 [rows,nb,256])."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    nb = blocks_per_row(K)
    if packed.size != packed_bytes(rows, K):
        raise ValueError("packed size %d != %d" % (packed.size, packed_bytes(rows, K)))
    blk = packed.reshape(rows, nb, BLOCK_BYTES)
    scale = blk[:, :, 0:4].copy().view("<f4").reshape(rows, nb)
    zero = blk[:, :, 4:8].copy().view("<f4").reshape(rows, nb)
    cb = blk[:, :, 8:]
    q = np.empty((rows, nb, BLOCK), dtype=np.uint8)
    q[:, :, 0::2] = cb & 0x0F
    q[:, :, 1::2] = cb >> 4
    return scale, zero, q


def dequantize(packed, rows, K):
    """w_hat = zero + scale * q per block, in float64 (exact: an f32 times a
    4-bit integer fits in 53 bits).  Returns float64 [rows, K]; padding dropped."""
    scale, zero, q = decode_fields(packed, rows, K)
    w = zero.astype(np.float64)[:, :, None] + scale.astype(np.float64)[:, :, None] * q.astype(np.float64)
    return w.reshape(rows, -1)[:, :K]


def matvec(packed, rows, K, x):
    """y[r] = sum_{i<K} w_hat[r, i] * x[i], float64 accumulation.  x may be
    [K] or [B, K] (then y is [B, rows])."""
    W = dequantize(packed, rows, K)
    x = np.asarray(x, dtype=np.float64)
    return x @ W.T
