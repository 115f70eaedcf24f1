"""CPU oracle for the 8-bit floating-point KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline may import this module.  It shares no code with the HIP library.

The pages name an fp8 KV cache as a serving option that doubles the cache's
capacity and halves the bytes attention reads (zihan-zhang.net vLLM study,
4.2.1: KV cache quantization; the same page's 4.2.3 lists it for long
contexts at high concurrency).  They fix neither the 8-bit format nor how
values are scaled into it.  Readings taken here:

* Format: E4M3 of the OCP 8-bit floating-point specification, the format
  vLLM's ``fp8`` cache type refers to: 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent field 0 holds zero and the subnormals
  (m / 8 * 2^-6); S.1111.111 is NaN; there are no infinities, so the largest
  finite magnitude is 1.75 * 2^8 = 448.
* Scaling: one fp32 scale per pool (``k_scale`` for the K pool, ``v_scale``
  for the V pool).  A code c stands for value(c) * scale.
* Quantization of an incoming value x (bf16): the quotient x / scale is
  taken in fp32 (one correctly rounded division), then mapped to the nearest
  E4M3 value, ties to the even code (mantissa LSB 0).  Magnitudes beyond 448,
  infinities included, saturate to 448 with x's sign; a NaN gives 0x7F with
  x's sign bit.  The sign bit of the code is always x's sign bit, so a
  negative x that rounds to zero gives 0x80.
* Attention over an fp8 pool is the same attention as over a bf16 pool, with
  each K and V element replaced by its dequantized value; queries and
  outputs stay bf16.

Everything is plain NumPy over the 256-entry table of code values.
"""

from __future__ import annotations

import numpy as np

from . import paged_attention
from .paged_attention import BLOCK_SIZE, widen

FP8_MAX = 448.0
NAN_CODE = 0x7F


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code from the format's definition (float64; NaN for
    the two NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# value of every code, index = code
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)

# finite non-negative magnitudes in code order (codes 0x00 .. 0x7E increase)
_MAGS = E4M3_TABLE[:0x7F]


def decode(codes: np.ndarray) -> np.ndarray:
    """float64 value of each code."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_f32(x: np.ndarray) -> np.ndarray:
    """E4M3 code of each float32 value: nearest value, ties to even, saturating
    at 448, NaN -> 0x7F; the sign bit is x's sign bit."""
    x = np.asarray(x, dtype=np.float32)
    sign = ((x.view(np.uint32) >> np.uint32(31)).astype(np.uint8)) << np.uint8(7)
    a = np.abs(x.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, FP8_MAX))
    # neighbours: _MAGS[hi - 1] < a <= _MAGS[hi]
    hi = np.searchsorted(_MAGS, a, side="left")
    hi = np.clip(hi, 0, len(_MAGS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    mag = np.where(nan, np.uint8(NAN_CODE), mag)
    return (mag | sign).astype(np.uint8)


def quantize(raw: np.ndarray, dtype: str, scale) -> np.ndarray:
    """Codes of raw bf16 (or fp32) values under ``scale`` (> 0): x / scale in
    fp32, then ``encode_f32``; a NaN input gives 0x7F with its own sign bit."""
    x = widen(raw, dtype).astype(np.float32)  # exact: the inputs are fp32-representable
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        qt = x / np.float32(scale)
    codes = encode_f32(qt)
    nan = np.isnan(x)
    sign = ((x.view(np.uint32) >> np.uint32(31)).astype(np.uint8)) << np.uint8(7)
    return np.where(nan, np.uint8(NAN_CODE) | sign, codes).astype(np.uint8)


def dequantize(codes: np.ndarray, scale) -> np.ndarray:
    """float64 value each code stands for: value(code) * scale."""
    return decode(codes) * float(np.float32(scale))


# ----------------------------------------------------------------------------
# pools of codes, logical view [num_blocks, 16, Hkv, D] (uint8)


def new_pool(num_blocks: int, num_kv_heads: int, head_dim: int, fill: int) -> np.ndarray:
    return np.full((num_blocks, BLOCK_SIZE, num_kv_heads, head_dim), fill, dtype=np.uint8)


def reshape_and_cache(pool_k, pool_v, k, v, slot_mapping, k_scale, v_scale, dtype="bf16") -> None:
    """Quantize token i's K and V rows and store the codes in its slot (slot
    s >= 0 names block s // 16, offset s % 16; negative slots write nothing)."""
    kc = quantize(k, dtype, k_scale)
    vc = quantize(v, dtype, v_scale)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    s = slots[keep]
    pool_k[s // BLOCK_SIZE, s % BLOCK_SIZE] = kc[keep]
    pool_v[s // BLOCK_SIZE, s % BLOCK_SIZE] = vc[keep]


# ----------------------------------------------------------------------------
# attention over dequantized pools: the same attention as over a bf16 pool
# (the generic decode / prefill of paged_attention, pinned on their own), with
# every gathered K and V code replaced by the value it stands for


def decode_attention(q, pool_k, pool_v, block_tables, context_lens, scale, k_scale, v_scale,
                     q_dtype="bf16", seqs=None):
    """Decode attention (one query per sequence, whole context visible) over
    fp8 pools; float64 [S, Hq, D], zeros for empty contexts."""
    return paged_attention.decode(q, pool_k, pool_v, block_tables, context_lens, scale, q_dtype,
                                  seqs=seqs, k_value=lambda c: dequantize(c, k_scale),
                                  v_value=lambda c: dequantize(c, v_scale))


def prefill_attention(q, pool_k, pool_v, block_tables, query_start_loc, context_lens, scale,
                      k_scale, v_scale, q_dtype="bf16", rows=None):
    """Causal attention of each request's query chunk (its last n_r tokens)
    against its paged fp8 context; float64 [total_q, Hq, D]."""
    return paged_attention.prefill_chunk(q, pool_k, pool_v, block_tables, query_start_loc,
                                         context_lens, scale, q_dtype, rows=rows,
                                         k_value=lambda c: dequantize(c, k_scale),
                                         v_value=lambda c: dequantize(c, v_scale))
