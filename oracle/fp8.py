"""Oracle: an 8-bit floating-point (e4m3) paged KV cache (TEST INFRASTRUCTURE ONLY).

The pages do not describe a quantised cache.  They put the cost of decoding in
the memory bandwidth it needs [profile; abstract], and the attention's traffic
is the KV cache, which halving the bytes of every cached value attacks.
Everything below is therefore a stated reading, not a statement of the pages.

Format: the OCP 8-bit floating point format E4M3 (the "OFP8" specification's
E4M3, called float8_e4m3fn by PyTorch).  One sign bit, four exponent bits with
bias 7 and three mantissa bits:
  * exponent field e = 1..15: (-1)^s * (1 + m/8) * 2^(e-7);
  * e = 0 (subnormal): (-1)^s * (m/8) * 2^-6;
  * S.1111.111 is NaN; there is no infinity; the largest magnitude is 448.

Quantisation of a bf16 value x of KV head h with that head's fp32 scale s_h
(one scale for K and one for V per head and layer):
  code = round_e4m3(fp32(x) / s_h)
where the division is IEEE fp32 (rounded to nearest even; a quotient beyond
the fp32 range is an infinity) and round_e4m3 takes the nearest e4m3 value,
ties to the even code, and maps magnitudes beyond 448 to 448 (saturating; the
sign of a zero result is kept).  The value the
attention sees is decode(code) * s_h.

Which K/V are quantised: every key and value the attention reads, the cached
ones and the block's own rows alike.  Greedy decoding with such a cache writes a
token's K/V and reads them back from the cache, so the verify pass must see the
block's keys exactly as the cache will hold them for its tokens to equal greedy
decoding's [gist §2.3 step 3; HN #21, identical output distribution].  The
commit then copies the quantised rows unchanged.

Pinned by (tests/test_oracle_fp8.py): the closed-form values of the format's
landmark codes; PyTorch's float8_e4m3fn decoding of all 256 codes and its
rounding of in-range values (a library routine); exact round trips of every
finite code; the ties-to-even rule at every midpoint between neighbouring
codes; saturation; the direction of the scale (power-of-two scales reduce to
exact shifts); and, for attention, the identities a per-head K scale equals a
per-head change of the score scale and a per-head V scale multiplies that
head's output, plus constant-V and brute-force pure-Python decoding.
"""
from __future__ import annotations

import numpy as np

from .attention import block_attention, from_bf16

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """uint8 e4m3 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# every non-negative finite value with its code, in increasing order
_POS_CODES = np.arange(0x7F, dtype=np.uint8)            # 0x00 .. 0x7E
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(x) -> np.ndarray:
    """Floats -> nearest e4m3 codes (ties to the even code, magnitudes beyond
    448, infinities included, saturating to +-448, the sign of zero kept)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("e4m3_encode: NaN has no saturating code")
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")         # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    neg = np.signbit(x)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def quantize_kv(x_bits, scale, head_axis: int = -2) -> np.ndarray:
    """bf16 bit patterns -> e4m3 codes, divided by the per-KV-head fp32 scale
    (scale[h] applies along head_axis) in fp32 arithmetic."""
    x32 = from_bf16(x_bits).astype(np.float32)
    s = _along(np.asarray(scale, dtype=np.float32), x32.ndim, head_axis)
    with np.errstate(over="ignore"):
        q = (x32 / s).astype(np.float32)
    return e4m3_encode(q)


def dequantize_kv(codes, scale, head_axis: int = -2) -> np.ndarray:
    """e4m3 codes -> float64 values decode(code) * scale[h]."""
    v = e4m3_decode(codes)
    s = _along(np.asarray(scale, dtype=np.float32).astype(np.float64), v.ndim, head_axis)
    return v * s


def _along(s: np.ndarray, ndim: int, axis: int) -> np.ndarray:
    shape = [1] * ndim
    shape[axis] = s.shape[0]
    return s.reshape(shape)


def block_attention_fp8(q_bits, k_blk, v_blk, k_pages, v_pages, k_scale, v_scale,
                        block_table, seq_lens, mode: str, scale: float | None = None,
                        page_size: int = 16) -> np.ndarray:
    """Attention [B, K, Hq, D] (fp64) over an e4m3 cache.

    q_bits: bf16 [B,K,Hq,D]; k_blk, v_blk: e4m3 codes [B,K,Hkv,D] (the block's
    own rows, quantised like the cache); k_pages, v_pages: e4m3 codes
    [num_pages,Hkv,page_size,D]; k_scale, v_scale: fp32 [Hkv].  The keys and
    values are dequantised and the attention is the bf16 cache's
    (oracle.attention.block_attention) on those values."""
    return block_attention(from_bf16(q_bits),
                           dequantize_kv(k_blk, k_scale, head_axis=2),
                           dequantize_kv(v_blk, v_scale, head_axis=2),
                           dequantize_kv(k_pages, k_scale, head_axis=1),
                           dequantize_kv(v_pages, v_scale, head_axis=1),
                           block_table, seq_lens, mode, scale=scale, page_size=page_size)
