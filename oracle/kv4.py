"""4-bit min/max group quantization of the KV cache (FlexGen), fp64 / exact.

Follows the FlexGen digest (kwkr.cn), section "方法细节": groups of 64 elements,
min and max per group, values quantized to 4-bit integers and dequantized back
to FP16 before compute; the KV cache is grouped along the hidden dimension.

Readings where the page is silent (each is a choice of this library):

* a group is 64 contiguous channels of one token's key (or value) row;
* scale s16 = fp16((max - min) / 15), the exact quotient rounded once to
  binary16 (nearest, ties to even); min is stored as binary16 (exact, since it
  is one of the fp16 inputs);
* code c = clamp(round_half_even((x - min) / s16), 0, 15) against the stored
  s16; when s16 == 0 every code of the group is 0;
* two codes per byte, the even channel in the low nibble;
* dequantized value x_hat = fp16(min + c * s16), rounded once.

Exactness: fp16 values are multiples of 2^-24 below 2^16 in magnitude, so
max - min and min + c * s16 are exact in float64; the float64 quotients are
correctly rounded and (by the size of the numerators and denominators) can
neither land on nor cross a rounding tie unless the exact value is one, so
float64 followed by one rounding equals the exact-rational definition.
"""
from __future__ import annotations

import numpy as np

from .attention import decode_attention

GROUP = 64


def quantize_kv4(x: np.ndarray):
    """x float16 [..., R] with R % 64 == 0.

    Returns (codes uint8 [..., R/2], gmin float16 [..., R/64],
    gscale float16 [..., R/64]).
    """
    assert x.dtype == np.float16 and x.shape[-1] % GROUP == 0
    lead = x.shape[:-1]
    R = x.shape[-1]
    g = x.astype(np.float64).reshape(*lead, R // GROUP, GROUP)
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    s16 = ((mx - mn) / 15.0).astype(np.float16)          # one rounding
    s = s16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.rint((g - mn[..., None]) / s)              # ties to even
    c = np.where(s == 0.0, 0.0, c)
    c = np.clip(c, 0, 15).astype(np.uint8).reshape(*lead, R)
    codes = (c[..., 0::2] | (c[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return codes, mn.astype(np.float16), s16


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """uint8 [..., R/2] -> integer codes [..., R] (even channel = low nibble)."""
    lo = codes & np.uint8(0x0F)
    hi = codes >> np.uint8(4)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequantize_kv4(codes: np.ndarray, gmin: np.ndarray,
                   gscale: np.ndarray) -> np.ndarray:
    """x_hat = fp16(min + c * s16) per element; returns float16 [..., R]."""
    c = unpack_codes(codes).astype(np.float64)
    lead = c.shape[:-1]
    R = c.shape[-1]
    c = c.reshape(*lead, R // GROUP, GROUP)
    xh = gmin.astype(np.float64)[..., None] + c * gscale.astype(np.float64)[..., None]
    return xh.reshape(*lead, R).astype(np.float16)


def kv4_attention(q: np.ndarray, k_codes, k_min, k_scale, v_codes, v_min,
                  v_scale, scale: float) -> np.ndarray:
    """Decode attention over the dequantized (FP16) cache.

    q float64 [B][Hq][D]; codes [B][Hkv][N][D/2]; min/scale [B][Hkv][N][D/64].
    """
    k = dequantize_kv4(k_codes, k_min, k_scale).astype(np.float64)
    v = dequantize_kv4(v_codes, v_min, v_scale).astype(np.float64)
    return decode_attention(q, k, v, scale)
