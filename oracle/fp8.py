"""fp8 (E4M3) K/V cache rows for the oracle (test infrastructure).

The long-prompt prefill page ("qwen CUDA: long-prompt prefill 5.4x faster",
the Kernels list: F8) keeps the key/value cache as e4m3 rows with one fp32
scale per row and widens them to bf16 before the attention products.  The
pages give no quantisation recipe; the plainest one is taken (and pinned in
tests/test_fp8_pins.py):

* E4M3 as in the OCP 8-bit floating point specification (OFP8, 2023): one
  sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
  subnormal (m/8 * 2^-6); no infinities; S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448.
* Encoding rounds to the nearest code, ties to the code with an even
  mantissa, and saturates finite values beyond 448 to +-448.
* A row (one key or value of one KV head, 256 values) is scaled by
  ``scale = amax / 448`` (fp32 division; 1 for an all-zero row), each value
  encoded from ``x / scale`` (fp32 division), and widened back as
  ``bf16(decode(code) * scale)`` (fp32 product, rounded to bf16 once).

Everything here is plain numpy on the definitions above; nothing is shared
with the HIP library.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each code (uint8 array) as float32; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    val = sign * mag
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return val.astype(np.float32)


# All finite non-negative codes in increasing order of value (0x00 .. 0x7E).
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3_decode(_POS_CODES).astype(np.float64)


def e4m3_encode(x) -> np.ndarray:
    """Nearest code to each float32 value, ties to the even mantissa,
    finite values beyond 448 saturated to +-448, NaN to 0x7F."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")          # first value >= a
    hi = np.minimum(hi, _POS_VALUES.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    exact = d_hi == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(exact | pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def quantize_rows(x) -> tuple:
    """Rows of float32 values [..., n] -> (codes uint8 [..., n], scales float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0))
    scale = scale.astype(np.float32)
    q = (x / scale[..., None]).astype(np.float32)
    return e4m3_encode(q), scale


def dequantize_rows_bf16(codes, scales) -> np.ndarray:
    """bf16 bits of decode(code) * scale (fp32 product, rounded to bf16 once)."""
    import synth
    v = (e4m3_decode(codes) * np.asarray(scales, dtype=np.float32)[..., None]).astype(np.float32)
    return synth.f32_to_bf16_bits(v)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def fp8_cache_kv(orc, p):
    """The keys and values a fp8 cache holds for problem p, as the attention
    sees them: prepared keys [Hkv][T][D] and values [T][Hkv][D] (bf16 bits),
    each row quantised and widened; plus the codes and scales themselves
    (k_codes [Hkv][T][D], k_scales [Hkv][T], v_codes [Hkv][T][D], v_scales [Hkv][T])."""
    kp = orc.prepare_keys(p)                                   # [Hkv][T][D]
    kc, ks = quantize_rows(bf16_bits_to_f32(kp))
    vh = np.ascontiguousarray(np.transpose(p.v, (1, 0, 2)))    # [Hkv][T][D]
    vc, vs = quantize_rows(bf16_bits_to_f32(vh))
    k_eff = dequantize_rows_bf16(kc, ks)
    v_eff = np.ascontiguousarray(np.transpose(dequantize_rows_bf16(vc, vs), (1, 0, 2)))
    return dict(kp=k_eff, v=v_eff, k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs)


def attention_fp8(orc, p, rows=None, threads: int = 1):
    """Gated outputs of p over a fp8 K/V cache (keys and values widened as above)."""
    import dataclasses
    kv = fp8_cache_kv(orc, p)
    q = dataclasses.replace(p, v=kv["v"])
    return orc.attention(q, rows=rows, kp=kv["kp"], threads=threads)
