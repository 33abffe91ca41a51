"""Plain model of a KV cache stored in 8-bit floating point.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[KVB] ("How KV-cache memory limits concurrency") and [DCP] (decode-bottleneck
section) count the bytes of a cached token with the element size as a factor and
list FP8 at one byte; [DCP] (the passage that sets DCP beside KV-cache
quantisation) describes quantisation as storing the cache in a low-precision type
such as FP8 so each token takes fewer bytes.  The pages fix neither the 8-bit
format nor how values are scaled into it.  Readings taken here:

* format: FP8 E4M3 as in the OCP 8-bit floating point specification -- 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
  subnormals m/8 * 2^-6; sign.1111.111 is NaN; there are no infinities, the
  largest finite magnitude is 448;
* scaling: a stored code is E4M3(x / s) and reads back as value(code) * s, with ``s``
  a float32 per tensor or per KV head, one set for keys and one for values (a
  latent cache has keys only);
* rounding: x / s is formed in float32 (IEEE division), then rounded to the nearest
  E4M3 value, ties to the code with an even last bit; magnitudes above 448 and
  infinities saturate to +-448; NaN stays NaN with its sign.

A step reads the cache by dequantising every stored element (value(code) * s, in
float64) and then runs the ordinary attention of ``paged_attention`` on those
values.
"""
from __future__ import annotations

import numpy as np

from . import paged_attention as pa

NAN_CODE = 0x7F          # sign.1111.111 (the sign bit is kept)
MAX_CODE = 0x7E          # 0.1111.110 = 448


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code, from the field definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3 = np.array([e4m3_value(c) for c in range(256)])
_POS = E4M3[:MAX_CODE + 1]        # codes 0 .. 0x7E, values ascending from 0 to 448


def to_f32(x) -> np.ndarray:
    """Input rows (bf16 bit patterns as uint16, or float32) as float32, exactly."""
    return pa.widen(x).astype(np.float32)


def quantize(x, scale) -> np.ndarray:
    """E4M3 codes (uint8) of ``x / scale`` under the readings above.  ``scale`` is a
    float32 scalar or an array that broadcasts against ``x``."""
    y = to_f32(x) / np.asarray(scale, dtype=np.float32)           # float32 division
    y = np.asarray(y, dtype=np.float32)
    sign = np.signbit(y)
    a = np.abs(y).astype(np.float64)                                # exact
    hi = np.searchsorted(_POS, a, side="left").clip(0, MAX_CODE)    # first value >= a
    lo = (hi - 1).clip(0, MAX_CODE)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    code = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), code)
    code = np.where(a >= 448.0, MAX_CODE, code)                      # saturate (and +-inf)
    code = np.where(np.isnan(y), NAN_CODE, code)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def dequantize(codes, scale) -> np.ndarray:
    """float64 values ``value(code) * scale`` (``scale`` broadcasts against ``codes``)."""
    return E4M3[np.asarray(codes, dtype=np.uint8)] * np.asarray(scale, dtype=np.float64)


def head_scales(scales, n_kv_heads: int) -> np.ndarray:
    """float32 [n_kv_heads]: one scale for every head (per tensor) or one each."""
    s = np.asarray(scales, dtype=np.float32).reshape(-1)
    if s.size == 1:
        return np.repeat(s, n_kv_heads)
    if s.size != n_kv_heads:
        raise ValueError("need 1 or n_kv_heads scales")
    return s


def kv_append(k_cache, v_cache, k_new, v_new, slots, block_size: int, k_scale, v_scale):
    """Quantise each new token's key (and value) row with its head's scale and store
    the codes in its slot ([KVB], "What does the KV cache hold?": a step stores the
    new key and value before attending).  Returns new code arrays; a negative slot
    is padding."""
    hkv = k_cache.shape[1]
    ks = head_scales(k_scale, hkv)
    vs = None if v_cache is None else head_scales(v_scale, hkv)
    k_out = k_cache.copy()
    v_out = None if v_cache is None else v_cache.copy()
    for n, slot in enumerate(np.asarray(slots)):
        if slot < 0:
            continue
        blk, off = int(slot) // block_size, int(slot) % block_size
        for h in range(hkv):
            k_out[blk, h, off, :] = quantize(k_new[n, h], ks[h])
            if v_out is not None:
                v_out[blk, h, :, off] = quantize(v_new[n, h], vs[h])
    return k_out, v_out


def dequantize_cache(k_cache, v_cache, k_scale, v_scale):
    """float64 caches of the same layout: every code times its head's scale."""
    hkv = k_cache.shape[1]
    kd = dequantize(k_cache, head_scales(k_scale, hkv)[None, :, None, None])
    vd = None if v_cache is None else dequantize(v_cache, head_scales(v_scale, hkv)[None, :, None, None])
    return kd, vd


def decode_step(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                n_shards: int, interleave: int, block_size: int, partition_tokens: int,
                max_partitions_: int, scale: float, dv: int):
    """The step on an E4M3 cache: route, quantise-and-append, then attend over the
    dequantised cache exactly as ``paged_attention.decode`` does.  Returns the same
    dict as ``paged_attention.decode_step`` (caches as codes)."""
    slots = pa.slot_mapping(block_table, context_lens, n_shards, interleave, block_size)
    kc, vc = kv_append(k_cache, v_cache, k_new, v_new, slots, block_size, k_scale, v_scale)
    kd, vd = dequantize_cache(kc, vc, k_scale, v_scale)
    o, lse, part_o, part_lse = pa.decode(q, kd, vd, block_table, context_lens, n_shards,
                                         interleave, block_size, partition_tokens,
                                         max_partitions_, scale, dv)
    return dict(slots=slots, k_cache=kc, v_cache=vc, o=o, lse=lse, part_o=part_o,
                part_lse=part_lse)
