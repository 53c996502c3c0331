"""Plain reference for the FP8 latent cache -- TEST INFRASTRUCTURE ONLY.

Only the test suite and the bench's CPU leg may import this module; the HIP
library shares no code with it.

The pages use FP8 for matrix products, training and communication
(DeepSeek-V3 hardware paper summary, section on FP8 mixed precision), not
for the attention cache; storing the latent cache in FP8 is this library's
own extension.  Format, per token (656 bytes):

  [0, 512)    the 512 latent values as OCP FP8 E4M3 codes (1 sign, 4 exponent
              bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is
              NaN; largest finite magnitude 448, smallest normal 2^-6,
              smallest subnormal 2^-9),
  [512, 528)  four float32 scales, one per block of 128 latent values, each an
              exact power of two 2^e,
  [528, 656)  the 64 rotary values, bf16, unchanged.

A block's exponent e is the smallest integer with max|x| <= 448 * 2^e (0 for
an all-zero block); each value is stored as the E4M3 code nearest to
x * 2^-e, ties to the even code (last mantissa bit 0), the sign bit taken from
x.  Dequantized, a value is decode(code) * 2^e: with at most four significant
bits it is exactly a bf16 value (for blocks whose scale keeps it in bf16's
normal range, checked), so the latent decode over an FP8 cache equals the
decode over the bf16 cache of the dequantized values.
"""

from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 576
V_DIM = 512
PAGE = 64
BLOCK = 128
TOKEN_BYTES = 656
E4M3_MAX = 448.0


def _e4m3_table() -> np.ndarray:
    """float64 value of each of the 256 E4M3 codes, from the format's fields."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            vals[code] = np.nan
        elif exp == 0:
            vals[code] = sign * man * 2.0 ** -9            # subnormal: 0.mmm * 2^(1-7)
        else:
            vals[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return vals


E4M3_VALUES = _e4m3_table()
# the 127 finite non-negative magnitudes, indexed by the code's low 7 bits
_MAGS = E4M3_VALUES[:127]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to each value (ties to the even code), sign bit
    from the value's sign; magnitudes above 448 saturate to 448."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.searchsorted(_MAGS, a, side="left")      # first magnitude >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    mag = np.where(a == _MAGS[hi], hi, mag).astype(np.uint8)  # exact hits
    sign = np.signbit(y).astype(np.uint8) << np.uint8(7)
    return (mag | sign).astype(np.uint8)


def block_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e (0 for amax = 0)."""
    if amax == 0.0:
        return 0
    f, k = math.frexp(amax)              # amax = f * 2^k, f in [0.5, 1)
    e = (k - 1) - 8                      # 448 * 2^(k - 9) = 1.75 * 2^(k - 1)
    if 2.0 * f > 1.75:
        e += 1
    return e


def _bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def quantize_token(x_bits: np.ndarray) -> np.ndarray:
    """One 576-value bf16 cache entry -> its 656-byte FP8 record."""
    x = _bf16_bits_to_f64(x_bits)
    rec = np.zeros(TOKEN_BYTES, dtype=np.uint8)
    scales = np.zeros(V_DIM // BLOCK, dtype=np.float32)
    for blk in range(V_DIM // BLOCK):
        xs = x[BLOCK * blk:BLOCK * (blk + 1)]
        e = block_exponent(float(np.max(np.abs(xs))))
        rec[BLOCK * blk:BLOCK * (blk + 1)] = e4m3_encode(xs * 2.0 ** (-e))
        scales[blk] = np.float32(2.0 ** e)
    rec[V_DIM:V_DIM + 16] = scales.view(np.uint8)
    rec[V_DIM + 16:] = np.asarray(x_bits[V_DIM:], dtype=np.uint16).view(np.uint8)
    return rec


def quantize_cache(kv_bits: np.ndarray) -> np.ndarray:
    """bf16 cache [pages, 64, 576] -> FP8 cache [pages, 64, 656] (uint8)."""
    kv_bits = np.asarray(kv_bits, dtype=np.uint16)
    P = kv_bits.shape[0]
    out = np.empty((P, PAGE, TOKEN_BYTES), dtype=np.uint8)
    for p in range(P):
        for t in range(PAGE):
            out[p, t] = quantize_token(kv_bits[p, t])
    return out


def dequantize_cache_f64(kv8: np.ndarray) -> np.ndarray:
    """FP8 cache [pages, 64, 656] -> float64 values [pages, 64, 576]."""
    kv8 = np.asarray(kv8, dtype=np.uint8)
    codes = kv8[..., :V_DIM]
    scales = np.ascontiguousarray(kv8[..., V_DIM:V_DIM + 16]).view(np.float32).astype(np.float64)
    lat = e4m3_decode(codes) * np.repeat(scales, BLOCK, axis=-1)
    rope = _bf16_bits_to_f64(np.ascontiguousarray(kv8[..., V_DIM + 16:]).view(np.uint16))
    return np.concatenate([lat, rope], axis=-1)


def dequantize_cache_bf16_bits(kv8: np.ndarray) -> np.ndarray:
    """The dequantized cache as bf16 bit patterns (exact; raises if a value
    is not a bf16 value, i.e. a block's scale left bf16's range)."""
    v = dequantize_cache_f64(kv8)
    f32 = v.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), v, equal_nan=True):
        raise ValueError("dequantized value not exact in float32")
    u = f32.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("dequantized value not exact in bf16")
    return (u >> np.uint32(16)).astype(np.uint16)
