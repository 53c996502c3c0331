"""Pins of the FP8 latent-cache oracle (CPU): the E4M3 format's published
facts, encoding by nearest value with ties to even, the minimal block
exponent by brute force, the quantization error bound, exactness of the
dequantized values in bf16, and a hand-worked block."""

import os

import numpy as np

import oracle
from workloads import bf16_bits_from_f32

F = oracle.fp8_cache
HERE = os.path.dirname(os.path.abspath(__file__))


def test_e4m3_format_facts():
    v = F.E4M3_VALUES
    assert v[0x38] == 1.0
    assert v[0x7E] == 448.0                       # largest finite
    assert v[0x08] == 2.0 ** -6                   # smallest normal
    assert v[0x01] == 2.0 ** -9                   # smallest subnormal
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    nan = np.isnan(v)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(v[0x80:][~nan[0x80:]], -v[:0x80][~nan[:0x80]])
    assert np.all(np.diff(v[:0x7F]) > 0)          # magnitudes strictly increase
    # a normal code is (1 + m/8) 2^(e - 7): spot values
    assert v[0x3C] == 1.5 and v[0x7C] == 384.0 and v[0x55] == 13.0


def test_encode_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_encode_ties_to_even_and_nearest():
    mags = F.E4M3_VALUES[:127]
    mid = (mags[:-1] + mags[1:]) / 2
    got = F.e4m3_encode(mid)
    lo = np.arange(126)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))
    # just off the midpoint goes to the nearer neighbour
    eps = (mags[1:] - mags[:-1]) / 64
    assert np.array_equal(F.e4m3_encode(mid - eps), lo.astype(np.uint8))
    assert np.array_equal(F.e4m3_encode(mid + eps), (lo + 1).astype(np.uint8))
    assert F.e4m3_encode(np.array([1.0625]))[0] == 0x38   # 1 and 1.125: even is 1
    assert F.e4m3_encode(np.array([1.1875]))[0] == 0x3A   # 1.125 and 1.25: even is 1.25


def test_encode_sign_and_saturation():
    assert F.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert F.e4m3_encode(np.array([-(2.0 ** -11)]))[0] == 0x80  # rounds to -0
    assert F.e4m3_encode(np.array([500.0]))[0] == 0x7E
    assert F.e4m3_encode(np.array([-1e9]))[0] == 0xFE


def test_block_exponent_is_minimal():
    rng = np.random.Generator(np.random.PCG64(5))
    a = np.abs(rng.standard_normal(2000) * 10.0 ** rng.uniform(-6, 6, 2000)).astype(np.float32)
    a = oracle.bf16_to_f64(bf16_bits_from_f32(a))
    for x in list(a) + [448.0, 3.5, 1.75, 2.0 ** -100, 1e30]:
        e = F.block_exponent(float(x))
        assert x <= 448.0 * 2.0 ** e and x > 448.0 * 2.0 ** (e - 1), (x, e)
    assert F.block_exponent(0.0) == 0


def _random_tokens(n, seed, spread=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((n, 576)).astype(np.float32)
    if spread:  # blocks with very different magnitudes
        x *= (10.0 ** rng.uniform(-3, 3, (n, 1))).astype(np.float32)
    return bf16_bits_from_f32(x)


def test_quantize_error_bound_exact_bf16_and_layout():
    bits = _random_tokens(64, 6)
    kv8 = F.quantize_cache(bits.reshape(1, 64, 576))
    assert kv8.shape == (1, 64, 656) and kv8.dtype == np.uint8
    x = oracle.bf16_to_f64(bits)
    deq = F.dequantize_cache_f64(kv8)[0]
    scales = np.ascontiguousarray(kv8[0, :, 512:528]).view(np.float32).astype(np.float64)
    # scales are powers of two and minimal for their block
    m, _ = np.frexp(scales)
    assert np.all(m == 0.5)
    amax = np.abs(x[:, :512]).reshape(64, 4, 128).max(-1)
    assert np.all(amax <= 448 * scales) and np.all(amax > 224 * scales)
    # half a unit of the last place of E4M3 (2^-4 relative), or half the
    # subnormal step (2^-10 of the scale)
    err = np.abs(deq[:, :512] - x[:, :512])
    bound = 2.0 ** -4 * np.abs(x[:, :512]) + 2.0 ** -10 * np.repeat(scales, 128, axis=1)
    assert np.all(err <= bound)
    # rotary part untouched, dequantized values exact in bf16
    assert np.array_equal(deq[:, 512:], x[:, 512:])
    d16 = F.dequantize_cache_bf16_bits(kv8)
    assert np.array_equal(oracle.bf16_to_f64(d16), F.dequantize_cache_f64(kv8))


def test_golden_block_example():
    """A block worked by hand (tests/golden/fp8_block_example.txt)."""
    bits = np.zeros(576, dtype=np.uint16)
    want = {}
    scale = None
    with open(os.path.join(HERE, "golden", "fp8_block_example.txt")) as f:
        for line in f:
            tok = line.split()
            if not tok or tok[0].startswith("#"):
                continue
            if tok[0] == "scale_bytes":
                scale = bytes(int(t, 16) for t in tok[1:])
            elif tok[0] == "value":
                i = int(tok[1])
                bits[i] = int(tok[2], 16)
                want[i] = int(tok[3], 16)
    rec = F.quantize_token(bits)
    assert bytes(rec[512:516]) == scale
    for i, code in want.items():
        assert rec[i] == code, (i, hex(rec[i]), hex(code))
    assert np.all(rec[5:128] == 0)
