"""Small helpers for tests: cases built from explicit values."""

import numpy as np

from workloads import DecodeCase, bf16_bits_from_f32


def exact_bf16_bits(x) -> np.ndarray:
    """bf16 bits of values that bf16 holds exactly (asserts they do)."""
    x = np.asarray(x, dtype=np.float32)
    bits = bf16_bits_from_f32(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, x), "value not exactly representable in bf16"
    return bits


def case_from_values(q, kv, block_table, seqlens, scale, causal) -> DecodeCase:
    return DecodeCase(
        q=exact_bf16_bits(q),
        kv=exact_bf16_bits(kv),
        block_table=np.asarray(block_table, dtype=np.int32),
        cache_seqlens=np.asarray(seqlens, dtype=np.int32),
        softmax_scale=float(np.float32(scale)),
        causal=bool(causal),
    )


def permute_pool(case: DecodeCase, seed: int) -> DecodeCase:
    """Move every physical page to a new random place; rewrite the table."""
    rng = np.random.Generator(np.random.PCG64(seed))
    P = case.kv.shape[0]
    new_of_old = rng.permutation(P)
    kv = np.empty_like(case.kv)
    kv[new_of_old] = case.kv
    bt = case.block_table.copy()
    used = bt >= 0
    bt[used] = new_of_old[bt[used]]
    return DecodeCase(q=case.q.copy(), kv=kv, block_table=bt,
                      cache_seqlens=case.cache_seqlens.copy(),
                      softmax_scale=case.softmax_scale, causal=case.causal,
                      info=dict(case.info))


def read_golden(path):
    vals = {}
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if len(parts) == 2:
                vals[parts[0]] = float(parts[1])
            else:
                rows.append(parts)
    return vals, rows
