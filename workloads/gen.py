"""Seeded synthetic decode inputs: lengths, page pool, block table, bf16 bits.

Every array is drawn on the host from ``numpy.random.Generator(PCG64(seed))``
in a fixed order, so the same seed gives the same bits everywhere:

1. the per-sequence cache lengths (when the case draws them),
2. the index of the long sequence (skewed case only), then the permutation of
   the physical page pool,
3. the absorbed queries, float32 N(0, 1),
4. the latent cache pool, float32 N(0, 1), drawn in chunks of 1024 pages.

Queries and cache are rounded once to bfloat16 (round to nearest, ties to
even) and kept as raw uint16 bit patterns.  Logical page ``j`` of sequence
``b`` lives at physical page ``block_table[b, j]``; entries past the last
used page are -1.  The pool either holds exactly the pages needed or 1.25x
that many, with the unused ones left where the permutation puts them.

The latent cache entry of a token is 576 values: the 512-d compressed latent
followed by the 64-d rotary part (FlashMLA release note on shoujike.com.cn,
paragraph on the released paged BF16 cache with block size 64; DeepSeek-V3
hardware paper summary, paragraph on memory efficiency: one latent per token
shared by all heads).

Only input generation lives here; no attention arithmetic.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

HEAD_DIM = 576  # latent (512) + rotary (64), bf16
V_DIM = 512  # the latent part doubles as the value
PAGE = 64  # tokens per cache page
POOL_CHUNK = 1024  # pages drawn per call to the generator

BF16_NAN = np.uint16(0x7FC0)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs are finite draws, so no NaN special case is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def default_scale() -> float:
    """1/sqrt(192) rounded to float32 (returned as the Python float of it)."""
    return float(np.float32(1.0 / math.sqrt(192.0)))


@dataclass
class DecodeCase:
    """One batch of decode inputs, host side, as raw bits and int32 tables."""

    q: np.ndarray  # uint16 [batch, s_q, h_q, 576]
    kv: np.ndarray  # uint16 [num_pages, 64, 576]
    block_table: np.ndarray  # int32 [batch, max_pages]
    cache_seqlens: np.ndarray  # int32 [batch]
    softmax_scale: float
    causal: bool
    info: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def s_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def h_q(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_pages(self) -> int:
        return int(self.kv.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])


def _pages_for(L: int) -> int:
    return (int(L) + PAGE - 1) // PAGE


def make_case(
    seqlens: Sequence[int],
    s_q: int,
    h_q: int,
    causal: bool,
    seed: int,
    pool_factor: float = 1.0,
    softmax_scale: Optional[float] = None,
    max_pages: Optional[int] = None,
    poison_unused: bool = False,
    poison_tail: bool = False,
    rng: Optional[np.random.Generator] = None,
    info: Optional[dict] = None,
) -> DecodeCase:
    """Build a case for given cache lengths.

    ``rng`` continues a generator that already drew the lengths (the named
    workloads do that); otherwise a fresh ``PCG64(seed)`` is used.
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    seqlens = np.asarray(seqlens, dtype=np.int64)
    batch = int(seqlens.shape[0])
    if batch <= 0:
        raise ValueError("batch must be positive")
    if np.any(seqlens < 0):
        raise ValueError("cache lengths must be >= 0")
    n_pages = np.array([_pages_for(L) for L in seqlens], dtype=np.int64)
    needed = int(n_pages.sum())
    num_pages = max(1, int(math.ceil(needed * float(pool_factor))))
    if max_pages is None:
        max_pages = max(1, int(n_pages.max()))
    if max_pages < int(n_pages.max()):
        raise ValueError("max_pages smaller than the longest sequence")

    perm = rng.permutation(num_pages).astype(np.int32)
    block_table = np.full((batch, max_pages), -1, dtype=np.int32)
    k = 0
    for b in range(batch):
        nb = int(n_pages[b])
        block_table[b, :nb] = perm[k : k + nb]
        k += nb

    q = bf16_bits_from_f32(
        rng.standard_normal((batch, s_q, h_q, HEAD_DIM), dtype=np.float32)
    )
    kv = np.empty((num_pages, PAGE, HEAD_DIM), dtype=np.uint16)
    for p0 in range(0, num_pages, POOL_CHUNK):
        p1 = min(num_pages, p0 + POOL_CHUNK)
        kv[p0:p1] = bf16_bits_from_f32(
            rng.standard_normal((p1 - p0, PAGE, HEAD_DIM), dtype=np.float32)
        )

    if poison_unused and num_pages > needed:
        kv[perm[needed:]] = BF16_NAN
    if poison_tail:
        for b in range(batch):
            L = int(seqlens[b])
            if L % PAGE:
                kv[block_table[b, L // PAGE], L % PAGE :, :] = BF16_NAN

    scale = default_scale() if softmax_scale is None else float(np.float32(softmax_scale))
    meta = dict(seed=int(seed), pool_factor=float(pool_factor), needed_pages=needed)
    if info:
        meta.update(info)
    return DecodeCase(
        q=q,
        kv=kv,
        block_table=block_table,
        cache_seqlens=seqlens.astype(np.int32),
        softmax_scale=scale,
        causal=bool(causal),
        info=meta,
    )


@dataclass(frozen=True)
class CaseSpec:
    """A named decode workload: shapes and how its cache lengths are drawn."""

    name: str
    batch: int
    s_q: int
    h_q: int
    lengths: tuple  # ("fixed", L) | ("uniform", lo, hi) | ("skewed", lo, hi, long_len)
    pool_factor: float
    causal: bool

    @property
    def rows(self) -> int:
        return self.s_q * self.h_q


# The five workloads: tiny, memory-bound, compute-bound, two query tokens with
# a causal mask, and skewed long context.  Seed of workload k is 1000 + k.
CONFIGS = {
    1: CaseSpec("tiny", 1, 1, 16, ("fixed", 256), 1.0, False),
    2: CaseSpec("memory_bound", 8, 1, 16, ("uniform", 1024, 4096), 1.25, False),
    3: CaseSpec("compute_bound", 64, 1, 128, ("fixed", 4096), 1.0, False),
    4: CaseSpec("multi_token_causal", 128, 2, 128, ("uniform", 2048, 16384), 1.0, True),
    5: CaseSpec("skewed_long", 16, 1, 64, ("skewed", 1024, 32768, 131072), 1.25, False),
}


def draw_lengths(spec: CaseSpec, rng: np.random.Generator) -> tuple:
    """Draw the cache lengths of a named workload; returns (lengths, info)."""
    kind = spec.lengths[0]
    info = {}
    if kind == "fixed":
        L = np.full(spec.batch, spec.lengths[1], dtype=np.int64)
    elif kind == "uniform":
        lo, hi = spec.lengths[1], spec.lengths[2]
        L = rng.integers(lo, hi, size=spec.batch, endpoint=True).astype(np.int64)
    elif kind == "skewed":
        lo, hi, long_len = spec.lengths[1], spec.lengths[2], spec.lengths[3]
        short = rng.integers(lo, hi, size=spec.batch - 1, endpoint=True).astype(np.int64)
        idx = int(rng.integers(0, spec.batch))
        L = np.insert(short, idx, long_len)
        info["long_index"] = idx
    else:  # pragma: no cover - specs are fixed above
        raise ValueError(kind)
    return L, info


def make_config_case(k: int, poison_unused: bool = False, poison_tail: bool = False,
                     seed: Optional[int] = None) -> DecodeCase:
    """Inputs of named workload ``k`` (1..5) from seed ``1000 + k``."""
    spec = CONFIGS[k]
    seed = 1000 + k if seed is None else int(seed)
    rng = np.random.Generator(np.random.PCG64(seed))
    L, info = draw_lengths(spec, rng)
    info.update(config=k, name=spec.name)
    return make_case(
        L,
        spec.s_q,
        spec.h_q,
        spec.causal,
        seed,
        pool_factor=spec.pool_factor,
        poison_unused=poison_unused,
        poison_tail=poison_tail,
        rng=rng,
        info=info,
    )


# --------------------------------------------------------------------------
# inputs of the absorption products around the decode
# --------------------------------------------------------------------------
NOPE_DIM = 128  # per-head query part before absorption, and value head width
ROPE_DIM = 64


@dataclass
class AbsorbCase:
    """Inputs of the query and output absorption for one batch of query
    tokens, as raw bf16 bits.  ``w_uk`` and ``w_uv`` are the per-head
    up-projections as stored, ``[h, 128, 512]`` (head h's key part is
    ``w_uk[h] @ c``, its value ``w_uv[h] @ c`` for a 512-d latent c);
    ``w_uk_t`` is ``w_uk`` with its last two axes swapped, the layout the
    query absorption reads.  ``lat_out`` stands for a decode output."""
    batch: int
    s_q: int
    h_q: int
    seed: int
    q_nope: np.ndarray   # uint16 [b, s_q, h, 128]
    q_rope: np.ndarray   # uint16 [b, s_q, h, 64]
    w_uk: np.ndarray     # uint16 [h, 128, 512]
    w_uk_t: np.ndarray   # uint16 [h, 512, 128]
    w_uv: np.ndarray     # uint16 [h, 128, 512]
    lat_out: np.ndarray  # uint16 [b, s_q, h, 512]


def make_absorb_case(batch: int, s_q: int, h_q: int, seed: int) -> AbsorbCase:
    """Draw, in this order from PCG64(seed): q_nope and q_rope ~ N(0, 1), the
    weights ~ N(0, 1/512) (so an absorbed query entry has variance 1/4 and an
    output entry variance 1), and the latent output ~ N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    def draw(shape, sd=1.0):
        return bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32) * np.float32(sd))
    q_nope = draw((batch, s_q, h_q, NOPE_DIM))
    q_rope = draw((batch, s_q, h_q, ROPE_DIM))
    w_uk = draw((h_q, NOPE_DIM, V_DIM), 1.0 / math.sqrt(V_DIM))
    w_uv = draw((h_q, NOPE_DIM, V_DIM), 1.0 / math.sqrt(V_DIM))
    lat_out = draw((batch, s_q, h_q, V_DIM))
    w_uk_t = np.ascontiguousarray(w_uk.transpose(0, 2, 1))
    return AbsorbCase(batch, s_q, h_q, seed, q_nope, q_rope, w_uk, w_uk_t, w_uv, lat_out)


# --------------------------------------------------------------------------
# inputs of the paged KV append
# --------------------------------------------------------------------------
@dataclass
class AppendCase:
    """A paged cache, its block table and lengths, a stack of free pages and
    the new cache entries to append, as raw bits.  Pool pages: the held ones,
    then the free ones, then 3 spare pages that nothing references, all at
    positions drawn by one permutation; unused table entries are -1."""
    kv: np.ndarray          # uint16 [num_pages, 64, 576]
    block_table: np.ndarray  # int32 [batch, max_pages]
    seqlens: np.ndarray     # int32 [batch]
    new_kv: np.ndarray      # uint16 [batch, n_new, 576]
    free_pages: np.ndarray  # int32 [free]


def make_append_case(seqlens: Sequence[int], n_new: int, free: int, seed: int,
                     max_pages: Optional[int] = None) -> AppendCase:
    """Draw, in this order from PCG64(seed): the pool permutation, the cache
    pool ~ N(0, 1) and the new entries ~ N(0, 1), rounded to bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    batch = len(seqlens)
    held = [(int(L) + PAGE - 1) // PAGE for L in seqlens]
    if max_pages is None:
        max_pages = max(held + [1]) + (n_new + PAGE - 1) // PAGE + 1
    num_pages = sum(held) + free + 3
    perm = rng.permutation(num_pages).astype(np.int32)
    kv = bf16_bits_from_f32(rng.standard_normal((num_pages, PAGE, HEAD_DIM), dtype=np.float32))
    bt = np.full((batch, max_pages), -1, dtype=np.int32)
    k = 0
    for b, h in enumerate(held):
        bt[b, :h] = perm[k:k + h]
        k += h
    free_pages = perm[k:k + free].copy()
    new_kv = bf16_bits_from_f32(rng.standard_normal((batch, n_new, HEAD_DIM), dtype=np.float32))
    return AppendCase(kv, bt, np.array(seqlens, dtype=np.int32), new_kv, free_pages)


# --------------------------------------------------------------------------
# inputs of MLA prefill (per-head form)
# --------------------------------------------------------------------------
@dataclass
class PrefillCase:
    """Packed prompts: sequence s holds tokens cu_seqlens[s] .. cu_seqlens[s+1]-1.
    Raw bf16 bits throughout."""
    cu_seqlens: np.ndarray  # int32 [batch + 1]
    latent: np.ndarray      # uint16 [T, 576]: the cache entry [c (512) ; r (64)] of each token
    q: np.ndarray           # uint16 [T, H, 192]: [q_nope (128) ; q_rope (64)] per head
    w_uk: np.ndarray        # uint16 [H, 128, 512]: W_UK,h
    w_uv: np.ndarray        # uint16 [H, 128, 512]: W_UV,h
    softmax_scale: float

    @property
    def tokens(self) -> int:
        return int(self.latent.shape[0])

    @property
    def heads(self) -> int:
        return int(self.q.shape[1])


def make_prefill_case(seqlens: Sequence[int], h_q: int, seed: int,
                      softmax_scale: Optional[float] = None) -> PrefillCase:
    """Draw, in this order from PCG64(seed): the latents [c ; r] ~ N(0, 1),
    the queries ~ N(0, 1), W_UK then W_UV ~ N(0, 1/512) (so a widened key
    or value entry has variance about 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seqlens = [int(x) for x in seqlens]
    if any(x < 0 for x in seqlens) or not seqlens:
        raise ValueError("lengths must be non-negative, at least one sequence")
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    T = int(cu[-1])

    def draw(shape, sd=1.0):
        return bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32) * np.float32(sd))

    latent = draw((T, HEAD_DIM))
    q = draw((T, h_q, NOPE_DIM + ROPE_DIM))
    w_uk = draw((h_q, NOPE_DIM, V_DIM), 1.0 / math.sqrt(V_DIM))
    w_uv = draw((h_q, NOPE_DIM, V_DIM), 1.0 / math.sqrt(V_DIM))
    scale = default_scale() if softmax_scale is None else float(np.float32(softmax_scale))
    return PrefillCase(cu, latent, q, w_uk, w_uv, scale)
