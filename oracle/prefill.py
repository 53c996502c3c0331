"""Plain fp64 reference for MLA prefill in per-head form -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the bench may
import or call this.  It shares no code with the HIP library.

What is computed (sources, by page and paragraph):

* FlashMLA release note (shoujike.com.cn), paragraph on the MLA core
  principles: the per-token latent is widened again at compute time.  With a
  whole prompt to attend over, the widened form is the cheaper one: head h's
  key for token t is [W_UK,h c_t ; r_t] (128 values from the 512-value latent
  c_t, then the 64-value rotary key r_t shared by every head) and its value
  W_UV,h c_t (128 values).  DeepSeek-V3 summary, paragraph on memory
  efficiency: the up-projections fold every head's K and V into the latent.
* Same release note, introduction: FlashMLA itself is a decode kernel; the
  DeepSeek-V3 summary, paragraph on inference speed, runs prefill and decode
  as separate stages.  Prefill is causal self-attention over the prompt:
  query t sees tokens 0 .. t of its own sequence.

Readings (the pages give no prefill interface): several prompts are packed one
after another, sequence s holding tokens cu_seqlens[s] .. cu_seqlens[s+1]-1;
the query of token t is [q_nope ; q_rope] (128 + 64 values per head, rotary
embedding already applied); the scale is used as its float32 value; lse is
the natural log of the sum of exp(scaled scores); an empty row cannot occur
with the causal mask (a token always sees itself).

Everything is float64; bf16 inputs are widened exactly by the caller.
"""

from __future__ import annotations

import math
from typing import Sequence

import numpy as np

NOPE = 128
ROPE = 64
QK_DIM = NOPE + ROPE  # 192
V_HEAD = 128


def _scale64(scale: float) -> float:
    return float(np.float64(np.float32(scale)))


def expand_kv(c: np.ndarray, W_UK: np.ndarray, W_UV: np.ndarray):
    """Per-head keys' latent part and values from the latents.

    ``c [T, 512]``, ``W_UK`` and ``W_UV`` ``[H, 128, 512]`` ->
    ``k_nope [T, H, 128]`` with ``k_nope[t, h] = W_UK[h] c_t`` and
    ``v [T, H, 128]`` with ``v[t, h] = W_UV[h] c_t``.
    """
    c = np.asarray(c, dtype=np.float64)
    k_nope = np.einsum("hdk,tk->thd", np.asarray(W_UK, dtype=np.float64), c)
    v = np.einsum("hdk,tk->thd", np.asarray(W_UV, dtype=np.float64), c)
    return k_nope, v


def attention_ref(q: np.ndarray, k_nope: np.ndarray, k_rope: np.ndarray, v: np.ndarray,
                  cu_seqlens: Sequence[int], scale: float, causal: bool = True):
    """Per-head attention over packed prompts.

    ``q [T, H, 192]`` (latent part then rotary part), ``k_nope [T, H, 128]``,
    ``k_rope [T, 64]`` (shared by the heads), ``v [T, H, 128]``.  Head h's
    key of token t is ``[k_nope[t, h] ; k_rope[t]]``.  Within sequence s
    (tokens ``cu_seqlens[s] .. cu_seqlens[s+1] - 1``) query t sees the keys
    of tokens ``cu_seqlens[s] .. t`` (causal) or all of its sequence.
    Returns ``o [T, H, 128]`` and ``lse [T, H]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k_nope = np.asarray(k_nope, dtype=np.float64)
    k_rope = np.asarray(k_rope, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, _ = q.shape
    sc = _scale64(scale)
    o = np.zeros((T, H, V_HEAD))
    lse = np.full((T, H), -np.inf)
    cu = [int(x) for x in cu_seqlens]
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        n = b - a
        if n <= 0:
            continue
        mask = np.triu(np.ones((n, n), dtype=bool), k=1) if causal else np.zeros((n, n), bool)
        for h in range(H):
            K = np.concatenate([k_nope[a:b, h], k_rope[a:b]], axis=1)  # [n, 192]
            S = sc * (q[a:b, h] @ K.T)
            S = np.where(mask, -np.inf, S)
            M = S.max(axis=1)
            ls = M + np.log(np.exp(S - M[:, None]).sum(axis=1))
            P = np.exp(S - ls[:, None])
            o[a:b, h] = P @ v[a:b, h]
            lse[a:b, h] = ls
    return o, lse


def prefill_ref(c: np.ndarray, r: np.ndarray, q: np.ndarray, W_UK: np.ndarray,
                W_UV: np.ndarray, cu_seqlens: Sequence[int], scale: float, causal: bool = True):
    """MLA prefill from the latents: widen them per head (expand_kv), then
    attend (attention_ref).  ``c [T, 512]``, ``r [T, 64]``, ``q [T, H, 192]``."""
    k_nope, v = expand_kv(c, W_UK, W_UV)
    return attention_ref(q, k_nope, r, v, cu_seqlens, scale, causal)


def attention_rows(q: np.ndarray, k_nope: np.ndarray, k_rope: np.ndarray, v: np.ndarray,
                   cu_seqlens: Sequence[int], scale: float, causal: bool, rows):
    """Rows ``(t, h)`` of attention_ref, one by one (for prompts too long for
    the whole reference).  Returns a list of ``(o [128], lse)``."""
    cu = [int(x) for x in cu_seqlens]
    sc = _scale64(scale)
    res = []
    for t, h in rows:
        s = max(i for i in range(len(cu) - 1) if cu[i] <= t)
        a, b = cu[s], cu[s + 1]
        end = t + 1 if causal else b
        K = np.concatenate([np.asarray(k_nope[a:end, h], np.float64),
                            np.asarray(k_rope[a:end], np.float64)], axis=1)
        S = sc * (K @ np.asarray(q[t, h], np.float64))
        M = S.max()
        ls = M + math.log(np.exp(S - M).sum())
        P = np.exp(S - ls)
        res.append((P @ np.asarray(v[a:end, h], np.float64), ls))
    return res


def attention_bruteforce(q, k_nope, k_rope, v, cu_seqlens, scale, causal=True):
    """Scalar loops with exact sums (math.fsum); tiny inputs only.  Builds
    each head's key from its two parts itself and walks positions."""
    T, H, _ = q.shape
    sc = _scale64(scale)
    o = np.zeros((T, H, V_HEAD))
    lse = np.zeros((T, H))
    cu = [int(x) for x in cu_seqlens]
    for s in range(len(cu) - 1):
        for t in range(cu[s], cu[s + 1]):
            last = t if causal else cu[s + 1] - 1
            for h in range(H):
                qv = [float(x) for x in q[t, h]]
                scores = []
                for u in range(cu[s], last + 1):
                    key = [float(x) for x in k_nope[u, h]] + [float(x) for x in k_rope[u]]
                    scores.append(sc * math.fsum(qv[d] * key[d] for d in range(QK_DIM)))
                m = max(scores)
                z = math.fsum(math.exp(x - m) for x in scores)
                ls = m + math.log(z)
                w = [math.exp(x - ls) for x in scores]
                for d in range(V_HEAD):
                    o[t, h, d] = math.fsum(w[i] * float(v[cu[s] + i, h, d]) for i in range(len(w)))
                lse[t, h] = ls
    return o, lse
