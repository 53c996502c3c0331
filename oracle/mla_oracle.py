"""Plain, slow fp64 reference for MLA decode over a paged latent cache.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
bench's CPU-baseline leg, never by the product path.  It shares no code with
the HIP library; both sides take their inputs from the ``workloads`` package.

What is computed (sources, by page and paragraph):

* FlashMLA release note (shoujike.com.cn), paragraph on the MLA core
  principles: keys and values are held as one compressed low-dimensional
  latent per token and widened again at compute time.  DeepSeek-V3 hardware
  paper summary (news.chathome.org), paragraph on memory efficiency: the
  projection matrices fold the KV of every head into that one latent.  So one
  576-value cache entry per token serves as the key of every query head, and
  its first 512 values serve as the value.  Queries arrive already absorbed
  into the 576-d latent space.
* Same release note, paragraph on what was released: the cache is paged,
  bf16, 64 tokens per block; Tom's Hardware FR article, paragraph on the
  techniques: block-based paging allocated on demand.  Logical page j of a
  sequence is found through its block-table row.
* Same release note, paragraphs on variable-length optimisation and dynamic
  sequence processing: each sequence has its own cache length.
* Same release note, acknowledgements paragraph: the design follows
  FlashAttention, i.e. exact softmax attention; the tiling and online
  softmax only reorder the same sum, so the reference is the plain definition.

Readings where the pages say nothing (each one also listed in the design
notes): the log-sum-exp is the natural log of the sum of exp(scaled scores);
it is laid out [batch, s_q, h_q]; with several query tokens and a causal mask
the queries are the last s_q positions of the cache (query i sees keys
t <= L - s_q + i); an empty row gives out = 0 and lse = -inf; rotary
embedding is already applied upstream; the scale is used as its float32
value.

Everything is float64.  bf16 inputs are widened exactly (bf16 -> f32 is a
shift, f32 -> f64 is exact).
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

HEAD_DIM = 576
V_DIM = 512
PAGE = 64


# --------------------------------------------------------------------------
# exact widening of inputs
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64, exactly."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _scale64(softmax_scale: float) -> float:
    """The scale as used by the kernels: its float32 value, widened."""
    return float(np.float64(np.float32(softmax_scale)))


# --------------------------------------------------------------------------
# which cached tokens a query row sees
# --------------------------------------------------------------------------
def visible_tokens(L: int, s_q: int, i: int, causal: bool) -> int:
    """Number of cached tokens query token ``i`` of ``s_q`` attends to.

    Non-causal: all ``L``.  Causal: the query tokens are the last ``s_q``
    cache positions, so query ``i`` sits at position ``L - s_q + i`` and sees
    positions ``0 .. L - s_q + i``.  Clamped to ``[0, L]``.
    """
    n = (L - s_q + 1 + i) if causal else L
    return max(0, min(int(L), int(n)))


# --------------------------------------------------------------------------
# paging: logical token t of sequence b -> physical page/slot
# --------------------------------------------------------------------------
def gather_latents(kv_bits: np.ndarray, block_row: np.ndarray, L: int) -> np.ndarray:
    """The first ``L`` cached latents of one sequence, in logical order, fp64.

    Token ``t`` is at physical page ``block_row[t // 64]``, slot ``t % 64``.
    Returns an ``[L, 576]`` float64 array.
    """
    L = int(L)
    if L == 0:
        return np.zeros((0, HEAD_DIM), dtype=np.float64)
    n_pages = (L + PAGE - 1) // PAGE
    pages = np.asarray(block_row[:n_pages], dtype=np.int64)
    if np.any(pages < 0):
        raise ValueError("block table entry < 0 inside the used range")
    lat = kv_bits[pages].reshape(n_pages * PAGE, HEAD_DIM)[:L]
    return bf16_to_f64(lat)


# --------------------------------------------------------------------------
# the attention definition, on fp64 arrays
# --------------------------------------------------------------------------
def attend_f64(Q: np.ndarray, K: np.ndarray, n_rows: Sequence[int], scale: float,
               return_p: bool = False):
    """Softmax attention of rows ``Q`` over latents ``K`` (both fp64).

    Row ``r`` attends to the first ``n_rows[r]`` rows of ``K``.  Scores are
    ``scale * Q K^T``; values are ``K[:, :512]``.  Returns ``(out [R,512],
    lse [R])`` and, if asked, the weights ``P [R, len(K)]`` (zero where masked).
    The log-sum-exp is max-shifted; an empty row gives out 0 and lse -inf.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    R = Q.shape[0]
    T = K.shape[0]
    n_rows = np.asarray(n_rows, dtype=np.int64)
    S = scale * (Q @ K.T) if T else np.zeros((R, 0))
    mask = np.arange(T)[None, :] >= n_rows[:, None]
    S = np.where(mask, -np.inf, S)
    out = np.zeros((R, V_DIM), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    P = np.zeros((R, T), dtype=np.float64)
    live = n_rows > 0
    if np.any(live):
        Sl = S[live]
        M = Sl.max(axis=1)
        Z = np.exp(Sl - M[:, None]).sum(axis=1)
        lse_l = M + np.log(Z)
        Pl = np.exp(Sl - lse_l[:, None])
        P[live] = Pl
        lse[live] = lse_l
        out[live] = Pl @ K[:, :V_DIM]
    if return_p:
        return out, lse, P
    return out, lse


def _case_arrays(case):
    return (case.q, case.kv, case.block_table, case.cache_seqlens,
            case.softmax_scale, case.causal)


def decode_ref(case, batches: Optional[Iterable[int]] = None):
    """Reference decode of a whole case (or of the listed batches).

    Returns ``out [batch, s_q, h_q, 512]`` and ``lse [batch, s_q, h_q]`` in
    float64.  Rows of batches not listed are left NaN.
    """
    q_bits, kv_bits, bt, seqlens, scale, causal = _case_arrays(case)
    B, s_q, h_q, _ = q_bits.shape
    sc = _scale64(scale)
    out = np.full((B, s_q, h_q, V_DIM), np.nan)
    lse = np.full((B, s_q, h_q), np.nan)
    todo = range(B) if batches is None else batches
    for b in todo:
        L = int(seqlens[b])
        K = gather_latents(kv_bits, bt[b], L)
        Q = bf16_to_f64(q_bits[b]).reshape(s_q * h_q, HEAD_DIM)
        n_rows = [visible_tokens(L, s_q, r // h_q, causal) for r in range(s_q * h_q)]
        o, l = attend_f64(Q, K, n_rows, sc)
        out[b] = o.reshape(s_q, h_q, V_DIM)
        lse[b] = l.reshape(s_q, h_q)
    return out, lse


def decode_ref_rows(case, rows: Iterable[tuple]):
    """Reference output of single rows ``(b, i, h)``, one by one.

    For full-size workloads where the whole reference is too slow.  Returns a
    list of ``(out [512], lse)`` pairs in the order given.
    """
    q_bits, kv_bits, bt, seqlens, scale, causal = _case_arrays(case)
    s_q = q_bits.shape[1]
    sc = _scale64(scale)
    res = []
    cache = {}
    for (b, i, h) in rows:
        L = int(seqlens[b])
        if b not in cache:
            cache.clear()
            cache[b] = gather_latents(kv_bits, bt[b], L)
        K = cache[b]
        Q = bf16_to_f64(q_bits[b, i, h])[None, :]
        o, l = attend_f64(Q, K, [visible_tokens(L, s_q, i, causal)], sc)
        res.append((o[0], float(l[0])))
    return res


def softmax_weights(case, b: int) -> np.ndarray:
    """The attention weights of batch ``b``: ``[s_q*h_q, L]`` float64."""
    q_bits, kv_bits, bt, seqlens, scale, causal = _case_arrays(case)
    _, s_q, h_q, _ = q_bits.shape
    L = int(seqlens[b])
    K = gather_latents(kv_bits, bt[b], L)
    Q = bf16_to_f64(q_bits[b]).reshape(s_q * h_q, HEAD_DIM)
    n_rows = [visible_tokens(L, s_q, r // h_q, causal) for r in range(s_q * h_q)]
    return attend_f64(Q, K, n_rows, _scale64(scale), return_p=True)[2]


# --------------------------------------------------------------------------
# scalar brute force (tiny inputs only): its own loops, positions and sums
# --------------------------------------------------------------------------
def decode_bruteforce(case):
    """Scalar triple loops with exact summation (``math.fsum``).

    Written independently of ``attend_f64``: it walks positions explicitly,
    looks each token up through the block table itself, and masks by
    position.  Only for tiny inputs.
    """
    q_bits, kv_bits, bt, seqlens, scale, causal = _case_arrays(case)
    B, s_q, h_q, D = q_bits.shape
    sc = _scale64(scale)
    out = np.zeros((B, s_q, h_q, V_DIM))
    lse = np.zeros((B, s_q, h_q))
    for b in range(B):
        L = int(seqlens[b])
        keys = []
        for t in range(L):
            page = int(bt[b][t // PAGE])
            slot = t % PAGE
            keys.append([float(x) for x in bf16_to_f64(kv_bits[page, slot])])
        for i in range(s_q):
            # query i is cache position L - s_q + i when causal
            last = (L - s_q + i) if causal else (L - 1)
            for h in range(h_q):
                qv = [float(x) for x in bf16_to_f64(q_bits[b, i, h])]
                scores = []
                for t in range(L):
                    if t <= last:
                        scores.append(sc * math.fsum(qv[d] * keys[t][d] for d in range(D)))
                if not scores:
                    out[b, i, h, :] = 0.0
                    lse[b, i, h] = -math.inf
                    continue
                m = max(scores)
                z = math.fsum(math.exp(s - m) for s in scores)
                ls = m + math.log(z)
                w = [math.exp(s - ls) for s in scores]
                for c in range(V_DIM):
                    out[b, i, h, c] = math.fsum(w[t] * keys[t][c] for t in range(len(w)))
                lse[b, i, h] = ls
    return out, lse


# --------------------------------------------------------------------------
# explicit per-head form (keys/values widened from the latent per head)
# --------------------------------------------------------------------------
def explicit_heads(c: np.ndarray, r: np.ndarray, q_c: np.ndarray, q_r: np.ndarray,
                   W_UK: np.ndarray, W_UV: np.ndarray, scale: float):
    """Attention with keys and values restored per head from the latent.

    ``c [T,512]`` latents, ``r [T,64]`` rotary keys shared by all heads,
    ``q_c [H,128]`` and ``q_r [H,64]`` per-head query parts, ``W_UK`` and
    ``W_UV`` ``[H,128,512]`` up-projections.  Head ``h`` uses keys
    ``[W_UK[h] c_t ; r_t]`` (192-d) and values ``W_UV[h] c_t`` (128-d).
    This is the un-absorbed form that the latent trick rewrites (release note,
    MLA principles: widen the compressed latent at compute time).
    Returns ``o [H,128]`` and ``lse [H]``.
    """
    H = q_c.shape[0]
    T = c.shape[0]
    o = np.zeros((H, W_UV.shape[1]))
    lse = np.zeros(H)
    for h in range(H):
        k_h = np.concatenate([c @ W_UK[h].T, r], axis=1)  # [T, 192]
        v_h = c @ W_UV[h].T  # [T, 128]
        q_h = np.concatenate([q_c[h], q_r[h]])  # [192]
        s = scale * (k_h @ q_h)
        m = s.max()
        ls = m + np.log(np.exp(s - m).sum())
        p = np.exp(s - ls)
        o[h] = p @ v_h
        lse[h] = ls
        assert T == k_h.shape[0]
    return o, lse


def absorb_query(q_c: np.ndarray, q_r: np.ndarray, W_UK: np.ndarray) -> np.ndarray:
    """Absorbed query ``[W_UK[h]^T q_c[h] ; q_r[h]]`` (576-d) per head."""
    return np.concatenate([np.einsum("hdk,hd->hk", W_UK, q_c), q_r], axis=1)


def absorb_output(out: np.ndarray, W_UV: np.ndarray) -> np.ndarray:
    """Per-head output ``W_UV[h] out[h]`` (512 -> 128 values): head h's values
    are ``W_UV[h] c_t``, and the weights sum over tokens commutes with the
    linear map (release note, MLA principles).  ``out [H,512]`` -> ``[H,128]``."""
    return np.einsum("hdk,hk->hd", W_UV, out)


def absorb_ref(case):
    """Both absorption products of a ``workloads.AbsorbCase``, in float64 from
    the exactly widened bf16 inputs: ``q_out [b,s_q,h,576]`` (from q_nope,
    q_rope and w_uk as stored) and ``o [b,s_q,h,128]`` (from lat_out, w_uv).
    Each query token is an independent application of ``absorb_query`` /
    ``absorb_output``."""
    qn = bf16_to_f64(case.q_nope)
    qr = bf16_to_f64(case.q_rope)
    wk = bf16_to_f64(case.w_uk)
    wv = bf16_to_f64(case.w_uv)
    lo = bf16_to_f64(case.lat_out)
    b, s, h = case.batch, case.s_q, case.h_q
    q_out = np.zeros((b, s, h, HEAD_DIM))
    o = np.zeros((b, s, h, wv.shape[1]))
    for bi in range(b):
        for i in range(s):
            q_out[bi, i] = absorb_query(qn[bi, i], qr[bi, i], wk)
            o[bi, i] = absorb_output(lo[bi, i], wv)
    return q_out, o


# --------------------------------------------------------------------------
# splitting the key range and merging by log-sum-exp
# --------------------------------------------------------------------------
def merge_partials(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]):
    """Merge per-range results ``(o_s, lse_s)`` into the full-range result.

    ``o_s`` is each range's own normalised output; the merged output is
    ``sum_s exp(lse_s - lse) o_s`` with ``lse = log sum_s exp(lse_s)``.
    Ranges with ``lse_s = -inf`` carry no weight; all empty gives 0 / -inf.
    """
    lses = np.stack([np.asarray(x, dtype=np.float64) for x in lses])  # [S, R]
    outs = np.stack([np.asarray(x, dtype=np.float64) for x in outs])  # [S, R, C]
    M = lses.max(axis=0)
    finite = np.isfinite(M)
    Msafe = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Msafe[None, :]), 0.0)
    Z = w.sum(axis=0)
    lse = np.where(finite, Msafe + np.log(np.where(finite, Z, 1.0)), -np.inf)
    coef = np.where(finite[None, :], w / np.where(finite, Z, 1.0)[None, :], 0.0)
    out = np.einsum("sr,src->rc", coef, outs)
    return out, lse


def attend_chunks_and_merge(Q: np.ndarray, K: np.ndarray, n_rows: Sequence[int],
                            scale: float, cuts: Sequence[int]):
    """Attend over key ranges ``[cuts[j], cuts[j+1])`` separately, then merge.

    Each range's result uses only the keys in it that the row can see.
    """
    n_rows = np.asarray(n_rows, dtype=np.int64)
    outs, lses = [], []
    for a, z in zip(cuts[:-1], cuts[1:]):
        Kc = K[a:z]
        n_c = np.clip(n_rows - a, 0, z - a)
        o, l = attend_f64(Q, Kc, n_c, scale)
        outs.append(o)
        lses.append(l)
    return merge_partials(outs, lses)


# --------------------------------------------------------------------------
# paged KV append with page allocation
# --------------------------------------------------------------------------
def kv_append_ref(kv_bits: np.ndarray, block_table: np.ndarray, seqlens: np.ndarray,
                  new_kv_bits: np.ndarray, free_pages: np.ndarray, free_count: int):
    """Append ``new_kv_bits [b, n, 576]`` to each sequence of a paged cache.

    The cache is paged, 64 tokens per block, blocks handed out on demand as a
    sequence grows (release note, released paged cache; Tom's Hardware FR
    article, techniques paragraph).  Token ``t`` of sequence ``b`` lives at
    page ``block_table[b, t // 64]``, slot ``t % 64``.  Sequence ``b`` needs
    ``ceil((L+n)/64) - ceil(L/64)`` new pages; they are popped from the top
    of the free-page stack (``free_pages[:free_count]``) in batch order, i.e.
    sequence b's i-th new page is ``free_pages[F - 1 - (K_b + i)]``.  If the
    stack is too short or a row of the table too short, nothing changes and
    the status is 1.  Works on copies; returns
    ``(kv, block_table, seqlens, free_count, status)``.
    """
    kv = kv_bits.copy()
    bt = block_table.copy()
    sl = seqlens.copy()
    batch, n, _ = new_kv_bits.shape
    max_pages = bt.shape[1]
    old = [(int(L) + PAGE - 1) // PAGE for L in sl]
    new = [(int(L) + n + PAGE - 1) // PAGE for L in sl]
    need = [new[b] - old[b] for b in range(batch)]
    if sum(need) > free_count or any(x > max_pages for x in new):
        return kv, bt, sl, free_count, 1
    taken = 0
    for b in range(batch):
        for i in range(need[b]):
            bt[b, old[b] + i] = free_pages[free_count - 1 - taken]
            taken += 1
        L = int(sl[b])
        for i in range(n):
            t = L + i
            kv[bt[b, t // PAGE], t % PAGE, :] = new_kv_bits[b, i, :]
        sl[b] = L + n
    return kv, bt, sl, free_count - taken, 0
