"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each check is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, an off-by-one mask, a misread
block table) breaks at least one of them; the last tests plant such slips and
confirm they are caught.
"""

import math
import os

import numpy as np
import pytest

import oracle
from oracle import mla_oracle
import workloads
from workloads import make_case, make_config_case, CONFIGS, PAGE, HEAD_DIM, V_DIM
from casebuild import case_from_values, permute_pool, read_golden

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(seqlens, s_q, h_q, causal, seed, pool_factor=1.0):
    return make_case(seqlens, s_q, h_q, causal, seed, pool_factor=pool_factor)


# ---------------------------------------------------------------- (a) brute force
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seqlens,s_q,h_q", [
    ([1, 5], 1, 3),
    ([63, 64], 2, 2),
    ([65, 7, 130], 2, 2),
    ([2, 1], 2, 1),
])
def test_bruteforce_matches_vectorized(seqlens, s_q, h_q, causal):
    case = _tiny(seqlens, s_q, h_q, causal, seed=7, pool_factor=1.25)
    o_ref, l_ref = oracle.decode_ref(case)
    o_bf, l_bf = oracle.decode_bruteforce(case)
    assert np.array_equal(np.isinf(l_ref), np.isinf(l_bf))
    fin = np.isfinite(l_ref)
    assert np.allclose(l_ref[fin], l_bf[fin], rtol=0, atol=1e-12)
    assert np.allclose(o_ref, o_bf, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- (b) absorbed == explicit heads
def test_absorbed_equals_explicit_heads():
    rng = np.random.Generator(np.random.PCG64(11))
    H, T = 4, 37
    c = rng.standard_normal((T, 512))
    r = rng.standard_normal((T, 64))
    q_c = rng.standard_normal((H, 128))
    q_r = rng.standard_normal((H, 64))
    W_UK = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    W_UV = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    scale = 1.0 / math.sqrt(192.0)
    o_exp, lse_exp = oracle.explicit_heads(c, r, q_c, q_r, W_UK, W_UV, scale)
    q_abs = oracle.absorb_query(q_c, q_r, W_UK)  # [H, 576]
    K = np.concatenate([c, r], axis=1)  # cache entries [c_t ; r_t]
    out, lse = oracle.attend_f64(q_abs, K, [T] * H, scale)
    o_abs = oracle.absorb_output(out, W_UV)
    assert np.allclose(lse, lse_exp, rtol=1e-12, atol=0)
    rel = np.linalg.norm(o_abs - o_exp) / np.linalg.norm(o_exp)
    assert rel < 1e-10


# ---------------------------------------------------------------- (c) paging
def test_page_permutation_is_bitwise_invariant():
    case = _tiny([130, 64, 1, 200], 2, 3, True, seed=3, pool_factor=1.25)
    o1, l1 = oracle.decode_ref(case)
    o2, l2 = oracle.decode_ref(permute_pool(case, seed=99))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_paged_equals_contiguous():
    case = _tiny([130, 77], 1, 4, False, seed=5, pool_factor=1.25)
    # rebuild the same logical cache contiguously: sequence b occupies pages
    # in order, starting where the previous one ended
    n = [(int(L) + PAGE - 1) // PAGE for L in case.cache_seqlens]
    kv = np.zeros((sum(n), PAGE, HEAD_DIM), dtype=np.uint16)
    bt = np.full_like(case.block_table, -1)
    k = 0
    for b, nb in enumerate(n):
        for j in range(nb):
            kv[k] = case.kv[case.block_table[b, j]]
            bt[b, j] = k
            k += 1
    flat = type(case)(q=case.q, kv=kv, block_table=bt, cache_seqlens=case.cache_seqlens,
                      softmax_scale=case.softmax_scale, causal=case.causal)
    o1, l1 = oracle.decode_ref(case)
    o2, l2 = oracle.decode_ref(flat)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_unused_pages_and_tail_slots_do_not_matter():
    clean = _tiny([70, 129], 1, 2, False, seed=8, pool_factor=1.25)
    dirty = make_case([70, 129], 1, 2, False, 8, pool_factor=1.25,
                      poison_unused=True, poison_tail=True)
    o1, l1 = oracle.decode_ref(clean)
    o2, l2 = oracle.decode_ref(dirty)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- (d) weights sum to one
def test_weights_sum_to_one():
    case = _tiny([300, 65], 2, 4, True, seed=21)
    for b in range(case.batch):
        P = oracle.softmax_weights(case, b)
        assert np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert np.all(P >= 0)


# ---------------------------------------------------------------- closed forms
def test_single_token_gives_its_value_and_score():
    case = _tiny([1], 1, 5, False, seed=31)
    o, l = oracle.decode_ref(case)
    k0 = oracle.bf16_to_f64(case.kv[case.block_table[0, 0], 0])
    q = oracle.bf16_to_f64(case.q[0, 0])
    s0 = float(np.float32(case.softmax_scale)) * (q @ k0)
    assert np.allclose(o[0, 0], np.broadcast_to(k0[:V_DIM], (5, V_DIM)), atol=1e-12)
    assert np.allclose(l[0, 0], s0, atol=1e-12)


def test_zero_scale_gives_mean_and_log_n():
    case = _tiny([150], 1, 3, False, seed=41)
    case.softmax_scale = 0.0
    o, l = oracle.decode_ref(case)
    K = oracle.gather_latents(case.kv, case.block_table[0], 150)
    assert np.allclose(l, math.log(150), atol=1e-12)
    assert np.allclose(o[0, 0], K[:, :V_DIM].mean(axis=0), atol=1e-12)


def test_identical_tokens():
    rng = np.random.Generator(np.random.PCG64(51))
    tok = np.round(rng.standard_normal(HEAD_DIM) * 4) / 4  # bf16-exact
    kv = np.broadcast_to(tok, (2, PAGE, HEAD_DIM)).astype(np.float32)
    q = (np.round(rng.standard_normal((1, 1, 2, HEAD_DIM)) * 4) / 4).astype(np.float32)
    case = case_from_values(q, kv, [[1, 0]], [100], 0.125, False)
    o, l = oracle.decode_ref(case)
    for h in range(2):
        s = 0.125 * float(q[0, 0, h].astype(np.float64) @ tok)
        assert abs(l[0, 0, h] - (s + math.log(100))) < 1e-12
        assert np.allclose(o[0, 0, h], tok[:V_DIM], atol=1e-12)


def test_identical_queries_give_identical_rows():
    case = _tiny([90], 1, 4, False, seed=61)
    case.q[0, 0, 1:] = case.q[0, 0, 0]
    o, l = oracle.decode_ref(case)
    for h in range(1, 4):
        assert np.array_equal(o[0, 0, h], o[0, 0, 0]) and l[0, 0, h] == l[0, 0, 0]


def test_value_all_ones_gives_ones():
    case = _tiny([333, 20], 2, 3, True, seed=71)
    one_bits = np.uint16(0x3F80)  # bf16 1.0
    case.kv[:, :, :V_DIM] = one_bits
    o, _ = oracle.decode_ref(case)
    assert np.allclose(o, 1.0, atol=1e-12)


def test_empty_sequence_convention():
    case = _tiny([0, 5], 1, 2, False, seed=81)
    o, l = oracle.decode_ref(case)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(l[0]))
    assert np.all(np.isfinite(l[1]))


# ---------------------------------------------------------------- causal alignment
def test_causal_row_equals_shorter_decode():
    L = 150
    case = _tiny([L], 2, 3, True, seed=91)
    o, l = oracle.decode_ref(case)
    for i in range(2):
        single = type(case)(q=case.q[:, i:i + 1].copy(), kv=case.kv, block_table=case.block_table,
                            cache_seqlens=np.array([L - 1 + i], dtype=np.int32),
                            softmax_scale=case.softmax_scale, causal=False)
        o1, l1 = oracle.decode_ref(single)
        assert np.allclose(o[:, i], o1[:, 0], atol=1e-12)
        assert np.allclose(l[:, i], l1[:, 0], atol=1e-12)


def test_single_query_causal_equals_noncausal():
    a = _tiny([77, 300], 1, 2, True, seed=101)
    b = _tiny([77, 300], 1, 2, False, seed=101)
    oa, la = oracle.decode_ref(a)
    ob, lb = oracle.decode_ref(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


# ---------------------------------------------------------------- single rows
# rows (b, i, h) chosen so that a swapped (i, h), a wrong query index handed to
# the causal mask or a stale cached sequence changes the result
_ROW_CASES = [
    # lengths, s_q, h_q, causal
    ([130, 0, 65, 3], 3, 2, True),
    ([70, 64, 1], 2, 3, True),
    ([129, 5], 3, 2, False),
]


def _all_rows(case, order_seed=None):
    rows = [(b, i, h) for b in range(case.batch) for i in range(case.s_q) for h in range(case.h_q)]
    if order_seed is not None:  # jump between sequences, so the gather cache is refreshed
        rng = np.random.Generator(np.random.PCG64(order_seed))
        rows = [rows[k] for k in rng.permutation(len(rows))]
    return rows


@pytest.mark.parametrize("seqlens,s_q,h_q,causal", _ROW_CASES)
def test_rows_match_bruteforce(seqlens, s_q, h_q, causal):
    """Every row of decode_ref_rows against the scalar brute force (its own
    loops, its own position walk and block-table lookups), rows visited in a
    shuffled order; the empty sequence gives 0 / -inf."""
    case = _tiny(seqlens, s_q, h_q, causal, seed=121 + s_q * h_q, pool_factor=1.25)
    o_bf, l_bf = oracle.decode_bruteforce(case)
    rows = _all_rows(case, order_seed=5)
    got = oracle.decode_ref_rows(case, rows)
    for (b, i, h), (o, l) in zip(rows, got):
        if math.isinf(l_bf[b, i, h]):
            assert math.isinf(l) and l < 0 and np.all(o == 0.0), (b, i, h)
            continue
        assert abs(l - l_bf[b, i, h]) <= 1e-12, (b, i, h)
        assert np.max(np.abs(o - o_bf[b, i, h])) <= 1e-12, (b, i, h)


@pytest.mark.parametrize("seqlens,s_q,h_q,causal", _ROW_CASES)
def test_rows_match_whole_reference(seqlens, s_q, h_q, causal):
    """decode_ref_rows equals decode_ref row for row (the same definition,
    one row at a time instead of one sequence at a time)."""
    case = _tiny(seqlens, s_q, h_q, causal, seed=131 + s_q, pool_factor=1.25)
    o_ref, l_ref = oracle.decode_ref(case)
    rows = _all_rows(case)
    got = oracle.decode_ref_rows(case, rows)
    for (b, i, h), (o, l) in zip(rows, got):
        if math.isinf(l_ref[b, i, h]):
            assert math.isinf(l) and np.all(o == 0.0)
            continue
        assert abs(l - l_ref[b, i, h]) <= 1e-12
        assert np.max(np.abs(o - o_ref[b, i, h])) <= 1e-12


def test_rows_distinguish_token_and_head():
    """Rows (b, i, h) and (b, h, i) of a causal case differ, so a swapped
    index cannot pass unnoticed."""
    case = _tiny([90], 3, 3, True, seed=141)
    a = oracle.decode_ref_rows(case, [(0, 0, 2)])[0]
    b = oracle.decode_ref_rows(case, [(0, 2, 0)])[0]
    assert abs(a[1] - b[1]) > 1e-3


def test_planted_row_index_swap_is_caught(monkeypatch):
    """decode_ref_rows reading q[b, h, i] instead of q[b, i, h] fails the
    brute-force pin."""
    good = mla_oracle.decode_ref_rows

    def bad(case, rows):
        return good(case, [(b, h, i) if h < case.s_q and i < case.h_q else (b, i, h)
                           for (b, i, h) in rows])

    monkeypatch.setattr(oracle, "decode_ref_rows", bad)
    with pytest.raises(AssertionError):
        test_rows_match_bruteforce([130, 0, 65, 3], 3, 2, True)


def test_planted_row_mask_index_is_caught(monkeypatch):
    """A causal mask taken for the head index instead of the query token
    fails the brute-force pin."""
    good_vis = mla_oracle.visible_tokens
    calls = {"n": 0}

    def bad_rows(case, rows):
        out = []
        for (b, i, h) in rows:
            monkeypatch.setattr(mla_oracle, "visible_tokens",
                                lambda L, s_q, _i, c, hh=h: good_vis(L, s_q, min(hh, s_q - 1), c))
            out += mla_oracle.decode_ref_rows(case, [(b, i, h)])
            monkeypatch.setattr(mla_oracle, "visible_tokens", good_vis)
            calls["n"] += 1
        return out

    monkeypatch.setattr(oracle, "decode_ref_rows", bad_rows)
    with pytest.raises(AssertionError):
        test_rows_match_bruteforce([70, 64, 1], 2, 3, True)
    assert calls["n"] > 0


# ---------------------------------------------------------------- split + merge
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_split_and_merge_equals_unsplit(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    T, R = 257, 6
    Q = rng.standard_normal((R, HEAD_DIM))
    K = rng.standard_normal((T, HEAD_DIM))
    n_rows = rng.integers(0, T + 1, size=R)
    n_rows[0] = T
    n_rows[1] = 0
    scale = 1.0 / math.sqrt(192)
    o_full, l_full = oracle.attend_f64(Q, K, n_rows, scale)
    cuts = sorted(set([0, T] + list(rng.integers(1, T, size=5))))
    o_m, l_m = oracle.attend_chunks_and_merge(Q, K, n_rows, scale, cuts)
    assert np.array_equal(np.isinf(l_full), np.isinf(l_m))
    fin = np.isfinite(l_full)
    assert np.allclose(l_full[fin], l_m[fin], atol=1e-12)
    assert np.allclose(o_full, o_m, atol=1e-12)


# ---------------------------------------------------------------- golden worked examples
def test_golden_two_token_example():
    vals, _ = read_golden(os.path.join(GOLDEN, "two_token_example.txt"))
    kv = np.zeros((1, PAGE, HEAD_DIM), dtype=np.float32)
    kv[0, 0, 1] = 4.0
    kv[0, 1, 0] = 1.0
    kv[0, 1, 2] = 2.0
    q = np.zeros((1, 1, 1, HEAD_DIM), dtype=np.float32)
    q[0, 0, 0, 0] = 1.0
    case = case_from_values(q, kv, [[0]], [2], math.log(3.0), False)
    for fn in (oracle.decode_ref, oracle.decode_bruteforce):
        o, l = fn(case)
        o = o[0, 0, 0]
        assert abs(o[0] - vals["out_0"]) < 1e-7
        assert abs(o[1] - vals["out_1"]) < 1e-7
        assert abs(o[2] - vals["out_2"]) < 1e-7
        assert np.all(np.abs(o[3:]) <= vals["out_rest"] + 1e-12)
        assert abs(l[0, 0, 0] - vals["lse"]) < 1e-7


def test_golden_causal_example():
    vals, _ = read_golden(os.path.join(GOLDEN, "causal_example.txt"))
    kv = np.zeros((1, PAGE, HEAD_DIM), dtype=np.float32)
    for t in range(3):
        kv[0, t, t] = t + 1.0
    q = np.zeros((1, 2, 1, HEAD_DIM), dtype=np.float32)
    case = case_from_values(q, kv, [[0]], [3], 1.0, True)
    for fn in (oracle.decode_ref, oracle.decode_bruteforce):
        o, l = fn(case)
        for i in range(2):
            for d in range(3):
                assert abs(o[0, i, 0, d] - vals[f"q{i}_out_{d}"]) < 1e-12
            assert abs(l[0, i, 0] - vals[f"q{i}_lse"]) < 1e-12


def test_golden_kv_bytes_per_token():
    _, rows = read_golden(os.path.join(GOLDEN, "kv_bytes_per_token.txt"))
    assert len(rows) == 3
    for name, layers, per_layer, nbytes, printed_kb in rows:
        total = int(layers) * int(per_layer) * int(nbytes)
        assert total // 1000 == int(printed_kb), name  # printed figures are truncated
    # the MLA row is exactly the oracle's per-token geometry
    assert int(rows[0][2]) == HEAD_DIM and int(rows[0][3]) == 2


# ---------------------------------------------------------------- workloads
def test_config_shapes_and_tables():
    case = make_config_case(2)
    spec = CONFIGS[2]
    assert case.q.shape == (8, 1, 16, HEAD_DIM)
    L = case.cache_seqlens
    assert np.all((L >= 1024) & (L <= 4096))
    n = (L + PAGE - 1) // PAGE
    used = np.concatenate([case.block_table[b, :n[b]] for b in range(8)])
    assert len(set(used.tolist())) == len(used)  # no page shared
    assert case.num_pages == math.ceil(n.sum() * spec.pool_factor)
    for b in range(8):
        assert np.all(case.block_table[b, n[b]:] == -1)
    again = make_config_case(2)
    assert np.array_equal(again.kv, case.kv) and np.array_equal(again.q, case.q)


# ---------------------------------------------------------------- planted mistakes
def test_planted_mask_off_by_one_is_caught(monkeypatch):
    """A causal mask shifted by one breaks the hand-derived causal example."""
    good = mla_oracle.visible_tokens
    monkeypatch.setattr(mla_oracle, "visible_tokens",
                        lambda L, s_q, i, c: good(L, s_q, i, c) - (1 if c else 0))
    with pytest.raises(AssertionError):
        test_golden_causal_example()


def test_planted_dropped_rope_is_caught(monkeypatch):
    """Scores that skip the 64 rotary dims disagree with the brute force."""
    good = mla_oracle.attend_f64

    def bad(Q, K, n_rows, scale, return_p=False):
        K2 = np.array(K, dtype=np.float64)
        K2[:, V_DIM:] = 0.0
        res = good(Q, K2, n_rows, scale, return_p=True)
        P = res[2]
        out = P @ np.asarray(K, dtype=np.float64)[:, :V_DIM]
        return (out, res[1], P) if return_p else (out, res[1])

    monkeypatch.setattr(mla_oracle, "attend_f64", bad)
    with pytest.raises(AssertionError):
        test_bruteforce_matches_vectorized([65, 7, 130], 2, 2, False)


def test_planted_page_misread_is_caught(monkeypatch):
    """Reading physical page j instead of block_table[b, j] breaks invariance."""
    def bad_gather(kv_bits, block_row, L):
        L = int(L)
        n_pages = (L + PAGE - 1) // PAGE
        lat = kv_bits[np.arange(n_pages)].reshape(n_pages * PAGE, HEAD_DIM)[:L]
        return mla_oracle.bf16_to_f64(lat)

    monkeypatch.setattr(mla_oracle, "gather_latents", bad_gather)
    with pytest.raises(AssertionError):
        test_page_permutation_is_bitwise_invariant()


def test_planted_transposed_value_is_caught(monkeypatch):
    """Weighting the rotary tail instead of the latent breaks V == 1."""
    good = mla_oracle.attend_f64

    def bad(Q, K, n_rows, scale, return_p=False):
        res = good(Q, K, n_rows, scale, return_p=True)
        K = np.asarray(K, dtype=np.float64)
        out = res[2] @ np.concatenate([K[:, 64:], K[:, :64]], axis=1)[:, :V_DIM]
        return (out, res[1], res[2]) if return_p else (out, res[1])

    monkeypatch.setattr(mla_oracle, "attend_f64", bad)
    with pytest.raises(AssertionError):
        test_value_all_ones_gives_ones()


# ---------------------------------------------------------------- absorption products
def test_absorb_ref_bruteforce():
    """Both absorption products against scalar fsum loops over every output
    value of a tiny case (pins the index order of both einsums: a swapped
    operand or axis changes values)."""
    case = workloads.make_absorb_case(2, 2, 3, seed=41)
    q_out, o = oracle.absorb_ref(case)
    qn = oracle.bf16_to_f64(case.q_nope)
    qr = oracle.bf16_to_f64(case.q_rope)
    wk = oracle.bf16_to_f64(case.w_uk)
    wv = oracle.bf16_to_f64(case.w_uv)
    lo = oracle.bf16_to_f64(case.lat_out)
    for b in range(2):
        for i in range(2):
            for h in range(3):
                for c in range(0, 512, 37):
                    ref = math.fsum(wk[h, d, c] * qn[b, i, h, d] for d in range(128))
                    assert abs(q_out[b, i, h, c] - ref) <= 1e-12 * (1 + abs(ref))
                assert np.array_equal(q_out[b, i, h, 512:], qr[b, i, h])
                for d in range(0, 128, 11):
                    ref = math.fsum(wv[h, d, c] * lo[b, i, h, c] for c in range(512))
                    assert abs(o[b, i, h, d] - ref) <= 1e-12 * (1 + abs(ref))


def test_absorb_layouts_of_the_inputs():
    """The transposed query weight the HIP path reads holds the same values."""
    case = workloads.make_absorb_case(1, 1, 2, seed=43)
    assert case.w_uk_t.shape == (2, 512, 128)
    assert np.array_equal(case.w_uk_t[1, 300, 7], case.w_uk[1, 7, 300])


def test_absorbed_pipeline_equals_explicit_heads_per_token():
    """absorb_ref's query and output products wrapped around the latent
    attention give the explicit per-head attention for every query token."""
    case = workloads.make_absorb_case(2, 1, 2, seed=47)
    q_out, _ = oracle.absorb_ref(case)
    rng = np.random.Generator(np.random.PCG64(53))
    T = 29
    c = rng.standard_normal((T, 512))
    r = rng.standard_normal((T, 64))
    K = np.concatenate([c, r], axis=1)
    wk = oracle.bf16_to_f64(case.w_uk)
    wv = oracle.bf16_to_f64(case.w_uv)
    scale = 1.0 / math.sqrt(192.0)
    for b in range(2):
        qn = oracle.bf16_to_f64(case.q_nope[b, 0])
        qr = oracle.bf16_to_f64(case.q_rope[b, 0])
        o_exp, lse_exp = oracle.explicit_heads(c, r, qn, qr, wk, wv, scale)
        out, lse = oracle.attend_f64(q_out[b, 0], K, [T] * 2, scale)
        o_abs = oracle.absorb_output(out, wv)
        assert np.allclose(lse, lse_exp, rtol=1e-12, atol=0)
        assert np.linalg.norm(o_abs - o_exp) <= 1e-10 * np.linalg.norm(o_exp)


# ---------------------------------------------------------------- paged KV append
def _append_case(seqlens, n_new, free, seed, max_pages=None):
    c = workloads.make_append_case(seqlens, n_new, free, seed, max_pages)
    return c.kv, c.block_table, c.seqlens, c.new_kv, c.free_pages


def test_kv_append_worked_example():
    """Hand-worked allocation: lengths 63, 64, 0, 130 with 2 new tokens need
    1, 1, 1, 0 new pages; the stack [10 11 12 13 14] (top = 14) gives 14, 13,
    12 in batch order and keeps 2 entries."""
    kv = np.zeros((15, PAGE, HEAD_DIM), dtype=np.uint16)
    bt = np.full((4, 4), -1, dtype=np.int32)
    bt[0, 0] = 0
    bt[1, 0] = 1
    bt[3, :3] = [2, 3, 4]
    sl = np.array([63, 64, 0, 130], dtype=np.int32)
    new_kv = np.arange(4 * 2 * HEAD_DIM, dtype=np.uint16).reshape(4, 2, HEAD_DIM)
    free = np.array([10, 11, 12, 13, 14], dtype=np.int32)
    kv2, bt2, sl2, fc, st = oracle.kv_append_ref(kv, bt, sl, new_kv, free, 5)
    assert st == 0 and fc == 2
    assert bt2[0, 1] == 14 and bt2[1, 1] == 13 and bt2[2, 0] == 12
    assert list(sl2) == [65, 66, 2, 132]
    # sequence 0: token 63 -> page 0 slot 63, token 64 -> page 14 slot 0
    assert np.array_equal(kv2[0, 63], new_kv[0, 0]) and np.array_equal(kv2[14, 0], new_kv[0, 1])
    # sequence 1: tokens 64, 65 -> page 13 slots 0, 1; sequence 3: page 4 slots 2, 3
    assert np.array_equal(kv2[13, 1], new_kv[1, 1]) and np.array_equal(kv2[4, 3], new_kv[3, 1])
    assert np.array_equal(kv2[12, 1], new_kv[2, 1])


def test_kv_append_logical_view():
    """After the append every sequence reads back as its old tokens followed
    by the new ones, through its updated block table."""
    seqlens = [0, 1, 63, 64, 65, 200, 127]
    for n_new in (1, 2, 64, 130):
        kv, bt, sl, new_kv, free = _append_case(seqlens, n_new, free=40, seed=n_new)
        kv2, bt2, sl2, fc, st = oracle.kv_append_ref(kv, bt, sl, new_kv, free, len(free))
        assert st == 0
        for b, L in enumerate(seqlens):
            before = oracle.gather_latents(kv, bt[b], L)
            after = oracle.gather_latents(kv2, bt2[b], L + n_new)
            assert np.array_equal(after[:L], before)
            assert np.array_equal(after[L:], oracle.bf16_to_f64(new_kv[b]))
        taken = [int(p) for b in range(len(seqlens)) for p in bt2[b] if p >= 0 and p not in bt[b]]
        assert sorted(taken) == sorted(int(p) for p in free[fc:])  # the top of the stack
        assert len(set(taken)) == len(taken)


def test_kv_append_shortage_writes_nothing():
    kv, bt, sl, new_kv, free = _append_case([63, 64, 0], 2, free=2, seed=9)
    kv2, bt2, sl2, fc, st = oracle.kv_append_ref(kv, bt, sl, new_kv, free, len(free))
    assert st == 1 and fc == 2
    assert np.array_equal(kv2, kv) and np.array_equal(bt2, bt) and np.array_equal(sl2, sl)
    # a table row too short also stops everything
    kv, bt, sl, new_kv, free = _append_case([64], 1, free=4, seed=10, max_pages=1)
    assert oracle.kv_append_ref(kv, bt, sl, new_kv, free, len(free))[4] == 1


def test_kv_append_nothing_new():
    kv, bt, sl, new_kv, free = _append_case([5, 64], 0, free=3, seed=11)
    kv2, bt2, sl2, fc, st = oracle.kv_append_ref(kv, bt, sl, new_kv, free, len(free))
    assert st == 0 and fc == 3 and np.array_equal(kv2, kv) and np.array_equal(sl2, sl)
