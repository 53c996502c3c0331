"""Pins of the MLA prefill oracle (oracle/prefill.py) against facts that do
not come from it: scalar brute force, the explicit per-head form of the
decode oracle (itself pinned by the absorbed == explicit equivalence), the
absorbed latent decode, packing invariance, and planted mistakes."""

import math

import numpy as np
import pytest

import oracle
from oracle import prefill as pf
from workloads import make_prefill_case


def _f64(case):
    lat = oracle.bf16_to_f64(case.latent)
    return (lat[:, :512], lat[:, 512:], oracle.bf16_to_f64(case.q),
            oracle.bf16_to_f64(case.w_uk), oracle.bf16_to_f64(case.w_uv))


def _parts(case):
    c, r, q, wk, wv = _f64(case)
    k_nope, v = pf.expand_kv(c, wk, wv)
    return q, k_nope, r, v


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("seqlens,h", [([5], 2), ([4, 1, 6], 3), ([0, 7], 1)])
def test_attention_matches_bruteforce(seqlens, h, causal):
    case = make_prefill_case(seqlens, h, seed=11 + len(seqlens))
    q, k_nope, r, v = _parts(case)
    o, l = pf.attention_ref(q, k_nope, r, v, case.cu_seqlens, case.softmax_scale, causal)
    ob, lb = pf.attention_bruteforce(q, k_nope, r, v, case.cu_seqlens, case.softmax_scale, causal)
    assert np.max(np.abs(o - ob)) <= 1e-12
    assert np.max(np.abs(l - lb)) <= 1e-12


def test_expand_kv_by_hand():
    """k_nope[t, h, d] = sum_c W_UK[h, d, c] c_t[c], summed in plain loops."""
    case = make_prefill_case([3], 2, seed=21)
    c, r, q, wk, wv = _f64(case)
    k_nope, v = pf.expand_kv(c, wk, wv)
    for t in range(3):
        for h in range(2):
            for d in (0, 63, 127):
                assert abs(k_nope[t, h, d] - math.fsum(wk[h, d, x] * c[t, x] for x in range(512))) < 1e-12
                assert abs(v[t, h, d] - math.fsum(wv[h, d, x] * c[t, x] for x in range(512))) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_rows_equal_explicit_heads(causal):
    """Query t of a prompt, every head, equals the explicit per-head
    attention of the decode oracle over the tokens it sees."""
    case = make_prefill_case([6, 9], 3, seed=31)
    c, r, q, wk, wv = _f64(case)
    o, l = pf.prefill_ref(c, r, q, wk, wv, case.cu_seqlens, case.softmax_scale, causal)
    scale = float(np.float32(case.softmax_scale))
    cu = case.cu_seqlens
    for s in range(2):
        for t in range(cu[s], cu[s + 1]):
            end = t + 1 if causal else cu[s + 1]
            oe, le = oracle.explicit_heads(c[cu[s]:end], r[cu[s]:end], q[t, :, :128], q[t, :, 128:],
                                           wk, wv, scale)
            assert np.max(np.abs(o[t] - oe)) <= 1e-12
            assert np.max(np.abs(l[t] - le)) <= 1e-12


def test_equals_absorbed_latent_decode():
    """Prefill in per-head form equals the absorbed form: queries folded into
    the latent ([W_UK,h^T q_nope ; q_rope], 576 values), attention over the
    cached [c ; r] with the causal mask (query t sees t + 1 tokens), then
    W_UV,h applied to the 512-value latent output."""
    case = make_prefill_case([11], 2, seed=41)
    c, r, q, wk, wv = _f64(case)
    o, l = pf.prefill_ref(c, r, q, wk, wv, case.cu_seqlens, case.softmax_scale, True)
    lat = np.concatenate([c, r], axis=1)
    scale = float(np.float32(case.softmax_scale))
    T = 11
    for h in range(2):
        Qt = oracle.absorb_query(q[:, h, :128], q[:, h, 128:], np.broadcast_to(wk[h], (T,) + wk[h].shape))
        out, lse = oracle.attend_f64(Qt, lat, [t + 1 for t in range(T)], scale)
        oh = oracle.absorb_output(out, np.broadcast_to(wv[h], (T,) + wv[h].shape))
        assert np.max(np.abs(oh - o[:, h])) <= 1e-10
        assert np.max(np.abs(lse - l[:, h])) <= 1e-10


def test_packing_is_invisible():
    """Two prompts packed together give what each gives alone."""
    case = make_prefill_case([7, 5], 2, seed=51)
    q, k_nope, r, v = _parts(case)
    o, l = pf.attention_ref(q, k_nope, r, v, case.cu_seqlens, case.softmax_scale)
    o0, l0 = pf.attention_ref(q[:7], k_nope[:7], r[:7], v[:7], [0, 7], case.softmax_scale)
    o1, l1 = pf.attention_ref(q[7:], k_nope[7:], r[7:], v[7:], [0, 5], case.softmax_scale)
    assert np.array_equal(o[:7], o0) and np.array_equal(o[7:], o1)
    assert np.array_equal(l[:7], l0) and np.array_equal(l[7:], l1)


def test_first_token_sees_only_itself():
    """Causal row 0 of a prompt: out is its own value, lse its own score."""
    case = make_prefill_case([4], 2, seed=61)
    q, k_nope, r, v = _parts(case)
    o, l = pf.attention_ref(q, k_nope, r, v, case.cu_seqlens, case.softmax_scale)
    sc = float(np.float32(case.softmax_scale))
    for h in range(2):
        key = np.concatenate([k_nope[0, h], r[0]])
        assert abs(l[0, h] - sc * float(q[0, h] @ key)) <= 1e-12
        assert np.max(np.abs(o[0, h] - v[0, h])) <= 1e-12


def test_rows_helper_matches_whole():
    case = make_prefill_case([9, 6], 2, seed=71)
    q, k_nope, r, v = _parts(case)
    o, l = pf.attention_ref(q, k_nope, r, v, case.cu_seqlens, case.softmax_scale)
    rows = [(0, 0), (8, 1), (9, 0), (14, 1), (12, 0)]
    got = pf.attention_rows(q, k_nope, r, v, case.cu_seqlens, case.softmax_scale, True, rows)
    for (t, h), (oo, ll) in zip(rows, got):
        assert np.max(np.abs(oo - o[t, h])) <= 1e-12 and abs(ll - l[t, h]) <= 1e-12


def test_planted_mask_off_by_one_is_caught(monkeypatch):
    """A causal mask that hides the diagonal fails the explicit-heads pin."""
    good = np.triu

    def bad(m, k=0):
        return good(m, k=0 if k == 1 else k)

    monkeypatch.setattr(pf.np, "triu", bad)
    with pytest.raises(AssertionError):
        test_rows_equal_explicit_heads(True)


def test_planted_dropped_rope_is_caught(monkeypatch):
    """Keys without their rotary part fail the brute force."""
    good = pf.attention_ref

    def bad(q, k_nope, k_rope, v, cu, scale, causal=True):
        return good(q, k_nope, np.zeros_like(np.asarray(k_rope, np.float64)), v, cu, scale, causal)

    monkeypatch.setattr(pf, "attention_ref", bad)
    with pytest.raises(AssertionError):
        test_attention_matches_bruteforce([5], 2, True)


def test_planted_swapped_weights_are_caught(monkeypatch):
    """Values widened with W_UK instead of W_UV fail the explicit-heads pin."""
    good = pf.expand_kv
    monkeypatch.setattr(pf, "expand_kv", lambda c, wk, wv: good(c, wk, wk))
    with pytest.raises(AssertionError):
        test_rows_equal_explicit_heads(True)
