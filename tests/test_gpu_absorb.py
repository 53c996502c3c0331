"""GPU parity of the absorption products (query 128 -> 512 values per head,
output 512 -> 128) through the C ABI, against the fp64 oracle.

Gates as for the decode output: every element within 1e-2 absolute plus 2e-2
relative, the normwise relative error at most 2e-2; the rotary part of the
absorbed query is a copy and must match bit for bit.
"""

import math
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import make_absorb_case, make_case  # noqa: E402

ATOL = 1e-2
RTOL = 2e-2
NORM_RTOL = 2e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import mla_paged_kv_06_amd as m
    m.load_library()  # raises if the HIP library is missing
    return m


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(
        torch.bfloat16)


def _host(t):
    return oracle.bf16_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


def _close(got, ref):
    err = np.abs(got - ref)
    excess = float((err - (ATOL + RTOL * np.abs(ref))).max())
    nrm = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert np.all(np.isfinite(got)), "non-finite output"
    assert excess <= 0.0, f"outside atol+rtol*|ref| (max abs err {float(err.max())})"
    assert nrm <= NORM_RTOL, f"normwise rel err {nrm}"
    return float(err.max()), nrm


def _oracle_tokens(case, tokens):
    """Oracle of both products for the (b, i) query tokens listed."""
    qn = oracle.bf16_to_f64(case.q_nope)
    qr = oracle.bf16_to_f64(case.q_rope)
    wk = oracle.bf16_to_f64(case.w_uk)
    wv = oracle.bf16_to_f64(case.w_uv)
    lo = oracle.bf16_to_f64(case.lat_out)
    q_ref = np.stack([oracle.absorb_query(qn[b, i], qr[b, i], wk) for b, i in tokens])
    o_ref = np.stack([oracle.absorb_output(lo[b, i], wv) for b, i in tokens])
    return q_ref, o_ref


# (batch, s_q, h_q): one head; the memory-bound shape; two query tokens; a
# ragged 16-row tile (37 rows); more than one 256-row chunk with a ragged
# end (300); the compute-bound and multi-token shapes (sampled tokens); the
# tile-pipeline edges: whole tiles then a ragged one right where the
# prefetch ring ends (81 rows for the query product's 5 tiles ahead, 33 for
# the output product's 2), and whole-tile counts that are and are not a
# multiple of the ring (96, 48)
SHAPES = [(1, 1, 1), (8, 1, 16), (3, 2, 128), (37, 1, 64), (300, 1, 16), (64, 1, 128),
          (128, 2, 128), (81, 1, 16), (33, 1, 16), (96, 1, 4), (48, 1, 4)]


@pytest.mark.parametrize("batch,s_q,h_q", SHAPES)
def test_absorb_parity(mla, batch, s_q, h_q):
    _say(f"[absorb] batch={batch} s_q={s_q} h_q={h_q}")
    case = make_absorb_case(batch, s_q, h_q, seed=1000 + batch + 7 * s_q + h_q)
    q_out = mla.absorb_query(_dev(case.q_nope), _dev(case.q_rope), _dev(case.w_uk_t))
    o = mla.absorb_output(_dev(case.lat_out), _dev(case.w_uv))
    torch.cuda.synchronize()
    q_got, o_got = _host(q_out), _host(o)
    tokens = [(b, i) for b in range(batch) for i in range(s_q)]
    if len(tokens) > 48:
        rng = np.random.Generator(np.random.PCG64(batch * 131 + h_q))
        pick = sorted(set([0, len(tokens) - 1, 15, 16, 255, 256] +
                          [int(x) for x in rng.integers(0, len(tokens), 24)]))
        tokens = [tokens[t] for t in pick if t < len(tokens)]
    q_ref, o_ref = _oracle_tokens(case, tokens)
    q_sel = np.stack([q_got[b, i] for b, i in tokens])
    o_sel = np.stack([o_got[b, i] for b, i in tokens])
    # the rotary part is copied
    qr = oracle.bf16_to_f64(case.q_rope)
    assert np.array_equal(q_sel[..., 512:], np.stack([qr[b, i] for b, i in tokens]))
    eq = _close(q_sel[..., :512], q_ref[..., :512])
    eo = _close(o_sel, o_ref)
    _say(f"[absorb] query max|err| {eq[0]:.2e} norm {eq[1]:.2e}; output {eo[0]:.2e} {eo[1]:.2e}")


def test_absorb_repeat_is_deterministic(mla):
    case = make_absorb_case(40, 1, 16, seed=3)
    a = mla.absorb_output(_dev(case.lat_out), _dev(case.w_uv))
    b = mla.absorb_output(_dev(case.lat_out), _dev(case.w_uv))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_absorb_errors_raise(mla):
    case = make_absorb_case(2, 1, 4, seed=5)
    with pytest.raises(ValueError):
        mla.absorb_query(_dev(case.q_nope), _dev(case.q_rope), _dev(case.w_uv))  # wrong layout
    with pytest.raises(mla.MlaError):
        bad = torch.empty((70000, 1, 4, 512), dtype=torch.bfloat16, device="cuda:0")
        mla.absorb_output(bad, _dev(case.w_uv))  # batch above the limit


def test_mla_layer_through_the_gpu_equals_explicit_heads(mla):
    """Query absorption -> paged latent decode -> output absorption, all on
    the GPU, against the explicit per-head attention (keys [W_UK c ; r],
    values W_UV c) in fp64 on the same bf16 inputs.

    lse gates.  The GPU forms the absorbed query q~ in float32 (128 terms)
    and rounds it to bf16 before the decode; the explicit form never forms
    q~.  Each element then moves by at most e_d = 2^-8 |q~_d| (bf16 has 8
    significant bits) + 128 * 2^-24 * sum_k |W_UK[k,d] q_k| (float32
    accumulation), so score t moves by at most d_t = scale * sum_d e_d |c_t,d|
    (the rotary part is copied exactly), and the log-sum-exp of the scores
    by at most max_t d_t (it is 1-Lipschitz in the max norm).  So:
      * against the decode oracle fed the GPU's own bf16 q~: 1e-3, the
        decode's gate;
      * against the explicit heads: 1e-3 + max_t d_t, computed per row."""
    _say("[absorb] layer: absorb -> decode -> absorb vs explicit heads")
    h_q = 16
    dcase = make_case([100, 300, 64], 1, h_q, False, seed=59, pool_factor=1.25)
    acase = make_absorb_case(3, 1, h_q, seed=61)
    q_t = mla.absorb_query(_dev(acase.q_nope), _dev(acase.q_rope), _dev(acase.w_uk_t))
    kv = _dev(dcase.kv)
    bt = torch.from_numpy(dcase.block_table).to("cuda:0")
    sl = torch.from_numpy(dcase.cache_seqlens).to("cuda:0")
    out, lse = mla.mla_decode(q_t, kv, bt, sl, dcase.softmax_scale, False)
    o = mla.absorb_output(out, _dev(acase.w_uv))
    torch.cuda.synchronize()
    o_got = _host(o)
    lse_got = lse.cpu().numpy().astype(np.float64)
    q_t_bits = q_t.view(torch.int16).cpu().numpy().view(np.uint16)
    # the decode oracle on the GPU's rounded absorbed query
    rcase = type(dcase)(q=q_t_bits, kv=dcase.kv, block_table=dcase.block_table,
                        cache_seqlens=dcase.cache_seqlens, softmax_scale=dcase.softmax_scale,
                        causal=False)
    _, lse_dec = oracle.decode_ref(rcase)
    assert np.abs(lse_got - lse_dec).max() <= 1e-3, "lse against the decode oracle"
    wk = oracle.bf16_to_f64(acase.w_uk)
    wv = oracle.bf16_to_f64(acase.w_uv)
    scale = float(np.float32(dcase.softmax_scale))
    worst = 0.0
    for b in range(3):
        lat = oracle.gather_latents(dcase.kv, dcase.block_table[b], int(dcase.cache_seqlens[b]))
        c, r = lat[:, :512], lat[:, 512:]
        qn = oracle.bf16_to_f64(acase.q_nope[b, 0])
        qr = oracle.bf16_to_f64(acase.q_rope[b, 0])
        o_ref, lse_ref = oracle.explicit_heads(c, r, qn, qr, wk, wv, scale)
        _close(o_got[b, 0], o_ref)
        # only the 512 absorbed values are rounded; the rotary part is copied
        q_abs = np.abs(oracle.absorb_query(qn, qr, wk))[:, :512]  # [h, 512], unrounded
        q_sum = np.abs(oracle.absorb_query(np.abs(qn), qr, np.abs(wk)))[:, :512]
        e = 2.0 ** -8 * q_abs + 128 * 2.0 ** -24 * q_sum
        bound = scale * (np.abs(c) @ e.T).max(axis=0)  # [h]
        err = np.abs(lse_got[b, 0] - lse_ref)
        assert np.all(err <= 1e-3 + bound), "lse of the layer"
        worst = max(worst, float((err / (1e-3 + bound)).max()))
    _say(f"[absorb] layer lse error at most {worst:.2f} of its derived bound")
    assert math.isfinite(float(np.abs(o_got).max()))
