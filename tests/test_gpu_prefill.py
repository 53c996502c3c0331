"""GPU parity of MLA prefill (per-head form) through the C ABI.

* the expansion (latent -> per-head key part and value) against the oracle's
  fp64 products of the same bf16 inputs;
* the attention against the oracle fed the very bf16 keys and values the
  GPU expansion produced (so only the attention's own rounding is measured):
  |o - ref| <= 1e-2 + 2e-2 |ref| per element, normwise <= 2e-2, lse <= 1e-3;
* end to end (expansion + attention) against the oracle's prefill from the
  latents in fp64, whose rows are pinned to the explicit per-head form.  The
  GPU rounds k_nope and v to bf16 (2^-8 relative) after a float32 sum of 512
  terms; score t moves by at most d_t = scale * sum_d |q_d| e_d with
  e_d = 2^-8 |k_d| + 512 * 2^-24 sum_c |W_UK[d, c] c_c|, and lse by at most
  max_t d_t, so lse is gated at 1e-3 + that bound per row.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from oracle import prefill as pf  # noqa: E402
from workloads import make_prefill_case  # noqa: E402

ATOL, RTOL, NORM_RTOL, LSE_ATOL = 1e-2, 2e-2, 2e-2, 1e-3


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import mla_paged_kv_06_amd as m
    m.load_library()
    return m


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(
        torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _close(got, ref):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), "non-finite output"
    excess = float((err - (ATOL + RTOL * np.abs(ref))).max())
    nrm = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert excess <= 0.0, f"outside atol + rtol |ref| (max abs err {float(err.max())})"
    assert nrm <= NORM_RTOL, f"normwise rel err {nrm}"
    return float(err.max()), nrm


def _run(mla, case, causal=True, max_seqlen=None):
    lat = _dev(case.latent)
    k_nope, v = mla.prefill_expand_kv(lat, _dev(case.w_uk), _dev(case.w_uv))
    cu = torch.from_numpy(case.cu_seqlens).to("cuda:0")
    L = np.diff(case.cu_seqlens)
    ms = int(L.max()) if max_seqlen is None else max_seqlen
    o, lse = mla.prefill_attention(_dev(case.q), k_nope, lat[:, 512:], v, cu, ms,
                                   case.softmax_scale, causal)
    torch.cuda.synchronize()
    return _bits(k_nope), _bits(v), _bits(o), lse.cpu().numpy().astype(np.float64)


SHAPES = [
    # lengths, heads, causal
    ([1, 63, 64, 65, 300, 257], 4, True),
    ([700], 16, True),
    ([700, 129], 16, False),
    ([513, 0, 1000], 8, True),
    ([300, 45], 3, True),  # odd head count: the expansion's last column tile is half empty
]


@pytest.mark.parametrize("seqlens,h,causal", SHAPES)
def test_prefill_parity(mla, seqlens, h, causal):
    print(f"[prefill] lengths {seqlens} heads {h} causal {causal}", flush=True)
    case = make_prefill_case(seqlens, h, seed=401 + h + len(seqlens))
    kn_b, v_b, o_b, lse = _run(mla, case, causal)
    lat = oracle.bf16_to_f64(case.latent)
    c, r = lat[:, :512], lat[:, 512:]
    q = oracle.bf16_to_f64(case.q)
    wk, wv = oracle.bf16_to_f64(case.w_uk), oracle.bf16_to_f64(case.w_uv)
    # the expansion
    kn_ref, v_ref = pf.expand_kv(c, wk, wv)
    _close(oracle.bf16_to_f64(kn_b), kn_ref)
    _close(oracle.bf16_to_f64(v_b), v_ref)
    # the attention, on the GPU's own keys and values
    kn, vv = oracle.bf16_to_f64(kn_b), oracle.bf16_to_f64(v_b)
    o_ref, l_ref = pf.attention_ref(q, kn, r, vv, case.cu_seqlens, case.softmax_scale, causal)
    o = oracle.bf16_to_f64(o_b)
    e = _close(o, o_ref)
    assert np.abs(lse - l_ref).max() <= LSE_ATOL
    # end to end, from the latents, against the explicit per-head form
    o_x, l_x = pf.prefill_ref(c, r, q, wk, wv, case.cu_seqlens, case.softmax_scale, causal)
    _close(o, o_x)
    e_d = 2.0 ** -8 * np.abs(kn_ref) + 512 * 2.0 ** -24 * np.einsum("hdk,tk->thd", np.abs(wk),
                                                                   np.abs(c))
    sc = float(np.float32(case.softmax_scale))
    bound = np.zeros_like(l_x)
    cu = case.cu_seqlens
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        # d[t', h, u] = scale * sum_d |q[t', h, d]| e[u, h, d]; lse moves by the max over visible u
        d = sc * np.einsum("thd,uhd->thu", np.abs(q[a:b, :, :128]), e_d[a:b])
        if causal:
            d = np.where(np.tril(np.ones((b - a, b - a), bool))[:, None, :], d, 0.0)
        bound[a:b] = d.max(axis=2)
    assert np.all(np.abs(lse - l_x) <= LSE_ATOL + bound), "lse end to end"
    print(f"[prefill] attention max|err| {e[0]:.2e} norm {e[1]:.2e}", flush=True)


def test_prefill_long_prompt_sampled(mla):
    """A 4096-token prompt at 128 heads (16 query blocks per head, the
    causal diagonal in every one): sampled rows of every part of the
    prompt, the oracle on the GPU's own keys and values, row by row."""
    print("[prefill] 4096 tokens x 128 heads, sampled rows", flush=True)
    case = make_prefill_case([4096], 128, seed=451)
    kn_b, v_b, o_b, lse = _run(mla, case, True)
    rng = np.random.Generator(np.random.PCG64(452))
    rows = [(0, 0), (4095, 127), (255, 3), (256, 3), (257, 90), (1023, 64), (1024, 64),
            (2047, 17), (3071, 100), (4094, 5)]
    rows += [(int(t), int(h)) for t, h in zip(rng.integers(0, 4096, 40), rng.integers(0, 128, 40))]
    r = oracle.bf16_to_f64(case.latent[:, 512:])
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for h in sorted({h for _, h in rows}):
        ts = [t for t, hh in rows if hh == h]
        qh = oracle.bf16_to_f64(case.q[:, h:h + 1])
        kh = oracle.bf16_to_f64(kn_b[:, h:h + 1])
        vh = oracle.bf16_to_f64(v_b[:, h:h + 1])
        ref = pf.attention_rows(qh, kh, r, vh, case.cu_seqlens, case.softmax_scale, True,
                                [(t, 0) for t in ts])
        for t, (oo, ll) in zip(ts, ref):
            got_o.append(oracle.bf16_to_f64(o_b[t, h]))
            got_l.append(lse[t, h])
            ref_o.append(oo)
            ref_l.append(ll)
    _close(np.stack(got_o), np.stack(ref_o))
    assert np.abs(np.array(got_l) - np.array(ref_l)).max() <= LSE_ATOL


def test_prefill_max_seqlen_above_longest(mla):
    """max_seqlen only sizes the grid: a larger value gives the same bits."""
    case = make_prefill_case([300, 70], 4, seed=461)
    a = _run(mla, case, True)
    b = _run(mla, case, True, max_seqlen=2000)
    assert np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3])


def test_prefill_errors(mla):
    case = make_prefill_case([10], 2, seed=471)
    lat = _dev(case.latent)
    k_nope, v = mla.prefill_expand_kv(lat, _dev(case.w_uk), _dev(case.w_uv))
    cu = torch.from_numpy(case.cu_seqlens).to("cuda:0")
    with pytest.raises(mla.MlaError):
        mla.prefill_attention(_dev(case.q), k_nope, lat[:, 512:], v, cu, 10, 0.0)
    with pytest.raises(mla.MlaError):
        mla.prefill_attention(_dev(case.q), k_nope, lat[:, 512:], v, cu, 10, float("nan"))


def test_expansion_rows_are_independent_of_tiling(mla):
    """Every output value is one fixed-order float32 sum over its latent row
    and weight row, so a token's k_nope and v do not depend on where its row
    falls in the 256-row tiles, on how many tokens share the launch, or on
    the latent row stride: the same bits from 300 tokens at stride 576
    (cache entries [c ; r]), from their first 37, and from rows 200 .. 299
    packed at stride 512."""
    case = make_prefill_case([300], 6, seed=481)
    lat = _dev(case.latent)                      # [300, 576]
    wk, wv = _dev(case.w_uk), _dev(case.w_uv)
    kn_all, v_all = mla.prefill_expand_kv(lat, wk, wv)
    kn_head, v_head = mla.prefill_expand_kv(lat[:37], wk, wv)
    packed = lat[200:, :512].contiguous()        # stride 512, rows 200 .. 299
    kn_tail, v_tail = mla.prefill_expand_kv(packed, wk, wv)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16).cpu()  # noqa: E731
    assert torch.equal(bits(kn_all[:37]), bits(kn_head))
    assert torch.equal(bits(v_all[:37]), bits(v_head))
    assert torch.equal(bits(kn_all[200:]), bits(kn_tail))
    assert torch.equal(bits(v_all[200:]), bits(v_tail))


def test_expansion_refuses_a_huge_latent_stride(mla):
    case = make_prefill_case([4], 2, seed=491)
    wk, wv = _dev(case.w_uk), _dev(case.w_uv)
    big = torch.empty((2, (1 << 21) + 8), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(mla.MlaError):
        mla.prefill_expand_kv(big, wk, wv)


def _random_prompts(n, seed):
    """Seeded small prompt mixes: 1..4 prompts of 0..400 tokens (with block
    edges), 1..9 heads, causal or not."""
    rng = np.random.Generator(np.random.PCG64(seed))
    edges = [0, 1, 63, 64, 65, 255, 256, 257]
    out = []
    for i in range(n):
        k = int(rng.integers(1, 5))
        lens = [int(rng.choice(edges)) if rng.random() < 0.4 else int(rng.integers(1, 401))
                for _ in range(k)]
        if sum(lens) == 0:
            lens[0] = 1
        out.append((lens, int(rng.integers(1, 10)), bool(rng.random() < 0.7), seed * 100 + i))
    return out


@pytest.mark.parametrize("seqlens,h,causal,seed", _random_prompts(12, 7001))
def test_prefill_random_mixes(mla, seqlens, h, causal, seed):
    print(f"[prefill random] lengths {seqlens} heads {h} causal {causal} seed {seed}", flush=True)
    case = make_prefill_case(seqlens, h, seed=seed)
    kn_b, v_b, o_b, lse = _run(mla, case, causal)
    lat = oracle.bf16_to_f64(case.latent)
    c, r = lat[:, :512], lat[:, 512:]
    q = oracle.bf16_to_f64(case.q)
    wk, wv = oracle.bf16_to_f64(case.w_uk), oracle.bf16_to_f64(case.w_uv)
    kn_ref, v_ref = pf.expand_kv(c, wk, wv)
    _close(oracle.bf16_to_f64(kn_b), kn_ref)
    _close(oracle.bf16_to_f64(v_b), v_ref)
    kn, vv = oracle.bf16_to_f64(kn_b), oracle.bf16_to_f64(v_b)
    o_ref, l_ref = pf.attention_ref(q, kn, r, vv, case.cu_seqlens, case.softmax_scale, causal)
    _close(oracle.bf16_to_f64(o_b), o_ref)
    assert np.abs(lse - l_ref).max() <= LSE_ATOL
