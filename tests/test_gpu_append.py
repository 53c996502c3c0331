"""GPU parity of the paged KV append with page allocation (mla_kv_append)
through the C ABI, against the oracle: integer and byte work, so every
output -- the whole cache pool, the block table, the lengths, the free-page
count and the status word -- must match bit for bit."""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import bf16_bits_from_f32, make_append_case, make_case  # noqa: E402


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


def _bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


def _run(mla, case, free_count=None):
    fc0 = len(case.free_pages) if free_count is None else free_count
    kv = _bits(case.kv)
    bt = _i32(case.block_table)
    sl = _i32(case.seqlens)
    fp = _i32(case.free_pages if len(case.free_pages) else np.zeros(1, np.int32))
    fc = _i32(np.array([fc0]))
    st = mla.kv_append(kv, bt, sl, _bits(case.new_kv), fp, fc)
    torch.cuda.synchronize()
    got = (kv.view(torch.int16).cpu().numpy().view(np.uint16), bt.cpu().numpy(), sl.cpu().numpy(),
           int(fc.cpu()[0]), int(st.cpu()[0]))
    ref = oracle.kv_append_ref(case.kv, case.block_table, case.seqlens, case.new_kv,
                               case.free_pages, fc0)
    return got, ref


def _same(got, ref):
    assert got[4] == ref[4], f"status {got[4]} != {ref[4]}"
    assert got[3] == ref[3], f"free count {got[3]} != {ref[3]}"
    assert np.array_equal(got[2], ref[2]), "lengths"
    assert np.array_equal(got[1], ref[1]), "block table"
    assert np.array_equal(got[0], ref[0]), "cache pool"


EDGE = [0, 1, 63, 64, 65, 200, 127]


@pytest.mark.parametrize("n_new", [0, 1, 2, 64, 130])
def test_append_parity(mla, n_new):
    _say(f"[append] edge lengths n_new={n_new}")
    case = make_append_case(EDGE, n_new, free=40, seed=300 + n_new)
    got, ref = _run(mla, case)
    _same(got, ref)
    assert got[4] == 0


def test_append_many_sequences(mla):
    """More sequences than the allocator's block (1024): its chunked scan."""
    _say("[append] 1500 sequences")
    rng = np.random.Generator(np.random.PCG64(77))
    L = [int(x) for x in rng.integers(0, 400, size=1500)]
    case = make_append_case(L, 2, free=1600, seed=78)
    got, ref = _run(mla, case)
    _same(got, ref)
    assert got[4] == 0


def test_append_shortage_and_short_rows_write_nothing(mla):
    _say("[append] shortage")
    case = make_append_case([63, 64, 0, 5], 2, free=2, seed=81)
    got, ref = _run(mla, case)
    _same(got, ref)
    assert got[4] == 1
    case = make_append_case([64, 10], 1, free=4, seed=82, max_pages=1)
    got, ref = _run(mla, case)
    _same(got, ref)
    assert got[4] == 1
    # a stack shorter than the array: only free_count entries are free
    case = make_append_case([63, 64, 0], 2, free=8, seed=83)
    got, ref = _run(mla, case, free_count=3)
    _same(got, ref)
    assert got[3] == 0


def test_append_then_decode(mla):
    """Two decode steps' worth of appends (1 then 2 tokens), each followed by
    a decode, against the oracle decode of the cache the oracle appended."""
    _say("[append] append then decode")
    dcase = make_case([100, 64, 1, 300], 2, 16, True, seed=91, pool_factor=1.25)
    held = set(int(p) for p in dcase.block_table.ravel() if p >= 0)
    free = np.array([p for p in range(dcase.num_pages) if p not in held], dtype=np.int32)
    kv = _bits(dcase.kv)
    bt = _i32(dcase.block_table)
    sl = _i32(dcase.cache_seqlens)
    fp = _i32(free)
    fc = _i32(np.array([len(free)]))
    kv_h, bt_h, sl_h, fc_h = dcase.kv.copy(), dcase.block_table.copy(), dcase.cache_seqlens.copy(), len(free)
    rng = np.random.Generator(np.random.PCG64(92))
    q = torch.from_numpy(dcase.q.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    for n_new in (1, 2):
        new_kv = bf16_bits_from_f32(rng.standard_normal((4, n_new, 576), dtype=np.float32))
        st = mla.kv_append(kv, bt, sl, _bits(new_kv), fp, fc)
        kv_h, bt_h, sl_h, fc_h, st_h = oracle.kv_append_ref(kv_h, bt_h, sl_h, new_kv, free, fc_h)
        out, lse = mla.mla_decode(q, kv, bt, sl, dcase.softmax_scale, True)
        torch.cuda.synchronize()
        assert int(st.cpu()[0]) == 0 and st_h == 0
        assert np.array_equal(sl.cpu().numpy(), sl_h)
        dcase.kv, dcase.block_table, dcase.cache_seqlens = kv_h, bt_h, sl_h
        ref_out, ref_lse = oracle.decode_ref(dcase)
        o = oracle.bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
        err = np.abs(o - ref_out)
        assert float((err - (1e-2 + 2e-2 * np.abs(ref_out))).max()) <= 0.0
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-3
