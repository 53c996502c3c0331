"""Debug checks of device contents (MLA_DEBUG): a decode whose cache lengths
or used block-table entries are out of range returns a status and launches
no decode kernel; in-range inputs give the same bits as without the checks.

Every case here is safe to run: the check pass reads only the lengths and
the entries j < min(ceil(L/64), max_pages) of each row, and the decode is not
launched when they are out of range, so no kernel reads outside a buffer.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from workloads import make_case  # noqa: E402

STATUS_DEVICE_CONTENTS = 5


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import mla_paged_kv_06_amd as m
    m.load_library()
    prev = m.set_debug_checks(True)
    yield m
    m.set_debug_checks(prev)


def _dev(case):
    dev = torch.device("cuda:0")
    q = torch.from_numpy(case.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kv = torch.from_numpy(case.kv.view(np.int16)).to(dev).view(torch.bfloat16)
    return q, kv, torch.from_numpy(case.block_table).to(dev), \
        torch.from_numpy(case.cache_seqlens).to(dev)


def _base():
    return make_case([130, 64, 0, 700], 1, 16, False, seed=201, pool_factor=1.25)


@pytest.mark.parametrize("what", ["entry_past_pool", "entry_negative", "length_past_table",
                                  "length_negative"])
@pytest.mark.parametrize("schedule", ["separate", "in_decode"])
def test_bad_contents_are_flagged(mla, what, schedule):
    case = _base()
    q, kv, bt, sl = _dev(case)
    if what == "entry_past_pool":
        bt[3, 5] = case.num_pages          # a used entry (700 tokens use 11 pages)
    elif what == "entry_negative":
        bt[0, 2] = -1                      # the third page of 130 tokens
    elif what == "length_past_table":
        sl[1] = case.max_pages * 64 + 1
    else:
        sl[2] = -3
    out = torch.full((case.batch, 1, 16, 512), 7.0, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.full((case.batch, 1, 16), 7.0, dtype=torch.float32, device="cuda:0")
    with pytest.raises(mla.MlaError) as e:
        if schedule == "separate":
            meta, splits = mla.get_metadata(sl, 1, 16)
        else:
            meta, splits = None, torch.zeros((case.batch + 1,), dtype=torch.int32, device="cuda:0")
        mla.decode_paged(q, kv, bt, sl, case.softmax_scale, False, meta, splits, out=out, lse=lse)
    assert e.value.status == STATUS_DEVICE_CONTENTS
    torch.cuda.synchronize()
    # nothing was launched: the outputs keep their fill
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)


def test_unused_entries_are_not_checked(mla):
    """Entries past a sequence's last page are never read, so garbage there
    is not an error, and the result equals the one without checks."""
    case = _base()
    q, kv, bt, sl = _dev(case)
    ref_out, ref_lse = mla.mla_decode(q, kv, bt, sl, case.softmax_scale, False)
    bt2 = bt.clone()
    bt2[0, 3:] = 10 ** 9   # 130 tokens use pages 0..2
    bt2[2, :] = -5         # an empty sequence uses none
    out, lse = mla.mla_decode(q, kv, bt2, sl, case.softmax_scale, False)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse, ref_lse)


def test_checks_off_gives_the_same_bits(mla):
    case = make_case([1, 200, 4097, 65, 0, 3000], 2, 64, True, seed=203, pool_factor=1.25)
    q, kv, bt, sl = _dev(case)
    on = mla.mla_decode(q, kv, bt, sl, case.softmax_scale, True)
    mla.set_debug_checks(False)
    try:
        off = mla.mla_decode(q, kv, bt, sl, case.softmax_scale, True)
    finally:
        mla.set_debug_checks(True)
    torch.cuda.synchronize()
    assert torch.equal(on[0].view(torch.int16), off[0].view(torch.int16))
    assert torch.equal(on[1], off[1])


def test_checks_refuse_graph_capture(mla):
    """With the checks on, a decode must wait for them: under capture it
    returns MLA_ERR_UNSUPPORTED instead."""
    case = _base()
    q, kv, bt, sl = _dev(case)
    meta, splits = mla.get_metadata(sl, 1, 16)
    out = torch.empty((case.batch, 1, 16, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((case.batch, 1, 16), dtype=torch.float32, device="cuda:0")
    ws = torch.empty((mla.workspace_bytes(case.batch, 1, 16),), dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g, stream=s):
        try:
            mla.decode_paged(q, kv, bt, sl, case.softmax_scale, False, meta, splits,
                             workspace=ws, out=out, lse=lse)
        except mla.MlaError as e:
            err = e
    assert err is not None and err.status == 2
