"""The decode step that allocates nothing (mla_decode_step_noalloc), called
through the C ABI, against the existing entry points (mla_decode_paged +
mla_combine with caller-given buffers): the same kernels, so the same bits.
Two calls in a row share the library's static scratch, the second on a
smaller input; a shape that needs more scratch than there is is refused
before anything is launched."""

import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from workloads import make_case  # noqa: E402

SCRATCH_TOO_SMALL = 6


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import mla_paged_kv_06_amd as m
    m.load_library()
    return m


def _dev(case):
    dev = torch.device("cuda:0")
    q = torch.from_numpy(case.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kv = torch.from_numpy(case.kv.view(np.int16)).to(dev).view(torch.bfloat16)
    return q, kv, torch.from_numpy(case.block_table).to(dev), \
        torch.from_numpy(case.cache_seqlens).to(dev)


def _noalloc(mla, case, tensors):
    """The entry point itself, through ctypes; returns (status, out, lse)."""
    q, kv, bt, sl = tensors
    lib = mla.load_library()
    out = torch.full((case.batch, case.s_q, case.h_q, 512), 3.0, dtype=torch.bfloat16,
                     device="cuda:0")
    lse = torch.full((case.batch, case.s_q, case.h_q), 3.0, dtype=torch.float32, device="cuda:0")
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.mla_decode_step_noalloc(vp(q), vp(kv), vp(bt), vp(sl), case.batch, case.s_q,
                                     case.h_q, kv.shape[0], bt.shape[1], case.softmax_scale,
                                     int(case.causal), vp(out), vp(lse),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, out, lse


def _reference(mla, case, tensors):
    """mla_decode_paged + mla_combine with caller-given workspace, the same
    schedule choice (inside the decode wherever it can go)."""
    q, kv, bt, sl = tensors
    return mla.mla_decode(q, kv, bt, sl, case.softmax_scale, case.causal, schedule="auto")


@pytest.mark.parametrize("first,second", [
    # (lengths, s_q, h_q) of the first call, then a smaller second call
    (([3000, 129, 64, 4097, 0], 1, 16), ([700, 65], 1, 16)),          # 16-row kernel, split
    (([5000, 1, 2200], 2, 128), ([300, 1900], 2, 64)),                # 64-row kernel, row groups
    (([1200] * 3, 2, 16), ([70], 1, 8)),                              # 32-row kernel
    (([40] * 1100, 1, 16), ([90] * 1030, 1, 16)),                     # separate schedule (> 1024)
])
def test_noalloc_matches_the_entry_points(mla, first, second):
    for i, (L, s_q, h_q) in enumerate((first, second)):
        print(f"[noalloc] call {i}: batch {len(L)} s_q {s_q} h_q {h_q}", flush=True)
        case = make_case(L, s_q, h_q, s_q > 1, seed=300 + 7 * i + s_q * h_q, pool_factor=1.25,
                         poison_unused=True, poison_tail=True)
        t = _dev(case)
        st, out, lse = _noalloc(mla, case, t)
        assert st == 0, mla.load_library().mla_status_string(st)
        ref_out, ref_lse = _reference(mla, case, t)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"out, call {i}"
        assert torch.equal(lse, ref_lse), f"lse, call {i}"


def test_noalloc_refuses_shapes_beyond_its_scratch(mla):
    """2048 rows per sequence over 40 sequences need about 100 MB of
    partials: refused with its own status, nothing launched."""
    case = make_case([64] * 40, 16, 128, True, seed=333)
    t = _dev(case)
    need = mla.workspace_bytes(40, 16, 128)
    assert need > mla.NOALLOC_SCRATCH_BYTES
    st, out, lse = _noalloc(mla, case, t)
    torch.cuda.synchronize()
    assert st == SCRATCH_TOO_SMALL
    assert torch.all(out == 3.0) and torch.all(lse == 3.0)
    # and a call after the refusal still works
    small = make_case([100, 3], 1, 16, False, seed=334)
    ts = _dev(small)
    st, out, lse = _noalloc(mla, small, ts)
    ref_out, ref_lse = _reference(mla, small, ts)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse, ref_lse)


def test_noalloc_in_a_graph(mla):
    """The no-allocation step captured in a HIP graph (its purpose): every
    replay, with eager work in between, gives the eager bits."""
    case = make_case([3000, 129, 64, 0, 700], 2, 64, True, seed=351, pool_factor=1.25,
                     poison_unused=True, poison_tail=True)
    q, kv, bt, sl = _dev(case)
    out = torch.empty((case.batch, 2, 64, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((case.batch, 2, 64), dtype=torch.float32, device="cuda:0")
    mla.decode_step_noalloc(q, kv, bt, sl, case.softmax_scale, True, out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = out.view(torch.int16).clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mla.decode_step_noalloc(q, kv, bt, sl, case.softmax_scale, True, out, lse)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(-3.0)
        lse.fill_(-3.0)
        small = make_case([100, 3], 1, 16, False, seed=352 + r)
        ts = _dev(small)
        st, _, _ = _noalloc(mla, small, ts)  # another call on the same scratch
        assert st == 0
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o), f"out, replay {r}"
        assert torch.equal(lse, ref_l), f"lse, replay {r}"
