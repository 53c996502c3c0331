"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Gates: every output element within 1e-2 absolute plus 2e-2 relative
(|g - r| <= 1e-2 + 2e-2 |r|, the allclose form of the stated tolerance), the
normwise relative error of ``out`` at most 2e-2, and ``lse`` within 1e-3
absolute; empty rows must give exactly out = 0 and lse = -inf on both sides.
The output is bf16: for |out| in [2, 4) one bf16 ulp is 2^-6, so rounding
alone may cost 7.8e-3, which is why the relative term is needed.
"""

import math
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import make_case, make_config_case  # noqa: E402
from casebuild import permute_pool  # noqa: E402
from sched_model import schedule  # noqa: E402

OUT_ATOL = 1e-2
OUT_RTOL = 2e-2
OUT_NORM_RTOL = 2e-2
LSE_ATOL = 1e-3


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


def to_dev(case):
    dev = torch.device("cuda:0")
    q = torch.from_numpy(case.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kv = torch.from_numpy(case.kv.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.cache_seqlens).to(dev)
    return q, kv, bt, sl


def run(mla, case, num_cus=0):
    q, kv, bt, sl = to_dev(case)
    out, lse = mla.mla_decode(q, kv, bt, sl, case.softmax_scale, case.causal, num_cus=num_cus)
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return oracle.bf16_to_f64(o), lse.cpu().numpy().astype(np.float64)


def compare(out, lse, ref_out, ref_lse, batches=None):
    if batches is not None:
        out, lse = out[batches], lse[batches]
        ref_out, ref_lse = ref_out[batches], ref_lse[batches]
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), "empty rows differ"
    assert np.all(out[empty] == 0.0)
    assert np.all(np.isfinite(out)), "non-finite output"
    live = ~empty
    if not np.any(live):
        return 0.0, 0.0, 0.0
    err = np.abs(out - ref_out)
    max_abs = float(err.max())
    excess = float((err - (OUT_ATOL + OUT_RTOL * np.abs(ref_out))).max())
    nrm = float(np.linalg.norm(out[live] - ref_out[live]) / max(np.linalg.norm(ref_out[live]), 1e-30))
    lse_err = float(np.abs(lse[live] - ref_lse[live]).max())
    assert excess <= 0.0, f"out outside atol+rtol*|ref| (max abs err {max_abs})"
    assert nrm <= OUT_NORM_RTOL, f"out normwise rel err {nrm}"
    assert lse_err <= LSE_ATOL, f"lse max abs err {lse_err}"
    return max_abs, nrm, lse_err


# ---------------------------------------------------------------- the five workloads
def _report(name, case, errs):
    """Append one workload's errors to the file named by MLA_PARITY_REPORT
    (a summary of how far inside the gates each workload sits)."""
    path = os.environ.get("MLA_PARITY_REPORT")
    if not path:
        return
    import json

    rec = {"workload": name, "batch": case.batch, "s_q": case.s_q, "h_q": case.h_q,
           "causal": bool(case.causal), "sum_seqlen": int(case.cache_seqlens.sum()),
           "out_max_abs_err": errs[0], "out_normwise_rel_err": errs[1],
           "lse_max_abs_err": errs[2], "gates": {"out_atol": OUT_ATOL, "out_rtol": OUT_RTOL,
                                                 "out_norm_rtol": OUT_NORM_RTOL,
                                                 "lse_atol": LSE_ATOL}}
    with open(path, "a") as fh:
        fh.write(json.dumps(rec) + "\n")


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_config_full_parity(mla, k):
    """Every row of every sequence of the five workloads against the oracle,
    with unused pool pages and the tail slots of every last page poisoned
    with NaN (the kernels must never read them)."""
    _say(f"[parity] workload {k}: full oracle")
    case = make_config_case(k, poison_unused=True, poison_tail=True)
    out, lse = run(mla, case)
    ref_out, ref_lse = oracle.decode_ref(case)
    errs = compare(out, lse, ref_out, ref_lse)
    _say(f"[parity] workload {k}: max|err| {errs[0]:.2e} norm {errs[1]:.2e} lse {errs[2]:.2e}")
    _report(k, case, errs)


def test_batch_at_the_limit(mla):
    """65536 sequences (the batch limit), one query row each: one in 64 holds
    1 to 200 tokens, the rest are empty.  The chunked scheduler's largest
    case; the empty rows must come out as 0 / -inf, sampled live ones
    against the oracle."""
    _say("[parity] 65536 sequences")
    batch = 65536
    rng = np.random.Generator(np.random.PCG64(91))
    L = np.zeros(batch, dtype=np.int64)
    live = np.arange(0, batch, 64) + rng.integers(0, 64, batch // 64)
    L[live] = rng.integers(1, 201, live.size)
    case = make_case([int(x) for x in L], 1, 1, False, seed=92, pool_factor=1.1,
                     poison_unused=True, poison_tail=True)
    out, lse = run(mla, case)
    empty = L == 0
    assert np.all(np.isneginf(lse[empty])) and np.all(out[empty] == 0.0)
    assert np.all(np.isfinite(lse[~empty]))
    pick = sorted(set([int(live[0]), int(live[-1])] + [int(x) for x in rng.choice(live, 30)]))
    ref_out, ref_lse = oracle.decode_ref(case, batches=pick)
    errs = compare(out, lse, ref_out, ref_lse, batches=pick)
    _say(f"[parity] 65536 sequences, {len(pick)} sampled: {errs}")


# ---------------------------------------------------------------- query chunks
@pytest.mark.parametrize("L,s_q,h_q,causal,num_cus", [
    ([500, 70], 3, 683, False, 0),            # 2049 rows: 33 row groups, 7 partitions
    ([64, 1000, 2100], 32, 128, True, 0),     # 4096 rows: 4 partitions
    ([200, 1500], 128, 128, True, 0),         # 16384 rows: one partition, no combine
    ([300, 90, 1200], 16, 128, True, 5),      # 2048 rows on 5 CUs: one partition
])
def test_query_chunk_parity(mla, L, s_q, h_q, causal, num_cus):
    """Thousands of query rows per sequence (a chunk of new tokens at every
    head), the same decode: fewer partitions than XCDs, one partition (no
    split, nothing to combine), full oracle."""
    _say(f"[parity] chunk L={L} s_q={s_q} h_q={h_q} causal={causal} num_cus={num_cus}")
    case = make_case(L, s_q, h_q, causal, seed=81 + s_q, pool_factor=1.25,
                     poison_unused=True, poison_tail=True)
    out, lse = run(mla, case, num_cus)
    ref_out, ref_lse = oracle.decode_ref(case)
    errs = compare(out, lse, ref_out, ref_lse)
    _say(f"[parity] chunk: max|err| {errs[0]:.2e} norm {errs[1]:.2e} lse {errs[2]:.2e}")


def test_query_chunk_at_the_row_limit(mla):
    """65536 rows (512 query tokens x 128 heads, causal, 1024 row groups):
    sampled rows against the oracle, one by one."""
    _say("[parity] chunk of 512 tokens x 128 heads, sampled rows")
    case = make_case([1024, 700], 512, 128, True, seed=83, pool_factor=1.25,
                     poison_unused=True, poison_tail=True)
    out, lse = run(mla, case)
    rng = np.random.Generator(np.random.PCG64(84))
    rows = [(0, 0, 0), (0, 511, 127), (1, 0, 5), (1, 511, 0), (0, 255, 64), (1, 300, 127)]
    rows += [(int(b), int(i), int(h)) for b, i, h in zip(rng.integers(0, 2, 30),
                                                          rng.integers(0, 512, 30),
                                                          rng.integers(0, 128, 30))]
    ref = oracle.decode_ref_rows(case, rows)
    got_o = np.stack([out[b, i, h] for b, i, h in rows])
    got_l = np.array([lse[b, i, h] for b, i, h in rows])
    ref_o = np.stack([r[0] for r in ref])
    ref_l = np.array([r[1] for r in ref])
    errs = compare(got_o[None], got_l[None], ref_o[None], ref_l[None])
    _say(f"[parity] chunk at the limit: {errs}")


# ---------------------------------------------------------------- edge cases
EDGE_L = [1, 63, 64, 65, 127, 128, 4097]


@pytest.mark.parametrize("h_q", [1, 16, 64, 128])
@pytest.mark.parametrize("s_q,causal", [(1, False), (2, True), (2, False)])
def test_edge_lengths(mla, h_q, s_q, causal):
    _say(f"[parity] edge lengths h_q={h_q} s_q={s_q} causal={causal}")
    case = make_case(EDGE_L, s_q, h_q, causal, seed=17 + h_q, pool_factor=1.25,
                     poison_unused=True, poison_tail=True)
    out, lse = run(mla, case)
    ref_out, ref_lse = oracle.decode_ref(case)
    compare(out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("s_q,h_q,causal", [(1, 8, False), (1, 20, False), (5, 7, True),
                                             (3, 40, True), (8, 16, True), (4, 128, True),
                                             (16, 128, True)])
def test_row_shapes(mla, s_q, h_q, causal):
    """Row counts R = s_q * h_q that are not multiples of 16 (partial row tiles
    in every kernel variant), several row groups, and 2048 rows (32 row
    groups of 64, the most that still leaves 8 partitions on 256 CUs)."""
    _say(f"[parity] rows s_q={s_q} h_q={h_q} causal={causal}")
    case = make_case([1, 100, 700, 65, 0, 130], s_q, h_q, causal, seed=31 + s_q * h_q,
                     pool_factor=1.25, poison_unused=True, poison_tail=True)
    out, lse = run(mla, case)
    ref_out, ref_lse = oracle.decode_ref(case)
    compare(out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("h_q", [16, 64])
def test_many_short_sequences(mla, h_q):
    """1100 short sequences: the chunked scheduler path, many sequences per
    partition, and both combine kernels; sampled against the oracle."""
    _say(f"[parity] 1100 short sequences h_q={h_q}")
    rng = np.random.Generator(np.random.PCG64(97 + h_q))
    L = [int(x) for x in rng.integers(0, 300, size=1100)]
    L[5] = 0
    L[17] = 4000
    case = make_case(L, 1, h_q, False, seed=37 + h_q, pool_factor=1.1,
                     poison_unused=True, poison_tail=True)
    out, lse = run(mla, case)
    pick = sorted({0, 5, 17, 511, 512, 1023, 1024, 1099} | {int(x) for x in rng.integers(0, 1100, 12)})
    ref_out, ref_lse = oracle.decode_ref(case, batches=pick)
    compare(out, lse, ref_out, ref_lse, batches=pick)


@pytest.mark.parametrize("short", [0, 519])
def test_combine_beyond_128_splits(mla, short):
    """One 300-page sequence cut at every page (4096 partitions): its rows
    merge more than 128 partials, so the combine reads split weights from
    three places (lanes t, t + 64, and memory past 128).  Alone it takes the
    wide combine; behind 519 one-token sequences (partitions below eight per
    sequence) the one-wave-per-row combine."""
    _say(f"[parity] 300-way split behind {short} short sequences")
    L = [64 * 300 - 5] + [1] * short
    case = make_case(L, 1, 16, False, seed=61 + short, pool_factor=1.1,
                     poison_unused=True, poison_tail=True)
    parts = mla.num_partitions(1, 16, 4096)
    splits = schedule(L, parts, 1)[1]  # 16 rows: one page unit of fixed cost
    assert parts == 4096 and splits[1] - splits[0] > 128
    assert (parts >= 8 * len(L)) == (short == 0)  # which combine runs
    out, lse = run(mla, case, num_cus=4096)
    pick = [0, 1, short] if short else [0]
    ref_out, ref_lse = oracle.decode_ref(case, batches=pick)
    compare(out, lse, ref_out, ref_lse, batches=pick)


@pytest.mark.parametrize("num_cus", [1, 3, 64, 256, 1024, 4096, 5000])
def test_forced_partition_counts(mla, num_cus):
    _say(f"[parity] num_cus={num_cus}")
    case = make_case([1, 200, 4097, 65, 0, 3000], 2, 16, True, seed=23, pool_factor=1.25,
                     poison_unused=True, poison_tail=True)
    out, lse = run(mla, case, num_cus=num_cus)
    ref_out, ref_lse = oracle.decode_ref(case)
    compare(out, lse, ref_out, ref_lse)


def _both_schedules(mla, case, num_cus=0):
    q, kv, bt, sl = to_dev(case)
    res = {}
    for sched in ("separate", "in_decode"):
        meta, splits = None, None
        if sched == "separate":
            meta, splits = mla.get_metadata(sl, case.s_q, case.h_q, num_cus)
        else:
            splits = torch.full((case.batch + 1,), -7, dtype=torch.int32, device="cuda:0")
        out, lse, ws = mla.decode_paged(q, kv, bt, sl, case.softmax_scale, case.causal, meta,
                                        splits, num_cus)
        mla.combine(ws, splits, case.batch, case.s_q, case.h_q, out, lse, num_cus)
        torch.cuda.synchronize()
        res[sched] = (out.view(torch.int16).cpu().numpy(), lse.cpu().numpy(), splits.cpu().numpy())
    return res


@pytest.mark.parametrize("L,s_q,h_q,num_cus", [
    ([256], 1, 16, 0),
    (EDGE_L, 1, 16, 0),
    (EDGE_L, 2, 8, 3),
    ([1, 200, 4097, 65, 0, 3000], 2, 8, 64),
    ([0, 0, 0], 1, 1, 256),
    ([5000] * 3, 1, 16, 1024),
    (EDGE_L, 2, 16, 0),                        # 32 rows: the 4-wave 32-row kernel
    (EDGE_L, 1, 64, 0),                        # 64 rows: the 64-row kernel
    ([1, 200, 4097, 65, 0, 3000], 1, 64, 7),   # 64 rows, 7 partitions
    ([700, 0, 2100, 64], 2, 128, 0),           # 4 row groups x 64 partitions
    ([300, 1200], 32, 128, 0),                 # 64 row groups, 4 partitions
    ([900, 65], 3, 40, 1),                     # 120 rows, one partition
    ([4096] * 16, 1, 16, 0),                   # 16 full rows of a 64-entry block table
    ([4097] + [4096] * 15, 1, 16, 0),          # one longer row: 65 entries each
    ([40000, 3000, 9000], 1, 64, 0),           # 64-row kernel, long rows
])
def test_schedule_in_decode_matches_separate(mla, L, s_q, h_q, num_cus):
    """The decode that schedules itself cuts the key range exactly as the
    separate scheduler does: the same split counts and bit-identical output."""
    _say(f"[parity] in-decode schedule L={L[:4]} s_q={s_q} h_q={h_q} num_cus={num_cus}")
    case = make_case(L, s_q, h_q, s_q > 1, seed=71 + len(L), pool_factor=1.25,
                     poison_unused=True, poison_tail=True)
    r = _both_schedules(mla, case, num_cus)
    assert np.array_equal(r["separate"][2], r["in_decode"][2]), "num_splits"
    assert np.array_equal(r["separate"][0], r["in_decode"][0]), "out bits"
    assert np.array_equal(r["separate"][1], r["in_decode"][1]), "lse"


def test_schedule_in_decode_batch_limits(mla):
    """1024 sequences schedule in the decode; 1025 need the separate one."""
    _say("[parity] in-decode schedule at 1024 sequences")
    rng = np.random.Generator(np.random.PCG64(73))
    L = [int(x) for x in rng.integers(0, 200, size=1024)]
    case = make_case(L, 1, 16, False, seed=74, pool_factor=1.1)
    r = _both_schedules(mla, case)
    assert np.array_equal(r["separate"][2], r["in_decode"][2])
    assert np.array_equal(r["separate"][0], r["in_decode"][0])
    q, kv, bt, sl = to_dev(make_case(L + [3], 1, 16, False, seed=75, pool_factor=1.1))
    with pytest.raises(mla.MlaError):
        mla.mla_decode(q, kv, bt, sl, 0.07, False, schedule="in_decode")


def test_empty_and_single_token(mla):
    _say("[parity] empty / single-token sequences")
    case = make_case([0, 1, 0, 2], 1, 16, False, seed=29)
    out, lse = run(mla, case)
    ref_out, ref_lse = oracle.decode_ref(case)
    compare(out, lse, ref_out, ref_lse)
    assert np.all(np.isneginf(lse[0])) and np.all(out[0] == 0)


def test_fully_masked_split_partials(mla):
    """s_q = 2 causal with L = 64k + 1: a split holding only the last token is
    empty for query 0 (lse_s = -inf) and must carry no weight."""
    _say("[parity] masked partials")
    case = make_case([64 * 40 + 1, 64 * 7 + 1], 2, 64, True, seed=31)
    for num_cus in (64, 256, 1024):
        out, lse = run(mla, case, num_cus=num_cus)
        ref_out, ref_lse = oracle.decode_ref(case)
        compare(out, lse, ref_out, ref_lse)


# ---------------------------------------------------------------- properties
def test_value_all_ones_probe(mla):
    _say("[parity] V == 1 probe")
    case = make_case([700, 64, 3], 2, 16, True, seed=37)
    case.kv[:, :, :512] = np.uint16(0x3F80)
    out, lse = run(mla, case)
    assert np.max(np.abs(out - 1.0)) <= OUT_ATOL + OUT_RTOL


def test_deterministic_and_page_permutation_invariant(mla):
    _say("[parity] determinism and page permutation")
    case = make_case([3000, 129, 64], 1, 64, False, seed=41, pool_factor=1.25)
    a = run(mla, case)
    b = run(mla, case)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = run(mla, permute_pool(case, seed=5))
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


@pytest.mark.parametrize("s_q,h_q,num_cus", [(1, 16, 0), (2, 128, 0), (1, 64, 3), (1, 16, 1024)])
def test_device_schedule_matches_model(mla, s_q, h_q, num_cus):
    _say(f"[sched] s_q={s_q} h_q={h_q} num_cus={num_cus}")
    rng = np.random.Generator(np.random.PCG64(43))
    L = list(rng.integers(0, 20000, size=37)) + [131072, 0, 1, 64]
    _check_schedule(mla, L, s_q, h_q, num_cus)


@pytest.mark.gpu
@pytest.mark.parametrize("batch", [1, 64, 65, 200, 256, 257, 700, 1024, 1025, 1500])
def test_device_schedule_batch_sizes(mla, batch):
    """Every scheduler path (one workgroup of 64, 256 or 1024 threads, and the
    chunked path past 1024 sequences) against the model."""
    _say(f"[sched] batch={batch}")
    rng = np.random.Generator(np.random.PCG64(1000 + batch))
    L = [int(x) for x in rng.integers(0, 9000, size=batch)]
    L[0] = 0
    for num_cus in (0, 7, 1024):
        _check_schedule(mla, L, 1, 16, num_cus)
        _check_schedule(mla, L, 2, 128, num_cus)


@pytest.mark.gpu
@pytest.mark.parametrize("batch", [3, 100, 600])
def test_device_schedule_huge_lengths(mla, batch):
    """A sequence of 2^26+ tokens (2^20 page units) takes the 64-bit
    arithmetic of the small-batch scheduler; only the schedule is computed."""
    _say(f"[sched] huge lengths, batch={batch}")
    rng = np.random.Generator(np.random.PCG64(7 + batch))
    L = [int(x) for x in rng.integers(0, 5000, size=batch)]
    L[batch // 2] = 70_000_000
    L[-1] = 2**26 + 5
    for num_cus in (0, 13):
        _check_schedule(mla, L, 1, 64, num_cus)


def _check_schedule(mla, L, s_q, h_q, num_cus):
    sl = torch.tensor(L, dtype=torch.int32, device="cuda:0")
    meta, splits = mla.get_metadata(sl, s_q, h_q, num_cus)
    torch.cuda.synchronize()
    meta = meta.cpu().numpy()
    splits = splits.cpu().numpy()
    parts = meta.shape[0]
    c0 = int(meta[0, 6])
    ref_meta, ref_splits, _ = schedule(L, parts, c0)
    assert np.array_equal(meta, np.array(ref_meta, dtype=np.int32))
    assert np.array_equal(splits, np.array(ref_splits, dtype=np.int32))


def test_error_codes(mla):
    q = torch.zeros((2, 1, 16, 576), dtype=torch.bfloat16, device="cuda:0")
    kv = torch.zeros((4, 64, 576), dtype=torch.bfloat16, device="cuda:0")
    bt = torch.zeros((2, 2), dtype=torch.int32, device="cuda:0")
    sl = torch.full((2,), 64, dtype=torch.int32, device="cuda:0")
    meta, splits = mla.get_metadata(sl, 1, 16)
    with pytest.raises(mla.MlaError):
        mla.decode_paged(q, kv, bt, sl, float("inf"), False, meta, splits)
    with pytest.raises(mla.MlaError):
        mla.decode_paged(q, kv, bt, sl, 0.0, False, meta, splits)
    small = torch.empty((64,), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(mla.MlaError) as e:
        mla.decode_paged(q, kv, bt, sl, 0.1, False, meta, splits, workspace=small)
    assert e.value.status == 3
    with pytest.raises(TypeError):
        mla.decode_paged(q.float(), kv, bt, sl, 0.1, False, meta, splits)


# ---------------------------------------------------------------- HIP graphs
def _graph_replays_match(mla, case, step, replays=3):
    """Capture `step` (which writes fresh outputs it returns) in a HIP graph,
    replay it several times with eager work and host synchronisation in
    between, and compare every replay with the eager result bit for bit."""
    out0, lse0 = step()
    torch.cuda.synchronize()
    ref_o = out0.view(torch.int16).clone()
    ref_l = lse0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out_g, lse_g = step()
    torch.cuda.synchronize()
    for r in range(replays):
        step()  # eager work between replays (the same step, launched eagerly)
        torch.cuda.synchronize()
        out_g.fill_(-3.0)  # only the replay can restore the outputs
        lse_g.fill_(-3.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), ref_o), f"out, replay {r}"
        assert torch.equal(lse_g, ref_l), f"lse, replay {r}"


@pytest.mark.parametrize("L,s_q,h_q", [([3000, 129, 64, 0, 700], 1, 16), ([5000, 70, 2100], 2, 128),
                                       ([40] * 1100, 1, 16)])
def test_graph_replays_equal_eager(mla, L, s_q, h_q):
    """Whole decode steps (schedule, decode, combine) captured in a HIP graph
    give the eager bits on every replay: no memset nodes, nothing left over
    between replays."""
    _say(f"[graph] L={L[:3]} s_q={s_q} h_q={h_q}")
    case = make_case(L, s_q, h_q, s_q > 1, seed=211 + h_q, pool_factor=1.25, poison_unused=True,
                     poison_tail=True)
    q, kv, bt, sl = to_dev(case)
    b = case.batch
    out = torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device="cuda:0")
    fused = mla.prefers_in_decode(b, s_q, h_q, case.max_pages)
    ws = torch.empty((mla.workspace_bytes(b, s_q, h_q),), dtype=torch.uint8, device="cuda:0")
    splits = torch.empty((b + 1,), dtype=torch.int32, device="cuda:0")
    meta = torch.empty((mla.num_partitions(s_q, h_q), mla.META_INTS), dtype=torch.int32,
                       device="cuda:0")
    lib = mla.load_library()

    def step():
        st = torch.cuda.current_stream()
        if not fused:
            mla._check("mla_get_metadata", lib.mla_get_metadata(
                mla._ptr(sl), b, s_q, h_q, 0, mla._ptr(meta), mla._ptr(splits), mla._stream(st)))
        mla.decode_paged(q, kv, bt, sl, case.softmax_scale, case.causal,
                         None if fused else meta, splits, workspace=ws, out=out, lse=lse,
                         stream=st)
        mla.combine(ws, splits, b, s_q, h_q, out, lse, stream=st)
        return out, lse

    _graph_replays_match(mla, case, step)
    o, l = out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()
    ref_out, ref_lse = oracle.decode_ref(case, batches=[0, 1])
    compare(oracle.bf16_to_f64(o), l.astype(np.float64), ref_out, ref_lse, batches=[0, 1])


def _random_cases(n, seed):
    """Small random decode batches the oracle finishes quickly: lengths 0..400
    (empty, single-token, page-edge and ragged), 1..3 query tokens, head
    counts on both sides of every kernel's row limit, causal or not, and a
    partition count from one to a few hundred."""
    rng = np.random.Generator(np.random.PCG64(seed))
    edges = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129]
    out = []
    for i in range(n):
        batch = int(rng.integers(1, 7))
        L = [int(rng.choice(edges)) if rng.random() < 0.4 else int(rng.integers(0, 401))
             for _ in range(batch)]
        s_q = int(rng.integers(1, 4))
        h_q = int(rng.choice([1, 3, 8, 16, 20, 32, 48, 64, 128]))
        causal = bool(rng.random() < 0.5)
        num_cus = int(rng.choice([1, 3, 16, 77, 256, 300]))
        out.append((L, s_q, h_q, causal, num_cus, seed * 100 + i))
    return out


@pytest.mark.parametrize("L,s_q,h_q,causal,num_cus,seed", _random_cases(24, 9001))
def test_random_small_cases(mla, L, s_q, h_q, causal, num_cus, seed):
    _say(f"[random] L={L} s_q={s_q} h_q={h_q} causal={causal} num_cus={num_cus} seed={seed}")
    case = make_case(L, s_q, h_q, causal, seed=seed, pool_factor=1.5, poison_unused=True,
                     poison_tail=True)
    out, lse = run(mla, case, num_cus=num_cus)
    ref_out, ref_lse = oracle.decode_ref(case)
    compare(out, lse, ref_out, ref_lse)
