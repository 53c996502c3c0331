"""GPU parity of the FP8 latent cache through the C ABI.

Quantization: every live token's 656-byte record bit for bit against the
oracle (codes, power-of-two scales, rotary bytes).  Decode over the FP8
cache: against the oracle's decode over its own dequantized cache, at the
decode's tolerances (the dequantized values are exact bf16 values, so this
is the same bar as the bf16 decode).  The GPU decode reads the cache the GPU
quantized; the oracle quantizes the same bf16 input on its own.
"""

import dataclasses
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import bf16_bits_from_f32, make_case, make_config_case  # noqa: E402

F = oracle.fp8_cache
OUT_ATOL, OUT_RTOL, OUT_NORM_RTOL, LSE_ATOL = 1e-2, 2e-2, 2e-2, 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import mla_paged_kv_06_amd as m
    m.load_library()
    return m


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(
        torch.bfloat16)


def _live_tokens(case):
    """(page, slot) of every token some sequence holds."""
    out = []
    for b in range(case.batch):
        L = int(case.cache_seqlens[b])
        for t in range(L):
            out.append((int(case.block_table[b, t // 64]), t % 64))
    return out


def _oracle_dequantized_case(case):
    """The same case over the oracle's own quantize -> dequantize of its cache."""
    return dataclasses.replace(case, kv=F.dequantize_cache_bf16_bits(F.quantize_cache(case.kv)))


def _compare(out, lse, ref_out, ref_lse):
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty)
    assert np.all(out[empty] == 0.0)
    live = ~empty
    if not np.any(live):
        return
    err = np.abs(out - ref_out)
    assert float((err - (OUT_ATOL + OUT_RTOL * np.abs(ref_out))).max()) <= 0.0
    nrm = np.linalg.norm(out[live] - ref_out[live]) / max(np.linalg.norm(ref_out[live]), 1e-30)
    assert nrm <= OUT_NORM_RTOL, nrm
    assert float(np.abs(lse[live] - ref_lse[live]).max()) <= LSE_ATOL
    return float(err.max()), float(nrm)


def test_quantize_bit_exact_on_live_tokens(mla):
    _say("[fp8] quantize: live tokens bit for bit")
    case = make_case([1, 63, 64, 65, 700, 0, 4097], 1, 16, False, seed=201, pool_factor=1.25,
                     poison_unused=True, poison_tail=True)
    got = mla.kv_quantize_fp8(_dev_bf16(case.kv)).cpu().numpy()
    want = F.quantize_cache(case.kv)
    live = _live_tokens(case)
    g = np.stack([got[p, s] for p, s in live])
    w = np.stack([want[p, s] for p, s in live])
    assert np.array_equal(g, w)


def test_quantize_bit_exact_on_edge_blocks(mla):
    """All-zero blocks, a lone large value, tiny values, signed zeros, exact
    E4M3 ties and values on the 448 * 2^e boundary."""
    _say("[fp8] quantize: edge blocks")
    rng = np.random.Generator(np.random.PCG64(202))
    x = rng.standard_normal((2, 64, 576)).astype(np.float32)
    x[0, 0, :128] = 0.0                                 # zero block
    x[0, 1, :128] = 0.0
    x[0, 1, 7] = -3.0e4                                 # lone large value
    x[0, 2, 128:256] *= 1e-30                           # tiny block (scale 2^-1xx)
    x[0, 3, 256:384] = -0.0                             # negative zeros
    x[0, 4, :128] = 448.0 * 2.0 ** -3                   # exactly on the boundary
    x[0, 5, :8] = [1.0625, 1.1875, 3.0, -0.5, 2.0 ** -20, 7.0, 448.0 * 2.0 ** -7, 0.0]
    x[0, 5, 8:128] = 0.0                                # so that amax = 7, e = -6: ties at scale
    x[1] *= (10.0 ** rng.uniform(-4, 4, (64, 1))).astype(np.float32)
    bits = bf16_bits_from_f32(x)
    got = mla.kv_quantize_fp8(_dev_bf16(bits)).cpu().numpy()
    want = F.quantize_cache(bits)
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"first mismatches {mism[:5]}"


@pytest.mark.parametrize("lengths,s_q,h_q,causal,num_cus", [
    ([1, 63, 64, 65, 127, 128, 4097], 1, 16, False, 0),
    ([1, 63, 64, 65, 127, 128, 4097], 2, 8, True, 0),
    ([300, 0, 2000, 64], 1, 1, False, 5),
    ([1, 200, 4097, 65, 0, 3000], 2, 8, True, 1024),
])
def test_decode_fp8_parity(mla, lengths, s_q, h_q, causal, num_cus):
    _say(f"[fp8] decode L={lengths[:4]} s_q={s_q} h_q={h_q} causal={causal} num_cus={num_cus}")
    case = make_case(lengths, s_q, h_q, causal, seed=203 + h_q, pool_factor=1.25,
                     poison_unused=True, poison_tail=True)
    kv8 = mla.kv_quantize_fp8(_dev_bf16(case.kv))
    q = _dev_bf16(case.q)
    bt = torch.from_numpy(case.block_table).to("cuda:0")
    sl = torch.from_numpy(case.cache_seqlens).to("cuda:0")
    out, lse = mla.mla_decode_fp8(q, kv8, bt, sl, case.softmax_scale, causal, num_cus=num_cus)
    torch.cuda.synchronize()
    o = oracle.bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    l = lse.cpu().numpy().astype(np.float64)
    ref_out, ref_lse = oracle.decode_ref(_oracle_dequantized_case(case))
    _say(f"[fp8] decode errors {_compare(o, l, ref_out, ref_lse)}")


def test_decode_fp8_memory_bound_workload(mla):
    """The memory-bound workload's shape (8 sequences of 1024 to 4096 tokens,
    16 heads), whole, against the oracle over the dequantized cache."""
    _say("[fp8] decode, memory-bound workload")
    case = make_config_case(2, poison_unused=True, poison_tail=True)
    kv8 = mla.kv_quantize_fp8(_dev_bf16(case.kv))
    q = _dev_bf16(case.q)
    bt = torch.from_numpy(case.block_table).to("cuda:0")
    sl = torch.from_numpy(case.cache_seqlens).to("cuda:0")
    out, lse = mla.mla_decode_fp8(q, kv8, bt, sl, case.softmax_scale, case.causal)
    torch.cuda.synchronize()
    o = oracle.bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    l = lse.cpu().numpy().astype(np.float64)
    ref_out, ref_lse = oracle.decode_ref(_oracle_dequantized_case(case))
    _say(f"[fp8] workload 2 errors {_compare(o, l, ref_out, ref_lse)}")
    # and the FP8 step stays close to the bf16 one on the original cache
    # (quantization error only; a loose sanity bound, not a parity gate)
    ref16, _ = oracle.decode_ref(case)
    nrm = np.linalg.norm(o - ref16) / np.linalg.norm(ref16)
    _say(f"[fp8] normwise distance to the bf16-cache result {nrm:.3e}")
    assert nrm < 0.1


def test_fp8_shapes_outside_the_kernel_raise(mla):
    case = make_case([100], 2, 16, True, seed=204)
    kv8 = mla.kv_quantize_fp8(_dev_bf16(case.kv))
    q = _dev_bf16(case.q)
    bt = torch.from_numpy(case.block_table).to("cuda:0")
    sl = torch.from_numpy(case.cache_seqlens).to("cuda:0")
    with pytest.raises(mla.MlaError):
        mla.mla_decode_fp8(q, kv8, bt, sl, case.softmax_scale, True)  # 32 rows
