"""GPU parity of the 8-bit packet quantisation against the CPU oracle (bit for bit)."""
import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
import oracle
from gpu_util import assert_bits_equal, device, host, to_dev
from test_oracle_quant import _straddling_case

pytestmark = pytest.mark.gpu


def gpu_quant(vals, idx, e):
    dev = device()
    ed = to_dev(e, dev)
    q, sc = efg.ef_quantize_int8(to_dev(vals, dev), to_dev(idx, dev), ed)
    return host(q), float(host(sc)[0]), host(ed)


def check(vals, idx, e, what):
    q, sc, e2 = gpu_quant(vals, idx, e)
    oq, osc, oe = oracle.quantize_int8(vals, idx, e)
    assert_bits_equal(q, oq, f"q {what}")
    assert np.float32(sc).view(np.uint32) == np.float32(osc).view(np.uint32), (what, sc, osc)
    nan = np.isnan(e2) & np.isnan(oe)
    assert np.array_equal(np.isnan(e2), np.isnan(oe))
    assert_bits_equal(e2[~nan], oe[~nan], f"e {what}")


@pytest.mark.parametrize("k", [1, 2, 63, 256, 257, 5000, 300_001])
@pytest.mark.parametrize("kind", ["normal", "lognormal", "ties", "specials"])
def test_packets(k, kind):
    n = 4 * k + 7
    idx = gen.sorted_unique_indices(n, k, 400, k)
    v = {"normal": lambda: gen.normal_small(k, 401, k),
         "lognormal": lambda: gen.large_gradient(9, n=k),
         "ties": lambda: gen.uniform_ties(k, 7, 402, k),
         "specials": lambda: gen.specials(k, 403, k)}[kind]()
    check(v, idx, gen.normal_small(n, 404, k), f"{kind} k={k}")


def test_edge_cases():
    e = np.arange(8, dtype=np.float32)
    check(np.array([2.5e-38, 0.0, -2.5e-38, 1e-45], np.float32), np.array([0, 2, 5, 7], np.int32), e, "tiny amax")
    check(np.zeros(3, np.float32), np.array([1, 2, 3], np.int32), e, "zeros")
    check(np.array([np.nan, np.inf, -np.inf], np.float32), np.array([0, 1, 2], np.int32), e, "no finite value")
    amax, v = _straddling_case()
    check(np.array([amax, v], np.float32), np.array([3, 4], np.int32), e, "straddling")
    # out-of-range indices update nothing
    q, sc, e2 = gpu_quant(np.array([1.0, 2.0], np.float32), np.array([-1, 100], np.int32), e)
    assert np.array_equal(e2, e) and q.tolist() == [64, 127]


def test_empty_packet():
    dev = device()
    e = torch.ones(4, device=dev)
    q, sc = efg.ef_quantize_int8(torch.zeros(0, device=dev), torch.zeros(0, dtype=torch.int32, device=dev), e)
    assert float(host(sc)[0]) == 0.0 and host(e).tolist() == [1.0] * 4


def test_after_topk_chain():
    """top-k then 8-bit values over 5 chained steps, GPU against oracle end to end."""
    dev = device()
    n, k = 200_003, 2000
    ed = torch.zeros(n, device=dev)
    e_ref = np.zeros(n, np.float32)
    for t in range(5):
        g = gen.large_gradient(t, n=n)
        v, i = efg.ef_topk_compress(to_dev(g, dev), ed, k)
        q, sc = efg.ef_quantize_int8(v, i, ed)
        ov, oi, e_ref, _ = oracle.topk(g, e_ref, k)
        oq, osc, e_ref = oracle.quantize_int8(ov, oi, e_ref)
        assert_bits_equal(host(q), oq, f"q step {t}")
        assert_bits_equal(host(ed), e_ref, f"e step {t}")


def test_full_size_packet():
    """k = 1,300,000 values of the large workload's law at indices in [0, 1.3e9):
    the oracle runs on a compact copy of the residual (one slot per entry)."""
    dev = device()
    n, k = gen.LARGE_N, gen.LARGE_K
    idx = gen.sorted_unique_indices(n, k, 405)
    v = gen.large_gradient(11, n=k)
    ed = torch.zeros(n, device=dev)
    idd = to_dev(idx, dev)
    q, sc = efg.ef_quantize_int8(to_dev(v, dev), idd, ed)
    oq, osc, oe = oracle.quantize_int8(v, np.arange(k, dtype=np.int32), np.zeros(k, np.float32))
    assert_bits_equal(host(q), oq, "q full size")
    assert np.float32(float(host(sc)[0])) == np.float32(osc)
    assert_bits_equal(host(ed[idd.long()]), oe, "e full size")
