"""Steps of the library captured in HIP graphs (torch.cuda.graph) replay bit
for bit like the same calls made eagerly: single-tensor top-k with block
encoding, layer-wise top-k calls over 12 and 60 tensors (whose plans go in
kernel-argument chunks under capture), sign compression, random
sparsification, the 1-bit Adam update and the one-pass decode + SGD.
Every call launches kernels only (no memset or host-staged copies for these
shapes), so capture records the whole step.  Each replay is followed by some
eager work and a synchronisation before it is checked."""
import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
from gpu_util import device

pytestmark = pytest.mark.gpu

T = 5


def bits_equal(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def run_chain(step_of, state, outputs, dev):
    """Runs T steps eagerly from a copy of `state`, then captures one graph per
    step on the live state and replays them in order; returns True when every
    replay's outputs and state equal the eager ones.  `outputs()` returns the
    defined parts of the output buffers (a packet's length is read back)."""
    eager_state = [s.clone() for s in state]
    ref = []
    for t in range(T):
        step_of(t, eager_state)
        torch.cuda.synchronize()
        ref.append([o.clone() for o in outputs()] + [s.clone() for s in eager_state])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on scratch state, off the chain
        step_of(0, [s.clone() for s in state])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for t in range(T):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_of(t, state)
        graphs.append(g)
    torch.cuda.synchronize()
    ok = True
    for t in range(T):
        graphs[t].replay()
        torch.cuda.synchronize()
        got = outputs() + [s for s in state]
        float(sum(o.float().sum() for o in got))  # eager work between replays
        ok &= all(bits_equal(a, b) for a, b in zip(got, ref[t]))
    return ok


def test_topk_and_blocks_in_a_graph():
    dev = device()
    n, k = 300_007, 3000
    grads = [torch.from_numpy(gen.large_gradient(t, n=n)).to(dev) for t in range(T)]
    ws = efg.workspace(efg.ef_topk_workspace_bytes(n, k), dev)
    vals = torch.empty(k, device=dev)
    idx = torch.empty(k, dtype=torch.int32, device=dev)
    nb = (n + 255) // 256
    mask = torch.empty((nb + 7) // 8, dtype=torch.uint8, device=dev)
    counts = torch.empty(min(k, nb), dtype=torch.uint8, device=dev)
    offs = torch.empty(k, dtype=torch.uint8, device=dev)
    nblk = torch.empty(1, dtype=torch.int64, device=dev)
    wsb = efg.workspace(efg.lib().blocks_workspace_bytes(k, n), dev)

    def step(t, st):
        efg.ef_topk_compress(grads[t], st[0], k, vals=vals, idx=idx, ws=ws)
        efg.encode_blocks(idx, n, mask=mask, counts_m1=counts, offs=offs, nblk_out=nblk, ws=wsb)

    state = [torch.zeros(n, device=dev)]
    assert run_chain(step, state, lambda: [vals, idx, mask, counts[:int(nblk.item())], offs, nblk], dev)


@pytest.mark.parametrize("layout", ["12 tensors", "60 tensors"])
def test_layerwise_topk_in_a_graph(layout):
    """Plans of 512 words and of about 2,700 words (six kernel-argument chunks
    under capture)."""
    dev = device()
    if layout == "12 tensors":
        sizes = [768, 3072, 100_003, 768, 250_000, 4096, 77, 590_000, 768, 3072, 200_001, 33]
    else:
        sizes = [int(m) for m in gen.rng(141).integers(1, 60_000, size=60)]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    ks = np.array([max(1, m // 100) for m in sizes], np.int64)
    n, K = int(off[-1]), int(ks.sum())
    grads = [torch.from_numpy(gen.normal_small(n, 140, t)).to(dev) for t in range(T)]
    ws = efg.workspace(efg.ef_topk_segmented_workspace_bytes(off, ks), dev)
    vals = torch.empty(K, device=dev)
    idx = torch.empty(K, dtype=torch.int32, device=dev)

    def step(t, st):
        efg.ef_topk_compress_segmented(grads[t], st[0], off, ks, vals=vals, idx=idx, ws=ws)

    assert run_chain(step, [torch.zeros(n, device=dev)], lambda: [vals, idx], dev)


def test_sign_random_and_onebit_in_graphs():
    dev = device()
    n = 200_003
    gs = [torch.from_numpy(gen.sign_gradient(t, n=n)).to(dev) for t in range(T)]
    sgn = torch.empty(n, dtype=torch.int8, device=dev)
    bits = torch.empty((n + 7) // 8, dtype=torch.uint8, device=dev)
    assert run_chain(lambda t, st: efg.ef_sign_compress(gs[t], st[0], st[1], 0.9, 5.0, sign_out=sgn, bits=bits),
                     [torch.zeros(n, device=dev), torch.zeros(n, device=dev)], lambda: [sgn, bits], dev)

    k = 2000
    cap = 2 * k + 64
    rv = torch.empty(cap, device=dev)
    ri = torch.empty(cap, dtype=torch.int32, device=dev)
    rc = torch.empty(1, dtype=torch.int64, device=dev)
    wsr = efg.workspace(efg.lib().ef_random_sparsify_workspace_bytes(n), dev)
    lg = [torch.from_numpy(gen.large_gradient(10 + t, n=n)).to(dev) for t in range(T)]
    assert run_chain(lambda t, st: efg.ef_random_sparsify(lg[t], st[0], k, 7, t, cap=cap, vals=rv, idx=ri, count=rc,
                                                          ws=wsr),
                     [torch.zeros(n, device=dev)],
                     lambda: [rv[:min(cap, int(rc.item()))], ri[:min(cap, int(rc.item()))], rc], dev)

    v = torch.from_numpy(np.abs(gen.normal_small(n, 811, scale=1e-3))).to(dev)
    ss, sb = efg.adam_scalars(1e-3, 0.9, 0.999, 10, 3)

    def onebit(t, st):
        efg.ef_sign_compress(gs[t], st[0], None, 0.9, 5.0, sign_out=sgn, want_bits=False)
        efg.ef_onebit_adam_update(sgn, 1, st[1], v, st[2], 0.9, ss, sb, 1e-8)

    assert run_chain(onebit, [torch.zeros(n, device=dev), torch.zeros(n, device=dev),
                              torch.from_numpy(gen.normal_small(n, 812)).to(dev)], lambda: [sgn], dev)


def test_decode_sgd_in_a_graph():
    """The one-pass receiver step (sparse_decode_sgd) with its invalid-entry
    count: the weights carry from step to step, G and the count are outputs."""
    dev = device()
    n, P, kp = 300_007, 6, 3000
    r = gen.rng(150)
    idx = np.concatenate([np.sort(r.choice(n, size=kp, replace=False)) for _ in range(P)]).astype(np.int32)
    vals = [torch.from_numpy(gen.normal_small(P * kp, 151, t)).to(dev) for t in range(T)]
    idd = torch.from_numpy(idx).to(dev)
    off = torch.arange(0, (P + 1) * kp, kp, dtype=torch.int64, device=dev)
    G = torch.empty(n, device=dev)
    inv = torch.empty(1, dtype=torch.int32, device=dev)

    def step(t, st):
        efg.sparse_decode_sgd(st[0], vals[t], idd, off, 0.1, G=G, invalid=inv)

    assert run_chain(step, [torch.from_numpy(gen.normal_small(n, 152)).to(dev)], lambda: [G, inv], dev)
