"""Checkpoint / resume: the whole carried state of a chain is the residual e
(top-k) or e and the momentum m (1-bit sign path), so a chain split at step
5, its state saved with torch.save, reloaded into fresh buffers and resumed
with a fresh workspace, gives every later packet and the final state bit for
bit as the unsplit chain does, and as the oracle's chain does.  The pages
list the error buffer (and the momentum) as state a worker must keep and
synchronise ("1bit Adam" page, section 3.1)."""
import numpy as np
import pytest
import torch

import error_feedback_gradient_amd as efg
import gen
import oracle
from gpu_util import assert_bits_equal, device, host

pytestmark = pytest.mark.gpu

SPLIT = 5


def topk_chain(steps, e, dev, k):
    ws = efg.workspace(efg.ef_topk_workspace_bytes(e.numel(), k), dev)
    out = []
    for t in steps:
        v, i = efg.ef_topk_compress(torch.from_numpy(gen.flat_gradient(t)).to(dev), e, k, ws=ws)
        out.append((host(v), host(i)))
    return out


def test_topk_chain_split_and_resumed(tmp_path):
    dev = device()
    n, k, T = gen.FLAT_N, gen.FLAT_K, gen.FLAT_STEPS
    e_full = torch.zeros(n, device=dev)
    full = topk_chain(range(T), e_full, dev, k)
    # first half, checkpoint, fresh process state, second half
    e = torch.zeros(n, device=dev)
    first = topk_chain(range(SPLIT), e, dev, k)
    path = tmp_path / "ef_state.pt"
    torch.save({"e": e.cpu(), "step": SPLIT}, path)
    del e
    torch.cuda.empty_cache()
    st = torch.load(path, weights_only=True)
    e2 = st["e"].to(dev)
    second = topk_chain(range(st["step"], T), e2, dev, k)
    for t, ((va, ia), (vb, ib)) in enumerate(zip(full, first + second)):
        assert_bits_equal(ib, ia, f"idx step {t}")
        assert_bits_equal(vb, va, f"vals step {t}")
    assert_bits_equal(host(e2), host(e_full), "final e")
    # the oracle's chain, split the same way through np.save / np.load
    e_ref = np.zeros(n, np.float32)
    for t in range(SPLIT):
        _, _, e_ref, _ = oracle.topk(gen.flat_gradient(t), e_ref, k)
    np.save(tmp_path / "e_ref.npy", e_ref)
    e_ref = np.load(tmp_path / "e_ref.npy")
    for t in range(SPLIT, T):
        ov, oi, e_ref, _ = oracle.topk(gen.flat_gradient(t), e_ref, k)
        assert_bits_equal(second[t - SPLIT][1], oi, f"idx vs oracle step {t}")
        assert_bits_equal(second[t - SPLIT][0], ov, f"vals vs oracle step {t}")
    assert_bits_equal(host(e2), e_ref, "final e vs oracle")


def sign_chain(steps, e, m, dev, n):
    out = []
    for t in steps:
        g = torch.from_numpy(gen.sign_gradient(t, n=n)).to(dev)
        s, b = efg.ef_sign_compress(g, e, m, gen.SIGN_BETA1, gen.SIGN_CLIP)
        out.append((host(s), host(b)))
    return out


def test_sign_chain_split_and_resumed(tmp_path):
    dev = device()
    n, T = 1_000_003, 10
    e_full, m_full = torch.zeros(n, device=dev), torch.zeros(n, device=dev)
    full = sign_chain(range(T), e_full, m_full, dev, n)
    e, m = torch.zeros(n, device=dev), torch.zeros(n, device=dev)
    first = sign_chain(range(SPLIT), e, m, dev, n)
    path = tmp_path / "sign_state.pt"
    torch.save({"e": e.cpu(), "m": m.cpu(), "step": SPLIT}, path)
    del e, m
    st = torch.load(path, weights_only=True)
    e2, m2 = st["e"].to(dev), st["m"].to(dev)
    second = sign_chain(range(st["step"], T), e2, m2, dev, n)
    for t, ((sa, ba), (sb, bb)) in enumerate(zip(full, first + second)):
        assert np.array_equal(sa, sb) and np.array_equal(ba, bb), f"sign / bits step {t}"
    assert_bits_equal(host(e2), host(e_full), "final e")
    assert_bits_equal(host(m2), host(m_full), "final m")
    z = np.zeros(n, np.float32)
    er, mr = z, z
    for t in range(T):
        er, mr, _, _, _ = oracle.sign(gen.sign_gradient(t, n=n), er, mr, gen.SIGN_BETA1, gen.SIGN_CLIP)
    assert_bits_equal(host(e2), er, "final e vs oracle")
    assert_bits_equal(host(m2), mr, "final m vs oracle")
