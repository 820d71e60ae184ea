"""Helpers shared by the GPU parity tests (not a test module)."""
import sys

import numpy as np
import pytest
import torch


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_bits_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.float32 or want.dtype == np.float32:
        g, w = bits(got), bits(want)
    else:
        g, w = got, want
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5].tolist()}: got {got[bad[:5]]} want {want[bad[:5]]}"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def check_topk_invariants_device(x, vals, idx, e_after, k):
    """Asserts that (vals, idx, e_after) is the top-k of x (device tensors, any
    size): k strictly increasing in-range indices; vals = x[idx] bit for bit;
    every kept key (|x| bits) >= every dropped key, equal keys kept by lower
    index; e_after = x except +0 at idx.  These fix the result uniquely.
    Overwrites x."""
    n = x.numel()
    ik = idx.long()
    assert idx.numel() == k
    if k > 0:
        assert bool((ik[1:] > ik[:-1]).all()) and int(ik[0]) >= 0 and int(ik[-1]) < n
        assert torch.equal(vals.view(torch.int32), x[ik].view(torch.int32))
    if 0 < k < n:
        key = x.view(torch.int32) & 0x7FFFFFFF
        kept = torch.zeros(n, dtype=torch.bool, device=x.device)
        kept[ik] = True
        T = int(key[ik].min())
        drop_max = int(key.masked_fill(kept, -1).max())
        assert T >= drop_max
        if T == drop_max:  # ties at the threshold: the lower indices are kept
            assert int(ik[key[ik] == T].max()) < int(torch.nonzero((key == T) & ~kept)[0, 0])
        del key, kept
    x[ik] = 0.0
    assert torch.equal(e_after.view(torch.int32), x.view(torch.int32))
