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
