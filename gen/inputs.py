"""Seeded synthetic gradients, residuals and weights for every workload.

Every array is drawn from ``numpy.random.default_rng(SeedSequence(key))`` in
chunks of 2**24 elements, where ``key = [workload, step, chunk, stream]``.
Each random stream (normal values, masks, signs) has its own key, so the first
``n`` elements of an array are the same whatever total length is asked for and
however many threads fill it.  Chunks are filled by a thread pool: numpy's
generators and ufuncs release the GIL on large arrays.

Workloads (sizes are exact):

* ``flat``   N = 1,000,000 values N(0,1), k = 10,000, 10 chained steps.
* ``bert``   the 194 tensors of a BERT-base encoder (two embeddings, 12 layers of
             Q/K/V/O 768x768 + biases, 768x3072 and 3072x768 FFN + biases, two
             LayerNorms); per tensor Student-t(3) values times 10**u, u ~ U(-4,-2)
             drawn once per tensor; k = n//1000 for tensors above one million
             elements, else n//100, at least 1; 20 chained steps.
* ``sign``   N = 340,000,000 values 1e-3 * N(0,1) with a Bernoulli(0.01) mask of
             entries multiplied by 100; 50 chained steps.
* ``decode`` N = 25,600,000; 16 independent N(0,1) gradients (one per packet) and
             N(0,1) starting weights.
* ``large``  N = 1,300,000,000 magnitudes exp(-7 + 2 z), z ~ N(0,1), with random
             signs from a separate bit stream, k = 1,300,000, 5 chained steps.
* ``adam``   the sign workload's size and gradient law (N = 340,000,000, the
             parameter count of BERT-large) for a full 1-bit Adam run: weights
             0.02 N(0,1), lr = 2e-5, beta1 = 0.9, beta2 = 0.999, eps = 1e-8, clip 5,
             3 full-precision warm-up steps, then 1-bit compression steps.
* ``random`` the large workload's gradients and sizes with k = 1,300,000 the
             expected count of random sparsification; its draws are keyed by
             RANDOM_SEED and the step number.

Nothing in this module computes any part of the compression method.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 24

# workload ids (first element of every seed key)
FLAT, BERT, SIGN, DECODE, LARGE, SMALL = 1, 2, 3, 4, 5, 9

FLAT_N, FLAT_K, FLAT_STEPS = 1_000_000, 10_000, 10
SIGN_N, SIGN_STEPS, SIGN_BETA1, SIGN_CLIP = 340_000_000, 50, 0.9, 5.0
DECODE_N, DECODE_PACKETS, DECODE_K, DECODE_LR = 25_600_000, 16, 25_600, 0.1
LARGE_N, LARGE_K, LARGE_STEPS, LARGE_BLOCK = 1_300_000_000, 1_300_000, 5, 256
BERT_STEPS = 20
RANDOM_SEED = 0x5EED_0001
ADAM_N, ADAM_LR, ADAM_BETA1, ADAM_BETA2, ADAM_EPS, ADAM_WARMUP, ADAM_STEPS = 340_000_000, 2e-5, 0.9, 0.999, 1e-8, 3, 8
ADAM = 6


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(n: int, fill, dtype=np.float32, out: np.ndarray | None = None) -> np.ndarray:
    """Fill ``out[0:n]`` chunk by chunk; ``fill(c, m)`` returns chunk c of length m."""
    if out is None:
        out = np.empty(n, dtype=dtype)
    nchunks = (n + CHUNK - 1) // CHUNK

    def one(c):
        lo = c * CHUNK
        m = min(CHUNK, n - lo)
        out[lo:lo + m] = fill(c, m)

    if nchunks <= 1:
        for c in range(nchunks):
            one(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, range(nchunks)))
    return out


def normal_f32(n: int, *key: int) -> np.ndarray:
    """n float32 N(0,1) values, stream key + [chunk, 0]."""
    return _chunked(n, lambda c, m: rng(*key, c, 0).standard_normal(m, dtype=np.float32))


# ----------------------------------------------------------------- flat
def flat_gradient(step: int, n: int = FLAT_N) -> np.ndarray:
    return normal_f32(n, FLAT, step)


# ----------------------------------------------------------------- bert
def bert_base_tensors() -> list[tuple[str, int]]:
    """(name, element count) of the 194 BERT-base tensors, in packing order."""
    h, f, L = 768, 3072, 12
    t = [("embeddings.word", 30522 * h), ("embeddings.position", 512 * h)]
    for layer in range(L):
        p = f"layer{layer}."
        for m in ("q", "k", "v", "o"):
            t += [(p + m + ".weight", h * h), (p + m + ".bias", h)]
        t += [(p + "ln1.weight", h), (p + "ln1.bias", h)]
        t += [(p + "ffn_in.weight", h * f), (p + "ffn_in.bias", f)]
        t += [(p + "ffn_out.weight", f * h), (p + "ffn_out.bias", h)]
        t += [(p + "ln2.weight", h), (p + "ln2.bias", h)]
    return t


def layerwise_k(n: int) -> int:
    """Per-tensor k of the layer-wise workload: 0.1 % above one million
    elements, 1 % otherwise, at least one."""
    return max(1, n // 1000) if n > 1_000_000 else max(1, n // 100)


def bert_segments() -> tuple[np.ndarray, np.ndarray]:
    """(seg_off int64[nseg+1], seg_k int64[nseg]) of the packed BERT-base gradient."""
    sizes = [n for _, n in bert_base_tensors()]
    off = np.zeros(len(sizes) + 1, dtype=np.int64)
    off[1:] = np.cumsum(sizes)
    ks = np.array([layerwise_k(n) for n in sizes], dtype=np.int64)
    return off, ks


def bert_scales() -> np.ndarray:
    """One exponent u ~ U(-4, -2) per tensor, fixed for every step."""
    nt = len(bert_base_tensors())
    return np.array([rng(BERT, 999, t).uniform(-4.0, -2.0) for t in range(nt)])


def bert_gradient(step: int) -> np.ndarray:
    off, _ = bert_segments()
    u = bert_scales()
    out = np.empty(int(off[-1]), dtype=np.float32)

    def one(t):
        n = int(off[t + 1] - off[t])
        v = rng(BERT, step, t).standard_t(3, size=n) * (10.0 ** u[t])
        out[off[t]:off[t + 1]] = v.astype(np.float32)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(len(u))))
    return out


# ----------------------------------------------------------------- sign
def sign_gradient(step: int, n: int = SIGN_N) -> np.ndarray:
    def fill(c, m):
        z = rng(SIGN, step, c, 0).standard_normal(m, dtype=np.float32).astype(np.float64) * 1e-3
        hit = rng(SIGN, step, c, 1).random(m) < 0.01
        z[hit] *= 100.0
        return z.astype(np.float32)
    return _chunked(n, fill)


# ----------------------------------------------------------------- decode
def decode_packet_gradient(p: int, n: int = DECODE_N) -> np.ndarray:
    return normal_f32(n, DECODE, p)


def decode_weights(n: int = DECODE_N) -> np.ndarray:
    return normal_f32(n, DECODE, 1000)


# ----------------------------------------------------------------- large
def large_gradient(step: int, n: int = LARGE_N, out: np.ndarray | None = None) -> np.ndarray:
    """Log-normal magnitudes exp(-7 + 2 z) (computed in float64, stored as
    float32) with signs from a separate bit stream."""
    def fill(c, m):
        z = rng(LARGE, step, c, 0).standard_normal(m, dtype=np.float32).astype(np.float64)
        mag = np.exp(-7.0 + 2.0 * z).astype(np.float32)
        neg = rng(LARGE, step, c, 1).integers(0, 2, size=m, dtype=np.uint8).astype(bool)
        mag[neg] = -mag[neg]
        return mag
    return _chunked(n, fill, out=out)


# ----------------------------------------------------------------- small / adversarial
def uniform_ties(n: int, levels: int, *key: int) -> np.ndarray:
    """Values drawn from a few magnitudes (many exact ties in |x|), random signs."""
    r = rng(SMALL, *key)
    mags = r.integers(0, levels, size=n).astype(np.float32) * np.float32(0.25)
    sgn = np.where(r.integers(0, 2, size=n) == 1, 1.0, -1.0).astype(np.float32)
    return mags * sgn


def specials(n: int, *key: int) -> np.ndarray:
    """N(0,1) values salted with +-0, subnormals, +-max, +-inf and NaN."""
    r = rng(SMALL, *key)
    x = r.standard_normal(n, dtype=np.float32)
    pool = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, -3e-39, 3.4028235e38,
                     -3.4028235e38, np.inf, -np.inf, np.nan], dtype=np.float32)
    pos = r.integers(0, n, size=max(1, n // 8))
    x[pos] = pool[r.integers(0, len(pool), size=len(pos))]
    return x


def normal_small(n: int, *key: int, scale: float = 1.0) -> np.ndarray:
    return (rng(SMALL, *key).standard_normal(n, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def sorted_unique_indices(n: int, k: int, *key: int) -> np.ndarray:
    """k distinct indices in [0, n), ascending, int32 (for decode / encoding inputs)."""
    r = rng(SMALL, *key)
    if k == 0:
        return np.zeros(0, dtype=np.int32)
    if k * 4 < n:
        s = set()
        while len(s) < k:
            s.update(r.integers(0, n, size=k - len(s)).tolist())
        return np.array(sorted(s), dtype=np.int32)
    return np.sort(r.permutation(n)[:k]).astype(np.int32)


def large_gradient_device(step: int, n: int, device, chunk: int = 1 << 27):
    """Same law as large_gradient (exp(-7 + 2 z) magnitudes, random signs), drawn
    on the device with torch's seeded generator so that benchmark inputs for
    many steps at N = 1.3e9 cost milliseconds.  The values differ from the
    numpy stream; parity tests use large_gradient."""
    import torch

    gz = torch.Generator(device=device)
    gz.manual_seed(LARGE * 1_000_003 + step)
    out = torch.empty(n, dtype=torch.float32, device=device)
    for lo in range(0, n, chunk):
        m = min(chunk, n - lo)
        z = torch.randn(m, generator=gz, device=device, dtype=torch.float32).double()
        mag = torch.exp(z.mul_(2.0).add_(-7.0)).float()
        neg = torch.randint(0, 2, (m,), generator=gz, device=device, dtype=torch.uint8).bool()
        out[lo:lo + m] = torch.where(neg, -mag, mag)
    return out


def adam_weights(n: int = ADAM_N) -> np.ndarray:
    """Initial weights of the adam workload: 0.02 * N(0, 1)."""
    def fill(c, m):
        return (0.02 * rng(ADAM, 0, c, 0).standard_normal(m)).astype(np.float32)
    return _chunked(n, fill)


def adam_weights_device(n: int, device):
    """The same law drawn on the device (values differ from the numpy stream)."""
    import torch

    gz = torch.Generator(device=device)
    gz.manual_seed(ADAM * 1_000_003)
    return torch.randn(n, generator=gz, device=device, dtype=torch.float32).mul_(0.02)


def sign_gradient_device(step: int, n: int, device):
    """Same law as sign_gradient (1e-3 N(0,1) with a Bernoulli(0.01) set of
    entries times 100), drawn on the device with torch's seeded generator for
    long full-size chains; the values differ from the numpy stream."""
    import torch

    gz = torch.Generator(device=device)
    gz.manual_seed(SIGN * 1_000_003 + step)
    z = torch.randn(n, generator=gz, device=device, dtype=torch.float32).double().mul_(1e-3)
    hit = torch.rand(n, generator=gz, device=device, dtype=torch.float32) < 0.01
    z[hit] *= 100.0
    return z.float()
