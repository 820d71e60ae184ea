"""CPU oracle (test infrastructure only).

Plain, slow, single-threaded C (``oracle.c``) behind ctypes, with numpy in and
out.  Only tests, the smoke check and the benchmark's CPU-baseline leg may use
it; the GPU library neither imports nor links anything here.

``build()`` compiles ``liboracle.so`` next to this file with gcc; ``lib()``
loads it, building it first only if it is missing.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# EFG_ORACLE_LIB names another build of oracle.c (the sanitizer test's)
_LIB = os.environ.get("EFG_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-builtin",
          "-shared", "-fPIC", "-Wall", "-Wextra"]


def build() -> str:
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp])
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        p, i64, i32, u32p, f = C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_float
        sig = {
            "orc_topk": [p, p, i64, i64, p, p, u32p],
            "orc_topk_segmented": [p, p, i32, p, p, p, p, u32p],
            "orc_sign": [p, p, p, i64, f, f, p, p, u32p],
            "orc_decode": [p, i64, i32, p, p, p],
            "orc_sgd": [p, p, i64, f],
            "orc_bitmap_encode": [p, i64, i64, p],
            "orc_bitmap_decode": [p, i64, p, i64, p],
            "orc_delta_encode": [p, i64, p, p],
            "orc_delta_decode": [p, i64, i64, p],
            "orc_blocks_encode": [p, i64, i64, p, p, p, p],
            "orc_blocks_decode": [p, p, p, i64, p, i64, p],
            "orc_quantize_int8": [p, p, i64, p, p, p],
            "orc_random_keep_at": [p, p, i64, i64, f, C.c_uint64, C.c_uint64, p],
            "orc_adam_step": [p, p, p, p, i64, f, f, f, f, f, u32p],
            "orc_onebit_adam_update": [p, i32, p, p, p, i64, f, f, f, f, u32p],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = C.c_int
        L.orc_sumsq.argtypes = [p, i64]
        L.orc_sumsq.restype = C.c_double
        L.orc_philox4x32_10.argtypes = [p, p, p]
        L.orc_philox4x32_10.restype = None
        L.orc_sum_abs_exact.argtypes = [p, i64]
        L.orc_sum_abs_exact.restype = C.c_double
        L.orc_uniform.argtypes = [C.c_uint64, C.c_uint64, i64]
        L.orc_uniform.restype = C.c_float
        L.orc_keep_probability.argtypes = [f, i64, f]
        L.orc_keep_probability.restype = C.c_float
        L.orc_random_sparsify.argtypes = [p, p, i64, i64, C.c_uint64, C.c_uint64, i64, p, p, p, p, u32p]
        L.orc_random_sparsify.restype = C.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def topk(g, e, k):
    """Returns (vals, idx, e_new, nonfinite); e is not modified."""
    g = _f32(g)
    e2 = _f32(e).copy()
    n = g.size
    vals = np.empty(k, np.float32)
    idx = np.empty(k, np.int32)
    bad = np.zeros(1, np.uint32)
    _check(lib().orc_topk(_ptr(g), _ptr(e2), n, k, _ptr(vals), _ptr(idx), _ptr(bad)), "topk")
    return vals, idx, e2, int(bad[0])


def topk_segmented(g, e, seg_off, seg_k):
    g = _f32(g)
    e2 = _f32(e).copy()
    off = np.ascontiguousarray(seg_off, dtype=np.int64)
    ks = np.ascontiguousarray(seg_k, dtype=np.int64)
    K = int(ks.sum())
    vals = np.empty(K, np.float32)
    idx = np.empty(K, np.int32)
    bad = np.zeros(1, np.uint32)
    _check(lib().orc_topk_segmented(_ptr(g), _ptr(e2), len(ks), _ptr(off), _ptr(ks),
                                    _ptr(vals), _ptr(idx), _ptr(bad)), "topk_segmented")
    return vals, idx, e2, int(bad[0])


def sign(g, e, m, beta1=0.9, clip=5.0):
    """Returns (e_new, m_new, sign int8, bits uint8, nonfinite); m may be None
    (compress only: m_new is then None)."""
    g = _f32(g)
    e2 = _f32(e).copy()
    m2 = None if m is None else _f32(m).copy()
    n = g.size
    s = np.empty(n, np.int8)
    bits = np.empty((n + 7) // 8, np.uint8)
    bad = np.zeros(1, np.uint32)
    _check(lib().orc_sign(_ptr(g), _ptr(e2), None if m2 is None else _ptr(m2), n, beta1, clip, _ptr(s),
                          _ptr(bits), _ptr(bad)), "sign")
    return e2, m2, s, bits, int(bad[0])


def decode(G, vals, idx, pk_off):
    G2 = _f32(G).copy()
    vals = _f32(vals)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    off = np.ascontiguousarray(pk_off, dtype=np.int64)
    _check(lib().orc_decode(_ptr(G2), G2.size, len(off) - 1, _ptr(vals), _ptr(idx), _ptr(off)),
           "decode")
    return G2


def sgd(w, G, lr):
    w2 = _f32(w).copy()
    G = _f32(G)
    _check(lib().orc_sgd(_ptr(w2), _ptr(G), w2.size, lr), "sgd")
    return w2


def bitmap_encode(idx, n):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    bits = np.empty((n + 7) // 8, np.uint8)
    _check(lib().orc_bitmap_encode(_ptr(idx), idx.size, n, _ptr(bits)), "bitmap_encode")
    return bits


def bitmap_decode(bits, n, k_cap=None):
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    if k_cap is None:
        k_cap = n
    idx = np.empty(max(k_cap, 1), np.int32)
    k = np.zeros(1, np.int64)
    _check(lib().orc_bitmap_decode(_ptr(bits), n, _ptr(idx), k_cap, _ptr(k)), "bitmap_decode")
    return idx[:min(int(k[0]), k_cap)], int(k[0])


def delta_encode(idx):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    out = np.empty(5 * idx.size + 1, np.uint8)
    nb = np.zeros(1, np.int64)
    _check(lib().orc_delta_encode(_ptr(idx), idx.size, _ptr(out), _ptr(nb)), "delta_encode")
    return out[:int(nb[0])].copy()


def delta_decode(stream, k):
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    idx = np.empty(max(k, 1), np.int32)
    _check(lib().orc_delta_decode(_ptr(stream), stream.size, k, _ptr(idx)), "delta_decode")
    return idx[:k]


def blocks_encode(idx, n):
    """Returns (mask, counts_m1, offs)."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    nb = (n + 255) // 256
    mask = np.empty((nb + 7) // 8, np.uint8)
    counts = np.empty(max(1, min(idx.size, nb)), np.uint8)
    offs = np.empty(max(1, idx.size), np.uint8)
    nblk = np.zeros(1, np.int64)
    _check(lib().orc_blocks_encode(_ptr(idx), idx.size, n, _ptr(mask), _ptr(counts), _ptr(offs),
                                   _ptr(nblk)), "blocks_encode")
    return mask, counts[:int(nblk[0])].copy(), offs[:idx.size].copy()


def blocks_decode(mask, counts_m1, offs, n, k_cap=None):
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    counts_m1 = np.ascontiguousarray(counts_m1, dtype=np.uint8)
    offs = np.ascontiguousarray(offs, dtype=np.uint8)
    if k_cap is None:
        k_cap = offs.size
    idx = np.empty(max(k_cap, 1), np.int32)
    k = np.zeros(1, np.int64)
    _check(lib().orc_blocks_decode(_ptr(mask), _ptr(counts_m1 if counts_m1.size else np.zeros(1, np.uint8)),
                                   _ptr(offs if offs.size else np.zeros(1, np.uint8)), n, _ptr(idx),
                                   k_cap, _ptr(k)), "blocks_decode")
    return idx[:min(int(k[0]), k_cap)], int(k[0])


def quantize_int8(vals, idx, e):
    """Returns (q int8, scale, e_new); e is not modified."""
    vals = _f32(vals)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    e2 = _f32(e).copy()
    q = np.empty(max(1, vals.size), np.int8)
    sc = np.zeros(1, np.float32)
    _check(lib().orc_quantize_int8(_ptr(vals), _ptr(idx), vals.size, _ptr(e2), _ptr(q), _ptr(sc)), "quantize_int8")
    return q[:vals.size], float(sc[0]), e2


def sumsq(a):
    """Sum of squares of the finite entries, float64, in index order."""
    a = _f32(a)
    return float(lib().orc_sumsq(_ptr(a), a.size))


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return [int(v) for v in out]


def sum_abs_exact(x):
    """Sum of |x| over the finite entries, exact, rounded once to float64."""
    x = _f32(x)
    return float(lib().orc_sum_abs_exact(_ptr(x), x.size))


def uniform(seed, step, i):
    return float(lib().orc_uniform(seed, step, i))


def keep_probability(x, k, s32):
    return float(lib().orc_keep_probability(x, k, s32))


def random_sparsify(g, e, k, seed, step, cap=None):
    """Returns (vals, idx, e_new, count, S32, nonfinite); vals/idx hold min(count, cap) entries."""
    g = _f32(g)
    e2 = _f32(e).copy()
    n = g.size
    if cap is None:
        cap = n
    vals = np.empty(max(cap, 1), np.float32)
    idx = np.empty(max(cap, 1), np.int32)
    cnt = np.zeros(1, np.int64)
    s32 = np.zeros(1, np.float32)
    bad = np.zeros(1, np.uint32)
    _check(lib().orc_random_sparsify(_ptr(g), _ptr(e2), n, k, seed, step, cap, _ptr(vals), _ptr(idx), _ptr(cnt),
                                     _ptr(s32), _ptr(bad)), "random_sparsify")
    c = int(cnt[0])
    w = min(c, cap)
    return vals[:w].copy(), idx[:w].copy(), e2, c, float(s32[0]), int(bad[0])


def random_keep_at(x_at, pos, k, s32, seed, step):
    """Keep decisions (bool array) for elements pos whose x values are x_at."""
    x_at = _f32(x_at)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    keep = np.zeros(max(pos.size, 1), np.uint8)
    _check(lib().orc_random_keep_at(_ptr(x_at), _ptr(pos), pos.size, k, s32, seed, step, _ptr(keep)),
           "random_keep_at")
    return keep[:pos.size].astype(bool)


def adam_scalars(lr, beta1, beta2, t, t_v=None):
    """(step_size, sqrt_bc2) of step t (1-based): lr / (1 - beta1^t) and
    sqrt(1 - beta2^t_v), t_v = t unless v is frozen, evaluated in float64 with
    the float32 betas the EMAs use, then rounded to float32."""
    t_v = t if t_v is None else t_v
    b1, b2 = float(np.float32(beta1)), float(np.float32(beta2))
    return float(np.float32(lr / (1.0 - b1 ** t))), float(np.float32(np.sqrt(1.0 - b2 ** t_v)))


def adam_step(g, m, v, w, beta1, beta2, step_size, sqrt_bc2, eps):
    """Returns (m_new, v_new, w_new, nonfinite)."""
    g = _f32(g)
    m2, v2, w2 = _f32(m).copy(), _f32(v).copy(), _f32(w).copy()
    bad = np.zeros(1, np.uint32)
    _check(lib().orc_adam_step(_ptr(g), _ptr(m2), _ptr(v2), _ptr(w2), g.size, beta1, beta2, step_size, sqrt_bc2,
                               eps, _ptr(bad)), "adam_step")
    return m2, v2, w2, int(bad[0])


def onebit_adam_update_var(qsum, nworkers, m, v, w, beta1, beta2, step_size, sqrt_bc2, eps):
    """The compression-phase step with the variance still updated: the Adam
    step (adam_step) fed ghat = qsum / nworkers, a correctly rounded float32
    division.  Returns (m_new, v_new, w_new, nonfinite)."""
    ghat = np.ascontiguousarray(qsum, dtype=np.int8).astype(np.float32) / np.float32(nworkers)
    return adam_step(ghat, m, v, w, beta1, beta2, step_size, sqrt_bc2, eps)


def onebit_adam_update(qsum, nworkers, m, v, w, beta1, step_size, sqrt_bc2, eps):
    """Returns (m_new, w_new, nonfinite); v is read only."""
    q = np.ascontiguousarray(qsum, dtype=np.int8)
    m2, w2 = _f32(m).copy(), _f32(w).copy()
    v = _f32(v)
    bad = np.zeros(1, np.uint32)
    _check(lib().orc_onebit_adam_update(_ptr(q), nworkers, _ptr(m2), _ptr(v), _ptr(w2), q.size, beta1, step_size,
                                        sqrt_bc2, eps, _ptr(bad)), "onebit_adam_update")
    return m2, w2, int(bad[0])
