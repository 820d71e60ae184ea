"""Python binding of libefgrad.so: error-feedback gradient compression on MI355X.

Each function has the name of the C entry point it calls and only marshals
arguments: it checks tensor devices, dtypes and shapes, allocates outputs and
workspaces with torch when the caller does not pass them, and hands raw device
pointers and the current HIP stream to the library.  Every step of the
computation runs in the library's HIP kernels; there is no fallback path.
If libefgrad.so is missing, importing the symbols raises.

Build the library with ``python -m error_feedback_gradient_amd.build``.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libefgrad.so")

EF_OK, EF_EINVAL, EF_EWS, EF_EHIP, EF_ENOTIMPL = 0, 1, 2, 3, 4
EF_FLAG_FORCE_FALLBACK = 1

# name -> (restype, argtypes); the full C ABI of include/efgrad.h
_p, _i64, _i32, _u32, _f, _sz = C.c_void_p, C.c_int64, C.c_int32, C.c_uint32, C.c_float, C.c_size_t
SIGNATURES = {
    "ef_last_error": (C.c_char_p, []),
    "ef_version": (C.c_char_p, []),
    "ef_topk_workspace_bytes": (_sz, [_i64, _i64]),
    "ef_topk_compress": (C.c_int, [_p, _p, _i64, _i64, _p, _p, _p, _sz, _p, _p, _u32, _p]),
    "ef_topk_compress_noalloc": (C.c_int, [_p, _p, _i64, _i64, _p, _p, _p, _p, _u32, _p]),
    "ef_topk_workspace_status": (C.c_int, [_p, _p, _p]),
    "ef_topk_workspace_paths": (C.c_int, [_p, _sz, _i32, _p, _p]),
    "ef_topk_segmented_workspace_bytes": (_sz, [_i32, _p, _p]),
    "ef_topk_compress_segmented": (C.c_int, [_p, _p, _i32, _p, _p, _p, _p, _p, _sz, _p, _p, _u32, _p]),
    "ef_sign_workspace_bytes": (_sz, [_i64]),
    "ef_sign_compress": (C.c_int, [_p, _p, _p, _i64, _f, _f, _p, _p, _p, _p, _p, _sz, _p]),
    "ef_adam_scalars": (C.c_int, [C.c_double, _f, _f, _i64, _i64, C.POINTER(_f), C.POINTER(_f)]),
    "ef_adam_step": (C.c_int, [_p, _p, _p, _p, _i64, _f, _f, _f, _f, _f, _p, _p]),
    "ef_onebit_adam_update": (C.c_int, [_p, _i32, _p, _p, _p, _i64, _f, _f, _f, _f, _p, _p]),
    "ef_onebit_adam_update_var": (C.c_int, [_p, _i32, _p, _p, _p, _i64, _f, _f, _f, _f, _f, _p, _p]),
    "ef_quantize_workspace_bytes": (_sz, [_i64]),
    "ef_quantize_int8": (C.c_int, [_p, _p, _i64, _p, _i64, _p, _p, _p, _sz, _p]),
    "ef_random_sparsify_workspace_bytes": (_sz, [_i64]),
    "ef_random_sparsify": (C.c_int, [_p, _p, _i64, _i64, C.c_uint64, C.c_uint64, _p, _p, _i64, _p, _p, _p, _p, _sz,
                                     _u32, _p]),
    "sparse_decode_accumulate": (C.c_int, [_p, _i64, _i32, _p, _p, _p, _p, _p]),
    "sgd_apply": (C.c_int, [_p, _p, _i64, _f, _p]),
    "sparse_decode_sgd": (C.c_int, [_p, _p, _i64, _i32, _p, _p, _p, _f, _p, _p]),
    "encode_bitmap": (C.c_int, [_p, _i64, _i64, _p, _p]),
    "decode_bitmap_workspace_bytes": (_sz, [_i64]),
    "decode_bitmap": (C.c_int, [_p, _i64, _p, _i64, _p, _p, _sz, _p]),
    "encode_delta_bound": (_i64, [_i64]),
    "delta_workspace_bytes": (_sz, [_i64]),
    "encode_delta": (C.c_int, [_p, _i64, _p, _p, _p, _sz, _p]),
    "decode_delta": (C.c_int, [_p, _i64, _i64, _p, _p, _p, _sz, _p]),
    "blocks_workspace_bytes": (_sz, [_i64, _i64]),
    "encode_blocks": (C.c_int, [_p, _i64, _i64, _p, _p, _p, _p, _p, _sz, _p]),
    "decode_blocks": (C.c_int, [_p, _p, _p, _i64, _i64, _p, _p, _sz, _p]),
    "ef_profile_enable": (C.c_int, [C.c_int, C.c_char_p]),
    "ef_profile_read": (C.c_int, [C.c_char_p, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
}

_lib = None


class EfError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: status {code}: {msg}")
        self.code = code


def lib() -> C.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m error_feedback_gradient_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().ef_last_error().decode()


def _check(rc: int, where: str):
    if rc != EF_OK:
        raise EfError(rc, where, last_error())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, device, name, numel=None):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")


def _gpu(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    return t.device


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- top-k
def ef_topk_workspace_bytes(n: int, k: int) -> int:
    return int(lib().ef_topk_workspace_bytes(n, k))


def ef_topk_compress(g, e, k, vals=None, idx=None, ws=None, nonfinite=None, flags=0, stats=None):
    """x = g + e; keep the k largest |x| (ties: lower index); returns (vals, idx);
    e is updated in place.  stats (float64 GPU tensor of 2) receives
    {sum vals^2, sum new e^2}."""
    dev = _gpu(g, "g")
    n = g.numel()
    _need(g, torch.float32, dev, "g")
    _need(e, torch.float32, dev, "e", n)
    if vals is None:
        vals = torch.empty(k, dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(k, dtype=torch.int32, device=dev)
    _need(vals, torch.float32, dev, "vals", k)
    _need(idx, torch.int32, dev, "idx", k)
    if ws is None:
        ws = workspace(ef_topk_workspace_bytes(n, k), dev)
    if nonfinite is not None:
        _need(nonfinite, torch.int32, dev, "nonfinite", 1)
    if stats is not None:
        _need(stats, torch.float64, dev, "stats", 2)
    _check(lib().ef_topk_compress(_ptr(g), _ptr(e), n, k, _ptr(vals), _ptr(idx), _ptr(ws), ws.numel(),
                                  _ptr(nonfinite), _ptr(stats), flags, _stream(dev)), "ef_topk_compress")
    return vals, idx


def ef_topk_workspace_status(ws, stray=None, device=None):
    """Device uint32 (as int32[1]): indices the last top-k call on ws found
    out of range in its own workspace entries (0 unless the workspace was
    overwritten during the call).  ws=None: the allocation-free call's static
    scratch on `device`."""
    dev = ws.device if ws is not None else torch.device(device if device is not None else "cuda")
    if stray is None:
        stray = torch.empty(1, dtype=torch.int32, device=dev)
    _need(stray, torch.int32, dev, "stray", 1)
    _check(lib().ef_topk_workspace_status(_ptr(ws), _ptr(stray), _stream(dev)), "ef_topk_workspace_status")
    return stray


def ef_topk_workspace_paths(ws, nseg=1, out=None, device=None):
    """Device int32 [nseg, 2]: per tensor of the last top-k call on ws (nseg
    tensors), 1 if it took the exact full-pass selection else 0, and the
    candidates its streaming pass collected.  ws=None: the allocation-free
    call's static scratch on `device`."""
    dev = ws.device if ws is not None else torch.device(device if device is not None else "cuda")
    if out is None:
        out = torch.empty((max(0, nseg), 2), dtype=torch.int32, device=dev)
    _need(out, torch.int32, dev, "out", 2 * nseg)
    _check(lib().ef_topk_workspace_paths(_ptr(ws), 0 if ws is None else ws.numel(), nseg, _ptr(out),
                                         _stream(dev)),
           "ef_topk_workspace_paths")
    return out


EF_TOPK_NOALLOC_SCRATCH_BYTES = 32 << 20


def ef_topk_compress_noalloc(g, e, k, vals=None, idx=None, nonfinite=None, flags=0, stats=None):
    """ef_topk_compress with the library's static scratch instead of a workspace
    (the C call allocates nothing; vals and idx are allocated here only when
    the caller does not pass them).  Returns (vals, idx)."""
    dev = _gpu(g, "g")
    n = g.numel()
    _need(g, torch.float32, dev, "g")
    _need(e, torch.float32, dev, "e", n)
    if vals is None:
        vals = torch.empty(k, dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(k, dtype=torch.int32, device=dev)
    _need(vals, torch.float32, dev, "vals", k)
    _need(idx, torch.int32, dev, "idx", k)
    if nonfinite is not None:
        _need(nonfinite, torch.int32, dev, "nonfinite", 1)
    if stats is not None:
        _need(stats, torch.float64, dev, "stats", 2)
    _check(lib().ef_topk_compress_noalloc(_ptr(g), _ptr(e), n, k, _ptr(vals), _ptr(idx), _ptr(nonfinite),
                                          _ptr(stats), flags, _stream(dev)), "ef_topk_compress_noalloc")
    return vals, idx


def _i64_host(a):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a, a.ctypes.data_as(C.c_void_p)


def _segment_tables(seg_off, seg_k):
    """Host int64 copies of the segment tables and their pointers; seg_off must
    hold one entry more than seg_k (the library reads seg_off[nseg])."""
    off, po = _i64_host(seg_off)
    ks, pk = _i64_host(seg_k)
    if off.ndim != 1 or ks.ndim != 1 or off.size != ks.size + 1:
        raise ValueError(f"seg_off needs len(seg_k) + 1 = {ks.size + 1} entries, has {off.size}")
    return off, po, ks, pk


def ef_topk_segmented_workspace_bytes(seg_off, seg_k) -> int:
    off, po, ks, pk = _segment_tables(seg_off, seg_k)
    return int(lib().ef_topk_segmented_workspace_bytes(len(ks), po, pk))


def ef_topk_compress_segmented(g, e, seg_off, seg_k, vals=None, idx=None, ws=None, nonfinite=None, flags=0,
                               stats=None):
    """Top-k EF of every tensor [seg_off[s], seg_off[s+1]) with its own seg_k[s]
    (host integer sequences); returns (vals, idx) concatenated in tensor order.
    stats (float64 GPU tensor of 2*nseg) receives per tensor {sum vals^2, sum new e^2}."""
    dev = _gpu(g, "g")
    off, po, ks, pk = _segment_tables(seg_off, seg_k)
    K = int(ks.sum())
    _need(g, torch.float32, dev, "g", int(off[-1]) if len(off) else 0)
    _need(e, torch.float32, dev, "e", int(off[-1]) if len(off) else 0)
    if vals is None:
        vals = torch.empty(K, dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(K, dtype=torch.int32, device=dev)
    _need(vals, torch.float32, dev, "vals", K)
    _need(idx, torch.int32, dev, "idx", K)
    if ws is None:
        ws = workspace(lib().ef_topk_segmented_workspace_bytes(len(ks), po, pk), dev)
    if nonfinite is not None:
        _need(nonfinite, torch.int32, dev, "nonfinite", 1)
    if stats is not None:
        _need(stats, torch.float64, dev, "stats", 2 * len(ks))
    _check(lib().ef_topk_compress_segmented(_ptr(g), _ptr(e), len(ks), po, pk, _ptr(vals), _ptr(idx), _ptr(ws),
                                            ws.numel(), _ptr(nonfinite), _ptr(stats), flags, _stream(dev)),
           "ef_topk_compress_segmented")
    return vals, idx


# ---------------------------------------------------------------- sign
def ef_sign_compress(g, e, m, beta1=0.9, clip=5.0, sign_out=None, bits=None, nonfinite=None,
                     want_sign=True, want_bits=True, stats=None, ws=None):
    """1-bit sign EF with momentum; e and m updated in place.  Returns (sign int8, bits uint8).
    m may be None (compress only).  stats (float64 GPU tensor of 4) receives
    {sum e'^2, sum m'^2, #(+1), #(-1)}."""
    dev = _gpu(g, "g")
    n = g.numel()
    _need(g, torch.float32, dev, "g")
    _need(e, torch.float32, dev, "e", n)
    if m is not None:
        _need(m, torch.float32, dev, "m", n)
    if sign_out is None and want_sign:
        sign_out = torch.empty(n, dtype=torch.int8, device=dev)
    if bits is None and want_bits:
        bits = torch.empty((n + 7) // 8, dtype=torch.uint8, device=dev)
    if sign_out is not None:
        _need(sign_out, torch.int8, dev, "sign_out", n)
    if bits is not None:
        _need(bits, torch.uint8, dev, "bits", (n + 7) // 8)
    if nonfinite is not None:
        _need(nonfinite, torch.int32, dev, "nonfinite", 1)
    if stats is not None:
        _need(stats, torch.float64, dev, "stats", 4)
        if ws is None:
            ws = workspace(lib().ef_sign_workspace_bytes(n), dev)
    _check(lib().ef_sign_compress(_ptr(g), _ptr(e), _ptr(m), n, beta1, clip, _ptr(sign_out), _ptr(bits),
                                  _ptr(nonfinite), _ptr(stats), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(dev)), "ef_sign_compress")
    return sign_out, bits


# ---------------------------------------------------------------- Adam around 1-bit compression
def adam_scalars(lr, beta1, beta2, t, t_v=None):
    """(step_size, sqrt_bc2) of step t (1-based) from ef_adam_scalars: lr / (1 -
    beta1^t) and sqrt(1 - beta2^t_v), t_v = t unless the variance is frozen."""
    ss, sb = C.c_float(0.0), C.c_float(0.0)
    _check(lib().ef_adam_scalars(lr, beta1, beta2, t, t if t_v is None else t_v, C.byref(ss), C.byref(sb)),
           "ef_adam_scalars")
    return ss.value, sb.value


def ef_adam_step(g, m, v, w, beta1, beta2, step_size, sqrt_bc2, eps, nonfinite=None):
    """One full-precision Adam step in place on m, v, w."""
    dev = _gpu(g, "g")
    n = g.numel()
    for t, name in ((g, "g"), (m, "m"), (v, "v"), (w, "w")):
        _need(t, torch.float32, dev, name, n)
    if nonfinite is not None:
        _need(nonfinite, torch.int32, dev, "nonfinite", 1)
    _check(lib().ef_adam_step(_ptr(g), _ptr(m), _ptr(v), _ptr(w), n, beta1, beta2, step_size, sqrt_bc2, eps,
                              _ptr(nonfinite), _stream(dev)), "ef_adam_step")


def ef_onebit_adam_update(qsum, nworkers, m, v, w, beta1, step_size, sqrt_bc2, eps, nonfinite=None):
    """One 1-bit Adam compression-phase update in place on m, w (v read only)."""
    dev = _gpu(m, "m")
    n = m.numel()
    _need(qsum, torch.int8, dev, "qsum", n)
    for t, name in ((m, "m"), (v, "v"), (w, "w")):
        _need(t, torch.float32, dev, name, n)
    if nonfinite is not None:
        _need(nonfinite, torch.int32, dev, "nonfinite", 1)
    _check(lib().ef_onebit_adam_update(_ptr(qsum), nworkers, _ptr(m), _ptr(v), _ptr(w), n, beta1, step_size,
                                       sqrt_bc2, eps, _ptr(nonfinite), _stream(dev)), "ef_onebit_adam_update")


def ef_onebit_adam_update_var(qsum, nworkers, m, v, w, beta1, beta2, step_size, sqrt_bc2, eps, nonfinite=None):
    """One 1-bit Adam compression-phase update with the variance still updated
    from ghat = qsum / nworkers; in place on m, v, w."""
    dev = _gpu(m, "m")
    n = m.numel()
    _need(qsum, torch.int8, dev, "qsum", n)
    for t, name in ((m, "m"), (v, "v"), (w, "w")):
        _need(t, torch.float32, dev, name, n)
    if nonfinite is not None:
        _need(nonfinite, torch.int32, dev, "nonfinite", 1)
    _check(lib().ef_onebit_adam_update_var(_ptr(qsum), nworkers, _ptr(m), _ptr(v), _ptr(w), n, beta1, beta2,
                                           step_size, sqrt_bc2, eps, _ptr(nonfinite), _stream(dev)),
           "ef_onebit_adam_update_var")


# ---------------------------------------------------------------- 8-bit packet values
def ef_quantize_int8(vals, idx, e, q=None, scale=None, ws=None):
    """q = rint(vals * 127/amax), e[idx] = vals - q*scale; returns (q int8, scale float32[1])."""
    dev = _gpu(vals, "vals")
    k = vals.numel()
    _need(vals, torch.float32, dev, "vals")
    _need(idx, torch.int32, dev, "idx", k)
    _need(e, torch.float32, dev, "e")
    if q is None:
        q = torch.empty(max(k, 1), dtype=torch.int8, device=dev)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(lib().ef_quantize_workspace_bytes(k), dev)
    _check(lib().ef_quantize_int8(_ptr(vals), _ptr(idx), k, _ptr(e), e.numel(), _ptr(q), _ptr(scale), _ptr(ws),
                                  ws.numel(), _stream(dev)), "ef_quantize_int8")
    return q[:k], scale


# ---------------------------------------------------------------- random sparsification
def ef_random_sparsify(g, e, k, seed, step, cap=None, vals=None, idx=None, count=None, sum_out=None,
                       nonfinite=None, ws=None, flags=0):
    """Keep x = g + e with probability min(1, k|x|/S) (Philox draws keyed by
    seed and step); e <- residual in place.  Returns (vals, idx, count) where
    vals/idx hold cap slots of which the first min(count, cap) are written and
    count is a device int64[1]."""
    dev = _gpu(g, "g")
    n = g.numel()
    _need(g, torch.float32, dev, "g")
    _need(e, torch.float32, dev, "e", n)
    if cap is None:
        cap = max(1, 2 * k + 64)
    if vals is None:
        vals = torch.empty(max(cap, 1), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    _need(vals, torch.float32, dev, "vals")
    _need(idx, torch.int32, dev, "idx")
    if vals.numel() < cap or idx.numel() < cap:
        raise ValueError("vals and idx need at least cap slots")
    if count is None:
        count = torch.empty(1, dtype=torch.int64, device=dev)
    _need(count, torch.int64, dev, "count", 1)
    if sum_out is not None:
        _need(sum_out, torch.float32, dev, "sum_out", 1)
    if nonfinite is not None:
        _need(nonfinite, torch.int32, dev, "nonfinite", 1)
    if ws is None:
        ws = workspace(lib().ef_random_sparsify_workspace_bytes(n), dev)
    _check(lib().ef_random_sparsify(_ptr(g), _ptr(e), n, k, seed, step, _ptr(vals), _ptr(idx), cap, _ptr(count),
                                    _ptr(sum_out), _ptr(nonfinite), _ptr(ws), ws.numel(), flags, _stream(dev)),
           "ef_random_sparsify")
    return vals, idx, count


# ---------------------------------------------------------------- decode / sgd
def _packets(vals, idx, pk_off):
    """Packet count passed to the library.  Packets without a single entry
    between them come as empty (NULL) vals/idx, which the library refuses for
    npk > 0; pk_off must then describe only empty packets, which add nothing,
    so they are passed as none."""
    return 0 if vals.numel() == 0 or idx.numel() == 0 else pk_off.numel() - 1


def sparse_decode_accumulate(G, vals, idx, pk_off, invalid=None):
    """G[idx] += vals packet by packet, in packet order.  pk_off: int64 GPU tensor [npk+1]."""
    dev = _gpu(G, "G")
    _need(G, torch.float32, dev, "G")
    _need(vals, torch.float32, dev, "vals")
    _need(idx, torch.int32, dev, "idx")
    _need(pk_off, torch.int64, dev, "pk_off")
    if invalid is not None:
        _need(invalid, torch.int32, dev, "invalid", 1)
    _check(lib().sparse_decode_accumulate(_ptr(G), G.numel(), _packets(vals, idx, pk_off), _ptr(vals), _ptr(idx),
                                          _ptr(pk_off), _ptr(invalid), _stream(dev)), "sparse_decode_accumulate")
    return G


def sgd_apply(w, G, lr):
    dev = _gpu(w, "w")
    _need(w, torch.float32, dev, "w")
    _need(G, torch.float32, dev, "G", w.numel())
    _check(lib().sgd_apply(_ptr(w), _ptr(G), w.numel(), lr, _stream(dev)), "sgd_apply")
    return w


def sparse_decode_sgd(w, vals, idx, pk_off, lr, G=None, invalid=None):
    """The receiver's step in one pass: G = the packets summed from zero (as
    sparse_decode_accumulate on a zeroed G), then w -= lr * G (as sgd_apply).
    G (optional float32 GPU tensor of w's size) receives the sum.  Returns w."""
    dev = _gpu(w, "w")
    _need(w, torch.float32, dev, "w")
    if G is not None:
        _need(G, torch.float32, dev, "G", w.numel())
    _need(vals, torch.float32, dev, "vals")
    _need(idx, torch.int32, dev, "idx")
    _need(pk_off, torch.int64, dev, "pk_off")
    if invalid is not None:
        _need(invalid, torch.int32, dev, "invalid", 1)
    _check(lib().sparse_decode_sgd(_ptr(w), _ptr(G), w.numel(), _packets(vals, idx, pk_off), _ptr(vals), _ptr(idx),
                                   _ptr(pk_off), lr, _ptr(invalid), _stream(dev)), "sparse_decode_sgd")
    return w


# ---------------------------------------------------------------- encodings
def encode_bitmap(idx, n, bits=None):
    dev = _gpu(idx, "idx")
    _need(idx, torch.int32, dev, "idx")
    if bits is None:
        bits = torch.empty((n + 7) // 8, dtype=torch.uint8, device=dev)
    _need(bits, torch.uint8, dev, "bits", (n + 7) // 8)
    _check(lib().encode_bitmap(_ptr(idx), idx.numel(), n, _ptr(bits), _stream(dev)), "encode_bitmap")
    return bits


def decode_bitmap(bits, n, k_cap, idx=None, k_out=None, ws=None):
    """Returns (idx[k_cap], k_out int64[1]); the first min(k_out, k_cap) entries are valid."""
    dev = _gpu(bits, "bits")
    _need(bits, torch.uint8, dev, "bits", (n + 7) // 8)
    if idx is None:
        idx = torch.empty(max(k_cap, 1), dtype=torch.int32, device=dev)
    if k_out is None:
        k_out = torch.empty(1, dtype=torch.int64, device=dev)
    if ws is None:
        ws = workspace(lib().decode_bitmap_workspace_bytes(n), dev)
    _check(lib().decode_bitmap(_ptr(bits), n, _ptr(idx), k_cap, _ptr(k_out), _ptr(ws), ws.numel(), _stream(dev)),
           "decode_bitmap")
    return idx, k_out


def encode_delta(idx, out=None, nbytes_out=None, ws=None):
    """Returns (stream bytes [bound], nbytes int64[1])."""
    dev = _gpu(idx, "idx")
    _need(idx, torch.int32, dev, "idx")
    k = idx.numel()
    if out is None:
        out = torch.empty(max(1, int(lib().encode_delta_bound(k))), dtype=torch.uint8, device=dev)
    if nbytes_out is None:
        nbytes_out = torch.empty(1, dtype=torch.int64, device=dev)
    if ws is None:
        ws = workspace(lib().delta_workspace_bytes(k), dev)
    _check(lib().encode_delta(_ptr(idx), k, _ptr(out), _ptr(nbytes_out), _ptr(ws), ws.numel(), _stream(dev)),
           "encode_delta")
    return out, nbytes_out


def decode_delta(stream_bytes, nbytes, k, idx=None, status=None, ws=None):
    dev = _gpu(stream_bytes, "stream")
    _need(stream_bytes, torch.uint8, dev, "stream", nbytes)
    if idx is None:
        idx = torch.empty(max(k, 1), dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(lib().delta_workspace_bytes(nbytes), dev)
    _check(lib().decode_delta(_ptr(stream_bytes), nbytes, k, _ptr(idx), _ptr(status), _ptr(ws), ws.numel(),
                              _stream(dev)), "decode_delta")
    return idx[:k], status


def encode_blocks(idx, n, mask=None, counts_m1=None, offs=None, nblk_out=None, ws=None):
    """Returns (mask, counts_m1 [min(k, nb)], offs [k], nblk int64[1])."""
    dev = _gpu(idx, "idx")
    _need(idx, torch.int32, dev, "idx")
    k = idx.numel()
    nb = (n + 255) // 256
    if mask is None:
        mask = torch.empty(max(1, (nb + 7) // 8), dtype=torch.uint8, device=dev)
    if counts_m1 is None:
        counts_m1 = torch.empty(max(1, min(k, nb)), dtype=torch.uint8, device=dev)
    if offs is None:
        offs = torch.empty(max(1, k), dtype=torch.uint8, device=dev)
    if nblk_out is None:
        nblk_out = torch.empty(1, dtype=torch.int64, device=dev)
    if ws is None:
        ws = workspace(lib().blocks_workspace_bytes(k, n), dev)
    _check(lib().encode_blocks(_ptr(idx), k, n, _ptr(mask), _ptr(counts_m1), _ptr(offs), _ptr(nblk_out), _ptr(ws),
                               ws.numel(), _stream(dev)), "encode_blocks")
    return mask, counts_m1, offs, nblk_out


def decode_blocks(mask, counts_m1, offs, n, k, idx=None, ws=None):
    dev = _gpu(mask, "mask")
    nb = (n + 255) // 256
    _need(mask, torch.uint8, dev, "mask", (nb + 7) // 8)
    _need(counts_m1, torch.uint8, dev, "counts_m1")
    _need(offs, torch.uint8, dev, "offs", k)
    if idx is None:
        idx = torch.empty(max(k, 1), dtype=torch.int32, device=dev)
    _need(idx, torch.int32, dev, "idx", k)
    if ws is not None:
        _need(ws, torch.uint8, dev, "ws")
    if ws is None:
        ws = workspace(lib().blocks_workspace_bytes(k, n), dev)
    _check(lib().decode_blocks(_ptr(mask), _ptr(counts_m1), _ptr(offs), n, k, _ptr(idx), _ptr(ws), ws.numel(),
                               _stream(dev)), "decode_blocks")
    return idx[:k]


# ---------------------------------------------------------------- timing
def profile_enable(on: bool = True, only: str | None = None):
    """Record HIP events around later launches whose label contains `only` (all if None)."""
    _check(lib().ef_profile_enable(1 if on else 0, only.encode() if only else None), "ef_profile_enable")


def profile_read(name: str):
    """(total ms, launches) of recorded kernels whose label contains `name`."""
    ms = C.c_double(0.0)
    cnt = C.c_int64(0)
    _check(lib().ef_profile_read(name.encode(), C.byref(ms), C.byref(cnt)), "ef_profile_read")
    return ms.value, cnt.value
