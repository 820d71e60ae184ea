"""The C ABI on the CPU: the library loads, exports every symbol declared in
include/efgrad.h, and rejects bad arguments on the host before any HIP call
(so these run without a GPU)."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

import error_feedback_gradient_amd as efg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "efgrad.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced by the paths tested here
FAKE_ODD = 0x10004


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_matches_binding():
    decl = declared_functions()
    assert len(decl) >= 20
    assert set(decl) == set(efg.SIGNATURES), set(decl) ^ set(efg.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = efg.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", efg.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_is_gfx950_only():
    out = subprocess.run(["/opt/rocm/bin/roc-obj-ls", efg.LIB_PATH], capture_output=True, text=True)
    if out.returncode != 0:
        pytest.skip("roc-obj-ls unavailable")
    targets = set(re.findall(r"gfx\d+", out.stdout))
    assert targets == {"gfx950"}, targets


def rc_msg(rc):
    return rc, efg.last_error()


def test_version_and_error_string():
    assert b"gfx950" in efg.lib().ef_version()
    assert isinstance(efg.last_error(), str)


def test_topk_argument_checks():
    L = efg.lib()
    ws = efg.ef_topk_workspace_bytes(1000, 10)
    assert ws > 0
    assert efg.ef_topk_workspace_bytes(10, 11) == 0
    assert efg.ef_topk_workspace_bytes(-1, 0) == 0
    assert efg.ef_topk_workspace_bytes(2**31, 1) == 0
    call = lambda g, e, n, k, v, i, w, wb, flags=0: L.ef_topk_compress(g, e, n, k, v, i, w, wb, None, None, flags, None)
    assert call(FAKE, FAKE, -1, 0, FAKE, FAKE, FAKE, ws) == efg.EF_EINVAL
    assert call(FAKE, FAKE, 10, 11, FAKE, FAKE, FAKE, ws) == efg.EF_EINVAL
    assert call(FAKE, FAKE, 2**31, 1, FAKE, FAKE, FAKE, ws) == efg.EF_EINVAL
    assert call(None, FAKE, 1000, 10, FAKE, FAKE, FAKE, ws) == efg.EF_EINVAL
    assert call(FAKE_ODD, FAKE, 1000, 10, FAKE, FAKE, FAKE, ws) == efg.EF_EINVAL
    assert "aligned" in efg.last_error()
    assert call(FAKE, FAKE, 1000, 10, None, FAKE, FAKE, ws) == efg.EF_EINVAL
    assert call(FAKE, FAKE, 1000, 10, FAKE, FAKE, FAKE, ws, flags=8) == efg.EF_EINVAL
    assert call(FAKE, FAKE, 1000, 10, FAKE, FAKE, None, ws) == efg.EF_EWS
    assert call(FAKE, FAKE, 1000, 10, FAKE, FAKE, FAKE, ws - 1) == efg.EF_EWS
    assert call(FAKE, FAKE, 1000, 10, FAKE, FAKE, FAKE_ODD, ws) == efg.EF_EINVAL


def test_topk_noalloc_argument_checks():
    """The allocation-free call checks its arguments, and its scratch need
    against the static array, on the host before it touches the GPU."""
    L = efg.lib()
    lim = efg.EF_TOPK_NOALLOC_SCRATCH_BYTES
    call = lambda g, e, n, k, v, i, flags=0: L.ef_topk_compress_noalloc(g, e, n, k, v, i, None, None, flags, None)
    assert call(FAKE, FAKE, -1, 0, FAKE, FAKE) == efg.EF_EINVAL
    assert call(FAKE, FAKE, 10, 11, FAKE, FAKE) == efg.EF_EINVAL
    assert call(FAKE, FAKE, 2**31, 1, FAKE, FAKE) == efg.EF_EINVAL
    assert call(None, FAKE, 1000, 10, FAKE, FAKE) == efg.EF_EINVAL
    assert call(FAKE_ODD, FAKE, 1000, 10, FAKE, FAKE) == efg.EF_EINVAL
    assert call(FAKE, FAKE, 1000, 10, FAKE, None) == efg.EF_EINVAL
    assert call(FAKE, FAKE, 1000, 10, FAKE, FAKE, flags=8) == efg.EF_EINVAL
    # beyond the static scratch: a clear error, nothing enqueued
    n, k = 1 << 24, (1 << 24) // 10
    assert efg.ef_topk_workspace_bytes(n, k) > lim
    assert call(FAKE, FAKE, n, k, FAKE, FAKE) == efg.EF_EWS
    assert "static" in efg.last_error() and str(lim) in efg.last_error()
    # the sizes the header promises fit
    assert efg.ef_topk_workspace_bytes(1_000_000, 10_000) < lim
    assert efg.ef_topk_workspace_bytes(1 << 26, 1 << 16) < lim


def test_topk_workspace_sizes():
    # sample-based candidate capacity keeps the workspace far below the data
    n, k = 1_300_000_000, 1_300_000
    ws = efg.ef_topk_workspace_bytes(n, k)
    assert 0 < ws < 0.06 * 4 * n
    assert efg.ef_topk_workspace_bytes(1_000_000, 10_000) < 4 * 1_000_000
    # dense selections need no candidate slots
    assert efg.ef_topk_workspace_bytes(1 << 20, 1 << 19) < efg.ef_topk_workspace_bytes(1 << 20, 1 << 12) * 4


def test_segmented_argument_checks():
    L = efg.lib()
    off = np.array([0, 10, 5], np.int64)
    ks = np.array([1, 1], np.int64)
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    assert L.ef_topk_segmented_workspace_bytes(2, p(off), p(ks)) == 0
    rc = L.ef_topk_compress_segmented(FAKE, FAKE, 2, p(off), p(ks), FAKE, FAKE, FAKE, 1 << 30, None, None, 0, None)
    assert rc == efg.EF_EINVAL and "non-decreasing" in efg.last_error()
    off = np.array([0, 10, 20], np.int64)
    ks = np.array([1, 11], np.int64)
    rc = L.ef_topk_compress_segmented(FAKE, FAKE, 2, p(off), p(ks), FAKE, FAKE, FAKE, 1 << 30, None, None, 0, None)
    assert rc == efg.EF_EINVAL and "segment 1" in efg.last_error()
    off = np.array([0, 10, 20], np.int64)
    ks = np.array([1, 2], np.int64)
    need = L.ef_topk_segmented_workspace_bytes(2, p(off), p(ks))
    assert need > 0
    rc = L.ef_topk_compress_segmented(FAKE, FAKE, 2, p(off), p(ks), FAKE, FAKE, FAKE, need - 1, None, None, 0, None)
    assert rc == efg.EF_EWS
    assert L.ef_topk_compress_segmented(FAKE, FAKE, -1, None, None, FAKE, FAKE, FAKE, 0, None, None, 0, None) == efg.EF_EINVAL


def test_workspace_paths_argument_checks():
    """ef_topk_workspace_paths refuses, on the host, a workspace too small for
    the state of nseg tensors (its kernel would read past it), a NULL output
    and a negative nseg; nseg = 0 is a no-op."""
    L = efg.lib()
    off = np.array([0, 100_000, 300_000], np.int64)
    ks = np.array([100, 200], np.int64)
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    need = L.ef_topk_segmented_workspace_bytes(2, p(off), p(ks))
    assert L.ef_topk_workspace_paths(FAKE, 256, 2, FAKE, None) == efg.EF_EWS
    assert "workspace" in efg.last_error()
    assert L.ef_topk_workspace_paths(FAKE, need, 1_000_000, FAKE, None) == efg.EF_EWS
    assert L.ef_topk_workspace_paths(FAKE, need, 2, None, None) == efg.EF_EINVAL
    assert L.ef_topk_workspace_paths(FAKE, need, -1, FAKE, None) == efg.EF_EINVAL
    assert L.ef_topk_workspace_paths(FAKE, 0, 0, None, None) == efg.EF_OK


def test_bert_layout_workspace():
    import gen
    off, ks = gen.bert_segments()
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    need = efg.lib().ef_topk_segmented_workspace_bytes(len(ks), p(off), p(ks))
    assert 0 < need < 4 * int(off[-1])


def test_sign_argument_checks():
    L = efg.lib()
    ok = lambda **kw: L.ef_sign_compress(kw.get("g", FAKE), kw.get("e", FAKE), kw.get("m", FAKE), kw.get("n", 64),
                                         kw.get("b", 0.9), kw.get("c", 5.0), kw.get("s", FAKE), kw.get("bits", FAKE),
                                         None, kw.get("stats", None), kw.get("ws", None), kw.get("wsb", 0), None)
    assert ok(n=-1) == efg.EF_EINVAL
    assert ok(b=1.5) == efg.EF_EINVAL
    assert ok(b=float("nan")) == efg.EF_EINVAL
    assert ok(c=0.0) == efg.EF_EINVAL
    assert ok(m=None, e=None) == efg.EF_EINVAL  # m may be NULL (compress only), e may not
    assert ok(m=FAKE_ODD) == efg.EF_EINVAL
    assert ok(e=FAKE_ODD) == efg.EF_EINVAL
    assert ok(s=FAKE + 2) == efg.EF_EINVAL
    assert ok(stats=FAKE) == efg.EF_EWS
    assert ok(stats=FAKE, ws=FAKE, wsb=efg.lib().ef_sign_workspace_bytes(64) - 1) == efg.EF_EWS
    assert ok(stats=FAKE, ws=FAKE + 16, wsb=1 << 20) == efg.EF_EINVAL


def test_decode_and_sgd_argument_checks():
    L = efg.lib()
    assert L.sparse_decode_accumulate(FAKE, -1, 1, FAKE, FAKE, FAKE, None, None) == efg.EF_EINVAL
    assert L.sparse_decode_accumulate(FAKE, 10, -1, FAKE, FAKE, FAKE, None, None) == efg.EF_EINVAL
    assert L.sparse_decode_accumulate(FAKE, 10, 2, FAKE, None, FAKE, None, None) == efg.EF_EINVAL
    assert L.sgd_apply(FAKE, FAKE, -1, 0.1, None) == efg.EF_EINVAL
    assert L.sgd_apply(FAKE_ODD, FAKE, 16, 0.1, None) == efg.EF_EINVAL
    assert L.sgd_apply(None, FAKE, 16, 0.1, None) == efg.EF_EINVAL
    # the fused receiver step: sizes, missing packets, missing or misaligned w and G
    assert L.sparse_decode_sgd(FAKE, FAKE, -1, 1, FAKE, FAKE, FAKE, 0.1, None, None) == efg.EF_EINVAL
    assert L.sparse_decode_sgd(FAKE, FAKE, 10, -1, FAKE, FAKE, FAKE, 0.1, None, None) == efg.EF_EINVAL
    assert L.sparse_decode_sgd(FAKE, FAKE, 10, 2, FAKE, None, FAKE, 0.1, None, None) == efg.EF_EINVAL
    assert L.sparse_decode_sgd(None, FAKE, 10, 0, None, None, None, 0.1, None, None) == efg.EF_EINVAL
    assert L.sparse_decode_sgd(FAKE_ODD, FAKE, 16, 0, None, None, None, 0.1, None, None) == efg.EF_EINVAL
    assert L.sparse_decode_sgd(FAKE, FAKE_ODD, 16, 0, None, None, None, 0.1, None, None) == efg.EF_EINVAL


def test_encoding_argument_checks():
    L = efg.lib()
    assert L.encode_bitmap(FAKE, -1, 10, FAKE, None) == efg.EF_EINVAL
    assert L.encode_bitmap(None, 5, 10, FAKE, None) == efg.EF_EINVAL
    assert L.decode_bitmap(FAKE, 100, FAKE, 10, None, FAKE, 1 << 20, None) == efg.EF_EINVAL
    assert L.decode_bitmap(FAKE, 100, FAKE, 10, FAKE, FAKE, 0, None) == efg.EF_EWS
    assert L.encode_delta_bound(7) == 35
    assert L.encode_delta(FAKE, 10, FAKE, None, FAKE, 1 << 20, None) == efg.EF_EINVAL
    assert L.encode_delta(FAKE, 10, FAKE, FAKE, FAKE, 0, None) == efg.EF_EWS
    assert L.decode_delta(FAKE, -1, 10, FAKE, None, FAKE, 1 << 20, None) == efg.EF_EINVAL
    assert L.encode_blocks(FAKE, 10, 1000, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == efg.EF_EINVAL
    assert L.encode_blocks(FAKE, 10, 1000, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == efg.EF_EWS
    assert L.decode_blocks(FAKE, FAKE, FAKE, 1000, -1, FAKE, FAKE, 1 << 20, None) == efg.EF_EINVAL
    assert efg.lib().blocks_workspace_bytes(1_300_000, 1_300_000_000) < 64 << 20


def test_binding_never_uses_the_oracle():
    pkg = os.path.join(ROOT, "error_feedback_gradient_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                with open(os.path.join(dirpath, f)) as fh:
                    text = fh.read()
                assert "oracle" not in text.lower(), f


def test_random_sparsify_argument_checks():
    L = efg.lib()
    ws = L.ef_random_sparsify_workspace_bytes(100_000)
    assert ws > 100_000 // 8
    assert L.ef_random_sparsify_workspace_bytes(-1) == 0
    assert L.ef_random_sparsify_workspace_bytes(2**31) == 0
    call = lambda **kw: L.ef_random_sparsify(
        kw.get("g", FAKE), kw.get("e", FAKE), kw.get("n", 100_000), kw.get("k", 100), 1, 2, kw.get("v", FAKE),
        kw.get("i", FAKE), kw.get("cap", 300), kw.get("cnt", FAKE), None, None, kw.get("ws", FAKE),
        kw.get("wsb", ws), kw.get("flags", 0), None)
    assert call(n=-1) == efg.EF_EINVAL
    assert call(n=2**31) == efg.EF_EINVAL
    assert call(k=-1) == efg.EF_EINVAL
    assert call(cap=-1) == efg.EF_EINVAL
    assert call(flags=2) == efg.EF_EINVAL
    assert call(cnt=None) == efg.EF_EINVAL
    assert call(g=None) == efg.EF_EINVAL
    assert call(e=FAKE_ODD) == efg.EF_EINVAL and "aligned" in efg.last_error()
    assert call(v=None) == efg.EF_EINVAL
    assert call(ws=None) == efg.EF_EWS
    assert call(wsb=ws - 1) == efg.EF_EWS
    assert call(ws=FAKE + 16) == efg.EF_EINVAL
    # the bitmap dominates the workspace: about n/8 bytes
    assert L.ef_random_sparsify_workspace_bytes(1_300_000_000) < 1_300_000_000 // 8 + (8 << 20)


def test_adam_argument_checks():
    L = efg.lib()
    step = lambda **kw: L.ef_adam_step(kw.get("g", FAKE), kw.get("m", FAKE), kw.get("v", FAKE), kw.get("w", FAKE),
                                       kw.get("n", 64), kw.get("b1", 0.9), kw.get("b2", 0.999), 1e-3,
                                       kw.get("sb", 0.1), kw.get("eps", 1e-8), None, None)
    assert step(n=-1) == efg.EF_EINVAL
    assert step(b1=1.5) == efg.EF_EINVAL
    assert step(b2=float("nan")) == efg.EF_EINVAL
    assert step(sb=0.0) == efg.EF_EINVAL
    assert step(eps=-1.0) == efg.EF_EINVAL
    assert step(g=None) == efg.EF_EINVAL
    assert step(v=FAKE_ODD) == efg.EF_EINVAL
    upd = lambda **kw: L.ef_onebit_adam_update(kw.get("q", FAKE), kw.get("nw", 1), kw.get("m", FAKE), FAKE, FAKE,
                                               64, 0.9, 1e-3, 0.1, 1e-8, None, None)
    assert upd(nw=0) == efg.EF_EINVAL
    assert upd(nw=128) == efg.EF_EINVAL
    assert upd(q=None) == efg.EF_EINVAL
    assert upd(q=FAKE + 2) == efg.EF_EINVAL
    assert upd(m=None) == efg.EF_EINVAL
    var = lambda **kw: L.ef_onebit_adam_update_var(FAKE, kw.get("nw", 1), FAKE, FAKE, FAKE, 64, 0.9,
                                                   kw.get("b2", 0.999), 1e-3, 0.1, 1e-8, None, None)
    assert var(nw=0) == efg.EF_EINVAL
    assert var(b2=1.5) == efg.EF_EINVAL


def test_adam_scalars_match_the_oracle_helper():
    """ef_adam_scalars (the library's host arithmetic) gives the oracle's
    scalars, which test_oracle_adam pins through torch.optim.Adam."""
    import oracle
    for args in [(2e-5, 0.9, 0.999, 1), (1e-3, 0.9, 0.999, 100, 10), (0.1, 0.5, 0.9, 7, 7)]:
        assert efg.adam_scalars(*args) == oracle.adam_scalars(*args)
    r = np.random.default_rng(77)
    for _ in range(2000):
        lr = float(10.0 ** r.uniform(-7, 0))
        b1, b2 = float(r.choice([0.0, 0.5, 0.9, 0.95, r.uniform(0, 1)])), float(r.choice([0.9, 0.99, 0.999, 0.9999]))
        t = int(r.integers(1, 100_000))
        tv = int(r.integers(1, t + 1))
        assert efg.adam_scalars(lr, b1, b2, t, tv) == oracle.adam_scalars(lr, b1, b2, t, tv), (lr, b1, b2, t, tv)
    L = efg.lib()
    a, b = C.c_float(), C.c_float()
    assert L.ef_adam_scalars(1e-3, 1.0, 0.999, 1, 1, C.byref(a), C.byref(b)) == efg.EF_EINVAL
    assert L.ef_adam_scalars(1e-3, 0.9, 0.999, 0, 1, C.byref(a), C.byref(b)) == efg.EF_EINVAL
    assert L.ef_adam_scalars(1e-3, 0.9, 0.999, 1, 0, C.byref(a), C.byref(b)) == efg.EF_EINVAL
    assert L.ef_adam_scalars(float("inf"), 0.9, 0.999, 1, 1, C.byref(a), C.byref(b)) == efg.EF_EINVAL
    assert L.ef_adam_scalars(1e-3, 0.9, 0.999, 1, 1, None, C.byref(b)) == efg.EF_EINVAL
