"""Host-side fuzz of libefgrad: the plan and layout builders, the plan cache
and every entry point's argument checks, called through the C ABI with
random sizes, layouts and pointers that no kernel ever dereferences (nothing
is enqueued: each call stops at a host check, or at the first HIP call where
there is no GPU).  Run by tests/test_sanitizers.py against a build whose host
code has AddressSanitizer and UndefinedBehaviorSanitizer, so that a host-side
out-of-bounds access or undefined operation aborts it.

    python tests/host_fuzz.py LIBRARY [CASES]
"""
import ctypes as C
import os
import sys

import numpy as np

FAKE = 0x10000  # 16- and 256-byte aligned, never dereferenced on these paths


def main(path, cases=3000):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import torch

    if torch.cuda.device_count() > 0:
        # the pointers below are fake: with a GPU, calls that pass their host
        # checks would launch kernels on them
        raise SystemExit("host_fuzz runs only where no GPU is visible")
    import error_feedback_gradient_amd as efg

    efg.LIB_PATH = path
    L = efg.lib()
    r = np.random.default_rng(20261202)
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    sizes = lambda: int(r.choice([0, 1, 2, 3, 255, 256, 4095, 4096, 4097, r.integers(0, 1 << 20),
                                  r.integers(0, 1 << 31)]))
    for case in range(cases):
        # flat top-k: workspace query and argument checks
        n = sizes()
        k = int(r.choice([0, 1, n, max(0, n - 1), n // 1000, n // 100, n // 3, n + 1, -1]))
        L.ef_topk_workspace_bytes(n, k)
        L.ef_topk_compress(FAKE, FAKE, n, k, FAKE, FAKE, None, 0, None, None, int(r.integers(0, 3)), None)
        L.ef_topk_compress_noalloc(FAKE, FAKE, n, k, FAKE, FAKE, None, None, int(r.integers(0, 3)), None)
        # layer-wise: random tables (some invalid), through the plan cache
        nseg = int(r.choice([0, 1, 2, 11, 12, 40, int(r.integers(1, 300))]))
        lens = r.integers(0, int(r.choice([10, 5000, 3_000_000])), size=nseg)
        off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        ks = np.array([int(r.integers(0, m + 1)) for m in lens], np.int64)
        if nseg and r.random() < 0.1:
            ks[int(r.integers(0, nseg))] = -1 if r.random() < 0.5 else int(lens.max()) + 1
        if nseg and r.random() < 0.05:
            off[int(r.integers(1, nseg + 1))] = -5
        need = L.ef_topk_segmented_workspace_bytes(nseg, p(off), p(ks))
        ws = FAKE if r.random() < 0.5 else None
        L.ef_topk_compress_segmented(FAKE, FAKE, nseg, p(off), p(ks), FAKE, FAKE, ws,
                                     int(need) if r.random() < 0.5 else int(need) // 2, None, None, 0, None)
        # the other entry points' checks
        L.ef_sign_workspace_bytes(n)
        L.ef_sign_compress(FAKE, FAKE, FAKE if r.random() < 0.5 else None, n, float(r.uniform(-0.5, 1.5)),
                           float(r.choice([5.0, 0.0, -1.0, np.inf])), FAKE, FAKE, None, None, None, 0, None)
        L.ef_random_sparsify_workspace_bytes(n)
        L.ef_random_sparsify(FAKE, FAKE, n, k, 1, 2, FAKE, FAKE, int(r.integers(-1, 100)), FAKE, None, None,
                             FAKE if r.random() < 0.5 else None, int(r.integers(0, 1 << 30)), 0, None)
        L.ef_quantize_workspace_bytes(k)
        L.ef_quantize_int8(FAKE, FAKE, k, FAKE, n, FAKE, None, FAKE, int(r.integers(0, 8192)), None)
        npk = int(r.integers(-1, 70))
        L.sparse_decode_accumulate(FAKE, n, npk, FAKE, FAKE, FAKE, None, None) if npk < 0 else None
        L.sgd_apply(FAKE if r.random() < 0.9 else None, FAKE, -abs(n) if r.random() < 0.1 else 0, 0.1, None)
        L.encode_delta_bound(k)
        L.delta_workspace_bytes(k)
        L.blocks_workspace_bytes(k, n)
        L.decode_bitmap_workspace_bytes(n)
        L.encode_blocks(None, k, n, None, None, None, None, None, 0, None)
        L.decode_blocks(None, None, None, n, k, None, None, 0, None)
        a, b = C.c_float(), C.c_float()
        L.ef_adam_scalars(float(10.0 ** r.uniform(-8, 1)), float(r.uniform(-0.1, 1.1)), float(r.uniform(-0.1, 1.1)),
                          int(r.integers(-2, 1 << 20)), int(r.integers(-2, 1 << 20)), C.byref(a), C.byref(b))
        L.ef_adam_step(FAKE, FAKE, FAKE, FAKE, -1 if r.random() < 0.5 else n, 0.9, 0.999, 1e-3, 0.0, 1e-8, None, None)
        L.ef_onebit_adam_update(FAKE, int(r.integers(-1, 200)), FAKE, FAKE, FAKE, -1, 0.9, 1e-3, 0.5, 1e-8,
                                None, None)
        L.ef_last_error()
    print(f"host fuzz: {cases} cases", flush=True)


if __name__ == "__main__":
    main(sys.argv[1], int(sys.argv[2]) if len(sys.argv) > 2 else 3000)
