"""Benchmark of the error-feedback top-k step on one MI355X.

Workload: a flat float32 gradient of N = 1,300,000,000 log-normal magnitudes
(mu = -7, sigma = 2) with random signs, k = 1,300,000 (0.1 %), residual
carried from step to step, output also block-encoded (256-element blocks).
One step = ef_topk_compress + encode_blocks on fresh gradient data already
resident in HBM.

    python bench.py [--gpus 1] [--steps 5] [--warmup 2]

Prints one JSON line: elements/s of the whole step, HBM roofline of the
streaming kernel (12 algorithmic bytes per element: read g, read e, write e)
timed with HIP events that its own dispatches record on the library's
stream, over the timed region's K steps run once more right after it
(events on each launch slow the issue of a short step, so the timed steps
carry none), and the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "EF top-k compress elems/s & HBM GB/s (% of peak) at 1.3B fp32, 1 GPU"
PEAK_HBM_GBPS = 8000.0
STREAM_BYTES_PER_ELEM = 12  # read g, read e, write e


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# committed rocprofv3 traffic summaries of the roofline kernel of other workloads
TRAFFIC_PROFILES = {"random": "rs_accum_large_1p3e9_traffic", "adam": "onebit_update_adam_340m_traffic",
                    "decode": "decode_sgd_25p6m_traffic",
                    "sign": "sign_ef_340m_traffic"}


def measured_traffic(name="topk_stream_large_1p3e9_traffic"):
    """HBM bytes per launch of a kernel from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (profiles/<name>.json), or None if the kernel sources
    changed since."""
    import hashlib

    path = os.path.join(ROOT, "profiles", name + ".json")
    try:
        rec = json.load(open(path))
        src = b"".join(open(os.path.join(ROOT, p), "rb").read() for p in rec["sources"])
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return rec["traffic_bytes"]


def pin_one_core():
    """Pins the calling thread to its first allowed core (the oracle is
    single-threaded); returns the previous affinity set, or None if pinning is
    not available."""
    try:
        prev = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {sorted(prev)[0]})
        return prev
    except (AttributeError, OSError):
        return None


def unpin(prev):
    if prev:
        os.sched_setaffinity(0, prev)


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "the host CPU"


def cpu_baseline(n_sample: int, k_sample: int):
    """The oracle as it stands, single-threaded, on the first n_sample elements
    of the step-0 gradient (numpy stream), e = 0."""
    import numpy as np

    import gen
    import oracle

    g = gen.large_gradient(0, n=n_sample)
    e = np.zeros(n_sample, np.float32)
    prev = pin_one_core()
    cores = 1  # the oracle runs on one thread
    t0 = time.perf_counter()
    oracle.topk(g, e, k_sample)
    dt = time.perf_counter() - t0
    unpin(prev)
    model = host_cpu_model()
    return {
        "value": n_sample / dt,
        "unit": "elems/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"first {n_sample:,} elements of the step-0 log-normal gradient, k = {k_sample:,}, e = 0; "
                  f"{dt:.2f} s on one core of {model} ({os.cpu_count()} logical CPUs); the oracle ranks by a full "
                  f"sort (O(n log n)), so at the configured N = 1.3e9 its rate per element would be lower still",
        "seconds": dt,
        "GBps_algorithmic": STREAM_BYTES_PER_ELEM * n_sample / dt / 1e9,
    }


# chained steps of each workload's recipe; the default number of timed steps
CHAIN_STEPS = {"flat": 10, "bert": 20, "sign": 50, "large": 5}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: the workload's chained steps: 10 flat, 20 bert, 50 sign, else 5)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--n", type=int, default=None, help="override N (testing only)")
    ap.add_argument("--k", type=int, default=None, help="override k (testing only)")
    ap.add_argument("--cpu-sample", type=int, default=80_000_000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stats", action="store_true", help="also compute the fused monitoring statistics")
    ap.add_argument("--workload", default="large", choices=["large", "flat", "bert", "sign", "decode", "quant", "random", "adam"],
                    help="large (default, the headline) or one of the other workloads")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = CHAIN_STEPS.get(args.workload, 5)
    if args.gpus != 1:
        print(f"bench.py: this library measures one GPU's share of the gradient; --gpus {args.gpus} is not "
              "supported (run with --gpus 1).", file=sys.stderr, flush=True)
        sys.exit(2)

    if args.workload != "large":
        other_workload(args)
        return

    import torch

    import error_feedback_gradient_amd as efg
    import gen

    dev = torch.device("cuda:0")
    n = args.n or gen.LARGE_N
    k = args.k or (gen.LARGE_K if args.n is None else max(1, n // 1000))
    W, K = args.warmup, args.steps
    log(f"bench: N={n:,} k={k:,} warmup={W} steps={K}; drawing {W + K} gradients on the device")
    grads = [gen.large_gradient_device(t, n, dev) for t in range(W + K)]
    e = torch.zeros(n, dtype=torch.float32, device=dev)
    vals = torch.empty(k, dtype=torch.float32, device=dev)
    idx = torch.empty(k, dtype=torch.int32, device=dev)
    ws = efg.workspace(efg.ef_topk_workspace_bytes(n, k), dev)
    nb = (n + 255) // 256
    mask = torch.empty((nb + 7) // 8, dtype=torch.uint8, device=dev)
    counts = torch.empty(min(k, nb), dtype=torch.uint8, device=dev)
    offs = torch.empty(k, dtype=torch.uint8, device=dev)
    nblk = torch.empty(1, dtype=torch.int64, device=dev)
    wsb = efg.workspace(efg.lib().blocks_workspace_bytes(k, n), dev)
    nonfinite = torch.zeros(1, dtype=torch.int32, device=dev)

    stats = torch.zeros(2, dtype=torch.float64, device=dev) if args.stats else None

    def step(t):
        efg.ef_topk_compress(grads[t], e, k, vals=vals, idx=idx, ws=ws, nonfinite=nonfinite, stats=stats)
        efg.encode_blocks(idx, n, mask=mask, counts_m1=counts, offs=offs, nblk_out=nblk, ws=wsb)

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    log("bench: warmup done")

    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for t in range(W, W + K):
        step(t)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    stream_ms, launches = kernel_ms(step, range(W, W + K), "topk_stream")
    ms_per_step = total_ms / K
    stream_avg_ms = stream_ms / max(1, launches)
    achieved = STREAM_BYTES_PER_ELEM * n / (stream_avg_ms * 1e-3) / 1e9
    log(f"bench: {ms_per_step:.3f} ms/step, stream kernel {stream_avg_ms:.3f} ms ({achieved:.0f} GB/s)")

    # one more step with every kernel timed, for the breakdown (not part of the timed region)
    efg.profile_enable(True)
    step(0)
    torch.cuda.synchronize()
    labels = ["topk_init", "topk_sample_hist", "topk_sample_select", "topk_stream", "topk_compact",
              "topk_hist", "topk_write",
              "blocks_clear", "blocks_count", "blocks_scan", "blocks_write", "blocks_mask"]
    breakdown = {}
    for lab in labels:
        ms, cnt = efg.profile_read(lab)
        if cnt:
            breakdown[lab] = round(ms, 4)
    efg.profile_enable(False)

    # per-step spread of the whole step and of the compression alone
    steps_ms = per_step_ms(step, range(W, W + K), dev)
    compress_ms = per_step_ms(
        lambda t: efg.ef_topk_compress(grads[t], e, k, vals=vals, idx=idx, ws=ws, nonfinite=nonfinite, stats=stats),
        range(W, W + K), dev)
    # one more step, verified: the packet and the residual are the top-k of
    # x = g + e by the invariants that fix it, and the block encoding decodes
    # back to the packet
    t_last = W + K - 1
    x = grads[t_last] + e
    step(t_last)
    torch.cuda.synchronize()
    ok = topk_invariants(x, vals, idx, k, e) and int(nonfinite.item()) == 0
    del x
    back = efg.decode_blocks(mask, counts, offs, n, k)
    ok = ok and torch.equal(back, idx)
    if not ok:
        raise SystemExit("bench: the last step's packet is not the top-k of its input")

    # Same-run references, outside the timed region: the step forced onto the
    # exact full-pass selection, and the stream alone (k = 0: read g, read e,
    # write e, no selection), i.e. the rate of the bare 12 B/element pattern on
    # this box beside the streaming kernel's.
    forced_ms = per_step_ms(
        lambda t: efg.ef_topk_compress(grads[t], e, k, vals=vals, idx=idx, ws=ws,
                                       flags=efg.EF_FLAG_FORCE_FALLBACK), range(W, W + min(K, 3)), dev)
    efg.profile_enable(True, "topk_stream")
    for t in range(W, W + K):
        efg.ef_topk_compress(grads[t], e, 0, ws=ws)
    bare_ms, bare_n = efg.profile_read("topk_stream")
    efg.profile_enable(False)
    bare_gbps = STREAM_BYTES_PER_ELEM * n / (bare_ms / max(1, bare_n) * 1e-3) / 1e9
    log(f"bench: forced fallback {forced_ms['median']:.3f} ms/step, bare stream {bare_gbps:.0f} GB/s")
    drift = drift_chain(lambda g_, e_: efg.ef_topk_compress(g_, e_, k, vals=vals, idx=idx, ws=ws),
                        grads[:2], n, ws, [k], 1000 if args.n is None else 200, dev)
    log(f"bench: {drift['steps']} drifted steps: median {drift['median_ms']:.3f} ms, "
        f"{drift['fallback_steps']} on the exact fallback")

    del grads
    add_gbps = add_ceiling(dev)  # before the copies: those calibrate the counters
    copy_gbps = torch_copy(dev)

    result = {
        "metric": METRIC,
        "value": n / (ms_per_step * 1e-3),
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "EF top-k step on a flat fp32 gradient, N=1.3e9 log-normal(-7,2) magnitudes with random "
                        "signs, k=1.3e6 (0.1%), residual carried, block-sparse output (256-element blocks)"
            if args.n is None else f"reduced test size N={n}",
            "n": n,
            "k": k,
            "step": "ef_topk_compress + encode_blocks" + (" (with monitoring statistics)" if args.stats else ""),
            "parallelism": "single GPU",
        },
        "hbm_GBps_step": STREAM_BYTES_PER_ELEM * n / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac_step": STREAM_BYTES_PER_ELEM * n / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {
            "kernel": "topk_stream",
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": measured_traffic(),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "avg_ms": stream_avg_ms,
            "launches": launches,
        },
        "bare_stream_GBps": bare_gbps,
        "bare_stream_frac": bare_gbps / PEAK_HBM_GBPS,
        "forced_fallback_ms": forced_ms,
        "drift_chain": drift,
        "torch_copy_GBps": copy_gbps,
        "torch_add_GBps": add_gbps,
        "kernel_ms_one_step": breakdown,
        "step_ms": steps_ms,
        "compress_only_ms": compress_ms,
        "verified": ok,
    }
    if not args.no_cpu_baseline:
        log(f"bench: CPU oracle on {args.cpu_sample:,} elements")
        result["cpu_baseline"] = cpu_baseline(args.cpu_sample, max(1, args.cpu_sample // 1000))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def add_ceiling(dev):
    """torch's own elementwise a += b over 2^29 float32, ten times: read a, read
    b, write a, the streaming pass's 12 B/element with no selection work.  GB/s
    on that traffic, beside the streaming kernel's."""
    import torch

    stream = torch.cuda.current_stream(dev)
    a = torch.zeros(1 << 29, dtype=torch.float32, device=dev)
    b = torch.ones_like(a)
    a.add_(b)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        a.add_(b)
    c1.record(stream)
    torch.cuda.synchronize()
    gbps = 12 * a.numel() * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del a, b
    return gbps


def torch_copy(dev):
    """torch's device copy of 2 GiB, ten times (read + write GB/s): a reference
    rate of the same box (not a ceiling: the streaming kernel runs faster), and
    the known-size kernel that calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE
    counters in the same process."""
    import torch

    stream = torch.cuda.current_stream(dev)
    a = torch.empty(1 << 29, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        b.copy_(a)
    c1.record(stream)
    torch.cuda.synchronize()
    gbps = 2 * a.numel() * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del a, b
    return gbps


def topk_invariants(x, vals, idx, k, e_after):
    """True when (vals, idx, e_after) is the top-k of x: k strictly increasing
    in-range indices, vals = x[idx] bit for bit, every kept key (|x| bits) >=
    every dropped key with ties kept by lower index, and e_after = x except
    +0 at idx.  These properties fix the result uniquely, so the check needs
    no second implementation of the selection.  Device tensors."""
    import torch

    n = x.numel()
    ik = idx.long()
    if idx.numel() != k:
        return False
    if k == 0:
        return torch.equal(e_after.view(torch.int32), x.view(torch.int32))
    ok = bool((ik[1:] > ik[:-1]).all()) and int(ik[0]) >= 0 and int(ik[-1]) < n
    ok = ok and torch.equal(vals.view(torch.int32), x[ik].view(torch.int32))
    if ok and k < n:
        key = x.view(torch.int32) & 0x7FFFFFFF
        kept = torch.zeros(n, dtype=torch.bool, device=x.device)
        kept[ik] = True
        T = int(key[ik].min())
        dmax = int(key.masked_fill(kept, -1).max())
        ok = T >= dmax
        if ok and T == dmax:
            ok = int(ik[key[ik] == T].max()) < int(torch.nonzero((key == T) & ~kept)[0, 0])
        del key, kept
    if ok:
        want = x.clone()
        want[ik] = 0.0
        ok = torch.equal(e_after.view(torch.int32), want.view(torch.int32))
    return ok


def sign_bits_agree(sgn, bits):
    """int8 signs in {-1, 0, +1} and the packed bits equal (sign == +1), LSB
    first, zero padding.  Device tensors."""
    import torch

    n = sgn.numel()
    if not bool(((sgn >= -1) & (sgn <= 1)).all()):
        return False
    pos = torch.zeros(((n + 7) // 8) * 8, dtype=torch.int32, device=sgn.device)
    pos[:n] = (sgn == 1).int()
    w = torch.tensor([1, 2, 4, 8, 16, 32, 64, 128], dtype=torch.int32, device=sgn.device)
    return torch.equal((pos.view(-1, 8) * w).sum(1).to(torch.uint8), bits)


def kernel_ms(step, steps, kernel_label):
    """The steps once more, right after the timed region, with every launch of
    the kernels labelled kernel_label timed by a HIP event pair that its own
    dispatch records (on the stream the library launches on): (total ms,
    launches).  Kept out of the timed region: a launch that records events
    takes longer to issue, which would show in a short step."""
    import torch

    import error_feedback_gradient_amd as efg

    efg.profile_enable(True, kernel_label)
    for t in steps:
        step(t)
    torch.cuda.synchronize()
    ms, launches = efg.profile_read(kernel_label)
    efg.profile_enable(False)
    return ms, launches


def time_steps(step, W, K, kernel_label):
    """Runs W untimed and K timed steps (HIP events on the current stream), then
    times the labelled kernel over the same K steps (kernel_ms); returns (ms per
    step, ms of the labelled kernels per step, their launch count)."""
    import torch

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for t in range(W, W + K):
        step(t)
    stop.record()
    torch.cuda.synchronize()
    kms, launches = kernel_ms(step, range(W, W + K), kernel_label)
    # time of the labelled kernels per step (equal to the mean launch when one kernel matches)
    return start.elapsed_time(stop) / K, kms / K, launches


def drift_chain(call, g_pair, n, ws, ks, steps, dev):
    """Outside the timed region: `steps` chained top-k calls from a zero
    residual with two gradients alternating.  That is a drift: the residual of
    every coordinate that is not kept grows step after step until it is, so
    the values crowd just below the threshold, the regime where the sample's
    candidate window matters most.  Each call is timed by its own HIP events,
    and ef_topk_workspace_paths records each tensor's path and candidates.
    Returns {"steps", "median_ms", "p90_ms", "fallback_steps" (steps on which
    some tensor took the exact full-pass selection), "max_candidates_over_k"}."""
    import numpy as np
    import torch

    import error_feedback_gradient_amd as efg

    ks = np.asarray(ks, np.int64)
    e = torch.zeros(n, dtype=torch.float32, device=dev)
    paths = torch.empty((steps, ks.size, 2), dtype=torch.int32, device=dev)
    evs = []
    for t in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call(g_pair[t % 2], e)
        b.record()
        efg.ef_topk_workspace_paths(ws, int(ks.size), out=paths[t])
        evs.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    p = paths.cpu().numpy()
    sel = ks > 0
    ratio = float((p[:, sel, 1] / ks[sel][None, :]).max()) if sel.any() else 0.0
    del e
    return {"steps": steps, "gradients": "two of the workload's gradients alternating, from a zero residual",
            "median_ms": ms[len(ms) // 2], "p90_ms": ms[int(0.9 * (len(ms) - 1))],
            "fallback_steps": int((p[:, :, 0].sum(axis=1) > 0).sum()), "max_candidates_over_k": ratio}


def per_step_ms(step, steps, dev, flush_bytes=0):
    """Each step bracketed by its own HIP events (outside the contract's timed
    region): {"median", "min"} in ms.  With flush_bytes, a scratch buffer of
    that size is read (summed) before every step, so that the step starts with
    a cold 256 MB Infinity Cache and no dirty lines of other data waiting to be
    written back (a write flush would charge the step with writing the
    scratch's last 256 MB to HBM)."""
    import statistics

    import torch

    scratch = torch.ones(flush_bytes // 4, dtype=torch.float32, device=dev) if flush_bytes else None
    times = []
    for t in steps:
        if scratch is not None:
            float(scratch.sum())
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step(t)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    return {"median": statistics.median(times), "min": min(times), "steps": len(times)}


def other_workload(args):
    """One JSON line for a non-headline workload (per-kernel roofline evidence)."""
    import numpy as np
    import torch

    import error_feedback_gradient_amd as efg
    import gen
    import oracle

    dev = torch.device("cuda:0")
    W, K = args.warmup, args.steps
    wl = args.workload
    cpu = None
    # the oracle timings below run on one pinned core (the thread is unpinned
    # before the GPU is timed)
    pinned = None if args.no_cpu_baseline else pin_one_core()
    if wl == "flat":
        n, k = gen.FLAT_N, gen.FLAT_K
        grads = [torch.from_numpy(gen.flat_gradient(t)).to(dev) for t in range(W + K)]
        e = torch.zeros(n, device=dev)
        ws = efg.workspace(efg.ef_topk_workspace_bytes(n, k), dev)
        vals = torch.empty(k, device=dev)
        idx = torch.empty(k, dtype=torch.int32, device=dev)
        step = lambda t: efg.ef_topk_compress(grads[t], e, k, vals=vals, idx=idx, ws=ws)
        label, bpe, units, unit = "topk_stream", 12, n, "elems/s"
        metric = "EF top-k compress elems/s, flat N=1e6 fp32, k=1e4"
        desc = "flat fp32 gradient N=1e6 N(0,1), k=1e4 (1%), residual carried"
        if not args.no_cpu_baseline:
            g0 = gen.flat_gradient(0)
            t0 = time.perf_counter()
            oracle.topk(g0, np.zeros(n, np.float32), k)
            cpu = (n, time.perf_counter() - t0, f"one full step, N = {n:,}, k = {k:,}")
    elif wl == "bert":
        off, ks = gen.bert_segments()
        n = int(off[-1])
        grads = [torch.from_numpy(gen.bert_gradient(t)).to(dev) for t in range(W + K)]
        e = torch.zeros(n, device=dev)
        ws = efg.workspace(efg.ef_topk_segmented_workspace_bytes(off, ks), dev)
        K_ = int(ks.sum())
        vals = torch.empty(K_, device=dev)
        idx = torch.empty(K_, dtype=torch.int32, device=dev)
        step = lambda t: efg.ef_topk_compress_segmented(grads[t], e, off, ks, vals=vals, idx=idx, ws=ws)
        label, bpe, units, unit = "topk_stream", 12, n, "elems/s"
        metric = "Layer-wise EF top-k compress elems/s, BERT-base 194 tensors fp32"
        desc = "BERT-base layer-wise top-k (194 tensors, 108,888,576 elements, K=368,208), residual carried"
        if not args.no_cpu_baseline:
            g0 = gen.bert_gradient(0)
            t0 = time.perf_counter()
            oracle.topk_segmented(g0, np.zeros(n, np.float32), off, ks)
            cpu = (n, time.perf_counter() - t0, "one full layer-wise step over all 194 tensors")
    elif wl == "sign":
        n = gen.SIGN_N
        grads = [gen.sign_gradient_device(t, n, dev) for t in range(W + K)]
        e = torch.zeros(n, device=dev)
        m = torch.zeros(n, device=dev)
        sgn = torch.empty(n, dtype=torch.int8, device=dev)
        bits = torch.empty((n + 7) // 8, dtype=torch.uint8, device=dev)
        step = lambda t: efg.ef_sign_compress(grads[t], e, m, gen.SIGN_BETA1, gen.SIGN_CLIP, sign_out=sgn, bits=bits)
        label, bpe, units, unit = "sign_ef", 21.125, n, "elems/s"
        metric = "1-bit sign EF + momentum elems/s, N=340M fp32"
        desc = "1-bit sign EF + momentum, N=340M, int8 sign + packed bits, beta1=0.9, clip 5"
        if not args.no_cpu_baseline:
            ns = 40_000_000
            g0 = gen.sign_gradient(0, n=ns)
            z = np.zeros(ns, np.float32)
            t0 = time.perf_counter()
            oracle.sign(g0, z, z, gen.SIGN_BETA1, gen.SIGN_CLIP)
            cpu = (ns, time.perf_counter() - t0, f"first {ns:,} elements of the step-0 gradient")
    elif wl == "quant":
        n, k = gen.LARGE_N, gen.LARGE_K
        idx_h = gen.sorted_unique_indices(n, k, 405)
        v_h = gen.large_gradient(11, n=k)
        vals = torch.from_numpy(v_h).to(dev)
        idx = torch.from_numpy(idx_h).to(dev)
        e = torch.zeros(n, device=dev)
        q = torch.empty(k, dtype=torch.int8, device=dev)
        sc = torch.empty(1, device=dev)
        wsq = efg.workspace(efg.lib().ef_quantize_workspace_bytes(k), dev)
        step = lambda t: efg.ef_quantize_int8(vals, idx, e, q=q, scale=sc, ws=wsq)
        # read v twice and idx once, write q and one residual word per entry
        label, bpe, units, unit = "quant_", 17, k, "entries/s"
        metric = "8-bit packet quantisation entries/s, k=1.3e6 of N=1.3e9"
        desc = "8-bit quantisation of a 1.3e6-entry packet (values of the large workload's law) into int8 with one scale, error kept in the residual"
        if not args.no_cpu_baseline:
            t0 = time.perf_counter()
            oracle.quantize_int8(v_h, np.arange(k, dtype=np.int32), np.zeros(k, np.float32))
            cpu = (k, time.perf_counter() - t0, f"one full packet, k = {k:,}")
    elif wl == "adam":
        n = gen.ADAM_N
        b1, b2, eps, lr = gen.ADAM_BETA1, gen.ADAM_BETA2, gen.ADAM_EPS, gen.ADAM_LR
        grads = [gen.sign_gradient_device(t, n, dev) for t in range(W + K)]
        w = gen.adam_weights_device(n, dev)
        m, v, e = torch.zeros(n, device=dev), torch.zeros(n, device=dev), torch.zeros(n, device=dev)
        q = torch.empty(n, dtype=torch.int8, device=dev)
        bits = torch.empty((n + 7) // 8, dtype=torch.uint8, device=dev)
        # the state after the warm-up phase: full-precision steps first (untimed)
        for t in range(1, gen.ADAM_WARMUP + 1):
            ss, sb = efg.adam_scalars(lr, b1, b2, t)
            efg.ef_adam_step(grads[0], m, v, w, b1, b2, ss, sb, eps)

        def step(t):
            # one compression-phase step on one worker: signs (int8 for the local
            # sum, packed bits for the wire), then momentum and update
            ss, sb = efg.adam_scalars(lr, b1, b2, gen.ADAM_WARMUP + 1 + t, gen.ADAM_WARMUP)
            efg.ef_sign_compress(grads[t], e, None, b1, gen.SIGN_CLIP, sign_out=q, bits=bits)
            efg.ef_onebit_adam_update(q, 1, m, v, w, b1, ss, sb, eps)
        label, bpe, units, unit = "onebit_update", 21, n, "elems/s"
        metric = "1-bit Adam compression-phase step elems/s, N=340M fp32"
        desc = ("1-bit Adam step on one worker, N=340M: compress-only sign EF (int8 + packed bits), then momentum "
                "on the signs, frozen variance and the Adam parameter update; lr 2e-5, betas 0.9/0.999")
        if not args.no_cpu_baseline:
            ns = 20_000_000
            g0 = gen.sign_gradient(0, n=ns)
            z = np.zeros(ns, np.float32)
            w0 = gen.adam_weights(ns)
            vv = np.full(ns, 1e-6, np.float32)
            ss, sb = efg.adam_scalars(lr, b1, b2, 4, 3)
            t0 = time.perf_counter()
            _, _, q0, _, _ = oracle.sign(g0, z, None, b1, gen.SIGN_CLIP)
            oracle.onebit_adam_update(q0, 1, z, vv, w0, b1, ss, sb, eps)
            cpu = (ns, time.perf_counter() - t0, f"first {ns:,} elements of one compression-phase step")
    elif wl == "random":
        n, k, seed = gen.LARGE_N, gen.LARGE_K, gen.RANDOM_SEED
        grads = [gen.large_gradient_device(t, n, dev) for t in range(W + K)]
        e = torch.zeros(n, device=dev)
        cap = 2 * k + 64
        vals = torch.empty(cap, device=dev)
        idx = torch.empty(cap, dtype=torch.int32, device=dev)
        cnt = torch.empty(1, dtype=torch.int64, device=dev)
        wsr = efg.workspace(efg.lib().ef_random_sparsify_workspace_bytes(n), dev)
        step = lambda t: efg.ef_random_sparsify(grads[t], e, k, seed, t, cap=cap, vals=vals, idx=idx, count=cnt,
                                                ws=wsr)
        # rs_accum reads g and e and writes e back (x = g + e)
        label, bpe, units, unit = "rs_accum", 12, n, "elems/s"
        metric = "EF random sparsification elems/s, N=1.3e9 fp32, expected k=1.3e6"
        desc = ("random magnitude-proportional sparsification of the large workload's gradient law, N=1.3e9, "
                "expected k=1.3e6, Philox draws, index-ordered output, residual carried")
        if not args.no_cpu_baseline:
            ns = 10_000_000
            g0 = gen.large_gradient(0, n=ns)
            t0 = time.perf_counter()
            oracle.random_sparsify(g0, np.zeros(ns, np.float32), ns // 1000, seed, 0)
            cpu = (ns, time.perf_counter() - t0, f"first {ns:,} elements of the step-0 gradient, k = {ns // 1000:,}")
    else:
        n, P, kp = gen.DECODE_N, gen.DECODE_PACKETS, gen.DECODE_K
        idx_l, val_l = [], []
        for p in range(P):
            g = gen.decode_packet_gradient(p)
            sel = np.sort(np.argpartition(-np.abs(g), kp - 1)[:kp]).astype(np.int32)
            idx_l.append(sel)
            val_l.append(g[sel])
        vals = torch.from_numpy(np.concatenate(val_l)).to(dev)
        idx = torch.from_numpy(np.concatenate(idx_l)).to(dev)
        pk_off = torch.arange(0, (P + 1) * kp, kp, dtype=torch.int64, device=dev)
        G = torch.zeros(n, device=dev)
        w = torch.from_numpy(gen.decode_weights()).to(dev)

        def step(t):
            # the receiver's step in one pass: G from zero, the packets, w -= lr G
            efg.sparse_decode_sgd(w, vals, idx, pk_off, gen.DECODE_LR, G=G)

        def three_calls(t):
            G.zero_()
            efg.sparse_decode_accumulate(G, vals, idx, pk_off)
            efg.sgd_apply(w, G, gen.DECODE_LR)
        # decode_sgd must read w and write G whole (8 B per element), read the
        # packets (8 B per entry) and write w where it changes (at most one
        # float per entry): 8 + 12 * 409,600 / 25.6e6 = 8.19 B per element.
        # Writing every element of w back would make it 12.
        label, bpe, units, unit = "decode_sgd", 8 + 12 * P * kp / n, n, "elems/s"
        metric = "Sparse decode (16 packets) + SGD elems/s, N=25.6M fp32"
        desc = ("16 top-0.1% packets (25,600 entries each) scatter-added in packet order into G[25.6M] from zero, "
                "then w -= 0.1 G, in one pass (sparse_decode_sgd); w and G (205 MB) fit the 256 MB last-level cache, "
                "so cold_step_ms reports each step after a 1 GiB read")
        if not args.no_cpu_baseline:
            Gh = np.zeros(n, np.float32)
            w0 = gen.decode_weights()
            offs = np.arange(0, (P + 1) * kp, kp, dtype=np.int64)
            t0 = time.perf_counter()
            Gr = oracle.decode(Gh, np.concatenate(val_l), np.concatenate(idx_l), offs)
            oracle.sgd(w0, Gr, gen.DECODE_LR)
            cpu = (n, time.perf_counter() - t0, "one full decode + SGD step")
    unpin(pinned)
    ms, kms, launches = time_steps(step, W, K, label)
    extra = {"step_ms": per_step_ms(step, range(W, W + K), dev)}
    if wl in ("flat", "bert"):
        # host time to issue one call (argument checks, plan, launches), the GPU
        # running behind: it must stay below the GPU time per step
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(W, W + K):
            step(t)
        extra["host_issue_us"] = (time.perf_counter() - t0) / K * 1e6
        torch.cuda.synchronize()
        if wl == "flat":
            extra["drift_chain"] = drift_chain(
                lambda g_, e_: efg.ef_topk_compress(g_, e_, k, vals=vals, idx=idx, ws=ws), grads[:2], n, ws, [k],
                400, dev)
        else:
            extra["drift_chain"] = drift_chain(
                lambda g_, e_: efg.ef_topk_compress_segmented(g_, e_, off, ks, vals=vals, idx=idx, ws=ws),
                grads[:2], n, ws, ks, 400, dev)
    if wl in ("flat", "decode"):
        # inputs fit the 256 MB Infinity Cache: also time each step after a 1 GiB write
        extra["cold_step_ms"] = per_step_ms(step, range(W, W + K), dev, flush_bytes=1 << 30)
    if wl == "decode":
        # the same step as three calls: zero G, sparse_decode_accumulate, sgd_apply
        extra["three_call_step_ms"] = per_step_ms(three_calls, range(W, W + K), dev)
        _, dms, dl = time_steps(three_calls, 1, K, "decode_scatter")
        extra["decode_scatter_ms"] = dms
        extra["decode_entries_per_s"] = P * kp / (dms * 1e-3)
        # index encodings of every packet, encoded and decoded (16 packets per timed call)
        pk = [idx[p * kp:(p + 1) * kp] for p in range(P)]
        bm = [torch.empty((n + 7) // 8, dtype=torch.uint8, device=dev) for _ in range(P)]
        bidx = [torch.empty(kp, dtype=torch.int32, device=dev) for _ in range(P)]
        bk = torch.empty(1, dtype=torch.int64, device=dev)
        wsb = efg.workspace(efg.lib().decode_bitmap_workspace_bytes(n), dev)
        ds = [efg.encode_delta(pk[p]) for p in range(P)]
        torch.cuda.synchronize()
        dn = [int(ds[p][1].item()) for p in range(P)]
        didx = [torch.empty(kp, dtype=torch.int32, device=dev) for _ in range(P)]
        dst = torch.empty(1, dtype=torch.int32, device=dev)
        wsd = efg.workspace(max(efg.lib().delta_workspace_bytes(kp), efg.lib().delta_workspace_bytes(max(dn))), dev)
        enc = {
            "bitmap_encode": lambda t: [efg.encode_bitmap(pk[p], n, bits=bm[p]) for p in range(P)],
            "bitmap_decode": lambda t: [efg.decode_bitmap(bm[p], n, kp, idx=bidx[p], k_out=bk, ws=wsb) for p in range(P)],
            "delta_encode": lambda t: [efg.encode_delta(pk[p], out=ds[p][0], nbytes_out=ds[p][1], ws=wsd) for p in range(P)],
            "delta_decode": lambda t: [efg.decode_delta(ds[p][0], dn[p], kp, idx=didx[p], status=dst, ws=wsd)
                                       for p in range(P)],
        }
        for name, fn in enc.items():
            fn(0)
            r = per_step_ms(fn, range(K), dev)
            extra[name + "_ms"] = r["median"]
        torch.cuda.synchronize()
        extra["encodings_round_trip"] = all(torch.equal(bidx[p], pk[p]) and torch.equal(didx[p], pk[p])
                                            for p in range(P))
        extra["delta_bytes_per_index"] = sum(dn) / (P * kp)
    if wl == "adam":
        _, cms, _ = time_steps(step, 1, K, "sign_ef")
        extra["sign_compress_ms"] = cms
        extra["sign_compress_GBps"] = 13.125 * n / (cms * 1e-3) / 1e9
        extra["path_GBps"] = 34.125 * n / ((cms + kms) * 1e-3) / 1e9

        def warm(t):
            ss, sb = efg.adam_scalars(lr, b1, b2, 1 + t)
            efg.ef_adam_step(grads[t], m, v, w, b1, b2, ss, sb, eps)
        _, ams, _ = time_steps(warm, 1, K, "adam_step")
        extra["adam_step_ms"] = ams
        extra["adam_step_GBps"] = 28 * n / (ams * 1e-3) / 1e9
    if wl == "random":
        # which way the last call decided, from the call state at the start of
        # the workspace (float32 S32 at byte 8, S_lo at 24, overflow flag at 28)
        b = wsr[:64].cpu().numpy().tobytes()
        s32_, slo_ = np.frombuffer(b, np.float32, 1, 8)[0], np.frombuffer(b, np.float32, 1, 24)[0]
        slots = slo_ > 0 and np.frombuffer(b, np.uint32, 1, 28)[0] == 0 and s32_ >= slo_
        extra["decided_by"] = "candidate slots" if slots else "second pass"
        # every kernel of the path, one at a time; whole-path algorithmic bytes:
        # accum 12 B, then 16 B per kept element (the candidates and the sample
        # are below 0.1 %), plus mark 4 B + 2 bits when the second pass runs
        for kl in ("rs_sample", "rs_mark", "rs_filter", "rs_write", "rs_total", "rs_exact", "rs_scan", "rs_"):
            _, kms_l, nl = time_steps(step, 1, K, kl)
            extra[f"{kl}_ms"] = kms_l
        path_bytes = n * 12 + 16 * k if slots else n * (12 + 4 + 0.25) + 16 * k
        extra["path_GBps"] = path_bytes / (extra["rs__ms"] * 1e-3) / 1e9
        # the same step made to take the exact integer sum and the second pass
        forced = lambda t: efg.ef_random_sparsify(grads[t], e, k, seed, t, cap=cap, vals=vals, idx=idx, count=cnt,
                                                  ws=wsr, flags=efg.EF_FLAG_FORCE_FALLBACK)
        extra["forced_two_pass_step_ms"] = time_steps(forced, 1, K, "rs_")[0]
    # one more step, verified by properties that need no second implementation
    t_last = W + K - 1
    if wl in ("flat", "bert", "random"):
        x = grads[t_last] + e
    if wl == "adam":
        step(t_last)  # the int8 signs and their packed bits of this step agree
        ok = sign_bits_agree(q, bits) and bool(torch.isfinite(w).all()) and bool(torch.isfinite(m).all())
    elif wl == "sign":
        step(t_last)
        ok = sign_bits_agree(sgn, bits) and bool(torch.isfinite(e).all()) and bool(torch.isfinite(m).all())
    elif wl == "flat":
        step(t_last)
        ok = topk_invariants(x, vals, idx, k, e)
    elif wl == "bert":
        step(t_last)
        ok, o = True, 0
        for s_, kk in enumerate(ks):  # each tensor is the top-k_s of its slice
            a, b = int(off[s_]), int(off[s_ + 1])
            ok = ok and topk_invariants(x[a:b], vals[o:o + kk], idx[o:o + kk] - a, int(kk), e[a:b])
            o += int(kk)
    elif wl == "random":
        step(t_last)  # bookkeeping: vals = x[idx] in increasing index order, e = x except +0 there
        c = int(cnt.item())
        ik = idx[:min(c, cap)].long()
        want = x.clone()
        want[ik] = 0.0
        ok = (0 < c <= cap and bool((ik[1:] > ik[:-1]).all()) and int(ik[0]) >= 0 and int(ik[-1]) < n
              and torch.equal(vals[:c].view(torch.int32), x[ik].view(torch.int32))
              and torch.equal(e.view(torch.int32), want.view(torch.int32)))
        del want
    elif wl == "quant":
        step(t_last)  # codes within +-127, a finite positive scale, zero values coded 0
        scale = float(sc.item())
        ok = (bool((q >= -127).all()) and 0.0 < scale < float("inf")
              and bool((q[vals == 0] == 0).all()))
    else:
        w_before = w.clone()
        step(t_last)  # G is zero wherever no packet entry lands, and there w is untouched
        touched = torch.zeros(n, dtype=torch.bool, device=dev)
        touched[idx.long()] = True
        ok = bool((G[~touched] == 0).all()) and torch.equal(w[G == 0], w_before[G == 0])
        del w_before, touched
    torch.cuda.synchronize()
    if wl in ("flat", "bert", "random"):
        del x
    if not ok:
        raise SystemExit(f"bench: the {wl} workload's last step failed its check")
    extra["verified"] = ok
    # the box's copy rate, and the known-size kernel for the traffic counters
    extra["torch_copy_GBps"] = torch_copy(dev)
    achieved = bpe * units / (kms * 1e-3) / 1e9
    res = {
        "metric": metric, "value": units / (ms * 1e-3), "unit": unit, "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": {"workload": desc, "n": units},
        "roofline": {"kernel": label, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": measured_traffic(TRAFFIC_PROFILES[wl]) if wl in TRAFFIC_PROFILES else None,
                     "kernel_ms_per_step": kms,
                     "launches": launches, "bytes_per_elem": bpe},
    }
    res.update(extra)
    if cpu is not None:
        cores = 1  # the oracle runs on one thread
        res["cpu_baseline"] = {"value": cpu[0] / cpu[1], "unit": unit, "cores": cores, "kind": "oracle",
                               "sample": cpu[2] + f"; {cpu[1]:.2f} s on one core of {host_cpu_model()}"}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
