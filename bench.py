#!/usr/bin/env python3
"""Throughput of the SSD scan hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
the chunked scan of the 30B-shaped prefill (b=1, L=8192, H=64, P=64, N=128,
G=8, chunk 128, bf16 x/B/C, fp32 dt/A/D and state, final state returned;
kernels chunk_prep, chunk_state, chunk_output) followed by one decode token on
the returned state (state_update).  Inputs are resident in HBM before timing
starts; the step cycles over several copies of the inputs so that consecutive
steps do not hit in the 256 MB MALL.

Prints ONE JSON line with the throughput (host clock over the timed steps),
a roofline entry for the whole scan call (its compulsory bytes over the sum of
its dispatches' durations, each timed by HIP events that the library binds to
the dispatch on the stream it launches on, over the same number of steps right
after the timed ones; the GPU time of the whole call between plain stream
events, launch gaps included, is reported beside it), and the fp64 CPU oracle
timed on the host cores.  A "workloads" object measures the other workloads
the same way: 16 packed sequences of 16K tokens in all, a 128K-token row from
an initial state (chunk 256), and a 64 x 4096 prefill with its batch-64 decode
step.

The defaults warm up for about 30 ms (the clocks settle within about 20 ms of
sustained work) and time about 0.1 s of steps.

The line also carries a "backward" object for the gradients of the same scan
(ssd_chunk_scan_bwd on the same inputs, seeded dy and final-state gradient):
its tokens/s, per-kernel times, a roofline entry for its per-chunk gradient
kernel against the compulsory bytes of the whole backward pass, and the fp64
oracle's gradients timed on the heads of one group; and a "mixer" object for
the steps beside the scan (causal conv1d into the scan's x/B/C, gated group
RMSNorm of its output) at the same shape; and a "cache" object for continuous
batching on state caches (a 256-row decode step on slots of a 512-slot cache
with its HBM roofline, the prefill of 8 prompts of different lengths from and
back into cache slots, the same prompts packed back to back (cu_seqlens), and the
strict chunk-emulating decode of 64 rows).
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSD scan tokens/s (bf16, H=64,P=64,N=128) and % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
MALL_BYTES = 256 << 20
COPY_BYTES = 1 << 30  # calibration copy, 4x the MALL
WORKLOADS_BY_NAME = {"prefill_8k": 1, "packed_16k": 2, "long_128k": 3}
WORKLOADS_BY_NAME_ALL = dict(WORKLOADS_BY_NAME, prefill_decode=4)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash():
    """Hash of the HIP sources; a counter summary taken on other sources is stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mamba_ssd_selective_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def profile_bytes(fname, key="hbm_bytes_per_call"):
    """HBM bytes per call (all its dispatches) that a committed rocprofv3
    counter summary under profiles/ gives for `key`, if the summary was taken
    on the current sources; else None."""
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(re.escape(key) + r":\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash():
        return None
    return float(m_bytes.group(1))


def counter_traffic(workload):
    """HBM bytes per ssd_chunk_scan_fwd call of a scan workload (see profile_bytes)."""
    return profile_bytes("scan_%s_counters.md" % workload)


def compulsory_bytes(b, L, H, P, N, G, *, es=2, seq_idx=False, init=False, final=True):
    """Each input read once and each output written once: x, dt, B, C in, y
    out (plus seq_idx), the fp32 final states (and initial states)."""
    per_token = 2 * H * P * es + 2 * G * N * es + H * 4 + (4 if seq_idx else 0)
    state = b * H * P * N * 4
    return b * L * per_token + (state if final else 0) + (state if init else 0)


def scan_flops(b, L, H, P, N, G, Q):
    """MFMA work of the chunked form on the lower triangle: chunk states and
    the carried-state term (2PN each), the intra-chunk product (PQ) and the
    group's C.B^T (NQ, shared by H/G heads), per token and head."""
    return b * L * H * (2 * P * N + P * Q + 2 * P * N + N * Q / (H // G))


def bound_pass(lib, hip, fn, nk, reps):
    """Every dispatch of `reps` rounds of library calls timed by HIP events
    bound to it (the library passes them to the launch, on the stream it
    launches on).  fn is one call, or a list of calls made in turn each round;
    nk is its number of dispatches (or the list of them).  Returns the mean
    duration of each dispatch of a round, in order, in us."""
    import numpy as np
    fns = fn if isinstance(fn, (list, tuple)) else [fn]
    nks = nk if isinstance(nk, (list, tuple)) else [nk]
    tot = sum(nks)
    evs = hip.events(2 * tot * reps)
    launched = ctypes.c_int(0)
    vp = ctypes.sizeof(ctypes.c_void_p)
    for i in range(reps):
        first = tot * i
        for f, n in zip(fns, nks):
            lib.ssd_set_timing_events(ev_slice_of(evs, 2 * first, 2 * n, vp), 2 * n,
                                      ctypes.byref(launched))
            f(i)
            if launched.value != n:
                raise RuntimeError("expected %d dispatches, got %d" % (n, launched.value))
            first += n
    lib.ssd_set_timing_events(None, 0, None)
    import torch
    torch.cuda.synchronize()
    us = [1e3 * float(np.mean([hip.elapsed_ms(evs[2 * (tot * i + k)], evs[2 * (tot * i + k) + 1])
                               for i in range(reps)])) for k in range(tot)]
    hip.destroy(evs)
    return us


def count_dispatches(lib, fn):
    launched = ctypes.c_int(0)
    no_events = (ctypes.c_void_p * 32)()
    lib.ssd_set_timing_events(no_events, 32, ctypes.byref(launched))
    fn(0)
    lib.ssd_set_timing_events(None, 0, None)
    return launched.value


def roofline_entry(nbytes, us, traffic=None):
    ach = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}


class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        out = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            rc = self.lib.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError("hipEventCreate failed: %d" % rc)
            out[i] = e
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


def cpu_baseline(p, w, budget_s):
    """The fp64 oracle (as it stands) on the host cores, on a bounded sample of
    the same workload: all L tokens of blocks of heads, cycling over the heads
    until the time budget is spent; tokens/s of the whole workload (all heads)."""
    import numpy as np
    import oracle
    threads = oracle.max_threads()
    H = w.nheads
    block = max(8, min(H, threads))
    hpg = H // w.ngroups
    head_tokens = 0  # tokens x heads processed
    t0 = time.perf_counter()
    start = 0
    while time.perf_counter() - t0 < budget_s:
        heads = (start + np.arange(block)) % H
        groups = heads // hpg
        oracle.scan(p["x"][:, :, heads], p["dt_raw"][:, :, heads], p["A"][heads],
                    p["B"][:, :, groups], p["C"][:, :, groups], dt_bias=p["dt_bias"][heads],
                    D=p["D"][heads], h_init=None if p.get("h_init") is None else p["h_init"][:, heads],
                    seq_idx=p.get("seq_idx"))
        head_tokens += w.batch * w.seqlen * len(heads)
        start = (start + block) % H
    el = time.perf_counter() - t0
    return {"value": head_tokens / H / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%s: all %d tokens of blocks of %d heads, cycling over the %d heads for "
                      "%.1f s (%.1f passes over all heads; fp64 sequential recurrence, OpenMP "
                      "over heads); tokens/s of the whole workload"
                      % (w.name, w.seqlen, block, H, el, head_tokens / (w.batch * w.seqlen * H))}


def backward_measure(ssd, lib, hip, torch, base, A, D, bias, w, steps, cpu_seconds, p):
    """The backward pass (ssd_chunk_scan_bwd) on the same workload: tokens/s
    over `steps` timed calls, the gradient kernel's duration from events bound
    to its dispatch, its roofline against the compulsory bytes of the whole
    backward, and the oracle's gradients timed on one group of heads."""
    import numpy as np
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    if not (P == 64 and N == 128 and Q == 128):
        return None
    dev = base["x"].device
    gen = torch.Generator(device="cpu").manual_seed(2024)
    dy = torch.randn((b, L, H, P), generator=gen).to(torch.bfloat16).to(dev)
    dfin = torch.randn((b, H, P, N), generator=gen).to(dev)
    ws = torch.empty(ssd.bwd_workspace_bytes(b, L, H, P, N, G, Q), dtype=torch.uint8, device=dev)

    def call():
        return ssd.chunk_scan_bwd(base["x"], base["dt"], A, base["B"], base["C"], dy, chunk_size=Q,
                                  D=D, dt_bias=bias, initial_states=base["h0"], seq_idx=base["seq"],
                                  d_final_states=dfin, workspace=ws)

    launched = ctypes.c_int(0)
    no_events = (ctypes.c_void_p * 16)()
    lib.ssd_set_timing_events(no_events, 16, ctypes.byref(launched))
    call()
    lib.ssd_set_timing_events(None, 0, None)
    nk = launched.value
    # segmented state walks add the segment ends and a pass per direction
    names = (["chunk_meta", "seg_ends", "seg_pass_fwd", "seg_pass_bwd", "chunk_states", "chunk_grad",
              "grad_sums"] if nk == 7 else ["chunk_meta", "chunk_states", "chunk_grad", "grad_sums"][:nk])
    kg = names.index("chunk_grad")
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    vp = ctypes.sizeof(ctypes.c_void_p)
    evs = hip.events(2 * nk * steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        sl = (ctypes.c_void_p * (2 * nk))()
        sl[2 * kg] = evs[2 * nk * i + 2 * kg]
        sl[2 * kg + 1] = evs[2 * nk * i + 2 * kg + 1]
        lib.ssd_set_timing_events(sl, 2 * nk, ctypes.byref(launched))
        call()
    lib.ssd_set_timing_events(None, 0, None)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    grad_us = 1e3 * float(np.mean([hip.elapsed_ms(evs[2 * nk * i + 2 * kg], evs[2 * nk * i + 2 * kg + 1])
                                   for i in range(steps)]))
    diag = min(steps, 10)
    for i in range(diag):
        lib.ssd_set_timing_events(ev_slice_of(evs, 2 * nk * i, 2 * nk, vp), 2 * nk, ctypes.byref(launched))
        call()
    lib.ssd_set_timing_events(None, 0, None)
    torch.cuda.synchronize()
    kus = {n: round(1e3 * float(np.mean([hip.elapsed_ms(evs[2 * nk * i + 2 * k], evs[2 * nk * i + 2 * k + 1])
                                        for i in range(diag)])), 2) for k, n in enumerate(names)}
    hip.destroy(evs)
    # compulsory bytes: x, dy, B, C, dt in; dx, dB, dC, d(dt) out (three (b,L,H,P)
    # bf16 tensors, four (b,L,G,N) ones, two fp32 dt-shaped ones); the states in and out
    per_token = 3 * H * P * 2 + 4 * G * N * 2 + 2 * H * 4
    state_bytes = b * H * P * N * 4
    bwd_bytes = b * L * per_token + 3 * state_bytes + (b * L * 4 if base["seq"] is not None else 0)
    call_us = sum(kus.values())
    out = {"value": round(b * L * steps / el, 1), "unit": "tokens/s", "steps": steps,
           "ms_per_step": round(1e3 * el / steps, 5), "dtype": "bf16",
           "grad_kernel_us": round(grad_us, 2), "kernels_us": kus,
           "call_kernel_us": round(call_us, 2), "compulsory_bytes": bwd_bytes,
           # the whole backward call: its compulsory bytes over the sum of its dispatches
           "roofline": roofline_entry(bwd_bytes, call_us, profile_bytes("bwd_prefill_8k_counters.md")),
           "grad_kernel_roofline_frac": round(bwd_bytes / (grad_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "cpu_baseline": None}
    if cpu_seconds > 0:
        import oracle
        grp = 0
        hs = slice(0, H // G)
        pin = {k: (None if v is None else v) for k, v in p.items()}
        dy_np = dy.float().cpu().numpy()
        df_np = dfin.cpu().numpy()
        t0 = time.perf_counter()
        runs = 0
        while runs == 0 or time.perf_counter() - t0 < cpu_seconds:
            oracle.scan_bwd(pin["x"][:, :L, hs], pin["dt_raw"][:, :L, hs], pin["A"][hs],
                            pin["B"][:, :L, grp:grp + 1], pin["C"][:, :L, grp:grp + 1], dy_np[:, :, hs],
                            dh_final=df_np[:, hs], dt_bias=pin["dt_bias"][hs], D=pin["D"][hs],
                            h_init=None if pin.get("h_init") is None else pin["h_init"][:, hs],
                            seq_idx=None if pin.get("seq_idx") is None else pin["seq_idx"][:, :L])
            runs += 1
        cel = time.perf_counter() - t0
        out["cpu_baseline"] = {
            "value": round(b * L * runs * (H // G) / H / cel, 1), "unit": "tokens/s",
            "cores": min(oracle.max_threads(), b * (H // G)), "kind": "oracle",
            "sample": "%s: gradients of all %d tokens for the %d heads of group 0, %d run(s) in "
                      "%.1f s (fp64 reverse-mode recurrence, OpenMP over heads); tokens/s of the "
                      "whole workload" % (w.name, L, H // G, runs, cel)}
    return out


def mixer_measure(ssd, lib, hip, torch, w, steps, cpu_seconds):
    """The mixer steps beside the scan at the workload's shape: the causal conv1d
    over the xBC channels (written as the scan's x, B, C) and the gated group
    RMSNorm of the scan's output (group 512).  Dispatch-timed durations, HBM
    rooflines against each kernel's compulsory bytes, and the oracle timed on
    a sample of tokens."""
    import numpy as np
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    dev = torch.device("cuda:0")
    nx, nb = H * P, G * N
    dim = nx + 2 * nb
    gen = torch.Generator(device="cpu").manual_seed(77)
    bf = torch.bfloat16
    xbc = torch.randn((b, L, dim), generator=gen).to(bf).to(dev)
    cw = (0.5 * torch.randn((dim, 4), generator=gen)).to(dev)
    cb = torch.randn((dim,), generator=gen).to(dev)
    cst = torch.randn((b, dim, 3), generator=gen).to(bf).to(dev)
    y = torch.randn((b, L, nx), generator=gen).to(bf).to(dev)
    z = torch.randn((b, L, nx), generator=gen).to(bf).to(dev)
    nw = torch.randn((nx,), generator=gen).to(dev)
    xo = torch.empty((b, L, H, P), dtype=bf, device=dev)
    bo = torch.empty((b, L, G, N), dtype=bf, device=dev)
    co = torch.empty((b, L, G, N), dtype=bf, device=dev)
    so = torch.empty((b, dim, 3), dtype=bf, device=dev)
    out = torch.empty_like(y)
    calls = {
        "conv1d": lambda: lib.ssd_conv1d_fwd(b, L, dim, nx, nb, 1, xbc.data_ptr(), cw.data_ptr(), 4,
                                             cb.data_ptr(), cst.data_ptr(), None, xo.data_ptr(),
                                             bo.data_ptr(), co.data_ptr(), so.data_ptr(),
                                             torch.cuda.current_stream().cuda_stream),
        "gated_norm": lambda: lib.ssd_gated_rmsnorm(b * L, nx, 512, 1, y.data_ptr(), z.data_ptr(),
                                                    nw.data_ptr(), 1e-6, out.data_ptr(),
                                                    torch.cuda.current_stream().cuda_stream),
    }
    nbytes = {"conv1d": 2 * b * L * dim * 2 + 2 * b * dim * 3 * 2 + dim * 5 * 4,
              "gated_norm": 3 * b * L * nx * 2 + nx * 4}
    res = {}
    for name, fn in calls.items():
        for _ in range(5):
            if fn() != 0:
                raise RuntimeError("%s failed" % name)
        torch.cuda.synchronize()
        evs = hip.events(2 * steps)
        launched = ctypes.c_int(0)
        for i in range(steps):
            lib.ssd_set_timing_events(ev_slice_of(evs, 2 * i, 2, ctypes.sizeof(ctypes.c_void_p)), 2,
                                      ctypes.byref(launched))
            fn()
        lib.ssd_set_timing_events(None, 0, None)
        torch.cuda.synchronize()
        us = 1e3 * float(np.mean([hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps)]))
        hip.destroy(evs)
        ach = nbytes[name] / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 2), "tokens_per_s": round(b * L / (us * 1e-6), 1),
                     "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                                  "traffic": None}}
    res["shape"] = {"tokens": b * L, "xbc_channels": dim, "norm_channels": nx, "norm_group": 512,
                    "dtype": "bf16"}
    res["cpu_baseline"] = None
    if cpu_seconds > 0:
        from oracle import mixer
        T = min(L, 1024)
        xs = xbc[:, :T].float().cpu().numpy(); ys = y[:, :T].float().cpu().numpy()
        zs = z[:, :T].float().cpu().numpy()
        cwn, cbn, csn, nwn = cw.cpu().numpy(), cb.cpu().numpy(), cst.float().cpu().numpy(), nw.cpu().numpy()
        t0 = time.perf_counter()
        runs = 0
        while runs == 0 or time.perf_counter() - t0 < cpu_seconds:
            mixer.conv1d(xs, cwn, cbn, csn)
            mixer.gated_rmsnorm(ys, zs, nwn, 512)
            runs += 1
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(b * T * runs / el, 1), "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": "conv1d + gated norm of the first %d tokens, %d run(s) in %.1f s "
                                         "(numpy fp64, one thread)" % (T, runs, el)}
    return res


def cache_measure(ssd, lib, hip, torch, w, steps, cpu_seconds):
    """Continuous batching on state caches at the workload's head shape: one
    decode token for 256 rows whose fp32 states sit in slots of a 512-slot
    cache (the state update; HBM roofline against its compulsory bytes), and
    the prefill of 8 prompts of seeded lengths 512..2048 (rows of 2048 tokens)
    from and back into the slots of a 16-slot cache (every dispatch timed); and
    the strict chunk-emulating decode of 64 rows at offset 63 of their chunks.
    The oracle's decode step is timed on 16 of the rows."""
    import numpy as np
    H, P, N, G, Q = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    dev = torch.device("cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(91)
    bf = torch.bfloat16
    stream = lambda: torch.cuda.current_stream().cuda_stream
    A = (-torch.rand((H,), generator=gen) * 3 - 0.5).to(dev)
    D = torch.randn((H,), generator=gen).to(dev)
    bias = (torch.rand((H,), generator=gen) - 4.0).to(dev)
    res = {}
    vp = ctypes.sizeof(ctypes.c_void_p)

    def timed(fn, nk, n):
        for _ in range(5):
            if fn() != 0:
                raise RuntimeError("cache call failed")
        torch.cuda.synchronize()
        # wall time per call, back to back, with no events between the dispatches
        t0 = time.perf_counter()
        for i in range(n):
            fn()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / n
        # each dispatch's duration from events bound to it
        evs = hip.events(2 * nk * n)
        launched = ctypes.c_int(0)
        for i in range(n):
            lib.ssd_set_timing_events(ev_slice_of(evs, 2 * nk * i, 2 * nk, vp), 2 * nk,
                                      ctypes.byref(launched))
            fn()
        lib.ssd_set_timing_events(None, 0, None)
        torch.cuda.synchronize()
        if launched.value != nk:
            raise RuntimeError("expected %d dispatches, got %d" % (nk, launched.value))
        us = [1e3 * float(np.mean([hip.elapsed_ms(evs[2 * (nk * i + k)], evs[2 * (nk * i + k) + 1])
                                   for i in range(n)])) for k in range(nk)]
        hip.destroy(evs)
        return us, wall

    # ---- decode: 256 rows, 512 slots
    rows, slots = 256, 512
    cache = torch.randn((slots, H, P, N), generator=gen).to(dev)
    idx = torch.randperm(slots, generator=gen)[:rows].to(torch.int32).to(dev)
    x = torch.randn((rows, H, P), generator=gen).to(bf).to(dev)
    dt = torch.randn((rows, H), generator=gen).to(dev)
    Bm = torch.randn((rows, G, N), generator=gen).to(bf).to(dev)
    Cm = torch.randn((rows, G, N), generator=gen).to(bf).to(dev)
    y = torch.empty((rows, H, P), dtype=bf, device=dev)
    dec = lambda: lib.ssd_state_update_cached(rows, slots, H, P, N, G, 1, cache.data_ptr(),
                                              idx.data_ptr(), x.data_ptr(), dt.data_ptr(),
                                              bias.data_ptr(), 1, 0.0, math.inf, A.data_ptr(),
                                              Bm.data_ptr(), Cm.data_ptr(), D.data_ptr(),
                                              y.data_ptr(), stream())
    (us,), _ = timed(dec, 1, steps)
    nbytes = rows * (2 * H * P * N * 4 + 2 * H * P * 2 + 2 * G * N * 2 + H * 4 + 4) + 3 * H * 4
    ach = nbytes / (us * 1e-6) / 1e9
    res["decode"] = {"rows": rows, "slots": slots, "us": round(us, 2),
                     "tokens_per_s": round(rows / (us * 1e-6), 1),
                     "roofline": roofline_entry(nbytes, us, profile_bytes(
                         "cache_kernels_counters.md", "hbm_bytes_per_call[cache decode]"))}

    # ---- prefill: 8 prompts of 512..2048 tokens into a 16-slot cache
    b, L, pslots = 8, 2048, 16
    lens = torch.randint(512, L + 1, (b,), generator=gen, dtype=torch.int32)
    px = torch.randn((b, L, H, P), generator=gen).to(bf)
    pB = torch.randn((b, L, G, N), generator=gen).to(bf)
    pC = torch.randn((b, L, G, N), generator=gen).to(bf)
    pdt = torch.randn((b, L, H), generator=gen)
    for r in range(b):  # padding positions hold zeros
        n = int(lens[r])
        px[r, n:] = 0
        pB[r, n:] = 0
        pC[r, n:] = 0
    px, pB, pC, pdt = px.to(dev), pB.to(dev), pC.to(dev), pdt.to(dev)
    pcache = torch.randn((pslots, H, P, N), generator=gen).to(dev)
    pidx = torch.randperm(pslots, generator=gen)[:b].to(torch.int32).to(dev)
    plens = lens.to(dev)
    py = torch.empty((b, L, H, P), dtype=bf, device=dev)
    d = ssd._dims(b, L, H, P, N, G, Q)
    need = int(lib.ssd_chunk_scan_cached_workspace_bytes(ctypes.byref(d), 1))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    nseg = ssd.segments(b, L, H, P, N, G, Q)
    names = ["gather", "chunk_prep"] + (["chunk_state"] if nseg > 1 else []) + ["chunk_output",
                                                                                  "scatter"]
    pre = lambda: lib.ssd_chunk_scan_fwd_cached(
        ctypes.byref(d), 1, px.data_ptr(), pdt.data_ptr(), bias.data_ptr(), 1, 0.0, math.inf,
        A.data_ptr(), pB.data_ptr(), pC.data_ptr(), D.data_ptr(), plens.data_ptr(),
        pcache.data_ptr(), pslots, pidx.data_ptr(), 1, 0, py.data_ptr(), ws.data_ptr(), need,
        stream())
    us_k, wall = timed(pre, len(names), max(steps // 2, 10))
    real = int(lens.sum())
    # the same prompts packed back to back (cu_seqlens)
    cu = torch.zeros(b + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0)
    vx = torch.cat([px[r, :int(lens[r])] for r in range(b)])
    vdt = torch.cat([pdt[r, :int(lens[r])] for r in range(b)])
    vB = torch.cat([pB[r, :int(lens[r])] for r in range(b)])
    vC = torch.cat([pC[r, :int(lens[r])] for r in range(b)])
    vy = torch.empty_like(vx)
    cud = cu.to(dev)
    vneed = int(lib.ssd_chunk_scan_varlen_workspace_bytes(ctypes.byref(d), 1))
    vws = torch.empty(vneed, dtype=torch.uint8, device=dev)
    var = lambda: lib.ssd_chunk_scan_fwd_varlen(
        ctypes.byref(d), real, 1, vx.data_ptr(), vdt.data_ptr(), bias.data_ptr(), 1, 0.0, math.inf,
        A.data_ptr(), vB.data_ptr(), vC.data_ptr(), D.data_ptr(), cud.data_ptr(), pcache.data_ptr(),
        pslots, pidx.data_ptr(), 1, 0, vy.data_ptr(), vws.data_ptr(), vneed, stream())
    # the same dispatches as the cached prefill, on the packed layout in place
    vus, vwall = timed(var, len(names), max(steps // 2, 10))
    res["packed_prefill"] = {"sequences": b, "real_tokens": real, "max_seqlen": L,
                             "kernels_us": {n: round(u, 2) for n, u in zip(names, vus)},
                             "kernels_total_us": round(sum(vus), 2),
                             "ms_per_call": round(1e3 * vwall, 4),
                             "real_tokens_per_s": round(real / vwall, 1)}
    res["prefill"] = {"rows": b, "row_capacity": L, "real_tokens": real,
                      "lengths": [int(v) for v in lens], "slots": pslots,
                      "kernels_us": {n: round(u, 2) for n, u in zip(names, us_k)},
                      "kernels_total_us": round(sum(us_k), 2),
                      "ms_per_call": round(1e3 * wall, 4),
                      "real_tokens_per_s": round(real / wall, 1)}
    # ---- strict decode (chunk-emulating): 64 rows at offset 63 of their chunks
    er, eslots, epos = 64, 64, 63
    ecache = torch.randn((eslots, H, P, N), generator=gen).to(dev)
    ech = (torch.randn((eslots, Q, H, P), generator=gen).to(bf).to(dev),
           torch.randn((eslots, Q, H), generator=gen).to(dev),
           torch.randn((eslots, Q, G, N), generator=gen).to(bf).to(dev),
           torch.randn((eslots, Q, G, N), generator=gen).to(bf).to(dev))
    eidx = torch.randperm(eslots, generator=gen).to(torch.int32).to(dev)
    eposd = torch.full((er,), epos, dtype=torch.int32, device=dev)
    ey = torch.empty((er, H, P), dtype=bf, device=dev)
    ed = ssd._dims(er, Q, H, P, N, G, Q)
    eneed = int(lib.ssd_decode_emulated_workspace_bytes(ctypes.byref(ed), 1))
    ews = torch.empty(eneed, dtype=torch.uint8, device=dev)
    ex, edt, eB, eC = x[:er], dt[:er], Bm[:er], Cm[:er]
    emu = lambda: lib.ssd_decode_emulated(
        ctypes.byref(ed), 1, ex.data_ptr(), edt.data_ptr(), bias.data_ptr(), 1, 0.0, math.inf,
        A.data_ptr(), eB.data_ptr(), eC.data_ptr(), D.data_ptr(), ecache.data_ptr(),
        ech[0].data_ptr(), ech[1].data_ptr(), ech[2].data_ptr(), ech[3].data_ptr(), eslots,
        eidx.data_ptr(), eposd.data_ptr(), ey.data_ptr(), ews.data_ptr(), eneed, stream())
    # the output kernel in two passes: rows whose chunk does not complete, then the others
    enames = ["chunk_prep", "chunk_output", "chunk_output_commit"]
    eus, ewall = timed(emu, len(enames), max(steps // 2, 10))
    res["strict_decode"] = {"rows": er, "slots": eslots, "offset_in_chunk": epos,
                            "kernels_us": {n: round(u, 2) for n, u in zip(enames, eus)},
                            "kernels_total_us": round(sum(eus), 2),
                            "ms_per_call": round(1e3 * ewall, 4),
                            "tokens_per_s": round(er / ewall, 1)}
    # the step at the end of every row's chunk (offset Q - 1): every row also
    # replaces its slot's chunk-start state (the repeated calls rewrite the
    # same slots from the states they left; the work per call is the same)
    eposd.fill_(Q - 1)
    cus, cwall = timed(emu, len(enames), max(steps // 2, 10))
    res["strict_decode_chunk_end"] = {"rows": er, "slots": eslots, "offset_in_chunk": Q - 1,
                                      "kernels_us": {n: round(u, 2) for n, u in zip(enames, cus)},
                                      "kernels_total_us": round(sum(cus), 2),
                                      "ms_per_call": round(1e3 * cwall, 4),
                                      "tokens_per_s": round(er / cwall, 1)}
    res["cpu_baseline"] = None
    if cpu_seconds > 0:
        import oracle
        k = 16
        st0 = cache[idx[:k].long()].double().cpu().numpy()
        args = (x[:k].float().cpu().numpy(), dt[:k].cpu().numpy(), A.cpu().numpy(),
                Bm[:k].float().cpu().numpy(), Cm[:k].float().cpu().numpy())
        t0 = time.perf_counter()
        runs = 0
        while runs == 0 or time.perf_counter() - t0 < cpu_seconds:
            oracle.step(st0, *args, dt_bias=bias.cpu().numpy(), D=D.cpu().numpy())
            runs += 1
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(k * runs / el, 1), "unit": "decode tokens/s",
                               "cores": 1, "kind": "oracle",
                               "sample": "decode step of %d of the %d rows, %d run(s) in %.1f s "
                                         "(fp64, one thread)" % (k, rows, runs, el)}
    return res


def scan_workload_measure(ssd, lib, hip, torch, w, reps):
    """One ssd_chunk_scan_fwd call over workload w (inputs drawn on the device,
    resident in HBM): tokens/s from the host clock over `reps` calls, every
    dispatch's duration from events bound to it over another `reps` calls, and
    the whole call's HBM roofline against its compulsory bytes.  For the
    prefill+decode workload, also its batch decode step (ssd_state_update on
    the rows' final states, one token per row, cycling over the decode tokens)."""
    import workloads
    dev = torch.device("cuda:0")
    b, H, P, N, G, Q = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    Lp = w.prefill or w.seqlen
    inp = workloads.make_inputs_device(w, dev)
    x, dt, B, C = (inp[k][:, :Lp].contiguous() for k in ("x", "dt_raw", "B", "C"))
    seq = inp["seq_idx"]
    h0 = inp["h_init"]
    y = torch.empty_like(x)
    fs = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, ssd.workspace_bytes(b, Lp, H, P, N, G, Q)), dtype=torch.uint8, device=dev)
    A, D, bias = inp["A"], inp["D"], inp["dt_bias"]

    def scan(i):
        ssd.chunk_scan_fwd(x, dt, A, B, C, chunk_size=Q, D=D, dt_bias=bias, initial_states=h0,
                           seq_idx=seq, return_final_states=True, out=y, final_states_out=fs,
                           workspace=ws)

    for i in range(3):
        scan(i)
    torch.cuda.synchronize()
    nk = count_dispatches(lib, scan)
    t0 = time.perf_counter()
    for i in range(reps):
        scan(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / reps
    kus = bound_pass(lib, hip, scan, nk, reps)
    nbytes = compulsory_bytes(b, Lp, H, P, N, G, seq_idx=seq is not None, init=h0 is not None)
    ksum = sum(kus)
    res = {"workload": w.name, "batch": b, "seq_len": Lp, "chunk": Q,
           "segments": ssd.segments(b, Lp, H, P, N, G, Q),
           "packed_sequences": w.packed or None, "initial_states": h0 is not None,
           "value": round(b * Lp / wall, 1), "unit": "tokens/s", "calls": reps,
           "ms_per_call": round(1e3 * wall, 4), "kernels_us": [round(u, 2) for u in kus],
           "call_kernel_us": round(ksum, 2), "compulsory_bytes": nbytes,
           "roofline": roofline_entry(nbytes, ksum, counter_traffic(w.name)),
           "mfma_frac": round(scan_flops(b, Lp, H, P, N, G, Q) / (ksum * 1e-6) / 1e12
                              / MFMA_BF16_PEAK_TFLOPS, 4)}
    if w.decode_steps:
        steps = w.decode_steps
        xs, dts = inp["x"][:, Lp:], inp["dt_raw"][:, Lp:]
        Bs, Cs = inp["B"][:, Lp:], inp["C"][:, Lp:]
        xd = [xs[:, t].contiguous() for t in range(steps)]
        dtd = [dts[:, t].contiguous() for t in range(steps)]
        Bd = [Bs[:, t].contiguous() for t in range(steps)]
        Cd = [Cs[:, t].contiguous() for t in range(steps)]
        yd = torch.empty((b, H, P), dtype=x.dtype, device=dev)

        def step(i):
            t = i % steps
            ssd.state_update(fs, xd[t], dtd[t], A, Bd[t], Cd[t], D=D, dt_bias=bias, out=yd)

        for i in range(3):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        dwall = (time.perf_counter() - t0) / steps
        (dus,) = bound_pass(lib, hip, step, 1, steps)
        dbytes = b * (2 * H * P * N * 4 + 2 * H * P * 2 + 2 * G * N * 2 + H * 4)
        res["decode"] = {"rows": b, "steps": steps, "value": round(b / dwall, 1),
                         "unit": "decode tokens/s", "ms_per_step": round(1e3 * dwall, 4),
                         "kernel_us": round(dus, 2), "compulsory_bytes": dbytes,
                         "roofline": roofline_entry(dbytes, dus, profile_bytes(
                             "scan_prefill_decode_counters.md", "hbm_bytes_per_decode_step"))}
    del inp, x, dt, B, C, y, ws
    torch.cuda.empty_cache()
    return res


def ev_slice_of(evs, first, count, vp):
    return (ctypes.c_void_p * count).from_buffer(evs, first * vp)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="prefill_8k", choices=sorted(WORKLOADS_BY_NAME))
    ap.add_argument("--backward-steps", type=int, default=30,
                    help="timed calls of the backward pass (reported under \"backward\")")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the CPU oracle baseline (0 = skip)")
    ap.add_argument("--skip-workloads", action="store_true",
                    help="measure only the headline workload (no packed_16k, long_128k, "
                         "prefill_decode objects)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (for scaling HBM "
                         "byte counters) and print its size")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library runs on one GPU only (the SSD scan's data-parallel path "
              "on one GPU's share); --gpus %d is not supported." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if args.calibrate_copy:
        # a plain copy of COPY_BYTES, five times: rocprofv3 FETCH_SIZE / WRITE_SIZE of
        # this kernel give the counter-to-bytes factor (each launch reads and writes
        # COPY_BYTES; the buffers are larger than the 256 MB MALL)
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": COPY_BYTES, "launches": 5}), flush=True)
        return
    import mamba_ssd_selective_amd as ssd
    import workloads

    lib = ssd.library()
    hip = Hip()
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS[WORKLOADS_BY_NAME[args.workload]]
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    log("bench: drawing %s inputs" % w.name)
    p = workloads.make_inputs(w, seqlen=L + 1)  # last token feeds the decode update
    bf = torch.bfloat16

    def dev_t(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return t.to(dtype) if dtype is not None else t

    base = dict(x=dev_t(p["x"][:, :L], bf), dt=dev_t(p["dt_raw"][:, :L]),
                B=dev_t(p["B"][:, :L], bf), C=dev_t(p["C"][:, :L], bf),
                xd=dev_t(p["x"][:, L], bf), dtd=dev_t(p["dt_raw"][:, L]),
                Bd=dev_t(p["B"][:, L], bf), Cd=dev_t(p["C"][:, L], bf),
                seq=None if p.get("seq_idx") is None else dev_t(p["seq_idx"][:, :L]),
                h0=None if p.get("h_init") is None else dev_t(p["h_init"]))
    A, D, bias = dev_t(p["A"]), dev_t(p["D"]), dev_t(p["dt_bias"])
    es = 2
    state_bytes = b * H * P * N * 4
    scan_bytes = compulsory_bytes(b, L, H, P, N, G, seq_idx=base["seq"] is not None,
                                  init=base["h0"] is not None)
    nsets = max(2, math.ceil(2 * MALL_BYTES / scan_bytes) + 1)
    sets = []
    for _ in range(nsets):
        s = {k: (v.clone() if v is not None else None) for k, v in base.items()}
        s["y"] = torch.empty((b, L, H, P), dtype=bf, device=dev)
        s["fs"] = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
        s["yd"] = torch.empty((b, H, P), dtype=bf, device=dev)
        sets.append(s)
    ws = torch.empty(max(1, ssd.workspace_bytes(b, L, H, P, N, G, Q)), dtype=torch.uint8,
                     device=dev)
    nseg = ssd.segments(b, L, H, P, N, G, Q)

    def scan(i):
        s = sets[i % nsets]
        ssd.chunk_scan_fwd(s["x"], s["dt"], A, s["B"], s["C"], chunk_size=Q, D=D, dt_bias=bias,
                           initial_states=s["h0"], seq_idx=s["seq"], return_final_states=True,
                           out=s["y"], final_states_out=s["fs"], workspace=ws)

    def decode(i):
        s = sets[i % nsets]
        ssd.state_update(s["fs"], s["xd"], s["dtd"], A, s["Bd"], s["Cd"], D=D, dt_bias=bias,
                         out=s["yd"])

    nk = count_dispatches(lib, scan)
    kernels = {2: ["chunk_prep", "chunk_output"],
               3: ["chunk_prep", "chunk_state", "chunk_output"],
               4: ["chunk_prep", "chunk_state", "state_pass", "chunk_output"]}[nk]

    log("bench: %d warmup steps" % args.warmup)
    for i in range(args.warmup):
        scan(i)
        decode(i)
    torch.cuda.synchronize()
    # the timed steps: a plain stream event on each side of the scan (GPU time
    # of the whole call, launch gaps included)
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    log("bench: %d timed steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        e0[i].record()
        scan(i)
        e1[i].record()
        decode(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    call_us = 1e3 * float(np.mean([e0[i].elapsed_time(e1[i]) for i in range(args.steps)]))
    ms_per_step = 1e3 * elapsed / args.steps
    tokens_per_step = b * L + b
    value = tokens_per_step * args.steps / elapsed
    # the same steps again with HIP events bound to every dispatch of the scan
    # and of the decode update (each pair on the stream its kernel runs on)
    log("bench: %d steps with events bound to every dispatch" % args.steps)

    kus = bound_pass(lib, hip, [scan, decode], [nk, 1], args.steps)
    names = kernels + ["state_update"]
    avg_us = dict(zip(names, kus))
    kernel_sum = sum(kus[:nk])

    # roofline of the whole scan call: its compulsory bytes over the sum of
    # its dispatches' durations
    roof = roofline_entry(scan_bytes, kernel_sum, counter_traffic(w.name))
    step_bytes = scan_bytes + 2 * state_bytes + b * (H * P * 2 * es + 2 * G * N * es + H * 4)
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": b, "seq_len": L, "nheads": H, "headdim": P,
                   "dstate": N, "ngroups": G, "chunk": Q, "decode_tokens_per_step": b,
                   "segments": nseg, "input_copies": nsets},
        "roofline": roof,
        "scan_kernel_us": round(kernel_sum, 2),
        "scan_call_us": round(call_us, 2),
        "kernels_us": {n: round(v, 2) for n, v in avg_us.items()},
        # share of the call's kernel time per dispatch, and the call's bytes
        # over the output kernel's time alone (the figure earlier lines reported)
        "kernel_time_share": {n: round(avg_us[n] / kernel_sum, 4) for n in kernels},
        "chunk_output_frac_of_call_bytes": round(
            scan_bytes / (avg_us["chunk_output"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "scan_mfma_frac": round(scan_flops(b, L, H, P, N, G, Q) / (kernel_sum * 1e-6) / 1e12
                                / MFMA_BF16_PEAK_TFLOPS, 4),
        "source_hash": source_hash(),
    }
    if not args.skip_workloads:
        result["workloads"] = {}
        for name in ("packed_16k", "long_128k", "prefill_decode"):
            log("bench: workload %s" % name)
            ww = workloads.WORKLOADS[WORKLOADS_BY_NAME_ALL[name]]
            result["workloads"][name] = scan_workload_measure(
                ssd, lib, hip, torch, ww, 20 if name != "packed_16k" else 50)
    log("bench: backward pass")
    result["backward"] = backward_measure(ssd, lib, hip, torch, sets[0], A, D, bias, w,
                                          args.backward_steps, min(args.cpu_seconds, 5.0), p)
    log("bench: mixer steps")
    result["mixer"] = mixer_measure(ssd, lib, hip, torch, w, 50, min(args.cpu_seconds, 3.0))
    log("bench: state caches")
    result["cache"] = cache_measure(ssd, lib, hip, torch, w, 50, min(args.cpu_seconds, 2.0))
    if args.cpu_seconds > 0:
        log("bench: CPU oracle baseline (budget %.0f s)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline({k: (v[:, :L] if k in ("x", "dt_raw", "B", "C", "seq_idx") and v is not None else v)
                                               for k, v in p.items()}, w, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
