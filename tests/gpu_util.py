"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
HIP path through its binding, run the oracle on the same values."""
import sys

import numpy as np

import oracle


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device():
    import torch
    return torch.device("cuda:0")


def to_dev(p, io, keys=("x", "dt_raw", "B", "C", "dt_bias", "A", "D", "h_init", "seq_idx")):
    """numpy problem dict -> torch tensors on cuda:0; x, B, C in the io dtype
    (their values are already representable in it)."""
    import torch
    dev = device()
    io_t = torch.bfloat16 if io == "bf16" else torch.float32
    out = {}
    for k in keys:
        v = p.get(k)
        if v is None:
            out[k] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(v)).to(dev)
        if k in ("x", "B", "C"):
            t = t.to(io_t)
        out[k] = t.contiguous()
    return out


def run_scan(t, chunk, *, final=True, zero_D=False, **kw):
    import torch
    import mamba_ssd_selective_amd as ssd
    D = torch.zeros_like(t["D"]) if zero_D else t["D"]
    r = ssd.chunk_scan_fwd(t["x"], t["dt_raw"], t["A"], t["B"], t["C"], chunk_size=chunk, D=D,
                           dt_bias=t["dt_bias"], initial_states=t["h_init"],
                           seq_idx=t["seq_idx"], return_final_states=final, **kw)
    torch.cuda.synchronize()
    return r


def run_oracle(p, *, zero_D=False, **kw):
    D = np.zeros_like(p["D"]) if zero_D else p["D"]
    return oracle.scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], dt_bias=p["dt_bias"], D=D,
                       h_init=p.get("h_init"), seq_idx=p.get("seq_idx"), **kw)


def host(t):
    return t.float().cpu().numpy()


def tol(io):
    """Relative L2 tolerance: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs with fp32 state."""
    return 1e-4 if io == "f32" else 2e-2


def head_subset(p, heads):
    """The sub-problem of a head subset, each head with its own copy of its
    group's B/C (G' = len(heads)); the recurrence is independent per head."""
    H = p["A"].shape[0]
    G = p["B"].shape[2]
    hpg = H // G
    heads = np.asarray(heads)
    groups = heads // hpg
    sub = dict(p)
    sub["x"] = p["x"][:, :, heads, :]
    sub["dt_raw"] = p["dt_raw"][:, :, heads]
    sub["B"] = p["B"][:, :, groups, :]
    sub["C"] = p["C"][:, :, groups, :]
    for k in ("A", "D", "dt_bias"):
        sub[k] = p[k][heads]
    if p.get("h_init") is not None:
        sub["h_init"] = p["h_init"][:, heads]
    return sub
