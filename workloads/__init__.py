"""Seeded synthetic inputs for the SSD scan workloads.

This module is shared by the fp64 oracle side and the HIP side; it therefore
holds none of the method's arithmetic (no softplus, no decay, no scan): it
only draws the raw inputs, rounds the low-precision ones to bfloat16 with
round-to-nearest-even, and builds the packed-sequence index.

Workloads (shapes of the Nemotron-3-Nano-30B Mamba-2 layer: H=64 heads,
head dim P=64, state N=128, G=8 B/C groups; RL-Kernel RFC
"Nemotron-3-Nano-30B-A3B", section 3 Figure 2: in_proj splits into z 4096,
xBC 6144 and dt 64, so H*P = 4096 and 2*G*N = 2048; SSD chunk 128):

  0 tiny_fp32      b=1  L=256     H=4  P=16 N=16  G=1 Q=64   all fp32
  1 prefill_8k     b=1  L=8192    H=64 P=64 N=128 G=8 Q=128  x/B/C bf16, final state
  2 packed_16k     b=1  L=16384 = 16 packed sequences, Q=128, seq_idx
  3 long_128k      b=1  L=131072  Q=256, random fp32 initial state ~ 0.1*N(0,1)
  4 prefill_decode b=64 rows of 4352 tokens: 4096-token prefill (Q=128)
                   then 256 single-token state updates

Recipe (seeded by 1000 + the workload's index in the table above):
  per-head parameters from the parent generator, in order:
    dt_bias ~ U[-4,-2], A = -exp(U[0, ln 16]), D ~ N(0,1)
  packed lengths (packed_16k) next: u_i ~ U[ln 64, ln 4096], l_i = e^{u_i}
    rescaled to sum to L, floored, remainder given to the largest fractional
    parts (ties to the lower index), each length >= 1;
  per batch row, from SeedSequence(1000+k).spawn(b)[row], in order:
    x ~ N(0,1) (L,H,P), dt_raw ~ N(0,1) (L,H), B ~ N(0,1)/sqrt(N) (L,G,N),
    C ~ N(0,1)/sqrt(N) (L,G,N), then h_init ~ 0.1*N(0,1) (H,P,N) if used.
  x, B, C are rounded to bf16 (RNE) for the bf16 workloads; dt, A, D, states
  stay fp32.  All arrays are returned as float32 numpy arrays whose values are
  exactly representable in the io dtype.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    io: str                 # "f32" or "bf16"
    init_states: bool = False
    final_states: bool = True
    packed: int = 0         # number of packed sequences (0 = no seq_idx)
    prefill: Optional[int] = None   # prefill_decode: tokens scanned before decode
    decode_steps: int = 0

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


WORKLOADS = {
    0: Workload(0, "tiny_fp32", 1, 256, 4, 16, 16, 1, 64, "f32", final_states=True),
    1: Workload(1, "prefill_8k", 1, 8192, 64, 64, 128, 8, 128, "bf16"),
    2: Workload(2, "packed_16k", 1, 16384, 64, 64, 128, 8, 128, "bf16", packed=16),
    3: Workload(3, "long_128k", 1, 131072, 64, 64, 128, 8, 256, "bf16", init_states=True),
    4: Workload(4, "prefill_decode", 64, 4352, 64, 64, 128, 8, 128, "bf16",
                prefill=4096, decode_steps=256),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return them as float32.  Implemented on the bit pattern; NaN stays NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.float32("nan")
    return out.reshape(a.shape)


def packed_lengths(rng: np.random.Generator, count: int, total: int,
                   lo: float = 64.0, hi: float = 4096.0):
    u = rng.uniform(math.log(lo), math.log(hi), size=count)
    raw = np.exp(u)
    scaled = raw * (total / raw.sum())
    base = np.floor(scaled).astype(np.int64)
    base = np.maximum(base, 1)
    rem = total - int(base.sum())
    frac = scaled - np.floor(scaled)
    # remainder to the largest fractional parts, ties to the lower index
    order = sorted(range(count), key=lambda i: (-frac[i], i))
    i = 0
    while rem > 0:
        base[order[i % count]] += 1
        rem -= 1
        i += 1
    while rem < 0:  # only when the >=1 floor pushed the sum over
        j = int(np.argmax(base))
        base[j] -= 1
        rem += 1
    assert int(base.sum()) == total and (base >= 1).all()
    return base


def make_inputs(w: Workload, *, rows: Optional[range] = None, seqlen: Optional[int] = None,
                seed: Optional[int] = None):
    """Draw the inputs of workload ``w``.

    ``rows`` restricts generation to a subset of batch rows (each row has its
    own spawned stream, so a row's values do not depend on which other rows
    are drawn).  ``seqlen`` overrides L (used for reduced-size parity cases).
    Returns a dict of numpy arrays (float32 unless noted).
    """
    k = w.cid if seed is None else seed
    L = w.seqlen if seqlen is None else int(seqlen)
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    parent = np.random.default_rng(1000 + k)
    dt_bias = parent.uniform(-4.0, -2.0, size=H).astype(np.float32)
    A = (-np.exp(parent.uniform(0.0, math.log(16.0), size=H))).astype(np.float32)
    D = parent.standard_normal(H).astype(np.float32)
    seq_idx = None
    lengths = None
    if w.packed:
        lengths = packed_lengths(parent, w.packed, L)
    rows = range(w.batch) if rows is None else rows
    children = np.random.SeedSequence(1000 + k).spawn(w.batch)
    xs, dts, Bs, Cs, h0s = [], [], [], [], []
    rnd = round_bf16 if w.io == "bf16" else (lambda a: np.asarray(a, dtype=np.float32))
    for r in rows:
        g = np.random.default_rng(children[r])
        x = g.standard_normal((L, H, P), dtype=np.float32)
        dt_raw = g.standard_normal((L, H), dtype=np.float32)
        B = (g.standard_normal((L, G, N), dtype=np.float32) / np.float32(math.sqrt(N)))
        C = (g.standard_normal((L, G, N), dtype=np.float32) / np.float32(math.sqrt(N)))
        xs.append(rnd(x))
        dts.append(dt_raw)
        Bs.append(rnd(B))
        Cs.append(rnd(C))
        if w.init_states:
            h0s.append((np.float32(0.1) * g.standard_normal((H, P, N), dtype=np.float32)))
    def stack(parts, shape):
        return np.stack(parts) if parts else np.zeros((0,) + shape, dtype=np.float32)

    out = dict(
        x=stack(xs, (L, H, P)), dt_raw=stack(dts, (L, H)), B=stack(Bs, (L, G, N)),
        C=stack(Cs, (L, G, N)), dt_bias=dt_bias, A=A, D=D,
        h_init=stack(h0s, (H, P, N)) if w.init_states else None,
    )
    if lengths is not None:
        seq_idx = np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)
        out["seq_idx"] = np.broadcast_to(seq_idx, (len(xs), L)).copy()
        out["lengths"] = lengths
    else:
        out["seq_idx"] = None
    return out


def random_problem(rng: np.random.Generator, b, L, H, P, N, G, *, io="f32",
                   init=False, dt_scale=1.0):
    """Small random problem with the workloads' value distributions, for
    parity and property tests at arbitrary shapes."""
    rnd = round_bf16 if io == "bf16" else (lambda a: np.asarray(a, dtype=np.float32))
    return dict(
        x=rnd(rng.standard_normal((b, L, H, P), dtype=np.float32)),
        dt_raw=(dt_scale * rng.standard_normal((b, L, H))).astype(np.float32),
        B=rnd(rng.standard_normal((b, L, G, N), dtype=np.float32) / np.float32(math.sqrt(N))),
        C=rnd(rng.standard_normal((b, L, G, N), dtype=np.float32) / np.float32(math.sqrt(N))),
        dt_bias=rng.uniform(-4.0, -2.0, size=H).astype(np.float32),
        A=(-np.exp(rng.uniform(0.0, math.log(16.0), size=H))).astype(np.float32),
        D=rng.standard_normal(H).astype(np.float32),
        h_init=((np.float32(0.1) * rng.standard_normal((b, H, P, N), dtype=np.float32))
                if init else None),
        seq_idx=None,
    )


def make_inputs_device(w: Workload, device, *, seed: Optional[int] = None,
                       seqlen: Optional[int] = None):
    """The inputs of workload ``w`` drawn directly on ``device`` with torch's
    seeded generator: the same distributions and shapes as ``make_inputs``
    (dt_bias ~ U[-4,-2], A = -exp(U[0, ln 16]), D ~ N(0,1); x, dt_raw ~ N(0,1);
    B, C ~ N(0,1)/sqrt(N); h_init ~ 0.1 N(0,1); packed lengths by the same
    recipe), from a different random stream.  For throughput measurement of
    the large workloads, whose host-side generation takes tens of seconds;
    nothing compares these values with the oracle.  x, B and C come back in
    bfloat16 for the bf16 workloads (torch's conversion rounds to nearest
    even), everything else in float32.  Returns a dict of torch tensors."""
    import torch
    k = w.cid if seed is None else seed
    L = w.seqlen if seqlen is None else int(seqlen)
    b, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    gen = torch.Generator(device=device)
    gen.manual_seed(2000 + k)
    f32 = torch.float32
    io = torch.bfloat16 if w.io == "bf16" else f32

    def u(shape, lo, hi):
        return torch.rand(shape, generator=gen, device=device, dtype=f32) * (hi - lo) + lo

    def n(shape):
        return torch.randn(shape, generator=gen, device=device, dtype=f32)

    out = dict(dt_bias=u((H,), -4.0, -2.0), A=-torch.exp(u((H,), 0.0, math.log(16.0))), D=n((H,)))
    out["x"] = n((b, L, H, P)).to(io)
    out["dt_raw"] = n((b, L, H))
    out["B"] = (n((b, L, G, N)) / math.sqrt(N)).to(io)
    out["C"] = (n((b, L, G, N)) / math.sqrt(N)).to(io)
    out["h_init"] = 0.1 * n((b, H, P, N)) if w.init_states else None
    out["seq_idx"] = None
    if w.packed:
        lengths = packed_lengths(np.random.default_rng(2000 + k), w.packed, L)
        sid = np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)
        out["seq_idx"] = torch.from_numpy(np.broadcast_to(sid, (b, L)).copy()).to(device)
        out["lengths"] = lengths
    return out
