"""Chunked decomposition of the SSD scan in numpy fp64, for any chunk size.

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

The pages name the training-side algorithm a chunked parallel scan with chunk
128 (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 1 operator family 1 and
section 3 Figure 2, box [F2] "SSD chunked scan"; "Nemotron 3 Nano - JAX
Implementation", Key Components item 1: the chunked SSD keeps memory bounded).
They do not print its steps; the ones below follow from the recurrence
h_t = e^{a_t} h_{t-1} + dt_t x_t (outer) B_t, y_t = h_t . C_t + D x_t, because
token j's contribution to the state at token i (j <= i, no reset between them)
is e^{cs_i - cs_j} dt_j x_j (outer) B_j with cs the running sum of a:

1. per chunk, the inclusive sum cs of a_t = dt_t A restarted at the chunk start;
2. chunk state S_c = sum_{j in c, same sequence as the chunk's last token}
   e^{cs_last - cs_j} dt_j x_j (outer) B_j;
3. state passing h_c = [no reset since the previous chunk's last token]
   * e^{cs_last} h_{c-1} + S_c, starting from h_init;
4. chunk output y_i = sum_{j<=i, same sequence} (C_i . B_j) e^{cs_i - cs_j} dt_j x_j
   + [same sequence as the previous chunk's last token] e^{cs_i} h_{c-1} . C_i
   + D x_i.

The "previous chunk's last token" of chunk 0 is token 0 (the initial state
belongs to the sequence holding token 0).  L need not be a multiple of Q: the
last chunk is shorter.  The library routines used per step are numpy matmul
and cumsum only; nothing is blocked or fused beyond the four steps above.
"""
from __future__ import annotations

import numpy as np


def _dt(dt_raw, dt_bias, softplus, dt_min, dt_max):
    v = np.asarray(dt_raw, dtype=np.float64)
    if dt_bias is not None:
        v = v + np.asarray(dt_bias, dtype=np.float64)
    if softplus:
        v = np.logaddexp(0.0, v)
    return np.clip(v, dt_min, dt_max)


def chunked_scan(x, dt_raw, A, B, C, *, chunk, dt_bias=None, D=None, h_init=None,
                 seq_idx=None, dt_softplus=True, dt_min=0.0, dt_max=np.inf):
    x = np.asarray(x, dtype=np.float64)
    Bm = np.asarray(B, dtype=np.float64)
    Cm = np.asarray(C, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    b, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    Q = int(chunk)
    assert Q >= 1
    dt = _dt(dt_raw, dt_bias, dt_softplus, dt_min, dt_max)
    Dv = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    seq = np.zeros((b, L), dtype=np.int64) if seq_idx is None else np.asarray(seq_idx)
    y = np.zeros((b, L, H, P))
    hf = np.zeros((b, H, P, N))
    nc = (L + Q - 1) // Q
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            state = (np.zeros((P, N)) if h_init is None
                     else np.asarray(h_init, dtype=np.float64)[bi, h].copy())
            prev_last_seq = seq[bi, 0] if L > 0 else 0
            for c in range(nc):
                t0, t1 = c * Q, min((c + 1) * Q, L)
                xs = x[bi, t0:t1, h, :]            # (q, P)
                Bs = Bm[bi, t0:t1, g, :]           # (q, N)
                Cs = Cm[bi, t0:t1, g, :]           # (q, N)
                dts = dt[bi, t0:t1, h]             # (q,)
                sq = seq[bi, t0:t1]
                # step 1: chunk-local inclusive cumsum of a = dt * A
                cs = np.cumsum(dts * A[h])
                # step 4 (uses h_{c-1}): intra-chunk quadratic part + carried state
                diff = cs[:, None] - cs[None, :]
                causal = np.tril(np.ones((t1 - t0, t1 - t0), dtype=bool))
                same = sq[:, None] == sq[None, :]
                Lmat = np.where(causal & same, np.exp(np.where(causal, diff, 0.0)), 0.0)
                G_ = (Cs @ Bs.T) * Lmat * dts[None, :]
                yc = G_ @ xs
                carried = np.exp(cs)[:, None] * (Cs @ state.T)
                yc += np.where((sq == prev_last_seq)[:, None], carried, 0.0)
                yc += Dv[h] * xs
                y[bi, t0:t1, h, :] = yc
                # step 2: chunk state from the tokens of the chunk's last sequence
                w = np.where(sq == sq[-1], np.exp(cs[-1] - cs) * dts, 0.0)
                S = (xs * w[:, None]).T @ Bs       # (P, N)
                # step 3: state passing
                if sq[-1] == prev_last_seq:
                    state = np.exp(cs[-1]) * state + S
                else:
                    state = S
                prev_last_seq = sq[-1]
            hf[bi, h] = state
    return y, hf
