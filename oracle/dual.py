"""Brute-force matrix ("dual", quadratic) form of the SSD scan, fp64.

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

The recurrence h_t = e^{a_t} h_{t-1} + dt_t x_t (outer) B_t, y_t = h_t . C_t + D x_t
(RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 1 operator family 1) unrolls
into one lower-triangular matrix per (batch, head):

    y_t = sum_{s<=t, same sequence} (C_t . B_s) * prod_{r=s+1..t} e^{a_r} * dt_s * x_s
          + [t in the first sequence] * prod_{r=0..t} e^{a_r} * (h_init . C_t)
          + D x_t

This module builds that matrix with explicit running products of the per-step
decays (no cumulative sums, no chunking), so it shares no intermediate with
either the sequential oracle or the chunked form.  O(L^2) per head: tiny inputs
only.
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


def quadratic_scan(x, dt_raw, A, B, C, *, dt_bias=None, D=None, h_init=None,
                   seq_idx=None, dt_softplus=True, dt_min=0.0, dt_max=np.inf):
    x = np.asarray(x, dtype=np.float64)
    Bm = np.asarray(B, dtype=np.float64)
    Cm = np.asarray(C, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    b, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    dt = _dt(dt_raw, dt_bias, dt_softplus, dt_min, dt_max)  # (b,L,H)
    Dv = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    seq = np.zeros((b, L), dtype=np.int64) if seq_idx is None else np.asarray(seq_idx)
    y = np.zeros((b, L, H, P))
    hf = np.zeros((b, H, P, N))
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            decay = np.exp(dt[bi, :, h] * A[h])  # e^{a_t}
            # prod[t, s] = prod_{r=s+1..t} decay_r for s <= t (explicit products)
            prod = np.zeros((L, L))
            for t in range(L):
                run = 1.0
                prod[t, t] = 1.0
                for s in range(t - 1, -1, -1):
                    run *= decay[s + 1]
                    prod[t, s] = run
            same = seq[bi][:, None] == seq[bi][None, :]
            causal = np.tril(np.ones((L, L), dtype=bool))
            cb = Cm[bi, :, g, :] @ Bm[bi, :, g, :].T  # (L, L): C_t . B_s
            M = np.where(causal & same, cb * prod * dt[bi, :, h][None, :], 0.0)
            y[bi, :, h, :] = M @ x[bi, :, h, :] + Dv[h] * x[bi, :, h, :]
            # final state: tokens of the last sequence, decayed to t = L-1
            last_seq = seq[bi, L - 1]
            for s in range(L):
                if seq[bi, s] == last_seq:
                    hf[bi, h] += prod[L - 1, s] * dt[bi, s, h] * np.outer(
                        x[bi, s, h, :], Bm[bi, s, g, :])
            if h_init is not None:
                h0 = np.asarray(h_init, dtype=np.float64)[bi, h]  # (P, N)
                run = 1.0
                for t in range(L):
                    run *= decay[t]  # prod_{r=0..t} decay_r
                    if seq[bi, t] == seq[bi, 0]:
                        y[bi, t, h, :] += run * (h0 @ Cm[bi, t, g, :])
                if seq[bi, L - 1] == seq[bi, 0]:
                    hf[bi, h] += run * h0
    return y, hf
