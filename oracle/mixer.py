"""fp64 oracle of the steps beside the scan in the Mamba-2 mixer: the causal
depthwise conv1d with bias and SiLU (with its conv-state cache) that produces
the scan's x, B and C, and the gated group RMSNorm applied to the scan's
output (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 3, Figure 2, box
[F2]: "causal conv1d k=4 + bias + SiLU, conv-state cache" feeding the SSD scan,
and "gated group RMSNorm norm(y * silu(z)), group 512" after it; the kernel
width 4 and the RMSNorm epsilon 1e-6 are the "Nemotron 3 Nano - JAX
Implementation" page's Configuration values mamba_d_conv and rms_norm_eps).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): shares no code with the
HIP library.

Readings (the pages name the operations; their plainest forms):
* conv: out_t[c] = silu(bias[c] + sum_{k=0}^{K-1} w[c, k] in_{t-K+1+k}[c]),
  weight (channels, K); inputs before the first token come from the conv
  state (the last K-1 inputs of the previous call, oldest first) or are zero;
  with packed sequences, inputs of another sequence count as zero (the state
  belongs to the sequence of token 0, like the scan's initial state).  The
  new conv state holds the last K-1 inputs (the old state's tail when L < K-1),
  zero where they belong to another sequence than the last token's.
* the conv output channels split into x (first H*P), B (next G*N) and C
  (last G*N), the scan's three inputs.
* gated norm: v = y * silu(z); per group of `group` consecutive channels,
  out = v / sqrt(mean(v^2) + eps) * weight.
"""
from __future__ import annotations

import numpy as np


def silu(v):
    """v * sigmoid(v), without overflow for large |v|."""
    v = np.asarray(v, dtype=np.float64)
    return v * np.where(v >= 0, 1.0 / (1.0 + np.exp(-np.abs(v))),
                        np.exp(-np.abs(v)) / (1.0 + np.exp(-np.abs(v))))


def conv1d(xbc, weight, bias=None, conv_state=None, seq_idx=None):
    """Causal depthwise conv + bias + SiLU over (b, L, D).

    Returns (out (b, L, D), new_state (b, D, K-1)), float64."""
    xbc = np.asarray(xbc, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    b, L, D = xbc.shape
    K = w.shape[1]
    assert w.shape == (D, K)
    st = (np.zeros((b, D, K - 1)) if conv_state is None
          else np.asarray(conv_state, dtype=np.float64))
    assert st.shape == (b, D, K - 1)
    # the input stream with the state in front: ext[:, K-1+t] = in_t
    ext = np.concatenate([np.transpose(st, (0, 2, 1)), xbc], axis=1)  # (b, K-1+L, D)
    seq = None if seq_idx is None else np.asarray(seq_idx)
    acc = np.zeros((b, L, D))
    for k in range(K):
        # tap k reads in_{t-K+1+k} = ext[:, t+k]
        src = ext[:, k:k + L, :].copy()
        if seq is not None:
            lag = K - 1 - k
            for r in range(b):
                for t in range(L):
                    j = t - lag
                    # inputs of another sequence (and state inputs, which belong
                    # to the sequence of token 0) count as zero
                    if j >= 0 and seq[r, j] != seq[r, t]:
                        src[r, t] = 0.0
                    elif j < 0 and seq[r, 0] != seq[r, t]:
                        src[r, t] = 0.0
        acc += src * w[None, None, :, k]
    if bias is not None:
        acc += np.asarray(bias, dtype=np.float64)[None, None, :]
    new_state = np.transpose(ext[:, L:, :], (0, 2, 1)).copy()  # last K-1 inputs
    if seq is not None and L > 0:
        # only inputs of the last token's sequence are carried on
        for r in range(b):
            for k in range(K - 1):
                j = L - (K - 1) + k  # token index of state slot k (negative: old state)
                same = seq[r, j] == seq[r, L - 1] if j >= 0 else seq[r, 0] == seq[r, L - 1]
                if not same:
                    new_state[r, :, k] = 0.0
    return silu(acc), new_state


def conv1d_update(xbc_t, weight, bias, conv_state):
    """One decode token: xbc_t (b, D), conv_state (b, D, K-1).  Returns
    (out (b, D), new_state)."""
    out, st = conv1d(np.asarray(xbc_t)[:, None, :], weight, bias, conv_state)
    return out[:, 0, :], st


def split_xbc(out, H, P, G, N):
    """The conv output's channels as the scan's x (b, L, H, P), B, C (b, L, G, N)."""
    b, L, D = out.shape
    assert D == H * P + 2 * G * N
    x = out[:, :, :H * P].reshape(b, L, H, P)
    Bm = out[:, :, H * P:H * P + G * N].reshape(b, L, G, N)
    Cm = out[:, :, H * P + G * N:].reshape(b, L, G, N)
    return x, Bm, Cm


def gated_rmsnorm(y, z, weight, group, eps=1e-6):
    """norm(y * silu(z)) per group of `group` channels of the last axis, times
    weight; float64."""
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    v = y * silu(z)
    shape = v.shape
    D = shape[-1]
    assert D % group == 0
    vg = v.reshape(shape[:-1] + (D // group, group))
    ms = np.mean(vg * vg, axis=-1, keepdims=True)
    out = (vg / np.sqrt(ms + eps)).reshape(shape)
    return out * np.asarray(weight, dtype=np.float64)
