"""GPU parity of the scan's gradients (ssd_chunk_scan_bwd through the C-ABI)
against the fp64 oracle's reverse-mode gradients, on the same bf16-rounded
inputs: every gradient within the bf16 tolerance (relative L2 2e-2)."""
import numpy as np
import pytest

import oracle
import workloads


def to_dev(a, dtype=None):
    """numpy array -> contiguous tensor on cuda:0 (optionally cast; the values
    of bf16 inputs are already representable)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.device("cuda:0"))
    return (t.to(dtype) if dtype is not None else t).contiguous()

pytestmark = pytest.mark.gpu

P, N, Q = 64, 128, 128
TOL = 2e-2
NAMES = {"dx": "dx", "ddt": "ddt_raw", "dA": "dA", "dB": "dB", "dC": "dC", "dD": "dD",
         "ddt_bias": "ddt_bias", "d_initial_states": "dh_init"}


def _problem(seed, b, L, H, G, *, init=False, seq=None, dfinal=False, no_D=False, no_bias=False,
             n=N):
    rng = np.random.default_rng(seed)
    p = workloads.random_problem(rng, b, L, H, P, n, G, io="bf16", init=init)
    p["seq_idx"] = seq
    p["dy"] = workloads.round_bf16(rng.standard_normal((b, L, H, P), dtype=np.float32))
    p["dfinal"] = (rng.standard_normal((b, H, P, n)).astype(np.float32) if dfinal else None)
    if no_D:
        p["D"] = None
    if no_bias:
        p["dt_bias"] = None
    return p


def _run(p, dt_limit=(0.0, float("inf")), softplus=True):
    import torch
    import mamba_ssd_selective_amd as ssd
    bf = torch.bfloat16
    t = lambda k, dtype=None: None if p.get(k) is None else to_dev(p[k], dtype)
    g = ssd.chunk_scan_bwd(t("x", bf), t("dt_raw"), t("A"), t("B", bf), t("C", bf), t("dy", bf),
                           chunk_size=Q, D=t("D"), dt_bias=t("dt_bias"),
                           initial_states=t("h_init"), seq_idx=t("seq_idx"),
                           d_final_states=t("dfinal"), dt_softplus=softplus, dt_limit=dt_limit)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.float().cpu().numpy()) for k, v in g.items()}


def _reference(p, dt_limit=(0.0, float("inf")), softplus=True):
    return oracle.scan_bwd(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], p["dy"],
                           dh_final=p["dfinal"], dt_bias=p["dt_bias"], D=p["D"],
                           h_init=p["h_init"], seq_idx=p["seq_idx"], dt_softplus=softplus,
                           dt_min=dt_limit[0], dt_max=dt_limit[1])


def _compare(gpu, ref, p, tol=TOL):
    errs = {}
    for k, rk in NAMES.items():
        if gpu[k] is None:
            continue
        if k == "dD" and p["D"] is None:
            continue
        errs[k] = oracle.rel_l2(gpu[k], ref[rk])
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, "gradients off the oracle: %s (all: %s)" % (bad, errs)
    return errs


@pytest.mark.parametrize("b,L,H,G", [(1, 128, 4, 1), (2, 300, 8, 2), (1, 1, 2, 1),
                                     (1, 257, 4, 4), (3, 640, 8, 1)])
def test_bwd_parity_shapes(b, L, H, G):
    """Single chunks, ragged tails, one token, a head per group, several rows."""
    p = _problem(100 + L, b, L, H, G, init=True, dfinal=True)
    print("case b=%d L=%d H=%d G=%d" % (b, L, H, G), flush=True)
    _compare(_run(p), _reference(p), p)


def test_bwd_parity_packed_sequences():
    """Resets at a chunk start, in the middle of chunks and near a chunk end;
    the initial state belongs to the first sequence."""
    b, L, H, G = 2, 700, 4, 2
    seq = np.zeros((b, L), dtype=np.int32)
    seq[0, 128:300] = 1
    seq[0, 300:505] = 2
    seq[0, 505:] = 3
    seq[1, 57:] = 4
    p = _problem(7, b, L, H, G, init=True, seq=seq, dfinal=True)
    _compare(_run(p), _reference(p), p)


def test_bwd_parity_clamp_and_optional_inputs():
    """A clamp that binds on both sides (those tokens pass no dt gradient), no
    D, no dt_bias and no final-state gradient."""
    b, L, H, G = 1, 384, 4, 1
    p = _problem(9, b, L, H, G, no_D=True, no_bias=True)
    p["dt_raw"] = (p["dt_raw"] * 2.0 - 3.0).astype(np.float32)
    lim = (0.02, 0.3)
    g = _run(p, dt_limit=lim)
    ref = _reference(p, dt_limit=lim)
    sp = np.logaddexp(0.0, p["dt_raw"].astype(np.float64))
    clamped = (sp < lim[0]) | (sp > lim[1])
    assert clamped.any() and (~clamped).any()
    assert np.all(g["ddt"][clamped] == 0.0)
    _compare(g, ref, p)


def test_bwd_deterministic():
    """Two calls give the same bits (no atomics; fixed summation order)."""
    p = _problem(3, 2, 520, 8, 2, init=True, dfinal=True)
    g1, g2 = _run(p), _run(p)
    for k in g1:
        if g1[k] is not None:
            assert np.array_equal(g1[k], g2[k]), k


def test_bwd_batch_invariant():
    """A row's gradients (dx, d(dt_raw), dB, dC, d(initial_states)) are
    bitwise the same computed alone and inside a batch of three (RFC section
    4.1: batch invariance, forward and backward).  2500 tokens: 20 chunks, so
    the state walks run in two segments.  dA, dD and d(dt_bias) sum over the
    batch and are not per-row quantities."""
    b, L, H, G = 3, 2500, 4, 2
    p = _problem(19, b, L, H, G, init=True, dfinal=True)
    whole = _run(p)
    for r in range(b):
        q = {k: (v[r:r + 1] if k in ("x", "dt_raw", "B", "C", "dy", "h_init", "dfinal") and v is not None
                 else v) for k, v in p.items()}
        alone = _run(q)
        for k in ("dx", "ddt", "dB", "dC", "d_initial_states"):
            assert np.array_equal(whole[k][r:r + 1], alone[k]), (r, k)
    # and the gradients themselves are right
    _compare(whole, _reference(p), p)


def test_bwd_rejects_unsupported():
    """Outside the compiled set the call fails closed before any launch."""
    import torch
    import mamba_ssd_selective_amd as ssd
    p = _problem(1, 1, 64, 2, 1)
    bf = torch.bfloat16
    with pytest.raises(ssd.SSDError):
        ssd.chunk_scan_bwd(to_dev(p["x"], bf), to_dev(p["dt_raw"]), to_dev(p["A"]),
                           to_dev(p["B"], bf), to_dev(p["C"], bf), to_dev(p["dy"], bf),
                           chunk_size=32)


@pytest.mark.parametrize("Q", [64, 128])
def test_bwd_state_size_64(Q):
    """State size N = 64 (with P = 64, chunk 64: the JAX page's Configuration
    defaults), on a ragged length with an initial state, a final-state
    gradient and packed sequences, against the oracle."""
    import torch
    import mamba_ssd_selective_amd as ssd
    b, L, H, G = 2, 700, 4, 2
    seq = np.zeros((b, L), dtype=np.int32)
    seq[:, 300:] = 1
    seq[1, 517:] = 2
    p = _problem(29, b, L, H, G, init=True, dfinal=True, seq=seq, n=64)
    bf = torch.bfloat16
    t = lambda k, dtype=None: to_dev(p[k], dtype)
    g = ssd.chunk_scan_bwd(t("x", bf), t("dt_raw"), t("A"), t("B", bf), t("C", bf), t("dy", bf),
                           chunk_size=Q, D=t("D"), dt_bias=t("dt_bias"), initial_states=t("h_init"),
                           seq_idx=t("seq_idx"), d_final_states=t("dfinal"))
    torch.cuda.synchronize()
    got = {k: (None if v is None else v.float().cpu().numpy()) for k, v in g.items()}
    _compare(got, _reference(p), p)


@pytest.mark.parametrize("Q", [64, 256])
def test_bwd_other_chunk_sizes(Q):
    """The forward's other chunk sizes of this shape: the gradients of the
    same recurrence (run as 128-token chunks), against the oracle."""
    import torch
    import mamba_ssd_selective_amd as ssd
    p = _problem(23, 2, 600, 4, 2, init=True, dfinal=True)
    bf = torch.bfloat16
    t = lambda k, dtype=None: to_dev(p[k], dtype)
    g = ssd.chunk_scan_bwd(t("x", bf), t("dt_raw"), t("A"), t("B", bf), t("C", bf), t("dy", bf),
                           chunk_size=Q, D=t("D"), dt_bias=t("dt_bias"), initial_states=t("h_init"),
                           d_final_states=t("dfinal"))
    torch.cuda.synchronize()
    got = {k: (None if v is None else v.float().cpu().numpy()) for k, v in g.items()}
    _compare(got, _reference(p), p)


def test_bwd_prefill_8k_one_group():
    """The 8K-token prefill shape (b 1, L 8192, H 64, G 8) on the GPU; the
    oracle runs on the heads of group 3, whose gradients (dB, dC of that
    group included) are compared."""
    rng = np.random.default_rng(41)
    b, L, H, G = 1, 8192, 64, 8
    p = workloads.random_problem(rng, b, L, H, P, N, G, io="bf16", init=True)
    p["seq_idx"] = None
    p["dy"] = workloads.round_bf16(rng.standard_normal((b, L, H, P), dtype=np.float32))
    p["dfinal"] = rng.standard_normal((b, H, P, N)).astype(np.float32)
    g = _run(p)
    grp = 3
    hs = slice(8 * grp, 8 * grp + 8)
    ref = oracle.scan_bwd(p["x"][:, :, hs], p["dt_raw"][:, :, hs], p["A"][hs],
                          p["B"][:, :, grp:grp + 1], p["C"][:, :, grp:grp + 1], p["dy"][:, :, hs],
                          dh_final=p["dfinal"][:, hs], dt_bias=p["dt_bias"][hs], D=p["D"][hs],
                          h_init=p["h_init"][:, hs])
    sub = {"dx": g["dx"][:, :, hs], "ddt": g["ddt"][:, :, hs], "dA": g["dA"][hs],
           "dB": g["dB"][:, :, grp:grp + 1], "dC": g["dC"][:, :, grp:grp + 1],
           "dD": g["dD"][hs], "ddt_bias": g["ddt_bias"][hs],
           "d_initial_states": g["d_initial_states"][:, hs]}
    print(_compare(sub, ref, p), flush=True)
