"""The fp64 oracle against an independent implementation of the same operation:
the naive (pure torch) SSD path of transformers' NemotronH model.

The RL-Kernel RFC "Nemotron-3-Nano-30B-A3B" (section 2, "Reference-implementation
hazards") names that torch path as a numerical reference worth keeping beside
the kernels.  It shares nothing with the oracle: it computes the chunked form
(segment sums, chunk states, an inter-chunk recurrence) in fp32 torch, while
the oracle runs the sequential recurrence in fp64 C.  Agreement pins the
readings the oracle takes where the pages are silent (exp(dt*A) decay, the
Euler input term dt*x*B, the output after the update, contiguous head groups,
softplus then clamp, the D skip on the input, the initial state entering the
first token's decay) against a third party's choices.

Skipped when transformers is not importable.  Run offline: nothing is fetched.
"""
import os

import numpy as np
import pytest

import oracle

os.environ.setdefault("HF_HUB_OFFLINE", "1")
os.environ.setdefault("TRANSFORMERS_OFFLINE", "1")

torch = pytest.importorskip("torch")
nh = pytest.importorskip("transformers.models.nemotron_h.modeling_nemotron_h")

# fp32 torch against fp64: the bound is fp32 rounding over a few hundred terms
TOL = 1e-5


def _problem(seed, b, L, H, P, N, G, init):
    rng = np.random.default_rng(seed)
    p = {
        "x": rng.standard_normal((b, L, H, P)),
        "dt_raw": rng.standard_normal((b, L, H)),
        "A": -np.exp(rng.uniform(0.0, np.log(16.0), H)),
        "B": rng.standard_normal((b, L, G, N)) / np.sqrt(N),
        "C": rng.standard_normal((b, L, G, N)) / np.sqrt(N),
        "D": rng.standard_normal(H),
        "dt_bias": rng.uniform(-4.0, -2.0, H),
        "h_init": 0.1 * rng.standard_normal((b, H, P, N)) if init else None,
    }
    # values exactly representable in fp32, so both sides see the same inputs
    return {k: (None if v is None else v.astype(np.float32).astype(np.float64)) for k, v in p.items()}


def _t(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


@pytest.mark.parametrize("L,chunk,init,with_D,limit", [
    (64, 16, False, True, None),
    (200, 64, True, True, None),       # ragged last chunk, initial state
    (128, 32, True, False, None),      # no D
    (150, 64, False, True, (0.02, 0.3)),  # a clamp that binds on both sides
])
def test_scan_matches_transformers_naive_ssd(L, chunk, init, with_D, limit):
    b, H, P, N, G = 2, 4, 8, 16, 2
    p = _problem(100 + L, b, L, H, P, N, G, init)
    lo, hi = limit if limit else (0.0, float("inf"))
    y, hf = oracle.scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], dt_bias=p["dt_bias"],
                        D=p["D"] if with_D else None, h_init=p["h_init"], dt_min=lo, dt_max=hi)
    with torch.no_grad():
        yr, hr = nh.mamba2_chunk_scan(_t(p["x"]), _t(p["dt_raw"]), _t(p["A"]), _t(p["B"]), _t(p["C"]),
                                      chunk, D=_t(p["D"]) if with_D else None,
                                      dt_bias=_t(p["dt_bias"]), initial_states=_t(p["h_init"]),
                                      dt_softplus=True, dt_limit=(lo, hi), return_final_states=True)
    e_y = oracle.rel_l2(yr.double().numpy(), y)
    e_h = oracle.rel_l2(hr.double().numpy(), hf)
    assert e_y < TOL and e_h < TOL, (e_y, e_h)
    if with_D:
        # without the D skip the scan terms alone must agree too (they are
        # about a hundredth of D x, which would hide a mistake in them)
        y0, _ = oracle.scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], dt_bias=p["dt_bias"],
                            h_init=p["h_init"], dt_min=lo, dt_max=hi)
        with torch.no_grad():
            yr0 = nh.mamba2_chunk_scan(_t(p["x"]), _t(p["dt_raw"]), _t(p["A"]), _t(p["B"]), _t(p["C"]),
                                       chunk, dt_bias=_t(p["dt_bias"]), initial_states=_t(p["h_init"]),
                                       dt_softplus=True, dt_limit=(lo, hi))
        assert oracle.rel_l2(yr0.double().numpy(), y0) < TOL


@pytest.mark.parametrize("with_D", [True, False])
def test_step_matches_transformers_state_update(with_D):
    """One decode token.  The torch routine takes dt per (head, p) and A per
    (head, p, n); the head's scalars are broadcast to those shapes."""
    b, H, P, N, G = 3, 4, 8, 16, 2
    p = _problem(7, b, 1, H, P, N, G, True)
    state0 = p["h_init"]
    s_new, y = oracle.step(state0, p["x"][:, 0], p["dt_raw"][:, 0], p["A"], p["B"][:, 0], p["C"][:, 0],
                           dt_bias=p["dt_bias"], D=p["D"] if with_D else None)
    st = _t(state0).clone()
    dt_hp = np.repeat(p["dt_raw"][:, 0][:, :, None], P, axis=2)
    A_hpn = np.broadcast_to(p["A"][:, None, None], (H, P, N))
    with torch.no_grad():
        yr = nh.mamba2_selective_state_update(
            st, _t(p["x"][:, 0]), _t(dt_hp), _t(A_hpn), _t(p["B"][:, 0]), _t(p["C"][:, 0]),
            D=_t(p["D"][:, None]) if with_D else None, dt_bias=_t(p["dt_bias"][:, None]),
            dt_softplus=True)
    assert oracle.rel_l2(yr.double().numpy(), y) < TOL
    assert oracle.rel_l2(st.double().numpy(), s_new) < TOL
