"""CPU pins for the oracle's gradients (oracle.scan_bwd, no GPU).

The gradients are tied to the forward recurrence through checks that never
run the reverse-mode code: central finite differences of the forward oracle
along random directions of every input, and the exact identities that follow
from the outputs being linear in (x, h_init), in B (zero initial state) and in
C.  Planted mistakes in a copy of the reverse-mode source must fail them.
"""
import numpy as np
import pytest

import oracle
import workloads

DT_MIN, DT_MAX = 0.03, 0.3  # some tokens of the case below are clamped on each side
INPUTS = ("x", "dt_raw", "A", "B", "C", "D", "dt_bias", "h_init")


def _case(seed=5, b=2, L=70, H=4, P=3, N=5, G=2):
    """Two rows crossing one oracle checkpoint (64 tokens): row 0 packs three
    sequences, row 1 holds one; groups of two heads, an initial state, D and
    dt_bias, softplus and a clamp that binds on both sides."""
    rng = np.random.default_rng(seed)
    p = workloads.random_problem(rng, b, L, H, P, N, G, init=True, dt_scale=2.0)
    p = {k: (None if v is None else np.asarray(v, dtype=np.float64)) for k, v in p.items()}
    seq = np.zeros((b, L), dtype=np.int32)
    seq[0, 20:45] = 1
    seq[0, 45:] = 2
    seq[1, :] = 7
    p["seq_idx"] = seq
    wy = rng.standard_normal((b, L, H, P))
    wh = rng.standard_normal((b, H, P, N))
    return p, wy, wh


def _loss(p, wy, wh, lib=None):
    y, hf = oracle.scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], dt_bias=p["dt_bias"],
                        D=p["D"], h_init=p["h_init"], seq_idx=p["seq_idx"], dt_min=DT_MIN,
                        dt_max=DT_MAX, lib=lib)
    return float(np.sum(wy * y) + np.sum(wh * hf)), y, hf


def _grads(p, wy, wh, lib=None):
    return oracle.scan_bwd(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], wy, dh_final=wh,
                           dt_bias=p["dt_bias"], D=p["D"], h_init=p["h_init"],
                           seq_idx=p["seq_idx"], dt_min=DT_MIN, dt_max=DT_MAX, lib=lib)


GRAD_OF = {"x": "dx", "dt_raw": "ddt_raw", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
           "dt_bias": "ddt_bias", "h_init": "dh_init"}


def _directional_failures(lib=None, eps=1e-6, rtol=1e-6):
    """Names of the inputs whose gradient disagrees with the central difference
    of the forward loss along two random directions."""
    p, wy, wh = _case()
    g = _grads(p, wy, wh, lib=lib)
    rng = np.random.default_rng(11)
    bad = []
    for name in INPUTS:
        for _ in range(2):
            v = rng.standard_normal(p[name].shape)
            plus = dict(p); plus[name] = p[name] + eps * v
            minus = dict(p); minus[name] = p[name] - eps * v
            fd = (_loss(plus, wy, wh, lib)[0] - _loss(minus, wy, wh, lib)[0]) / (2 * eps)
            an = float(np.sum(g[GRAD_OF[name]] * v))
            if not abs(fd - an) <= rtol * max(1.0, abs(an)):
                bad.append(name)
                break
    return bad


def test_gradients_match_finite_differences():
    """Every gradient, projected on random directions, equals the central
    difference of the forward oracle's loss (fp64, step 1e-6)."""
    assert _directional_failures() == []


def test_elementwise_finite_differences_at_special_tokens():
    """Single entries at the places a reverse pass most easily gets wrong: the
    first token, a sequence start (no state flows in), the token before it,
    the last token (final-state gradient) and a clamped dt (zero gradient)."""
    p, wy, wh = _case()
    g = _grads(p, wy, wh)
    dt = np.clip(np.logaddexp(0.0, p["dt_raw"] + p["dt_bias"]), DT_MIN, DT_MAX)
    sp = np.logaddexp(0.0, p["dt_raw"] + p["dt_bias"])
    clamped = np.argwhere((sp < DT_MIN) | (sp > DT_MAX))
    assert len(clamped) > 0 and np.any(sp > DT_MAX) and np.any(sp < DT_MIN)
    eps = 1e-6
    picks = [("dt_raw", (0, 0, 1)), ("dt_raw", (0, 20, 2)), ("dt_raw", (0, 19, 0)),
             ("dt_raw", (1, 69, 3)), ("dt_raw", tuple(clamped[0])), ("x", (0, 20, 1, 2)),
             ("x", (1, 0, 3, 0)), ("B", (0, 45, 1, 4)), ("C", (1, 69, 0, 2)),
             ("h_init", (0, 2, 1, 3)), ("h_init", (1, 0, 2, 4))]
    for name, idx in picks:
        plus = dict(p); plus[name] = p[name].copy(); plus[name][idx] += eps
        minus = dict(p); minus[name] = p[name].copy(); minus[name][idx] -= eps
        fd = (_loss(plus, wy, wh)[0] - _loss(minus, wy, wh)[0]) / (2 * eps)
        an = g[GRAD_OF[name]][idx]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an)
    # a clamped dt passes no gradient to dt_raw
    for idx in clamped:
        assert g["ddt_raw"][tuple(idx)] == 0.0
    assert np.all(dt[tuple(clamped.T)] != 0)


def test_linearity_identities():
    """y and the final state are linear in (x, h_init) jointly; with zero
    initial state they are linear in B; y - D x is linear in C.  Hence
    <dy, y> + <dh, h_final> = <dx, x> + <dh_init, h_init> = <dB, B> (h_init = 0),
    <dy, y - D x> = <dC, C> and <dy, D x> = <dD, D>."""
    p, wy, wh = _case(seed=8)
    lval, y, hf = _loss(p, wy, wh)
    g = _grads(p, wy, wh)
    lhs = np.sum(g["dx"] * p["x"]) + np.sum(g["dh_init"] * p["h_init"])
    assert abs(lhs - lval) <= 1e-12 * np.sum(np.abs(wy * y)) + 1e-12
    dx_part = np.sum(wy * p["D"][None, None, :, None] * p["x"])
    assert abs(np.sum(g["dD"] * p["D"]) - dx_part) <= 1e-12 * abs(dx_part) + 1e-12
    assert abs(np.sum(g["dC"] * p["C"]) - (np.sum(wy * y) - dx_part)) <= 1e-10
    p0 = dict(p); p0["h_init"] = None
    l0, _, _ = _loss(p0, wy, wh)
    g0 = _grads(p0, wy, wh)
    assert abs(np.sum(g0["dB"] * p0["B"]) - (l0 - dx_part)) <= 1e-10


# ------------------------------------------------------ planted mistakes

MUTATIONS = {
    "no_decay_term_in_ddt": ("ddt += Ah * a * gh;", "(void)gh;"),
    "no_dA": ("accA += dt * a * gh;", "(void)0;"),
    "no_reset_in_reverse": ("} else {\n                    memset(gs, 0, sizeof(double) * (size_t)PN);",
                            "} else {\n                    for (int64_t i = 0; i < PN; ++i) gs[i] *= a;"),
    "dB_without_dt": ("dbt[n] = dt * acc;", "dbt[n] = acc;"),
    "dC_from_previous_state": ("acc += cur[p * N + n] * dyt[p];", "acc += prev[p * N + n] * dyt[p];"),
    "dx_without_D": ("dx[((b * L + t) * H + h) * P + p] = dt * acc + Dh * dyt[p];",
                     "dx[((b * L + t) * H + h) * P + p] = dt * acc;"),
    "clamp_passes_gradient": ("const int pass = sp >= dt_min && sp <= dt_max;", "const int pass = 1;"),
    "no_softplus_derivative": ("draw = dt_softplus ? ddt / (1.0 + exp(-v)) : ddt;", "draw = ddt;"),
    "gradient_before_output_term": ("for (int64_t n = 0; n < N; ++n) gs[p * N + n] += dyt[p] * ct[n];",
                                    "for (int64_t n = 0; n < N; ++n) gs[p * N + n] += 0.0 * dyt[p] * ct[n];"),
    "dh_final_ignored": ("if (dh_final) memcpy(gs, dh_final", "if (0) memcpy(gs, dh_final"),
}


def test_gradient_pins_catch_planted_mistakes(tmp_path):
    """Each plausible mistake planted in the reverse-mode code of a copy of the
    oracle source makes the finite-difference pin fail; the unmodified source
    passes."""
    src = oracle.source_text()
    assert _directional_failures(oracle._load()) == []
    for name, (old, new) in MUTATIONS.items():
        assert src.count(old) == 1, name
        path = oracle.compile_variant(src.replace(old, new), str(tmp_path / ("b_%s.so" % name)))
        assert _directional_failures(oracle._load(path)), "mutation %s went undetected" % name


@pytest.mark.parametrize("L", [1, 64, 65])
def test_checkpoint_boundaries(L):
    """Lengths at and around the oracle's checkpoint stride give the same
    gradients as a run whose stretches hold every token (directional pin at
    these lengths)."""
    rng = np.random.default_rng(L)
    p = workloads.random_problem(rng, 1, L, 2, 3, 4, 1, init=True)
    p = {k: (None if v is None else np.asarray(v, dtype=np.float64)) for k, v in p.items()}
    wy = rng.standard_normal((1, L, 2, 3))
    g = oracle.scan_bwd(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], wy, dt_bias=p["dt_bias"],
                        D=p["D"], h_init=p["h_init"])
    eps = 1e-6
    for name in ("x", "dt_raw", "B", "h_init"):
        v = rng.standard_normal(p[name].shape)
        vals = []
        for sgn in (1, -1):
            q = dict(p); q[name] = p[name] + sgn * eps * v
            y, _ = oracle.scan(q["x"], q["dt_raw"], q["A"], q["B"], q["C"], dt_bias=q["dt_bias"],
                               D=q["D"], h_init=q["h_init"])
            vals.append(np.sum(wy * y))
        fd = (vals[0] - vals[1]) / (2 * eps)
        an = np.sum(g[GRAD_OF[name]] * v)
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), name
