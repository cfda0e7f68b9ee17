"""CPU pins for the fp64 oracle (no GPU).

Every check here ties the oracle to something other than itself: hand-derived
closed forms (tests/golden), a textbook library routine (scipy.signal.lfilter),
the brute-force matrix form written independently (oracle.dual), the chunk
decomposition (oracle.chunked) and invariants the pages imply (sequence-split
and batch invariance, RL-Kernel RFC "Nemotron-3-Nano-30B-A3B" section 4.1;
packing and resets, same RFC section 8 question 4).
"""
import math
import os

import numpy as np
import pytest
import scipy.signal

import oracle
import workloads
from oracle.chunked import chunked_scan
from oracle.dual import quadratic_scan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _scan(p, **kw):
    return oracle.scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], dt_bias=p["dt_bias"],
                       D=p["D"], h_init=p["h_init"], seq_idx=p.get("seq_idx"), **kw)


def _problem(seed, b, L, H, P, N, G, init=False, seq=None):
    rng = np.random.default_rng(seed)
    p = workloads.random_problem(rng, b, L, H, P, N, G, init=init)
    if seq is not None:
        p["seq_idx"] = seq
    return p


def _packed_seq(rng, b, L, nseq):
    rows = []
    for _ in range(b):
        cuts = np.sort(rng.choice(np.arange(1, L), size=nseq - 1, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [L]]))
        rows.append(np.repeat(np.arange(nseq, dtype=np.int32) + 3, lens))
    return np.stack(rows)


# ---------------------------------------------------------------- generator


def test_round_bf16_matches_torch_rne():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1e-40, 3.4e38, -3.4e38, np.inf, -np.inf],
                                 dtype=np.float32)])
    # values exactly halfway between two bf16 numbers: ties go to even
    halves = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    a = np.concatenate([a, halves])
    ours = workloads.round_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_packed_lengths_recipe():
    w = workloads.WORKLOADS[2]
    p = workloads.make_inputs(w, seqlen=w.seqlen, rows=range(0))  # no rows: params only
    lens = p["lengths"]
    assert len(lens) == 16 and lens.sum() == 16384 and (lens >= 1).all()
    # drawn log-uniform on [64, 4096] then rescaled by one common factor
    ratio = lens.max() / lens.min()
    assert ratio <= 4096 / 64 + 1


def test_generator_row_streams_independent():
    w = workloads.WORKLOADS[4]
    a = workloads.make_inputs(w, rows=range(2, 3), seqlen=64)
    b = workloads.make_inputs(w, rows=range(0, 4), seqlen=64)
    assert np.array_equal(a["x"][0], b["x"][2])
    assert np.array_equal(a["B"][0], b["B"][2])


# ------------------------------------------------------- closed forms (pins)


def _scalar(x, A, *, D=0.0, h0=None, dt_raw=1.0):
    L = len(x)
    return dict(
        x=np.asarray(x, dtype=np.float64).reshape(1, L, 1, 1),
        dt_raw=np.full((1, L, 1), dt_raw), B=np.ones((1, L, 1, 1)), C=np.ones((1, L, 1, 1)),
        A=np.array([A]), D=np.array([D]), dt_bias=np.zeros(1),
        h_init=None if h0 is None else np.full((1, 1, 1, 1), h0), seq_idx=None)


def test_golden_cumsum_when_A_is_zero():
    """P-1: A = 0, dt = 1, B = C = 1, D = 0 gives a running sum (exact)."""
    with open(os.path.join(GOLDEN, "cumsum_a_zero.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    x = [float(v) for v in rows[0][1:]]
    want = [float(v) for v in rows[1][1:]]
    y, hf = _scan(_scalar(x, 0.0), dt_softplus=False)
    assert np.array_equal(y.reshape(-1), np.array(want))
    assert hf.reshape(-1)[0] == want[-1]


def test_golden_geometric_halving():
    """Hand-derived closed form: decay exactly 1/2 per step, D = 1/2, h0 = 4."""
    with open(os.path.join(GOLDEN, "geometric_halving.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    ys = {int(r[0]): float(r[1]) for r in rows if r[0] != "final"}
    final = [float(r[1]) for r in rows if r[0] == "final"][0]
    L = len(ys)
    y, hf = _scan(_scalar(np.ones(L), -math.log(2.0), D=0.5, h0=4.0), dt_softplus=False)
    np.testing.assert_allclose(y.reshape(-1), [ys[t] for t in range(L)], rtol=1e-14, atol=0)
    np.testing.assert_allclose(hf.reshape(-1)[0], final, rtol=1e-14)


def test_single_token_formula():
    """P-2: for L = 1 the output is dt (C.B) x + e^{dt A} (h0 . C) + D x."""
    p = _problem(11, 2, 1, 6, 5, 7, 3, init=True)
    y, hf = _scan(p)
    dt = np.logaddexp(0.0, p["dt_raw"].astype(np.float64) + p["dt_bias"])  # (b,1,H)
    for b in range(2):
        for h in range(6):
            g = h // 2
            Bv = p["B"][b, 0, g].astype(np.float64)
            Cv = p["C"][b, 0, g].astype(np.float64)
            xv = p["x"][b, 0, h].astype(np.float64)
            h0 = p["h_init"][b, h].astype(np.float64)
            d = dt[b, 0, h]
            want = d * (Cv @ Bv) * xv + math.exp(d * p["A"][h]) * (h0 @ Cv) + p["D"][h] * xv
            np.testing.assert_allclose(y[b, 0, h], want, rtol=1e-13, atol=1e-15)
            want_h = math.exp(d * p["A"][h]) * h0 + d * np.outer(xv, Bv)
            np.testing.assert_allclose(hf[b, h], want_h, rtol=1e-13, atol=1e-15)


def test_scalar_iir_matches_lfilter():
    """P-3: H=P=N=G=1, constant dt: a first-order IIR filter (scipy.signal.lfilter)
    plus the decaying initial state."""
    rng = np.random.default_rng(3)
    L = 300
    x = rng.standard_normal(L)
    dt, A, D, h0 = 0.37, -1.9, 0.8, 1.3
    p = _scalar(x, A, D=D, h0=h0, dt_raw=dt)
    y, _ = _scan(p, dt_softplus=False)
    r = math.exp(dt * A)
    want = scipy.signal.lfilter([dt], [1.0, -r], x) + D * x + h0 * r ** (np.arange(L) + 1)
    np.testing.assert_allclose(y.reshape(-1), want, rtol=1e-12, atol=1e-13)


def test_softplus_and_clamp_against_numpy():
    """dt = clamp(softplus(raw + bias)): L = 1, B = C = 1, x = 1, A = 0 gives y = dt."""
    raw = np.array([-40.0, -3.0, -0.5, 0.0, 0.5, 3.0, 40.0, 700.0])
    L = len(raw)
    for lo, hi in [(0.0, math.inf), (0.05, 2.5)]:
        for t in range(L):
            p = _scalar([1.0], 0.0, dt_raw=raw[t])
            y, _ = _scan(p, dt_min=lo, dt_max=hi)
            want = min(max(float(np.logaddexp(0.0, raw[t])), lo), hi)
            np.testing.assert_allclose(y.reshape(-1)[0], want, rtol=1e-15)
    assert abs(_scan(_scalar([1.0], 0.0, dt_raw=0.0))[0].item() - math.log(2.0)) < 1e-16


# ------------------------------------------------- independent formulations


@pytest.mark.parametrize("shape", [(1, 17, 2, 3, 5, 1), (2, 40, 4, 4, 6, 2), (1, 64, 6, 2, 3, 3)])
@pytest.mark.parametrize("init", [False, True])
@pytest.mark.parametrize("packed", [False, True])
def test_dual_matches_sequential(shape, init, packed):
    """P-4: brute-force matrix form with explicit decay products equals the
    sequential recurrence to 1e-12 (relative)."""
    b, L, H, P, N, G = shape
    rng = np.random.default_rng(hash((shape, init, packed)) % 2**32)
    seq = _packed_seq(rng, b, L, 3) if packed else None
    p = _problem(5, b, L, H, P, N, G, init=init, seq=seq)
    y1, h1 = _scan(p)
    y2, h2 = quadratic_scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], dt_bias=p["dt_bias"],
                            D=p["D"], h_init=p["h_init"], seq_idx=seq)
    assert oracle.rel_l2(y1, y2) < 1e-12
    assert oracle.rel_l2(h1, h2) < 1e-12


def test_dual_matches_sequential_with_clamp_no_softplus():
    p = _problem(8, 1, 30, 3, 4, 4, 1, init=True)
    kw = dict(dt_softplus=False, dt_min=0.01, dt_max=0.2)
    y1, h1 = _scan(p, **kw)
    y2, h2 = quadratic_scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], dt_bias=p["dt_bias"],
                            D=p["D"], h_init=p["h_init"], **kw)
    assert oracle.rel_l2(y1, y2) < 1e-12 and oracle.rel_l2(h1, h2) < 1e-12


@pytest.mark.parametrize("Q", [1, 2, 3, 7, 16, 64, 128, 256, 300, 305])
def test_chunked_matches_sequential_any_chunk(Q):
    """P-5: results are independent of the chunk size (ragged L = 300)."""
    rng = np.random.default_rng(Q)
    seq = _packed_seq(rng, 2, 300, 4)
    p = _problem(9, 2, 300, 4, 8, 6, 2, init=True, seq=seq)
    y1, h1 = _scan(p)
    y2, h2 = chunked_scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], chunk=Q,
                          dt_bias=p["dt_bias"], D=p["D"], h_init=p["h_init"], seq_idx=seq)
    assert oracle.rel_l2(y1, y2) < 1e-12
    assert oracle.rel_l2(h1, h2) < 1e-12


def test_chunked_strong_decay_no_overflow():
    """A = -16 with large dt: chunk-local cumsums reach far below -700; the
    chunk form must evaluate exp of differences only (no inf/nan)."""
    p = _problem(4, 1, 512, 2, 4, 4, 1)
    p["A"] = np.array([-16.0, -16.0], dtype=np.float32)
    p["dt_bias"] = np.array([3.0, 3.0], dtype=np.float32)
    y1, h1 = _scan(p)
    y2, h2 = chunked_scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], chunk=256,
                          dt_bias=p["dt_bias"], D=p["D"])
    assert np.isfinite(y2).all() and np.isfinite(h2).all()
    assert oracle.rel_l2(y1, y2) < 1e-12


# ---------------------------------------------------------------- invariants


def test_split_invariance_prefix_then_steps():
    """P-6: a prefix scan followed by single-token steps equals the full scan,
    bitwise (RL-Kernel RFC section 4.1: the same token's output whether
    produced by a full-sequence pass, a prefill or a decode step)."""
    p = _problem(12, 3, 50, 4, 4, 8, 2, init=True)
    yfull, hfull = _scan(p)
    k = 37
    pre = {key: (v[:, :k] if key in ("x", "dt_raw", "B", "C") else v) for key, v in p.items()}
    ypre, state = _scan(pre)
    assert np.array_equal(ypre, yfull[:, :k])
    for t in range(k, 50):
        state, yt = oracle.step(state, p["x"][:, t], p["dt_raw"][:, t], p["A"], p["B"][:, t],
                                p["C"][:, t], dt_bias=p["dt_bias"], D=p["D"])
        assert np.array_equal(yt, yfull[:, t])
    assert np.array_equal(state, hfull)


def test_packing_equals_concatenation():
    """P-7: a packed row with seq_idx equals the per-sequence runs, bitwise;
    the initial state belongs to the first sequence only."""
    rng = np.random.default_rng(2)
    L = 90
    seq = _packed_seq(rng, 1, L, 4)
    p = _problem(13, 1, L, 4, 3, 5, 2, init=True, seq=seq)
    y, hf = _scan(p)
    starts = np.flatnonzero(np.diff(seq[0], prepend=seq[0, 0] - 1))
    bounds = list(starts) + [L]
    for i in range(len(starts)):
        a, e = bounds[i], bounds[i + 1]
        sub = {key: (v[:, a:e] if key in ("x", "dt_raw", "B", "C") else v)
               for key, v in p.items() if key != "seq_idx"}
        sub["seq_idx"] = None
        if i > 0:
            sub["h_init"] = None
        ys, hs = _scan(sub)
        assert np.array_equal(ys, y[:, a:e])
        if i == len(starts) - 1:
            assert np.array_equal(hs, hf)


def test_linearity_in_x_and_h_init():
    """P-8: y is linear in (x, h_init) jointly (D included)."""
    p = _problem(14, 1, 60, 3, 4, 4, 3, init=True)
    q = _problem(15, 1, 60, 3, 4, 4, 3, init=True)
    q.update({k: p[k] for k in ("dt_raw", "A", "B", "C", "D", "dt_bias")})
    a, bcoef = 0.7, -1.3
    r = dict(p)
    r["x"] = a * p["x"].astype(np.float64) + bcoef * q["x"].astype(np.float64)
    r["h_init"] = a * p["h_init"].astype(np.float64) + bcoef * q["h_init"].astype(np.float64)
    yp, hp = _scan(p)
    yq, hq = _scan(q)
    yr, hr = _scan(r)
    assert oracle.rel_l2(yr, a * yp + bcoef * yq) < 1e-12
    assert oracle.rel_l2(hr, a * hp + bcoef * hq) < 1e-12


def test_group_equivalence():
    """P-9: G < H equals G = H with each head given its group's B/C
    (contiguous head -> group map, h // (H/G))."""
    p = _problem(16, 2, 40, 6, 3, 4, 2, init=True)
    y1, h1 = _scan(p)
    rep = dict(p)
    gmap = np.arange(6) // 3
    rep["B"] = p["B"][:, :, gmap, :]
    rep["C"] = p["C"][:, :, gmap, :]
    y2, h2 = _scan(rep)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)
    # a wrong (interleaved) map gives a different answer, so the test can fail
    bad = dict(p)
    bad["B"] = p["B"][:, :, np.arange(6) % 2, :]
    bad["C"] = p["C"][:, :, np.arange(6) % 2, :]
    assert oracle.rel_l2(_scan(bad)[0], y1) > 1e-3


def test_batch_equivalence():
    """P-10: each batch row equals a batch-of-one run of that row."""
    p = _problem(17, 3, 33, 2, 4, 4, 1, init=True)
    y, hf = _scan(p)
    for r in range(3):
        sub = {k: (v[r:r + 1] if k in ("x", "dt_raw", "B", "C", "h_init") else v)
               for k, v in p.items()}
        ys, hs = _scan(sub)
        assert np.array_equal(ys, y[r:r + 1]) and np.array_equal(hs, hf[r:r + 1])


def test_contraction_bound():
    """P-11: e^{a} in (0, 1], so ||h_t|| <= ||h_{t-1}|| + dt_t ||x_t|| ||B_t||."""
    p = _problem(18, 1, 200, 2, 4, 8, 1, init=True)
    state = p["h_init"].astype(np.float64)
    dt = np.logaddexp(0.0, p["dt_raw"].astype(np.float64) + p["dt_bias"])
    for t in range(200):
        prev = np.linalg.norm(state, axis=(2, 3))
        state, _ = oracle.step(state, p["x"][:, t], p["dt_raw"][:, t], p["A"], p["B"][:, t],
                               p["C"][:, t], dt_bias=p["dt_bias"], D=p["D"])
        now = np.linalg.norm(state, axis=(2, 3))
        bound = prev + dt[:, t] * np.linalg.norm(p["x"][:, t].astype(np.float64), axis=-1) * \
            np.linalg.norm(p["B"][:, t, 0].astype(np.float64), axis=-1)[:, None]
        assert (now <= bound * (1 + 1e-12)).all() and np.isfinite(now).all()


# ------------------------------------------------------ planted mistakes


MUTATIONS = {
    "dropped_D": ("yt[p] = acc + Dh * xt[p];", "yt[p] = acc;"),
    "pre_update_output": ("row[n] = decay * row[n] + dt * xt[p] * bt[n];\n            acc += row[n] * ct[n];",
                          "acc += row[n] * ct[n];\n            row[n] = decay * row[n] + dt * xt[p] * bt[n];"),
    "decay_sign": ("double decay = exp(dt * A);", "double decay = exp(-dt * A);"),
    "no_dt_on_input": ("+ dt * xt[p] * bt[n]", "+ xt[p] * bt[n]"),
    "interleaved_groups": ("const int64_t g = h / heads_per_group;\n        double* s",
                           "const int64_t g = h % G;\n        double* s"),
    "no_reset": ("memset(s, 0, sizeof(double) * (size_t)(P * N));\n            const double dt",
                 "(void)0;\n            const double dt"),
    "dropped_bias": ("const double bias = dt_bias ? dt_bias[h] : 0.0;", "const double bias = 0.0;"),
    "C_for_B": ("+ dt * xt[p] * bt[n]", "+ dt * xt[p] * ct[n]"),
    "no_softplus": ("if (softplus) v = oracle_softplus(v);", "(void)softplus;"),
    "init_ignored": ("memcpy(s, h_init + (b * H + h) * P * N", "memset(s, 0, 0 * sizeof(int)); if(0) memcpy(s, h_init + (b * H + h) * P * N"),
}


def _pin_suite(lib):
    """The pins above, rerun against a given oracle build; returns the names of
    the pins that fail."""
    failed = []
    # closed form: geometric halving with D and h0
    try:
        y, _ = oracle.scan(**{k: v for k, v in _scalar(np.ones(12), -math.log(2.0), D=0.5,
                                                        h0=4.0).items() if k != "seq_idx"},
                           dt_softplus=False, lib=lib)
        np.testing.assert_allclose(y.reshape(-1), 2.5 + 2.0 ** -np.arange(12), rtol=1e-14)
    except AssertionError:
        failed.append("geometric")
    # brute force, with groups, packing, init, bias, softplus
    rng = np.random.default_rng(99)
    seq = _packed_seq(rng, 1, 40, 3)
    p = _problem(21, 1, 40, 4, 3, 5, 2, init=True, seq=seq)
    y1, h1 = oracle.scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], dt_bias=p["dt_bias"],
                         D=p["D"], h_init=p["h_init"], seq_idx=seq, lib=lib)
    y2, h2 = quadratic_scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], dt_bias=p["dt_bias"],
                            D=p["D"], h_init=p["h_init"], seq_idx=seq)
    if not (oracle.rel_l2(y1, y2) < 1e-12 and oracle.rel_l2(h1, h2) < 1e-12):
        failed.append("dual")
    return failed


def test_pins_catch_planted_mistakes(tmp_path):
    """Each plausible mistake planted in a copy of the oracle source (on the
    CPU) makes at least one pin fail; the unmodified source passes them all."""
    src = oracle.source_text()
    assert _pin_suite(oracle._load()) == []
    for name, (old, new) in MUTATIONS.items():
        assert old in src, name
        # planted in the forward recurrence (the first occurrence in the source)
        path = oracle.compile_variant(src.replace(old, new, 1), str(tmp_path / ("m_%s.so" % name)))
        lib = oracle._load(path)
        assert _pin_suite(lib), "mutation %s went undetected" % name
