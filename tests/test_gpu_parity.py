"""GPU parity of the HIP path against the fp64 oracle at sizes the oracle
finishes in seconds (several chunks, ragged tails, packed sequences, segment
chaining), plus the decode update, determinism and sequence-boundary exactness.

Tolerance (relative L2 over all elements): 1e-4 for fp32 inputs, 2e-2 for bf16
inputs with fp32 state.  Because D*x dominates y for these input distributions,
every case is also checked with D = 0, where y is the state-space part alone.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import head_subset, host, log, run_oracle, run_scan, tol, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_ssd_selective_amd as ssd
    ssd.library()


def _packed(rng, b, L, nseq):
    rows = []
    for _ in range(b):
        cuts = np.sort(rng.choice(np.arange(1, L), size=nseq - 1, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [L]]))
        rows.append(np.repeat(np.arange(nseq, dtype=np.int32), lens))
    return np.stack(rows)


def _check_case(p, io, Q, label):
    t = to_dev(p, io)
    for zero_D in (False, True):
        y, fs = run_scan(t, Q, zero_D=zero_D)
        yr, hr = run_oracle(p, zero_D=zero_D)
        ey, eh = oracle.rel_l2(host(y), yr), oracle.rel_l2(host(fs), hr)
        log("%s D=%s: rel_l2 y=%.3e final=%.3e" % (label, "0" if zero_D else "D", ey, eh))
        assert ey < tol(io) and eh < tol(io), (label, zero_D, ey, eh)
        assert np.isfinite(host(y)).all()


def test_config0_tiny_fp32():
    w = workloads.WORKLOADS[0]
    p = workloads.make_inputs(w)
    _check_case(p, "f32", w.chunk, "config0")


FP32_CASES = [
    # b, L, H, P, N, G, Q, init, packed
    (2, 300, 8, 64, 128, 2, 64, True, False),
    (1, 1000, 4, 64, 128, 1, 128, True, True),
    (3, 77, 4, 16, 16, 2, 32, False, True),
    (1, 1, 4, 16, 16, 1, 64, True, False),
    (1, 64, 4, 16, 16, 1, 64, True, False),
    (1, 65, 4, 16, 16, 1, 64, False, False),
    (2, 500, 4, 16, 16, 4, 128, True, True),
    # chunk 256 run as two 128-token blocks by the chunk-128 kernels
    (1, 700, 4, 64, 128, 2, 256, True, True),
    # state size 64, head dim 128, state size 256
    (2, 300, 4, 64, 64, 2, 64, True, True),
    (1, 400, 4, 64, 64, 1, 128, True, False),
    (1, 300, 4, 128, 128, 2, 64, True, True),
    (2, 200, 4, 64, 256, 2, 64, False, True),
]


@pytest.mark.parametrize("case", FP32_CASES, ids=lambda c: "b%dL%dH%dP%dN%dG%dQ%d_i%d_p%d" % c)
def test_fp32_parity(case):
    b, L, H, P, N, G, Q, init, packed = case
    rng = np.random.default_rng(hash(case) % 2**32)
    p = workloads.random_problem(rng, b, L, H, P, N, G, io="f32", init=init)
    if packed:
        p["seq_idx"] = _packed(rng, b, L, 3)
    _check_case(p, "f32", Q, "fp32 %s" % (case,))


BF16_CASES = [
    (1, 4096, 64, 64, 128, 8, 128, True, False),  # 4 segments of 8 chunks
    (2, 777, 16, 64, 128, 4, 256, True, True),
    (4, 333, 8, 64, 128, 2, 64, False, True),
    (1, 2000, 8, 64, 64, 2, 128, True, False),
    (2, 150, 4, 16, 16, 1, 64, True, True),
    (1, 129, 64, 64, 128, 8, 128, False, False),
    # the JAX page's Configuration defaults (d_state 64, head dim 64, chunk 64)
    (2, 333, 8, 64, 64, 2, 64, True, True),
    (1, 1000, 64, 64, 64, 8, 64, True, False),
    # chunk 256 at N = 64, run as two 128-token blocks
    (1, 900, 8, 64, 64, 2, 256, True, True),
    # the generic kernel's other shapes: state size 256, head dims 128 and 32,
    # chunk 32, state size 32
    (1, 300, 4, 64, 256, 1, 64, True, True),
    (2, 333, 4, 64, 256, 2, 128, True, False),
    (1, 400, 4, 128, 128, 2, 128, True, True),
    (2, 300, 4, 32, 128, 2, 128, False, True),
    (2, 200, 4, 64, 128, 2, 32, True, True),
    (2, 150, 4, 64, 32, 1, 64, True, False),
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "b%dL%dH%dP%dN%dG%dQ%d_i%d_p%d" % c)
def test_bf16_parity(case):
    b, L, H, P, N, G, Q, init, packed = case
    rng = np.random.default_rng(hash(case) % 2**32)
    p = workloads.random_problem(rng, b, L, H, P, N, G, io="bf16", init=init)
    if packed:
        p["seq_idx"] = _packed(rng, b, L, 4)
    _check_case(p, "bf16", Q, "bf16 %s" % (case,))


@pytest.mark.parametrize("packed", [False, True])
def test_mixed_sign_decay_exponent(packed):
    """dt without softplus and of mixed sign: some dt * A > 0, so the output
    kernel cannot factor its intra-chunk decays and every step takes the exact
    per-element form."""
    b, L, H, P, N, G, Q = 1, 600, 8, 64, 128, 2, 128
    rng = np.random.default_rng(4242 + packed)
    p = workloads.random_problem(rng, b, L, H, P, N, G, io="bf16", init=True)
    p["dt_raw"] = (0.05 + 0.04 * rng.standard_normal((b, L, H))).astype(np.float32)
    p["dt_bias"] = np.zeros(H, dtype=np.float32)
    assert (p["dt_raw"] < 0).any()
    if packed:
        p["seq_idx"] = _packed(rng, b, L, 4)
    t = to_dev(p, "bf16")
    for zero_D in (False, True):
        y, fs = run_scan(t, Q, zero_D=zero_D, dt_softplus=False)
        yr, hr = run_oracle(p, zero_D=zero_D, dt_softplus=False)
        ey, eh = oracle.rel_l2(host(y), yr), oracle.rel_l2(host(fs), hr)
        log("mixed-sign dt packed=%s D=%s: rel_l2 y=%.3e final=%.3e"
            % (packed, "0" if zero_D else "D", ey, eh))
        assert ey < tol("bf16") and eh < tol("bf16"), (packed, zero_D, ey, eh)


@pytest.mark.parametrize("Q", [64, 128, 256])
def test_chunk_size_sweep_config1_shapes(Q):
    """Results are independent of the chunk size (within tolerance) at the
    30B layer shape (H=64, P=64, N=128, G=8)."""
    w = workloads.WORKLOADS[1]
    p = workloads.make_inputs(w, seqlen=2048)
    t = to_dev(p, "bf16")
    sub_heads = [0, 9, 36, 63]
    for zero_D in (False, True):
        y, fs = run_scan(t, Q, zero_D=zero_D)
        sub = head_subset(p, sub_heads)
        yr, hr = run_oracle(sub, zero_D=zero_D)
        ey = oracle.rel_l2(host(y)[:, :, sub_heads], yr)
        eh = oracle.rel_l2(host(fs)[:, sub_heads], hr)
        log("chunk sweep Q=%d D=%s: y=%.3e final=%.3e" % (Q, not zero_D, ey, eh))
        assert ey < 2e-2 and eh < 2e-2


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("PN", [(16, 16), (64, 128), (64, 256), (32, 64), (24, 32), (80, 16)])
@pytest.mark.parametrize("bH", [(5, 8), (16, 64)], ids=["few_heads", "many_heads"])
def test_decode_step_parity(io, PN, bH):
    """One decode token three times; both grid layouts of the update (few rows x
    heads split each head's rows over blocks, many loop over them)."""
    import torch
    import mamba_ssd_selective_amd as ssd
    P, N = PN
    (b, H), G = bH, 2
    rng = np.random.default_rng(P * 1000 + N)
    p = workloads.random_problem(rng, b, 3, H, P, N, G, io=io, init=True)
    t = to_dev(p, io)
    state = t["h_init"].clone()
    st_ref = p["h_init"].astype(np.float64)
    for k in range(3):
        y = ssd.state_update(state, t["x"][:, k].contiguous(), t["dt_raw"][:, k].contiguous(),
                             t["A"], t["B"][:, k].contiguous(), t["C"][:, k].contiguous(),
                             D=t["D"], dt_bias=t["dt_bias"])
        torch.cuda.synchronize()
        st_ref, yr = oracle.step(st_ref, p["x"][:, k], p["dt_raw"][:, k], p["A"], p["B"][:, k],
                                 p["C"][:, k], dt_bias=p["dt_bias"], D=p["D"])
        ey = oracle.rel_l2(host(y), yr)
        es = oracle.rel_l2(host(state), st_ref)
        log("decode %s P=%d N=%d step %d: y=%.3e state=%.3e" % (io, P, N, k, ey, es))
        assert es < 1e-5
        assert ey < (1e-5 if io == "f32" else 2e-2)


def test_determinism_bitwise():
    """Fixed reduction order, no atomics: two runs are bitwise equal."""
    w = workloads.WORKLOADS[2]
    p = workloads.make_inputs(w, seqlen=4096)
    p["seq_idx"] = np.repeat(np.arange(5, dtype=np.int32), [700, 900, 33, 2000, 463])[None]
    t = to_dev(p, "bf16")
    y1, f1 = run_scan(t, 128)
    y2, f2 = run_scan(t, 128)
    import torch
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_other_sequence_perturbation_is_bitwise_invisible():
    """Changing one packed sequence's (finite) inputs leaves every other
    sequence's outputs bitwise unchanged (masks are selects)."""
    rng = np.random.default_rng(77)
    b, L, H, P, N, G = 1, 1500, 8, 64, 128, 2
    p = workloads.random_problem(rng, b, L, H, P, N, G, io="bf16", init=True)
    lens = [300, 77, 500, 623]
    p["seq_idx"] = np.repeat(np.arange(4, dtype=np.int32), lens)[None]
    starts = np.cumsum([0] + lens)
    t = to_dev(p, "bf16")
    y0, f0 = run_scan(t, 128)
    k = 1  # perturb sequence 1 (tokens 300..376, mid-chunk on both sides)
    q = {kk: (v.copy() if isinstance(v, np.ndarray) else v) for kk, v in p.items()}
    a, e = starts[k], starts[k + 1]
    q["x"][:, a:e] = workloads.round_bf16(rng.standard_normal(q["x"][:, a:e].shape).astype(np.float32) * 3)
    q["B"][:, a:e] = workloads.round_bf16(rng.standard_normal(q["B"][:, a:e].shape).astype(np.float32))
    q["C"][:, a:e] = workloads.round_bf16(rng.standard_normal(q["C"][:, a:e].shape).astype(np.float32))
    q["dt_raw"][:, a:e] = rng.standard_normal(q["dt_raw"][:, a:e].shape).astype(np.float32) + 2
    y1, f1 = run_scan(to_dev(q, "bf16"), 128)
    Y0, Y1 = host(y0), host(y1)
    assert not np.array_equal(Y0[:, a:e], Y1[:, a:e])
    mask = np.ones(L, dtype=bool)
    mask[a:e] = False
    assert np.array_equal(Y0[:, mask], Y1[:, mask])
    assert np.array_equal(host(f0), host(f1))


def test_chunk_aligned_sequence_matches_standalone_run_bitwise():
    """A sequence that starts on a chunk boundary of a packed row gives bitwise
    the same outputs and final state as a run of that sequence alone (same
    chunk grid, one segment per row), and the carry at the reset is exactly 0."""
    import mamba_ssd_selective_amd as ssd
    rng = np.random.default_rng(5)
    b, H, P, N, G, Q = 8, 64, 64, 128, 8, 128
    La, Lb = 256, 300
    p = workloads.random_problem(rng, b, La + Lb, H, P, N, G, io="bf16", init=True)
    p["seq_idx"] = np.repeat(np.array([4, 9], dtype=np.int32), [La, Lb])[None].repeat(b, 0)
    assert ssd.segments(b, La + Lb, H, P, N, G, Q) == 1
    assert ssd.segments(b, Lb, H, P, N, G, Q) == 1
    y, f = run_scan(to_dev(p, "bf16"), Q)
    alone = {k: (v[:, La:] if k in ("x", "dt_raw", "B", "C") else v) for k, v in p.items()}
    alone["seq_idx"] = None
    alone["h_init"] = None
    ya, fa = run_scan(to_dev(alone, "bf16"), Q)
    assert np.array_equal(host(y)[:, La:], host(ya))
    assert np.array_equal(host(f), host(fa))


def test_empty_and_tiny_lengths():
    import torch
    import mamba_ssd_selective_amd as ssd
    dev = torch.device("cuda:0")
    b, H, P, N, G = 2, 4, 16, 16, 1
    h0 = torch.randn(b, H, P, N, device=dev)
    z = lambda *s, dt=torch.float32: torch.zeros(*s, device=dev, dtype=dt)
    A = -torch.ones(H, device=dev)
    y, fs = ssd.chunk_scan_fwd(z(b, 0, H, P), z(b, 0, H), A, z(b, 0, G, N), z(b, 0, G, N),
                               chunk_size=64, initial_states=h0, return_final_states=True)
    torch.cuda.synchronize()
    assert y.shape == (b, 0, H, P) and torch.equal(fs, h0)
    y, fs = ssd.chunk_scan_fwd(z(b, 0, H, P), z(b, 0, H), A, z(b, 0, G, N), z(b, 0, G, N),
                               chunk_size=64, return_final_states=True)
    torch.cuda.synchronize()
    assert torch.equal(fs, torch.zeros_like(fs))
    y = ssd.chunk_scan_fwd(z(0, 10, H, P), z(0, 10, H), A, z(0, 10, G, N), z(0, 10, G, N),
                           chunk_size=64)
    assert y.shape == (0, 10, H, P)


def test_final_state_may_alias_initial_state():
    import torch
    rng = np.random.default_rng(9)
    p = workloads.random_problem(rng, 2, 700, 8, 64, 128, 2, io="bf16", init=True)
    t = to_dev(p, "bf16")
    y1, f1 = run_scan(t, 128)
    st = t["h_init"].clone()
    t2 = dict(t)
    t2["h_init"] = st
    y2, f2 = run_scan(t2, 128, final_states_out=st)
    assert f2.data_ptr() == st.data_ptr()
    assert torch.equal(y1, y2) and torch.equal(f1, st)


def test_rejects_unsupported_geometry_on_device():
    import torch
    import mamba_ssd_selective_amd as ssd
    dev = torch.device("cuda:0")
    x = torch.zeros(1, 64, 4, 48, device=dev)
    with pytest.raises(ssd.SSDError) as e:
        ssd.chunk_scan_fwd(x, torch.zeros(1, 64, 4, device=dev), -torch.ones(4, device=dev),
                           torch.zeros(1, 64, 1, 16, device=dev), torch.zeros(1, 64, 1, 16, device=dev),
                           chunk_size=64)
    assert e.value.status == 4


def test_graph_replay_matches_eager_bitwise():
    """The prefill scan and a decode step captured into a HIP graph give, on
    every replay, bitwise the outputs of the same calls launched eagerly (the
    library records no memset nodes; eager work and synchronisations run
    between the replays)."""
    import torch
    import mamba_ssd_selective_amd as ssd
    rng = np.random.default_rng(31)
    b, L, H, P, N, G, Q = 1, 2000, 16, 64, 128, 2, 128
    p = workloads.random_problem(rng, b, L + 1, H, P, N, G, io="bf16", init=True)
    p["seq_idx"] = _packed(rng, b, L + 1, 3)
    t = to_dev(p, "bf16")
    x, dt, B, C = (t[k][:, :L].contiguous() for k in ("x", "dt_raw", "B", "C"))
    xd, dtd, Bd, Cd = (t[k][:, L].contiguous() for k in ("x", "dt_raw", "B", "C"))
    seq = t["seq_idx"][:, :L].contiguous()
    ws = torch.empty(max(1, ssd.workspace_bytes(b, L, H, P, N, G, Q)), dtype=torch.uint8,
                     device=x.device)
    y = torch.empty_like(x)
    fs = torch.empty(b, H, P, N, device=x.device)
    yd = torch.empty_like(xd)

    def step():
        ssd.chunk_scan_fwd(x, dt, t["A"], B, C, chunk_size=Q, D=t["D"], dt_bias=t["dt_bias"],
                           initial_states=t["h_init"], seq_idx=seq, return_final_states=True,
                           out=y, final_states_out=fs, workspace=ws)
        ssd.state_update(fs, xd, dtd, t["A"], Bd, Cd, D=t["D"], dt_bias=t["dt_bias"], out=yd)

    step()
    torch.cuda.synchronize()
    ref = (y.clone(), fs.clone(), yd.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for o in (y, fs, yd):
            o.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log("graph replay %d" % r)
        assert torch.equal(y, ref[0]) and torch.equal(fs, ref[1]) and torch.equal(yd, ref[2]), r


def _report_diff(Y0, Y1, mask):
    """Log the tokens (outside the poisoned sequence) whose outputs differ."""
    d = (Y0 != Y1) & mask[None, :, None, None]
    if d.any():
        toks = np.unique(np.nonzero(d)[1])
        heads = np.unique(np.nonzero(d)[2])
        log("differing tokens %s (%d), heads %s, non-finite %d"
            % (toks[:40].tolist(), len(toks), heads.tolist(), int((~np.isfinite(Y1) & d).sum())))


def _poison(q, a, e, kind, rng):
    """Non-finite values in tokens [a, e) of one packed sequence: at its first
    and last token and at a few tokens between (so that chunks it shares with
    its neighbours are hit)."""
    toks = sorted({a, e - 1, (a + e) // 2} | set(rng.integers(a, e, size=3).tolist()))
    bad = {"nan": np.float32("nan"), "inf": np.float32("inf"), "-inf": np.float32("-inf")}[kind]
    for t in toks:
        q["x"][:, t, :, ::7] = bad
        q["B"][:, t, :, 3] = bad
        q["C"][:, t, :, 5] = -bad
        q["dt_raw"][:, t, 1] = bad
    return toks


@pytest.mark.parametrize("kind", ["nan", "inf", "-inf"])
@pytest.mark.parametrize("victim", [1, 3])
def test_nonfinite_inputs_stay_inside_their_sequence(kind, victim):
    """NaN or +-Inf in one packed sequence's x, B, C and dt leave every other
    sequence's y bitwise unchanged, and the final state too unless the poisoned
    sequence is the row's last (masks are selects).  12
    segments of one chunk each, so the segment-state pass and the carry between
    segments are on the path."""
    rng = np.random.default_rng(99)
    b, L, H, P, N, G = 1, 1500, 8, 64, 128, 2
    p = workloads.random_problem(rng, b, L, H, P, N, G, io="bf16", init=True)
    lens = [300, 77, 500, 623]
    p["seq_idx"] = np.repeat(np.arange(4, dtype=np.int32), lens)[None]
    starts = np.cumsum([0] + lens)
    y0, f0 = run_scan(to_dev(p, "bf16"), 128)
    q = {kk: (v.copy() if isinstance(v, np.ndarray) else v) for kk, v in p.items()}
    a, e = starts[victim], starts[victim + 1]
    toks = _poison(q, a, e, kind, rng)
    log("nonfinite %s in sequence %d (tokens %s)" % (kind, victim, toks))
    y1, f1 = run_scan(to_dev(q, "bf16"), 128)
    Y0, Y1 = host(y0), host(y1)
    mask = np.ones(L, dtype=bool)
    mask[a:e] = False
    _report_diff(Y0, Y1, mask)
    assert np.array_equal(Y0[:, mask], Y1[:, mask])
    assert not np.isfinite(Y1[:, a:e]).all()
    if victim != 3:
        assert np.array_equal(host(f0), host(f1))


def test_nonfinite_inputs_stay_inside_their_sequence_packed_16k():
    """The same at the packed 16K workload's shape (64 heads, 16 sequences,
    most starting mid-chunk), for one sequence in the middle."""
    w = workloads.WORKLOADS[2]
    p = workloads.make_inputs(w)
    lens = p["lengths"]
    starts = np.concatenate([[0], np.cumsum(lens)])
    victim = 6
    a, e = int(starts[victim]), int(starts[victim + 1])
    y0, f0 = run_scan(to_dev(p, "bf16"), w.chunk)
    q = {kk: (v.copy() if isinstance(v, np.ndarray) else v) for kk, v in p.items()}
    toks = _poison(q, a, e, "nan", np.random.default_rng(3))
    log("nonfinite nan in packed_16k sequence %d [%d, %d) tokens %s" % (victim, a, e, toks))
    y1, f1 = run_scan(to_dev(q, "bf16"), w.chunk)
    Y0, Y1 = host(y0), host(y1)
    mask = np.ones(w.seqlen, dtype=bool)
    mask[a:e] = False
    assert np.array_equal(Y0[:, mask], Y1[:, mask])
    assert np.array_equal(host(f0), host(f1))


def test_seq_idx_order_check_on_the_device():
    """The opt-in check reads a device seq_idx and rejects a decreasing row;
    the scan entry point runs it first when asked."""
    import torch
    import mamba_ssd_selective_amd as ssd
    dev = torch.device("cuda:0")
    good = torch.tensor([[0, 0, 1, 2, 2, 7]] * 2, dtype=torch.int32, device=dev)
    bad = good.clone()
    bad[1, 4] = 1
    ssd.check_seq_idx(good)
    with pytest.raises(ssd.SSDError) as e:
        ssd.check_seq_idx(bad)
    assert e.value.status == 10
    b, L, H, P, N, G = 2, 6, 4, 16, 16, 1
    z = lambda *s, dt=torch.float32: torch.zeros(*s, device=dev, dtype=dt)
    with pytest.raises(ssd.SSDError):
        ssd.chunk_scan_fwd(z(b, L, H, P), z(b, L, H), -torch.ones(H, device=dev), z(b, L, G, N),
                           z(b, L, G, N), chunk_size=64, seq_idx=bad, check_seq_idx_order=True)
