"""Chunk-emulating decode (ssd_decode_emulated through the C-ABI): decode
tokens give bitwise the strict chunked prefill's outputs and chunk-start
states, so the split of a sequence into prefill and decode steps changes no bit
(RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 1, operator family 1, and
section 3, Figure 2, box [F2]).  The strict prefill runs each row as one
segment and forms every intra-chunk decay per element; the oracle checks the
values."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import tol

pytestmark = pytest.mark.gpu

H, P, N, G, Q = 64, 64, 128, 8, 128
# the shape of the tests below unless one says otherwise
SH = dict(H=H, P=P, N=N, G=G, Q=Q, io="bf16")


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.device("cuda:0"))
    return (t.to(dtype) if dtype is not None else t).contiguous()


def _host(t):
    return t.float().cpu().numpy()


def _io(sh):
    import torch
    return torch.bfloat16 if sh["io"] == "bf16" else torch.float32


class _Slots:
    def __init__(self, rows, sh=SH):
        import torch
        dev, io = torch.device("cuda:0"), _io(sh)
        h, p, n, g, q = sh["H"], sh["P"], sh["N"], sh["G"], sh["Q"]
        self.state = torch.zeros((rows, h, p, n), dtype=torch.float32, device=dev)
        self.chunks = (torch.zeros((rows, q, h, p), dtype=io, device=dev),
                       torch.zeros((rows, q, h), dtype=torch.float32, device=dev),
                       torch.zeros((rows, q, g, n), dtype=io, device=dev),
                       torch.zeros((rows, q, g, n), dtype=io, device=dev))


def _full_prefill(p, L, sh=SH):
    """The strict prefill of every row's first L tokens: (y, final states)."""
    b = p["x"].shape[0]
    s = _Slots(b, sh)
    y = _cached(p, list(range(b)), L, s, list(range(b)), True, sh=sh)
    return y, _host(s.state)


def _step(p, slots, toks, idx, pos, sh=SH):
    """One emulated decode step; toks[r] = the token index of row r (ignored
    for padding rows)."""
    import torch
    import mamba_ssd_selective_amd as ssd
    io = _io(sh)
    pick = lambda a: np.stack([a[r, max(t, 0)] for r, t in enumerate(toks)])
    y = torch.full((len(toks), sh["H"], sh["P"]), 7.0, dtype=io, device=torch.device("cuda:0"))
    ssd.decode_emulated(_dev(pick(p["x"]), io), _dev(pick(p["dt_raw"])), _dev(p["A"]),
                        _dev(pick(p["B"]), io), _dev(pick(p["C"]), io), slots.state, slots.chunks,
                        _dev(np.asarray(idx, dtype=np.int32)), _dev(np.asarray(pos, dtype=np.int32)),
                        chunk_size=sh["Q"], D=_dev(p["D"]), dt_bias=_dev(p["dt_bias"]), out=y)
    return y


def test_emulated_decode_bitwise_equals_prefill():
    """Four rows: 256 prompt tokens prefilled into slots, then 150 decode
    tokens (across a chunk boundary).  Every decode output equals the
    406-token prefill's bit for bit, and after the boundary each slot holds the
    384-token prefill's final state bit for bit."""
    import torch
    import mamba_ssd_selective_amd as ssd
    b, T, L0 = 4, 2 * Q + 150, 2 * Q
    rng = np.random.default_rng(5)
    p = workloads.random_problem(rng, b, T, H, P, N, G, io="bf16", init=False)
    y_full, _ = _full_prefill(p, T)
    _, fs3 = _full_prefill(p, 3 * Q)
    idx = [3, 0, 5, 1]
    slots = _Slots(6)
    bf = torch.bfloat16
    ssd.chunk_scan_fwd_cached(_dev(p["x"][:, :L0], bf), _dev(p["dt_raw"][:, :L0]), _dev(p["A"]),
                              _dev(p["B"][:, :L0], bf), _dev(p["C"][:, :L0], bf), slots.state,
                              _dev(np.asarray(idx, dtype=np.int32)), chunk_size=Q,
                              init_from_cache=False, strict=True, D=_dev(p["D"]),
                              dt_bias=_dev(p["dt_bias"]))
    ys = []
    for t in range(L0, T):
        ys.append(_host(_step(p, slots, [t] * b, idx, [t % Q] * b)))
    torch.cuda.synchronize()
    ys = np.stack(ys, axis=1)  # (b, T - L0, H, P)
    bad = [(r, t) for r in range(b) for t in range(T - L0) if not np.array_equal(ys[r, t], y_full[r, L0 + t])]
    assert not bad, "decode tokens differing from the prefill: %d, first %s" % (len(bad), bad[:3])
    st = _host(slots.state)
    for r in range(b):
        assert np.array_equal(st[idx[r]], fs3[r]), r
    # the values themselves: the oracle on row 2
    yr, _ = oracle.scan(p["x"][2:3], p["dt_raw"][2:3], p["A"], p["B"][2:3], p["C"][2:3],
                        dt_bias=p["dt_bias"], D=p["D"])
    assert oracle.rel_l2(ys[2], yr[0, L0:]) < 2e-2


def test_emulated_decode_staggered_rows_and_padding():
    """Prompts of 256, 128, 0 and 384 tokens; each row starts decoding at
    another step (a padding row before that, its y left alone), so the rows
    sit at different chunk offsets in one call.  Bitwise the prefill's
    outputs."""
    import torch
    import mamba_ssd_selective_amd as ssd
    b, T = 4, 3 * Q + 140
    rng = np.random.default_rng(9)
    p = workloads.random_problem(rng, b, T, H, P, N, G, io="bf16", init=False)
    y_full, _ = _full_prefill(p, T)
    lens = np.array([2 * Q, Q, 0, 3 * Q], dtype=np.int32)
    start = [0, 5, 37, 90]
    steps = 140
    idx = [4, 2, 0, 1]
    slots = _Slots(5)
    L = 3 * Q
    q = {k: p[k][:, :L].copy() for k in ("x", "dt_raw", "B", "C")}
    for k in q:
        for r in range(b):
            q[k][r, lens[r]:] = 0
    bf = torch.bfloat16
    ssd.chunk_scan_fwd_cached(_dev(q["x"], bf), _dev(q["dt_raw"]), _dev(p["A"]), _dev(q["B"], bf),
                              _dev(q["C"], bf), slots.state, _dev(np.asarray(idx, dtype=np.int32)),
                              chunk_size=Q, seq_lens=_dev(lens), init_from_cache=False,
                              strict=True, D=_dev(p["D"]), dt_bias=_dev(p["dt_bias"]))
    got = {r: [] for r in range(b)}
    for k in range(steps):
        toks, ii, pp = [], [], []
        for r in range(b):
            t = lens[r] + k - start[r]
            live = k >= start[r] and t < T
            toks.append(t if live else -1)
            ii.append(idx[r] if live else -1)
            pp.append(t % Q if live else 0)
        y = _host(_step(p, slots, toks, ii, pp))
        for r in range(b):
            if toks[r] >= 0:
                got[r].append((toks[r], y[r]))
            else:
                assert np.all(y[r] == 7.0)
    torch.cuda.synchronize()
    for r in range(b):
        assert got[r]
        for t, yv in got[r]:
            assert np.array_equal(yv, y_full[r, t]), (r, t)


def _cached(p, rows_sel, L, slots, idx, strict, lens=None, sh=SH):
    import torch
    import mamba_ssd_selective_amd as ssd
    io = _io(sh)
    sel = lambda k: p[k][rows_sel, :L]
    y = ssd.chunk_scan_fwd_cached(_dev(sel("x"), io), _dev(sel("dt_raw")), _dev(p["A"]),
                                  _dev(sel("B"), io), _dev(sel("C"), io), slots.state,
                                  _dev(np.asarray(idx, dtype=np.int32)), chunk_size=sh["Q"],
                                  seq_lens=None if lens is None else _dev(lens),
                                  init_from_cache=False, strict=strict, D=_dev(p["D"]),
                                  dt_bias=_dev(p["dt_bias"]))
    torch.cuda.synchronize()
    return _host(y)


def test_strict_prefill_is_batch_invariant_and_decode_continues_it():
    """Strict mode: a row alone and the same row inside a batch of three give
    the same bits (the row is one segment either way), and one row's strict
    prefill of 256 tokens continued by 40 emulated decode tokens equals its
    strict prefill of 296 tokens bit for bit."""
    import mamba_ssd_selective_amd as ssd
    rng = np.random.default_rng(13)
    T = 2 * Q + 40
    p = workloads.random_problem(rng, 3, T, H, P, N, G, io="bf16", init=False)
    assert ssd.segments(1, T, H, P, N, G, Q) > 1   # the default split of one row differs
    s1, s3 = _Slots(1), _Slots(3)
    y1 = _cached(p, [1], T, s1, [0], True)
    y3 = _cached(p, [0, 1, 2], T, s3, [2, 0, 1], True)
    assert np.array_equal(y1[0], y3[1])
    assert np.array_equal(_host(s1.state)[0], _host(s3.state)[0])
    # one row: prefill 256 tokens, then decode 40
    s = _Slots(1)
    _cached(p, [1], 2 * Q, s, [0], True)
    for t in range(2 * Q, T):
        yd = _host(_step({k: (p[k][1:2] if k in ("x", "dt_raw", "B", "C") else p[k]) for k in p},
                         s, [t], [0], [t % Q]))
        assert np.array_equal(yd[0], y1[0, t]), t


def test_strict_states_and_outputs_against_the_oracle():
    """The strict path's values against the fp64 oracle (its bitwise tests
    above compare GPU with GPU): the strict prefill's y with D and with D = 0
    (D x dominates y), its final states, and the chunk-start states the
    emulated decode commits to the slots as it crosses chunk boundaries."""
    import torch
    rng = np.random.default_rng(31)
    b, L0, T = 2, Q + 37, 3 * Q
    p = workloads.random_problem(rng, b, T, H, P, N, G, io="bf16", init=False)
    for zero_D in (False, True):
        q = dict(p, D=np.zeros_like(p["D"]) if zero_D else p["D"])
        s = _Slots(b)
        y = _cached(q, list(range(b)), L0, s, list(range(b)), True)
        yr, hr = oracle.scan(q["x"][:, :L0], q["dt_raw"][:, :L0], q["A"], q["B"][:, :L0],
                             q["C"][:, :L0], dt_bias=q["dt_bias"], D=q["D"])
        ey, eh = oracle.rel_l2(y, yr), oracle.rel_l2(_host(s.state), hr)
        print("strict prefill D=%s: y %.3e final %.3e" % ("0" if zero_D else "D", ey, eh), flush=True)
        assert ey < 2e-2 and eh < 2e-2
    # the emulated decode from a chunk-aligned prompt of Q tokens: after the
    # boundary at 2Q each slot holds the oracle's state after 2Q tokens, and
    # the decode outputs with D = 0 match the oracle's
    q = dict(p, D=np.zeros_like(p["D"]))
    s = _Slots(b)
    _cached(q, list(range(b)), Q, s, list(range(b)), True)
    ys = []
    for t in range(Q, T):
        ys.append(_host(_step(q, s, [t] * b, list(range(b)), [t % Q] * b)))
        if t == 2 * Q - 1:
            torch.cuda.synchronize()
            committed = _host(s.state)
    torch.cuda.synchronize()
    yr, _ = oracle.scan(q["x"], q["dt_raw"], q["A"], q["B"], q["C"], dt_bias=q["dt_bias"], D=q["D"])
    _, h2 = oracle.scan(q["x"][:, :2 * Q], q["dt_raw"][:, :2 * Q], q["A"], q["B"][:, :2 * Q],
                        q["C"][:, :2 * Q], dt_bias=q["dt_bias"], D=q["D"])
    ed = oracle.rel_l2(np.stack(ys, axis=1), yr[:, Q:])
    ec = oracle.rel_l2(committed, h2)
    print("emulated decode D=0: y %.3e, committed chunk-start state %.3e" % (ed, ec), flush=True)
    assert ed < 2e-2 and ec < 2e-2


@pytest.mark.parametrize("n,q,io", [(64, 64, "bf16"), (128, 64, "bf16"), (64, 128, "bf16"),
                                    (128, 256, "bf16"), (128, 128, "f32"), (256, 64, "bf16")])
def test_emulated_decode_other_shapes(n, q, io):
    """The decode forms of the other compiled shapes and of fp32: two rows,
    one after a Q-token prompt and one from an empty slot that starts seven
    steps later (a padding row until then), decoded across a chunk boundary
    each.  Bitwise the strict prefill's outputs and, at the boundary, its
    states; the values against the oracle."""
    import torch
    sh = dict(H=16, P=64, N=n, G=2, Q=q, io=io)
    rng = np.random.default_rng(41)
    T = 2 * q + 30
    p = workloads.random_problem(rng, 2, T, sh["H"], sh["P"], n, sh["G"], io=io, init=False)
    y_full, _ = _full_prefill(p, T, sh)
    _, fs2 = _full_prefill(p, 2 * q, sh)
    lens = np.array([q, 0], dtype=np.int32)
    start = [0, 7]
    idx = [1, 0]
    slots = _Slots(2, sh)
    _cached({k: (v[:, :q] if k in ("x", "dt_raw", "B", "C") else v) for k, v in p.items()},
            [0, 1], q, slots, idx, True, lens=lens, sh=sh)
    got = {0: [], 1: []}
    for k in range(q + 30):
        toks = [int(lens[r]) + k - start[r] if k >= start[r] else -1 for r in range(2)]
        toks = [t if t < T else -1 for t in toks]
        ii = [idx[r] if toks[r] >= 0 else -1 for r in range(2)]
        pp = [toks[r] % q if toks[r] >= 0 else 0 for r in range(2)]
        y = _host(_step(p, slots, toks, ii, pp, sh))
        for r in range(2):
            if toks[r] >= 0:
                got[r].append((toks[r], y[r]))
            else:
                assert np.all(y[r] == 7.0)
        if toks[0] == 2 * q - 1:
            torch.cuda.synchronize()
            assert np.array_equal(_host(slots.state)[idx[0]], fs2[0])
    torch.cuda.synchronize()
    for r in range(2):
        bad = [t for t, yv in got[r] if not np.array_equal(yv, y_full[r, t])]
        assert not bad, (r, bad[:5])
    yr, _ = oracle.scan(p["x"], p["dt_raw"], p["A"], p["B"], p["C"], dt_bias=p["dt_bias"], D=p["D"])
    err = oracle.rel_l2(np.stack([yv for _, yv in got[0]]), yr[0, [t for t, _ in got[0]]])
    assert err < tol(io), err


def test_emulated_decode_graph_replay_matches_eager_bitwise():
    """One emulated decode step captured into a HIP graph and replayed for 130
    tokens (across a chunk boundary, so the commit pass runs inside the
    graph), with the next token's inputs and offsets copied into the
    captured buffers between replays: every replay's y, and the slots at the
    end, equal those of the same steps launched eagerly on a copy of the
    slots, bit for bit."""
    import torch
    import mamba_ssd_selective_amd as ssd
    rng = np.random.default_rng(23)
    b, T = 3, 2 * Q + 2
    p = workloads.random_problem(rng, b, T, H, P, N, G, io="bf16", init=False)
    bf = torch.bfloat16
    idx = [2, 0, 1]
    ga, eg = _Slots(3), _Slots(3)
    for s in (ga, eg):
        _cached(p, list(range(b)), Q, s, idx, True)
    dev_idx = _dev(np.asarray(idx, dtype=np.int32))
    # the captured step's inputs, refilled before every replay
    xs = _dev(p["x"][:, Q], bf)
    dts, Bs, Cs = _dev(p["dt_raw"][:, Q]), _dev(p["B"][:, Q], bf), _dev(p["C"][:, Q], bf)
    pos = _dev(np.zeros(b, dtype=np.int32))
    y = torch.empty((b, H, P), dtype=bf, device=xs.device)
    A, D, bias = _dev(p["A"]), _dev(p["D"]), _dev(p["dt_bias"])

    def step(slots, x, dt, Bt, Ct, ps, out):
        ssd.decode_emulated(x, dt, A, Bt, Ct, slots.state, slots.chunks, dev_idx, ps,
                            chunk_size=Q, D=D, dt_bias=bias, out=out)

    # warm-up outside the capture, on scratch slots
    warm = _Slots(3)
    step(warm, xs, dts, Bs, Cs, pos, y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(ga, xs, dts, Bs, Cs, pos, y)
    for t in range(Q, T):
        xs.copy_(_dev(p["x"][:, t], bf))
        dts.copy_(_dev(p["dt_raw"][:, t]))
        Bs.copy_(_dev(p["B"][:, t], bf))
        Cs.copy_(_dev(p["C"][:, t], bf))
        pos.fill_(t % Q)
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        ye = torch.empty_like(y)
        step(eg, xs, dts, Bs, Cs, pos, ye)
        torch.cuda.synchronize()
        assert torch.equal(y, ye), t
    assert torch.equal(ga.state, eg.state)
    for a, e in zip(ga.chunks, eg.chunks):
        assert torch.equal(a, e)


def test_emulated_decode_many_rows_bitwise():
    """520 rows x 64 heads (33,280 work items), decoded from empty slots for
    130 tokens in lockstep, so that every row completes its chunk in the same
    step: the pass for completing rows then walks up to 65 items per
    workgroup (two rounds of 64 candidates).  Every step's outputs equal the
    strict prefill's bit for bit, and after the chunk end every slot holds
    the strict prefill's state after Q tokens."""
    import torch
    import mamba_ssd_selective_amd as ssd
    dev, bf = torch.device("cuda:0"), torch.bfloat16
    b, T = 520, Q + 2
    gen = torch.Generator(device=dev).manual_seed(77)
    x = torch.randn((b, T, H, P), generator=gen, device=dev).to(bf)
    dt = torch.randn((b, T, H), generator=gen, device=dev)
    Bm = (torch.randn((b, T, G, N), generator=gen, device=dev) / N ** 0.5).to(bf)
    Cm = (torch.randn((b, T, G, N), generator=gen, device=dev) / N ** 0.5).to(bf)
    A = -torch.exp(torch.rand(H, generator=gen, device=dev) * 2.7)
    D = torch.randn(H, generator=gen, device=dev)
    bias = -2.0 - 2.0 * torch.rand(H, generator=gen, device=dev)
    idx = torch.randperm(b, generator=gen, device=dev).to(torch.int32)

    def prefill(L):
        st = torch.zeros((b, H, P, N), device=dev)
        y = ssd.chunk_scan_fwd_cached(x[:, :L].contiguous(), dt[:, :L].contiguous(), A,
                                      Bm[:, :L].contiguous(), Cm[:, :L].contiguous(), st,
                                      torch.arange(b, dtype=torch.int32, device=dev), chunk_size=Q,
                                      init_from_cache=False, strict=True, D=D, dt_bias=bias)
        return y, st

    y_full, _ = prefill(T)
    _, st_q = prefill(Q)
    slots = _Slots(b)
    for t in range(T):
        pos = torch.full((b,), t % Q, dtype=torch.int32, device=dev)
        y = ssd.decode_emulated(x[:, t].contiguous(), dt[:, t].contiguous(), A, Bm[:, t].contiguous(),
                                Cm[:, t].contiguous(), slots.state, slots.chunks, idx, pos,
                                chunk_size=Q, D=D, dt_bias=bias)
        assert torch.equal(y, y_full[:, t]), t
        if t == Q - 1:
            assert torch.equal(slots.state[idx.long()], st_q)
    torch.cuda.synchronize()
