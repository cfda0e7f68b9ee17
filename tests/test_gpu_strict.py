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

pytestmark = pytest.mark.gpu

H, P, N, G, Q = 64, 64, 128, 8, 128


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.device("cuda:0"))
    return (t.to(dtype) if dtype is not None else t).contiguous()


def _host(t):
    return t.float().cpu().numpy()


class _Slots:
    def __init__(self, rows):
        import torch
        dev, bf = torch.device("cuda:0"), torch.bfloat16
        self.state = torch.zeros((rows, H, P, N), dtype=torch.float32, device=dev)
        self.chunks = (torch.zeros((rows, Q, H, P), dtype=bf, device=dev),
                       torch.zeros((rows, Q, H), dtype=torch.float32, device=dev),
                       torch.zeros((rows, Q, G, N), dtype=bf, device=dev),
                       torch.zeros((rows, Q, G, N), dtype=bf, device=dev))


def _full_prefill(p, L):
    """The strict prefill of every row's first L tokens: (y, final states)."""
    b = p["x"].shape[0]
    s = _Slots(b)
    y = _cached(p, list(range(b)), L, s, list(range(b)), True)
    return y, _host(s.state)


def _step(p, slots, toks, idx, pos):
    """One emulated decode step; toks[r] = the token index of row r (ignored
    for padding rows)."""
    import torch
    import mamba_ssd_selective_amd as ssd
    bf = torch.bfloat16
    pick = lambda a: np.stack([a[r, max(t, 0)] for r, t in enumerate(toks)])
    y = torch.full((len(toks), H, P), 7.0, dtype=bf, device=torch.device("cuda:0"))
    ssd.decode_emulated(_dev(pick(p["x"]), bf), _dev(pick(p["dt_raw"])), _dev(p["A"]),
                        _dev(pick(p["B"]), bf), _dev(pick(p["C"]), bf), slots.state, slots.chunks,
                        _dev(np.asarray(idx, dtype=np.int32)), _dev(np.asarray(pos, dtype=np.int32)),
                        chunk_size=Q, D=_dev(p["D"]), dt_bias=_dev(p["dt_bias"]), out=y)
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


def _cached(p, rows_sel, L, slots, idx, strict, lens=None):
    import torch
    import mamba_ssd_selective_amd as ssd
    bf = torch.bfloat16
    sel = lambda k: p[k][rows_sel, :L]
    y = ssd.chunk_scan_fwd_cached(_dev(sel("x"), bf), _dev(sel("dt_raw")), _dev(p["A"]),
                                  _dev(sel("B"), bf), _dev(sel("C"), bf), slots.state,
                                  _dev(np.asarray(idx, dtype=np.int32)), chunk_size=Q,
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
