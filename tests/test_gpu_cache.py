"""Decode on state caches (continuous batching): the SSM state update and the
conv update with per-row int32 slot indices into caches that outlive the
batch (the per-sequence conv and fp32 SSM states of RL-Kernel RFC
"Nemotron-3-Nano-30B-A3B", section 1, operator family 2).  Checked against the
unindexed entry points on gathered states (bitwise: the same arithmetic), the
fp64 oracle, and untouched slots and padding rows."""
import numpy as np
import pytest

import oracle
import workloads
from oracle import mixer

pytestmark = pytest.mark.gpu


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.device("cuda:0"))
    return (t.to(dtype) if dtype is not None else t).contiguous()


def _host(t):
    return t.float().cpu().numpy()


def _slots(rng, b, rows, pad):
    """b distinct slots of [0, rows), with `pad` of them replaced by indices
    outside the cache (padding rows)."""
    idx = rng.permutation(rows)[:b].astype(np.int32)
    if pad:
        where = rng.choice(b, size=pad, replace=False)
        idx[where] = np.array([-1, rows, rows + 7, -100][:pad], dtype=np.int32)
    return idx


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("bH,rows,pad", [((5, 8), 37, 2), ((16, 64), 40, 3), ((1, 2), 1, 0)],
                         ids=["few_heads", "many_heads", "one_slot"])
def test_state_update_cached(io, bH, rows, pad):
    import torch
    import mamba_ssd_selective_amd as ssd
    (b, H), G, P, N = bH, 2 if bH[1] % 2 == 0 else 1, 64, 128
    rng = np.random.default_rng(rows * 10 + b)
    p = workloads.random_problem(rng, b, 1, H, P, N, G, io=io, init=False)
    cache = rng.standard_normal((rows, H, P, N)).astype(np.float32)
    idx = _slots(rng, b, rows, pad)
    live = (idx >= 0) & (idx < rows)
    print("case io=%s b=%d H=%d rows=%d idx=%s" % (io, b, H, rows, idx.tolist()), flush=True)
    t = torch.bfloat16 if io == "bf16" else torch.float32
    x, dt = _dev(p["x"][:, 0], t), _dev(p["dt_raw"][:, 0])
    Bm, Cm = _dev(p["B"][:, 0], t), _dev(p["C"][:, 0], t)
    A, D, bias = _dev(p["A"]), _dev(p["D"]), _dev(p["dt_bias"])
    c = _dev(cache)
    y = torch.full((b, H, P), 3.0, dtype=t, device=c.device)
    ssd.state_update(c, x, dt, A, Bm, Cm, D=D, dt_bias=bias, out=y, state_indices=_dev(idx))
    # the unindexed update on the gathered states (padding rows get zeros)
    g = np.zeros((b, H, P, N), dtype=np.float32)
    g[live] = cache[idx[live]]
    gd = _dev(g)
    y2 = ssd.state_update(gd, x, dt, A, Bm, Cm, D=D, dt_bias=bias)
    torch.cuda.synchronize()
    got_c, got_y, ref_g, ref_y = _host(c), _host(y), _host(gd), _host(y2)
    assert np.array_equal(got_c[idx[live]], ref_g[live])
    assert np.array_equal(got_y[live], ref_y[live])
    untouched = np.setdiff1d(np.arange(rows), idx[live])
    assert np.array_equal(got_c[untouched], cache[untouched])
    assert np.all(got_y[~live] == 3.0)
    # and the oracle on the live rows
    st, yr = oracle.step(g.astype(np.float64), p["x"][:, 0], p["dt_raw"][:, 0], p["A"],
                         p["B"][:, 0], p["C"][:, 0], dt_bias=p["dt_bias"], D=p["D"])
    assert oracle.rel_l2(got_c[idx[live]], st[live]) < 1e-5
    assert oracle.rel_l2(got_y[live], yr[live]) < (1e-5 if io == "f32" else 2e-2)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_update_cached(io):
    import torch
    import mamba_ssd_selective_amd as ssd
    H, P, G, N = 64, 64, 8, 128
    dim = H * P + 2 * G * N
    b, rows = 12, 50
    rng = np.random.default_rng(5)
    rnd = workloads.round_bf16 if io == "bf16" else (lambda a: a.astype(np.float32))
    t = torch.bfloat16 if io == "bf16" else torch.float32
    xbc = rnd(rng.standard_normal((b, dim), dtype=np.float32))
    w = (rng.standard_normal((dim, 4)) * 0.5).astype(np.float32)
    bias = rng.standard_normal(dim).astype(np.float32)
    cache = rnd(rng.standard_normal((rows, dim, 3), dtype=np.float32))
    idx = _slots(rng, b, rows, 3)
    live = (idx >= 0) & (idx < rows)
    print("case io=%s idx=%s" % (io, idx.tolist()), flush=True)
    c = _dev(cache, t)
    dev = c.device
    out = (torch.full((b, H, P), 5.0, dtype=t, device=dev),
           torch.full((b, G, N), 5.0, dtype=t, device=dev),
           torch.full((b, G, N), 5.0, dtype=t, device=dev))
    xd, wd, bd = _dev(xbc, t), _dev(w), _dev(bias)
    ssd.conv1d_update(xd, c, wd, nheads=H, headdim=P, ngroups=G, dstate=N, bias=bd,
                      state_indices=_dev(idx), out=out)
    g = np.zeros((b, dim, 3), dtype=np.float32)
    g[live] = cache[idx[live]]
    gd = _dev(g, t)
    ref = ssd.conv1d_update(xd, gd, wd, nheads=H, headdim=P, ngroups=G, dstate=N, bias=bd)
    torch.cuda.synchronize()
    got_c = _host(c)
    assert np.array_equal(got_c[idx[live]], _host(gd)[live])
    untouched = np.setdiff1d(np.arange(rows), idx[live])
    assert np.array_equal(got_c[untouched], cache[untouched])
    for o, r in zip(out, ref):
        assert np.array_equal(_host(o)[live], _host(r)[live])
        assert np.all(_host(o)[~live] == 5.0)
    ro, rs = mixer.conv1d_update(xbc[live], w, bias, g[live])
    assert np.array_equal(got_c[idx[live]], rs)   # the state holds inputs as they are
    gx = _host(out[0]).reshape(b, -1)[live]
    assert oracle.rel_l2(gx, ro[:, :H * P]) < (1e-4 if io == "f32" else 2e-2)


def test_continuous_batching_decode():
    """Four sequences on a 6-slot cache decode over five steps whose batches
    change in membership and order (a sequence joins, one sits out a step);
    every sequence's outputs and final slot equal its own oracle decode."""
    import torch
    import mamba_ssd_selective_amd as ssd
    H, P, N, G, rows = 8, 64, 128, 2, 6
    rng = np.random.default_rng(17)
    nseq, T = 4, 5
    slot = {0: 4, 1: 0, 2: 5, 3: 2}
    # per-sequence tokens (T each) and initial states
    seqs = [workloads.random_problem(rng, 1, T, H, P, N, G, io="bf16", init=True)
            for _ in range(nseq)]
    A, D, bias = _dev(seqs[0]["A"]), _dev(seqs[0]["D"]), _dev(seqs[0]["dt_bias"])
    cache = np.zeros((rows, H, P, N), dtype=np.float32)
    for s in range(nseq):
        cache[slot[s]] = seqs[s]["h_init"][0]
    c = _dev(cache)
    batches = [[2, 0, 1], [0, 1, 2, 3], [3, 1], [1, 3, 0, 2], [2, 3, 0, 1]]
    pos = [0] * nseq
    ys = {s: [] for s in range(nseq)}
    bf = torch.bfloat16
    for members in batches:
        rows_x = np.stack([seqs[s]["x"][0, pos[s]] for s in members])
        rows_dt = np.stack([seqs[s]["dt_raw"][0, pos[s]] for s in members])
        rows_B = np.stack([seqs[s]["B"][0, pos[s]] for s in members])
        rows_C = np.stack([seqs[s]["C"][0, pos[s]] for s in members])
        idx = np.array([slot[s] for s in members], dtype=np.int32)
        y = ssd.state_update(c, _dev(rows_x, bf), _dev(rows_dt), A, _dev(rows_B, bf),
                             _dev(rows_C, bf), D=D, dt_bias=bias, state_indices=_dev(idx))
        yh = _host(y)
        for r, s in enumerate(members):
            ys[s].append(yh[r])
            pos[s] += 1
    torch.cuda.synchronize()
    got = _host(c)
    p0 = seqs[0]
    for s in range(nseq):
        q = seqs[s]
        n = pos[s]
        st = q["h_init"].astype(np.float64)
        yr = []
        for k in range(n):
            st, y1 = oracle.step(st, q["x"][:, k], q["dt_raw"][:, k], p0["A"], q["B"][:, k],
                                 q["C"][:, k], dt_bias=p0["dt_bias"], D=p0["D"])
            yr.append(y1[0])
        assert oracle.rel_l2(got[slot[s]], st[0]) < 1e-5
        assert oracle.rel_l2(np.stack(ys[s]), np.stack(yr)) < 2e-2
    # the slots no sequence holds stayed zero
    assert not got[[1, 3]].any()


def _prefill_case(seed, b, L, H, G, io, rows):
    rng = np.random.default_rng(seed)
    p = workloads.random_problem(rng, b, L, H, 64, 128, G, io=io, init=False)
    p["cache"] = rng.standard_normal((rows, H, 64, 128)).astype(np.float32)
    return rng, p


def _run_prefill(p, idx, lens, io, Q, init_from_cache=True, zero_D=False):
    import torch
    import mamba_ssd_selective_amd as ssd
    t = torch.bfloat16 if io == "bf16" else torch.float32
    c = _dev(p["cache"])
    D = np.zeros_like(p["D"]) if zero_D else p["D"]
    y = ssd.chunk_scan_fwd_cached(_dev(p["x"], t), _dev(p["dt_raw"]), _dev(p["A"]), _dev(p["B"], t),
                                  _dev(p["C"], t), c, _dev(idx), chunk_size=Q,
                                  seq_lens=None if lens is None else _dev(lens),
                                  init_from_cache=init_from_cache, D=_dev(D),
                                  dt_bias=_dev(p["dt_bias"]))
    torch.cuda.synchronize()
    return _host(y), _host(c)


def _oracle_row(p, r, n, h0, heads=None, grp=None, zero_D=False):
    hs = slice(None) if heads is None else heads
    gs = slice(None) if grp is None else grp
    D = np.zeros_like(p["D"]) if zero_D else p["D"]
    return oracle.scan(p["x"][r:r + 1, :n, hs], p["dt_raw"][r:r + 1, :n, hs], p["A"][hs],
                       p["B"][r:r + 1, :n, gs], p["C"][r:r + 1, :n, gs],
                       dt_bias=p["dt_bias"][hs], D=D[hs],
                       h_init=None if h0 is None else h0[None])


@pytest.mark.parametrize("io,Q", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("init_from_cache", [True, False])
def test_prefill_cached_rows(io, Q, init_from_cache):
    """Rows of lengths 300 (all), 0, 1, one chunk, a ragged 200 and a padding
    row: each row's y up to its length and its slot equal the oracle's scan of
    that row's real tokens from the slot's state; other slots are untouched."""
    b, L, H, G, rows = 6, 300, 8, 2, 9
    rng, p = _prefill_case(3, b, L, H, G, io, rows)
    idx = np.array([7, 2, 0, 5, -1, 3], dtype=np.int32)
    lens = np.array([300, 0, 1, Q, 137, 200], dtype=np.int32)
    tol = 1e-4 if io == "f32" else 2e-2
    # with D, and with D = 0 (D x dominates y, which would hide the scan terms)
    for zero_D in (False, True):
        print("case io=%s Q=%d init=%s D=%s" % (io, Q, init_from_cache, "0" if zero_D else "D"),
              flush=True)
        y, c = _run_prefill(p, idx, lens, io, Q, init_from_cache, zero_D=zero_D)
        for r in range(b):
            s, n = idx[r], lens[r]
            if not 0 <= s < rows:
                continue
            h0 = p["cache"][s] if init_from_cache else None
            if n == 0:
                want = p["cache"][s] if init_from_cache else np.zeros_like(p["cache"][s])
                assert np.array_equal(c[s], want)
                continue
            yr, hr = _oracle_row(p, r, n, h0, zero_D=zero_D)
            assert oracle.rel_l2(y[r, :n], yr[0]) < tol, (r, zero_D)
            assert oracle.rel_l2(c[s], hr[0]) < tol, (r, zero_D)
        untouched = [s for s in range(rows) if s not in idx]
        assert np.array_equal(c[untouched], p["cache"][untouched])


def test_prefill_cached_matches_plain_scan():
    """All rows full and slots 0..b-1 in order: the same y and final states
    as the plain scan with those initial states, bit for bit."""
    import torch
    import mamba_ssd_selective_amd as ssd
    b, L, H, G = 3, 700, 8, 2
    rng, p = _prefill_case(8, b, L, H, G, "bf16", b)
    bf = torch.bfloat16
    y0, fs = ssd.chunk_scan_fwd(_dev(p["x"], bf), _dev(p["dt_raw"]), _dev(p["A"]), _dev(p["B"], bf),
                                _dev(p["C"], bf), chunk_size=128, D=_dev(p["D"]),
                                dt_bias=_dev(p["dt_bias"]), initial_states=_dev(p["cache"]),
                                return_final_states=True)
    y, c = _run_prefill(p, np.arange(b, dtype=np.int32), None, "bf16", 128)
    assert np.array_equal(y, _host(y0))
    assert np.array_equal(c, _host(fs))


def test_prefill_cached_8k_shape():
    """The 8K-token shape (H 64, G 8) as a two-row batch of lengths 8192 and
    5000 on an 8-slot cache; the oracle runs the heads of group 5."""
    b, L, H, G, rows = 2, 8192, 64, 8, 8
    rng, p = _prefill_case(12, b, L, H, G, "bf16", rows)
    idx = np.array([6, 1], dtype=np.int32)
    lens = np.array([8192, 5000], dtype=np.int32)
    grp = 5
    hs = slice(8 * grp, 8 * grp + 8)
    for zero_D in (False, True):
        y, c = _run_prefill(p, idx, lens, "bf16", 128, zero_D=zero_D)
        for r in range(b):
            s, n = idx[r], lens[r]
            yr, hr = _oracle_row(p, r, n, p["cache"][s][hs], heads=hs, grp=slice(grp, grp + 1),
                                 zero_D=zero_D)
            ey, eh = oracle.rel_l2(y[r, :n, hs], yr[0]), oracle.rel_l2(c[s][hs], hr[0])
            print("row %d D=%s: y %.3e state %.3e" % (r, "0" if zero_D else "D", ey, eh), flush=True)
            assert ey < 2e-2 and eh < 2e-2


def test_prefill_then_decode_on_cache():
    """Prompts of different lengths prefilled into their slots, then three
    decode tokens each on the same slots: every sequence's decode outputs and
    final slot equal the oracle's scan of its prompt plus the three tokens."""
    import torch
    import mamba_ssd_selective_amd as ssd
    b, L, H, G, rows = 4, 260, 8, 2, 6
    T = 3
    rng, p = _prefill_case(21, b, L + T, H, G, "bf16", rows)
    idx = np.array([4, 0, 5, 2], dtype=np.int32)
    lens = np.array([260, 77, 128, 1], dtype=np.int32)
    # the prompts: each row's first lens[r] tokens, zeros after
    q = {k: p[k].copy() for k in ("x", "dt_raw", "B", "C")}
    for k in q:
        q[k] = q[k][:, :L].copy()
        for r in range(b):
            q[k][r, lens[r]:] = 0
    q.update({k: p[k] for k in ("A", "D", "dt_bias", "cache")})
    _, c = _run_prefill(q, idx, lens, "bf16", 128)
    cd = _dev(c)
    bf = torch.bfloat16
    ys = []
    for k in range(T):
        # decode token k of row r is the row's token lens[r] + k
        pick = lambda a: np.stack([a[r, lens[r] + k] for r in range(b)])
        ys.append(_host(ssd.state_update(cd, _dev(pick(p["x"]), bf), _dev(pick(p["dt_raw"])),
                                         _dev(p["A"]), _dev(pick(p["B"]), bf), _dev(pick(p["C"]), bf),
                                         D=_dev(p["D"]), dt_bias=_dev(p["dt_bias"]),
                                         state_indices=_dev(idx))))
    torch.cuda.synchronize()
    got = _host(cd)
    for r in range(b):
        n = lens[r] + T
        yr, hr = _oracle_row(p, r, n, p["cache"][idx[r]])
        dec = np.stack([ys[k][r] for k in range(T)])
        assert oracle.rel_l2(dec, yr[0, lens[r]:n]) < 2e-2, r
        assert oracle.rel_l2(got[idx[r]], hr[0]) < 2e-2, r


def _varlen_case(seed, lens, H, G, io, rows):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    p = workloads.random_problem(rng, 1, T, H, 64, 128, G, io=io, init=False)
    p = {k: (v[0] if k in ("x", "dt_raw", "B", "C") else v) for k, v in p.items()}
    p["cache"] = rng.standard_normal((rows, H, 64, 128)).astype(np.float32)
    p["cu"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return p


@pytest.mark.parametrize("io,Q", [("bf16", 128), ("f32", 64)])
def test_varlen_packed_sequences(io, Q):
    """Five packed sequences of 300, 1, 128, 0 and 77 tokens: each one's y
    and final slot equal the oracle's scan of that sequence from its slot's
    state; the slots of no sequence are untouched."""
    import torch
    import mamba_ssd_selective_amd as ssd
    lens = [300, 1, 128, 0, 77]
    H, G, rows = 8, 2, 9
    p = _varlen_case(17, lens, H, G, io, rows)
    idx = np.array([6, 0, 3, 8, 1], dtype=np.int32)
    t = torch.bfloat16 if io == "bf16" else torch.float32
    tol = 1e-4 if io == "f32" else 2e-2
    for zero_D in (False, True):
        D = np.zeros_like(p["D"]) if zero_D else p["D"]
        c = _dev(p["cache"])
        y = ssd.chunk_scan_fwd_varlen(_dev(p["x"], t), _dev(p["dt_raw"]), _dev(p["A"]), _dev(p["B"], t),
                                      _dev(p["C"], t), _dev(p["cu"]), c, _dev(idx),
                                      # fp32: the wrapper reads the longest length back
                                      max_seqlen=max(lens) if io == "bf16" else None,
                                      chunk_size=Q, D=_dev(D), dt_bias=_dev(p["dt_bias"]),
                                      check_seqlens=True)
        torch.cuda.synchronize()
        y, c = _host(y), _host(c)
        for r, n in enumerate(lens):
            s, a = idx[r], p["cu"][r]
            if n == 0:
                assert np.array_equal(c[s], p["cache"][s])
                continue
            yr, hr = oracle.scan(p["x"][None, a:a + n], p["dt_raw"][None, a:a + n], p["A"],
                                 p["B"][None, a:a + n], p["C"][None, a:a + n], dt_bias=p["dt_bias"],
                                 D=D, h_init=p["cache"][s][None])
            assert oracle.rel_l2(y[a:a + n], yr[0]) < tol, (r, zero_D)
            assert oracle.rel_l2(c[s], hr[0]) < tol, (r, zero_D)
        untouched = [s for s in range(rows) if s not in idx]
        assert np.array_equal(c[untouched], p["cache"][untouched])


@pytest.mark.parametrize("strict", [True, False])
def test_varlen_equals_cached_rows_bitwise(strict):
    """The packed prefill gives the bits of the cached prefill on the same
    sequences laid out as rows of one batch.  The rows' padding holds NaN:
    it is never read.  Non-strict, 4 rows x 16 heads cut each row into four
    segments of two chunks, so that short rows have segments with no chunk."""
    import torch
    import mamba_ssd_selective_amd as ssd
    lens = [700, 129, 1000, 64]
    H, G, rows = 16, 2, 4
    p = _varlen_case(23, lens, H, G, "bf16", rows)
    idx = np.array([2, 3, 0, 1], dtype=np.int32)
    bf = torch.bfloat16
    Lm = max(lens)
    if not strict:
        assert ssd.segments(len(lens), Lm, H, 64, 128, G, 128) == 4
    c1 = _dev(p["cache"])
    y = ssd.chunk_scan_fwd_varlen(_dev(p["x"], bf), _dev(p["dt_raw"]), _dev(p["A"]), _dev(p["B"], bf),
                                  _dev(p["C"], bf), _dev(p["cu"]), c1, _dev(idx), max_seqlen=Lm,
                                  chunk_size=128, strict=strict, D=_dev(p["D"]),
                                  dt_bias=_dev(p["dt_bias"]))
    rowsd = {}
    for k in ("x", "dt_raw", "B", "C"):
        a = np.full((len(lens), Lm) + p[k].shape[1:], np.nan, dtype=p[k].dtype)
        for r, n in enumerate(lens):
            a[r, :n] = p[k][p["cu"][r]:p["cu"][r] + n]
        rowsd[k] = a
    c2 = _dev(p["cache"])
    y2 = ssd.chunk_scan_fwd_cached(_dev(rowsd["x"], bf), _dev(rowsd["dt_raw"]), _dev(p["A"]),
                                   _dev(rowsd["B"], bf), _dev(rowsd["C"], bf), c2, _dev(idx),
                                   chunk_size=128, seq_lens=_dev(np.array(lens, dtype=np.int32)),
                                   strict=strict, D=_dev(p["D"]), dt_bias=_dev(p["dt_bias"]))
    torch.cuda.synchronize()
    y, y2 = _host(y), _host(y2)
    for r, n in enumerate(lens):
        a = p["cu"][r]
        assert np.array_equal(y[a:a + n], y2[r, :n]), r
        assert np.isfinite(y2[r, :n]).all(), r
    assert np.array_equal(_host(c1), _host(c2))
    assert np.isfinite(_host(c1)).all()


@pytest.mark.parametrize("init_from_cache", [False, True])
def test_cached_prefill_of_no_tokens(init_from_cache):
    """L = 0: a row that starts from zeros ends in zeros, written to its slot;
    a row that starts from its slot leaves it as it is; padding rows and
    other slots are untouched either way."""
    import torch
    import mamba_ssd_selective_amd as ssd
    b, H, P, N, G, Q, slots = 3, 4, 64, 128, 2, 128, 6
    rng = np.random.default_rng(31)
    cache = rng.standard_normal((slots, H, P, N)).astype(np.float32)
    idx = np.array([4, -1, 1], dtype=np.int32)  # the middle row is padding
    c = _dev(cache)
    bf = torch.bfloat16
    z = lambda *s: torch.zeros(s, dtype=bf, device="cuda:0")
    f = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda:0")
    ssd.chunk_scan_fwd_cached(z(b, 0, H, P), f(b, 0, H), f(H), z(b, 0, G, N), z(b, 0, G, N), c,
                              _dev(idx), chunk_size=Q, init_from_cache=init_from_cache)
    torch.cuda.synchronize()
    got = c.cpu().numpy()
    live = np.array([4, 1])
    want = cache[live] if init_from_cache else np.zeros_like(cache[live])
    assert np.array_equal(got[live], want)
    others = np.setdiff1d(np.arange(slots), live)
    assert np.array_equal(got[others], cache[others])
