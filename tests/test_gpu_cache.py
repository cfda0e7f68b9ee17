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
