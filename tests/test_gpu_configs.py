"""The five workloads at full size, in the launch configuration bench.py times,
checked against the fp64 oracle on sampled heads (the recurrence is
independent per head, so the oracle runs on a head subset of the same
inputs) and, for the decode workload, on sampled rows.  Every check is
repeated with D = 0 (the state-space part alone).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import head_subset, host, log, run_oracle, run_scan, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_sampled(p, t, Q, heads, label, first_chunk=False):
    for zero_D in (False, True):
        y, fs = run_scan(t, Q, zero_D=zero_D)
        Y, F = host(y), host(fs)
        sub = head_subset(p, heads)
        yr, hr = run_oracle(sub, zero_D=zero_D)
        ey = oracle.rel_l2(Y[:, :, heads], yr)
        eh = oracle.rel_l2(F[:, heads], hr)
        log("%s D=%s heads=%s: rel_l2 y=%.3e final=%.3e" % (label, not zero_D, heads, ey, eh))
        assert np.isfinite(Y).all() and np.isfinite(F).all()
        assert ey < 2e-2 and eh < 2e-2
        if first_chunk:
            e1 = oracle.rel_l2(Y[:, :Q][:, :, heads], yr[:, :Q])
            log("%s first chunk D=%s: rel_l2 %.3e" % (label, not zero_D, e1))
            assert e1 < 2e-2


def test_config1_prefill_8k():
    w = workloads.WORKLOADS[1]
    p = workloads.make_inputs(w)
    t = to_dev(p, "bf16")
    # one head of every B/C group
    _check_sampled(p, t, w.chunk, [0, 9, 18, 27, 36, 45, 54, 63], "config1")


def test_config2_packed_16k():
    w = workloads.WORKLOADS[2]
    p = workloads.make_inputs(w)
    assert p["seq_idx"] is not None and len(np.unique(p["seq_idx"])) == 16
    t = to_dev(p, "bf16")
    _check_sampled(p, t, w.chunk, [3, 12, 21, 30, 39, 48, 57, 60], "config2")


def test_config3_long_128k():
    w = workloads.WORKLOADS[3]
    p = workloads.make_inputs(w)
    t = to_dev(p, "bf16")
    # one head of every B/C group (the oracle runs them one thread each)
    _check_sampled(p, t, w.chunk, [5, 14, 23, 32, 41, 50, 58, 62], "config3", first_chunk=True)


def _token(t, k):
    return t["x"][:, k].contiguous(), t["dt_raw"][:, k].contiguous()


def _token_bc(t, k):
    return t["B"][:, k].contiguous(), t["C"][:, k].contiguous()


def test_config4_prefill_then_decode():
    """64 rows: 4096-token chunked prefill, then 256 single-token updates on
    the fp32 state; compared with the oracle's single 4352-token scan."""
    import torch
    import mamba_ssd_selective_amd as ssd
    w = workloads.WORKLOADS[4]
    pre, steps = w.prefill, w.decode_steps
    p = workloads.make_inputs(w)
    log("config4: inputs drawn")
    t = to_dev(p, "bf16")
    pre_t = {k: (v[:, :pre].contiguous() if k in ("x", "dt_raw", "B", "C") else v)
             for k, v in t.items()}
    y_pre, state = run_scan(pre_t, w.chunk)
    ys = []
    for k in range(pre, pre + steps):
        ys.append(ssd.state_update(state, *_token(t, k), t["A"], *_token_bc(t, k), D=t["D"],
                                   dt_bias=t["dt_bias"]))
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, dim=1)
    # the single 4352-token chunked scan on the GPU as well
    y_full, f_full = run_scan(t, w.chunk)
    rows, heads = [0, 37, 63], [0, 17, 63]
    sub = head_subset({k: (v[rows] if k in ("x", "dt_raw", "B", "C") else v)
                       for k, v in p.items()}, heads)
    yr, hr = run_oracle(sub)
    Ypre = host(y_pre)[rows][:, :, heads]
    Ydec = host(y_dec)[rows][:, :, heads]
    Yfull = host(y_full)[rows][:, :, heads]
    e_pre = oracle.rel_l2(Ypre, yr[:, :pre])
    e_dec = oracle.rel_l2(Ydec, yr[:, pre:])
    e_st = oracle.rel_l2(host(state)[rows][:, heads], hr)
    e_full = oracle.rel_l2(Yfull, yr)
    e_ffull = oracle.rel_l2(host(f_full)[rows][:, heads], hr)
    log("config4: prefill y=%.3e decode y=%.3e state=%.3e | single scan y=%.3e final=%.3e"
        % (e_pre, e_dec, e_st, e_full, e_ffull))
    for e in (e_pre, e_dec, e_st, e_full, e_ffull):
        assert e < 2e-2
    # D = 0: the state-space part alone, prefill and decode
    y_pre0, state0 = run_scan(pre_t, w.chunk, zero_D=True)
    zD = torch.zeros_like(t["D"])
    ys0 = [ssd.state_update(state0, *_token(t, k), t["A"], *_token_bc(t, k), D=zD,
                            dt_bias=t["dt_bias"])
           for k in range(pre, pre + steps)]
    torch.cuda.synchronize()
    yr0, _ = run_oracle(sub, zero_D=True)
    e_pre0 = oracle.rel_l2(host(y_pre0)[rows][:, :, heads], yr0[:, :pre])
    e_dec0 = oracle.rel_l2(host(torch.stack(ys0, dim=1))[rows][:, :, heads], yr0[:, pre:])
    log("config4 D=0: prefill y=%.3e decode y=%.3e" % (e_pre0, e_dec0))
    assert e_pre0 < 2e-2 and e_dec0 < 2e-2
