"""Final states written over the initial states they start from.

ssd_chunk_scan_fwd accepts final_states == initial_states, and the cached
prefill always scans in place (its gathered slot states are both).  When a
row is cut into several segments, every segment's workgroup reads the initial
state while the last segment's writes the final one; with more workgroups
than fit at once the two must still not meet.  The shapes below are chosen
so that the grid exceeds one workgroup per CU (three rows of 64 heads, two
segments each), and every result must be bitwise the out-of-place one."""
import numpy as np
import pytest

import workloads
from gpu_util import log

pytestmark = pytest.mark.gpu


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.device("cuda:0"))
    return (t.to(dtype) if dtype is not None else t).contiguous()


def _inputs(seed, b, L, H, P, N, G):
    import torch
    p = workloads.random_problem(np.random.default_rng(seed), b, L, H, P, N, G, io="bf16", init=True)
    bf = torch.bfloat16
    return p, dict(x=_dev(p["x"], bf), dt=_dev(p["dt_raw"]), A=_dev(p["A"]), B=_dev(p["B"], bf),
                   C=_dev(p["C"], bf), D=_dev(p["D"]), bias=_dev(p["dt_bias"]), h0=_dev(p["h_init"]))


def test_chunk_scan_final_over_initial_states():
    import torch
    import mamba_ssd_selective_amd as ssd
    b, L, H, P, N, G, Q = 3, 4096, 64, 64, 128, 8, 128
    assert ssd.segments(b, L, H, P, N, G, Q) == 2
    log("alias: chunk_scan_fwd b=%d L=%d H=%d" % (b, L, H))
    _, t = _inputs(5, b, L, H, P, N, G)
    y_ref, fs_ref = ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], chunk_size=Q, D=t["D"],
                                       dt_bias=t["bias"], initial_states=t["h0"], return_final_states=True)
    st = t["h0"].clone()
    y, fs = ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], chunk_size=Q, D=t["D"],
                               dt_bias=t["bias"], initial_states=st, return_final_states=True,
                               final_states_out=st)
    torch.cuda.synchronize()
    assert fs.data_ptr() == st.data_ptr()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    assert torch.equal(st.view(torch.int32), fs_ref.view(torch.int32))


def test_cached_prefill_in_place_matches_out_of_place():
    import torch
    import mamba_ssd_selective_amd as ssd
    b, L, H, P, N, G, Q = 3, 4096, 64, 64, 128, 8, 128
    log("alias: cached prefill b=%d L=%d H=%d" % (b, L, H))
    p, t = _inputs(6, b, L, H, P, N, G)
    slots = 5
    cache = np.random.default_rng(9).standard_normal((slots, H, P, N)).astype(np.float32)
    idx = np.array([3, 0, 4], dtype=np.int32)
    c = _dev(cache)
    y = ssd.chunk_scan_fwd_cached(t["x"], t["dt"], t["A"], t["B"], t["C"], c, _dev(idx), chunk_size=Q,
                                  D=t["D"], dt_bias=t["bias"], init_from_cache=True)
    # out of place: the same rows from separate initial and final states
    h0 = _dev(cache[idx])
    y_ref, fs_ref = ssd.chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], chunk_size=Q, D=t["D"],
                                       dt_bias=t["bias"], initial_states=h0, return_final_states=True)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    got = c.cpu().numpy()
    assert np.array_equal(got[idx], fs_ref.cpu().numpy())
    others = np.setdiff1d(np.arange(slots), idx)
    assert np.array_equal(got[others], cache[others])
