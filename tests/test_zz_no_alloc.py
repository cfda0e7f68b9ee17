"""ssd_chunk_scan_fwd_noalloc (the entry point that takes its scratch from the
library's static device array instead of a caller workspace) against
ssd_chunk_scan_fwd: same kernels, so the outputs must be bitwise equal.  Two
calls in a row, the second on a smaller input (the array keeps the first
call's contents), then a problem too large for the array, which must be
rejected before any launch."""
import ctypes
import math

import numpy as np
import pytest

import workloads
from gpu_util import log

pytestmark = pytest.mark.gpu


def _call_fwd(lib, d, t, y, fs, ws, noalloc):
    import torch
    import mamba_ssd_selective_amd as ssd
    st = torch.cuda.current_stream().cuda_stream
    args = [ctypes.byref(d), 1, t["x"].data_ptr(), t["dt"].data_ptr(), t["bias"].data_ptr(), 1,
            0.0, math.inf, t["A"].data_ptr(), t["B"].data_ptr(), t["C"].data_ptr(), t["D"].data_ptr(),
            t["h0"].data_ptr(), None, y.data_ptr(), fs.data_ptr()]
    if noalloc:
        return lib.ssd_chunk_scan_fwd_noalloc(*args, st)
    return lib.ssd_chunk_scan_fwd(*args, ws.data_ptr(), ws.numel(), st)


def _problem(seed, b, L, H, P, N, G):
    import torch
    rng = np.random.default_rng(seed)
    p = workloads.random_problem(rng, b, L, H, P, N, G, io="bf16", init=True)
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    return {"x": torch.from_numpy(p["x"]).to(dev).to(bf).contiguous(),
            "dt": torch.from_numpy(p["dt_raw"]).to(dev).contiguous(),
            "B": torch.from_numpy(p["B"]).to(dev).to(bf).contiguous(),
            "C": torch.from_numpy(p["C"]).to(dev).to(bf).contiguous(),
            "A": torch.from_numpy(p["A"]).to(dev), "D": torch.from_numpy(p["D"]).to(dev),
            "bias": torch.from_numpy(p["dt_bias"]).to(dev),
            "h0": torch.from_numpy(p["h_init"]).to(dev).contiguous()}


def test_noalloc_matches_workspace_entry_point():
    import torch
    import mamba_ssd_selective_amd as ssd
    lib = ssd.library()
    H, P, N, G, Q = 64, 64, 128, 8, 128
    # a large call, then a smaller one on the same (now dirty) scratch
    for seed, b, L in ((11, 1, 4096 + 77), (12, 2, 333)):
        log("noalloc: b=%d L=%d" % (b, L))
        t = _problem(seed, b, L, H, P, N, G)
        d = ssd._dims(b, L, H, P, N, G, Q)
        need = int(lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d), 1))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda:0")
        y_ref = torch.empty_like(t["x"])
        fs_ref = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda:0")
        assert _call_fwd(lib, d, t, y_ref, fs_ref, ws, False) == 0
        y = torch.full_like(t["x"], float("nan"))
        fs = torch.full_like(fs_ref, float("nan"))
        assert _call_fwd(lib, d, t, y, fs, None, True) == 0
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
        assert torch.equal(fs.view(torch.int32), fs_ref.view(torch.int32))


def test_noalloc_rejects_problems_beyond_the_static_scratch():
    import torch
    import mamba_ssd_selective_amd as ssd
    lib = ssd.library()
    H, P, N, G, Q = 64, 64, 128, 8, 128
    L = 1 << 20  # needs far more scratch than the static array holds
    d = ssd._dims(1, L, H, P, N, G, Q)
    assert int(lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d), 1)) > 64 << 20
    x = torch.zeros(16, dtype=torch.uint8, device="cuda:0")  # never read: rejected first
    p = x.data_ptr()
    st = lib.ssd_chunk_scan_fwd_noalloc(ctypes.byref(d), 1, p, p, None, 1, 0.0, math.inf, p, p, p,
                                        None, None, None, p, None,
                                        torch.cuda.current_stream().cuda_stream)
    assert st == 9  # SSD_ERR_TOO_LARGE
