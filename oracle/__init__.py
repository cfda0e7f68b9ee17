"""fp64 CPU oracle for the Mamba-2 SSD selective scan.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library under ``mamba_ssd_selective_amd`` and never imports
it; the two meet only in the seeded input generator (``workloads``), which
holds none of the method's arithmetic.

Three independent formulations of the same operation live here:

* ``scan`` / ``step`` -- the plain sequential recurrence in C (``ssd_oracle.c``),
  the authority every GPU result is compared against;
* ``scan_bwd`` -- its gradients, by reverse mode of the same recurrence in C;
* ``mixer`` -- the steps beside the scan (causal conv1d + bias + SiLU with its
  conv state, the split into x/B/C, gated group RMSNorm), numpy fp64;
* ``dual.quadratic_scan`` -- the brute-force matrix ("dual") form with explicit
  products of per-step decays, for tiny inputs;
* ``chunked.chunked_scan`` -- the chunk decomposition (chunk states, state
  passing, chunk outputs) in numpy fp64, for any chunk size.

The operation (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 1 operator
families 1 and 2, section 3 Figure 2 box [F2]; "Nemotron 3 Nano - JAX
Implementation", Key Components item 1):

    dt_t = clamp(softplus(dt_raw_t + dt_bias), dt_min, dt_max)
    h_t  = exp(dt_t A) h_{t-1} + dt_t x_t (outer) B_t
    y_t  = h_t . C_t + D x_t
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_ssd.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ssd_oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load(path=None):
    """Load the compiled oracle (or, for mutation tests, another build of the
    same source at ``path``)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    i64, dp, ip = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p
    lib.oracle_ssd_scan.argtypes = [i64, i64, i64, i64, i64, i64,
                                    dp, dp, dp, ctypes.c_int, ctypes.c_double,
                                    ctypes.c_double, dp, dp, dp, dp, dp, ip,
                                    dp, dp, ctypes.c_int]
    lib.oracle_ssd_scan.restype = ctypes.c_int
    lib.oracle_ssd_step.argtypes = [i64, i64, i64, i64, i64, dp, dp, dp, dp,
                                    ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                    dp, dp, dp, dp, dp]
    lib.oracle_ssd_step.restype = ctypes.c_int
    lib.oracle_ssd_scan_bwd.argtypes = [i64, i64, i64, i64, i64, i64,
                                        dp, dp, dp, ctypes.c_int, ctypes.c_double,
                                        ctypes.c_double, dp, dp, dp, dp, dp, ip,
                                        dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.oracle_ssd_scan_bwd.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def compile_variant(src_text: str, out_path: str) -> str:
    """Compile an edited copy of the oracle source (mutation tests only)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                    "-shared", "-fPIC", "-o", out_path, src, "-lm"], check=True)
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def scan(x, dt_raw, A, B, C, *, dt_bias=None, D=None, h_init=None, seq_idx=None,
         dt_softplus=True, dt_min=0.0, dt_max=float("inf"), nthreads=0, lib=None):
    """Sequential fp64 recurrence over a whole batch.

    x (b,L,H,P), dt_raw (b,L,H), A (H), B/C (b,L,G,N), dt_bias/D (H),
    h_init (b,H,P,N), seq_idx (b,L) int.  Returns (y (b,L,H,P), h_final (b,H,P,N)),
    both float64.
    """
    x, dt_raw, A, B, C = map(_f64, (x, dt_raw, A, B, C))
    dt_bias, D, h_init = map(_f64, (dt_bias, D, h_init))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt_raw.shape == (b, L, H) and B.shape == (b, L, G, N) and C.shape == B.shape
    assert A.shape == (H,)
    if h_init is not None:
        assert h_init.shape == (b, H, P, N)
    sp = None
    if seq_idx is not None:
        seq_idx = np.ascontiguousarray(np.asarray(seq_idx, dtype=np.int32))
        assert seq_idx.shape == (b, L)
        sp = seq_idx.ctypes.data_as(ctypes.c_void_p)
    y = np.empty((b, L, H, P), dtype=np.float64)
    hf = np.empty((b, H, P, N), dtype=np.float64)
    rc = (lib or _load()).oracle_ssd_scan(
        b, L, H, P, N, G, _ptr(x), _ptr(dt_raw), _ptr(dt_bias), int(bool(dt_softplus)),
        float(dt_min), float(dt_max), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h_init),
        sp, _ptr(y), _ptr(hf), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_ssd_scan failed with code %d" % rc)
    return y, hf


def scan_bwd(x, dt_raw, A, B, C, dy, *, dh_final=None, dt_bias=None, D=None, h_init=None,
             seq_idx=None, dt_softplus=True, dt_min=0.0, dt_max=float("inf"), nthreads=0,
             lib=None):
    """Gradients of the sequential recurrence (reverse mode, fp64) for a loss
    with gradients dy (b,L,H,P) with respect to y and dh_final (b,H,P,N, or
    None = 0) with respect to the final state.

    Returns a dict of float64 arrays: dx (b,L,H,P), ddt_raw (b,L,H), dA (H),
    dB, dC (b,L,G,N), dD (H), ddt_bias (H), dh_init (b,H,P,N).
    """
    x, dt_raw, A, B, C, dy = map(_f64, (x, dt_raw, A, B, C, dy))
    dt_bias, D, h_init, dh_final = map(_f64, (dt_bias, D, h_init, dh_final))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt_raw.shape == (b, L, H) and B.shape == (b, L, G, N) and C.shape == B.shape
    assert dy.shape == x.shape and A.shape == (H,)
    for st in (h_init, dh_final):
        if st is not None:
            assert st.shape == (b, H, P, N)
    sp = None
    if seq_idx is not None:
        seq_idx = np.ascontiguousarray(np.asarray(seq_idx, dtype=np.int32))
        assert seq_idx.shape == (b, L)
        sp = seq_idx.ctypes.data_as(ctypes.c_void_p)
    out = {"dx": np.empty((b, L, H, P)), "ddt_raw": np.empty((b, L, H)), "dA": np.empty(H),
           "dB": np.empty((b, L, G, N)), "dC": np.empty((b, L, G, N)), "dD": np.empty(H),
           "ddt_bias": np.empty(H), "dh_init": np.empty((b, H, P, N))}
    rc = (lib or _load()).oracle_ssd_scan_bwd(
        b, L, H, P, N, G, _ptr(x), _ptr(dt_raw), _ptr(dt_bias), int(bool(dt_softplus)),
        float(dt_min), float(dt_max), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h_init),
        sp, _ptr(dy), _ptr(dh_final), _ptr(out["dx"]), _ptr(out["ddt_raw"]), _ptr(out["dA"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["ddt_bias"]),
        _ptr(out["dh_init"]), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_ssd_scan_bwd failed with code %d" % rc)
    return out


def step(state, x, dt_raw, A, B, C, *, dt_bias=None, D=None, dt_softplus=True,
         dt_min=0.0, dt_max=float("inf"), lib=None):
    """One decode token: state (b,H,P,N) -> (new_state, y (b,H,P)), float64."""
    s = np.array(state, dtype=np.float64, copy=True, order="C")
    x, dt_raw, A, B, C = map(_f64, (x, dt_raw, A, B, C))
    dt_bias, D = _f64(dt_bias), _f64(D)
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    assert s.shape == (b, H, P, N) and dt_raw.shape == (b, H) and C.shape == B.shape
    y = np.empty((b, H, P), dtype=np.float64)
    rc = (lib or _load()).oracle_ssd_step(
        b, H, P, N, G, _ptr(s), _ptr(x), _ptr(dt_raw), _ptr(dt_bias), int(bool(dt_softplus)),
        float(dt_min), float(dt_max), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(y))
    if rc != 0:
        raise RuntimeError("oracle_ssd_step failed with code %d" % rc)
    return s, y


def rel_l2(a, ref) -> float:
    """||a - ref||_2 / ||ref||_2 in fp64 over all elements."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum((a - ref) ** 2)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
