"""C-ABI checks that need no GPU: the library loads, exports every function
include/ssd.h declares, and rejects bad arguments before launching anything
(fail closed: RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 4.1 WS1 rules
and section 7 "Fail closed").  Only calls that validation rejects, or that
return before any launch (batch = 0), are made here."""
import ctypes
import math
import os
import re

import pytest

import mamba_ssd_selective_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, NULL_ARG, BAD_SHAPE, BAD_DTYPE, UNSUPPORTED, WORKSPACE, BAD_ARG, ALIAS, HIP = range(9)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.library_path()):
        pytest.fail("libssd.so is not built; run __graft_entry__.build()")
    return ssd.library()


def test_exports_every_declared_symbol(lib):
    text = open(HEADER).read()
    names = set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text))
    assert {"ssd_chunk_scan_fwd", "ssd_state_update", "ssd_chunk_scan_workspace_bytes",
            "ssd_status_string", "ssd_abi_version"} <= names
    raw = ctypes.CDLL(ssd.library_path())
    for n in sorted(names):
        assert hasattr(raw, n), "libssd.so does not export %s" % n


def test_one_hip_runtime_when_the_library_loads_first():
    # the binding loads torch's HIP runtime ahead of the library, so that the
    # library binds that copy (same soname) and not the system one beside it
    import subprocess
    import sys
    code = ("import mamba_ssd_selective_amd as s; s.library(); import torch; "
            "print(len({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    env = dict(os.environ, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_version_and_status_strings(lib):
    assert lib.ssd_abi_version() == 1
    for s in range(11):
        assert lib.ssd_status_string(s) and b"unknown" not in lib.ssd_status_string(s)
    assert b"unknown" in lib.ssd_status_string(99)


def test_supported_set(lib):
    assert ssd.supported(ssd.BF16, 64, 128, 128)
    assert ssd.supported(ssd.BF16, 64, 128, 256)
    assert ssd.supported(ssd.F32, 16, 16, 64)
    for io, P, N, Q in ((ssd.BF16, 64, 256, 64), (ssd.BF16, 64, 256, 128), (ssd.BF16, 128, 128, 128),
                        (ssd.BF16, 32, 128, 128), (ssd.BF16, 64, 128, 32), (ssd.BF16, 64, 32, 64),
                        (ssd.F32, 64, 64, 64), (ssd.F32, 64, 64, 128), (ssd.F32, 128, 128, 64),
                        (ssd.F32, 64, 256, 64)):
        assert ssd.supported(io, P, N, Q), (io, P, N, Q)
    assert not ssd.supported(ssd.F32, 128, 128, 128)   # its tiles do not fit the LDS
    assert not ssd.supported(ssd.BF16, 48, 128, 128)
    assert not ssd.supported(ssd.BF16, 64, 128, 100)
    assert not ssd.supported(5, 64, 128, 128)


def test_workspace_and_segments(lib):
    # one 8192-token row, 64 heads: 64 chunks of 128 -> 4 segments of 16 chunks (256 workgroups)
    ws = ssd.workspace_bytes(1, 8192, 64, 64, 128, 8, 128)
    # chunk metadata (cs, dt, weights: fp32 per row, head, token), C.B^T tiles
    # (lower-triangular 16x16 bf16 tiles in 20 pairs of 64 lanes x 8 elements
    # per row, chunk, group), the C rows in the output kernel's operand order
    # (bf16 Q x N per row, chunk, group), segment states (fp32 P x N per row,
    # head, segment) and segment multipliers, and room for the final states
    # (fp32 P x N per row, head) for calls whose final states overwrite their
    # initial states
    meta = 3 * 64 * 8192 * 4
    tiles = 64 * 8 * 20 * 512 * 2
    cops = 64 * 8 * 128 * 128 * 2
    seg = 64 * 4 * 64 * 128 * 4 + 256 * math.ceil(64 * 4 * 4 / 256)
    fin = 64 * 64 * 128 * 4
    assert ws == meta + tiles + cops + seg + fin
    assert ssd.segments(1, 8192, 64, 64, 128, 8, 128) == 4
    # enough rows x heads: one segment, no segment scratch
    assert ssd.segments(64, 4096, 64, 64, 128, 8, 128) == 1
    assert ssd.workspace_bytes(64, 4096, 64, 64, 128, 8, 128) == (
        3 * 64 * 64 * 4096 * 4 + 64 * 32 * 8 * 20 * 512 * 2 + 64 * 32 * 8 * 128 * 128 * 2)
    # ragged L: 3 chunks, one segment each
    assert ssd.segments(1, 300, 64, 64, 128, 8, 128) == 3
    assert ssd.workspace_bytes(1, 0, 64, 64, 128, 8, 128) == 0
    assert ssd.workspace_bytes(1, 128, 64, 48, 128, 8, 128) == 0  # unsupported


class _Buf:
    """Fake, never-dereferenced device addresses, 256-byte aligned and far apart."""

    def __init__(self):
        self.next = 0x10000000

    def __call__(self, nbytes=1 << 24):
        a = self.next
        self.next += (nbytes + (1 << 24)) // 256 * 256
        return a


def _scan_call(lib, dims=(1, 256, 4, 16, 16, 1, 64), io=ssd.F32, **over):
    buf = _Buf()
    args = dict(x=buf(), dt=buf(), dt_bias=None, softplus=1, lo=0.0, hi=math.inf, A=buf(),
                B=buf(), C=buf(), D=None, init=None, seq=None, y=buf(), final=None,
                ws=buf(), ws_bytes=1 << 30)
    args.update(over)
    d = ssd._Dims(*dims) if dims is not None else None
    return lib.ssd_chunk_scan_fwd(
        ctypes.byref(d) if d is not None else None, io, args["x"], args["dt"], args["dt_bias"],
        args["softplus"], args["lo"], args["hi"], args["A"], args["B"], args["C"], args["D"],
        args["init"], args["seq"], args["y"], args["final"], args["ws"], args["ws_bytes"], None)


def test_scan_rejects_bad_arguments(lib):
    assert _scan_call(lib, dims=None) == NULL_ARG
    assert _scan_call(lib, io=7) == BAD_DTYPE
    assert _scan_call(lib, dims=(1, 256, 6, 16, 16, 4, 64)) == BAD_SHAPE   # H % G
    assert _scan_call(lib, dims=(-1, 256, 4, 16, 16, 1, 64)) == BAD_SHAPE
    assert _scan_call(lib, dims=(1, 256, 4, 16, 16, 1, 0)) == BAD_SHAPE
    assert _scan_call(lib, dims=(1, 256, 4, 24, 16, 1, 64)) == UNSUPPORTED
    assert _scan_call(lib, dims=(1, 256, 4, 16, 16, 1, 256)) == UNSUPPORTED  # f32, Q=256
    assert _scan_call(lib, x=None) == NULL_ARG
    assert _scan_call(lib, A=None) == NULL_ARG
    assert _scan_call(lib, y=None) == NULL_ARG
    assert _scan_call(lib, dims=(1, 1024, 4, 16, 16, 1, 64), ws=None) == WORKSPACE
    assert _scan_call(lib, dims=(1, 1024, 4, 16, 16, 1, 64), ws_bytes=16) == WORKSPACE
    # not 256-byte aligned
    assert _scan_call(lib, dims=(1, 1024, 4, 16, 16, 1, 64), ws=0x70000010) == WORKSPACE
    assert _scan_call(lib, lo=1.0, hi=0.5) == BAD_ARG
    assert _scan_call(lib, lo=float("nan")) == BAD_ARG
    assert _scan_call(lib, x=0x70000004) == BAD_ARG  # not 16-byte aligned


def test_scan_rejects_aliasing(lib):
    buf = _Buf()
    x = buf()
    assert _scan_call(lib, x=x, y=x + 1024) == ALIAS          # y overlaps x
    st = buf()
    assert _scan_call(lib, init=st, final=st + 256) == ALIAS  # partial overlap
    w = buf()
    assert _scan_call(lib, dims=(1, 1024, 4, 16, 16, 1, 64), ws=w, y=w) == ALIAS
    assert _scan_call(lib, final=x) == ALIAS


def test_scan_empty_batch_launches_nothing(lib):
    # batch = 0 passes validation and returns before any HIP call
    assert _scan_call(lib, dims=(0, 256, 4, 16, 16, 1, 64), x=None, y=None) == OK


def _step_call(lib, b=2, H=4, P=16, N=16, G=1, io=ssd.F32, **over):
    buf = _Buf()
    a = dict(state=buf(), x=buf(), dt=buf(), bias=None, sp=1, lo=0.0, hi=math.inf, A=buf(),
             B=buf(), C=buf(), D=None, y=buf())
    a.update(over)
    return lib.ssd_state_update(b, H, P, N, G, io, a["state"], a["x"], a["dt"], a["bias"],
                                a["sp"], a["lo"], a["hi"], a["A"], a["B"], a["C"], a["D"],
                                a["y"], None)


def test_state_update_rejects_bad_arguments(lib):
    assert _step_call(lib, io=3) == BAD_DTYPE
    assert _step_call(lib, H=6, G=4) == BAD_SHAPE
    assert _step_call(lib, N=48) == UNSUPPORTED
    assert _step_call(lib, state=None) == NULL_ARG
    assert _step_call(lib, lo=2.0, hi=1.0) == BAD_ARG
    assert _step_call(lib, state=0x70000008) == BAD_ARG
    buf = _Buf()
    s = buf()
    assert _step_call(lib, state=s, y=s + 64) == ALIAS
    assert _step_call(lib, b=0) == OK


def _cached_step_call(lib, b=2, rows=1000, H=4, P=16, N=16, G=1, io=ssd.F32, **over):
    buf = _Buf()
    a = dict(state=buf(), idx=buf(), x=buf(), dt=buf(), bias=None, sp=1, lo=0.0, hi=math.inf,
             A=buf(), B=buf(), C=buf(), D=None, y=buf())
    a.update(over)
    return lib.ssd_state_update_cached(b, rows, H, P, N, G, io, a["state"], a["idx"], a["x"],
                                       a["dt"], a["bias"], a["sp"], a["lo"], a["hi"], a["A"],
                                       a["B"], a["C"], a["D"], a["y"], None)


def test_cached_state_update_rejects_bad_arguments(lib):
    assert _cached_step_call(lib, idx=None) == NULL_ARG
    assert _cached_step_call(lib, rows=-1) == BAD_SHAPE
    assert _cached_step_call(lib, rows=1 << 31) == BAD_SHAPE
    assert _cached_step_call(lib, rows=(1 << 30), H=1 << 16, P=1 << 10) == BAD_SHAPE  # bytes > 2^62
    assert _cached_step_call(lib, N=48) == UNSUPPORTED
    buf = _Buf()
    s = buf()
    # the cache spans all its rows (1000 x 4 KiB), not the batch's two
    assert _cached_step_call(lib, state=s, y=s + 2 * 1024 * 1024) == ALIAS
    assert _cached_step_call(lib, state=s, idx=s + 4096) == ALIAS
    y = buf()
    assert _cached_step_call(lib, idx=y, y=y) == ALIAS
    assert _cached_step_call(lib, b=0, idx=None) == OK


def _cached_conv_call(lib, b=2, rows=1000, nx=64, nb=32, io=ssd.BF16, **over):
    buf = _Buf()
    a = dict(xbc=buf(), w=buf(), bias=None, st=buf(), idx=buf(), xo=buf(), bo=buf(), co=buf())
    a.update(over)
    return lib.ssd_conv1d_update_cached(b, rows, nx + 2 * nb, nx, nb, io, a["xbc"], a["w"], 4,
                                        a["bias"], a["st"], a["idx"], a["xo"], a["bo"], a["co"],
                                        None)


def test_cached_conv_update_rejects_bad_arguments(lib):
    assert _cached_conv_call(lib, idx=None) == NULL_ARG
    assert _cached_conv_call(lib, rows=-1) == BAD_SHAPE
    assert _cached_conv_call(lib, rows=(1 << 31) + 1) == BAD_SHAPE
    assert _cached_conv_call(lib, nx=60, nb=34) == UNSUPPORTED
    buf = _Buf()
    s = buf()
    # 1000 rows x 128 channels x 3 bf16 = 768 KB of cache
    assert _cached_conv_call(lib, st=s, xo=s + 512 * 1024) == ALIAS
    assert _cached_conv_call(lib, st=s, idx=s + 256) == ALIAS
    assert _cached_conv_call(lib, b=0, idx=None) == OK


def test_cached_prefill_workspace_and_rejections(lib):
    # the scan's workspace, then the gathered states (fp32 P x N per row, head)
    plain = ssd.workspace_bytes(2, 300, 8, 64, 128, 2, 128)
    assert ssd.cached_workspace_bytes(2, 300, 8, 64, 128, 2, 128) == plain + 2 * 8 * 64 * 128 * 4
    assert ssd.cached_workspace_bytes(2, 0, 8, 64, 128, 2, 128) == 0
    buf = _Buf()

    def call(dims=(2, 300, 8, 64, 128, 2, 128), rows=16, **over):
        a = dict(x=buf(), dt=buf(), A=buf(), B=buf(), C=buf(), lens=None, cache=buf(1 << 26),
                 idx=buf(), y=buf(), ws=buf(1 << 23), ws_bytes=1 << 23, lo=0.0, hi=math.inf)
        a.update(over)
        d = ssd._Dims(*dims)
        return lib.ssd_chunk_scan_fwd_cached(
            ctypes.byref(d), ssd.BF16, a["x"], a["dt"], None, 1, a["lo"], a["hi"], a["A"], a["B"],
            a["C"], None, a["lens"], a["cache"], rows, a["idx"], 1, 0, a["y"], a["ws"],
            a["ws_bytes"], None)

    assert call(idx=None) == NULL_ARG
    assert call(cache=None) == NULL_ARG
    assert call(rows=-1) == BAD_SHAPE
    assert call(rows=1 << 31) == BAD_SHAPE
    assert call(cache=0x70000008) == BAD_ARG
    assert call(lo=1.0, hi=0.0) == BAD_ARG
    assert call(ws=None) == WORKSPACE
    assert call(ws_bytes=1 << 20) == WORKSPACE
    assert call(dims=(2, 300, 8, 64, 96, 2, 128)) == UNSUPPORTED
    c = buf(1 << 26)
    assert call(cache=c, y=c + 4096) == ALIAS              # y over the cache
    assert call(cache=c, idx=c + (4 << 20) - 64) == ALIAS   # indices inside the last slot (16 x 256 KiB)
    w = buf(1 << 23)
    assert call(ws=w, y=w + 4096) == ALIAS                 # y over the workspace
    assert call(dims=(0, 300, 8, 64, 128, 2, 128), idx=None, cache=None) == OK
    assert call(dims=(2, 0, 8, 64, 128, 2, 128), ws=None) == OK   # nothing to scan


def test_emulated_decode_workspace_and_rejections(lib):
    d = (4, 128, 64, 64, 128, 8, 128)
    need = ssd.library().ssd_decode_emulated_workspace_bytes(ctypes.byref(ssd._Dims(*d)), ssd.BF16)
    # the one-chunk scan's workspace (the slots and new tokens are read in place)
    scan = ssd.workspace_bytes(*d)
    al = lambda v: (v + 255) // 256 * 256
    assert need == al(scan)
    buf = _Buf()

    def call(dims=d, rows=8, **over):
        a = dict(x=buf(), dt=buf(), A=buf(), B=buf(), C=buf(), st=buf(1 << 26), xc=buf(1 << 28),
                 dtc=buf(), bc=buf(1 << 26), cc=buf(1 << 26), idx=buf(), pos=buf(), y=buf(),
                 ws=buf(1 << 26), ws_bytes=1 << 26)
        a.update(over)
        return lib.ssd_decode_emulated(
            ctypes.byref(ssd._Dims(*dims)), ssd.BF16, a["x"], a["dt"], None, 1, 0.0, math.inf, a["A"],
            a["B"], a["C"], None, a["st"], a["xc"], a["dtc"], a["bc"], a["cc"], rows, a["idx"],
            a["pos"], a["y"], a["ws"], a["ws_bytes"], None)

    assert call(dims=(4, 256, 64, 64, 128, 8, 128)) == BAD_SHAPE   # seqlen must be one chunk
    assert call(dims=(4, 128, 64, 64, 96, 8, 128)) == UNSUPPORTED
    assert call(rows=-1) == BAD_SHAPE
    assert call(xc=None) == NULL_ARG
    assert call(pos=None) == NULL_ARG
    assert call(st=0x70000008) == BAD_ARG
    assert call(xc=buf(1 << 28) + 8) == BAD_ARG   # the scan reads the chunk buffers: 16-byte aligned
    assert call(ws=None) == WORKSPACE
    assert call(ws_bytes=1 << 20) == WORKSPACE
    s = buf(1 << 26)
    assert call(st=s, y=s + 4096) == ALIAS                   # y inside the state cache
    x = buf(1 << 28)
    assert call(xc=x, bc=x + (1 << 20)) == ALIAS            # two caches overlap
    w = buf(1 << 26)
    assert call(ws=w, y=w + 1024) == ALIAS                   # y over the workspace
    assert call(dims=(0, 128, 64, 64, 128, 8, 128), x=None, xc=None) == OK


def test_varlen_prefill_workspace_and_rejections(lib):
    d = ssd._Dims(3, 300, 8, 64, 128, 2, 128)
    need = lib.ssd_chunk_scan_varlen_workspace_bytes(ctypes.byref(d), ssd.BF16)
    # the packed rows are read in place: the cached prefill's workspace
    assert need == ssd.cached_workspace_bytes(3, 300, 8, 64, 128, 2, 128)
    buf = _Buf()

    def call(dims=(3, 300, 8, 64, 128, 2, 128), T=500, **over):
        a = dict(x=buf(), dt=buf(), A=buf(), B=buf(), C=buf(), cu=buf(), st=buf(1 << 26), idx=buf(),
                 y=buf(), ws=buf(1 << 26), ws_bytes=1 << 26)
        a.update(over)
        return lib.ssd_chunk_scan_fwd_varlen(
            ctypes.byref(ssd._Dims(*dims)), T, ssd.BF16, a["x"], a["dt"], None, 1, 0.0, math.inf,
            a["A"], a["B"], a["C"], None, a["cu"], a["st"], 16, a["idx"], 1, 0, a["y"], a["ws"],
            a["ws_bytes"], None)

    assert call(T=-1) == BAD_SHAPE
    assert call(cu=None) == NULL_ARG
    assert call(st=None) == NULL_ARG        # before the packing copy is launched
    assert call(idx=None) == NULL_ARG
    assert call(st=0x70000008) == BAD_ARG
    assert call(ws=None) == WORKSPACE
    assert call(ws_bytes=1 << 20) == WORKSPACE
    assert call(x=0x70000008) == BAD_ARG
    assert call(dims=(3, 300, 8, 64, 96, 2, 128)) == UNSUPPORTED
    x = buf()
    assert call(x=x, y=x + 4096) == ALIAS
    s = buf(1 << 26)
    assert call(st=s, dt=s + 64) == ALIAS
    assert call(dims=(0, 300, 8, 64, 128, 2, 128)) == OK


# ---------------------------------------------------------- gradients, mixer


def test_bwd_workspace_bytes(lib):
    # metadata (3 x Q fp32 per row, head, chunk), the state before and the
    # gradient after every chunk (bf16 P x N each), per-chunk sums (3 fp32)
    b, L, H, G = 1, 8192, 64, 8
    nc = 64
    meta = b * H * nc * 128 * 3 * 4
    states = b * H * nc * 64 * 128 * 2
    parts = 256 * math.ceil(b * H * nc * 3 * 4 / 256)
    # 2 x 64 walks, cut into segments of 16 chunks: end states (fp32 P x N) and decay products
    segs = 2 * b * H * 4
    seg = segs * 64 * 128 * 4 + 256 * math.ceil(segs * 4 / 256)
    assert ssd.bwd_workspace_bytes(b, L, H, 64, 128, G, 128) == meta + 2 * states + parts + seg
    # segments fixed in chunks, whatever the batch: four rows, four times the bytes
    assert ssd.bwd_workspace_bytes(4, L, H, 64, 128, G, 128) == 4 * (meta + 2 * states + parts + seg)
    # up to 16 chunks: one segment, no segment scratch
    assert ssd.bwd_workspace_bytes(1, 2048, H, 64, 128, G, 128) == (meta + 2 * states + parts) // 4
    assert ssd.bwd_workspace_bytes(1, 0, H, 64, 128, G, 128) == 0
    # chunk 64 and 256 run as 128-token chunks: the same workspace
    assert ssd.bwd_workspace_bytes(1, 8192, H, 64, 128, G, 64) == ssd.bwd_workspace_bytes(1, 8192, H, 64, 128, G, 128)
    assert ssd.bwd_workspace_bytes(1, 8192, H, 64, 128, G, 256) == ssd.bwd_workspace_bytes(1, 8192, H, 64, 128, G, 128)
    assert ssd.bwd_workspace_bytes(1, 128, H, 64, 128, G, 32) == 0   # not a compiled chunk
    assert ssd.bwd_workspace_bytes(1, 128, H, 64, 64, G, 64) > 0     # N 64
    assert ssd.bwd_workspace_bytes(1, 128, H, 64, 32, G, 64) == 0    # N 32: not built
    assert ssd.bwd_workspace_bytes(1, 128, H, 64, 128, G, 128, io=ssd.F32) == 0   # fp32: not built


def _bwd_call(lib, dims=(1, 256, 4, 64, 128, 1, 128), io=ssd.BF16, **over):
    buf = _Buf()
    args = dict(x=buf(), dt=buf(), dt_bias=None, softplus=1, lo=0.0, hi=math.inf, A=buf(), B=buf(),
                C=buf(), D=None, init=None, seq=None, dy=buf(), dfin=None, dx=buf(), ddt=buf(),
                dA=buf(), dB=buf(), dC=buf(), dD=None, dbias=None, dinit=None, ws=buf(1 << 28),
                ws_bytes=1 << 28)
    args.update(over)
    d = ssd._Dims(*dims)
    return lib.ssd_chunk_scan_bwd(
        ctypes.byref(d), io, args["x"], args["dt"], args["dt_bias"], args["softplus"], args["lo"],
        args["hi"], args["A"], args["B"], args["C"], args["D"], args["init"], args["seq"], args["dy"],
        args["dfin"], args["dx"], args["ddt"], args["dA"], args["dB"], args["dC"], args["dD"],
        args["dbias"], args["dinit"], args["ws"], args["ws_bytes"], None)


def test_bwd_rejects_bad_arguments(lib):
    assert _bwd_call(lib, io=ssd.F32) == UNSUPPORTED
    assert _bwd_call(lib, dims=(1, 256, 4, 64, 32, 1, 128)) == UNSUPPORTED
    assert _bwd_call(lib, dims=(1, 256, 4, 64, 128, 1, 32)) == UNSUPPORTED
    assert _bwd_call(lib, dims=(1, 256, 6, 64, 128, 4, 128)) == BAD_SHAPE   # H % G
    assert _bwd_call(lib, dy=None) == NULL_ARG
    assert _bwd_call(lib, dA=None) == NULL_ARG
    assert _bwd_call(lib, ws=None) == WORKSPACE
    assert _bwd_call(lib, ws_bytes=16) == WORKSPACE
    assert _bwd_call(lib, lo=1.0, hi=0.5) == BAD_ARG
    assert _bwd_call(lib, dx=0x70000008) == BAD_ARG   # not 16-byte aligned
    buf = _Buf()
    x = buf()
    assert _bwd_call(lib, x=x, dx=x + 4096) == ALIAS   # an output over an input
    o = buf()
    assert _bwd_call(lib, dB=o, dC=o + 64) == ALIAS    # two outputs overlap
    w = buf(1 << 28)
    assert _bwd_call(lib, ws=w, ddt=w + 4096) == ALIAS  # an output over the workspace


def _conv_call(lib, b=1, L=64, nx=64, nb=32, io=ssd.BF16, width=4, dim=None, **over):
    """Every call here fails validation (or has nothing to do) before any launch."""
    buf = _Buf()
    args = dict(xbc=buf(), w=buf(), bias=None, sin=None, seq=None, xo=buf(), bo=buf(), co=buf(),
                sout=None)
    args.update(over)
    return lib.ssd_conv1d_fwd(b, L, nx + 2 * nb if dim is None else dim, nx, nb, io, args["xbc"],
                              args["w"], width, args["bias"], args["sin"], args["seq"], args["xo"],
                              args["bo"], args["co"], args["sout"], None)


def test_conv_rejects_bad_arguments(lib):
    assert _conv_call(lib, width=3) == UNSUPPORTED
    assert _conv_call(lib, nx=60, nb=34) == UNSUPPORTED          # not multiples of 8
    assert _conv_call(lib, io=7) == BAD_DTYPE
    assert _conv_call(lib, dim=100) == BAD_SHAPE                  # dim != nx + 2 nb
    assert _conv_call(lib, w=None) == NULL_ARG
    assert _conv_call(lib, xo=None) == NULL_ARG
    assert _conv_call(lib, xbc=0x70000002) == BAD_ARG
    buf = _Buf()
    x = buf()
    assert _conv_call(lib, xbc=x, co=x + 512) == ALIAS
    s = buf()
    assert _conv_call(lib, sin=s, sout=s + 2) == ALIAS            # partial overlap (in place is allowed)
    assert _conv_call(lib, b=0) == OK                             # nothing to launch


def test_gated_norm_rejects_bad_arguments(lib):
    buf = _Buf()

    def call(rows=8, dim=1024, group=512, io=ssd.BF16, eps=1e-6, **over):
        a = dict(y=buf(), z=buf(), w=buf(), out=buf())
        a.update(over)
        return lib.ssd_gated_rmsnorm(rows, dim, group, io, a["y"], a["z"], a["w"], eps, a["out"], None)

    assert call(dim=1200, group=12) == UNSUPPORTED      # divides dim, but not a multiple of 8
    assert call(group=8192, dim=8192) == UNSUPPORTED
    assert call(dim=1000, group=512) == BAD_SHAPE
    assert call(eps=-1.0) == BAD_ARG
    assert call(eps=float("inf")) == BAD_ARG
    assert call(w=None) == NULL_ARG
    y = buf()
    assert call(y=y, out=y) == ALIAS
    assert call(rows=0) == OK


def test_seq_idx_order_check_on_the_host(lib):
    import numpy as np
    ok = np.array([[0, 0, 1, 1, 5], [2, 2, 2, 3, 3]], dtype=np.int32)
    bad = ok.copy()
    bad[1, 3] = 1  # decreases inside row 1
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert lib.ssd_check_seq_idx_host(ptr(ok), 2, 5) == OK
    assert lib.ssd_check_seq_idx_host(ptr(bad), 2, 5) == 10  # SSD_ERR_BAD_SEQ_IDX
    # a decrease across rows is allowed (rows are independent)
    assert lib.ssd_check_seq_idx_host(ptr(np.array([[4, 5], [0, 1]], dtype=np.int32)), 2, 2) == OK
    assert lib.ssd_check_seq_idx_host(None, 2, 5) == NULL_ARG
    assert lib.ssd_check_seq_idx_host(None, 0, 5) == OK
    assert lib.ssd_check_seq_idx_host(ptr(ok), -1, 5) == BAD_SHAPE
    import torch
    ssd.check_seq_idx(torch.from_numpy(ok))
    with pytest.raises(ssd.SSDError):
        ssd.check_seq_idx(torch.from_numpy(bad))


def test_varlen_seqlen_checks_on_the_host(lib):
    """check_seqlens reads cu_seqlens back and rejects offsets that decrease,
    that do not end at the token count, or a sequence longer than max_seqlen,
    before anything is launched."""
    import torch
    T, H, P, N, G = 10, 2, 64, 128, 1
    x = torch.zeros(T, H, P)
    dt = torch.zeros(T, H)
    B = torch.zeros(T, G, N)
    cache = torch.zeros(3, H, P, N)
    idx = torch.zeros(3, dtype=torch.int32)

    def call(cu, max_seqlen):
        ssd.chunk_scan_fwd_varlen(x, dt, torch.zeros(H), B, B, torch.tensor(cu, dtype=torch.int32),
                                  cache, idx[:len(cu) - 1], chunk_size=64, max_seqlen=max_seqlen,
                                  check_seqlens=True)

    with pytest.raises(ValueError):
        call([0, 4, 3, 10], 8)      # decreases
    with pytest.raises(ValueError):
        call([0, 4, 9], 8)          # ends before T
    with pytest.raises(ValueError):
        call([0, 4, 10], 5)         # a sequence of 6 tokens
