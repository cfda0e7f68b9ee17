"""MI355X (gfx950) Mamba-2 SSD selective scan: Python binding of libssd.so.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libssd.so`` (built from ``csrc/`` by ``_build.build()``); PyTorch
supplies device memory and the current stream.  There is no CPU or PyTorch
fallback: if the library is missing or fails to load, every call raises.

The operation (RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 1 operator
families 1 and 2, section 3 Figure 2 box [F2]; "Nemotron 3 Nano - JAX
Implementation", Key Components item 1), per row and head:

    dt_t = clamp(softplus(dt_raw_t + dt_bias), dt_min, dt_max)
    h_t  = exp(dt_t A) h_{t-1} + dt_t x_t (outer) B_t       (fp32 state, P x N)
    y_t  = h_t . C_t + D x_t

``chunk_scan_fwd`` computes it for whole sequences as a chunked parallel scan
(prefill / training forward); ``state_update`` advances a decode state by one
token.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = ["chunk_scan_fwd", "state_update", "workspace_bytes", "supported", "segments",
           "SSDError", "library", "library_path", "F32", "BF16"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssd.so")
F32, BF16 = 0, 1

_lib = None


class SSDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        msg = library().ssd_status_string(self.status).decode()
        super().__init__("%s failed: status %d (%s)" % (where, self.status, msg))


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk_size")]


def library_path() -> str:
    return _LIB_PATH


def library():
    """Load libssd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libssd.so not found at %s: build it with "
                               "mamba_ssd_selective_amd._build.build()" % _LIB_PATH)
        # torch's HIP runtime first: the library then binds that same copy
        # (both carry the soname libamdhip64.so.7).  Loaded before torch, it
        # would bind the system copy and torch would add its own, two HIP
        # runtimes in one process, where the library's launches have failed.
        import torch  # noqa: F401
        lib = ctypes.CDLL(_LIB_PATH)
        vp, f, i64, i = ctypes.c_void_p, ctypes.c_float, ctypes.c_int64, ctypes.c_int
        dims_p = ctypes.POINTER(_Dims)
        lib.ssd_abi_version.restype = i
        lib.ssd_status_string.argtypes = [i]
        lib.ssd_status_string.restype = ctypes.c_char_p
        lib.ssd_chunk_scan_workspace_bytes.argtypes = [dims_p, i]
        lib.ssd_chunk_scan_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_chunk_scan_segments.argtypes = [dims_p, i]
        lib.ssd_chunk_scan_segments.restype = i64
        lib.ssd_chunk_scan_supported.argtypes = [i, i64, i64, i64]
        lib.ssd_chunk_scan_supported.restype = i
        lib.ssd_chunk_scan_fwd.argtypes = [dims_p, i, vp, vp, vp, i, f, f, vp, vp, vp, vp, vp,
                                           vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.ssd_chunk_scan_fwd.restype = i
        lib.ssd_chunk_scan_fwd_noalloc.argtypes = [dims_p, i, vp, vp, vp, i, f, f, vp, vp, vp, vp,
                                                   vp, vp, vp, vp, vp]
        lib.ssd_chunk_scan_fwd_noalloc.restype = i
        lib.ssd_chunk_scan_bwd_workspace_bytes.argtypes = [dims_p, i]
        lib.ssd_chunk_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_chunk_scan_bwd.argtypes = [dims_p, i, vp, vp, vp, i, f, f, vp, vp, vp, vp, vp, vp,
                                           vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           ctypes.c_size_t, vp]
        lib.ssd_chunk_scan_bwd.restype = i
        lib.ssd_conv1d_fwd.argtypes = [i64, i64, i64, i64, i64, i, vp, vp, i64, vp, vp, vp, vp, vp,
                                       vp, vp, vp]
        lib.ssd_conv1d_fwd.restype = i
        lib.ssd_conv1d_update.argtypes = [i64, i64, i64, i64, i, vp, vp, i64, vp, vp, vp, vp, vp, vp]
        lib.ssd_conv1d_update.restype = i
        lib.ssd_chunk_scan_cached_workspace_bytes.argtypes = [ctypes.POINTER(_Dims), i]
        lib.ssd_chunk_scan_cached_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_chunk_scan_fwd_cached.argtypes = [ctypes.POINTER(_Dims), i, vp, vp, vp, i, f, f,
                                                  vp, vp, vp, vp, vp, vp, i64, vp, i, i, vp, vp,
                                                  ctypes.c_size_t, vp]
        lib.ssd_chunk_scan_fwd_cached.restype = i
        lib.ssd_chunk_scan_varlen_workspace_bytes.argtypes = [ctypes.POINTER(_Dims), i]
        lib.ssd_chunk_scan_varlen_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_chunk_scan_fwd_varlen.argtypes = [ctypes.POINTER(_Dims), i64, i, vp, vp, vp, i, f,
                                                  f, vp, vp, vp, vp, vp, vp, i64, vp, i, i, vp, vp,
                                                  ctypes.c_size_t, vp]
        lib.ssd_chunk_scan_fwd_varlen.restype = i
        lib.ssd_decode_emulated_workspace_bytes.argtypes = [ctypes.POINTER(_Dims), i]
        lib.ssd_decode_emulated_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_decode_emulated.argtypes = [ctypes.POINTER(_Dims), i, vp, vp, vp, i, f, f, vp, vp,
                                            vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp,
                                            ctypes.c_size_t, vp]
        lib.ssd_decode_emulated.restype = i
        lib.ssd_conv1d_update_cached.argtypes = [i64, i64, i64, i64, i64, i, vp, vp, i64, vp, vp, vp,
                                                 vp, vp, vp, vp]
        lib.ssd_conv1d_update_cached.restype = i
        lib.ssd_gated_rmsnorm.argtypes = [i64, i64, i64, i, vp, vp, vp, f, vp, vp]
        lib.ssd_gated_rmsnorm.restype = i
        lib.ssd_state_update.argtypes = [i64, i64, i64, i64, i64, i, vp, vp, vp, vp, i, f, f,
                                         vp, vp, vp, vp, vp, vp]
        lib.ssd_state_update.restype = i
        lib.ssd_state_update_cached.argtypes = [i64, i64, i64, i64, i64, i64, i, vp, vp, vp, vp, vp,
                                                i, f, f, vp, vp, vp, vp, vp, vp]
        lib.ssd_state_update_cached.restype = i
        lib.ssd_check_seq_idx_host.argtypes = [vp, i64, i64]
        lib.ssd_check_seq_idx_host.restype = i
        lib.ssd_check_seq_idx.argtypes = [vp, i64, i64, vp]
        lib.ssd_check_seq_idx.restype = i
        lib.ssd_set_timing_events.argtypes = [ctypes.POINTER(vp), i, ctypes.POINTER(i)]
        lib.ssd_set_timing_events.restype = None
        if lib.ssd_abi_version() != 1:
            raise RuntimeError("libssd.so ABI version %d, expected 1" % lib.ssd_abi_version())
        _lib = lib
    return _lib


def _io_code(dtype) -> int:
    import torch
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float32:
        return F32
    raise TypeError("x/B/C must be torch.bfloat16 or torch.float32, got %s" % dtype)


def _dims(b, L, H, P, N, G, Q) -> _Dims:
    return _Dims(int(b), int(L), int(H), int(P), int(N), int(G), int(Q))


def workspace_bytes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, io=BF16) -> int:
    d = _dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size)
    return int(library().ssd_chunk_scan_workspace_bytes(ctypes.byref(d), int(io)))


def segments(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, io=BF16) -> int:
    d = _dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size)
    return int(library().ssd_chunk_scan_segments(ctypes.byref(d), int(io)))


def supported(io, headdim, dstate, chunk_size) -> bool:
    return bool(library().ssd_chunk_scan_supported(int(io), int(headdim), int(dstate),
                                                   int(chunk_size)))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if t.device != device:
        raise ValueError("%s: expected device %s, got %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream_handle(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def check_seq_idx(seq_idx):
    """Raise SSDError (SSD_ERR_BAD_SEQ_IDX) if a row of seq_idx (b, L) int32
    decreases.  A host tensor is checked in place; a device tensor is copied
    to the host on the current stream first (which synchronises it)."""
    import torch
    lib = library()
    if seq_idx.dtype != torch.int32 or seq_idx.dim() != 2 or not seq_idx.is_contiguous():
        raise ValueError("seq_idx must be a contiguous (b, L) int32 tensor")
    b, L = seq_idx.shape
    if seq_idx.is_cuda:
        st = lib.ssd_check_seq_idx(_ptr(seq_idx), b, L, _stream_handle(seq_idx.device))
    else:
        st = lib.ssd_check_seq_idx_host(seq_idx.data_ptr() if seq_idx.numel() else None, b, L)
    if st != 0:
        raise SSDError(st, "ssd_check_seq_idx")


def chunk_scan_fwd(x, dt, A, B, C, *, chunk_size: int, D=None, dt_bias=None,
                   initial_states=None, seq_idx=None, dt_softplus: bool = True,
                   dt_limit: Tuple[float, float] = (0.0, math.inf),
                   return_final_states: bool = False, out=None, final_states_out=None,
                   workspace=None, check_seq_idx_order: bool = False):
    """Chunked SSD scan.

    x (b, L, H, P), B/C (b, L, G, N) in bf16 or fp32 (same dtype); dt (b, L, H),
    A/D/dt_bias (H), initial_states (b, H, P, N) fp32; seq_idx (b, L) int32.
    Returns y (b, L, H, P) in x's dtype, and the final fp32 states
    (b, H, P, N) when ``return_final_states``.  ``check_seq_idx_order``: first
    verify that seq_idx never decreases along a row (a device-to-host copy
    and a stream synchronisation; off by default).
    """
    import torch
    lib = library()
    if check_seq_idx_order and seq_idx is not None:
        check_seq_idx(seq_idx)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    io = _io_code(x.dtype)
    f32 = torch.float32
    _check(x, "x", (b, L, H, P), x.dtype, dev)
    _check(B, "B", (b, L, G, N), x.dtype, dev)
    _check(C, "C", (b, L, G, N), x.dtype, dev)
    _check(dt, "dt", (b, L, H), f32, dev)
    _check(A, "A", (H,), f32, dev)
    _check(D, "D", (H,), f32, dev)
    _check(dt_bias, "dt_bias", (H,), f32, dev)
    _check(initial_states, "initial_states", (b, H, P, N), f32, dev)
    _check(seq_idx, "seq_idx", (b, L), torch.int32, dev)
    y = out if out is not None else torch.empty((b, L, H, P), dtype=x.dtype, device=dev)
    _check(y, "out", (b, L, H, P), x.dtype, dev)
    fs = None
    if return_final_states:
        fs = final_states_out if final_states_out is not None else \
            torch.empty((b, H, P, N), dtype=f32, device=dev)
        _check(fs, "final_states_out", (b, H, P, N), f32, dev)
    d = _dims(b, L, H, P, N, G, chunk_size)
    need = int(lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d), io))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssd_chunk_scan_fwd(
        ctypes.byref(d), io, _ptr(x), _ptr(dt), _ptr(dt_bias), int(bool(dt_softplus)),
        float(dt_limit[0]), float(dt_limit[1]), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(initial_states), _ptr(seq_idx), _ptr(y), _ptr(fs), _ptr(workspace), ws_bytes,
        _stream_handle(dev))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd")
    return (y, fs) if return_final_states else y


def cached_workspace_bytes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size,
                           io=BF16) -> int:
    d = _dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size)
    return int(library().ssd_chunk_scan_cached_workspace_bytes(ctypes.byref(d), io))


def chunk_scan_fwd_cached(x, dt, A, B, C, state_cache, state_indices, *, chunk_size: int,
                          seq_lens=None, init_from_cache: bool = True, strict: bool = False,
                          D=None, dt_bias=None,
                          dt_softplus: bool = True,
                          dt_limit: Tuple[float, float] = (0.0, math.inf), out=None,
                          workspace=None):
    """Chunked SSD scan of a batch of prompts on a state cache: row r is one
    sequence of seq_lens[r] real tokens (None: all L; later tokens are
    padding), starting from slot state_indices[r] of ``state_cache``
    (slots, H, P, N) fp32 (zeros unless ``init_from_cache``) and writing its
    final state back to that slot.  An index outside the cache marks a
    padding row.  ``strict`` runs each row as one segment (bitwise the same
    in any batch, continued bit for bit by ``decode_emulated``).  Returns
    y (b, L, H, P); rows past a row's length are not meaningful."""
    import torch
    lib = library()
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    io = _io_code(x.dtype)
    f32 = torch.float32
    _check(x, "x", (b, L, H, P), x.dtype, dev)
    _check(B, "B", (b, L, G, N), x.dtype, dev)
    _check(C, "C", (b, L, G, N), x.dtype, dev)
    _check(dt, "dt", (b, L, H), f32, dev)
    _check(A, "A", (H,), f32, dev)
    _check(D, "D", (H,), f32, dev)
    _check(dt_bias, "dt_bias", (H,), f32, dev)
    rows = state_cache.shape[0]
    _check(state_cache, "state_cache", (rows, H, P, N), f32, dev)
    _check(state_indices, "state_indices", (b,), torch.int32, dev)
    _check(seq_lens, "seq_lens", (b,), torch.int32, dev)
    y = out if out is not None else torch.empty((b, L, H, P), dtype=x.dtype, device=dev)
    _check(y, "out", (b, L, H, P), x.dtype, dev)
    d = _dims(b, L, H, P, N, G, chunk_size)
    need = int(lib.ssd_chunk_scan_cached_workspace_bytes(ctypes.byref(d), io))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssd_chunk_scan_fwd_cached(
        ctypes.byref(d), io, _ptr(x), _ptr(dt), _ptr(dt_bias), int(bool(dt_softplus)),
        float(dt_limit[0]), float(dt_limit[1]), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(seq_lens), _ptr(state_cache), rows, _ptr(state_indices), int(bool(init_from_cache)),
        int(bool(strict)), _ptr(y), _ptr(workspace), ws_bytes, _stream_handle(dev))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd_cached")
    return y


def chunk_scan_fwd_varlen(x, dt, A, B, C, cu_seqlens, state_cache, state_indices, *,
                          chunk_size: int, max_seqlen: Optional[int] = None,
                          init_from_cache: bool = True, strict: bool = False, D=None,
                          dt_bias=None, dt_softplus: bool = True,
                          dt_limit: Tuple[float, float] = (0.0, math.inf), out=None,
                          workspace=None, check_seqlens: bool = False):
    """Packed variable-length prefill: x (T, H, P), dt (T, H), B/C (T, G, N)
    hold the sequences back to back at offsets ``cu_seqlens`` (nseq + 1,
    int32); sequence r is chunked from its own start, begins at slot
    state_indices[r] of ``state_cache`` (zeros unless ``init_from_cache``) and
    leaves its final state there.  Returns y (T, H, P).

    ``max_seqlen`` bounds every sequence's length (the library cuts longer
    ones to it).  None: it is computed from cu_seqlens, which reads the
    offsets back to the host (a synchronisation).  ``check_seqlens``: read
    them back and raise ValueError unless they run from 0 to T without
    decreasing and no sequence is longer than max_seqlen."""
    import torch
    lib = library()
    if max_seqlen is None or check_seqlens:
        cu = cu_seqlens.detach().to("cpu", torch.int64)
        lens = cu[1:] - cu[:-1]
        longest = int(lens.max()) if lens.numel() else 0
        if check_seqlens:
            if cu.numel() == 0 or int(cu[0]) != 0 or int(cu[-1]) != x.shape[0] or \
                    (lens.numel() and int(lens.min()) < 0):
                raise ValueError("cu_seqlens must rise from 0 to the packed token count")
            if max_seqlen is not None and longest > max_seqlen:
                raise ValueError("a sequence of %d tokens is longer than max_seqlen %d"
                                 % (longest, max_seqlen))
        if max_seqlen is None:
            max_seqlen = longest
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    S = cu_seqlens.shape[0] - 1
    dev = x.device
    io = _io_code(x.dtype)
    f32 = torch.float32
    _check(x, "x", (T, H, P), x.dtype, dev)
    _check(dt, "dt", (T, H), f32, dev)
    _check(B, "B", (T, G, N), x.dtype, dev)
    _check(C, "C", (T, G, N), x.dtype, dev)
    _check(A, "A", (H,), f32, dev)
    _check(D, "D", (H,), f32, dev)
    _check(dt_bias, "dt_bias", (H,), f32, dev)
    _check(cu_seqlens, "cu_seqlens", (S + 1,), torch.int32, dev)
    rows = state_cache.shape[0]
    _check(state_cache, "state_cache", (rows, H, P, N), f32, dev)
    _check(state_indices, "state_indices", (S,), torch.int32, dev)
    y = out if out is not None else torch.empty((T, H, P), dtype=x.dtype, device=dev)
    _check(y, "out", (T, H, P), x.dtype, dev)
    d = _dims(S, max_seqlen, H, P, N, G, chunk_size)
    need = int(lib.ssd_chunk_scan_varlen_workspace_bytes(ctypes.byref(d), io))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssd_chunk_scan_fwd_varlen(
        ctypes.byref(d), T, io, _ptr(x), _ptr(dt), _ptr(dt_bias), int(bool(dt_softplus)),
        float(dt_limit[0]), float(dt_limit[1]), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(cu_seqlens), _ptr(state_cache), rows, _ptr(state_indices), int(bool(init_from_cache)),
        int(bool(strict)), _ptr(y), _ptr(workspace), ws_bytes, _stream_handle(dev))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_fwd_varlen")
    return y


def decode_emulated(x, dt, A, B, C, state_cache, chunks, state_indices, positions, *,
                    chunk_size: int, D=None, dt_bias=None, dt_softplus: bool = True,
                    dt_limit: Tuple[float, float] = (0.0, math.inf), out=None, workspace=None):
    """Chunk-emulating decode: one token per row (x (b, H, P), dt (b, H),
    B/C (b, G, N)) at offset positions[r] of the current chunk of slot
    state_indices[r].  ``state_cache`` (slots, H, P, N) fp32 holds each slot's
    chunk-start state and ``chunks`` = (x_chunks (slots, Q, H, P),
    dt_chunks (slots, Q, H), B_chunks, C_chunks (slots, Q, G, N)) the chunk's
    tokens so far; both are updated in place.  Returns y (b, H, P), bitwise
    the chunked prefill's value for each token."""
    import torch
    lib = library()
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    Q = int(chunk_size)
    dev = x.device
    io = _io_code(x.dtype)
    f32 = torch.float32
    xc, dtc, bc, cc = chunks
    rows = state_cache.shape[0]
    _check(x, "x", (b, H, P), x.dtype, dev)
    _check(dt, "dt", (b, H), f32, dev)
    _check(B, "B", (b, G, N), x.dtype, dev)
    _check(C, "C", (b, G, N), x.dtype, dev)
    _check(A, "A", (H,), f32, dev)
    _check(D, "D", (H,), f32, dev)
    _check(dt_bias, "dt_bias", (H,), f32, dev)
    _check(state_cache, "state_cache", (rows, H, P, N), f32, dev)
    _check(xc, "x_chunks", (rows, Q, H, P), x.dtype, dev)
    _check(dtc, "dt_chunks", (rows, Q, H), f32, dev)
    _check(bc, "B_chunks", (rows, Q, G, N), x.dtype, dev)
    _check(cc, "C_chunks", (rows, Q, G, N), x.dtype, dev)
    _check(state_indices, "state_indices", (b,), torch.int32, dev)
    _check(positions, "positions", (b,), torch.int32, dev)
    y = out if out is not None else torch.empty((b, H, P), dtype=x.dtype, device=dev)
    _check(y, "out", (b, H, P), x.dtype, dev)
    d = _dims(b, Q, H, P, N, G, Q)
    need = int(lib.ssd_decode_emulated_workspace_bytes(ctypes.byref(d), io))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssd_decode_emulated(
        ctypes.byref(d), io, _ptr(x), _ptr(dt), _ptr(dt_bias), int(bool(dt_softplus)),
        float(dt_limit[0]), float(dt_limit[1]), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(state_cache), _ptr(xc), _ptr(dtc), _ptr(bc), _ptr(cc), rows, _ptr(state_indices),
        _ptr(positions), _ptr(y), _ptr(workspace), ws_bytes, _stream_handle(dev))
    if st != 0:
        raise SSDError(st, "ssd_decode_emulated")
    return y


def bwd_workspace_bytes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size,
                        io=BF16) -> int:
    d = _dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size)
    return int(library().ssd_chunk_scan_bwd_workspace_bytes(ctypes.byref(d), io))


def chunk_scan_bwd(x, dt, A, B, C, dy, *, chunk_size: int, D=None, dt_bias=None,
                   initial_states=None, seq_idx=None, d_final_states=None,
                   dt_softplus: bool = True, dt_limit: Tuple[float, float] = (0.0, math.inf),
                   workspace=None):
    """Gradients of ``chunk_scan_fwd`` for a loss with gradients ``dy``
    (b, L, H, P, x's dtype) with respect to y and ``d_final_states``
    (b, H, P, N fp32, or None) with respect to the final states.

    Returns a dict: dx (b, L, H, P) and dB, dC (b, L, G, N) in x's dtype;
    ddt (b, L, H), dA, dD, ddt_bias (H), d_initial_states (b, H, P, N) fp32
    (dD only when D is given, ddt_bias only when dt_bias is given).
    """
    import torch
    lib = library()
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    io = _io_code(x.dtype)
    f32 = torch.float32
    _check(x, "x", (b, L, H, P), x.dtype, dev)
    _check(B, "B", (b, L, G, N), x.dtype, dev)
    _check(C, "C", (b, L, G, N), x.dtype, dev)
    _check(dy, "dy", (b, L, H, P), x.dtype, dev)
    _check(dt, "dt", (b, L, H), f32, dev)
    _check(A, "A", (H,), f32, dev)
    _check(D, "D", (H,), f32, dev)
    _check(dt_bias, "dt_bias", (H,), f32, dev)
    _check(initial_states, "initial_states", (b, H, P, N), f32, dev)
    _check(d_final_states, "d_final_states", (b, H, P, N), f32, dev)
    _check(seq_idx, "seq_idx", (b, L), torch.int32, dev)
    g = {"dx": torch.empty((b, L, H, P), dtype=x.dtype, device=dev),
         "ddt": torch.empty((b, L, H), dtype=f32, device=dev),
         "dA": torch.empty((H,), dtype=f32, device=dev),
         "dB": torch.empty((b, L, G, N), dtype=x.dtype, device=dev),
         "dC": torch.empty((b, L, G, N), dtype=x.dtype, device=dev),
         "dD": torch.empty((H,), dtype=f32, device=dev) if D is not None else None,
         "ddt_bias": torch.empty((H,), dtype=f32, device=dev) if dt_bias is not None else None,
         "d_initial_states": torch.empty((b, H, P, N), dtype=f32, device=dev)}
    d = _dims(b, L, H, P, N, G, chunk_size)
    need = int(lib.ssd_chunk_scan_bwd_workspace_bytes(ctypes.byref(d), io))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssd_chunk_scan_bwd(
        ctypes.byref(d), io, _ptr(x), _ptr(dt), _ptr(dt_bias), int(bool(dt_softplus)),
        float(dt_limit[0]), float(dt_limit[1]), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(initial_states), _ptr(seq_idx), _ptr(dy), _ptr(d_final_states), _ptr(g["dx"]),
        _ptr(g["ddt"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
        _ptr(g["ddt_bias"]), _ptr(g["d_initial_states"]), _ptr(workspace), ws_bytes,
        _stream_handle(dev))
    if st != 0:
        raise SSDError(st, "ssd_chunk_scan_bwd")
    return g


def conv1d_fwd(xbc, weight, *, nheads: int, headdim: int, ngroups: int, dstate: int, bias=None,
               conv_state=None, seq_idx=None, return_conv_state: bool = False,
               conv_state_out=None):
    """Causal conv1d (width 4) + bias + SiLU over xbc (b, L, H*P + 2*G*N),
    written as the scan's inputs: returns x (b, L, H, P), B, C (b, L, G, N) in
    xbc's dtype, and the new conv state (b, dim, 3) when ``return_conv_state``
    (``conv_state_out`` may be ``conv_state`` itself: updated in place)."""
    import torch
    lib = library()
    b, L, dim = xbc.shape
    nx, nb = nheads * headdim, ngroups * dstate
    dev = xbc.device
    io = _io_code(xbc.dtype)
    _check(xbc, "xbc", (b, L, dim), xbc.dtype, dev)
    _check(weight, "weight", (dim, 4), torch.float32, dev)
    _check(bias, "bias", (dim,), torch.float32, dev)
    _check(conv_state, "conv_state", (b, dim, 3), xbc.dtype, dev)
    _check(seq_idx, "seq_idx", (b, L), torch.int32, dev)
    x = torch.empty((b, L, nheads, headdim), dtype=xbc.dtype, device=dev)
    Bm = torch.empty((b, L, ngroups, dstate), dtype=xbc.dtype, device=dev)
    Cm = torch.empty((b, L, ngroups, dstate), dtype=xbc.dtype, device=dev)
    st = None
    if return_conv_state:
        st = conv_state_out if conv_state_out is not None else \
            torch.empty((b, dim, 3), dtype=xbc.dtype, device=dev)
        _check(st, "conv_state_out", (b, dim, 3), xbc.dtype, dev)
    rc = lib.ssd_conv1d_fwd(b, L, dim, nx, nb, io, _ptr(xbc), _ptr(weight), 4, _ptr(bias),
                            _ptr(conv_state), _ptr(seq_idx), _ptr(x), _ptr(Bm), _ptr(Cm), _ptr(st),
                            _stream_handle(dev))
    if rc != 0:
        raise SSDError(rc, "ssd_conv1d_fwd")
    return (x, Bm, Cm, st) if return_conv_state else (x, Bm, Cm)


def conv1d_update(xbc, conv_state, weight, *, nheads: int, headdim: int, ngroups: int,
                  dstate: int, bias=None, state_indices=None, out=None):
    """One decode token of the conv: xbc (b, dim); conv_state (b, dim, 3) is
    updated in place.  Returns x (b, H, P), B, C (b, G, N).

    With ``state_indices`` (b,) int32, conv_state is a cache (rows, dim, 3):
    row r reads and updates cache row state_indices[r]; an index outside the
    cache marks a padding row (cache untouched, outputs not written).  ``out``
    optionally gives the (x, B, C) tensors to write."""
    import torch
    lib = library()
    b, dim = xbc.shape
    nx, nb = nheads * headdim, ngroups * dstate
    dev = xbc.device
    io = _io_code(xbc.dtype)
    _check(xbc, "xbc", (b, dim), xbc.dtype, dev)
    rows = conv_state.shape[0] if state_indices is not None else b
    _check(conv_state, "conv_state", (rows, dim, 3), xbc.dtype, dev)
    _check(state_indices, "state_indices", (b,), torch.int32, dev)
    _check(weight, "weight", (dim, 4), torch.float32, dev)
    _check(bias, "bias", (dim,), torch.float32, dev)
    if out is None:
        out = (torch.empty((b, nheads, headdim), dtype=xbc.dtype, device=dev),
               torch.empty((b, ngroups, dstate), dtype=xbc.dtype, device=dev),
               torch.empty((b, ngroups, dstate), dtype=xbc.dtype, device=dev))
    x, Bm, Cm = out
    _check(x, "x", (b, nheads, headdim), xbc.dtype, dev)
    _check(Bm, "B", (b, ngroups, dstate), xbc.dtype, dev)
    _check(Cm, "C", (b, ngroups, dstate), xbc.dtype, dev)
    if state_indices is None:
        rc = lib.ssd_conv1d_update(b, dim, nx, nb, io, _ptr(xbc), _ptr(weight), 4, _ptr(bias),
                                   _ptr(conv_state), _ptr(x), _ptr(Bm), _ptr(Cm),
                                   _stream_handle(dev))
        name = "ssd_conv1d_update"
    else:
        rc = lib.ssd_conv1d_update_cached(b, rows, dim, nx, nb, io, _ptr(xbc), _ptr(weight), 4,
                                          _ptr(bias), _ptr(conv_state), _ptr(state_indices),
                                          _ptr(x), _ptr(Bm), _ptr(Cm), _stream_handle(dev))
        name = "ssd_conv1d_update_cached"
    if rc != 0:
        raise SSDError(rc, name)
    return x, Bm, Cm


def gated_rmsnorm(y, z, weight, *, group: int, eps: float = 1e-6, out=None):
    """norm(y * silu(z)) over groups of ``group`` channels of the last axis,
    times weight (fp32, last-axis size).  y, z of the same shape and dtype."""
    import torch
    lib = library()
    dim = y.shape[-1]
    rows = y.numel() // dim if dim else 0
    dev = y.device
    io = _io_code(y.dtype)
    _check(y, "y", tuple(y.shape), y.dtype, dev)
    _check(z, "z", tuple(y.shape), y.dtype, dev)
    _check(weight, "weight", (dim,), torch.float32, dev)
    o = out if out is not None else torch.empty_like(y)
    _check(o, "out", tuple(y.shape), y.dtype, dev)
    rc = lib.ssd_gated_rmsnorm(rows, dim, group, io, _ptr(y), _ptr(z), _ptr(weight), float(eps),
                               _ptr(o), _stream_handle(dev))
    if rc != 0:
        raise SSDError(rc, "ssd_gated_rmsnorm")
    return o


def state_update(state, x, dt, A, B, C, *, D=None, dt_bias=None, dt_softplus: bool = True,
                 dt_limit: Tuple[float, float] = (0.0, math.inf), out=None, state_indices=None):
    """One decode token: updates ``state`` (b, H, P, N) fp32 in place and
    returns y (b, H, P) in x's dtype.  x (b, H, P), dt (b, H), B/C (b, G, N).

    With ``state_indices`` (b,) int32, state is a cache (slots, H, P, N): row
    r reads and updates slot state_indices[r]; an index outside the cache
    marks a padding row (slot untouched, its y rows not written)."""
    import torch
    lib = library()
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dev = x.device
    io = _io_code(x.dtype)
    f32 = torch.float32
    rows = state.shape[0] if state_indices is not None else b
    _check(state, "state", (rows, H, P, N), f32, dev)
    _check(state_indices, "state_indices", (b,), torch.int32, dev)
    _check(B, "B", (b, G, N), x.dtype, dev)
    _check(C, "C", (b, G, N), x.dtype, dev)
    _check(dt, "dt", (b, H), f32, dev)
    _check(A, "A", (H,), f32, dev)
    _check(D, "D", (H,), f32, dev)
    _check(dt_bias, "dt_bias", (H,), f32, dev)
    y = out if out is not None else torch.empty((b, H, P), dtype=x.dtype, device=dev)
    _check(y, "out", (b, H, P), x.dtype, dev)
    if state_indices is None:
        st = lib.ssd_state_update(b, H, P, N, G, io, _ptr(state), _ptr(x), _ptr(dt),
                                  _ptr(dt_bias), int(bool(dt_softplus)), float(dt_limit[0]),
                                  float(dt_limit[1]), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(y),
                                  _stream_handle(dev))
        name = "ssd_state_update"
    else:
        st = lib.ssd_state_update_cached(b, rows, H, P, N, G, io, _ptr(state),
                                         _ptr(state_indices), _ptr(x), _ptr(dt), _ptr(dt_bias),
                                         int(bool(dt_softplus)), float(dt_limit[0]),
                                         float(dt_limit[1]), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                         _ptr(y), _stream_handle(dev))
        name = "ssd_state_update_cached"
    if st != 0:
        raise SSDError(st, name)
    return y
