"""Thin ctypes binding of libsmla.so (the C ABI in include/smla.h).

Argument marshalling only: torch tensors -> device pointers, the current HIP
stream -> a stream handle, C status codes -> exceptions.  Every computation runs
in the library's HIP kernels; there is no fallback path.  If the library is
missing, every call raises.

Function names follow the C entry points: smla_fwd, smla_bwd, smla_bwd_phased,
smla_bwd_noalloc, smla_delta, smla_dq, smla_interm, smla_build_csr, smla_gather,
smla_dsink, and the has_pe=True variant smla_fwd_pe, smla_bwd_pe.  Above them:
sparse_mla_bwd_dsv4 (the backward under the page's call form), sparse_mla /
SparseMLA (a torch.autograd.Function whose forward is smla_fwd and whose
backward is smla_bwd) and sparse_mla_pe / SparseMLAPE (the same over
smla_fwd_pe / smla_bwd_pe).
"""
from __future__ import annotations

import collections
import ctypes
import math
import os
import threading

import torch

D = 512
DPE = 64   # positional part of the has_pe=True variant
_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsmla.so")

_lib = None
_lib_lock = threading.Lock()

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
_U = ctypes.c_uint32

_SIGNATURES = {
    "smla_status_string": ([_I], ctypes.c_char_p),
    "smla_fwd": ([_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P], _I),
    "smla_bwd_workspace_bytes": ([_I, _I, _I, _I, _U], _Z),
    "smla_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _U, _P, _P, _P, _P, _P, _Z, _P], _I),
    "smla_bwd_timed": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _U, _P, _P, _P, _P, _P, _Z,
                        _P, _P], _I),
    "smla_bwd_phased_workspace_bytes": ([_I, _I, _I, _I, _I, _U], _Z),
    "smla_bwd_phased": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _U, _I, _P, _P, _P, _P, _P,
                         _Z, _P], _I),
    "smla_bwd_noalloc": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _U, _P, _P, _P, _P, _P], _I),
    "smla_delta": ([_P, _P, _P, _I, _I, _P, _P], _I),
    "smla_dq": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P], _I),
    "smla_interm": ([_P, _P, _P, _P, _I, _I, _I, _I, _P, _P], _I),
    "smla_csr_workspace_bytes": ([_I, _I, _I], _Z),
    "smla_build_csr": ([_P, _I, _I, _I, _P, _P, _P, _P, _Z, _P], _I),
    "smla_gather_workspace_bytes": ([_I, _I, _I], _Z),
    "smla_gather": ([_P, _P, _P, _I, _I, _I, _P, _P, _Z, _P], _I),
    "smla_dsp_bytes": ([_I, _I, _I], _Z),
    "smla_dsink_workspace_bytes": ([_I, _I], _Z),
    "smla_dsink": ([_P, _P, _P, _I, _I, _P, _P, _Z, _P], _I),
    "smla_fwd_pe": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P], _I),
    "smla_bwd_pe_workspace_bytes": ([_I, _I, _I, _I, _U], _Z),
    "smla_bwd_pe": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _U, _P, _P, _P, _P, _P, _P,
                     _P, _Z, _P], _I),
}
EXPORTED = tuple(_SIGNATURES)


class SmlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


def lib():
    """Load libsmla.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m sparse_mla_attention_smla_amd.build`")
                h = ctypes.CDLL(LIB_PATH)
                for name, (args, res) in _SIGNATURES.items():
                    f = getattr(h, name)
                    f.argtypes = args
                    f.restype = res
                _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().smla_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise SmlaError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None, device=None):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _workspace(ws, name, device, need=None):
    """Check a caller-given workspace (contiguous uint8 on `device`, at least
    `need` bytes when given); returns its size in bytes, which is what the C
    entry point is told (so that its own size check sees the real buffer)."""
    _need(ws, name, torch.uint8, device=device)
    n = ws.numel() * ws.element_size()
    if need is not None and n < need:
        raise ValueError(f"{name} holds {n} bytes, {need} are needed")
    return n


def _default_scale(scale):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


# ---------------------------------------------------------------------------
# forward / backward
# ---------------------------------------------------------------------------

def smla_fwd(q, kv, idx, sink=None, scale=None, out=None):
    """Sparse MLA forward: (o bf16 [T,H,512], lse fp32 [T,H]).  lse includes the sink.
    out, if given, is a tuple (o, lse) of preallocated outputs."""
    T, H, _ = q.shape
    N, K = kv.shape[0], idx.shape[1]
    _need(q, "q", torch.bfloat16, (T, H, D))
    _need(kv, "kv", torch.bfloat16, (N, D), q.device)
    _need(idx, "idx", torch.int32, (T, K), q.device)
    if sink is not None:
        _need(sink, "sink", torch.float32, (H,), q.device)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _need(o, "o", torch.bfloat16, (T, H, D), q.device)
        _need(lse, "lse", torch.float32, (T, H), q.device)
    _check("smla_fwd", lib().smla_fwd(_ptr(q), _ptr(kv), _ptr(idx), _ptr(sink), T, H, N, K,
                                      _default_scale(scale), _ptr(o), _ptr(lse), _stream(q.device)))
    return o, lse


def bwd_workspace_bytes(T, H, num_kv, topk) -> int:
    n = lib().smla_bwd_workspace_bytes(T, H, num_kv, topk, 0)
    if n == 0:
        raise SmlaError("smla_bwd_workspace_bytes", 2)
    return n


_WS_CACHE_MAX = 2
_ws_cache: "collections.OrderedDict" = collections.OrderedDict()
_ws_lock = threading.Lock()


def bwd_workspace(T, H, num_kv, topk, device):
    """A cached workspace buffer for this shape, device and current stream.  Calls
    on one stream run in order and may share it; a call on another stream (say,
    from another host thread) gets its own, so concurrent calls never share one.
    At most two buffers are kept (least recently used evicted first); an evicted
    buffer returns to torch's allocator on the stream it was made for, so work
    still queued there finishes before the memory is reused."""
    key = (T, H, num_kv, topk, str(device), torch.cuda.current_stream(device).cuda_stream)
    with _ws_lock:
        ws = _ws_cache.get(key)
        if ws is not None:
            _ws_cache.move_to_end(key)
            return ws
        while len(_ws_cache) >= _WS_CACHE_MAX:
            _ws_cache.popitem(last=False)
        ws = torch.empty(bwd_workspace_bytes(T, H, num_kv, topk), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
        return ws


def clear_workspace_cache():
    """Drop every cached backward workspace."""
    with _ws_lock:
        _ws_cache.clear()


def _bwd_outputs(q, kv, H, sink, out):
    """Preallocated (dq, dkv, d_sink) checked like the inputs, or new tensors."""
    T = q.shape[0]
    N = kv.shape[0]
    if out is None:
        dq = torch.empty_like(q)
        dkv = torch.empty_like(kv)
        d_sink = torch.empty((H,), dtype=torch.float32, device=q.device) if sink is not None else None
        return dq, dkv, d_sink
    dq, dkv, d_sink = out
    _need(dq, "dq", torch.bfloat16, (T, H, D), q.device)
    _need(dkv, "dkv", torch.bfloat16, (N, D), q.device)
    if (sink is None) != (d_sink is None):
        raise ValueError("out: d_sink must be given exactly when sink is")
    if d_sink is not None:
        _need(d_sink, "d_sink", torch.float32, (H,), q.device)
    return dq, dkv, d_sink


def _check_bwd_inputs(q, kv, dO, o, lse, idx, sink, dlse):
    T, H, _ = q.shape
    N, K = kv.shape[0], idx.shape[1]
    dv = q.device
    _need(q, "q", torch.bfloat16, (T, H, D))
    _need(kv, "kv", torch.bfloat16, (N, D), dv)
    _need(dO, "dO", torch.bfloat16, (T, H, D), dv)
    _need(o, "o", torch.bfloat16, (T, H, D), dv)
    _need(lse, "lse", torch.float32, (T, H), dv)
    _need(idx, "idx", torch.int32, (T, K), dv)
    if sink is not None:
        _need(sink, "sink", torch.float32, (H,), dv)
    if dlse is not None:
        _need(dlse, "dlse", torch.float32, (T, H), dv)
    return T, H, N, K


def smla_bwd(q, kv, dO, o, lse, idx, sink=None, scale=None, workspace=None, out=None,
             count_invalid=False, dlse=None, events=None):
    """Sparse MLA backward: returns (dq, dkv, d_sink[, n_invalid]).

    out, if given, is a tuple (dq, dkv, d_sink) of preallocated outputs.
    dlse, if given, is the upstream gradient of lse (fp32 [T, H]).
    events, if given, are five torch.cuda.Event objects (timing enabled) that the
    call records on its stream at the stage boundaries (smla_bwd_timed): before
    delta and after delta, dQ, the intermediate and the gather.
    """
    T, H, N, K = _check_bwd_inputs(q, kv, dO, o, lse, idx, sink, dlse)
    dq, dkv, d_sink = _bwd_outputs(q, kv, H, sink, out)
    if workspace is None:
        workspace = bwd_workspace(T, H, N, K, q.device)
    ws_bytes = _workspace(workspace, "workspace", q.device)
    n_inv = torch.empty((1,), dtype=torch.int32, device=q.device) if count_invalid else None
    args = (_ptr(q), _ptr(kv), _ptr(dO), _ptr(o), _ptr(lse), _ptr(idx), _ptr(sink), _ptr(dlse), T, H, N, K,
            _default_scale(scale), 0, _ptr(dq), _ptr(dkv), _ptr(d_sink), _ptr(n_inv),
            _ptr(workspace), ws_bytes, _stream(q.device))
    if events is None:
        _check("smla_bwd", lib().smla_bwd(*args))
    else:
        if len(events) != 5:
            raise ValueError("smla_bwd: events must hold five torch.cuda.Event objects")
        for e in events:
            if e.cuda_event == 0:   # torch creates the underlying event at its first record
                e.record()
        handles = (ctypes.c_void_p * 5)(*[e.cuda_event for e in events])
        _check("smla_bwd_timed", lib().smla_bwd_timed(*args, handles))
    if count_invalid:
        return dq, dkv, d_sink, n_inv
    return dq, dkv, d_sink


def smla_bwd_phased(q, kv, dO, o, lse, idx, sink=None, scale=None, phase_tokens=1024, workspace=None,
                    out=None, count_invalid=False, dlse=None):
    """The backward with a workspace bounded by `phase_tokens` tokens: returns
    (dq, dkv, d_sink[, n_invalid]) like smla_bwd."""
    T, H, N, K = _check_bwd_inputs(q, kv, dO, o, lse, idx, sink, dlse)
    dq, dkv, d_sink = _bwd_outputs(q, kv, H, sink, out)
    if workspace is None:
        n = lib().smla_bwd_phased_workspace_bytes(T, H, N, K, int(phase_tokens), 0)
        if n == 0:
            raise SmlaError("smla_bwd_phased_workspace_bytes", 2)
        workspace = torch.empty((n,), dtype=torch.uint8, device=q.device)
    ws_bytes = _workspace(workspace, "workspace", q.device)
    n_inv = torch.empty((1,), dtype=torch.int32, device=q.device) if count_invalid else None
    _check("smla_bwd_phased", lib().smla_bwd_phased(
        _ptr(q), _ptr(kv), _ptr(dO), _ptr(o), _ptr(lse), _ptr(idx), _ptr(sink), _ptr(dlse), T, H, N, K,
        _default_scale(scale), 0, int(phase_tokens), _ptr(dq), _ptr(dkv), _ptr(d_sink), _ptr(n_inv),
        _ptr(workspace), ws_bytes, _stream(q.device)))
    if count_invalid:
        return dq, dkv, d_sink, n_inv
    return dq, dkv, d_sink


def smla_bwd_noalloc(q, kv, dO, o, lse, idx, sink=None, scale=None, out=None, count_invalid=False,
                     dlse=None):
    """The backward on the library's fixed device scratch (no workspace, no
    allocation inside the call).  With `out` (and count_invalid False) this
    function allocates nothing either.  Returns (dq, dkv, d_sink[, n_invalid])."""
    T, H, N, K = _check_bwd_inputs(q, kv, dO, o, lse, idx, sink, dlse)
    dq, dkv, d_sink = _bwd_outputs(q, kv, H, sink, out)
    n_inv = torch.empty((1,), dtype=torch.int32, device=q.device) if count_invalid else None
    _check("smla_bwd_noalloc", lib().smla_bwd_noalloc(
        _ptr(q), _ptr(kv), _ptr(dO), _ptr(o), _ptr(lse), _ptr(idx), _ptr(sink), _ptr(dlse), T, H, N, K,
        _default_scale(scale), 0, _ptr(dq), _ptr(dkv), _ptr(d_sink), _ptr(n_inv), _stream(q.device)))
    if count_invalid:
        return dq, dkv, d_sink, n_inv
    return dq, dkv, d_sink


# ---------------------------------------------------------------------------
# stages
# ---------------------------------------------------------------------------

def smla_delta(o, dO, delta=None, dlse=None):
    """delta = rowsum(o * dO) (minus dlse when given), fp32 [T, H]."""
    T, H, _ = o.shape
    _need(o, "o", torch.bfloat16, (T, H, D))
    _need(dO, "dO", torch.bfloat16, (T, H, D), o.device)
    if dlse is not None:
        _need(dlse, "dlse", torch.float32, (T, H), o.device)
    if delta is None:
        delta = torch.empty((T, H), dtype=torch.float32, device=o.device)
    else:
        _need(delta, "delta", torch.float32, (T, H), o.device)
    _check("smla_delta", lib().smla_delta(_ptr(o), _ptr(dO), _ptr(dlse), T, H, _ptr(delta),
                                          _stream(o.device)))
    return delta


def dsp_numel(T, H, topk) -> int:
    """bf16 elements of the dS/P block buffer of smla_dq / smla_interm."""
    return lib().smla_dsp_bytes(T, H, topk) // 2


def smla_dq(q, kv, dO, lse, delta, idx, scale=None, dsp=None, dq=None):
    """Returns (dq bf16 [T,H,512], dsp bf16 blocks): per token, compacted tiles of
    32 valid slots, each a block of 2H x 32 values (rows scale*dS then P) in the
    piece layout documented with smla_dq in include/smla.h."""
    T, H, _ = q.shape
    N, K = kv.shape[0], idx.shape[1]
    for t, n, dt, sh in ((q, "q", torch.bfloat16, (T, H, D)), (kv, "kv", torch.bfloat16, (N, D)),
                         (dO, "dO", torch.bfloat16, (T, H, D)), (lse, "lse", torch.float32, (T, H)),
                         (delta, "delta", torch.float32, (T, H)), (idx, "idx", torch.int32, (T, K))):
        _need(t, n, dt, sh, q.device)
    if dq is None:
        dq = torch.empty_like(q)
    else:
        _need(dq, "dq", torch.bfloat16, (T, H, D), q.device)
    if dsp is None:
        dsp = torch.empty((dsp_numel(T, H, K),), dtype=torch.bfloat16, device=q.device)
    else:
        _need(dsp, "dsp", torch.bfloat16, (dsp_numel(T, H, K),), q.device)
    _check("smla_dq", lib().smla_dq(_ptr(q), _ptr(kv), _ptr(dO), _ptr(lse), _ptr(delta), _ptr(idx),
                                    T, H, N, K, _default_scale(scale), _ptr(dq), _ptr(dsp),
                                    _stream(q.device)))
    return dq, dsp


def smla_interm(q, dO, dsp, idx, num_kv, interm=None):
    T, H, _ = q.shape
    K = idx.shape[1]
    _need(q, "q", torch.bfloat16, (T, H, D))
    _need(dO, "dO", torch.bfloat16, (T, H, D), q.device)
    _need(dsp, "dsp", torch.bfloat16, (dsp_numel(T, H, K),), q.device)
    _need(idx, "idx", torch.int32, (T, K), q.device)
    if interm is None:
        interm = torch.empty((T * K, D), dtype=torch.bfloat16, device=q.device)
    else:
        _need(interm, "interm", torch.bfloat16, (T * K, D), q.device)
    _check("smla_interm", lib().smla_interm(_ptr(q), _ptr(dO), _ptr(dsp), _ptr(idx), T, H, num_kv, K,
                                            _ptr(interm), _stream(q.device)))
    return interm


def smla_build_csr(idx, num_kv, count_invalid=False, out=None, workspace=None):
    """Returns (row_ptr int32 [num_kv+1], slots int32 [T*topk] capacity[, n_invalid])."""
    T, K = idx.shape
    _need(idx, "idx", torch.int32, (T, K))
    if out is None:
        row_ptr = torch.empty((num_kv + 1,), dtype=torch.int32, device=idx.device)
        slots = torch.empty((max(T * K, 1),), dtype=torch.int32, device=idx.device)
    else:
        row_ptr, slots = out
        _need(row_ptr, "row_ptr", torch.int32, (num_kv + 1,), idx.device)
        _need(slots, "slots", torch.int32, None, idx.device)
        if slots.numel() < T * K:
            raise ValueError(f"slots holds {slots.numel()} entries, T*topk = {T * K} are needed")
    n = lib().smla_csr_workspace_bytes(T, K, num_kv)
    if n == 0:
        raise SmlaError("smla_csr_workspace_bytes", 2)
    ws = torch.empty((n,), dtype=torch.uint8, device=idx.device) if workspace is None else workspace
    ws_bytes = _workspace(ws, "workspace", idx.device)
    n_inv = torch.empty((1,), dtype=torch.int32, device=idx.device) if count_invalid else None
    _check("smla_build_csr", lib().smla_build_csr(_ptr(idx), T, K, num_kv, _ptr(row_ptr), _ptr(slots),
                                                  _ptr(n_inv), _ptr(ws), ws_bytes, _stream(idx.device)))
    return (row_ptr, slots, n_inv) if count_invalid else (row_ptr, slots)


def smla_gather(interm, row_ptr, slots, T, topk, num_kv, dkv=None, workspace=None):
    dv = interm.device
    _need(interm, "interm", torch.bfloat16, (T * topk, D))
    _need(row_ptr, "row_ptr", torch.int32, (num_kv + 1,), dv)
    _need(slots, "slots", torch.int32, None, dv)
    if dkv is None:
        dkv = torch.empty((num_kv, D), dtype=torch.bfloat16, device=dv)
    else:
        _need(dkv, "dkv", torch.bfloat16, (num_kv, D), dv)
    n = lib().smla_gather_workspace_bytes(T, topk, num_kv)
    if n == 0:
        raise SmlaError("smla_gather_workspace_bytes", 2)
    ws = torch.empty((n,), dtype=torch.uint8, device=dv) if workspace is None else workspace
    ws_bytes = _workspace(ws, "workspace", dv)
    _check("smla_gather", lib().smla_gather(_ptr(interm), _ptr(row_ptr), _ptr(slots), T, topk, num_kv,
                                            _ptr(dkv), _ptr(ws), ws_bytes, _stream(dv)))
    return dkv


def smla_dsink(lse, delta, sink, d_sink=None, workspace=None):
    T, H = lse.shape
    dv = lse.device
    _need(lse, "lse", torch.float32, (T, H))
    _need(delta, "delta", torch.float32, (T, H), dv)
    _need(sink, "sink", torch.float32, (H,), dv)
    if d_sink is None:
        d_sink = torch.empty((H,), dtype=torch.float32, device=dv)
    else:
        _need(d_sink, "d_sink", torch.float32, (H,), dv)
    n = lib().smla_dsink_workspace_bytes(T, H)
    ws = torch.empty((max(n, 4),), dtype=torch.uint8, device=dv) if workspace is None else workspace
    ws_bytes = _workspace(ws, "workspace", dv)
    _check("smla_dsink", lib().smla_dsink(_ptr(lse), _ptr(delta), _ptr(sink), T, H, _ptr(d_sink),
                                          _ptr(ws), ws_bytes, _stream(dv)))
    return d_sink


# ---------------------------------------------------------------------------
# the has_pe=True variant (positional parts q_pe [T,H,64], k_pe [num_kv,64])
# ---------------------------------------------------------------------------

def _default_scale_pe(scale):
    return 1.0 / math.sqrt(D + DPE) if scale is None else float(scale)


def smla_fwd_pe(q, q_pe, kv, k_pe, idx, sink=None, scale=None, out=None):
    """Forward with the positional part: (o bf16 [T,H,512], lse fp32 [T,H])."""
    T, H, _ = q.shape
    N, K = kv.shape[0], idx.shape[1]
    dv = q.device
    _need(q, "q", torch.bfloat16, (T, H, D))
    _need(q_pe, "q_pe", torch.bfloat16, (T, H, DPE), dv)
    _need(kv, "kv", torch.bfloat16, (N, D), dv)
    _need(k_pe, "k_pe", torch.bfloat16, (N, DPE), dv)
    _need(idx, "idx", torch.int32, (T, K), dv)
    if sink is not None:
        _need(sink, "sink", torch.float32, (H,), dv)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((T, H), dtype=torch.float32, device=dv)
    else:
        o, lse = out
        _need(o, "o", torch.bfloat16, (T, H, D), dv)
        _need(lse, "lse", torch.float32, (T, H), dv)
    _check("smla_fwd_pe", lib().smla_fwd_pe(_ptr(q), _ptr(q_pe), _ptr(kv), _ptr(k_pe), _ptr(idx), _ptr(sink),
                                            T, H, N, K, _default_scale_pe(scale), _ptr(o), _ptr(lse),
                                            _stream(dv)))
    return o, lse


def bwd_pe_workspace_bytes(T, H, num_kv, topk) -> int:
    n = lib().smla_bwd_pe_workspace_bytes(T, H, num_kv, topk, 0)
    if n == 0:
        raise SmlaError("smla_bwd_pe_workspace_bytes", 2)
    return n


def smla_bwd_pe(q, q_pe, kv, k_pe, dO, o, lse, idx, sink=None, scale=None, workspace=None, out=None,
                count_invalid=False, dlse=None):
    """Backward with the positional part: returns (dq, dq_pe, dkv, dk_pe, d_sink[, n_invalid]).
    out, if given, is a tuple (dq, dq_pe, dkv, dk_pe, d_sink) of preallocated outputs."""
    T, H, N, K = _check_bwd_inputs(q, kv, dO, o, lse, idx, sink, dlse)
    dv = q.device
    _need(q_pe, "q_pe", torch.bfloat16, (T, H, DPE), dv)
    _need(k_pe, "k_pe", torch.bfloat16, (N, DPE), dv)
    if out is None:
        dq, dkv, d_sink = _bwd_outputs(q, kv, H, sink, None)
        dq_pe = torch.empty_like(q_pe)
        dk_pe = torch.empty_like(k_pe)
    else:
        dq, dq_pe, dkv, dk_pe, d_sink = out
        dq, dkv, d_sink = _bwd_outputs(q, kv, H, sink, (dq, dkv, d_sink))
        _need(dq_pe, "dq_pe", torch.bfloat16, (T, H, DPE), dv)
        _need(dk_pe, "dk_pe", torch.bfloat16, (N, DPE), dv)
    if workspace is None:
        workspace = torch.empty((bwd_pe_workspace_bytes(T, H, N, K),), dtype=torch.uint8, device=dv)
    ws_bytes = _workspace(workspace, "workspace", dv)
    n_inv = torch.empty((1,), dtype=torch.int32, device=dv) if count_invalid else None
    _check("smla_bwd_pe", lib().smla_bwd_pe(
        _ptr(q), _ptr(q_pe), _ptr(kv), _ptr(k_pe), _ptr(dO), _ptr(o), _ptr(lse), _ptr(idx), _ptr(sink),
        _ptr(dlse), T, H, N, K, _default_scale_pe(scale), 0, _ptr(dq), _ptr(dq_pe), _ptr(dkv), _ptr(dk_pe),
        _ptr(d_sink), _ptr(n_inv), _ptr(workspace), ws_bytes, _stream(dv)))
    res = (dq, dq_pe, dkv, dk_pe, d_sink)
    return res + (n_inv,) if count_invalid else res


# ---------------------------------------------------------------------------
# the page's call form, and autograd (argument marshalling only)
# ---------------------------------------------------------------------------

def sparse_mla_bwd_dsv4(q, kv, do, o, lse, topk, attn_sink=None, scale=None):
    """The backward under the page's call form (same argument order, `topk` the
    [T, topk] int32 index tensor, `attn_sink` the optional per-head sink):
    returns (dq, dkv, d_sink), d_sink None without a sink."""
    return smla_bwd(q, kv, do, o, lse, topk, attn_sink, scale)


class SparseMLA(torch.autograd.Function):
    """o, lse = smla_fwd(q, kv, idx, sink); its backward is smla_bwd, with the
    gradient of lse (when lse is used) passed on as dlse.  Gradients flow to q,
    kv and sink; idx takes none."""

    @staticmethod
    def forward(ctx, q, kv, idx, sink, scale):
        o, lse = smla_fwd(q, kv, idx, sink, scale)
        ctx.save_for_backward(q, kv, idx, o, lse, *(() if sink is None else (sink,)))
        ctx.has_sink = sink is not None
        ctx.scale = scale
        return o, lse

    @staticmethod
    def backward(ctx, do, dlse):
        q, kv, idx, o, lse, *rest = ctx.saved_tensors
        sink = rest[0] if ctx.has_sink else None
        do = torch.zeros_like(o) if do is None else do.to(torch.bfloat16).contiguous()
        dlse = None if dlse is None else dlse.to(torch.float32).contiguous()
        dq, dkv, d_sink = smla_bwd(q, kv, do, o, lse, idx, sink, ctx.scale, dlse=dlse)
        return dq, dkv, None, d_sink, None


def sparse_mla(q, kv, idx, sink=None, scale=None):
    """Differentiable sparse MLA attention: (o bf16 [T,H,512], lse fp32 [T,H])."""
    return SparseMLA.apply(q, kv, idx, sink, scale)


class SparseMLAPE(torch.autograd.Function):
    """The has_pe=True variant under autograd: o, lse = smla_fwd_pe(q, q_pe, kv,
    k_pe, idx, sink); its backward is smla_bwd_pe, lse's gradient going in as
    dlse.  Gradients flow to q, q_pe, kv, k_pe and sink."""

    @staticmethod
    def forward(ctx, q, q_pe, kv, k_pe, idx, sink, scale):
        o, lse = smla_fwd_pe(q, q_pe, kv, k_pe, idx, sink, scale)
        ctx.save_for_backward(q, q_pe, kv, k_pe, idx, o, lse, *(() if sink is None else (sink,)))
        ctx.has_sink = sink is not None
        ctx.scale = scale
        return o, lse

    @staticmethod
    def backward(ctx, do, dlse):
        q, q_pe, kv, k_pe, idx, o, lse, *rest = ctx.saved_tensors
        sink = rest[0] if ctx.has_sink else None
        do = torch.zeros_like(o) if do is None else do.to(torch.bfloat16).contiguous()
        dlse = None if dlse is None else dlse.to(torch.float32).contiguous()
        dq, dq_pe, dkv, dk_pe, d_sink = smla_bwd_pe(q, q_pe, kv, k_pe, do, o, lse, idx, sink, ctx.scale, dlse=dlse)
        return dq, dq_pe, dkv, dk_pe, None, d_sink, None


def sparse_mla_pe(q, q_pe, kv, k_pe, idx, sink=None, scale=None):
    """Differentiable has_pe=True sparse MLA attention: (o, lse)."""
    return SparseMLAPE.apply(q, q_pe, kv, k_pe, idx, sink, scale)
