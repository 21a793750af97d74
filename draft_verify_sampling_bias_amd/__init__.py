"""Python binding of libdspark (the DSpark draft -> schedule -> verify hot path
on MI355X / gfx950).

Argument marshalling only: tensors are checked for device, dtype and layout,
outputs and workspaces are allocated with torch on the inputs' device (from
the pool of the stream the call is launched on, so a buffer freed after the
call is not handed to other work while the call's kernels still use it), and
the C entry points of ``libdspark.so`` (declared in include/dspark.h) are
called on that stream (the current torch stream unless ``stream`` is given).
Every step of the computation runs in the library's HIP kernels; there is no
other implementation to fall back to, and the first call fails loudly
(ImportError) if the library has not been built.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "LIB_PATH", "get_lib", "Status", "DsparkError", "dspark_draft_block", "dspark_schedule",
    "dspark_schedule_cutoff", "dspark_pack_w2", "dspark_w2_packed_bytes", "PackArgs",
    "dspark_verify", "dspark_schedule_rows", "dspark_draft_workspace_size",
    "dspark_verify_workspace_size", "dspark_status_string", "dspark_abi_version",
    "DraftArgs", "ScheduleArgs", "CutoffArgs", "VerifyArgs", "EXPORTED_SYMBOLS",
    "dspark_capacity", "CapacityArgs", "dspark_sts_fit", "dspark_sts_apply", "StsFitArgs", "StsApplyArgs",
    "dspark_check", "InputCheckError", "CHECK_INPUTS", "BAD_TOKEN", "BAD_UNIFORM", "BAD_LENGTH",
    "BAD_CONFIDENCE", "WORKSPACE_HEADER", "dspark_schedule_workspace_size", "dspark_cutoff_workspace_size",
    "dspark_draft_block_noalloc", "NOALLOC_SCRATCH_BYTES", "HEAD_MARKOV", "HEAD_RNN", "ACT_IDENTITY",
    "ACT_TANH", "ABI_VERSION",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdspark.so")

W_F32, W_BF16 = 0, 1
HEAD_MARKOV, HEAD_RNN = 0, 1      # dspark_head
ACT_IDENTITY, ACT_TANH = 0, 1     # dspark_act
ABI_VERSION = 3                   # DSPARK_ABI_VERSION these structs follow

# flags and input-check bits (include/dspark.h)
CHECK_INPUTS = 1
BAD_TOKEN, BAD_UNIFORM, BAD_LENGTH, BAD_CONFIDENCE = 1, 2, 4, 8
WORKSPACE_HEADER = 256
NOALLOC_SCRATCH_BYTES = 64 << 20   # the static workspace of dspark_draft_block_noalloc

EXPORTED_SYMBOLS = (
    "dspark_draft_workspace_size", "dspark_verify_workspace_size", "dspark_draft_block",
    "dspark_schedule", "dspark_schedule_cutoff", "dspark_verify", "dspark_schedule_rows",
    "dspark_status_string", "dspark_abi_version", "dspark_pack_w2", "dspark_w2_packed_bytes",
    "dspark_capacity", "dspark_sts_fit", "dspark_sts_apply", "dspark_schedule_workspace_size",
    "dspark_cutoff_workspace_size", "dspark_check", "dspark_draft_block_noalloc",
)


class Status:
    (OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_ABI, ERR_HIP,
     ERR_INPUT) = range(10)


class DsparkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({dspark_status_string(status)})")


class InputCheckError(DsparkError):
    """The device input checks (check_inputs=True) found values outside the
    contract; ``bits`` holds the BAD_* bits.  The call's outputs were still
    written (with clamped inputs), but are unspecified."""

    def __init__(self, fn: str, bits: int):
        self.bits = bits
        names = [n for n, b in (("BAD_TOKEN", BAD_TOKEN), ("BAD_UNIFORM", BAD_UNIFORM), ("BAD_LENGTH", BAD_LENGTH),
                                ("BAD_CONFIDENCE", BAD_CONFIDENCE)) if bits & b]
        super().__init__(fn, Status.ERR_INPUT)
        self.args = (f"{fn}: device input check failed: {' | '.join(names) or hex(bits)}",)


_p = ctypes.c_void_p


class DraftArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("R", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("V", ctypes.c_int32), ("rank", ctypes.c_int32), ("wdtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32),
                ("U", _p), ("W1", _p), ("W2", _p), ("anchor", _p), ("temp", _p), ("u_draft", _p),
                ("y", _p), ("q_tok", _p), ("q_stats", _p), ("workspace", _p),
                ("workspace_bytes", ctypes.c_size_t), ("stream", _p), ("prof_events", _p), ("W2_packed", _p),
                ("W2_packed_bytes", ctypes.c_size_t), ("head", ctypes.c_int32), ("act", ctypes.c_int32),
                ("A", _p), ("h", _p)]


class ScheduleArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("R", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("K", ctypes.c_int64), ("flags", ctypes.c_uint32), ("c", _p), ("anchor", _p), ("y", _p),
                ("a", _p), ("l", _p), ("row_offsets", _p), ("row_req", _p), ("row_pos", _p), ("row_tok", _p),
                ("expected_tokens", _p), ("workspace", _p), ("workspace_bytes", ctypes.c_size_t),
                ("stream", _p)]


class CutoffArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("R", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("conf_min", ctypes.c_float), ("flags", ctypes.c_uint32), ("c", _p), ("anchor", _p),
                ("y", _p), ("a", _p), ("l", _p), ("row_offsets", _p), ("row_req", _p), ("row_pos", _p),
                ("row_tok", _p), ("expected_tokens", _p), ("workspace", _p),
                ("workspace_bytes", ctypes.c_size_t), ("stream", _p)]


class VerifyArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("R", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("V", ctypes.c_int32), ("rank", ctypes.c_int32), ("wdtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("n_rows", ctypes.c_int64), ("target", _p), ("row_offsets", _p),
                ("U", _p), ("W1", _p), ("W2", _p), ("anchor", _p), ("temp", _p), ("y", _p), ("q_tok", _p),
                ("q_stats", _p), ("u_accept", _p), ("u_final", _p), ("n_accept", _p), ("out_tok", _p),
                ("p_tok", _p), ("workspace", _p), ("workspace_bytes", ctypes.c_size_t), ("stream", _p),
                ("W2_packed", _p), ("W2_packed_bytes", ctypes.c_size_t), ("head", ctypes.c_int32),
                ("h", _p)]


class CapacityArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("R", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("n_sps", ctypes.c_int32), ("a_lag", _p), ("sps", _p), ("K", _p), ("expected", _p),
                ("theta", _p), ("stream", _p)]


class StsFitArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("N", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("z", _p), ("n_acc", _p), ("tau", _p), ("stream", _p)]


class StsApplyArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("R", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("z", _p), ("tau", _p), ("c", _p), ("stream", _p)]


class PackArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("V", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("W2", _p), ("W2_packed", _p), ("W2_packed_bytes", ctypes.c_size_t), ("stream", _p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m draft_verify_sampling_bias_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.dspark_draft_workspace_size.argtypes = [P(DraftArgs), P(ctypes.c_size_t)]
    L.dspark_verify_workspace_size.argtypes = [P(VerifyArgs), P(ctypes.c_size_t)]
    L.dspark_schedule_workspace_size.argtypes = [P(ScheduleArgs), P(ctypes.c_size_t)]
    L.dspark_cutoff_workspace_size.argtypes = [P(CutoffArgs), P(ctypes.c_size_t)]
    L.dspark_check.argtypes = [_p, _p, P(ctypes.c_uint32)]
    L.dspark_draft_block.argtypes = [P(DraftArgs)]
    L.dspark_draft_block_noalloc.argtypes = [P(DraftArgs)]
    L.dspark_schedule.argtypes = [P(ScheduleArgs)]
    L.dspark_schedule_cutoff.argtypes = [P(CutoffArgs)]
    L.dspark_pack_w2.argtypes = [P(PackArgs)]
    L.dspark_w2_packed_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
    L.dspark_w2_packed_bytes.restype = ctypes.c_size_t
    L.dspark_verify.argtypes = [P(VerifyArgs)]
    L.dspark_capacity.argtypes = [P(CapacityArgs)]
    L.dspark_sts_fit.argtypes = [P(StsFitArgs)]
    L.dspark_sts_apply.argtypes = [P(StsApplyArgs)]
    for f in ("dspark_draft_workspace_size", "dspark_verify_workspace_size", "dspark_draft_block",
              "dspark_schedule", "dspark_schedule_cutoff", "dspark_verify", "dspark_abi_version",
              "dspark_pack_w2", "dspark_capacity", "dspark_sts_fit", "dspark_sts_apply",
              "dspark_schedule_workspace_size", "dspark_cutoff_workspace_size", "dspark_check",
              "dspark_draft_block_noalloc"):
        getattr(L, f).restype = ctypes.c_int
    L.dspark_schedule_rows.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]
    L.dspark_schedule_rows.restype = ctypes.c_int64
    L.dspark_status_string.argtypes = [ctypes.c_int]
    L.dspark_status_string.restype = ctypes.c_char_p
    L.dspark_abi_version.argtypes = []
    got = L.dspark_abi_version()
    if got != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has C ABI version {got}, these bindings follow {ABI_VERSION}: rebuild it")
    return L


_LIB = None


def get_lib():
    """The loaded libdspark.so (ctypes.CDLL); raises ImportError if it has not
    been built."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def dspark_status_string(status: int) -> str:
    return get_lib().dspark_status_string(int(status)).decode()


def dspark_abi_version() -> int:
    return int(get_lib().dspark_abi_version())


def dspark_schedule_rows(R: int, gamma: int, K: int) -> int:
    return int(get_lib().dspark_schedule_rows(int(R), int(gamma), int(K)))


def _check(fn: str, status: int):
    if status != Status.OK:
        raise DsparkError(fn, status)


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _want(t, name: str, dtype, shape: Sequence[int], device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _wdtype(W1, W2):
    torch = _torch()
    if W1.dtype != W2.dtype:
        raise TypeError("W1 and W2 must share a dtype")
    if W1.dtype == torch.bfloat16:
        return W_BF16
    if W1.dtype == torch.float32:
        return W_F32
    raise TypeError(f"W1/W2 dtype {W1.dtype}: expected torch.bfloat16 or torch.float32")


def _stream(device, stream):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def _alloc_on(stream):
    """Allocation context for a call's outputs and workspace: the pool of the
    stream the call runs on (a given side stream), so that freeing a buffer
    after the call waits for that stream's work in torch's caching
    allocator."""
    torch = _torch()
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _workspace(nbytes: int, device, workspace):
    torch = _torch()
    if workspace is not None:
        if (workspace.device != device or workspace.numel() * workspace.element_size() < nbytes
                or not workspace.is_contiguous()):
            raise ValueError(f"workspace must be a contiguous buffer of {nbytes} bytes on {device}")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _w2_packed(W2_packed, device, V: int, rank: int):
    """(pointer, bytes) of an optional fragment-packed W2: a contiguous uint8
    tensor on the inputs' device holding at least dspark_w2_packed_bytes."""
    torch = _torch()
    if W2_packed is None:
        return None, 0
    need = dspark_w2_packed_bytes(V, rank)
    if not isinstance(W2_packed, torch.Tensor) or W2_packed.dtype != torch.uint8:
        raise TypeError("W2_packed must be the uint8 tensor made by dspark_pack_w2")
    if W2_packed.device != device or not W2_packed.is_contiguous():
        raise ValueError(f"W2_packed must be contiguous on {device}")
    if W2_packed.numel() < need:
        raise ValueError(f"W2_packed holds {W2_packed.numel()} bytes, V={V} rank={rank} needs {need}")
    return W2_packed.data_ptr(), W2_packed.numel()


def dspark_check(workspace, stream=None) -> int:
    """Error word of the device input checks of the last call on this
    workspace (include/dspark.h, dspark_check): waits for the stream and
    returns the BAD_* bits (0 when every checked input is inside the
    contract)."""
    bits = ctypes.c_uint32(0)
    st = get_lib().dspark_check(ctypes.c_void_p(workspace.data_ptr()), _stream(workspace.device, stream),
                                ctypes.byref(bits))
    if st not in (Status.OK, Status.ERR_INPUT):
        raise DsparkError("dspark_check", st)
    return int(bits.value)


def _raise_on_check(fn: str, ws, stream):
    bits = dspark_check(ws, stream)
    if bits:
        raise InputCheckError(fn, bits)


def _sched_workspace(fn: str, args, device, workspace):
    n = ctypes.c_size_t(0)
    _check(fn, getattr(get_lib(), fn)(ctypes.byref(args), ctypes.byref(n)))
    if n.value == 0:
        return None
    return _workspace(int(n.value), device, workspace)


def draft_workspace_bytes(R: int, gamma: int, V: int, rank: int, wdtype: int, flags: int = 0, *,
                          head: int = 0, act: int = 0) -> int:
    a = DraftArgs(struct_size=ctypes.sizeof(DraftArgs), R=R, gamma=gamma, V=V, rank=rank, wdtype=wdtype,
                  flags=flags, head=head, act=act)
    n = ctypes.c_size_t(0)
    _check("dspark_draft_workspace_size", get_lib().dspark_draft_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return int(n.value)


def verify_workspace_bytes(R: int, gamma: int, V: int, rank: int, wdtype: int, n_rows: int,
                           flags: int = 0, *, head: int = 0) -> int:
    a = VerifyArgs(struct_size=ctypes.sizeof(VerifyArgs), R=R, gamma=gamma, V=V, rank=rank, wdtype=wdtype,
                   n_rows=n_rows, flags=flags, head=head)
    n = ctypes.c_size_t(0)
    _check("dspark_verify_workspace_size", get_lib().dspark_verify_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return int(n.value)


dspark_draft_workspace_size = draft_workspace_bytes
dspark_verify_workspace_size = verify_workspace_bytes


def dspark_schedule_workspace_size(R: int, gamma: int, flags: int = 0) -> int:
    a = ScheduleArgs(struct_size=ctypes.sizeof(ScheduleArgs), R=R, gamma=gamma, flags=flags)
    n = ctypes.c_size_t(0)
    _check("dspark_schedule_workspace_size", get_lib().dspark_schedule_workspace_size(ctypes.byref(a),
                                                                                      ctypes.byref(n)))
    return int(n.value)


def dspark_cutoff_workspace_size(R: int, gamma: int, flags: int = 0) -> int:
    a = CutoffArgs(struct_size=ctypes.sizeof(CutoffArgs), R=R, gamma=gamma, flags=flags)
    n = ctypes.c_size_t(0)
    _check("dspark_cutoff_workspace_size", get_lib().dspark_cutoff_workspace_size(ctypes.byref(a),
                                                                                  ctypes.byref(n)))
    return int(n.value)


def dspark_w2_packed_bytes(V: int, rank: int) -> int:
    return int(get_lib().dspark_w2_packed_bytes(int(V), int(rank)))


def dspark_pack_w2(W2, *, out=None, stream=None):
    """W2 [V, rank] bf16 in the fragment-packed layout of the 16-row fused
    kernel (include/dspark.h, dspark_pack_w2): a uint8 tensor of
    dspark_w2_packed_bytes(V, rank) bytes, to pass as W2_packed."""
    torch = _torch()
    dev = W2.device
    V, rank = W2.shape
    _want(W2, "W2", torch.bfloat16, (V, rank), dev)
    nbytes = dspark_w2_packed_bytes(V, rank)
    if nbytes == 0:
        raise ValueError("invalid V / rank")
    if out is None:
        with _alloc_on(stream):
            out = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    a = PackArgs(struct_size=ctypes.sizeof(PackArgs), V=V, rank=rank, W2=_ptr(W2), W2_packed=_ptr(out),
                 W2_packed_bytes=out.numel() * out.element_size(), stream=_stream(dev, stream))
    _check("dspark_pack_w2", get_lib().dspark_pack_w2(ctypes.byref(a)))
    return out


def _rnn_head(A, act, h, dev, R, gamma, rank, wd, *, alloc: bool):
    """(head, act, A ptr, h tensor) of a draft call: the Markov head when A
    is None, else the RNN head with recurrence A [rank, rank] (the weights'
    dtype) and state output h [R, gamma, rank] fp32 (allocated if None and
    ``alloc``)."""
    torch = _torch()
    if A is None:
        if h is not None:
            raise ValueError("h is the RNN head's state output: give A too")
        return HEAD_MARKOV, ACT_IDENTITY, None, None
    _want(A, "A", torch.bfloat16 if wd == W_BF16 else torch.float32, (rank, rank), dev)
    if h is None:
        if not alloc:
            raise ValueError("the RNN head needs h (the state output) here")
        h = torch.empty((R, gamma, rank), dtype=torch.float32, device=dev)
    _want(h, "h", torch.float32, (R, gamma, rank), dev)
    return HEAD_RNN, int(act), _ptr(A), h


def dspark_draft_block(U, W1, W2, anchor, temp, u_draft, *, out=None, workspace=None, stream=None,
                       prof_events=None, W2_packed=None, check_inputs: bool = False, A=None, act: int = 1,
                       h=None):
    """Draft gamma tokens per request (include/dspark.h, dspark_draft_block).

    U [R, gamma, V] fp32; W1, W2 [V, rank] bf16 or fp32; anchor [R] int32;
    temp [R] fp32; u_draft [R, gamma] fp32.  Returns (y int32 [R, gamma],
    q_tok fp32 [R, gamma], q_stats fp32 [R, gamma, 2]).  ``out`` may supply
    those three tensors; ``prof_events`` a list of 2*gamma timing events
    (torch.cuda.Event already recorded once, or raw hipEvent_t handles)
    attached to each position's fused bias kernel dispatch (start / stop of
    that kernel alone); ``W2_packed`` the output of dspark_pack_w2 for W2.
    ``check_inputs`` runs the device input checks (DSPARK_CHECK_INPUTS) and
    then waits for them: InputCheckError if an input is outside the
    contract (debug only: it synchronises).  ``A`` selects the RNN head
    (DSPARK_HEAD_RNN) with recurrence A [rank, rank] and activation ``act``
    (ACT_IDENTITY / ACT_TANH); the call then returns the states h [R, gamma,
    rank] fp32 as a fourth value (written into ``h`` if given)."""
    torch = _torch()
    dev = U.device
    R, gamma, V = U.shape
    rank = W1.shape[1]
    wd = _wdtype(W1, W2)
    _want(U, "U", torch.float32, (R, gamma, V), dev)
    _want(W1, "W1", W1.dtype, (V, rank), dev)
    _want(W2, "W2", W1.dtype, (V, rank), dev)
    _want(anchor, "anchor", torch.int32, (R,), dev)
    _want(temp, "temp", torch.float32, (R,), dev)
    _want(u_draft, "u_draft", torch.float32, (R, gamma), dev)
    w2p, w2p_bytes = _w2_packed(W2_packed, dev, V, rank)
    flags = CHECK_INPUTS if check_inputs else 0
    with _alloc_on(stream):
        if out is None:
            y = torch.empty((R, gamma), dtype=torch.int32, device=dev)
            q_tok = torch.empty((R, gamma), dtype=torch.float32, device=dev)
            q_stats = torch.empty((R, gamma, 2), dtype=torch.float32, device=dev)
        else:
            y, q_tok, q_stats = out
            _want(y, "y", torch.int32, (R, gamma), dev)
            _want(q_tok, "q_tok", torch.float32, (R, gamma), dev)
            _want(q_stats, "q_stats", torch.float32, (R, gamma, 2), dev)
        head, act_v, a_ptr, h = _rnn_head(A, act, h, dev, R, gamma, rank, wd, alloc=True)
        nbytes = draft_workspace_bytes(R, gamma, V, rank, wd, flags, head=head, act=act_v)
        ws = _workspace(nbytes, dev, workspace)
    ev_arr = None
    if prof_events is not None:
        if len(prof_events) != 2 * gamma:
            raise ValueError(f"prof_events needs {2 * gamma} events")
        # torch.cuda.Event objects or raw hipEvent_t handles (int)
        ev_arr = (ctypes.c_void_p * len(prof_events))(
            *[e if isinstance(e, int) else e.cuda_event for e in prof_events])
    a = DraftArgs(struct_size=ctypes.sizeof(DraftArgs), R=R, gamma=gamma, V=V, rank=rank, wdtype=wd, flags=flags,
                  U=_ptr(U), W1=_ptr(W1), W2=_ptr(W2), anchor=_ptr(anchor), temp=_ptr(temp),
                  u_draft=_ptr(u_draft), y=_ptr(y), q_tok=_ptr(q_tok), q_stats=_ptr(q_stats),
                  workspace=_ptr(ws), workspace_bytes=ws.numel() * ws.element_size(),
                  stream=_stream(dev, stream),
                  prof_events=ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None,
                  W2_packed=w2p, W2_packed_bytes=w2p_bytes, head=head, act=act_v, A=a_ptr,
                  h=_ptr(h) if h is not None else None)
    _check("dspark_draft_block", get_lib().dspark_draft_block(ctypes.byref(a)))
    if check_inputs and R > 0:
        _raise_on_check("dspark_draft_block", ws, stream)
    if head == HEAD_RNN:
        return y, q_tok, q_stats, h
    return y, q_tok, q_stats


def dspark_draft_block_noalloc(U, W1, W2, anchor, temp, u_draft, *, out, stream=None, W2_packed=None, A=None,
                               act: int = 1, h=None):
    """dspark_draft_block with the library's static device workspace
    (include/dspark.h, dspark_draft_block_noalloc): nothing is allocated, so
    ``out`` = (y, q_tok, q_stats) must be given (and ``h`` with the RNN
    head).  Calls that overlap in time on one device share that workspace
    and race."""
    torch = _torch()
    dev = U.device
    R, gamma, V = U.shape
    rank = W1.shape[1]
    wd = _wdtype(W1, W2)
    _want(U, "U", torch.float32, (R, gamma, V), dev)
    _want(W1, "W1", W1.dtype, (V, rank), dev)
    _want(W2, "W2", W1.dtype, (V, rank), dev)
    _want(anchor, "anchor", torch.int32, (R,), dev)
    _want(temp, "temp", torch.float32, (R,), dev)
    _want(u_draft, "u_draft", torch.float32, (R, gamma), dev)
    y, q_tok, q_stats = out
    _want(y, "y", torch.int32, (R, gamma), dev)
    _want(q_tok, "q_tok", torch.float32, (R, gamma), dev)
    _want(q_stats, "q_stats", torch.float32, (R, gamma, 2), dev)
    w2p, w2p_bytes = _w2_packed(W2_packed, dev, V, rank)
    head, act_v, a_ptr, h = _rnn_head(A, act, h, dev, R, gamma, rank, wd, alloc=False)
    a = DraftArgs(struct_size=ctypes.sizeof(DraftArgs), R=R, gamma=gamma, V=V, rank=rank, wdtype=wd,
                  U=_ptr(U), W1=_ptr(W1), W2=_ptr(W2), anchor=_ptr(anchor), temp=_ptr(temp),
                  u_draft=_ptr(u_draft), y=_ptr(y), q_tok=_ptr(q_tok), q_stats=_ptr(q_stats),
                  stream=_stream(dev, stream), W2_packed=w2p, W2_packed_bytes=w2p_bytes, head=head, act=act_v,
                  A=a_ptr, h=_ptr(h) if h is not None else None)
    _check("dspark_draft_block_noalloc", get_lib().dspark_draft_block_noalloc(ctypes.byref(a)))
    if head == HEAD_RNN:
        return y, q_tok, q_stats, h
    return y, q_tok, q_stats


def dspark_schedule(c, K: int, anchor, y, *, out=None, want_expected: bool = True, stream=None,
                    check_inputs: bool = False, workspace=None):
    """Survival + causal prefix-closed top-K schedule (include/dspark.h,
    dspark_schedule).  c [R, gamma] fp32; anchor [R] int32; y [R, gamma] int32.
    Returns a dict with a, l, row_offsets, row_req, row_pos, row_tok and
    expected_tokens (or None)."""
    torch = _torch()
    dev = c.device
    R, gamma = c.shape
    _want(c, "c", torch.float32, (R, gamma), dev)
    _want(anchor, "anchor", torch.int32, (R,), dev)
    _want(y, "y", torch.int32, (R, gamma), dev)
    n_rows = dspark_schedule_rows(R, gamma, K)
    if n_rows < 0:
        raise ValueError("invalid R / gamma")
    flags = CHECK_INPUTS if check_inputs else 0
    given = out is not None
    a = ScheduleArgs(struct_size=ctypes.sizeof(ScheduleArgs), R=R, gamma=gamma, K=int(K), flags=flags)
    with _alloc_on(stream):
        ws = _sched_workspace("dspark_schedule_workspace_size", a, dev, workspace)
        if out is None:
            out = dict(a=torch.empty((R, gamma), dtype=torch.float32, device=dev),
                       l=torch.empty(R, dtype=torch.int32, device=dev),
                       row_offsets=torch.empty(R + 1, dtype=torch.int32, device=dev),
                       row_req=torch.empty(n_rows, dtype=torch.int32, device=dev),
                       row_pos=torch.empty(n_rows, dtype=torch.int32, device=dev),
                       row_tok=torch.empty(n_rows, dtype=torch.int32, device=dev),
                       expected_tokens=torch.empty(1, dtype=torch.float32, device=dev) if want_expected else None)
    if given:
        _want(out["a"], "a", torch.float32, (R, gamma), dev)
        _want(out["l"], "l", torch.int32, (R,), dev)
        _want(out["row_offsets"], "row_offsets", torch.int32, (R + 1,), dev)
        for f in ("row_req", "row_pos", "row_tok"):
            _want(out[f], f, torch.int32, (n_rows,), dev)
    a = ScheduleArgs(struct_size=ctypes.sizeof(ScheduleArgs), R=R, gamma=gamma, K=int(K), flags=flags, c=_ptr(c),
                     anchor=_ptr(anchor), y=_ptr(y), a=_ptr(out["a"]), l=_ptr(out["l"]),
                     row_offsets=_ptr(out["row_offsets"]), row_req=_ptr(out["row_req"]),
                     row_pos=_ptr(out["row_pos"]), row_tok=_ptr(out["row_tok"]),
                     expected_tokens=_ptr(out.get("expected_tokens")), workspace=_ptr(ws),
                     workspace_bytes=0 if ws is None else ws.numel(), stream=_stream(dev, stream))
    _check("dspark_schedule", get_lib().dspark_schedule(ctypes.byref(a)))
    if check_inputs and R > 0:
        _raise_on_check("dspark_schedule", ws, stream)
    return out


def dspark_schedule_cutoff(c, conf_min: float, anchor, y, *, out=None, want_expected: bool = True, stream=None,
                           check_inputs: bool = False, workspace=None):
    """Survival + static confidence-cutoff schedule (include/dspark.h,
    dspark_schedule_cutoff).  c [R, gamma] fp32; anchor [R] int32; y [R, gamma]
    int32.  Returns a dict like dspark_schedule's; the row arrays have room
    for R * (gamma + 1) rows, of which row_offsets[R] are written."""
    torch = _torch()
    dev = c.device
    R, gamma = c.shape
    _want(c, "c", torch.float32, (R, gamma), dev)
    _want(anchor, "anchor", torch.int32, (R,), dev)
    _want(y, "y", torch.int32, (R, gamma), dev)
    cap = R * (gamma + 1)
    flags = CHECK_INPUTS if check_inputs else 0
    given = out is not None
    a = CutoffArgs(struct_size=ctypes.sizeof(CutoffArgs), R=R, gamma=gamma, conf_min=float(conf_min), flags=flags)
    with _alloc_on(stream):
        ws = _sched_workspace("dspark_cutoff_workspace_size", a, dev, workspace)
        if out is None:
            out = dict(a=torch.empty((R, gamma), dtype=torch.float32, device=dev),
                       l=torch.empty(R, dtype=torch.int32, device=dev),
                       row_offsets=torch.empty(R + 1, dtype=torch.int32, device=dev),
                       row_req=torch.empty(cap, dtype=torch.int32, device=dev),
                       row_pos=torch.empty(cap, dtype=torch.int32, device=dev),
                       row_tok=torch.empty(cap, dtype=torch.int32, device=dev),
                       expected_tokens=torch.empty(1, dtype=torch.float32, device=dev) if want_expected else None)
    if given:
        _want(out["a"], "a", torch.float32, (R, gamma), dev)
        _want(out["l"], "l", torch.int32, (R,), dev)
        _want(out["row_offsets"], "row_offsets", torch.int32, (R + 1,), dev)
        for f in ("row_req", "row_pos", "row_tok"):
            _want(out[f], f, torch.int32, (cap,), dev)
    a = CutoffArgs(struct_size=ctypes.sizeof(CutoffArgs), R=R, gamma=gamma, conf_min=float(conf_min), flags=flags,
                   c=_ptr(c), anchor=_ptr(anchor), y=_ptr(y), a=_ptr(out["a"]), l=_ptr(out["l"]),
                   row_offsets=_ptr(out["row_offsets"]), row_req=_ptr(out["row_req"]),
                   row_pos=_ptr(out["row_pos"]), row_tok=_ptr(out["row_tok"]),
                   expected_tokens=_ptr(out.get("expected_tokens")), workspace=_ptr(ws),
                   workspace_bytes=0 if ws is None else ws.numel(), stream=_stream(dev, stream))
    _check("dspark_schedule_cutoff", get_lib().dspark_schedule_cutoff(ctypes.byref(a)))
    if check_inputs and R > 0:
        _raise_on_check("dspark_schedule_cutoff", ws, stream)
    return out


def dspark_capacity(a_lag, sps, *, out=None, stream=None):
    """Hardware-aware capacity for a later step (include/dspark.h,
    dspark_capacity).  a_lag [R, gamma] fp32: survival of an earlier step;
    sps [n_sps] fp32: step rate of a verify batch of B rows, n_sps >= R + 1.
    Returns a dict of device tensors: K int32 [1], expected float64 [1] (E(K))
    and theta float64 [1] (Theta(K))."""
    torch = _torch()
    dev = sps.device
    R, gamma = a_lag.shape
    _want(a_lag, "a_lag", torch.float32, (R, gamma), dev)
    (n_sps,) = sps.shape
    _want(sps, "sps", torch.float32, (n_sps,), dev)
    if out is None:
        with _alloc_on(stream):
            out = dict(K=torch.empty(1, dtype=torch.int32, device=dev),
                       expected=torch.empty(1, dtype=torch.float64, device=dev),
                       theta=torch.empty(1, dtype=torch.float64, device=dev))
    else:
        _want(out["K"], "K", torch.int32, (1,), dev)
        for f in ("expected", "theta"):
            if out.get(f) is not None:
                _want(out[f], f, torch.float64, (1,), dev)
    a = CapacityArgs(struct_size=ctypes.sizeof(CapacityArgs), R=R, gamma=gamma, n_sps=n_sps,
                     a_lag=_ptr(a_lag) if R > 0 else None, sps=_ptr(sps), K=_ptr(out["K"]),
                     expected=_ptr(out.get("expected")), theta=_ptr(out.get("theta")),
                     stream=_stream(dev, stream))
    _check("dspark_capacity", get_lib().dspark_capacity(ctypes.byref(a)))
    return out


def dspark_sts_fit(z, n_acc, *, out=None, stream=None):
    """Sequential temperature scaling fit (include/dspark.h, dspark_sts_fit).
    z [N, gamma] fp32 confidence logits of calibration blocks; n_acc [N]
    int32 accepted counts.  Returns tau [gamma] fp32 (device)."""
    torch = _torch()
    dev = z.device
    N, gamma = z.shape
    _want(z, "z", torch.float32, (N, gamma), dev)
    _want(n_acc, "n_acc", torch.int32, (N,), dev)
    with _alloc_on(stream):
        tau = torch.empty(gamma, dtype=torch.float32, device=dev) if out is None else out
    _want(tau, "tau", torch.float32, (gamma,), dev)
    a = StsFitArgs(struct_size=ctypes.sizeof(StsFitArgs), N=N, gamma=gamma, z=_ptr(z) if N else None,
                   n_acc=_ptr(n_acc) if N else None, tau=_ptr(tau), stream=_stream(dev, stream))
    _check("dspark_sts_fit", get_lib().dspark_sts_fit(ctypes.byref(a)))
    return tau


def dspark_sts_apply(z, tau, *, out=None, stream=None):
    """Calibrated confidence c = sigmoid(z / tau) (include/dspark.h,
    dspark_sts_apply).  z [R, gamma] fp32, tau [gamma] fp32; returns c
    [R, gamma] fp32 (device)."""
    torch = _torch()
    dev = z.device
    R, gamma = z.shape
    _want(z, "z", torch.float32, (R, gamma), dev)
    _want(tau, "tau", torch.float32, (gamma,), dev)
    with _alloc_on(stream):
        c = torch.empty((R, gamma), dtype=torch.float32, device=dev) if out is None else out
    _want(c, "c", torch.float32, (R, gamma), dev)
    a = StsApplyArgs(struct_size=ctypes.sizeof(StsApplyArgs), R=R, gamma=gamma, z=_ptr(z), tau=_ptr(tau),
                     c=_ptr(c), stream=_stream(dev, stream))
    _check("dspark_sts_apply", get_lib().dspark_sts_apply(ctypes.byref(a)))
    return c


def dspark_verify(target, row_offsets, U, W1, W2, anchor, temp, y, q_tok, q_stats, u_accept, u_final, *,
                  out=None, workspace=None, stream=None, W2_packed=None, check_inputs: bool = False, h=None):
    """Accept / reject against target logits (include/dspark.h, dspark_verify).

    target [n_rows, V] fp32; row_offsets [R+1] int32; the draft inputs and
    outputs; u_accept [R, gamma] fp32; u_final [R] fp32; ``h`` the RNN
    head's states from dspark_draft_block (None: Markov head).  Returns
    (n_accept int32 [R], out_tok int32 [R], p_tok fp32 [R, gamma])."""
    torch = _torch()
    dev = target.device
    R, gamma, V = U.shape
    rank = W1.shape[1]
    wd = _wdtype(W1, W2)
    n_rows = target.shape[0]
    _want(target, "target", torch.float32, (n_rows, V), dev)
    _want(row_offsets, "row_offsets", torch.int32, (R + 1,), dev)
    _want(U, "U", torch.float32, (R, gamma, V), dev)
    _want(W1, "W1", W1.dtype, (V, rank), dev)
    _want(W2, "W2", W1.dtype, (V, rank), dev)
    _want(anchor, "anchor", torch.int32, (R,), dev)
    _want(temp, "temp", torch.float32, (R,), dev)
    _want(y, "y", torch.int32, (R, gamma), dev)
    _want(q_tok, "q_tok", torch.float32, (R, gamma), dev)
    _want(q_stats, "q_stats", torch.float32, (R, gamma, 2), dev)
    _want(u_accept, "u_accept", torch.float32, (R, gamma), dev)
    _want(u_final, "u_final", torch.float32, (R,), dev)
    w2p, w2p_bytes = _w2_packed(W2_packed, dev, V, rank)
    flags = CHECK_INPUTS if check_inputs else 0
    head = HEAD_MARKOV
    if h is not None:
        _want(h, "h", torch.float32, (R, gamma, rank), dev)
        head = HEAD_RNN
    with _alloc_on(stream):
        if out is None:
            n_accept = torch.empty(R, dtype=torch.int32, device=dev)
            out_tok = torch.empty(R, dtype=torch.int32, device=dev)
            p_tok = torch.empty((R, gamma), dtype=torch.float32, device=dev)
        else:
            n_accept, out_tok, p_tok = out
            _want(n_accept, "n_accept", torch.int32, (R,), dev)
            _want(out_tok, "out_tok", torch.int32, (R,), dev)
            _want(p_tok, "p_tok", torch.float32, (R, gamma), dev)
        nbytes = verify_workspace_bytes(R, gamma, V, rank, wd, n_rows, flags, head=head)
        ws = _workspace(nbytes, dev, workspace)
    a = VerifyArgs(struct_size=ctypes.sizeof(VerifyArgs), R=R, gamma=gamma, V=V, rank=rank, wdtype=wd, flags=flags,
                   n_rows=n_rows, target=_ptr(target), row_offsets=_ptr(row_offsets), U=_ptr(U),
                   W1=_ptr(W1), W2=_ptr(W2), anchor=_ptr(anchor), temp=_ptr(temp), y=_ptr(y),
                   q_tok=_ptr(q_tok), q_stats=_ptr(q_stats), u_accept=_ptr(u_accept), u_final=_ptr(u_final),
                   n_accept=_ptr(n_accept), out_tok=_ptr(out_tok), p_tok=_ptr(p_tok), workspace=_ptr(ws),
                   workspace_bytes=ws.numel() * ws.element_size(), stream=_stream(dev, stream),
                   W2_packed=w2p, W2_packed_bytes=w2p_bytes, head=head, h=_ptr(h) if h is not None else None)
    _check("dspark_verify", get_lib().dspark_verify(ctypes.byref(a)))
    if check_inputs and R > 0:
        _raise_on_check("dspark_verify", ws, stream)
    return n_accept, out_tok, p_tok
