"""ctypes binding of liblinrec.so (include/linrec.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
of the library.  PyTorch provides device memory and the current stream.
Importing this module never loads the library; the first call does, and
raises if it has not been built -- there is no fallback path.

Layer (per batch b, head h): S_0 = S_in, S_t = a_t S_{t-1} + k_t^T v_t,
o_t = q_t S_t, S_out = S_T; the backward returns dq, dk, dv and dS_in for the
loss <dO, o> + <dS_out, S_out>.  Sub-sequences chain through S_out -> S_in
forward and dS_in -> dS_out backward (StateFlow, Abstract; Sequence
Accumulation and Beyond, "Approach").
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblinrec.so")

CHUNK = 64
BF16, F32 = 0, 1
DECAY_NONE, DECAY_HEAD, DECAY_TOKEN = 0, 1, 2

STATUS = {
    0: "LINREC_OK", 1: "LINREC_E_NULL", 2: "LINREC_E_SHAPE", 3: "LINREC_E_DTYPE",
    4: "LINREC_E_LAYOUT", 5: "LINREC_E_ALIGN", 6: "LINREC_E_WORKSPACE",
    7: "LINREC_E_DEVICE", 8: "LINREC_E_LAUNCH", 9: "LINREC_E_SCRATCH",
}

# Fixed device scratch of linrec_bwd_noalloc (LINREC_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 32 << 20
# Largest T of a call (LINREC_MAX_T).
MAX_T = 2147479552

# Every function include/linrec.h declares.
EXPORTS = (
    "linrec_ctx_create", "linrec_ctx_destroy", "linrec_states_bytes", "linrec_seq_states_bytes",
    "linrec_bwd_workspace_bytes", "linrec_fwd", "linrec_bwd", "linrec_fwd_seq",
    "linrec_bwd_seq_workspace_bytes", "linrec_bwd_seq", "linrec_status_str",
    "linrec_last_hip_error", "linrec_version", "linrec_ctx_set_timing",
    "linrec_ctx_kernel_times", "linrec_bwd_recompute_workspace_bytes", "linrec_bwd_recompute",
    "linrec_bwd_da_workspace_bytes", "linrec_bwd_da", "linrec_bwd_noalloc",
    "linrec_delta_workspace_bytes", "linrec_delta_fwd", "linrec_delta_saved_bytes",
    "linrec_delta_bwd_workspace_bytes", "linrec_delta_bwd", "linrec_delta_seq_saved_bytes",
    "linrec_delta_fwd_seq_workspace_bytes", "linrec_delta_bwd_seq_workspace_bytes",
    "linrec_delta_fwd_seq", "linrec_delta_bwd_seq",
)

KERNEL_KINDS = {0: "fwd_sum", 1: "fwd_fold", 2: "fwd_seg", 3: "bwd_sum", 4: "bwd_fold",
                5: "bwd_seg", 6: "da_finish", 7: "delta_fwd", 8: "delta_bwd"}


class LinrecError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} "
                         f"({_lib().linrec_status_str(status).decode()}; "
                         f"hip error {_lib().linrec_last_hip_error()})")


class Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("sb", ctypes.c_int64),
                ("sh", ctypes.c_int64), ("st", ctypes.c_int64)]


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("decay", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -m state_passing_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, T, D = ctypes.c_void_p, Tensor, ctypes.POINTER(Desc)
    I32 = ctypes.c_int32
    sig = {
        "linrec_ctx_create": ([ctypes.POINTER(P), ctypes.c_int], ctypes.c_int),
        "linrec_ctx_destroy": ([P], ctypes.c_int),
        "linrec_states_bytes": ([D], ctypes.c_size_t),
        "linrec_bwd_workspace_bytes": ([D], ctypes.c_size_t),
        "linrec_bwd_seq_workspace_bytes": ([D, I32, P], ctypes.c_size_t),
        "linrec_seq_states_bytes": ([D, I32, P], ctypes.c_size_t),
        "linrec_fwd": ([P, D, T, T, T, T, P, T, P, P, P], ctypes.c_int),
        "linrec_bwd": ([P, D, T, T, T, T, P, T, P, T, T, T, P, P, P], ctypes.c_int),
        "linrec_bwd_recompute_workspace_bytes": ([D], ctypes.c_size_t),
        "linrec_bwd_recompute": ([P, D, T, T, T, T, P, T, P, T, T, T, P, P, P], ctypes.c_int),
        "linrec_bwd_da_workspace_bytes": ([D], ctypes.c_size_t),
        "linrec_bwd_noalloc": ([P, D, T, T, T, T, P, T, P, T, T, T, P, P], ctypes.c_int),
        "linrec_delta_workspace_bytes": ([D], ctypes.c_size_t),
        "linrec_delta_fwd": ([P, D, T, T, T, T, T, P, T, P, P, P, P], ctypes.c_int),
        "linrec_delta_saved_bytes": ([D], ctypes.c_size_t),
        "linrec_delta_bwd_workspace_bytes": ([D], ctypes.c_size_t),
        "linrec_delta_bwd": ([P, D, T, T, T, T, T, P, T, P, T, T, T, T, P, P, P], ctypes.c_int),
        "linrec_delta_seq_saved_bytes": ([D, I32, P], ctypes.c_size_t),
        "linrec_delta_fwd_seq_workspace_bytes": ([D, I32, P], ctypes.c_size_t),
        "linrec_delta_bwd_seq_workspace_bytes": ([D, I32, P], ctypes.c_size_t),
        "linrec_delta_fwd_seq": ([P, D, I32, P, T, T, T, T, T, P, T, P, P, P, P], ctypes.c_int),
        "linrec_delta_bwd_seq": ([P, D, I32, P, T, T, T, T, T, P, T, P, T, T, T, T, P, P, P],
                                 ctypes.c_int),
        "linrec_bwd_da": ([P, D, T, T, T, T, P, T, P, T, T, T, P, T, P, P, P, P], ctypes.c_int),
        "linrec_fwd_seq": ([P, D, I32, P, T, T, T, T, P, T, P, P, P], ctypes.c_int),
        "linrec_bwd_seq": ([P, D, I32, P, T, T, T, T, P, T, P, T, T, T, P, P, P], ctypes.c_int),
        "linrec_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "linrec_last_hip_error": ([], ctypes.c_int),
        "linrec_version": ([], ctypes.c_int),
        "linrec_ctx_set_timing": ([P, ctypes.c_int], ctypes.c_int),
        "linrec_ctx_kernel_times": ([P, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _LIB = lib
    return lib


def exported_symbols():
    """Names from EXPORTS that the loaded library resolves."""
    lib = _lib()
    return [n for n in EXPORTS if hasattr(lib, n)]


# ----------------------------------------------------------------- context

_CTX = {}


def context(device: Optional[int] = None) -> int:
    """The (cached) linrec_ctx of a device, as an opaque pointer value."""
    if device is None:
        device = torch.cuda.current_device()
    if device not in _CTX:
        p = ctypes.c_void_p()
        rc = _lib().linrec_ctx_create(ctypes.byref(p), int(device))
        if rc != 0:
            raise LinrecError(rc, "linrec_ctx_create")
        _CTX[device] = p.value
    return _CTX[device]


def set_kernel_timing(enable: bool, device: Optional[int] = None) -> None:
    """Turn the context's per-kernel event timing on or off (resets totals)."""
    _check(_lib().linrec_ctx_set_timing(context(device), 1 if enable else 0),
           "linrec_ctx_set_timing")


def kernel_times(device: Optional[int] = None) -> dict:
    """{kernel name: (launches, total ms)} since timing was enabled."""
    out = {}
    for kind, name in KERNEL_KINDS.items():
        n, ms = ctypes.c_int64(), ctypes.c_double()
        _check(_lib().linrec_ctx_kernel_times(context(device), kind, ctypes.byref(n),
                                              ctypes.byref(ms)), "linrec_ctx_kernel_times")
        out[name] = (int(n.value), float(ms.value))
    return out


# ----------------------------------------------------------------- marshalling

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported activation dtype {t.dtype}")


def _act(t: Optional[torch.Tensor]) -> Tensor:
    if t is None:
        return Tensor(None, 0, 0, 0)
    if t.dim() != 4:
        raise ValueError(f"activation must be [B,H,T,d], got {tuple(t.shape)}")
    s = t.stride()
    return Tensor(t.data_ptr(), s[0], s[1], s[2])


def _decay(a: Optional[torch.Tensor]):
    if a is None:
        return DECAY_NONE, Tensor(None, 0, 0, 0)
    if a.dtype != torch.float32:
        raise TypeError("decay must be float32")
    if a.dim() == 1:
        return DECAY_HEAD, Tensor(a.data_ptr(), 0, a.stride(0), 0)
    if a.dim() == 3:
        s = a.stride()
        return DECAY_TOKEN, Tensor(a.data_ptr(), s[0], s[1], s[2])
    raise ValueError("decay must be [H] or [B,H,T]")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def desc(B, H, T, dk, dv, dtype_code, decay_kind, out_code=None) -> Desc:
    return Desc(B, H, T, dk, dv, CHUNK, dtype_code, decay_kind,
                dtype_code if out_code is None else out_code)


def _desc_of(q, v, decay_kind, out_dtype=None) -> Desc:
    B, H, T, dk = q.shape
    code = _dtype_code(q)
    out = code if out_dtype is None else _dtype_code(torch.empty(0, dtype=out_dtype))
    return desc(B, H, T, dk, v.shape[3], code, decay_kind, out)


def states_bytes(d: Desc) -> int:
    return int(_lib().linrec_states_bytes(ctypes.byref(d)))


def bwd_workspace_bytes(d: Desc) -> int:
    return int(_lib().linrec_bwd_workspace_bytes(ctypes.byref(d)))


def seq_states_bytes(d: Desc, lengths: Sequence[int]) -> int:
    arr = (ctypes.c_int32 * len(lengths))(*lengths)
    return int(_lib().linrec_seq_states_bytes(ctypes.byref(d), len(lengths), arr))


def bwd_seq_workspace_bytes(d: Desc, lengths: Sequence[int]) -> int:
    arr = (ctypes.c_int32 * len(lengths))(*lengths)
    return int(_lib().linrec_bwd_seq_workspace_bytes(ctypes.byref(d), len(lengths), arr))


def _state_out(like: torch.Tensor, B, H, dk, dv, given):
    if given is not None:
        return given
    return torch.empty(B, H, dk, dv, dtype=torch.float32, device=like.device)


def _check(rc, where):
    if rc != 0:
        raise LinrecError(rc, where)



# ----------------------------------------------------------------- validation
#
# The C ABI checks what it can see (shapes in the descriptor, alignment,
# strides, NULL pointers).  It cannot see tensor shapes, dtypes, devices or
# buffer sizes, so a mismatch there would become an out-of-bounds access on
# the GPU.  These checks run before any library call; the device check comes
# last so that every structural mistake is reported as such.

def _fail(msg: str, exc=ValueError):
    raise exc(msg)


def _check_act(name, t, shape, dtype=None):
    # conditions first, messages only on failure (this runs on every call)
    if not isinstance(t, torch.Tensor):
        _fail(f"{name}: expected a tensor", TypeError)
    if t.dim() != 4:
        _fail(f"{name}: must be [B,H,T,d], got {tuple(t.shape)}")
    if t.shape != shape:
        _fail(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        _fail(f"{name}: dtype {t.dtype} != {dtype}", TypeError)
    if t.stride(-1) != 1:
        _fail(f"{name}: the feature dimension must be contiguous (stride 1)")


def _check_state(name, t, shape):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        _fail(f"{name}: expected a tensor", TypeError)
    if t.dtype != torch.float32:
        _fail(f"{name}: must be float32, got {t.dtype}", TypeError)
    if t.shape != shape:
        _fail(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if not t.is_contiguous():
        _fail(f"{name}: must be contiguous")


def _check_decay(decay, B, H, T):
    if decay is None:
        return
    if not isinstance(decay, torch.Tensor):
        _fail("decay: expected a tensor", TypeError)
    if decay.dtype != torch.float32:
        _fail("decay must be float32", TypeError)
    if decay.shape != (H,) and decay.shape != (B, H, T):
        _fail(f"decay must be [H] or [B,H,T], got {tuple(decay.shape)} for B={B} H={H} T={T}")


def _check_buffer(name, t, nbytes):
    if not isinstance(t, torch.Tensor):
        _fail(f"{name}: expected a tensor", TypeError)
    if not t.is_contiguous():
        _fail(f"{name}: must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        _fail(f"{name}: {have} bytes, the call needs {nbytes}")


def _check_device(q, *others):
    if not q.is_cuda:
        _fail(f"tensors must be on a GPU, got {q.device}")
    dev = q.device
    for name, t in others:
        if t is not None and t.device != dev:
            _fail(f"{name}: on {t.device}, q on {dev}")


def _validate(q, k, v, decay, *, dO=None, outs=(), states_in=(), states_out=(), extra=()):
    """Check every tensor of a call against q's [B,H,T,d_k] and v's d_v.

    outs: (name, tensor or None, out dtype, d) activation outputs;
    states_in / states_out: (name, tensor or None) fp32 [B,H,d_k,d_v];
    extra: (name, tensor or None) other tensors that only need the device check.
    Returns the (name, tensor) pairs for _check_device, which the caller runs
    after its buffer-size checks, so that structural errors are reported first."""
    if not isinstance(q, torch.Tensor):
        _fail("q: expected a tensor", TypeError)
    if q.dim() != 4:
        _fail(f"q: must be [B,H,T,d_k], got {tuple(q.shape)}")
    B, H, T, DK = q.shape
    if q.dtype not in (torch.bfloat16, torch.float32):
        _fail(f"unsupported activation dtype {q.dtype}", TypeError)
    qs = q.shape
    _check_act("q", q, qs, q.dtype)
    _check_act("k", k, qs, q.dtype)
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        _fail("v: must be [B,H,T,d_v]")
    DV = v.shape[3]
    vs = torch.Size((B, H, T, DV))
    _check_act("v", v, vs, q.dtype)
    if dO is not None:
        _check_act("dO", dO, vs, q.dtype)
    _check_decay(decay, B, H, T)
    odts = set()
    for name, t, odt, d in outs:
        if t is not None:
            _check_act(name, t, torch.Size((B, H, T, d)))
            odts.add(t.dtype)
        else:
            odts.add(odt)
    if len(odts) > 1:
        _fail(f"outputs must share one dtype, got {sorted(map(str, odts))}", TypeError)
    ss = torch.Size((B, H, DK, DV))
    for name, t in states_in:
        _check_state(name, t, ss)
    for name, t in states_out:
        _check_state(name, t, ss)
    return (("k", k), ("v", v), ("dO", dO), ("decay", decay),
            *((n, t) for n, t, _, _ in outs), *states_in, *states_out, *extra)

# ----------------------------------------------------------------- calls

def _out_dtype(q, out_dtype, given):
    if given is not None:
        return given.dtype
    return q.dtype if out_dtype is None else out_dtype


def _piece_lengths(lengths, T):
    lengths = [int(x) for x in lengths]
    if not lengths:
        _fail("lengths: need at least one piece")
    if sum(lengths) != T:
        _fail(f"lengths sum to {sum(lengths)}, the sequence has {T} tokens")
    return lengths


def _outs(q, v, odt, **given):
    """(name, tensor or None, dtype, width) for the activation outputs."""
    DK, DV = q.shape[3], v.shape[3]
    width = {"o": DV, "dq": DK, "dk": DK, "dv": DV}
    return tuple((n, t, odt, width[n]) for n, t in given.items())


def _new_act(q, d, odt, t):
    B, H, T = q.shape[:3]
    return torch.empty(B, H, T, d, dtype=odt, device=q.device) if t is None else t


def fwd(q, k, v, decay=None, S_in=None, *, o=None, S_out=None, states=None, out_dtype=None):
    """Forward over one piece.  Returns (o, S_out, states)."""
    odt = _out_dtype(q, out_dtype, o)
    devs = _validate(q, k, v, decay, outs=_outs(q, v, odt, o=o), states_in=(("S_in", S_in),),
              states_out=(("S_out", S_out),), extra=(("states", states),))
    kind, dec = _decay(decay)
    d = _desc_of(q, v, kind, odt)
    B, H, T, dk = q.shape
    dv = v.shape[3]
    if states is not None:
        _check_buffer("states", states, states_bytes(d))
    _check_device(q, *devs)
    o = _new_act(q, dv, odt, o)
    S_out = _state_out(q, B, H, dk, dv, S_out)
    if states is None:
        states = torch.empty(max(states_bytes(d), 16), dtype=torch.uint8, device=q.device)
    rc = _lib().linrec_fwd(context(q.device.index), ctypes.byref(d), _act(q), _act(k), _act(v),
                           dec, _ptr(S_in), _act(o), _ptr(S_out), _ptr(states),
                           _stream(q.device))
    _check(rc, "linrec_fwd")
    return o, S_out, states


def bwd(q, k, v, decay, states, dO, dS_out=None, *, dq=None, dk=None, dv=None,
        dS_in=None, workspace=None, out_dtype=None):
    """Backward over one piece.  Returns (dq, dk, dv, dS_in)."""
    odt = _out_dtype(q, out_dtype, dq)
    devs = _validate(q, k, v, decay, dO=dO, outs=_outs(q, v, odt, dq=dq, dk=dk, dv=dv),
              states_in=(("dS_out", dS_out),), states_out=(("dS_in", dS_in),),
              extra=(("states", states), ("workspace", workspace)))
    kind, dec = _decay(decay)
    d = _desc_of(q, v, kind, odt)
    B, H, T, DK = q.shape
    DV = v.shape[3]
    _check_buffer("states", states, states_bytes(d))
    if workspace is not None:
        _check_buffer("workspace", workspace, bwd_workspace_bytes(d))
    _check_device(q, *devs)
    dq, dk, dv = _new_act(q, DK, odt, dq), _new_act(q, DK, odt, dk), _new_act(q, DV, odt, dv)
    dS_in = _state_out(q, B, H, DK, DV, dS_in)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(d), 16), dtype=torch.uint8, device=q.device)
    rc = _lib().linrec_bwd(context(q.device.index), ctypes.byref(d), _act(q), _act(k), _act(v),
                           dec, _ptr(states), _act(dO), _ptr(dS_out), _act(dq), _act(dk),
                           _act(dv), _ptr(dS_in), _ptr(workspace), _stream(q.device))
    _check(rc, "linrec_bwd")
    return dq, dk, dv, dS_in


def bwd_noalloc(q, k, v, decay, states, dO, dS_out=None, *, dq=None, dk=None, dv=None,
                dS_in=None, out_dtype=None):
    """linrec_bwd_noalloc: the backward of one piece in the library's fixed
    device scratch (no workspace).  The library call allocates nothing; pass
    dq, dk, dv and dS_in to keep this wrapper from allocating them.  Returns
    (dq, dk, dv, dS_in)."""
    odt = _out_dtype(q, out_dtype, dq)
    devs = _validate(q, k, v, decay, dO=dO, outs=_outs(q, v, odt, dq=dq, dk=dk, dv=dv),
                     states_in=(("dS_out", dS_out),), states_out=(("dS_in", dS_in),),
                     extra=(("states", states),))
    kind, dec = _decay(decay)
    d = _desc_of(q, v, kind, odt)
    B, H, T, DK = q.shape
    DV = v.shape[3]
    _check_buffer("states", states, states_bytes(d))
    _check_device(q, *devs)
    dq, dk, dv = _new_act(q, DK, odt, dq), _new_act(q, DK, odt, dk), _new_act(q, DV, odt, dv)
    dS_in = _state_out(q, B, H, DK, DV, dS_in)
    rc = _lib().linrec_bwd_noalloc(context(q.device.index), ctypes.byref(d), _act(q), _act(k),
                                   _act(v), dec, _ptr(states), _act(dO), _ptr(dS_out), _act(dq),
                                   _act(dk), _act(dv), _ptr(dS_in), _stream(q.device))
    _check(rc, "linrec_bwd_noalloc")
    return dq, dk, dv, dS_in


def bwd_recompute_workspace_bytes(d: Desc) -> int:
    return int(_lib().linrec_bwd_recompute_workspace_bytes(ctypes.byref(d)))


def bwd_recompute(q, k, v, decay, S_in, dO, dS_out=None, *, dq=None, dk=None, dv=None,
                  dS_in=None, workspace=None, out_dtype=None):
    """Backward over one piece from its boundary state S_in alone (the
    per-segment states are rebuilt).  Returns (dq, dk, dv, dS_in)."""
    odt = _out_dtype(q, out_dtype, dq)
    devs = _validate(q, k, v, decay, dO=dO, outs=_outs(q, v, odt, dq=dq, dk=dk, dv=dv),
              states_in=(("S_in", S_in), ("dS_out", dS_out)), states_out=(("dS_in", dS_in),),
              extra=(("workspace", workspace),))
    kind, dec = _decay(decay)
    d = _desc_of(q, v, kind, odt)
    B, H, T, DK = q.shape
    DV = v.shape[3]
    if workspace is not None:
        _check_buffer("workspace", workspace, bwd_recompute_workspace_bytes(d))
    _check_device(q, *devs)
    dq, dk, dv = _new_act(q, DK, odt, dq), _new_act(q, DK, odt, dk), _new_act(q, DV, odt, dv)
    dS_in = _state_out(q, B, H, DK, DV, dS_in)
    if workspace is None:
        workspace = torch.empty(max(bwd_recompute_workspace_bytes(d), 16), dtype=torch.uint8,
                                device=q.device)
    rc = _lib().linrec_bwd_recompute(context(q.device.index), ctypes.byref(d), _act(q), _act(k),
                                     _act(v), dec, _ptr(S_in), _act(dO), _ptr(dS_out), _act(dq),
                                     _act(dk), _act(dv), _ptr(dS_in), _ptr(workspace),
                                     _stream(q.device))
    _check(rc, "linrec_bwd_recompute")
    return dq, dk, dv, dS_in


def bwd_da_workspace_bytes(d: Desc) -> int:
    return int(_lib().linrec_bwd_da_workspace_bytes(ctypes.byref(d)))


def bwd_da(q, k, v, decay, states, dO, dS_out=None, da_carry=None, *, dq=None, dk=None,
           dv=None, dS_in=None, da=None, da_carry_out=None, workspace=None, out_dtype=None):
    """Backward over one piece plus the decay gradient.

    da_carry: fp32 [B,H], the gradient carried from later pieces (<dS_out,
    S_out>; None = 0).  Returns (dq, dk, dv, dS_in, da, da_carry_out) with
    da fp32 [B,H,T] and da_carry_out the carry for the previous piece."""
    odt = _out_dtype(q, out_dtype, dq)
    devs = _validate(q, k, v, decay, dO=dO, outs=_outs(q, v, odt, dq=dq, dk=dk, dv=dv),
              states_in=(("dS_out", dS_out),), states_out=(("dS_in", dS_in),),
              extra=(("states", states), ("workspace", workspace), ("da", da),
                     ("da_carry", da_carry), ("da_carry_out", da_carry_out)))
    if decay is None:
        _fail("bwd_da: needs a decay tensor")
    B, H, T, DK = q.shape
    DV = v.shape[3]
    if da is not None and (da.dtype != torch.float32 or da.shape != (B, H, T)):
        _fail(f"da: must be float32 [B,H,T] = {(B, H, T)}, got {da.dtype} {tuple(da.shape)}")
    for name, t in (("da_carry", da_carry), ("da_carry_out", da_carry_out)):
        if t is not None and (t.dtype != torch.float32 or t.shape != (B, H) or
                              not t.is_contiguous()):
            _fail(f"{name}: must be contiguous float32 [B,H] = {(B, H)}")
    kind, dec = _decay(decay)
    d = _desc_of(q, v, kind, odt)
    _check_buffer("states", states, states_bytes(d))
    if workspace is not None:
        _check_buffer("workspace", workspace, bwd_da_workspace_bytes(d))
    _check_device(q, *devs)
    dq, dk, dv = _new_act(q, DK, odt, dq), _new_act(q, DK, odt, dk), _new_act(q, DV, odt, dv)
    dS_in = _state_out(q, B, H, DK, DV, dS_in)
    da = torch.empty(B, H, T, dtype=torch.float32, device=q.device) if da is None else da
    if da_carry_out is None:
        da_carry_out = torch.empty(B, H, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(bwd_da_workspace_bytes(d), 16), dtype=torch.uint8,
                                device=q.device)
    rc = _lib().linrec_bwd_da(context(q.device.index), ctypes.byref(d), _act(q), _act(k), _act(v),
                              dec, _ptr(states), _act(dO), _ptr(dS_out), _act(dq), _act(dk),
                              _act(dv), _ptr(dS_in), Tensor(da.data_ptr(), da.stride(0),
                                                            da.stride(1), da.stride(2)),
                              _ptr(da_carry), _ptr(da_carry_out), _ptr(workspace),
                              _stream(q.device))
    _check(rc, "linrec_bwd_da")
    return dq, dk, dv, dS_in, da, da_carry_out


def fwd_seq(q, k, v, decay, lengths: Sequence[int], S_in=None, *, o=None, S_out=None,
            states=None, out_dtype=None):
    """Sequence accumulation forward over consecutive pieces (native driver).

    Returns (o, S_out, states) with states covering the whole sequence."""
    odt = _out_dtype(q, out_dtype, o)
    devs = _validate(q, k, v, decay, outs=_outs(q, v, odt, o=o), states_in=(("S_in", S_in),),
              states_out=(("S_out", S_out),), extra=(("states", states),))
    lengths = _piece_lengths(lengths, q.shape[2])
    kind, dec = _decay(decay)
    d = _desc_of(q, v, kind, odt)
    B, H, T, dk = q.shape
    dv = v.shape[3]
    if states is not None:
        _check_buffer("states", states, seq_states_bytes(d, lengths))
    _check_device(q, *devs)
    o = _new_act(q, dv, odt, o)
    S_out = _state_out(q, B, H, dk, dv, S_out)
    if states is None:
        states = torch.empty(max(seq_states_bytes(d, lengths), 16), dtype=torch.uint8,
                             device=q.device)
    arr = (ctypes.c_int32 * len(lengths))(*lengths)
    rc = _lib().linrec_fwd_seq(context(q.device.index), ctypes.byref(d), len(lengths), arr,
                               _act(q), _act(k), _act(v), dec, _ptr(S_in), _act(o),
                               _ptr(S_out), _ptr(states), _stream(q.device))
    _check(rc, "linrec_fwd_seq")
    return o, S_out, states


def bwd_seq(q, k, v, decay, lengths: Sequence[int], states, dO, dS_out=None, *, dq=None,
            dk=None, dv=None, dS_in=None, workspace=None, out_dtype=None):
    """Sequence accumulation backward (pieces in reverse, dS carried back)."""
    odt = _out_dtype(q, out_dtype, dq)
    devs = _validate(q, k, v, decay, dO=dO, outs=_outs(q, v, odt, dq=dq, dk=dk, dv=dv),
              states_in=(("dS_out", dS_out),), states_out=(("dS_in", dS_in),),
              extra=(("states", states), ("workspace", workspace)))
    lengths = _piece_lengths(lengths, q.shape[2])
    kind, dec = _decay(decay)
    d = _desc_of(q, v, kind, odt)
    B, H, T, DK = q.shape
    DV = v.shape[3]
    _check_buffer("states", states, seq_states_bytes(d, lengths))
    if workspace is not None:
        _check_buffer("workspace", workspace, bwd_seq_workspace_bytes(d, lengths))
    _check_device(q, *devs)
    dq, dk, dv = _new_act(q, DK, odt, dq), _new_act(q, DK, odt, dk), _new_act(q, DV, odt, dv)
    dS_in = _state_out(q, B, H, DK, DV, dS_in)
    if workspace is None:
        workspace = torch.empty(max(bwd_seq_workspace_bytes(d, lengths), 16), dtype=torch.uint8,
                                device=q.device)
    arr = (ctypes.c_int32 * len(lengths))(*lengths)
    rc = _lib().linrec_bwd_seq(context(q.device.index), ctypes.byref(d), len(lengths), arr,
                               _act(q), _act(k), _act(v), dec, _ptr(states), _act(dO),
                               _ptr(dS_out), _act(dq), _act(dk), _act(dv), _ptr(dS_in),
                               _ptr(workspace), _stream(q.device))
    _check(rc, "linrec_bwd_seq")
    return dq, dk, dv, dS_in


# ----------------------------------------------------------------- delta rule

def delta_workspace_bytes(d: Desc) -> int:
    return int(_lib().linrec_delta_workspace_bytes(ctypes.byref(d)))


def delta_saved_bytes(d: Desc) -> int:
    return int(_lib().linrec_delta_saved_bytes(ctypes.byref(d)))


def delta_bwd_workspace_bytes(d: Desc) -> int:
    return int(_lib().linrec_delta_bwd_workspace_bytes(ctypes.byref(d)))


def _beta_arg(name, x, B, H, T):
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.shape != (B, H, T):
        _fail(f"{name}: must be float32 [B,H,T] = {(B, H, T)}")
    st = x.stride()
    return Tensor(x.data_ptr(), st[0], st[1], st[2])


def delta_fwd(q, k, v, beta, decay=None, S_in=None, *, o=None, S_out=None, saved=None,
              save=False, workspace=None, out_dtype=None):
    """Gated delta rule, forward over one piece (linrec_delta_fwd):
    S_t = a_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t, o_t = q_t S_t.
    beta: fp32 [B,H,T].  With save=True (or a `saved` buffer) the states and
    values the backward needs are kept.  Returns (o, S_out, saved or None)."""
    odt = _out_dtype(q, out_dtype, o)
    devs = _validate(q, k, v, decay, outs=_outs(q, v, odt, o=o), states_in=(("S_in", S_in),),
                     states_out=(("S_out", S_out),),
                     extra=(("beta", beta), ("workspace", workspace), ("saved", saved)))
    B, H, T, DK = q.shape
    DV = v.shape[3]
    barg = _beta_arg("beta", beta, B, H, T)
    kind, dec = _decay(decay)
    d = _desc_of(q, v, kind, odt)
    if workspace is not None:
        _check_buffer("workspace", workspace, delta_workspace_bytes(d))
    if saved is not None:
        _check_buffer("saved", saved, delta_saved_bytes(d))
    _check_device(q, *devs)
    o = _new_act(q, DV, odt, o)
    S_out = _state_out(q, B, H, DK, DV, S_out)
    if workspace is None:
        workspace = torch.empty(max(delta_workspace_bytes(d), 16), dtype=torch.uint8, device=q.device)
    if saved is None and save:
        saved = torch.empty(max(delta_saved_bytes(d), 16), dtype=torch.uint8, device=q.device)
    rc = _lib().linrec_delta_fwd(context(q.device.index), ctypes.byref(d), _act(q), _act(k), _act(v),
                                 barg, dec, _ptr(S_in), _act(o), _ptr(S_out), _ptr(saved),
                                 _ptr(workspace), _stream(q.device))
    _check(rc, "linrec_delta_fwd")
    return o, S_out, saved


def delta_bwd(q, k, v, beta, decay, saved, dO, dS_out=None, *, dq=None, dk=None, dv=None,
              dbeta=None, dS_in=None, workspace=None, out_dtype=None):
    """Gated delta rule, backward over one piece (linrec_delta_bwd) from the
    forward's `saved` buffer.  Returns (dq, dk, dv, dbeta, dS_in)."""
    odt = _out_dtype(q, out_dtype, dq)
    devs = _validate(q, k, v, decay, dO=dO, outs=_outs(q, v, odt, dq=dq, dk=dk, dv=dv),
                     states_in=(("dS_out", dS_out),), states_out=(("dS_in", dS_in),),
                     extra=(("beta", beta), ("saved", saved), ("workspace", workspace),
                            ("dbeta", dbeta)))
    B, H, T, DK = q.shape
    DV = v.shape[3]
    barg = _beta_arg("beta", beta, B, H, T)
    kind, dec = _decay(decay)
    d = _desc_of(q, v, kind, odt)
    _check_buffer("saved", saved, delta_saved_bytes(d))
    if workspace is not None:
        _check_buffer("workspace", workspace, delta_bwd_workspace_bytes(d))
    if dbeta is not None:
        _beta_arg("dbeta", dbeta, B, H, T)
    _check_device(q, *devs)
    dq, dk, dv = _new_act(q, DK, odt, dq), _new_act(q, DK, odt, dk), _new_act(q, DV, odt, dv)
    dS_in = _state_out(q, B, H, DK, DV, dS_in)
    if dbeta is None:
        dbeta = torch.empty(B, H, T, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(delta_bwd_workspace_bytes(d), 16), dtype=torch.uint8,
                                device=q.device)
    rc = _lib().linrec_delta_bwd(context(q.device.index), ctypes.byref(d), _act(q), _act(k), _act(v),
                                 barg, dec, _ptr(saved), _act(dO), _ptr(dS_out), _act(dq), _act(dk),
                                 _act(dv), _beta_arg("dbeta", dbeta, B, H, T), _ptr(dS_in),
                                 _ptr(workspace), _stream(q.device))
    _check(rc, "linrec_delta_bwd")
    return dq, dk, dv, dbeta, dS_in


def _lengths_arg(lengths):
    return (ctypes.c_int32 * len(lengths))(*lengths)


def delta_seq_saved_bytes(d: Desc, lengths: Sequence[int]) -> int:
    return int(_lib().linrec_delta_seq_saved_bytes(ctypes.byref(d), len(lengths),
                                                   _lengths_arg(lengths)))


def delta_fwd_seq_workspace_bytes(d: Desc, lengths: Sequence[int]) -> int:
    return int(_lib().linrec_delta_fwd_seq_workspace_bytes(ctypes.byref(d), len(lengths),
                                                           _lengths_arg(lengths)))


def delta_bwd_seq_workspace_bytes(d: Desc, lengths: Sequence[int]) -> int:
    return int(_lib().linrec_delta_bwd_seq_workspace_bytes(ctypes.byref(d), len(lengths),
                                                           _lengths_arg(lengths)))


def delta_fwd_seq(q, k, v, beta, decay, lengths: Sequence[int], S_in=None, *, o=None,
                  S_out=None, saved=None, save=False, workspace=None, out_dtype=None):
    """Gated delta rule forward over consecutive pieces, S carried (native
    driver, linrec_delta_fwd_seq).  Returns (o, S_out, saved or None)."""
    odt = _out_dtype(q, out_dtype, o)
    devs = _validate(q, k, v, decay, outs=_outs(q, v, odt, o=o), states_in=(("S_in", S_in),),
                     states_out=(("S_out", S_out),),
                     extra=(("beta", beta), ("workspace", workspace), ("saved", saved)))
    lengths = _piece_lengths(lengths, q.shape[2])
    B, H, T, DK = q.shape
    DV = v.shape[3]
    barg = _beta_arg("beta", beta, B, H, T)
    kind, dec = _decay(decay)
    d = _desc_of(q, v, kind, odt)
    if workspace is not None:
        _check_buffer("workspace", workspace, delta_fwd_seq_workspace_bytes(d, lengths))
    if saved is not None:
        _check_buffer("saved", saved, delta_seq_saved_bytes(d, lengths))
    _check_device(q, *devs)
    o = _new_act(q, DV, odt, o)
    S_out = _state_out(q, B, H, DK, DV, S_out)
    if workspace is None:
        workspace = torch.empty(max(delta_fwd_seq_workspace_bytes(d, lengths), 16),
                                dtype=torch.uint8, device=q.device)
    if saved is None and save:
        saved = torch.empty(max(delta_seq_saved_bytes(d, lengths), 16), dtype=torch.uint8,
                            device=q.device)
    rc = _lib().linrec_delta_fwd_seq(context(q.device.index), ctypes.byref(d), len(lengths),
                                     _lengths_arg(lengths), _act(q), _act(k), _act(v), barg, dec,
                                     _ptr(S_in), _act(o), _ptr(S_out), _ptr(saved),
                                     _ptr(workspace), _stream(q.device))
    _check(rc, "linrec_delta_fwd_seq")
    return o, S_out, saved


def delta_bwd_seq(q, k, v, beta, decay, lengths: Sequence[int], saved, dO, dS_out=None, *,
                  dq=None, dk=None, dv=None, dbeta=None, dS_in=None, workspace=None,
                  out_dtype=None):
    """Gated delta rule backward over consecutive pieces in reverse, dS
    carried (linrec_delta_bwd_seq), from delta_fwd_seq's `saved`.  Returns
    (dq, dk, dv, dbeta, dS_in)."""
    odt = _out_dtype(q, out_dtype, dq)
    devs = _validate(q, k, v, decay, dO=dO, outs=_outs(q, v, odt, dq=dq, dk=dk, dv=dv),
                     states_in=(("dS_out", dS_out),), states_out=(("dS_in", dS_in),),
                     extra=(("beta", beta), ("saved", saved), ("workspace", workspace),
                            ("dbeta", dbeta)))
    lengths = _piece_lengths(lengths, q.shape[2])
    B, H, T, DK = q.shape
    DV = v.shape[3]
    barg = _beta_arg("beta", beta, B, H, T)
    kind, dec = _decay(decay)
    d = _desc_of(q, v, kind, odt)
    _check_buffer("saved", saved, delta_seq_saved_bytes(d, lengths))
    if workspace is not None:
        _check_buffer("workspace", workspace, delta_bwd_seq_workspace_bytes(d, lengths))
    if dbeta is not None:
        _beta_arg("dbeta", dbeta, B, H, T)
    _check_device(q, *devs)
    dq, dk, dv = _new_act(q, DK, odt, dq), _new_act(q, DK, odt, dk), _new_act(q, DV, odt, dv)
    dS_in = _state_out(q, B, H, DK, DV, dS_in)
    if dbeta is None:
        dbeta = torch.empty(B, H, T, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(delta_bwd_seq_workspace_bytes(d, lengths), 16),
                                dtype=torch.uint8, device=q.device)
    rc = _lib().linrec_delta_bwd_seq(context(q.device.index), ctypes.byref(d), len(lengths),
                                     _lengths_arg(lengths), _act(q), _act(k), _act(v), barg, dec,
                                     _ptr(saved), _act(dO), _ptr(dS_out), _act(dq), _act(dk),
                                     _act(dv), _beta_arg("dbeta", dbeta, B, H, T), _ptr(dS_in),
                                     _ptr(workspace), _stream(q.device))
    _check(rc, "linrec_delta_bwd_seq")
    return dq, dk, dv, dbeta, dS_in


def piece_loop(q, k, v, decay, lengths: Sequence[int], S_in=None, dO=None, dS_out=None,
               out_dtype=None):
    """Sequence accumulation through the per-piece calls, one call per piece
    (S carried forward, dS carried back).  Returns (o, S_out, dq, dk, dv, dS_in)
    -- the gradients are None when dO is None."""
    B, H, T, DK = q.shape
    DV = v.shape[3]
    odt = q.dtype if out_dtype is None else out_dtype
    o = torch.empty(B, H, T, DV, dtype=odt, device=q.device)
    S = S_in
    bounds = [0]
    for L in lengths:
        bounds.append(bounds[-1] + L)

    def dsl(i):
        if decay is None or decay.dim() == 1:
            return decay
        return decay[:, :, bounds[i]:bounds[i + 1]]

    saved = []
    for i in range(len(lengths)):
        sl = slice(bounds[i], bounds[i + 1])
        _, S, st = fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], dsl(i), S, o=o[:, :, sl])
        saved.append(st)
    if dO is None:
        return o, S, None, None, None, None
    dq, dk, dv = (torch.empty(x.shape, dtype=odt, device=q.device) for x in (q, k, v))
    dS = dS_out
    for i in reversed(range(len(lengths))):
        sl = slice(bounds[i], bounds[i + 1])
        _, _, _, dS = bwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], dsl(i), saved[i],
                          dO[:, :, sl], dS, dq=dq[:, :, sl], dk=dk[:, :, sl], dv=dv[:, :, sl])
    return o, S, dq, dk, dv, dS
