"""ctypes binding of libswitchffn.so: the C-ABI names, argument marshalling only.

Tensors are torch tensors in device memory (torch provides the allocations
and the stream); every step of the layer runs in the library's HIP kernels.
The library must be built (``__graft_entry__.build()``); loading fails loudly
when it is missing.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswitchffn.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "switch_ffn.h")

SFFN_OK = 0
SFFN_EINVAL = -1
SFFN_EDTYPE = -2
SFFN_EWORKSPACE = -3
SFFN_EUNSUPPORTED = -4
SFFN_EHIP = -5
SFFN_ESCRATCH = -6
SFFN_FP32 = 0
SFFN_BF16 = 1
SFFN_NO_RESIDUAL = 1
SFFN_REROUTE_OVERFLOW = 2
SFFN_GEGLU = 4


class sffn_stats(ctypes.Structure):
    _fields_ = [("expert_count", ctypes.c_void_p), ("accepted_count", ctypes.c_void_p),
                ("n_dropped", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_FWD_ARGS = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_double, ctypes.c_int,
             _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]

_lib = None


def load_library(path: str = LIB_PATH):
    """ctypes handle of a libswitchffn build with argument types set."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: the HIP library must be built "
                           "(__graft_entry__.build()); there is no fallback path")
    # One HIP runtime per process: torch ships its own libamdhip64 (soname
    # libamdhip64.so.7) and asks for it by another name, so if this library
    # loaded the system's copy first, torch would load a second runtime beside
    # it and the two would not share the device.  With torch loaded first, the
    # library's libamdhip64.so.7 resolves to torch's copy.
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    L.switch_ffn_capacity.restype = ctypes.c_int64
    L.switch_ffn_capacity.argtypes = [_I64, _I64, ctypes.c_double]
    L.switch_ffn_workspace_bytes.restype = ctypes.c_size_t
    L.switch_ffn_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_double,
                                             ctypes.c_int]
    L.switch_ffn_forward.restype = ctypes.c_int
    L.switch_ffn_forward.argtypes = _FWD_ARGS
    L.switch_ffn_forward_ex.restype = ctypes.c_int
    L.switch_ffn_forward_ex.argtypes = _FWD_ARGS + [ctypes.c_uint32, ctypes.POINTER(sffn_stats)]
    L.switch_ffn_workspace_bytes_topk.restype = ctypes.c_size_t
    L.switch_ffn_workspace_bytes_topk.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_double,
                                                  ctypes.c_int, ctypes.c_int]
    L.switch_ffn_forward_topk.restype = ctypes.c_int
    L.switch_ffn_forward_topk.argtypes = (_FWD_ARGS[:11] + [ctypes.c_int] + _FWD_ARGS[11:] +
                                          [ctypes.c_uint32, ctypes.POINTER(sffn_stats), _P])
    L.switch_ffn_backward_workspace_bytes.restype = ctypes.c_size_t
    L.switch_ffn_backward_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_double,
                                                      ctypes.c_int]
    L.switch_ffn_backward.restype = ctypes.c_int
    L.switch_ffn_backward.argtypes = (_FWD_ARGS[:12] + [_P, _P, _P, ctypes.c_size_t, _P,
                                                        ctypes.c_float] + [_P] * 6 +
                                      [_P, ctypes.c_size_t, _P, _P])
    L.switch_ffn_backward_num_stages.restype = ctypes.c_int
    L.switch_ffn_backward_num_stages.argtypes = []
    L.switch_ffn_backward_stage_name.restype = ctypes.c_char_p
    L.switch_ffn_backward_stage_name.argtypes = [ctypes.c_int]
    L.switch_ffn_num_stages.restype = ctypes.c_int
    L.switch_ffn_num_stages.argtypes = []
    L.switch_ffn_stage_name.restype = ctypes.c_char_p
    L.switch_ffn_stage_name.argtypes = [ctypes.c_int]
    L.switch_ffn_noalloc_scratch_bytes.restype = ctypes.c_size_t
    L.switch_ffn_noalloc_scratch_bytes.argtypes = []
    L.switch_ffn_forward_noalloc.restype = ctypes.c_int
    L.switch_ffn_forward_noalloc.argtypes = _FWD_ARGS[:17] + [_P]
    L.switch_ffn_status_string.restype = ctypes.c_char_p
    L.switch_ffn_status_string.argtypes = [ctypes.c_int]
    return L


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def header_functions() -> list:
    """Names of the functions include/switch_ffn.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(switch_ffn_\w+)\s*\(", text)))


def switch_ffn_capacity(T: int, N: int, CF: float) -> int:
    return lib().switch_ffn_capacity(T, N, CF)


def switch_ffn_workspace_bytes(T, d, F, N, CF, dtype) -> int:
    return lib().switch_ffn_workspace_bytes(T, d, F, N, CF, dtype)


def switch_ffn_workspace_bytes_topk(T, d, F, N, CF, k, dtype) -> int:
    return lib().switch_ffn_workspace_bytes_topk(T, d, F, N, CF, k, dtype)


def switch_ffn_backward_workspace_bytes(T, d, F, N, CF, dtype) -> int:
    return lib().switch_ffn_backward_workspace_bytes(T, d, F, N, CF, dtype)


def switch_ffn_backward_num_stages() -> int:
    return lib().switch_ffn_backward_num_stages()


def switch_ffn_backward_stage_name(i: int):
    s = lib().switch_ffn_backward_stage_name(i)
    return None if s is None else s.decode()


def switch_ffn_num_stages() -> int:
    return lib().switch_ffn_num_stages()


def switch_ffn_stage_name(i: int):
    s = lib().switch_ffn_stage_name(i)
    return None if s is None else s.decode()


def switch_ffn_noalloc_scratch_bytes() -> int:
    return lib().switch_ffn_noalloc_scratch_bytes()


def switch_ffn_forward_noalloc(x, Wr, W1, b1, W2, b2, CF: float, *, y, expert_idx, slot, gate,
                               aux_loss, stream=None, check: bool = True) -> int:
    """The allocation-free forward into caller-given outputs (no workspace argument: the
    library's built-in scratch).  Allocates nothing; returns the status."""
    import torch

    T, d, F, N = _check_layer(x, Wr, W1, b1, W2, b2, False)
    dev = x.device
    _check("y", y, (T, d), x.dtype, dev)
    _check("expert_idx", expert_idx, (T,), torch.int32, dev)
    _check("slot", slot, (T,), torch.int32, dev)
    _check("gate", gate, (T,), torch.float32, dev)
    _check("aux_loss", aux_loss, (1,), torch.float32, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib().switch_ffn_forward_noalloc(
        _ptr(x), _ptr(Wr), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), T, d, F, N, CF,
        _dtype_code(x), _ptr(y), _ptr(expert_idx), _ptr(slot), _ptr(gate), _ptr(aux_loss),
        stream)
    if check and rc != SFFN_OK:
        raise RuntimeError(f"switch_ffn_forward_noalloc failed ({rc}): "
                           f"{switch_ffn_status_string(rc)}")
    return rc


def switch_ffn_status_string(status: int) -> str:
    return lib().switch_ffn_status_string(status).decode()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SFFN_BF16
    if t.dtype == torch.float32:
        return SFFN_FP32
    raise TypeError(f"x must be float32 or bfloat16, not {t.dtype}")


def _check(name, t, shape, dtype, device, nullable=False):
    """A tensor argument as the C-ABI reads it: this shape and dtype, contiguous, on the
    layer's device (the library reads it through a raw pointer, so anything else would
    make it read the wrong bytes or past the allocation)."""
    if t is None:
        if nullable:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the layer's tensors on {device}")


def _check_workspace(name, ws, nbytes, device):
    import torch
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device != device:
        raise ValueError(f"{name} must be a contiguous uint8 tensor on {device}")
    if ws.numel() < nbytes:
        raise ValueError(f"{name} holds {ws.numel()} bytes, {nbytes} needed")


def _check_layer(x, Wr, W1, b1, W2, b2, glu: bool):
    """Shapes, dtypes, contiguity and device of the layer's inputs; returns T, d, F, N."""
    import torch
    if x.dim() != 2 or W2.dim() != 3 or Wr.dim() != 2:
        raise ValueError("x must be [T, d], Wr [N, d], W2 [N, d, F]")
    _dtype_code(x)
    T, d = x.shape
    N, F = Wr.shape[0], W2.shape[2]
    F1 = 2 * F if glu else F
    dev = x.device
    _check("x", x, (T, d), x.dtype, dev)
    _check("Wr", Wr, (N, d), torch.float32, dev)
    _check("W1", W1, (N, F1, d), x.dtype, dev)
    _check("b1", b1, (N, F1), x.dtype, dev, nullable=True)
    _check("W2", W2, (N, d, F), x.dtype, dev)
    _check("b2", b2, (N, d), x.dtype, dev, nullable=True)
    if dev.type != "cuda":
        raise ValueError(f"the layer's tensors must be GPU tensors, not on {dev}")
    return T, d, F, N


def switch_ffn_forward(x, Wr, W1, b1, W2, b2, CF: float, *, y=None, expert_idx=None, slot=None,
                       gate=None, aux_loss=None, workspace=None, stream=None, flags: int = 0,
                       stats=None, stage_events=None, check: bool = True, k: int = 1) -> dict:
    """Run the layer on device tensors; returns the output tensors (allocated when not given).

    x [T, d], Wr [N, d] fp32, W1 [N, F, d], b1 [N, F] | None, W2 [N, d, F], b2 [N, d] | None
    (flags with SFFN_GEGLU: W1 [N, 2F, d], b1 [N, 2F]).
    k: experts per token (1, or 2 for top-2 routing through switch_ffn_forward_topk; then
    expert_idx, slot and gate are [T, 2]).
    stats: optional dict of int32 device tensors 'expert_count' [N], 'accepted_count' [N],
    'n_dropped' [1].  stage_events: optional list of torch.cuda.Event (already recorded once
    so that the handle exists), switch_ffn_num_stages()+1 of them.
    """
    import torch

    if k not in (1, 2):
        raise ValueError("k must be 1 or 2")
    T, d, F, N = _check_layer(x, Wr, W1, b1, W2, b2, bool(flags & SFFN_GEGLU))
    dt = _dtype_code(x)
    dev = x.device
    shape = (T,) if k == 1 else (T, k)
    if y is None:
        y = torch.empty_like(x)
    if expert_idx is None:
        expert_idx = torch.empty(shape, dtype=torch.int32, device=dev)
    if slot is None:
        slot = torch.empty(shape, dtype=torch.int32, device=dev)
    if gate is None:
        gate = torch.empty(shape, dtype=torch.float32, device=dev)
    if aux_loss is None:
        aux_loss = torch.empty(1, dtype=torch.float32, device=dev)
    _check("y", y, (T, d), x.dtype, dev)
    _check("expert_idx", expert_idx, shape, torch.int32, dev)
    _check("slot", slot, shape, torch.int32, dev)
    _check("gate", gate, shape, torch.float32, dev)
    _check("aux_loss", aux_loss, (1,), torch.float32, dev)
    nbytes = switch_ffn_workspace_bytes_topk(T, d, F, N, CF, k, dt)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check_workspace("workspace", workspace, nbytes, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    st = None
    if stats is not None:
        for key, n in (("expert_count", N), ("accepted_count", N), ("n_dropped", 1)):
            _check(f"stats['{key}']", stats.get(key), (n,), torch.int32, dev, nullable=True)
        st = sffn_stats(_ptr(stats.get("expert_count")), _ptr(stats.get("accepted_count")),
                        _ptr(stats.get("n_dropped")))
    ev = None
    if stage_events is not None:
        handles = [e.cuda_event for e in stage_events]
        if any(h == 0 for h in handles):
            raise ValueError("stage events must be recorded once before use (handle is null)")
        ev = (ctypes.c_void_p * len(handles))(*handles)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(x), _ptr(Wr), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), T, d, F, N, CF, dt,
            _ptr(y), _ptr(expert_idx), _ptr(slot), _ptr(gate), _ptr(aux_loss), _ptr(workspace),
            ws_bytes, stream)
    if k != 1 or ev is not None:
        name = "switch_ffn_forward_topk"
        rc = lib().switch_ffn_forward_topk(*args[:11], k, *args[11:], flags,
                                           None if st is None else ctypes.byref(st),
                                           None if ev is None else ctypes.cast(ev, ctypes.c_void_p))
    elif flags == 0 and st is None:
        name = "switch_ffn_forward"
        rc = lib().switch_ffn_forward(*args)
    else:
        name = "switch_ffn_forward_ex"
        rc = lib().switch_ffn_forward_ex(*args, flags, None if st is None else ctypes.byref(st))
    if check and rc != SFFN_OK:
        raise RuntimeError(f"{name} failed ({rc}): {switch_ffn_status_string(rc)}")
    # k and flags travel with the workspace: the backward reads only a top-1 forward's
    # workspace without rerouting or GEGLU experts (the library checks its tag as well).
    return {"status": rc, "y": y, "expert_idx": expert_idx, "slot": slot, "gate": gate,
            "aux_loss": aux_loss, "workspace": workspace, "k": k, "flags": flags}


# forward_ex's and forward_topk's extra arguments are keyword arguments of switch_ffn_forward.
switch_ffn_forward_ex = switch_ffn_forward
switch_ffn_forward_topk = switch_ffn_forward


def switch_ffn_backward(x, Wr, W1, b1, W2, b2, CF: float, fwd: dict, dy, d_aux: float = 0.0, *,
                        dx=None, dWr=None, dW1=None, db1=None, dW2=None, db2=None,
                        workspace=None, stream=None, stage_events=None,
                        check: bool = True) -> dict:
    """Gradients of the top-1 ReLU layer (switch_ffn_backward).

    fwd: what switch_ffn_forward returned for the same inputs (its expert_idx, slot and
    workspace, untouched since).  dy [T, d] like x; d_aux = dL/d(aux_loss).  Returns dx,
    dWr (fp32), dW1, db1, dW2, db2 (db1/db2 None when the bias is absent).
    """
    import torch

    if fwd.get("k", 1) != 1 or fwd.get("flags", 0) & (SFFN_REROUTE_OVERFLOW | SFFN_GEGLU):
        raise ValueError("the backward pass covers the top-1 layer with ReLU experts: fwd must "
                         "come from a k = 1 forward without SFFN_REROUTE_OVERFLOW or SFFN_GEGLU")
    T, d, F, N = _check_layer(x, Wr, W1, b1, W2, b2, False)
    dt = _dtype_code(x)
    dev = x.device
    _check("dy", dy, (T, d), x.dtype, dev)
    _check("fwd['expert_idx']", fwd["expert_idx"], (T,), torch.int32, dev)
    _check("fwd['slot']", fwd["slot"], (T,), torch.int32, dev)
    dx = torch.empty_like(x) if dx is None else dx
    dWr = torch.empty((N, d), dtype=torch.float32, device=dev) if dWr is None else dWr
    dW1 = torch.empty_like(W1) if dW1 is None else dW1
    dW2 = torch.empty_like(W2) if dW2 is None else dW2
    if db1 is None and b1 is not None:
        db1 = torch.empty_like(b1)
    if db2 is None and b2 is not None:
        db2 = torch.empty_like(b2)
    _check("dx", dx, (T, d), x.dtype, dev)
    _check("dWr", dWr, (N, d), torch.float32, dev)
    _check("dW1", dW1, (N, F, d), x.dtype, dev)
    _check("dW2", dW2, (N, d, F), x.dtype, dev)
    _check("db1", db1, (N, F), x.dtype, dev, nullable=True)
    _check("db2", db2, (N, d), x.dtype, dev, nullable=True)
    _check_workspace("fwd['workspace']", fwd["workspace"],
                     switch_ffn_workspace_bytes(T, d, F, N, CF, dt), dev)
    nbytes = switch_ffn_backward_workspace_bytes(T, d, F, N, CF, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check_workspace("workspace", workspace, nbytes, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ev = None
    if stage_events is not None:
        handles = [e.cuda_event for e in stage_events]
        if any(h == 0 for h in handles):
            raise ValueError("stage events must be recorded once before use (handle is null)")
        ev = (ctypes.c_void_p * len(handles))(*handles)
    fws = fwd["workspace"]
    rc = lib().switch_ffn_backward(
        _ptr(x), _ptr(Wr), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), T, d, F, N, CF, dt,
        _ptr(fwd["expert_idx"]), _ptr(fwd["slot"]), _ptr(fws), fws.numel() * fws.element_size(),
        _ptr(dy), float(d_aux), _ptr(dx), _ptr(dWr), _ptr(dW1), _ptr(db1), _ptr(dW2), _ptr(db2),
        _ptr(workspace), workspace.numel() * workspace.element_size(), stream,
        None if ev is None else ctypes.cast(ev, ctypes.c_void_p))
    if check and rc != SFFN_OK:
        raise RuntimeError(f"switch_ffn_backward failed ({rc}): {switch_ffn_status_string(rc)}")
    return {"status": rc, "dx": dx, "dWr": dWr, "dW1": dW1, "db1": db1, "dW2": dW2, "db2": db2,
            "workspace": workspace}
