"""Draw the synthetic inputs of a Workload, on the host or in place on the GPU.

Both fillers evaluate the element definition in ``csrc/synth_common.h``; the
host one is used for everything the CPU oracle reads (and for the small router
matrix, which is uploaded), the device one for the large expert tensors and x.

Tensor layouts (row-major):
  x  [T, d]     Wr [N, d]     W1 [N, F, d]   b1 [N, F]   W2 [N, d, F]   b2 [N, d]
  (GEGLU experts: W1 [N, 2F, d] and b1 [N, 2F])
bf16 tensors travel as uint16 bit patterns on the host.
"""
from __future__ import annotations

import math
import os

import numpy as np

from . import _native
from .workloads import Workload

STREAMS = {"x": 1, "Wr": 2, "W1": 3, "b1": 4, "W2": 5, "b2": 6}
BF16_ONE = 0x3F80  # bit pattern of 1.0 in bfloat16


def shape_of(w: Workload, name: str) -> tuple:
    return {
        "x": (w.T, w.d),
        "Wr": (w.N, w.d),
        "W1": (w.N, 2 * w.F if w.glu else w.F, w.d),
        "b1": (w.N, 2 * w.F if w.glu else w.F),
        "W2": (w.N, w.d, w.F),
        "b2": (w.N, w.d),
    }[name]


def sigma_of(w: Workload, name: str) -> float:
    if name == "x":
        return w.x_sigma
    if name in ("Wr", "W1", "W2"):
        return w.w_sigma
    return w.bias_sigma


def is_bf16(w: Workload, name: str) -> bool:
    # The router matrix is always fp32; everything else follows the workload dtype.
    return name != "Wr" and w.dtype == "bf16"


def zipf_router_bias(w: Workload) -> np.ndarray:
    """Per-expert router bias beta * sigma_z * ln(pi_i), pi_i ~ (i+1)^-s (fp32).

    sigma_z = w_sigma * sqrt(d - 1) is the spread of the other d-1 logit terms,
    so beta sets the bias in units of the random logit's standard deviation.
    The bias enters through x[:, d-1] = 1 and Wr[:, d-1] = bias.
    """
    assert w.zipf_s is not None
    i = np.arange(w.N, dtype=np.float64)
    pi = (i + 1.0) ** (-w.zipf_s)
    pi /= pi.sum()
    sigma_z = w.w_sigma * math.sqrt(w.d - 1)
    return (w.zipf_beta * sigma_z * np.log(pi)).astype(np.float32)


def _threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(16, os.cpu_count() or 1))


def host_array(w: Workload, name: str, start: int = 0, count: int | None = None) -> np.ndarray:
    """Flat elements [start, start+count) of tensor `name` (uint16 bits or fp32)."""
    total = int(np.prod(shape_of(w, name)))
    if count is None:
        count = total - start
    if start < 0 or count < 0 or start + count > total:
        raise ValueError(f"slice [{start}, {start + count}) outside {name} of {total} elements")
    bf = is_bf16(w, name)
    out = np.empty(count, dtype=np.uint16 if bf else np.float32)
    _native.fill_host(out, start, w.seed, STREAMS[name], sigma_of(w, name), bf, _threads())
    if w.zipf_s is not None and name in ("x", "Wr"):
        # Column d-1 carries the popularity bias: x[:, d-1] = 1, Wr[:, d-1] = bias.
        idx = np.arange(start, start + count, dtype=np.int64)
        col = (idx % w.d) == (w.d - 1)
        if name == "x":
            out[col] = BF16_ONE if bf else np.float32(1.0)
        else:
            out[col] = zipf_router_bias(w)[idx[col] // w.d]
    return out


def host_inputs(w: Workload, max_elems: int = 1 << 29) -> dict:
    """All six tensors on the host (shaped).  Biases are None when absent."""
    out = {}
    for name in STREAMS:
        if name in ("b1", "b2") and not w.has_bias:
            out[name] = None
            continue
        shp = shape_of(w, name)
        n = int(np.prod(shp))
        if n > max_elems:
            raise MemoryError(f"{name} has {n} elements; draw it per expert instead")
        out[name] = host_array(w, name).reshape(shp)
    return out


def host_rows(w: Workload, name: str, rows: np.ndarray) -> np.ndarray:
    """Selected leading-axis rows of x or Wr (shaped [len(rows), d])."""
    shp = shape_of(w, name)
    width = int(np.prod(shp[1:]))
    rows = np.asarray(rows, dtype=np.int64)
    parts = [host_array(w, name, int(r) * width, width) for r in rows]
    if not parts:
        return np.empty((0,) + tuple(shp[1:]), dtype=np.uint16 if is_bf16(w, name) else np.float32)
    return np.stack(parts).reshape((len(rows),) + tuple(shp[1:]))


def expert_weights_host(w: Workload, e: int) -> dict:
    """Expert e's W1 [F1, d], b1 [F1], W2 [d, F], b2 [d] (None when absent); F1 = F, or
    2F for GEGLU experts."""
    F1 = 2 * w.F if w.glu else w.F
    Fd = w.F * w.d
    out = {
        "W1": host_array(w, "W1", e * F1 * w.d, F1 * w.d).reshape(F1, w.d),
        "W2": host_array(w, "W2", e * Fd, Fd).reshape(w.d, w.F),
        "b1": None,
        "b2": None,
    }
    if w.has_bias:
        out["b1"] = host_array(w, "b1", e * F1, F1)
        out["b2"] = host_array(w, "b2", e * w.d, w.d)
    return out


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def decode(a, w: Workload | None = None, name: str | None = None) -> np.ndarray | None:
    """Host tensor (uint16 bf16 bits or fp32) -> float64 values, exactly."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def device_inputs(w: Workload, device: str = "cuda") -> dict:
    """All six tensors resident on the GPU (torch tensors; biases None when absent).

    x and the expert tensors are drawn in place by the device filler; Wr is
    drawn on the host and uploaded, so the oracle and the GPU see the same bytes.
    """
    import torch

    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    stream = torch.cuda.current_stream(device).cuda_stream
    out = {}
    for name in STREAMS:
        if name in ("b1", "b2") and not w.has_bias:
            out[name] = None
            continue
        shp = shape_of(w, name)
        if name == "Wr":
            out[name] = torch.from_numpy(host_array(w, "Wr").reshape(shp)).to(device)
            continue
        t = torch.empty(shp, dtype=tdt, device=device)
        _native.fill_device(t.data_ptr(), t.numel(), 0, w.seed, STREAMS[name], sigma_of(w, name),
                            is_bf16(w, name), stream)
        out[name] = t
    if w.zipf_s is not None:
        out["x"][:, w.d - 1] = 1.0
    torch.cuda.synchronize(device)
    return out
