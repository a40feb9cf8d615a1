"""GPU parity of the backward pass (switch_ffn_backward, top-1 ReLU layer) against the
CPU oracle's backward on the same seeded inputs, replaying the GPU's routing: dx, dWr,
dW1, db1, dW2, db2 within rel-L2 2e-2 (bf16 layer) or 1e-5 (fp32 layer); experts without
tokens get exactly zero gradients; two calls agree bit for bit."""
import numpy as np
import pytest

import oracle
import switchffn_synth as synth
from gpu_harness import announce, host_x, rel_l2

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": 2e-2, "fp32": 1e-5}


def _dy(w, seed=1234):
    """dL/dy ~ N(0, 1), seeded, in the layer's dtype (host bits and float64 values)."""
    v = np.random.default_rng(seed).standard_normal((w.T, w.d)).astype(np.float32)
    if w.dtype == "bf16":
        u = v.view(np.uint32)
        bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        return bits, synth.bf16_bits_to_f32(bits).astype(np.float64)
    return v, v.astype(np.float64)


def _host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(
            np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def _case(w, d_aux=0.37, sampled=False, twice=False, expert_dx=False):
    """expert_dx: also hold dx - dy (the expert and router terms) to the tolerance; for
    weights large enough that those terms are not lost in dy's rounding."""
    import torch

    import sparse_mixture_experts_switchffn_amd as sffn

    announce(f"backward d_aux={d_aux} " + w.describe())
    dev_in = synth.device_inputs(w, DEV)
    args = (dev_in["x"], dev_in["Wr"], dev_in["W1"], dev_in["b1"], dev_in["W2"], dev_in["b2"])
    fwd = sffn.switch_ffn_forward(*args, w.CF)
    dy_raw, dy64 = _dy(w)
    if w.dtype == "bf16":
        dy = torch.from_numpy(dy_raw.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        dy = torch.from_numpy(dy_raw).to(DEV)
    g = sffn.switch_ffn_backward(*args, w.CF, fwd, dy, d_aux)
    torch.cuda.synchronize()
    if twice:
        g2 = sffn.switch_ffn_backward(*args, w.CF, fwd, dy, d_aux)
        torch.cuda.synchronize()
        for k in ("dx", "dWr", "dW1", "dW2", "db1", "db2"):
            if g[k] is not None:
                assert torch.equal(g[k], g2[k]), f"{k} differs between two calls"
    eidx = fwd["expert_idx"].cpu().numpy().astype(np.int64)
    x64 = synth.decode(host_x(w))
    Wr64 = synth.decode(synth.host_array(w, "Wr").reshape(w.N, w.d))

    def experts(e):
        ew = synth.expert_weights_host(w, e)
        return (synth.decode(ew["W1"]), synth.decode(ew["b1"]), synth.decode(ew["W2"]),
                synth.decode(ew["b2"]))

    C = oracle.capacity(w.T, w.N, w.CF)
    acc = np.bincount(eidx, minlength=w.N).clip(max=C)
    only = None
    if sampled:
        live = np.nonzero(acc > 0)[0]
        only = sorted({int(live[0]), int(live[-1]), int(np.argmax(acc))} |
                      set(int(e) for e in np.random.default_rng(0).choice(live, 5)))
    ref = oracle.backward(x64, Wr64, experts, w.CF, dy64, d_aux, expert_idx=eidx,
                          only_experts=only)
    assert np.array_equal(fwd["slot"].cpu().numpy(), ref["slot"])
    tol = TOL[w.dtype]
    errs = {}
    rows = np.nonzero(np.all(np.isfinite(ref["dx"]), axis=1))[0]
    assert rows.size > 0
    errs["dx"] = rel_l2(_host(g["dx"])[rows], ref["dx"][rows])
    if expert_dx:
        errs["dx-dy"] = rel_l2(_host(g["dx"])[rows] - dy64[rows], ref["dx"][rows] - dy64[rows])
    todo = range(w.N) if only is None else only
    for k in ("dW1", "dW2", "db1", "db2"):
        if g[k] is None:
            continue
        got = _host(g[k])
        errs[k] = rel_l2(np.stack([got[e] for e in todo]), np.stack([ref[k][e] for e in todo]))
    if only is None:
        errs["dWr"] = rel_l2(g["dWr"].cpu().numpy().astype(np.float64), ref["dWr"])
    # experts without tokens: exactly zero gradients, every one of them
    empty = torch.from_numpy(np.nonzero(acc == 0)[0]).to(DEV)
    if empty.numel():
        for k in ("dW1", "dW2", "db1", "db2"):
            if g[k] is not None:
                assert float(g[k][empty].float().abs().max()) == 0.0, f"{k} of an empty expert"
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) +
          f" dropped={int(np.sum(ref['slot'] < 0))}", flush=True)
    for k, v in errs.items():
        assert v <= tol, f"{k} rel-L2 {v:.3e} > {tol}"
    del dev_in, fwd, g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("case", [
    dict(T=100, d=5, F=7, N=3, CF=1.0, bias_sigma=0.1),
    dict(T=333, d=33, F=65, N=9, CF=1.25, bias_sigma=0.02),
])
def test_backward_fp32(case):
    _case(synth.workload("tiny").replace(**case), twice=True)


@pytest.mark.parametrize("case", [
    dict(T=300, d=72, F=136, N=6, CF=1.0, bias_sigma=0.02),      # ragged K, M and N tails
    dict(T=640, d=256, F=512, N=16, CF=0.5),                     # heavy dropping, no bias
    dict(T=1100, d=200, F=64, N=260, CF=2.0, bias_sigma=0.02),   # many experts, N % 4 != 0
    dict(T=4096, d=64, F=96, N=4, CF=1.25, bias_sigma=0.02),     # long expert row ranges
])
def test_backward_bf16(case):
    _case(synth.workload("switch_base").replace(**case), twice=True)


@pytest.mark.parametrize("case", [
    dict(T=300, d=72, F=136, N=6, CF=1.0, bias_sigma=0.02, w_sigma=0.2),   # ragged tails
    dict(T=700, d=128, F=640, N=8, CF=1.0, bias_sigma=0.02, w_sigma=0.1),  # 20 k-steps of E2
    dict(T=2000, d=64, F=520, N=4, CF=1.25, w_sigma=0.15),                 # 4 row chunks, K tail
])
def test_backward_expert_dx(case):
    """Weights large enough that dx - dy (W1^T dA + Wr^T dz) is of the size of dy, so that
    an error in the expert or router part of dx cannot hide in dy's rounding."""
    _case(synth.workload("switch_base").replace(**case), twice=True, expert_dx=True)


@pytest.mark.parametrize("case", [
    dict(T=1, d=64, F=128, N=4, CF=4.0, bias_sigma=0.02),      # one token
    dict(T=256, d=64, F=96, N=1, CF=1.0, bias_sigma=0.02),     # N = 1: dense FFN, dz = 0
    dict(T=130, d=40, F=200, N=3, CF=1.0),                     # K tails of every GEMM
    dict(T=500, d=96, F=128, N=6, CF=1.25, bias_sigma=0.02),   # weight rows off the line grid
])
def test_backward_edges(case):
    _case(synth.workload("switch_base").replace(**case), twice=True)


def test_backward_capacity_zero():
    """C = 0: every token dropped; dx = dy + Wr^T dz from the aux term; dW = 0."""
    _case(synth.workload("switch_base").replace(T=200, d=32, F=64, N=5, CF=0.0, bias_sigma=0.02),
          d_aux=1.5)


def test_backward_no_aux():
    _case(synth.workload("switch_base").replace(T=512, d=128, F=256, N=8, CF=1.0), d_aux=0.0)


def test_backward_switch_base():
    """The Switch-Base-like workload at full size, every expert in the oracle: dx of every
    token, dWr (a sum over all tokens), and the weight and bias gradients of all experts."""
    _case(synth.workload("switch_base"))


@pytest.mark.parametrize("name", ["skewed", "switch_large"])
def test_backward_full_size_sampled(name):
    """The skewed (many drops, C = 128) and Switch-Large-like (C = 320: two row chunks per
    expert) workloads at full size: gradients of sampled experts, dx of their tokens and of
    the dropped tokens."""
    _case(synth.workload(name), sampled=True)


@pytest.mark.parametrize("name", ["switch_base", "skewed", "switch_large"])
def test_backward_full_size_expert_terms(name):
    """Full-size shapes with weights large enough (sigma 0.15) that the expert and router
    terms of dx (W1^T dA + Wr^T dz) outweigh dy: dx - dy held to the tolerance on the
    sampled experts' tokens and the dropped tokens, at the benchmark's tile structure."""
    _case(synth.workload(name).replace(w_sigma=0.15), sampled=True, expert_dx=True)


@pytest.mark.parametrize("name", ["switch_base", "skewed", "switch_large"])
def test_backward_aux_only_full_size(name):
    """dy = 0 at full size: the aux loss alone drives the gradient.  Then dO = g dy = 0 and
    dg = dy . o = 0, so dx = Wr^T dz and dWr = dz^T x for every token (accepted or
    dropped), with dz = p * (u - p . u), u_i = d_aux N f_i / T; every expert gradient is
    exactly zero.  The expert weights drop out of the exact result, so the oracle runs
    with zero experts and covers all tokens."""
    import torch

    import sparse_mixture_experts_switchffn_amd as sffn

    w = synth.workload(name)
    announce(f"backward, dy = 0, d_aux = 1: {w.describe()}")
    dev_in = synth.device_inputs(w, DEV)
    args = (dev_in["x"], dev_in["Wr"], dev_in["W1"], dev_in["b1"], dev_in["W2"], dev_in["b2"])
    fwd = sffn.switch_ffn_forward(*args, w.CF)
    dy = torch.zeros_like(dev_in["x"])
    g = sffn.switch_ffn_backward(*args, w.CF, fwd, dy, 1.0)
    torch.cuda.synchronize()
    eidx = fwd["expert_idx"].cpu().numpy().astype(np.int64)
    x64 = synth.decode(host_x(w))
    Wr64 = synth.decode(synth.host_array(w, "Wr").reshape(w.N, w.d))
    zero = (np.zeros((w.F, w.d)), None, np.zeros((w.d, w.F)), None)
    ref = oracle.backward(x64, Wr64, lambda e: zero, w.CF, np.zeros((w.T, w.d)), 1.0,
                          expert_idx=eidx)
    errs = {"dx": rel_l2(_host(g["dx"]), ref["dx"]),
            "dWr": rel_l2(g["dWr"].cpu().numpy().astype(np.float64), ref["dWr"])}
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= TOL[w.dtype], f"{k} rel-L2 {v:.3e}"
    for k in ("dW1", "dW2", "db1", "db2"):
        if g[k] is not None:
            assert float(g[k].float().abs().max()) == 0.0, f"{k} not zero"
    del dev_in, fwd, g
    torch.cuda.empty_cache()


def _raw_backward(w, dev_in, fwd, dy, stream):
    """switch_ffn_backward through the C-ABI directly (past the binding's own checks)."""
    import torch

    import sparse_mixture_experts_switchffn_amd as sffn
    from sparse_mixture_experts_switchffn_amd.binding import _ptr

    dt = sffn.SFFN_BF16 if w.dtype == "bf16" else sffn.SFFN_FP32
    out = {"dx": torch.empty_like(dev_in["x"]),
           "dWr": torch.empty((w.N, w.d), dtype=torch.float32, device=DEV),
           "dW1": torch.empty_like(dev_in["W1"]), "dW2": torch.empty_like(dev_in["W2"]),
           "db1": None if dev_in["b1"] is None else torch.empty_like(dev_in["b1"]),
           "db2": None if dev_in["b2"] is None else torch.empty_like(dev_in["b2"])}
    nb = sffn.switch_ffn_backward_workspace_bytes(w.T, w.d, w.F, w.N, w.CF, dt)
    out["workspace"] = torch.empty(nb, dtype=torch.uint8, device=DEV)
    fws = fwd["workspace"]
    rc = sffn.lib().switch_ffn_backward(
        _ptr(dev_in["x"]), _ptr(dev_in["Wr"]), _ptr(dev_in["W1"]), _ptr(dev_in["b1"]),
        _ptr(dev_in["W2"]), _ptr(dev_in["b2"]), w.T, w.d, w.F, w.N, w.CF, dt,
        _ptr(fwd["expert_idx"]), _ptr(fwd["slot"]), _ptr(fws), fws.numel(), _ptr(dy), 0.37,
        _ptr(out["dx"]), _ptr(out["dWr"]), _ptr(out["dW1"]), _ptr(out["db1"]),
        _ptr(out["dW2"]), _ptr(out["db2"]), _ptr(out["workspace"]), nb, stream, None)
    return rc, out


def _other_forms(w, dev_in):
    import sparse_mixture_experts_switchffn_amd as sffn
    args = (dev_in["x"], dev_in["Wr"], dev_in["W1"], dev_in["b1"], dev_in["W2"], dev_in["b2"],
            w.CF)
    return {"top2": sffn.switch_ffn_forward(*args, k=2),
            "reroute": sffn.switch_ffn_forward(*args, flags=sffn.SFFN_REROUTE_OVERFLOW)}


def test_backward_refuses_other_forward_workspaces():
    """A workspace left by a top-2 or rerouting forward, by a forward of another shape, or
    never written by a forward: the C-ABI returns SFFN_EINVAL before enqueueing anything;
    a top-1 forward's workspace (with or without SFFN_NO_RESIDUAL) is accepted."""
    import torch

    import sparse_mixture_experts_switchffn_amd as sffn

    w = synth.workload("switch_base").replace(T=256, d=64, F=128, N=8, CF=1.0, bias_sigma=0.02)
    announce("backward refuses foreign workspaces " + w.describe())
    dev_in = synth.device_inputs(w, DEV)
    dy = torch.ones_like(dev_in["x"])
    stream = torch.cuda.current_stream().cuda_stream
    for name, fwd in _other_forms(w, dev_in).items():
        torch.cuda.synchronize()
        fwd1 = dict(fwd, expert_idx=fwd["expert_idx"][:, 0].contiguous() if fwd["expert_idx"].dim() == 2
                    else fwd["expert_idx"],
                    slot=fwd["slot"][:, 0].contiguous() if fwd["slot"].dim() == 2 else fwd["slot"])
        rc, _ = _raw_backward(w, dev_in, fwd1, dy, stream)
        assert rc == sffn.SFFN_EINVAL, (name, rc)
    args = (dev_in["x"], dev_in["Wr"], dev_in["W1"], dev_in["b1"], dev_in["W2"], dev_in["b2"],
            w.CF)
    for flags in (0, sffn.SFFN_NO_RESIDUAL):
        fwd = sffn.switch_ffn_forward(*args, flags=flags)
        rc, out = _raw_backward(w, dev_in, fwd, dy, stream)
        assert rc == sffn.SFFN_OK, (flags, rc)
    # a GEGLU forward (W1 of 2F rows; the call is refused before any weight is read)
    wg = w.replace(glu=True)
    gin = synth.device_inputs(wg, DEV)
    gfwd = sffn.switch_ffn_forward(gin["x"], gin["Wr"], gin["W1"], gin["b1"], gin["W2"],
                                   gin["b2"], w.CF, flags=sffn.SFFN_GEGLU)
    rc, _ = _raw_backward(w, dev_in, gfwd, dy, stream)
    assert rc == sffn.SFFN_EINVAL
    # a workspace of the right size that no forward wrote
    blank = dict(fwd, workspace=torch.zeros_like(fwd["workspace"]))
    rc, _ = _raw_backward(w, dev_in, blank, dy, stream)
    assert rc == sffn.SFFN_EINVAL
    # a top-1 forward of another capacity (same buffers, CF 2.0)
    other = sffn.switch_ffn_forward(*args[:6], 2.0)
    rc, _ = _raw_backward(w, dev_in, other, dy, stream)
    assert rc == sffn.SFFN_EINVAL
    torch.cuda.synchronize()


def test_backward_captured_with_foreign_workspace_gives_nan():
    """Under graph capture the host cannot read the tag (the forward has not run); the
    guard kernel checks it on the device.  A captured backward fed a top-2 forward's
    workspace reads none of its row maps and returns NaN gradients; the same graph fed a
    top-1 workspace afterwards (the maps copied in) gives the eager result bit for bit."""
    import torch

    import sparse_mixture_experts_switchffn_amd as sffn

    w = synth.workload("switch_base").replace(T=256, d=64, F=128, N=8, CF=1.0, bias_sigma=0.02)
    announce("captured backward on a foreign workspace " + w.describe())
    dev_in = synth.device_inputs(w, DEV)
    dy = torch.ones_like(dev_in["x"])
    forms = _other_forms(w, dev_in)
    top2 = forms["top2"]
    args = (dev_in["x"], dev_in["Wr"], dev_in["W1"], dev_in["b1"], dev_in["W2"], dev_in["b2"],
            w.CF)
    top1 = sffn.switch_ffn_forward(*args)
    torch.cuda.synchronize()
    rc, eager = _raw_backward(w, dev_in, top1, dy, torch.cuda.current_stream().cuda_stream)
    assert rc == sffn.SFFN_OK
    torch.cuda.synchronize()
    # one buffer set for the capture: the top-2 workspace (larger), top-1 sized views of
    # the choice arrays
    ws = top2["workspace"].clone()
    eidx = torch.zeros(w.T, dtype=torch.int32, device=DEV)
    slot = torch.zeros(w.T, dtype=torch.int32, device=DEV)
    fwd = {"workspace": ws, "expert_idx": eidx, "slot": slot}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        rc, out = _raw_backward(w, dev_in, fwd, dy, side.cuda_stream)
    assert rc == sffn.SFFN_OK
    eidx.copy_(top2["expert_idx"][:, 0])
    slot.copy_(top2["slot"][:, 0])
    g.replay()
    torch.cuda.synchronize()
    for k in ("dx", "dWr", "dW1", "dW2", "db1", "db2"):
        assert bool(torch.isnan(out[k].float()).all()), f"{k} not all NaN"
    # the same graph on a top-1 forward's workspace and outputs
    ws.zero_()
    ws[: top1["workspace"].numel()].copy_(top1["workspace"])
    eidx.copy_(top1["expert_idx"])
    slot.copy_(top1["slot"])
    g.replay()
    torch.cuda.synchronize()
    for k in ("dx", "dWr", "dW1", "dW2", "db1", "db2"):
        assert torch.equal(out[k], eager[k]), k
    del g
