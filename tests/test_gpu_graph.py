"""The forward pass, and a forward + backward training step, captured in a HIP graph:
replays reproduce eager launches bit for bit, also when other eager work (on the same
workspaces) runs between the replays."""
import pytest
import torch

import sparse_mixture_experts_switchffn_amd as S
import switchffn_synth as synth

pytestmark = pytest.mark.gpu

OUT_KEYS = ("y", "expert_idx", "slot", "gate", "aux_loss")


def _run(inp, w, bufs):
    S.switch_ffn_forward(inp["x"], inp["Wr"], inp["W1"], inp["b1"], inp["W2"], inp["b2"], w.CF,
                         **bufs)


@pytest.mark.parametrize("name,over", [
    ("graph_small", dict(T=1000, d=256, F=512, N=8, CF=1.0, bias_sigma=0.02)),
    ("graph_many_tiles", dict(T=4096, d=512, F=1024, N=16, CF=1.25)),
])
def test_graph_replay_matches_eager(name, over):
    dev = "cuda:0"
    w = synth.workload("switch_base", **over)
    inp = synth.device_inputs(w, dev)
    other = synth.device_inputs(w.replace(seed=w.seed + 7), dev)
    out = S.switch_ffn_forward(inp["x"], inp["Wr"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                               w.CF)
    bufs = {k: out[k] for k in OUT_KEYS + ("workspace",)}
    torch.cuda.synchronize()
    ref = {k: bufs[k].clone() for k in OUT_KEYS}
    # The other input's eager outputs go to their own buffers but share the workspace.
    obufs = {k: torch.empty_like(bufs[k]) for k in OUT_KEYS}
    obufs["workspace"] = bufs["workspace"]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(inp, w, bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run(inp, w, bufs)
    torch.cuda.synchronize()
    for rep in range(4):
        for k in OUT_KEYS:
            bufs[k].zero_()
        _run(other, w, obufs)          # eager work in between, same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in OUT_KEYS:
            assert torch.equal(bufs[k], ref[k]), f"{name}: replay {rep} differs in {k}"
    del g


GRAD_KEYS = ("dx", "dWr", "dW1", "db1", "dW2", "db2")


def test_graph_replay_training_step():
    """Forward + backward captured together: every replay reproduces the eager gradients bit
    for bit, with an eager training step on other inputs (same workspaces) in between."""
    dev = "cuda:0"
    w = synth.workload("switch_base", T=1500, d=256, F=512, N=8, CF=1.25, bias_sigma=0.02)
    inp = synth.device_inputs(w, dev)
    other = synth.device_inputs(w.replace(seed=w.seed + 3), dev)
    gen = torch.Generator(device=dev).manual_seed(5)
    dy = torch.randn(w.T, w.d, generator=gen, device=dev).to(torch.bfloat16)
    args = lambda i: (i["x"], i["Wr"], i["W1"], i["b1"], i["W2"], i["b2"])  # noqa: E731
    fwd = S.switch_ffn_forward(*args(inp), w.CF)
    fbufs = {k: fwd[k] for k in OUT_KEYS + ("workspace",)}
    g0 = S.switch_ffn_backward(*args(inp), w.CF, fwd, dy, 0.25)
    gbufs = {k: g0[k] for k in GRAD_KEYS + ("workspace",)}
    torch.cuda.synchronize()
    ref = {k: gbufs[k].clone() for k in GRAD_KEYS}

    def step(i, fb, gb):
        S.switch_ffn_forward(*args(i), w.CF, **fb)
        S.switch_ffn_backward(*args(i), w.CF, fb, dy, 0.25, **gb)

    obufs = {k: torch.empty_like(fbufs[k]) for k in OUT_KEYS}
    obufs["workspace"] = fbufs["workspace"]
    ogbufs = {k: torch.empty_like(gbufs[k]) for k in GRAD_KEYS}
    ogbufs["workspace"] = gbufs["workspace"]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(inp, fbufs, gbufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(inp, fbufs, gbufs)
    torch.cuda.synchronize()
    for rep in range(4):
        for k in GRAD_KEYS:
            gbufs[k].zero_()
        step(other, obufs, ogbufs)     # eager work in between, same workspaces
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in GRAD_KEYS:
            assert torch.equal(gbufs[k], ref[k]), f"replay {rep} differs in {k}"
    del g
