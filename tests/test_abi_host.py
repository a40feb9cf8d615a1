"""The C-ABI library on the host: it loads, exports what the header declares, and its
host-only entry points and argument checks behave (no GPU, no compute calls)."""
import ctypes
import math

import pytest

import oracle
import sparse_mixture_experts_switchffn_amd as S
from sparse_mixture_experts_switchffn_amd import binding as B


def test_library_exports_every_declared_function():
    names = S.header_functions()
    assert set(names) >= {"switch_ffn_capacity", "switch_ffn_workspace_bytes",
                          "switch_ffn_forward", "switch_ffn_forward_ex",
                          "switch_ffn_status_string", "switch_ffn_num_stages",
                          "switch_ffn_stage_name"}
    raw = ctypes.CDLL(S.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


@pytest.mark.parametrize("T,N,CF", [(64, 4, 1.0), (8192, 64, 1.25), (16384, 128, 1.0),
                                    (32768, 128, 1.25), (65536, 2048, 1.0), (10, 4, 1.0),
                                    (10, 4, 1.25), (7, 3, 0.0), (7, 3, 3.0), (0, 3, 1.0),
                                    (1, 1, 0.999), (1000, 7, 0.3), (12345, 17, 2.75)])
def test_capacity_matches_oracle(T, N, CF):
    assert S.switch_ffn_capacity(T, N, CF) == oracle.capacity(T, N, CF)


@pytest.mark.parametrize("args", [(5, 0, 1.0), (-1, 2, 1.0), (5, 2, -0.5), (5, 2, math.nan),
                                  (5, 2, math.inf)])
def test_capacity_rejects(args):
    assert S.switch_ffn_capacity(*args) == -1


def test_workspace_bytes():
    base = S.switch_ffn_workspace_bytes(8192, 768, 3072, 64, 1.25, S.SFFN_BF16)
    assert base > 8192 * 64 * 4 + 8192 * 3072 * 2       # logits + hidden activations
    assert S.switch_ffn_workspace_bytes(8192, 768, 3072, 64, 1.25, S.SFFN_FP32) > base
    assert S.switch_ffn_workspace_bytes(16384, 768, 3072, 64, 1.25, S.SFFN_BF16) > base
    assert S.switch_ffn_workspace_bytes(8192, 768, 4096, 64, 1.25, S.SFFN_BF16) > base
    assert S.switch_ffn_workspace_bytes(8192, 768, 3072, 64, 0.0, S.SFFN_BF16) < base
    for bad in ((0, 8, 8, 2, 1.0, 1), (8, 8, 8, 2, -1.0, 1), (8, 8, 8, 2, 1.0, 7),
                (8, 8, 8, 5000, 1.0, 1), (8, 12, 8, 2, 1.0, 1)):
        assert S.switch_ffn_workspace_bytes(*bad) == 0


def test_stage_names():
    n = S.switch_ffn_num_stages()
    names = [S.switch_ffn_stage_name(i) for i in range(n)]
    assert names == ["router_logits", "softmax_route", "dispatch_scan", "dispatch_scatter",
                     "ffn1", "ffn2"]
    assert S.switch_ffn_stage_name(n) is None and S.switch_ffn_stage_name(-1) is None


def test_backward_stage_names():
    n = S.switch_ffn_backward_num_stages()
    names = [S.switch_ffn_backward_stage_name(i) for i in range(n)]
    assert names == ["expert_dgrad_hidden", "router_grad", "expert_dgrad_input", "dx",
                     "router_wgrad", "expert_wgrad", "bias_grad"]
    assert S.switch_ffn_backward_stage_name(n) is None
    assert S.switch_ffn_backward_stage_name(-1) is None


def _call(**over):
    # Fake, never-dereferenced addresses: every case below must be rejected before
    # anything touches a device.
    fake = 0x100000
    a = dict(x=fake, Wr=fake, W1=fake, b1=None, W2=fake, b2=None, T=64, d=32, F=64, N=4, CF=1.0,
             dtype=S.SFFN_BF16, y=fake, expert_idx=fake, slot=fake, gate=fake, aux=fake,
             ws=fake, ws_bytes=1 << 40, stream=None, flags=0)
    a.update(over)
    return B.lib().switch_ffn_forward_ex(
        a["x"], a["Wr"], a["W1"], a["b1"], a["W2"], a["b2"], a["T"], a["d"], a["F"], a["N"],
        a["CF"], a["dtype"], a["y"], a["expert_idx"], a["slot"], a["gate"], a["aux"], a["ws"],
        a["ws_bytes"], a["stream"], a["flags"], None)


def test_forward_ex_signature_is_forward_plus_flags_and_stats():
    # switch_ffn_forward's 20 arguments, then flags and the nullable stats pointer.
    assert len(B.lib().switch_ffn_forward.argtypes) == 20
    assert len(B.lib().switch_ffn_forward_ex.argtypes) == 22
    assert B.lib().switch_ffn_forward_ex.argtypes[:20] == B.lib().switch_ffn_forward.argtypes


@pytest.mark.parametrize("over,code", [
    (dict(x=None), S.SFFN_EINVAL), (dict(Wr=None), S.SFFN_EINVAL), (dict(W1=None), S.SFFN_EINVAL),
    (dict(W2=None), S.SFFN_EINVAL), (dict(y=None), S.SFFN_EINVAL),
    (dict(expert_idx=None), S.SFFN_EINVAL), (dict(slot=None), S.SFFN_EINVAL),
    (dict(gate=None), S.SFFN_EINVAL), (dict(aux=None), S.SFFN_EINVAL),
    (dict(T=0), S.SFFN_EINVAL), (dict(d=-1), S.SFFN_EINVAL), (dict(F=0), S.SFFN_EINVAL),
    (dict(N=0), S.SFFN_EINVAL), (dict(CF=-1.0), S.SFFN_EINVAL), (dict(CF=math.nan), S.SFFN_EINVAL),
    (dict(flags=8), S.SFFN_EINVAL), (dict(dtype=3), S.SFFN_EDTYPE),
    (dict(N=5000), S.SFFN_EUNSUPPORTED), (dict(d=36), S.SFFN_EUNSUPPORTED),
    (dict(F=70), S.SFFN_EUNSUPPORTED), (dict(T=1 << 25, d=64), S.SFFN_EUNSUPPORTED), (dict(d=32768, F=32768), S.SFFN_EUNSUPPORTED),
    # fp32 logits of 2^29 elements (2 GiB) and an expert of 2^29 weights: past the limits
    (dict(T=1 << 18, N=2048, d=64, F=64), S.SFFN_EUNSUPPORTED), (dict(d=16384, F=32768), S.SFFN_EUNSUPPORTED),
    (dict(x=0x100004), S.SFFN_EUNSUPPORTED), (dict(ws=None), S.SFFN_EWORKSPACE),
    (dict(ws_bytes=1000), S.SFFN_EWORKSPACE), (dict(ws=0x100010), S.SFFN_EUNSUPPORTED),
])
def test_forward_rejects_before_launch(over, code):
    assert _call(**over) == code
    assert S.switch_ffn_status_string(code)


def test_status_strings():
    for c in (S.SFFN_OK, S.SFFN_EINVAL, S.SFFN_EDTYPE, S.SFFN_EWORKSPACE, S.SFFN_EUNSUPPORTED,
              S.SFFN_EHIP, -99):
        assert isinstance(S.switch_ffn_status_string(c), str)


def _call_topk(k, **over):
    fake = 0x100000
    a = dict(x=fake, Wr=fake, W1=fake, b1=None, W2=fake, b2=None, T=64, d=32, F=64, N=4, CF=1.0,
             dtype=S.SFFN_BF16, y=fake, expert_idx=fake, slot=fake, gate=fake, aux=fake,
             ws=fake, ws_bytes=1 << 40, stream=None, flags=0)
    a.update(over)
    return B.lib().switch_ffn_forward_topk(
        a["x"], a["Wr"], a["W1"], a["b1"], a["W2"], a["b2"], a["T"], a["d"], a["F"], a["N"],
        a["CF"], k, a["dtype"], a["y"], a["expert_idx"], a["slot"], a["gate"], a["aux"], a["ws"],
        a["ws_bytes"], a["stream"], a["flags"], None, None)


@pytest.mark.parametrize("k,over,code", [
    (0, {}, S.SFFN_EINVAL), (3, {}, S.SFFN_EINVAL), (2, dict(N=1), S.SFFN_EINVAL),
    (2, dict(x=None), S.SFFN_EINVAL), (2, dict(dtype=3), S.SFFN_EDTYPE),
    (2, dict(d=36), S.SFFN_EUNSUPPORTED), (2, dict(ws_bytes=1000), S.SFFN_EWORKSPACE),
    (2, dict(T=1 << 20, d=512, F=512, N=2, CF=1.0), S.SFFN_EUNSUPPORTED),  # 2T rows x F x 4 >= 2^31
])
def test_forward_topk_rejects_before_launch(k, over, code):
    assert _call_topk(k, **over) == code


@pytest.mark.parametrize("k,over,code", [
    (1, dict(N=1), S.SFFN_EINVAL),                 # rerouting needs a second choice
    (2, {}, S.SFFN_EINVAL),                        # rerouting is a top-1 form
    (1, dict(flags=S.SFFN_REROUTE_OVERFLOW | 8), S.SFFN_EINVAL),  # unknown flag bit
    (1, dict(ws_bytes=1000), S.SFFN_EWORKSPACE),
])
def test_reroute_rejects_before_launch(k, over, code):
    over = dict(over)
    over["flags"] = over.get("flags", S.SFFN_REROUTE_OVERFLOW)
    assert _call_topk(k, **over) == code
    if k == 1:
        assert _call(**over) == code


def test_workspace_bytes_topk():
    one = S.switch_ffn_workspace_bytes(8192, 768, 3072, 64, 1.25, S.SFFN_BF16)
    assert S.switch_ffn_workspace_bytes_topk(8192, 768, 3072, 64, 1.25, 1, S.SFFN_BF16) == one
    two = S.switch_ffn_workspace_bytes_topk(8192, 768, 3072, 64, 1.25, 2, S.SFFN_BF16)
    # twice the expert rows (H and the per-row outputs), top-1 counts, two ranks per token
    assert two > one + 8192 * 3072 * 2 + 2 * 8192 * 768 * 2 - 8192 * 768 * 2
    assert S.switch_ffn_workspace_bytes_topk(8192, 768, 3072, 1, 1.25, 2, S.SFFN_BF16) == 0
    assert S.switch_ffn_workspace_bytes_topk(8192, 768, 3072, 64, 1.25, 3, S.SFFN_BF16) == 0


def _call_bwd(**over):
    # Fake, never-dereferenced addresses: every case below is rejected before the
    # layout tag is read or anything is enqueued.
    fake = 0x100000
    T, d, F, N, CF, dt = 64, 32, 64, 4, 1.0, S.SFFN_BF16
    fwd_need = S.switch_ffn_workspace_bytes(T, d, F, N, CF, dt)
    bwd_need = S.switch_ffn_backward_workspace_bytes(T, d, F, N, CF, dt)
    a = dict(x=fake, Wr=fake, W1=fake, b1=None, W2=fake, b2=None, T=T, d=d, F=F, N=N, CF=CF,
             dtype=dt, expert_idx=fake, slot=fake, fws=fake, fws_bytes=fwd_need, dy=fake,
             d_aux=0.01, dx=fake, dWr=fake, dW1=fake, db1=None, dW2=fake, db2=None, ws=fake,
             ws_bytes=bwd_need, stream=None)
    a.update(over)
    return B.lib().switch_ffn_backward(
        a["x"], a["Wr"], a["W1"], a["b1"], a["W2"], a["b2"], a["T"], a["d"], a["F"], a["N"],
        a["CF"], a["dtype"], a["expert_idx"], a["slot"], a["fws"], a["fws_bytes"], a["dy"],
        a["d_aux"], a["dx"], a["dWr"], a["dW1"], a["db1"], a["dW2"], a["db2"], a["ws"],
        a["ws_bytes"], a["stream"], None)


@pytest.mark.parametrize("over,code", [
    (dict(x=None), S.SFFN_EINVAL), (dict(Wr=None), S.SFFN_EINVAL), (dict(W1=None), S.SFFN_EINVAL),
    (dict(W2=None), S.SFFN_EINVAL), (dict(expert_idx=None), S.SFFN_EINVAL),
    (dict(slot=None), S.SFFN_EINVAL), (dict(fws=None), S.SFFN_EINVAL),
    (dict(dy=None), S.SFFN_EINVAL), (dict(dx=None), S.SFFN_EINVAL),
    (dict(dWr=None), S.SFFN_EINVAL), (dict(dW1=None), S.SFFN_EINVAL),
    (dict(dW2=None), S.SFFN_EINVAL), (dict(d_aux=math.nan), S.SFFN_EINVAL),
    (dict(d_aux=math.inf), S.SFFN_EINVAL), (dict(T=0), S.SFFN_EINVAL), (dict(N=0), S.SFFN_EINVAL),
    (dict(CF=-1.0), S.SFFN_EINVAL), (dict(dtype=5), S.SFFN_EDTYPE),
    (dict(N=5000), S.SFFN_EUNSUPPORTED), (dict(d=36), S.SFFN_EUNSUPPORTED),
    (dict(dy=0x100004), S.SFFN_EUNSUPPORTED), (dict(dx=0x100008), S.SFFN_EUNSUPPORTED),
    (dict(dW1=0x100002), S.SFFN_EUNSUPPORTED), (dict(dW2=0x100002), S.SFFN_EUNSUPPORTED),
    (dict(fws_bytes=1000), S.SFFN_EWORKSPACE), (dict(ws=None), S.SFFN_EWORKSPACE),
    (dict(ws_bytes=1000), S.SFFN_EWORKSPACE), (dict(ws=0x100010), S.SFFN_EUNSUPPORTED),
    (dict(fws=0x100010), S.SFFN_EUNSUPPORTED),
])
def test_backward_rejects_before_launch(over, code):
    assert _call_bwd(**over) == code


def test_backward_workspace_bytes():
    one = S.switch_ffn_backward_workspace_bytes(8192, 768, 3072, 64, 1.25, S.SFFN_BF16)
    # dz [T, N] fp32, dA [rows, F] bf16 and the expert part of dx [T, d] fp32 at least
    assert one > 8192 * 64 * 4 + 8192 * 3072 * 2 + 8192 * 768 * 4
    assert S.switch_ffn_backward_workspace_bytes(8192, 768, 3072, 64, 1.25, 9) == 0
    assert S.switch_ffn_backward_workspace_bytes(0, 768, 3072, 64, 1.25, S.SFFN_BF16) == 0


# ---------------------------------------------------------------------------
# The binding refuses tensors the C-ABI would read wrongly (CPU tensors stand in:
# every check below fires before anything reaches the library).
# ---------------------------------------------------------------------------
def _layer(T=16, d=8, F=16, N=4, dtype=None, device="cpu"):
    import torch
    dt = torch.bfloat16 if dtype is None else dtype
    return dict(x=torch.zeros(T, d, dtype=dt, device=device),
                Wr=torch.zeros(N, d, dtype=torch.float32, device=device),
                W1=torch.zeros(N, F, d, dtype=dt, device=device), b1=None,
                W2=torch.zeros(N, d, F, dtype=dt, device=device), b2=None)


def _fwd(L, **kw):
    return B.switch_ffn_forward(L["x"], L["Wr"], L["W1"], L["b1"], L["W2"], L["b2"], 1.0, **kw)


def test_binding_rejects_wrong_dtypes_and_shapes():
    import torch
    L = _layer()
    with pytest.raises(TypeError):
        _fwd(dict(L, x=L["x"].to(torch.float16)))
    with pytest.raises(TypeError):
        _fwd(dict(L, Wr=L["Wr"].to(torch.bfloat16)))          # the router is fp32
    with pytest.raises(TypeError):
        _fwd(dict(L, W1=L["W1"].float()))                      # experts share x's dtype
    with pytest.raises(TypeError):
        _fwd(dict(L, W2=L["W2"].float()))
    with pytest.raises(TypeError):
        _fwd(dict(L, b1=torch.zeros(4, 16, dtype=torch.float32)))
    with pytest.raises(ValueError):
        _fwd(dict(L, W1=torch.zeros(4, 8, 16, dtype=torch.bfloat16)))   # [N, d, F]: transposed
    with pytest.raises(ValueError):
        _fwd(dict(L, W2=torch.zeros(4, 16, 16, dtype=torch.bfloat16)))
    with pytest.raises(ValueError):
        _fwd(dict(L, Wr=torch.zeros(4, 9, dtype=torch.float32)))
    with pytest.raises(ValueError):
        _fwd(dict(L, b2=torch.zeros(4, 16, dtype=torch.bfloat16)))
    with pytest.raises(ValueError):
        _fwd(dict(L, x=L["x"][:, None]))                        # not [T, d]
    with pytest.raises(ValueError):
        _fwd(L, flags=B.SFFN_GEGLU)                             # GEGLU needs W1 [N, 2F, d]
    with pytest.raises(ValueError):
        _fwd(L, k=3)


def test_binding_rejects_strided_and_host_tensors():
    import torch
    L = _layer()
    with pytest.raises(ValueError):
        _fwd(dict(L, x=torch.zeros(8, 16, dtype=torch.bfloat16).t()))   # a transposed view
    with pytest.raises(ValueError):
        _fwd(dict(L, W1=torch.zeros(4, 8, 16, dtype=torch.bfloat16).transpose(1, 2)))
    with pytest.raises(ValueError, match="GPU"):
        _fwd(L)                                                 # host memory


def test_binding_backward_refuses_other_forward_forms():
    L = _layer()
    for fwd in (dict(k=2, flags=0), dict(k=1, flags=B.SFFN_REROUTE_OVERFLOW),
                dict(k=1, flags=B.SFFN_GEGLU)):
        with pytest.raises(ValueError, match="top-1"):
            B.switch_ffn_backward(L["x"], L["Wr"], L["W1"], L["b1"], L["W2"], L["b2"], 1.0, fwd,
                                  L["x"], 0.0)


def test_noalloc_rejects_before_any_device_call():
    fake = 0x100000
    L = B.lib()
    assert L.switch_ffn_noalloc_scratch_bytes() == 64 << 20

    def call(T=8192, d=768, F=3072, N=64, CF=1.25, dtype=S.SFFN_BF16, x=fake):
        return L.switch_ffn_forward_noalloc(x, fake, fake, None, fake, None, T, d, F, N, CF, dtype,
                                            fake, fake, fake, fake, fake, None)
    assert call(T=65536, d=2080, F=6144, N=2048, CF=1.0) == S.SFFN_ESCRATCH
    assert call(T=32768, d=1024, F=4096, N=128) == S.SFFN_ESCRATCH
    assert call(T=0) == S.SFFN_EINVAL
    assert call(x=None) == S.SFFN_EINVAL
    assert call(dtype=4) == S.SFFN_EDTYPE
    assert call(d=36) == S.SFFN_EUNSUPPORTED
    assert "scratch" in S.switch_ffn_status_string(S.SFFN_ESCRATCH)
