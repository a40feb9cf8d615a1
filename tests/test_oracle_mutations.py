"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each.

A pin set that a dropped term, a wrong sign or index, or a transposed operand
slips through would not pin the oracle; every mutant below must make at least
one pin fail.
"""
import math

import numpy as np
import pytest

import oracle.switchffn_oracle as O
from oracle_pins import ALL_PINS

_orig = {name: getattr(O, name) for name in
         ("capacity", "router_logits", "softmax", "top1", "dispatch", "aux_loss", "expert_ffn",
          "round_to_bf16", "forward", "second_choice", "topk_gates", "dispatch_topk",
          "reroute_overflow", "gelu", "expert_backward", "aux_prob_grad", "softmax_backward",
          "backward", "near_tie_tokens", "near_tie_second")}


def _ffn_no_b2(xe, W1e, b1e, W2e, b2e, activation="relu"):
    return _orig["expert_ffn"](xe, W1e, b1e, W2e, None, activation)


def _ffn_no_b1(xe, W1e, b1e, W2e, b2e, activation="relu"):
    return _orig["expert_ffn"](xe, W1e, None, W2e, b2e, activation)


def _ffn_no_relu(xe, W1e, b1e, W2e, b2e, activation="relu"):
    a = xe @ np.asarray(W1e).T + (0 if b1e is None else b1e)
    return a @ np.asarray(W2e).T + (0 if b2e is None else b2e)


def _ffn_relu_after(xe, W1e, b1e, W2e, b2e, activation="relu"):
    return np.maximum(_ffn_no_relu(xe, W1e, b1e, W2e, b2e), 0.0)


def _ffn_transposed_w1(xe, W1e, b1e, W2e, b2e, activation="relu"):
    W1e = np.asarray(W1e)
    return _orig["expert_ffn"](xe, W1e.reshape(W1e.shape[::-1]), b1e, W2e, b2e, activation)


def _logits_sign(x, Wr):
    return -_orig["router_logits"](x, Wr)


def _logits_untransposed(x, Wr):
    Wr = np.asarray(Wr, np.float64)
    return np.asarray(x, np.float64) @ Wr.reshape(Wr.shape[::-1])


def _softmax_axis0(z):
    m = z.max(axis=0, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=0, keepdims=True)


def _softmax_no_norm(z):
    return np.exp(z - z.max(axis=1, keepdims=True))


def _top1_last_tie(z):
    z32 = z.astype(np.float32)[:, ::-1]
    return (z.shape[1] - 1 - np.argmax(z32, axis=1)).astype(np.int64)


def _top1_argmin(z):
    return np.argmin(z.astype(np.float32), axis=1).astype(np.int64)


def _dispatch_one_based(eidx, N, C):
    dp = _orig["dispatch"](eidx, N, C)
    rank = dp["rank"] + 1
    dp["rank"] = rank
    dp["slot"] = np.where(rank < C, rank, -1)
    return dp


def _dispatch_le(eidx, N, C):
    return _orig["dispatch"](eidx, N, C + 1)


def _dispatch_reverse_order(eidx, N, C):
    T = len(eidx)
    dp = _orig["dispatch"](np.asarray(eidx)[::-1], N, C)
    out = dict(dp)
    for k in ("rank", "slot"):
        out[k] = dp[k][::-1]
    out["row2tok"] = T - 1 - dp["row2tok"]
    return out


def _aux_no_n(eidx, probs):
    return _orig["aux_loss"](eidx, probs) / probs.shape[1]


def _aux_gate_only(eidx, probs):
    T, N = probs.shape
    onehot = np.zeros_like(probs)
    onehot[np.arange(T), eidx] = probs[np.arange(T), eidx]
    return _orig["aux_loss"](eidx, onehot)


def _aux_f_squared(eidx, probs):
    T, N = probs.shape
    f = np.bincount(eidx, minlength=N) / T
    return float(N * np.dot(f, f))


def _capacity_ceil(T, N, CF):
    _orig["capacity"](T, N, CF)
    return int(math.ceil(CF * T / N))


def _capacity_floor_first(T, N, CF):
    _orig["capacity"](T, N, CF)
    return int(math.floor(T / N) * CF)


def _bf16_truncate(v):
    m, e = np.frexp(np.asarray(v, np.float64))
    return np.ldexp(np.trunc(m * 256.0), e - 8)


def _forward_no_residual(*a, **k):
    k = dict(k)
    r = _orig["forward"](*a, **k)
    if not k.get("no_residual"):
        x = np.asarray(a[0], np.float64)
        acc = r["slot"] >= 0
        r["y64"] = r["y64"].copy()
        r["y64"][acc] -= x[acc]
    return r


def _forward_dropped_zero(*a, **k):
    r = _orig["forward"](*a, **k)
    r["y64"] = r["y64"].copy()
    r["y64"][r["slot"] < 0] = 0.0
    return r


def _forward_gate_outside_b2(*a, **k):
    # y = x + g * (W2 h) + b2 instead of x + g * (W2 h + b2)
    r = _orig["forward"](*a, **k)
    experts = a[2] if len(a) > 2 else k["experts"]
    b2 = experts[3] if not callable(experts) else None
    if b2 is not None:
        r["y64"] = r["y64"].copy()
        for t in np.nonzero(r["slot"] >= 0)[0]:
            e = r["expert_idx"][t]
            r["y64"][t] += (1.0 - r["gate"][t]) * b2[e]
    return r


def _second_ties_to_highest(z, first):
    z32 = z.astype(np.float32).copy()
    z32[np.arange(z.shape[0]), first] = -np.inf
    return (z.shape[1] - 1 - np.argmax(z32[:, ::-1], axis=1)).astype(np.int64)


def _gates_renormalised(probs, choices):
    g = _orig["topk_gates"](probs, choices)
    return g / g.sum(axis=1, keepdims=True)


def _dispatch_first_choices_first(choices, N, C):
    # All first choices in token order, then all second choices (a different
    # priority rule from filling each expert column in token order).
    T, k = choices.shape
    count = np.zeros(N, dtype=np.int64)
    rank = np.empty((T, k), dtype=np.int64)
    for c in range(k):
        for t in range(T):
            e = int(choices[t, c])
            rank[t, c] = count[e]
            count[e] += 1
    dp = _orig["dispatch_topk"](choices, N, C)
    slot = np.where(rank < C, rank, -1)
    dp.update(rank=rank, slot=slot)
    return dp


def _dispatch_topk_capacity_without_k(choices, N, C):
    return _orig["dispatch_topk"](choices, N, C // 2)


def _reroute_ignores_first_stage(first, second, N, C):
    # Stage 2 placed from position 0 instead of after the stage-1 tokens.
    d1 = _orig["dispatch"](first, N, C)
    r = _orig["reroute_overflow"](first, second, N, C)
    slot = r["slot"].copy()
    over = d1["slot"] < 0
    slot[over & (slot >= 0)] -= d1["accepted"][r["expert"][over & (slot >= 0)]]
    r["slot"] = slot
    return r


def _reroute_reverse_order(first, second, N, C):
    T = len(first)
    d1 = _orig["dispatch"](first, N, C)
    r = _orig["reroute_overflow"](first, second, N, C)
    # redo stage 2 from the last overflowed token to the first
    used = d1["accepted"].copy()
    count2 = np.zeros(N, dtype=np.int64)
    slot = d1["slot"].copy()
    expert = np.asarray(first).copy()
    for t in reversed(range(T)):
        if d1["slot"][t] >= 0:
            continue
        e = int(second[t])
        pos = used[e] + count2[e]
        count2[e] += 1
        if pos < C:
            slot[t], expert[t] = pos, e
    r.update(slot=slot, expert=expert)
    return r


def _reroute_none(first, second, N, C):
    r = _orig["reroute_overflow"](first, second, N, C)
    d1 = _orig["dispatch"](first, N, C)
    r.update(slot=d1["slot"], expert=np.asarray(first).copy(), accepted=d1["accepted"],
             offset=d1["offset"], row2tok=d1["row2tok"])
    return r


def _gelu_tanh(a):
    # the tanh approximation instead of the exact a * Phi(a)
    return 0.5 * a * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (a + 0.044715 * a ** 3)))


def _geglu_halves_swapped(xe, W1e, b1e, W2e, b2e, activation="relu"):
    if activation != "geglu":
        return _orig["expert_ffn"](xe, W1e, b1e, W2e, b2e, activation)
    F = np.asarray(W1e).shape[0] // 2
    W1s = np.concatenate([np.asarray(W1e)[F:], np.asarray(W1e)[:F]])
    b1s = None if b1e is None else np.concatenate([np.asarray(b1e)[F:], np.asarray(b1e)[:F]])
    return _orig["expert_ffn"](xe, W1s, b1s, W2e, b2e, activation)


def _geglu_relu_gate(xe, W1e, b1e, W2e, b2e, activation="relu"):
    if activation != "geglu":
        return _orig["expert_ffn"](xe, W1e, b1e, W2e, b2e, activation)
    a = xe @ np.asarray(W1e).T + (0 if b1e is None else b1e)
    F = a.shape[1] // 2
    h = np.maximum(a[:, :F], 0.0) * a[:, F:]
    return h @ np.asarray(W2e).T + (0 if b2e is None else b2e)


def _eb_no_relu_mask(xe, W1e, b1e, W2e, b2e, dye, ge):
    g = _orig["expert_backward"](xe, W1e, b1e, W2e, b2e, dye, ge)
    da = (ge[:, None] * dye) @ np.asarray(W2e, np.float64)   # mask forgotten
    g.update(dW1=da.T @ xe, db1=da.sum(axis=0), dx=da @ np.asarray(W1e, np.float64))
    return g


def _eb_no_gate(xe, W1e, b1e, W2e, b2e, dye, ge):
    return _orig["expert_backward"](xe, W1e, b1e, W2e, b2e, dye, np.ones_like(ge))


def _eb_dg_without_b2(xe, W1e, b1e, W2e, b2e, dye, ge):
    g = _orig["expert_backward"](xe, W1e, b1e, W2e, b2e, dye, ge)
    if b2e is not None:
        g["dg"] = g["dg"] - dye @ np.asarray(b2e, np.float64)
    return g


def _eb_db2_ungated(xe, W1e, b1e, W2e, b2e, dye, ge):
    g = _orig["expert_backward"](xe, W1e, b1e, W2e, b2e, dye, ge)
    g["db2"] = dye.sum(axis=0)
    return g


def _aux_grad_without_n(hist, T, d_aux):
    return _orig["aux_prob_grad"](hist, T, d_aux) / len(hist)


def _softmax_bwd_uncentred(p, u):
    return p * u


def _softmax_bwd_sign(p, u):
    return -_orig["softmax_backward"](p, u)


def _bwd_no_residual(*a, **k):
    g = _orig["backward"](*a, **k)
    g["dx"] = g["dx"] - np.asarray(a[4], np.float64)
    return g


def _near_tie_strict(z, tol=1e-5):
    if z.shape[1] < 2:
        return np.zeros(z.shape[0], dtype=bool)
    part = np.partition(z, -2, axis=1)
    return (part[:, -1] - part[:, -2]) < tol


def _near_tie_top1_top3(z, tol=1e-5):
    if z.shape[1] < 3:
        return _orig["near_tie_tokens"](z, tol)
    srt = np.sort(z, axis=1)
    return (srt[:, -1] - srt[:, -3]) <= tol


def _near_tie_top2_top3(z, tol=1e-5):
    if z.shape[1] < 3:
        return _orig["near_tie_tokens"](z, tol)
    srt = np.sort(z, axis=1)
    return (srt[:, -2] - srt[:, -3]) <= tol


def _near_tie_sign(z, tol=1e-5):
    if z.shape[1] < 2:
        return np.zeros(z.shape[0], dtype=bool)
    part = np.partition(z, -2, axis=1)
    return (part[:, -2] - part[:, -1]) <= tol


def _near_tie_second_strict(z, tol=1e-5):
    if z.shape[1] < 3:
        return np.zeros(z.shape[0], dtype=bool)
    srt = np.sort(z, axis=1)
    return (srt[:, -2] - srt[:, -3]) < tol


def _near_tie_second_top1_top2(z, tol=1e-5):
    if z.shape[1] < 3:
        return np.zeros(z.shape[0], dtype=bool)
    srt = np.sort(z, axis=1)
    return (srt[:, -1] - srt[:, -2]) <= tol


def _top1_ignores_nan(z):
    return np.nanargmax(z.astype(np.float32), axis=1).astype(np.int64)


def _second_by_minus_inf(z, first):
    z32 = z.astype(np.float32).copy()
    z32[np.arange(z.shape[0]), first] = -np.inf
    return np.argmax(z32, axis=1).astype(np.int64)


MUTANTS = {
    "near_tie_strict_inequality": ("near_tie_tokens", _near_tie_strict),
    "near_tie_top1_top3_gap": ("near_tie_tokens", _near_tie_top1_top3),
    "near_tie_top2_top3_gap": ("near_tie_tokens", _near_tie_top2_top3),
    "near_tie_sign_flip": ("near_tie_tokens", _near_tie_sign),
    "near_tie_second_strict_inequality": ("near_tie_second", _near_tie_second_strict),
    "near_tie_second_top1_top2_gap": ("near_tie_second", _near_tie_second_top1_top2),
    "top1_ignores_nan": ("top1", _top1_ignores_nan),
    "second_choice_masks_by_minus_inf": ("second_choice", _second_by_minus_inf),
    "ffn_drops_b2": ("expert_ffn", _ffn_no_b2),
    "ffn_drops_b1": ("expert_ffn", _ffn_no_b1),
    "ffn_no_relu": ("expert_ffn", _ffn_no_relu),
    "ffn_relu_after_w2": ("expert_ffn", _ffn_relu_after),
    "ffn_w1_transposed": ("expert_ffn", _ffn_transposed_w1),
    "logits_sign_flip": ("router_logits", _logits_sign),
    "logits_wr_untransposed": ("router_logits", _logits_untransposed),
    "softmax_wrong_axis": ("softmax", _softmax_axis0),
    "softmax_unnormalised": ("softmax", _softmax_no_norm),
    "top1_ties_to_highest": ("top1", _top1_last_tie),
    "top1_argmin": ("top1", _top1_argmin),
    "dispatch_one_based_rank": ("dispatch", _dispatch_one_based),
    "dispatch_capacity_off_by_one": ("dispatch", _dispatch_le),
    "dispatch_reverse_token_order": ("dispatch", _dispatch_reverse_order),
    "aux_missing_n": ("aux_loss", _aux_no_n),
    "aux_gate_only": ("aux_loss", _aux_gate_only),
    "aux_f_times_f": ("aux_loss", _aux_f_squared),
    "capacity_ceil": ("capacity", _capacity_ceil),
    "capacity_floor_then_scale": ("capacity", _capacity_floor_first),
    "bf16_truncates": ("round_to_bf16", _bf16_truncate),
    "combine_no_residual": ("forward", _forward_no_residual),
    "dropped_rows_zeroed": ("forward", _forward_dropped_zero),
    "gate_outside_b2": ("forward", _forward_gate_outside_b2),
    "top2_second_ties_to_highest": ("second_choice", _second_ties_to_highest),
    "top2_gates_renormalised": ("topk_gates", _gates_renormalised),
    "top2_first_choices_first": ("dispatch_topk", _dispatch_first_choices_first),
    "top2_capacity_without_k": ("dispatch_topk", _dispatch_topk_capacity_without_k),
    "reroute_ignores_first_stage": ("reroute_overflow", _reroute_ignores_first_stage),
    "reroute_reverse_order": ("reroute_overflow", _reroute_reverse_order),
    "reroute_none": ("reroute_overflow", _reroute_none),
    "gelu_tanh_approximation": ("gelu", _gelu_tanh),
    "geglu_halves_swapped": ("expert_ffn", _geglu_halves_swapped),
    "geglu_relu_gate": ("expert_ffn", _geglu_relu_gate),
    "bwd_no_relu_mask": ("expert_backward", _eb_no_relu_mask),
    "bwd_no_gate": ("expert_backward", _eb_no_gate),
    "bwd_dg_without_b2": ("expert_backward", _eb_dg_without_b2),
    "bwd_db2_ungated": ("expert_backward", _eb_db2_ungated),
    "bwd_aux_grad_without_n": ("aux_prob_grad", _aux_grad_without_n),
    "bwd_softmax_uncentred": ("softmax_backward", _softmax_bwd_uncentred),
    "bwd_softmax_sign": ("softmax_backward", _softmax_bwd_sign),
    "bwd_dx_without_residual": ("backward", _bwd_no_residual),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception as exc:  # noqa: BLE001 -- any failure of a pin counts
            caught.append(f"{pin.__name__}: {type(exc).__name__}")
    assert caught, f"mutant {name} passed every pin"
