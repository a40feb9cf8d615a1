"""Brute-force SwitchFFN forward: pure Python, one token at a time.

An independent second reading of the layer for tiny inputs, used to pin the
oracle.  It shares nothing with the oracle: no numpy, a token's rank is found
by scanning every earlier token, each dot product is an exactly rounded
math.fsum, and the fp32 rounding of a logit goes through struct.
"""
from __future__ import annotations

import math
import struct


def to_f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def dot(a, b) -> float:
    return math.fsum(ai * bi for ai, bi in zip(a, b))


def brute_gelu(a: float) -> float:
    return a * 0.5 * math.erfc(-a / math.sqrt(2.0))


def brute_hidden(xt, W1e, b1e, F, activation):
    """Hidden activations of one token: ReLU of F pre-activations, or (geglu) GELU of
    the first F times the next F."""
    pre = [dot(W1e[j], xt) + (b1e[j] if b1e is not None else 0.0) for j in range(len(W1e))]
    if activation == "relu":
        return [a if a > 0.0 else 0.0 for a in pre]
    return [brute_gelu(pre[j]) * pre[F + j] for j in range(F)]


def brute_forward(x, Wr, W1, b1, W2, b2, CF, no_residual=False, activation="relu"):
    """All arguments are nested lists of floats (b1/b2 may be None)."""
    T = len(x)
    N = len(Wr)
    d = len(x[0]) if T else len(Wr[0])
    F = len(W2[0][0])
    C = math.floor(CF * T / N)

    choice, probs = [], []
    for t in range(T):
        z = [dot(x[t], Wr[i]) for i in range(N)]
        z32 = [to_f32(v) for v in z]
        best = 0
        for i in range(1, N):
            if z32[i] > z32[best]:
                best = i
        m = max(z)
        ex = [math.exp(v - m) for v in z]
        s = math.fsum(ex)
        choice.append(best)
        probs.append([v / s for v in ex])

    slot, y = [], []
    for t in range(T):
        e = choice[t]
        rank = sum(1 for s_ in range(t) if choice[s_] == e)
        accepted = rank < C
        slot.append(rank if accepted else -1)
        if not accepted:
            y.append([0.0] * d if no_residual else list(x[t]))
            continue
        g = probs[t][e]
        h = brute_hidden(x[t], W1[e], None if b1 is None else b1[e], F, activation)
        row = []
        for i in range(d):
            o = dot(W2[e][i], h) + (b2[e][i] if b2 is not None else 0.0)
            row.append(g * o if no_residual else x[t][i] + g * o)
        y.append(row)

    aux = 0.0
    for i in range(N):
        f_i = sum(1 for t in range(T) if choice[t] == i) / T
        P_i = math.fsum(probs[t][i] for t in range(T)) / T
        aux += f_i * P_i
    aux *= N
    gate = [probs[t][choice[t]] for t in range(T)]
    return {"C": C, "expert_idx": choice, "slot": slot, "gate": gate, "aux_loss": aux, "y": y,
            "probs": probs}


def brute_forward_top2(x, Wr, W1, b1, W2, b2, CF, no_residual=False):
    """Top-2 routing, one token at a time: the two largest fp32 logits (ties to the
    lowest index), raw gates, capacity floor(CF * 2T / N), expert columns filled in
    token order, y = x + the gated outputs of the accepted choices."""
    T = len(x)
    N = len(Wr)
    d = len(x[0]) if T else len(Wr[0])
    F = len(W1[0])
    C = math.floor(CF * (2 * T) / N)

    choices, probs = [], []
    for t in range(T):
        z = [dot(x[t], Wr[i]) for i in range(N)]
        z32 = [to_f32(v) for v in z]
        first = 0
        for i in range(1, N):
            if z32[i] > z32[first]:
                first = i
        second = 1 if first == 0 else 0
        for i in range(N):
            if i != first and z32[i] > z32[second]:
                second = i
        m = max(z)
        ex = [math.exp(v - m) for v in z]
        s = math.fsum(ex)
        choices.append((first, second))
        probs.append([v / s for v in ex])

    slot, gate, y = [], [], []
    for t in range(T):
        row = [0.0] * d if no_residual else list(x[t])
        slots, gates = [], []
        for e in choices[t]:
            rank = sum(1 for s_ in range(t) if e in choices[s_])
            g = probs[t][e]
            gates.append(g)
            if rank >= C:
                slots.append(-1)
                continue
            slots.append(rank)
            h = []
            for j in range(F):
                a = dot(W1[e][j], x[t]) + (b1[e][j] if b1 is not None else 0.0)
                h.append(a if a > 0.0 else 0.0)
            for i in range(d):
                row[i] += g * (dot(W2[e][i], h) + (b2[e][i] if b2 is not None else 0.0))
        slot.append(slots)
        gate.append(gates)
        y.append(row)

    aux = 0.0
    for i in range(N):
        f_i = sum(1 for t in range(T) if choices[t][0] == i) / T
        P_i = math.fsum(probs[t][i] for t in range(T)) / T
        aux += f_i * P_i
    aux *= N
    return {"C": C, "expert_idx": [list(c) for c in choices], "slot": slot, "gate": gate,
            "aux_loss": aux, "y": y, "probs": probs}


def brute_forward_reroute(x, Wr, W1, b1, W2, b2, CF, no_residual=False):
    """Top-1 routing with No-Token-Left-Behind rerouting, one token at a time: a token
    refused by its first choice (rank >= C) takes the next free position of its second
    choice after that expert's first-stage tokens, if one is left."""
    T = len(x)
    N = len(Wr)
    d = len(x[0]) if T else len(Wr[0])
    F = len(W1[0])
    C = math.floor(CF * T / N)
    choices, probs = [], []
    for t in range(T):
        z = [dot(x[t], Wr[i]) for i in range(N)]
        z32 = [to_f32(v) for v in z]
        first = 0
        for i in range(1, N):
            if z32[i] > z32[first]:
                first = i
        second = 1 if first == 0 else 0
        for i in range(N):
            if i != first and z32[i] > z32[second]:
                second = i
        m = max(z)
        ex = [math.exp(v - m) for v in z]
        s = math.fsum(ex)
        choices.append((first, second))
        probs.append([v / s for v in ex])

    first_rank = [sum(1 for s_ in range(t) if choices[s_][0] == choices[t][0]) for t in range(T)]
    stage1 = [first_rank[t] < C for t in range(T)]
    used = [min(C, sum(1 for t in range(T) if choices[t][0] == e)) for e in range(N)]
    expert, slot = [], []
    for t in range(T):
        if stage1[t]:
            expert.append(choices[t][0])
            slot.append(first_rank[t])
            continue
        e = choices[t][1]
        before = sum(1 for s_ in range(t) if not stage1[s_] and choices[s_][1] == e)
        pos = used[e] + before
        if pos < C:
            expert.append(e)
            slot.append(pos)
        else:
            expert.append(choices[t][0])
            slot.append(-1)

    y, gate = [], []
    for t in range(T):
        e = expert[t]
        g = probs[t][e]
        gate.append(g)
        if slot[t] < 0:
            y.append([0.0] * d if no_residual else list(x[t]))
            continue
        h = []
        for j in range(F):
            a = dot(W1[e][j], x[t]) + (b1[e][j] if b1 is not None else 0.0)
            h.append(a if a > 0.0 else 0.0)
        row = []
        for i in range(d):
            o = dot(W2[e][i], h) + (b2[e][i] if b2 is not None else 0.0)
            row.append(g * o if no_residual else x[t][i] + g * o)
        y.append(row)

    aux = 0.0
    for i in range(N):
        f_i = sum(1 for t in range(T) if choices[t][0] == i) / T
        P_i = math.fsum(probs[t][i] for t in range(T)) / T
        aux += f_i * P_i
    aux *= N
    return {"C": C, "expert_idx": expert, "slot": slot, "gate": gate, "aux_loss": aux, "y": y}
