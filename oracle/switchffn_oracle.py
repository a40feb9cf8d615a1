"""CPU oracle for the SwitchFFN forward pass (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It shares no code with
the HIP path; the two meet only in the seeded inputs of switchffn_synth.

Every step below is the plain definition the pages give, written out in the
pages' order, with a library matmul as the only primitive.  Sources:
  [Switch summary] "Switch Transformers: Scaling to Trillion Parameter Models
      with Simple and Efficient Sparsity" (paper-graph-ui summary), section 3.4
      "Detailed, Sentence-Based Technical Breakdown" and section 3.2
      "Big-Picture Architecture (Diagram in Words)".
  [Paper note] "Switch Transformer" (eightmm.github.io note), sections
      "Router", "Expert FFN Layer", "Capacity Factor", "Load-Balancing Loss",
      "Implementation Notes".
  [Explainer] "Switch Transformer, explained." (vibeengines.com), the nine-step
      recipe (steps 2-5).
  [Math-LLMs card] "Chapter 8 - Attention and Transformers" companion reader,
      card 08 "Penalize uneven expert traffic".

Readings where the pages are silent or disagree (each also listed in the
design notes): capacity C = floor(CF*T/N) in IEEE double; the first C tokens of
an expert in flattened token order are accepted; argmax ties go to the lowest
expert index and the decision is taken on fp32 logits (the router precision);
f_i counts the argmax before capacity; P_i averages over all T tokens; the
aux loss is returned without the alpha factor; y = x + g*E(x) for accepted
tokens and y = x for dropped ones; b2 sits inside the gate scaling.

Top-2 routing (the MoE baseline the Switch summary contrasts with, section
"Why Top-1 Routing Matters" and the routing formula before "Switch uses"):
y = x + sum over the two largest p_{t,i} of p_{t,i} E_i(x), raw (not
renormalised) gates; the second choice is the largest of the remaining fp32
logits, ties to the lowest index; the capacity is floor(CF * (k*T) / N)
([Switch summary] 3.4, k x tokens per batch / N x capacity factor); each
expert column is filled in token order (a token holds at most one position
per expert, so both choices of a token are ranked by token); f_i of the aux
loss stays the top-1 (argmax) share.

No-Token-Left-Behind rerouting ([Switch summary] "Distributed Implementation
and Expert Capacity", the No-Token-Left-Behind experiment, and section 5 on
Appendix B / Figure 11): tokens that overflow their first choice are sent to
their second choice.  Reading: two stages (the figure's two-stage process);
stage 1 is the top-1 dispatch; stage 2 takes the overflowed tokens in token
order and fills each expert's slots left after stage 1 (positions
accepted_1[e] ..  C-1) with those whose second choice it is; a token accepted
in stage 2 uses that expert and its gate p[t, e2]; a token refused twice
passes through (y = x) and reports its first choice.

GEGLU experts ([Switch summary] 3.2 "Expert FFNs" names GEGLU beside ReLU and
gives no formula): the gated-GELU unit GELU(W x + b_W) * (V x + b_V) with the
exact GELU a * Phi(a) (Phi the standard normal CDF); W1 then holds the two
up-projections, W in rows 0..F-1 and V in rows F..2F-1, and b1 both biases.

Backward pass (top-1, ReLU experts): the chain rule through the gate and
through P_i of the aux loss, f_i and the routing carrying no gradient (see
backward() for the readings); pinned against central finite differences of
forward() and the closed forms below.

Pins (tests/test_oracle_pins.py): the worked aux-loss example of the
Math-LLMs card (1.15), the uniform-routing closed forms (aux = 1), the
one-expert limit (aux -> N, closed form), N = 1 dense-FFN reduction, the x = 0
and Wr = 0 closed forms, a hand-computed FFN example, capacity edge cases and
a brute-force per-token loop (up to 1200 tokens and 128 experts).  The pages
print no values of a full forward pass at the workload sizes, so none are
stored; every function here is pinned at the sizes above and runs unchanged at
every size.
"""
from __future__ import annotations

import math
from typing import Callable, Iterable, Optional

import numpy as np
from scipy.special import erf as scipy_erf


# ----------------------------------------------------------------------------
# Capacity ([Switch summary] 3.4 "Distributed Implementation and Expert
# Capacity", expert capacity formula; [Paper note] "Capacity Factor";
# [Explainer] step 3).  The three pages round differently; the reading used
# here is floor((CF * T) / N) evaluated in IEEE double in that order.
# ----------------------------------------------------------------------------
def capacity(T: int, N: int, CF: float) -> int:
    if T < 0 or N <= 0 or not math.isfinite(CF) or CF < 0:
        raise ValueError("capacity needs T >= 0, N > 0 and a finite CF >= 0")
    return int(math.floor((float(CF) * float(T)) / float(N)))


# ----------------------------------------------------------------------------
# Router ([Switch summary] 3.4 "Switch Routing: The k=1 Simplification":
# h(x) = W_r . x, p_i(x) = softmax, selected expert = argmax_i p_i(x), gate
# p_{i*}(x); [Paper note] "Router"; [Explainer] step 2 and [Switch summary]
# 3.4 "Selective Precision Training": the router works in float32).
# ----------------------------------------------------------------------------
def router_logits(x: np.ndarray, Wr: np.ndarray) -> np.ndarray:
    """z[t, i] = sum_k x[t, k] * Wr[i, k]  (Wr stored [N, d]), in float64."""
    return np.asarray(x, np.float64) @ np.asarray(Wr, np.float64).T


def softmax(z: np.ndarray) -> np.ndarray:
    """p[t, i] = exp(z[t, i] - m_t) / sum_j exp(z[t, j] - m_t), m_t = max_i z[t, i]."""
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=1, keepdims=True)


def top1(z: np.ndarray) -> np.ndarray:
    """Lowest expert index among the largest fp32 logits of each token.

    numpy's argmax order: the first maximum wins, and a NaN counts as larger than
    every number (the pages never meet non-finite logits; this reading gives every
    token an expert in [0, N) whatever its logits hold).
    """
    z32 = z.astype(np.float32)
    return np.argmax(z32, axis=1).astype(np.int64)


def router(x: np.ndarray, Wr: np.ndarray) -> dict:
    z = router_logits(x, Wr)
    probs = softmax(z)
    expert_idx = top1(z)
    gate = probs[np.arange(z.shape[0]), expert_idx]
    return {"logits": z, "probs": probs, "expert_idx": expert_idx, "gate": gate}


# ----------------------------------------------------------------------------
# Dispatch with the capacity mask ([Switch summary] 3.4 "Distributed
# Implementation and Expert Capacity": a running count per expert column gives
# each token its position; positions past the capacity are masked out and the
# token overflows).  Token order is the flattened order t = b*L + l
# ([Paper note] "Implementation Notes -- Batch and Sequence Shape").
# ----------------------------------------------------------------------------
def dispatch(expert_idx: np.ndarray, N: int, C: int) -> dict:
    T = len(expert_idx)
    count = np.zeros(N, dtype=np.int64)
    rank = np.empty(T, dtype=np.int64)
    for t in range(T):
        e = int(expert_idx[t])
        rank[t] = count[e]          # tokens of expert e seen before t
        count[e] += 1
    slot = np.where(rank < C, rank, -1)
    accepted = np.minimum(count, C)
    offset = np.zeros(N + 1, dtype=np.int64)
    offset[1:] = np.cumsum(accepted)
    row2tok = np.empty(int(offset[-1]), dtype=np.int64)
    for t in range(T):
        if slot[t] >= 0:
            row2tok[offset[int(expert_idx[t])] + slot[t]] = t
    return {"hist": count, "rank": rank, "slot": slot, "accepted": accepted,
            "offset": offset, "row2tok": row2tok}


def second_choice(z: np.ndarray, first: np.ndarray) -> np.ndarray:
    """Lowest expert index among the largest fp32 logits other than the first choice.

    The first choice is removed from each row (not masked by -inf, which would tie
    with a row of -inf logits); argmax over the remaining experts in index order.
    """
    z32 = z.astype(np.float32)
    T, N = z32.shape
    j = np.arange(N - 1)[None, :]
    rest = j + (j >= np.asarray(first)[:, None])      # the other experts, increasing
    pick = np.argmax(np.take_along_axis(z32, rest, axis=1), axis=1)
    return rest[np.arange(T), pick].astype(np.int64)


def topk_gates(probs: np.ndarray, choices: np.ndarray) -> np.ndarray:
    """Raw gates p[t, e_{t,c}] of the chosen experts (not renormalised)."""
    return probs[np.arange(probs.shape[0])[:, None], choices]


def dispatch_topk(choices: np.ndarray, N: int, C: int) -> dict:
    """Dispatch of k choices per token: each expert column is filled in token order."""
    T, k = choices.shape
    count = np.zeros(N, dtype=np.int64)
    rank = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        for c in range(k):
            e = int(choices[t, c])
            rank[t, c] = count[e]   # tokens holding a choice of e before t
            count[e] += 1
    slot = np.where(rank < C, rank, -1)
    accepted = np.minimum(count, C)
    offset = np.zeros(N + 1, dtype=np.int64)
    offset[1:] = np.cumsum(accepted)
    row2tok = np.empty(int(offset[-1]), dtype=np.int64)
    row2choice = np.empty(int(offset[-1]), dtype=np.int64)
    for t in range(T):
        for c in range(k):
            if slot[t, c] >= 0:
                row = offset[int(choices[t, c])] + slot[t, c]
                row2tok[row] = t
                row2choice[row] = c
    return {"hist": count, "rank": rank, "slot": slot, "accepted": accepted,
            "offset": offset, "row2tok": row2tok, "row2choice": row2choice}


# ----------------------------------------------------------------------------
# Load-balancing auxiliary loss ([Switch summary] 3.4 "The Load-Balancing
# Auxiliary Loss": f_i = (1/T) sum_x 1{argmax p(x) = i}, P_i = (1/T) sum_x
# p_i(x), loss = alpha * N * sum_i f_i P_i; [Math-LLMs card] card 08).  Returned
# without alpha.
# ----------------------------------------------------------------------------
def aux_loss(expert_idx: np.ndarray, probs: np.ndarray) -> float:
    T, N = probs.shape
    f = np.bincount(expert_idx, minlength=N).astype(np.float64) / T
    P = probs.sum(axis=0) / T
    return float(N * np.dot(f, P))


# ----------------------------------------------------------------------------
# Expert FFN ([Paper note] "Expert FFN Layer": E_i(x) = W_{2,i} sigma(W_{1,i} x
# + b_{1,i}) + b_{2,i}; sigma = ReLU, [Switch summary] 3.2 "Expert FFNs").
# W1 is stored [F, d] and W2 [d, F] per expert.
# ----------------------------------------------------------------------------
def gelu(a: np.ndarray) -> np.ndarray:
    """GELU(a) = a * Phi(a), Phi the standard normal CDF (the exact form, via erf)."""
    return 0.5 * a * (1.0 + scipy_erf(a / math.sqrt(2.0)))


def expert_ffn(xe: np.ndarray, W1e: np.ndarray, b1e, W2e: np.ndarray, b2e,
               activation: str = "relu") -> np.ndarray:
    """E(x) = W2 sigma(W1 x + b1) + b2 for the rows of xe.

    activation "geglu" ([Switch summary] 3.2 names it beside ReLU): W1e holds
    2F rows, the gate projection W (rows 0..F-1) then the linear projection V
    (rows F..2F-1), b1e likewise, and h = GELU(W x + b_W) * (V x + b_V).
    """
    a = xe @ np.asarray(W1e, np.float64).T
    if b1e is not None:
        a = a + np.asarray(b1e, np.float64)
    if activation == "relu":
        h = np.maximum(a, 0.0)
    elif activation == "geglu":
        F = a.shape[1] // 2
        h = gelu(a[:, :F]) * a[:, F:]
    else:
        raise ValueError(activation)
    o = h @ np.asarray(W2e, np.float64).T
    if b2e is not None:
        o = o + np.asarray(b2e, np.float64)
    return o


# ----------------------------------------------------------------------------
# Rounding of the layer output to the storage type (once, from float64).
# ----------------------------------------------------------------------------
def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each float64, returned as float64."""
    v = np.asarray(v, np.float64)
    m, e = np.frexp(v)                 # v = m * 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0)             # 8 significant bits, round half to even
    return np.ldexp(q, e - 8)


def round_to_dtype(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_to_bf16(v)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# The whole layer ([Switch summary] 3.2 "Information flow through a Switch
# layer": route, dispatch, expert, scale by the gate, add on the residual;
# overflow tokens bypass the expert and pass through unchanged; [Explainer]
# step 4).
# ----------------------------------------------------------------------------
ExpertSource = Callable[[int], tuple]


def forward(x, Wr, experts, CF: float, dtype: str = "fp32", *, no_residual: bool = False,
            expert_idx: Optional[np.ndarray] = None,
            only_experts: Optional[Iterable[int]] = None, k: int = 1,
            activation: str = "relu") -> dict:
    """Run the layer on float64 inputs.

    k: experts per token, 1 (Switch routing) or 2 (top-2 routing; expert_idx,
        slot, gate and rank are then [T, 2], choice minor).

    experts: (W1 [N,F,d], b1 [N,F] | None, W2 [N,d,F], b2 [N,d] | None), or a
        callable e -> (W1e, b1e, W2e, b2e) for weights drawn one expert at a time.
    expert_idx: replay a given routing instead of the oracle's own top-1 (the
        probabilities, gate and aux loss still come from the oracle's logits).
    only_experts: compute expert outputs for these experts only; the y rows of
        other experts' accepted tokens are NaN.
    no_residual: y = g * E(x) for accepted tokens and 0 for dropped ones.
    activation: "relu", or "geglu" (W1 [N, 2F, d] and b1 [N, 2F]; see expert_ffn).
    """
    if k == 2:
        return _forward_top2(x, Wr, experts, CF, dtype, no_residual=no_residual,
                             expert_idx=expert_idx, only_experts=only_experts,
                             activation=activation)
    if k != 1:
        raise ValueError("k must be 1 or 2")
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    N = np.asarray(Wr).shape[0]
    C = capacity(T, N, CF)
    r = router(x, Wr)
    eidx = r["expert_idx"] if expert_idx is None else np.asarray(expert_idx, np.int64)
    gate = r["probs"][np.arange(T), eidx]
    dp = dispatch(eidx, N, C)
    aux = aux_loss(eidx, r["probs"])

    if callable(experts):
        get = experts
    else:
        W1, b1, W2, b2 = experts
        def get(e):
            return (W1[e], None if b1 is None else b1[e], W2[e], None if b2 is None else b2[e])

    y = np.zeros_like(x) if no_residual else x.copy()
    todo = range(N) if only_experts is None else sorted(set(int(e) for e in only_experts))
    if only_experts is not None:
        for e in range(N):
            if e not in todo:
                y[dp["row2tok"][dp["offset"][e]:dp["offset"][e + 1]]] = np.nan
    for e in todo:
        rows = dp["row2tok"][dp["offset"][e]:dp["offset"][e + 1]]
        if len(rows) == 0:
            continue
        W1e, b1e, W2e, b2e = get(e)
        o = expert_ffn(x[rows], W1e, b1e, W2e, b2e, activation)
        contrib = gate[rows, None] * o
        y[rows] = contrib if no_residual else x[rows] + contrib

    return {
        "C": C, "logits": r["logits"], "probs": r["probs"], "expert_idx": eidx,
        "router_expert_idx": r["expert_idx"], "gate": gate, "aux_loss": aux,
        "y64": y, "y": round_to_dtype(y, dtype), **dp,
    }


def reroute_overflow(first: np.ndarray, second: np.ndarray, N: int, C: int) -> dict:
    """Two-stage dispatch: top-1 first, then overflowed tokens to their second choice."""
    T = len(first)
    d1 = dispatch(first, N, C)
    used = d1["accepted"].copy()            # stage-1 rows of each expert
    expert = first.copy()
    slot = d1["slot"].copy()
    count2 = np.zeros(N, dtype=np.int64)
    for t in range(T):                      # stage 2, token order
        if slot[t] >= 0:
            continue
        e = int(second[t])
        pos = used[e] + count2[e]           # next free position after stage 1
        count2[e] += 1
        if pos < C:
            slot[t] = pos
            expert[t] = e
    accepted = np.minimum(used + count2, C)
    offset = np.zeros(N + 1, dtype=np.int64)
    offset[1:] = np.cumsum(accepted)
    row2tok = np.empty(int(offset[-1]), dtype=np.int64)
    for t in range(T):
        if slot[t] >= 0:
            row2tok[offset[int(expert[t])] + slot[t]] = t
    return {"hist": d1["hist"], "rank": d1["rank"], "slot": slot, "accepted": accepted,
            "offset": offset, "row2tok": row2tok, "expert": expert, "rerouted": count2}


def forward_reroute(x, Wr, experts, CF: float, dtype: str = "fp32", *, no_residual: bool = False,
                    expert_idx: Optional[np.ndarray] = None,
                    only_experts: Optional[Iterable[int]] = None,
                    activation: str = "relu") -> dict:
    """The top-1 layer with No-Token-Left-Behind rerouting (see the header).

    expert_idx: replay a given pair of choices [T, 2] (first, second) instead of the
    oracle's own; the returned expert_idx is the expert each token ends in.
    """
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    N = np.asarray(Wr).shape[0]
    if N < 2:
        raise ValueError("rerouting needs N >= 2")
    C = capacity(T, N, CF)
    r = router(x, Wr)
    first = r["expert_idx"]
    own = np.stack([first, second_choice(r["logits"], first)], axis=1)
    choices = own if expert_idx is None else np.asarray(expert_idx, np.int64).reshape(T, 2)
    dp = reroute_overflow(choices[:, 0], choices[:, 1], N, C)
    eidx = dp.pop("expert")
    gate = r["probs"][np.arange(T), eidx]
    aux = aux_loss(choices[:, 0], r["probs"])

    if callable(experts):
        get = experts
    else:
        W1, b1, W2, b2 = experts
        def get(e):
            return (W1[e], None if b1 is None else b1[e], W2[e], None if b2 is None else b2[e])

    y = np.zeros_like(x) if no_residual else x.copy()
    todo = range(N) if only_experts is None else sorted(set(int(e) for e in only_experts))
    if only_experts is not None:
        for e in range(N):
            if e not in todo:
                y[dp["row2tok"][dp["offset"][e]:dp["offset"][e + 1]]] = np.nan
    for e in todo:
        rows = dp["row2tok"][dp["offset"][e]:dp["offset"][e + 1]]
        if len(rows) == 0:
            continue
        W1e, b1e, W2e, b2e = get(e)
        o = expert_ffn(x[rows], W1e, b1e, W2e, b2e, activation)
        contrib = gate[rows, None] * o
        y[rows] = contrib if no_residual else x[rows] + contrib

    return {
        "C": C, "logits": r["logits"], "probs": r["probs"], "expert_idx": eidx,
        "choices": choices, "router_choices": own, "gate": gate, "aux_loss": aux,
        "y64": y, "y": round_to_dtype(y, dtype), **dp,
    }


def _forward_top2(x, Wr, experts, CF, dtype, *, no_residual, expert_idx, only_experts,
                  activation) -> dict:
    """Top-2 routing: y_t = x_t + sum_c [accepted] p_{t,e_c} E_{e_c}(x_t) (see the header)."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    N = np.asarray(Wr).shape[0]
    if N < 2:
        raise ValueError("top-2 routing needs N >= 2")
    C = capacity(2 * T, N, CF)
    r = router(x, Wr)
    first = r["expert_idx"]
    own = np.stack([first, second_choice(r["logits"], first)], axis=1)
    choices = own if expert_idx is None else np.asarray(expert_idx, np.int64).reshape(T, 2)
    gate = topk_gates(r["probs"], choices)
    dp = dispatch_topk(choices, N, C)
    aux = aux_loss(choices[:, 0], r["probs"])

    if callable(experts):
        get = experts
    else:
        W1, b1, W2, b2 = experts
        def get(e):
            return (W1[e], None if b1 is None else b1[e], W2[e], None if b2 is None else b2[e])

    y = np.zeros_like(x) if no_residual else x.copy()
    todo = range(N) if only_experts is None else sorted(set(int(e) for e in only_experts))
    if only_experts is not None:
        for e in range(N):
            if e not in todo:
                y[dp["row2tok"][dp["offset"][e]:dp["offset"][e + 1]]] = np.nan
    for e in todo:
        lo, hi = dp["offset"][e], dp["offset"][e + 1]
        rows = dp["row2tok"][lo:hi]
        if len(rows) == 0:
            continue
        W1e, b1e, W2e, b2e = get(e)
        o = expert_ffn(x[rows], W1e, b1e, W2e, b2e, activation)
        y[rows] += gate[rows, dp["row2choice"][lo:hi], None] * o   # distinct rows per expert

    return {
        "C": C, "logits": r["logits"], "probs": r["probs"], "expert_idx": choices,
        "router_expert_idx": own, "gate": gate, "aux_loss": aux,
        "y64": y, "y": round_to_dtype(y, dtype), **dp,
    }


# ----------------------------------------------------------------------------
# Backward pass of the top-1 ReLU layer.  The routing (argmax, capacity) is a
# piecewise-constant choice and carries no gradient; the router learns through
# the gate p_{t,e_t} that scales the expert output ([Switch summary] 3.4
# "Switch Routing: The k=1 Simplification"; [Explainer] "Why one expert is
# enough") and through P_i of the aux loss, f_i being a count with no gradient
# ([Explainer] symbol list under "Why one expert is enough"; [Switch summary]
# 3.4 "The Load-Balancing Auxiliary Loss").  Chain rule, for accepted t with
# expert e, a_t = W1_e x_t + b1_e, h_t = ReLU(a_t), o_t = W2_e h_t + b2_e:
#   dO_t = g_t dy_t,  dg_t = dy_t . o_t
#   dW2_e = sum_t dO_t h_t^T,  db2_e = sum_t dO_t
#   da_t = (W2_e^T dO_t) * [a_t > 0]          (ReLU'(0) taken as 0)
#   dW1_e = sum_t da_t x_t^T,  db1_e = sum_t da_t
#   u_{t,i} = d_aux N f_i / T + [t accepted][i = e_t] dg_t
#   dz_t = p_t * (u_t - p_t . u_t)            (softmax Jacobian)
#   dWr = sum_t dz_t x_t^T
#   dx_t = dy_t + [t accepted] W1_e^T da_t + Wr^T dz_t
# where d_aux is the gradient of the loss with respect to the aux value.
# ----------------------------------------------------------------------------
def expert_backward(xe, W1e, b1e, W2e, b2e, dye, ge) -> dict:
    """One expert's rows: forward recomputed in float64, then the chain rule."""
    W1e = np.asarray(W1e, np.float64)
    W2e = np.asarray(W2e, np.float64)
    a = xe @ W1e.T + (0.0 if b1e is None else np.asarray(b1e, np.float64))
    h = np.maximum(a, 0.0)
    o = h @ W2e.T + (0.0 if b2e is None else np.asarray(b2e, np.float64))
    dO = ge[:, None] * dye
    da = (dO @ W2e) * (a > 0.0)
    return {"dW1": da.T @ xe, "db1": da.sum(axis=0), "dW2": dO.T @ h, "db2": dO.sum(axis=0),
            "dx": da @ W1e, "dg": np.sum(dye * o, axis=1)}


def aux_prob_grad(hist: np.ndarray, T: int, d_aux: float) -> np.ndarray:
    """dL/dp_{t,i} from the aux term: d_aux * N * f_i / T (the same for every t)."""
    N = len(hist)
    return d_aux * N * (np.asarray(hist, np.float64) / T) / T


def softmax_backward(p: np.ndarray, u: np.ndarray) -> np.ndarray:
    """dz from dL/dp through p = softmax(z): p * (u - p . u), row by row."""
    return p * (u - np.sum(p * u, axis=1, keepdims=True))


def backward(x, Wr, experts, CF: float, dy, d_aux: float = 0.0, *,
             expert_idx: Optional[np.ndarray] = None,
             only_experts: Optional[Iterable[int]] = None) -> dict:
    """Gradients of L(y, aux) given dy = dL/dy [T, d] and d_aux = dL/daux.

    experts, expert_idx and only_experts as for forward (expert_idx replays a given
    routing).  only_experts: the weight and bias gradients of the other experts are
    NaN, and so are the dz and dx rows of their accepted tokens (whose dg is then
    unknown); dWr, a sum over every token, is computed only when only_experts is None.
    Returns dx [T, d], dWr [N, d], dW1 [N, F, d], db1 [N, F], dW2 [N, d, F],
    db2 [N, d] (float64), and dg [T] and dz [T, N].
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    Wr = np.asarray(Wr, np.float64)
    T, d = x.shape
    N = Wr.shape[0]
    C = capacity(T, N, CF)
    r = router(x, Wr)
    p = r["probs"]
    eidx = r["expert_idx"] if expert_idx is None else np.asarray(expert_idx, np.int64)
    gate = p[np.arange(T), eidx]
    dp = dispatch(eidx, N, C)

    if callable(experts):
        get = experts
    else:
        W1, b1, W2, b2 = experts
        def get(e):
            return (W1[e], None if b1 is None else b1[e], W2[e], None if b2 is None else b2[e])

    F = None
    dx = dy.copy()
    dg = np.zeros(T)
    grads = {}
    todo = range(N) if only_experts is None else sorted(set(int(e) for e in only_experts))
    for e in todo:
        W1e, b1e, W2e, b2e = get(e)
        F = np.asarray(W1e).shape[0]
        rows = dp["row2tok"][dp["offset"][e]:dp["offset"][e + 1]]
        g = expert_backward(x[rows], W1e, b1e, W2e, b2e, dy[rows], gate[rows])
        dg[rows] = g["dg"]
        grads[e] = (g["dW1"], g["db1"], g["dW2"], g["db2"])
        dx[rows] += g["dx"]
    if F is None:
        F = np.asarray(get(0)[0]).shape[0]
    dW1 = np.full((N, F, d), np.nan)
    db1 = np.full((N, F), np.nan)
    dW2 = np.full((N, d, F), np.nan)
    db2 = np.full((N, d), np.nan)
    for e, (g1, gb1, g2, gb2) in grads.items():
        dW1[e], db1[e], dW2[e], db2[e] = g1, gb1, g2, gb2

    out = {"C": C, "expert_idx": eidx, "slot": dp["slot"], "gate": gate, "dg": dg,
           "dW1": dW1, "db1": db1, "dW2": dW2, "db2": db2}
    u = np.broadcast_to(aux_prob_grad(dp["hist"], T, d_aux), (T, N)).copy()
    acc = dp["slot"] >= 0
    u[np.nonzero(acc)[0], eidx[acc]] += dg[acc]
    dz = softmax_backward(p, u)
    dx = dx + dz @ Wr
    if only_experts is not None:
        for e in range(N):
            if e not in grads:
                rows = dp["row2tok"][dp["offset"][e]:dp["offset"][e + 1]]
                dz[rows] = np.nan
                dx[rows] = np.nan
        out.update(dz=dz, dx=dx)
        return out
    out.update(dz=dz, dWr=dz.T @ x, dx=dx)
    return out


# ----------------------------------------------------------------------------
# Where the routing choice is ambiguous.  The router decides on fp32 logits
# ([Switch summary] 3.4 "Selective Precision Training"); two fp32 dot products
# of the same operands summed in different orders can differ by a few fp32
# ulps, so where the largest logits lie within tol of each other either choice
# is a correct fp32 router.  Parity checks exempt these tokens from the
# bit-exact expert comparison (and check the choice lies within tol instead).
# ----------------------------------------------------------------------------
def near_tie_tokens(logits: np.ndarray, tol: float = 1e-5) -> np.ndarray:
    """Tokens whose largest and second-largest logits differ by at most tol."""
    if logits.shape[1] < 2:
        return np.zeros(logits.shape[0], dtype=bool)
    part = np.partition(logits, -2, axis=1)
    return (part[:, -1] - part[:, -2]) <= tol


def near_tie_second(logits: np.ndarray, tol: float = 1e-5) -> np.ndarray:
    """Tokens whose second- and third-largest logits differ by at most tol (the
    second choice of top-2 routing or rerouting is then ambiguous)."""
    if logits.shape[1] < 3:
        return np.zeros(logits.shape[0], dtype=bool)
    srt = np.sort(logits, axis=1)
    return (srt[:, -2] - srt[:, -3]) <= tol
