"""Pins of the CPU oracle: facts fixed by the pages or by the mathematics.

Each pin is a plain function that raises AssertionError on failure, so the
same set can be run against the oracle as written (test_oracle_pins.py) and
against deliberately broken copies of it (test_oracle_mutations.py).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle.switchffn_oracle as O
from bruteforce import brute_forward, brute_forward_reroute, brute_forward_top2

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f32(a):
    return np.asarray(a, np.float32).astype(np.float64)


def random_case(seed, T, d, F, N, bias=False, wscale=0.3):
    rng = np.random.default_rng(seed)
    x = _f32(rng.standard_normal((T, d)))
    Wr = _f32(rng.standard_normal((N, d)) * wscale)
    W1 = _f32(rng.standard_normal((N, F, d)) * wscale)
    W2 = _f32(rng.standard_normal((N, d, F)) * wscale)
    b1 = _f32(rng.standard_normal((N, F)) * wscale) if bias else None
    b2 = _f32(rng.standard_normal((N, d)) * wscale) if bias else None
    return x, Wr, W1, b1, W2, b2


def _tolist(a):
    return None if a is None else np.asarray(a).tolist()


def _close(a, b, tol):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.abs(a - b) <= tol * (1.0 + np.abs(b))), float(np.max(np.abs(a - b)))


def _zero_ffn(N, F, d):
    return (np.zeros((N, F, d)), None, np.zeros((N, d, F)), None)


# ---------------------------------------------------------------------------
# Aux loss: the worked example of the Math-LLMs card 08 and its closed forms.
# ---------------------------------------------------------------------------
def pin_aux_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "aux_worked_example.json")))
    rows = np.array(g["book_batch_rows"], np.float64)
    N = g["book_batch"]["experts"]
    assert rows.shape == (g["book_batch"]["tokens"], N)
    x = np.log(rows)
    Wr = np.eye(N)
    r = O.forward(x, Wr, _zero_ffn(N, 4, N), CF=2.0)
    T = rows.shape[0]
    f = np.bincount(r["expert_idx"], minlength=N) / T
    _close(f, g["book_batch"]["f"], 1e-15)
    _close(r["probs"].mean(axis=0), g["book_batch"]["p"], 1e-12)
    assert abs(r["aux_loss"] - g["book_batch"]["loss"]) < 1e-12, r["aux_loss"]

    rows = np.array(g["check_question_rows"], np.float64)
    r = O.forward(np.log(rows), np.eye(4), _zero_ffn(4, 4, 4), CF=2.0)
    f = np.bincount(r["expert_idx"], minlength=4) / rows.shape[0]
    _close(f, g["check_question"]["f"], 1e-15)
    assert abs(r["aux_loss"] - g["check_question"]["loss"]) < 1e-12, r["aux_loss"]


def pin_aux_uniform_probs():
    # Wr = 0: every logit is 0, p is uniform, and the aux loss is 1 whatever f is
    # (all tokens tie and go to expert 0).
    for N in (1, 3, 8):
        x, _, W1, b1, W2, b2 = random_case(1, 20, 6, 5, N)
        r = O.forward(x, np.zeros((N, 6)), (W1, b1, W2, b2), CF=1.0)
        assert np.all(r["expert_idx"] == 0)
        _close(r["gate"], np.full(20, 1.0 / N), 1e-15)
        assert abs(r["aux_loss"] - 1.0) < 1e-12


def pin_aux_uniform_f():
    # x_t = s * e_{t mod N}, Wr = I: each expert gets T/N tokens, sum_i P_i = 1, aux = 1.
    N, T, s = 4, 12, 3.0
    x = np.zeros((T, N))
    x[np.arange(T), np.arange(T) % N] = s
    r = O.forward(x, np.eye(N), _zero_ffn(N, 2, N), CF=1.0)
    assert np.all(np.bincount(r["expert_idx"], minlength=N) == T // N)
    assert abs(r["aux_loss"] - 1.0) < 1e-12


def pin_aux_one_expert_limit():
    # Every token prefers expert 0 by a margin s: p_0 = 1 / (1 + (N-1) e^-s), so
    # aux = N * 1 * p_0, which tends to N as s grows.
    N, T = 6, 10
    for s in (1.0, 5.0, 40.0):
        x = np.zeros((T, N))
        x[:, 0] = s
        r = O.forward(x, np.eye(N), _zero_ffn(N, 2, N), CF=float(N))
        expect = N / (1.0 + (N - 1) * math.exp(-s))
        assert abs(r["aux_loss"] - expect) < 1e-12 * N, (r["aux_loss"], expect)


def pin_aux_can_fall_below_one():
    # The inner sum is not bounded below by 1/N for arbitrary routings: with
    # p rows (.51,.49), (.51,.49), (.01,.99): f = (2/3, 1/3), P = (1.03/3, 1.97/3),
    # aux = 2 * (2.06 + 1.97) / 9 = 8.06 / 9.
    rows = np.array([[0.51, 0.49], [0.51, 0.49], [0.01, 0.99]])
    r = O.forward(np.log(rows), np.eye(2), _zero_ffn(2, 2, 2), CF=2.0)
    assert abs(r["aux_loss"] - 8.06 / 9.0) < 1e-12, r["aux_loss"]


# ---------------------------------------------------------------------------
# Capacity and dispatch.
# ---------------------------------------------------------------------------
def pin_capacity_values():
    assert O.capacity(64, 4, 1.0) == 16
    assert O.capacity(8192, 64, 1.25) == 160
    assert O.capacity(16384, 128, 1.0) == 128
    assert O.capacity(32768, 128, 1.25) == 320
    assert O.capacity(65536, 2048, 1.0) == 32
    assert O.capacity(10, 4, 1.0) == 2       # 2.5 rounds down
    assert O.capacity(10, 4, 1.25) == 3      # 3.125
    assert O.capacity(7, 3, 1.0) == 2
    assert O.capacity(7, 3, 0.0) == 0
    assert O.capacity(7, 3, 3.0) == 7        # CF = N admits every token
    assert O.capacity(0, 3, 1.0) == 0
    for bad in ((5, 0, 1.0), (5, 2, -0.5), (5, 2, float("nan")), (5, 2, float("inf"))):
        try:
            O.capacity(*bad)
        except ValueError:
            continue
        raise AssertionError(f"capacity{bad} accepted")


def pin_dispatch_bruteforce():
    rng = np.random.default_rng(7)
    for T, N, C in ((1, 1, 0), (1, 1, 1), (50, 3, 10), (200, 7, 20), (64, 4, 64), (33, 5, 0)):
        skew = rng.dirichlet(np.ones(N) * 0.5)
        eidx = rng.choice(N, size=T, p=skew)
        dp = O.dispatch(eidx, N, C)
        for t in range(T):
            rank = sum(1 for s in range(t) if eidx[s] == eidx[t])
            assert dp["rank"][t] == rank
            assert dp["slot"][t] == (rank if rank < C else -1)
        hist = np.bincount(eidx, minlength=N)
        assert np.array_equal(dp["hist"], hist)
        assert np.array_equal(dp["accepted"], np.minimum(hist, C))
        assert int(dp["offset"][-1]) + int(np.sum(dp["slot"] < 0)) == T
        for e in range(N):
            toks = dp["row2tok"][dp["offset"][e]:dp["offset"][e + 1]]
            assert np.all(eidx[toks] == e)
            assert np.array_equal(dp["slot"][toks], np.arange(len(toks)))
            assert np.all(np.diff(toks) > 0)


def pin_capacity_special_cases():
    x, Wr, W1, b1, W2, b2 = random_case(3, 40, 6, 7, 4, bias=True)
    r = O.forward(x, Wr, (W1, b1, W2, b2), CF=0.0)          # C = 0: all dropped
    assert r["C"] == 0 and np.all(r["slot"] == -1)
    assert np.array_equal(r["y64"], x)
    r = O.forward(x, Wr, (W1, b1, W2, b2), CF=4.0)          # CF = N: none dropped
    assert np.all(r["slot"] >= 0)
    r = O.forward(x, np.zeros_like(Wr), (W1, b1, W2, b2), CF=1.0)   # Wr = 0
    assert r["C"] == 10
    assert np.array_equal(r["slot"][:10], np.arange(10)) and np.all(r["slot"][10:] == -1)
    assert np.array_equal(r["y64"][10:], x[10:])


# ---------------------------------------------------------------------------
# Expert FFN, gate and combine.
# ---------------------------------------------------------------------------
def pin_ffn_hand_example():
    # One expert (gate 1), d = 2, F = 3, worked by hand:
    #   a = W1 x + b1 = (1*2 - 1*1 + 0.5, 0*2 + 2*1 - 3, -1*2 + 0*1 + 4) = (1.5, -1, 2)
    #   h = ReLU(a) = (1.5, 0, 2)
    #   o = W2 h + b2 = (1*1.5 + 5*0 - 1*2 + 0.25, 2*1.5 + 0*0 + 0.5*2 - 1) = (-0.25, 3)
    #   y = x + o = (1.75, 4)
    x = np.array([[2.0, 1.0]])
    W1 = np.array([[[1.0, -1.0], [0.0, 2.0], [-1.0, 0.0]]])
    b1 = np.array([[0.5, -3.0, 4.0]])
    W2 = np.array([[[1.0, 5.0, -1.0], [2.0, 0.0, 0.5]]])
    b2 = np.array([[0.25, -1.0]])
    r = O.forward(x, np.zeros((1, 2)), (W1, b1, W2, b2), CF=1.0)
    assert r["gate"][0] == 1.0 and r["expert_idx"][0] == 0
    assert np.array_equal(r["y64"], np.array([[1.75, 4.0]]))
    r = O.forward(x, np.zeros((1, 2)), (W1, b1, W2, b2), CF=1.0, no_residual=True)
    assert np.array_equal(r["y64"], np.array([[-0.25, 3.0]]))


def pin_dense_ffn_n1():
    # N = 1 and CF >= 1: every token goes to the one expert with gate exactly 1 and
    # the layer is x + FFN(x), the dense baseline of the paper note.
    x, Wr, W1, b1, W2, b2 = random_case(11, 9, 5, 7, 1, bias=True)
    r = O.forward(x, Wr, (W1, b1, W2, b2), CF=1.0)
    assert np.all(r["gate"] == 1.0) and np.all(r["slot"] == np.arange(9))
    for t in range(9):
        h = [max(0.0, math.fsum(W1[0, j, k] * x[t, k] for k in range(5)) + b1[0, j]) for j in range(7)]
        for i in range(5):
            o = math.fsum(W2[0, i, j] * h[j] for j in range(7)) + b2[0, i]
            assert abs(r["y64"][t, i] - (x[t, i] + o)) < 1e-12


def pin_x_zero_closed_form():
    # x = 0: all logits tie at 0, every token goes to expert 0 with gate 1/N and
    # the accepted ones get y = (W2_0 ReLU(b1_0) + b2_0) / N; the rest stay 0.
    N, T, d, F = 4, 16, 3, 5
    _, _, W1, b1, W2, b2 = random_case(5, T, d, F, N, bias=True)
    _, Wr, _, _, _, _ = random_case(6, T, d, F, N)
    r = O.forward(np.zeros((T, d)), Wr, (W1, b1, W2, b2), CF=1.0)
    C = r["C"]
    h = [max(0.0, b1[0, j]) for j in range(F)]
    o = [math.fsum(W2[0, i, j] * h[j] for j in range(F)) + b2[0, i] for i in range(d)]
    for t in range(T):
        want = [v / N for v in o] if t < C else [0.0] * d
        _close(r["y64"][t], want, 1e-14)


def pin_bruteforce_agreement():
    cases = [
        dict(seed=21, T=1, d=3, F=4, N=1, CF=1.0, bias=False),
        dict(seed=22, T=7, d=5, F=6, N=3, CF=1.0, bias=True),
        dict(seed=23, T=64, d=8, F=12, N=4, CF=1.0, bias=False),
        dict(seed=24, T=100, d=6, F=9, N=8, CF=0.5, bias=True),
        dict(seed=25, T=40, d=4, F=3, N=3, CF=1.25, bias=True),
        dict(seed=26, T=30, d=7, F=5, N=5, CF=2.0, bias=False),
        dict(seed=27, T=25, d=3, F=2, N=4, CF=4.0, bias=True),
        # larger layers: many route blocks, many experts with drops at CF = 1
        dict(seed=28, T=1200, d=16, F=24, N=40, CF=1.0, bias=True),
        dict(seed=29, T=1000, d=8, F=8, N=128, CF=1.0, bias=False),
    ]
    for c in cases:
        x, Wr, W1, b1, W2, b2 = random_case(c["seed"], c["T"], c["d"], c["F"], c["N"], c["bias"])
        for nr in (False, True):
            r = O.forward(x, Wr, (W1, b1, W2, b2), CF=c["CF"], no_residual=nr)
            b = brute_forward(_tolist(x), _tolist(Wr), _tolist(W1), _tolist(b1), _tolist(W2),
                              _tolist(b2), c["CF"], no_residual=nr)
            assert r["C"] == b["C"]
            assert list(r["expert_idx"]) == b["expert_idx"]
            assert list(r["slot"]) == b["slot"]
            _close(r["gate"], b["gate"], 1e-12)
            _close(r["probs"], b["probs"], 1e-12)
            assert abs(r["aux_loss"] - b["aux_loss"]) < 1e-12
            _close(r["y64"], b["y"], 1e-12)


def pin_ties_lowest_index():
    # Logit ties (exact in fp32) go to the lowest expert index.
    x = np.array([[1.0, 1.0, 0.0], [0.0, 2.0, 2.0], [3.0, 3.0, 3.0], [0.0, 0.0, 5.0]])
    r = O.forward(x, np.eye(3), _zero_ffn(3, 2, 3), CF=3.0)
    assert list(r["expert_idx"]) == [0, 1, 0, 2]


def pin_nan_logits_routing_order():
    # numpy's argmax order: a NaN logit counts as the largest, the first one wins;
    # the second choice is the same order over the other experts (a row of -inf
    # logits still gets a second expert distinct from the first).
    z = np.array([[1.0, np.nan, 3.0], [np.nan, np.nan, 0.0], [-np.inf, -np.inf, -np.inf],
                  [0.0, -np.inf, np.nan]])
    first = O.top1(z)
    assert list(first) == [1, 0, 0, 2], first
    assert list(O.second_choice(z, first)) == [2, 1, 1, 0]
    # A NaN row of x: all its logits are NaN, so it goes to expert 0 with a NaN gate,
    # the aux loss is NaN, and every other token routes and ranks as it would by itself.
    rng = np.random.default_rng(5)
    x = _f32(rng.standard_normal((6, 3)))
    x[2] = np.nan
    r = O.forward(x, np.eye(3), _zero_ffn(3, 2, 3), CF=3.0)
    assert r["expert_idx"][2] == 0 and np.isnan(r["gate"][2]) and math.isnan(r["aux_loss"])
    others = [0, 1, 3, 4, 5]
    assert list(r["expert_idx"][others]) == list(np.argmax(x[others], axis=1))
    assert np.all(np.isnan(r["y64"][2]))
    ranks = [sum(1 for s in range(t) if r["expert_idx"][s] == r["expert_idx"][t]) for t in range(6)]
    assert list(r["slot"]) == ranks


def pin_near_tie_rule():
    # The exemption set of the routing parity rule: largest minus second-largest logit
    # <= tol (1e-5), wherever the two maxima sit; hand-checked rows.
    z = np.array([
        [0.3, 0.3, -1.0, -2.0],              # exact tie                       -> exempt
        [1.0, 1.0 - 0.5e-5, 0.0, 0.5],       # gap 0.5e-5                      -> exempt
        [0.0, -1e-5, -2.0, -3.0],            # gap exactly 1e-5 (0 - (-1e-5))  -> exempt
        [2e-5, 0.0, -3.0, -4.0],             # gap 2e-5                        -> not
        [-5.0, 0.0, 3e-6, -1.0],             # maxima in columns 2 and 1       -> exempt
        [7.0, -2.0, 7.0 - 4e-5, 7.0 - 4e-5], # second and third tie, gap 4e-5  -> not
        [5.0, 5.0, 5.0, 0.0],                # three-way tie                   -> exempt
        [1.0, 4.0, 4.0 - 1e-6, 1.0],         # maxima in columns 1 and 2       -> exempt
        [-3.0, -3.0 - 1e-6, -7.0, -9.0],     # negative logits, gap 1e-6       -> exempt
        [5.0, 1.0, 1.0, 0.0],                # clear winner                    -> not
        [np.nan, 1.0, 1.0, 0.0],             # NaN: the choice is fixed, never exempt
    ])
    want = [True, True, True, False, True, False, True, True, True, False, False]
    assert list(O.near_tie_tokens(z, 1e-5)) == want
    assert not O.near_tie_tokens(np.array([[3.0], [3.0]]), 1e-5).any()   # one expert: no tie
    assert list(O.near_tie_tokens(np.array([[1.0, 1.0 + 2e-5]]), 3e-5)) == [True]


def pin_near_tie_second_rule():
    # Top-2 routing's extra exemption: second- minus third-largest logit <= tol.
    z = np.array([
        [5.0, 1.0, 1.0],                     # second and third tie            -> exempt
        [5.0, 1.0, 1.0 - 2e-5],              # gap 2e-5                        -> not
        [1.0, 1.0, 1.0],                     # three-way tie                   -> exempt
        [0.0, 0.0, -1e-5],                   # gap exactly 1e-5                -> exempt
        [3.0, 2.0 - 0.5e-5, 2.0],            # gap 0.5e-5, columns swapped     -> exempt
        [9.0, 9.0, 1.0],                     # top-1/top-2 tie only            -> not
    ])
    assert list(O.near_tie_second(z, 1e-5)) == [True, False, True, True, True, False]
    assert not O.near_tie_second(np.array([[1.0, 1.0]]), 1e-5).any()      # two experts


def pin_round_to_bf16():
    ulp = 2.0 ** -7
    vals = np.array([1.0, 1.0 + ulp / 2, 1.0 + 1.5 * ulp, 1.0 + 0.75 * ulp, -1.0 - ulp / 2,
                     3.0 + 0.3 * 2 * ulp, 0.0, 255.5, 256.5, 1.0 + 2.0 ** -30])
    want = np.array([1.0, 1.0, 1.0 + 2 * ulp, 1.0 + ulp, -1.0, 3.0, 0.0, 256.0, 256.0, 1.0])
    got = O.round_to_bf16(vals)
    assert np.array_equal(got, want), got


# ---------------------------------------------------------------------------
# Top-2 routing (the MoE baseline: y = x + sum over the two largest p of p E(x)).
# ---------------------------------------------------------------------------
def pin_top2_bruteforce_agreement():
    cases = [
        dict(seed=31, T=1, d=3, F=4, N=2, CF=1.0, bias=False),
        dict(seed=32, T=9, d=5, F=6, N=3, CF=1.0, bias=True),
        dict(seed=33, T=48, d=6, F=7, N=5, CF=0.5, bias=True),
        dict(seed=34, T=40, d=4, F=3, N=4, CF=1.25, bias=False),
        dict(seed=35, T=30, d=7, F=5, N=6, CF=3.0, bias=True),
    ]
    for c in cases:
        x, Wr, W1, b1, W2, b2 = random_case(c["seed"], c["T"], c["d"], c["F"], c["N"], c["bias"])
        for nr in (False, True):
            r = O.forward(x, Wr, (W1, b1, W2, b2), CF=c["CF"], no_residual=nr, k=2)
            b = brute_forward_top2(_tolist(x), _tolist(Wr), _tolist(W1), _tolist(b1), _tolist(W2),
                                   _tolist(b2), c["CF"], no_residual=nr)
            assert r["C"] == b["C"]
            assert r["expert_idx"].tolist() == b["expert_idx"]
            assert r["slot"].tolist() == b["slot"]
            _close(r["gate"], b["gate"], 1e-12)
            assert abs(r["aux_loss"] - b["aux_loss"]) < 1e-12
            _close(r["y64"], b["y"], 1e-12)


def pin_top2_two_experts_is_dense_mixture():
    # N = k = 2 and C >= T: every token visits both experts and the layer is the
    # soft mixture x + sum_i p_i E_i(x) (p = softmax of the logits), written here
    # with scipy's softmax and one plain matmul chain per expert.
    from scipy.special import softmax as sp_softmax
    x, Wr, W1, b1, W2, b2 = random_case(41, 25, 6, 8, 2, bias=True)
    r = O.forward(x, Wr, (W1, b1, W2, b2), CF=1.0, k=2)
    assert r["C"] == 25 and np.all(r["slot"] >= 0)
    p = sp_softmax(x @ Wr.T, axis=1)
    want = x.copy()
    for e in range(2):
        want += p[:, e:e + 1] * (np.maximum(x @ W1[e].T + b1[e], 0.0) @ W2[e].T + b2[e])
    _close(r["y64"], want, 1e-12)
    _close(np.sort(r["gate"], axis=1), np.sort(p, axis=1), 1e-12)


def pin_top2_router_zero_ties():
    # Wr = 0: all logits tie, so every token picks experts 0 then 1 with gates 1/N,
    # C = floor(CF 2T / N), and tokens 0..C-1 get x + (E_0(x) + E_1(x)) / N.
    N, T = 4, 20
    x, _, W1, b1, W2, b2 = random_case(43, T, 5, 6, N, bias=True)
    r = O.forward(x, np.zeros((N, 5)), (W1, b1, W2, b2), CF=1.0, k=2)
    C = r["C"]
    assert C == 10
    assert np.all(r["expert_idx"] == np.array([0, 1]))
    _close(r["gate"], np.full((T, 2), 1.0 / N), 1e-15)
    for t in range(T):
        want = x[t].copy()
        if t < C:
            for e in (0, 1):
                want += (np.maximum(W1[e] @ x[t] + b1[e], 0.0) @ W2[e].T + b2[e]) / N
            assert np.all(r["slot"][t] == t)
        else:
            assert np.all(r["slot"][t] == -1)
        _close(r["y64"][t], want, 1e-13)


def pin_top2_second_choice_ties():
    # Second choices with exact ties go to the lowest remaining index.
    x = np.array([[1.0, 1.0, 0.0], [0.0, 2.0, 2.0], [3.0, 3.0, 3.0], [0.0, 0.0, 5.0],
                  [4.0, 0.0, 4.0]])
    r = O.forward(x, np.eye(3), _zero_ffn(3, 2, 3), CF=3.0, k=2)
    assert r["expert_idx"].tolist() == [[0, 1], [1, 2], [0, 1], [2, 0], [0, 2]]


def pin_top2_capacity_and_aux():
    # Capacity counts k choices per token; aux keeps the top-1 share f_i, so it
    # equals the top-1 layer's on the same inputs; CF = 0 drops every choice.
    assert O.capacity(2 * 8192, 64, 1.25) == 320
    assert O.capacity(2 * 10, 4, 1.0) == 5
    x, Wr, W1, b1, W2, b2 = random_case(45, 36, 6, 5, 4, bias=True)
    r1 = O.forward(x, Wr, (W1, b1, W2, b2), CF=1.0)
    r2 = O.forward(x, Wr, (W1, b1, W2, b2), CF=1.0, k=2)
    assert r2["C"] == 2 * r1["C"] == 18
    assert abs(r1["aux_loss"] - r2["aux_loss"]) < 1e-15
    assert np.array_equal(r2["expert_idx"][:, 0], r1["expert_idx"])
    assert np.all(r2["expert_idx"][:, 0] != r2["expert_idx"][:, 1])
    acc = np.bincount(r2["expert_idx"][r2["slot"] >= 0], minlength=4)
    assert np.array_equal(acc, np.minimum(r2["hist"], 18))
    r0 = O.forward(x, Wr, (W1, b1, W2, b2), CF=0.0, k=2)
    assert np.all(r0["slot"] == -1) and np.array_equal(r0["y64"], x)


# ---------------------------------------------------------------------------
# No-Token-Left-Behind rerouting (overflow tokens to their second choice).
# ---------------------------------------------------------------------------
def pin_reroute_bruteforce_agreement():
    cases = [
        dict(seed=51, T=12, d=4, F=5, N=3, CF=0.5, bias=True),
        dict(seed=52, T=40, d=5, F=6, N=4, CF=1.0, bias=False),
        dict(seed=53, T=60, d=6, F=4, N=6, CF=0.75, bias=True),
        dict(seed=54, T=33, d=3, F=7, N=2, CF=0.6, bias=True),
    ]
    for c in cases:
        x, Wr, W1, b1, W2, b2 = random_case(c["seed"], c["T"], c["d"], c["F"], c["N"], c["bias"])
        for nr in (False, True):
            r = O.forward_reroute(x, Wr, (W1, b1, W2, b2), CF=c["CF"], no_residual=nr)
            b = brute_forward_reroute(_tolist(x), _tolist(Wr), _tolist(W1), _tolist(b1),
                                      _tolist(W2), _tolist(b2), c["CF"], no_residual=nr)
            assert r["C"] == b["C"]
            assert list(r["expert_idx"]) == b["expert_idx"]
            assert list(r["slot"]) == b["slot"]
            _close(r["gate"], b["gate"], 1e-12)
            assert abs(r["aux_loss"] - b["aux_loss"]) < 1e-12
            _close(r["y64"], b["y"], 1e-12)


def pin_reroute_without_overflow_is_top1():
    # CF = N: nothing overflows, so rerouting changes nothing.
    x, Wr, W1, b1, W2, b2 = random_case(55, 30, 5, 6, 4, bias=True)
    r0 = O.forward(x, Wr, (W1, b1, W2, b2), CF=4.0)
    r1 = O.forward_reroute(x, Wr, (W1, b1, W2, b2), CF=4.0)
    assert np.array_equal(r0["slot"], r1["slot"]) and np.array_equal(r0["expert_idx"], r1["expert_idx"])
    assert np.array_equal(r0["y64"], r1["y64"]) and r0["aux_loss"] == r1["aux_loss"]


def pin_reroute_router_zero():
    # Wr = 0: every token picks expert 0 then expert 1 (ties), gate 1/N.  Tokens 0..C-1
    # stay with expert 0, tokens C..2C-1 are rerouted into expert 1's empty buffer at
    # positions 0..C-1, the rest pass through.
    N, T = 4, 20
    x, _, W1, b1, W2, b2 = random_case(57, T, 5, 6, N, bias=True)
    r = O.forward_reroute(x, np.zeros((N, 5)), (W1, b1, W2, b2), CF=1.0)
    C = r["C"]
    assert C == 5
    for t in range(T):
        e, want_slot = (0, t) if t < C else ((1, t - C) if t < 2 * C else (0, -1))
        assert r["expert_idx"][t] == e and r["slot"][t] == want_slot, (t, r["expert_idx"][t], r["slot"][t])
        want = x[t].copy()
        if want_slot >= 0:
            want += (np.maximum(W1[e] @ x[t] + b1[e], 0.0) @ W2[e].T + b2[e]) / N
        _close(r["y64"][t], want, 1e-13)
    assert np.array_equal(r["accepted"], [5, 5, 0, 0])


def pin_reroute_fills_after_first_stage():
    # Experts 0 and 1, C = 3.  Logits put tokens 0-4 first on expert 0 (second 1) and
    # tokens 5-6 first on expert 1 (second 0): expert 0 takes 0, 1, 2 and refuses 3, 4;
    # expert 1 takes 5, 6 in stage 1 and has one position left, which goes to token 3
    # (the earlier of the two overflowed tokens); token 4 passes through.
    x = np.array([[2.0, 1.0]] * 5 + [[1.0, 2.0]] * 2)
    r = O.forward_reroute(x, np.eye(2), _zero_ffn(2, 3, 2), CF=1.0)
    assert r["C"] == 3
    assert list(r["expert_idx"]) == [0, 0, 0, 1, 0, 1, 1]
    assert list(r["slot"]) == [0, 1, 2, 2, -1, 0, 1]
    assert np.array_equal(r["accepted"], [3, 3])
    p = np.exp(1.0) / (np.exp(1.0) + np.exp(2.0))   # token 3's gate on its second choice
    assert abs(r["gate"][3] - p) < 1e-15


# ---------------------------------------------------------------------------
# GEGLU experts.
# ---------------------------------------------------------------------------
# Standard normal CDF values from the printed tables: Phi(1), Phi(2), Phi(3).
PHI_1, PHI_2, PHI_3 = 0.8413447460685429, 0.9772498680518208, 0.9986501019683699


def pin_gelu_closed_forms():
    a = np.array([0.0, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0, 12.0, -12.0])
    want = np.array([0.0, PHI_1, -(1 - PHI_1), 2 * PHI_2, -2 * (1 - PHI_2), 3 * PHI_3,
                     -3 * (1 - PHI_3), 12.0, 0.0])
    got = O.gelu(a)
    assert np.all(np.abs(got - want) <= 1e-15 * np.maximum(1.0, np.abs(want)) + 1e-30), got - want
    # GELU(a) - GELU(-a) = a (Phi(a) + Phi(-a) = 1), at any a
    b = np.linspace(-7, 7, 57)
    assert np.max(np.abs(O.gelu(b) - O.gelu(-b) - b)) < 1e-14


def pin_geglu_expert_hand_example():
    # d = 2, F = 1: W = [1, 0], V = [0, 1], b_W = 0, b_V = 0.5, W2 = [[2], [-1]], b2 = 0.
    # x = (1, 1.5): GELU(1) * (1.5 + 0.5) = 2 Phi(1); o = (4 Phi(1), -2 Phi(1)).
    W1e = np.array([[1.0, 0.0], [0.0, 1.0]])
    b1e = np.array([0.0, 0.5])
    W2e = np.array([[2.0], [-1.0]])
    o = O.expert_ffn(np.array([[1.0, 1.5]]), W1e, b1e, W2e, None, "geglu")
    _close(o, [[4 * PHI_1, -2 * PHI_1]], 1e-15)


def pin_geglu_bruteforce_agreement():
    for seed, T, d, F, N, CF, bias in ((61, 20, 4, 3, 3, 1.0, True), (62, 33, 6, 5, 2, 0.7, False),
                                       (63, 48, 5, 8, 4, 1.5, True)):
        x, Wr, W1, b1, _, _ = random_case(seed, T, d, 2 * F, N, bias)
        rng = np.random.default_rng(seed + 100)
        W2 = rng.normal(0, 0.5, (N, d, F))
        b2 = rng.normal(0, 0.1, (N, d)) if bias else None
        for nr in (False, True):
            r = O.forward(x, Wr, (W1, b1, W2, b2), CF=CF, no_residual=nr, activation="geglu")
            b = brute_forward(_tolist(x), _tolist(Wr), _tolist(W1), _tolist(b1), _tolist(W2),
                              _tolist(b2), CF, no_residual=nr, activation="geglu")
            assert list(r["slot"]) == b["slot"]
            _close(r["y64"], b["y"], 1e-12)


def pin_geglu_linear_branch_identity():
    # V = 0 and b_V = 1: h = GELU(W x + b_W), so E(x) matches a one-expert GELU FFN
    # evaluated through the Phi table at pre-activations 1, -1, 2 (x = e_i, W = diag).
    W1e = np.vstack([np.diag([1.0, -1.0, 2.0]), np.zeros((3, 3))])
    b1e = np.concatenate([np.zeros(3), np.ones(3)])
    o = O.expert_ffn(np.eye(3), W1e, b1e, np.eye(3), None, "geglu")
    _close(np.diag(o), [PHI_1, -(1 - PHI_1), 2 * PHI_2], 1e-15)
    assert np.all(o[~np.eye(3, dtype=bool)] == 0.0)


# ---------------------------------------------------------------------------
# Backward pass.
# ---------------------------------------------------------------------------
def _fd_check(x, Wr, experts, CF, dy, d_aux, entries=5, eps=1e-6, tol=2e-8, seed=0):
    """Central differences of L = sum(y * dy) + d_aux * aux, through forward(), at
    sampled entries of every input; the routing must not move within +-eps."""
    g = O.backward(x, Wr, experts, CF, dy, d_aux)
    W1, b1, W2, b2 = experts
    base = O.forward(x, Wr, experts, CF)
    arrays = {"dx": x, "dWr": Wr, "dW1": W1, "db1": b1, "dW2": W2, "db2": b2}
    rng = np.random.default_rng(seed)

    def loss():
        r = O.forward(x, Wr, experts, CF)
        assert np.array_equal(r["slot"], base["slot"]) and \
            np.array_equal(r["expert_idx"], base["expert_idx"]), "routing moved"
        return float(np.sum(r["y64"] * dy) + d_aux * r["aux_loss"])

    for key, arr in arrays.items():
        if arr is None:
            continue
        for _ in range(entries):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss()
            arr[idx] = old - eps
            lm = loss()
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[key][idx]) <= tol * max(1.0, abs(fd)), (key, idx, fd, g[key][idx])
    return g


def pin_backward_finite_differences():
    cases = [dict(seed=71, T=24, d=5, F=6, N=3, CF=0.8, bias=True, d_aux=0.7),   # drops
             dict(seed=72, T=16, d=4, F=3, N=4, CF=2.0, bias=False, d_aux=0.0),
             dict(seed=73, T=30, d=6, F=5, N=2, CF=1.0, bias=True, d_aux=-1.3),
             dict(seed=74, T=12, d=3, F=4, N=1, CF=1.0, bias=True, d_aux=2.0)]   # dense
    for c in cases:
        x, Wr, W1, b1, W2, b2 = random_case(c["seed"], c["T"], c["d"], c["F"], c["N"], c["bias"])
        x, Wr, W1, W2 = (np.array(a, np.float64) for a in (x, Wr, W1, W2))
        b1 = None if b1 is None else np.array(b1, np.float64)
        b2 = None if b2 is None else np.array(b2, np.float64)
        dy = np.random.default_rng(c["seed"] + 1).standard_normal((c["T"], c["d"]))
        g = _fd_check(x, Wr, (W1, b1, W2, b2), c["CF"], dy, c["d_aux"], seed=c["seed"])
        if c["N"] == 1:
            assert np.all(g["dz"] == 0.0) and np.all(g["dWr"] == 0.0)


def pin_backward_aux_only_router_zero():
    # Wr = 0, dy = 0, d_aux = 1: every token picks expert 0 (ties), f = (1, 0, ..), p = 1/N,
    # so dz_{t,0} = (N-1)/(N T), dz_{t,j} = -1/(N T) for j > 0; dWr_j = dz_j * sum_t x_t;
    # dx = Wr^T dz = 0 and every expert gradient is 0.
    N, T, d = 4, 10, 3
    x, _, W1, b1, W2, b2 = random_case(75, T, d, 5, N, bias=True)
    g = O.backward(x, np.zeros((N, d)), (W1, b1, W2, b2), 4.0, np.zeros((T, d)), 1.0)
    sx = np.asarray(x, np.float64).sum(axis=0)
    want = np.vstack([(N - 1) / (N * T) * sx] + [-1.0 / (N * T) * sx] * (N - 1))
    _close(g["dWr"], want, 1e-15)
    assert np.all(g["dx"] == 0.0)
    for k in ("dW1", "db1", "dW2", "db2"):
        assert np.all(g[k] == 0.0), k


def pin_backward_dropped_token_passes_gradient():
    # CF = 0: every token is dropped, y = x, so dx = dy + Wr^T dz with dz from the aux
    # term alone, and the expert gradients vanish.
    x, Wr, W1, b1, W2, b2 = random_case(76, 14, 4, 5, 3, bias=True)
    dy = np.random.default_rng(9).standard_normal((14, 4))
    g = O.backward(x, Wr, (W1, b1, W2, b2), 0.0, dy, 0.0)
    _close(g["dx"], dy, 0.0)
    assert np.all(g["dWr"] == 0.0)
    g = O.backward(x, Wr, (W1, b1, W2, b2), 0.0, dy, 1.0)
    r = O.forward(x, Wr, (W1, b1, W2, b2), 0.0)
    f = np.bincount(r["expert_idx"], minlength=3) / 14
    p = r["probs"]
    c = 3 * f / 14
    dz = p * (c - (p @ c)[:, None])
    _close(g["dx"], dy + dz @ np.asarray(Wr, np.float64), 1e-14)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
