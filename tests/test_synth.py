"""The seeded input generator (host side; the device filler is checked in the GPU tests)."""
import numpy as np
import pytest

import switchffn_synth as S
from switchffn_synth.generate import BF16_ONE, shape_of


def test_slices_match_full_draw():
    w = S.workload("tiny")
    full = S.host_array(w, "W1")
    assert full.shape == (w.N * w.F * w.d,)
    for start, count in ((0, 5), (17, 100), (w.F * w.d, w.F * w.d)):
        assert np.array_equal(S.host_array(w, "W1", start, count), full[start:start + count])
    ew = S.expert_weights_host(w, 2)
    assert np.array_equal(ew["W1"].ravel(), full[2 * w.F * w.d:3 * w.F * w.d])


def test_deterministic_and_seeded():
    w = S.workload("tiny")
    a = S.host_array(w, "x")
    assert np.array_equal(a, S.host_array(w, "x"))
    assert not np.array_equal(a, S.host_array(w.replace(seed=1), "x"))
    wr = S.host_array(w, "Wr")
    assert not np.array_equal(a[: wr.size], wr)          # streams differ


@pytest.mark.parametrize("name,sigma", [("x", 1.0), ("W1", 0.02)])
def test_moments(name, sigma):
    w = S.workload("switch_base")
    v = S.decode(S.host_array(w, name, 0, 1 << 20))
    assert abs(v.mean()) < 5e-3 * sigma
    assert abs(v.std() / sigma - 1.0) < 5e-3
    assert np.max(np.abs(v)) <= 6.0 * sigma * 1.01          # Irwin-Hall(12) support
    kurt = np.mean((v - v.mean()) ** 4) / v.var() ** 2
    assert abs(kurt - 2.9) < 0.05                            # 3 - 6/5/12 = 2.9


def test_bf16_bits_are_round_to_nearest_even():
    w = S.workload("switch_base")
    bits = S.host_array(w, "x", 0, 4096)
    wf = w.replace(dtype="fp32")
    f32 = S.host_array(wf, "x", 0, 4096)
    # nearest bf16 of each fp32 value, ties to even, by exhaustive neighbour check
    lo = (f32.view(np.uint32) >> 16).astype(np.uint32)
    cand = np.stack([lo, lo + 1])
    vals = (cand << 16).view(np.float32).astype(np.float64)
    err = np.abs(vals - f32.astype(np.float64))
    pick = np.where(err[0] < err[1], cand[0], np.where(err[1] < err[0], cand[1],
                    np.where(cand[0] % 2 == 0, cand[0], cand[1])))
    assert np.array_equal(bits.astype(np.uint32), pick)


def test_skew_bias_columns():
    w = S.workload("skewed").replace(T=64)
    x = S.host_array(w, "x").reshape(shape_of(w, "x"))
    assert np.all(x[:, -1] == BF16_ONE)
    Wr = S.host_array(w, "Wr").reshape(shape_of(w, "Wr"))
    bias = S.zipf_router_bias(w)
    assert np.array_equal(Wr[:, -1], bias)
    assert np.all(np.diff(bias) < 0)                         # popularity falls with index
    pi = np.exp(bias.astype(np.float64) / (w.zipf_beta * w.w_sigma * np.sqrt(w.d - 1)))
    assert abs(pi.sum() - 1.0) < 1e-5
    assert abs(pi[0] / pi[1] - 2.0 ** 1.1) < 1e-4


def test_rows_helper():
    w = S.workload("tiny")
    x = S.host_array(w, "x").reshape(w.T, w.d)
    rows = np.array([3, 0, 63])
    assert np.array_equal(S.host_rows(w, "x", rows), x[rows])
