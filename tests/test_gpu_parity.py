"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle on the same
seeded inputs.  Routing, slots and the drop mask bit-exact outside near-ties of the
top-2 logits (gap <= 1e-5), gate within 1e-6, aux within 1e-5, y within rel-L2 2e-2
(bf16 experts) or 1e-5 (fp32), dropped rows bit-exact."""
import numpy as np
import pytest

import oracle
import switchffn_synth as synth
from gpu_harness import (announce, check_routing, check_y, host_x, oracle_ref, rows_of, run_gpu,
                         sample_experts)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _full_case(w, mutate=None, no_residual_too=True):
    """Small shapes: the oracle computes every row."""
    announce(w.describe())
    dev_in = synth.device_inputs(w, DEV)
    x_raw = host_x(w)
    Wr_raw = synth.host_array(w, "Wr").reshape(w.N, w.d)
    if mutate is not None:
        x_raw, Wr_raw = mutate(dev_in, x_raw, Wr_raw)
    gpu = run_gpu(w, dev_in)
    ref = oracle_ref(w, x_raw, Wr_raw, gpu["expert_idx"])
    ties = check_routing(gpu, ref)
    err = check_y(w, gpu, ref, x_raw)
    out = {"ties": ties, "y_err": err, "dropped": int(np.sum(ref["slot"] < 0)), "ref": ref}
    if no_residual_too:
        from sparse_mixture_experts_switchffn_amd import SFFN_NO_RESIDUAL
        gnr = run_gpu(w, dev_in, flags=SFFN_NO_RESIDUAL)
        assert np.array_equal(gnr["slot"], gpu["slot"])
        rnr = oracle_ref(w, x_raw, Wr_raw, gnr["expert_idx"], no_residual=True)
        out["y_err_nr"] = check_y(w, gnr, rnr, x_raw, no_residual=True)
    print(f"  ties={ties} dropped={out['dropped']} y_err={err:.2e} "
          f"y_err_nr={out.get('y_err_nr', float('nan')):.2e}", flush=True)
    return out


def test_device_filler_matches_host_filler():
    import torch
    w = synth.workload("switch_base").replace(T=512, N=4, bias_sigma=0.02)
    announce("device filler vs host filler " + w.describe())
    dev_in = synth.device_inputs(w, DEV)
    for name in ("x", "W1", "b1", "W2", "b2"):
        t = dev_in[name]
        got = t.view(torch.int16).cpu().numpy().view(np.uint16).ravel()
        assert np.array_equal(got, synth.host_array(w, name)), name
    wf = w.replace(dtype="fp32")
    t = synth.device_inputs(wf, DEV)["W2"]
    assert np.array_equal(t.cpu().numpy().ravel(), synth.host_array(wf, "W2"))


def test_tiny_fp32():
    r = _full_case(synth.workload("tiny"))
    assert r["y_err"] <= 1e-6


@pytest.mark.parametrize("case", [
    dict(T=300, d=72, F=136, N=6, CF=1.0, bias_sigma=0.02),      # ragged T, K tail, column tail
    dict(T=257, d=64, F=128, N=1, CF=1.0, bias_sigma=0.02),      # one expert: dense FFN, gate 1
    dict(T=200, d=32, F=64, N=5, CF=0.0),                        # C = 0: every token dropped
    dict(T=199, d=40, F=48, N=3, CF=3.0, bias_sigma=0.02),       # CF = N: nothing dropped
    dict(T=1, d=16, F=24, N=3, CF=1.0),                          # a single token (C = 0)
    dict(T=2, d=16, F=24, N=2, CF=2.0, bias_sigma=0.02),         # two tokens, C = 2
    dict(T=2048, d=64, F=96, N=4, CF=1.0),                       # C = 512: two row chunks
    dict(T=1000, d=128, F=256, N=130, CF=1.5),                   # N > 128, N % 4 != 0: scalar path
    dict(T=1100, d=200, F=64, N=260, CF=2.0, bias_sigma=0.02),   # tiled logits: partial group, k tail
    dict(T=530, d=2080, F=32, N=132, CF=4.0),                    # tiled logits: odd step count, ragged T
    dict(T=300, d=72, F=16, N=4096, CF=16.0),                    # the most experts: widest softmax
    dict(T=33000, d=64, F=32, N=128, CF=1.0, bias_sigma=0.02),   # tiled logits, 128-token blocks, ragged T
    dict(T=33000, d=40, F=16, N=68, CF=1.0),                     # tiled logits, partial expert group
    dict(T=700, d=2080, F=64, N=7, CF=1.0),                      # d = 2080 (32 x 65) K tail
    dict(T=300, d=32, F=64, N=4, CF=1.0, bias_sigma=0.02),       # d = 32: half a k-step
    dict(T=500, d=96, F=128, N=6, CF=1.25, bias_sigma=0.02),     # d = 96: rows off the line grid
    dict(T=640, d=256, F=512, N=16, CF=0.5, bias_sigma=0.05),    # heavy dropping
])
def test_bf16_edge_shapes(case):
    w = synth.workload("switch_base").replace(**case)
    _full_case(w)


@pytest.mark.parametrize("case", [
    dict(T=1200, d=128, F=192, N=4, CF=1.0, bias_sigma=0.02),    # C = 300: both GEMMs in two row parts
    dict(T=1100, d=64, F=136, N=4, CF=1.0),                      # C = 275: FFN1 split, column tail
    dict(T=1290, d=64, F=128, N=4, CF=1.0, bias_sigma=0.02),     # C = 322: 11 row tiles, two chunks
    dict(T=1030, d=192, F=64, N=4, CF=1.0),                      # C = 257: 9 row tiles, one row
])
def test_tall_expert_tiles(case):
    """Experts of 257..320 rows at small sizes: two row chunks (too few tiles to split)."""
    w = synth.workload("switch_base").replace(**case)
    _full_case(w)


@pytest.mark.parametrize("case", [
    dict(T=2000, d=96, F=256, N=64, CF=1.0, bias_sigma=0.02),    # C = 31: one row tile, K tail of half a step
    dict(T=3000, d=160, F=128, N=48, CF=1.0),                    # C = 62: two row tiles, three k-steps
    dict(T=1500, d=2080, F=256, N=40, CF=1.0, bias_sigma=0.02),  # the many-expert row length, C = 37
    dict(T=1000, d=32, F=128, N=32, CF=1.0),                     # K = 32: half a k-step
])
def test_rows_off_the_line_grid(case):
    """Token rows of x and weight rows that start mid-line (2d % 128 == 64) in tiles of one
    or two row tiles, the many-expert layer's tile shape."""
    _full_case(synth.workload("switch_base").replace(**case))


@pytest.mark.parametrize("case", [
    dict(T=8192, d=64, F=64, N=64, CF=1.0, bias_sigma=0.02),     # 256 blocks: the folded scan's limit
    dict(T=8193, d=64, F=64, N=64, CF=1.0, bias_sigma=0.02),     # 257 blocks: the separate scan
    dict(T=4000, d=64, F=64, N=128, CF=1.0),                     # 128 experts folded, router planes
    dict(T=700, d=64, F=64, N=60, CF=1.0, bias_sigma=0.02),      # 15 chunks a row: idle threads
    dict(T=3000, d=96, F=64, N=100, CF=1.0),                     # four partial expert tiles
])
def test_scan_fold_boundaries(case):
    """Top-1 dispatch with the column scan in the scatter (the count table small enough)
    and without it, and the fused router with and without the planes pass."""
    _full_case(synth.workload("switch_base").replace(**case), no_residual_too=False)


def test_rows_off_the_line_grid_offset_x():
    """The same with x starting 64 bytes past a line (a view one row into a larger
    buffer), so that the even tokens are the ones that start mid-line."""
    import torch
    w = synth.workload("switch_base").replace(T=2000, d=96, F=256, N=64, CF=1.0, bias_sigma=0.02)

    def offset_x(dev_in, x_raw, Wr_raw):
        x = dev_in["x"]
        big = torch.zeros((w.T + 1, w.d), dtype=x.dtype, device=x.device)
        big[1:] = x
        dev_in["x"] = big[1:]
        assert dev_in["x"].data_ptr() % 128 == 64
        return x_raw, Wr_raw

    _full_case(w, mutate=offset_x)


@pytest.mark.parametrize("case", [
    dict(T=76800, d=64, F=512, N=256, CF=1.0, bias_sigma=0.02),   # FFN1 split: 1024 tiles
    dict(T=76790, d=512, F=64, N=256, CF=1.0),                    # FFN2 split, ragged T
])
def test_split_row_tiles(case):
    """C = 300 with enough column tiles (four rounds of the grid) for the split-row GEMM:
    one tile of two row parts sharing each weight step, every weight byte read once."""
    w = synth.workload("switch_base").replace(**case)
    _full_case(w, no_residual_too=False)


def test_split_row_tiles_top2():
    """Top-2 routing with C = floor(1.0 * 2T / N) = 300: the split-row tiles with the
    row-output FFN2 epilogue and the combine."""
    w = synth.workload("switch_base").replace(T=600, d=128, F=192, N=4, CF=1.0, bias_sigma=0.02)
    announce("split rows, top-2 " + w.describe())
    dev_in = synth.device_inputs(w, DEV)
    x_raw = host_x(w)
    Wr_raw = synth.host_array(w, "Wr").reshape(w.N, w.d)
    gpu = run_gpu(w, dev_in, k=2)
    ref = oracle_ref(w, x_raw, Wr_raw, gpu["expert_idx"], k=2)
    check_routing(gpu, ref)
    check_y(w, gpu, ref, x_raw)


@pytest.mark.parametrize("case", [
    dict(T=100, d=5, F=7, N=3, CF=1.0, bias_sigma=0.1),
    dict(T=333, d=33, F=65, N=9, CF=1.25, bias_sigma=0.02),
    dict(T=64, d=32, F=64, N=4, CF=0.0),
])
def test_fp32_edge_shapes(case):
    w = synth.workload("tiny").replace(**case)
    r = _full_case(w)
    assert r["y_err"] <= 1e-5


def test_router_zero_all_ties():
    """Wr = 0: every logit ties at 0, all tokens go to expert 0 with gate 1/N and only the
    first C tokens are accepted."""
    import torch
    w = synth.workload("switch_base").replace(T=320, d=64, F=128, N=8, CF=2.0, bias_sigma=0.02)

    def mutate(dev_in, x_raw, Wr_raw):
        dev_in["Wr"].zero_()
        torch.cuda.synchronize()
        return x_raw, np.zeros_like(Wr_raw)

    r = _full_case(w, mutate)
    ref = r["ref"]
    assert np.all(ref["expert_idx"] == 0)
    C = ref["C"]
    assert np.array_equal(ref["slot"][:C], np.arange(C)) and np.all(ref["slot"][C:] == -1)


def test_zero_tokens_closed_form():
    """x = 0: all tokens tie into expert 0; accepted rows are (W2_0 ReLU(b1_0) + b2_0) / N."""
    import torch
    w = synth.workload("switch_base").replace(T=256, d=64, F=128, N=4, CF=1.0, bias_sigma=0.05)

    def mutate(dev_in, x_raw, Wr_raw):
        dev_in["x"].zero_()
        torch.cuda.synchronize()
        return np.zeros_like(x_raw), Wr_raw

    _full_case(w, mutate)


@pytest.mark.parametrize("name", ["switch_base", "skewed", "switch_large", "many_expert"])
def test_measured_workloads(name):
    """The full-size workloads, in the launch configuration the benchmark times: routing,
    slots, gate, aux and the drop mask for every token; y for every dropped row (bit-exact)
    and for all accepted rows of sampled experts."""
    import torch
    w = synth.workload(name)
    announce(w.describe())
    dev_in = synth.device_inputs(w, DEV)
    gpu = run_gpu(w, dev_in)
    x_raw = host_x(w)
    Wr_raw = synth.host_array(w, "Wr").reshape(w.N, w.d)
    C = oracle.capacity(w.T, w.N, w.CF)
    experts = sample_experts(oracle.dispatch(gpu["expert_idx"], w.N, C), 8)
    ref = oracle_ref(w, x_raw, Wr_raw, gpu["expert_idx"], only_experts=experts)
    ties = check_routing(gpu, ref)
    rows = rows_of(ref, experts)
    err = check_y(w, gpu, ref, x_raw, rows=rows)
    from sparse_mixture_experts_switchffn_amd import SFFN_NO_RESIDUAL
    gnr = run_gpu(w, dev_in, flags=SFFN_NO_RESIDUAL)
    rnr = oracle_ref(w, x_raw, Wr_raw, gnr["expert_idx"], only_experts=experts, no_residual=True)
    err_nr = check_y(w, gnr, rnr, x_raw, rows=rows, no_residual=True)
    hist = ref["hist"]
    print(f"  ties={ties} dropped={int(np.sum(ref['slot'] < 0))} accepted={int(ref['offset'][-1])}"
          f" hist[min,max]=({hist.min()},{hist.max()}) aux={gpu['aux_loss']:.6f}"
          f" y_err={err:.2e} y_err_nr={err_nr:.2e} experts={experts}", flush=True)
    del dev_in
    torch.cuda.empty_cache()


def test_deterministic():
    w = synth.workload("switch_base")
    announce("determinism " + w.describe())
    dev_in = synth.device_inputs(w, DEV)
    a = run_gpu(w, dev_in)
    b = run_gpu(w, dev_in)
    for k in ("expert_idx", "slot", "gate", "y_bits"):
        assert np.array_equal(a[k], b[k]), k
    assert a["aux_loss"] == b["aux_loss"]


@pytest.mark.parametrize("case,k,reroute", [
    (dict(T=300, d=72, F=64, N=6, CF=1.0), 1, False),             # fused router, top-1
    (dict(T=300, d=72, F=64, N=6, CF=1.0), 2, False),             # fused router, top-2 mode
    (dict(T=300, d=72, F=64, N=6, CF=0.6, zipf_s=1.1), 1, True),  # fused router, rerouting mode
    (dict(T=1100, d=200, F=64, N=260, CF=2.0), 1, False),         # tiled logits
    (dict(T=1000, d=128, F=64, N=130, CF=1.5), 1, False),         # N % 4 != 0: scalar logits
    (dict(T=333, d=33, F=65, N=9, CF=1.25, dtype="fp32"), 1, False),  # fp32 layer
])
def test_stored_router_logits(case, k, reroute):
    """Every router path leaves z = Wr x (fp32) at the start of the forward workspace, where
    the backward pass reads it.  Bound: an fp32 sum of n exact products, in any order, is
    within about n * 2^-24 * sum |products| of the exact sum.  The bf16 paths add 3d
    products (bf16 x times the exact bf16 planes hi, mid, lo of Wr, each exact in fp32), the
    fp32 path d fused multiply-adds; 3d * 2^-24 * 1.01 * sum_k |x_k Wr_ik| covers both."""
    import torch

    import sparse_mixture_experts_switchffn_amd as sffn
    w = synth.workload("switch_base").replace(**case)
    announce(f"stored logits k={k} reroute={reroute} " + w.describe())
    dev_in = synth.device_inputs(w, DEV)
    flags = sffn.SFFN_REROUTE_OVERFLOW if reroute else 0
    out = sffn.switch_ffn_forward(dev_in["x"], dev_in["Wr"], dev_in["W1"], dev_in["b1"],
                                  dev_in["W2"], dev_in["b2"], w.CF, flags=flags, k=k)
    torch.cuda.synchronize()
    # the header: a 16-word layout tag in the first 256 bytes, the logits from byte 256
    tag = out["workspace"][:64].view(torch.int32).cpu().numpy().view(np.uint32)
    C = sffn.switch_ffn_capacity(k * w.T, w.N, w.CF)
    want = [0x4E464653, 1, k, flags, w.T, w.d, w.F, w.N, min(C, w.T),
            sffn.SFFN_BF16 if w.dtype == "bf16" else sffn.SFFN_FP32] + [0] * 6
    assert list(tag) == want, list(tag)
    z = out["workspace"][256: 256 + w.T * w.N * 4].view(torch.float32).cpu().numpy().reshape(
        w.T, w.N)
    x64 = synth.decode(host_x(w))
    Wr64 = synth.decode(synth.host_array(w, "Wr").reshape(w.N, w.d))
    ref = oracle.router_logits(x64, Wr64)
    bound = 3 * w.d * 2.0 ** -24 * 1.01 * (np.abs(x64) @ np.abs(Wr64).T)
    err = np.abs(z.astype(np.float64) - ref)
    assert np.all(err <= bound), f"max excess {np.max(err - bound):.3e}"
    print(f"  max |z - z64| = {err.max():.2e} (bound {bound.max():.2e})", flush=True)
