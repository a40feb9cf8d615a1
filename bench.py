#!/usr/bin/env python3
"""SwitchFFN forward benchmark on one MI355X.

One step = one switch_ffn_forward call over one batch of the workload (router,
softmax/top-1, dispatch, both expert GEMMs with the combine, aux loss), with
inputs already resident in HBM.  Prints ONE JSON line:
  value       tokens/s over the K timed steps (HIP events around the timed region);
              the steps are replayed from a HIP graph of --graph forward calls
              (default 10; the remainder launched eagerly), used only when a replay
              reproduces the eager output bit for bit -- `launch` reports the eager
              rate of the same K steps as well
  roofline    the dominant kernel's algorithmic HBM bytes per launch / its average
              duration (per-stage HIP events recorded on the launch stream inside
              the timed region) against the 8 TB/s HBM peak; `traffic` is the HBM
              byte count rocprofv3 measured for that kernel (profiles/), or null
              when the kernel source changed since it was measured
  cpu_baseline the CPU oracle (float64 numpy) timed on this host on a bounded
              sample of the same workload
              (many_expert: the bounded sample described in cpu_baseline_extrapolated),
              with the host's CPUs and one-thread rates of Tiny and Switch-Base-like
  roofline.layer  the whole layer's minimum HBM bytes (the weights of experts with
              accepted tokens, Wr, x read once, y written once) / ms_per_step
Default workload: the many-expert Switch-C-shaped layer, the largest configuration
that fits one GPU (T=65536 tokens, d_model 2080, d_ff 6144, 2048 experts, CF 1.0,
105 GB of bf16 expert weights, fp32 router).  --config picks another (tiny,
switch_base, skewed, switch_large).  Variants of the step: --topk 2 (top-2 routing),
--reroute (No-Token-Left-Behind), --geglu (GEGLU experts), --backward (a training
step: forward then backward; metric "SwitchFFN fwd+bwd tokens/s").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KERNEL_SOURCES = {"ffn1": ("ffn.hip", "sffn_device.h"), "ffn2": ("ffn.hip", "sffn_device.h"),
                  "router_logits": ("router.hip", "sffn_device.h"),
                  "softmax_route": ("router.hip", "sffn_device.h"),
                  "dispatch_scan": ("dispatch.hip", "sffn_device.h"),
                  "dispatch_scatter": ("dispatch.hip", "sffn_device.h")}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="many_expert",
                   help="workload: tiny, switch_base, skewed, switch_large, many_expert")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU work budget of the oracle baseline (0 = skip)")
    p.add_argument("--graph", type=int, default=10,
                   help="forward calls per captured HIP graph in the timed region (0 = eager launches)")
    p.add_argument("--quiet", action="store_true", help="only the JSON line on stdout")
    p.add_argument("--topk", type=int, default=1, choices=(1, 2),
                   help="experts per token: 1 (Switch routing, the headline) or 2 (top-2)")
    p.add_argument("--reroute", action="store_true",
                   help="top-1 routing with No-Token-Left-Behind rerouting of overflowed tokens "
                        "to their second choice")
    p.add_argument("--backward", action="store_true",
                   help="a training step of the layer: forward then backward (dy ~ N(0, 1), "
                        "d_aux = 0.01), top-1 ReLU experts")
    p.add_argument("--geglu", action="store_true",
                   help="GEGLU experts (two up-projections, W1 [N, 2F, d])")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain device copy of 1 GiB three times (calibrates the "
                        "rocprofv3 FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


def measured_peaks(dev):
    """This GPU's own reference points, beside the published peaks: a plain device copy
    (read + write bytes per second) and a large bf16 GEMM through torch (hipBLASLt)."""
    import torch
    out = {"hbm_spec_GBps": HBM_PEAK_GBS, "bf16_mfma_spec_TFLOPs": MFMA_BF16_PEAK_TFLOPS}
    try:
        n = 1 << 29  # 1 GiB of bf16
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize(dev)
        out["copy_GBps"] = 5 * 2 * n * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst
        m = 8192
        a = torch.randn(m, m, device=dev).to(torch.bfloat16)
        b = torch.randn(m, m, device=dev).to(torch.bfloat16)
        c = a @ b
        e0.record()
        for _ in range(5):
            c = a @ b
        e1.record()
        torch.cuda.synchronize(dev)
        out["bf16_gemm_8192_TFLOPs"] = 5 * 2.0 * m ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12
        del a, b, c
        torch.cuda.empty_cache()
    except Exception as exc:  # a reference only; never fails the benchmark
        out["error"] = str(exc)[:200]
    return out


def copy_calibration():
    """A plain copy of known size: 1 GiB read and 1 GiB written per launch."""
    import torch
    n = 1 << 29  # bf16 elements = 1 GiB
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_launch": n * 2,
                      "copy_calibration_bytes_written_per_launch": n * 2, "launches": 3}))


def log(args, msg):
    if not args.quiet:
        print(msg, file=sys.stderr, flush=True)


def source_digest(fnames) -> str:
    """First 16 hex digits of the sha256 over the kernel's source files, in order."""
    h = hashlib.sha256()
    for fname in fnames:
        path = os.path.join(ROOT, "sparse_mixture_experts_switchffn_amd", "csrc", fname)
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if still valid."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    srcs = KERNEL_SOURCES.get(kernel) or (("bwd.hip", "sffn_device.h") if kernel.startswith("bwd_")
                                          else None)
    if srcs is None or kv.get("source_sha256_16") != source_digest(srcs):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measured_mfma(stage: str, workload: str):
    """Matrix-core counters of a stage from the committed rocprofv3 summary, if still valid:
    {mfma_flops, busy_frac} per launch (profiles/<stage>_<workload>_mfma.txt)."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}_mfma.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    srcs = KERNEL_SOURCES.get(stage)
    if srcs is None or kv.get("source_sha256_16") != source_digest(srcs):
        return None
    try:
        return {"mfma_flops": float(kv["mfma_flops_per_launch"]), "busy_frac": float(kv["busy_frac"]),
                "kernel": kv.get("kernel")}
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(w, stage, accepted, active, esize, dropped=0, k=1, reroute=False):
    """Bytes a stage must move at minimum, from what it reads and writes once.

    The router runs one of two ways (the library's choice, mirrored here):
    fused (bf16, N <= 128, fewer than 32768 tokens when N > 64): the whole
          router is in the softmax_route stage (router_logits launches nothing):
          Wr read, its three bf16 planes written and read once, x read, and the
          fp32 logits, expert/gate/rank per token and the per-block p sums and
          counts written;
    tiled / staged (otherwise): router_logits reads x and Wr (and, tiled, writes
          and reads the planes once) and writes the fp32 logits; softmax_route
          reads the logits and writes the same per-token and per-block outputs.
    dispatch_scan: per-block counts and p sums read, per-block bases written, and the
          per-expert counts / accepted / p totals.
    dispatch_scatter: expert, rank, block base and gate per token read; slot per token,
          the row-to-token and row-to-gate maps, and the dropped rows (read + write).
    ffn1: W1 of every expert with accepted tokens + the gathered x rows + the H rows
          written + b1 + the row-to-token map.
    ffn2: W2 of active experts + H rows + the x rows of the residual + the y rows
          written + b2 + gate and row-to-token entries.
    Top-2 (k = 2): A counts accepted choices; the router (fused or tiled as above)
    writes two choices, gates and ranks per token; dispatch_scatter copies no rows;
    ffn2 writes the gate-scaled expert rows and its stage also holds the combine
    (x and those rows read once, y written).
    GEGLU experts: ffn1 reads both up-projections (2F rows of W1 and of b1).
    Rerouting (k = 1): the router writes both choices and gates and the first-choice
    rank per token; dispatch_scan also reads the choices and
    ranks again, writes the first-stage slot and the overflow ranks and scans the
    overflow counts; dispatch_scatter reads both choices and gates, the first-stage
    slot and the overflow rank, and writes expert, gate and slot per token.
    """
    A = accepted
    T, N, d = w.T, w.N, w.d
    nblk = (T + 31) // 32
    bf16 = w.dtype == "bf16"
    tiled = bf16 and N % 4 == 0 and (N > 128 or (N > 64 and T >= 256 * 128))
    fused = bf16 and N <= 128 and not tiled
    wbytes = active * w.F * w.d * esize
    w1mul = 2 if w.glu else 1  # GEGLU: two up-projections (W1 and b1 of 2F rows)
    bias1 = w1mul * active * w.F * esize if w.has_bias else 0
    bias2 = active * w.d * esize if w.has_bias else 0
    outs = T * 12 * k + nblk * N * (8 + 4 * (k - 1))
    if reroute:
        outs = T * 20 + nblk * N * 8
    if stage == "ffn1":
        return w1mul * wbytes + A * w.d * esize + A * w.F * esize + bias1 + A * 4
    if stage == "ffn2":
        if k == 2:
            return (wbytes + A * w.F * esize + A * w.d * esize + bias2 + A * 8
                    + 2 * T * d * esize + A * d * esize)
        return wbytes + A * w.F * esize + 2 * A * w.d * esize + bias2 + A * 8
    if stage == "router_logits":
        if fused:
            return None
        return T * d * esize + N * d * 4 + (12 * N * d if tiled else 0) + T * N * 4
    if stage == "softmax_route":
        if fused:
            return T * d * 2 + N * d * 4 + 12 * N * d + T * N * 4 + outs
        return T * N * 4 + outs
    if stage == "dispatch_scan":
        if reroute:
            return 2 * (nblk * N * 12 + N * 16) + T * 24
        return nblk * N * 12 + N * 16
    if stage == "dispatch_scatter":
        if reroute:
            return T * 36 + A * 8 + 2 * dropped * d * esize
        if k == 2:
            return T * 40 + A * 8
        return T * 20 + A * 8 + 2 * dropped * d * esize
    return None


def backward_bytes(w, stage, accepted, active, esize, parts):
    """Bytes a backward stage must move at minimum (each operand read once, each
    result written once; A accepted rows, `active` experts with rows):
    expert_dgrad_hidden: W2 of active experts, dy and H rows read, dA rows and the
        partial dg (one fp32 per row and 128-column tile) written;
    router_grad: the forward's logits read, dz written, partial dg read (plus dy . b2);
    expert_dgrad_input: W1 of active experts and dA rows read, fp32 dXe rows written;
    dx: dz, Wr, dy and dXe read, dx written;
    router_wgrad: dz and x read, per-part fp32 sums written, read back and summed;
    expert_wgrad: dy, H, dA and x rows read, dW2 and dW1 of every expert written;
    bias_grad: dy and dA rows read, db2 and db1 written.
    """
    A, T, N, d, F = accepted, w.T, w.N, w.d, w.F
    n_dgp = (F + 127) // 128 if w.dtype == "bf16" else 1
    wb = active * d * F * esize
    if stage == "expert_dgrad_hidden":
        return wb + A * d * esize + 2 * A * F * esize + n_dgp * A * 4 + A * 8
    if stage == "router_grad":
        return 2 * T * N * 4 + n_dgp * A * 4 + (A * d * esize if w.has_bias else 0) + T * 8
    if stage == "expert_dgrad_input":
        return wb + A * F * esize + A * d * 4 + A * 4
    if stage == "dx":
        return T * N * 4 + N * d * 4 + 2 * T * d * esize + A * d * 4 + T * 4
    if stage == "router_wgrad":
        return T * N * 4 + T * d * esize + 2 * parts * N * d * 4 + N * d * 4
    if stage == "expert_wgrad":
        return 2 * N * d * F * esize + 2 * A * d * esize + 2 * A * F * esize + A * 8
    if stage == "bias_grad":
        return (A * d * esize + A * F * esize + N * (d + F) * esize) if w.has_bias else None
    return None


def host_cpu():
    """The host the oracle runs on: logical CPUs, the ones this process may use, the CPU
    model and the BLAS thread count numpy's matmuls use."""
    info = {"nproc": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    info["omp_num_threads"] = os.environ.get("OMP_NUM_THREADS")
    try:
        from threadpoolctl import threadpool_info
        info["blas_threads"] = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        info["blas_threads"] = int(os.environ.get("OMP_NUM_THREADS", "1"))
    return info


def one_thread_rates(args):
    """The oracle's forward on Tiny and Switch-Base-like with numpy's BLAS on one thread
    (tokens/s; Tiny repeated for about a second, Switch-Base-like one pass)."""
    import oracle
    import switchffn_synth as synth
    from threadpoolctl import threadpool_limits

    out = {}
    for name, min_s in (("tiny", 1.0), ("switch_base", 0.0)):
        w = synth.workload(name)
        dec = {k: synth.decode(v) for k, v in synth.host_inputs(w).items()}
        experts = (dec["W1"], dec["b1"], dec["W2"], dec["b2"])
        with threadpool_limits(limits=1):
            passes, t0 = 0, time.perf_counter()
            while True:
                oracle.forward(dec["x"], dec["Wr"], experts, w.CF, w.dtype)
                passes += 1
                el = time.perf_counter() - t0
                if el >= min_s or passes >= 10000:
                    break
        out[name] = {"tokens_per_s": w.T * passes / el, "passes": passes, "seconds": el}
        log(args, f"cpu_baseline: {name} on one thread, {passes} passes in {el:.2f} s")
    return out


def cpu_baseline_extrapolated(w, args):
    """The many-expert oracle, bounded: the router (logits, softmax, top-1), dispatch and
    aux loss over every token, and the expert FFNs of 64 experts stratified by load;
    the FFN time is scaled by A / A_subset (accepted rows) to the whole layer."""
    import numpy as np

    import oracle
    import switchffn_synth as synth

    log(args, f"cpu_baseline: drawing x and Wr for {w.name}")
    x = synth.decode(synth.host_array(w, "x").reshape(w.T, w.d))
    Wr = synth.decode(synth.host_array(w, "Wr").reshape(w.N, w.d))
    C = oracle.capacity(w.T, w.N, w.CF)
    # routing only (no expert computed): the router, dispatch and aux loss in full
    t0 = time.perf_counter()
    r0 = oracle.forward(x, Wr, lambda e: None, w.CF, w.dtype, only_experts=[])
    t_route = time.perf_counter() - t0
    acc = r0["accepted"]
    order = np.argsort(acc, kind="stable")
    pick = sorted(int(order[i]) for i in np.linspace(0, w.N - 1, 64).round().astype(int))
    A, A_sub = int(acc.sum()), int(acc[pick].sum())
    log(args, f"cpu_baseline: routing {t_route:.1f} s; drawing 64 experts' weights "
              f"({A_sub} of {A} accepted rows)")
    raw = {e: synth.expert_weights_host(w, e) for e in pick}

    def experts(e):
        ew = raw[e]
        return (synth.decode(ew["W1"]), synth.decode(ew["b1"]), synth.decode(ew["W2"]),
                synth.decode(ew["b2"]))

    t0 = time.perf_counter()
    oracle.forward(x, Wr, experts, w.CF, w.dtype, only_experts=pick)
    t_sub = time.perf_counter() - t0
    t_ffn = max(t_sub - t_route, 0.0) * A / max(A_sub, 1)
    total = t_route + t_ffn
    log(args, f"cpu_baseline: routing + 64 experts {t_sub:.1f} s; extrapolated layer "
              f"{total:.1f} s")
    return {"value": w.T / total, "unit": "tokens/s", "kind": "oracle",
            "extrapolated": True,
            "sample": (f"{w.name}: router, softmax, top-1, dispatch and aux loss of all "
                       f"{w.T} tokens in full ({t_route:.1f} s, float64 numpy); expert FFNs of "
                       f"64 of {w.N} experts stratified by load ({A_sub} of {A} accepted rows, "
                       f"{t_sub - t_route:.1f} s), extrapolated by A/A_subset to "
                       f"{t_ffn:.1f} s: layer {total:.1f} s (extrapolated)"),
            "seconds": {"routing": t_route, "ffn_subset": t_sub - t_route,
                        "ffn_extrapolated": t_ffn}, "capacity": C}


def cpu_baseline(w, budget_s, args):
    """The oracle as it stands on this host: full forward passes until the budget is used
    (many_expert: the bounded, extrapolated sample of cpu_baseline_extrapolated), with the
    host's description and one-thread rates of the two small workloads beside it."""
    host = host_cpu()
    if w.name == "many_expert" and not (args.backward or args.reroute or args.topk != 1
                                        or w.glu):
        out = cpu_baseline_extrapolated(w, args)
    else:
        out = cpu_baseline_full(w, budget_s, args)
    out["cores"] = host["blas_threads"]
    out["host"] = host
    try:
        out["one_thread"] = one_thread_rates(args)
    except Exception as exc:  # noqa: BLE001 -- a reference figure only
        out["one_thread"] = {"error": str(exc)[:200]}
    return out


def cpu_baseline_full(w, budget_s, args):
    """Full forward (or training-step) passes of the oracle until the budget is used."""
    import numpy as np

    import oracle
    import switchffn_synth as synth

    log(args, f"cpu_baseline: drawing inputs for {w.name}")
    host = synth.host_inputs(w, max_elems=1 << 31)
    dec = {k: synth.decode(v) for k, v in host.items()}
    experts = (dec["W1"], dec["b1"], dec["W2"], dec["b2"])
    passes, t0 = 0, time.perf_counter()
    while True:
        act = "geglu" if w.glu else "relu"
        if getattr(args, "backward", False):
            dy = np.random.default_rng(1).standard_normal((w.T, w.d))
            oracle.forward(dec["x"], dec["Wr"], experts, w.CF, w.dtype)
            oracle.backward(dec["x"], dec["Wr"], experts, w.CF, dy, 0.01)
        elif getattr(args, "reroute", False):
            oracle.forward_reroute(dec["x"], dec["Wr"], experts, w.CF, w.dtype, activation=act)
        else:
            oracle.forward(dec["x"], dec["Wr"], experts, w.CF, w.dtype,
                           k=getattr(args, "topk", 1), activation=act)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s or passes >= 1000:
            break
    log(args, f"cpu_baseline: {passes} passes in {el:.2f} s")
    kind = "forward + backward" if getattr(args, "backward", False) else "forward"

    return {"value": w.T * passes / el, "unit": "tokens/s", "kind": "oracle",
            "extrapolated": False,
            "sample": f"{passes} full {kind} pass(es) of the {w.name} workload "
                      f"(T={w.T}) in float64 numpy, {el:.1f} s"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.stderr.write("bench.py: multi-GPU runs are not supported (one GPU only)\n")
        return 2

    import torch

    import sparse_mixture_experts_switchffn_amd as sffn
    import switchffn_synth as synth

    w = synth.workload(args.config)
    if args.geglu:
        w = w.replace(glu=True)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(args, f"bench: {w.describe()}")
    inp = synth.device_inputs(w, dev)
    T, N = w.T, w.N
    esize = 2 if w.dtype == "bf16" else 4
    stats = {"expert_count": torch.zeros(N, dtype=torch.int32, device=dev),
             "accepted_count": torch.zeros(N, dtype=torch.int32, device=dev),
             "n_dropped": torch.zeros(1, dtype=torch.int32, device=dev)}
    K = args.topk
    if args.reroute and K != 1:
        sys.stderr.write("bench.py: --reroute is a top-1 form; it needs --topk 1\n")
        return 2
    FLAGS = (sffn.SFFN_REROUTE_OVERFLOW if args.reroute else 0) | (sffn.SFFN_GEGLU if w.glu else 0)
    BWD = bool(args.backward)
    if BWD and (K != 1 or FLAGS):
        sys.stderr.write("bench.py: --backward covers the top-1 ReLU layer only\n")
        return 2
    out = sffn.switch_ffn_forward(inp["x"], inp["Wr"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                                  w.CF, stats=stats, k=K, flags=FLAGS)
    bufs = {k: out[k] for k in ("y", "expert_idx", "slot", "gate", "aux_loss", "workspace")}
    nst = sffn.switch_ffn_num_stages()
    names = [sffn.switch_ffn_stage_name(i) for i in range(nst)]
    nbs = sffn.switch_ffn_backward_num_stages() if BWD else 0
    bnames = [sffn.switch_ffn_backward_stage_name(i) for i in range(nbs)]
    stream = torch.cuda.current_stream(dev)
    grads = None
    if BWD:
        gen = torch.Generator(device=dev).manual_seed(1)
        dy = torch.randn(T, w.d, generator=gen, device=dev).to(inp["x"].dtype)
        grads = sffn.switch_ffn_backward(inp["x"], inp["Wr"], inp["W1"], inp["b1"], inp["W2"],
                                         inp["b2"], w.CF, out, dy, 0.01)
        gbufs = {k: grads[k] for k in ("dx", "dWr", "dW1", "db1", "dW2", "db2", "workspace")}

    def step(events=None, bevents=None):
        sffn.switch_ffn_forward(inp["x"], inp["Wr"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                                w.CF, stats=stats, stage_events=events, k=K, flags=FLAGS,
                                **bufs)
        if BWD:
            sffn.switch_ffn_backward(inp["x"], inp["Wr"], inp["W1"], inp["b1"], inp["W2"],
                                     inp["b2"], w.CF, bufs, dy, 0.01, stage_events=bevents,
                                     **gbufs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    y_ref = bufs["y"].clone()
    dx_ref = gbufs["dx"].clone() if BWD else None

    def timed(run, n_steps):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        w0 = time.perf_counter()
        t0.record(stream)
        run()
        t1.record(stream)
        torch.cuda.synchronize(dev)
        return t0.elapsed_time(t1) / n_steps, time.perf_counter() - w0

    # Eager launches: exactly K steps, events only at the two ends (an event between
    # kernels costs a few microseconds of GPU time, so stage events stay out).
    eager_ms, eager_wall = timed(lambda: [step() for _ in range(args.steps)], args.steps)

    # The same K steps replayed from a HIP graph of `graph` forward calls (the
    # remainder launched eagerly), which removes the host launch gaps between the
    # kernels; used only if a replay reproduces the eager output bit for bit.
    graph_info = {"calls_per_graph": 0, "used": False}
    ms_per_step, wall = eager_ms, eager_wall
    if args.graph > 0:
        try:
            side = torch.cuda.Stream(dev)
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for _ in range(2):
                    step()
            stream.wait_stream(side)
            torch.cuda.synchronize(dev)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(args.graph):
                    step()
            torch.cuda.synchronize(dev)
            bufs["y"].zero_()
            if BWD:
                gbufs["dx"].zero_()
            g.replay()
            torch.cuda.synchronize(dev)
            exact = bool(torch.equal(bufs["y"], y_ref))
            if BWD:
                exact = exact and bool(torch.equal(gbufs["dx"], dx_ref))
            graph_info = {"calls_per_graph": args.graph, "replay_matches_eager": exact,
                          "used": exact}
            if exact:
                for _ in range(5):  # the first replays of a new graph carry a set-up cost
                    g.replay()
                torch.cuda.synchronize(dev)
                reps, rest = divmod(args.steps, args.graph)

                def run_graph():
                    for _ in range(reps):
                        g.replay()
                    for _ in range(rest):
                        step()
                ms_per_step, wall = timed(run_graph, args.steps)
            del g
        except Exception as exc:  # capture unsupported: keep the eager timing
            graph_info = {"calls_per_graph": args.graph, "used": False, "error": str(exc)[:200]}
    total_ms = ms_per_step * args.steps

    # Stage region: K more steps with an event before each stage and after the last,
    # recorded on the launch stream; per-stage averages give the kernels' durations.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(args.steps)]
    for row in evs:  # create the underlying handles
        for e in row:
            e.record(stream)
    torch.cuda.synchronize(dev)
    bevs = [[torch.cuda.Event(enable_timing=True) for _ in range(nbs + 1)] for _ in range(args.steps)]
    for row in bevs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize(dev)
    for k in range(args.steps):
        step(evs[k], bevs[k] if BWD else None)
    torch.cuda.synchronize(dev)
    stage_ms = {names[i]: sum(evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps))
                / args.steps for i in range(nst)}
    bwd_ms = {bnames[i]: sum(bevs[k][i].elapsed_time(bevs[k][i + 1]) for k in range(args.steps))
              / args.steps for i in range(nbs)}

    # Per-call wall time on the stream: an event between consecutive eager calls.
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize(dev)
    cev[0].record(stream)
    for k in range(args.steps):
        step()
        cev[k + 1].record(stream)
    torch.cuda.synchronize(dev)
    per_call = sorted(cev[k].elapsed_time(cev[k + 1]) for k in range(args.steps))

    def pct(q):
        return per_call[min(len(per_call) - 1, int(round(q * (len(per_call) - 1))))]

    acc = stats["accepted_count"].cpu()
    accepted = int(acc.sum())
    active = int((acc > 0).sum())
    dropped = int(stats["n_dropped"].cpu()[0])
    parts = None
    if BWD:
        tiles = ((N + 127) // 128) * ((w.d + 127) // 128)
        parts = max(1, min((1024 + tiles - 1) // tiles, (T + 127) // 128))

    def stage_bytes(name):
        if name.startswith("bwd_"):
            return backward_bytes(w, name[4:], accepted, active, esize, parts)
        return algorithmic_bytes(w, name, accepted, active, esize, dropped, K, args.reroute)

    all_ms = dict(stage_ms)
    all_ms.update({"bwd_" + k: v for k, v in bwd_ms.items()})
    dominant = max(all_ms, key=all_ms.get)
    alg = stage_bytes(dominant)
    stage_table = {}
    for name, ms in all_ms.items():
        b = stage_bytes(name)
        gbs = b / (ms * 1e-3) / 1e9 if (b and ms > 0) else None
        stage_table[name] = {"ms": ms, "algorithmic_bytes": b, "GB_per_s": gbs,
                             "hbm_frac": gbs / HBM_PEAK_GBS if gbs else None}
    achieved = alg / (all_ms[dominant] * 1e-3) / 1e9 if alg else None
    gemm_flops = (6.0 if w.glu else 4.0) * accepted * w.d * w.F
    gemm_ms = stage_ms.get("ffn1", 0.0) + stage_ms.get("ffn2", 0.0)
    wname = (w.name + ("_top2" if K == 2 else "") + ("_reroute" if args.reroute else "")
             + ("_geglu" if w.glu else "") + ("_train" if BWD else ""))
    traffic = measured_traffic(dominant, wname)
    counter_gemm = {}
    for st in ("ffn1", "ffn2"):
        mm = measured_mfma(st, wname)
        if mm and stage_ms.get(st):
            alg_flops = (2.0 * (2 if (w.glu and st == "ffn1") else 1)) * accepted * w.d * w.F
            tf = mm["mfma_flops"] / (stage_ms[st] * 1e-3) / 1e12
            counter_gemm[st] = {"kernel": mm["kernel"], "mfma_flops": mm["mfma_flops"],
                                "tflops": tf, "frac_of_bf16_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                                "mfma_busy_frac": mm["busy_frac"],
                                "padded_over_algorithmic": mm["mfma_flops"] / alg_flops}
    w1mul = 2 if w.glu else 1
    layer_bytes = (active * (w1mul + 1) * w.F * w.d * esize + N * w.d * 4 + 2 * T * w.d * esize
                   + (active * (w1mul * w.F + w.d) * esize if w.has_bias else 0))

    result = {
        "metric": "SwitchFFN fwd+bwd tokens/s" if BWD else "SwitchFFN fwd tokens/s",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded counter-based generator; x ~ N(0,1), W ~ N(0,0.02^2))",
        "config": {"workload": wname, "tokens": T, "d_model": w.d, "d_ff": w.F, "experts": N,
                   "capacity_factor": w.CF, "capacity": sffn.switch_ffn_capacity(K * T, N, w.CF),
                   "experts_per_token": K, "reroute_overflow": bool(args.reroute),
                   "expert_activation": "geglu" if w.glu else "relu",
                   "router_dtype": "fp32", "accepted_tokens": accepted, "dropped_tokens": dropped,
                   "active_experts": active, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
                     "traffic": traffic, "algorithmic_bytes": alg,
                     "layer": {"bytes": layer_bytes, "ms_per_step": ms_per_step,
                               "GB_per_s": layer_bytes / (ms_per_step * 1e-3) / 1e9,
                               "frac": layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                               "note": "weights of experts with accepted tokens (W1, W2, "
                                       "biases), Wr, x read once and y written once"}},
        "stages_ms": all_ms,
        "stages": stage_table,
        "per_call_ms": {"median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9),
                        "note": "eager calls with an event between consecutive calls"},
        "accepted_tokens_per_s": accepted / (ms_per_step * 1e-3),
        "measured_peaks": measured_peaks(dev),
        "expert_gemm": {"tflops": gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None,
                        "frac_of_bf16_mfma_peak": (gemm_flops / (gemm_ms * 1e-3) / 1e12
                                                   / MFMA_BF16_PEAK_TFLOPS) if gemm_ms else None,
                        "note": "analytic: (4 or 6 for GEGLU) * accepted * d * F flops over the two "
                                "stages' event times; counter: rocprofv3 bf16 MFMA flops per launch "
                                "(padded tile rows included) over this run's stage time",
                        "counter": counter_gemm},
        "wall_s_timed_region": wall,
        "launch": {"graph": graph_info, "eager_ms_per_step": eager_ms,
                   "eager_tokens_per_s": T / (eager_ms * 1e-3)},
    }
    del inp, bufs, out
    torch.cuda.empty_cache()
    if args.cpu_seconds > 0 and (w.name != "many_expert" or not (BWD or args.reroute or K != 1
                                                                  or w.glu)):
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, args)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
