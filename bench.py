"""Benchmark of the fused attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

A step is one pass of the attention over one batch of synthetic input of the
chosen standing workload (default: the causal GQA long-context workload B=2,
Hq=32, Hkv=8, N=8192, d=128, bf16): one fa_fwd (or fa_fwd_f32) call, or for
the fp8 workload (config 5) fa_fp8_prepare (Hadamard rotation of Q and K,
per-tensor scales, e4m3 codes) followed by fa_fwd_fp8.  Inputs are resident
in HBM before timing starts; K steps are timed back to back with HIP events
on the stream the kernels run on.  Prints one JSON line on stdout
(diagnostics go to stderr):

  value     attention forward TFLOP/s = 4*B*Hq*Nq*Nk*d (halved when causal) / step time
  roofline  the attention kernel (its own launch time, from events around
            each launch) against the MI355X dense MFMA peak for its dtype, and
            the HBM traffic measured by rocprofv3 counters for the same kernel
            source (null when the source changed since the counters were taken)
  cpu_baseline  the fp64 oracle timed on this host's cores over a bounded
            sample of the same workload (whole heads), as a reported baseline

--config backward measures the backward pass (fa_bwd_dq then fa_bwd_dkdv:
dQ, dK, dV for a seeded upstream gradient dO, probabilities recomputed from
the saved LSE) on the same causal GQA workload, O and LSE from one fa_fwd
before timing.  value = 10*B*Hq*Nq*Nk*d (halved when causal) per step, the
five matrix products of the gradient; the roofline is the dK/dV kernel with
its four of them (S, dP, dV, dK) against its own launch time.  The dQ kernel
recomputes S and dP, so only its dQ product counts as algorithmic work.

--config decode measures the key-split path (fa_fwd_splitkv: parts over key
ranges merged on the GPU) on a GQA decoding step, B=8 sequences, Hq=32,
Hkv=8, one query each over Nk=32768 keys, d=128.  That path is bound by HBM
bandwidth, so its line reports algorithmic bytes per second (Q, K, V, O, LSE
once) against the 8 TB/s of HBM3E; the step includes the merge kernel.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % of MFMA peak (bf16, causal GQA, N=8K, d=128)"
# MI355X published dense peaks (no sparsity), TFLOP/s
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 2500.0, "fp8": 5000.0}
# sources of the attention kernel of each dtype (the traffic summary is valid
# only for the sources it was measured on)
_CSRC = "exact_attention_07_amd/csrc/"
KERNEL_SOURCES = {
    "bf16": [_CSRC + f for f in ("fa_fwd.hip", "fa_frag.h", "fa_device.h", "plan.h")],
    "f32": [_CSRC + f for f in ("fa_fwd.hip", "fa_frag.h", "fa_device.h", "plan.h")],
    "fp8": [_CSRC + f for f in ("fa_fwd_fp8.hip", "fa_device.h", "plan.h")],
    "bwd": [_CSRC + f for f in ("fa_bwd.hip", "fa_frag.h", "fa_device.h", "plan.h")],
}
KERNEL_NAME = {"bf16": "fa_fwd_bf16_kernel", "f32": "fa_fwd_f32_kernel", "fp8": "fa_fwd_fp8_kernel",
               "bwd": "fa_bwd_dkdv_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(dtype: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[dtype]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(tag: str, dtype: str):
    """HBM bytes per launch of the measured kernel from the committed
    rocprofv3 counter summary profiles/traffic_<tag>.txt, if it was taken on
    the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != source_hash(dtype):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, x, budget_s: float):
    """Time the fp64 oracle on whole (b, h) heads of the workload until budget_s elapsed."""
    from oracle import attention_fp64
    from oracle.formats import bf16_bits_to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    g = w.Hq // w.Hkv
    done, flops, t_total = 0, 0.0, 0.0
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    for b, h in heads:
        q = bf16_bits_to_f64(x["q"][b:b + 1, h:h + 1])
        k = bf16_bits_to_f64(x["k"][b:b + 1, h // g:h // g + 1])
        v = bf16_bits_to_f64(x["v"][b:b + 1, h // g:h // g + 1])
        t0 = time.perf_counter()
        attention_fp64(q, k, v, w.softmax_scale, w.causal)
        t_total += time.perf_counter() - t0
        done += 1
        f = 4.0 * w.Nq * w.Nk * w.d
        flops += f / 2 if w.causal else f
        if t_total >= budget_s:
            break
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {len(heads)} (b,h) heads of the same workload, fp64 two-pass oracle "
                      f"(S and P materialised), {t_total:.1f} s"}


def cpu_baseline_backward(w, x, dout, budget_s: float):
    """Time the fp64 gradient oracle on whole (b, h) heads until budget_s elapsed."""
    from oracle import attention_backward_fp64
    from oracle.formats import bf16_bits_to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    g = w.Hq // w.Hkv
    done, flops, t_total = 0, 0.0, 0.0
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    for b, h in heads:
        q = bf16_bits_to_f64(x["q"][b:b + 1, h:h + 1])
        k = bf16_bits_to_f64(x["k"][b:b + 1, h // g:h // g + 1])
        v = bf16_bits_to_f64(x["v"][b:b + 1, h // g:h // g + 1])
        do = bf16_bits_to_f64(dout[b:b + 1, h:h + 1])
        t0 = time.perf_counter()
        attention_backward_fp64(q, k, v, do, w.softmax_scale, w.causal)
        t_total += time.perf_counter() - t0
        done += 1
        f = 10.0 * w.Nq * w.Nk * w.d
        flops += f / 2 if w.causal else f
        if t_total >= budget_s:
            break
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {len(heads)} (b,h) heads of the same workload, fp64 gradient oracle "
                      f"(P, dP, dS materialised), {t_total:.1f} s"}


def bench_backward(args, torch, api, gen):
    w, x = gen.make_config(3)
    dout = gen.make_dout(w, (3,))
    log(f"workload: backward of {w.name}")
    dev = torch.device("cuda:0")

    def dev_tensor(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = (dev_tensor(a) for a in (x["q"], x["k"], x["v"], dout))
    stream = torch.cuda.current_stream()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    api.fa_fwd(q, k, v, o, lse, w.softmax_scale, w.causal, stream)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(api.bwd_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal) // 4, dtype=torch.float32,
                     device=dev)

    def stage_dq():
        api.fa_bwd_dq(q, k, v, o, lse, do, dq, w.softmax_scale, w.causal, ws, stream)

    def stage_dkdv():
        api.fa_bwd_dkdv(q, k, v, o, lse, do, dk, dv, w.softmax_scale, w.causal, ws, stream)

    for _ in range(args.warmup):
        stage_dq()
        stage_dkdv()
    torch.cuda.synchronize()

    def event():
        return torch.cuda.Event(enable_timing=True)

    marks = [(event(), event(), event()) for _ in range(args.steps)]
    e0, e1 = event(), event()
    t0 = time.perf_counter()
    e0.record(stream)
    for a, m, b in marks:
        a.record(stream)
        stage_dq()
        m.record(stream)
        stage_dkdv()
        b.record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    dq_ms = sum(a.elapsed_time(m) for a, m, _ in marks) / args.steps
    dkdv_ms = sum(m.elapsed_time(b) for _, m, b in marks) / args.steps
    fwd_flops = w.flops()                 # one product pair of the forward pass = 2 products
    flops = 2.5 * fwd_flops               # S, dP, dV, dK, dQ
    tflops = flops / (ms * 1e-3) / 1e12
    dkdv_tflops = 2.0 * fwd_flops / (dkdv_ms * 1e-3) / 1e12   # S, dP, dV, dK
    dq_exec_tflops = 1.5 * fwd_flops / (dq_ms * 1e-3) / 1e12  # S, dP, dQ as executed
    log(f"{args.steps} steps: {ms:.4f} ms/step (events), {wall / args.steps * 1e3:.4f} ms/step (wall), "
        f"{tflops:.1f} TFLOP/s; dQ kernel {dq_ms:.4f} ms ({dq_exec_tflops:.1f} TFLOP/s executed), "
        f"dK/dV kernel {dkdv_ms:.4f} ms ({dkdv_tflops:.1f} TFLOP/s)")

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB device copy done")

    if args.check:
        # one query row of dQ against the oracle's gradient of one head (stderr only)
        from oracle import attention_backward_fp64
        from oracle.formats import bf16_bits_to_f64
        b_, h_ = w.B - 1, w.Hq - 1
        g = w.Hq // w.Hkv
        rq, rk, rv = attention_backward_fp64(bf16_bits_to_f64(x["q"][b_:b_ + 1, h_:h_ + 1]),
                                             bf16_bits_to_f64(x["k"][b_:b_ + 1, h_ // g:h_ // g + 1]),
                                             bf16_bits_to_f64(x["v"][b_:b_ + 1, h_ // g:h_ // g + 1]),
                                             bf16_bits_to_f64(dout[b_:b_ + 1, h_:h_ + 1]), w.softmax_scale, w.causal)
        got = dq[b_, h_].float().cpu().numpy()
        err = np.abs(got - rq[0, 0])
        log(f"check dQ of head ({b_},{h_}): rms err / rms ref = "
            f"{np.sqrt((err ** 2).mean()) / np.sqrt((rq ** 2).mean()):.2e}")

    traffic = load_traffic("backward", "bwd")
    line = {
        "metric": "attention bwd TFLOP/s + % of MFMA peak (bf16, causal GQA, N=8K, d=128)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q, K, V, dO; O and LSE from fa_fwd; resident in HBM before timing)",
        "config": {"workload": "backward of " + w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk,
                   "d": w.d, "causal": w.causal, "kernel": KERNEL_NAME["bwd"],
                   "steps_in_a_step": "fa_bwd_dq (dQ, D, LSE log2 e) + fa_bwd_dkdv (dK, dV)"},
        "roofline": {"bound": "mfma", "achieved": round(dkdv_tflops, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(dkdv_tflops / PEAK_TFLOPS["bf16"], 4), "traffic": traffic,
                     "kernel_ms": round(dkdv_ms, 5)},
        "dq_kernel": {"ms": round(dq_ms, 5), "executed_tflops": round(dq_exec_tflops, 2),
                      "algorithmic_tflops": round(0.5 * fwd_flops / (dq_ms * 1e-3) / 1e12, 2)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_backward(w, x, dout, args.cpu_budget)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="3", help="standing workload 1..5, decode or backward")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--check", action="store_true", help="compare sampled rows with the oracle (stderr)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one 1 GiB device copy (reference for rocprofv3 byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_attention_07_amd import api, gen

    if args.config == "backward":
        bench_backward(args, torch, api, gen)
        return
    cfg = args.config if args.config == "decode" else int(args.config)
    args.config = cfg
    w, x = gen.make_config(cfg)
    log(f"workload: {w.name}")
    dev = torch.device("cuda:0")

    def dev_tensor(a):
        if w.dtype == "f32":
            return torch.from_numpy(a).to(dev)
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = (dev_tensor(x[t]) for t in "qkv")
    o = torch.empty(q.shape, dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    decode = cfg == "decode"
    if decode:
        ws_bytes = api.splitkv_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, 0)
        ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=dev)

        def prepare():
            pass

        def attend():
            api.fa_fwd_splitkv(q, k, v, o, lse, w.softmax_scale, w.causal, 0, ws, stream)
    elif w.dtype == "fp8":
        signs = torch.from_numpy(x["signs"]).to(dev)
        q8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
        k8 = torch.empty(k.shape, dtype=torch.uint8, device=dev)
        v8t = torch.empty((w.B, w.Hkv, w.d, api.padded_keys(w.Nk)), dtype=torch.uint8, device=dev)
        descale = torch.empty(3, dtype=torch.float32, device=dev)
        amax_ws = torch.empty(3, dtype=torch.int32, device=dev)

        def prepare():
            api.fa_fp8_prepare(q, k, v, q8, k8, v8t, descale, amax_ws, signs, stream)

        def attend():
            api.fa_fwd_fp8(q8, k8, v8t, descale, o, lse, w.softmax_scale, w.causal, stream)
    else:
        fwd = api.fa_fwd if w.dtype == "bf16" else api.fa_fwd_f32

        def prepare():
            pass

        def attend():
            fwd(q, k, v, o, lse, w.softmax_scale, w.causal, stream)

    for _ in range(args.warmup):
        prepare()
        attend()
    torch.cuda.synchronize()

    def event():
        return torch.cuda.Event(enable_timing=True)

    # events around every attention launch give its own duration; the step
    # time is the span from the first to the last event
    marks = [(event(), event()) for _ in range(args.steps)]
    e0, e1 = event(), event()
    t0 = time.perf_counter()
    e0.record(stream)
    for a, b in marks:
        prepare()
        a.record(stream)
        attend()
        b.record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    kernel_ms = sum(a.elapsed_time(b) for a, b in marks) / args.steps
    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    kernel_tflops = flops / (kernel_ms * 1e-3) / 1e12
    log(f"{args.steps} steps: {ms:.4f} ms/step (events), {wall / args.steps * 1e3:.4f} ms/step (wall), "
        f"{tflops:.1f} TFLOP/s; attention kernel {kernel_ms:.4f} ms/launch, {kernel_tflops:.1f} TFLOP/s")

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB device copy done")

    if args.check:
        from oracle import attention_rows_fp64
        from oracle.formats import bf16_bits_to_f64
        rows = [(0, 0, 0), (w.B - 1, w.Hq - 1, w.Nq - 1), (0, w.Hq // 2, w.Nq // 3)]
        conv = (lambda a: a.astype(np.float64)) if w.dtype == "f32" else bf16_bits_to_f64
        o_ref, l_ref = attention_rows_fp64(conv(x["q"]), conv(x["k"]), conv(x["v"]), w.softmax_scale, w.causal,
                                           rows)
        oo = o.float().cpu().numpy()
        ll = lse.cpu().numpy()
        err = max(float(np.abs(oo[b, h, i] - o_ref[r]).max()) for r, (b, h, i) in enumerate(rows))
        lerr = max(abs(float(ll[b, h, i]) - l_ref[r]) for r, (b, h, i) in enumerate(rows))
        log(f"check on {len(rows)} rows: max|O err|={err:.2e} max|LSE err|={lerr:.2e}")

    if decode:
        # the same step without the split, for comparison (stderr)
        for _ in range(3):
            api.fa_fwd(q, k, v, o, lse, w.softmax_scale, w.causal, stream)
        a, b = event(), event()
        a.record(stream)
        for _ in range(args.steps):
            api.fa_fwd(q, k, v, o, lse, w.softmax_scale, w.causal, stream)
        b.record(stream)
        torch.cuda.synchronize()
        log(f"without the key split (fa_fwd): {a.elapsed_time(b) / args.steps:.4f} ms/step")
        nbytes = 2 * (q.numel() + k.numel() + v.numel() + o.numel()) + 4 * lse.numel()
        gbs = nbytes / (ms * 1e-3) / 1e9
        log(f"key split: {ws_bytes / 4 / (w.B * w.Hq * w.Nq * (w.d + 1)):.0f} ranges, {gbs:.0f} GB/s")
        line = {
            "metric": "attention decode step HBM GB/s (bf16, GQA, Nq=1, Nk=32K, d=128)",
            "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic (seeded N(0,1), resident in HBM before timing)",
            "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                       "causal": w.causal, "path": "fa_fwd_splitkv (attention kernel over key ranges + merge)"},
            # achieved: algorithmic bytes over the whole step (attention kernel
            # over the key ranges + the merge, one library call); traffic: HBM
            # bytes of the attention kernel (rocprofv3 counters)
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                         "frac": round(gbs / 8000.0, 4), "traffic": load_traffic("decode", "bf16"),
                         "step_ms": round(ms, 5), "call_ms": round(kernel_ms, 5), "tflops": round(tflops, 2)},
        }
        print(json.dumps(line), flush=True)
        return

    peak = PEAK_TFLOPS[w.dtype]
    traffic = load_traffic(f"config{args.config}", w.dtype)
    data = "synthetic (seeded N(0,1), generated on the host, resident in HBM before timing)"
    if w.dtype == "fp8":
        data = ("synthetic (seeded N(0,1) bf16, Q and K with +-50 outliers at p=0.001; quantised to e4m3 "
                "inside every step; resident in HBM before timing)")
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": data,
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "kernel": KERNEL_NAME[w.dtype]},
        "roofline": {"bound": "mfma", "achieved": round(kernel_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(kernel_tflops / peak, 4), "traffic": traffic,
                     "kernel_ms": round(kernel_ms, 5)},
    }
    if w.dtype == "fp8":
        line["config"]["steps_in_a_step"] = "fa_fp8_prepare (rotation, scales, e4m3) + fa_fwd_fp8"
        line["prepare_ms"] = round(ms - kernel_ms, 5)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
