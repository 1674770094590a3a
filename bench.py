"""Benchmark of the fused attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

A step is one pass of the attention over one batch of synthetic input of the
chosen standing workload (default: the causal GQA long-context workload B=2,
Hq=32, Hkv=8, N=8192, d=128, bf16): one fa_fwd (or fa_fwd_f32) call, or for
the fp8 workload (--config 5: B=4, H=16, N=8192, d=128, e4m3) fa_fp8_prepare (Hadamard rotation of Q and K,
per-tensor scales, e4m3 codes) followed by fa_fwd_fp8.  Inputs are resident
in HBM before timing starts; the step first runs untimed for --prewarm-ms
(default 250 ms of wall time; from a cold start the GPU's clocks need tens
of milliseconds of load to leave their idle state, and launches of the
default step fall from ~1.2 ms to a steady ~0.92 ms over the first ~30),
then W warmup steps; K steps are timed back to back with HIP events on the
stream the kernels run on.  Prints one JSON line on stdout
(diagnostics go to stderr):

  value     attention forward TFLOP/s = 4*B*Hq*Nq*Nk*d (halved when causal) / step time
  roofline  the attention kernel (its own launch time, from events around
            each launch: mean, median and min over the K launches) against
            the MI355X dense MFMA peak for its dtype; the HBM traffic, the
            sustained clock, the MFMA-busy share, the LDS bank-conflict rate
            and the VALU mix measured by rocprofv3 counters on the same kernel
            source (profiles/counters_config<N>.txt; hbm_gbs = those bytes over the launch time;
            omitted or null when the source changed since they were taken),
            with the fraction of the peak at that clock; and the measured MFMA
            ceiling (fa_mfma_ceiling, a loop of the same matrix instruction on
            toggling operands, timed right after the steps) with the fraction
            of it reached
  cpu_baseline  the fp64 oracle timed on this host's cores over a bounded
            sample of the same workload (whole (b, h) heads, one per task over
            a pool of processes), with the CPU model, as a reported baseline

--config backward measures the backward pass (fa_bwd_dq then fa_bwd_dkdv:
dQ, dK, dV for a seeded upstream gradient dO, probabilities recomputed from
the saved LSE) on the same causal GQA workload, O and LSE from one fa_fwd
before timing.  value = 10*B*Hq*Nq*Nk*d (halved when causal) per step, the
five matrix products of the gradient; the roofline is the dK/dV kernel with
its four of them (S, dP, dV, dK) against its own launch time.  The dQ kernel
recomputes S and dP, so only its dQ product counts as algorithmic work.

--ceiling-sweep measures only fa_mfma_ceiling (bf16 and fp8 MFMA loops, two
waves per SIMD) with random operands and with constant ones, and prints one
JSON line with the rate of each and the clock that rate implies (the loop is
bound by the matrix pipe: rate / (CUs x 4 SIMDs x flops per clock per SIMD)).
Under rocprofv3 counters (GRBM_GUI_ACTIVE) the same run shows the clock
directly: the evidence that on this chip the clock under dense matrix work,
and hence the reachable matrix rate, depends on the data the MFMAs toggle.

--issue-sweep measures only fa_issue_cost: rounds of MFMAs (bf16, or the
fp8 kernel's e4m3 forms) with exponentials, e4m3 packings and FMAs beside
them (the bf16 and fp8 kernels' mixes, and the same with part of the
exponentials replaced by seven FMA-pipe instructions each), each case's
median launch time against the MFMA-only case of the same instruction;
--issue-summary PATH writes the table to PATH.

--exp2-emulated Q times fa_fwd_exp2_emulated (Q of every four exponentials
computed by a polynomial on the FMA pipe) in place of fa_fwd on a bf16
workload; the line's config then names it.

--config decode measures the key-split path (fa_fwd_splitkv: parts over key
ranges merged on the GPU) on a GQA decoding step, B=8 sequences, Hq=32,
Hkv=8, one query each over Nk=32768 keys, d=128.  That path is bound by HBM
bandwidth, so its line reports algorithmic bytes per second (Q, K, V, O, LSE
once) against the 8 TB/s of HBM3E; the step includes the merge kernel.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from exact_attention_07_amd import profsum  # noqa: E402  (reads profiler summaries; no GPU, no oracle)

METRIC = "attention fwd TFLOP/s + % of MFMA peak (bf16, causal GQA, N=8K, d=128)"
# MI355X published dense peaks (no sparsity), TFLOP/s
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 2500.0, "fp8": 5000.0}
NOMINAL_CLOCK_GHZ = 2.4  # the clock the published peaks assume


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def load_counters(config):
    """The committed rocprofv3 counter summary of this workload's attention
    kernel (profiles/counters_config<N>.txt, counters_decode.txt,
    counters_backward.txt), if taken on the current kernel sources; else None."""
    return profsum.load(config, ROOT)


def load_traffic(tag: str, dtype: str, counters=None):
    """HBM bytes per launch of the measured kernel: from the counter summary
    of the workload, or from profiles/traffic_<tag>.txt, if taken on the
    current kernel sources; else None."""
    if counters and "hbm_bytes_per_launch" in counters:
        return float(counters["hbm_bytes_per_launch"])
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != profsum.source_hash(dtype):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # noqa: BLE001
        pass


def _oracle_head(args):
    """One (b, h) head of the fp64 oracle (forward, or its gradient when dO is given)."""
    import time as _t
    from oracle import attention_backward_fp64, attention_fp64
    from oracle.formats import bf16_bits_to_f64
    q, k, v, do, scale, causal = args
    q, k, v = (bf16_bits_to_f64(a)[None, None] for a in (q, k, v))
    t0 = _t.perf_counter()
    if do is None:
        attention_fp64(q, k, v, scale, causal)
    else:
        attention_backward_fp64(q, k, v, bf16_bits_to_f64(do)[None, None], scale, causal)
    return _t.perf_counter() - t0


def cpu_baseline_pool(w, x, budget_s: float, dout=None, bytes_total=None):
    """The fp64 oracle timed on this host: whole (b, h) heads of the workload,
    one per task over a pool of host processes (one BLAS thread each), until
    budget_s of wall time has passed; value = oracle flops of the finished
    heads / wall time, or, given the workload's algorithmic bytes
    (bytes_total), that share of them per second in GB/s."""
    import multiprocessing as mp
    cores = host_cores()
    g = w.Hq // w.Hkv
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    per_head = (10.0 if dout is not None else 4.0) * w.Nq * w.Nk * w.d / (2 if w.causal else 1)
    tasks = [(x["q"][b, h], x["k"][b, h // g], x["v"][b, h // g], None if dout is None else dout[b, h],
              w.softmax_scale, w.causal) for b, h in heads]
    pool = mp.get_context("spawn").Pool(cores, initializer=_pool_init)
    try:
        pool.map(abs, range(cores))  # workers started before the clock runs
        t0 = time.perf_counter()
        done, t_last = 0, t0
        for _ in pool.imap_unordered(_oracle_head, tasks):
            done += 1
            t_last = time.perf_counter()
            if t_last - t0 >= budget_s:
                break
    finally:
        pool.terminate()
        pool.join()
    wall = t_last - t0
    what = "fp64 gradient oracle (P, dP, dS materialised)" if dout is not None else \
        "fp64 two-pass oracle (S and P materialised)"
    value, unit = done * per_head / wall / 1e12, "TFLOP/s"
    if bytes_total is not None:
        value, unit = bytes_total * done / len(heads) / wall / 1e9, "GB/s"
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} of {len(heads)} (b,h) heads of the same workload, {what}, one head per task on "
                      f"{cores} processes with one BLAS thread each, {wall:.1f} s wall"}



def prewarm(torch, step, ms: float) -> int:
    """Run `step` untimed, in batches of 10 with a synchronisation after each,
    until `ms` milliseconds of wall time have passed; returns the number of
    steps run.  From a cold start the GPU's clocks take tens of milliseconds
    of load to leave their idle state: launches of the causal GQA step fall
    from about 1.2 ms to a steady 0.92 ms over the first ~30 (one box), so a
    few warmup steps alone would time the ramp rather than the kernel."""
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        n += 10
    return n

def cold_start_trace(torch, stream, step, n: int, flops: float):
    """`n` steps right after setup, no untimed ones before them, each timed
    with its own events: the launch-by-launch settling the prewarm exists
    for.  Prints one JSON line with the per-launch milliseconds."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [round(a.elapsed_time(b), 4) for a, b in ev]
    tail = ms[len(ms) // 2:]
    log(f"cold start: launches 1-10 {ms[:10]}; second half mean {np.mean(tail):.4f} ms")
    print(json.dumps({"metric": "per-launch time from a cold start", "unit": "ms", "launch_ms": ms,
                      "second_half_mean_ms": round(float(np.mean(tail)), 4),
                      "second_half_tflops": round(flops / (float(np.mean(tail)) * 1e-3) / 1e12, 2)}), flush=True)


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

    prewarm_steps = prewarm(torch, lambda: (stage_dq(), stage_dkdv()), args.prewarm_ms)
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

    traffic = load_traffic("backward", "bwd", load_counters("backward"))
    line = {
        "metric": "attention bwd TFLOP/s + % of MFMA peak (bf16, causal GQA, N=8K, d=128)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "prewarm": {"ms": args.prewarm_ms, "steps": prewarm_steps},
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q, K, V, dO; O and LSE from fa_fwd; resident in HBM before timing)",
        "config": {"workload": "backward of " + w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk,
                   "d": w.d, "causal": w.causal, "kernel": "fa_bwd_dkdv_kernel",
                   "steps_in_a_step": "fa_bwd_dq (dQ, D, LSE log2 e) + fa_bwd_dkdv (dK, dV)"},
        "roofline": {"bound": "mfma", "achieved": round(dkdv_tflops, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(dkdv_tflops / PEAK_TFLOPS["bf16"], 4), "traffic": traffic,
                     "kernel_ms": round(dkdv_ms, 5)},
        "dq_kernel": {"ms": round(dq_ms, 5), "executed_tflops": round(dq_exec_tflops, 2),
                      "algorithmic_tflops": round(0.5 * fwd_flops / (dq_ms * 1e-3) / 1e12, 2)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_pool(w, x, args.cpu_budget, dout)
    print(json.dumps(line), flush=True)


def measured_ceiling(torch, api, fp8: bool, stream, span_ms: float):
    """Time the MFMA-only loop (fa_mfma_ceiling: the attention kernels' matrix
    instruction, two waves per SIMD, operands toggling like random data) for
    about as long as the attention launches ran, right after them: the rate
    the chip sustains for pure matrix work at that moment."""
    out = torch.empty(api.mfma_ceiling_out_bytes() // 4, dtype=torch.float32, device="cuda")
    iters = 250 if fp8 else 500
    for _ in range(3):
        api.mfma_ceiling(out, fp8, iters, True, stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 4
    a.record(stream)
    for _ in range(n):
        api.mfma_ceiling(out, fp8, iters, True, stream)
    b.record(stream)
    torch.cuda.synchronize()
    one = a.elapsed_time(b) / n
    n = max(10, int(span_ms / max(one, 1e-3)))
    launches = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in launches:
        a.record(stream)
        api.mfma_ceiling(out, fp8, iters, True, stream)
        b.record(stream)
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(b) for a, b in launches]))
    tf = api.mfma_ceiling_flops(fp8, iters) / (t * 1e-3) / 1e12
    log(f"measured MFMA ceiling ({'fp8' if fp8 else 'bf16'}, random operands): {tf:.1f} TFLOP/s "
        f"({n} launches of {t:.3f} ms)")
    return {"tflops": round(tf, 1),
            "what": f"fa_mfma_ceiling: {'v_mfma_f32_32x32x64_f8f6f4' if fp8 else 'v_mfma_f32_32x32x16_bf16'} only, "
                    f"two waves per SIMD, toggling operands, median of {n} launches right after the timed steps"}


def ceiling_sweep(torch, api, launches: int, warm: int):
    """fa_mfma_ceiling for bf16 and fp8 with random operands, then constant
    ones: median rate over `launches` launches, after `warm` untimed ones
    that bring the clock to its steady state under that load, and the clock
    the rate implies.  Dispatch order (for counter runs): per dtype, random
    then constant, each `warm` + `launches` launches."""
    stream = torch.cuda.current_stream()
    out = torch.empty(api.mfma_ceiling_out_bytes() // 4, dtype=torch.float32, device="cuda")
    rows = []
    for fp8 in (False, True):
        iters = 250 if fp8 else 500
        per_clock = 256 * 4 * (2048 if fp8 else 1024)   # dense flops per clock of the chip
        for random in (True, False):
            for _ in range(warm):
                api.mfma_ceiling(out, fp8, iters, random, stream)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
            for a, b in ev:
                a.record(stream)
                api.mfma_ceiling(out, fp8, iters, random, stream)
                b.record(stream)
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
            tf = api.mfma_ceiling_flops(fp8, iters) / (ms * 1e-3) / 1e12
            rows.append({"mfma": "v_mfma_f32_32x32x64_f8f6f4" if fp8 else "v_mfma_f32_32x32x16_bf16",
                         "operands": "random" if random else "constant", "launch_ms": round(ms, 4),
                         "tflops": round(tf, 1), "implied_clock_ghz": round(tf * 1e12 / per_clock / 1e9, 3),
                         "nominal_peak_tflops": 5000.0 if fp8 else 2500.0})
            log(f"ceiling {rows[-1]['mfma']} {rows[-1]['operands']}: {tf:.1f} TFLOP/s, "
                f"{rows[-1]['implied_clock_ghz']} GHz implied ({launches} launches of {ms:.3f} ms)")
    print(json.dumps({"metric": "MFMA-only loop rate by operand data", "unit": "TFLOP/s", "launches": launches,
                      "warm_launches": warm, "rows": rows}), flush=True)


def issue_sweep(torch, api, launches: int, warm: int, iters: int, summary: str | None, command: str):
    """fa_issue_cost: every case (rounds of MFMAs with exponentials, e4m3
    packings and FMAs beside them, two waves per SIMD), median launch time
    over `launches` launches after `warm` untimed ones, against the
    MFMA-only case of the same matrix instruction.  With `summary`, also
    writes the table there."""
    stream = torch.cuda.current_stream()
    out = torch.empty(api.mfma_ceiling_out_bytes() // 4, dtype=torch.float32, device="cuda")
    cases = api.issue_cost_cases()
    rows = []
    for i, c in enumerate(cases):
        for _ in range(warm):
            api.issue_cost(out, i, iters, stream)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
        for a, b in ev:
            a.record(stream)
            api.issue_cost(out, i, iters, stream)
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        rows.append(dict(c, case=i, launch_ms=round(ms, 4)))
    # each case against the MFMA-only round of its own instruction (the
    # cases without matrix work against the bf16 one)
    base = {}
    for r in rows:
        if r["mfmas"] > 0 and r["exps"] == r["cvts"] == r["fmas"] == 0:
            base.setdefault(r["mfma"], r["launch_ms"])
    for r in rows:
        ref = base[r["mfma"]] if r["mfmas"] > 0 else base["bf16"]
        r["vs_mfma_only"] = round(r["launch_ms"] / ref, 3)
        log(f"issue cost case {r['case']}: {r['mfmas']} {r['mfma']} MFMA, {r['exps']} exp, {r['cvts']} e4m3 "
            f"packings, {r['fmas']} FMA per round: {r['launch_ms']:.4f} ms ({r['vs_mfma_only']:.3f} x MFMA only)")
    line = {"metric": "issue cost of vector work beside MFMA", "unit": "ms per launch", "iters": iters,
            "launches": launches, "warm_launches": warm, "rows": rows}
    print(json.dumps(line), flush=True)
    if summary:
        with open(summary, "w") as f:
            f.write("# fa_issue_cost: rounds of MFMAs (random operands; bf16 = v_mfma_f32_32x32x16_bf16,\n"
                    "# fp8 = v_mfma_f32_32x32x64_f8f6f4 on e4m3, fp8_scaled = the same with E8M0 scale operands,\n"
                    "# fp8_alternating = the two e4m3 forms in turn) with v_exp_f32, v_cvt_pk_fp8_f32 and\n"
                    "# v_fma_f32 beside them, per wave, two waves per SIMD on every CU; each case against the\n"
                    "# MFMA-only case of the same instruction (cases without MFMAs against the bf16 one);\n"
                    f"# median launch time of {launches} launches after {warm} untimed ones, {iters} rounds per wave\n"
                    f"# command (from the repository root on the MI355X box):\n#   {command}\n")
            f.write("case  mfmas  mfma             exps  cvts  fmas  launch_ms  vs_mfma_only\n")
            for r in rows:
                f.write(f"{r['case']:4d}  {r['mfmas']:5d}  {r['mfma']:15s}  {r['exps']:4d}  {r['cvts']:4d}  "
                        f"{r['fmas']:4d}  {r['launch_ms']:9.4f}  {r['vs_mfma_only']:12.3f}\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cold-start", type=int, default=0, metavar="N",
                    help="time N launches one by one right after setup (no prewarm, no warmup), print them, exit")
    ap.add_argument("--prewarm-ms", type=float, default=250.0,
                    help="untimed steps for at least this long (wall time) before the warmup steps, so that the "
                         "GPU's clocks have left their idle state")
    ap.add_argument("--config", default="3", help="standing workload 1..5, decode or backward")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--check", action="store_true", help="compare sampled rows with the oracle (stderr)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the measured MFMA ceiling (profiling runs)")
    ap.add_argument("--no-compare", action="store_true",
                    help="decode: skip the comparison run without the key split (profiling runs)")
    ap.add_argument("--exp2-emulated", type=int, default=0, choices=(0, 1, 2),
                    help="time fa_fwd_exp2_emulated with 1 or 2 of every 4 exponentials on the FMA pipe "
                         "(bf16, d = 64 or 128) instead of fa_fwd")
    ap.add_argument("--ceiling-sweep", action="store_true",
                    help="measure only the MFMA-only loop, random against constant operands (see above)")
    ap.add_argument("--issue-sweep", action="store_true",
                    help="measure only fa_issue_cost (vector work beside MFMA) and exit")
    ap.add_argument("--issue-summary", default=None, help="with --issue-sweep: write the table to this file")
    ap.add_argument("--sweep-launches", type=int, default=60)
    ap.add_argument("--sweep-warm", type=int, default=600, help="untimed launches before each case")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one 1 GiB device copy (reference for rocprofv3 byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_attention_07_amd import api, gen

    if args.ceiling_sweep:
        ceiling_sweep(torch, api, args.sweep_launches, args.sweep_warm)
        return
    if args.issue_sweep:
        issue_sweep(torch, api, args.sweep_launches, min(args.sweep_warm, 200), 4000, args.issue_summary,
                    "python3 " + " ".join(sys.argv))
        return
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
            api.fa_fp8_prepare(q, k, v, q8, k8, v8t, descale, amax_ws, signs, w.softmax_scale, stream)

        def attend():
            api.fa_fwd_fp8(q8, k8, v8t, descale, o, lse, w.causal, stream)
    elif args.exp2_emulated:
        if w.dtype != "bf16" or w.d not in (64, 128):
            raise SystemExit("--exp2-emulated needs a bf16 workload with d = 64 or 128")

        def prepare():
            pass

        def attend():
            api.fa_fwd_exp2_emulated(q, k, v, o, lse, w.softmax_scale, w.causal, args.exp2_emulated, stream)
    else:
        fwd = api.fa_fwd if w.dtype == "bf16" else api.fa_fwd_f32

        def prepare():
            pass

        def attend():
            fwd(q, k, v, o, lse, w.softmax_scale, w.causal, stream)

    if args.cold_start:
        cold_start_trace(torch, stream, lambda: (prepare(), attend()), args.cold_start, w.flops())
        return
    prewarm_steps = prewarm(torch, lambda: (prepare(), attend()), args.prewarm_ms)
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
    launch_ms = [a.elapsed_time(b) for a, b in marks]
    kernel_ms = sum(launch_ms) / args.steps
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

    if decode and not args.no_compare:
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
    if decode:
        nbytes = 2 * (q.numel() + k.numel() + v.numel() + o.numel()) + 4 * lse.numel()
        gbs = nbytes / (ms * 1e-3) / 1e9
        log(f"key split: {ws_bytes / 4 / (w.B * w.Hq * w.Nq * (w.d + 1)):.0f} ranges, {gbs:.0f} GB/s")
        line = {
            "metric": "attention decode step HBM GB/s (bf16, GQA, Nq=1, Nk=32K, d=128)",
            "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "prewarm": {"ms": args.prewarm_ms, "steps": prewarm_steps},
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic (seeded N(0,1), resident in HBM before timing)",
            "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                       "causal": w.causal, "path": "fa_fwd_splitkv (attention kernel over key ranges + merge)"},
            # achieved: algorithmic bytes over the whole step (attention kernel
            # over the key ranges + the merge, one library call); traffic: HBM
            # bytes of the attention kernel (rocprofv3 counters)
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                         "frac": round(gbs / 8000.0, 4), "traffic": load_traffic("decode", "bf16", load_counters("decode")),
                         "step_ms": round(ms, 5), "call_ms": round(kernel_ms, 5), "tflops": round(tflops, 2)},
        }
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_pool(w, x, args.cpu_budget, bytes_total=nbytes)
        print(json.dumps(line), flush=True)
        return

    peak = PEAK_TFLOPS[w.dtype]
    # the counter summaries describe fa_fwd's kernels, not the emulated variant
    counters = None if args.exp2_emulated else load_counters(args.config)
    traffic = None if args.exp2_emulated else load_traffic(f"config{args.config}", w.dtype, counters)
    ceiling = None if args.no_ceiling else measured_ceiling(torch, api, w.dtype == "fp8", stream,
                                                            args.steps * kernel_ms)
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
        "prewarm": {"ms": args.prewarm_ms, "steps": prewarm_steps},
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": data,
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "kernel": {"bf16": "fa_fwd_bf16_kernel", "f32": "fa_fwd_f32_kernel", "fp8": "fa_fwd_fp8_kernel"}[w.dtype]},
        "roofline": {"bound": "mfma", "achieved": round(kernel_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(kernel_tflops / peak, 4), "traffic": traffic,
                     "kernel_ms": round(kernel_ms, 5),
                     "kernel_ms_median": round(float(np.median(launch_ms)), 5),
                     "kernel_ms_min": round(float(np.min(launch_ms)), 5), "launches": len(launch_ms)},
    }
    if traffic:
        # the HBM bytes the counters saw per launch over this run's launch time,
        # against the 8 TB/s of HBM3E (the kernel is matrix-bound; this shows by how far)
        hbm_gbs = traffic / (kernel_ms * 1e-3) / 1e9
        line["roofline"].update({"hbm_gbs": round(hbm_gbs, 1), "hbm_frac": round(hbm_gbs / 8000.0, 4)})
    if counters:
        # the same kernel under rocprofv3 counters: the clock it sustains and
        # the share of SIMD cycles its matrix pipe was busy
        clk = float(counters.get("sustained_clock_ghz", "nan"))
        if not clk <= NOMINAL_CLOCK_GHZ:
            clk = float("nan")  # the counter spanned more than the kernel: no clock (see the summary)
        peak_clk = peak * clk / NOMINAL_CLOCK_GHZ
        line["roofline"].update({
            "sustained_clock_ghz": None if clk != clk else round(clk, 4),
            "mfma_busy": float(counters.get("mfma_busy", "nan")),
            "peak_at_sustained_clock": None if clk != clk else round(peak_clk, 1),
            "frac_at_sustained_clock": None if clk != clk else round(kernel_tflops / peak_clk, 4),
            "lds_bank_conflict_rate": float(counters.get("lds_bank_conflict_rate", "nan")),
            "valu_insts_per_mfma": float(counters.get("valu_insts_per_mfma", "nan")),
            "trans_share_of_valu": float(counters.get("trans_share", "nan")),
            "counters": "profiles/" + profsum.summary_name(args.config)})
    if ceiling:
        line["roofline"].update({"measured_mfma_ceiling": ceiling["tflops"],
                                 "frac_of_measured_ceiling": round(kernel_tflops / ceiling["tflops"], 4),
                                 "ceiling_measurement": ceiling["what"]})
    if args.exp2_emulated:
        line["config"]["entry_point"] = (f"fa_fwd_exp2_emulated: {args.exp2_emulated} of every 4 exponentials "
                                         "on the FMA pipe")
    if w.dtype == "fp8":
        line["config"]["steps_in_a_step"] = "fa_fp8_prepare (rotation, scales, e4m3) + fa_fwd_fp8"
        line["prepare_ms"] = round(ms - kernel_ms, 5)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_pool(w, x, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
