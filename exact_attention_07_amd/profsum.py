"""Summaries of rocprofv3 counter runs of the attention kernels.

    python -m exact_attention_07_amd.profsum --config 3 --out profiles/counters_config3.txt \\
        --cmd "<command of pass 1>" ... DIR [DIR ...]

Each DIR is the output directory of one `rocprofv3 --pmc ... --output-format
csv` run of `bench.py --config N` (one counter pass).  The summary averages
every counter over the dispatches of the workload's attention kernel, derives
the quantities the measurement reports, and records the sha256 of the
kernel's sources, so that bench.py uses it only while it describes the
current code:

  sustained_clock_ghz   GRBM_GUI_ACTIVE / 8 XCDs / kernel duration (the
                        counter sums the busy clocks of the 8 XCDs)
  mfma_busy             SQ_VALU_MFMA_BUSY_CYCLES / (clocks * 4 SIMDs * CUs):
                        the share of SIMD cycles the matrix pipe was busy
  mfma_flops_executed   512 * SQ_INSTS_VALU_MFMA_MOPS_* (one MOP = 512 flops)
  mfma_peak_at_clock    CUs * 4 SIMDs * flops per clock per SIMD (1024 bf16,
                        2048 fp8) * sustained clock
  trans_share           SQ_INSTS_VALU_TRANS_F32 / non-matrix VALU instructions
  lds_bank_conflict_rate SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS (cycles)
  hbm_bytes_per_launch  FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
                        scaled by true bytes / counted bytes of the 1 GiB
                        device copy bench.py --copy-calibration runs

Measurement tooling: it reads profiler output only and computes nothing of
the attention.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_CSRC = "exact_attention_07_amd/csrc/"
# sources of the attention kernel of each dtype
KERNEL_SOURCES = {
    "bf16": [_CSRC + f for f in ("fa_fwd.hip", "fa_frag.h", "fa_device.h", "plan.h", "fa_exp2.h", "fa_exp2_coef.h")],
    "f32": [_CSRC + f for f in ("fa_fwd.hip", "fa_frag.h", "fa_device.h", "plan.h", "fa_exp2.h", "fa_exp2_coef.h")],
    "fp8": [_CSRC + f for f in ("fa_fwd_fp8.hip", "fa_device.h", "plan.h")],
    "bwd": [_CSRC + f for f in ("fa_bwd.hip", "fa_frag.h", "fa_device.h", "plan.h")],
    "ceiling": [_CSRC + "fa_ceiling.hip"],
}
KERNEL_NAME = {"bf16": "fa_fwd_bf16_kernel", "f32": "fa_fwd_f32_kernel", "fp8": "fa_fwd_fp8_kernel",
               "bwd": "fa_bwd_dkdv_kernel"}
CONFIG_DTYPE = {1: "f32", 2: "bf16", 3: "bf16", 4: "bf16", 5: "fp8", "decode": "bf16", "backward": "bwd"}
N_XCD = 8
N_CU = 256
COPY_BYTES = 1 << 30


def source_hash(dtype: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[dtype]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _dispatch_counters(path: str, name_part: str):
    """{dispatch id: {counter: value, "_ns": duration}} of the dispatches whose
    kernel name contains name_part, summed over the counter's dimensions."""
    out = {}
    for r in csv.DictReader(open(path)):
        if name_part not in r["Kernel_Name"]:
            continue
        d = out.setdefault(r["Dispatch_Id"], {"_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _mean(rows, key):
    vals = [r[key] for r in rows if key in r]
    return sum(vals) / len(vals) if vals else None


def summarize(config, dirs, commands, out_path):
    dtype = CONFIG_DTYPE[config]
    kname = KERNEL_NAME[dtype]
    fields = {}
    copy = {}
    durations = []
    clocks = []
    busy = None
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        rows = list(_dispatch_counters(files[0], kname).values())
        if not rows:
            raise SystemExit(f"no dispatch of {kname} in {files[0]}")
        for key in rows[0]:
            if key != "_ns":
                fields[key] = _mean(rows, key)
        durations += [r["_ns"] for r in rows]
        # clock and matrix-pipe share from the dispatches of the same pass
        if "GRBM_GUI_ACTIVE" in rows[0]:
            clocks += [r["GRBM_GUI_ACTIVE"] / N_XCD / r["_ns"] for r in rows]
            if "SQ_VALU_MFMA_BUSY_CYCLES" in rows[0]:
                busy = sum(r["SQ_VALU_MFMA_BUSY_CYCLES"] / (r["GRBM_GUI_ACTIVE"] / N_XCD * 4 * N_CU)
                           for r in rows) / len(rows)
        for r in _dispatch_counters(files[0], "copyBuffer").values():
            for key in ("FETCH_SIZE", "WRITE_SIZE"):
                if key in r:
                    copy[key] = r[key]
    ns = sum(durations) / len(durations)
    lines = [f"# rocprofv3 counters of {kname}: workload config {config}",
             "# commands (from the repository root on the MI355X box), one counter pass each:"]
    lines += [f"#   {c}" for c in commands]
    lines += ["# values: mean per dispatch of the attention kernel over the profiled launches",
              f"kernel: {kname}", f"dispatches_per_pass: {len(durations) // max(1, len(dirs))}",
              f"kernel_ns_under_counters: {ns:.0f}"]
    for key in sorted(fields):
        lines.append(f"{key}: {fields[key]:.0f}")
    if clocks:
        clk = sum(clocks) / len(clocks)  # GHz
        lines.append(f"sustained_clock_ghz: {clk:.4f}")
        if clk > 2.4:
            # above the chip's maximum: the counter spans more than the
            # kernel's own duration (short or memory-bound launches), so this
            # is no clock
            lines.append("sustained_clock_note: above the 2.4 GHz maximum, not a clock (GRBM_GUI_ACTIVE spans "
                         "more than this kernel's duration)")
        per_simd = 1024.0 * (2 if dtype == "fp8" else 1)
        lines.append(f"mfma_peak_at_clock_tflops: {N_CU * 4 * per_simd * clk * 1e9 / 1e12:.1f}")
    if busy is not None:
        lines.append(f"mfma_busy: {busy:.4f}")
    mops = fields.get("SQ_INSTS_VALU_MFMA_MOPS_F8" if dtype == "fp8" else "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    if mops:
        lines.append(f"mfma_flops_executed: {512.0 * mops:.4e}")
        lines.append(f"mfma_tflops_executed_under_counters: {512.0 * mops / ns / 1e3:.1f}")
    valu, mfma, trans = (fields.get(k) for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_TRANS_F32"))
    if valu and mfma and trans is not None:
        lines.append(f"valu_insts_per_mfma: {(valu - mfma) / mfma:.3f}")
        lines.append(f"trans_share: {trans / (valu - mfma):.4f}")
    if fields.get("SQ_ACTIVE_INST_LDS"):
        lines.append(f"lds_bank_conflict_rate: {fields.get('SQ_LDS_BANK_CONFLICT', 0.0) / fields['SQ_ACTIVE_INST_LDS']:.5f}")
    if "FETCH_SIZE" in fields and "WRITE_SIZE" in fields and "FETCH_SIZE" in copy and "WRITE_SIZE" in copy:
        fs = COPY_BYTES / (copy["FETCH_SIZE"] * 1024.0)
        ws = COPY_BYTES / (copy["WRITE_SIZE"] * 1024.0)
        fb = fields["FETCH_SIZE"] * 1024.0 * fs
        wb = fields["WRITE_SIZE"] * 1024.0 * ws
        lines += [f"copy_fetch_kib_raw: {copy['FETCH_SIZE']:.1f}", f"copy_write_kib_raw: {copy['WRITE_SIZE']:.1f}",
                  f"fetch_scale: {fs:.4f}", f"write_scale: {ws:.4f}",
                  f"fetch_bytes_per_launch: {fb:.0f}", f"write_bytes_per_launch: {wb:.0f}",
                  f"hbm_bytes_per_launch: {fb + wb:.0f}"]
    lines.append(f"kernel_source_sha256: {source_hash(dtype)}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_path


def summarize_ceiling(dirs, commands, out_path, launches, warm):
    """Counters of a `bench.py --ceiling-sweep` run: per MFMA loop (bf16,
    fp8) and operand data (random, then constant, in dispatch order; each
    `warm` untimed + `launches` timed launches), the mean clock and
    matrix-pipe share over the timed launches."""
    groups = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        disp = _dispatch_counters(files[0], "mfma_loop_kernel")
        for did in sorted(disp, key=int):
            r = disp[did]
            name = "fp8" if "<true>" in _kernel_name(files[0], did) else "bf16"
            groups.setdefault((d, name), []).append(r)
    lines = ["# rocprofv3 counters of fa_mfma_ceiling (MFMA-only loops, two waves per SIMD):",
             "# random operands, then constant ones (bf16: 0.5 and 0.25; fp8: 1.0 in every byte)",
             "# commands (from the repository root on the MI355X box), one counter pass each:"]
    lines += [f"#   {c}" for c in commands]
    lines.append("# values: mean over the timed launches of each case")
    for (d, name), rows in sorted(groups.items(), key=lambda t: (t[0][1] != "bf16", t[0][0])):
        per = warm + launches
        if len(rows) != 2 * per:
            raise SystemExit(f"{d} {name}: {len(rows)} dispatches, expected {2 * per}")
        for k, what in enumerate(("random", "constant")):
            part = rows[k * per + warm:(k + 1) * per]
            ns = sum(r["_ns"] for r in part) / len(part)
            lines.append(f"{name}_{what}_kernel_ns_under_counters: {ns:.0f}")
            if "GRBM_GUI_ACTIVE" in part[0]:
                clk = sum(r["GRBM_GUI_ACTIVE"] / N_XCD / r["_ns"] for r in part) / len(part)
                lines.append(f"{name}_{what}_clock_ghz: {clk:.4f}")
                if "SQ_VALU_MFMA_BUSY_CYCLES" in part[0]:
                    busy = sum(r["SQ_VALU_MFMA_BUSY_CYCLES"] / (r["GRBM_GUI_ACTIVE"] / N_XCD * 4 * N_CU)
                               for r in part) / len(part)
                    lines.append(f"{name}_{what}_mfma_busy: {busy:.4f}")
    lines.append(f"kernel_source_sha256: {source_hash('ceiling')}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_path


def summarize_cold_start(dirs, commands, out_path, first: int = 40):
    """GRBM_GUI_ACTIVE per dispatch of a `bench.py --cold-start N` run: the
    clock (counter / 8 XCDs / duration) and duration of each of the first
    `first` dispatches of the attention kernel, then the mean over the rest."""
    files = glob.glob(os.path.join(dirs[0], "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {dirs[0]}")
    disp = _dispatch_counters(files[0], "fa_fwd_bf16_kernel")
    rows = [disp[d] for d in sorted(disp, key=int)]
    if len(rows) <= first:
        raise SystemExit(f"{len(rows)} dispatches, need more than {first}")
    lines = ["# rocprofv3 GRBM_GUI_ACTIVE of fa_fwd_bf16_kernel, launch by launch from a cold start",
             "# (no untimed launches before them), with the clock each launch ran at",
             "# (GRBM_GUI_ACTIVE / 8 XCDs / duration)",
             "# command (from the repository root on the MI355X box):"]
    lines += [f"#   {c}" for c in commands]
    lines.append("launch  ms  clock_ghz")
    for i, r in enumerate(rows[:first]):
        lines.append(f"{i + 1:4d}  {r['_ns'] * 1e-6:.4f}  {r['GRBM_GUI_ACTIVE'] / N_XCD / r['_ns']:.3f}")
    rest = rows[first:]
    ns = sum(r["_ns"] for r in rest) / len(rest)
    clk = sum(r["GRBM_GUI_ACTIVE"] / N_XCD / r["_ns"] for r in rest) / len(rest)
    lines.append(f"launches {first + 1}-{len(rows)}: mean {ns * 1e-6:.4f} ms at {clk:.3f} GHz")
    lines.append(f"kernel_source_sha256: {source_hash('bf16')}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_path


def _kernel_name(path: str, dispatch_id: str) -> str:
    for r in csv.DictReader(open(path)):
        if r["Dispatch_Id"] == dispatch_id:
            return r["Kernel_Name"]
    return ""


def summary_name(config) -> str:
    """File name of a workload's counter summary under profiles/."""
    return f"counters_config{config}.txt" if isinstance(config, int) else f"counters_{config}.txt"


def load(config, root=ROOT):
    """Fields of the workload's counter summary under profiles/ if it
    describes the current kernel sources, else None."""
    path = os.path.join(root, "profiles", summary_name(config))
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != source_hash(CONFIG_DTYPE[config]):
        return None
    return fields


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", required=True, help="workload (1..5, decode, backward), ceiling or cold_start")
    ap.add_argument("--launches", type=int, default=60, help="ceiling: timed launches per case")
    ap.add_argument("--warm", type=int, default=600, help="ceiling: untimed launches before each case")
    ap.add_argument("--out", required=True)
    ap.add_argument("--cmd", action="append", default=[], help="command of a pass (repeat, in order)")
    ap.add_argument("dirs", nargs="+")
    a = ap.parse_args(argv)
    if a.config == "ceiling":
        print(summarize_ceiling(a.dirs, a.cmd, a.out, a.launches, a.warm))
        return
    if a.config == "cold_start":
        print(summarize_cold_start(a.dirs, a.cmd, a.out))
        return
    cfg = int(a.config) if a.config.isdigit() else a.config
    print(summarize(cfg, a.dirs, a.cmd, a.out))


if __name__ == "__main__":
    sys.exit(main())
