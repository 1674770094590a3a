"""The counter summaries bench.py reads (exact_attention_07_amd/profsum.py),
on synthetic rocprofv3 counter files: the derived quantities follow their
definitions, the copy calibration scales the byte counters, a summary is
used only while the kernel sources it names are unchanged, and the ceiling
summary splits its dispatches into the random and constant cases."""
import csv
import os

import pytest

from exact_attention_07_amd import profsum

FIELDS = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Counter_Name", "Counter_Value"]


def write_pass(d, dispatches):
    """dispatches: list of (id, kernel name, ns, {counter: value})."""
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    with open(os.path.join(d, "host", "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        t = 1000
        for did, name, ns, counters in dispatches:
            for cname, val in counters.items():
                w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Start_Timestamp": t,
                            "End_Timestamp": t + ns, "Counter_Name": cname, "Counter_Value": val})
            t += ns + 100


def fields_of(path):
    out = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def test_summary_quantities(tmp_path):
    k = "void fa::fa_fwd_bf16_kernel<128, true, 8, 0>(...)"
    ns = 1_000_000
    clk = 1.7  # GHz
    grbm = clk * ns * profsum.N_XCD          # GRBM_GUI_ACTIVE sums the XCDs' busy clocks
    busy_cycles = 0.6 * clk * ns * 4 * profsum.N_CU
    a = str(tmp_path / "a")
    write_pass(a, [(1, k, ns, {"GRBM_GUI_ACTIVE": grbm, "SQ_VALU_MFMA_BUSY_CYCLES": busy_cycles,
                               "SQ_INSTS_VALU_MFMA_MOPS_BF16": 2.0e9, "SQ_INSTS_VALU": 5e8, "SQ_INSTS_MFMA": 1e8}),
                   (2, "other_kernel", 10, {"GRBM_GUI_ACTIVE": 1.0})])
    b = str(tmp_path / "b")
    write_pass(b, [(1, k, ns, {"SQ_INSTS_VALU_TRANS_F32": 1e8, "SQ_ACTIVE_INST_LDS": 1000.0,
                               "SQ_LDS_BANK_CONFLICT": 10.0})])
    # fetch / write passes with the 1 GiB copy: FETCH counts half the bytes
    f = str(tmp_path / "f")
    write_pass(f, [(1, k, ns, {"FETCH_SIZE": 100_000.0}),
                   (2, "__amd_rocclr_copyBuffer", 5, {"FETCH_SIZE": profsum.COPY_BYTES / 2 / 1024})])
    wdir = str(tmp_path / "w")
    write_pass(wdir, [(1, k, ns, {"WRITE_SIZE": 50_000.0}),
                      (2, "__amd_rocclr_copyBuffer", 5, {"WRITE_SIZE": profsum.COPY_BYTES / 1024})])
    out = str(tmp_path / "s.txt")
    profsum.summarize(3, [a, b, f, wdir], ["cmd a", "cmd b", "cmd f", "cmd w"], out)
    s = fields_of(out)
    assert s["kernel"] == "fa_fwd_bf16_kernel"
    assert abs(float(s["sustained_clock_ghz"]) - clk) < 1e-4
    assert abs(float(s["mfma_busy"]) - 0.6) < 1e-4
    assert abs(float(s["mfma_flops_executed"]) - 512 * 2.0e9) / (512 * 2.0e9) < 1e-3
    assert abs(float(s["valu_insts_per_mfma"]) - 4.0) < 1e-3
    assert abs(float(s["trans_share"]) - 0.25) < 1e-4
    assert abs(float(s["lds_bank_conflict_rate"]) - 0.01) < 1e-6
    assert abs(float(s["fetch_scale"]) - 2.0) < 1e-4 and abs(float(s["write_scale"]) - 1.0) < 1e-4
    assert int(s["hbm_bytes_per_launch"]) == 2 * 100_000 * 1024 + 50_000 * 1024
    assert s["kernel_source_sha256"] == profsum.source_hash("bf16")
    assert "sustained_clock_note" not in s


def test_impossible_clock_is_flagged(tmp_path):
    k = "fa_fwd_bf16_kernel<64, true, 4, 0>"
    a = str(tmp_path / "a")
    write_pass(a, [(1, k, 1000, {"GRBM_GUI_ACTIVE": 3.0 * 1000 * profsum.N_XCD})])
    out = str(tmp_path / "s.txt")
    profsum.summarize(2, [a], ["cmd"], out)
    assert "sustained_clock_note" in fields_of(out)


def test_summary_is_used_only_for_the_sources_it_names(tmp_path, monkeypatch):
    os.makedirs(tmp_path / "profiles")
    path = tmp_path / "profiles" / profsum.summary_name(5)
    path.write_text(f"mfma_busy: 0.4\nkernel_source_sha256: {profsum.source_hash('fp8')}\n")
    assert profsum.load(5, root=str(tmp_path))["mfma_busy"] == "0.4"
    path.write_text("mfma_busy: 0.4\nkernel_source_sha256: 0123456789abcdef\n")
    assert profsum.load(5, root=str(tmp_path)) is None
    assert profsum.load(4, root=str(tmp_path)) is None       # no summary at all
    assert profsum.summary_name("decode") == "counters_decode.txt"


def test_ceiling_summary_splits_random_and_constant(tmp_path):
    warm, launches = 3, 4
    rows, did = [], 1
    for name, clocks in (("mfma_loop_kernel<false>(float*, int, int)", (1.9, 2.4)),
                         ("mfma_loop_kernel<true>(float*, int, int)", (2.2, 2.4))):
        for clk in clocks:
            for i in range(warm + launches):
                c = 1.0 if i < warm else clk   # warm-up launches at another clock
                rows.append((did, name, 1000, {"GRBM_GUI_ACTIVE": c * 1000 * profsum.N_XCD,
                                               "SQ_VALU_MFMA_BUSY_CYCLES": 0.9 * c * 1000 * 4 * profsum.N_CU}))
                did += 1
    a = str(tmp_path / "a")
    write_pass(a, rows)
    out = str(tmp_path / "c.txt")
    profsum.summarize_ceiling([a], ["cmd"], out, launches, warm)
    s = fields_of(out)
    assert abs(float(s["bf16_random_clock_ghz"]) - 1.9) < 1e-4
    assert abs(float(s["bf16_constant_clock_ghz"]) - 2.4) < 1e-4
    assert abs(float(s["fp8_random_clock_ghz"]) - 2.2) < 1e-4
    assert abs(float(s["fp8_random_mfma_busy"]) - 0.9) < 1e-4
    with pytest.raises(SystemExit):
        profsum.summarize_ceiling([a], ["cmd"], out, launches + 1, warm)


def test_cold_start_summary_lists_each_early_launch_and_averages_the_rest(tmp_path):
    k = "void fa::fa_fwd_bf16_kernel<128, true, 8, 0>(...)"
    d = str(tmp_path / "c")
    # 50 launches: the clock dips on launches 3-5, then holds 1.8 GHz; each
    # launch's duration follows from a fixed cycle count at its clock
    clocks = [1.75, 1.73, 1.45, 1.5, 1.6] + [1.8] * 45
    cycles = 1.7e6
    disp = []
    for i, c in enumerate(clocks):
        ns = int(round(cycles / c))
        disp.append((i + 1, k, ns, {"GRBM_GUI_ACTIVE": c * ns * profsum.N_XCD}))
    disp.append((99, "other_kernel", 10, {"GRBM_GUI_ACTIVE": 1.0}))
    write_pass(d, disp)
    out = str(tmp_path / "cold.txt")
    profsum.summarize_cold_start([d], ["cmd"], out, first=10)
    lines = [l for l in open(out) if not l.startswith("#")]
    rows = [l.split() for l in lines[1:11]]
    assert [int(r[0]) for r in rows] == list(range(1, 11))
    assert [float(r[2]) for r in rows] == pytest.approx(clocks[:10], abs=2e-3)
    assert float(rows[2][1]) == pytest.approx(cycles / 1.45 * 1e-6, rel=1e-3)
    assert "launches 11-50" in lines[11] and "1.800 GHz" in lines[11]
    assert fields_of(out)["kernel_source_sha256"] == profsum.source_hash("bf16")
