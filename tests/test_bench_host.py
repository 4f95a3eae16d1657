"""Host logic of bench.py: the attribution of rocprofv3 counter rows to the
benchmark's launches and the copy calibration (no GPU; synthetic CSVs)."""

import csv
import json

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id",
          "Thread_Id", "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size",
          "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
          "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
          "End_Timestamp"]

PREP64 = "_ZN3gdn14prepare_kernelILi64EDF16bLb0EEEvPKT0_S3_PKfS5_PfiiiiNS_6QkArgsE"
PREP64G = "void gdn::prepare_kernel<64, bool _Accum, bool, E>(bool _Accum const*)"
SCAN64 = "_ZN3gdn11scan_kernelILi64EDF16bDF16bLi4ELi1ELb0EEEvPKT0_S3_S3_PKfPT1_PfS5_iiiiiS8_"
PREP128 = "_ZN3gdn14prepare_kernelILi128EDF16bLb0EEEvPKT0_S3_PKfS5_PfiiiiNS_6QkArgsE"
SCAN128 = "_ZN3gdn11scan_kernelILi128EDF16bDF16bLi4ELi1ELb0EEEvPKT0_S3_S3_PKfPT1_PfS5_iiiiiS8_"
# the state-storing instance the backward pass launches at the same grid
SCAN128_ST = "_ZN3gdn11scan_kernelILi128EDF16bDF16bLi4ELi1ELb1EEEvPKT0_S3_S3_PKfPT1_PfS5_iiiiiS8_"
DEC64 = "_ZN3gdn13decode_kernelILi64ELi4EDF16bDF16bLi0EEEvPKT1_S3_S3_PKfS5_S5_PfPT2_iiiiNS_6QkArgsE"


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for i, (name, grid, val) in enumerate(rows, 1):
            r = {k: 0 for k in FIELDS}
            r.update(Dispatch_Id=i, Grid_Size=grid, Kernel_Name=name,
                     Counter_Name=counter, Counter_Value=val)
            w.writerow(r)


def args(**kw):
    a = bench.main.__globals__["argparse"].Namespace(
        skip_prefill=True, skip_decode=True, skip_batched=True, skip_qk=True,
        skip_gated=True, skip_backward=True, qk_gather_only=False, decode_batch=[64, 1])
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_kernel_keys():
    assert bench._kernel_key("_ZN3gdn15backward_kernelILi128ELi2EDF16bEEvPKT1_S3_S3_PKfS5_") == (
        "backward_kernel", 128, 2)
    assert bench._kernel_key("void gdn::backward_reduce_kernel<128>(float const*, float*)") == (
        "backward_reduce_kernel", 128, None)
    assert bench._kernel_key(PREP64) == ("prepare_kernel", 64, 0)
    assert bench._kernel_key(PREP64G) == ("prepare_kernel", 64, None)
    assert bench._kernel_key(DEC64) == ("decode_kernel", 64, 0)
    assert bench._kernel_key("void gdn::prepare_kernel<128, __bf16, true>(int)") == (
        "prepare_kernel", 128, 1)
    assert bench._kernel_key("__amd_rocclr_copyBuffer")[0] == "__amd_rocclr_copyBuffer"
    # prepare_kernel<dk, type, gather, no-P>: keyed by the gather flag
    assert bench._kernel_key(
        "_ZN3gdn14prepare_kernelILi128EDF16bLb0ELb1EEEvPKT0_S3_PKfS5_PfiiiiNS_6QkArgsE") == (
        "prepare_kernel", 128, 0)
    assert bench._kernel_key(
        "_ZN3gdn14prepare_kernelILi64EDF16bLb1ELb0EEEvPKT0_S3_PKfS5_PfiiiiNS_6QkArgsE") == (
        "prepare_kernel", 64, 1)
    assert bench._kernel_key("void gdn::prepare_kernel<64, __bf16, true, false>(int)") == (
        "prepare_kernel", 64, 1)


def test_counters_attribution_and_calibration(tmp_path):
    # an upload copy, two batched dk=64 launches, a decode prompt's prepare
    # (other grid: not counted), then the 23 calibration copies of 512 MiB
    # that read as half their bytes (FETCH) and as all of them (WRITE)
    g_prep, g_scan = 64 * 16 * 8 * 64, 8 * 16 * 2 * 256
    common = [("__amd_rocclr_copyBuffer", 131072, 1000.0),
              (PREP128, g_prep, 7.0), (SCAN128, g_scan, 9.0),
              (PREP64, g_prep, None), (SCAN64, g_scan, None),
              (PREP64, g_prep, None), (SCAN64, g_scan, None),
              (PREP64, 2097152, None)]
    fetch = [(n, g, v if v is not None else {PREP64: 100.0, SCAN64: 300.0}[n])
             for n, g, v in common] + [("__amd_rocclr_copyBuffer", 131072, 262144.0)] * 23
    write = [(n, g, v if v is not None else {PREP64: 50.0, SCAN64: 70.0}[n])
             for n, g, v in common] + [("__amd_rocclr_copyBuffer", 131072, 524288.0)] * 23
    fetch[7] = (PREP64, 2097152, 9e9)               # the prompt's prepare must not count
    write[7] = (PREP64, 2097152, 9e9)
    fetch.insert(8, (SCAN128_ST, g_scan, 9e9))      # nor a state-storing scan
    write.insert(8, (SCAN128_ST, g_scan, 9e9))
    write_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    write_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    bench.summarize_counters(args(skip_batched=False), str(tmp_path / "f.csv"),
                             str(tmp_path / "w.csv"), out_path=str(out))
    d = json.loads(out.read_text())
    assert d["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert d["calibration"]["write_factor"] == pytest.approx(1.0)
    e = d["kernels"]["batched_dk64"]
    assert e["parts"]["prepare_kernel"]["dispatches"] == 2
    assert e["hbm_bytes_per_launch"] == pytest.approx((100 * 2 + 50 + 300 * 2 + 70) * 1024)
    assert d["kernels"]["batched_dk128"]["hbm_bytes_per_launch"] == pytest.approx(
        (7 * 2 + 7 + 9 * 2 + 9) * 1024)
    assert d["source_hash"] == bench.kernel_source_hash()


def test_counters_refuse_pooled_legs(tmp_path):
    write_csv(tmp_path / "f.csv", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1, 1.0)])
    write_csv(tmp_path / "w.csv", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1, 1.0)])
    # the plain and the fused norm-only batched legs launch the same kernels
    with pytest.raises(SystemExit):
        bench.summarize_counters(args(skip_batched=False, skip_qk=False),
                                 str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                 out_path=str(tmp_path / "t.json"))


def test_trace_legs_split_in_run_order(tmp_path, capsys):
    # three legs launch prepare_kernel<64, 0> at one grid, in the order the
    # benchmark runs them (plain batched, the norm-only input path, then the
    # backward pass), seconds apart, with the gathering input path's
    # prepare_kernel<64, 1> between the first two; the backward's
    # state-storing scan must not be taken for the forward scan of the
    # batched legs
    import sqlite3
    SCAN64_ST = SCAN64.replace("Lb0E", "Lb1E")
    PREP64_G = PREP64.replace("Lb0E", "Lb1E")
    db = tmp_path / "t.db"
    con = sqlite3.connect(db)
    con.execute("create table rocpd_info_kernel_symbol (id integer, kernel_name text)")
    con.execute("create table rocpd_kernel_dispatch (kernel_id integer, grid_size_x integer, "
                "grid_size_y integer, grid_size_z integer, start integer, end integer)")
    for i, n in enumerate((PREP64, SCAN64, SCAN64_ST, PREP64_G)):
        con.execute("insert into rocpd_info_kernel_symbol values (?, ?)", (i, n))
    g_prep, g_scan = 64 * 16 * 8 * 64, 8 * 16 * 2 * 256
    t = 0
    # (dispatch pairs, prepare kernel id, prepare us, scan kernel id, scan
    # us) per leg in run order
    for npair, prep_id, prep_us, scan_id, scan_us in ((5, 0, 60, 1, 180), (2, 3, 140, 1, 185),
                                                       (4, 0, 70, 1, 190), (3, 0, 95, 2, 210)):
        for _ in range(npair):
            con.execute("insert into rocpd_kernel_dispatch values (?, ?, 1, 1, ?, ?)",
                        (prep_id, g_prep, t, t + prep_us * 1000))
            t += prep_us * 1000 + 1000
            con.execute("insert into rocpd_kernel_dispatch values (?, ?, 1, 1, ?, ?)",
                        (scan_id, g_scan, t, t + scan_us * 1000))
            t += scan_us * 1000 + 1000
        t += 5 * 10**9
    con.commit()
    con.close()
    bench.summarize_trace(args(skip_qk=False, skip_backward=False, skip_batched=False,
                               decode_batch=[1]), str(db))
    rows = {}
    for line in capsys.readouterr().out.splitlines()[2:]:
        c = [x.strip() for x in line.split("|")]
        rows[(c[1], c[2])] = (int(c[4]), float(c[5]))
    assert rows[("batched_dk64", "prepare_kernel<64, 0>")] == (5, 60.0)
    assert rows[("batched_dk64", "scan_kernel<64, 0>")] == (5, 180.0)
    assert rows[("batched_qk_dk64", "prepare_kernel<64, 1>")] == (2, 140.0)
    assert rows[("batched_qk_dk64", "scan_kernel<64, 0>")] == (2, 185.0)
    assert rows[("batched_qk_norm_dk64", "prepare_kernel<64, 0>")] == (4, 70.0)
    assert rows[("batched_qk_norm_dk64", "scan_kernel<64, 0>")] == (4, 190.0)
    assert rows[("backward_B8_T4096_dk64", "prepare_kernel<64, 0>")] == (3, 95.0)
    assert rows[("backward_B8_T4096_dk64", "scan_kernel<64, 1>")] == (3, 210.0)
