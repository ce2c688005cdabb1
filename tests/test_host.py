"""Host-side logic of the measurement tools (no GPU): the code digest that
keys stored traffic measurements, and the markdown formatting of bench
output lines."""

import json

from io_aware_softmax_02_amd.profile_summary import code_digest, configs_md


def test_code_digest_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {  // one\n  return x + 1;  /* two\n lines */\n}\n")
    b.write_text("int f(int x) {\n\treturn x + 1; // another comment\n}")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert code_digest(str(a)) == code_digest(str(b))
    assert code_digest(str(a)) != code_digest(str(c))


def test_code_digest_sees_every_kernel_source_change(tmp_path):
    # a one-character change of code in a real kernel source changes the digest
    import io_aware_softmax_02_amd.profile_summary as ps
    import os
    src = os.path.join(ps.ROOT, "io_aware_softmax_02_amd", "csrc", "attn_fwd_bf16.hip")
    text = open(src, encoding="utf-8").read()
    p = tmp_path / "k.hip"
    p.write_text(text)
    d0 = code_digest(str(p))
    p.write_text(text.replace("constexpr float kSlack = 8.0f;", "constexpr float kSlack = 7.0f;"))
    assert code_digest(str(p)) != d0
    p.write_text(text + "\n// trailing comment\n")
    assert code_digest(str(p)) == d0


def test_configs_markdown(tmp_path):
    line = {"workload": "w", "B": 1, "H": 2, "N": 3, "d": 64, "dtype": "bf16", "launches": 1,
            "ms_fwd": 0.5, "ms_bwd": 1.5, "fwd_tflops": 100.0, "fwdbwd_tflops": 250.0,
            "peak_tflops": 2500.0}
    log = tmp_path / "log"
    log.write_text("noise\n" + json.dumps(line) + "\n")
    md = configs_md(str(log))
    row = [r for r in md.splitlines() if r.startswith("| `w`")]
    assert row == ["| `w` | 1, 2, 3, 64 | bf16 | 500.0 | 100.0 | 1500.0 | 250.0 | 10.0 |"]


def test_trace_markdown_average_and_median(tmp_path):
    # A kernel-trace database with the two tables the summary reads: the
    # median column is the middle per-launch duration, which stays at the
    # working-clock value when the first launches run slow after idle.
    import sqlite3
    from io_aware_softmax_02_amd.profile_summary import trace
    db = tmp_path / "t_results.db"
    con = sqlite3.connect(str(db))
    con.execute("create table kernels (name text, duration integer, lds_size integer, "
                "vgpr_count integer, accum_vgpr_count integer, sgpr_count integer, "
                "grid_x integer, workgroup_x integer)")
    durs_ns = [1500000, 1200000, 1000000, 1000000, 1000000]
    for d in durs_ns:
        con.execute("insert into kernels values ('void fa::k<128>(int)', ?, 1024, 128, 0, 32, "
                    "262144, 256)", (d,))
    con.execute("create table top_kernels (name text, total_calls integer, "
                "total_duration real, average real, percentage real)")
    con.execute("insert into top_kernels values ('void fa::k<128>(int)', 5, 5700.0, 1140.0, 100.0)")
    con.commit()
    con.close()
    md = trace(str(tmp_path / "*_results.db"), "T", "C")
    row = [r for r in md.splitlines() if r.startswith("| `k<128>`")]
    assert row == ["| `k<128>` | 5 | 5700.0 | 1140.0 | 1000.0 | 100.0 | 262144 | 256 | 1024 | 128 | 0 |"]


def test_cpu_markdown_labels_extrapolation(tmp_path):
    from io_aware_softmax_02_amd.profile_summary import cpu_md
    lines = [{"cpu_oracle": "a", "B": 1, "H": 2, "N": 8, "d": 4, "cores": 16,
              "sample": "1 of 2 heads, forward", "seconds": 1.5, "tflops": 0.25,
              "extrapolated_all_heads_seconds": 3.0},
             {"cpu_oracle": "b", "B": 1, "H": 1, "N": 9, "d": 4, "cores": 16,
              "sample": "2 sampled query rows", "seconds": 0.5, "tflops": 0.125,
              "extrapolated_full_forward_seconds": 2.25}]
    log = tmp_path / "log"
    log.write_text("\n".join(json.dumps(x) for x in lines) + "\n")
    md = cpu_md(str(log))
    assert "**extrapolation**" in md and "16 BLAS threads" in md
    rows = [r for r in md.splitlines() if r.startswith("| `")]
    assert rows == ["| `a` | 1, 2, 8, 4 | 1 of 2 heads, forward | 1.5 | 0.2500 | 3.0 |",
                    "| `b` | 1, 1, 9, 4 | 2 sampled query rows | 0.5 | 0.1250 | 2.25 |"]


def test_traffic_calibration_uses_only_the_large_copy(tmp_path):
    # Copies of tensors a few tens of MB large share the calibration copy's
    # grid; only dispatches near the largest value calibrate.
    from io_aware_softmax_02_amd.profile_summary import calibration
    rows = ["Dispatch_Id,Grid_Size,Kernel_Name,Counter_Name,Counter_Value"]
    for d, v in ((2, 262160.0), (3, 262156.0), (10, 16400.0), (11, 16399.0), (19, 1.5)):
        rows.append(f'{d},131072,"__amd_rocclr_copyBuffer",FETCH_SIZE,{v}')
    rows.append('5,262144,"fa::fwd_bf16_kernel<128>(...)",FETCH_SIZE,49232.0')
    p = tmp_path / "c.csv"
    p.write_text("\n".join(rows) + "\n")
    assert calibration(str(p), "FETCH_SIZE") == 262158.0


def test_apicalls_counts_calls_inside_the_marker_range(tmp_path):
    """The HIP-call summary counts only calls that start inside the roctx
    range fa_steps, on the range's thread, and reports allocation calls."""
    from io_aware_softmax_02_amd import profile_summary as ps
    hdr = '"Domain","Function","Process_Id","Thread_Id","Correlation_Id","Start_Timestamp","End_Timestamp"\n'
    (tmp_path / "x_marker_api_trace.csv").write_text(
        hdr + '"MARKER_CORE_RANGE_API","fa_steps",1,7,9,1000,2000\n')
    rows = [("hipMalloc", 7, 500), ("hipLaunchKernel", 7, 1100), ("hipLaunchKernel", 7, 1900),
            ("hipGetLastError", 7, 1200), ("hipLaunchKernel", 8, 1500), ("hipFree", 7, 2500),
            ("hipMemsetAsync", 7, 1300)]
    (tmp_path / "x_hip_api_trace.csv").write_text(hdr + "".join(
        f'"HIP_RUNTIME_API","{f}",1,{t},1,{s},{s + 10}\n' for f, t, s in rows))
    md = ps.apicalls(str(tmp_path), "T", "C")
    assert "| `hipLaunchKernel` | 2 |" in md and "| `hipGetLastError` | 1 |" in md
    assert "hipMalloc" not in md and "hipFree" not in md
    assert "Allocation, free, memset or copy calls inside the range: 1 ({'hipMemsetAsync': 1})." in md
    assert "HIP calls on other threads inside the range: 1." in md
