"""Host-side logic of bench.py, on the CPU: the algorithmic byte counts
behind the roofline line, the rocprofv3 --pmc traffic summary and its
source-hash guard, and the one-GPU guard of the command line."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

MiB = 1 << 20


def test_algorithmic_bytes_of_the_main_workload():
    # q, k, v: 3 x 128 MiB (bf16); alpha, beta: 2 x 2 MiB (fp32); o: 128 MiB
    # (bf16); final state: 64 heads x 128 x 128 fp32 = 4 MiB; no initial state
    assert bench.alg_bytes_main(4, 16, 8192, 128) == (3 * 128 + 2 * 2 + 128 + 4) * MiB


def test_algorithmic_bytes_of_a_decode_step():
    # the fp32 state is read and written once (2 x 256 MiB); per head q, k, v
    # in (bf16), alpha, beta in (fp32) and o out (bf16)
    heads = 256 * 16
    per_head = 3 * 128 * 2 + 2 * 4 + 128 * 2
    assert bench.alg_bytes_decode(256, 16, 128) == 2 * 256 * MiB + heads * per_head


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "1_counter_collection.csv"), "w") as fh:
        fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, value) in enumerate(rows):
            fh.write('%d,"%s",%s,%r\n' % (i + 1, name, counter, value))


def test_pmc_summary_scales_by_the_copy_and_averages_the_last_launches(tmp_path, monkeypatch):
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    copy_kib = 512 * 1024.0
    # FETCH_SIZE reads half the copy's 512 MiB (scale 2); WRITE_SIZE reads it all
    chunk = "void gdn::pipe::chunk_fwd_pipe_kernel<false>(...)"
    early = [(chunk, 9.0e5)] * 5                      # before the clocks settle: ignored
    last_fetch = [(chunk, 2.0e5 + 1000.0 * i) for i in range(bench.PMC_LAUNCHES)]
    last_write = [(chunk, 1.3e5)] * bench.PMC_LAUNCHES
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", [("copyBuffer", copy_kib / 2)] + early + last_fetch)
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", [("copyBuffer", copy_kib)] + early + last_write)
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"))
    vals = {}
    for line in out.read_text().splitlines():
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    mean_fetch = sum(v for _, v in last_fetch) / len(last_fetch)
    assert float(vals["fetch_scale"]) == pytest.approx(2.0)
    assert float(vals["write_scale"]) == pytest.approx(1.0)
    assert int(vals["hbm_fetch_bytes"]) == int(mean_fetch * 1024 * 2)
    assert int(vals["hbm_write_bytes"]) == int(1.3e5 * 1024)
    assert vals["kernel_source_hash"] == bench.kernel_source_hash()
    # the guard: the summary counts while the kernel sources are the ones it was taken on
    assert bench.read_traffic() == int(vals["hbm_bytes_per_launch"])
    out.write_text(out.read_text().replace(vals["kernel_source_hash"], "0" * 16))
    assert bench.read_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_trace(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_kernel_trace.csv"), "w") as fh:
        fh.write("Kernel_Name,Grid_Size_X,Workgroup_Size_X,Start_Timestamp,End_Timestamp\n")
        t = 0
        for name, wgs, threads, dur in rows:
            fh.write('"%s",%d,%d,%d,%d\n' % (name, wgs * threads, threads, t, t + dur))
            t += dur + 1000


def test_trace_summary_groups_by_kernel_and_shape_and_prices_the_main_launches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    chunk = "void gdn::pipe::chunk_fwd_pipe_kernel<false, true, 4>(unsigned short const*, int)"
    rows = [(chunk, 256, 512, 300000)] * 50 + [(chunk, 256, 512, 200000)] * 100
    rows += [(chunk, 8, 512, 150000)] * 3
    rows += [("void at::native::copy_kernel(int)", 1024, 256, 5000)] * 2  # not the library's
    _write_trace(str(tmp_path / "tr"), rows)
    bench.summarize_trace(str(tmp_path / "tr"), "x", command="rocprofv3 --kernel-trace -- python3 bench.py")
    text = (tmp_path / "profiles" / "x.txt").read_text()
    assert "rocprofv3 --kernel-trace -- python3 bench.py" in text
    assert "copy_kernel" not in text
    lines = [l for l in text.splitlines() if l.startswith("gdn::pipe::chunk_fwd_pipe_kernel")]
    assert len(lines) == 2
    big = lines[0].split()[-7:]  # wgs, threads, launches, mean, min, max, tail (the name has a space)
    assert big[0:3] == ["256", "512", "150"]
    # the tail mean covers the last 100 launches only; the mean all 150
    assert float(big[-1]) == pytest.approx(200.0)
    assert float(big[3]) == pytest.approx((50 * 300 + 100 * 200) / 150.0, abs=0.01)
    frac = [l for l in text.splitlines() if "fraction_of_8000_GBps" in l][0]
    alg = bench.alg_bytes_main(4, 16, 8192, 128)
    assert float(frac.split("=")[1]) == pytest.approx(alg / 200000.0 / 8000.0, rel=1e-3)


def test_trace_summary_prices_each_decode_step_variant(tmp_path, monkeypatch):
    """The three decode steps (scalar gate, per-dimension gate, no delta rule)
    keep rows of their own, and the per-dimension gate's extra bytes count."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    step = "void gdn::recurrent_step_kernel<unsigned short, 128, 128, 512, %d>(unsigned short const*, long)"
    rows = [[(step % g, 4096, 512, 80000 + 1000 * g)] * 64 for g in (0, 1, 2)]
    _write_trace(str(tmp_path / "tr"), [r for rs in rows for r in rs])
    bench.summarize_trace(str(tmp_path / "tr"), "x", command="c", tail=64)
    text = (tmp_path / "profiles" / "x.txt").read_text()
    assert len([l for l in text.splitlines() if l.startswith("gdn::recurrent_step_kernel")]) == 3
    fr = [float(l.split("=")[1]) for l in text.splitlines() if "fraction_of_8000_GBps" in l]
    base = bench.alg_bytes_decode(256, 16, 128)
    vec = base + 256 * 16 * 127 * 4
    assert fr == pytest.approx([base / 80000.0 / 8000.0, vec / 81000.0 / 8000.0, base / 82000.0 / 8000.0],
                               rel=1e-3)
    assert "per-dimension gate" in text and "gated linear attention" in text


def test_host_info_names_the_cpu():
    info = bench.host_info()
    assert info["nproc"] >= 1 and isinstance(info["cpu_model"], str)


def test_kernel_hash_follows_code_not_comments():
    """The traffic summaries stay valid across comment edits of a kernel and
    are voided by any change of its code."""
    base = "int f(int a) {  // sum\n  return a + 1; /* one */\n}\n"
    read = lambda text: (lambda f: text)
    h0 = bench.kernel_source_hash(["x.hpp"], read(base))
    assert bench.kernel_source_hash(["x.hpp"], read(base.replace("// sum", "// the sum\n  "))) == h0
    assert bench.kernel_source_hash(["x.hpp"], read(base.replace("/* one */", ""))) == h0
    assert bench.kernel_source_hash(["x.hpp"], read(base.replace("a + 1", "a + 2"))) != h0
    # one function of a file: edits elsewhere in the file do not matter
    two = base + "int g(int b) {\n  return b;\n}\n"
    hf = bench.kernel_source_hash(["x.hip:f"], read(two))
    assert bench.kernel_source_hash(["x.hip:f"], read(two.replace("return b;", "return b * 2;"))) == hf
    assert bench.kernel_source_hash(["x.hip:f"], read(two.replace("a + 1", "a - 1"))) != hf
