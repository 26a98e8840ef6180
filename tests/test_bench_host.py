"""Host-side checks of bench.py (no GPU): the one-GPU refusal and the kernel code hash
that ties a counter summary under profiles/ to the kernel it measured."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_kernel_hash_ignores_comments(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n  return x + 1;  // one\n}\n/* block */\n")
    h1 = bench.kernel_code_hash([str(src)])
    src.write_text("int f(int x) {   return x + 1;  // two, longer\n}\n")
    assert bench.kernel_code_hash([str(src)]) == h1
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_code_hash([str(src)]) != h1


def test_counter_summaries_name_their_kernel_hash():
    """Every committed HBM-byte summary records the code hash it was taken with, and the
    bytes per launch that bench.py reports as `traffic`."""
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.endswith("_hbm_bytes.txt")]
    assert names
    for n in names:
        text = open(os.path.join(prof, n)).read()
        assert "kernel code sha256" in text and "traffic bytes per launch:" in text, n
        assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text, n


def test_host_info_and_streaming_oracle_baseline():
    """The oracle baseline states the host it ran on, and the streaming workload's baseline
    runs the CLOCK step and the attention of a step within its time budget."""
    import argparse
    sys.path.insert(0, ROOT)
    import bench
    info = bench.host_info()
    assert info["usable_cores"] >= 1 and info["os_cpu_count"] >= 1
    assert set(info) == {"cpu_model", "usable_cores", "os_cpu_count", "blas"}
    res = bench.cpu_baseline_streaming(argparse.Namespace(host_tokens=65536, cpu_seconds=0.01))
    assert res["kind"] == "oracle" and res["value"] > 0 and res["cores"] >= 1
    assert "16 layers" in res["sample"] and res["host"] == info


def test_trace_and_counter_summaries(tmp_path):
    """--summarize-trace and --summarize-counters read rocprofv3's CSV layout."""
    d = tmp_path / "t" / "host"
    d.mkdir(parents=True)
    (d / "1_kernel_trace.csv").write_text(
        "Kernel_Name,Start_Timestamp,End_Timestamp\n"
        '"void kvc::(anonymous namespace)::decode_split<1, 1, 4, false, true>(x)",1000,41000\n'
        '"void kvc::(anonymous namespace)::decode_split<1, 1, 4, false, true>(x)",50000,88000\n'
        '"void kvc::(anonymous namespace)::decode_combine(y)",90000,95000\n')
    r = run_bench("--summarize-trace", str(tmp_path / "t"), "--last", "1")
    assert r.returncode == 0, r.stderr
    assert "decode_split<1, 1, 4, false, true>" in r.stdout and "38.00" in r.stdout
    c = tmp_path / "c" / "host"
    c.mkdir(parents=True)
    (c / "1_counter_collection.csv").write_text(
        "Kernel_Name,Counter_Name,Counter_Value\n"
        '"decode_split<1, 1, 4, false, true>",FETCH_SIZE,100\n"decode_split<1, 1, 4, false, true>",FETCH_SIZE,300\n')
    r = run_bench("--summarize-counters", str(tmp_path / "c"))
    assert r.returncode == 0, r.stderr
    assert "FETCH_SIZE" in r.stdout and "200.0" in r.stdout
