"""bench.py's command line, without a GPU: more than one GPU is refused with
a message and exit status 2 before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_contract_flags():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--graph", "--no-fp8"):
        assert flag in r.stdout


def test_power_sampler_reads_a_sysfs_tree(tmp_path):
    """bench.py's power / clock sampler on a fake sysfs tree: an AMD card with
    hwmon power1_input and power1_cap (microwatts) and a DPM sclk table whose
    current level is marked '*'.  Run in a child process: importing bench.py
    sets BLAS thread variables."""
    dev = tmp_path / "card0" / "device"
    (dev / "hwmon" / "hwmon3").mkdir(parents=True)
    (dev / "vendor").write_text("0x1002\n")
    (dev / "hwmon" / "hwmon3" / "power1_input").write_text("1390000000\n")
    (dev / "hwmon" / "hwmon3" / "power1_cap").write_text("1400000000\n")
    (dev / "pp_dpm_sclk").write_text("0: 500Mhz\nS: 1882Mhz *\n1: 2400Mhz\n")
    code = (
        "import json, time, bench\n"
        f"s = bench.PowerSampler({str(tmp_path)!r})\n"
        "s.start(); time.sleep(0.05); s.stop()\n"
        "print(json.dumps(s.summary()))\n"
        "print(json.dumps(bench.PowerSampler('/nonexistent').summary()))\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr
    import json
    got, none = (json.loads(line) for line in r.stdout.strip().splitlines())
    assert got["samples"] >= 2
    assert got["power_w_mean"] == got["power_w_max"] == 1390.0
    assert got["power_cap_w"] == 1400.0
    assert got["sclk_mhz_mean"] == got["sclk_mhz_min"] == 1882.0
    assert none is None


def test_source_hash_ignores_comments_and_layout():
    """The hash that ties profiles/traffic.json to the kernel sources changes
    with the code, not with comments or whitespace; comment markers inside
    string literals (inline assembly) are code."""
    import bench
    src = 'int a = 1; // one\n/* block\n comment */ asm("s_nop 1 // not a comment");\n'
    assert bench.strip_comments(src).split() == ['int', 'a', '=', '1;', 'asm("s_nop', '1', '//', 'not', 'a', 'comment");']
    assert " ".join(bench.strip_comments("x /* a */ + y // b\n").split()) == "x + y"
    assert len(bench.source_hash()) == 16
