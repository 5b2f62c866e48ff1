"""Host-side pieces of bench.py (CPU only): the committed profile figures it
reports are parsed and tied to the GEMM sources they were taken from, and a
request for more than one GPU is refused before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_profile_figures_parse_or_are_withheld():
    traffic, alg = bench.gemm_traffic()
    clock, busy = bench.gemm_clock()
    # either both figures match the current GEMM sources, or they are withheld
    assert (traffic is None) == (alg is None)
    assert (clock is None) == (busy is None)
    if traffic is not None:
        assert traffic > alg > 0
    if clock is not None:
        assert 0.5 < clock < 2.5 and 0.0 < busy <= 1.0


def test_figures_withheld_for_other_sources(tmp_path, monkeypatch):
    src = tmp_path / "gemm.hip"
    src.write_text("// a different kernel source\n")
    monkeypatch.setattr(bench, "GEMM_SOURCES", [str(src)])
    assert bench.gemm_traffic() == (None, None)
    assert bench.gemm_clock() == (None, None)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_profile_commands_use_valid_bench_flags(monkeypatch):
    """Every bench.py command recorded in profiles/ parses with bench.py's own
    argument parser, and a counter run (--pmc) never also asks for a trace."""
    import glob
    import shlex
    cmds = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if line.startswith("rocprofv3 ") and "bench.py" in line:
                cmds.append((os.path.basename(path), line.strip()))
    assert cmds, "no recorded bench commands"
    for name, line in cmds:
        words = shlex.split(line)
        if "--pmc" in words:
            assert not any(w in words for w in ("--kernel-trace", "--sys-trace", "-s",
                                                "--runtime-trace", "-r")), name
        args = words[words.index(next(w for w in words if w.endswith("bench.py"))) + 1:]
        monkeypatch.setattr(sys, "argv", ["bench.py"] + args)
        a = bench.parse()
        assert a.gpus == 1 and a.steps >= 1, name


def test_per_kernel_medians():
    """Per-kernel step times are sums over a step's launches of each launch's
    median across the timed steps, so one slow step does not move them."""
    class Ev:
        def __init__(self, t):
            self.t = t

        def elapsed_time(self, other):
            return other.t - self.t

    events = []
    for scale in (1.0, 5.0, 1.2):                      # the second step is an outlier
        events.append(("gemm", 10.0, "FLOP", Ev(0.0), Ev(2.0 * scale)))
        events.append(("quant", 4.0, "B", Ev(0.0), Ev(1.0 * scale)))
        events.append(("gemm", 20.0, "FLOP", Ev(0.0), Ev(3.0 * scale)))
    per = bench.per_kernel_medians(events, 3)
    assert per["gemm"]["launches"] == 2 and per["gemm"]["work"] == 30.0
    assert abs(per["gemm"]["ms"] - (2.0 * 1.2 + 3.0 * 1.2)) < 1e-12
    assert per["quant"]["launches"] == 1 and abs(per["quant"]["ms"] - 1.2) < 1e-12
