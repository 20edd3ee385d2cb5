"""Host-side checks of the benchmark script (no GPU): it refuses more than
one GPU, the committed counter summaries it reads are current and
self-consistent, its rocprofv3 summary writer round-trips counters through
the same parser, and its CPU baseline runs the oracle on a small trace."""
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("mode", ["fused", "noio"])
def test_committed_traffic_is_current(mode):
    """The PMC summaries behind the headline's traffic figures (the 16 x 8
    shared-selection workload) were taken on the kernel sources in the tree
    (else the bench reports no traffic), over the 20 steps the default run
    times, and the scaled byte counts are of the size the workload implies."""
    t = bench.committed_traffic("resolve_kernel", "tokens_b16x8_L256k", mode)
    assert t is not None, "PMC summaries missing or taken on other kernel sources"
    # the driver's run: 20 timed steps x 8 layers after 5 warm-up steps
    assert bench.traffic_matches(t, 20, 5, 160, serial=False)
    assert not bench.traffic_matches(t, 32, 5, 256, serial=False)
    assert not bench.traffic_matches(t, 20, 0, 160, serial=False)
    assert not bench.traffic_matches(t, 20, 5, 160, serial=True)
    # per launch: 16 streams x 2048 selections of metadata at least; with the
    # copies, about 9.4 MB of miss rows read and written on average
    assert t["FETCH_SIZE"] > 16 * 2048 * 4 and t["WRITE_SIZE"] > 16 * 2048 * 4
    if mode == "fused":
        assert 9.0e6 < t["FETCH_SIZE"] < 2.0e7
        assert 9.0e6 < t["WRITE_SIZE"] < 2.0e7
    else:
        assert t["FETCH_SIZE"] < 5.0e6 and t["WRITE_SIZE"] < 5.0e6


def test_committed_traffic_of_attention_and_topk():
    """The attention and top-k counter summaries are current for their own
    kernel sources: attention reads every attended row about once (16 x 2048
    rows of 1152 B) plus the split partials; top-k reads the 16 x 131072
    scores twice (histogram, filter)."""
    rows = 16 * 2048 * 1152
    m = bench.committed_traffic(("mla_decode_kernel", "mla_combine_kernel"),
                                "tokens_b16x8_L256k_h16", "mla")
    assert m is not None
    assert rows < m["FETCH_SIZE"] < 1.6 * rows
    scores = 16 * 131072 * 4
    t = bench.committed_traffic(("topk_hist_kernel", "topk_filter_kernel", "topk_finish_kernel"),
                                "tokens_b16x8_L128k", "topk")
    assert t is not None
    assert 2 * scores < t["FETCH_SIZE"] < 3 * scores


def test_summary_writer_round_trip(tmp_path, monkeypatch):
    """A synthetic rocprofv3 counter CSV -> the Markdown summary -> the parser
    the bench uses: the calibration copy's reading scales the kernel's."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    d = tmp_path / "raw" / "node"
    d.mkdir(parents=True)
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    rows += ["1,hsp::resolve_kernel<4>(args),FETCH_SIZE,100.0",
             "2,hsp::resolve_kernel<4>(args),FETCH_SIZE,300.0",
             "3,hsp::probe_host_read_kernel(args),FETCH_SIZE,131072.0"]
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_rocprof(str(tmp_path / "raw"), "pmc_fetch_size_x_fused", "cmd")
    rows[1:] = [r.replace("FETCH_SIZE", "WRITE_SIZE") for r in rows[1:]]
    rows[-1] = "3,hsp::probe_host_read_kernel(args),WRITE_SIZE,262144.0"
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_rocprof(str(tmp_path / "raw"), "pmc_write_size_x_fused", "cmd")
    t = bench.committed_traffic("resolve_kernel", "x", "fused")
    # mean 200 KiB per dispatch; the 256 MiB copy read as 128 MiB -> x2, written as 256 MiB -> x1
    assert t["FETCH_SIZE"] == pytest.approx(200 * 1024 * 2.0)
    assert t["WRITE_SIZE"] == pytest.approx(200 * 1024 * 1.0)
    text = (tmp_path / "profiles" / "pmc_fetch_size_x_fused.md").read_text()
    assert "Command: `cmd`" in text and "| resolve_kernel | FETCH_SIZE | 2 | 200.0 | 400.0 |" in text
    # with a tail, the means cover each kernel's last dispatches only
    bench.summarize_rocprof(str(tmp_path / "raw"), "pmc_write_size_x_fused",
                            "bench.py --steps 1 --warmup 1", tail=1)
    rows[1:] = [r.replace("WRITE_SIZE", "FETCH_SIZE") for r in rows[1:]]
    rows[-1] = "3,hsp::probe_host_read_kernel(args),FETCH_SIZE,131072.0"
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_rocprof(str(tmp_path / "raw"), "pmc_fetch_size_x_fused",
                            "bench.py --steps 1 --warmup 1", tail=1)
    t = bench.committed_traffic("resolve_kernel", "x", "fused")
    assert t["FETCH_SIZE"] == pytest.approx(300 * 1024 * 2.0)   # the last dispatch only
    assert bench.traffic_matches(t, 1, 1, 1, serial=False)
    assert not bench.traffic_matches(t, 1, 1, 2, serial=False)


def test_cpu_baseline_runs_the_oracle():
    from tests.harness import fill_host, make_trace
    from workload import WORKLOADS
    cfg = WORKLOADS[2].scaled(B=2, L0=6000, C=1200, R=16, k=600, steps=3)
    trace = make_trace(cfg)
    hosts = {(b, l): (None, np.zeros((cfg.l_cap, cfg.row_bytes), np.uint8))
             for b in range(cfg.B) for l in range(cfg.layers)}
    fill_host(cfg, lambda b, l: hosts[(b, l)][1], trace, list(hosts))
    setup = types.SimpleNamespace(cfg=cfg, trace=trace, hosts=hosts, queries=1, W=1)
    r = bench.cpu_baseline(setup, cfg.steps - 1, threads=2, min_seconds=0.2, no_io_seconds=0.1)
    assert r["kind"] == "oracle" and r["cores"] == 2 and r["unit"] == "entries/s"
    assert r["value"] > 0 and r["no_io_value"] > 0
    assert "steps 1 .. 2 of the trace (after 1 untimed warm-up steps) on all 2 streams" in r["sample"]


def test_only_the_cpu_baseline_legs_reach_the_oracle():
    """The benchmark's setup and timed code have no import edge into oracle/
    or tests/: every such import sits inside a function whose name says it
    is a CPU-baseline leg, and importing the benchmark (and the package, the
    instance helper and the input preparation it uses) loads neither."""
    import ast
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())

    def walk(node, fn=None):
        for child in ast.iter_child_nodes(node):
            name = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else fn
            if isinstance(child, (ast.Import, ast.ImportFrom)):
                mods = ([a.name for a in child.names] if isinstance(child, ast.Import)
                        else [child.module or ""])
                for m in mods:
                    if m.split(".")[0] in ("oracle", "tests"):
                        assert name and "cpu_baseline" in name, (m, name, child.lineno)
            walk(child, name)

    walk(tree)
    code = ("import sys; sys.path.insert(0, %r); import bench; "
            "import hierarchical_kv_cache_hisparse_amd.instance, workload.prepare; "
            "bad = [m for m in sys.modules if m.split('.')[0] in ('oracle', 'tests')]; "
            "assert not bad, bad" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       cwd="/")
    assert r.returncode == 0, r.stderr
