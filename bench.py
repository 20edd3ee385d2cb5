#!/usr/bin/env python3
"""Benchmark of the per-layer selection-resolution step on one MI355X.

A step is one decode step of the whole hot path: for every layer, resolve
every request's top-k selections (hit detection, LRU victim choice, metadata
update, slot map) and fetch the missing rows from pinned host memory into the
HBM slot cache.  Inputs (selections, context lengths, appended rows) are
resident in HBM before the timed region; the host histories live in pinned
host memory, which is where the method keeps them.

Prints one JSON line.  ``value`` is resolved top-k entries per second over
the timed region: all K steps captured as one HIP graph (as a decode graph
holds them) and replayed once from a cold cache.  When each layer call is one
launch (the fused copy), the dominant kernel's average launch duration comes
from HIP events on the launch stream around that timed replay; otherwise
(separate fetch launches, which events cannot split inside a graph) from an
eager pass over the same K steps with the library's HIP events around each
launch, whose throughput is reported too.  Also reported: miss-fetch GB/s against the host link
(theoretical PCIe Gen5 x16 and the measured peak of this machine), the resolve
kernel against HBM, the no-IO (copies suppressed) per-layer call time under
graph replay, and the CPU oracle timed on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

LINK_PEAK_THEORETICAL_GBPS = 64.0      # PCIe Gen5 x16, per direction
HBM_PEAK_GBPS = 8000.0                  # MI355X HBM3E
DECODE_STEP_BUDGET_US = 20000.0         # reading: 20 ms decode step ...
BUDGET_LAYERS = 64                      # ... spread over a 64-layer model
NOIO_STEP_BUDGET_US = 1000.0            # whole-step resolution without copies, all layers


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: the workload's own step count, 64 for workload 2)")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", type=int, default=4,
                    help="workload 1..5 of workload/configs.py (default 4: 16 requests x 8 layers "
                         "sharing one selection, 262144 token rows, the next layer prefetched on "
                         "a second stream; the largest workload of the five)")
    ap.add_argument("--serial", action="store_true",
                    help="shared-selection workloads: resolve every layer on the main stream "
                         "instead of the workload's layer-wise prefetch schedule")
    ap.add_argument("--no-prefetch-study", action="store_true",
                    help="skip the prefetch hidden-fraction study of the default run")
    ap.add_argument("--numa-node", type=int, default=-1,
                    help="NUMA node of the pinned host histories (-1: the GPU's own node, "
                         "-2: the process's default policy)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the link-peak probe")
    ap.add_argument("--no-io", action="store_true",
                    help="with --only-timed: time the instance that suppresses the row copies "
                         "(metadata only), for profiling the resolve kernel alone")
    ap.add_argument("--only-timed", action="store_true",
                    help="only the eager timed region (for profiler runs)")
    ap.add_argument("--with-graph", action="store_true",
                    help="with --only-timed: also the timed graph replay (for profiler runs "
                         "of the launches the roofline times)")
    ap.add_argument("--host-noncoherent", action="store_true",
                    help="allocate host histories non-coherent (GPU-cacheable)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after the timed region, copy 256 MiB device->device with the "
                         "library's 16-byte copy kernel (known bytes for PMC scaling)")
    ap.add_argument("--prefetch-study", action="store_true",
                    help="shared-selection workloads: serial vs layer-wise prefetch vs no-IO, "
                         "with a fixed-duration stand-in for each layer's compute")
    ap.add_argument("--layer-compute-us", type=float, default=312.5,
                    help="stand-in compute per layer for --prefetch-study (20 ms / 64 layers)")
    ap.add_argument("--layer-compute", choices=("busy", "attention", "none"), default="busy",
                    help="--prefetch-study per-layer compute: the calibrated busy kernel, the "
                         "sparse MLA decode attention over the layer's slot map (--heads), or "
                         "none (the schedules' own overlap)")
    ap.add_argument("--mla-attention", action="store_true",
                    help="time sparse MLA decode attention over the slot map (one layer)")
    ap.add_argument("--heads", type=int, default=16, help="query heads for --mla-attention")
    ap.add_argument("--topk", action="store_true",
                    help="time the top-k selection producer over synthetic indexer scores at "
                         "the workload's per-layer shape (requests x context rows, k)")
    ap.add_argument("--pipeline", action="store_true",
                    help="time the layer step as a DSA-style decode step runs it: indexer scores "
                         "-> top-k -> resolve with miss fetch -> sparse MLA attention (--heads), "
                         "every layer, all steps in one HIP graph; also with the copies "
                         "suppressed")
    ap.add_argument("--queries", type=int, default=1,
                    help="query tokens per request and step (multi-token prediction): each "
                         "brings the workload's k selections; resolved in one pass per layer")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="summarize rocprofv3 CSV output in DIR into profiles/ and exit")
    ap.add_argument("--label", help="summary name (with --summarize-rocprof)")
    ap.add_argument("--command", help="the profiled command line (with --summarize-rocprof)")
    ap.add_argument("--trace-tail", type=int, default=0,
                    help="with --summarize-rocprof: also the mean over each kernel's last N launches")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_mem_available_gib():
    """MemAvailable of /proc/meminfo, GiB (None where unreadable)."""
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    return round(int(line.split()[1]) / 2**20, 1)
    except OSError:
        pass
    return None


class Setup:
    """Host histories, two library instances (IO and no-IO) and device inputs."""

    def __init__(self, cfg, host_flags, queries=1, numa_node=-1, prefetch=False, warmup=0):
        import torch
        from hierarchical_kv_cache_hisparse_amd import binding as hb
        from hierarchical_kv_cache_hisparse_amd.instance import GpuInstance, host_view
        from workload.prepare import appended_row, fill_host, make_trace
        self.torch, self.hb, self.cfg, self.queries = torch, hb, cfg, queries
        self.W = warmup    # untimed decode steps before every timed region
        # the workload's layer-wise prefetch schedule (shared selections only)
        self.prefetch = bool(prefetch and cfg.shared_selection and cfg.layers > 1 and queries == 1)
        self.side = torch.cuda.Stream() if self.prefetch else None
        t0 = time.time()
        self.trace = make_trace(cfg, queries=queries)                  # [S, L, B, k]
        nbytes = cfg.l_cap * cfg.row_bytes
        # pinning fails loudly (the binding raises); nothing is shrunk to fit
        self.host_memory = {"available_before_GiB": host_mem_available_gib(),
                            "pinned_GiB": round(cfg.streams * nbytes / 2**30, 3)}
        self.hosts = {}
        for l in range(cfg.layers):
            for b in range(cfg.B):
                ptr = hb.hisparse_host_alloc(nbytes, host_flags, numa_node)
                self.hosts[(b, l)] = (ptr, host_view(ptr, nbytes).reshape(cfg.l_cap, cfg.row_bytes))
        streams = list(self.hosts)
        fill_host(cfg, lambda b, l: self.hosts[(b, l)][1], self.trace, streams)
        # where the histories landed: the node of a few touched pages of the
        # first and last history, next to the GPU's own node
        import glob
        self.host_memory["numa_node_requested"] = numa_node
        self.host_memory["host_numa_nodes"] = len(glob.glob("/sys/devices/system/node/node[0-9]*"))
        self.host_memory["gpu_numa_node"] = hb.hisparse_device_numa_node()
        nodes = set()
        for key in (streams[0], streams[-1]):
            ptr, view = self.hosts[key]
            for frac in (0.0, 0.5, 0.999):
                row = int(frac * (cfg.l_cap - 1))
                nodes.add(hb.hisparse_host_numa_node(ptr + row * cfg.row_bytes))
        self.host_memory["history_numa_nodes"] = sorted(nodes)
        log(f"host histories: {len(streams)} x {nbytes / 2**20:.1f} MiB pinned on NUMA node(s) "
            f"{sorted(nodes)} (GPU node {self.host_memory['gpu_numa_node']}), filled in "
            f"{time.time() - t0:.1f}s")
        self.io = GpuInstance(cfg, flags=0, hosts=self.hosts)
        self.noio = GpuInstance(cfg, flags=hb.HISPARSE_NO_IO, hosts=self.hosts)
        dev = "cuda:0"
        S = cfg.steps
        self.sel = torch.from_numpy(self.trace).to(dev)
        self.ctx = torch.from_numpy(
            np.array([[cfg.ctx_at(s)] * cfg.B for s in range(S)], np.int32)).to(dev)
        self.out = torch.empty((cfg.layers, cfg.B, cfg.k), dtype=torch.int32, device=dev)
        self.rows = self.pos = None
        if cfg.growth:
            rows = np.zeros((S, cfg.layers, cfg.B, cfg.row_bytes), np.uint8)
            for s in range(1, S):
                for l in range(cfg.layers):
                    for b in range(cfg.B):
                        rows[s, l, b] = appended_row(cfg, b, l, cfg.ctx_at(s) - 1)
            self.rows = torch.from_numpy(rows).to(dev)
            self.pos = torch.from_numpy(
                np.array([[cfg.ctx_at(s) - 1] * cfg.B for s in range(S)], np.int32)).to(dev)
        torch.cuda.synchronize()

    def reset(self, inst):
        hb, s = self.hb, self.torch.cuda.current_stream().cuda_stream
        hb.hisparse_reset(inst.h, s, -1, -1)
        hb.hisparse_load_window(inst.h, s, -1, self.ctx[0].data_ptr())
        self.torch.cuda.synchronize()

    def warm(self, inst):
        """Reset `inst`, then run the W warm-up steps (0 .. W-1) eagerly: the
        state every timed region starts from.  Returns the running totals
        (misses, evictions, hits) after them."""
        self.reset(inst)
        for s in range(self.W):
            self.step(inst, s)
        self.torch.cuda.synchronize()
        return self.totals(inst)

    def step(self, inst, s, stream=None):
        hb, cfg = self.hb, self.cfg
        st = self.torch.cuda.current_stream().cuda_stream if stream is None else stream
        if self.prefetch:
            # shared selections: layer 0 on the main stream; every layer l+1
            # prefetched on the side stream (forked after layer l's call) and
            # joined by its resolve
            ctx = self.ctx[s].data_ptr()
            hb.hisparse_resolve(inst.h, st, self.sel[s, 0].data_ptr(), ctx, 0,
                                self.out[0].data_ptr())
            for l in range(cfg.layers - 1):
                hb.hisparse_prefetch(inst.h, st, self.side.cuda_stream,
                                     self.sel[s, l + 1].data_ptr(), ctx, l + 1,
                                     self.out[l + 1].data_ptr())
                hb.hisparse_resolve(inst.h, st, self.sel[s, l + 1].data_ptr(), ctx, l + 1,
                                    self.out[l + 1].data_ptr())
            return
        for l in range(cfg.layers):
            if cfg.growth and s > 0:
                # the decode step of a growing context: append + resolve, one call
                if self.queries > 1:
                    hb.hisparse_append_resolve_multi(
                        inst.h, st, l, self.rows[s, l].data_ptr(), self.pos[s].data_ptr(),
                        self.sel[s, l].data_ptr(), self.queries, cfg.k // self.queries,
                        self.ctx[s].data_ptr(), self.out[l].data_ptr())
                else:
                    hb.hisparse_append_resolve(inst.h, st, l, self.rows[s, l].data_ptr(),
                                               self.pos[s].data_ptr(), self.sel[s, l].data_ptr(),
                                               self.ctx[s].data_ptr(), self.out[l].data_ptr())
                continue
            if self.queries > 1:
                hb.hisparse_resolve_multi(inst.h, st, self.sel[s, l].data_ptr(), self.queries,
                                          cfg.k // self.queries, self.ctx[s].data_ptr(), l,
                                          self.out[l].data_ptr())
            else:
                hb.hisparse_resolve(inst.h, st, self.sel[s, l].data_ptr(), self.ctx[s].data_ptr(),
                                    l, self.out[l].data_ptr())

    def totals(self, inst):
        """Summed running counters of every stream (misses, evictions, hits)."""
        return inst.totals()

    def close(self):
        self.io.close()
        self.noio.close()
        for ptr, _ in self.hosts.values():
            self.hb.hisparse_host_free(ptr)


def link_probe(torch, hb, numa_node=-1):
    """Host->device peak of this machine, from pinned memory on the histories'
    NUMA node: hipMemcpyAsync of 256 MiB (through torch's copy), and a
    zero-copy 16-byte-load kernel over 256 MiB at several grid sizes; best
    of 5 each.  torch's own pinned allocator is measured too, for context."""
    from hierarchical_kv_cache_hisparse_amd.instance import host_view
    nbytes = 256 << 20
    dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")

    def best_of(fn, n=5):
        best = 0.0
        for _ in range(n):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            best = max(best, nbytes / (time.perf_counter() - t0) / 1e9)
        return round(best, 2)

    res = {}
    ptr = hb.hisparse_host_alloc(nbytes, hb.HISPARSE_HOST_COHERENT, numa_node)
    try:
        view = host_view(ptr, nbytes)
        view[:] = 1
        res["numa_node"] = hb.hisparse_host_numa_node(ptr)
        src = torch.from_numpy(view)   # the pinned allocation, as a CPU tensor
        res["memcpy_h2d_GBps"] = best_of(lambda: dev.copy_(src, non_blocking=True))
        stream = torch.cuda.current_stream().cuda_stream
        per_wg = {}
        for wgs in (1, 4, 8, 16, 64, 256, 1024):
            per_wg[wgs] = best_of(
                lambda: hb.hisparse_probe_host_read(stream, ptr, dev.data_ptr(), nbytes, wgs))
        res["zero_copy_read_GBps"] = per_wg
        del src, view
    finally:
        hb.hisparse_host_free(ptr)
    pinned = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    pinned.fill_(1)
    res["memcpy_h2d_torch_pinned_GBps"] = best_of(lambda: dev.copy_(pinned, non_blocking=True))
    del pinned
    res["measured_peak_GBps"] = max(res["memcpy_h2d_GBps"], *res["zero_copy_read_GBps"].values())
    return res


PROFILES = os.path.join(ROOT, "profiles")
# the resolve and fetch kernels' sources: PMC summaries taken on other sources
# are not used for the traffic figure
CSRC = os.path.join(ROOT, "hierarchical_kv_cache_hisparse_amd", "csrc")
# the sources each kernel family is built from; a counter summary is used only
# while the hash of its family's sources matches the one it recorded
SOURCE_FAMILIES = {
    "resolve": ("hisparse_kernels.hip", "hisparse_device.h", "hisparse_internal.h",
                "hisparse_align.h"),
    "mla": ("hisparse_mla.hip", "hisparse_device.h", "hisparse_mla_internal.h"),
    "topk": ("hisparse_topk.hip", "hisparse_device.h", "hisparse_topk_internal.h",
             "hisparse_align.h"),
}
SHA_LINE = {"resolve": "Kernel source sha256[:16]", "mla": "MLA kernel source sha256[:16]",
            "topk": "Top-k kernel source sha256[:16]"}
CALIBRATION_BYTES = 256 << 20


def _code_only(text):
    """Source text without comments and blank lines: edits to comments leave
    the recorded hash (and the counters taken on that code) valid."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_sha(family="resolve"):
    import hashlib
    h = hashlib.sha256()
    for name in SOURCE_FAMILIES[family]:
        with open(os.path.join(CSRC, name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def kernel_family(kernel):
    if kernel.startswith("mla_"):
        return "mla"
    if kernel.startswith("topk_"):
        return "topk"
    return "resolve"


def calibration_copy():
    """The known-size device copy (256 MiB with 16-byte loads) whose counter
    readings scale FETCH_SIZE and WRITE_SIZE in the PMC runs."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(3)
    torch.cuda.synchronize()
    hb.hisparse_probe_host_read(torch.cuda.current_stream().cuda_stream, src.data_ptr(),
                                dst.data_ptr(), CALIBRATION_BYTES, 1024)
    torch.cuda.synchronize()
    del src, dst


KERNEL_NAMES = ("mla_decode_kernel", "mla_combine_kernel", "topk_hist_kernel", "topk_filter_kernel",
                "topk_finish_kernel", "resolve_kernel", "fetch_stream_kernel", "fetch_kernel",
                "prefetch_join_kernel")


def short_kernel_name(name):
    for key in ("mla_decode_kernel", "mla_combine_kernel", "topk_hist_kernel", "topk_filter_kernel",
                "topk_finish_kernel", "resolve_kernel", "fetch_stream_kernel", "fetch_kernel",
                "probe_host_read_kernel", "init_kernel",
                "load_window_kernel", "append_kernel", "prefetch_join_kernel"):
        if key in name:
            return key
    return name.split("(")[0][-48:]


def summarize_rocprof(directory, label, command, tail=0):
    """Turn rocprofv3 CSV output (kernel trace + stats, or one PMC counter)
    into a short Markdown summary under profiles/.  With tail > 0 the trace
    table also gives each kernel's mean over its last `tail` launches (in
    start order), e.g. the launches of the timed graph replay."""
    import csv
    import glob
    lines = [f"# {label}", "", f"Command: `{command}`", ""]
    sha_at = len(lines)  # the hashes of the kernel families measured here go here
    stats = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    pmc = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if stats:
        lines += ["## rocprofv3 --stats (kernel durations)", "",
                  "| kernel | calls | total us | average us | min us | max us |",
                  "|---|---|---|---|---|---|"]
        with open(stats[0]) as f:
            for row in csv.DictReader(f):
                lines.append("| {} | {} | {:.1f} | {:.3f} | {:.3f} | {:.3f} |".format(
                    short_kernel_name(row["Name"]), row["Calls"],
                    float(row["TotalDurationNs"]) / 1e3, float(row["AverageNs"]) / 1e3,
                    float(row["MinNs"]) / 1e3, float(row["MaxNs"]) / 1e3))
        lines.append("")
    if trace:
        import statistics
        per = {}
        with open(trace[0]) as f:
            rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
        for row in rows:
            d = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            per.setdefault(short_kernel_name(row["Kernel_Name"]), []).append(d)
        head = "| kernel | launches | mean | median | first launch |"
        rule = "|---|---|---|---|---|"
        if tail:
            head += f" mean of the last {tail} |"
            rule += "---|"
        lines += ["## kernel trace: per-launch durations (us)", "", head, rule]
        for k, v in per.items():
            line = (f"| {k} | {len(v)} | {statistics.mean(v):.3f} | "
                    f"{statistics.median(v):.3f} | {v[0]:.3f} |")
            if tail:
                line += f" {statistics.mean(v[-tail:]):.3f} |" if len(v) >= tail else " - |"
            lines.append(line)
        lines.append("")
    if pmc:
        agg = {}
        with open(pmc[0]) as f:
            rows = list(csv.DictReader(f))
        if rows and "Dispatch_Id" in rows[0]:
            rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        for row in rows:
            key = (short_kernel_name(row["Kernel_Name"]), row["Counter_Name"])
            agg.setdefault(key, []).append(float(row["Counter_Value"]))
        if tail:   # each kernel's last `tail` dispatches (e.g. the timed steps)
            agg = {key: v[-tail:] for key, v in agg.items()}
            lines += [f"PMC means over the last {tail} dispatches of each kernel "
                      f"(all of them where it has fewer)", ""]
        lines += ["## PMC counters (per dispatch)", "",
                  "| kernel | counter | dispatches | mean per dispatch | total |",
                  "|---|---|---|---|---|"]
        for (k, c), v in sorted(agg.items()):
            lines.append(f"| {k} | {c} | {len(v)} | {sum(v) / len(v):.1f} | {sum(v):.1f} |")
        lines.append("")
        for (k, c), v in sorted(agg.items()):
            lines.append(f"pmc: kernel={k} counter={c} mean={sum(v) / len(v):.3f} "
                         f"dispatches={len(v)}")
    measured = {kernel_family(k) for k in KERNEL_NAMES
                if any(f"| {k} |" in line or f"kernel={k} " in line for line in lines)}
    lines[sha_at:sha_at] = [f"{SHA_LINE[fam]}: {kernel_source_sha(fam)}"
                            for fam in SOURCE_FAMILIES if fam in measured] + [""]
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, label + ".md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def committed_traffic(kernels, label, mode):
    """HBM+link bytes per call from the committed PMC summaries: FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch) of each kernel in `kernels` (one name,
    or several launched once per call, summed), each scaled by the counter's
    reading for a device copy of known size.  None when a summary is absent
    or was taken on other sources of the kernels' family."""
    import re
    kernels = (kernels,) if isinstance(kernels, str) else tuple(kernels)
    fam = kernel_family(kernels[0])
    vals = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        path = os.path.join(PROFILES, f"pmc_{counter.lower()}_{label}_{mode}.md")
        if not os.path.exists(path):
            return None
        text = open(path).read()
        rec = re.search(r"^" + re.escape(SHA_LINE[fam]) + r": (\w+)$", text, re.M)
        if not rec or rec.group(1) != kernel_source_sha(fam):
            return None
        got = {}
        for m in re.finditer(r"pmc: kernel=(\S+) counter=(\S+) mean=([0-9.eE+-]+)", text):
            got[m.group(1)] = float(m.group(3))
        if any(k not in got for k in kernels) or "probe_host_read_kernel" not in got:
            return None
        scale = (CALIBRATION_BYTES / 1024.0) / got["probe_host_read_kernel"]
        vals[counter] = sum(got[k] for k in kernels) * scale * 1024.0
        # the profiled run: its step and warm-up counts (dispatch means are
        # over its launches, so the algorithmic bytes must be of the same steps)
        cmd = re.search(r"^Command: `(.*)`$", text, re.M)
        cmd = cmd.group(1) if cmd else ""
        st = re.search(r"--steps (\d+)", cmd)
        wu = re.search(r"--warmup (\d+)", cmd)
        tl = re.search(r"^PMC means over the last (\d+) dispatches", text, re.M)
        vals.setdefault("profiled", []).append({
            "counter": counter, "steps": int(st.group(1)) if st else None,
            "warmup": int(wu.group(1)) if wu else None, "serial": "--serial" in cmd,
            "tail": int(tl.group(1)) if tl else None})
    return vals


def traffic_matches(t, K, W, launches, serial):
    """True when every counter run of `t` profiled the same K timed steps
    after the same W warm-up steps on the same schedule, and its
    per-dispatch means are over exactly those steps' `launches` launches
    (the whole run when there is no warm-up)."""
    return bool(t) and all(
        p["steps"] == K and p["warmup"] == W and p["serial"] == serial
        and (p["tail"] == launches or (W == 0 and p["tail"] is None))
        for p in t["profiled"])


def traffic_fields(t):
    """The roofline's traffic entries from committed_traffic's result."""
    return {"traffic": round(t["FETCH_SIZE"] + t["WRITE_SIZE"]) if t else None,
            "traffic_read_bytes": round(t["FETCH_SIZE"]) if t else None,
            "traffic_write_bytes": round(t["WRITE_SIZE"]) if t else None}


def prefetch_study(setup, K, compute_us, compute="busy", heads=16):
    """Exact layer-wise prefetch on a shared-selection workload.

    Per layer a stand-in compute kernel (torch's fixed-cycle busy kernel,
    calibrated to `compute_us`; the sparse attention; or nothing) runs on the
    main stream.  Four schedules, each captured as one HIP graph of K steps
    and replayed after the warm-up steps:
      serial:    resolve(l); compute(l)                       for every layer
      prefetch:  resolve(0); then per layer prefetch(l+1) on a side stream,
                 compute(l), resolve(l+1) joins it
      two ahead: resolve(0), prefetch(1); then per layer prefetch(l+2) on the
                 other of two side streams, compute(l), resolve(l+1) joins:
                 two layers' launches in flight at once
      no-IO:     the serial schedule with copies suppressed
    hidden = 1 - (T_prefetch - T_noIO) / (T_serial - T_noIO).
    """
    torch, hb, cfg = setup.torch, setup.hb, setup.cfg
    if not cfg.shared_selection:
        raise SystemExit("--prefetch-study needs a workload whose layers share selections")
    # calibrate the busy kernel
    cycles = 1_000_000
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        ev0.record(); torch.cuda._sleep(cycles); ev1.record(); torch.cuda.synchronize()
    us_per_cycle = ev0.elapsed_time(ev1) * 1e3 / cycles
    cyc = max(1, int(round(compute_us / us_per_cycle)))
    attn = {}
    if compute == "attention":
        from workload.rows import make_queries
        for inst in (setup.io, setup.noio):
            attn[id(inst)] = torch.empty(hb.hisparse_mla_workspace_bytes(inst.h, heads),
                                         dtype=torch.uint8, device="cuda:0")
        qs = [torch.from_numpy(make_queries(cfg.B, heads, 3000 + cfg.data_seed, l)).to("cuda:0")
              for l in range(cfg.layers)]
        a_out = torch.empty((cfg.B, heads, 512), dtype=torch.float32, device="cuda:0")
        a_lse = torch.empty((cfg.B, heads), dtype=torch.float32, device="cuda:0")

    def layer_compute(inst, l, ms):
        if compute == "attention":
            hb.hisparse_sparse_mla_decode(inst.h, ms, l, qs[l].data_ptr(), setup.out[l].data_ptr(),
                                          heads, 1.0 / np.sqrt(576.0), attn[id(inst)].data_ptr(),
                                          a_out.data_ptr(), a_lse.data_ptr())
        elif compute == "busy":
            torch.cuda._sleep(cyc)

    def serial(inst, s, ms, ss, ss2):
        for l in range(cfg.layers):
            hb.hisparse_resolve(inst.h, ms, setup.sel[s, l].data_ptr(), setup.ctx[s].data_ptr(), l,
                                setup.out[l].data_ptr())
            layer_compute(inst, l, ms)

    def prefetched(inst, s, ms, ss, ss2):
        hb.hisparse_resolve(inst.h, ms, setup.sel[s, 0].data_ptr(), setup.ctx[s].data_ptr(), 0,
                            setup.out[0].data_ptr())
        for l in range(cfg.layers):
            if l + 1 < cfg.layers:
                hb.hisparse_prefetch(inst.h, ms, ss, setup.sel[s, l + 1].data_ptr(),
                                     setup.ctx[s].data_ptr(), l + 1, setup.out[l + 1].data_ptr())
            layer_compute(inst, l, ms)
            if l + 1 < cfg.layers:
                hb.hisparse_resolve(inst.h, ms, setup.sel[s, l + 1].data_ptr(),
                                    setup.ctx[s].data_ptr(), l + 1, setup.out[l + 1].data_ptr())

    def two_ahead(inst, s, ms, ss, ss2):
        sides = (ss, ss2)
        hb.hisparse_resolve(inst.h, ms, setup.sel[s, 0].data_ptr(), setup.ctx[s].data_ptr(), 0,
                            setup.out[0].data_ptr())
        if cfg.layers > 1:
            hb.hisparse_prefetch(inst.h, ms, sides[1], setup.sel[s, 1].data_ptr(),
                                 setup.ctx[s].data_ptr(), 1, setup.out[1].data_ptr())
        for l in range(cfg.layers):
            if l + 2 < cfg.layers:
                hb.hisparse_prefetch(inst.h, ms, sides[l % 2], setup.sel[s, l + 2].data_ptr(),
                                     setup.ctx[s].data_ptr(), l + 2, setup.out[l + 2].data_ptr())
            layer_compute(inst, l, ms)
            if l + 1 < cfg.layers:
                hb.hisparse_resolve(inst.h, ms, setup.sel[s, l + 1].data_ptr(),
                                    setup.ctx[s].data_ptr(), l + 1, setup.out[l + 1].data_ptr())

    W = setup.W

    def timed(inst, schedule):
        main, side, side2 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(main):
            with torch.cuda.graph(g, stream=main):
                for s in range(W, W + K):
                    schedule(inst, s, main.cuda_stream, side.cuda_stream, side2.cuda_stream)
        torch.cuda.synchronize()
        best = None
        for _ in range(2):
            setup.warm(inst)
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
        assert inst.status() == 0
        return best

    t_serial = timed(setup.io, serial)
    t_pref = timed(setup.io, prefetched)
    t_two = timed(setup.io, two_ahead)
    t_noio = timed(setup.noio, serial)
    t_noio_two = timed(setup.noio, two_ahead)

    def hidden_of(t):
        return round(1.0 - (t - t_noio) / (t_serial - t_noio), 4) if t_serial > t_noio else None

    return {"metric": "layer-wise prefetch: hidden fraction of the miss overhead",
            "value": hidden_of(t_pref), "unit": "fraction",
            "value_two_ahead": hidden_of(t_two),
            "workload": cfg.name, "steps": K, "layers": cfg.layers,
            "layer_compute": (f"sparse MLA attention, {heads} heads" if compute == "attention"
                              else "none" if compute == "none"
                              else f"busy kernel, {round(cyc * us_per_cycle, 2)} us"),
            "ms_per_step": {"serial": round(t_serial / K * 1e3, 4),
                            "prefetch": round(t_pref / K * 1e3, 4),
                            "two_ahead": round(t_two / K * 1e3, 4),
                            "no_io": round(t_noio / K * 1e3, 4),
                            "no_io_two_ahead": round(t_noio_two / K * 1e3, 4)},
            "miss_overhead_us_per_step": {"serial": round((t_serial - t_noio) / K * 1e6, 1),
                                          "prefetch": round((t_pref - t_noio) / K * 1e6, 1),
                                          "two_ahead": round((t_two - t_noio) / K * 1e6, 1)},
            "mode": f"one HIP graph per schedule of steps {W} .. {W + K - 1}, best of 2 replays "
                    f"after the {W} warm-up steps"}


def _mla_cpu_baseline(setup, K, q_np, rows, Q, per, scale):
    """The float64 oracle attention on the host over the host rows at the
    last step's selections, for as many attention rows as fit ~10 s (at
    least one): (seconds, rows timed)."""
    from oracle.attention import bf16_to_f64, mla_decode_attention_lse
    t_cpu, n_cpu = 0.0, 0
    for r in range(rows):
        b, j = divmod(r, Q)
        sel = setup.trace[K - 1, 0, b].reshape(Q, per)[j]
        host = setup.hosts[(b, 0)][1]
        tok = host[sel[sel >= 0]].reshape(-1, 1152)
        t0 = time.perf_counter()
        mla_decode_attention_lse(bf16_to_f64(q_np[r]), bf16_to_f64(tok), scale)
        t_cpu += time.perf_counter() - t0
        n_cpu += 1
        if t_cpu > 10.0:
            break
    return t_cpu, n_cpu


def _topk_cpu_baseline(scores, N, k):
    """The top-k oracle on the host, one row at a time, for as many rows as
    fit ~10 s (at least one): (seconds, rows timed)."""
    from oracle.topk import topk_rows
    t_cpu, n_cpu = 0.0, 0
    for b in range(scores.shape[0]):
        t0 = time.perf_counter()
        topk_rows(scores[b:b + 1], [N], k)
        t_cpu += time.perf_counter() - t0
        n_cpu += 1
        if t_cpu > 10.0:
            break
    return t_cpu, n_cpu


def mla_study(setup, K, H):
    """Sparse MLA decode attention over the slot map of layer 0, after each of
    K resolve steps; timed with torch events on the launching stream.  With
    several query tokens per request (--queries Q) every token attends to its
    own entries of the multi-query slot map.

    Algorithmic bytes per call: the attended rows (B * Q * k_q * T * 1152),
    the queries, outputs and lse; FLOPs: 2 * B * Q * H * k_q * T * (576 + 512)."""
    torch, hb, cfg = setup.torch, setup.hb, setup.cfg
    from workload.rows import make_queries
    io = setup.io
    T = cfg.row_bytes // 1152
    Q = setup.queries               # query tokens per request (rows of attention)
    per = cfg.k // Q
    rows = cfg.B * Q
    ws = torch.empty(hb.hisparse_mla_workspace_bytes_multi(io.h, Q, per, H), dtype=torch.uint8,
                     device="cuda:0")
    q_np = make_queries(rows, H, 3000 + cfg.data_seed, 0)
    q = torch.from_numpy(q_np).to("cuda:0")
    out = torch.empty((rows, H, 512), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((rows, H), dtype=torch.float32, device="cuda:0")
    scale = 1.0 / np.sqrt(576.0)
    stream = torch.cuda.current_stream().cuda_stream
    setup.reset(io)
    times = []
    for s in range(K):
        setup.step(io, s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if Q == 1:
            hb.hisparse_sparse_mla_decode(io.h, stream, 0, q.data_ptr(), setup.out[0].data_ptr(),
                                          H, scale, ws.data_ptr(), out.data_ptr(), lse.data_ptr())
        else:
            hb.hisparse_sparse_mla_decode_multi(io.h, stream, 0, Q, per, q.data_ptr(),
                                                setup.out[0].data_ptr(), H, scale, ws.data_ptr(),
                                                out.data_ptr(), lse.data_ptr())
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    us = float(np.median(times[1:] if len(times) > 1 else times))
    t_cpu, n_cpu = _mla_cpu_baseline(setup, K, q_np, rows, Q, per, scale)
    cpu_us_per_call = t_cpu / n_cpu * rows * 1e6
    n_tok = per * T
    byts = rows * n_tok * 1152 + rows * H * (1152 + 512 * 4 + 4)
    flops = 2.0 * rows * H * n_tok * (576 + 512)
    return {"metric": "sparse MLA decode attention over the slot map", "value": round(us, 3),
            "unit": "us per layer call", "higher_is_better": False, "workload": cfg.name,
            "requests": cfg.B, "query_tokens_per_request": Q, "heads": H,
            "attended_rows_per_query_token": n_tok,
            "roofline": {"bound": "hbm", "kernel": "mla_decode_kernel + mla_combine_kernel",
                         "achieved": round(byts / us / 1e3, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(byts / us / 1e3 / HBM_PEAK_GBPS, 4),
                         "per_launch_bytes": byts,
                         **traffic_fields(committed_traffic(
                             ("mla_decode_kernel", "mla_combine_kernel"),
                             f"{cfg.label}_h{H}" + (f"_q{Q}" if Q > 1 else ""), "mla"))},
            "mfma": {"achieved_TFLOPs": round(flops / us / 1e6, 2), "peak_TFLOPs": 2500.0,
                     "frac": round(flops / us / 1e6 / 2500.0, 5)},
            "timing": "torch events around each launch, median of steps 1..",
            "cpu_baseline": {"value": round(cpu_us_per_call, 1), "unit": "us per layer call",
                             "cores": 1, "kind": "oracle",
                             "sample": f"float64 numpy oracle on {n_cpu} of {rows} attention rows "
                                       f"of the last step, scaled to all rows"}}


def topk_study(cfg, K, W):
    """hisparse_topk on one layer's scores (requests x context rows, the
    workload's k), on fresh drifting scores each step; torch events on the
    launching stream around the three launches.

    Algorithmic bytes per call: every eligible score read once (4 B) plus the
    selection written (4 B per entry).  The kernels read the scores twice
    (histogram, filter), so at best half the HBM peak is reachable."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from workload.scores import score_rows
    B, N, k = cfg.B, cfg.L0, cfg.k
    stride = ((N + 3) // 4) * 4
    ws = torch.zeros(hb.hisparse_topk_workspace_bytes(B, N), dtype=torch.uint8, device="cuda:0")
    n_sets = 4
    host_scores = [score_rows(B, N, 5000 + cfg.data_seed, 0, s, ties=True) for s in range(n_sets)]
    scores = torch.zeros((n_sets, B, stride), dtype=torch.float32, device="cuda:0")
    for i, sc in enumerate(host_scores):
        scores[i, :, :N].copy_(torch.from_numpy(sc))
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda:0")
    out = torch.empty((B, k), dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream

    def call(i):
        hb.hisparse_topk(stream, scores[i % n_sets].data_ptr(), stride, B, N, ctx.data_ptr(), k,
                         ws.data_ptr(), out.data_ptr())

    for i in range(W):
        call(i)
    torch.cuda.synchronize()
    times = []
    for i in range(K):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call(i)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    us = float(np.median(times))
    # the graph-replayed per-call time (launch gaps removed)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            s2 = torch.cuda.current_stream().cuda_stream
            for i in range(16):
                hb.hisparse_topk(s2, scores[i % n_sets].data_ptr(), stride, B, N, ctx.data_ptr(),
                                 k, ws.data_ptr(), out.data_ptr())
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) / (5 * 16) * 1e6
    t_cpu, n_cpu = _topk_cpu_baseline(host_scores[0], N, k)
    byts = B * N * 4 + B * k * 4
    return {"metric": "top-k selection over indexer scores", "value": round(us, 3),
            "unit": "us per layer call", "higher_is_better": False, "workload": cfg.name,
            "rows": B, "positions_per_row": N, "k": k,
            "scores_per_s": round(B * N / us * 1e6, 1),
            "graph_us_per_call": round(graph_us, 3),
            "roofline": {"bound": "hbm",
                         "kernel": "topk_hist_kernel + topk_filter_kernel + topk_finish_kernel",
                         "achieved": round(byts / us / 1e3, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(byts / us / 1e3 / HBM_PEAK_GBPS, 4),
                         "per_launch_bytes": byts,
                         "achieved_graph": round(byts / graph_us / 1e3, 1),
                         **traffic_fields(committed_traffic(
                             ("topk_hist_kernel", "topk_filter_kernel", "topk_finish_kernel"),
                             cfg.label, "topk"))},
            "timing": "torch events around the three launches, median of K calls",
            "cpu_baseline": {"value": round(t_cpu / n_cpu * B * 1e6, 1), "unit": "us per layer call",
                             "cores": 1, "kind": "oracle",
                             "sample": f"numpy lexsort oracle on {n_cpu} of {B} rows, scaled"}}


def capture_steps(setup, inst, K, first=0):
    """Steps first .. first+K-1 of `inst` captured into one HIP graph (on a
    side stream); capturing runs nothing, so the caller sets the state each
    replay starts from (setup.warm, or setup.reset for first = 0)."""
    import torch
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for s in range(first, first + K):
                setup.step(inst, s)
    torch.cuda.synchronize()
    return g


def pipeline_study(setup, K, H):
    """Scores -> top-k -> resolve (+ miss fetch) -> sparse MLA attention for
    every layer of every step, captured as one HIP graph and replayed once
    from a cold cache, on the IO instance and on the instance that suppresses
    the copies.  Scores drift as the indexer's would: per layer a fixed N(0,1)
    base, plus 0.35 x N(0,1) noise per (step, layer), drawn on the device with
    a seeded generator before the timed region.  The selections therefore
    differ from the workload's trace, and host rows outside the trace's are
    zero: timing only; the pieces are parity-tested separately."""
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from workload.rows import make_queries
    cfg = setup.cfg
    dev = "cuda:0"
    B, N, k, L = cfg.B, cfg.L0, cfg.k, cfg.layers
    stride = ((cfg.l_cap + 3) // 4) * 4
    gen = torch.Generator(device=dev)
    gen.manual_seed(6000 + cfg.data_seed)
    base = torch.randn((L, B, N), generator=gen, device=dev)
    scores = torch.zeros((K * L, B, stride), dtype=torch.float32, device=dev)
    for s in range(K):
        for l in range(L):
            scores[s * L + l, :, :N] = base[l] + 0.35 * torch.randn((B, N), generator=gen,
                                                                     device=dev)
    del base
    tk_ws = torch.zeros(hb.hisparse_topk_workspace_bytes(B, cfg.l_cap), dtype=torch.uint8,
                        device=dev)
    sel = torch.empty((L, B, k), dtype=torch.int32, device=dev)
    q = torch.from_numpy(make_queries(B, H, 3000 + cfg.data_seed, 0)).to(dev)
    att = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    scale = 1.0 / np.sqrt(576.0)

    def run(inst, label):
        ws = torch.empty(hb.hisparse_mla_workspace_bytes(inst.h, H), dtype=torch.uint8,
                         device=dev)
        setup.reset(inst)
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                st = torch.cuda.current_stream().cuda_stream
                for s in range(K):
                    for l in range(L):
                        hb.hisparse_topk(st, scores[s * L + l].data_ptr(), stride, B,
                                         cfg.l_cap, setup.ctx[s].data_ptr(), k, tk_ws.data_ptr(),
                                         sel[l].data_ptr())
                        if cfg.growth and s > 0:
                            hb.hisparse_append_resolve(inst.h, st, l, setup.rows[s, l].data_ptr(),
                                                       setup.pos[s].data_ptr(), sel[l].data_ptr(),
                                                       setup.ctx[s].data_ptr(),
                                                       setup.out[l].data_ptr())
                        else:
                            hb.hisparse_resolve(inst.h, st, sel[l].data_ptr(),
                                                setup.ctx[s].data_ptr(), l, setup.out[l].data_ptr())
                        hb.hisparse_sparse_mla_decode(inst.h, st, l, q.data_ptr(),
                                                      setup.out[l].data_ptr(), H, scale,
                                                      ws.data_ptr(), att.data_ptr(), lse.data_ptr())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        setup.reset(inst)
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        assert inst.status() == 0
        misses = int(setup.totals(inst)[0])
        log(f"pipeline {label}: {K} steps x {L} layers in {dt * 1e3:.2f} ms, {misses} misses")
        return dt, misses

    dt_io, misses = run(setup.io, "IO")
    dt_noio, _ = run(setup.noio, "no-IO")
    calls = K * L
    return {"metric": "decode layer step: indexer top-k -> resolve -> sparse MLA attention",
            "value": round(dt_io / calls * 1e6, 3), "unit": "us per layer call",
            "higher_is_better": False, "workload": cfg.name, "heads": H, "steps": K,
            "layers": L,
            "no_io_us_per_layer_call": round(dt_noio / calls * 1e6, 3),
            "miss_bytes_per_layer_call": round(misses * cfg.row_bytes / calls),
            "miss_fetch_share": round(1.0 - dt_noio / dt_io, 4) if dt_io > 0 else None,
            "mode": "one HIP graph of all steps and layers, one timed replay from a cold cache",
            "note": "selections come from top-k over synthetic scores (not the workload trace)"}


def cpu_baseline(setup, steps, threads=1, min_seconds=10.0, no_io_seconds=0.0):
    """The CPU oracle (plain C) on the same trace and host rows: the timed
    steps W .. W+steps-1 after the W untimed warm-up steps (setup.W, 0 if
    absent), repeated until at least `min_seconds` of wall time are measured.  With
    threads > 1 the independent streams are spread over that many threads
    (the C oracle runs without the Python lock).  With no_io_seconds > 0 the
    same trace is also timed with the row copies suppressed, and the copy rate
    (miss bytes / the time difference) is reported."""
    from concurrent.futures import ThreadPoolExecutor
    from tests.harness import OracleRun
    cfg = setup.cfg
    streams = [(b, l) for b in range(cfg.B) for l in range(cfg.layers)]
    host_of = lambda b, l: setup.hosts[(b, l)][1]
    groups = [streams[i::threads] for i in range(threads)]

    W = getattr(setup, "W", 0)

    def warm_group(group, no_io):
        """Oracle streams after the W warm-up steps (untimed)."""
        run = OracleRun(cfg, group, host_of=host_of)
        for s in range(W):
            if cfg.growth and s > 0:
                run.append(s)
            run.step(s, setup.trace, no_io=no_io, queries=setup.queries)
        return run

    def run_group(run, no_io):
        missed = 0
        for s in range(W, W + steps):
            if cfg.growth and s > 0:
                run.append(s)
            res = run.step(s, setup.trace, no_io=no_io, queries=setup.queries)
            missed += sum(int(r.counters["n_miss"]) for r in res.values())
        return missed

    def timed(no_io, seconds):
        elapsed, entries, reps, missed = 0.0, 0, 0, 0
        with ThreadPoolExecutor(threads) as pool:
            while elapsed < seconds and reps < 2000:
                runs = list(pool.map(lambda g: warm_group(g, no_io), groups))
                t0 = time.perf_counter()
                missed += sum(pool.map(lambda r: run_group(r, no_io), runs))
                elapsed += time.perf_counter() - t0
                entries += steps * cfg.layers * cfg.B * cfg.k
                reps += 1
        return elapsed, entries, reps, missed

    elapsed, entries, reps, missed = timed(False, min_seconds)
    out = {"value": entries / elapsed, "unit": "entries/s", "cores": threads, "kind": "oracle",
           "sample": f"{reps} x steps {W} .. {W + steps - 1} of the trace (after {W} untimed "
                     f"warm-up steps) on all {len(streams)} streams with row copies "
                     f"({elapsed:.1f}s wall, {threads} thread(s))",
           "cpu_model": cpu_model()}
    if no_io_seconds > 0:
        e2, n2, r2, _ = timed(True, no_io_seconds)
        out["no_io_value"] = n2 / e2
        out["no_io_sample"] = f"{r2} x the same steps, row copies suppressed ({e2:.1f}s wall)"
        copy_s = elapsed / reps - e2 / r2
        out["memcpy_GBps"] = (round(missed / reps * cfg.row_bytes / copy_s / 1e9, 3)
                              if copy_s > 0 else None)
    return out


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.label or "profile", args.command or "",
                          tail=args.trace_tail)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the resolve path has no cross-GPU step, and this "
              f"build runs on a single MI355X (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    from hierarchical_kv_cache_hisparse_amd import binding as hb
    from workload import WORKLOADS

    torch.cuda.set_device(0)
    base = WORKLOADS[args.workload]
    if args.steps is None:
        args.steps = base.steps
    if args.topk:
        result = topk_study(base, max(1, args.steps), args.warmup)
        if args.calibration_copy:
            calibration_copy()
        print(json.dumps(result), flush=True)
        return
    S = max(args.warmup + args.steps, 1)   # warm-up steps, then the timed ones
    Q = max(1, args.queries)
    cfg = base.scaled(steps=S) if S != base.steps else base
    if Q > 1:   # Q query tokens, each with the workload's k selections
        cfg = cfg.scaled(k=Q * base.k)
    host_flags = hb.HISPARSE_HOST_NONCOHERENT if args.host_noncoherent else hb.HISPARSE_HOST_COHERENT
    setup = Setup(cfg, host_flags, queries=Q, numa_node=args.numa_node, prefetch=not args.serial,
                  warmup=args.warmup)
    K, W = args.steps, args.warmup
    io = setup.noio if (args.no_io and args.only_timed) else setup.io
    if args.pipeline:
        try:
            print(json.dumps(pipeline_study(setup, K, args.heads)), flush=True)
        finally:
            setup.close()
        return
    if args.mla_attention:
        try:
            result = mla_study(setup, K, args.heads)
            if args.calibration_copy:
                calibration_copy()
            print(json.dumps(result), flush=True)
        finally:
            setup.close()
        return
    if args.prefetch_study:
        try:
            print(json.dumps(prefetch_study(setup, K, args.layer_compute_us, args.layer_compute,
                                            args.heads)), flush=True)
        finally:
            setup.close()
        return
    try:
        # ---- the W warm-up steps (0 .. W-1, the cold fill among them), then
        # a kernel-timing pass over steps W .. W+K-1: eager launches with the
        # library's timing events attached to each kernel's dispatch (events
        # cannot be recorded inside a captured graph) --------------------------
        base_tot = setup.warm(io)
        hb.hisparse_set_timing(io.h, True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(W, W + K):
            setup.step(io, s)
        torch.cuda.synchronize()
        elapsed_eager = time.perf_counter() - t0
        timing = hb.hisparse_get_timing(io.h)
        hb.hisparse_set_timing(io.h, False)
        end_tot = setup.totals(io)
        tot_miss, tot_evict, tot_hit = (int(x) for x in end_tot - base_tot)
        assert io.status() == 0, "device status word set during the benchmark"
        entries = K * cfg.layers * cfg.B * cfg.k
        miss_bytes = tot_miss * cfg.row_bytes
        log(f"eager: {K} steps after {W} warm-up steps in {elapsed_eager * 1e3:.2f} ms; misses "
            f"{tot_miss}, evictions {tot_evict}, hits {tot_hit}; kernel time resolve "
            f"{timing['resolve_ms']:.3f} ms / {timing['resolve_launches']}, fetch "
            f"{timing['fetch_ms']:.3f} ms / {timing['fetch_launches']}")

        # ---- the timed region: steps W .. W+K-1 (every layer's call) captured
        # as one HIP graph, as a decode graph holds them, replayed once after
        # the warm-up steps (and after one untimed replay) ---------------------
        graph_ev_ms = None
        if args.only_timed and not args.with_graph:
            elapsed = elapsed_eager
            mode = "eager, library kernel timing on"
        else:
            graph = capture_steps(setup, io, K, first=W)
            setup.warm(io)
            graph.replay()
            torch.cuda.synchronize()
            setup.warm(io)
            # HIP events on the stream the graph is launched on, around the
            # timed replay
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            ev0.record()
            graph.replay()
            ev1.record()
            torch.cuda.synchronize()
            elapsed = time.perf_counter() - t0
            graph_ev_ms = ev0.elapsed_time(ev1)
            assert io.status() == 0, "device status word set during the benchmark"
            assert tuple(int(x) for x in setup.totals(io)) == tuple(int(x) for x in end_tot), \
                "graph replay and eager pass disagree"
            del graph
            mode = (f"one HIP graph of steps {W} .. {W + K - 1}, one timed replay after the "
                    f"{W} warm-up steps" + (
                        "; every layer l+1 prefetched on a second stream (forked after layer l) "
                        "and joined by its resolve" if setup.prefetch else ""))
            log(f"timed: {K} steps in {elapsed * 1e3:.3f} ms (graph replay)")
        value = entries / elapsed

        if args.calibration_copy:
            calibration_copy()

        fused = timing["fetch_launches"] == 0
        resolve_avg_s = timing["resolve_ms"] / max(1, timing["resolve_launches"]) / 1e3
        # one launch per layer call (the resolve kernel, with the append fused
        # in when the context grows): then the timed graph holds nothing else.
        # The prefetch schedule adds a join launch per prefetched layer, so
        # there the eager pass's per-launch events are used.
        one_launch = fused and (not cfg.growth or cfg.R > 0) and not setup.prefetch
        launch_timing = "eager pass, library HIP events around each launch"
        if fused:   # the resolve workgroups copy their own misses
            fetch_avg_s = resolve_avg_s
            fetch_bytes_per_launch = miss_bytes / max(1, timing["resolve_launches"])
            if one_launch and graph_ev_ms is not None:
                fetch_avg_s = graph_ev_ms / 1e3 / (K * cfg.layers)
                launch_timing = ("timed region: HIP events on the launch stream around the graph "
                                 "replay, whose K x layers nodes are the resolve launches")
        else:
            fetch_avg_s = timing["fetch_ms"] / max(1, timing["fetch_launches"]) / 1e3
            fetch_bytes_per_launch = miss_bytes / max(1, timing["fetch_launches"])
        fetch_gbps = fetch_bytes_per_launch / fetch_avg_s / 1e9 if fetch_avg_s > 0 else 0.0
        # algorithmic metadata bytes per stream-step: sel + gathers + out +
        # LRU-order and slot2pos reads and rewrites + last_use stamps + per-miss
        # updates (position->slot clear/set, eviction log, miss list)
        n_calls = K * cfg.layers
        avg_miss = tot_miss / max(1, n_calls * cfg.B)
        avg_hit = tot_hit / max(1, n_calls * cfg.B)
        meta_bytes = cfg.B * (12 * cfg.k + 16 * cfg.C + 4 * (avg_hit + avg_miss) + 24 * avg_miss + 64)
        # the library's split fetch: sliced per stream below 8 streams per call
        dominant = ("resolve_kernel" if fused else
                    "fetch_stream_kernel" if cfg.B < 8 else "fetch_kernel")
        alg_traffic = 2 * fetch_bytes_per_launch + (meta_bytes if fused else 0)
        traffic = committed_traffic(dominant, cfg.label, "fused" if fused else "split")
        # counters are reported only when taken over the same K steps (from a
        # cold cache, no warm-up) and schedule as this run
        traffic_note = None
        n_launch = K * cfg.layers
        if traffic and not traffic_matches(traffic, K, W, n_launch, not setup.prefetch):
            traffic_note = (f"counter summaries were taken over other steps or another schedule "
                            f"({traffic['profiled']}); this run times {K} steps after {W} "
                            f"warm-up steps")
            traffic = None

        result = {
            "metric": "resolved top-k entries/s; miss-fetch GB/s vs host-link peak; no-IO overhead",
            "value": round(value, 1),
            "unit": "entries/s",
            "n_gpus": 1,
            "steps": K,
            "warmup": W,
            "ms_per_step": round(elapsed / K * 1e3, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "int32",
            "data": "synthetic",
            "config": {"workload": cfg.name, "requests": cfg.B, "layers": cfg.layers,
                       "context_rows": cfg.L0, "row_bytes": cfg.row_bytes, "cache_slots": cfg.C,
                       "resident_window": cfg.R, "top_k": cfg.k, "steps": K,
                       "carry_over_pct": cfg.carry_pct, "replacement": cfg.replacement,
                       "shared_selection": cfg.shared_selection,
                       "timed_steps": f"{W} .. {W + K - 1}, after {W} untimed warm-up steps "
                                      f"(step 0, the cold fill, among them)",
                       "schedule": "layer-wise prefetch" if setup.prefetch else "serial",
                       "timed_launch_mode": mode},
            "roofline": {"bound": "host_link", "kernel": dominant, "fused_fetch": fused,
                         "bound_note": "the miss fetch moves missed rows from pinned host memory "
                                       "over PCIe Gen5 x16; it is bound by that link, not by HBM "
                                       "(see traffic) or MFMA (none is used): peak = the link's "
                                       "64 GB/s, peak_measured = this host's measured H2D peak",
                         "achieved": round(fetch_gbps, 3), "peak": LINK_PEAK_THEORETICAL_GBPS,
                         "unit": "GB/s", "frac": round(fetch_gbps / LINK_PEAK_THEORETICAL_GBPS, 4),
                         "traffic": (round(traffic["FETCH_SIZE"] + traffic["WRITE_SIZE"])
                                     if traffic else None),
                         "traffic_read_bytes": round(traffic["FETCH_SIZE"]) if traffic else None,
                         "traffic_write_bytes": round(traffic["WRITE_SIZE"]) if traffic else None,
                         "per_launch_bytes": round(fetch_bytes_per_launch),
                         # what `traffic` counts, algorithmically: the missed rows read
                         # over the link and written to HBM, plus (fused) the metadata
                         "algorithmic_traffic_bytes": round(alg_traffic),
                         "traffic_over_algorithmic": (
                             round((traffic["FETCH_SIZE"] + traffic["WRITE_SIZE"]) / alg_traffic, 3)
                             if traffic else None),
                         "traffic_source": (
                             f"rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE summaries "
                             f"profiles/pmc_{{fetch,write}}_size_{cfg.label}_"
                             f"{'fused' if fused else 'split'}.md, the same {K} steps after {W} "
                             f"warm-up steps, scaled by the 256 MiB device copy"
                             if traffic else traffic_note),
                         "avg_launch_us": round(fetch_avg_s * 1e6, 3),
                         "launch_timing": launch_timing,
                         "avg_launch_us_eager": round(
                             (resolve_avg_s if fused else
                              timing["fetch_ms"] / max(1, timing["fetch_launches"]) / 1e3) * 1e6, 3)},
            "resolve_kernel": {"bound": "hbm", "per_launch_bytes": round(meta_bytes),
                               "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                               "note": "metadata only: the kernel timed on the instance "
                                       "that suppresses the row copies"},
            "miss_fetch": {"bytes": miss_bytes, "misses": tot_miss, "evictions": tot_evict,
                           "hits": tot_hit,
                           "GBps_over_fetch_kernels": round(fetch_gbps, 3),
                           "GBps_over_timed_region": round(miss_bytes / elapsed / 1e9, 3)},
            "host_memory": setup.host_memory,
            "eager": {"entries_per_s": round(entries / elapsed_eager, 1),
                      "ms_per_step": round(elapsed_eager / K * 1e3, 4),
                      "mode": "eager launches, library HIP-event timing on (the kernel-timing "
                              "pass behind the roofline figures)"},
        }

        if Q > 1:
            result["metric"] = "resolved query-token entries/s, several query tokens per step"
            result["config"]["queries"] = Q
            result["config"]["selections_per_query"] = cfg.k // Q
            result["config"]["top_k"] = cfg.k
            distinct = tot_hit + tot_miss
            result["multi_query"] = {
                "entries_per_request_step": cfg.k,
                "avg_distinct_nonresident_per_request_step": round(
                    distinct / max(1, K * cfg.layers * cfg.B), 1),
                "reading": "the union of the queries' selections is resolved once per layer "
                           "call; every entry is served its position's slot"}

        if not args.only_timed:
            # ---- graph replay, best of 3 (IO and no-IO) --------------------
            def graph_pass(inst):
                """Steps W .. W+K-1 in one HIP graph, replayed after the warm-up
                steps: best wall time and best HIP-event time (ms) of 3 replays."""
                g = capture_steps(setup, inst, K, first=W)
                setup.warm(inst)
                g.replay()                      # untimed replay
                torch.cuda.synchronize()
                best, best_ev = None, None
                for _ in range(3):
                    setup.warm(inst)
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    t0 = time.perf_counter()
                    e0.record()
                    g.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    dt = time.perf_counter() - t0
                    best = dt if best is None else min(best, dt)
                    ev = e0.elapsed_time(e1)
                    best_ev = ev if best_ev is None else min(best_ev, ev)
                assert inst.status() == 0
                return best, best_ev

            dt_io, _ = graph_pass(io)
            dt_noio, ev_noio_ms = graph_pass(setup.noio)
            # resolve kernel alone, copies suppressed: eager launches, HIP events
            setup.warm(setup.noio)
            hb.hisparse_set_timing(setup.noio.h, True)
            for s in range(W, W + K):
                setup.step(setup.noio, s)
            t_noio = hb.hisparse_get_timing(setup.noio.h)
            hb.hisparse_set_timing(setup.noio.h, False)
            noio_kernel_us = t_noio["resolve_ms"] / max(1, t_noio["resolve_launches"]) * 1e3
            rk = result["resolve_kernel"]
            # copies suppressed, every layer call is one launch (the append is
            # fused in when the context grows and a window exists): the graph's
            # nodes are the K x layers resolve launches
            if (not cfg.growth or cfg.R > 0) and not setup.prefetch:
                rk_us = ev_noio_ms * 1e3 / (K * cfg.layers)
                rk["launch_timing"] = ("HIP events around the copy-free graph replay (best of 3), "
                                       "whose K x layers nodes are the resolve launches")
            else:
                rk_us = noio_kernel_us
                rk["launch_timing"] = "eager pass, library HIP events around each launch"
            rk["avg_launch_us"] = round(rk_us, 3)
            rk["avg_launch_us_eager"] = round(noio_kernel_us, 3)
            rk["achieved"] = round(meta_bytes / (rk_us * 1e-6) / 1e9, 3)
            rk["frac"] = round(rk["achieved"] / HBM_PEAK_GBPS, 6)
            t_meta = committed_traffic("resolve_kernel", cfg.label, "noio")
            if t_meta and not traffic_matches(t_meta, K, W, K * cfg.layers, not setup.prefetch):
                t_meta = None
            rk["traffic"] = round(t_meta["FETCH_SIZE"] + t_meta["WRITE_SIZE"]) if t_meta else None
            rk["traffic_read_bytes"] = round(t_meta["FETCH_SIZE"]) if t_meta else None
            rk["traffic_write_bytes"] = round(t_meta["WRITE_SIZE"]) if t_meta else None
            per_call_us = dt_noio / (K * cfg.layers) * 1e6
            budget_us = DECODE_STEP_BUDGET_US / BUDGET_LAYERS * 0.05
            result["graph_replay"] = {"entries_per_s": round(entries / dt_io, 1),
                                      "ms_per_step": round(dt_io / K * 1e3, 4),
                                      "mode": "one HIP graph of all steps, best of 3"}
            result["no_io"] = {"us_per_layer_call": round(per_call_us, 3),
                               "resolve_kernel_us": round(noio_kernel_us, 3),
                               "includes_append": bool(cfg.growth),
                               "append": ("fused into the resolve launch" if cfg.growth and cfg.R > 0
                                          else "separate launch" if cfg.growth else None),
                               "target_us": budget_us,
                               "frac_of_decode_step_budget": round(
                                   per_call_us / (DECODE_STEP_BUDGET_US / BUDGET_LAYERS), 5),
                               "entries_per_s": round(entries / dt_noio, 1),
                               "mode": "one HIP graph of all steps, copies suppressed, best of 3"}
            io_minus_noio = dt_io - dt_noio
            result["miss_fetch"]["GBps_io_minus_noio"] = round(
                miss_bytes / io_minus_noio / 1e9, 3) if io_minus_noio > 0 else None
            result["no_io"]["us_per_step"] = round(dt_noio / K * 1e6, 3)
            result["no_io"]["step_budget_us"] = NOIO_STEP_BUDGET_US
            # ---- step 0 alone (the cold fill: about k misses per stream) ----
            def cold_step(inst):
                setup.reset(inst)
                g = capture_steps(setup, inst, 1)
                g.replay()
                torch.cuda.synchronize()
                best = None
                for _ in range(3):
                    setup.reset(inst)
                    t0 = time.perf_counter()
                    g.replay()
                    torch.cuda.synchronize()
                    dt = time.perf_counter() - t0
                    best = dt if best is None else min(best, dt)
                return best, int(setup.totals(inst)[0])
            dt0_io, miss0 = cold_step(io)
            dt0_noio, _ = cold_step(setup.noio)
            b0 = miss0 * cfg.row_bytes
            result["miss_fetch"]["cold_step"] = {
                "bytes": b0, "misses": miss0, "us": round(dt0_io * 1e6, 1),
                "us_no_io": round(dt0_noio * 1e6, 1),
                "GBps": round(b0 / dt0_io / 1e9, 3),
                "GBps_io_minus_noio": (round(b0 / (dt0_io - dt0_noio) / 1e9, 3)
                                       if dt0_io > dt0_noio else None),
                "mode": "step 0 alone from a cold cache, one HIP graph, best of 3"}
            if not args.no_probe:
                lp = link_probe(torch, hb, args.numa_node)
                result["link_peak"] = lp
                result["roofline"]["peak_measured"] = lp["measured_peak_GBps"]
                result["roofline"]["frac_of_measured"] = round(fetch_gbps / lp["measured_peak_GBps"], 4)
                cs = result["miss_fetch"]["cold_step"]
                cs["frac_of_measured"] = round(cs["GBps"] / lp["measured_peak_GBps"], 4)
            if setup.prefetch and not args.no_prefetch_study:
                # the pages' claim for shared selections: prefetching the next
                # layer during this layer's compute hides part of the misses
                result["prefetch"] = {
                    "stand_in_compute": prefetch_study(setup, K, args.layer_compute_us, "busy"),
                    "attention_compute": prefetch_study(setup, K, 0.0, "attention",
                                                        args.heads),
                    "no_compute": prefetch_study(setup, K, 0.0, "none")}
                log("prefetch study: hidden fraction {} (stand-in compute), {} (attention)".format(
                    result["prefetch"]["stand_in_compute"]["value"],
                    result["prefetch"]["attention_compute"]["value"]))
            if not args.no_cpu_baseline:
                result["cpu_baseline"] = cpu_baseline(setup, K, no_io_seconds=3.0)
                result["cpu_baseline_threads"] = cpu_baseline(
                    setup, K, threads=min(cfg.streams, len(os.sched_getaffinity(0))),
                    min_seconds=5.0)
    finally:
        setup.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
