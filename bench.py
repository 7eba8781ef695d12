"""Benchmark of the fused graph attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one pass of the whole path over one batch of synthetic input:
gattn_build_csr (COO -> CSR on the device) followed by gattn_forward (the
fused SDDMM / softmax / SpMM).  The default workload is the RTMScore-style
batch of 64 kNN graphs (8 heads x 16, fp32, clipped softmax with an edge
projection), the setting of the gattn-triton article's headline table.

Honest HBM numbers: the step cycles through R copies of the batch whose
total size is well above the 256 MB Infinity Cache, so every step streams
its inputs from HBM.  Before a timed region a sleep kernel holds the GPU
while the host enqueues all K steps, so the GPU then runs them back to back.
Two timed regions of K steps each: the first has events only at its two ends
and gives the throughput (an event recorded between kernels costs the GPU a
few microseconds, a fifth of a small step); the second records HIP events
around the CSR build and around the op of every step, and their averages give
the per-kernel durations of the roofline.

Output: one JSON line (metric, value in GEdges/s of the whole step, roofline
of the forward kernel against 8 TB/s HBM, the CPU oracle's rate on the host).

--variant picks what follows the CSR build (default: forward):
    e_out      the forward also writes the RTMScore per-edge update
    edge_ids   E stays in COO order and is read through the CSR's edge_perm
    aggregate  gattn_aggregate: V summed with seeded fp32 weights per edge and
               head, normalized by the summed weights + eps (no logits)

Counter mode (used under rocprofv3 --pmc, one counter per run):
    python bench.py --counters-run        one copy kernel of known size, then
                                          forward launches, no timing
    python bench.py --ingest-counters DIR summarise rocprofv3 CSVs into
                                          profiles/<kernel>_<workload>_counters.json
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused graph attention GEdges/s at 1 MI355X; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = {"gather": ["graph_sparse_attention_amd/csrc/gather_kernel.hpp",
                         "graph_sparse_attention_amd/csrc/forward_gather.hip",
                         "graph_sparse_attention_amd/csrc/forward_gather_split.hip"],
              "mfma": ["graph_sparse_attention_amd/csrc/forward_mfma.hip"]}
KERNEL_SRC["hybrid"] = KERNEL_SRC["mfma"] + KERNEL_SRC["gather"]
COPY_BYTES = 512 << 20      # calibration copy for the traffic counters
VARIANTS = {"forward": "gattn_forward", "e_out": "gattn_forward + edge update",
            "edge_ids": "gattn_forward, E through edge ids", "aggregate": "gattn_aggregate (normalized)"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=2,
                   help="1-5: the benchmark configurations; 6: the mixed-density batch of the hybrid dispatch")
    p.add_argument("--path", default="auto", choices=["auto", "gather", "mfma", "hybrid"])
    p.add_argument("--min-density", type=float, default=0.125, help="hybrid path: tile density of an MFMA window")
    p.add_argument("--variant", default="forward", choices=list(VARIANTS))
    p.add_argument("--partition", default="node", choices=["balanced", "node"],
                   help="gather path: edge-balanced workgroups with cut heavy rows (workspace) or equal node counts")
    p.add_argument("--pipeline", action="store_true",
                   help="build the CSR of batch i+1 on a second stream while batch i runs its forward")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="bound of the CPU oracle sample")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--counters-run", action="store_true")
    p.add_argument("--ingest-counters", default=None)
    return p.parse_args()


def src_hash(path_key):
    h = hashlib.sha256()
    for rel in KERNEL_SRC[path_key]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# workload and algorithmic bytes
# ---------------------------------------------------------------------------

def algorithmic_bytes(n, nnz, h, d, s, has_e, variant="forward"):
    """Compulsory HBM bytes of one launch: every input once, output once.
    forward:   B_min = 4(N+1) + 4 nnz + 3 N H D s + nnz H D s [E] + N H D s
    e_out:     B_min + nnz H D s (the edge update written)
    edge_ids:  B_min + 4 nnz (the id per edge)
    aggregate: 4(N+1) + 4 nnz + N H D s (x) + 4 nnz H (w) + N H D s (out)"""
    if variant == "aggregate":
        return 4 * (n + 1) + 4 * nnz + n * h * d * s + 4 * nnz * h + n * h * d * s
    b = 4 * (n + 1) + 4 * nnz + 3 * n * h * d * s + (nnz * h * d * s if has_e else 0) + n * h * d * s
    if variant == "e_out":
        b += nnz * h * d * s
    elif variant == "edge_ids":
        b += 4 * nnz
    return b


class Batch:
    def __init__(self, wl, dev, host, variant="forward", partition="node"):
        import torch
        import graph_sparse_attention_amd as gsa
        self.src = host["src"].to(dev)
        self.dst = host["dst"].to(dev)
        self.q, self.k, self.v = (host[x].to(dev) for x in ("q", "k", "v"))
        self.e = host["e"].to(dev) if host["e"] is not None else None
        self.out = torch.empty_like(self.q)
        self.w = host["w"].to(dev) if host.get("w") is not None else None
        self.e_out = torch.empty_like(self.e) if host.get("e_out") and self.e is not None else None
        self.csr = gsa.CsrBuilder(wl.num_nodes, wl.nnz, dev)
        self.rw = None
        self.hy = None
        self.ws = None
        if partition == "balanced":
            rp, ci = self.csr.row_ptr, self.csr.col_idx
            nbytes = (gsa.gattn_aggregate_workspace(rp, ci, self.v) if variant == "aggregate" else
                      gsa.gattn_forward_workspace(rp, ci, self.q, self.k, self.v, self.e, wl.mode,
                                                  e_out=self.e_out is not None))
            self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None


def make_host_inputs(wl, variant="forward"):
    import torch
    import workloads as W
    h = {"src": torch.from_numpy(wl.src), "dst": torch.from_numpy(wl.dst)}
    for x in ("q", "k", "v"):
        h[x] = W.cast(getattr(wl, x)(), wl.dtype)
    h["e"] = W.cast(wl.e(), wl.dtype) if wl.has_e else None
    if variant == "aggregate":
        h["w"] = torch.from_numpy(wl.w())
    h["e_out"] = variant == "e_out"
    return h


def batch_bytes(wl, es, variant="forward"):
    n, m, hd = wl.num_nodes, wl.nnz, wl.heads * wl.head_dim
    e = m * hd * es if wl.has_e else 0
    return 8 * m + 4 * n + 8 * m + 4 * n * hd * es + e * (2 if variant == "e_out" else 1) + \
        (4 * m * wl.heads if variant == "aggregate" else 0)


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def cpu_baseline(wl, host, seconds, variant="forward"):
    import oracle
    cores = len(os.sched_getaffinity(0))
    q64, k64, v64 = (oracle.widen(host[x]) for x in ("q", "k", "v"))
    e64 = oracle.widen(host["e"]) if host["e"] is not None else None
    w64 = host["w"].numpy().astype(np.float64) if variant == "aggregate" else None
    reps, t0 = 0, time.perf_counter()
    while True:
        rp, ci, pe = oracle.build_csr(wl.num_nodes, wl.src, wl.dst)
        if variant == "aggregate":
            oracle.aggregate(rp, ci, v64, w64, normalize=True, eps=wl.eps, threads=cores)
        else:
            oracle.forward(rp, ci, q64, k64, v64, e64, mode=wl.mode, scale=wl.scale, clip=wl.clip, eps=wl.eps,
                           threads=cores, edge_ids=pe if variant == "edge_ids" else None,
                           want_e_out=variant == "e_out")
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 100000:
            break
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(wl.nnz * reps / el / 1e9, 6), "unit": "GEdges/s", "cores": cores, "kind": "oracle",
            "sample": f"the full batch ({wl.nnz} edges), oracle CSR build (1 thread) + fp64 {VARIANTS[variant]} "
                      f"({cores} OpenMP threads), repeated {reps}x in {el:.1f} s; host CPU: {cpu_model}"}


# ---------------------------------------------------------------------------
# counters
# ---------------------------------------------------------------------------

def counters_file(path_key, config, variant="forward", partition="node"):
    suffix = ("" if variant == "forward" else f"_{variant}") + ("_balanced" if partition == "balanced" and path_key == "gather" else "")
    return os.path.join(PROFILES, f"forward_{path_key}_config{config}{suffix}_counters.json")


def load_traffic(path_key, config, variant="forward", partition="node"):
    f = counters_file(path_key, config, variant, partition)
    if not os.path.exists(f):
        return None
    d = json.load(open(f))
    if d.get("kernel_source_sha256_16") != src_hash(path_key):
        return None           # the kernel changed since the counters were taken
    return d


def ingest_counters(dirname, config, path_key, variant="forward", partition="node"):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the forward kernel
    and of the calibration copy; scale by the copy's bytes-per-count."""
    rows = []
    import csv
    for f in glob.glob(os.path.join(dirname, "**", "*counter_collection*.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no counter CSV under {dirname}")
    kerns = {"gather": ["gather_kernel"], "mfma": ["mfma_kernel"], "hybrid": ["mfma_kernel", "gather_kernel"]}[path_key]
    kern = " + ".join(kerns)
    acc = {}
    for r in rows:
        name = r.get("Kernel_Name", "")
        ctr = r.get("Counter_Name", "")
        val = float(r.get("Counter_Value", "nan"))
        key = "copy" if "copyBuffer" in name else next((k for k in kerns if k in name), None)
        if key is None or ctr not in ("FETCH_SIZE", "WRITE_SIZE"):
            continue
        acc.setdefault((key, ctr), []).append(val)
    # the calibration copy is the largest copyBuffer dispatch (the run also
    # makes small runtime copies, which would drag an average down); one
    # launch of the op is one dispatch of each of its kernels
    res = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        if ("copy", ctr) in acc:
            res["copy_" + ctr] = float(np.max(acc[("copy", ctr)]))
        if all((k, ctr) in acc for k in kerns):
            res["fwd_" + ctr] = float(sum(np.mean(acc[(k, ctr)]) for k in kerns))
    copy_read = res.get("copy_FETCH_SIZE")
    copy_write = res.get("copy_WRITE_SIZE")
    fr = COPY_BYTES / (copy_read * 1024.0) if copy_read else None
    fw = COPY_BYTES / (copy_write * 1024.0) if copy_write else None
    out = {"kernel": kern, "config": config, "variant": variant, "partition": partition if path_key == "gather" else None,
           "kernel_source_sha256_16": src_hash(path_key),
           "fetch_kib_per_dispatch": res.get("fwd_FETCH_SIZE"), "write_kib_per_dispatch": res.get("fwd_WRITE_SIZE"),
           "copy_fetch_kib": copy_read, "copy_write_kib": copy_write, "copy_bytes_each_way": COPY_BYTES,
           "read_scale": fr, "write_scale": fw,
           "commands": [f"rocprofv3 --pmc {ctr} -d {os.path.join(dirname, ctr.split('_')[0].lower())} -o run "
                        f"--output-format csv -- python -u bench.py --config {config} --path {path_key}"
                        + (f" --variant {variant}" if variant != "forward" else "")
                        + (" --partition balanced" if partition == "balanced" and path_key == "gather" else "")
                        + " --counters-run" for ctr in ("FETCH_SIZE", "WRITE_SIZE")]
                       + [f"python bench.py --config {config} --path {path_key}"
                          + (f" --variant {variant}" if variant != "forward" else "")
                          + (" --partition balanced" if partition == "balanced" and path_key == "gather" else "")
                          + f" --ingest-counters {dirname}"]}
    if res.get("fwd_FETCH_SIZE") is not None and fr and res.get("fwd_WRITE_SIZE") is not None and fw:
        out["hbm_bytes_per_launch"] = res["fwd_FETCH_SIZE"] * 1024.0 * fr + res["fwd_WRITE_SIZE"] * 1024.0 * fw
    os.makedirs(PROFILES, exist_ok=True)
    with open(counters_file(path_key, config, variant, partition), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the library has no multi-GPU path; "
              "each GPU would build and run the graphs of its own share of the batch.", file=sys.stderr)
        sys.exit(2)
    import workloads as W
    if args.ingest_counters:
        path_key = args.path if args.path in ("mfma", "hybrid") else "gather"
        ingest_counters(args.ingest_counters, args.config, path_key, args.variant, args.partition)
        return

    import torch
    import graph_sparse_attention_amd as gsa
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# generating workload config {args.config}", file=sys.stderr, flush=True)
    wl = W.make(args.config)
    if args.variant in ("e_out", "edge_ids") and not wl.has_e:
        sys.exit(f"--variant {args.variant} needs a workload with an edge tensor (config 2)")
    if args.variant == "e_out" and wl.mode != "clipped":
        sys.exit("--variant e_out needs the clipped softmax (config 2)")
    host = make_host_inputs(wl, args.variant)
    es = 4 if wl.dtype == "f32" else 2

    def run_op(b, rp, ci, pe):
        if args.variant == "aggregate":
            gsa.gattn_aggregate(rp, ci, b.v, b.w, normalize=True, eps=wl.eps, out=b.out, workspace=b.ws)
        else:
            gsa.gattn_forward(rp, ci, b.q, b.k, b.v, b.e, mode=wl.mode, scale=wl.scale, clip=wl.clip, eps=wl.eps,
                              path=args.path, rw=b.rw, out=b.out,
                              edge_ids=pe if args.variant == "edge_ids" else None, e_out=b.e_out,
                              workspace=b.ws, hybrid=b.hy)

    def plans(b, rp, ci):
        """Row windows (and the hybrid plan) once per graph: they synchronize,
        so they are built in the warmup, never inside the timed region."""
        if b.rw is None:
            b.rw = gsa.gattn_build_rowwindows(rp, ci, wl.num_nodes)
        if args.path == "hybrid" and b.hy is None:
            b.hy = gsa.gattn_build_hybrid(rp, ci, b.rw, b.q, min_density=args.min_density)

    if args.counters_run:
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)                      # calibration: COPY_BYTES read + COPY_BYTES written (runtime copyBuffer kernel)
        torch.cuda.synchronize()
        bt = Batch(wl, dev, host, args.variant, args.partition)
        rp, ci, pe = bt.csr(bt.src, bt.dst)
        if args.path in ("mfma", "hybrid"):
            plans(bt, rp, ci)
        for _ in range(5):
            run_op(bt, rp, ci, pe)
        torch.cuda.synchronize()
        print("# counters run done", file=sys.stderr, flush=True)
        return

    # R rotating copies so that one step's inputs are not cache-resident
    R = max(2, min(16, math.ceil(3 * MALL_BYTES / max(batch_bytes(wl, es, args.variant), 1)) + 1))
    print(f"# {wl.name}: N={wl.num_nodes} nnz={wl.nnz}; {R} rotating batches", file=sys.stderr, flush=True)
    batches = [Batch(wl, dev, host, args.variant, args.partition) for _ in range(R)]
    use_rw = args.variant == "forward" and (args.path in ("mfma", "hybrid") or (
        args.path == "auto" and wl.dtype != "f32" and wl.mode == "standard" and not wl.has_e))

    main_stream = torch.cuda.current_stream()
    side = torch.cuda.Stream() if args.pipeline else None        # default priority
    built = [torch.cuda.Event() for _ in range(R)]
    used = [torch.cuda.Event() for _ in range(R)]

    def step(i, ev=None):
        b = batches[i % R]
        if side is None:
            if ev is not None:
                ev[0].record()
            rp, ci, pe = b.csr(b.src, b.dst)
            if use_rw:
                plans(b, rp, ci)
            if ev is not None:
                ev[1].record()
            run_op(b, rp, ci, pe)
            if ev is not None:
                ev[2].record()
            return
        # pipelined: the side stream builds batch i's CSR once the forward that
        # last read this batch slot (step i - R) is done; the main stream waits
        # for the build, then runs the forward
        with torch.cuda.stream(side):
            side.wait_event(used[i % R])
            if ev is not None:
                ev[0].record(side)
            rp, ci, pe = b.csr(b.src, b.dst)
            if use_rw:
                plans(b, rp, ci)
            if ev is not None:
                ev[3].record(side)
            built[i % R].record(side)
        main_stream.wait_event(built[i % R])
        if ev is not None:
            ev[1].record(main_stream)
        run_op(b, rp, ci, pe)
        if ev is not None:
            ev[2].record(main_stream)
        used[i % R].record(main_stream)

    # warmup (also builds the row windows of every batch)
    for i in range(max(args.warmup, R)):
        step(i)
    torch.cuda.synchronize()
    for b in batches:
        assert int(b.csr.status.item()) == 0, "bad graph"
    path = "gather" if args.variant == "aggregate" else gsa.gattn_forward_path(batches[0].csr.row_ptr, batches[0].csr.col_idx, batches[0].q, batches[0].k,
                                  batches[0].v, batches[0].e, mode=wl.mode, path=args.path, rw=batches[0].rw,
                                  hybrid=batches[0].hy)

    # host enqueue rate, to size the sleep that keeps the GPU backlogged
    t0 = time.perf_counter()
    for i in range(R):
        step(i)
    enqueue_s = (time.perf_counter() - t0) / R
    torch.cuda.synchronize()

    K = args.steps

    def timed(evs):
        """K steps behind a sleep that lasts until the host has enqueued them
        all; returns the start-to-end time of the K steps in ms."""
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        sleep_s = 1.5 * enqueue_s * K + 2e-3
        torch.cuda._sleep(int(sleep_s * 2.4e9))
        start.record()
        if side is not None:
            side.wait_event(start)      # no build starts before the timed region
        for i in range(K):
            step(i, evs[i] if evs else None)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    # throughput: the K steps alone (an event record between kernels costs the
    # GPU several microseconds, so the per-kernel events get their own run)
    total_ms = timed(None)
    # kernel durations: the same K steps with events around the build and the op
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    evented_ms = timed(evs)
    build_ms = float(np.mean([e[0].elapsed_time(e[3] if side is not None else e[1]) for e in evs]))
    fwd_ms_all = np.array([e[1].elapsed_time(e[2]) for e in evs])
    fwd_ms = float(np.mean(fwd_ms_all))
    ms_per_step = total_ms / K

    nnz = wl.nnz
    bmin = algorithmic_bytes(wl.num_nodes, nnz, wl.heads, wl.head_dim, es, wl.has_e, args.variant)
    achieved = bmin / (fwd_ms * 1e-3) / 1e9
    pk = path if path in ("mfma", "hybrid") else "gather"
    tr = load_traffic(pk, args.config, args.variant, args.partition)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": (round(tr["hbm_bytes_per_launch"]) if tr and tr.get("hbm_bytes_per_launch") else None),
                "kernel": {"gather": "gather_kernel", "mfma": "mfma_kernel", "hybrid": "mfma_kernel + gather_kernel"}[pk],
                "algorithmic_bytes_per_launch": bmin, "bytes_per_edge": round(bmin / nnz, 2),
                "kernel_ms": round(fwd_ms, 5), "kernel_ms_median": round(float(np.median(fwd_ms_all)), 5),
                "kernel_ms_min": round(float(fwd_ms_all.min()), 5)}
    res = {"metric": METRIC, "value": round(nnz / (ms_per_step * 1e-3) / 1e9, 4), "unit": "GEdges/s",
           "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
           "data": "synthetic",
           "config": {"workload": wl.name, "config_index": args.config, "nodes": wl.num_nodes, "edges": nnz,
                      "heads": wl.heads, "head_dim": wl.head_dim,
                      "softmax": "none (given weights)" if args.variant == "aggregate" else wl.mode,
                      "edge_projection": wl.has_e and args.variant != "aggregate",
                      "step": f"gattn_build_csr + {VARIANTS[args.variant]}", "variant": args.variant,
                      "pipeline": ("CSR build of batch i+1 on a second stream during the forward of batch i"
                                   if side is not None else None),
                      "partition": args.partition if path == "gather" else None,
                      "forward_path": path,
                      "rotating_batches": R},
           "roofline": roofline,
           "forward_gedges_per_s": round(nnz / (fwd_ms * 1e-3) / 1e9, 4),
           "gedge_heads_per_s": round(nnz * wl.heads / (ms_per_step * 1e-3) / 1e9, 4),
           "ms_per_step_with_kernel_events": round(evented_ms / K, 5),
           "build_csr_ms": round(build_ms, 5)}
    if not args.no_cpu:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, host, args.cpu_seconds, args.variant)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
