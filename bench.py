"""Benchmark of the fused graph attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4]

A step is one gattn_forward (the fused SDDMM / softmax / SpMM) over one
batch of synthetic input whose CSR was built on the device beforehand: the
CSR build runs once per graph and is timed on its own (``build_csr_ms``), as
the gattn-triton article builds its CSC index outside the timed kernel.
``--include-build`` times gattn_build_csr + gattn_forward per step instead.
The default workload is the largest configuration that fits one GPU: the
power-law graph of 2.45M destinations and 101M edges (lognormal in-degree,
uniform sources), one head of 64, bf16, standard softmax.  K and V sit in
one [N, 2, H, D] buffer, as a layer's fused K|V projection writes them
(``--kv-layout separate`` gives two packed tensors instead); the op reads them
as two row views, and the gathered bytes per edge are the same either way.

Honest HBM numbers: the step cycles through R copies of the batch whose
total size is well above the 256 MB Infinity Cache, so every step streams
its inputs from HBM.  Before a timed region a sleep kernel holds the GPU
while the host enqueues all K steps, so the GPU then runs them back to back.
Two timed regions of K steps each: the first has events only at its two ends
and gives the throughput (an event recorded between kernels costs the GPU a
few microseconds, a fifth of a small step); the second records HIP events
around the op of every step, and their averages give the kernel duration of
the roofline.

Output: one JSON line (metric, value in GEdges/s, the roofline of the
forward kernel against 8 TB/s HBM with both byte models, the counter-measured
HBM traffic when a profile of this kernel source is committed, and the CPU
oracle on one thread and on every core of the host, whose outputs also check
the rows of the timed GPU output they cover: the run fails on a mismatch).

--partition picks the gather path's workgroup partition (default auto: the
balanced one when the largest in-degree is above 32x the mean on a graph
below 2^24 edges, the rule of the Python graph layer; else equal node counts).

--variant picks the op (default: forward):
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
    p.add_argument("--config", type=int, default=4,
                   help="1-5: the benchmark configurations; 6: the mixed-density batch of the hybrid dispatch")
    p.add_argument("--path", default="auto", choices=["auto", "gather", "mfma", "hybrid"])
    p.add_argument("--min-density", type=float, default=0.09, help="hybrid path: tile density of an MFMA window")
    p.add_argument("--variant", default="forward", choices=list(VARIANTS))
    p.add_argument("--partition", default="auto", choices=["auto", "balanced", "node"],
                   help="gather path: edge-balanced workgroups with cut heavy rows (workspace), equal node "
                        "counts, or auto: the graph layer's rule (balanced when the largest in-degree is above "
                        "32x the mean on a graph below 2^24 edges)")
    p.add_argument("--include-build", action="store_true",
                   help="a step is gattn_build_csr + the op (default: the op on a CSR built once per batch)")
    p.add_argument("--pipeline", action="store_true",
                   help="with --include-build: build the CSR of batch i+1 on a second stream while batch i runs")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="single-thread oracle time the CPU sample is sized for")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle (and with it the parity check)")
    p.add_argument("--eager", action="store_true",
                   help="also time an eager PyTorch formulation of the same forward (context only)")
    p.add_argument("--ceiling", action="store_true",
                   help="gather rate against the size of the gathered table (graphs shaped like config 4)")
    p.add_argument("--kv-layout", default="interleaved", choices=["separate", "interleaved"],
                   help="K and V as the halves of one [N, 2, H, D] buffer, as one fused K|V projection "
                        "writes them (row views with a row stride of 2 H D: a row's K and V bytes adjacent), "
                        "or as two packed [N, H, D] tensors")
    p.add_argument("--counters-run", action="store_true")
    p.add_argument("--ingest-counters", default=None)
    args = p.parse_args()
    if args.pipeline and not args.include_build:
        p.error("--pipeline overlaps CSR builds with forwards: it needs --include-build")
    return args


def src_hash(path_key):
    """Hash of the kernel sources' code: line comments, trailing blanks and
    empty lines are left out, so that an edit of a comment does not mark the
    committed counters as taken on another kernel."""
    h = hashlib.sha256()
    for rel in KERNEL_SRC[path_key]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# workload and algorithmic bytes
# ---------------------------------------------------------------------------

def algorithmic_bytes(n, nnz, h, d, s, has_e, variant="forward"):
    """B_min, the compulsory HBM bytes of one launch: every input once, the
    output once.
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


def gather_bytes(n, nnz, h, d, s, has_e, variant="forward"):
    """B_gather, the bytes of the method as the pages state it: every edge
    loads its source's K and V rows (V only for the aggregation, with the
    edge's weights) and its E row; Q is read and O written once per node.
    B_gather = 4(N+1) + nnz (4 + 2 H D s + H D s [E]) + 2 N H D s."""
    if variant == "aggregate":
        return 4 * (n + 1) + nnz * (4 + h * d * s + 4 * h) + n * h * d * s
    b = 4 * (n + 1) + nnz * (4 + 2 * h * d * s + (h * d * s if has_e else 0)) + 2 * n * h * d * s
    if variant == "e_out":
        b += nnz * h * d * s
    elif variant == "edge_ids":
        b += 4 * nnz
    return b


def roofline_basis(n, h, d, s, variant="forward"):
    """Which byte model is the algorithmic one.  When the rows the edges
    gather (K and V, or X for the aggregation) exceed the 256 MB Infinity
    Cache, the last level of cache on the chip, and the sources are spread
    over the whole table, each edge's rows have to come over the memory
    fabric: B_gather is what the method moves.  When they fit, a row can be
    served on chip after its first fetch, and B_min is the floor."""
    table = (1 if variant == "aggregate" else 2) * n * h * d * s
    return "gather" if table > MALL_BYTES else "min"


class Batch:
    def __init__(self, wl, dev, host, variant="forward", partition="node", kv_layout="interleaved"):
        import torch
        import graph_sparse_attention_amd as gsa
        self.src = host["src"].to(dev)
        self.dst = host["dst"].to(dev)
        self.q, self.k, self.v = (host[x].to(dev) for x in ("q", "k", "v"))
        if kv_layout == "interleaved" and variant != "aggregate":
            # one [N, 2, H, D] buffer; k and v are its halves (row stride 2 H D)
            kv = torch.stack((self.k, self.v), dim=1)
            self.k, self.v = kv[:, 0], kv[:, 1]
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


def resolve_partition(wl):
    """The gather partition the graph layer picks for this workload's graph."""
    import graph_sparse_attention_amd as gsa
    max_degree = int(np.bincount(wl.dst, minlength=wl.num_nodes).max()) if wl.nnz else 0
    return "balanced" if gsa.Graph.skewed_degrees(wl.num_nodes, wl.nnz, max_degree) else "node"


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

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def parity_of(y, ref, mag, dtype):
    """The parity bounds of the test suite on the sampled rows: fp32
    componentwise |y - y*| / max(|y*|, S) <= 1e-5; fp16 / bf16 relative L2
    over the sample <= 2e-3 / 8e-3 and per element |y - y*| <= 4u max(|y*|, S)
    + f (u = 2^-11 / 2^-8, f = 2^-25 / 2^-134); rows without in-edges exactly
    0.  Returns the figures and whether they pass."""
    y, ref, mag = (np.asarray(x, np.float64) for x in (y, ref, mag))
    scale = np.maximum(np.abs(ref), mag)
    zero = scale == 0
    res = {"zero_rows_exact": bool(np.all(y[zero] == 0.0))}
    ok = res["zero_rows_exact"]
    if dtype == "f32":
        err = float((np.abs(y - ref)[~zero] / scale[~zero]).max()) if (~zero).any() else 0.0
        res["fp32_componentwise"] = err
        return res, ok and err <= 1e-5
    u, f, tol = {"f16": (2.0 ** -11, 2.0 ** -25, 2e-3), "bf16": (2.0 ** -8, 2.0 ** -134, 8e-3)}[dtype]
    nr = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(y - ref) / nr) if nr > 0 else 0.0
    elem = float((np.abs(y - ref) / (4.0 * u * scale + f)).max()) if y.size else 0.0
    res.update({"rel_l2": rel, "element_of_bound": elem})
    return res, ok and rel <= tol and elem <= 1.0


def cpu_baseline(wl, host, gpu_out, seconds, variant="forward"):
    """The oracle (fp64, plain loops) on the host cores: its CSR build, then
    the op on a sample of destinations, once on one thread and repeatedly on
    every core of the process's affinity mask (OpenMP over destinations;
    identical bits).  The sample is the 64 highest-degree destinations plus
    a leading block of rows sized for about `seconds` of single-thread work,
    or the whole batch when that is less.  The same oracle outputs check the
    sampled rows of the GPU output of the timed region."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    n = wl.num_nodes
    t0 = time.perf_counter()
    rp, ci, pe = oracle.build_csr(n, wl.src, wl.dst)
    t_build = time.perf_counter() - t0
    deg = np.diff(rp.astype(np.int64))
    q64, k64, v64 = (oracle.widen(host[x]) for x in ("q", "k", "v"))
    e64 = oracle.widen(host["e"]) if host["e"] is not None else None

    def run(rows, threads):
        if variant == "aggregate":
            w64 = host["w"].numpy().astype(np.float64)
            out = oracle.aggregate(rp, ci, v64, w64, normalize=True, eps=wl.eps, threads=threads)
            mag = oracle.aggregate(rp, ci, np.abs(v64), np.abs(w64), normalize=True, eps=wl.eps, threads=threads)
            return out[rows], mag[rows]
        return oracle.forward(rp, ci, q64, k64, v64, e64, mode=wl.mode, scale=wl.scale, clip=wl.clip, eps=wl.eps,
                              rows=rows, want_mag=True, threads=threads,
                              edge_ids=pe if variant == "edge_ids" else None)

    if variant == "aggregate":
        rows = np.arange(n, dtype=np.int32)          # the oracle's aggregation has no row subset
    else:
        # calibrate the single-thread rate on a probe of about 200k edges
        probe = np.arange(int(np.searchsorted(np.cumsum(deg), 200_000)) + 1, dtype=np.int32)[:n]
        t0 = time.perf_counter()
        run(probe, 1)
        rate = max(deg[probe].sum(), 1) / max(time.perf_counter() - t0, 1e-6)
        lead = int(np.searchsorted(np.cumsum(deg), rate * seconds)) + 1
        if lead >= n:
            rows = np.arange(n, dtype=np.int32)
        else:
            hubs = np.argsort(deg, kind="stable")[-64:]
            rows = np.unique(np.concatenate([np.arange(lead), hubs])).astype(np.int32)
    edges = int(deg[rows].sum())
    t0 = time.perf_counter()
    ref, mag = run(rows, 1)
    t1 = time.perf_counter() - t0
    reps, t0 = 0, time.perf_counter()
    while True:
        ref_mt, _ = run(rows, cores)
        reps += 1
        tm = time.perf_counter() - t0
        if tm >= 2.0 or reps >= 1000:
            break
    assert np.array_equal(ref, ref_mt), "the oracle's result depends on its thread count"
    y = gpu_out.detach().float().cpu().double().numpy()[rows]
    figures, ok = parity_of(y, ref, mag, wl.dtype)
    sample = (f"{'all' if rows.shape[0] == n else rows.shape[0]} of {n} destinations"
              + ("" if rows.shape[0] == n else " (a leading block + the 64 highest in-degrees)")
              + f", {edges} of {wl.nnz} edges; fp64 {VARIANTS[variant]}; one thread once ({t1:.2f} s), "
              f"{cores} OpenMP threads {reps}x ({tm:.2f} s); oracle CSR build of the whole batch "
              f"{t_build:.2f} s (1 thread); host CPU: {cpu_model()}")
    base = {"value": round(edges * reps / tm / 1e9, 6), "unit": "GEdges/s", "cores": cores, "kind": "oracle",
            "sample": sample, "value_1_thread": round(edges / t1 / 1e9, 6), "csr_build_s_1_thread": round(t_build, 3)}
    check = {"rows": int(rows.shape[0]), "edges": edges, "passed": bool(ok), **figures}
    return base, check


# ---------------------------------------------------------------------------
# eager PyTorch context
# ---------------------------------------------------------------------------

def eager_forward(torch, dst, src, q, k, v, e, mode, scale, clip, eps):
    """The forward as separate PyTorch ops on per-edge tensors, in the order
    the gattn-triton article's eager reference takes (gather the endpoint
    rows, the logit, clamp and exp or a max-subtracted exp, scatter-add the
    weights and the weighted rows, divide): a timing context for the fused
    kernel, never a result of the library and never used for parity."""
    N, H, D = q.shape
    if mode == "clipped":
        t = (q[dst] * k[src] * scale).clamp(clip[0], clip[1])
        if e is not None:
            t = t * e
        w = t.sum(-1).clamp(clip[0], clip[1]).exp()
        den = torch.zeros((N, H), dtype=w.dtype, device=q.device).index_add_(0, dst, w) + eps
    else:
        t = q[dst] * k[src]
        if e is not None:
            t = t * e
        lg = t.sum(-1) * scale
        mx = torch.full((N, H), float("-inf"), dtype=lg.dtype, device=q.device)
        mx = mx.scatter_reduce(0, dst[:, None].expand(-1, H), lg, "amax", include_self=True)
        w = (lg - mx[dst]).exp()
        den = torch.zeros((N, H), dtype=w.dtype, device=q.device).index_add_(0, dst, w)
        den = torch.where(den > 0, den, torch.ones_like(den))
    num = torch.zeros((N, H, D), dtype=v.dtype, device=q.device).index_add_(0, dst, w[..., None] * v[src])
    return num / den[..., None]


def eager_context(torch, wl, b, fwd_ms_median, reps=20):
    rp, ci = b.csr.row_ptr, b.csr.col_idx
    deg = (rp[1:] - rp[:-1]).long()
    dst = torch.repeat_interleave(torch.arange(wl.num_nodes, device=rp.device), deg)
    src = ci.long()
    f = lambda: eager_forward(torch, dst, src, b.q, b.k, b.v, b.e, wl.mode, wl.scale, wl.clip, wl.eps)
    for _ in range(3):
        y = f()
    ts = []
    for _ in range(reps):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        f()
        a1.record()
        torch.cuda.synchronize()
        ts.append(a0.elapsed_time(a1))
    ms = float(np.median(ts))
    diff = float((y.float() - b.out.float()).abs().max())
    return {"ms_median": round(ms, 5), "speedup_of_fused": round(ms / fwd_ms_median, 2),
            "max_abs_diff_to_fused": diff, "reps": reps,
            "formulation": "per-edge gather, logit, exp, index_add_ of weights and weighted rows, divide "
                           "(PyTorch ops in the input dtype, same device, same CSR)"}


# ---------------------------------------------------------------------------
# counters
# ---------------------------------------------------------------------------

def counters_file(path_key, config, variant="forward", partition="node", kv_layout="interleaved"):
    suffix = (("" if variant == "forward" else f"_{variant}") + ("_balanced" if partition == "balanced" and path_key == "gather" else "")
              + ("_kv_separate" if kv_layout == "separate" else ""))
    return os.path.join(PROFILES, f"forward_{path_key}_config{config}{suffix}_counters.json")


def load_traffic(path_key, config, variant="forward", partition="node", kv_layout="interleaved"):
    f = counters_file(path_key, config, variant, partition, kv_layout)
    if not os.path.exists(f):
        return None
    d = json.load(open(f))
    if d.get("kernel_source_sha256_16") != src_hash(path_key):
        return None           # the kernel changed since the counters were taken
    return d


def counter_commands(dirname, config, path_key, variant, partition, kv_layout="interleaved"):
    """The runs behind a counter file: from /tmp with TMPDIR=/tmp, R = the
    repository root, one run per counter, the CSVs under DIR/FETCH and
    DIR/WRITE, then the ingestion from the repository root."""
    args = (f"--config {config} --path {path_key}" + (f" --variant {variant}" if variant != "forward" else "")
            + (f" --partition {partition}" if path_key == "gather" else "")
            + (" --kv-layout separate" if kv_layout == "separate" else ""))
    rel = os.path.relpath(os.path.abspath(dirname), ROOT)
    return ([f"rocprofv3 --pmc {ctr} -d $R/{rel}/{ctr.split('_')[0]} -o run --output-format csv -- "
             f"python3 -u $R/bench.py {args} --counters-run" for ctr in ("FETCH_SIZE", "WRITE_SIZE")]
            + [f"python3 bench.py {args} --ingest-counters {rel}"])


def ingest_counters(dirname, config, path_key, variant="forward", partition="node", kv_layout="interleaved"):
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
           "kv_layout": kv_layout,
           "kernel_source_sha256_16": src_hash(path_key),
           "fetch_kib_per_dispatch": res.get("fwd_FETCH_SIZE"), "write_kib_per_dispatch": res.get("fwd_WRITE_SIZE"),
           "copy_fetch_kib": copy_read, "copy_write_kib": copy_write, "copy_bytes_each_way": COPY_BYTES,
           "read_scale": fr, "write_scale": fw,
           "commands": counter_commands(dirname, config, path_key, variant, partition, kv_layout)}
    if res.get("fwd_FETCH_SIZE") is not None and fr and res.get("fwd_WRITE_SIZE") is not None and fw:
        out["hbm_bytes_per_launch"] = res["fwd_FETCH_SIZE"] * 1024.0 * fr + res["fwd_WRITE_SIZE"] * 1024.0 * fw
    os.makedirs(PROFILES, exist_ok=True)
    with open(counters_file(path_key, config, variant, partition, kv_layout), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


# ---------------------------------------------------------------------------

def ceiling():
    """The gather kernel on graphs shaped like config 4 (2.45M destinations of
    in-degree 41, H = 1, D = 64, bf16, standard softmax) whose sources are
    drawn uniformly from the first S nodes, S chosen so that the K and V rows
    that can be gathered take 16 MB ... 627 MB (all nodes): the rate of the
    gathered rows (B_gather per launch over the mean launch time) against the
    size of the table they come from.  If the caches on the chip served random
    128-byte rows faster than HBM, the smaller tables would run faster."""
    import torch
    import graph_sparse_attention_amd as gsa
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    N, deg, D = 2_450_000, 41, 64
    nnz = N * deg
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    q, k, v = (torch.randn(N, 1, D, device=dev, generator=g).to(torch.bfloat16) for _ in range(3))
    out = torch.empty_like(q)
    dst = torch.arange(N, device=dev, dtype=torch.int32).repeat_interleave(deg)
    rows = []
    for table_mb in (16, 32, 64, 128, 256, 627):
        S = min(N, (table_mb << 20) // (2 * D * 2 * 1))  # K and V: 2 D bytes each per node
        src = torch.randint(0, S, (nnz,), device=dev, dtype=torch.int32, generator=g)
        rp, ci, _ = gsa.gattn_build_csr(src, dst, N)
        del src
        f = lambda: gsa.gattn_forward(rp, ci, q, k, v, scale=1 / math.sqrt(D), path="gather", out=out)
        for _ in range(3):
            f()
        ts = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        t = sum(ts) / len(ts)
        b_gather = nnz * 2 * D * 2
        rows.append({"table_mb": round(S * 4 * D / 2**20, 1), "sources": S, "ms": round(t * 1e3, 4),
                     "gathered_tb_s": round(b_gather / t / 1e12, 3), "frac_gather": round(b_gather / t / 8e12, 4)})
        print(f"# K/V table {rows[-1]['table_mb']} MB ({S} sources): {t * 1e3:.3f} ms, "
              f"{b_gather / t / 1e12:.2f} TB/s of gathered rows", file=sys.stderr, flush=True)
        del rp, ci
    print(json.dumps({"ceiling": rows, "edges": nnz, "destinations": N}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the library has no multi-GPU path; "
              "each GPU would build and run the graphs of its own share of the batch.", file=sys.stderr)
        sys.exit(2)
    if args.ceiling:
        ceiling()
        return
    import workloads as W
    wl = None
    if args.partition == "auto":
        print(f"# generating workload config {args.config}", file=sys.stderr, flush=True)
        wl = W.make(args.config)
        args.partition = resolve_partition(wl)
    if args.ingest_counters:
        path_key = args.path if args.path in ("mfma", "hybrid") else "gather"
        ingest_counters(args.ingest_counters, args.config, path_key, args.variant, args.partition, args.kv_layout)
        return

    import torch
    import graph_sparse_attention_amd as gsa
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if wl is None:
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
        so they are built before any timed region."""
        if b.rw is None:
            b.rw = gsa.gattn_build_rowwindows(rp, ci, wl.num_nodes)
        if args.path == "hybrid" and b.hy is None:
            b.hy = gsa.gattn_build_hybrid(rp, ci, b.rw, b.q, min_density=args.min_density)

    use_rw = args.variant == "forward" and (args.path in ("mfma", "hybrid") or (
        args.path == "auto" and wl.dtype != "f32" and wl.mode == "standard" and not wl.has_e))

    if args.counters_run:
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)                      # calibration: COPY_BYTES read + COPY_BYTES written (runtime copyBuffer kernel)
        torch.cuda.synchronize()
        bt = Batch(wl, dev, host, args.variant, args.partition, args.kv_layout)
        rp, ci, pe = bt.csr(bt.src, bt.dst)
        if use_rw:
            plans(bt, rp, ci)
        for _ in range(5):
            run_op(bt, rp, ci, pe)
        torch.cuda.synchronize()
        print("# counters run done", file=sys.stderr, flush=True)
        return

    # R rotating copies so that one step's inputs are not cache-resident
    R = max(2, min(16, math.ceil(3 * MALL_BYTES / max(batch_bytes(wl, es, args.variant), 1)) + 1))
    print(f"# {wl.name}: N={wl.num_nodes} nnz={wl.nnz}; {R} rotating batches", file=sys.stderr, flush=True)
    batches = [Batch(wl, dev, host, args.variant, args.partition, args.kv_layout) for _ in range(R)]
    for b in batches:               # each batch's CSR once (rebuilt per step with --include-build)
        b.csr(b.src, b.dst)
        if use_rw:
            plans(b, b.csr.row_ptr, b.csr.col_idx)
    torch.cuda.synchronize()
    for b in batches:
        assert int(b.csr.status.item()) == 0, "bad graph"

    main_stream = torch.cuda.current_stream()
    side = torch.cuda.Stream() if args.pipeline else None        # default priority
    built = [torch.cuda.Event() for _ in range(R)]
    used = [torch.cuda.Event() for _ in range(R)]

    def step(i, ev=None):
        b = batches[i % R]
        if not args.include_build:
            if ev is not None:
                ev[1].record()
            run_op(b, b.csr.row_ptr, b.csr.col_idx, b.csr.edge_perm)
            if ev is not None:
                ev[2].record()
            return
        if side is None:
            if ev is not None:
                ev[0].record()
            rp, ci, pe = b.csr(b.src, b.dst)
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

    for i in range(max(args.warmup, R)):
        step(i)
    torch.cuda.synchronize()
    path = "gather" if args.variant == "aggregate" else gsa.gattn_forward_path(
        batches[0].csr.row_ptr, batches[0].csr.col_idx, batches[0].q, batches[0].k, batches[0].v, batches[0].e,
        mode=wl.mode, path=args.path, rw=batches[0].rw, hybrid=batches[0].hy)

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

    print(f"# timing {K} steps", file=sys.stderr, flush=True)
    # throughput: the K steps alone (an event record between kernels costs the
    # GPU several microseconds, so the per-kernel events get their own run)
    total_ms = timed(None)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    evented_ms = timed(evs)
    fwd_ms_all = np.array([e[1].elapsed_time(e[2]) for e in evs])
    fwd_ms = float(np.mean(fwd_ms_all))
    ms_per_step = total_ms / K
    if args.include_build:
        build_ms = float(np.mean([e[0].elapsed_time(e[3] if side is not None else e[1]) for e in evs]))
    else:
        # the once-per-graph CSR build, timed on its own: events around each of
        # a few builds of the rotating batches
        nb = max(3, min(20, K // 10))
        bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nb)]
        torch.cuda.synchronize()
        for i in range(nb):
            b = batches[i % R]
            bev[i][0].record()
            b.csr(b.src, b.dst)
            bev[i][1].record()
        torch.cuda.synchronize()
        build_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in bev]))
        for i in range(R):            # outputs of the timed op again, on the rebuilt CSR
            step(i)
        torch.cuda.synchronize()

    nnz = wl.nnz
    bmin = algorithmic_bytes(wl.num_nodes, nnz, wl.heads, wl.head_dim, es, wl.has_e, args.variant)
    bgat = gather_bytes(wl.num_nodes, nnz, wl.heads, wl.head_dim, es, wl.has_e, args.variant)
    basis = roofline_basis(wl.num_nodes, wl.heads, wl.head_dim, es, args.variant)
    balg = bgat if basis == "gather" else bmin
    achieved = balg / (fwd_ms * 1e-3) / 1e9
    pk = path if path in ("mfma", "hybrid") else "gather"
    tr = load_traffic(pk, args.config, args.variant, args.partition, args.kv_layout)
    traffic = round(tr["hbm_bytes_per_launch"]) if tr and tr.get("hbm_bytes_per_launch") else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": {"gather": "gather_kernel", "mfma": "mfma_kernel", "hybrid": "mfma_kernel + gather_kernel"}[pk],
                "basis": ("B_gather: the K and V rows of every edge (the gathered table exceeds the 256 MB "
                          "Infinity Cache)" if basis == "gather" else "B_min: every input once, the output once"),
                "algorithmic_bytes_per_launch": balg, "bytes_per_edge": round(balg / nnz, 2),
                "b_min": bmin, "b_gather": bgat,
                "frac_min": round(bmin / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "frac_gather": round(bgat / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "counter_gbs": round(traffic / (fwd_ms * 1e-3) / 1e9, 1) if traffic else None,
                "counter_frac": round(traffic / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if traffic else None,
                "kernel_ms": round(fwd_ms, 5), "kernel_ms_median": round(float(np.median(fwd_ms_all)), 5),
                "kernel_ms_min": round(float(fwd_ms_all.min()), 5)}
    op = VARIANTS[args.variant]
    res = {"metric": METRIC, "value": round(nnz / (ms_per_step * 1e-3) / 1e9, 4), "unit": "GEdges/s",
           "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
           "data": "synthetic",
           "config": {"workload": wl.name, "config_index": args.config, "nodes": wl.num_nodes, "edges": nnz,
                      "heads": wl.heads, "head_dim": wl.head_dim,
                      "softmax": "none (given weights)" if args.variant == "aggregate" else wl.mode,
                      "edge_projection": wl.has_e and args.variant != "aggregate",
                      "step": f"gattn_build_csr + {op}" if args.include_build else
                              f"{op} (CSR built on the device once per batch, timed apart)",
                      "variant": args.variant,
                      "pipeline": ("CSR build of batch i+1 on a second stream during the forward of batch i"
                                   if side is not None else None),
                      "partition": args.partition if path == "gather" else None,
                      "kv_layout": args.kv_layout if args.variant != "aggregate" else None,
                      "forward_path": path,
                      "rotating_batches": R},
           "roofline": roofline,
           "forward_gedges_per_s": round(nnz / (fwd_ms * 1e-3) / 1e9, 4),
           "gedge_heads_per_s": round(nnz * wl.heads / (ms_per_step * 1e-3) / 1e9, 4),
           "ms_per_step_with_kernel_events": round(evented_ms / K, 5),
           "build_csr_ms": round(build_ms, 5),
           "gedges_per_s_with_build": round(nnz / ((fwd_ms + build_ms) * 1e-3) / 1e9, 4)}
    if args.eager and args.variant == "forward":
        print("# timing the eager PyTorch formulation (context)", file=sys.stderr, flush=True)
        res["eager_torch"] = eager_context(torch, wl, batches[0], float(np.median(fwd_ms_all)))
    failed = False
    if not args.no_cpu:
        print("# timing the CPU oracle and checking the sampled output rows", file=sys.stderr, flush=True)
        res["cpu_baseline"], res["parity"] = cpu_baseline(wl, host, batches[0].out, args.cpu_seconds, args.variant)
        failed = not res["parity"]["passed"]
    print(json.dumps(res), flush=True)
    if failed:
        print(f"# PARITY FAILED on the sampled rows: {res['parity']}", file=sys.stderr, flush=True)
        sys.exit(1)


if __name__ == "__main__":
    main()
