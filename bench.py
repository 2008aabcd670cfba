"""Benchmark of the compressed-index matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]

Headline (``value``): decode-path throughput in GB/s of compressed weight
bytes on the largest single-GPU decode workload, the 70B-MLP-shaped linears
(28672x8192 and 8192x28672; one stage of 16-bit indices into a 65,536-entry
fp16 codebook, one fp16 scale per row, bf16 x, batch 1) with the randomized
Hadamard transform of x (blocks of 8192) before each product.  One step =
the input transform and the vq_gemv of each linear.  Weights are cycled
through enough identical copies (>= 512 MiB) that every launch reads its
indices from HBM, not from the 256 MiB Infinity Cache or the L2.  Every time
is the median of 5 replays of a HIP graph of `steps` steps (or launches),
bracketed by events on the launch stream.

The line carries:
  * ``roofline``: the dominant kernel of the headline step against HBM peak,
    with the HBM traffic counted by rocprofv3 (profiles/) when it was taken
    on the current kernel source;
  * ``rooflines``: the same for the dominant kernel of each target workload:
    Llama-3-8B decode at batch 1 (two 12-bit stages), the 70B MLP, and the
    2048-token prefill GEMM against the bf16 matrix-core peak (the published
    2.5 PFLOP/s and the peak at the engine clock measured during the run);
  * ``hbm_copy_gbs``: a plain 1 GiB device copy measured the same way;
  * ``cpu_baseline``: the float64 oracle on a bounded sample of the headline
    workload, unpack / dequant / transform / matmul timed separately (median
    of 3), with one BLAS thread and with all of them;
  * ``detail``: every other workload measured the same way (Llama-3-8B at
    1..64 tokens, tiny and SmolLM shapes, the residual ladders, the sparse
    correction, standalone dequant, the RHT fused into the decode kernel).
"""

from __future__ import annotations

import argparse
import json
import os
import re
import statistics
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, published
CUS, BF16_FLOP_PER_CLK_CU = 256, 4096  # the published peak is CUs x flop/clk x engine clock
MALL_DEFEAT_BYTES = 512 << 20  # rotate through at least this many weight bytes
MAX_COPIES = 128  # at most this many copies (the tiny and SmolLM weights stay warm in the 256 MB Infinity Cache)
REPLAYS = 5                    # timed graph replays; the median is reported
COPY_BYTES = 1 << 30           # the plain copy used for HBM calibration (4x the Infinity Cache)

# Kernel sources behind each roofline entry: a traffic figure taken on other
# sources is stale and reported as null.
SOURCES = {
    "k_gemv_lds": ["k_gemv.hip", "gemv_kernels.h", "vqmm_device.h"],
    "k_gemv_cbs": ["k_gemv_cbs.hip", "gemv_kernels.h", "vqmm_device.h"],
    "k_gemm_wide": ["k_gemm.hip", "gemm_kernels.h", "vqmm_device.h"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="headline and rooflines only (no other legs, no cpu)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu baseline")
    ap.add_argument("--only", default="", help="comma list of detail legs to run")
    ap.add_argument("--traffic-probe", default="", metavar="WORKLOAD:N,K[:M]",
                    help="launch only the product of one linear (rotating weight copies; M tokens, default 1) "
                         "and a plain 1 GiB device copy, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--traffic-summary", nargs=5, metavar=("SPEC", "KERNEL", "FETCH_CSV", "WRITE_CSV", "OUT_JSON"),
                    help="turn the two counter CSVs of --traffic-probe SPEC into a traffic summary for the "
                         "dispatches whose name contains KERNEL")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def graph_times_ms(launches, warmup_launches=None, reps=REPLAYS):
    """Capture `launches` (callables that enqueue on the current stream) in
    one HIP graph, replay it once untimed, then `reps` times, each between
    two events on the launch stream.  Returns the elapsed ms of each timed
    replay."""
    import torch
    for f in (warmup_launches or launches[: min(len(launches), 8)]):
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in launches:
            f()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    del g
    return out


def median_ms(launches, per, warmup_launches=None):
    """Median over the timed replays of one replay's ms, divided by `per`."""
    t = graph_times_ms(launches, warmup_launches)
    return statistics.median(t) / per, [v / per for v in t]


def copies_for(bytes_per_set):
    return max(2, -(-MALL_DEFEAT_BYTES // max(1, bytes_per_set)))


def weight_copies(sws):
    """Copies of a set of linears such that each linear timed alone also
    rotates through MALL_DEFEAT_BYTES of its own weights (at most
    MAX_COPIES: the tiny and SmolLM weights stay in the cache)."""
    return min(MAX_COPIES, max(copies_for(compressed_bytes(sw)) for sw in sws))


def upload_set(sws, ncopies):
    """ncopies identical copies of the weights at distinct device addresses."""
    base = [device_weight_(sw) for sw in sws]
    sets = [base]
    for _ in range(ncopies - 1):
        sets.append([w.clone() for w in base])
    return sets


def x_device(stored, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32)).cuda()


# ----------------------------------------------------------------------------
# legs
# ----------------------------------------------------------------------------

def run_decode_leg(vq, workload, steps, warmup, batch=1, rht=False, fused=False):
    """GEMV (and optionally the input RHT: a separate rht_apply launch, or
    with fused=True inside the decode kernel through vq_gemv_rht) over all
    linears of a workload.  Per-step time, GB/s and per-kernel times."""
    import torch
    import vqsynth
    ws, act_ss = vqsynth.workload_weights(workload)
    cfg = vqsynth.WORKLOADS[workload]
    kids = act_ss.spawn(2 * len(ws))
    xs, signs = [], []
    for i, sw in enumerate(ws):
        st, _ = vqsynth.make_x(batch, sw.k_in, cfg["x_dtype"], kids[i])
        xs.append(x_device(st, cfg["x_dtype"]))
        if rht:
            signs.append(torch.from_numpy(vqsynth.make_signs(sw.k_in, kids[len(ws) + i])).cuda())
    ncopies = weight_copies(ws)
    sets = upload_set(ws, ncopies)
    ys = [torch.empty((batch, sw.n_out), dtype=torch.float32, device="cuda") for sw in ws]
    xr = [torch.empty((batch, sw.k_in), dtype=torch.float32, device="cuda") for sw in ws] if rht else None
    wsp = [torch.empty(max(1, vq.vq_gemm_workspace_size(sets[0][j], batch)), dtype=torch.uint8, device="cuda")
           for j in range(len(ws))]

    def product(j, w):
        if rht and fused:
            return lambda: vq.vq_gemv_rht(w, xs[j], signs[j], cfg["rht"], y=ys[j])
        if rht:
            return lambda: vq.vq_gemv(w, xr[j], y=ys[j])
        if batch > 16:  # more tokens than vq_gemv takes: the same product through vq_gemm
            return lambda: vq.vq_gemm(w, xs[j], y=ys[j], workspace=wsp[j])
        return lambda: vq.vq_gemv(w, xs[j], y=ys[j])

    def launches_of(i, only=None):
        """Closures that enqueue step i (only linear `only` if given)."""
        out = []
        for j, w in enumerate(sets[i % ncopies]):
            if only is not None and j != only:
                continue
            if rht and not fused:
                out.append(lambda j=j: vq.rht_apply(xs[j], signs[j], cfg["rht"], out=xr[j]))
            out.append(product(j, w))
        return out

    for i in range(warmup):
        for f in launches_of(i):
            f()
    torch.cuda.synchronize()
    # eager timing of `steps` steps (includes host launch overhead)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        for f in launches_of(i):
            f()
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / steps
    ms_step, ms_all = median_ms([f for i in range(steps) for f in launches_of(i)], steps)
    x_bytes = 2 if cfg["x_dtype"] == "bf16" else 4
    per, tot_bytes = [], 0
    for j, sw in enumerate(ws):
        k_ms, k_all = median_ms([product(j, sets[i % ncopies][j]) for i in range(steps)], steps)
        ent = {}
        if rht and not fused:
            r_ms, _ = median_ms([lambda j=j: vq.rht_apply(xs[j], signs[j], cfg["rht"], out=xr[j])
                                 for _ in range(steps)], steps)
            ent["rht_us"] = r_ms * 1e3
        comp = compressed_bytes(sw)
        xb = batch * sw.k_in * (4 if rht and not fused else x_bytes) + (sw.k_in if fused else 0)  # (+ signs)
        yb = batch * sw.n_out * 4
        alg = comp + xb + yb
        tot_bytes += comp
        ent.update({"shape": [sw.n_out, sw.k_in], "compressed_bytes": comp, "algorithmic_bytes": alg,
                    "kernel_us": k_ms * 1e3, "kernel_us_replays": [v * 1e3 for v in k_all],
                    "gbs_algorithmic": alg / (k_ms * 1e-3) / 1e9})
        per.append(ent)
    return {"ms_per_step": ms_step, "ms_per_step_replays": ms_all, "ms_per_step_eager": ms_eager,
            "compressed_bytes_per_step": tot_bytes, "gbs_compressed": tot_bytes / (ms_step * 1e-3) / 1e9,
            "weight_copies": ncopies, "linears": per, "batch": batch}


def run_gemm_leg(vq, steps, warmup, workload="prefill", only=None, m=2048):
    """m-token vq_gemm over the linears of `workload` (TFLOP/s)."""
    import torch
    import vqsynth
    ws, act_ss = vqsynth.workload_weights(workload, only=only)
    kids = act_ss.spawn(len(ws))
    res = []
    for i, sw in enumerate(ws):
        st, _ = vqsynth.make_x(m, sw.k_in, "bf16", kids[i])
        x = x_device(st, "bf16")
        w = device_weight_(sw)
        y = torch.empty((m, sw.n_out), dtype=torch.float32, device="cuda")
        wsp = torch.empty(max(1, vq.vq_gemm_workspace_size(w, m)), dtype=torch.uint8, device="cuda")
        f = lambda: vq.vq_gemm(w, x, y=y, workspace=wsp)  # noqa: E731
        ms, ms_all = median_ms([f] * steps, steps, [f] * warmup)
        flops = 2.0 * m * sw.n_out * sw.k_in
        tf = flops / (ms * 1e-3) / 1e12
        res.append({"shape": [m, sw.n_out, sw.k_in], "flops": flops, "kernel_us": ms * 1e3,
                    "kernel_us_replays": [v * 1e3 for v in ms_all], "tflops": tf,
                    "frac_bf16_peak": tf / BF16_PEAK_TFLOPS})
        del w, x, y, wsp
    tot_f = sum(r["flops"] for r in res)
    tot_t = sum(r["kernel_us"] for r in res) * 1e-6
    return {"shapes": res, "tflops": tot_f / tot_t / 1e12, "frac_bf16_peak": tot_f / tot_t / 1e12 / BF16_PEAK_TFLOPS}


def run_dequant_leg(vq, steps, warmup):
    import torch
    import vqsynth
    ws, _ = vqsynth.workload_weights("llama8b", only=["gate_up"])
    sw = ws[0]
    w = device_weight_(sw)
    wt = torch.empty((sw.n_out, sw.k_in), dtype=torch.float16, device="cuda")
    L = vq.lib()

    def f():  # raw call: no per-call allocation; the stream is the capturing one
        st = L.vq_unpack_dequant(w.ref(), None, wt.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == 0
    ms, _ = median_ms([f] * steps, steps, [f] * warmup)
    moved = compressed_bytes(sw) + sw.n_out * sw.k_in * 2
    return {"shape": [sw.n_out, sw.k_in], "kernel_us": ms * 1e3, "gbs_read_plus_write": moved / (ms * 1e-3) / 1e9}


def run_copy_leg():
    """A plain device copy of COPY_BYTES (read + write) on the launch stream."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms, ms_all = median_ms([lambda: dst.copy_(src)] * 4, 4)
    del src, dst
    return {"bytes": 2 * COPY_BYTES, "us": ms * 1e3, "gbs": 2 * COPY_BYTES / (ms * 1e-3) / 1e9,
            "frac_hbm_peak": 2 * COPY_BYTES / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def sclk_under(fn, seconds=2.0):
    """Median engine clock (MHz) read by rocm-smi while fn() keeps the GPU busy
    (fn is called repeatedly); None when rocm-smi is missing or says nothing
    readable."""
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                                     timeout=10).stdout
            except Exception:  # pragma: no cover - tool missing
                return
            m = re.search(r"sclk clock level:\s*\d+:\s*\((\d+)\s*Mhz\)", out)
            if m:
                samples.append(int(m.group(1)))
    t = threading.Thread(target=sampler, daemon=True)
    t0 = time.time()
    t.start()
    while time.time() - t0 < seconds or (not samples and time.time() - t0 < 4 * seconds):
        fn()
        torch.cuda.synchronize()
    stop.set()
    t.join(timeout=15)
    busy = [s for s in samples if s > 1000]  # readings taken while the clock was up
    return statistics.median(busy) if busy else None


# ----------------------------------------------------------------------------
# helpers that avoid importing the tests package
# ----------------------------------------------------------------------------

def compressed_bytes(sw):
    """Index planes + fp16 scales + fp16 codebooks, each once (per group and
    stage: 16-bit 2 B, 12-bit 1.5 B, 8-bit 1 B, 4-bit 0.5 B)."""
    g = sw.n_out * (sw.k_in // 8)
    per = {4: (g + 1) // 2, 8: g, 12: g + (g + 1) // 2, 16: 2 * g}
    nblk = -(-sw.k_in // sw.scale_block)
    sp = 0 if sw.sparse is None else 4 * (sw.n_out + 1) + 6 * int(sw.sparse[0][-1])
    return sum(per[b] + (1 << b) * 16 for b in sw.widths) + 2 * sw.n_out * nblk + sp


def device_weight_(sw):
    from compressed_index_matmul_amd import VQWeight
    return VQWeight(sw.n_out, sw.k_in, sw.n_stages, sw.idx_bits, sw.scale_block, codebooks=sw.codebooks,
                    scales=sw.scales, lo=sw.lo, hi=sw.hi, idx16=sw.idx16, device="cuda",
                    stage_bits=sw.stage_bits, stage_scales=sw.stage_scales, sparse=sw.sparse)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def cpu_baseline(rows=8192, reps=3):
    """The float64 oracle as it stands on a bounded sample of the headline
    workload: `rows` rows of each 70B-MLP linear (every column), with the
    input transform of a fresh x.  Unpack, dequant, transform and matmul are
    timed separately, each the median of `reps` runs, once with one BLAS
    thread and once with all of them.  GB/s counts the sample's compressed
    bytes: its rows' indices and scales plus the codebook prorated by rows."""
    import oracle
    import vqsynth
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    ws, act_ss = vqsynth.workload_weights("mlp70b")
    cfg = vqsynth.WORKLOADS["mlp70b"]
    kids = act_ss.spawn(2 * len(ws))
    sample_bytes = 0.0
    jobs = []
    for i, sw in enumerate(ws):
        r = min(rows, sw.n_out)
        g = sw.k_in // 8
        sub = sw.idx16[0][: r * g]
        _, x64 = vqsynth.make_x(1, sw.k_in, "bf16", kids[i])
        signs = vqsynth.make_signs(sw.k_in, kids[len(ws) + i])
        jobs.append((sw, r, g, sub, x64, signs))
        sample_bytes += r * (2 * g + 2 * -(-sw.k_in // sw.scale_block)) + (65536 * 16) * r / sw.n_out

    def one_pass():
        t = {"unpack": 0.0, "dequant": 0.0, "rht": 0.0, "matmul": 0.0}
        for sw, r, g, sub, x64, signs in jobs:
            t0 = time.perf_counter()
            idx = oracle.unpack_indices(16, r * g, idx16=sub)
            t1 = time.perf_counter()
            w64 = oracle.dequant_exact(r, sw.k_in, [idx], sw.codebooks, sw.scales[:r], sw.scale_block)
            t2 = time.perf_counter()
            xr = oracle.rht_ref(x64, signs, cfg["rht"])
            t3 = time.perf_counter()
            oracle.matmul_ref(w64, xr)
            t4 = time.perf_counter()
            t["unpack"] += t1 - t0
            t["dequant"] += t2 - t1
            t["rht"] += t3 - t2
            t["matmul"] += t4 - t3
            del w64
        return t

    def timed(threads):
        lim = threadpool_limits(threads) if threadpool_limits is not None and threads else None
        try:
            runs = [one_pass() for _ in range(reps)]
        finally:
            if lim is not None:
                lim.restore_original_limits()
        ph = {k: statistics.median(r[k] for r in runs) for k in runs[0]}
        tot = sum(ph.values())
        return {"seconds_per_pass": tot, "phase_seconds": ph, "gbs": sample_bytes / tot / 1e9}

    t0 = time.perf_counter()
    one = timed(1)
    allc = timed(os.cpu_count())
    n_all = os.cpu_count()
    return {"value": allc["gbs"], "unit": "GB/s", "cores": n_all, "kind": "oracle",
            "sample": f"{rows} rows of each 70B-MLP linear (28672x8192, 8192x28672; every column, "
                      f"{sample_bytes / 1e6:.1f} MB of compressed weight), the input transform of a fresh x, "
                      "float64 unpack + exact dequant + transform + matmul, numpy; median of "
                      f"{reps} passes per phase",
            "all_threads": allc, "one_thread": one, "cpu_model": cpu_model(), "host_cpus": n_all,
            "seconds_total": time.perf_counter() - t0}


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in SOURCES[kernel]:
        with open(os.path.join(ROOT, "compressed_index_matmul_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(kernel, workload, shape):
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}_{'x'.join(str(v) for v in shape)}.json")


def stored_traffic(kernel, workload, shape):
    """HBM bytes per launch from profiles/ when they were taken on the current
    kernel source, else None."""
    try:
        with open(traffic_file(kernel, workload, shape)) as f:
            t = json.load(f)
        if t.get("source_hash") == kernel_source_hash(kernel):
            return t["traffic_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        pass
    return None


def parse_spec(spec):
    parts = spec.split(":")
    workload = parts[0]
    n, k = (int(v) for v in parts[1].split(","))
    m = int(parts[2]) if len(parts) > 2 else 1
    return workload, n, k, m


def traffic_probe(spec, launches=20):
    """Launch the product of one linear `launches` times (weights rotated
    through >= 512 MiB of copies; the input transform first for a workload
    that has one, as in the bench), then a plain 1 GiB float32 copy whose HBM
    bytes are known."""
    import torch
    import vqsynth
    import compressed_index_matmul_amd as vq
    workload, n, k, m = parse_spec(spec)
    ws, act_ss = vqsynth.workload_weights(workload)
    sw = [w for w in ws if (w.n_out, w.k_in) == (n, k)][0]
    cfg = vqsynth.WORKLOADS[workload]
    kids = act_ss.spawn(2)
    st, _ = vqsynth.make_x(m, k, cfg["x_dtype"], kids[0])
    x = x_device(st, cfg["x_dtype"])
    if cfg["rht"]:
        signs = torch.from_numpy(vqsynth.make_signs(k, kids[1])).cuda()
        x = vq.rht_apply(x, signs, cfg["rht"])
    sets = upload_set([sw], copies_for(compressed_bytes(sw)))
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for i in range(launches):
        w = sets[i % len(sets)][0]
        if m > 16:
            vq.vq_gemm(w, x, y=y)
        else:
            vq.vq_gemv(w, x, y=y)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe": [workload, n, k, m], "launches": launches, "copy_bytes": COPY_BYTES}), flush=True)


def traffic_summary(spec, kernel, fetch_csv, write_csv, out_json):
    """HBM bytes per dispatch of `kernel` from FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch), each scaled by bytes moved / counter of the plain copy (it
    reads COPY_BYTES and writes COPY_BYTES)."""
    import csv

    def read(path, counter):
        mine, other = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            (mine if kernel in r["Kernel_Name"] else other).append(v)
        return mine, other
    gf, of = read(fetch_csv, "FETCH_SIZE")
    gw, ow = read(write_csv, "WRITE_SIZE")
    f_scale = COPY_BYTES / max(of)  # the copy is the largest other dispatch
    w_scale = COPY_BYTES / max(ow)
    fetch = float(np.median(gf)) * f_scale
    write = float(np.median(gw)) * w_scale
    workload, n, k, m = parse_spec(spec)
    out = {"kernel": kernel, "workload": workload, "shape": [n, k], "tokens": m,
           "source_hash": kernel_source_hash(kernel), "dispatches": len(gf),
           "fetch_kib_raw_median": float(np.median(gf)) / 1024.0, "write_kib_raw_median": float(np.median(gw)) / 1024.0,
           "copy_fetch_kib_raw": max(of) / 1024.0, "copy_write_kib_raw": max(ow) / 1024.0,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "traffic_bytes_per_launch": fetch + write}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def hbm_roofline(kernel, workload, ent, label):
    """Roofline entry of one decode linear against HBM peak."""
    us = ent["kernel_us"]
    ach = ent["algorithmic_bytes"] / (us * 1e-6) / 1e9
    return {"workload": label, "kernel": kernel, "shape": ent["shape"], "bound": "hbm", "achieved": ach,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
            "traffic": stored_traffic(kernel, workload, ent["shape"]),
            "algorithmic_bytes": ent["algorithmic_bytes"], "kernel_us": us,
            "kernel_us_replays": ent["kernel_us_replays"]}


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (each product runs on a single "
              "MI355X; the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    import compressed_index_matmul_amd as vq
    if not os.path.exists(vq.LIB_PATH):
        from compressed_index_matmul_amd.build import build
        build()
    vq.lib()
    torch.cuda.set_device(0)

    if args.traffic_probe:
        traffic_probe(args.traffic_probe)
        return

    steps, warmup = args.steps, args.warmup
    log("headline: 70B-MLP input transform + 16-bit decode, batch 1")
    head = run_decode_leg(vq, "mlp70b", steps, warmup, rht=True)
    dom = max(head["linears"], key=lambda e: e["kernel_us"])
    roof = hbm_roofline("k_gemv_cbs", "mlp70b", dom, "mlp70b_rht_gemv_b1")
    log("llama8b decode, batch 1")
    c3 = run_decode_leg(vq, "llama8b", steps, warmup)
    log("prefill GEMM, 2048 tokens")
    c5 = run_gemm_leg(vq, max(5, steps // 2), 3)
    log("1 GiB copy")
    copy = run_copy_leg()
    log("engine clock under the prefill GEMM")
    import vqsynth
    ws5, act5 = vqsynth.workload_weights("prefill", only=["gate_up"])
    w5 = device_weight_(ws5[0])
    x5 = x_device(vqsynth.make_x(2048, ws5[0].k_in, "bf16", act5.spawn(1)[0])[0], "bf16")
    y5 = torch.empty((2048, ws5[0].n_out), dtype=torch.float32, device="cuda")
    ws5b = torch.empty(max(1, vq.vq_gemm_workspace_size(w5, 2048)), dtype=torch.uint8, device="cuda")
    sclk = sclk_under(lambda: [vq.vq_gemm(w5, x5, y=y5, workspace=ws5b) for _ in range(200)])
    del w5, x5, y5, ws5b
    peak_sclk = CUS * BF16_FLOP_PER_CLK_CU * sclk * 1e6 / 1e12 if sclk else None

    dom3 = max(c3["linears"], key=lambda e: e["kernel_us"])
    dom5 = max(c5["shapes"], key=lambda e: e["kernel_us"])
    ach5 = dom5["tflops"]
    rooflines = [
        dict(roof),
        hbm_roofline("k_gemv_lds", "llama8b", dom3, "llama8b_gemv_b1"),
        {"workload": "prefill_gemm_m2048", "kernel": "k_gemm_wide", "shape": dom5["shape"], "bound": "mfma",
         "achieved": ach5, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach5 / BF16_PEAK_TFLOPS,
         "peak_at_measured_sclk": peak_sclk, "frac_at_measured_sclk": ach5 / peak_sclk if peak_sclk else None,
         "traffic": stored_traffic("k_gemm_wide", "prefill", dom5["shape"][1:]),
         "flops": dom5["flops"], "kernel_us": dom5["kernel_us"], "kernel_us_replays": dom5["kernel_us_replays"]},
    ]
    detail = {"headline_linears": head["linears"], "weight_copies": head["weight_copies"],
              "headline_ms_per_step_replays": head["ms_per_step_replays"],
              "headline_ms_per_step_eager": head["ms_per_step_eager"],
              "llama8b_gemv_b1": c3, "prefill_gemm_m2048": c5}
    only = set(filter(None, args.only.split(",")))
    if only or not args.quick:
        short = max(5, steps // 4)
        legs = [("llama8b_gemv_b16", lambda: run_decode_leg(vq, "llama8b", steps, warmup, batch=16)),
                ("llama8b_tokens_2_to_64", lambda: {
                    f"m{m}": run_decode_leg(vq, "llama8b", short, 2, batch=m) for m in (2, 8, 32, 64)}),
                ("mlp70b_rht_fused_gemv_b1", lambda: run_decode_leg(vq, "mlp70b", short, 3, rht=True, fused=True)),
                ("smollm_gemv_b1", lambda: run_decode_leg(vq, "smollm", steps, warmup)),
                ("tiny_gemv_b1", lambda: run_decode_leg(vq, "tiny", steps, warmup)),
                ("dequant_14336x4096", lambda: run_dequant_leg(vq, steps, warmup)),
                # residual ladders: orka's rvq-12-4 (12 + 4 bits), GLQ's 3 bpw 16 + 8 with a residual scale
                ("smollm_rvq124_gemv_b1", lambda: run_decode_leg(vq, "smollm_rvq124", steps, warmup)),
                ("llama8b_rvq124_gemv_b1", lambda: run_decode_leg(vq, "llama8b_rvq124", steps, warmup)),
                ("llama8b_rvq124_gemv_b16", lambda: run_decode_leg(vq, "llama8b_rvq124", steps, warmup,
                                                                   batch=16)),
                ("llama8b_rvq124_gemm_m2048", lambda: run_gemm_leg(vq, short, 3, "llama8b_rvq124",
                                                                   only=["qo", "gate_up"])),
                ("mlp70b_e8p3_rht_gemv_b1", lambda: run_decode_leg(vq, "mlp70b_e8p3", short, 3, rht=True)),
                ("mlp70b_e8p3_rht_fused_gemv_b1", lambda: run_decode_leg(vq, "mlp70b_e8p3", short, 3,
                                                                         rht=True, fused=True)),
                ("mlp70b_e8p4_rht_gemv_b1", lambda: run_decode_leg(vq, "mlp70b_e8p4", short, 3, rht=True)),
                # sparse correction (0.5 % of the weights) on the Llama-3-8B format
                ("llama8b_sparse_gemv_b1", lambda: run_decode_leg(vq, "llama8b_sparse", steps, warmup)),
                ("llama8b_sparse_gemv_b16", lambda: run_decode_leg(vq, "llama8b_sparse", steps, warmup,
                                                                   batch=16))]
        for name, fn in legs:
            if only and name not in only:
                continue
            log(name)
            detail[name] = fn()
    cpu = None
    if not (args.quick or args.no_cpu):
        log("cpu baseline (oracle)")
        cpu = cpu_baseline()
    out = {
        "metric": "vq_gemv compressed-weight GB/s (% HBM peak); vq_gemm TFLOP/s (% MFMA peak)",
        "value": head["gbs_compressed"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32",
        "data": "synthetic",
        "config": {"workload": "mlp70b_rht_gemv_b1",
                   "shapes": [[28672, 8192], [8192, 28672]], "stages": 1, "idx_bits": 16,
                   "scale_block": "per row", "batch": 1, "x": "bf16", "rht_max_block": 8192,
                   "weight_copies": head["weight_copies"],
                   "launch": f"HIP graph of {steps} steps, median of {REPLAYS} replays (eager step time in detail)"},
        "frac_hbm_peak": head["gbs_compressed"] / HBM_PEAK_GBS,
        "roofline": roof,
        "rooflines": rooflines,
        "hbm_copy_gbs": copy,
        "sclk_mhz_under_gemm": sclk,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
