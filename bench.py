"""Benchmark of the compressed-index matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

Headline (``value``): decode-path throughput in GB/s of compressed weight
bytes for the Llama-3-8B-shaped linears (4096x4096, 14336x4096, 4096x14336;
two 12-bit bit-plane stages, per-row x 128-column fp16 scales, bf16 x, batch
1).  One step = one vq_gemv on each of the three linears.  Weights are
cycled through enough identical copies (>= 512 MiB) that every launch reads
its indices from HBM, not from the 256 MiB Infinity Cache or the L2.

The same JSON line carries, under ``detail``, the other workloads measured
the same way (70B-MLP RHT + 16-bit GEMV, batch-16 decode, 2048-token GEMM in
TFLOP/s, tiny and SmolLM-shaped linears in microseconds, standalone dequant,
the residual-ladder formats: rvq-12-4 on the SmolLM and Llama-3-8B
shapes, a 16 + 8-bit ladder with a residual scale on the 70B-MLP shapes,
and the headline format with a 0.5 % sparse correction),
``roofline`` for the dominant kernel of the headline step (HIP-event kernel
times on the launch stream), and ``cpu_baseline``: the float64 oracle timed
on the host on one full headline step.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
MALL_DEFEAT_BYTES = 512 << 20  # rotate through at least this many weight bytes


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="headline only (no detail, no cpu baseline)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu baseline")
    ap.add_argument("--only", default="", help="comma list of detail legs to run")
    ap.add_argument("--traffic-probe", default="", metavar="N,K",
                    help="launch only the GEMV of shape N x K (llama8b format, rotating copies) "
                         "and a plain 256 MiB device copy, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("N,K", "FETCH_CSV", "WRITE_CSV", "OUT_JSON"),
                    help="turn the two counter CSVs of --traffic-probe into a traffic summary")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """HIP events on the current (launch) stream around each launch."""

    def __init__(self):
        import torch
        self.torch = torch
        self.pairs = []

    def around(self, fn):
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.append((a, b))

    def durations_ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


def graph_time_ms(launches, warmup_launches=None):
    """Capture `launches` (callables that enqueue on the current stream) into
    one HIP graph, replay it once untimed, then once between two events on
    the launch stream.  Returns the elapsed milliseconds of the timed replay."""
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
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    del g
    return ms


def copies_for(bytes_per_set):
    return max(2, -(-MALL_DEFEAT_BYTES // max(1, bytes_per_set)))


def upload_set(vq, sws, ncopies):
    """ncopies identical copies of the weights at distinct device addresses."""
    base = [device_weight_(sw) for sw in sws]
    sets = [base]
    for _ in range(ncopies - 1):
        sets.append([w.clone() for w in base])
    return sets


# ----------------------------------------------------------------------------
# legs
# ----------------------------------------------------------------------------

def run_decode_leg(vq, workload, steps, warmup, batch=1, rht=False, fused=False):
    """GEMV (and optionally the input RHT: a separate rht_apply launch, or
    with fused=True inside the decode kernel through vq_gemv_rht) over all
    linears of a workload.  Returns a dict with per-step time, GB/s and
    per-kernel timings."""
    import torch
    import vqsynth
    ws, act_ss = vqsynth.workload_weights(workload)
    cfg = vqsynth.WORKLOADS[workload]
    kids = act_ss.spawn(2 * len(ws))
    xs = []
    signs = []
    for i, sw in enumerate(ws):
        st, _ = vqsynth.make_x(batch, sw.k_in, cfg["x_dtype"], kids[i])
        if cfg["x_dtype"] == "bf16":
            xs.append(torch.from_numpy(st.view(np.int16)).cuda().view(torch.bfloat16))
        else:
            xs.append(torch.from_numpy(st).cuda())
        if rht:
            signs.append(torch.from_numpy(vqsynth.make_signs(sw.k_in, kids[len(ws) + i])).cuda())
    set_bytes = sum(compressed_bytes(sw) for sw in ws)
    ncopies = copies_for(set_bytes)
    sets = upload_set(vq, ws, ncopies)
    ys = [torch.empty((batch, sw.n_out), dtype=torch.float32, device="cuda") for sw in ws]
    xr = [torch.empty((batch, sw.k_in), dtype=torch.float32, device="cuda") for sw in ws] if rht else None

    def launches_of(i, only=None):
        """Closures that enqueue step i (only linear `only` if given)."""
        wset = sets[i % ncopies]
        out = []
        for j, w in enumerate(wset):
            if only is not None and j != only:
                continue
            if rht and fused:
                out.append(lambda j=j, w=w: vq.vq_gemv_rht(w, xs[j], signs[j], cfg["rht"], y=ys[j]))
            elif rht:
                out.append(lambda j=j: vq.rht_apply(xs[j], signs[j], cfg["rht"], out=xr[j]))
                out.append(lambda j=j, w=w: vq.vq_gemv(w, xr[j], y=ys[j]))
            elif batch > 16:  # more tokens than vq_gemv takes: the same product through vq_gemm
                out.append(lambda j=j, w=w: vq.vq_gemm(w, xs[j], y=ys[j]))
            else:
                out.append(lambda j=j, w=w: vq.vq_gemv(w, xs[j], y=ys[j]))
        return out

    # eager warmup steps
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
    # graph timing: exactly `steps` steps captured in one graph
    ms_step = graph_time_ms([f for i in range(steps) for f in launches_of(i)]) / steps
    # per-kernel averages: `steps` launches of one linear (and its RHT) per graph
    x_bytes = 2 if cfg["x_dtype"] == "bf16" else 4
    per = []
    tot_bytes = 0
    for j, sw in enumerate(ws):
        if rht and fused:
            g_ms = graph_time_ms([f for i in range(steps) for f in launches_of(i, only=j)]) / steps
        elif rht:
            r_ms = graph_time_ms([lambda j=j: vq.rht_apply(xs[j], signs[j], cfg["rht"], out=xr[j])
                                  for _ in range(steps)]) / steps
            g_ms = graph_time_ms([lambda i=i, j=j: vq.vq_gemv(sets[i % ncopies][j], xr[j], y=ys[j])
                                  for i in range(steps)]) / steps
        else:
            g_ms = graph_time_ms([f for i in range(steps) for f in launches_of(i, only=j)]) / steps
        comp = compressed_bytes(sw)
        xb = batch * sw.k_in * (4 if rht and not fused else x_bytes) + (sw.k_in if fused else 0)  # (+ signs)
        yb = batch * sw.n_out * 4
        alg = comp + xb + yb
        tot_bytes += comp
        ent = {"shape": [sw.n_out, sw.k_in], "compressed_bytes": comp, "algorithmic_bytes": alg,
               "kernel_us_mean": g_ms * 1e3, "gbs_algorithmic": alg / (g_ms * 1e-3) / 1e9}
        if rht and not fused:
            ent["rht_us_mean"] = r_ms * 1e3
        per.append(ent)
    return {"ms_per_step": ms_step, "ms_per_step_eager": ms_eager, "compressed_bytes_per_step": tot_bytes,
            "gbs_compressed": tot_bytes / (ms_step * 1e-3) / 1e9, "weight_copies": ncopies,
            "linears": per, "batch": batch}


def run_gemm_leg(vq, steps, warmup, workload="prefill", only=None):
    """2048-token vq_gemm over the linears of `workload` (TFLOP/s)."""
    import torch
    import vqsynth
    ws, act_ss = vqsynth.workload_weights(workload, only=only)
    kids = act_ss.spawn(len(ws))
    res = []
    for i, sw in enumerate(ws):
        st, _ = vqsynth.make_x(2048, sw.k_in, "bf16", kids[i])
        x = torch.from_numpy(st.view(np.int16)).cuda().view(torch.bfloat16)
        w = device_weight_(sw)
        y = torch.empty((2048, sw.n_out), dtype=torch.float32, device="cuda")
        ms = graph_time_ms([lambda: vq.vq_gemm(w, x, y=y) for _ in range(steps)],
                           [lambda: vq.vq_gemm(w, x, y=y) for _ in range(warmup)]) / steps
        d = np.array([ms])
        flops = 2.0 * 2048 * sw.n_out * sw.k_in
        tf = flops / (d.mean() * 1e-3) / 1e12
        res.append({"shape": [2048, sw.n_out, sw.k_in], "kernel_us_mean": float(d.mean() * 1e3),
                    "tflops": float(tf), "frac_bf16_peak": float(tf / BF16_PEAK_TFLOPS)})
        del w, x, y
    tot_f = sum(2.0 * 2048 * sw.n_out * sw.k_in for sw in ws)
    tot_t = sum(r["kernel_us_mean"] for r in res) * 1e-6
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
    d = graph_time_ms([f for _ in range(steps)], [f for _ in range(warmup)]) / steps * 1e-3
    moved = compressed_bytes(sw) + sw.n_out * sw.k_in * 2
    return {"shape": [sw.n_out, sw.k_in], "kernel_us_mean": d * 1e6, "gbs_read_plus_write": moved / d / 1e9}


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


def cpu_baseline(min_seconds=10.0, max_steps=20):
    """The float64 oracle on full headline steps (all three Llama-3-8B
    linears, every row: unpack, exact dequant, matmul), single-threaded,
    repeated with a fresh x each step until about min_seconds have passed."""
    import oracle
    import vqsynth
    try:
        from threadpoolctl import threadpool_limits
        lim = threadpool_limits(1)
    except Exception:  # pragma: no cover
        lim = None
    ws, act_ss = vqsynth.workload_weights("llama8b")
    kids = act_ss.spawn(max_steps * len(ws))
    t0 = time.perf_counter()
    tot = 0
    steps = 0
    while steps < max_steps and (steps == 0 or time.perf_counter() - t0 < min_seconds):
        for i, sw in enumerate(ws):
            _, x64 = vqsynth.make_x(1, sw.k_in, "bf16", kids[steps * len(ws) + i])
            idx = [oracle.unpack_indices(sw.idx_bits, sw.n_groups, lo=sw.lo[t], hi=sw.hi[t])
                   for t in range(sw.n_stages)]
            w64 = oracle.dequant_exact(sw.n_out, sw.k_in, idx, sw.codebooks, sw.scales, sw.scale_block)
            oracle.matmul_ref(w64, x64)
            tot += compressed_bytes(sw)
            del w64
        steps += 1
    dt = time.perf_counter() - t0
    if lim is not None:
        lim.restore_original_limits()
    return {"value": tot / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full steps: all three Llama-3-8B-shaped linears (every row) with a fresh x each "
                      "step, float64 unpack + exact dequant + matmul, numpy with BLAS limited to 1 thread",
            "seconds": dt, "host_cpus": os.cpu_count()}


KERNEL_SOURCES = ["compressed_index_matmul_amd/csrc/k_gemv.hip", "compressed_index_matmul_amd/csrc/gemv_kernels.h",
                  "compressed_index_matmul_amd/csrc/vqmm_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemv_lds_llama8b_down_4096x14336_traffic.json")
COPY_BYTES = 256 << 20


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_probe(spec, launches=20):
    """Launch the batch-1 decode GEMV of one linear `launches` times (weights
    rotated through >= 512 MiB of copies), then a plain 256 MiB float32 copy
    (`dst = src * 1`) whose HBM bytes are known.  spec: "N,K" (Llama-3-8B
    format) or "workload:N,K"."""
    import torch
    import vqsynth
    import compressed_index_matmul_amd as vq
    workload, _, shape = spec.rpartition(":")
    workload = workload or "llama8b"
    n, k = (int(v) for v in shape.split(","))
    ws, act_ss = vqsynth.workload_weights(workload)
    sw = [w for w in ws if (w.n_out, w.k_in) == (n, k)][0]
    cfg = vqsynth.WORKLOADS[workload]
    st, _ = vqsynth.make_x(1, k, cfg["x_dtype"], act_ss.spawn(1)[0])
    if cfg["x_dtype"] == "bf16":
        x = torch.from_numpy(st.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        x = torch.from_numpy(st).cuda()
    sets = upload_set(vq, [sw], copies_for(compressed_bytes(sw)))
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for i in range(launches):
        vq.vq_gemv(sets[i % len(sets)][0], x, y=y)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"probe": [workload, n, k], "launches": launches, "copy_bytes": COPY_BYTES}), flush=True)


def traffic_summary(spec, fetch_csv, write_csv, out_json):
    """HBM bytes per GEMV dispatch from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by bytes-moved / counter of the plain copy: the
    copy reads COPY_BYTES and writes COPY_BYTES."""
    import csv

    def read(path, counter):
        gemv, other = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            (gemv if "k_gemv_lds" in r["Kernel_Name"] else other).append(v)
        return gemv, other
    gf, of = read(fetch_csv, "FETCH_SIZE")
    gw, ow = read(write_csv, "WRITE_SIZE")
    # the copy is the dispatch with the largest read (resp. write) besides the GEMV
    f_scale = COPY_BYTES / max(of)
    w_scale = COPY_BYTES / max(ow)
    fetch = float(np.median(gf)) * f_scale
    write = float(np.median(gw)) * w_scale
    n, k = (int(v) for v in spec.split(","))
    out = {"kernel": "k_gemv_lds", "shape": [n, k], "source_hash": kernel_source_hash(),
           "dispatches": len(gf),
           "fetch_kib_raw_median": float(np.median(gf)) / 1024.0, "write_kib_raw_median": float(np.median(gw)) / 1024.0,
           "copy_fetch_kib_raw": max(of) / 1024.0, "copy_write_kib_raw": max(ow) / 1024.0,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "traffic_bytes_per_launch": fetch + write}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library runs each "
              "product on a single MI355X and has no multi-GPU path)", file=sys.stderr)
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

    log("headline: llama8b decode, batch 1")
    head = run_decode_leg(vq, "llama8b", args.steps, args.warmup)
    # dominant kernel of the step: the linear with the largest kernel time
    dom = max(head["linears"], key=lambda e: e["kernel_us_mean"])
    traffic = None
    try:  # counters taken on this exact kernel source, else null
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("source_hash") == kernel_source_hash() and t.get("shape") == dom["shape"]:
            traffic = t["traffic_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None
    roof = {"bound": "hbm", "achieved": dom["gbs_algorithmic"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": dom["gbs_algorithmic"] / HBM_PEAK_GBS, "traffic": traffic,
            "kernel": "k_gemv_lds (2 stages, 12-bit)", "shape": dom["shape"],
            "kernel_us_mean": dom["kernel_us_mean"], "algorithmic_bytes": dom["algorithmic_bytes"]}
    detail = {"headline_linears": head["linears"], "weight_copies": head["weight_copies"],
              "headline_ms_per_step_eager": head["ms_per_step_eager"]}
    only = set(filter(None, args.only.split(",")))
    if only or not args.quick:
        legs = [("mlp70b_rht_gemv_b1", lambda: run_decode_leg(vq, "mlp70b", max(5, args.steps // 5), 3, rht=True)),
                ("llama8b_gemv_b16", lambda: run_decode_leg(vq, "llama8b", args.steps, args.warmup, batch=16)),
                ("llama8b_tokens_2_to_64", lambda: {
                    f"m{m}": run_decode_leg(vq, "llama8b", max(5, args.steps // 4), 2, batch=m)
                    for m in (2, 8, 32, 64)}),
                ("prefill_gemm_m2048", lambda: run_gemm_leg(vq, max(5, args.steps // 5), 3)),
                ("smollm_gemv_b1", lambda: run_decode_leg(vq, "smollm", args.steps, args.warmup)),
                ("tiny_gemv_b1", lambda: run_decode_leg(vq, "tiny", args.steps, args.warmup)),
                ("dequant_14336x4096", lambda: run_dequant_leg(vq, args.steps, args.warmup)),
                # residual ladders: orka's rvq-12-4 (12 + 4 bits), GLQ's 3 bpw 16 + 8 with a residual scale
                ("smollm_rvq124_gemv_b1", lambda: run_decode_leg(vq, "smollm_rvq124", args.steps, args.warmup)),
                ("llama8b_rvq124_gemv_b1", lambda: run_decode_leg(vq, "llama8b_rvq124", args.steps, args.warmup)),
                ("llama8b_rvq124_gemv_b16", lambda: run_decode_leg(vq, "llama8b_rvq124", args.steps, args.warmup,
                                                                   batch=16)),
                ("llama8b_rvq124_gemm_m2048", lambda: run_gemm_leg(vq, max(5, args.steps // 5), 3, "llama8b_rvq124",
                                                                   only=["qo", "gate_up"])),
                ("mlp70b_e8p3_rht_gemv_b1", lambda: run_decode_leg(vq, "mlp70b_e8p3", max(5, args.steps // 5), 3,
                                                                   rht=True)),
                # the same two workloads with the input transform inside the decode kernel (vq_gemv_rht)
                ("mlp70b_rht_fused_gemv_b1", lambda: run_decode_leg(vq, "mlp70b", max(5, args.steps // 5), 3,
                                                                    rht=True, fused=True)),
                ("mlp70b_e8p3_rht_fused_gemv_b1", lambda: run_decode_leg(vq, "mlp70b_e8p3", max(5, args.steps // 5),
                                                                         3, rht=True, fused=True)),
                # sparse correction (0.5 % of the weights) on the headline format
                ("llama8b_sparse_gemv_b1", lambda: run_decode_leg(vq, "llama8b_sparse", args.steps, args.warmup)),
                ("llama8b_sparse_gemv_b16", lambda: run_decode_leg(vq, "llama8b_sparse", args.steps, args.warmup,
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
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_linears_decode_b1",
                   "shapes": [[4096, 4096], [14336, 4096], [4096, 14336]],
                   "stages": 2, "idx_bits": 12, "scale_block": 128, "batch": 1,
                   "x": "bf16", "weight_copies": head["weight_copies"],
                   "launch": "HIP graph of the timed steps (eager step time in detail)"},
        "frac_hbm_peak": head["gbs_compressed"] / HBM_PEAK_GBS,
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
