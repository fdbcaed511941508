"""Throughput of the block-sparse masked attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = the whole hot path over one batch of seeded synthetic input that
is already resident in HBM: build the block mask on the device, then run the
forward.  Prints ONE JSON line.  `value` is effective TFLOP/s over unmasked
FLOPs, 2 * B * H * (D + Dv) * (visible query-key pairs) per step (4 * D with
equal head dims), divided by the measured step time; `roofline` reports the forward kernel alone, timed with
HIP events on the stream it is launched on; `cpu_baseline` times the fp64
oracle on a bounded sample of rows of the same workload.

`--pass bwd` measures the backward instead: one step = build both block-mask
arrays (per q-block and per kv-block) on the device, then the backward (the
per-row delta pass, the dq kernel and the dk/dv kernel) from the forward's
output and lse, computed once beforehand.  Its `value` counts 6 * D + 4 * Dv
FLOPs per visible pair (the five products the gradients need: S, dK and dQ
2 * D each, dP and dV 2 * Dv each; 10 * D with equal head dims; the kernels
recompute S and dP once more, which is not counted), and
its `cpu_baseline` times the oracle's backward on whole heads.

`--copy-calibration` instead runs only a plain device-to-device copy of a
known size, so that rocprofv3's FETCH_SIZE / WRITE_SIZE counters can be
scaled against it.

`--mfma-peak` runs only the matrix-unit microbenchmark (independent chains
of v_mfma_f32_32x32x16_bf16, 4 waves per SIMD, HIP-event timed) and prints
its measured dense bf16 rate and the shader clock it ran at; the default
forward line carries the same figures in `mfma_peak_measured`.

The default forward line also carries `sliding_window`: the sliding-window
workload (B=2, H=16, L=8192, window 256, 128x128 tiles) timed the same way
with the alpha-rescale subtiling off and on, each with its warm and
cold-cache forward time, its fraction of the bf16 peak and of the HBM
roofline of its algorithmic bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector (the fp32-input instance)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_prefix_causal_traffic.txt")


def visible_pairs(mask: dict, q_len: int, kv_len: int) -> int:
    """Number of (query, key) pairs the mask leaves visible in one head."""
    return int(_row_counts(mask, q_len, kv_len).sum())


def kernel_source_hash() -> str:
    """Hash of the sources the forward kernel is built from; the stored traffic
    figures are only reported while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_masked_flexattention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")) and (name.startswith("fwd_") or name == "internal.hpp"):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload_name: str):
    """HBM bytes per forward launch from the committed counter summary, or
    None when it is missing, for another workload, or for other sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                a, b = line.split("=", 1)
                kv[a.strip()] = b.strip()
    if kv.get("workload") != workload_name or kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or 'unknown'."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, q, k, v, target_seconds: float, seed: int = 0):
    """Time the fp64 oracle on randomly sampled query rows of the workload,
    growing the sample until it takes about `target_seconds`."""
    from oracle import oracle

    B, H, L, D = cfg["B"], cfg["H"], cfg["q_len"], cfg["d"]
    qf, kf, vf = (t.float().numpy() for t in (q, k, v))
    rng = np.random.default_rng(seed)
    threads = oracle.threads_used()
    # per-row visible counts, to price the sample in unmasked FLOPs
    counts = _row_counts(cfg["mask"], L, cfg["kv_len"])
    n = max(threads, 16)
    spent, flops, rows_done = 0.0, 0.0, 0
    while True:
        rows = rng.integers(0, B * H * L, size=n).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attention_rows(qf, kf, vf, cfg["mask"], cfg["score"], cfg["scale"], rows=rows,
                              threads=threads)
        dt = time.perf_counter() - t0
        spent += dt
        flops += 2.0 * (D + cfg.get("dv", D)) * float(counts[rows % L].sum())
        rows_done += n
        if spent >= target_seconds:
            break
        # aim the next batch at the remaining time
        per_row = dt / n
        n = int(min(max(n * 2, 16), max(16, (target_seconds - spent) / max(per_row, 1e-9))))
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": "%d query rows drawn uniformly from all B*H*Lq rows of the workload, "
                  "fp64 oracle, %.1f s" % (rows_done, spent),
    }


def cpu_baseline_bwd(cfg, q, k, v, dout, target_seconds: float):
    """Time the fp64 oracle backward on whole heads (one per host thread per
    round) until it has run about `target_seconds`."""
    from oracle import oracle

    B, H, L, D = cfg["B"], cfg["H"], cfg["q_len"], cfg["d"]
    qf, kf, vf, df = (t.float().numpy() for t in (q, k, v, dout))
    threads = oracle.threads_used()
    Dv = cfg.get("dv", D)
    per_head = 2.0 * (3 * D + 2 * Dv) * visible_pairs(cfg["mask"], L, cfg["kv_len"])
    spent, flops, heads_done, h0 = 0.0, 0.0, 0, 0
    while spent < target_seconds and heads_done < B * H:
        n = min(threads, B * H - h0)
        heads = np.arange(h0, h0 + n)
        t0 = time.perf_counter()
        oracle.attention_backward(qf, kf, vf, df, cfg["mask"], cfg["score"], cfg["scale"],
                                  threads=threads, heads=heads)
        spent += time.perf_counter() - t0
        flops += per_head * n
        heads_done += n
        h0 += n
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": "%d whole heads (of %d) of the workload, fp64 oracle backward, %.1f s"
                  % (heads_done, B * H, spent),
    }


def _printable_mask(mask: dict) -> dict:
    """The mask for the JSON line: document ids replaced by their count."""
    out = {k: v for k, v in mask.items() if k not in ("q_doc", "kv_doc")}
    if "q_doc" in mask:
        out["documents"] = int(len(np.unique(np.asarray(mask["q_doc"].cpu()))))
    return out


def run_bwd(args, cfg, name, q, k, v):
    """The backward measurement (see the module docstring)."""
    import torch
    from block_sparse_masked_flexattention_amd import flexattn as fa
    from block_sparse_masked_flexattention_amd.inputs import make_grad_inputs, with_doc_ids

    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    dout, _ = make_grad_inputs(cfg)
    dod = dout.to(dev)
    B, H, Lq, Lk, D = cfg["B"], cfg["H"], cfg["q_len"], cfg["kv_len"], cfg["d"]
    Dv = cfg.get("dv", D)
    bargs = (with_doc_ids(cfg, dev), Lq, Lk, cfg["q_block"], cfg["kv_block"])
    bm = fa.build_block_mask(*bargs, device=dev)
    bmt = fa.build_block_mask_t(*bargs, device=dev)
    out, lse = fa.fwd(qd, kd, vd, bm, cfg["score"], cfg["scale"], return_lse=True)
    gd = qd.dtype
    dq = torch.empty((B, H, Lq, D), dtype=gd, device=dev)
    dk = torch.empty((B, H, Lk, D), dtype=gd, device=dev)
    dv = torch.empty((B, H, Lk, Dv), dtype=gd, device=dev)
    ws = torch.empty(max(fa.bwd_workspace_floats(B, H, Lq), 1), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        fa.build_block_mask(*bargs, out=bm)
        fa.build_block_mask_t(*bargs, out=bmt)
        if ev is not None:
            ev[0].record(stream)
        fa.bwd(qd, kd, vd, out, dod, lse, bm, bmt, cfg["score"], cfg["scale"],
               grad_dtype=gd, workspace=ws, dq=dq, dk=dk, dv=dv)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    bwd_ms = [a.elapsed_time(b) for a, b in events]
    bwd_avg_ms = float(np.mean(bwd_ms))
    pairs = visible_pairs(cfg["mask"], Lq, Lk)
    flops = 2.0 * B * H * (3 * D + 2 * Dv) * pairs
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (bwd_avg_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS
    res = {
        "metric": "effective TFLOP/s (unmasked FLOPs) + % bf16 MFMA peak, flex-attn bwd",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {
            "workload": name, "B": B, "H": H, "q_len": Lq, "kv_len": Lk, "head_dim": D,
            "v_head_dim": Dv, "q_block": cfg["q_block"], "kv_block": cfg["kv_block"],
            "mask": _printable_mask(cfg["mask"]),
            "score_mod": cfg["score"]["kind"], "grad_dtype": cfg["dtype"],
            "visible_pairs_per_head": pairs,
            "step": "block-mask build (both layouts) + backward (delta, dq, dk/dv)",
        },
        "pct_peak": round(100.0 * value / peak, 2),
        "bwd_ms": round(bwd_avg_ms, 5),
        "bwd_ms_min": round(float(np.min(bwd_ms)), 5),
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": None,
            "kernels": "delta pass + dq + dk/dv, timed together",
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_bwd(cfg, q, k, v, dout, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


def _row_counts(mask, q_len, kv_len):
    """Visible keys per query row, from each row's visible interval."""
    i = np.arange(q_len, dtype=np.int64)
    lo = np.zeros(q_len, np.int64)
    hi = np.full(q_len, kv_len - 1, np.int64)
    if mask["kind"] in ("document", "document_causal"):
        # sorted ids: a row sees the run of keys with its own id
        qd = np.asarray(mask["q_doc"].cpu() if hasattr(mask["q_doc"], "cpu") else mask["q_doc"])
        kd = np.asarray(mask["kv_doc"].cpu() if hasattr(mask["kv_doc"], "cpu") else mask["kv_doc"])
        lo = np.searchsorted(kd[:kv_len], qd[:q_len], side="left").astype(np.int64)
        hi = np.searchsorted(kd[:kv_len], qd[:q_len], side="right").astype(np.int64) - 1
        if mask["kind"] == "document_causal":
            hi = np.minimum(hi, i)
    elif mask["kind"] == "causal":
        hi = np.minimum(hi, i)
    elif mask["kind"] == "sliding_window":
        lo = np.maximum(0, i - mask["window"])
        hi = np.minimum(hi, i - mask.get("window_min", 0))
    elif mask["kind"] == "prefix_causal":
        P = mask["prefix"]
        hi = np.minimum(hi, np.where(i <= P, np.maximum(P, i), i))
    return np.maximum(hi - lo + 1, 0)


def _counter_mean_kib(csv_path: str, kernel_substr: str, counter: str) -> float:
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"].startswith(counter)]
    if not vals:
        raise SystemExit("no %s samples for %r in %s" % (counter, kernel_substr, csv_path))
    return sum(vals) / len(vals)


def write_traffic_file(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv,
                       workload_name: str, nbytes: int = 1 << 30):
    """HBM bytes per forward launch from rocprofv3 FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for a plain
    device copy of `nbytes` (the copy reads and writes nbytes)."""
    copy = "copyBuffer"
    f_scale = nbytes / (1024.0 * _counter_mean_kib(copy_fetch_csv, copy, "FETCH_SIZE"))
    w_scale = nbytes / (1024.0 * _counter_mean_kib(copy_write_csv, copy, "WRITE_SIZE"))
    fetch = 1024.0 * _counter_mean_kib(fetch_csv, "fwd_kernel", "FETCH_SIZE") * f_scale
    write = 1024.0 * _counter_mean_kib(write_csv, "fwd_kernel", "WRITE_SIZE") * w_scale
    lines = [
        "# HBM traffic of the forward kernel, workload %s" % workload_name,
        "# from: rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -f csv -- python bench.py --steps 3 --warmup 1 --no-cpu-baseline --cold-reps 0 --no-extra",
        "#   and the same counters over: python bench.py --copy-calibration (a 1 GiB device copy)",
        "# counter scale factors from the copy: FETCH_SIZE x%.4f, WRITE_SIZE x%.4f" % (f_scale, w_scale),
        "workload = %s" % workload_name,
        "kernel_source_hash = %s" % kernel_source_hash(),
        "fetch_bytes_per_launch = %.0f" % fetch,
        "write_bytes_per_launch = %.0f" % write,
        "hbm_bytes_per_launch = %.0f" % (fetch + write),
    ]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def mfma_peak(reps: int = 5, iters: int = 20000) -> dict:
    """Measured dense bf16 matrix rate: the library's probe kernel (4
    independent v_mfma_f32_32x32x16_bf16 chains per wave, 4 work-groups of 4
    waves per compute unit) timed with HIP events on its stream, and the
    shader clock from each wave's cycle and real-time counters."""
    import torch
    from block_sparse_masked_flexattention_amd import flexattn as fa
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nwg = 4 * cus
    stream = torch.cuda.current_stream(dev)
    fa.mfma_peak_probe(nwg, iters, dev)  # warm-up
    torch.cuda.synchronize()
    times, clocks = [], None
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        flops, _, clocks = fa.mfma_peak_probe(nwg, iters, dev)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.median(times))
    c = clocks.cpu().numpy().reshape(-1, 2).astype(np.float64)
    ghz = float(np.median(0.1 * c[:, 0] / np.maximum(c[:, 1], 1.0)))
    tflops = flops / (ms * 1e-3) / 1e12
    return {"tflops": round(tflops, 1), "clock_ghz": round(ghz, 3), "ms": round(ms, 4),
            "frac_of_published": round(tflops / PEAK_BF16_TFLOPS, 4),
            "published_at_measured_clock": round(PEAK_BF16_TFLOPS * ghz / 2.4, 1),
            "kernel": "4 waves/SIMD x 4 independent v_mfma_f32_32x32x16_bf16 chains, %d work-groups"
                      " x %d rounds" % (nwg, iters)}


def fwd_timing(cfg, dmask, qd, kd, vd, steps: int, warmup: int, cold_reps: int,
               use_subtiling: bool = False) -> dict:
    """Warm and cold-cache forward times of one workload (HIP events on the
    launch stream), its fraction of the bf16 peak and, from its algorithmic
    bytes (q, k, v read once, out written once), of the HBM roofline."""
    import torch
    from block_sparse_masked_flexattention_amd import flexattn as fa
    dev = qd.device
    B, H, Lq, Lk, D = cfg["B"], cfg["H"], cfg["q_len"], cfg["kv_len"], cfg["d"]
    Dv = cfg.get("dv", D)
    out = torch.empty((B, H, Lq, Dv), dtype=qd.dtype, device=dev)
    bm = fa.build_block_mask(dmask, Lq, Lk, cfg["q_block"], cfg["kv_block"], device=dev)
    stream = torch.cuda.current_stream(dev)

    def run(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fwd(qd, kd, vd, bm, cfg["score"], cfg["scale"], out=out, use_subtiling=use_subtiling)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    warm = [a.elapsed_time(b) for a, b in evs]
    cold = []
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    for _ in range(cold_reps):
        flush.fill_(1.0)
        e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        run(e)
        torch.cuda.synchronize()
        cold.append(e[0].elapsed_time(e[1]))
    del flush
    pairs = visible_pairs(cfg["mask"], Lq, Lk)
    flops = 2.0 * B * H * (D + Dv) * pairs
    esz = 2 if cfg["dtype"] == "bf16" else 4
    hbm_bytes = float(esz) * B * H * (Lq * D + Lk * D + Lk * Dv + Lq * Dv)
    ms = float(np.mean(warm))
    ms_cold = float(np.median(cold)) if cold else None
    res = {"fwd_ms": round(ms, 5), "fwd_ms_min": round(float(np.min(warm)), 5),
           "fwd_ms_cold": round(ms_cold, 5) if ms_cold else None,
           "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "hbm_bytes": hbm_bytes,
           "hbm_frac": round(hbm_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "hbm_frac_cold": round(hbm_bytes / (ms_cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
           if ms_cold else None}
    return res


def sliding_window_lines(steps: int, warmup: int, cold_reps: int) -> dict:
    """The sliding-window workload with subtiling off and on (see the module
    docstring)."""
    import torch
    from block_sparse_masked_flexattention_amd.inputs import make_inputs, workload
    cfg = workload("sliding_window")
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in make_inputs(cfg))
    res = {"config": {"B": cfg["B"], "H": cfg["H"], "q_len": cfg["q_len"], "head_dim": cfg["d"],
                      "mask": cfg["mask"], "q_block": cfg["q_block"], "kv_block": cfg["kv_block"]}}
    for sub in (False, True):
        res["subtiling_on" if sub else "subtiling_off"] = fwd_timing(
            cfg, cfg["mask"], qd, kd, vd, steps, warmup, cold_reps, use_subtiling=sub)
    return res


def copy_calibration(nbytes: int, reps: int):
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    src.random_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--use-subtiling", action="store_true")
    ap.add_argument("--output-max", action="store_true",
                    help="forward: also write the row max of the scores (OUTPUT_MAX)")
    ap.add_argument("--prescale-qk", action="store_true",
                    help="forward: scale q before Q K^T (PRESCALE_QK)")
    ap.add_argument("--autotune", action="store_true",
                    help="forward: time every tile shape first and run the fastest")
    ap.add_argument("--v-head-dim", type=int, default=None,
                    help="forward: value head dim, when it should differ from the workload's head dim")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="only the matrix-unit microbenchmark: measured bf16 peak and clock")
    ap.add_argument("--no-extra", action="store_true",
                    help="forward: leave out the sliding-window and matrix-peak figures")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd"], default="fwd",
                    help="measure the forward (default) or the backward")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="forward launches timed after a cache-evicting write (0: skip)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write the traffic summary under profiles/ from rocprofv3 counter CSVs")
    args = ap.parse_args(argv)
    if args.traffic_from:
        write_traffic_file(*args.traffic_from, workload_name=args.workload or "prefix_causal")
        return 0

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested); run with --gpus 1" % args.gpus, file=sys.stderr)
        return 2

    import torch
    from block_sparse_masked_flexattention_amd import flexattn as fa
    from block_sparse_masked_flexattention_amd.inputs import (BENCH_WORKLOAD, make_inputs,
                                                              with_doc_ids, workload)

    if args.copy_calibration:
        copy_calibration(1 << 30, 5)
        return 0
    if args.mfma_peak:
        torch.cuda.set_device(0)
        fa.load()
        print(json.dumps({"mfma_peak_measured": mfma_peak()}), flush=True)
        return 0

    name = args.workload or BENCH_WORKLOAD
    cfg = workload(name, **({"dv": args.v_head_dim} if args.v_head_dim else {}))
    cfg["mask"] = with_doc_ids(cfg)  # document ids (CPU) for the oracle and the pair count
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fa.load()  # fails loudly if the HIP library is missing

    q, k, v = make_inputs(cfg)
    if args.which == "bwd":
        if cfg["dtype"] != "bf16" or cfg["d"] not in (64, 128) or cfg.get("dv", cfg["d"]) != cfg["d"]:
            print("the backward covers bf16 inputs with head dim 64 or 128 (value head dim equal); "
                  "workload %s has %s, d=%d" % (name, cfg["dtype"], cfg["d"]), file=sys.stderr)
            return 2
        return run_bwd(args, cfg, name, q, k, v)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    B, H, Lq, Lk, D = cfg["B"], cfg["H"], cfg["q_len"], cfg["kv_len"], cfg["d"]
    Dv = cfg.get("dv", D)
    out = torch.empty((B, H, Lq, Dv), dtype=qd.dtype, device=dev)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev) if cfg["lse"] else None
    mx = torch.empty((B, H, Lq), dtype=torch.float32, device=dev) if args.output_max else None
    dmask = with_doc_ids(cfg, dev)
    tuned = None
    if args.autotune:
        from block_sparse_masked_flexattention_amd import autotune
        tuned = autotune.tune_fwd(qd, kd, vd, dmask, cfg["score"], cfg["scale"], reps=10, warmup=3,
                                  use_subtiling=args.use_subtiling, prescale_qk=args.prescale_qk)
        cfg["q_block"], cfg["kv_block"] = tuned.q_block, tuned.kv_block
    bm = fa.build_block_mask(dmask, Lq, Lk, cfg["q_block"], cfg["kv_block"], device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        fa.build_block_mask(dmask, Lq, Lk, cfg["q_block"], cfg["kv_block"], out=bm)
        if ev is not None:
            ev[0].record(stream)
        fa.fwd(qd, kd, vd, bm, cfg["score"], cfg["scale"], out=out, lse=lse, max_out=mx,
               use_subtiling=args.use_subtiling, prescale_qk=args.prescale_qk)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_per_step = elapsed * 1e3 / args.steps
    fwd_ms = [a.elapsed_time(b) for a, b in events]

    # Cold-cache forward time (reported beside the warm figure, not `value`):
    # a 1 GiB write between launches evicts L2 and the 256 MB last-level cache.
    cold_ms = []
    if args.cold_reps > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        for _ in range(args.cold_reps):
            flush.fill_(1.0)
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            step(ev)
            torch.cuda.synchronize()
            cold_ms.append(ev[0].elapsed_time(ev[1]))
        del flush
    fwd_avg_ms = float(np.mean(fwd_ms))
    pairs = visible_pairs(cfg["mask"], Lq, Lk)
    flops = 2.0 * B * H * (D + Dv) * pairs  # Q K^T and P V
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (fwd_avg_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg["dtype"] == "bf16" else PEAK_FP32_TFLOPS
    traffic = stored_traffic(name)

    res = {
        "metric": "effective TFLOP/s (unmasked FLOPs) + % bf16 MFMA peak, flex-attn fwd",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {
            "workload": name, "B": B, "H": H, "q_len": Lq, "kv_len": Lk, "head_dim": D,
            "v_head_dim": Dv, "q_block": cfg["q_block"], "kv_block": cfg["kv_block"],
            "mask": _printable_mask(cfg["mask"]),
            "score_mod": cfg["score"]["kind"], "out_dtype": cfg["dtype"], "lse": cfg["lse"],
            "use_subtiling": args.use_subtiling, "output_max": args.output_max,
            "prescale_qk": args.prescale_qk, "visible_pairs_per_head": pairs,
            "autotune": None if tuned is None else {
                "chosen": [tuned.q_block, tuned.kv_block],
                "ms": {"%dx%d" % qk: round(t, 5) for qk, t in tuned.ms.items()}},
            "step": "block-mask build + forward",
        },
        "pct_peak": round(100.0 * value / peak, 2),
        "fwd_ms": round(fwd_avg_ms, 5),
        "fwd_ms_min": round(float(np.min(fwd_ms)), 5),
        "fwd_ms_cold": round(float(np.median(cold_ms)), 5) if cold_ms else None,
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic,
        },
    }
    if not args.no_extra and args.workload is None:
        res["sliding_window"] = sliding_window_lines(max(args.steps, 20), args.warmup,
                                                     args.cold_reps)
        peak = mfma_peak()
        peak["forward_frac_of_measured"] = round(achieved / peak["tflops"], 4)
        res["mfma_peak_measured"] = peak
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, q, k, v, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
