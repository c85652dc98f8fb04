"""Bench: Prox sparse SwiGLU FFN layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2_s70]

A step is one prox_ffn_forward (Stage 1 + Stage 2, every phase of the path)
over one batch of synthetic tokens for one FFN layer.  Inputs are resident in
HBM before timing starts.  Several copies of the layer's weights and proxy at
distinct addresses are rotated step by step so no step finds its weights in
the 256 MB last-level cache; x changes every step, so masks change too.

Prints ONE JSON line: the layer throughput in algorithmic HBM GB/s (the
metric's unit), microseconds per token, the roofline entry of the dominant
kernel (timed live with events on the launch stream) and the CPU oracle
timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from prox_workloads import gen_weights, gen_x, workloads  # noqa: E402

METRIC = "sparse FFN-layer µs/token and achieved HBM GB/s (% peak) at 70% sparsity"
PEAK_HBM_GBS = 8000.0
LLC_BYTES = 256 << 20
BATCH_MIN = 4   # the library's switch to the matrix-core path (tokens per call)


def algorithmic_bytes(d, F, kind, k_in_rows, k_ch, B):
    """Weight bytes one forward must read at minimum: proxy codes of the kept
    rows + proxy scales (Stage 1) and 3 bf16 rows per kept channel (Stage 2).
    For B > 1 the kept rows / channels are the union over the batch (measured
    from the call's own outputs)."""
    bits = 8 if kind == "int8" else 4
    groups = 1 if kind == "int8" else d // 128
    proxy = 2 * k_in_rows * F * bits // 8 + 2 * groups * F * 4
    stage2 = 3 * k_ch * d * 2
    return proxy, stage2


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2_s70")
    ap.add_argument("--copies", type=int, default=0, help="weight copies rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, --steps times (the reference "
                         "for scaling hardware byte counters)")
    args = ap.parse_args(argv)

    if args.copy_calibration:
        return copy_calibration(args.copy_calibration, args.steps)

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding plan is design-only.", file=sys.stderr)
        return 2

    import torch
    import free_ffn_activation_prox_amd as P

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = workloads()[args.workload]
    layer = 0
    d, F = wl.layers[layer].d, wl.layers[layer].F
    B, kind = wl.batch, wl.proxy
    k_in, k_ff = wl.k_in(layer), wl.k_ff(layer)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.time()
    w = gen_weights(wl.config_id, layer, d, F)
    base = P.Weights(up(w["wg_t"]), up(w["wu_t"]), up(w["wd"]))
    base_proxy = P.build_proxy(base, kind)
    layer_bytes = 3 * F * d * 2 + base_proxy.desc.bytes
    copies = args.copies or max(4, int(np.ceil(4 * LLC_BYTES / layer_bytes)))
    copies = min(copies, 64)
    sets = [(base, base_proxy)]
    for _ in range(copies - 1):
        wc = P.Weights(base.w_gate_t.clone(), base.w_up_t.clone(), base.w_down.clone())
        sets.append((wc, P.build_proxy(wc, kind)))
    n_x = 16
    xs = [up(gen_x(wl, layer, step=s)) for s in range(n_x)]
    ws = P.alloc_workspace(d, F, B, kind, dev)
    y = torch.empty(B, d, dtype=torch.float32, device=dev)
    mask = torch.empty(B, F, dtype=torch.uint8, device=dev)
    idx = torch.empty(B, max(k_ff, 1), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def step(i, events=None):
        wt, px = sets[i % copies]
        P.ffn_forward(xs[i % n_x], wt, px, k_in, k_ff, y=y, mask=mask, idx=idx, workspace=ws,
                      events=events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps (the library launches on torch's current stream)
    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        step(args.warmup + i)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / K

    # per-kernel durations: the same K steps again, with events at every phase
    # boundary recorded by the library on its launch stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(P.N_PHASES + 1)] for _ in range(K)]
    for row in ev:              # torch creates the HIP event on first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(K):
        step(args.warmup + i, ev[i])
    torch.cuda.synchronize()
    phase_ms = np.zeros(P.N_PHASES)
    for i in range(K):
        for p in range(P.N_PHASES):
            phase_ms[p] += ev[i][p].elapsed_time(ev[i][p + 1])
    phase_ms /= K

    # union of kept rows / channels over the batch, from the outputs of one call
    step(0)
    torch.cuda.synchronize()
    m = mask.cpu().numpy().astype(bool)
    ch_union = int(m.any(axis=0).sum())
    if B == 1:
        rows_union = k_in
    else:
        xb = xs[0].float().abs().cpu().numpy()
        order = np.lexsort((np.tile(np.arange(d), (B, 1)), -xb), axis=1)[:, :k_in]
        rows_union = int(len(np.unique(order)))
    proxy_b, stage2_b = algorithmic_bytes(d, F, kind, rows_union, ch_union, B)
    io_b = B * (2 * d + 4 * d + F + 4 * k_ff)       # x, y, mask, idx
    total_b = proxy_b + stage2_b + io_b
    gbs = total_b / (ms_per_step * 1e-3) / 1e9
    us_tok = ms_per_step * 1e3 / B

    # dominant kernel: the phase with the largest share of the step (fewer
    # than BATCH_MIN tokens: one kernel per phase; from BATCH_MIN tokens the
    # matrix-core path: stage1 = input selection + proxy GEMM, stage2 =
    # channel selection + gate/up + down)
    dom = int(np.argmax(phase_ms))
    dom_name = P.PHASES[dom]
    dom_bytes = {0: proxy_b, 1: stage2_b}.get(dom, total_b)
    dom_gbs = dom_bytes / (phase_ms[dom] * 1e-3) / 1e9
    if B < BATCH_MIN:
        dom_kernel = {0: "k_stage1", 1: "k_stage2"}.get(dom, "k_reduce_y")
    else:
        dom_kernel = {0: "xsel + k_proxy_batch", 1: "k_stage2 (selection) + k_gateup_batch + k_down_batch"}.get(dom, "k_reduce_y")
    traffic = measured_traffic(wl.name, dom_kernel) if B < BATCH_MIN else None

    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_token": round(us_tok, 3),
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "pct_of_peak_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": "Stage 2: bf16 weights, fp32 accumulation; Stage 1: int8/int4 codes x bf16 x, fp64 accumulation",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, Laplace x with outliers; random-init, no checkpoint)",
        "config": {"workload": f"{wl.name}: d_model={d} d_ff={F} batch={B} proxy={kind} "
                               f"keep={wl.keep_pct}% sparsity={wl.sparsity_pct}%",
                   "d_model": d, "d_ff": F, "batch": B, "proxy": kind, "k_in": k_in, "k_ff": k_ff,
                   "weight_copies_rotated": copies, "algorithmic_bytes_per_step": int(total_b)},
        "phase_us": {P.PHASES[p]: round(float(phase_ms[p] * 1e3), 2) for p in range(P.N_PHASES)},
        "roofline": {"bound": "hbm", "kernel": dom_kernel, "phase": dom_name, "achieved": round(dom_gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(dom_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": int(dom_bytes),
                     "layer_achieved": round(gbs, 1), "layer_frac": round(gbs / PEAK_HBM_GBS, 4)},
        "kernel_sources_sha256": kernel_sources_hash(),
        "setup_s": round(setup_s, 1),
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, layer, w, xs, k_in, k_ff, total_b / B, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def kernel_sources_hash():
    """sha256 (first 16 hex digits) of the library's kernel sources and header."""
    files = sorted(glob.glob(os.path.join(ROOT, "free_ffn_activation_prox_amd", "csrc", "*.hip")) +
                   glob.glob(os.path.join(ROOT, "free_ffn_activation_prox_amd", "csrc", "*.hpp")))
    files.append(os.path.join(ROOT, "include", "prox.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary of
    this workload (FETCH_SIZE + WRITE_SIZE, each scaled by the plain-copy
    factor), or None when there is none or the kernel sources have changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"prox_forward_{workload}_hbm_bytes.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"Kernel sources sha256: ([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_sources_hash():
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.split("|")]
        if len(cells) > 7 and f"prox::{kernel}<" in cells[1]:
            return int(round((float(cells[5]) + float(cells[6])) * 1e6))
    return None


def copy_calibration(mib, steps):
    """A plain device-to-device copy of known size: it reads and writes exactly
    mib MiB per launch, so hardware byte counters read on it give the factor
    between what they report and the bytes moved."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        dst.copy_(src)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": steps + 3,
                      "us_per_copy": round(ms * 1e3, 2), "GBps": round(2 * n / (ms * 1e-3) / 1e9, 1)}),
          flush=True)
    return 0


def cpu_baseline(wl, layer, w, xs, k_in, k_ff, bytes_per_token, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    tokens of the same layer, one oracle forward each, until about budget_s."""
    from oracle import prox_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    f64 = O.bf16_bits_to_f64
    wg, wu, wd = f64(w["wg_t"]), f64(w["wu_t"]), f64(w["wd"])
    proxies = (O.build_proxy(wg.T, wl.proxy), O.build_proxy(wu.T, wl.proxy))
    xs_h = [f64(x.view(__import__("torch").int16).cpu().numpy().view(np.uint16)) for x in xs]
    n = 0
    t0 = time.time()
    while True:
        xb = xs_h[n % len(xs_h)][:1]
        O.oracle_forward(xb, wg, wu, wd, wl.proxy, k_in, k_ff, proxies=proxies)
        n += 1
        if time.time() - t0 >= budget_s:
            break
    dt = time.time() - t0
    per_tok = dt / n
    return {"value": round(bytes_per_token / per_tok / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "us_per_token": round(per_tok * 1e6, 1),
            "sample": f"{n} single-token oracle forwards of {wl.name} layer {layer} "
                      f"(float64 numpy, proxies prebuilt), {dt:.1f} s"}


if __name__ == "__main__":
    sys.exit(main())
