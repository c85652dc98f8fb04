"""Bench: Prox sparse SwiGLU FFN on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2_s70]

A step is one pass of the whole path over one batch of synthetic tokens:
prox_ffn_forward (Stage 1 + Stage 2, every kernel of the path) for one FFN
layer, or, for the stacked workloads (c3_*: 32 layers, c5: 64 layers), for
every layer of the stack in order (µs per token = stack time / batch).
Inputs are resident in HBM before timing starts.  Single-layer workloads
rotate several copies of the layer's weights and proxy at distinct addresses
so no step finds its weights in the 256 MB last-level cache (a stack is
larger than the cache by itself); x changes every step, so masks change too.

Prints ONE JSON line: the throughput in algorithmic HBM GB/s (the metric's
unit), µs per token, the roofline entry of the dominant kernel (timed live
with events on the launch stream), the read rate of a plain streaming kernel
on the same GPU (the practical ceiling) and the CPU oracle timed on a bounded
sample of the same workload, with one thread and with every core.
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
PEAK_MFMA_BF16_TFLOPS = 2500.0
LLC_BYTES = 256 << 20
BATCH_MIN = 4   # the library's switch to the matrix-core path (tokens per call)


def algorithmic_bytes(d, F, kind, k_in_rows, k_ch, mode="proxy"):
    """Weight bytes one forward must read at minimum.  Stage 1: the proxy codes
    of the kept rows + the proxy scales (exact mode: every gate and up row,
    bf16).  Stage 2: 3 rows per kept channel, bf16 (q8: int8 rows + 3 fp32
    scales; exact mode: the W_down row only, h being known).  For several
    tokens the kept rows / channels are the union over the batch (measured
    from the call's own outputs)."""
    if mode == "exact":
        return 2 * F * d * 2, k_ch * d * 2
    if mode == "dense":
        return 0, 3 * F * d * 2
    bits = 8 if kind == "int8" else 4
    groups = 1 if kind == "int8" else d // 128
    proxy = 2 * k_in_rows * F * bits // 8 + 2 * groups * F * 4
    stage2 = 3 * k_ch * d + 3 * k_ch * 4 if mode == "q8" else 3 * k_ch * d * 2
    return proxy, stage2


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2_s70")
    ap.add_argument("--mode", default="proxy", choices=["proxy", "exact", "q8", "dense"],
                    help="proxy: the workload's proxy and bf16 Stage 2; exact: exact-mask mode (every input "
                         "kept); q8: int8 Stage-2 rows; dense: the dense bf16 SwiGLU FFN as three torch "
                         "(hipBLASLt) products, the same-GPU reference for the layer speed-up")
    ap.add_argument("--layers", type=int, default=0, help="stacked workloads: first N layers only (0 = all)")
    ap.add_argument("--copies", type=int, default=0, help="weight copies rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="per CPU leg")
    ap.add_argument("--no-read-probe", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="time a decode step of a Llama-2-7B-shaped 32-layer stack (dense vs Prox FFNs) instead")
    ap.add_argument("--context", type=int, default=512, help="--decode: tokens already in the KV cache")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, --steps times (the reference "
                         "for scaling hardware byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding plan is design-only.", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration, args.steps)
    if args.decode:
        return decode_bench(args)

    import torch
    import free_ffn_activation_prox_amd as P

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = workloads()[args.workload]
    n_layers = wl.n_layers if not args.layers else min(args.layers, wl.n_layers)
    stack = wl.n_layers > 1
    B, kind = wl.batch, (wl.proxy if args.mode not in ("exact", "dense") else
                         ("exact" if args.mode == "exact" else wl.proxy))
    k_in_of = (lambda l: wl.layers[l].d) if args.mode == "exact" else wl.k_in

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.time()
    # per layer: a list of (weights, proxy) copies; single layers rotate copies
    sets, w0 = [], None
    for layer in range(n_layers):
        d, F = wl.layers[layer].d, wl.layers[layer].F
        w = gen_weights(wl.config_id, layer, d, F)
        if layer == 0:
            w0 = w
        base = P.Weights(up(w["wg_t"]), up(w["wu_t"]), up(w["wd"]))

        def s2rows(wt):
            return P.build_qweights(wt) if args.mode == "q8" else wt
        copies_l = [(s2rows(base), P.build_proxy(base, kind))]
        if not stack:
            layer_bytes = 3 * F * d * 2 + copies_l[0][1].desc.bytes
            copies = args.copies or max(4, int(np.ceil(4 * LLC_BYTES / layer_bytes)))
            for _ in range(min(copies, 64) - 1):
                wc = P.Weights(base.w_gate_t.clone(), base.w_up_t.clone(), base.w_down.clone())
                copies_l.append((s2rows(wc), P.build_proxy(wc, kind)))
        if args.mode == "q8":
            del base
        sets.append(copies_l)
        del w
    n_copies = len(sets[0])
    n_x = 16
    xs = [[up(gen_x(wl, layer, step=s)) for s in range(n_x)] for layer in range(n_layers)]
    shapes = sorted({(wl.layers[l].d, wl.layers[l].F) for l in range(n_layers)})
    ws = P.alloc_workspace(max(s[0] for s in shapes), max(s[1] for s in shapes), B, kind, dev)
    ws_need = max(P.workspace_bytes(d, F, B, kind) for d, F in shapes)
    assert ws.numel() >= ws_need
    bufs = {}
    for d, F in shapes:
        k_ff_max = max(wl.k_ff(l) for l in range(n_layers) if (wl.layers[l].d, wl.layers[l].F) == (d, F))
        bufs[(d, F)] = (torch.empty(B, d, dtype=torch.float32, device=dev),
                        torch.empty(B, F, dtype=torch.uint8, device=dev),
                        torch.empty(B, max(k_ff_max, 1), dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def forward(layer, i, events=None):
        d, F = wl.layers[layer].d, wl.layers[layer].F
        wt, px = sets[layer][i % n_copies]
        y, mask, idx = bufs[(d, F)]
        if args.mode == "dense":
            xb = xs[layer][i % n_x]
            if events is not None:
                events[0].record()
            h = torch.nn.functional.silu(torch.nn.functional.linear(xb, wt.w_gate_t).float()) * \
                torch.nn.functional.linear(xb, wt.w_up_t).float()
            y.copy_(torch.matmul(h.to(torch.bfloat16), wt.w_down))
            if events is not None:       # the whole torch layer in phase 0, nothing in the others
                for e in events[1:]:
                    e.record()
            return
        P.ffn_forward(xs[layer][i % n_x], wt, px, k_in_of(layer), wl.k_ff(layer), y=y, mask=mask, idx=idx,
                      workspace=ws[:P.workspace_bytes(d, F, B, kind)], events=events,
                      kernel_events=events is not None)

    def step(i, events=None):
        for layer in range(n_layers):
            forward(layer, i, None if events is None else events[layer])

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

    # per-kernel durations: the same K steps again; the kernels of every phase
    # of every layer carry a pair of events (hipExtLaunchKernel: the start of
    # the phase's first kernel, the end of its last), so a one-kernel phase is
    # timed without the dispatch gap before it
    Kp = min(K, max(1, 400 // n_layers))
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2 * P.N_PHASES)] for _ in range(n_layers)]
          for _ in range(Kp)]
    for row in ev:              # torch creates the HIP event on first record
        for lay in row:
            for e in lay:
                e.record()
    torch.cuda.synchronize()
    for i in range(Kp):
        step(args.warmup + i, ev[i])
    torch.cuda.synchronize()
    phase_ms = np.zeros(P.N_PHASES)        # per step (summed over the layers)
    for i in range(Kp):
        for lay in ev[i]:
            for p in range(P.N_PHASES):
                phase_ms[p] += lay[2 * p].elapsed_time(lay[2 * p + 1])
    phase_ms /= Kp

    # algorithmic bytes: per layer, union of kept rows / channels over the
    # batch from the outputs of one call
    proxy_b = stage2_b = io_b = 0
    for layer in range(n_layers):
        d, F = wl.layers[layer].d, wl.layers[layer].F
        k_in, k_ff = k_in_of(layer), wl.k_ff(layer)
        forward(layer, 0)
        torch.cuda.synchronize()
        m = bufs[(d, F)][1].cpu().numpy().astype(bool)
        ch_union = int(m.any(axis=0).sum())
        if B == 1:
            rows_union = k_in
        else:
            xb = xs[layer][0].float().abs().cpu().numpy()
            order = np.lexsort((np.tile(np.arange(d), (B, 1)), -xb), axis=1)[:, :k_in]
            rows_union = int(len(np.unique(order)))
        pb, sb = algorithmic_bytes(d, F, kind, rows_union, ch_union, args.mode)
        proxy_b += pb
        stage2_b += sb
        io_b += B * (2 * d + 4 * d + F + 4 * k_ff)       # x, y, mask, idx
    total_b = proxy_b + stage2_b + io_b
    gbs = total_b / (ms_per_step * 1e-3) / 1e9
    us_tok = ms_per_step * 1e3 / B

    # dominant kernel: the phase with the largest share of the step (fewer
    # than BATCH_MIN tokens: one kernel per phase; from BATCH_MIN tokens the
    # matrix-core path: stage1 = input selection + proxy GEMM, stage2 =
    # channel selection + gate/up + down)
    dom = int(np.argmax(phase_ms))
    dom_name = P.PHASES[dom]
    dom_bytes = {0: proxy_b, 1: stage2_b}.get(dom, total_b) if args.mode != "dense" else stage2_b
    dom_gbs = dom_bytes / (phase_ms[dom] * 1e-3) / 1e9
    if args.mode == "dense":
        dom_kernel = "torch SwiGLU (3 hipBLASLt products + silu * u)"
    elif args.mode == "exact":
        dom_kernel = {0: "k_exact_h", 1: "k_stage2"}.get(dom, "k_reduce_y")
    elif B < BATCH_MIN or args.mode == "q8" and dom == 1:
        dom_kernel = {0: "k_stage1" if B < BATCH_MIN else "k_xsel + k_proxy_batch", 1: "k_stage2"}.get(dom, "k_reduce_y")
    else:
        dom_kernel = {0: "k_xsel + k_proxy_batch",
                      1: "k_stage2 (selection) + k_gateup_batch + k_down_batch"}.get(dom, "k_reduce_y")
    # prefill (more than 64 tokens per call): bound by the matrix cores; the
    # phase events time only the last 64-token sub-batch, so the roofline
    # entry is the whole call's algorithmic flops over its step time
    prefill = B > 64
    if prefill:
        flops = 0
        for layer in range(n_layers):
            d, F = wl.layers[layer].d, wl.layers[layer].F
            flops += B * (6 * F * d if args.mode == "dense" else 4 * k_in_of(layer) * F + 6 * wl.k_ff(layer) * d)
        tflops = flops / (ms_per_step * 1e-3) / 1e12
    src_hash = kernel_sources_hash()
    prof = committed_profile(wl.name, dom_kernel, src_hash, n_layers) if args.mode == "proxy" else {}
    probe = None if args.no_read_probe else read_probe_gbs(P, torch, dev)

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
        "pct_of_read_probe": round(100.0 * gbs / probe, 2) if probe else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": {"proxy": "Stage 2: bf16 weights, fp32 accumulation; Stage 1: int8/int4 codes x bf16 x, "
                                  "fp32 exact chunk sums into fp64 totals",
                         "exact": "Stage 1: bf16 gate/up rows x bf16 x, fp64 accumulation; Stage 2: bf16 W_down rows, "
                                  "fp32 accumulation",
                         "q8": "Stage 2: int8 rows x fp32 row scales, fp32 accumulation; Stage 1 as proxy",
                         "dense": "bf16 products, fp32 accumulation (torch)"}[args.mode],
        "data": "synthetic (seeded N(0,0.02) bf16 weights, Laplace x with outliers or RMS-normalised; "
                "random-init, no checkpoint)",
        "config": {"workload": f"{wl.name}: d_model={'/'.join(str(s[0]) for s in shapes)} "
                               f"d_ff={'/'.join(str(s[1]) for s in shapes)} layers={n_layers} batch={B} "
                               f"proxy={kind} keep={100 if args.mode == 'exact' else wl.keep_pct}% "
                               f"sparsity={wl.sparsity_pct}% stage2={'int8 rows' if args.mode == 'q8' else 'bf16'}",
                   "mode": args.mode,
                   "layers": n_layers, "batch": B, "proxy": kind,
                   "k_in": [k_in_of(l) for l in range(min(n_layers, 2))],
                   "k_ff": [wl.k_ff(l) for l in range(min(n_layers, 2))],
                   "weight_copies_rotated": n_copies, "algorithmic_bytes_per_step": int(total_b)},
        "phase_us": {P.PHASES[p]: round(float(phase_ms[p] * 1e3), 2) for p in range(P.N_PHASES)},
        "roofline": {"bound": "hbm", "kernel": dom_kernel, "phase": dom_name, "achieved": round(dom_gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(dom_gbs / PEAK_HBM_GBS, 4),
                     "traffic": prof.get("traffic"), "algorithmic_bytes": int(dom_bytes),
                     "timing": "events carried by the kernel's own launch (hipExtLaunchKernel): its execution, "
                               "averaged over the timed steps",
                     "rocprof_avg_us": prof.get("avg_us"),
                     "achieved_rocprof": round(dom_bytes / n_layers / (prof["avg_us"] * 1e-6) / 1e9, 1)
                     if prof.get("avg_us") else None,
                     "frac_rocprof": round(dom_bytes / n_layers / (prof["avg_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
                     if prof.get("avg_us") else None,
                     "profile": prof.get("file"),
                     "layer_achieved": round(gbs, 1), "layer_frac": round(gbs / PEAK_HBM_GBS, 4)},
        "read_probe_GBps": round(probe, 1) if probe else None,
        **({"roofline": {"bound": "mfma", "kernel": "whole call: sub-batches of 64 tokens (k_xsel, k_proxy_batch, "
                                                  "k_stage2 selection, k_gateup_batch, k_down_batch, k_reduce_y)"
                         if args.mode != "dense" else dom_kernel,
                         "achieved": round(tflops, 2), "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4), "traffic": None,
                         "algorithmic_flops": int(flops),
                         "flops_definition": "per token 4*k_in*d_ff (proxy) + 6*k_ff*d_model (Stage 2)"
                         if args.mode != "dense" else "per token 6*d_ff*d_model"}} if prefill else {}),
        "kernel_sources_sha256": src_hash,
        "library": {"path": os.path.relpath(P.LIB_PATH, ROOT), "sha256": P.library_sha256()},
        "setup_s": round(setup_s, 1),
    }

    if not args.no_cpu_baseline and args.mode == "proxy":
        out["cpu_baseline"] = cpu_baseline(wl, w0, xs[0], total_b / n_layers / B, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def read_probe_gbs(P, torch, dev, gib=2, reps=10):
    """Read rate of a plain streaming kernel over `gib` GiB (eight times the
    last-level cache, so the reads come from HBM): the practical ceiling.  The
    best median over a few grid sizes."""
    n = gib << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device=dev)
    best = 0.0
    for blocks in (256, 512, 1024, 2048):
        sink = torch.empty(blocks * 512, dtype=torch.int32, device=dev)
        for _ in range(3):
            P.read_probe(buf, sink, blocks)
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            P.read_probe(buf, sink, blocks)
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        best = max(best, n / (float(np.median(times)) * 1e-3) / 1e9)
    del buf
    return best


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


def committed_profile(workload, kernel, src_hash, n_layers):
    """rocprofv3 figures of the dominant kernel from the committed summaries of
    this workload (profiles/prox_forward_<workload>_kernel_stats.md and
    _hbm_bytes.md), used only while the kernel sources match the ones they were
    taken on: average kernel duration (µs) and HBM bytes per launch (FETCH_SIZE +
    WRITE_SIZE, each scaled by the plain-copy factor).  Empty when there is no
    matching summary."""
    out = {}
    names = [k.strip() for k in kernel.split("+")]
    if len(names) != 1 or n_layers != 1:
        return out            # several kernels per phase, or a stack: no single-kernel figure
    pat = f"prox::{names[0]}<" if "<" not in names[0] else names[0]

    def rows(path):
        if not os.path.exists(path):
            return None
        text = open(path).read()
        m = re.search(r"Kernel sources sha256: ([0-9a-f]+)", text)
        if not m or m.group(1) != src_hash:
            return None
        return [[c.strip() for c in line.split("|")] for line in text.splitlines() if line.startswith("|")]

    base = os.path.join(ROOT, "profiles", f"prox_forward_{workload}")
    st = rows(base + "_kernel_stats.md")
    if st:
        for cells in st:
            if len(cells) > 4 and (pat in cells[1] or f"prox::{names[0]}(" in cells[1]):
                out["avg_us"] = float(cells[3])
                out["file"] = os.path.relpath(base + "_kernel_stats.md", ROOT)
                break
    hb = rows(base + "_hbm_bytes.md")
    if hb:
        for cells in hb:
            if len(cells) > 7 and (pat in cells[1] or f"prox::{names[0]}(" in cells[1]):
                out["traffic"] = int(round((float(cells[5]) + float(cells[6])) * 1e6))
                break
    return out


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


def decode_bench(args):
    """One decode step (batch 1, one token through all 32 layers, KV cache of
    --context tokens) of a random-weight Llama-2-7B-shaped decoder (d 4096,
    d_ff 11008, 32 heads), with dense bf16 FFNs (torch / hipBLASLt) and with
    Prox FFNs (int8 proxy, keep 60 %, sparsity 70 %; bf16 and int8 Stage-2
    rows).  Attention and the rest of the block are the same torch code in
    every variant.  Steps are timed with events on the current stream."""
    import torch
    from free_ffn_activation_prox_amd.decode import DecodeHarness, DecoderShape, random_layers
    wl = workloads()["c2_s70"]
    sh = DecoderShape(n_layers=32, d=4096, F=11008, n_heads=32, n_kv=32)
    t0 = time.time()
    layers = random_layers(sh, lambda l: gen_weights(wl.config_id, l, sh.d, sh.F), seed=0)
    k_in, k_ff = wl.k_in(), wl.k_ff()
    variants = {"dense": DecodeHarness(sh, layers, args.context + args.steps + args.warmup + 1, ffn="dense")}
    # the dense FFN on this library's kernels: exact mode keeping every channel
    variants["dense_library"] = DecodeHarness(sh, layers, args.context + args.steps + args.warmup + 1, ffn="exact",
                                              k_in=sh.d, k_ff=sh.F)
    for name, ffn in (("prox_int8", "prox"), ("prox_int8_q8rows", "q8")):
        variants[name] = DecodeHarness(sh, layers, args.context + args.steps + args.warmup + 1, ffn=ffn,
                                       proxy="int8", k_in=k_in, k_ff=k_ff)
    for h in variants.values():
        h.fill_cache(args.context, seed=1)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    x0 = torch.from_numpy(np.random.default_rng(0).standard_normal((1, sh.d)).astype(np.float32)).cuda()
    ms, ms_graph = {}, {}
    for name, h in variants.items():
        x = x0
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(args.warmup):
                x = h.step(x)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            x = h.step(x)
        b.record()
        torch.cuda.synchronize()
        ms[name] = a.elapsed_time(b) / args.steps
        # the GPU time of a step without the host's per-op launch cost: one step
        # captured in a graph and replayed (every replay at the same cache
        # position, i.e. the same context length)
        g = torch.cuda.CUDAGraph()
        xs = x.clone()
        with torch.cuda.graph(g):
            ys = h.step(xs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        ms_graph[name] = a.elapsed_time(b) / args.steps
        del g, ys
    out = {"metric": "decode step ms (Llama-2-7B-shaped 32-layer stack, batch 1)", "unit": "ms",
           "higher_is_better": False, "steps": args.steps, "warmup": args.warmup,
           "config": {"workload": f"decode: 32 layers d=4096 d_ff=11008 heads=32 context={args.context} "
                                  f"batch=1; Prox FFN int8 proxy keep=60% sparsity=70% (k_in={k_in} k_ff={k_ff})"},
           "ms_per_step": {k: round(v, 4) for k, v in ms_graph.items()},
           "speedup_vs_dense": {k: round(ms_graph["dense"] / v, 3) for k, v in ms_graph.items() if k != "dense"},
           "speedup_vs_dense_library": {k: round(ms_graph["dense_library"] / v, 3) for k, v in ms_graph.items()
                                        if k.startswith("prox")},
           "variants": {"dense": "FFN as three bf16 torch products (hipBLASLt)",
                        "dense_library": "FFN through this library's exact mode with every channel kept (k_ff = d_ff)",
                        "prox_int8": "Prox FFN, bf16 Stage-2 rows", "prox_int8_q8rows": "Prox FFN, int8 Stage-2 rows"},
           "timing": "ms_per_step: one step captured in a HIP graph and replayed (GPU time; every replay at the "
                     "same cache position); eager_ms_per_step: the same step launched op by op from Python",
           "eager_ms_per_step": {k: round(v, 4) for k, v in ms.items()},
           "context_pages": "1.99x end-to-end decode at 70% FFN sparsity (hardware, model and batch not stated)",
           "data": "synthetic random-init weights (attention N(0,0.02), FFN as workload c2), random KV cache",
           "setup_s": round(setup_s, 1)}
    print(json.dumps(out), flush=True)
    return 0


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, w, xs, bytes_per_token, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    single-token forwards of layer 0, one token each, for about budget_s with
    one BLAS thread and again with every core."""
    from oracle import prox_oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    f64 = O.bf16_bits_to_f64
    wg, wu, wd = f64(w["wg_t"]), f64(w["wu_t"]), f64(w["wd"])
    proxies = (O.build_proxy(wg.T, wl.proxy), O.build_proxy(wu.T, wl.proxy))
    import torch
    xs_h = [f64(x.view(torch.int16).cpu().numpy().view(np.uint16)) for x in xs]
    k_in, k_ff = wl.k_in(0), wl.k_ff(0)

    def leg(threads):
        with threadpool_limits(limits=threads):
            used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
            n = 0
            t0 = time.time()
            while True:
                O.oracle_forward(xs_h[n % len(xs_h)][:1], wg, wu, wd, wl.proxy, k_in, k_ff, proxies=proxies)
                n += 1
                if time.time() - t0 >= budget_s:
                    break
            dt = time.time() - t0
        return n, dt, used

    all_cores = os.cpu_count() or 1
    n1, dt1, used1 = leg(1)
    nN, dtN, usedN = leg(all_cores)
    per1, perN = dt1 / n1, dtN / nN
    return {"value": round(bytes_per_token / perN / 1e9, 4), "unit": "GB/s", "cores": int(usedN),
            "kind": "oracle", "us_per_token": round(perN * 1e6, 1), "cpu_model": cpu_model(),
            "host_cpus": all_cores,
            "single_thread": {"value": round(bytes_per_token / per1 / 1e9, 4), "unit": "GB/s", "cores": int(used1),
                              "us_per_token": round(per1 * 1e6, 1)},
            "sample": f"single-token oracle forwards of {wl.name} layer 0 (float64 numpy, proxies prebuilt): "
                      f"{nN} in {dtN:.1f} s on {usedN} threads, {n1} in {dt1:.1f} s on 1 thread"}


if __name__ == "__main__":
    sys.exit(main())
