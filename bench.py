"""Benchmark of one DDTree verify step on one MI355X.

A step is the whole hot path on one batch of synthetic input: one layer of
tree-verify attention for a budget-22 tree (23 nodes) over a 128K-row Q4_0
KV cache (24 query / 4 KV heads, head_dim 256, no window), then greedy
acceptance over 23 x 152000 fp32 logits. Inputs are resident in HBM before
the timed region; the KV cache rotates over enough copies (>= 1 GiB) that
the 256 MB Infinity Cache cannot hold it between steps.

Prints one JSON line. `value` is verify steps per second. Extra fields give
the effective KV bandwidth, the chain-16 comparison, the roofline of the
attention launch and the CPU oracle's speed on a bounded sample.
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

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA

METRIC = "tree-verify steps/s and effective KV GB/s (% HBM peak), budget 22 @128K ctx"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # a cold device needs about a hundred milliseconds of work to reach its
    # steady clocks; the long timed bracket lets the host run ahead of the
    # device by a deep queue, so a brief host-side stall does not idle it
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="long", choices=["long", "27b", "window"])
    ap.add_argument("--kv", default="q4_0", choices=["q4_0", "f16"])
    ap.add_argument("--rotate-bytes", type=float, default=1.1e9, help="KV bytes the copies span at least")
    ap.add_argument("--window-mode", type=int, default=0, choices=[0, 1],
                    help="1: per-position sliding window (a node at depth k sees positions [n_ctx+k-W, n_ctx+k])")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=552, help="oracle output rows timed for the CPU baseline")
    ap.add_argument("--no-full-step", action="store_true", help="skip the 16-layer verify-step measurement")
    ap.add_argument("--sweep", action="store_true",
                    help="attention cost against tree size (1..64 nodes), context and KV type; one JSON line per "
                         "point, then a markdown table")
    ap.add_argument("--copy-calibration", type=float, default=0.0,
                    help="only copy a device buffer of this many bytes --steps times (HBM counter calibration)")
    return ap.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_128k_q4_0_hbm_traffic.md")


def kernel_sources_sha256():
    """Hash of the HIP sources and build flags of libtv.so: a stored counter
    figure applies only to the kernels it was measured on."""
    import hashlib
    pkg = os.path.join(ROOT, "tree_verify_attention_ddtree_amd")
    h = hashlib.sha256()
    for name in sorted(os.listdir(os.path.join(pkg, "csrc"))):
        with open(os.path.join(pkg, "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    with open(os.path.join(pkg, "build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per attention launch from the rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes (copy-calibrated) stored under profiles/, or None when
    the kernels have changed since they were taken."""
    try:
        fields = {}
        with open(TRAFFIC_PROFILE) as f:
            for line in f:
                if ":" in line and not line.startswith(" "):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("sources_sha256") != kernel_sources_sha256():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(nbytes, steps):
    """A plain device-to-device copy of known size, the yardstick that scales
    the HBM byte counters (FETCH_SIZE / WRITE_SIZE) of the other kernels."""
    import torch
    src = torch.ones(int(nbytes) // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4, "steps": steps}))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the step is measured on one GPU (the library runs one GPU's "
                                   "share of a sharded step); run with --gpus 1"}))
        sys.exit(2)
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration, args.steps)
        return
    if args.sweep:
        budget_sweep(args)
        return

    import torch

    import synth
    import tree_verify_attention_ddtree_amd as tv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = dict(synth.WORKLOADS[args.workload])
    Hq, Hkv, D, T = w["n_q_heads"], w["n_kv_heads"], w["head_dim"], w["n_ctx"]
    W = w.get("window", 0)
    vocab = synth.WORKLOADS["full"]["vocab"]
    kvt = tv.TV_KV_Q4_0 if args.kv == "q4_0" else tv.TV_KV_F16

    inp = synth.attn_inputs(**w, kv=args.kv)
    parent = inp["parent"]
    n = len(parent)
    s = synth.streams(w["seed"])
    tokens = synth.sibling_distinct_tokens(s["tokens"], parent, vocab)
    logits, planted_L, _ = synth.planted_logits(s["logits"], parent, tokens, vocab)

    kc0 = torch.from_numpy(inp["k_cache"]).to(dev)
    vc0 = torch.from_numpy(inp["v_cache"]).to(dev)
    kv_bytes_alloc = 2 * kc0.numel() * kc0.element_size()
    n_copies = max(1, int(np.ceil(args.rotate_bytes / kv_bytes_alloc)))
    caches = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(n_copies - 1)]
    q = torch.from_numpy(inp["q"]).to(dev)
    kt = torch.from_numpy(inp["k_tree"]).to(dev)
    vt = torch.from_numpy(inp["v_tree"]).to(dev)
    out = torch.empty((n, Hq, D), dtype=torch.float32, device=dev)
    ts, hs = tv.cache_strides(kc0, kvt)
    desc, _par = tv.make_desc(parent, Hq, Hkv, D, kvt, T, W, inp["scale"], ts, hs, window_mode=args.window_mode)
    wsb = tv.tv_attn_workspace_bytes(desc)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    lg = torch.from_numpy(logits).to(dev)
    am = torch.empty(n, dtype=torch.int32, device=dev)
    res = torch.empty(2 + 2 * n, dtype=torch.int32, device=dev)
    aws = torch.zeros(tv.tv_accept_workspace_bytes(n, vocab), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    # chain-16 comparison (same cache, block-size-16 chain instead of the tree)
    chain = synth.chain_tree(16)
    cdesc, _cpar = tv.make_desc(chain, Hq, Hkv, D, kvt, T, W, inp["scale"], ts, hs, window_mode=args.window_mode)
    cws = torch.empty(max(tv.tv_attn_workspace_bytes(cdesc), 16), dtype=torch.uint8, device=dev)
    cq, ckt, cvt = q[:16].contiguous(), kt[:16].contiguous(), vt[:16].contiguous()
    cout = torch.empty((16, Hq, D), dtype=torch.float32, device=dev)

    def attn(i):
        kc, vc = caches[i % n_copies]
        tv.tree_verify_attn(desc, kc, vc, q, kt, vt, out, ws, wsb, stream)

    def accept():
        tv.tree_accept(lg, parent, tokens, am, res, aws, stream)

    def step(i):
        attn(i)
        accept()

    def timed(fn, k):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(k):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k  # ms per call

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step = timed(step, args.steps)
    # per-launch durations of the parts, same stream, same rotation
    ms_attn = timed(attn, args.steps)
    ms_accept = timed(lambda i: accept(), args.steps)
    ms_chain = timed(lambda i: tv.tree_verify_attn(cdesc, caches[i % n_copies][0], caches[i % n_copies][1], cq,
                                                   ckt, cvt, cout, cws, None, stream), args.steps)
    assert int(res[0].item()) == planted_L


    # algorithmic work of one attention launch
    R = T - max(0, T - W) if W > 0 else T
    row_bytes = (D // 32 * 18) if args.kv == "q4_0" else 2 * D
    kv_bytes = 2 * Hkv * R * row_bytes
    flops = 4.0 * Hq * n * R * D
    kv_gbps = kv_bytes / (ms_attn * 1e-3) / 1e9
    tflops = flops / (ms_attn * 1e-3) / 1e12
    chain_kv_gbps = kv_bytes / (ms_chain * 1e-3) / 1e9

    traffic = measured_traffic() if (args.workload == "long" and args.kv == "q4_0") else None
    line = {
        "metric": METRIC,
        "value": 1e3 / ms_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": (f"one verify step: tree-verify attention (1 layer, {Hq} q / {Hkv} kv heads, head_dim {D}, "
                         f"ctx {T}, window {W}, {args.kv} KV, budget-22 tree of {n} nodes) + greedy acceptance "
                         f"over {n}x{vocab} fp32 logits"),
            "kv": args.kv, "n_ctx": T, "window": W, "window_mode": args.window_mode, "n_nodes": n, "vocab": vocab,
            "kv_copies_rotated": n_copies,
        },
        "kv_gbps": kv_gbps,
        "kv_frac_hbm_peak": kv_gbps / HBM_PEAK_GBPS,
        "attn_us": ms_attn * 1e3,
        "accept_us": ms_accept * 1e3,
        "chain16_attn_us": ms_chain * 1e3,
        "chain16_kv_gbps": chain_kv_gbps,
        "roofline": {
            "kernel": "tree_verify_attn launch (split kernel + merge kernel)",
            "bound": "mfma",
            "achieved": tflops,
            "peak": MFMA_FP16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_FP16_PEAK_TFLOPS,
            "traffic": traffic,
            "traffic_unit": "bytes per attention launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE x1, copy-calibrated)",
            "algorithmic_flops": flops,
            "algorithmic_kv_bytes": kv_bytes,
        },
    }

    if not args.no_full_step and args.workload == "long" and args.kv == "q4_0":
        line.update(full_step(tv, synth, dev, stream, max(5, args.steps // 2)))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, logits, parent, tokens, args.cpu_rows)
    print(json.dumps(line), flush=True)


def full_step(tv, synth, dev, stream, steps):
    """A whole decode step of a 16-layer model of the same head layout at 32K
    context: 16 tree-verify attention launches over 16 distinct Q4_0 layer
    caches (604 MB together), the acceptance, then the KV commit of the
    accepted path into each of the 16 caches (rows past n_ctx, so every step
    reads the same context). Timed back to back (pipelined) and with the
    step's result copied to the host and the stream synchronised after every
    step, as a decode loop must."""
    import torch
    w = dict(synth.WORKLOADS["full"])
    T = w["n_ctx"]
    cap = T + 64
    layers = []
    for layer in range(w["n_layers"]):
        inp = synth.attn_inputs(**dict(w, seed=5000 + 100 * layer))
        t = {k: torch.from_numpy(inp[k]).to(dev) for k in ("q", "k_tree", "v_tree")}
        for k in ("k_cache", "v_cache"):
            c = torch.empty((w["n_kv_heads"], cap, inp[k].shape[2]), dtype=torch.uint8, device=dev)
            c[:, :T] = torch.from_numpy(inp[k]).to(dev)
            t[k] = c
        ts, hs = tv.cache_strides(t["k_cache"], tv.TV_KV_Q4_0)
        desc, par = tv.make_desc(inp["parent"], w["n_q_heads"], w["n_kv_heads"], w["head_dim"], tv.TV_KV_Q4_0,
                                 T, 0, inp["scale"], ts, hs)
        wsb = tv.tv_attn_workspace_bytes(desc)
        t["ws"] = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        t["wsb"], t["desc"], t["par"] = wsb, desc, par
        t["cdesc"] = tv.make_commit_desc(len(inp["parent"]), w["n_kv_heads"], w["head_dim"], tv.TV_KV_Q4_0, T, cap,
                                         ts, hs)
        t["out"] = torch.empty((len(inp["parent"]), w["n_q_heads"], w["head_dim"]), dtype=torch.float32, device=dev)
        layers.append(t)
    parent = synth.attn_inputs(**dict(w, seed=5000))["parent"]
    s = synth.streams(w["seed"])
    tokens = synth.sibling_distinct_tokens(s["tokens"], parent, w["vocab"])
    logits, planted_L, _ = synth.planted_logits(s["logits"], parent, tokens, w["vocab"])
    n = len(parent)
    lg = torch.from_numpy(logits).to(dev)
    am = torch.empty(n, dtype=torch.int32, device=dev)
    res = torch.empty(2 + 2 * n, dtype=torch.int32, device=dev)
    aws = torch.zeros(tv.tv_accept_workspace_bytes(n, w["vocab"]), dtype=torch.uint8, device=dev)
    host = torch.empty(2 + 2 * n, dtype=torch.int32, pin_memory=True)
    # every layer's cache has the same shape and strides: one commit launch
    k_trees, v_trees = [t["k_tree"] for t in layers], [t["v_tree"] for t in layers]
    k_caches, v_caches = [t["k_cache"] for t in layers], [t["v_cache"] for t in layers]

    def one_step():
        for t in layers:
            tv.tree_verify_attn(t["desc"], t["k_cache"], t["v_cache"], t["q"], t["k_tree"], t["v_tree"], t["out"],
                                t["ws"], t["wsb"], stream)
        tv.tree_accept(lg, parent, tokens, am, res, aws, stream)
        tv.tree_commit_kv_layers(layers[0]["cdesc"], res, k_trees, v_trees, k_caches, v_caches, stream)

    for _ in range(3):
        one_step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        one_step()
    e1.record(stream)
    torch.cuda.synchronize()
    pipelined_ms = e0.elapsed_time(e1) / steps
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step()
        host.copy_(res, non_blocking=True)
        stream.synchronize()
    synced_ms = (time.perf_counter() - t0) * 1e3 / steps
    assert int(host[0]) == planted_L
    return {
        "full_step": {
            "workload": "16 layers x (24 q / 4 kv heads, head_dim 256, 32768 Q4_0 rows, budget-22 tree) + acceptance "
                        "over 23x152000 logits + KV commit of the accepted path into the 16 layers (one launch)",
            "steps_per_s_pipelined": 1e3 / pipelined_ms,
            "ms_per_step_pipelined": pipelined_ms,
            "steps_per_s_with_host_sync": 1e3 / synced_ms,
            "ms_per_step_with_host_sync": synced_ms,
            "kv_gbps": 16 * 2 * 4 * 32768 * 144 / (pipelined_ms * 1e-3) / 1e9,
        }
    }


def budget_sweep(args):
    """Attention launch time against the tree size n (1..64 nodes) at 8K, 32K
    and 128K context, Q4_0 and F16, with the 27B head layout (24 q / 4 kv
    heads, head_dim 256): random draft trees of depth <= 16, plus chains of
    the same size. The cache rotates over copies spanning >= 1.1 GB so that
    every launch streams it from HBM. Each point: the average of 200 launches
    after 50, the KV bandwidth, the MFMA rate and the fraction of the binding
    roofline (HBM below 312 FLOP per KV byte, MFMA above)."""
    import torch

    import synth
    import tree_verify_attention_ddtree_amd as tv
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    Hq, Hkv, D = 24, 4, 256
    sizes = [1, 2, 4, 8, 12, 16, 23, 32, 48, 64]
    rows = []
    for kv in ("q4_0", "f16"):
        for T in (8192, 32768, 131072):
            inp = synth.attn_inputs(Hq, Hkv, D, T, 64, 16, seed=900 + T, kv=kv)
            kc0 = torch.from_numpy(inp["k_cache"]).to(dev)
            vc0 = torch.from_numpy(inp["v_cache"]).to(dev)
            layer_bytes = 2 * kc0.numel() * kc0.element_size()
            ncp = max(1, int(np.ceil(1.1e9 / layer_bytes)))
            caches = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(ncp - 1)]
            kvt = tv.TV_KV_Q4_0 if kv == "q4_0" else tv.TV_KV_F16
            ts, hs = tv.cache_strides(kc0, kvt)
            rng = np.random.default_rng(T)
            for n in sizes:
                for shape in ("tree", "chain"):
                    if shape == "chain" and n not in (16, 23, 64):
                        continue
                    parent = synth.chain_tree(n) if shape == "chain" else synth.draft_tree(rng, n, 16)
                    q = torch.from_numpy(np.ascontiguousarray(inp["q"][:n])).to(dev)
                    kt = torch.from_numpy(np.ascontiguousarray(inp["k_tree"][:n])).to(dev)
                    vt = torch.from_numpy(np.ascontiguousarray(inp["v_tree"][:n])).to(dev)
                    out = torch.empty((n, Hq, D), dtype=torch.float32, device=dev)
                    desc, _par = tv.make_desc(parent, Hq, Hkv, D, kvt, T, 0, inp["scale"], ts, hs)
                    wsb = tv.tv_attn_workspace_bytes(desc)
                    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)

                    def launch(i):
                        kc, vc = caches[i % ncp]
                        tv.tree_verify_attn(desc, kc, vc, q, kt, vt, out, ws, wsb, stream)

                    for i in range(50):
                        launch(i)
                    torch.cuda.synchronize()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for i in range(200):
                        launch(i)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    us = e0.elapsed_time(e1) / 200 * 1e3
                    flops = 4.0 * Hq * n * T * D
                    kvb = layer_bytes
                    gbps = kvb / (us * 1e-6) / 1e9
                    tfl = flops / (us * 1e-6) / 1e12
                    mfma_bound = flops / kvb > MFMA_FP16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
                    frac = tfl / MFMA_FP16_PEAK_TFLOPS if mfma_bound else gbps / HBM_PEAK_GBPS
                    row = dict(kv=kv, n_ctx=T, n=n, tree=shape, us=us, kv_gbps=gbps, tflops=tfl,
                               bound="mfma" if mfma_bound else "hbm", frac=frac)
                    rows.append(row)
                    print(json.dumps(row), flush=True)
            del caches, kc0, vc0
            torch.cuda.empty_cache()
    print("| KV | ctx | n | tree | us | KV GB/s | TFLOP/s | bound | frac |")
    print("|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['kv']} | {r['n_ctx']} | {r['n']} | {r['tree']} | {r['us']:.1f} | {r['kv_gbps']:.0f} | "
              f"{r['tflops']:.0f} | {r['bound']} | {r['frac']:.3f} |")


def cpu_baseline(inp, logits, parent, tokens, n_rows):
    """The oracle (fp64, OpenMP) on a bounded sample of the same step: the
    first n_rows output rows of the attention, extrapolated to all rows, plus
    the full acceptance."""
    import oracle
    n = len(parent)
    Hq = inp["n_q_heads"]
    total = n * Hq
    k = min(n_rows, total)
    rows = list(range(k))
    t0 = time.perf_counter()
    oracle.attn(inp, rows=rows)
    t1 = time.perf_counter()
    oracle.accept(logits, parent, tokens)
    t2 = time.perf_counter()
    step_s = (t1 - t0) * total / k + (t2 - t1)
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or os.cpu_count()
    return {
        "value": 1.0 / step_s,
        "unit": "steps/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"attention rows 0..{k - 1} of {total} ({(t1 - t0):.1f} s, scaled by {total / k:.2f}) "
                  f"+ full acceptance ({(t2 - t1) * 1e3:.0f} ms)",
    }


if __name__ == "__main__":
    main()
