"""Benchmark of one DDTree verify step on one MI355X.

A step is the whole hot path on one batch of synthetic input: one layer of
tree-verify attention for a budget-22 tree (23 nodes) over a 128K-row Q4_0
KV cache (24 query / 4 KV heads, head_dim 256, no window), then greedy
acceptance over 23 x 152000 fp32 logits, as one tree_verify_step call (two
launches for one layer: the split kernel, then the merge rows and the
acceptance slices side by side). Inputs are resident in HBM before
the timed region; the KV cache rotates over enough copies (>= 1 GiB) that
the 256 MB Infinity Cache cannot hold it between steps.

Prints one JSON line (progress goes to stderr). `value` is verify steps per
second. Extra fields give the effective KV bandwidth, the roofline of the
attention launch, the stream probes on the same caches, one record per
workload (tiny, 27B-shaped at 8K, 128K tree and chain, 128K with an F16
cache, the 2048-token window uniform and per position, the 16-layer step at
32K over its 64 seeded trees) and the CPU oracle's speed on bounded samples
of each.

The per-workload measurements run before the headline's warm-up and timed
steps, so that the headline is taken on a device at its steady clocks.
"""

from __future__ import annotations

import argparse
import gc
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="only the headline step (for profiler runs)")
    ap.add_argument("--cpu-rows", type=int, default=552, help="oracle output rows timed for the CPU baseline")
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
    """HBM bytes per attention launch (split and merge kernels) from the
    rocprofv3 FETCH_SIZE and WRITE_SIZE passes (copy-calibrated) stored under
    profiles/, or None when the kernels have changed since they were taken."""
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


# ---------------------------------------------------------------------------
# helpers


def timed(torch, stream, fn, k, lead=0, lead_base=0):
    """Average ms per call of fn(i), i = 0..k-1, with HIP events on `stream`.
    With `lead`, that many untimed calls fn(lead_base + i) are queued after
    the synchronisation and before the first event, so that the timed calls
    find the device already running (an idle device restarts at lower
    clocks: a bracket of 50 calls that starts idle reads several percent
    slow)."""
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for i in range(lead):
        fn(lead_base + i)
    e0.record(stream)
    for i in range(k):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / k


def timed_median(torch, stream, fn, k, parts=6):
    """Median over `parts` runs of k / parts calls each of the average ms per
    call: a stall outside the kernels (seen once in a while on a freshly
    allocated gigabyte, tens of ms in one run) moves one part, not the
    figure. Each run is led by as many untimed calls (on other rotation
    indices), so that it times the device in steady state: the per-kernel
    figures (the roofline's launch time among them) then agree with the
    profiler's kernel durations."""
    per = max(1, k // parts)
    return float(np.median([timed(torch, stream, lambda i, j=j: fn(j * per + i), per, lead=per,
                                  lead_base=k + j * per + 3) for j in range(parts)]))


def rotated_q4_0(torch, dev, n_kv, rows, row_bytes, seed):
    """A head-major Q4_0 cache [n_kv, rows, row_bytes] drawn on the device:
    block scales fp16(|N(0,1)| * 0.05), uniform code bytes (the distribution
    of the seeded caches of the tests)."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    nb = row_bytes // 18
    codes = torch.randint(0, 256, (n_kv, rows, nb, 16), dtype=torch.uint8, device=dev, generator=g)
    sc = (torch.randn((n_kv, rows, nb), device=dev, generator=g).abs() * 0.05).half()
    blocks = torch.cat([sc.view(torch.uint8).reshape(n_kv, rows, nb, 2), codes], dim=3)
    return blocks.reshape(n_kv, rows, row_bytes).contiguous()


def rotated_f16(torch, dev, n_kv, rows, D, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (torch.randn((n_kv, rows, D), device=dev, generator=g) * 0.2).half()


def attn_record(us, kv_bytes, flops):
    kv_gbps = kv_bytes / (us * 1e-6) / 1e9
    tflops = flops / (us * 1e-6) / 1e12
    mfma_bound = flops / kv_bytes > MFMA_FP16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    return {
        "us": us, "steps_per_s": 1e6 / us, "kv_gbps": kv_gbps, "kv_frac_hbm_peak": kv_gbps / HBM_PEAK_GBPS,
        "tflops": tflops, "bound": "mfma" if mfma_bound else "hbm",
        "frac": tflops / MFMA_FP16_PEAK_TFLOPS if mfma_bound else kv_gbps / HBM_PEAK_GBPS,
        "algorithmic_kv_bytes": kv_bytes, "algorithmic_flops": flops,
    }


def oracle_times(inp, rows=None, single_thread=False):
    """Seconds the oracle takes for the attention of `inp` (all rows or the
    given ones), on all host threads and optionally on one."""
    import oracle
    t0 = time.perf_counter()
    oracle.attn(inp, rows=rows)
    out = {"oracle_s": time.perf_counter() - t0, "oracle_threads": oracle.max_threads()}
    if single_thread:
        n = oracle.max_threads()
        oracle.set_threads(1)
        t0 = time.perf_counter()
        oracle.attn(inp, rows=rows)
        out["oracle_s_1thread"] = time.perf_counter() - t0
        oracle.set_threads(n)
    return out


# ---------------------------------------------------------------------------
# per-workload records


def layer_config(torch, tv, dev, stream, name, Hq, Hkv, D, T, W, kv, parent, window_mode=0, launches=300,
                 seed=0):
    """One attention layer, timed over >= 1.1 GB of KV rows: the cache is
    allocated large and every call reads it through a view that starts R rows
    (the rows a call reads) after the previous one, so consecutive calls read
    disjoint memory."""
    from synth import f16_normal, streams
    n = len(parent)
    kvt = tv.TV_KV_Q4_0 if kv == "q4_0" else tv.TV_KV_F16
    R = min(T, W) if W > 0 else T
    row_bytes = (D // 32 * 18) if kv == "q4_0" else 2 * D
    n_views = max(1, int(np.ceil(1.1e9 / (2 * Hkv * R * row_bytes))))
    rows_alloc = (n_views - 1) * R + T
    if kv == "q4_0":
        kc = rotated_q4_0(torch, dev, Hkv, rows_alloc, row_bytes, seed + 1)
        vc = rotated_q4_0(torch, dev, Hkv, rows_alloc, row_bytes, seed + 2)
    else:
        kc = rotated_f16(torch, dev, Hkv, rows_alloc, D, seed + 1)
        vc = rotated_f16(torch, dev, Hkv, rows_alloc, D, seed + 2)
    ts, hs = tv.cache_strides(kc, kvt)
    s = streams(seed)
    q = torch.from_numpy(f16_normal(s["q"], (n, Hq, D))).to(dev)
    kt = torch.from_numpy(f16_normal(s["k_tree"], (n, Hkv, D))).to(dev)
    vt = torch.from_numpy(f16_normal(s["v_tree"], (n, Hkv, D))).to(dev)
    out = torch.empty((n, Hq, D), dtype=torch.float32, device=dev)
    desc, _par = tv.make_desc(parent, Hq, Hkv, D, kvt, T, W, 1.0 / np.sqrt(D), ts, hs, window_mode=window_mode)
    plan = tv.tv_attn_plan(desc)
    wsb = plan["workspace_bytes"]
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)

    def launch(i):
        off = (i % n_views) * R
        tv.tree_verify_attn(desc, kc[:, off:], vc[:, off:], q, kt, vt, out, ws, wsb, stream)

    timed(torch, stream, launch, 50)
    ms = timed_median(torch, stream, launch, launches)
    rec = attn_record(ms * 1e3, 2 * Hkv * R * row_bytes, 4.0 * Hq * n * R * D)
    rec.update({"n_ctx": T, "window": W, "window_mode": window_mode, "kv": kv, "n_nodes": n,
                "heads": f"{Hq}/{Hkv}", "head_dim": D, "kv_views_rotated": n_views, "launches_timed": launches,
                "plan": {k: plan[k] for k in ("splits", "row_groups", "own_tiles", "shared_tiles", "kernel")}})
    del kc, vc
    torch.cuda.empty_cache()
    log(f"{name}: {rec['us']:.1f} us, {rec['kv_gbps']:.0f} GB/s KV, frac {rec['frac']:.3f}")
    return rec


def stream_probes(torch, tv, stream, caches, kv_bytes):
    """tv_stream_probe over the same rotated 128K caches the headline reads:
    a plain read and a read with Q4_0-style decoding of every byte."""
    out = {}
    chk = torch.empty(2048, dtype=torch.int32, device=caches[0][0].device)
    for name, kind in (("read", tv.TV_PROBE_READ), ("q4_0_decode", tv.TV_PROBE_Q4_0_DECODE)):
        def probe(i):
            kc, vc = caches[i % len(caches)]
            tv.tv_stream_probe(kc, kind, chk, stream)
            tv.tv_stream_probe(vc, kind, chk, stream)
        timed(torch, stream, probe, 20)
        ms = timed_median(torch, stream, probe, 200)
        gbps = kv_bytes / (ms * 1e-3) / 1e9
        out[name] = {"us": ms * 1e3, "gbps": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS}
    out["bytes_per_call"] = kv_bytes
    out["note"] = ("K and V caches of the 128K layer (rotated copies), two launches of 2048 workgroups x 256 "
                   "threads per call, each workgroup one contiguous range read with streaming loads; "
                   "q4_0_decode unpacks every code byte into fp16 (code - 8) * scale")
    log(f"stream probes: read {out['read']['gbps']:.0f} GB/s, q4_0 decode {out['q4_0_decode']['gbps']:.0f} GB/s")
    return out


def full_step(torch, tv, synth, dev, stream, passes):
    """The 16-layer verify step at 32K context over its 64 seeded trees: step
    t uses tree t % 64 for every layer (its queries and tree K/V differ per
    layer), then the acceptance over that tree's planted 23 x 152000 logits,
    then the KV commit of the accepted path into all 16 layers (rows past
    n_ctx, so every step reads the same context). Timed back to back
    (pipelined) and with each step's result copied to the host and the stream
    synchronised, as a decode loop must."""
    w = dict(synth.WORKLOADS["full"])
    L, T, ntr = w["n_layers"], w["n_ctx"], w["n_trees"]
    Hq, Hkv, D = w["n_q_heads"], w["n_kv_heads"], w["head_dim"]
    cap = T + 64
    trees = [synth.full_step_tree(t) for t in range(ntr)]
    layers = []
    for layer in range(L):
        kc_np, vc_np = synth.full_step_cache(layer)
        t = {}
        for name, arr in (("k_cache", kc_np), ("v_cache", vc_np)):
            c = torch.empty((Hkv, cap, arr.shape[2]), dtype=torch.uint8, device=dev)
            c[:, :T] = torch.from_numpy(arr).to(dev)
            t[name] = c
        t["qkv"] = []
        for tr in range(ntr):
            x = synth.full_step_qkv(layer, tr, len(trees[tr]["parent"]))
            t["qkv"].append({k: torch.from_numpy(v).to(dev) for k, v in x.items()})
        layers.append(t)
    log("full step: inputs on the device")
    ts, hs = tv.cache_strides(layers[0]["k_cache"], tv.TV_KV_Q4_0)
    descs = [tv.make_desc(tr["parent"], Hq, Hkv, D, tv.TV_KV_Q4_0, T, 0, 1.0 / np.sqrt(D), ts, hs) for tr in trees]
    wsb = max(tv.tv_attn_workspace_bytes(d) for d, _ in descs)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    outs = torch.empty((23, Hq, D), dtype=torch.float32, device=dev)
    logits = [torch.from_numpy(tr["logits"]).to(dev) for tr in trees]
    am = torch.empty(23, dtype=torch.int32, device=dev)
    res = torch.empty((ntr, 2 + 2 * 23), dtype=torch.int32, device=dev)
    aws = torch.zeros(tv.tv_accept_workspace_bytes(23, w["vocab"]), dtype=torch.uint8, device=dev)
    host = torch.empty(2 + 2 * 23, dtype=torch.int32, pin_memory=True)
    cdesc = tv.make_commit_desc(23, Hkv, D, tv.TV_KV_Q4_0, T, cap, ts, hs)
    k_caches, v_caches = [t["k_cache"] for t in layers], [t["v_cache"] for t in layers]
    k_trees = [[t["qkv"][tr]["k_tree"] for t in layers] for tr in range(ntr)]
    v_trees = [[t["qkv"][tr]["v_tree"] for t in layers] for tr in range(ntr)]

    # the one-launch form: every layer's output kept, one work-queue launch
    step_outs = [torch.empty((23, Hq, D), dtype=torch.float32, device=dev) for _ in range(L)]
    step_layers = [tv.step_layers([(t["k_cache"], t["v_cache"], t["qkv"][tr]["q"], t["qkv"][tr]["k_tree"],
                                    t["qkv"][tr]["v_tree"], o) for t, o in zip(layers, step_outs)])
                   for tr in range(ntr)]
    sws = torch.zeros(max(tv.tv_step_workspace_bytes(d, L, w["vocab"]) for d, _ in descs), dtype=torch.uint8,
                      device=dev)
    splan = tv.tv_step_plan(descs[0][0], L, w["vocab"])

    def one_step(i, single):
        tr = i % ntr
        d, _p = descs[tr]
        if single:
            tv.tree_verify_step(d, step_layers[tr], logits[tr], trees[tr]["tokens"], am, res[tr], sws, stream)
        else:
            for t in layers:
                x = t["qkv"][tr]
                tv.tree_verify_attn(d, t["k_cache"], t["v_cache"], x["q"], x["k_tree"], x["v_tree"], outs, ws, wsb,
                                    stream)
            tv.tree_accept(logits[tr], trees[tr]["parent"], trees[tr]["tokens"], am, res[tr], aws, stream)
        tv.tree_commit_kv_layers(cdesc, res[tr], k_trees[tr], v_trees[tr], k_caches, v_caches, stream)

    kv_step = L * 2 * Hkv * T * 144
    rec = {
        "workload": "16 layers x (24 q / 4 kv heads, head_dim 256, 32768 Q4_0 rows), 64 seeded budget-22 trees "
                    "(one per step, shared by all layers), acceptance over 23x152000 logits, KV commit of the "
                    "accepted path into the 16 layers (one launch)",
        "one_launch_plan": splan,
    }
    accepted_ok = True
    for single in (True, False):
        for i in range(8):
            one_step(i, single)
        torch.cuda.synchronize()
        steps = passes * ntr
        res.fill_(-1)
        pipelined_ms = timed(torch, stream, lambda i: one_step(i, single), steps)
        got = res.cpu().numpy()
        ok = all(int(got[tr][0]) == trees[tr]["n_acc"] for tr in range(ntr))
        t0 = time.perf_counter()
        for i in range(ntr):
            one_step(i, single)
            host.copy_(res[i % ntr], non_blocking=True)
            stream.synchronize()
            ok = ok and int(host[0]) == trees[i % ntr]["n_acc"]
        synced_ms = (time.perf_counter() - t0) * 1e3 / ntr
        accepted_ok = accepted_ok and ok
        form = {"steps_timed_pipelined": steps, "steps_per_s_pipelined": 1e3 / pipelined_ms,
                "ms_per_step_pipelined": pipelined_ms, "steps_per_s_with_host_sync": 1e3 / synced_ms,
                "ms_per_step_with_host_sync": synced_ms, "kv_gbps": kv_step / (pipelined_ms * 1e-3) / 1e9,
                "accepted_lengths_match_planted": bool(ok)}
        if single:
            # the step and the commit: two launches
            form["launches_per_step"] = splan["launches"] + 1
            rec.update(form)
            rec["attention_and_acceptance"] = "tree_verify_step (work-queue kernel, one launch)"
        else:
            form["launches_per_step"] = 2 * L + 2
            rec["separate_launches"] = form
        log(f"full step ({'one launch' if single else 'separate launches'}): {pipelined_ms:.3f} ms pipelined, "
            f"{synced_ms:.3f} ms with host sync")
    rec["accepted_lengths_match_planted"] = bool(accepted_ok)
    del layers, logits, step_outs, step_layers, sws
    torch.cuda.empty_cache()
    return rec, trees


# ---------------------------------------------------------------------------


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures the verify step on one GPU: a tree-verify layer of "
                                   "one GPU's share of a sharded step (KV heads or cache rows) is the same kernel "
                                   "at a smaller head count or context, run with --gpus 1"}))
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
    stream = torch.cuda.current_stream()
    w = dict(synth.WORKLOADS["long"])
    Hq, Hkv, D, T = w["n_q_heads"], w["n_kv_heads"], w["head_dim"], w["n_ctx"]
    vocab = synth.WORKLOADS["full"]["vocab"]

    inp = synth.attn_inputs(**w)
    parent = inp["parent"]
    n = len(parent)
    s = synth.streams(w["seed"])
    tokens = synth.sibling_distinct_tokens(s["tokens"], parent, vocab)
    logits, planted_L, _ = synth.planted_logits(s["logits"], parent, tokens, vocab)
    log("headline inputs drawn")

    kc0 = torch.from_numpy(inp["k_cache"]).to(dev)
    vc0 = torch.from_numpy(inp["v_cache"]).to(dev)
    kv_bytes_alloc = 2 * kc0.numel() * kc0.element_size()
    n_copies = max(1, int(np.ceil(1.1e9 / kv_bytes_alloc)))
    caches = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(n_copies - 1)]
    q = torch.from_numpy(inp["q"]).to(dev)
    kt = torch.from_numpy(inp["k_tree"]).to(dev)
    vt = torch.from_numpy(inp["v_tree"]).to(dev)
    out = torch.empty((n, Hq, D), dtype=torch.float32, device=dev)
    ts, hs = tv.cache_strides(kc0, tv.TV_KV_Q4_0)
    desc, _par = tv.make_desc(parent, Hq, Hkv, D, tv.TV_KV_Q4_0, T, 0, inp["scale"], ts, hs)
    wsb = tv.tv_attn_workspace_bytes(desc)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    lg = torch.from_numpy(logits).to(dev)
    am = torch.empty(n, dtype=torch.int32, device=dev)
    res = torch.empty(2 + 2 * n, dtype=torch.int32, device=dev)
    aws = torch.zeros(tv.tv_accept_workspace_bytes(n, vocab), dtype=torch.uint8, device=dev)

    chain = synth.chain_tree(16)
    cdesc, _cpar = tv.make_desc(chain, Hq, Hkv, D, tv.TV_KV_Q4_0, T, 0, inp["scale"], ts, hs)
    cws = torch.empty(max(tv.tv_attn_workspace_bytes(cdesc), 16), dtype=torch.uint8, device=dev)
    cq, ckt, cvt = q[:16].contiguous(), kt[:16].contiguous(), vt[:16].contiguous()
    cout = torch.empty((16, Hq, D), dtype=torch.float32, device=dev)

    def attn(i):
        kc, vc = caches[i % n_copies]
        tv.tree_verify_attn(desc, kc, vc, q, kt, vt, out, ws, wsb, stream)

    def accept():
        tv.tree_accept(lg, parent, tokens, am, res, aws, stream)

    def step_separate(i):
        attn(i)
        accept()

    # the step: tree_verify_step over the layer and the acceptance (for one
    # layer two launches: the split kernel, then the merge rows and the
    # acceptance slices side by side in one kernel). The same step as the
    # separate calls (tree_verify_attn, then tree_accept: three launches) is
    # timed beside it.
    sws = torch.zeros(tv.tv_step_workspace_bytes(desc, 1, vocab), dtype=torch.uint8, device=dev)
    step_arrs = [tv.step_layers([(kc, vc, q, kt, vt, out)]) for kc, vc in caches]

    def step_one(i):
        tv.tree_verify_step(desc, step_arrs[i % n_copies], lg, tokens, am, res, sws, stream)

    step = step_one

    R = T
    kv_bytes = 2 * Hkv * R * (D // 32 * 18)
    flops = 4.0 * Hq * n * R * D

    extra = {}
    trees = None
    if not args.no_configs:
        # per-workload records first (they also bring the device to its steady clocks)
        cfg = {}
        ptiny = synth.draft_tree(synth.streams(1)["tree"], 8, 4)
        cfg["tiny_q4_0"] = layer_config(torch, tv, dev, stream, "tiny q4_0", 4, 2, 64, 256, 0, "q4_0", ptiny, seed=11)
        cfg["tiny_f16"] = layer_config(torch, tv, dev, stream, "tiny f16", 4, 2, 64, 256, 0, "f16", ptiny, seed=12)
        p27 = synth.draft_tree(synth.streams(2)["tree"], 23, 16)
        cfg["27b_8k_q4_0"] = layer_config(torch, tv, dev, stream, "27b 8K q4_0", 24, 4, 256, 8192, 0, "q4_0", p27,
                                          seed=21)
        cfg["27b_8k_f16"] = layer_config(torch, tv, dev, stream, "27b 8K f16", 24, 4, 256, 8192, 0, "f16", p27,
                                         seed=22)
        p61 = synth.draft_tree(synth.streams(4)["tree"], 23, 16)
        cfg["window_61k_w2048_uniform"] = layer_config(torch, tv, dev, stream, "61K window 2048", 24, 4, 256, 61440,
                                                       2048, "q4_0", p61, window_mode=0, seed=41)
        cfg["window_61k_w2048_per_position"] = layer_config(torch, tv, dev, stream, "61K per-position window 2048",
                                                            24, 4, 256, 61440, 2048, "q4_0", p61, window_mode=1,
                                                            seed=42)
        # the headline layer with an F16 cache (3.6x the KV bytes of Q4_0)
        cfg["long_128k_f16"] = layer_config(torch, tv, dev, stream, "128K f16", Hq, Hkv, D, T, 0, "f16", parent,
                                            seed=31)
        timed(torch, stream, attn, 50)
        ms_tree = timed_median(torch, stream, attn, 500)
        cfg["long_128k_tree"] = attn_record(ms_tree * 1e3, kv_bytes, flops)
        cfg["long_128k_tree"].update({"n_ctx": T, "n_nodes": n, "kv": "q4_0", "kv_copies_rotated": n_copies})
        ms_chain = timed_median(torch, stream, lambda i: tv.tree_verify_attn(
            cdesc, caches[i % n_copies][0], caches[i % n_copies][1], cq, ckt, cvt, cout, cws, None, stream), 500)
        cfg["long_128k_chain16"] = attn_record(ms_chain * 1e3, kv_bytes, 4.0 * Hq * 16 * R * D)
        cfg["long_128k_chain16"].update({"n_ctx": T, "n_nodes": 16, "kv": "q4_0", "kv_copies_rotated": n_copies})
        log(f"128K tree: {ms_tree * 1e3:.1f} us, chain-16: {ms_chain * 1e3:.1f} us")
        extra["stream_probes"] = stream_probes(torch, tv, stream, caches, kv_bytes)
        fs, trees = full_step(torch, tv, synth, dev, stream, passes=2)
        cfg["full_step_32k_16_layers"] = fs
        extra["configs"] = cfg

    # ---- headline: W warm-up steps, then exactly K timed steps. Before
    # them, 200 steps that settle the device after the per-workload records
    # (which allocate and free gigabytes: a short bracket right after that ran
    # 10-20% slow).
    # No garbage collection from here to the end of the timed runs: a
    # collection pass is a host stall of milliseconds, which a short run
    # cannot hide. (The collection it replaces runs first, before the
    # warm-up: taken between the warm-up and a short timed run, its pause
    # left the device idle long enough that a 20-step run took 15% longer.)
    gc.collect()
    gc.disable()
    if not args.no_configs:
        for i in range(200):
            step(i)
    res.fill_(-1)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step = timed(torch, stream, step, args.steps)
    assert int(res[0].item()) == planted_L
    # the parts of a step on their own and the step as separate calls
    # (medians of six runs of 50, each led by 50 untimed calls)
    ms_attn = timed_median(torch, stream, attn, max(args.steps, 300))
    ms_accept = timed_median(torch, stream, lambda i: accept(), max(args.steps, 300))
    ms_med = timed_median(torch, stream, step, max(args.steps, 300))
    res.fill_(-1)
    timed(torch, stream, step_separate, 50)
    ms_sep = timed_median(torch, stream, step_separate, max(args.steps, 300))
    assert int(res[0].item()) == planted_L
    gc.enable()
    log(f"headline: {ms_step * 1e3:.1f} us per step ({ms_med * 1e3:.1f} us median), attention {ms_attn * 1e3:.1f} us, "
        f"separate calls {ms_sep * 1e3:.1f} us")

    kv_gbps = kv_bytes / (ms_attn * 1e-3) / 1e9
    tflops = flops / (ms_attn * 1e-3) / 1e12
    tflops_sep = flops / (ms_sep * 1e-3) / 1e12
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
                         f"ctx {T}, no window, Q4_0 KV, budget-22 tree of {n} nodes) + greedy acceptance "
                         f"over {n}x{vocab} fp32 logits"),
            "kv": "q4_0", "n_ctx": T, "window": 0, "n_nodes": n, "vocab": vocab, "kv_copies_rotated": n_copies,
        },
        "kv_gbps": kv_gbps,
        "kv_frac_hbm_peak": kv_gbps / HBM_PEAK_GBPS,
        "ms_per_step_median": ms_med,
        "step_plan": tv.tv_step_plan(desc, 1, vocab),
        "attn_us": ms_attn * 1e3,
        "accept_us": ms_accept * 1e3,
        "separate_calls": {
            "ms_per_step": ms_sep, "steps_per_s": 1e3 / ms_sep, "tflops": tflops_sep,
            "frac_mfma": tflops_sep / MFMA_FP16_PEAK_TFLOPS,
            "note": "tree_verify_attn then tree_accept: three launches (median of six runs of 50, each led by 50 untimed steps)",
        },
        "roofline": {
            "kernel": "tree_verify_attn launch: split_q4ws_kernel<2, 1> + merge_kernel<256>",
            "bound": "mfma",
            "achieved": tflops,
            "peak": MFMA_FP16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_FP16_PEAK_TFLOPS,
            "launch_us": ms_attn * 1e3,
            "traffic": measured_traffic(),
            "traffic_unit": "bytes per attention launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE x1, copy-calibrated)",
            "algorithmic_flops": flops,
            "algorithmic_kv_bytes": kv_bytes,
        },
    }
    line.update(extra)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, logits, parent, tokens, args.cpu_rows)
        if not args.no_configs:
            line["cpu_baseline"]["per_config"] = cpu_per_config(synth, trees)
    print(json.dumps(line), flush=True)


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
    log(f"cpu baseline: {1.0 / step_s:.3f} steps/s")
    return {
        "value": 1.0 / step_s,
        "unit": "steps/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"attention rows 0..{k - 1} of {total} ({(t1 - t0):.1f} s, scaled by {total / k:.2f}) "
                  f"+ full acceptance ({(t2 - t1) * 1e3:.0f} ms)",
    }


def cpu_per_config(synth, trees):
    """The oracle per workload (seeded inputs of each): every row for tiny,
    27B 8K and the 2048-token windows, also on one thread for tiny and 27B
    8K; the 16-layer step from layer 0 of tree 0 (every row, scaled by 16
    layers) plus the acceptance of all 64 trees (averaged)."""
    import oracle
    out = {}
    for name, wl, kv, single in (("tiny_q4_0", "tiny", "q4_0", True), ("tiny_f16", "tiny", "f16", True),
                                 ("27b_8k_q4_0", "27b", "q4_0", True), ("27b_8k_f16", "27b", "f16", True),
                                 ("window_61k_w2048_uniform", "window", "q4_0", False)):
        inp = synth.attn_inputs(**synth.WORKLOADS[wl], kv=kv)
        out[name] = oracle_times(inp, single_thread=single)
    inp = dict(synth.attn_inputs(**synth.WORKLOADS["window"]), window_mode=1)
    out["window_61k_w2048_per_position"] = oracle_times(inp)
    layer = synth.full_step_layer(0, 0, tree_inputs=trees[0])
    t = oracle_times(layer)
    t0 = time.perf_counter()
    for x in trees:
        oracle.accept(x["logits"], x["parent"], x["tokens"])
    acc_s = (time.perf_counter() - t0) / len(trees)
    out["full_step_32k_16_layers"] = {"oracle_s_per_step": 16 * t["oracle_s"] + acc_s,
                                      "oracle_threads": t["oracle_threads"],
                                      "sample": "attention of layer 0 for tree 0 (every row) x 16 layers, plus the "
                                                f"acceptance averaged over {len(trees)} trees ({acc_s * 1e3:.0f} ms)"}
    log("cpu per-config oracle timings done")
    return out


def budget_sweep(args):
    """Attention launch time against the tree size n (1..64 nodes) at 8K, 32K
    and 128K context, Q4_0 and F16, with the 27B head layout (24 q / 4 kv
    heads, head_dim 256): random draft trees of depth <= 16, plus chains of
    the same size. The cache rotates over copies spanning >= 1.1 GB so that
    every launch streams it from HBM. Each point: the median of six runs of
    40 launches (each led by 40 untimed ones) after 50, the KV bandwidth, the
    MFMA rate and the fraction of the binding roofline (HBM below 312 FLOP
    per KV byte, MFMA above)."""
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

                    timed(torch, stream, launch, 50)
                    us = timed_median(torch, stream, launch, 240) * 1e3
                    rec = attn_record(us, layer_bytes, 4.0 * Hq * n * T * D)
                    row = dict(kv=kv, n_ctx=T, n=n, tree=shape, us=us, kv_gbps=rec["kv_gbps"], tflops=rec["tflops"],
                               bound=rec["bound"], frac=rec["frac"])
                    rows.append(row)
                    print(json.dumps(row), flush=True)
            del caches, kc0, vc0
            torch.cuda.empty_cache()
    print("| KV | ctx | n | tree | us | KV GB/s | TFLOP/s | bound | frac |")
    print("|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['kv']} | {r['n_ctx']} | {r['n']} | {r['tree']} | {r['us']:.1f} | {r['kv_gbps']:.0f} | "
              f"{r['tflops']:.0f} | {r['bound']} | {r['frac']:.3f} |")


if __name__ == "__main__":
    main()
