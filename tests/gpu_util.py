"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
call libtv.so through its binding, and compare with the oracle."""

import numpy as np

TOL = 2e-3  # row-normalised relative error bound for attention outputs


def rownorm_err(got, ref):
    """max over rows (node, head) of max_d |got - ref| / max_d |ref|."""
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((np.abs(got - ref).max(axis=-1) / den).max())


def to_dev(inp, dev):
    import torch
    t = {}
    for k in ("k_cache", "v_cache", "q", "k_tree", "v_tree"):
        t[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
    return t


def gpu_attn(inp, dev="cuda", n_ctx=None, window=None, tensors=None, strides=None, repeat=1):
    """Run tree_verify_attn on the device; returns float32 [n, H_q, D]."""
    import torch

    import tree_verify_attention_ddtree_amd as tv
    t = tensors if tensors is not None else to_dev(inp, dev)
    kv = tv.TV_KV_Q4_0 if inp["k_cache"].dtype == np.uint8 else tv.TV_KV_F16
    ts, hs = strides if strides is not None else tv.cache_strides(t["k_cache"], kv)
    ctx = inp["k_cache"].shape[1] if n_ctx is None else n_ctx
    W = inp.get("window", 0) if window is None else window
    desc, _par = tv.make_desc(inp["parent"], inp["n_q_heads"], inp["n_kv_heads"], inp["head_dim"], kv, ctx, W,
                              inp["scale"], ts, hs, window_mode=inp.get("window_mode", 0))
    wsb = tv.tv_attn_workspace_bytes(desc)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    n = len(inp["parent"])
    outs = []
    for _ in range(repeat):
        out = torch.full((n, inp["n_q_heads"], inp["head_dim"]), float("nan"), dtype=torch.float32, device=dev)
        tv.tree_verify_attn(desc, t["k_cache"], t["v_cache"], t["q"], t["k_tree"], t["v_tree"], out, ws, wsb)
        outs.append(out)
    torch.cuda.synchronize()
    res = [o.cpu().numpy() for o in outs]
    return res[0] if repeat == 1 else res


def gpu_accept(logits, parent, tokens, dev="cuda"):
    import torch

    import tree_verify_attention_ddtree_amd as tv
    n, vocab = logits.shape
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(dev)
    am = torch.full((n,), -7, dtype=torch.int32, device=dev)
    res = torch.full((2 + 2 * n,), -7, dtype=torch.int32, device=dev)
    ws = torch.zeros(tv.tv_accept_workspace_bytes(n, vocab), dtype=torch.uint8, device=dev)
    tv.tree_accept(lg, parent, tokens, am, res, ws)
    torch.cuda.synchronize()
    return am.cpu().numpy(), res.cpu().numpy()
