"""Seeded generators for the verify-step workloads.

Shapes follow the workloads the DFlash/DDTree pages describe for a 27B-class
target: 24 query heads over 4 KV heads with head_dim 256, a budget-22 draft
tree (23 nodes with the root, block size 16), a Q4_0 or F16 KV cache up to
128K rows and an optional 2048-row decode window.

Conventions (readings of the pages, stated once here):
  * Q4_0 storage is the ggml block: 18 bytes per 32 values, an fp16 scale
    followed by 16 code bytes. Each code is a 4-bit unsigned nibble. Because
    the two nibbles of every code byte are independent and uniform on 0..15,
    a uniformly random byte draws both at once, so the generator never has to
    know which nibble holds which element.
  * Caches are head-major: array [n_kv_heads, n_ctx, row_bytes].
  * Tree node 0 is the root; parent[0] == -1 and 0 <= parent[i] < i.

Random streams are spawned from one SeedSequence per workload in a fixed
order, so every array is reproducible on its own.
"""

from __future__ import annotations

import numpy as np

Q4_0_BLOCK = 32
Q4_0_BLOCK_BYTES = 18

STREAM_NAMES = ("k_cache", "v_cache", "q", "k_tree", "v_tree", "tree", "tokens", "logits")


def q4_0_row_bytes(head_dim: int) -> int:
    """Bytes of one Q4_0 row of `head_dim` values."""
    assert head_dim % Q4_0_BLOCK == 0
    return head_dim // Q4_0_BLOCK * Q4_0_BLOCK_BYTES


def streams(seed: int) -> dict:
    """Independent PCG64 generators, one per input, spawned in a fixed order."""
    children = np.random.SeedSequence(seed).spawn(len(STREAM_NAMES))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(STREAM_NAMES, children)}


def q4_0_cache(rng, n_heads: int, n_ctx: int, head_dim: int, scale_sigma: float = 0.05) -> np.ndarray:
    """Q4_0 cache bytes, uint8 [n_heads, n_ctx, row_bytes].

    Per block: scale = fp16(|N(0,1)| * scale_sigma) (round to nearest even, so
    a few scales land in the fp16 subnormal range), then 16 uniform bytes of
    codes.
    """
    nb = head_dim // Q4_0_BLOCK
    scales = (np.abs(rng.standard_normal((n_heads, n_ctx, nb))) * scale_sigma).astype(np.float16)
    out = np.empty((n_heads, n_ctx, nb, Q4_0_BLOCK_BYTES), np.uint8)
    out[..., 0:2] = scales.view(np.uint8).reshape(n_heads, n_ctx, nb, 2)
    out[..., 2:] = rng.integers(0, 256, size=(n_heads, n_ctx, nb, 16), dtype=np.uint8)
    return out.reshape(n_heads, n_ctx, nb * Q4_0_BLOCK_BYTES)


def f16_normal(rng, shape, sigma: float = 1.0) -> np.ndarray:
    """fp16(N(0, sigma^2)) with round to nearest even."""
    return (rng.standard_normal(shape) * sigma).astype(np.float16)


def f16_cache(rng, n_heads: int, n_ctx: int, head_dim: int, sigma: float = 0.2) -> np.ndarray:
    """An F16 cache drawn directly, fp16 [n_heads, n_ctx, head_dim].

    Its spread (0.2) is close to that of the Q4_0 caches above, whose values
    have standard deviation of about 0.05 * 0.8 * 4.6.
    """
    return f16_normal(rng, (n_heads, n_ctx, head_dim), sigma)


def draft_tree(rng, n: int, depth_cap: int, p_spine: float = 0.6) -> np.ndarray:
    """Random draft tree as a parent array, branching biased to the first child.

    A spine tip starts at the root. Each new node extends the spine with
    probability p_spine (while the tip is shallower than depth_cap); otherwise
    it hangs under a uniformly chosen earlier node that is shallower than
    depth_cap. Node numbering is topological (parent[i] < i).
    """
    parent = [-1]
    depth = [0]
    tip = 0
    for i in range(1, n):
        if rng.random() < p_spine and depth[tip] < depth_cap:
            p = tip
            tip = i
        else:
            cands = [j for j in range(i) if depth[j] < depth_cap]
            p = cands[int(rng.integers(len(cands)))]
        parent.append(p)
        depth.append(depth[p] + 1)
    return np.asarray(parent, np.int32)


def chain_tree(n: int) -> np.ndarray:
    """A chain: root then n-1 drafts, each the child of the previous one."""
    return np.arange(-1, n - 1, dtype=np.int32)


def sibling_distinct_tokens(rng, parent: np.ndarray, vocab: int) -> np.ndarray:
    """Draft tokens uniform on [0, vocab), redrawn until siblings differ."""
    n = len(parent)
    tok = np.empty(n, np.int32)
    tok[0] = int(rng.integers(vocab))
    used = {}
    for i in range(1, n):
        s = used.setdefault(int(parent[i]), set())
        while True:
            t = int(rng.integers(vocab))
            if t not in s:
                break
        s.add(t)
        tok[i] = t
    return tok


def planted_logits(rng, parent: np.ndarray, tokens: np.ndarray, vocab: int, p_first: float = 0.7):
    """Logits N(0,1) fp32 [n, vocab] with a planted accepted path.

    A root-to-leaf path is walked (first child with probability p_first, else
    a uniformly chosen later child) and a length L is drawn uniformly from
    0..len(path)-1. Along the first L edges the child's token gets logit 100
    at its parent's row, far above any N(0,1) draw; at the L-th node every
    child's token gets -100, so nothing below it can match. Returns
    (logits, L, planted_path[0..L]).
    """
    n = len(parent)
    logits = rng.standard_normal((n, vocab)).astype(np.float32)
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[int(parent[i])].append(i)
    path = [0]
    while children[path[-1]]:
        ch = children[path[-1]]
        if len(ch) == 1 or rng.random() < p_first:
            path.append(ch[0])
        else:
            path.append(ch[int(rng.integers(1, len(ch)))])
    L = int(rng.integers(0, len(path)))
    for k in range(L):
        logits[path[k], tokens[path[k + 1]]] = 100.0
    for c in children[path[L]]:
        logits[path[L], tokens[c]] = -100.0
    return logits, L, path[: L + 1]


# Workloads: shapes of the verify step the pages describe (27B-class target,
# budget 22, block 16, window 2048, Q4_0 KV up to 128K rows).
WORKLOADS = {
    "tiny": dict(n_q_heads=4, n_kv_heads=2, head_dim=64, n_ctx=256, n_nodes=8, depth_cap=4,
                 window=0, vocab=1024, seed=1),
    "27b": dict(n_q_heads=24, n_kv_heads=4, head_dim=256, n_ctx=8192, n_nodes=23, depth_cap=16,
                window=0, seed=2),
    "long": dict(n_q_heads=24, n_kv_heads=4, head_dim=256, n_ctx=131072, n_nodes=23, depth_cap=16,
                 window=0, seed=3),
    "window": dict(n_q_heads=24, n_kv_heads=4, head_dim=256, n_ctx=61440, n_nodes=23, depth_cap=16,
                   window=2048, seed=4),
    "full": dict(n_q_heads=24, n_kv_heads=4, head_dim=256, n_ctx=32768, n_nodes=23, depth_cap=16,
                 window=0, vocab=152000, n_layers=16, n_trees=64, seed=5),
}


def attn_inputs(n_q_heads: int, n_kv_heads: int, head_dim: int, n_ctx: int, n_nodes: int,
                depth_cap: int, seed: int, kv: str = "q4_0", parent=None, window: int = 0,
                **_unused) -> dict:
    """One layer's inputs for a verify step.

    Returns numpy arrays: k_cache, v_cache (Q4_0 bytes [H_kv, n_ctx, row] or
    fp16 [H_kv, n_ctx, D]), q fp16 [n, H_q, D], k_tree / v_tree fp16
    [n, H_kv, D], parent int32 [n]; plus the scalar fields.
    """
    s = streams(seed)
    if kv == "q4_0":
        kc = q4_0_cache(s["k_cache"], n_kv_heads, n_ctx, head_dim)
        vc = q4_0_cache(s["v_cache"], n_kv_heads, n_ctx, head_dim)
    elif kv == "f16":
        kc = f16_cache(s["k_cache"], n_kv_heads, n_ctx, head_dim)
        vc = f16_cache(s["v_cache"], n_kv_heads, n_ctx, head_dim)
    else:
        raise ValueError(kv)
    if parent is None:
        parent = draft_tree(s["tree"], n_nodes, depth_cap)
    parent = np.asarray(parent, np.int32)
    n = len(parent)
    return dict(
        kv=kv, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim, n_ctx=n_ctx,
        window=window, scale=1.0 / np.sqrt(head_dim), parent=parent,
        k_cache=kc, v_cache=vc,
        q=f16_normal(s["q"], (n, n_q_heads, head_dim)),
        k_tree=f16_normal(s["k_tree"], (n, n_kv_heads, head_dim)),
        v_tree=f16_normal(s["v_tree"], (n, n_kv_heads, head_dim)),
    )


def full_step_tree(tree: int) -> dict:
    """Tree `tree` (0..63) of the 16-layer verify step: the draft tree shared
    by every layer of that step, its sibling-distinct draft tokens and the
    planted logits of the acceptance (seed 5000 + tree)."""
    w = WORKLOADS["full"]
    s = streams(5000 + tree)
    parent = draft_tree(s["tree"], w["n_nodes"], w["depth_cap"])
    tokens = sibling_distinct_tokens(s["tokens"], parent, w["vocab"])
    logits, L, path = planted_logits(s["logits"], parent, tokens, w["vocab"])
    return dict(parent=parent, tokens=tokens, logits=logits, n_acc=L, path=path)


def full_step_cache(layer: int):
    """Layer `layer`'s committed Q4_0 caches (K, V) of the verify step
    (the cache streams of seed 5000 + 100 * layer)."""
    w = WORKLOADS["full"]
    s = streams(5000 + 100 * layer)
    kc = q4_0_cache(s["k_cache"], w["n_kv_heads"], w["n_ctx"], w["head_dim"])
    vc = q4_0_cache(s["v_cache"], w["n_kv_heads"], w["n_ctx"], w["head_dim"])
    return kc, vc


def full_step_qkv(layer: int, tree: int, n: int) -> dict:
    """Q, K_tree and V_tree of layer `layer` for tree `tree` (seed
    1000000 + 100 * layer + tree): fp16 N(0,1)."""
    w = WORKLOADS["full"]
    s = streams(1000000 + 100 * layer + tree)
    return dict(q=f16_normal(s["q"], (n, w["n_q_heads"], w["head_dim"])),
                k_tree=f16_normal(s["k_tree"], (n, w["n_kv_heads"], w["head_dim"])),
                v_tree=f16_normal(s["v_tree"], (n, w["n_kv_heads"], w["head_dim"])))


def full_step_layer(layer: int, tree: int, cache=None, tree_inputs=None) -> dict:
    """One layer's attention inputs of the verify step for tree `tree`, in
    the form attn_inputs returns (the caches may be passed in, since they do
    not depend on the tree)."""
    w = WORKLOADS["full"]
    t = tree_inputs if tree_inputs is not None else full_step_tree(tree)
    kc, vc = cache if cache is not None else full_step_cache(layer)
    n = len(t["parent"])
    return dict(kv="q4_0", n_q_heads=w["n_q_heads"], n_kv_heads=w["n_kv_heads"], head_dim=w["head_dim"],
                n_ctx=w["n_ctx"], window=0, scale=1.0 / np.sqrt(w["head_dim"]), parent=t["parent"],
                k_cache=kc, v_cache=vc, **full_step_qkv(layer, tree, n))
