"""GPU tests of tree_verify_step: one verify step (every layer's attention
plus the acceptance) in one launch of the work-queue kernel, or as the same
separate launches where the plan has no work-queue kernel.

The step's outputs must equal, bit for bit, those of tree_verify_attn per
layer followed by tree_accept (the same split and merge arithmetic) where
the step splits the keys as tree_verify_attn does (one layer); with several
layers it takes fewer splits per layer, and every layer is then compared
with the separate calls within the attention bound and some against the
oracle. The acceptance must equal the oracle's. Repeated calls on one
workspace check that the queue counters are left zero.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, rownorm_err, to_dev

pytestmark = pytest.mark.gpu


def _desc(tv, inp, t):
    kv = tv.TV_KV_Q4_0 if inp["k_cache"].dtype == np.uint8 else tv.TV_KV_F16
    ts, hs = tv.cache_strides(t["k_cache"], kv)
    return tv.make_desc(inp["parent"], inp["n_q_heads"], inp["n_kv_heads"], inp["head_dim"], kv,
                        inp["k_cache"].shape[1], inp.get("window", 0), inp["scale"], ts, hs,
                        window_mode=inp.get("window_mode", 0))


def _outs(torch, inp, L):
    n = len(inp["parent"])
    return [torch.full((n, inp["n_q_heads"], inp["head_dim"]), float("nan"), dtype=torch.float32, device="cuda")
            for _ in range(L)]


def run_step(tv, torch, desc, tens, inp, logits, tokens, ws):
    n = len(inp["parent"])
    outs = _outs(torch, inp, len(tens))
    am = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    res = torch.full((2 + 2 * n,), -7, dtype=torch.int32, device="cuda")
    layers = [(t["k_cache"], t["v_cache"], t["q"], t["k_tree"], t["v_tree"], o) for t, o in zip(tens, outs)]
    tv.tree_verify_step(desc, layers, logits, tokens, am, res, ws)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs], am.cpu().numpy(), res.cpu().numpy()


def run_separate(tv, torch, desc, tens, inp, logits, tokens):
    n, vocab = logits.shape
    outs = _outs(torch, inp, len(tens))
    wsb = tv.tv_attn_workspace_bytes(desc)
    aws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    for t, o in zip(tens, outs):
        tv.tree_verify_attn(desc, t["k_cache"], t["v_cache"], t["q"], t["k_tree"], t["v_tree"], o, aws, wsb)
    am = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    res = torch.full((2 + 2 * n,), -7, dtype=torch.int32, device="cuda")
    accws = torch.zeros(tv.tv_accept_workspace_bytes(n, vocab), dtype=torch.uint8, device="cuda")
    tv.tree_accept(logits, inp["parent"], tokens, am, res, accws)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs], am.cpu().numpy(), res.cpu().numpy()


def header_clear(ws):
    """The queue header (first 2048 bytes) is zero except the status word."""
    h = ws[:2048].cpu().numpy().view(np.uint32)
    return int(h[2]) == 0 and not h.any()


def check_step(inps, vocab, seed, expect_launches=None, oracle_layers=()):
    import torch

    import tree_verify_attention_ddtree_amd as tv
    tens = [to_dev(inp, "cuda") for inp in inps]
    desc, _par = _desc(tv, inps[0], tens[0])
    plan = tv.tv_step_plan(desc, len(inps), vocab)
    if expect_launches is not None:
        assert plan["launches"] == expect_launches, plan
    s = synth.streams(seed)
    parent = inps[0]["parent"]
    tokens = synth.sibling_distinct_tokens(s["tokens"], parent, vocab)
    logits_np, L, _ = synth.planted_logits(s["logits"], parent, tokens, vocab)
    logits = torch.from_numpy(logits_np).cuda()
    ws = torch.zeros(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
    assert plan["workspace_bytes"] == tv.tv_step_workspace_bytes(desc, len(inps), vocab)
    ref = run_separate(tv, torch, desc, tens, inps[0], logits, tokens)
    ram, rres = oracle.accept(logits_np, parent, tokens)
    assert np.array_equal(ref[1], ram) and np.array_equal(ref[2], rres)
    assert int(rres[0]) == L
    same_splits = plan["splits"] == tv.tv_attn_plan(desc)["splits"]
    for rep in range(2):
        got = run_step(tv, torch, desc, tens, inps[0], logits, tokens, ws)
        for l, (g, r) in enumerate(zip(got[0], ref[0])):
            if same_splits:
                assert np.array_equal(g, r), ("layer", l, "call", rep, np.nanmax(np.abs(g - r)))
            else:
                assert rownorm_err(g.astype(np.float64), r.astype(np.float64)) <= TOL, ("layer", l, "call", rep)
        assert np.array_equal(got[1], ram) and np.array_equal(got[2], rres), rep
        assert header_clear(ws), rep
    for l in oracle_layers:
        want = oracle.attn(inps[l])
        assert rownorm_err(ref[0][l].astype(np.float64), want) <= TOL, l
        err = rownorm_err(got[0][l].astype(np.float64), want)
        assert err <= TOL, (l, err)
    return plan


def _same_tree(inps):
    """attn_inputs draws the tree from the seed; give every layer layer 0's
    tree (the step shares one tree) with that layer's own tensors."""
    p = inps[0]["parent"]
    n = len(p)
    for x in inps[1:]:
        assert len(x["parent"]) == n
        x["parent"] = p
    return inps


# (H_q, H_kv, D, n_ctx, n, window, kv, layers, vocab, single launch: True,
# False, or None where the plan decides; for one layer of head_dim 256 the
# launches the plan must make). The single-launch shapes cover
# every tile layout of the work-queue kernel: M = 6 n query rows per KV head
# in T = ceil(M / 16) tiles; T = 9 -> (2, 1), 4 -> (1, 0), 5 -> (1, 1),
# 6 -> (2, 0) (two idle slots), 8 -> (2, 0); 12 tiles in two row groups
# (a 2048-row window) -> (1, 2).
SHAPES = [
    (24, 4, 256, 4096, 23, 0, "q4_0", 3, 152000, True),
    (24, 4, 256, 2048 + 64 * 5, 10, 0, "q4_0", 2, 16385, True),      # last acceptance slice of one logit
    (24, 4, 256, 4096, 12, 0, "q4_0", 2, 2000, True),
    (24, 4, 256, 4096, 16, 0, "q4_0", 2, 4099, True),
    (24, 4, 256, 4096, 20, 0, "q4_0", 2, 1000, True),
    (24, 4, 256, 33000, 23, 0, "q4_0", 2, 5000, True),        # 40 tail rows left to the merge
    (24, 4, 256, 8192, 23, 2048, "q4_0", 2, 777, True),       # 2048-row window: two row groups
    (24, 4, 256, 8192, 32, 2048, "q4_0", 2, 777, True),       # the same with 32 nodes: (1, 2) per group
    (24, 4, 256, 4096 + 37, 23, 0, "q4_0", 2, 5000, None),    # ragged end: masked split kernel
    (24, 4, 256, 6000, 30, 0, "q4_0", 2, 1000, None),         # three own tiles per wave
    (24, 4, 256, 50, 23, 0, "q4_0", 2, 64, False),            # no whole chunk: merge only
    (8, 2, 128, 3000, 12, 0, "f16", 2, 3000, False),          # F16, head_dim 128
    (4, 2, 256, 1000, 8, 0, "q4_0", 2, 1024, False),          # one tile (all shared)
    (24, 4, 256, 4096, 23, 0, "q4_0", 1, 152000, 2),          # one layer: split, then merge + acceptance
    (24, 4, 256, 4096 + 37, 23, 0, "q4_0", 1, 32769, 2),      # one layer, masked split kernel; 3 slices a row
    (8, 2, 256, 3000, 12, 0, "f16", 1, 3000, 2),              # one layer, F16
    (8, 2, 128, 3000, 12, 0, "f16", 1, 3000, 3),              # one layer, head_dim 128: separate launches
    (24, 4, 256, 50, 23, 0, "q4_0", 1, 64, 2),                # one layer, no whole chunk: merge, acceptance
    (8, 2, 128, 40, 12, 0, "f16", 1, 3000, 2),                # the same at head_dim 128
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}-{s[3]}-n{s[4]}-w{s[5]}-{s[6]}" for s in SHAPES])
def test_step_equals_separate_calls(shape):
    Hq, Hkv, D, T, n, W, kv, L, vocab, single = shape
    w = dict(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_ctx=T, n_nodes=n, depth_cap=16, kv=kv, window=W)
    inps = _same_tree([synth.attn_inputs(**dict(w, seed=9100 + 7 * l + T)) for l in range(L)])
    for x in inps:
        x["window"] = W
    expect = single if isinstance(single, int) and not isinstance(single, bool) else (1 if single else None)
    plan = check_step(inps, vocab, 9200 + T, expect_launches=expect, oracle_layers=range(L))
    if single is False:
        assert plan["launches"] > 1 and plan["workgroups"] == 0


def test_full_step_16_layers_one_launch():
    """The 16-layer verify step at 32768 rows (trees 0 and 1 of its 64 on one
    workspace): one launch, every layer within the attention bound of the
    separate calls, the planted acceptance exact, and layer 15 of tree 1
    against the oracle on every row."""
    import torch

    import tree_verify_attention_ddtree_amd as tv
    caches = [synth.full_step_cache(l) for l in range(16)]
    ws = None
    for tree in (0, 1):
        t = synth.full_step_tree(tree)
        inps = [synth.full_step_layer(l, tree, cache=caches[l], tree_inputs=t) for l in range(16)]
        tens = [to_dev(inp, "cuda") for inp in inps]
        desc, _par = _desc(tv, inps[0], tens[0])
        V = t["logits"].shape[1]
        plan = tv.tv_step_plan(desc, 16, V)
        assert plan["launches"] == 1 and plan["workgroups"] == plan["items"], plan
        if ws is None:
            ws = torch.zeros(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
        logits = torch.from_numpy(t["logits"]).cuda()
        got = run_step(tv, torch, desc, tens, inps[0], logits, t["tokens"], ws)
        ref = run_separate(tv, torch, desc, tens, inps[0], logits, t["tokens"])
        assert plan["splits"] == 32  # half the single-layer count: items of 16 chunks
        for l in range(16):
            assert rownorm_err(got[0][l].astype(np.float64), ref[0][l].astype(np.float64)) <= TOL, (tree, l)
        ram, rres = oracle.accept(t["logits"], t["parent"], t["tokens"])
        assert np.array_equal(got[1], ram) and np.array_equal(got[2], rres)
        assert int(got[2][0]) == t["n_acc"]
        assert header_clear(ws)
        del tens
    err = rownorm_err(got[0][15].astype(np.float64), oracle.attn(inps[15]))
    assert err <= TOL, err


def _random_step_shapes(k, seed):
    """k seeded step shapes: layer counts 1..4, head layouts, tree sizes,
    contexts (whole chunks or ragged), windows, both cache types, vocabularies
    from 64 logits to two 16384-logit slices and a bit; every third shape is
    one the work-queue kernel takes, and every third one layer of head_dim
    256 (two launches)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < k:
        D = int(rng.choice([128, 256, 256]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.integers(1, 8))
        n = int(rng.integers(1, 41))
        T = int(rng.choice([int(rng.integers(1, 3000)), 64 * int(rng.integers(1, 48))]))
        W = int(rng.choice([0, 0, int(rng.integers(1, 2500))]))
        kv = str(rng.choice(["q4_0", "q4_0", "f16"]))
        L = int(rng.integers(1, 5))
        # (at least as many tokens as a node can have children: the draft
        # tokens of siblings are distinct)
        vocab = int(rng.choice([64, int(rng.integers(65, 5000)), int(rng.integers(16000, 40000))]))
        if len(out) % 3 == 0:
            # a shape for the work-queue kernel: several layers of head_dim
            # 256 over enough whole chunks of a Q4_0 cache, no window
            D, kv, W, L = 256, "q4_0", 0, int(rng.integers(2, 5))
            T = 64 * int(rng.integers(64, 160))
        elif len(out) % 3 == 1:
            # one layer of head_dim 256: the two-launch form
            D, L = 256, 1
        if L * G * Hkv * n * T * D > 2e9:
            continue
        out.append((G * Hkv, Hkv, D, T, n, W, kv, L, vocab, int(rng.integers(1 << 20))))
    return out


RANDOM_STEPS = _random_step_shapes(24, 20261204)


@pytest.mark.parametrize("shape", RANDOM_STEPS,
                         ids=[f"{s[0]}x{s[1]}x{s[2]}-T{s[3]}-n{s[4]}-W{s[5]}-{s[6]}-L{s[7]}-V{s[8]}" for s in RANDOM_STEPS])
def test_random_step_shapes(shape):
    """Seeded random steps: whatever launch form the plan takes (work queue,
    two launches, separate launches) equals the separate calls, the
    acceptance the oracle's, and every layer the oracle within the bound."""
    Hq, Hkv, D, T, n, W, kv, L, vocab, seed = shape
    w = dict(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_ctx=T, n_nodes=n, depth_cap=16, kv=kv, window=W)
    inps = _same_tree([synth.attn_inputs(**dict(w, seed=seed + 7 * l)) for l in range(L)])
    for x in inps:
        x["window"] = W
    check_step(inps, vocab, seed + 1, oracle_layers=range(L))
