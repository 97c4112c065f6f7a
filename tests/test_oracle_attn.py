"""Pins of the oracle's tree-verify attention.

Each test checks the oracle against something it does not compute itself:
torch's CPU scaled_dot_product_attention in float64 (a library routine) with
an explicit mask, causal attention over a flat sequence, single-token decode,
closed forms, and structural invariants of the tree mask. A dropped
ancestor, a missing self term, a wrong KV head, a window off by one or a
transposed operand each break at least one of them.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

TOL = 1e-12


def deq_cache(inp):
    c = inp["k_cache"]
    D = inp["head_dim"]
    if c.dtype == np.uint8:
        return oracle.q4_0_dequant(inp["k_cache"], D), oracle.q4_0_dequant(inp["v_cache"], D)
    return inp["k_cache"].astype(np.float64), inp["v_cache"].astype(np.float64)


def root_path(i, parent):
    p = [i]
    while parent[p[-1]] >= 0:
        p.append(int(parent[p[-1]]))
    return p[::-1]


def sdpa_reference(inp, n_ctx=None):
    """Library attention: every node over the window rows plus its ancestors."""
    parent = inp["parent"]
    n = len(parent)
    Hq, Hkv, D = inp["n_q_heads"], inp["n_kv_heads"], inp["head_dim"]
    G = Hq // Hkv
    K, V = deq_cache(inp)
    T = K.shape[1] if n_ctx is None else n_ctx
    W = inp.get("window", 0)
    s0 = max(0, T - W) if W > 0 else 0
    mask = np.zeros((n, (T - s0) + n), bool)
    mask[:, : T - s0] = True
    for i in range(n):
        for a in root_path(i, parent):
            mask[i, T - s0 + a] = True
    out = np.empty((n, Hq, D))
    for h in range(Hq):
        g = h // G
        keys = np.concatenate([K[g, s0:T], inp["k_tree"][:, g].astype(np.float64)])
        vals = np.concatenate([V[g, s0:T], inp["v_tree"][:, g].astype(np.float64)])
        q = torch.from_numpy(inp["q"][:, h].astype(np.float64))[None, None]
        o = F.scaled_dot_product_attention(q, torch.from_numpy(keys)[None, None], torch.from_numpy(vals)[None, None],
                                           attn_mask=torch.from_numpy(mask), scale=float(inp["scale"]))
        out[:, h] = o[0, 0].numpy()
    return out


def rownorm_err(a, b):
    den = np.maximum(np.abs(b).max(axis=-1), 1e-300)
    return (np.abs(a - b).max(axis=-1) / den).max()


def f16_copy(inp):
    """Same tensor stored as F16: fp16 round-to-nearest of the Q4_0 values."""
    K, V = deq_cache(inp)
    out = dict(inp)
    out["k_cache"] = K.astype(np.float16)
    out["v_cache"] = V.astype(np.float16)
    return out


@pytest.mark.parametrize("kv", ["q4_0", "f16copy"])
def test_matches_library_sdpa_tiny(kv):
    inp = synth.attn_inputs(**synth.WORKLOADS["tiny"])
    if kv == "f16copy":
        inp = f16_copy(inp)
    assert rownorm_err(oracle.attn(inp), sdpa_reference(inp)) < TOL


@pytest.mark.parametrize("W", [1, 17, 100, 255, 256, 1000])
def test_window_matches_library_sdpa(W):
    inp = synth.attn_inputs(**synth.WORKLOADS["tiny"])
    inp["window"] = W
    assert rownorm_err(oracle.attn(inp), sdpa_reference(inp)) < TOL


def test_gqa_and_deeper_tree_matches_library():
    inp = synth.attn_inputs(n_q_heads=12, n_kv_heads=2, head_dim=96, n_ctx=77, n_nodes=23, depth_cap=16, seed=9)
    assert rownorm_err(oracle.attn(inp), sdpa_reference(inp)) < TOL


def test_chain_equals_causal_attention():
    """A chain tree is ordinary causal attention over [cache; chain]."""
    w = dict(synth.WORKLOADS["tiny"])
    n = 16
    inp = synth.attn_inputs(**w, parent=synth.chain_tree(n))
    K, V = deq_cache(inp)
    Hq, Hkv, D = w["n_q_heads"], w["n_kv_heads"], w["head_dim"]
    G = Hq // Hkv
    T = K.shape[1]
    got = oracle.attn(inp)
    for h in range(Hq):
        g = h // G
        keys = np.concatenate([K[g], inp["k_tree"][:, g].astype(np.float64)])
        vals = np.concatenate([V[g], inp["v_tree"][:, g].astype(np.float64)])
        qs = np.zeros((T + n, D))
        qs[T:] = inp["q"][:, h].astype(np.float64)
        o = F.scaled_dot_product_attention(torch.from_numpy(qs)[None, None], torch.from_numpy(keys)[None, None],
                                           torch.from_numpy(vals)[None, None], is_causal=True,
                                           scale=float(inp["scale"]))[0, 0].numpy()
        assert rownorm_err(got[:, h], o[T:]) < TOL


def test_budget_zero_equals_single_token_decode():
    """A one-node tree is plain decode of one token over [cache; its own row]."""
    w = dict(synth.WORKLOADS["tiny"])
    inp = synth.attn_inputs(**w, parent=np.array([-1], np.int32))
    K, V = deq_cache(inp)
    got = oracle.attn(inp)
    G = w["n_q_heads"] // w["n_kv_heads"]
    for h in range(w["n_q_heads"]):
        g = h // G
        keys = np.concatenate([K[g], inp["k_tree"][0:1, g].astype(np.float64)])
        vals = np.concatenate([V[g], inp["v_tree"][0:1, g].astype(np.float64)])
        s = keys @ inp["q"][0, h].astype(np.float64) * inp["scale"]
        p = np.exp(s - s.max())
        ref = (p @ vals) / p.sum()
        assert rownorm_err(got[0, h][None], ref[None]) < TOL


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
def test_window_equals_truncated_cache(kv):
    w = dict(synth.WORKLOADS["tiny"])
    inp = synth.attn_inputs(**w, kv=kv)
    W = 48
    a = dict(inp, window=W)
    b = dict(inp, window=0, k_cache=inp["k_cache"][:, -W:], v_cache=inp["v_cache"][:, -W:])
    assert np.array_equal(oracle.attn(a), oracle.attn(b))
    # a window at least as long as the cache is no window
    for big in (256, 257, 10 ** 6):
        assert np.array_equal(oracle.attn(dict(inp, window=big)), oracle.attn(dict(inp, window=0)))


def test_empty_cache_is_tree_only():
    w = dict(synth.WORKLOADS["tiny"])
    inp = synth.attn_inputs(**w)
    e = dict(inp, k_cache=inp["k_cache"][:, :0], v_cache=inp["v_cache"][:, :0])
    assert rownorm_err(oracle.attn(e), sdpa_reference(e)) < TOL
    # the root with an empty cache attends only to itself: output = its V row
    out = oracle.attn(e)
    G = w["n_q_heads"] // w["n_kv_heads"]
    for h in range(w["n_q_heads"]):
        assert np.array_equal(out[0, h], inp["v_tree"][0, h // G].astype(np.float64))


def test_identical_keys_give_mean_of_values():
    """Closed form: equal scores make the softmax uniform over attended keys."""
    w = dict(synth.WORKLOADS["tiny"])
    inp = synth.attn_inputs(**w)
    D = w["head_dim"]
    # every K row (cache and tree) is the same vector of exact fp16 values
    kc = inp["k_cache"].copy()
    kc[:, :, :] = kc[0, 0, :]
    # scale 0.5 in every block, so every value (code - 8) / 2 is exact in fp16
    blocks = kc.reshape(kc.shape[0], kc.shape[1], -1, 18)
    blocks[..., 0] = 0x00
    blocks[..., 1] = 0x38
    krow = oracle.q4_0_dequant(kc[0, 0][None], D)[0]
    kt = np.broadcast_to(krow.astype(np.float16), inp["k_tree"].shape).copy()
    assert np.array_equal(kt[0, 0].astype(np.float64), krow)
    inp = dict(inp, k_cache=kc, k_tree=kt)
    out = oracle.attn(inp)
    _, V = deq_cache(inp)
    G = w["n_q_heads"] // w["n_kv_heads"]
    for i in range(len(inp["parent"])):
        anc = root_path(i, inp["parent"])
        for h in range(w["n_q_heads"]):
            g = h // G
            vals = np.concatenate([V[g], inp["v_tree"][anc, g].astype(np.float64)])
            assert rownorm_err(out[i, h][None], vals.mean(axis=0)[None]) < 1e-13


def test_dominant_key_selects_its_value():
    """Closed form: a key scoring 60 above all others takes all the weight."""
    w = dict(synth.WORKLOADS["tiny"])
    inp = synth.attn_inputs(**w, kv="f16")
    D = w["head_dim"]
    q = np.zeros_like(inp["q"])
    q[..., 0] = 1.0
    kc = inp["k_cache"].copy()
    kc[..., 0] = 0.0
    j = 101
    kc[:, j, 0] = 480.0  # score 480 / sqrt(64) = 60 above every other key
    kt = inp["k_tree"].copy()
    kt[..., 0] = 0.0
    inp = dict(inp, q=q, k_cache=kc, k_tree=kt)
    out = oracle.attn(inp)
    nk = 256 + 8
    bound = nk * np.exp(-60.0) * 4
    G = w["n_q_heads"] // w["n_kv_heads"]
    for h in range(w["n_q_heads"]):
        ref = inp["v_cache"][h // G, j].astype(np.float64)
        assert np.abs(out[:, h] - ref).max() <= bound * np.abs(inp["v_cache"]).max()


def test_relabelling_permutes_outputs_exactly():
    """Another topological numbering of the same tree permutes the outputs."""
    inp = synth.attn_inputs(n_q_heads=4, n_kv_heads=2, head_dim=64, n_ctx=40, n_nodes=10, depth_cap=5, seed=11,
                            parent=np.array([-1, 0, 0, 1, 1, 2, 3, 3, 5, 8], np.int32))
    # BFS order of the same tree is another topological numbering
    parent = inp["parent"]
    order = [0]
    k = 0
    while k < len(order):
        u = order[k]
        order += [c for c in range(len(parent)) if parent[c] == u]
        k += 1
    new_of = {old: new for new, old in enumerate(order)}
    perm = np.array(order)
    p2 = np.array([-1] + [new_of[int(parent[old])] for old in order[1:]], np.int32)
    inp2 = dict(inp, parent=p2, q=inp["q"][perm], k_tree=inp["k_tree"][perm], v_tree=inp["v_tree"][perm])
    assert np.array_equal(oracle.attn(inp2), oracle.attn(inp)[perm])


def test_nodes_outside_ancestry_do_not_matter():
    """Adding nodes off node i's root path leaves node i's output unchanged."""
    base = np.array([-1, 0, 1, 2], np.int32)
    grown = np.array([-1, 0, 1, 2, 0, 4, 1, 6], np.int32)
    inp = synth.attn_inputs(n_q_heads=4, n_kv_heads=2, head_dim=64, n_ctx=50, n_nodes=8, depth_cap=8, seed=12,
                            parent=grown)
    small = dict(inp, parent=base, q=inp["q"][:4], k_tree=inp["k_tree"][:4], v_tree=inp["v_tree"][:4])
    assert np.array_equal(oracle.attn(small), oracle.attn(inp)[:4])


def test_row_subset_matches_full():
    inp = synth.attn_inputs(**synth.WORKLOADS["tiny"])
    full = oracle.attn(inp)
    rows = [0, 5, 31]
    part = oracle.attn(inp, rows=rows)
    Hq = inp["n_q_heads"]
    for r in rows:
        assert np.array_equal(part[r // Hq, r % Hq], full[r // Hq, r % Hq])


def test_rejects_bad_trees():
    assert oracle.check_tree(np.array([-1, 0, 1], np.int32)) == 0
    assert oracle.check_tree(np.array([0, 0], np.int32)) != 0
    assert oracle.check_tree(np.array([-1, 1], np.int32)) != 0
    assert oracle.check_tree(np.array([-1, 0, 3, 1], np.int32)) != 0
    assert oracle.check_tree(np.array([-1, -1], np.int32)) != 0


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
def test_cache_row_order_does_not_matter(kv):
    """Attention is a sum over keys: the same cache rows (K with its V) in any
    order give the same output (up to summation order), and exchanging the V
    rows of two keys alone changes it (a K/V row mismatch would not)."""
    w = dict(n_q_heads=6, n_kv_heads=2, head_dim=64, n_ctx=300, n_nodes=9, depth_cap=4, seed=515, kv=kv)
    inp = synth.attn_inputs(**w)
    base = oracle.attn(inp)
    perm = np.random.default_rng(7).permutation(300)
    shuf = dict(inp, k_cache=np.ascontiguousarray(inp["k_cache"][:, perm]),
                v_cache=np.ascontiguousarray(inp["v_cache"][:, perm]))
    assert rownorm_err(oracle.attn(shuf), base) <= TOL
    swapped_v = inp["v_cache"].copy()
    swapped_v[:, [3, 200]] = swapped_v[:, [200, 3]]
    assert rownorm_err(oracle.attn(dict(inp, v_cache=swapped_v)), base) > 1e-6
