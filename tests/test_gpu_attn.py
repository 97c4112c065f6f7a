"""GPU parity of tree_verify_attn against the CPU oracle.

Bar: row-normalised relative error <= 2e-3 (fp16 products, fp32
accumulation). Small workloads are compared element by element on every
row; the 128K and 32K workloads on sampled rows the oracle computes one by
one. Edge cases cover empty and ragged caches, windows, every tile layout of
the split kernel, strided caches, extreme Q4_0 scales and peaky scores.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, gpu_attn, rownorm_err

pytestmark = pytest.mark.gpu


def deq_copy(inp):
    """The same tensor stored as F16 (fp16 rounding of the Q4_0 values)."""
    D = inp["head_dim"]
    out = dict(inp)
    out["k_cache"] = oracle.q4_0_dequant(inp["k_cache"], D).astype(np.float16)
    out["v_cache"] = oracle.q4_0_dequant(inp["v_cache"], D).astype(np.float16)
    return out


def sample_rows(n, Hq, k, seed):
    rng = np.random.default_rng(seed)
    rows = {0, n * Hq - 1, (n - 1) * Hq, Hq - 1}
    while len(rows) < k:
        rows.add(int(rng.integers(n * Hq)))
    return sorted(rows)


def check_rows(got, ref, rows, Hq):
    g = np.stack([got[r // Hq, r % Hq] for r in rows]).astype(np.float64)
    f = np.stack([ref[r // Hq, r % Hq] for r in rows])
    return rownorm_err(g, f)


@pytest.mark.parametrize("kv", ["q4_0", "f16copy"])
def test_tiny(kv):
    inp = synth.attn_inputs(**synth.WORKLOADS["tiny"])
    if kv == "f16copy":
        inp = deq_copy(inp)
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


@pytest.mark.parametrize("kv", ["q4_0", "f16copy"])
def test_27b_shape_8k(kv):
    inp = synth.attn_inputs(**synth.WORKLOADS["27b"])
    if kv == "f16copy":
        inp = deq_copy(inp)
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


def test_27b_shape_f16_direct():
    inp = synth.attn_inputs(**synth.WORKLOADS["27b"], kv="f16")
    rows = sample_rows(23, 24, 48, 5)
    err = check_rows(gpu_attn(inp), oracle.attn(inp, rows=rows), rows, 24)
    assert err <= TOL, err


@pytest.mark.parametrize("tree", ["budget22", "chain16"])
def test_long_128k_sampled(tree):
    w = dict(synth.WORKLOADS["long"])
    parent = synth.chain_tree(16) if tree == "chain16" else None
    inp = synth.attn_inputs(**w, parent=parent)
    n = len(inp["parent"])
    rows = sample_rows(n, 24, 16, 3)
    err = check_rows(gpu_attn(inp), oracle.attn(inp, rows=rows), rows, 24)
    assert err <= TOL, err


@pytest.mark.parametrize("tree", ["budget22", "chain16"])
def test_long_128k_all_rows(tree):
    """The headline layer (131072 Q4_0 rows, 24 q / 4 kv heads, head_dim
    256) on every output row: 552 for the budget-22 tree, 384 for the
    chain of 16."""
    w = dict(synth.WORKLOADS["long"])
    parent = synth.chain_tree(16) if tree == "chain16" else None
    inp = synth.attn_inputs(**w, parent=parent)
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


@pytest.mark.parametrize("tree", ["budget22", "chain16"])
def test_long_128k_f16_all_rows(tree):
    """The same layer with an F16 cache (the warp-specialised F16 kernel at
    64 splits: two own tiles and one shared per wave for the budget-22 tree,
    two own for the chain), on every output row."""
    w = dict(synth.WORKLOADS["long"])
    parent = synth.chain_tree(16) if tree == "chain16" else None
    inp = synth.attn_inputs(**w, parent=parent, kv="f16")
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


@pytest.mark.parametrize("layer,tree", [(0, 0), (0, 1), (15, 0), (15, 1)])
def test_full_step_layer_tree_all_rows(layer, tree):
    """Layers 0 and 15 of the 16-layer verify step at 32768 rows, for trees 0
    and 1 of its 64 (one draft tree per step, shared by every layer), on every
    output row."""
    t = synth.full_step_tree(tree)
    inp = synth.full_step_layer(layer, tree, tree_inputs=t)
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, (layer, tree, err)


def test_window_61k():
    w = dict(synth.WORKLOADS["window"])
    inp = synth.attn_inputs(**w)
    got = gpu_attn(inp)
    err = rownorm_err(got.astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err
    # the same as full attention over the last 2048 rows
    trunc = dict(inp, window=0, k_cache=inp["k_cache"][:, -2048:], v_cache=inp["v_cache"][:, -2048:])
    assert rownorm_err(gpu_attn(trunc).astype(np.float64), got.astype(np.float64)) <= TOL


def test_full_step_layers_sampled():
    """Two layers (first and last) of the 16-layer, 32K verify step."""
    w = dict(synth.WORKLOADS["full"])
    for layer in (0, 15):
        inp = synth.attn_inputs(**dict(w, seed=5000 + 100 * layer))
        rows = sample_rows(23, 24, 12, layer)
        err = check_rows(gpu_attn(inp), oracle.attn(inp, rows=rows), rows, 24)
        assert err <= TOL, (layer, err)


# Head layouts and tree sizes that hit every tile layout of the split kernel:
# M = (H_q / H_kv) * n query rows per KV head -> T = ceil(M / 16) tiles.
LAYOUTS = [
    (2, 1, 1, 64),     # M=2,   T=1
    (2, 1, 16, 64),    # M=32,  T=2
    (6, 1, 8, 128),    # M=48,  T=3
    (4, 1, 16, 64),    # M=64,  T=4
    (6, 2, 13, 256),   # M=39 per KV head, T=3, two KV heads
    (5, 1, 16, 128),   # M=80,  T=5
    (6, 1, 16, 256),   # M=96,  T=6 (chain-16 shape)
    (7, 1, 16, 64),    # M=112, T=7
    (8, 1, 16, 128),   # M=128, T=8
    (6, 1, 23, 256),   # M=138, T=9 (budget-22 shape)
    (10, 1, 16, 64),   # M=160, T=10 -> two row groups
    (11, 1, 16, 128),  # M=176, T=11
    (12, 1, 16, 256),  # M=192, T=12
    (13, 1, 16, 64),   # M=208, T=13 -> three row groups
    (6, 1, 64, 256),   # M=384, T=24, 64 nodes
    (32, 4, 40, 128),  # G=8, 40 nodes
]


@pytest.mark.parametrize("Hq,Hkv,n,D", LAYOUTS)
@pytest.mark.parametrize("kv", ["q4_0", "f16"])
def test_tile_layouts(Hq, Hkv, n, D, kv):
    inp = synth.attn_inputs(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_ctx=700, n_nodes=n,
                            depth_cap=16, seed=1000 + Hq * 7 + n, kv=kv)
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
@pytest.mark.parametrize("n,layout", [(8, {"q4_0": (1, 0), "f16": (1, 0)}), (20, {"q4_0": (2, 0), "f16": (2, 0)}),
                                      (30, {"q4_0": (3, 0), "f16": (3, 0)}), (23, {"q4_0": (2, 1), "f16": (2, 1)}),
                                      (10, {"q4_0": (1, 0), "f16": (1, 0)}), (11, {"q4_0": (1, 1), "f16": (1, 1)}),
                                      (16, {"q4_0": (2, 0), "f16": (2, 0)}), (26, {"q4_0": (1, 1), "f16": (1, 1)}),
                                      (2, {"q4_0": (0, 1), "f16": (1, 0)})])
def test_tile_layouts_27b_heads(n, layout, kv):
    """The 27B head layout (24 q / 4 kv heads) over 256 whole chunks per KV
    head: 8, 20, 30, 23, 10, 11, 16 and 2 nodes make 3, 8, 12, 9, 4, 5, 6 and
    1 query tiles in one row group; 26 nodes make 10 tiles, cut into two row
    groups of five (a group holds at most three tile slots per wave). Small
    layouts the warp-specialised kernels lack run on one they have with idle
    tile slots (Q4_0: three and six tiles; F16: up to eight). The plan the library
    reports for this device is asserted first, so each case is known to run
    the tile layout and split kernel it is named for (unmasked; every layout
    of the warp-specialised Q4_0 and F16 kernels is among them)."""
    import tree_verify_attention_ddtree_amd as tv
    inp = synth.attn_inputs(n_q_heads=24, n_kv_heads=4, head_dim=256, n_ctx=16384, n_nodes=n, depth_cap=16,
                            seed=3000 + n, kv=kv)
    kvt = tv.TV_KV_Q4_0 if kv == "q4_0" else tv.TV_KV_F16
    row = inp["k_cache"].shape[2] * inp["k_cache"].itemsize
    desc, _par = tv.make_desc(inp["parent"], 24, 4, 256, kvt, 16384, 0, inp["scale"], row, row * 16384)
    plan = tv.tv_attn_plan(desc)
    assert (plan["own_tiles"], plan["shared_tiles"]) == layout[kv], plan
    assert plan["row_groups"] == (2 if n == 26 else 1) and plan["masked"] == 0, plan
    own, sh = layout[kv]
    want = {"f16": tv.TV_SPLIT_F16_WS if own in (1, 2) and sh <= 1 else tv.TV_SPLIT_F16,
            "q4_0": tv.TV_SPLIT_Q4_0_WS if own in (1, 2) else tv.TV_SPLIT_Q4_0}
    assert plan["kernel"] == want[kv], plan
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


@pytest.mark.parametrize("kv,n,layout", [("q4_0", 8, (0, 3)), ("f16", 16, (1, 2)), ("q4_0", 16, (1, 2))])
def test_masked_layouts_one_wave_kernels(kv, n, layout):
    """A ragged end (16384 + 31 rows: short splits, so the masked kernels):
    the layouts the warp-specialised kernels would otherwise take over (three
    shared Q4_0 tiles; one own and two shared F16 tiles) on the one-wave
    masked kernels, against the oracle."""
    import tree_verify_attention_ddtree_amd as tv
    T = 16384 + 31
    inp = synth.attn_inputs(n_q_heads=24, n_kv_heads=4, head_dim=256, n_ctx=T, n_nodes=n, depth_cap=16,
                            seed=3100 + n, kv=kv)
    kvt = tv.TV_KV_Q4_0 if kv == "q4_0" else tv.TV_KV_F16
    row = inp["k_cache"].shape[2] * inp["k_cache"].itemsize
    desc, _par = tv.make_desc(inp["parent"], 24, 4, 256, kvt, T, 0, inp["scale"], row, row * T)
    plan = tv.tv_attn_plan(desc)
    assert (plan["own_tiles"], plan["shared_tiles"], plan["masked"]) == layout + (1,), plan
    assert plan["kernel"] == (tv.TV_SPLIT_Q4_0 if kv == "q4_0" else tv.TV_SPLIT_F16), plan
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
@pytest.mark.parametrize("n_ctx", [0, 5, 63])
def test_no_workspace_without_splits(kv, n_ctx):
    """Fewer than 64 cache rows: no split runs, the workspace is 0 bytes and
    is passed as NULL (and so are the caches when they are empty)."""
    import torch

    import tree_verify_attention_ddtree_amd as tv
    w = dict(synth.WORKLOADS["27b"], n_ctx=max(n_ctx, 1))
    inp = synth.attn_inputs(**w, kv=kv)
    inp["k_cache"] = inp["k_cache"][:, :n_ctx]
    inp["v_cache"] = inp["v_cache"][:, :n_ctx]
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).cuda() for k in ("q", "k_tree", "v_tree")}
    kvt = tv.TV_KV_Q4_0 if kv == "q4_0" else tv.TV_KV_F16
    row = inp["k_cache"].shape[2] * inp["k_cache"].itemsize
    desc, _par = tv.make_desc(inp["parent"], 24, 4, 256, kvt, n_ctx, 0, inp["scale"], row, row * max(n_ctx, 1))
    assert tv.tv_attn_workspace_bytes(desc) == 0
    kc = vc = None
    if n_ctx > 0:
        kc = torch.from_numpy(np.ascontiguousarray(inp["k_cache"])).cuda()
        vc = torch.from_numpy(np.ascontiguousarray(inp["v_cache"])).cuda()
    out = torch.full((23, 24, 256), float("nan"), dtype=torch.float32, device="cuda")
    tv.tree_verify_attn(desc, kc, vc, t["q"], t["k_tree"], t["v_tree"], out, None, 0)
    torch.cuda.synchronize()
    err = rownorm_err(out.cpu().numpy().astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


def test_non_finite_scales_stay_in_their_kv_head():
    """Q4_0 blocks with +inf, -inf and NaN scales in KV head 1 only (a commit
    of a row holding +-inf writes such scales): the rows of that head's
    query heads are unspecified, every other row matches the oracle."""
    inp = synth.attn_inputs(**dict(synth.WORKLOADS["27b"], n_ctx=1000))
    for k, bits in (("k_cache", (0x7C00, 0xFE00)), ("v_cache", (0xFC00, 0x7C00))):
        c = inp[k].copy()
        blocks = c.reshape(c.shape[0], c.shape[1], -1, 18)
        for j, b in enumerate(bits):
            blocks[1, 100 + 300 * j, 2, 0:2] = np.array([b], np.uint16).view(np.uint8)
        inp[k] = c
    got = gpu_attn(inp).astype(np.float64)
    ref = oracle.attn(inp)
    keep = [h for h in range(24) if h // 6 != 1]
    assert np.isfinite(ref[:, keep]).all() and np.isfinite(got[:, keep]).all()
    err = rownorm_err(got[:, keep], ref[:, keep])
    assert err <= TOL, err


@pytest.mark.parametrize("Hq,Hkv,n,D", [(6, 1, 8, 256), (6, 1, 7, 64), (2, 1, 21, 128), (8, 1, 16, 256)])
def test_tile_layouts_whole_chunks(Hq, Hkv, n, D):
    """Q4_0 layouts on a cache of whole 64-row chunks (the unmasked split
    kernels; the 700-row cases above take the masked ones): three shared
    tiles (M = 48, 42, 42) and eight own tiles (M = 128)."""
    inp = synth.attn_inputs(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_ctx=4096, n_nodes=n,
                            depth_cap=16, seed=2000 + Hq * 7 + n)
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


@pytest.mark.parametrize("n_ctx", [0, 1, 5, 63, 64, 65, 127, 255, 1000, 4097])
def test_ragged_and_empty_caches(n_ctx):
    w = dict(synth.WORKLOADS["27b"], n_ctx=max(n_ctx, 1))
    inp = synth.attn_inputs(**w)
    inp["k_cache"] = inp["k_cache"][:, :n_ctx]
    inp["v_cache"] = inp["v_cache"][:, :n_ctx]
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


@pytest.mark.parametrize("W", [1, 63, 64, 100, 2047, 2048, 5000, 10 ** 9])
def test_windows(W):
    w = dict(synth.WORKLOADS["27b"], n_ctx=4500)
    inp = synth.attn_inputs(**w)
    inp["window"] = W
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


def test_budget_zero_decode():
    w = dict(synth.WORKLOADS["27b"])
    inp = synth.attn_inputs(**w, parent=np.array([-1], np.int32))
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


@pytest.mark.parametrize("kv,n_ctx", [("q4_0", 1500), ("f16", 1500), ("q4_0", 1536), ("f16", 1536)])
def test_token_major_strided_cache(kv, n_ctx):
    """Cache laid out [token][head][row] (ggml-like) instead of head-major:
    a ragged end (the masked one-wave kernels) and whole chunks (the
    warp-specialised kernels)."""
    import torch

    import tree_verify_attention_ddtree_amd as tv
    inp = synth.attn_inputs(**dict(synth.WORKLOADS["27b"], n_ctx=n_ctx), kv=kv)
    t = {}
    for k in ("k_cache", "v_cache"):
        tm = np.ascontiguousarray(inp[k].transpose(1, 0, 2))  # [T][H][row]
        t[k] = torch.from_numpy(tm).cuda()
    for k in ("q", "k_tree", "v_tree"):
        t[k] = torch.from_numpy(inp[k]).cuda()
    row = inp["k_cache"].shape[2] * inp["k_cache"].itemsize
    kvt = tv.TV_KV_Q4_0 if kv == "q4_0" else tv.TV_KV_F16
    desc, _par = tv.make_desc(inp["parent"], 24, 4, 256, kvt, n_ctx, 0, inp["scale"], row * 4, row)
    plan = tv.tv_attn_plan(desc)
    ws_kind = tv.TV_SPLIT_Q4_0_WS if kv == "q4_0" else tv.TV_SPLIT_F16_WS
    assert (plan["kernel"] == ws_kind) == (n_ctx % 64 == 0), plan
    got = gpu_attn(inp, tensors=t, strides=(row * inp["n_kv_heads"], row))
    err = rownorm_err(got.astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


def test_extreme_q4_0_scales():
    """Subnormal, zero and large fp16 scales decode exactly (no flushing)."""
    inp = synth.attn_inputs(**dict(synth.WORKLOADS["27b"], n_ctx=900))
    rng = np.random.default_rng(77)
    for k in ("k_cache", "v_cache"):
        c = inp[k].copy()
        blocks = c.reshape(c.shape[0], c.shape[1], -1, 18)
        sel = rng.random(blocks.shape[:3])
        sc = blocks[..., 0:2].copy().view(np.uint16)[..., 0]
        sc[sel < 0.2] = 0x0001          # smallest subnormal
        sc[(sel >= 0.2) & (sel < 0.3)] = 0x03FF  # largest subnormal
        sc[(sel >= 0.3) & (sel < 0.35)] = 0x0000
        sc[(sel >= 0.35) & (sel < 0.4)] = 0x8000
        blocks[..., 0:2] = sc[..., None].view(np.uint8).reshape(sc.shape + (2,))
        inp[k] = c
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


def test_peaky_scores_force_rescaling():
    """Large, growing scores move the running max by far more than the
    lazy-rescale threshold many times within a split."""
    inp = synth.attn_inputs(**dict(synth.WORKLOADS["27b"], n_ctx=6000), kv="f16")
    q = inp["q"].astype(np.float32) * 4
    inp["q"] = q.astype(np.float16)
    kc = inp["k_cache"].astype(np.float32)
    ramp = np.linspace(0.2, 6.0, kc.shape[1], dtype=np.float32)[None, :, None]
    inp["k_cache"] = (kc * ramp).astype(np.float16)
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


@pytest.mark.parametrize("n_nodes", [2, 4, 23])
def test_peaky_scores_force_rescaling_q4_0(n_nodes):
    """Q4_0 keys whose block scales rise 30-fold over every 256 rows (four
    64-key chunks; a split here covers four or five): the running maxima
    move by far more than the lazy-rescale threshold in later chunks of a
    split too, not only in its first. 2 and 4 nodes give one and two
    query tiles (shared tiles only), 23 nodes two own tiles and a shared one
    per wave, so both rescale paths of the Q4_0 split kernel run, the shared
    tiles' one with the waves' P quarters taken against different maxima.
    The key scales are rounded to powers of two, so that the dequantised
    keys are exact in fp16: at scores this large (up to ~55 in log2 units)
    the one rounding of an ordinary scale times a code moves a score by
    more than the tolerance allows (row errors 6e-3 to 8e-3 measured, with
    or without the rescaling), which this test is not about."""
    inp = synth.attn_inputs(**dict(synth.WORKLOADS["27b"], n_ctx=20000, n_nodes=n_nodes))
    inp["q"] = (inp["q"].astype(np.float32) * 16).astype(np.float16)
    c = inp["k_cache"].copy()
    blocks = c.reshape(c.shape[0], c.shape[1], -1, 18)
    sc = blocks[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float32)
    ramp = (0.2 + 5.8 * (np.arange(c.shape[1]) % 256) / 255.0).astype(np.float32)[None, :, None]
    scr = sc * ramp
    p2 = np.exp2(np.round(np.log2(np.where(scr > 0, scr, 1.0))))
    sc16 = np.where(scr > 0, p2, 0.0).astype(np.float16)
    blocks[..., 0:2] = sc16[..., None].view(np.uint8).reshape(sc16.shape + (2,))
    inp["k_cache"] = c
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


def _ramped_q4_0(alpha, n_ctx=20000, n_nodes=23, seed=2):
    """The 27B layout with queries scaled by alpha and Q4_0 key scales that
    rise 30-fold over every 256 rows, rounded to fp16 as they are (not to
    powers of two): scores grow with alpha."""
    inp = synth.attn_inputs(**dict(synth.WORKLOADS["27b"], n_ctx=n_ctx, n_nodes=n_nodes, seed=seed))
    inp["q"] = (inp["q"].astype(np.float32) * alpha).astype(np.float16)
    c = inp["k_cache"].copy()
    blocks = c.reshape(c.shape[0], c.shape[1], -1, 18)
    sc = blocks[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float32)
    ramp = (0.2 + 5.8 * (np.arange(c.shape[1]) % 256) / 255.0).astype(np.float32)[None, :, None]
    sc16 = (sc * ramp).astype(np.float16)
    blocks[..., 0:2] = sc16[..., None].view(np.uint8).reshape(sc16.shape + (2,))
    inp["k_cache"] = c
    return inp


def test_q4_0_precision_edge_ordinary_scales():
    """The documented limit of the Q4_0 path: each dequantised key is rounded
    to fp16 once, which moves a score by up to 2^-11 of its terms, so the row
    error grows with the scores. With ordinary key scales (rising 30-fold
    over every 256 rows) and queries x1.5 the largest |scale q.k| is about 23
    in log2 units, inside the stated bound of 29, and the error stays within
    2e-3 (measured 0.8e-3 at x1 and 2.0e-3 at x2, where the scores reach 31)."""
    inp = _ramped_q4_0(1.5)
    D, G = inp["head_dim"], inp["n_q_heads"] // inp["n_kv_heads"]
    k = oracle.q4_0_dequant(inp["k_cache"], D)
    q = inp["q"].astype(np.float64)
    c = inp["scale"] * np.log2(np.e)
    smax = max(float(np.abs((q[:, h, :] @ k[h // G].T) * c).max()) for h in range(inp["n_q_heads"]))
    assert 20.0 < smax < 29.0, smax
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
def test_split_count_invariance(kv):
    """The same attention under different split plans: the 24 q / 4 kv layer
    at 32768 rows runs 64 key-range splits per KV head; each KV head called
    alone (6 q / 1 kv heads, the same rows) runs 256. Both within 2e-3 of the
    oracle and of each other."""
    import tree_verify_attention_ddtree_amd as tv
    inp = synth.attn_inputs(**dict(synth.WORKLOADS["27b"], n_ctx=32768, seed=61), kv=kv)
    kvt = tv.TV_KV_Q4_0 if kv == "q4_0" else tv.TV_KV_F16
    row = inp["k_cache"].shape[2] * inp["k_cache"].itemsize
    whole = gpu_attn(inp).astype(np.float64)
    d4, _p4 = tv.make_desc(inp["parent"], 24, 4, 256, kvt, 32768, 0, inp["scale"], row, row * 32768)
    d1, _p1 = tv.make_desc(inp["parent"], 6, 1, 256, kvt, 32768, 0, inp["scale"], row, row * 32768)
    s4, s1 = tv.tv_attn_plan(d4)["splits"], tv.tv_attn_plan(d1)["splits"]
    assert s1 >= 2 * s4, (s4, s1)
    parts = []
    for g in range(4):
        sub = dict(inp, n_q_heads=6, n_kv_heads=1, q=np.ascontiguousarray(inp["q"][:, 6 * g:6 * g + 6]),
                   k_tree=np.ascontiguousarray(inp["k_tree"][:, g:g + 1]),
                   v_tree=np.ascontiguousarray(inp["v_tree"][:, g:g + 1]),
                   k_cache=np.ascontiguousarray(inp["k_cache"][g:g + 1]),
                   v_cache=np.ascontiguousarray(inp["v_cache"][g:g + 1]))
        parts.append(gpu_attn(sub).astype(np.float64))
    split = np.concatenate(parts, axis=1)
    rows = sample_rows(23, 24, 48, 61)
    ref = oracle.attn(inp, rows=rows)
    assert check_rows(whole, ref, rows, 24) <= TOL
    assert check_rows(split, ref, rows, 24) <= TOL
    assert rownorm_err(split, whole) <= TOL


def test_deterministic():
    inp = synth.attn_inputs(**synth.WORKLOADS["27b"])
    a, b = gpu_attn(inp, repeat=2)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
@pytest.mark.parametrize("W,n_ctx", [(1, 700), (5, 700), (12, 700), (63, 700), (64, 700), (65, 700), (100, 4097),
                                     (2047, 4097), (2048, 4097), (5000, 4097), (30, 40), (3, 10), (64, 64)])
def test_per_position_window(kv, W, n_ctx):
    """window_mode 1: a node at depth k sees positions [n_ctx + k - W, n_ctx + k];
    windows narrower than the tree's depth, around the 64-row head the merge
    kernel scores, wider than the context, and contexts shorter than a chunk."""
    inp = synth.attn_inputs(n_q_heads=24, n_kv_heads=4, head_dim=256, n_ctx=n_ctx, n_nodes=23, depth_cap=16,
                            seed=4000 + W, kv=kv)
    inp = dict(inp, window=W, window_mode=1)
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


def test_per_position_window_61k_and_deep_chain():
    w = dict(synth.WORKLOADS["window"])
    inp = dict(synth.attn_inputs(**w), window_mode=1)
    rows = sample_rows(23, 24, 24, 7)
    err = check_rows(gpu_attn(inp), oracle.attn(inp, rows=rows), rows, 24)
    assert err <= TOL, err
    # a 64-node chain with a window of 10: ancestors beyond the window drop out
    ch = dict(synth.attn_inputs(n_q_heads=8, n_kv_heads=2, head_dim=128, n_ctx=300, n_nodes=64, depth_cap=64,
                                seed=77, kv="q4_0", parent=synth.chain_tree(64)), window=10, window_mode=1)
    err = rownorm_err(gpu_attn(ch).astype(np.float64), oracle.attn(ch))
    assert err <= TOL, err


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
@pytest.mark.parametrize("mode", [0, 1])
def test_remainder_rows_left_to_merge_kernel(kv, mode):
    """With 16 KV heads the grid has 16 splits per head (256 CUs); 16415 cache
    rows are 256 whole chunks, 16 to a split, plus 31 rows. A remainder chunk
    would make one split longer, so the merge kernel scores those 31 rows.
    With a per-position window over the whole cache the split kernel also
    masks, per node, the first rows of its first chunk."""
    inp = synth.attn_inputs(n_q_heads=16, n_kv_heads=16, head_dim=64, n_ctx=16415, n_nodes=12, depth_cap=8,
                            seed=4242 + mode, kv=kv)
    if mode:
        inp = dict(inp, window=16415, window_mode=1)
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


def _random_shapes(k, seed):
    """k seeded layer shapes across the descriptor's range: head dims, head
    counts and GQA groups, tree sizes 1..64, contexts from a few rows to a few
    thousand (whole chunks or ragged), windows of either mode, both cache
    types; sized so the oracle takes at most a few seconds each."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < k:
        D = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.integers(1, 9))
        n = int(rng.integers(1, 65))
        T = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 6000)), 64 * int(rng.integers(1, 90))]))
        W = int(rng.choice([0, 0, int(rng.integers(1, 3000))]))
        wm = int(rng.integers(0, 2)) if W else 0
        kv = str(rng.choice(["q4_0", "f16"]))
        if G * Hkv * n * T * D > 3e9:
            continue
        out.append((G * Hkv, Hkv, D, T, n, W, wm, kv, int(rng.integers(1 << 30))))
    return out


RANDOM_SHAPES = _random_shapes(96, 20261203)


@pytest.mark.parametrize("shape", RANDOM_SHAPES,
                         ids=[f"{s[0]}x{s[1]}x{s[2]}-T{s[3]}-n{s[4]}-W{s[5]}m{s[6]}-{s[7]}" for s in RANDOM_SHAPES])
def test_random_shapes(shape):
    """Seeded random shapes against the oracle: whatever split kernel, tile
    layout, row grouping, masking and merge path the planner picks for each."""
    Hq, Hkv, D, T, n, W, wm, kv, seed = shape
    inp = synth.attn_inputs(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_ctx=T, n_nodes=n, depth_cap=16, seed=seed,
                            kv=kv, window=W)
    inp["window_mode"] = wm
    err = rownorm_err(gpu_attn(inp).astype(np.float64), oracle.attn(inp))
    assert err <= TOL, err


def test_two_streams_own_workspaces():
    """Calls on two streams at once, each with its own inputs, outputs and
    workspace (the header's threading note): both match the oracle."""
    import torch

    import tree_verify_attention_ddtree_amd as tv
    from gpu_util import to_dev
    inps = [synth.attn_inputs(**dict(synth.WORKLOADS["27b"], n_ctx=4096 + 64 * k, seed=6100 + k)) for k in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    keep = []
    for inp, st in zip(inps, streams):
        t = to_dev(inp, "cuda")
        ts, hs = tv.cache_strides(t["k_cache"], tv.TV_KV_Q4_0)
        desc, par = tv.make_desc(inp["parent"], 24, 4, 256, tv.TV_KV_Q4_0, inp["k_cache"].shape[1], 0, inp["scale"],
                                 ts, hs)
        wsb = tv.tv_attn_workspace_bytes(desc)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        out = torch.full((23, 24, 256), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        keep.append((t, desc, par, ws))
        outs.append(out)
    for (t, desc, par, ws), out, st in zip(keep, outs, streams):
        for _ in range(5):
            tv.tree_verify_attn(desc, t["k_cache"], t["v_cache"], t["q"], t["k_tree"], t["v_tree"], out, ws,
                                ws.numel(), st)
    torch.cuda.synchronize()
    for inp, out in zip(inps, outs):
        err = rownorm_err(out.cpu().numpy().astype(np.float64), oracle.attn(inp))
        assert err <= TOL, err
