"""GPU parity of tree_commit_kv (the KV commit of the accepted path) against
the oracle: the caches must come out bit for bit equal (Q4_0 bytes, F16
bits), for every head size, strided caches, special values, every path
length and results that are out of range; plus a closed decode loop of
verify -> accept -> commit steps run on the GPU and on the oracle side by
side."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _dev_commit(res, kt, vt, kc, vc, n_ctx, token_major=False):
    """Commit on the GPU; caches given head-major [H_kv][cap][row] and
    returned the same way."""
    import torch

    import tree_verify_attention_ddtree_amd as tv
    n, hkv, D = kt.shape
    kv = tv.TV_KV_Q4_0 if kc.dtype == np.uint8 else tv.TV_KV_F16
    cap = kc.shape[1]
    dev = "cuda"
    if token_major:
        tk = torch.from_numpy(np.ascontiguousarray(kc.transpose(1, 0, 2))).to(dev)
        tvv = torch.from_numpy(np.ascontiguousarray(vc.transpose(1, 0, 2))).to(dev)
        es = tk.element_size()
        ts, hs = tk.stride(0) * es, tk.stride(1) * es
    else:
        tk = torch.from_numpy(np.ascontiguousarray(kc)).to(dev)
        tvv = torch.from_numpy(np.ascontiguousarray(vc)).to(dev)
        ts, hs = tv.cache_strides(tk, kv)
    d = tv.make_commit_desc(n, hkv, D, kv, n_ctx, cap, ts, hs)
    r = torch.from_numpy(np.ascontiguousarray(res, np.int32)).to(dev)
    tv.tree_commit_kv(d, r, torch.from_numpy(kt).to(dev), torch.from_numpy(vt).to(dev), tk, tvv)
    torch.cuda.synchronize()
    k2, v2 = tk.cpu().numpy(), tvv.cpu().numpy()
    if token_major:
        k2, v2 = k2.transpose(1, 0, 2), v2.transpose(1, 0, 2)
    return k2, v2


def _caches(rng, kv, hkv, cap, D):
    if kv == "q4_0":
        return (rng.integers(0, 256, (hkv, cap, D // 32 * 18)).astype(np.uint8),
                rng.integers(0, 256, (hkv, cap, D // 32 * 18)).astype(np.uint8))
    return synth.f16_normal(rng, (hkv, cap, D)), synth.f16_normal(rng, (hkv, cap, D))


def _result(n, path):
    res = np.full(2 + 2 * n, -1, np.int32)
    res[0] = len(path) - 1
    res[1] = 7
    res[2:2 + len(path)] = path
    return res


def _check(res, kt, vt, kc, vc, n_ctx, token_major=False):
    gk, gv = _dev_commit(res, kt, vt, kc, vc, n_ctx, token_major)
    ok, ov = oracle.commit(res, kt, vt, kc, vc, n_ctx)
    assert np.array_equal(gk.view(np.uint8), ok.view(np.uint8))
    assert np.array_equal(gv.view(np.uint8), ov.view(np.uint8))


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
@pytest.mark.parametrize("D,hkv,n", [(64, 1, 5), (128, 2, 13), (256, 4, 23), (256, 1, 64)])
def test_commit_matches_oracle(kv, D, hkv, n):
    rng = np.random.default_rng(D + 7 * n)
    kt = synth.f16_normal(rng, (n, hkv, D), 0.7)
    vt = synth.f16_normal(rng, (n, hkv, D), 0.05)
    kc, vc = _caches(rng, kv, hkv, 3 * n + 9, D)
    for n_acc in (0, 1, n // 2, n - 1):
        path = [0] + sorted(rng.choice(np.arange(1, n), n_acc, replace=False).tolist()) if n_acc else [0]
        _check(_result(n, path), kt, vt, kc, vc, n_ctx=int(rng.integers(0, 2 * n + 10)))


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
def test_commit_token_major_cache(kv):
    rng = np.random.default_rng(4)
    n, hkv, D = 9, 3, 128
    kt, vt = synth.f16_normal(rng, (n, hkv, D)), synth.f16_normal(rng, (n, hkv, D))
    kc, vc = _caches(rng, kv, hkv, 40, D)
    _check(_result(n, [0, 1, 4, 8]), kt, vt, kc, vc, n_ctx=30, token_major=True)


def test_commit_special_values():
    """Ties of the largest magnitude (+m after -m and the reverse), zero
    blocks, fp16 subnormals, the largest finite fp16, infinities and NaN."""
    rng = np.random.default_rng(8)
    n, hkv, D = 6, 2, 256
    kt = synth.f16_normal(rng, (n, hkv, D))
    vt = synth.f16_normal(rng, (n, hkv, D))
    kt[0, 0, 0:32] = 0.0
    kt[0, 0, 32:64] = np.float16(2.0 ** -20) * rng.integers(-8, 8, 32)
    kt[0, 0, 64] = -3.0
    kt[0, 0, 70] = 3.0
    kt[0, 0, 96] = 3.0
    kt[0, 0, 100] = -3.0
    kt[0, 0, 128:160] = np.float16(65504.0) * np.sign(rng.standard_normal(32)).astype(np.float16)
    kt[0, 0, 160] = np.inf
    kt[0, 0, 192] = -np.inf
    kt[0, 0, 224] = np.nan
    vt[0, 1, :] = np.float16(2.0 ** -24)
    kc, vc = _caches(rng, "q4_0", hkv, 20, D)
    _check(_result(n, [0, 3]), kt, vt, kc, vc, n_ctx=11)


def test_commit_out_of_range_results_write_nothing():
    rng = np.random.default_rng(9)
    n, hkv, D = 7, 2, 64
    kt, vt = synth.f16_normal(rng, (n, hkv, D)), synth.f16_normal(rng, (n, hkv, D))
    kc, vc = _caches(rng, "q4_0", hkv, 16, D)
    for res in (_result(n, [0] * 8),           # n_acc = 7 is not below n
                np.array([-1] * (2 + 2 * n), np.int32)):  # n_acc = -1
        gk, gv = _dev_commit(res, kt, vt, kc, vc, 5)
        assert np.array_equal(gk, kc) and np.array_equal(gv, vc)
    # a path node out of range: that row alone is skipped
    res = _result(n, [0, 9, 2])
    gk, gv = _dev_commit(res, kt, vt, kc, vc, 5)
    ok, ov = oracle.commit(_result(n, [0]), kt, vt, kc, vc, 5)
    ok2, _ = oracle.commit(_result(n, [2, 2, 2]), kt, vt, kc, vc, 5)
    assert np.array_equal(gk[:, 5], ok[:, 5]) and np.array_equal(gk[:, 6], kc[:, 6])
    assert np.array_equal(gk[:, 7], ok2[:, 7])


def test_accept_then_commit_on_device():
    """The commit reads tree_accept's result where tree_accept left it."""
    import torch

    import tree_verify_attention_ddtree_amd as tv
    rng = np.random.default_rng(12)
    n, hkv, D, vocab = 23, 4, 256, 5000
    s = synth.streams(3)
    parent = synth.draft_tree(s["tree"], n, 16)
    tokens = synth.sibling_distinct_tokens(s["tokens"], parent, vocab)
    logits, L, _ = synth.planted_logits(s["logits"], parent, tokens, vocab)
    kt, vt = synth.f16_normal(rng, (n, hkv, D)), synth.f16_normal(rng, (n, hkv, D), 0.1)
    kc, vc = _caches(rng, "q4_0", hkv, 100, D)
    dev = "cuda"
    lg = torch.from_numpy(logits).to(dev)
    am = torch.empty(n, dtype=torch.int32, device=dev)
    res = torch.empty(2 + 2 * n, dtype=torch.int32, device=dev)
    ws = torch.zeros(tv.tv_accept_workspace_bytes(n, vocab), dtype=torch.uint8, device=dev)
    tk, tvv = torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)
    ts, hs = tv.cache_strides(tk, tv.TV_KV_Q4_0)
    tv.tree_accept(lg, parent, tokens, am, res, ws)
    tv.tree_commit_kv(tv.make_commit_desc(n, hkv, D, tv.TV_KV_Q4_0, 40, 100, ts, hs), res,
                      torch.from_numpy(kt).to(dev), torch.from_numpy(vt).to(dev), tk, tvv)
    torch.cuda.synchronize()
    _, ref = oracle.accept(logits, parent, tokens)
    assert ref[0] == L
    ok, ov = oracle.commit(ref, kt, vt, kc, vc, 40)
    assert np.array_equal(tk.cpu().numpy(), ok) and np.array_equal(tvv.cpu().numpy(), ov)


class _ToyLM:
    """Per-token Q/K/V embeddings and an output projection: the test's
    stand-in for the target model around the verify step."""

    def __init__(self, seed, vocab, hq, hkv, d):
        rng = np.random.default_rng(seed)
        self.qe = synth.f16_normal(rng, (vocab, hq, d), 0.5)
        self.ke = synth.f16_normal(rng, (vocab, hkv, d), 0.5)
        self.ve = synth.f16_normal(rng, (vocab, hkv, d), 1.0)
        self.wout = rng.standard_normal((vocab, hq * d))


def _toy_logits(lm, parent, tokens, kc, vc, n_ctx, hq, hkv, d):
    n = len(parent)
    inp = dict(n_q_heads=hq, n_kv_heads=hkv, head_dim=d, window=0, scale=d ** -0.5, parent=parent,
               k_cache=kc, v_cache=vc, q=lm.qe[tokens], k_tree=lm.ke[tokens], v_tree=lm.ve[tokens])
    o = oracle.attn(inp, n_ctx=n_ctx)
    flat = o.reshape(n, hq * d)
    return inp, o, np.stack([lm.wout @ flat[i] for i in range(n)]).astype(np.float32)


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
def test_decode_loop_matches_oracle(kv):
    """Ten steps of verify -> accept -> commit with the caches on the GPU,
    against the same loop on the oracle. Each step the GPU attention over the
    GPU-committed cache matches the oracle's within the attention bar; both
    acceptances get the same (oracle) logits, so the accepted paths and then
    the caches must agree bit for bit."""
    import torch

    from gpu_util import TOL, rownorm_err
    import tree_verify_attention_ddtree_amd as tv
    VOCAB, HQ, HKV, D, N, CAP = 8, 4, 2, 64, 8, 160
    lm = _ToyLM(5, VOCAB, HQ, HKV, D)
    rng = np.random.default_rng(77)
    kvt = tv.TV_KV_Q4_0 if kv == "q4_0" else tv.TV_KV_F16
    # a committed prefix of 40 tokens, stored by the oracle's own commit
    kc, vc = _caches(rng, kv, HKV, CAP, D)
    prefix = rng.integers(0, VOCAB, 40)
    for j, t in enumerate(prefix):
        kc, vc = oracle.commit(_result(1, [0]), lm.ke[[t]], lm.ve[[t]], kc, vc, j)
    n_ctx, root = 40, int(rng.integers(VOCAB))
    dev = "cuda"
    gk, gv = torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)
    ts, hs = tv.cache_strides(gk, kvt)
    accepted = []
    for step in range(10):
        parent = synth.draft_tree(rng, N, 4)
        tokens = synth.sibling_distinct_tokens(rng, parent, VOCAB)
        tokens[0] = root
        # a drafter that guesses the target's argmax along first children
        for i in range(1, N):
            if i == min(j for j in range(1, N) if parent[j] == parent[i]):
                tokens[i] = int(np.argmax(_toy_logits(lm, parent, tokens, kc, vc, n_ctx, HQ, HKV, D)[2][parent[i]]))
        inp, o_ref, lg = _toy_logits(lm, parent, tokens, kc, vc, n_ctx, HQ, HKV, D)
        _, res_ref = oracle.accept(lg, parent, tokens)
        # the GPU step over the GPU-committed cache
        desc, _p = tv.make_desc(parent, HQ, HKV, D, kvt, n_ctx, 0, D ** -0.5, ts, hs)
        wsb = tv.tv_attn_workspace_bytes(desc)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        out = torch.empty((N, HQ, D), dtype=torch.float32, device=dev)
        qd, ktd, vtd = (torch.from_numpy(inp[k]).to(dev) for k in ("q", "k_tree", "v_tree"))
        tv.tree_verify_attn(desc, gk, gv, qd, ktd, vtd, out, ws, wsb)
        am = torch.empty(N, dtype=torch.int32, device=dev)
        res = torch.empty(2 + 2 * N, dtype=torch.int32, device=dev)
        aws = torch.zeros(tv.tv_accept_workspace_bytes(N, VOCAB), dtype=torch.uint8, device=dev)
        tv.tree_accept(torch.from_numpy(lg).to(dev), parent, tokens, am, res, aws)
        tv.tree_commit_kv(tv.make_commit_desc(N, HKV, D, kvt, n_ctx, CAP, ts, hs), res, ktd, vtd, gk, gv)
        torch.cuda.synchronize()
        assert rownorm_err(out.cpu().numpy().astype(np.float64), o_ref) <= TOL, step
        assert np.array_equal(res.cpu().numpy(), res_ref), step
        kc, vc = oracle.commit(res_ref, inp["k_tree"], inp["v_tree"], kc, vc, n_ctx)
        assert np.array_equal(gk.cpu().numpy().view(np.uint8), kc.view(np.uint8)), step
        assert np.array_equal(gv.cpu().numpy().view(np.uint8), vc.view(np.uint8)), step
        accepted.append(int(res_ref[0]))
        n_ctx += int(res_ref[0]) + 1
        root = int(res_ref[1])  # the bonus token is the next step's root
    assert sum(accepted) >= 10, accepted


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
def test_commit_layers_matches_oracle(kv):
    """tree_commit_kv_layers: each layer's caches as the oracle commits them."""
    import torch

    import tree_verify_attention_ddtree_amd as tv
    rng = np.random.default_rng(31)
    n, hkv, D, cap, n_ctx, NL = 23, 4, 256, 60, 30, 5
    kvt = tv.TV_KV_Q4_0 if kv == "q4_0" else tv.TV_KV_F16
    res = _result(n, [0, 2, 5, 6, 11])
    kts = [synth.f16_normal(rng, (n, hkv, D), 0.3 + l) for l in range(NL)]
    vts = [synth.f16_normal(rng, (n, hkv, D), 0.1) for _ in range(NL)]
    caches = [_caches(rng, kv, hkv, cap, D) for _ in range(NL)]
    dev = "cuda"
    g_kt = [torch.from_numpy(x).to(dev) for x in kts]
    g_vt = [torch.from_numpy(x).to(dev) for x in vts]
    g_kc = [torch.from_numpy(c[0]).to(dev) for c in caches]
    g_vc = [torch.from_numpy(c[1]).to(dev) for c in caches]
    ts, hs = tv.cache_strides(g_kc[0], kvt)
    r = torch.from_numpy(res).to(dev)
    tv.tree_commit_kv_layers(tv.make_commit_desc(n, hkv, D, kvt, n_ctx, cap, ts, hs), r, g_kt, g_vt, g_kc, g_vc)
    torch.cuda.synchronize()
    for l in range(NL):
        ok, ov = oracle.commit(res, kts[l], vts[l], caches[l][0], caches[l][1], n_ctx)
        assert np.array_equal(g_kc[l].cpu().numpy().view(np.uint8), ok.view(np.uint8)), l
        assert np.array_equal(g_vc[l].cpu().numpy().view(np.uint8), ov.view(np.uint8)), l
