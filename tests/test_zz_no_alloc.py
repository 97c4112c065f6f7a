"""The no-allocation acceptance entry point against tree_accept: two calls
in a row through the C ABI, the second with a smaller tree and vocabulary,
each bit-exact against tree_accept on the same inputs (and the oracle)."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _inputs(seed, n, vocab):
    s = synth.streams(seed)
    parent = synth.draft_tree(s["tree"], n, 16)
    tok = synth.sibling_distinct_tokens(s["tokens"], parent, vocab)
    logits, L, _ = synth.planted_logits(s["logits"], parent, tok, vocab)
    return parent, tok, logits, L


def test_noalloc_matches_workspace_entry_point():
    import torch

    import tree_verify_attention_ddtree_amd as tv
    V = synth.WORKLOADS["full"]["vocab"]
    for seed, n, vocab in ((7301, 23, V), (7302, 8, 1024)):
        parent, tok, logits, L = _inputs(seed, n, vocab)
        lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
        outs = []
        for noalloc in (True, False):
            am = torch.full((n,), -7, dtype=torch.int32, device="cuda")
            res = torch.full((2 + 2 * n,), -7, dtype=torch.int32, device="cuda")
            if noalloc:
                tv.tree_accept_noalloc(lg, parent, tok, am, res)
            else:
                ws = torch.zeros(tv.tv_accept_workspace_bytes(n, vocab), dtype=torch.uint8, device="cuda")
                tv.tree_accept(lg, parent, tok, am, res, ws)
            torch.cuda.synchronize()
            outs.append((am.cpu().numpy(), res.cpu().numpy()))
        (am0, res0), (am1, res1) = outs
        assert np.array_equal(am0, am1) and np.array_equal(res0, res1), (n, vocab)
        ram, rres = oracle.accept(logits, parent, tok)
        assert np.array_equal(am0, ram) and np.array_equal(res0, rres), (n, vocab)
        assert int(res0[0]) == L


def test_noalloc_rejects_oversized_trees():
    import torch

    import tree_verify_attention_ddtree_amd as tv
    n = tv.TV_MAX_NODES + 1
    lg = torch.zeros((n, 16), dtype=torch.float32, device="cuda")
    am = torch.zeros(n, dtype=torch.int32, device="cuda")
    res = torch.zeros(2 + 2 * n, dtype=torch.int32, device="cuda")
    with pytest.raises(tv.TvError) as e:
        tv.tree_accept_noalloc(lg, [-1] + list(range(n - 1)), [0] * n, am, res)
    assert e.value.code == -3
