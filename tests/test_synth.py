"""The seeded generators are deterministic and produce the stated shapes."""

import numpy as np

import synth


def test_seed_determinism():
    a = synth.attn_inputs(**synth.WORKLOADS["tiny"])
    b = synth.attn_inputs(**synth.WORKLOADS["tiny"])
    for k in ("k_cache", "v_cache", "q", "k_tree", "v_tree", "parent"):
        assert np.array_equal(a[k], b[k])


def test_tree_shapes():
    for seed in range(50):
        s = synth.streams(seed)
        p = synth.draft_tree(s["tree"], 23, 16)
        assert p[0] == -1 and all(0 <= p[i] < i for i in range(1, 23))
        depth = [0] * 23
        for i in range(1, 23):
            depth[i] = depth[p[i]] + 1
        assert max(depth) <= 16
        tok = synth.sibling_distinct_tokens(s["tokens"], p, 50)
        for u in range(23):
            sib = [tok[c] for c in range(1, 23) if p[c] == u]
            assert len(sib) == len(set(sib))
    assert list(synth.chain_tree(4)) == [-1, 0, 1, 2]


def test_q4_0_cache_layout():
    s = synth.streams(0)
    c = synth.q4_0_cache(s["k_cache"], 2, 10, 256)
    assert c.shape == (2, 10, 144) and c.dtype == np.uint8
    assert synth.q4_0_row_bytes(64) == 36
