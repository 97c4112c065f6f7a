"""Pins of the oracle's per-position sliding window (window_mode 1): a tree
node at depth k (position n_ctx + k) sees the positions [n_ctx + k - W,
n_ctx + k] of its own sequence, cache rows and ancestors alike: the keys a
token at that position sees when decoding token by token with window W.

Pinned against: torch's float64 scaled_dot_product_attention over the flat
sequence [cache; chain] with a band mask (a library routine); for any tree,
each node against the uniform window shrunk by its depth (bit for bit) and,
once the depth reaches W, against the chain of its own root path; and the
uniform mode where the two must agree (depth 0, windows wider than the
context).
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from test_oracle_attn import TOL, deq_cache, rownorm_err


def _depth(parent):
    d = np.zeros(len(parent), int)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


@pytest.mark.parametrize("W", [1, 3, 8, 20, 100, 300])
def test_chain_equals_banded_causal_attention(W):
    w = dict(synth.WORKLOADS["tiny"])
    n = 16
    inp = dict(synth.attn_inputs(**w, parent=synth.chain_tree(n), kv="f16"), window=W, window_mode=1)
    K, V = deq_cache(inp)
    Hq, Hkv, D = w["n_q_heads"], w["n_kv_heads"], w["head_dim"]
    G = Hq // Hkv
    T = K.shape[1]
    got = oracle.attn(inp)
    pos = np.arange(T + n)
    band = (pos[None, :] <= pos[:, None]) & (pos[None, :] >= pos[:, None] - W)
    for h in range(Hq):
        g = h // G
        keys = np.concatenate([K[g], inp["k_tree"][:, g].astype(np.float64)])
        vals = np.concatenate([V[g], inp["v_tree"][:, g].astype(np.float64)])
        qs = np.zeros((T + n, D))
        qs[T:] = inp["q"][:, h].astype(np.float64)
        o = F.scaled_dot_product_attention(torch.from_numpy(qs)[None, None], torch.from_numpy(keys)[None, None],
                                           torch.from_numpy(vals)[None, None], attn_mask=torch.from_numpy(band),
                                           scale=float(inp["scale"]))[0, 0].numpy()
        assert rownorm_err(got[:, h], o[T:]) < TOL, h


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
@pytest.mark.parametrize("W", [2, 5, 9, 40, 250])
def test_each_node_equals_uniform_window_shrunk_by_its_depth(kv, W):
    w = dict(synth.WORKLOADS["tiny"], n_nodes=23, depth_cap=12)
    inp = synth.attn_inputs(**w, kv=kv)
    d = _depth(inp["parent"])
    got = oracle.attn(dict(inp, window=W, window_mode=1))
    for i in range(len(d)):
        if d[i] < W:
            ref = oracle.attn(dict(inp, window=W - int(d[i]), window_mode=0))[i]
        else:
            # the window holds no cache row and part of the node's path: the
            # node's output is that of the last node of the chain made of its
            # root path (subtree independence), which the band pin covers
            path = [i]
            while inp["parent"][path[-1]] >= 0:
                path.append(int(inp["parent"][path[-1]]))
            path = path[::-1]
            chain = dict(inp, parent=synth.chain_tree(len(path)), q=inp["q"][path], k_tree=inp["k_tree"][path],
                         v_tree=inp["v_tree"][path], window=W, window_mode=1)
            ref = oracle.attn(chain)[-1]
        assert np.array_equal(got[i], ref), (i, int(d[i]))


def test_depth_zero_and_wide_windows_match_uniform():
    w = dict(synth.WORKLOADS["tiny"], n_nodes=20, depth_cap=10)
    inp = synth.attn_inputs(**w)
    T = inp["k_cache"].shape[1]
    a = oracle.attn(dict(inp, window=30, window_mode=1))
    b = oracle.attn(dict(inp, window=30, window_mode=0))
    assert np.array_equal(a[0], b[0])  # the root is at depth 0
    assert not np.array_equal(a, b)     # deeper nodes see fewer cache rows
    wide = T + 64
    assert np.array_equal(oracle.attn(dict(inp, window=wide, window_mode=1)),
                          oracle.attn(dict(inp, window=0, window_mode=0)))
    # window 0 means the whole cache in both modes
    assert np.array_equal(oracle.attn(dict(inp, window=0, window_mode=1)),
                          oracle.attn(dict(inp, window=0, window_mode=0)))
