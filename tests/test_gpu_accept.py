"""GPU parity of tree_accept against the CPU oracle: bit-exact argmax,
accepted path, emitted tokens and bonus token."""

import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import gpu_accept

pytestmark = pytest.mark.gpu


def check(logits, parent, tokens):
    am, res = gpu_accept(logits, parent, tokens)
    ram, rres = oracle.accept(logits, parent, tokens)
    assert np.array_equal(am, ram), (am, ram)
    assert np.array_equal(res, rres), (res, rres)
    return rres


def test_tiny_planted():
    w = synth.WORKLOADS["tiny"]
    for seed in range(20):
        s = synth.streams(seed)
        parent = synth.draft_tree(s["tree"], 8, 4)
        tok = synth.sibling_distinct_tokens(s["tokens"], parent, w["vocab"])
        logits, L, _ = synth.planted_logits(s["logits"], parent, tok, w["vocab"])
        assert check(logits, parent, tok)[0] == L


def test_full_vocab_planted_64_trees():
    """23 x 152000 logits, planted paths, the 64 trees of the full step."""
    V = synth.WORKLOADS["full"]["vocab"]
    for t in range(64):
        s = synth.streams(5000 + t)
        parent = synth.draft_tree(s["tree"], 23, 16)
        tok = synth.sibling_distinct_tokens(s["tokens"], parent, V)
        logits, L, _ = synth.planted_logits(s["logits"], parent, tok, V)
        assert check(logits, parent, tok)[0] == L


@pytest.mark.parametrize("vocab", [1, 3, 7, 8191, 8192, 8193, 16383, 16384, 16385, 30001, 152000, 152003])
def test_vocab_sizes(vocab):
    rng = np.random.default_rng(vocab)
    parent = synth.draft_tree(rng, 23, 16)
    tok = rng.integers(0, vocab, size=23).astype(np.int32)
    logits = rng.standard_normal((23, vocab)).astype(np.float32)
    check(logits, parent, tok)


def test_ties_zeros_nan():
    V = 20000
    rng = np.random.default_rng(3)
    parent = np.array([-1, 0, 0, 1, 2, 3, 3, 5], np.int32)
    tok = np.array([0, 5, 9, 17000, 4, 12, 13, 8], np.int32)
    logits = rng.integers(-3, 3, size=(8, V)).astype(np.float32)  # many ties
    logits[0, 5] = 7.0
    logits[0, 17] = 7.0           # tie with a later index: 5 wins
    logits[1, :] = -0.0
    logits[1, 17000] = 0.0        # -0 == +0: index 0 wins
    logits[2, :] = np.nan         # all NaN -> 0
    logits[3, ::3] = np.nan
    logits[3, 4] = 100.0
    logits[4, :] = -np.inf
    logits[4, 12345] = np.nan     # NaN below -inf
    logits[5, 9999] = np.inf
    check(logits, parent, tok)


def test_duplicate_sibling_tokens():
    rng = np.random.default_rng(11)
    for trial in range(200):
        n = int(rng.integers(1, 30))
        parent = synth.draft_tree(rng, n, 8, p_spine=float(rng.random()))
        V = int(rng.integers(2, 5))
        tok = rng.integers(0, V, size=n).astype(np.int32)
        logits = rng.integers(-1, 2, size=(n, V)).astype(np.float32)
        check(logits, parent, tok)


def test_64_node_tree():
    rng = np.random.default_rng(64)
    parent = synth.draft_tree(rng, 64, 16)
    tok = synth.sibling_distinct_tokens(rng, parent, 1000)
    logits, L, _ = synth.planted_logits(rng, parent, tok, 1000)
    assert check(logits, parent, tok)[0] == L


def test_workspace_reused_across_calls():
    """One workspace for many calls of different sizes on one stream: the
    counters and maxima the last workgroup resets must be zero again for the
    next call (results bit-exact each time, workspace zero at the end)."""
    import torch

    import tree_verify_attention_ddtree_amd as tv
    V = synth.WORKLOADS["full"]["vocab"]
    ws = torch.zeros(tv.tv_accept_workspace_bytes(64, V), dtype=torch.uint8, device="cuda")
    for t, (n, vocab) in enumerate([(23, V), (8, 1024), (64, 5000), (23, V), (1, 7), (40, 70001)]):
        s = synth.streams(7100 + t)
        parent = synth.draft_tree(s["tree"], n, 16)
        tok = synth.sibling_distinct_tokens(s["tokens"], parent, vocab)
        logits, L, _ = synth.planted_logits(s["logits"], parent, tok, vocab)
        lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
        am = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        res = torch.full((2 + 2 * n,), -7, dtype=torch.int32, device="cuda")
        tv.tree_accept(lg, parent, tok, am, res, ws)
        torch.cuda.synchronize()
        ram, rres = oracle.accept(logits, parent, tok)
        assert np.array_equal(am.cpu().numpy(), ram) and np.array_equal(res.cpu().numpy(), rres), (n, vocab)
        assert int(rres[0]) == L
    assert int(ws.sum().item()) == 0


def test_stream_probe_reads_every_byte():
    """tv_stream_probe: the checksums of all workgroups XOR to the XOR of
    every dword of the buffer (each 16-byte piece is read by exactly one
    thread); the decoding kind runs on the same buffer."""
    import torch

    import tree_verify_attention_ddtree_amd as tv
    rng = np.random.default_rng(5)
    buf_np = rng.integers(0, 2 ** 32, size=(1 << 20) + 12, dtype=np.uint32)
    buf = torch.from_numpy(buf_np.view(np.int32)).cuda()
    chk = torch.zeros(96, dtype=torch.int32, device="cuda")
    tv.tv_stream_probe(buf, tv.TV_PROBE_READ, chk)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(chk.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(buf_np))
    tv.tv_stream_probe(buf, tv.TV_PROBE_Q4_0_DECODE, chk)
    torch.cuda.synchronize()
    # fewer 16-byte pieces than workgroups: the first ten read one each
    small = torch.from_numpy(buf_np[:40].view(np.int32)).cuda()
    tv.tv_stream_probe(small, tv.TV_PROBE_READ, chk)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(chk.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(buf_np[:40]))


@pytest.mark.parametrize("seed", range(40))
def test_random_trees_and_tied_logits(seed):
    """Seeded random trees (1..64 nodes, random depth caps), vocabularies
    from 1 to 40000 (slice edges included), logits drawn from a few values so
    that argmax ties are common, draft tokens that often match the parent's
    argmax (long accepted paths and competing equal-length paths), against
    the oracle bit for bit."""
    rng = np.random.default_rng(9000 + seed)
    n = int(rng.integers(1, 65))
    parent = synth.draft_tree(rng, n, int(rng.integers(1, 17)))
    vocab = int(rng.choice([1, 2, int(rng.integers(3, 3000)), 16384, 16385, int(rng.integers(3000, 40000))]))
    levels = rng.integers(1, 5)
    logits = rng.integers(0, levels + 1, size=(n, vocab)).astype(np.float32) * np.float32(0.5)
    am = logits.argmax(axis=1)  # first maximum: the smallest index on ties
    tok = np.where(rng.random(n) < 0.7, am[np.maximum(parent, 0)], rng.integers(0, vocab, size=n)).astype(np.int32)
    tok[0] = -1
    check(logits, parent, tok)
