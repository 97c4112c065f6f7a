"""Tree-speculative greedy decoding reproduces token-by-token greedy decoding.

The Luce DFlash post states that the target graph's output is bit-identical
to autoregressive decoding and that verification is greedy. This pins the
oracle's attention mask and its acceptance together on a toy one-layer model:
its per-token Q/K/V embeddings lie on the lattice {(c - 8) / 8}, which fp16
and Q4_0 (scale 1/8) both hold exactly, so committing a token's K/V to either
cache loses nothing. The token streams must be identical and the logits of
every accepted node must equal, bit for bit, the logits greedy decoding
computes at the same position.
"""

import numpy as np
import pytest

import oracle
import synth

VOCAB = 64
HQ, HKV, D = 4, 2, 64


class ToyLM:
    def __init__(self, seed):
        rng = np.random.default_rng(seed)
        lat = lambda shape: ((rng.integers(0, 16, size=shape) - 8) / 8.0)
        self.qe = lat((VOCAB, HQ, D)).astype(np.float16)
        self.ke = lat((VOCAB, HKV, D)).astype(np.float16)
        self.ve = lat((VOCAB, HKV, D)).astype(np.float16)
        self.codes_k = (self.ke.astype(np.float64) * 8 + 8).astype(np.uint8)
        self.codes_v = (self.ve.astype(np.float64) * 8 + 8).astype(np.uint8)
        self.wout = rng.standard_normal((VOCAB, HQ * D))

    def q4_0_row(self, codes):
        """Q4_0 bytes of one row with scale 1/8 (fp16 0x3000)."""
        out = np.zeros(D // 32 * 18, np.uint8)
        for b in range(D // 32):
            c = codes[32 * b:32 * b + 32]
            out[18 * b] = 0x00
            out[18 * b + 1] = 0x30
            out[18 * b + 2:18 * b + 18] = c[:16] | (c[16:] << 4)
        return out

    def cache_rows(self, toks, kv):
        if kv == "f16":
            return self.ke[toks].transpose(1, 0, 2), self.ve[toks].transpose(1, 0, 2)
        k = np.stack([[self.q4_0_row(self.codes_k[t, g]) for t in toks] for g in range(HKV)])
        v = np.stack([[self.q4_0_row(self.codes_v[t, g]) for t in toks] for g in range(HKV)])
        return k.reshape(HKV, len(toks), -1), v.reshape(HKV, len(toks), -1)

    def verify(self, committed, tree_tokens, parent, kv):
        """Logits (float64 [n, VOCAB]) of every tree node."""
        kc, vc = self.cache_rows(committed, kv)
        inp = dict(n_q_heads=HQ, n_kv_heads=HKV, head_dim=D, window=0, scale=1.0 / 8.0,
                   parent=np.asarray(parent, np.int32), k_cache=kc, v_cache=vc,
                   q=self.qe[tree_tokens], k_tree=self.ke[tree_tokens], v_tree=self.ve[tree_tokens])
        out = oracle.attn(inp).reshape(len(parent), HQ * D)
        # one matrix-vector product per node, the same call greedy decoding makes
        return np.stack([self.wout @ out[i] for i in range(len(parent))])


def greedy_ar(lm, prompt, n_new, kv):
    committed = list(prompt[:-1])
    cur = prompt[-1]
    toks, logits = [], []
    for _ in range(n_new):
        lg = lm.verify(committed, [cur], [-1], kv)[0]
        nxt = oracle.argmax_row(lg.astype(np.float32))
        logits.append(lg)
        toks.append(nxt)
        committed.append(cur)
        cur = nxt
    return toks, logits


@pytest.mark.parametrize("kv", ["f16", "q4_0"])
def test_tree_speculation_reproduces_greedy_ar(kv):
    lm = ToyLM(7)
    rng = np.random.default_rng(99)
    prompt = [int(t) for t in rng.integers(0, VOCAB, size=12)]
    n_new = 40
    ar_toks, ar_logits = greedy_ar(lm, prompt, n_new + 20, kv)

    committed = list(prompt[:-1])
    cur = prompt[-1]
    out = []
    out_logits = []
    steps = 0
    while len(out) < n_new:
        pos = len(out)  # ar_toks[pos] is the token greedy decoding emits next
        # draft tree: a first-child spine following the greedy continuation
        # for a random length, then random siblings and descendants
        L = int(rng.integers(0, 7))
        parent = [-1]
        toks = [cur]
        spine = [0]
        for k in range(L):
            parent.append(spine[-1])
            toks.append(ar_toks[pos + k])
            spine.append(len(parent) - 1)
        for _ in range(int(rng.integers(0, 8))):
            p = int(rng.integers(0, len(parent)))
            used = {toks[c] for c in range(1, len(parent)) if parent[c] == p}
            t = int(rng.integers(0, VOCAB))
            if t in used:
                continue
            parent.append(p)
            toks.append(t)
        # renumber topologically (parents already precede children)
        lg = lm.verify(committed, toks, parent, kv)
        tokens = np.array(toks, np.int32)
        _, res = oracle.accept(lg.astype(np.float32), np.array(parent, np.int32), tokens)
        n_acc = int(res[0])
        n = len(parent)
        path = [int(x) for x in res[2:2 + n_acc + 1]]
        emitted = [int(x) for x in res[2 + n:2 + n + n_acc + 1]]
        for k, node in enumerate(path):
            assert np.array_equal(lg[node], ar_logits[pos + k]), (steps, k)
        out += emitted
        out_logits += [lg[p] for p in path]
        committed += [toks[p] for p in path]
        cur = emitted[-1]
        steps += 1
    assert out[:n_new] == ar_toks[:n_new]
    assert steps < n_new  # speculation accepted something
