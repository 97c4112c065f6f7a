"""Host-side checks of libtv.so that need no GPU.

The library must load, export every function include/tree_verify.h
declares, and reject invalid arguments on the host with the documented
status codes before it touches the device (these calls make no HIP call).
"""

import ctypes
import os
import re

import numpy as np
import pytest

import tree_verify_attention_ddtree_amd as tv
from tree_verify_attention_ddtree_amd import build as tvbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    tvbuild.ensure_built()
    return tv.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "tree_verify.h")).read()
    return sorted(set(re.findall(r"^TV_API\s+[\w\s\*]*?\b(\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(tv.EXPORTS)
    for name in names:
        assert hasattr(L, name), name


def test_strerror(L):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert tv.tv_strerror(code)
    assert tv.tv_strerror(12345) == "unknown status"


def _desc(parent=(-1, 0, 1), Hq=4, Hkv=2, D=64, kv=tv.TV_KV_Q4_0, n_ctx=256, window=0, scale=0.125,
          ts=36, hs=36 * 256):
    return tv.make_desc(parent, Hq, Hkv, D, kv, n_ctx, window, scale, ts, hs)


def _call(L, desc, ptrs=None, ws=None, wsb=0):
    if ptrs is None:
        ptrs = tv.TvAttnPtrs(4096, 4096, 4096, 4096, 4096, 4096)
    return L.tree_verify_attn(ctypes.byref(desc), ctypes.byref(ptrs), ws, wsb, None)


@pytest.mark.parametrize("parent,code", [
    ((0, 0), -2),          # root must have parent -1
    ((-1, 1), -2),         # parent must precede child
    ((-1, 0, 3, 1), -2),   # forward reference
    ((-1, -1), -2),        # second root
    (tuple([-1] + list(range(64))), -3),  # 65 nodes
])
def test_bad_trees_rejected(L, parent, code):
    d, keep = _desc(parent=parent)
    assert _call(L, d) == code


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), -3),       # H_q not a multiple of H_kv
    (dict(D=96), -3),              # head_dim not supported
    (dict(kv=7), -1),              # bad KV type
    (dict(n_ctx=-1), -3),
    (dict(window=-5), -3),
    (dict(scale=0.0), -1),
    (dict(scale=float("nan")), -1),
    (dict(scale=-0.1), -1),
    (dict(ts=35), -3),             # token stride below the row size
    (dict(ts=38), -4),             # Q4_0 strides must be multiples of 4
    (dict(ts=(1 << 24) + 4, hs=0), -3),  # row offsets inside a chunk must fit 32 bits
    (dict(kv=tv.TV_KV_F16, ts=136, hs=136 * 256), -4),  # F16 strides: multiples of 16
])
def test_bad_shapes_rejected(L, kw, code):
    d, keep = _desc(**kw)
    assert _call(L, d) == code


def test_null_and_misaligned_pointers_rejected(L):
    """Every call here fails a host check, so nothing is launched even where a
    GPU is visible (the fake pointers are never dereferenced). That an empty
    cache may be NULL, with no workspace, is checked on the GPU."""
    d, keep = _desc()
    assert _call(L, d, tv.TvAttnPtrs(4096, 4096, None, 4096, 4096, 4096)) == -1
    assert _call(L, d, tv.TvAttnPtrs(None, 4096, 4096, 4096, 4096, 4096)) == -1
    assert _call(L, d, tv.TvAttnPtrs(4096, 4096, 4098, 4096, 4096, 4096)) == -4
    assert _call(L, d, tv.TvAttnPtrs(4104, 4096, 4096, 4096, 4096, 4096)) == -4
    d0, keep0 = _desc(n_ctx=0)
    assert _call(L, d0, tv.TvAttnPtrs(None, None, None, 4096, 4096, 4096)) == -1
    assert _call(L, d0, tv.TvAttnPtrs(None, None, 4096, 4096, 4096, 4100)) == -4
    assert L.tree_verify_attn(None, None, None, 0, None) == -1


def test_accept_argument_checks(L):
    par = np.array([-1, 0, 0], np.int32)
    tok = np.array([0, 1, 2], np.int32)
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    f = L.tree_accept
    assert f(4096, 3, 10, P(np.array([0, 0, 0], np.int32)), P(tok), 4096, 4096, 4096, 1 << 20, None) == -2
    assert f(4096, 3, 0, P(par), P(tok), 4096, 4096, 4096, 1 << 20, None) == -3
    assert f(4096, 65, 10, P(np.arange(-1, 64, dtype=np.int32)), P(np.zeros(65, np.int32)), 4096, 4096, 4096,
             1 << 20, None) == -3
    assert f(None, 3, 10, P(par), P(tok), 4096, 4096, 4096, 1 << 20, None) == -1
    assert f(4096, 3, 10, P(par), None, 4096, 4096, 4096, 1 << 20, None) == -1
    assert f(4100, 3, 10, P(par), P(tok), 4096, 4096, 4096, 1 << 20, None) == -4
    assert f(4096, 3, 10, P(par), P(tok), 4096, 4096, None, 0, None) == -5
    assert f(4096, 3, 10, P(par), P(tok), 4096, 4096, 4096, 7, None) == -5
    assert tv.tv_accept_workspace_bytes(23, 152000) == tv.tv_accept_workspace_bytes(1, 7) == 832
    assert tv.tv_accept_workspace_bytes(0, 10) == 0
    assert tv.tv_accept_workspace_bytes(3, 0) == 0


def test_stream_probe_argument_checks(L):
    f = L.tv_stream_probe
    assert f(None, 4096, 0, 4096, 8, None) == -1
    assert f(4096, 4096, 0, None, 8, None) == -1
    assert f(4096, 4096, 2, 4096, 8, None) == -1       # unknown kind
    assert f(4096, 0, 0, 4096, 8, None) == -3           # nothing to read
    assert f(4096, 4096, 0, 4096, 0, None) == -3        # no workgroup
    assert f(4096, 4100, 1, 4096, 8, None) == -4        # not a multiple of 16 bytes
    assert f(4104, 4096, 1, 4096, 8, None) == -4        # base not 16-byte aligned


def test_library_links_no_oracle():
    """The GPU library and the oracle share nothing: no oracle symbol, no
    oracle header."""
    import subprocess
    out = subprocess.run(["nm", "-D", tvbuild.LIB], capture_output=True, text=True).stdout
    assert "tvref" not in out
    for src in os.listdir(tvbuild.CSRC):
        text = open(os.path.join(tvbuild.CSRC, src)).read()
        assert "tvref" not in text and "oracle" not in text.lower(), src


def test_commit_argument_checks(L):
    def call(n=5, hkv=2, D=64, kv=tv.TV_KV_Q4_0, n_ctx=10, cap=20, ts=36, hs=36 * 20, ptrs=(4096,) * 5):
        d = tv.make_commit_desc(n, hkv, D, kv, n_ctx, cap, ts, hs)
        return L.tree_commit_kv(ctypes.byref(d), *ptrs, None)

    assert L.tree_commit_kv(None, 4096, 4096, 4096, 4096, 4096, None) == -1
    assert call(n=0) == -3 and call(n=65) == -3
    assert call(hkv=0) == -3
    assert call(D=96) == -3
    assert call(kv=9) == -1
    assert call(n_ctx=-1) == -3
    assert call(n_ctx=16) == -3             # 16 + 5 rows would pass the capacity of 20
    assert call(ts=35) == -3                # below the Q4_0 row size
    assert call(ts=38) == -4                # Q4_0 strides: multiples of 4
    assert call(kv=tv.TV_KV_F16, ts=136, hs=136 * 20) == -4
    assert call(ptrs=(None, 4096, 4096, 4096, 4096)) == -1
    assert call(ptrs=(4096, 4096, 4096, 4096, None)) == -1
    assert call(ptrs=(4098, 4096, 4096, 4096, 4096)) == -4   # result must be 4-byte aligned
    assert call(ptrs=(4096, 4104, 4096, 4096, 4096)) == -4   # tree rows 16-byte aligned
    assert call(ptrs=(4096, 4096, 4096, 4100, 4096)) == -4   # caches 16-byte aligned


def test_commit_layers_argument_checks(L):
    d = tv.make_commit_desc(5, 2, 64, tv.TV_KV_Q4_0, 10, 20, 36, 36 * 20)
    arr = lambda *p: (ctypes.c_void_p * len(p))(*p)
    ok = arr(4096, 4096, 4096)
    f = lambda nl, res=4096, kt=ok, vt=ok, kc=ok, vc=ok: L.tree_commit_kv_layers(
        ctypes.byref(d), nl, res, kt, vt, kc, vc, None)
    assert f(0) == -3
    assert f(3, res=None) == -1
    assert f(3, kt=None) == -1
    assert f(3, vc=arr(4096, None, 4096)) == -1      # a null pointer in layer 1
    assert f(3, kc=arr(4096, 4096, 4100)) == -4      # a misaligned cache in layer 2
    assert f(3, res=4098) == -4
    bad = tv.make_commit_desc(5, 2, 64, tv.TV_KV_Q4_0, 16, 20, 36, 36 * 20)
    assert L.tree_commit_kv_layers(ctypes.byref(bad), 3, 4096, ok, ok, ok, ok, None) == -3


def test_window_mode_checked(L):
    d, keep = _desc()
    d.window_mode = 2
    assert _call(L, d) == -1
    d.window_mode = 1
    assert tv.tv_attn_plan(d, 256)["splits"] > 0  # valid (host-only query: nothing launched)


def test_row_bytes_fit_32_bit_offsets(L):
    """q, out and each split's workspace block are addressed with 32-bit
    buffer offsets: n * H_q * 2 * head_dim must stay below 2^31."""
    parent = tuple([-1] + list(range(63)))
    d, keep = _desc(parent=parent, Hq=1 << 16, Hkv=1, D=256, ts=144, hs=144 * 256)
    assert _call(L, d) == -3
    d, keep = _desc(parent=parent, Hq=(1 << 16) - 4, Hkv=1, D=256, ts=144, hs=144 * 256)
    assert tv.tv_attn_plan(d, 256)["splits"] >= 1
    # more than 65535 KV heads do not fit the split grid
    d, keep = _desc(parent=(-1,), Hq=1 << 16, Hkv=1 << 16, D=64)
    assert _call(L, d) == -3


def _plan(Hq, Hkv, n, D, kv, n_ctx, window=0, window_mode=0, n_cu=256):
    par = [-1] + [max(0, i - 1) for i in range(1, n)]
    row = D // 32 * 18 if kv == tv.TV_KV_Q4_0 else 2 * D
    d, keep = tv.make_desc(par, Hq, Hkv, D, kv, n_ctx, window, 0.0625, row, row * max(n_ctx, 1),
                           window_mode=window_mode)
    return tv.tv_attn_plan(d, n_cu)


def test_plan_query_layouts():
    """The 27B head layout (24 q / 4 kv heads) on 256 compute units, 256
    whole chunks per KV head: 8, 20 and 30 nodes give 3, 8 and 12 query
    tiles, which the Q4_0 kernels take as one own tile per wave (three
    shared tiles moved onto the warp-specialised kernel, one slot idle), two
    own tiles per wave and three own tiles per wave, with one row group. F16
    plans of head_dim 256 up to 8 tiles take the warp-specialised F16 kernel
    with one or two own tiles per wave, and with at most one shared tile
    above; the others the one-wave F16 kernel."""
    Q, F = tv.TV_KV_Q4_0, tv.TV_KV_F16
    p = _plan(24, 4, 8, 256, Q, 16384)
    assert (p["own_tiles"], p["shared_tiles"], p["row_groups"], p["masked"]) == (1, 0, 1, 0)
    assert (p["splits"], p["chunks"], p["kernel"]) == (64, 256, tv.TV_SPLIT_Q4_0_WS)
    # ... but a masked plan keeps the three shared tiles (one-wave kernel)
    p = _plan(24, 4, 8, 256, Q, 16384 + 31)
    assert (p["own_tiles"], p["shared_tiles"], p["masked"], p["kernel"]) == (0, 3, 1, tv.TV_SPLIT_Q4_0)
    # one or two Q4_0 tiles stay all-shared on the one-wave kernel
    p = _plan(24, 4, 2, 256, Q, 16384)
    assert (p["own_tiles"], p["shared_tiles"], p["kernel"]) == (0, 1, tv.TV_SPLIT_Q4_0)
    p = _plan(24, 4, 8, 256, F, 16384)
    assert (p["own_tiles"], p["shared_tiles"], p["kernel"]) == (1, 0, tv.TV_SPLIT_F16_WS)
    for kv in (Q, F):
        p = _plan(24, 4, 20, 256, kv, 16384)
        assert (p["own_tiles"], p["shared_tiles"], p["row_groups"]) == (2, 0, 1)
        assert p["kernel"] == (tv.TV_SPLIT_Q4_0_WS if kv == Q else tv.TV_SPLIT_F16_WS)
        p = _plan(24, 4, 30, 256, kv, 16384)
        assert (p["own_tiles"], p["shared_tiles"], p["row_groups"]) == (3, 0, 1)
        # three own tiles per wave do not fit two waves per SIMD
        assert p["kernel"] == (tv.TV_SPLIT_Q4_0 if kv == Q else tv.TV_SPLIT_F16)
    # at most two chunks a split (8K and below): half the splits, two row
    # groups (budget 22: groups of 5 and 4 tiles, one own tile per wave)
    p = _plan(24, 4, 23, 256, Q, 8192)
    assert (p["splits"], p["row_groups"], p["own_tiles"], p["shared_tiles"]) == (32, 2, 1, 1)
    assert p["kernel"] == tv.TV_SPLIT_Q4_0_WS
    p = _plan(24, 4, 23, 256, Q, 16384)
    assert (p["splits"], p["row_groups"]) == (64, 1)
    # F16 likewise, on the warp-specialised F16 kernel; not where a group
    # would leave the warp-specialised layouts (10 nodes: groups of two
    # shared tiles)
    p = _plan(24, 4, 23, 256, F, 8192)
    assert (p["splits"], p["row_groups"], p["own_tiles"], p["shared_tiles"]) == (32, 2, 1, 1)
    assert p["kernel"] == tv.TV_SPLIT_F16_WS
    p = _plan(24, 4, 10, 256, Q, 8192)
    assert (p["splits"], p["row_groups"], p["kernel"]) == (64, 1, tv.TV_SPLIT_Q4_0_WS)
    p = _plan(24, 4, 23, 256, F, 16384)
    assert (p["splits"], p["row_groups"], p["kernel"]) == (64, 1, tv.TV_SPLIT_F16_WS)
    # F16 with six tiles (16 nodes): two own tiles per wave, two slots idle,
    # instead of (1, 2); one or two tiles: one own tile per wave
    p = _plan(24, 4, 16, 256, F, 16384)
    assert (p["own_tiles"], p["shared_tiles"], p["kernel"]) == (2, 0, tv.TV_SPLIT_F16_WS)
    p = _plan(24, 4, 2, 256, F, 16384)
    assert (p["own_tiles"], p["shared_tiles"], p["kernel"]) == (1, 0, tv.TV_SPLIT_F16_WS)
    # masked or head_dim 128: the one-wave F16 kernel
    assert _plan(24, 4, 23, 256, F, 8192 + 31)["kernel"] == tv.TV_SPLIT_F16
    assert _plan(24, 4, 23, 128, F, 16384)["kernel"] == tv.TV_SPLIT_F16
    # budget 22 at 128K: two own tiles per wave and a shared one, 64 splits,
    # on the warp-specialised kernel (head_dim 256)
    p = _plan(24, 4, 23, 256, Q, 131072)
    assert (p["own_tiles"], p["shared_tiles"], p["splits"], p["chunks"]) == (2, 1, 64, 2048)
    assert p["kernel"] == tv.TV_SPLIT_Q4_0_WS
    # the chain-16 (six tiles: two own tiles per wave, two slots idle) too;
    # head_dim 128 does not
    p16 = _plan(24, 4, 16, 256, Q, 131072)
    assert (p16["own_tiles"], p16["shared_tiles"], p16["kernel"]) == (2, 0, tv.TV_SPLIT_Q4_0_WS)
    # twelve tiles in the two row groups of a 2048-row window: (1, 2)
    p12 = _plan(24, 4, 32, 256, Q, 8192, window=2048)
    assert (p12["own_tiles"], p12["shared_tiles"], p12["row_groups"], p12["kernel"]) == (1, 2, 2, tv.TV_SPLIT_Q4_0_WS)
    assert _plan(24, 4, 23, 128, Q, 131072)["kernel"] == tv.TV_SPLIT_Q4_0
    assert p["workspace_bytes"] == 64 * 23 * 24 * (2 * 256 + 4)
    # a 2048-row window: 32 chunks cap the splits, the rows are cut in two groups
    p = _plan(24, 4, 23, 256, Q, 61440, window=2048)
    assert (p["splits"], p["row_groups"], p["chunks"]) == (32, 2, 32)
    # a ragged window end: the masked kernel while splits stay short
    p = _plan(24, 4, 23, 256, Q, 8192 + 31)
    assert p["masked"] == 1 and p["merge_rows"] == 0 and p["kernel"] == tv.TV_SPLIT_Q4_0
    # ... and the merge kernel's rows once they are long
    p = _plan(24, 4, 23, 256, Q, 131072 + 31)
    assert p["masked"] == 0 and p["merge_rows"] == 31


@pytest.mark.parametrize("n_ctx", [0, 5, 63])
def test_plan_without_splits_needs_no_workspace(n_ctx):
    for kv in (tv.TV_KV_Q4_0, tv.TV_KV_F16):
        p = _plan(24, 4, 23, 256, kv, n_ctx)
        assert p["splits"] == 0 and p["workspace_bytes"] == 0 and p["kernel"] == tv.TV_SPLIT_NONE
        assert p["merge_rows"] == n_ctx


def test_step_argument_checks(L):
    """tree_verify_step rejects bad arguments on the host, before it asks the
    device anything (so nothing here launches where a GPU is visible)."""
    d, keep = _desc(parent=(-1, 0, 1), Hq=24, Hkv=4, D=256, n_ctx=4096, ts=144, hs=144 * 4096)
    good = tv.TvAttnPtrs(4096, 4096, 4096, 4096, 4096, 4096)
    arr = (tv.TvAttnPtrs * 2)(good, good)
    tok = np.array([0, 1, 2], np.int32)
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    f = lambda dd, nl, ly, lg=4096, V=100, tk=P(tok), am=4096, res=4096, ws=4096: L.tree_verify_step(
        ctypes.byref(dd), nl, ly, lg, V, tk, am, res, ws, 1 << 40, None)
    assert f(d, 0, arr) == -3                      # no layer
    assert f(d, tv.TV_MAX_LAYERS + 1, arr) == -3   # too many layers
    assert f(d, 2, None) == -1
    bad = (tv.TvAttnPtrs * 2)(good, tv.TvAttnPtrs(4096, 4096, None, 4096, 4096, 4096))
    assert f(d, 2, bad) == -1                      # a null tensor in the second layer
    bad = (tv.TvAttnPtrs * 2)(good, tv.TvAttnPtrs(4096, 4096, 4096, 4096, 4100, 4096))
    assert f(d, 2, bad) == -4                      # a misaligned one
    assert f(d, 2, arr, lg=None) == -1
    assert f(d, 2, arr, V=0) == -3
    assert f(d, 2, arr, tk=None) == -1
    assert f(d, 2, arr, ws=None) == -5
    assert f(d, 2, arr, ws=4096 + 16) == -4        # the workspace is 256-byte aligned
    dt, keep2 = _desc(parent=(-1, 0, 2), Hq=24, Hkv=4, D=256, n_ctx=4096, ts=144, hs=144 * 4096)
    assert f(dt, 2, arr) == -2
    assert L.tree_verify_step(None, 1, arr, 4096, 10, P(tok), 4096, 4096, 4096, 1 << 20, None) == -1


def test_step_plan():
    """Several layers: one launch where the warp-specialised split kernel
    runs, one work item per workgroup (acceptance items of two 16384-logit
    slices, split items, merge items of 8 rows, 4 for the last layer); the
    separate launches otherwise. One layer of head_dim 256: two launches.
    The workspace is
    a 2048-byte header plus each layer's partials, rounded to 256 bytes."""
    Q, F = tv.TV_KV_Q4_0, tv.TV_KV_F16
    par = [-1] + [i // 2 for i in range(22)]

    def plan(kv, n_ctx, L, vocab, D=256, parent=par, window=0):
        row = D // 32 * 18 if kv == Q else 2 * D
        d, keep = tv.make_desc(parent, 24, 4, D, kv, n_ctx, window, 0.0625, row, row * max(n_ctx, 1))
        return tv.tv_step_plan(d, L, vocab, 256), tv.tv_attn_plan(d, 256)

    # one layer: the split count of tree_verify_attn, two launches (the split
    # kernel, then the merge rows and acceptance slices side by side)
    p, a = plan(Q, 131072, 1, 152000)
    assert a["kernel"] == tv.TV_SPLIT_Q4_0_WS and a["splits"] == 64 and p["splits"] == 64
    assert (p["launches"], p["workgroups"], p["items"]) == (2, 64 * 4 + 23 * 24 + 23 * 10, 0)
    assert p["workspace_bytes"] == 2048 + (a["workspace_bytes"] + 255) // 256 * 256
    # also for the other kernels of head_dim 256 (F16, two row groups)
    p, a = plan(F, 8192, 1, 1000)
    assert (p["launches"], p["workgroups"]) == (2, a["splits"] * 4 * a["row_groups"] + 23 * 24 + 23)
    # one layer of head_dim 128, or without a whole chunk: the separate launches
    for n_ctx, D in ((8192, 128), (50, 256), (40, 128)):
        p, a = plan(Q, n_ctx, 1, 1000, D=D)
        assert (p["workgroups"], p["items"]) == (0, 0) and p["launches"] == (2 if a["splits"] else 1) + 1
    # 16 layers at 32K: half the splits (at most 16 chunks per split item)
    p, a = plan(Q, 32768, 16, 152000)
    assert a["splits"] == 64 and (p["splits"], p["row_groups"]) == (32, 1)
    n_items = (23 * 10 + 1) // 2 + 16 * 32 * 4 + 15 * ((23 * 24 + 7) // 8) + (23 * 24 + 3) // 4
    assert (p["launches"], p["workgroups"], p["items"]) == (1, n_items, n_items)
    layer = 32 * 23 * 24 * (2 * 256 + 4)
    assert p["workspace_bytes"] == 2048 + 16 * ((layer + 255) // 256 * 256)
    # 16 layers at 8K: at least two rounds of split items over 256 CUs
    p, a = plan(Q, 8192, 16, 152000)
    assert (a["splits"], a["row_groups"], p["splits"], p["row_groups"]) == (32, 2, 8, 1)
    # a 2048-row window: two row groups per KV head
    p, a = plan(Q, 61440, 3, 1000, window=2048)
    assert a["row_groups"] == 2 and (p["splits"], p["row_groups"]) == (32, 2)
    assert p["items"] == (23 + 1) // 2 + 3 * 32 * 4 * 2 + 2 * 69 + 138
    # separate launches: F16, head_dim 128, no whole chunk, a masked plan
    for kv, n_ctx, D in ((F, 32768, 256), (Q, 32768, 128), (Q, 50, 256), (Q, 4096 + 37, 256)):
        p, a = plan(kv, n_ctx, 4, 1000, D=D)
        assert p["workgroups"] == 0 and p["items"] == 0
        assert p["launches"] == 4 * (2 if a["splits"] else 1) + 1
    with pytest.raises(tv.TvError):
        plan(Q, 32768, 0, 1000)
    with pytest.raises(tv.TvError):
        plan(Q, 32768, 2, 0)
