"""Python binding of libtv.so: DDTree tree-verify attention and greedy
acceptance on MI355X (gfx950).

The functions carry the names of the C ABI in include/tree_verify.h and only
marshal arguments: torch tensors become device pointers, host arrays become
int32 buffers, and a non-zero status becomes an exception. Every step of the
computation runs in the HIP kernels of libtv.so; there is no fallback. The
library must have been built (``python -m tree_verify_attention_ddtree_amd.build``
or ``__graft_entry__.build()``); importing works without it, calling does not.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

TV_OK = 0
TV_KV_F16 = 0
TV_KV_Q4_0 = 1
TV_MAX_NODES = 64
TV_MAX_LAYERS = 16

_lib = None


class TvAttnDesc(ctypes.Structure):
    _fields_ = [
        ("n_nodes", ctypes.c_int32),
        ("parent", ctypes.c_void_p),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_type", ctypes.c_int32),
        ("n_ctx", ctypes.c_int64),
        ("window", ctypes.c_int64),
        ("kv_token_stride", ctypes.c_int64),
        ("kv_head_stride", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("window_mode", ctypes.c_int32),
    ]


class TvAttnPtrs(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("k_tree", ctypes.c_void_p),
        ("v_tree", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
    ]


class TvAttnPlanInfo(ctypes.Structure):
    _fields_ = [
        ("splits", ctypes.c_int32),
        ("row_groups", ctypes.c_int32),
        ("own_tiles", ctypes.c_int32),
        ("shared_tiles", ctypes.c_int32),
        ("masked", ctypes.c_int32),
        ("kernel", ctypes.c_int32),
        ("chunks", ctypes.c_int64),
        ("merge_rows", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_uint64),
    ]


TV_SPLIT_NONE = 0
TV_SPLIT_F16 = 1
TV_SPLIT_Q4_0 = 2
TV_SPLIT_Q4_0_WS = 3
TV_SPLIT_F16_WS = 4


class TvStepPlanInfo(ctypes.Structure):
    _fields_ = [
        ("launches", ctypes.c_int32),
        ("workgroups", ctypes.c_int32),
        ("splits", ctypes.c_int32),
        ("row_groups", ctypes.c_int32),
        ("items", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_uint64),
    ]


class TvError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {tv_strerror(code)} ({code})")


def lib_path() -> str:
    """libtv.so next to this file, or the build TV_LIB names (the host-only
    sanitizer build of tests/sanitize/run_cpu_suite.sh, whose launches all
    fail with TV_E_HIP)."""
    return os.environ.get("TV_LIB") or _build.LIB


def lib():
    """The loaded libtv.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it first (python -m tree_verify_attention_ddtree_amd.build)")
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        L.tv_strerror.argtypes = [ctypes.c_int]
        L.tv_strerror.restype = ctypes.c_char_p
        L.tv_attn_workspace_bytes.argtypes = [ctypes.POINTER(TvAttnDesc)]
        L.tv_attn_workspace_bytes.restype = ctypes.c_size_t
        L.tree_verify_attn.argtypes = [ctypes.POINTER(TvAttnDesc), ctypes.POINTER(TvAttnPtrs), P, ctypes.c_size_t, P]
        L.tree_verify_attn.restype = ctypes.c_int
        L.tv_accept_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.tv_accept_workspace_bytes.restype = ctypes.c_size_t
        L.tree_accept.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, ctypes.c_size_t, P]
        L.tree_accept.restype = ctypes.c_int
        L.tree_commit_kv.argtypes = [ctypes.POINTER(TvCommitDesc), P, P, P, P, P, P]
        L.tree_commit_kv.restype = ctypes.c_int
        L.tree_commit_kv_layers.argtypes = [ctypes.POINTER(TvCommitDesc), ctypes.c_int32, P, P, P, P, P, P]
        L.tree_commit_kv_layers.restype = ctypes.c_int
        L.tree_accept_noalloc.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P]
        L.tree_accept_noalloc.restype = ctypes.c_int
        L.tv_stream_probe.argtypes = [P, ctypes.c_uint64, ctypes.c_int32, P, ctypes.c_int32, P]
        L.tv_stream_probe.restype = ctypes.c_int
        L.tv_attn_plan.argtypes = [ctypes.POINTER(TvAttnDesc), ctypes.c_int32, ctypes.POINTER(TvAttnPlanInfo)]
        L.tv_attn_plan.restype = ctypes.c_int
        L.tv_step_workspace_bytes.argtypes = [ctypes.POINTER(TvAttnDesc), ctypes.c_int32, ctypes.c_int32]
        L.tv_step_workspace_bytes.restype = ctypes.c_size_t
        L.tv_step_plan.argtypes = [ctypes.POINTER(TvAttnDesc), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.POINTER(TvStepPlanInfo)]
        L.tv_step_plan.restype = ctypes.c_int
        L.tree_verify_step.argtypes = [ctypes.POINTER(TvAttnDesc), ctypes.c_int32, ctypes.POINTER(TvAttnPtrs), P,
                                       ctypes.c_int32, P, P, P, P, ctypes.c_size_t, P]
        L.tree_verify_step.restype = ctypes.c_int
        _lib = L
    return _lib


class TvCommitDesc(ctypes.Structure):
    _fields_ = [
        ("n_nodes", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_type", ctypes.c_int32),
        ("n_ctx", ctypes.c_int64),
        ("capacity", ctypes.c_int64),
        ("kv_token_stride", ctypes.c_int64),
        ("kv_head_stride", ctypes.c_int64),
    ]


EXPORTS = ("tree_verify_attn", "tree_accept", "tree_commit_kv", "tree_commit_kv_layers", "tv_attn_workspace_bytes",
           "tv_accept_workspace_bytes", "tv_strerror", "tv_attn_plan", "tree_accept_noalloc", "tv_stream_probe",
           "tv_step_workspace_bytes", "tv_step_plan", "tree_verify_step")


def tv_strerror(code: int) -> str:
    return lib().tv_strerror(int(code)).decode()


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(int(t.data_ptr()))


def _stream_ptr(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(int(stream.cuda_stream))


def make_desc(parent, n_q_heads, n_kv_heads, head_dim, kv_type, n_ctx, window, scale, kv_token_stride=0,
              kv_head_stride=0, window_mode=0):
    """A TvAttnDesc plus the int32 buffer its parent pointer refers to (keep
    both alive while the descriptor is used)."""
    par = np.ascontiguousarray(np.asarray(parent), dtype=np.int32)
    d = TvAttnDesc(len(par), par.ctypes.data_as(ctypes.c_void_p).value, int(n_q_heads), int(n_kv_heads),
                   int(head_dim), int(kv_type), int(n_ctx), int(window), int(kv_token_stride),
                   int(kv_head_stride), float(scale), int(window_mode))
    return d, par


def cache_strides(cache, kv_type):
    """Token and head strides in bytes of a head-major cache tensor
    [H_kv, T, row] (uint8 rows for Q4_0, fp16 rows for F16)."""
    es = cache.element_size()
    return cache.stride(1) * es, cache.stride(0) * es


def tv_attn_workspace_bytes(desc: TvAttnDesc) -> int:
    return int(lib().tv_attn_workspace_bytes(ctypes.byref(desc)))


def tv_attn_plan(desc: TvAttnDesc, n_cu: int = 0) -> dict:
    """The split plan tree_verify_attn would use on a device with n_cu
    compute units (0: the current device). Host-only; raises TvError for an
    invalid descriptor."""
    info = TvAttnPlanInfo()
    rc = lib().tv_attn_plan(ctypes.byref(desc), int(n_cu), ctypes.byref(info))
    if rc != TV_OK:
        raise TvError(rc, "tv_attn_plan")
    return {name: int(getattr(info, name)) for name, _ in TvAttnPlanInfo._fields_}


def tree_verify_attn(desc: TvAttnDesc, k_cache, v_cache, q, k_tree, v_tree, out, workspace=None,
                     workspace_bytes=None, stream=None) -> None:
    """One layer of tree-verify attention (see include/tree_verify.h).

    Tensors are device tensors: caches laid out as the descriptor's strides
    say, q / k_tree / v_tree fp16, out fp32. ``workspace`` is a device
    tensor of at least tv_attn_workspace_bytes(desc) bytes (or None when that
    is 0).
    """
    ptrs = TvAttnPtrs(*(p.value if p is not None else None for p in
                        (_ptr(k_cache), _ptr(v_cache), _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(out))))
    wsb = workspace_bytes
    if wsb is None:
        wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().tree_verify_attn(ctypes.byref(desc), ctypes.byref(ptrs), _ptr(workspace), int(wsb),
                                _stream_ptr(stream))
    if rc != TV_OK:
        raise TvError(rc, "tree_verify_attn")


def _attn_ptrs(k_cache, v_cache, q, k_tree, v_tree, out):
    return TvAttnPtrs(*(p.value if p is not None else None for p in
                        (_ptr(k_cache), _ptr(v_cache), _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(out))))


def tv_step_workspace_bytes(desc: TvAttnDesc, n_layers: int, vocab: int) -> int:
    return int(lib().tv_step_workspace_bytes(ctypes.byref(desc), int(n_layers), int(vocab)))


def tv_step_plan(desc: TvAttnDesc, n_layers: int, vocab: int, n_cu: int = 0) -> dict:
    """How tree_verify_step runs this shape (host only): launches per call,
    work-queue workgroups and items, workspace bytes."""
    info = TvStepPlanInfo()
    rc = lib().tv_step_plan(ctypes.byref(desc), int(n_layers), int(vocab), int(n_cu), ctypes.byref(info))
    if rc != TV_OK:
        raise TvError(rc, "tv_step_plan")
    return {name: int(getattr(info, name)) for name, _ in TvStepPlanInfo._fields_}


def step_layers(layers):
    """The C array of per-layer tensors tree_verify_step takes, from a
    sequence of (k_cache, v_cache, q, k_tree, v_tree, out) device tensors
    (build it once to call the step many times)."""
    arr = (TvAttnPtrs * max(1, len(layers)))()
    for i, ly in enumerate(layers):
        arr[i] = _attn_ptrs(*ly)
    return arr


def tree_verify_step(desc: TvAttnDesc, layers, logits, tokens, argmax_out, result_out, workspace,
                     stream=None) -> None:
    """One verify step (see include/tree_verify.h): ``layers`` is a sequence
    of (k_cache, v_cache, q, k_tree, v_tree, out) device tensors, one per
    layer, all of the descriptor's shape (or the array step_layers made of
    one); ``logits`` device fp32
    [n, vocab]; ``tokens`` a host int sequence (the parent array is the
    descriptor's); ``workspace`` a device tensor of
    tv_step_workspace_bytes(desc, len(layers), vocab) bytes whose first 2048
    bytes are zero before its first use (allocate it with torch.zeros)."""
    n, vocab = int(logits.shape[0]), int(logits.shape[1])
    tok = np.ascontiguousarray(np.asarray(tokens), dtype=np.int32)
    if len(tok) != n or n != desc.n_nodes:
        raise ValueError("tokens length and logits.shape[0] must equal the descriptor's node count")
    arr = step_layers(layers) if not isinstance(layers, ctypes.Array) else layers
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().tree_verify_step(ctypes.byref(desc), len(layers), arr, _ptr(logits), vocab,
                                tok.ctypes.data_as(ctypes.c_void_p), _ptr(argmax_out), _ptr(result_out),
                                _ptr(workspace), int(wsb), _stream_ptr(stream))
    if rc != TV_OK:
        raise TvError(rc, "tree_verify_step")


def tv_accept_workspace_bytes(n_nodes: int, vocab: int) -> int:
    return int(lib().tv_accept_workspace_bytes(int(n_nodes), int(vocab)))


def tree_accept(logits, parent, tokens, argmax_out, result_out, workspace, stream=None) -> None:
    """Greedy acceptance (see include/tree_verify.h). ``logits`` is a device
    fp32 [n, vocab] tensor, ``parent``/``tokens`` host int sequences,
    ``argmax_out`` device int32 [n], ``result_out`` device int32 [2 + 2n].
    ``workspace`` holds tv_accept_workspace_bytes(n, vocab) bytes, zero
    before its first use (allocate it with torch.zeros); every call leaves it
    zero."""
    n, vocab = int(logits.shape[0]), int(logits.shape[1])
    par = np.ascontiguousarray(np.asarray(parent), dtype=np.int32)
    tok = np.ascontiguousarray(np.asarray(tokens), dtype=np.int32)
    if len(par) != n or len(tok) != n:
        raise ValueError("parent/tokens length must equal logits.shape[0]")
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().tree_accept(_ptr(logits), n, vocab, par.ctypes.data_as(ctypes.c_void_p),
                           tok.ctypes.data_as(ctypes.c_void_p), _ptr(argmax_out), _ptr(result_out),
                           _ptr(workspace), int(wsb), _stream_ptr(stream))
    if rc != TV_OK:
        raise TvError(rc, "tree_accept")


def tree_accept_noalloc(logits, parent, tokens, argmax_out, result_out, stream=None) -> None:
    """tree_accept without a workspace (the library's per-device static
    state; see include/tree_verify.h): for callers that cannot allocate.
    Calls on one device must not overlap."""
    n, vocab = int(logits.shape[0]), int(logits.shape[1])
    par = np.ascontiguousarray(np.asarray(parent), dtype=np.int32)
    tok = np.ascontiguousarray(np.asarray(tokens), dtype=np.int32)
    if len(par) != n or len(tok) != n:
        raise ValueError("parent/tokens length must equal logits.shape[0]")
    rc = lib().tree_accept_noalloc(_ptr(logits), n, vocab, par.ctypes.data_as(ctypes.c_void_p),
                                   tok.ctypes.data_as(ctypes.c_void_p), _ptr(argmax_out), _ptr(result_out),
                                   _stream_ptr(stream))
    if rc != TV_OK:
        raise TvError(rc, "tree_accept_noalloc")


TV_PROBE_READ = 0
TV_PROBE_Q4_0_DECODE = 1


def tv_stream_probe(buf, kind, checksums, stream=None) -> None:
    """Stream a device tensor's bytes (read, or read and unpack as Q4_0
    codes) with one checksum word per workgroup in ``checksums`` (device
    uint32/int32 tensor; its length is the workgroup count)."""
    nbytes = buf.numel() * buf.element_size()
    rc = lib().tv_stream_probe(_ptr(buf), nbytes, int(kind), _ptr(checksums), int(checksums.numel()),
                               _stream_ptr(stream))
    if rc != TV_OK:
        raise TvError(rc, "tv_stream_probe")


def make_commit_desc(n_nodes, n_kv_heads, head_dim, kv_type, n_ctx, capacity, kv_token_stride, kv_head_stride):
    return TvCommitDesc(int(n_nodes), int(n_kv_heads), int(head_dim), int(kv_type), int(n_ctx), int(capacity),
                        int(kv_token_stride), int(kv_head_stride))


def tree_commit_kv(desc: TvCommitDesc, result, k_tree, v_tree, k_cache, v_cache, stream=None) -> None:
    """Append the accepted path (tree_accept's device result) to one layer's
    caches: torch device tensors, caches head-major as for tree_verify_attn."""
    rc = lib().tree_commit_kv(ctypes.byref(desc), _ptr(result), _ptr(k_tree), _ptr(v_tree), _ptr(k_cache),
                              _ptr(v_cache), _stream_ptr(stream))
    if rc != TV_OK:
        raise TvError(rc, "tree_commit_kv")


def tree_commit_kv_layers(desc: TvCommitDesc, result, k_trees, v_trees, k_caches, v_caches, stream=None) -> None:
    """tree_commit_kv over several layers in one launch: lists of torch device
    tensors, one entry per layer, all of the shape `desc` describes."""
    nl = len(k_trees)
    if not (len(v_trees) == len(k_caches) == len(v_caches) == nl):
        raise ValueError("one K/V tree row buffer and one K/V cache per layer")
    arr = lambda ts: (ctypes.c_void_p * nl)(*[int(t.data_ptr()) for t in ts])
    rc = lib().tree_commit_kv_layers(ctypes.byref(desc), nl, _ptr(result), arr(k_trees), arr(v_trees),
                                     arr(k_caches), arr(v_caches), _stream_ptr(stream))
    if rc != TV_OK:
        raise TvError(rc, "tree_commit_kv_layers")
