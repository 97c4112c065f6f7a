"""CPU oracle for tree-verify attention and greedy acceptance.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. It shares no code with the GPU
library and never imports it.

The arithmetic lives in ``tvref.c`` (plain definitions in double precision,
OpenMP over output rows); this module only builds and loads it and marshals
numpy arrays. See the header of ``tvref.c`` for what each function computes
and which readings of the pages it takes.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tvref.c")
# TVREF_LIB names another build of tvref.c to load instead (the sanitizer
# run of tests/sanitize/run_cpu_suite.sh); it is loaded as it is
_LIB = os.environ.get("TVREF_LIB") or os.path.join(_HERE, "libtvref.so")

KV_F16 = 0
KV_Q4_0 = 1

_lib = None


def build() -> str:
    """Compile tvref.c into libtvref.so with gcc and OpenMP."""
    # no contraction: the Q4_0 quantiser rounds x * id and the + 8.5 separately
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp",
           "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.environ.get("TVREF_LIB") and (not os.path.exists(_LIB) or
                                                os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.tvref_half_to_double.argtypes = [ctypes.c_uint16]
        L.tvref_half_to_double.restype = dbl
        L.tvref_q4_0_dequant_row.argtypes = [P, i32, P]
        L.tvref_q4_0_dequant_row.restype = None
        L.tvref_q4_0_dequant_rows.argtypes = [P, i64, i32, P]
        L.tvref_q4_0_dequant_rows.restype = None
        L.tvref_check_tree.argtypes = [i32, P]
        L.tvref_check_tree.restype = i32
        L.tvref_ancestors.argtypes = [i32, P, P]
        L.tvref_ancestors.restype = i32
        L.tvref_attn.argtypes = [i32, P, i32, i32, i32, i64, i64, i32, dbl, i32, P, P, i64, i64, P, P, P, P, i32, P]
        L.tvref_attn.restype = i32
        L.tvref_argmax_row.argtypes = [P, i32]
        L.tvref_argmax_row.restype = i32
        L.tvref_accept.argtypes = [P, i32, i32, P, P, P, P]
        L.tvref_accept.restype = i32
        L.tvref_float_to_half.argtypes = [ctypes.c_float]
        L.tvref_float_to_half.restype = ctypes.c_uint16
        L.tvref_q4_0_quantize_block.argtypes = [P, P]
        L.tvref_q4_0_quantize_block.restype = None
        L.tvref_q4_0_quantize_rows.argtypes = [P, i64, i32, P]
        L.tvref_q4_0_quantize_rows.restype = None
        L.tvref_commit.argtypes = [i32, i32, i32, i32, i64, i64, P, P, P, P, P, i64, i64]
        L.tvref_commit.restype = i32
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """OpenMP threads the oracle uses from now on (the GNU OpenMP runtime the
    library is linked against)."""
    lib()
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def max_threads() -> int:
    lib()
    return int(ctypes.CDLL("libgomp.so.1").omp_get_max_threads())


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def half_to_double(bits: int) -> float:
    return lib().tvref_half_to_double(int(bits) & 0xFFFF)


def q4_0_dequant(rows: np.ndarray, head_dim: int) -> np.ndarray:
    """Q4_0 bytes [..., row_bytes] -> float64 [..., head_dim]."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    rb = head_dim // 32 * 18
    assert rows.shape[-1] == rb
    lead = rows.shape[:-1]
    nr = int(np.prod(lead)) if lead else 1
    out = np.empty(lead + (head_dim,), np.float64)
    lib().tvref_q4_0_dequant_rows(_ptr(rows), nr, head_dim, _ptr(out))
    return out


def ancestors(i: int, parent) -> list:
    parent = np.ascontiguousarray(parent, np.int32)
    buf = np.empty(len(parent), np.int32)
    k = lib().tvref_ancestors(int(i), _ptr(parent), _ptr(buf))
    return buf[:k].tolist()


def check_tree(parent) -> int:
    parent = np.ascontiguousarray(parent, np.int32)
    return lib().tvref_check_tree(len(parent), _ptr(parent))


def attn(inp: dict, rows=None, n_ctx=None) -> np.ndarray:
    """Oracle attention for one layer.

    ``inp`` holds the arrays of ``synth.attn_inputs`` (head-major caches);
    ``inp["window_mode"]`` (default 0) selects the per-position window (1).
    ``rows``: optional iterable of output rows r = i*H_q + h; other rows of the
    result are NaN. ``n_ctx`` overrides the number of committed rows used.
    Returns float64 [n, H_q, D].
    """
    parent = np.ascontiguousarray(inp["parent"], np.int32)
    n = len(parent)
    Hq, Hkv, D = inp["n_q_heads"], inp["n_kv_heads"], inp["head_dim"]
    kc = np.ascontiguousarray(inp["k_cache"])
    vc = np.ascontiguousarray(inp["v_cache"])
    kv = KV_Q4_0 if kc.dtype == np.uint8 else KV_F16
    if kv == KV_F16:
        kc = kc.astype(np.float16, copy=False)
        vc = vc.astype(np.float16, copy=False)
    ctx = kc.shape[1] if n_ctx is None else int(n_ctx)
    tok_stride = kc.strides[1]
    head_stride = kc.strides[0]
    assert vc.strides == kc.strides
    q = np.ascontiguousarray(inp["q"], np.float16)
    kt = np.ascontiguousarray(inp["k_tree"], np.float16)
    vt = np.ascontiguousarray(inp["v_tree"], np.float16)
    out = np.full((n, Hq, D), np.nan, np.float64)
    rws = None if rows is None else np.ascontiguousarray(list(rows), np.int32)
    rc = lib().tvref_attn(n, _ptr(parent), Hq, Hkv, D, ctx, int(inp.get("window", 0)),
                          int(inp.get("window_mode", 0)), float(inp["scale"]), kv,
                          _ptr(kc), _ptr(vc), tok_stride, head_stride, _ptr(q.view(np.uint16)),
                          _ptr(kt.view(np.uint16)), _ptr(vt.view(np.uint16)), _ptr(rws),
                          0 if rws is None else len(rws), _ptr(out))
    if rc != 0:
        raise ValueError(f"tvref_attn failed with {rc}")
    return out


def argmax_row(row: np.ndarray) -> int:
    row = np.ascontiguousarray(row, np.float32)
    return int(lib().tvref_argmax_row(_ptr(row), len(row)))


def accept(logits: np.ndarray, parent, tokens):
    """Oracle greedy acceptance. Returns (argmax int32[n], result int32[2+2n])."""
    logits = np.ascontiguousarray(logits, np.float32)
    parent = np.ascontiguousarray(parent, np.int32)
    tokens = np.ascontiguousarray(tokens, np.int32)
    n, vocab = logits.shape
    am = np.empty(n, np.int32)
    res = np.empty(2 + 2 * n, np.int32)
    rc = lib().tvref_accept(_ptr(logits), n, vocab, _ptr(parent), _ptr(tokens), _ptr(am), _ptr(res))
    if rc != 0:
        raise ValueError(f"tvref_accept failed with {rc}")
    return am, res


def float_to_half(x: float) -> int:
    """fp16 bits of an fp32 value, rounded to nearest even."""
    return int(lib().tvref_float_to_half(float(np.float32(x))))


def q4_0_quantize(x: np.ndarray) -> np.ndarray:
    """fp32 [..., D] (D a multiple of 32) -> Q4_0 bytes [..., 18*D/32], with
    the quantiser reading documented in tvref.c."""
    x = np.ascontiguousarray(x, np.float32)
    D = x.shape[-1]
    assert D % 32 == 0
    lead = x.shape[:-1]
    nr = int(np.prod(lead)) if lead else 1
    out = np.empty(lead + (18 * (D // 32),), np.uint8)
    lib().tvref_q4_0_quantize_rows(_ptr(x), nr, D, _ptr(out))
    return out


def commit(result, k_tree, v_tree, k_cache, v_cache, n_ctx):
    """Oracle KV commit of the accepted path into head-major caches.

    result: int32 [2 + 2n] from the acceptance; k_tree, v_tree: fp16 [n][H_kv][D];
    k_cache, v_cache: [H_kv][capacity][row] (uint8 Q4_0 rows or fp16 values).
    Returns new (k_cache, v_cache) arrays; the inputs are not modified.
    """
    result = np.ascontiguousarray(result, np.int32)
    kt = np.ascontiguousarray(k_tree, np.float16)
    vt = np.ascontiguousarray(v_tree, np.float16)
    n, Hkv, D = kt.shape
    kc = np.array(k_cache, copy=True, order="C")
    vc = np.array(v_cache, copy=True, order="C")
    kv = KV_Q4_0 if kc.dtype == np.uint8 else KV_F16
    rc = lib().tvref_commit(n, Hkv, D, kv, int(n_ctx), kc.shape[1], _ptr(result), _ptr(kt.view(np.uint16)),
                            _ptr(vt.view(np.uint16)), _ptr(kc), _ptr(vc), kc.strides[1], kc.strides[0])
    if rc != 0:
        raise ValueError(f"tvref_commit failed with {rc}")
    return kc, vc
