"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the benchmark's `cpu_baseline` leg may import
this package.  The product library (`exact_attention_08_amd`) never imports, links or calls
it, and this package imports nothing from the product library: the two share only the
seeded input generators in `attn_inputs`, which hold none of the method's arithmetic.

The arithmetic lives in `oracle.c` (plain C, IEEE fp64, program order, OpenMP over rows);
this file only builds it and marshals numpy arrays.  See `oracle.c` for what each function
computes and the passage of the pages it follows.

Parity pins (tests/test_oracle_pins.py) tie every function here to something other than
itself: the pages' worked examples, closed forms, torch's float64 scaled_dot_product_attention
and scipy's logsumexp.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16, FP16 = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                        "-fPIC", "-shared", "-Wall", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_widen16.argtypes = [ctypes.c_uint16, i32]
    lib.oracle_widen16.restype = f64
    lib.oracle_attention.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, f64, i32,
                                     P, i64, P, P, P]
    lib.oracle_attention.restype = i32
    lib.oracle_decode_paged.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i64,
                                        f64, i32, P, i64, P, P]
    lib.oracle_decode_paged.restype = i32
    lib.oracle_decode_cascade.argtypes = [P, P, P, i32, P, P, P, P, i32, i32, i32, i32, i32,
                                          i32, i64, f64, i32, P, i64, P, P]
    lib.oracle_decode_cascade.restype = i32
    lib.oracle_attention_variant.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, f64,
                                             f64, i32, P, i64, P, P]
    lib.oracle_attention_variant.restype = i32
    lib.oracle_prefill_paged.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i64,
                                         i32, i32, f64, i32, P, i64, P, P]
    lib.oracle_prefill_paged.restype = i32
    lib.oracle_online_row.argtypes = [P, P, i32, i32, i32, P, P, P, P, P, P, P]
    lib.oracle_online_row.restype = i32
    lib.oracle_merge.argtypes = [P, P, i32, i32, P, P]
    lib.oracle_merge.restype = i32
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_set_threads.restype = None
    return lib


def _load():
    """The default oracle library (built on first use if nothing is built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(_LIB)
    return _lib


_override = None


def use_library(path):
    """Route the functions below through another build of oracle.c (None = the default).
    Used only by the tests that plant a mistake in a copy of the oracle."""
    global _override
    _override = None if path is None else _bind(path)


def _L():
    return _override if _override is not None else _load()


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def threads() -> int:
    return int(_L().oracle_threads())


def set_threads(n: int) -> None:
    _L().oracle_set_threads(int(n))


def widen16(bits: int, dtype: int) -> float:
    return float(_L().oracle_widen16(int(bits), int(dtype)))


def attention(q, k, v, causal: bool, scale: float, dtype: int, rows=None, return_probs=False):
    """Standard attention over dense [B,H,N,d] 16-bit inputs.

    rows: optional flat row indices (b*Hq + h)*N + i.  Returns (O [n,d] f64, LSE [n] f64)
    and, with return_probs, P [n, N] (tiny cases only)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == k.shape
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = B * Hq * N if r is None else len(r)
    O = np.zeros((n, d), dtype=np.float64)
    L = np.zeros(n, dtype=np.float64)
    P = np.zeros((n, N), dtype=np.float64) if return_probs else None
    rc = _L().oracle_attention(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, N, d, int(bool(causal)),
                                  float(scale), int(dtype), _ptr(r), n, _ptr(O), _ptr(L), _ptr(P))
    if rc != 0:
        raise ValueError(f"oracle_attention rejected its arguments ({rc})")
    if rows is None:
        O, L = O.reshape(B, Hq, N, d), L.reshape(B, Hq, N)
        if P is not None:
            P = P.reshape(B, Hq, N, N)
    return (O, L, P) if return_probs else (O, L)


def attention_variant(q, k, v, causal: bool, window: int, softcap: float, scale: float,
                      dtype: int, rows=None):
    """Attention with a sliding window (window > 0, causal only) and/or logits soft-cap
    (softcap > 0).  Layouts and returns as attention()."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == k.shape
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = B * Hq * N if r is None else len(r)
    O = np.zeros((n, d), dtype=np.float64)
    L = np.zeros(n, dtype=np.float64)
    rc = _L().oracle_attention_variant(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, N, d,
                                       int(bool(causal)), int(window), float(softcap),
                                       float(scale), int(dtype), _ptr(r), n, _ptr(O), _ptr(L))
    if rc != 0:
        raise ValueError(f"oracle_attention_variant rejected its arguments ({rc})")
    if rows is None:
        O, L = O.reshape(B, Hq, N, d), L.reshape(B, Hq, N)
    return O, L


def decode_paged(q, k_pages, v_pages, block_table, ctx_lens, scale: float, dtype: int,
                 pairs=None):
    """Paged decode: q [B,Hq,d], pools [P,page,Hkv,d], table [B,max_pages], ctx [B].
    pairs: optional flat (r*Hq + h).  Returns (O [B,Hq,d] or [n,d], LSE)."""
    q, kp, vp = _u16(q), _u16(k_pages), _u16(v_pages)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    B, Hq, d = q.shape
    num_pages, page, Hkv, d2 = kp.shape
    assert d2 == d and vp.shape == kp.shape and bt.shape[0] == B and ctx.shape == (B,)
    pr = None if pairs is None else np.ascontiguousarray(pairs, dtype=np.int64)
    n = B * Hq if pr is None else len(pr)
    O = np.zeros((n, d), dtype=np.float64)
    L = np.zeros(n, dtype=np.float64)
    rc = _L().oracle_decode_paged(_ptr(q), _ptr(kp), _ptr(vp), _ptr(bt), _ptr(ctx), B, Hq, Hkv,
                                     d, page, bt.shape[1], num_pages, float(scale), int(dtype),
                                     _ptr(pr), n, _ptr(O), _ptr(L))
    if rc != 0:
        raise ValueError(f"oracle_decode_paged rejected its arguments ({rc})")
    if pairs is None:
        O, L = O.reshape(B, Hq, d), L.reshape(B, Hq)
    return O, L


def decode_cascade(q, k_prefix, v_prefix, k_pages, v_pages, block_table, ctx_lens,
                   scale: float, dtype: int, pairs=None):
    """Shared-prefix decode: every request attends to the shared prefix k/v_prefix
    [Hkv, P, d] followed by its own paged tokens (as decode_paged).  Returns (O, LSE) like
    decode_paged."""
    q, kp, vp = _u16(q), _u16(k_pages), _u16(v_pages)
    kpre, vpre = _u16(k_prefix), _u16(v_prefix)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    B, Hq, d = q.shape
    num_pages, page, Hkv, d2 = kp.shape
    Hkv2, P, d3 = kpre.shape
    assert d2 == d and d3 == d and Hkv2 == Hkv and vpre.shape == kpre.shape
    assert vp.shape == kp.shape and bt.shape[0] == B and ctx.shape == (B,)
    pr = None if pairs is None else np.ascontiguousarray(pairs, dtype=np.int64)
    n = B * Hq if pr is None else len(pr)
    O = np.zeros((n, d), dtype=np.float64)
    L = np.zeros(n, dtype=np.float64)
    rc = _L().oracle_decode_cascade(_ptr(q), _ptr(kpre), _ptr(vpre), P, _ptr(kp), _ptr(vp),
                                    _ptr(bt), _ptr(ctx), B, Hq, Hkv, d, page, bt.shape[1],
                                    num_pages, float(scale), int(dtype), _ptr(pr), n, _ptr(O),
                                    _ptr(L))
    if rc != 0:
        raise ValueError(f"oracle_decode_cascade rejected its arguments ({rc})")
    if pairs is None:
        O, L = O.reshape(B, Hq, d), L.reshape(B, Hq)
    return O, L


def prefill_paged(q, k_pages, v_pages, block_table, cu_seqlens_q, kv_lens, causal: bool,
                  scale: float, dtype: int, rows=None):
    """Paged / varlen prefill: q [total_q, Hq, d] packed by cu_seqlens_q [B+1]; each request's
    cache (pools [P,page,Hkv,d], table [B,max_pages]) holds kv_lens[r] tokens, its new ones
    last.  rows: optional flat (token*Hq + h).  Returns (O [total_q,Hq,d] or [n,d], LSE)."""
    q, kp, vp = _u16(q), _u16(k_pages), _u16(v_pages)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    kvl = np.ascontiguousarray(kv_lens, dtype=np.int32)
    total_q, Hq, d = q.shape
    num_pages, page, Hkv, d2 = kp.shape
    B = kvl.shape[0]
    assert d2 == d and vp.shape == kp.shape and bt.shape[0] == B and cu.shape == (B + 1,)
    pr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = total_q * Hq if pr is None else len(pr)
    O = np.zeros((n, d), dtype=np.float64)
    L = np.zeros(n, dtype=np.float64)
    rc = _L().oracle_prefill_paged(_ptr(q), _ptr(kp), _ptr(vp), _ptr(bt), _ptr(cu), _ptr(kvl),
                                   B, Hq, Hkv, d, page, bt.shape[1], num_pages, total_q,
                                   int(bool(causal)), float(scale), int(dtype), _ptr(pr), n,
                                   _ptr(O), _ptr(L))
    if rc != 0:
        raise ValueError(f"oracle_prefill_paged rejected its arguments ({rc})")
    if rows is None:
        O, L = O.reshape(total_q, Hq, d), L.reshape(total_q, Hq)
    return O, L


def online_row(s, v, bc: int):
    """FA2-order online softmax of one row.  s [n] scores, v [n, dv].  Returns a dict with
    O, m, l, lse and the per-tile trace (m, l, acc)."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    if v.ndim == 1:
        v = v[:, None]
    n, dv = v.shape
    assert s.shape == (n,)
    tiles = (n + bc - 1) // bc
    O = np.zeros(dv)
    m, l, lse = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    tm, tl, ta = np.zeros(max(tiles, 1)), np.zeros(max(tiles, 1)), np.zeros((max(tiles, 1), dv))
    rc = _L().oracle_online_row(_ptr(s), _ptr(v), n, dv, bc, _ptr(O), ctypes.byref(m),
                                   ctypes.byref(l), ctypes.byref(lse), _ptr(tm), _ptr(tl),
                                   _ptr(ta))
    if rc != 0:
        raise ValueError("oracle_online_row rejected its arguments")
    return dict(O=O, m=m.value, l=l.value, lse=lse.value, trace_m=tm[:tiles],
                trace_l=tl[:tiles], trace_acc=ta[:tiles])


def merge(O_s, lse_s):
    """Merge normalised part outputs O_s [S, dv] with their LSE_s [S] (ascending order)."""
    O_s = np.ascontiguousarray(O_s, dtype=np.float64)
    if O_s.ndim == 1:
        O_s = O_s[:, None]
    lse_s = np.ascontiguousarray(lse_s, dtype=np.float64)
    S, dv = O_s.shape
    O = np.zeros(dv)
    lse = ctypes.c_double()
    rc = _L().oracle_merge(_ptr(O_s), _ptr(lse_s), S, dv, _ptr(O), ctypes.byref(lse))
    if rc != 0:
        raise ValueError("oracle_merge rejected its arguments")
    return O, lse.value
