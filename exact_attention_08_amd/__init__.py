"""Python binding of libattn.so: exact attention forward on MI355X (gfx950).

The binding only marshals arguments: it reads shapes, device pointers and the current HIP
stream from torch tensors and calls the C ABI declared in include/attn.h.  Every step of
the computation runs in the library's HIP kernels.  There is no fallback: if libattn.so is
missing every call fails with ImportError, and a non-zero status from the library raises AttnError.

    attn_fwd(Q, K, V, O, LSE, causal, scale=None, stream=None)
    attn_decode_paged(q, k_pages, v_pages, block_table, ctx_lens, O, LSE, split_tokens,
                      workspace, scale=None, stream=None)
    attn_decode_paged_noalloc(q, k_pages, v_pages, block_table, ctx_lens, O, LSE, split_tokens,
                              scale=None, stream=None)
    attn_decode_paged_workspace_bytes(B, Hq, d, page_size, max_pages_per_seq, split_tokens)
    attn_decode_cascade(q, k_prefix, v_prefix, k_pages, v_pages, block_table, ctx_lens, O, LSE,
                        split_tokens, workspace, scale=None, stream=None)
    attn_decode_cascade_workspace_bytes(B, Hq, d, page_size, max_pages_per_seq, split_tokens,
                                        prefix_len)
    attn_prefill_paged(q, k_pages, v_pages, block_table, cu_seqlens_q, kv_lens, O, LSE,
                       max_q_len, causal=True, scale=None, stream=None)
    attn_fwd_variant(Q, K, V, O, LSE, causal, window=0, softcap=0.0, scale=None, stream=None)

split_tokens = 0 asks the decode calls for a split length chosen on the device.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")
_lib = None


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:  # pragma: no cover
        return []


def _load():
    """Load libattn.so on first use and declare its argument types.

    The package itself imports without the library, so that the build module
    (exact_attention_08_amd.build) works from a clean checkout; every compute call goes
    through here and fails with ImportError when the library is not built (there is no
    non-HIP implementation to fall back to)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m exact_attention_08_amd.build` "
            "(there is no non-HIP implementation to fall back to)")
    # One HIP runtime per process: torch brings its own libamdhip64 (same soname as ROCm's).
    # Loading torch first makes libattn.so's libamdhip64 dependency bind to that copy, so the
    # streams and device pointers torch hands over belong to the runtime that launches the
    # kernels.  Loading libattn.so first would pull in a second runtime.
    import torch  # noqa: F401  (imported for its HIP runtime)

    lib_ = ctypes.CDLL(LIB_PATH)
    if len(_hip_runtimes_mapped()) > 1:
        raise ImportError("two HIP runtimes are loaded in this process "
                          f"({_hip_runtimes_mapped()}); import torch before loading libattn.so")
    _P, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib_.attn_fwd.argtypes = [_P, _P, _P, _P, _P, _i, _i, _i, _i, _i, _i, _f, _i, _P]
    lib_.attn_fwd.restype = _i
    lib_.attn_decode_paged.argtypes = [_P, _P, _P, _P, _P, _P, _P, _i, _i, _i, _i, _i, _i, _i,
                                       _f, _i, _P, _sz, _P]
    lib_.attn_decode_paged.restype = _i
    lib_.attn_decode_paged_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _i, _i, _i, _i, _i,
                                               _i, _i, _f, _i, _P]
    lib_.attn_decode_paged_noalloc.restype = _i
    lib_.attn_decode_paged_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
    lib_.attn_decode_paged_workspace_bytes.restype = _sz
    lib_.attn_decode_cascade.argtypes = [_P, _P, _P, _i, _P, _P, _P, _P, _P, _P, _i, _i, _i, _i,
                                         _i, _i, _i, _f, _i, _P, _sz, _P]
    lib_.attn_decode_cascade.restype = _i
    lib_.attn_decode_cascade_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
    lib_.attn_decode_cascade_workspace_bytes.restype = _sz
    lib_.attn_fwd_variant.argtypes = [_P, _P, _P, _P, _P, _i, _i, _i, _i, _i, _i, _i, _f, _f,
                                      _i, _P]
    lib_.attn_fwd_variant.restype = _i
    lib_.attn_prefill_paged.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _i, _i, _i, _i, _i, _i,
                                        _i, _i, _f, _i, _P]
    lib_.attn_prefill_paged.restype = _i
    _lib = lib_
    return _lib


ATTN_OK = 0
STATUS = {0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_DTYPE",
          -4: "ATTN_ERR_UNSUPPORTED", -5: "ATTN_ERR_ALIGN", -6: "ATTN_ERR_WORKSPACE",
          -7: "ATTN_ERR_HIP", -8: "ATTN_ERR_TOO_LARGE"}
ATTN_BF16, ATTN_FP16 = 0, 1
EXPORTS = ("attn_fwd", "attn_decode_paged", "attn_decode_paged_noalloc",
           "attn_decode_paged_workspace_bytes",
           "attn_decode_cascade", "attn_decode_cascade_workspace_bytes", "attn_prefill_paged",
           "attn_fwd_variant")


class AttnError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {code} ({STATUS.get(code, 'unknown')})")
        self.code = code


def lib():
    """The raw ctypes handle (argument types set), for callers that pass pointers."""
    return _load()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_FP16
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float16")


def _stream_ptr(t, stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, code):
    if code != ATTN_OK:
        raise AttnError(fn, code)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def attn_fwd(Q, K, V, O, LSE, causal: bool, scale: float | None = None, stream=None) -> None:
    """O, LSE <- attention(Q, K, V).  Q,O [B,Hq,N,d]; K,V [B,Hkv,N,d]; LSE [B,Hq,N] fp32."""
    import torch
    for name, t in (("Q", Q), ("K", K), ("V", V), ("O", O), ("LSE", LSE)):
        _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
    _need(Q.dim() == 4 and K.dim() == 4 and V.shape == K.shape and O.shape == Q.shape,
          "shapes: Q,O [B,Hq,N,d]; K,V [B,Hkv,N,d]")
    B, Hq, N, d = Q.shape
    _need(K.shape[0] == B and K.shape[2] == N and K.shape[3] == d, "K/V must match Q in B, N, d")
    _need(LSE.dtype == torch.float32 and tuple(LSE.shape) == (B, Hq, N), "LSE must be fp32 [B,Hq,N]")
    dt = _dtype_code(Q)
    _need(K.dtype == Q.dtype and V.dtype == Q.dtype and O.dtype == Q.dtype, "dtypes must match")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _load().attn_fwd(Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), LSE.data_ptr(),
                         B, Hq, K.shape[1], N, d, int(bool(causal)), float(scale), dt,
                         _stream_ptr(Q, stream))
    _check("attn_fwd", code)


def attn_fwd_variant(Q, K, V, O, LSE, causal: bool, window: int = 0, softcap: float = 0.0,
                     scale: float | None = None, stream=None) -> None:
    """As attn_fwd, with a causal sliding window (window > 0: query i sees keys
    i - window < j <= i) and/or logits soft-cap (softcap > 0: s -> c tanh(s / c))."""
    import torch
    for name, t in (("Q", Q), ("K", K), ("V", V), ("O", O), ("LSE", LSE)):
        _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
    _need(Q.dim() == 4 and K.dim() == 4 and V.shape == K.shape and O.shape == Q.shape,
          "Q,O must be [B,Hq,N,d] and K,V [B,Hkv,N,d]")
    B, Hq, N, d = Q.shape
    _need(K.shape[0] == B and K.shape[2] == N and K.shape[3] == d, "K/V shape mismatch")
    _need(LSE.dtype == torch.float32 and tuple(LSE.shape) == (B, Hq, N), "LSE must be fp32 [B,Hq,N]")
    dt = _dtype_code(Q)
    _need(K.dtype == Q.dtype and V.dtype == Q.dtype and O.dtype == Q.dtype, "dtypes must match")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _load().attn_fwd_variant(Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(),
                                 LSE.data_ptr(), B, Hq, K.shape[1], N, d, int(bool(causal)),
                                 int(window), float(softcap), float(scale), dt,
                                 _stream_ptr(Q, stream))
    _check("attn_fwd_variant", code)


def attn_decode_paged_workspace_bytes(B, Hq, d, page_size, max_pages_per_seq,
                                      split_tokens) -> int:
    return int(_load().attn_decode_paged_workspace_bytes(B, Hq, d, page_size, max_pages_per_seq,
                                                      split_tokens))


def attn_decode_paged(q, k_pages, v_pages, block_table, ctx_lens, O, LSE, split_tokens: int,
                      workspace, scale: float | None = None, stream=None) -> None:
    """O (and LSE unless None) <- paged split-KV decode.  q,O [B,Hq,d]; pages
    [num_pages,page,Hkv,d]; block_table int32 [B,max_pages]; ctx_lens int32 [B];
    workspace: a device buffer of at least attn_decode_paged_workspace_bytes(...) bytes,
    zero-filled once after allocation (torch.zeros) and used by one call at a time."""
    import torch
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages),
                    ("block_table", block_table), ("ctx_lens", ctx_lens), ("O", O),
                    ("workspace", workspace)):
        _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
    _need(q.dim() == 3 and O.shape == q.shape, "q,O must be [B,Hq,d]")
    B, Hq, d = q.shape
    _need(k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "pages must be [P,page,Hkv,d]")
    _, page, Hkv, d2 = k_pages.shape
    _need(d2 == d, "page head dim must match q")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B,
          "block_table must be int32 [B,max_pages]")
    _need(ctx_lens.dtype == torch.int32 and tuple(ctx_lens.shape) == (B,), "ctx_lens must be int32 [B]")
    if LSE is not None:
        _need(LSE.is_cuda and LSE.is_contiguous() and LSE.dtype == torch.float32 and
              tuple(LSE.shape) == (B, Hq), "LSE must be fp32 [B,Hq]")
    dt = _dtype_code(q)
    _need(k_pages.dtype == q.dtype and v_pages.dtype == q.dtype and O.dtype == q.dtype,
          "dtypes must match")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = workspace.numel() * workspace.element_size()
    code = _load().attn_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                  block_table.data_ptr(), ctx_lens.data_ptr(), O.data_ptr(),
                                  None if LSE is None else LSE.data_ptr(), B, Hq, Hkv, d, page,
                                  block_table.shape[1], int(split_tokens), float(scale), dt,
                                  workspace.data_ptr(), ws_bytes, _stream_ptr(q, stream))
    _check("attn_decode_paged", code)


def attn_decode_paged_noalloc(q, k_pages, v_pages, block_table, ctx_lens, O, LSE,
                              split_tokens: int, scale: float | None = None, stream=None) -> None:
    """attn_decode_paged without a workspace: the library's fixed per-GPU scratch holds the
    partial states (for callers that cannot allocate).  Calls that overlap on one GPU race;
    a call whose partial states exceed the scratch raises AttnError (ATTN_ERR_TOO_LARGE)."""
    import torch
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages),
                    ("block_table", block_table), ("ctx_lens", ctx_lens), ("O", O)):
        _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
    _need(q.dim() == 3 and O.shape == q.shape, "q,O must be [B,Hq,d]")
    B, Hq, d = q.shape
    _need(k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "pages must be [P,page,Hkv,d]")
    _, page, Hkv, d2 = k_pages.shape
    _need(d2 == d, "page head dim must match q")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B,
          "block_table must be int32 [B,max_pages]")
    _need(ctx_lens.dtype == torch.int32 and tuple(ctx_lens.shape) == (B,), "ctx_lens must be int32 [B]")
    if LSE is not None:
        _need(LSE.is_cuda and LSE.is_contiguous() and LSE.dtype == torch.float32 and
              tuple(LSE.shape) == (B, Hq), "LSE must be fp32 [B,Hq]")
    dt = _dtype_code(q)
    _need(k_pages.dtype == q.dtype and v_pages.dtype == q.dtype and O.dtype == q.dtype,
          "dtypes must match")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _load().attn_decode_paged_noalloc(
        q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
        ctx_lens.data_ptr(), O.data_ptr(), None if LSE is None else LSE.data_ptr(), B, Hq, Hkv,
        d, page, block_table.shape[1], int(split_tokens), float(scale), dt,
        _stream_ptr(q, stream))
    _check("attn_decode_paged_noalloc", code)


def attn_decode_cascade_workspace_bytes(B, Hq, d, page_size, max_pages_per_seq, split_tokens,
                                        prefix_len) -> int:
    return int(_load().attn_decode_cascade_workspace_bytes(B, Hq, d, page_size, max_pages_per_seq,
                                                        split_tokens, prefix_len))


def attn_decode_cascade(q, k_prefix, v_prefix, k_pages, v_pages, block_table, ctx_lens, O, LSE,
                        split_tokens: int, workspace, scale: float | None = None,
                        stream=None) -> None:
    """O (and LSE unless None) <- decode over the shared prefix k/v_prefix [Hkv, P, d]
    followed by each request's own paged tokens (as attn_decode_paged)."""
    import torch
    for name, t in (("q", q), ("k_prefix", k_prefix), ("v_prefix", v_prefix),
                    ("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
                    ("ctx_lens", ctx_lens), ("O", O), ("workspace", workspace)):
        _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
    _need(q.dim() == 3 and O.shape == q.shape, "q,O must be [B,Hq,d]")
    B, Hq, d = q.shape
    _need(k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "pages must be [P,page,Hkv,d]")
    _, page, Hkv, d2 = k_pages.shape
    _need(d2 == d, "page head dim must match q")
    _need(k_prefix.dim() == 3 and v_prefix.shape == k_prefix.shape and k_prefix.shape[0] == Hkv
          and k_prefix.shape[2] == d, "prefix must be [Hkv, P, d]")
    P = k_prefix.shape[1]
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B,
          "block_table must be int32 [B,max_pages]")
    _need(ctx_lens.dtype == torch.int32 and tuple(ctx_lens.shape) == (B,), "ctx_lens must be int32 [B]")
    if LSE is not None:
        _need(LSE.is_cuda and LSE.is_contiguous() and LSE.dtype == torch.float32 and
              tuple(LSE.shape) == (B, Hq), "LSE must be fp32 [B,Hq]")
    dt = _dtype_code(q)
    _need(all(t.dtype == q.dtype for t in (k_pages, v_pages, k_prefix, v_prefix, O)),
          "dtypes must match")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = workspace.numel() * workspace.element_size()
    code = _load().attn_decode_cascade(q.data_ptr(), k_prefix.data_ptr() if P else None,
                                    v_prefix.data_ptr() if P else None, P, k_pages.data_ptr(),
                                    v_pages.data_ptr(), block_table.data_ptr(),
                                    ctx_lens.data_ptr(), O.data_ptr(),
                                    None if LSE is None else LSE.data_ptr(), B, Hq, Hkv, d, page,
                                    block_table.shape[1], int(split_tokens), float(scale), dt,
                                    workspace.data_ptr(), ws_bytes, _stream_ptr(q, stream))
    _check("attn_decode_cascade", code)



def attn_prefill_paged(q, k_pages, v_pages, block_table, cu_seqlens_q, kv_lens, O, LSE,
                       max_q_len: int, causal: bool = True, scale: float | None = None,
                       stream=None) -> None:
    """O (and LSE unless None) <- prefill of each request's new tokens (rows
    cu_seqlens_q[r] .. cu_seqlens_q[r+1]-1 of q [total_q, Hq, d]) over its paged cache of
    kv_lens[r] tokens, the new ones last.  max_q_len bounds every request's q_len."""
    import torch
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages),
                    ("block_table", block_table), ("cu_seqlens_q", cu_seqlens_q),
                    ("kv_lens", kv_lens), ("O", O)):
        _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
    _need(q.dim() == 3 and O.shape == q.shape, "q,O must be [total_q,Hq,d]")
    total_q, Hq, d = q.shape
    _need(k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "pages must be [P,page,Hkv,d]")
    _, page, Hkv, d2 = k_pages.shape
    _need(d2 == d, "page head dim must match q")
    _need(kv_lens.dtype == torch.int32 and kv_lens.dim() == 1, "kv_lens must be int32 [B]")
    B = kv_lens.shape[0]
    _need(cu_seqlens_q.dtype == torch.int32 and tuple(cu_seqlens_q.shape) == (B + 1,),
          "cu_seqlens_q must be int32 [B+1]")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B,
          "block_table must be int32 [B,max_pages]")
    if LSE is not None:
        _need(LSE.is_cuda and LSE.is_contiguous() and LSE.dtype == torch.float32 and
              tuple(LSE.shape) == (total_q, Hq), "LSE must be fp32 [total_q,Hq]")
    dt = _dtype_code(q)
    _need(all(t.dtype == q.dtype for t in (k_pages, v_pages, O)), "dtypes must match")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _load().attn_prefill_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                   block_table.data_ptr(), cu_seqlens_q.data_ptr(),
                                   kv_lens.data_ptr(), O.data_ptr(),
                                   None if LSE is None else LSE.data_ptr(), B, Hq, Hkv, d, page,
                                   block_table.shape[1], int(max_q_len), int(bool(causal)),
                                   float(scale), dt, _stream_ptr(q, stream))
    _check("attn_prefill_paged", code)
