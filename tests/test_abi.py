"""CPU-only checks of the C ABI: the library loads, exports every symbol include/attn.h
declares, and rejects bad arguments on the host with the documented status codes before
any HIP call (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

attn = pytest.importorskip("exact_attention_08_amd")
L = attn.lib()

A = 0x10000          # a 16-byte aligned fake device address; never dereferenced here
MIS = 0x10008        # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|size_t)\s+(attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_calls_and_the_helpers():
    assert declared_functions() == sorted(attn.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", attn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def status_codes():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(ATTN_\w+)\s*=\s*(-?\d+)", text)}


def test_status_codes_match_binding():
    codes = status_codes()
    for code, name in attn.STATUS.items():
        assert codes[name] == code


def fwd(Q=A, K=A, V=A, O=A, LSE=A, B=1, Hq=4, Hkv=2, N=16, d=64, causal=1, scale=0.125,
        dtype=0):
    return L.attn_fwd(Q, K, V, O, LSE, B, Hq, Hkv, N, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), -1), (dict(K=None), -1), (dict(V=None), -1), (dict(O=None), -1),
    (dict(LSE=None), -1),
    (dict(B=0), -2), (dict(Hq=0), -2), (dict(Hkv=0), -2), (dict(N=0), -2), (dict(d=0), -2),
    (dict(Hq=6, Hkv=4), -2), (dict(N=-5), -2), (dict(scale=0.0), -2), (dict(scale=-1.0), -2),
    (dict(scale=float("nan")), -2), (dict(scale=float("inf")), -2),
    (dict(dtype=2), -3), (dict(dtype=-1), -3),
    (dict(d=96), -4), (dict(d=256), -4), (dict(d=32), -4),
    (dict(Q=MIS), -5), (dict(O=MIS), -5), (dict(LSE=A + 4), -5),
])
def test_attn_fwd_rejects_bad_arguments(kw, code):
    assert fwd(**kw) == code


def dec(q=A, K=A, V=A, bt=A, ctx=A, O=A, LSE=A, B=2, Hq=8, Hkv=2, d=128, page=16, max_pages=8,
        split=64, scale=0.1, dtype=0, ws=A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.attn_decode_paged_workspace_bytes(B, Hq, d, 16, max_pages, max(split, 16))
    return L.attn_decode_paged(q, K, V, bt, ctx, O, LSE, B, Hq, Hkv, d, page, max_pages, split,
                               scale, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(K=None), -1), (dict(V=None), -1), (dict(bt=None), -1),
    (dict(ctx=None), -1), (dict(O=None), -1),
    (dict(B=0), -2), (dict(Hq=7), -2), (dict(max_pages=0), -2), (dict(split=-16), -2),
    (dict(scale=0.0), -2), (dict(page=0), -2),
    (dict(dtype=5), -3),
    (dict(d=80), -4), (dict(page=32), -4), (dict(page=8), -4), (dict(split=24), -4),
    (dict(Hq=64, Hkv=2), -4),
    (dict(q=MIS), -5), (dict(K=MIS), -5), (dict(O=MIS), -5), (dict(bt=A + 2), -5),
    (dict(LSE=A + 2), -5), (dict(ws=MIS), -5),
    (dict(ws=None), -6), (dict(ws_bytes=100), -6),
])
def test_attn_decode_paged_rejects_bad_arguments(kw, code):
    assert dec(**kw) == code


def test_workspace_helper():
    ws = L.attn_decode_paged_workspace_bytes
    # C5-like: 64 sequences x 32 heads, up to 2048 pages of 16 tokens, 1024-token splits
    S = (2048 * 16 + 1023) // 1024
    o = 64 * 32 * S * 128 * 4
    l = 64 * 32 * S * 4
    # the 256-byte control block, the partial states, then their LSEs padded to 256 bytes
    assert ws(64, 32, 128, 16, 2048, 1024) == 256 + o + ((l + 255) // 256) * 256
    assert ws(0, 32, 128, 16, 2048, 1024) == 0
    assert ws(1, 1, 64, 16, 1, 16) >= 64 * 4 + 4


def casc(q=A, Kp=A, Vp=A, P=100, K=A, V=A, bt=A, ctx=A, O=A, LSE=A, B=2, Hq=8, Hkv=2, d=128,
         page=16, max_pages=8, split=64, scale=0.1, dtype=0, ws=A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.attn_decode_cascade_workspace_bytes(B, Hq, d, 16, max_pages, max(split, 16),
                                                         max(P, 0))
    return L.attn_decode_cascade(q, Kp, Vp, P, K, V, bt, ctx, O, LSE, B, Hq, Hkv, d, page,
                                 max_pages, split, scale, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(K=None), -1), (dict(bt=None), -1), (dict(O=None), -1),
    (dict(Kp=None), -1), (dict(Vp=None), -1),
    (dict(P=-1), -2), (dict(B=0), -2), (dict(Hq=7), -2), (dict(split=-16), -2),
    (dict(scale=0.0), -2), (dict(P=(1 << 22) + 1), -2),
    (dict(dtype=5), -3),
    (dict(d=80), -4), (dict(page=32), -4), (dict(split=24), -4), (dict(Hq=64, Hkv=2), -4),
    (dict(q=MIS), -5), (dict(Kp=MIS), -5), (dict(Vp=MIS), -5), (dict(O=MIS), -5),
    (dict(ws=MIS), -5),
    (dict(ws=None), -6), (dict(ws_bytes=100), -6),
])
def test_attn_decode_cascade_rejects_bad_arguments(kw, code):
    assert casc(**kw) == code


def test_cascade_workspace_helper_adds_the_prefix_chunks():
    paged = L.attn_decode_paged_workspace_bytes
    cw = L.attn_decode_cascade_workspace_bytes
    # no prefix: the same workspace as the paged call
    assert cw(64, 32, 128, 16, 2048, 1024, 0) == paged(64, 32, 128, 16, 2048, 1024)
    # a prefix of 4097 tokens adds 9 partial states (chunks of 512 keys) per (request, head)
    S = (2048 * 16 + 1023) // 1024 + 9
    o = 64 * 32 * S * 128 * 4
    l = 64 * 32 * S * 4
    assert cw(64, 32, 128, 16, 2048, 1024, 4097) == 256 + o + ((l + 255) // 256) * 256
    assert cw(64, 32, 128, 16, 2048, 1024, -1) == 0



def ppre(q=A, K=A, V=A, bt=A, cu=A, kvl=A, O=A, LSE=A, B=2, Hq=8, Hkv=2, d=128, page=16,
         max_pages=8, max_q=64, causal=1, scale=0.1, dtype=0):
    return L.attn_prefill_paged(q, K, V, bt, cu, kvl, O, LSE, B, Hq, Hkv, d, page, max_pages,
                                max_q, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(K=None), -1), (dict(V=None), -1), (dict(bt=None), -1),
    (dict(cu=None), -1), (dict(kvl=None), -1), (dict(O=None), -1),
    (dict(B=0), -2), (dict(Hq=7), -2), (dict(max_q=-1), -2), (dict(max_pages=0), -2),
    (dict(scale=0.0), -2), (dict(scale=float("nan")), -2), (dict(max_q=(1 << 19) + 1), -2),
    (dict(dtype=5), -3),
    (dict(d=80), -4), (dict(page=32), -4),
    (dict(q=MIS), -5), (dict(K=MIS), -5), (dict(V=MIS), -5), (dict(O=MIS), -5),
    (dict(LSE=MIS + 1), -5),
])
def test_attn_prefill_paged_rejects_bad_arguments(kw, code):
    assert ppre(**kw) == code


def test_attn_prefill_paged_without_new_tokens_launches_nothing():
    # max_q_len = 0 is valid and returns before any HIP call (this host has no GPU)
    assert ppre(max_q=0) == 0
    assert ppre(max_q=0, LSE=None) == 0


def test_balanced_split_workspace_is_sized_for_the_shortest_split():
    ws = L.attn_decode_paged_workspace_bytes
    assert ws(64, 32, 128, 16, 2048, 0) == ws(64, 32, 128, 16, 2048, 256)
    assert ws(64, 32, 128, 16, 2048, -16) == 0
    cw = L.attn_decode_cascade_workspace_bytes
    assert cw(8, 32, 128, 16, 100, 0, 1000) == cw(8, 32, 128, 16, 100, 256, 1000)
    # a workspace sized for 1024-token splits is too small for the balanced choice
    small = ws(2, 8, 128, 16, 64, 1024)
    assert small < ws(2, 8, 128, 16, 64, 0)
    assert dec(split=0, max_pages=64, ws_bytes=small) == -6


def fvar(Q=A, K=A, V=A, O=A, LSE=A, B=2, Hq=8, Hkv=2, N=100, d=128, causal=1, window=16,
         softcap=30.0, scale=0.1, dtype=0):
    return L.attn_fwd_variant(Q, K, V, O, LSE, B, Hq, Hkv, N, d, causal, window, softcap,
                              scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), -1), (dict(LSE=None), -1),
    (dict(B=0), -2), (dict(Hq=7), -2), (dict(window=-1), -2), (dict(softcap=-1.0), -2),
    (dict(softcap=float("inf")), -2), (dict(scale=0.0), -2),
    (dict(dtype=4), -3),
    (dict(d=96), -4), (dict(causal=0), -4),
    (dict(Q=MIS), -5), (dict(O=MIS), -5),
])
def test_attn_fwd_variant_rejects_bad_arguments(kw, code):
    assert fvar(**kw) == code


def noalloc(q=A, K=A, V=A, bt=A, ctx=A, O=A, LSE=A, B=2, Hq=8, Hkv=2, d=128, page=16,
            max_pages=8, split=64, scale=0.1, dtype=0):
    return L.attn_decode_paged_noalloc(q, K, V, bt, ctx, O, LSE, B, Hq, Hkv, d, page, max_pages,
                                       split, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(ctx=None), -1), (dict(O=None), -1),
    (dict(B=0), -2), (dict(Hq=7), -2), (dict(split=-16), -2), (dict(scale=0.0), -2),
    (dict(dtype=5), -3),
    (dict(d=80), -4), (dict(page=32), -4), (dict(split=24), -4),
    (dict(q=MIS), -5), (dict(bt=A + 2), -5),
    # partial states beyond the fixed scratch: rejected before any HIP call
    (dict(B=64, Hq=32, max_pages=2048, split=0), -8),
    (dict(B=1, Hq=16, max_pages=65536, split=16), -2),
])
def test_attn_decode_paged_noalloc_rejects_bad_arguments(kw, code):
    assert noalloc(**kw) == code


def test_noalloc_scratch_limit_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    cap = int(m.group(1)) << int(m.group(2))
    ws = L.attn_decode_paged_workspace_bytes
    # the 64-sequence decode batch with 1024-token splits fits; with the balanced split not
    assert ws(64, 32, 128, 16, 2048, 1024) <= cap < ws(64, 32, 128, 16, 2048, 0)
