"""Seeded synthetic inputs for exact attention, shared by the fp64 oracle and the GPU path.

This module only *makes data*: it draws i.i.d. N(0,1) samples, rounds them to the 16-bit
storage type, and lays out paged KV pools with a shuffled block table.  It performs none of
the attention arithmetic; both the oracle and the HIP library receive exactly the 16-bit
patterns produced here.

Workload shapes follow the pages' examples:
  * dense layouts [B, H, N, d] (teaching kernel layout in the AI-infra handbook chapter
    "FlashAttention and inference operators"; the PyTorch example in the zwjcode.cn blog
    "FlashAttention tiling, online softmax and IO", section 05);
  * paged pools [num_pages, page, Hkv, d] with a block table [B, max_pages] whose unused
    entries are -1 and whose physical pages are a seeded shuffle (the paged decode test
    program of the same handbook chapter; LLM Internals section 10.3.7 for the
    `block_table` / `k_cache` shapes).
Seeds follow the handbook's test programs: Q=1, K=2, V=3, page shuffle=7; context
lengths use seed 5.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16 = 0
FP16 = 1
DTYPE_NAMES = {BF16: "bf16", FP16: "fp16"}

SEED_Q, SEED_K, SEED_V, SEED_CTX, SEED_PERM = 1, 2, 3, 5, 7


# ----------------------------------------------------------------------------- 16-bit codecs
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 with round-to-nearest-even; returns the uint16 patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bits_to_f64(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Widen 16-bit patterns to float64 exactly (numpy's own conversions)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == FP16:
        return bits.view(np.float16).astype(np.float64)
    raise ValueError(f"unknown dtype code {dtype}")


def normal_bits(shape, seed: int, dtype: int) -> np.ndarray:
    """i.i.d. N(0,1) in float32 from numpy's PCG64 stream `seed`, rounded (RNE) to 16 bits."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=int(np.prod(shape)), dtype=np.float32)
    if dtype == BF16:
        b = f32_to_bf16_bits(x)
    elif dtype == FP16:
        b = x.astype(np.float16).view(np.uint16)
    else:
        raise ValueError(f"unknown dtype code {dtype}")
    return b.reshape(shape)


# ----------------------------------------------------------------------------- prefill
@dataclass
class PrefillCase:
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    dtype: int
    scale: float
    q: np.ndarray  # uint16 [B, Hq, N, d]
    k: np.ndarray  # uint16 [B, Hkv, N, d]
    v: np.ndarray  # uint16 [B, Hkv, N, d]


def prefill_case(B, Hq, Hkv, N, d, causal, dtype=BF16, scale=None,
                 seeds=(SEED_Q, SEED_K, SEED_V)) -> PrefillCase:
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q = normal_bits((B, Hq, N, d), seeds[0], dtype)
    k = normal_bits((B, Hkv, N, d), seeds[1], dtype)
    v = normal_bits((B, Hkv, N, d), seeds[2], dtype)
    return PrefillCase(B, Hq, Hkv, N, d, bool(causal), dtype, float(scale), q, k, v)


# ----------------------------------------------------------------------------- paged decode
def log_uniform_ctx(B: int, lo: int, hi: int, seed: int = SEED_CTX) -> np.ndarray:
    """ctx = floor(exp(ln lo + u (ln hi - ln lo))), u ~ U[0,1) seeded, clipped to [lo, hi]."""
    u = np.random.default_rng(seed).random(B)
    ctx = np.floor(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))
    return np.clip(ctx, lo, hi).astype(np.int32)


def paged_layout(ctx_lens, page_size: int, seed: int = SEED_PERM, max_pages: int | None = None):
    """Block table for the given context lengths over a pool of exactly sum(ceil(ctx/page))
    physical pages, handed out in the order of a seeded random permutation; unused table
    entries are -1.  Returns (block_table int32 [B, max_pages], num_pages)."""
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    npages = (ctx_lens + page_size - 1) // page_size
    total = int(npages.sum())
    need = int(npages.max()) if len(npages) else 0
    if max_pages is None:
        max_pages = need
    if max_pages < need:
        raise ValueError("max_pages smaller than the longest context")
    perm = np.random.default_rng(seed).permutation(total).astype(np.int32)
    table = np.full((len(ctx_lens), max(max_pages, 1)), -1, dtype=np.int32)
    nxt = 0
    for r, n in enumerate(npages):
        table[r, :n] = perm[nxt:nxt + n]
        nxt += int(n)
    return table, total


@dataclass
class DecodeCase:
    B: int
    Hq: int
    Hkv: int
    d: int
    page_size: int
    dtype: int
    scale: float
    ctx_lens: np.ndarray     # int32 [B]
    block_table: np.ndarray  # int32 [B, max_pages]
    num_pages: int
    q: np.ndarray            # uint16 [B, Hq, d]
    k_pages: np.ndarray      # uint16 [num_pages, page, Hkv, d]
    v_pages: np.ndarray      # uint16 [num_pages, page, Hkv, d]
    extra: dict = field(default_factory=dict)

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]


def decode_case(B, Hq, Hkv, d, ctx_lens, page_size=16, dtype=BF16, scale=None,
                seeds=(SEED_Q, SEED_K, SEED_V), perm_seed=SEED_PERM, max_pages=None,
                identity_table=False) -> DecodeCase:
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    if identity_table:
        npages = (ctx_lens.astype(np.int64) + page_size - 1) // page_size
        mp = int(npages.max()) if max_pages is None else max_pages
        table = np.full((B, max(mp, 1)), -1, dtype=np.int32)
        nxt = 0
        for r, n in enumerate(npages):
            table[r, :n] = np.arange(nxt, nxt + n, dtype=np.int32)
            nxt += int(n)
        total = nxt
    else:
        table, total = paged_layout(ctx_lens, page_size, perm_seed, max_pages)
    q = normal_bits((B, Hq, d), seeds[0], dtype)
    kp = normal_bits((max(total, 1), page_size, Hkv, d), seeds[1], dtype)
    vp = normal_bits((max(total, 1), page_size, Hkv, d), seeds[2], dtype)
    return DecodeCase(B, Hq, Hkv, d, page_size, dtype, float(scale), ctx_lens, table, total,
                      q, kp, vp)


def permute_pages(case: DecodeCase, seed: int) -> DecodeCase:
    """Same logical KV, stored under a different physical page order (pure data movement)."""
    perm = np.random.default_rng(seed).permutation(case.num_pages).astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(case.num_pages, dtype=np.int32)
    kp = np.empty_like(case.k_pages)
    vp = np.empty_like(case.v_pages)
    kp[perm] = case.k_pages[: case.num_pages]
    vp[perm] = case.v_pages[: case.num_pages]
    table = case.block_table.copy()
    used = table >= 0
    table[used] = perm[table[used]]
    return DecodeCase(case.B, case.Hq, case.Hkv, case.d, case.page_size, case.dtype, case.scale,
                      case.ctx_lens.copy(), table, case.num_pages, case.q.copy(), kp, vp)


# ----------------------------------------------------------------------------- named workloads
# The five workloads this library is measured on; shapes from the GPT-2-medium and
# Llama-3-8B examples on the pages.
CONFIGS = {
    "single_head_n256_d64_fp16": dict(kind="prefill", B=1, Hq=1, Hkv=1, N=256, d=64,
                                      causal=False, dtype=FP16),
    "gpt2_medium_b64_h16_n1024_d64_causal": dict(kind="prefill", B=64, Hq=16, Hkv=16, N=1024,
                                                 d=64, causal=True, dtype=BF16),
    "llama3_8b_prefill_n8192_causal": dict(kind="prefill", B=1, Hq=32, Hkv=8, N=8192, d=128,
                                           causal=True, dtype=BF16),
    "llama3_8b_prefill_n32768_causal": dict(kind="prefill", B=1, Hq=32, Hkv=8, N=32768, d=128,
                                            causal=True, dtype=BF16),
    "paged_gqa_decode_b64_ctx512_32768": dict(kind="decode", B=64, Hq=32, Hkv=8, d=128,
                                              page_size=16, ctx_lo=512, ctx_hi=32768,
                                              split_tokens=1024, dtype=BF16),
}


def config_case(name: str):
    c = CONFIGS[name]
    if c["kind"] == "prefill":
        return prefill_case(c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["causal"], c["dtype"])
    ctx = log_uniform_ctx(c["B"], c["ctx_lo"], c["ctx_hi"])
    mp = (c["ctx_hi"] + c["page_size"] - 1) // c["page_size"]
    return decode_case(c["B"], c["Hq"], c["Hkv"], c["d"], ctx, c["page_size"], c["dtype"],
                       max_pages=mp)


# ----------------------------------------------------------------------------- shared prefix
SEED_PREFIX = 11    # prefix K; prefix V uses SEED_PREFIX + 1


def cascade_case(B, Hq, Hkv, d, prefix_len, own_ctx, page_size=16, dtype=BF16, scale=None,
                 seeds=(SEED_Q, SEED_K, SEED_V), prefix_seed=SEED_PREFIX, max_pages=None):
    """Requests sharing one prefix: a decode case for the requests' own tokens, plus the
    prefix K/V [Hkv, prefix_len, d] in case.extra["k_prefix"] / ["v_prefix"]."""
    case = decode_case(B, Hq, Hkv, d, own_ctx, page_size, dtype, scale, seeds, max_pages=max_pages)
    case.extra["k_prefix"] = normal_bits((Hkv, prefix_len, d), prefix_seed, dtype)
    case.extra["v_prefix"] = normal_bits((Hkv, prefix_len, d), prefix_seed + 1, dtype)
    return case


# The shared-prefix workload: Llama-3-8B decode shapes, 64 requests forked from one
# 8192-token prefix (a shared document or system prompt, the pages' motivating case), each
# with its own log-uniform tail of 128-4096 tokens.
CASCADE_WORKLOADS = {
    "cascade_gqa_decode_b64_prefix8192_own128_4096": dict(
        B=64, Hq=32, Hkv=8, d=128, page_size=16, prefix_len=8192, own_lo=128, own_hi=4096,
        split_tokens=1024, dtype=BF16),
}


def cascade_workload(name: str):
    c = CASCADE_WORKLOADS[name]
    own = log_uniform_ctx(c["B"], c["own_lo"], c["own_hi"])
    mp = (c["own_hi"] + c["page_size"] - 1) // c["page_size"]
    return cascade_case(c["B"], c["Hq"], c["Hkv"], c["d"], c["prefix_len"], own,
                        c["page_size"], c["dtype"], max_pages=mp)



# ----------------------------------------------------------------------------- paged / varlen prefill
@dataclass
class PagedPrefillCase:
    Hq: int
    Hkv: int
    d: int
    page_size: int
    dtype: int
    scale: float
    causal: bool
    q_lens: np.ndarray       # int32 [B] new tokens per request
    kv_lens: np.ndarray      # int32 [B] cached tokens per request, the new ones included
    cu_seqlens_q: np.ndarray  # int32 [B + 1]
    block_table: np.ndarray  # int32 [B, max_pages]
    num_pages: int
    q: np.ndarray            # uint16 [total_q, Hq, d]
    k_pages: np.ndarray      # uint16 [num_pages, page, Hkv, d]
    v_pages: np.ndarray

    @property
    def B(self) -> int:
        return len(self.kv_lens)

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if len(self.q_lens) else 0


def cu_seqlens(lengths) -> np.ndarray:
    """Packed-sequence offsets [0, l0, l0+l1, ...] (int32, length B + 1)."""
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


def paged_prefill_case(Hq, Hkv, d, q_lens, kv_lens, page_size=16, dtype=BF16, causal=True,
                       scale=None, seeds=(SEED_Q, SEED_K, SEED_V), perm_seed=SEED_PERM,
                       max_pages=None, pad_q=0) -> PagedPrefillCase:
    """New queries of several requests packed end to end ([total_q, Hq, d], total_q =
    sum(q_lens) + pad_q padding rows), over paged caches of kv_lens tokens each."""
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    table, total = paged_layout(kv_lens, page_size, perm_seed, max_pages)
    cu = cu_seqlens(q_lens)
    q = normal_bits((int(cu[-1]) + pad_q, Hq, d), seeds[0], dtype)
    kp = normal_bits((max(total, 1), page_size, Hkv, d), seeds[1], dtype)
    vp = normal_bits((max(total, 1), page_size, Hkv, d), seeds[2], dtype)
    return PagedPrefillCase(Hq, Hkv, d, page_size, dtype, float(scale), bool(causal), q_lens,
                            kv_lens, cu, table, total, q, kp, vp)


SEED_QLEN = 6

# Chunked prefill at Llama-3-8B shapes: 16 requests, each appending a chunk of new tokens
# (log-uniform 256-2048, seed 6) to a cached history (log-uniform 1024-16384 tokens, seed 5),
# the situation of incremental prefill and multi-turn chat on the pages.
PAGED_PREFILL_WORKLOADS = {
    "chunked_prefill_b16_hist1024_16384_chunk256_2048": dict(
        B=16, Hq=32, Hkv=8, d=128, page_size=16, hist_lo=1024, hist_hi=16384, q_lo=256,
        q_hi=2048, dtype=BF16),
}


def paged_prefill_workload(name: str) -> PagedPrefillCase:
    c = PAGED_PREFILL_WORKLOADS[name]
    hist = log_uniform_ctx(c["B"], c["hist_lo"], c["hist_hi"])
    qn = log_uniform_ctx(c["B"], c["q_lo"], c["q_hi"], seed=SEED_QLEN)
    return paged_prefill_case(c["Hq"], c["Hkv"], c["d"], qn, hist + qn, c["page_size"],
                              c["dtype"])
