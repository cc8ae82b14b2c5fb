"""GPU parity of attn_prefill_paged (chunked / varlen prefill over a paged KV cache) against
the fp64 oracle, through the C ABI binding.

Covered: GQA and MHA, both dtypes and head sizes, causal and not; requests with no new
token, a single new token (a decode step), a whole prompt (q_len = kv_len), a cache shorter
than its chunk (queries that see no key), chunks spanning several tiles with ragged tails;
bit-exact paging and masking (identity against shuffled block table, NaN poison in every
slot the cache does not use and in a guard page before the pool, zero queries counting
their visible keys exactly); a whole prompt equal bit for bit to attn_fwd; padding rows
left untouched; determinism; the full-size chunked-prefill workload on four rows of every
work item (request, kv head, 128-row tile), with every output row checked as written.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from attn_inputs import (BF16, FP16, PAGED_PREFILL_WORKLOADS, paged_prefill_case,
                         paged_prefill_workload)
from tests.gpu_util import assert_parity, bits_of, from_dev_f64, tdtype, to_dev

pytestmark = pytest.mark.gpu

NAN16 = {BF16: 0x7FC0, FP16: 0x7E00}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_paged(case, k_pages=None, v_pages=None, table=None, q=None, want_lse=True, O=None):
    import exact_attention_08_amd as attn
    qd = to_dev(case.q if q is None else q, case.dtype)
    K = k_pages if k_pages is not None else to_dev(case.k_pages, case.dtype)
    V = v_pages if v_pages is not None else to_dev(case.v_pages, case.dtype)
    bt = torch.from_numpy(case.block_table if table is None else table).cuda()
    cu = torch.from_numpy(case.cu_seqlens_q).cuda()
    kvl = torch.from_numpy(case.kv_lens).cuda()
    if O is None:
        # NaN until written: a row that should be computed and is not fails every check
        O = torch.full_like(qd, float("nan"))
    L = torch.full((case.total_q, case.Hq), 7.0, dtype=torch.float32, device="cuda") \
        if want_lse else None
    attn.attn_prefill_paged(qd, K, V, bt, cu, kvl, O, L, case.max_q_len, case.causal,
                            case.scale)
    torch.cuda.synchronize()
    return O, L


def oracle_paged(case, rows=None, q=None):
    return oracle.prefill_paged(case.q if q is None else q, case.k_pages, case.v_pages,
                                case.block_table, case.cu_seqlens_q, case.kv_lens, case.causal,
                                case.scale, case.dtype, rows=rows)


def check(case, O, L, O_ref, L_ref, what):
    O = from_dev_f64(O).reshape(O_ref.shape)
    L = L.cpu().numpy().astype(np.float64).reshape(L_ref.shape)
    empty = np.isneginf(L_ref)
    # a query that sees no key: O = 0 and LSE = -inf exactly
    assert np.all(np.isneginf(L[empty])), f"{what}: LSE of key-less rows"
    assert np.all(O[empty] == 0.0), f"{what}: O of key-less rows"
    assert_parity(O[~empty], O_ref[~empty], L[~empty], L_ref[~empty], what)


CASES = [
    # Hq, Hkv, d, dtype, causal, q_lens, kv_lens
    (32, 8, 128, BF16, True, [512, 1, 0, 77, 300], [4096, 1000, 50, 77, 301]),
    (32, 8, 128, FP16, True, [129, 33, 16], [129, 2000, 15]),          # last: cache < chunk
    (8, 8, 64, BF16, True, [200, 64, 5], [700, 64, 1029]),
    (16, 1, 128, BF16, True, [40, 9, 1], [40, 3000, 17]),
    (12, 4, 64, FP16, False, [100, 31, 1, 0], [2000, 31, 300, 9]),
    (32, 8, 128, BF16, False, [257, 2], [1100, 4]),
    (4, 2, 128, BF16, True, [1000], [1000]),
    (64, 8, 64, BF16, True, [17, 300], [5000, 333]),                    # G = 8
]


@pytest.mark.parametrize("Hq,Hkv,d,dtype,causal,q_lens,kv_lens", CASES)
def test_paged_prefill_small_all_rows(Hq, Hkv, d, dtype, causal, q_lens, kv_lens):
    say(f"paged prefill Hq{Hq} Hkv{Hkv} d{d} dtype{dtype} causal{causal} q{q_lens} kv{kv_lens}")
    case = paged_prefill_case(Hq, Hkv, d, q_lens, kv_lens, 16, dtype, causal)
    O, L = run_paged(case)
    O_ref, L_ref = oracle_paged(case)
    check(case, O, L, O_ref, L_ref, "paged prefill")


def test_paged_prefill_paging_and_masking_are_bit_exact():
    say("paged prefill: shuffled vs identity table, NaN poison, guard page")
    dt = BF16
    q_lens, kv_lens = [70, 1, 130, 9], [70, 517, 1000, 33]
    case = paged_prefill_case(32, 8, 128, q_lens, kv_lens, 16, dt, True, seeds=(31, 32, 33))
    O, L = run_paged(case)
    # the same cache stored under the identity table
    npg = case.num_pages
    ident = np.full_like(case.block_table, -1)
    kp = np.empty_like(case.k_pages)
    vp = np.empty_like(case.v_pages)
    nxt = 0
    for r in range(case.B):
        n = (int(case.kv_lens[r]) + 15) // 16
        ident[r, :n] = np.arange(nxt, nxt + n)
        kp[nxt:nxt + n] = case.k_pages[case.block_table[r, :n]]
        vp[nxt:nxt + n] = case.v_pages[case.block_table[r, :n]]
        nxt += n
    assert nxt == npg
    O2, L2 = run_paged(case, to_dev(kp, dt), to_dev(vp, dt), ident)
    assert torch.equal(O, O2) and torch.equal(L, L2)
    # NaN in every slot past a cache's end, in 3 unreferenced pages after the pool and in a
    # guard page just before it; the table shifts by one page
    big_k = np.full((npg + 4,) + case.k_pages.shape[1:], NAN16[dt], np.uint16)
    big_v = big_k.copy()
    big_k[1:npg + 1] = case.k_pages[:npg]
    big_v[1:npg + 1] = case.v_pages[:npg]
    for r in range(case.B):
        kl = int(case.kv_lens[r])
        if kl % 16:
            last = case.block_table[r, kl // 16] + 1
            big_k[last, kl % 16:] = NAN16[dt]
            big_v[last, kl % 16:] = NAN16[dt]
    dk, dv = to_dev(big_k, dt), to_dev(big_v, dt)
    O3, L3 = run_paged(case, dk[1:], dv[1:])
    assert torch.isfinite(O3.float()).all()
    assert torch.equal(O, O3) and torch.equal(L, L3)


def test_paged_prefill_zero_queries_count_visible_keys():
    say("paged prefill: zero queries count their visible keys")
    q_lens, kv_lens = [300, 1, 47, 129], [1300, 64, 47, 4000]
    case = paged_prefill_case(32, 8, 128, q_lens, kv_lens, 16, BF16, True, seeds=(34, 35, 36))
    q0 = np.zeros_like(case.q)
    _, L = run_paged(case, q=q0)
    cnt = np.round(np.exp(L.cpu().numpy().astype(np.float64)))
    want = np.concatenate([kl - ql + np.arange(ql) + 1 for ql, kl in zip(q_lens, kv_lens)])
    assert np.array_equal(cnt, np.repeat(want[:, None].astype(float), 32, 1))


# N = 4160 at d = 128: attn_fwd runs the 64-rows-per-wave kernel there, the paged mode the
# 32-rows-per-wave one, so the two kernels must agree bit for bit
@pytest.mark.parametrize("d,dtype,N", [(128, BF16, 1000), (64, FP16, 1000), (128, BF16, 4160),
                                       (128, FP16, 4160)])
def test_whole_prompt_equals_attn_fwd_bitwise(d, dtype, N):
    say(f"paged prefill of a whole prompt vs attn_fwd d{d} N{N}")
    import exact_attention_08_amd as attn
    case = paged_prefill_case(32, 8, d, [N], [N], 16, dtype, True, seeds=(37, 38, 39))
    O, L = run_paged(case)
    toks = np.arange(N)
    pages = case.block_table[0, toks // 16]
    K = case.k_pages[pages, toks % 16].transpose(1, 0, 2)[None]      # [1, Hkv, N, d]
    V = case.v_pages[pages, toks % 16].transpose(1, 0, 2)[None]
    Q = case.q.transpose(1, 0, 2)[None]                               # [1, Hq, N, d]
    Qd, Kd, Vd = (to_dev(np.ascontiguousarray(x), dtype) for x in (Q, K, V))
    Od = torch.empty_like(Qd)
    Ld = torch.empty(1, 32, N, dtype=torch.float32, device="cuda")
    attn.attn_fwd(Qd, Kd, Vd, Od, Ld, True, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(O, Od[0].transpose(0, 1)) and torch.equal(L, Ld[0].transpose(0, 1))


def test_padding_rows_untouched_lse_optional_and_deterministic():
    say("paged prefill: padding rows, no LSE, determinism")
    case = paged_prefill_case(16, 4, 128, [33, 200], [500, 260], 16, FP16, True,
                              seeds=(40, 41, 42), pad_q=5)
    fill = torch.full((case.total_q, 16, 128), 3.0, dtype=tdtype(FP16), device="cuda")
    O, L = run_paged(case, O=fill.clone())
    assert torch.equal(O[-5:], fill[-5:]) and torch.all(L[-5:] == 7.0)
    O2, _ = run_paged(case, O=fill.clone(), want_lse=False)
    assert torch.equal(O, O2)
    O3, L3 = run_paged(case, O=fill.clone())
    assert torch.equal(O, O3) and torch.equal(L, L3)
    O_ref, L_ref = oracle_paged(case, rows=np.arange(233 * 16))
    check(case, O[:233].reshape(-1, 128), L[:233].reshape(-1), O_ref, L_ref, "padded")


def item_rows(case, seed):
    """Four rows of every work item (request, kv head, 128-row tile of its G query heads x
    new tokens): the tile's first row, a random row in each of the second and third 32-row
    waves and the tile's last row, clipped to the request's rows.  A row t of a tile is new
    token t / G of the request and query head kvh * G + t % G; returned as flat indices
    token * Hq + head of O [total_q, Hq]."""
    rng = np.random.default_rng(seed)
    G = case.Hq // case.Hkv
    rows = []
    for r in range(case.B):
        a, b = int(case.cu_seqlens_q[r]), int(case.cu_seqlens_q[r + 1])
        n_rows = (b - a) * G
        for kvh in range(case.Hkv):
            for t0 in range(0, n_rows, 128):
                picks = {t0, t0 + 32 + int(rng.integers(0, 32)), t0 + 64 + int(rng.integers(0, 32)),
                         t0 + 127}
                for t in sorted(min(p, n_rows - 1) for p in picks):
                    rows.append((a + t // G) * case.Hq + kvh * G + t % G)
    return np.array(sorted(set(rows)), np.int64)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", sorted(PAGED_PREFILL_WORKLOADS))
def test_paged_prefill_named_workload_full_size_every_item(name):
    say(f"paged prefill full size {name}: rows of every work item")
    case = paged_prefill_workload(name)
    O, L = run_paged(case)
    # every row of every request was written (O started as NaN, LSE as 7.0)
    assert torch.isfinite(O.float()).all() and torch.isfinite(L).all()
    rows = item_rows(case, 43)
    say(f"  oracle over {len(rows)} rows")
    O_ref, L_ref = oracle_paged(case, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    check(case, O.view(-1, case.d)[idx], L.view(-1)[idx], O_ref, L_ref, name)
