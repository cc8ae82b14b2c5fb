"""Pins for the fp64 oracle: it is tied here to things other than itself.

* the pages' worked examples (tests/golden/*.json, each with its citation);
* closed forms (zero queries give uniform attention; a single visible key; constant V);
* library routines: torch's float64 CPU scaled_dot_product_attention (math path, with its
  own causal mask, scale and GQA expansion), scipy's softmax / logsumexp, numpy's 16-bit
  conversions;
* invariants the pages state: tiled equals untiled, the merge is order-free, paged equals
  contiguous exactly, rows of P sum to 1.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import torch
import torch.nn.functional as F

import oracle
from attn_inputs import (BF16, FP16, bits_to_f64, decode_case, f32_to_bf16_bits, normal_bits,
                         paged_prefill_case, permute_pages, prefill_case)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def half_ulp(printed: str) -> float:
    """Half a unit in the last printed digit."""
    s = str(printed)
    dec = len(s.split(".")[1]) if "." in s else 0
    return 0.5 * 10.0 ** (-dec)


def close_printed(value, printed, tol=None):
    t = half_ulp(printed) if tol is None else tol
    assert abs(value - float(printed)) <= t + 1e-12, (value, printed, t)


def bf16(vals):
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def scores_as_attention(scores, values, causal=False):
    """A one-dimensional attention problem whose every row has the given scores:
    d = 1, q = 1, k_j = score_j, v_j = value_j, scale = 1 (all exact in bf16)."""
    n = len(scores)
    q = bf16(np.ones(n)).reshape(1, 1, n, 1)
    k = bf16(scores).reshape(1, 1, n, 1)
    v = bf16(values).reshape(1, 1, n, 1)
    return q, k, v


# ----------------------------------------------------------------------------- 16-bit widening
@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_widen16_matches_numpy_for_every_pattern(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        ref = bits_to_f64(bits, dtype)
    got = np.array([oracle.widen16(int(b), dtype) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_single_visible_key_returns_v_bits_exactly():
    # O of a row with one visible key is that key's V row, widened exactly
    for dtype in (BF16, FP16):
        v = normal_bits((1, 1, 1, 64), 5, dtype)
        O, L = oracle.attention(np.zeros_like(v), np.zeros_like(v), v, causal=True, scale=1.0,
                                dtype=dtype)
        assert np.array_equal(O.reshape(-1), bits_to_f64(v.reshape(-1), dtype))
        assert L.reshape(-1)[0] == 0.0


# ----------------------------------------------------------------------------- worked examples
def test_three_scores_two_tiles_zwjcode_section04():
    g = gold("online_softmax_three_scores.json")
    r = oracle.online_row(g["scores"], g["values"], bc=2)
    for t, st in enumerate(g["after_tile"]):
        assert r["trace_m"][t] == st["m"]
        close_printed(r["trace_l"][t], st["l"])
        close_printed(r["trace_acc"][t, 0], st["acc"])
    close_printed(r["O"][0], g["output"])
    # the same numbers through the standard (untiled) oracle: every row of the 1-d problem
    q, k, v = scores_as_attention(g["scores"], g["values"])
    O, L = oracle.attention(q, k, v, causal=False, scale=1.0, dtype=BF16)
    for i in range(3):
        close_printed(O[0, 0, i, 0], g["output"])
        assert abs(O[0, 0, i, 0] - r["O"][0]) < 1e-12
        close_printed(math.exp(L[0, 0, i] - 3.0), g["after_tile"][-1]["l"])


def test_rechunk_lse_and_weights_llm_internals_10_3_2():
    g = gold("online_softmax_rechunk.json")
    for key in ("order_a", "order_b"):
        c = g[key]
        r = oracle.online_row(c["scores"], c["values"], bc=c["tile"])
        for t, st in enumerate(c["after_tile"]):
            assert r["trace_m"][t] == st["m"]
            close_printed(r["trace_l"][t], st["l"])
            close_printed(r["trace_acc"][t, 0], st["acc"])
        close_printed(r["O"][0], g["output"])
        close_printed(r["lse"], g["lse"])
    q, k, v = scores_as_attention(g["order_a"]["scores"], g["order_a"]["values"])
    O, L, P = oracle.attention(q, k, v, causal=False, scale=1.0, dtype=BF16, return_probs=True)
    close_printed(O[0, 0, 0, 0], g["output"])
    close_printed(L[0, 0, 0], g["lse"])
    for w, pw in zip(P[0, 0, 0], g["weights_for_scores_1_3_2"]):
        close_printed(w, pw)
    # LSE merge of the two chunks [1,3] and [2]: ln(e^L1 + e^L2), weights e^(Lk - L)
    a = oracle.online_row([1, 3], [10, 20], bc=2)
    b = oracle.online_row([2], [30], bc=1)
    Om, Lm = oracle.merge([a["O"], b["O"]], [a["lse"], b["lse"]])
    close_printed(Om[0], g["output"])
    close_printed(Lm, g["lse"])


def test_element_stream_cs349d_exercise1():
    g = gold("online_softmax_element_stream.json")
    r = oracle.online_row(g["scores"], np.zeros(3), bc=1)
    for t, st in enumerate(g["after_tile"]):
        assert r["trace_m"][t] == st["m"]
        close_printed(r["trace_l"][t], st["l"])
    close_printed(r["trace_l"][1] * math.exp(2 - 4), g["rescaled_l_before_last_add"])
    q, k, v = scores_as_attention(g["scores"], [0, 0, 0])
    O, L, P = oracle.attention(q, k, v, causal=False, scale=1.0, dtype=BF16, return_probs=True)
    for w, pw in zip(P[0, 0, 0], g["softmax"]):
        close_printed(w, pw)


def test_split_merge_max_refresh_handbook_exercise1():
    g = gold("split_merge_max_refresh.json")
    s = sum((b["scores"] for b in g["blocks"]), [])
    v = sum((b["values"] for b in g["blocks"]), [])
    r = oracle.online_row(s, v, bc=2)
    for t, st in enumerate(g["after_block"]):
        assert r["trace_m"][t] == st["m"]
        close_printed(r["trace_l"][t], st["l"])
        close_printed(r["trace_acc"][t, 0], st["acc"], st.get("acc_tol"))
    close_printed(math.exp(r["trace_m"][0] - r["trace_m"][1]), g["correction_second_block"])
    close_printed(r["O"][0], g["output"])
    # split-K form: each block normalised on its own, merged by the LSE rule
    parts = [oracle.online_row(b["scores"], b["values"], bc=len(b["scores"])) for b in g["blocks"]]
    Om, Lm = oracle.merge([p["O"] for p in parts], [p["lse"] for p in parts])
    close_printed(Om[0], g["output"])
    # direct: weights proportional to e^score
    q, k, vv = scores_as_attention(s, v)
    O, L = oracle.attention(q, k, vv, causal=False, scale=1.0, dtype=BF16)
    close_printed(O[0, 0, 0, 0], g["output"])
    for sc, pw in zip(s, g["direct_weights_unnormalised"]):
        close_printed(math.exp(sc), pw)
    close_printed(math.exp(L[0, 0, 0]), g["direct_weight_sum"])


# ----------------------------------------------------------------------------- library cross-checks
def _sdpa_ref(case, causal):
    q = torch.from_numpy(bits_to_f64(case.q, case.dtype))
    k = torch.from_numpy(bits_to_f64(case.k, case.dtype))
    v = torch.from_numpy(bits_to_f64(case.v, case.dtype))
    o = F.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=case.scale,
                                       enable_gqa=case.Hq != case.Hkv)
    # LSE through scipy: scores by a library matmul, masked, logsumexp
    rep = case.Hq // case.Hkv
    kk = np.repeat(bits_to_f64(case.k, case.dtype), rep, axis=1)
    s = case.scale * np.matmul(bits_to_f64(case.q, case.dtype), np.swapaxes(kk, -1, -2))
    if causal:
        n = s.shape[-1]
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
    return o.numpy(), sps.logsumexp(s, axis=-1)


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,dtype", [
    (2, 4, 2, 37, 16, True, BF16),
    (2, 4, 2, 37, 16, False, BF16),
    (1, 3, 1, 50, 8, True, FP16),
    (1, 2, 2, 1, 64, True, BF16),
    (3, 8, 8, 20, 32, False, FP16),
])
def test_attention_matches_torch_sdpa_float64(B, Hq, Hkv, N, d, causal, dtype):
    case = prefill_case(B, Hq, Hkv, N, d, causal, dtype, seeds=(11, 12, 13))
    O, L = oracle.attention(case.q, case.k, case.v, causal, case.scale, dtype)
    o_ref, l_ref = _sdpa_ref(case, causal)
    np.testing.assert_allclose(O, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, l_ref, rtol=1e-12, atol=1e-12)


def test_scale_is_applied_to_scores_not_values():
    case = prefill_case(1, 2, 1, 9, 16, False, BF16, scale=0.37, seeds=(21, 22, 23))
    O, L = oracle.attention(case.q, case.k, case.v, False, case.scale, BF16)
    o_ref, l_ref = _sdpa_ref(case, False)
    np.testing.assert_allclose(O, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, l_ref, rtol=1e-12, atol=1e-12)


def test_row_subset_equals_full_evaluation():
    case = prefill_case(2, 4, 2, 33, 16, True, BF16, seeds=(31, 32, 33))
    O, L = oracle.attention(case.q, case.k, case.v, True, case.scale, BF16)
    rows = np.array([0, 5, 32, 33 * 4 + 7, 2 * 4 * 33 - 1], dtype=np.int64)
    Os, Ls = oracle.attention(case.q, case.k, case.v, True, case.scale, BF16, rows=rows)
    assert np.array_equal(Os, O.reshape(-1, 16)[rows])
    assert np.array_equal(Ls, L.reshape(-1)[rows])


# ----------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [True, False])
def test_zero_queries_give_uniform_attention(causal):
    case = prefill_case(1, 2, 1, 40, 16, causal, BF16, seeds=(41, 42, 43))
    q0 = np.zeros_like(case.q)
    O, L = oracle.attention(q0, case.k, case.v, causal, case.scale, BF16)
    v = bits_to_f64(case.v, BF16)[0, 0]
    for i in range(40):
        n = i + 1 if causal else 40
        np.testing.assert_allclose(O[0, 1, i], v[:n].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert abs(L[0, 1, i] - math.log(n)) < 1e-14


def test_single_visible_key_and_constant_values():
    case = prefill_case(1, 1, 1, 16, 32, True, BF16, seeds=(51, 52, 53))
    O, L = oracle.attention(case.q, case.k, case.v, True, case.scale, BF16)
    v = bits_to_f64(case.v, BF16)[0, 0]
    assert np.array_equal(O[0, 0, 0], v[0])        # row 0 sees only key 0: P = 1 exactly
    s00 = case.scale * np.dot(bits_to_f64(case.q, BF16)[0, 0, 0], bits_to_f64(case.k, BF16)[0, 0, 0])
    assert abs(L[0, 0, 0] - s00) < 1e-14
    vc = np.full_like(case.v, f32_to_bf16_bits(np.array([1.5], np.float32))[0])
    O2, _ = oracle.attention(case.q, case.k, vc, True, case.scale, BF16)
    np.testing.assert_allclose(O2, 1.5, rtol=1e-14, atol=0)


def test_rows_of_p_sum_to_one_and_masked_entries_are_zero():
    case = prefill_case(1, 2, 2, 30, 16, True, BF16, seeds=(61, 62, 63))
    _, _, P = oracle.attention(case.q, case.k, case.v, True, case.scale, BF16, return_probs=True)
    assert np.all(np.abs(P.sum(-1) - 1.0) <= 1e-14)
    assert np.all(P[..., np.triu_indices(30, 1)[0], np.triu_indices(30, 1)[1]] == 0)
    assert np.all(P >= 0)


def test_gqa_equals_replicated_mha():
    case = prefill_case(2, 8, 2, 25, 16, True, BF16, seeds=(71, 72, 73))
    O, L = oracle.attention(case.q, case.k, case.v, True, case.scale, BF16)
    k_rep = np.repeat(case.k, 4, axis=1)
    v_rep = np.repeat(case.v, 4, axis=1)
    O2, L2 = oracle.attention(case.q, k_rep, v_rep, True, case.scale, BF16)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


# ----------------------------------------------------------------------------- tiled = untiled, merge
@pytest.mark.parametrize("n", [1, 2, 3, 17, 64, 257, 1000])
@pytest.mark.parametrize("bc", [1, 2, 3, 16, 64])
def test_tiled_online_equals_library_softmax(n, bc):
    rng = np.random.default_rng(1000 + n * 7 + bc)
    s = rng.standard_normal(n) * 3.0
    v = rng.standard_normal((n, 5))
    r = oracle.online_row(s, v, bc)
    ref = sps.softmax(s) @ v
    np.testing.assert_allclose(r["O"], ref, rtol=1e-12, atol=1e-13)
    assert abs(r["lse"] - sps.logsumexp(s)) <= 1e-12 * max(1.0, abs(r["lse"]))
    assert r["m"] == s.max()


def test_online_row_with_masked_scores():
    s = np.array([-np.inf, 0.5, -np.inf, 2.0, -np.inf])
    v = np.arange(10.0).reshape(5, 2)
    r = oracle.online_row(s, v, bc=2)       # first tile holds one visible score
    ref = sps.softmax(s) @ v
    np.testing.assert_allclose(r["O"], ref, rtol=1e-14)
    r2 = oracle.online_row(np.full(3, -np.inf), np.ones((3, 1)), bc=2)
    assert r2["lse"] == -np.inf and r2["O"][0] == 0.0


@pytest.mark.parametrize("segments", [2, 8, 64])
def test_merge_is_order_free(segments):
    rng = np.random.default_rng(segments)
    n = 10000
    s = rng.standard_normal(n) * 2.0
    v = rng.standard_normal((n, 3))
    cuts = np.sort(rng.choice(np.arange(1, n), segments - 1, replace=False))
    bounds = np.concatenate([[0], cuts, [n]])
    parts = [oracle.online_row(s[a:b], v[a:b], bc=64) for a, b in zip(bounds[:-1], bounds[1:])]
    O_s = np.array([p["O"] for p in parts])
    L_s = np.array([p["lse"] for p in parts])
    ref = sps.softmax(s) @ v
    for order in (np.arange(segments), np.arange(segments)[::-1], rng.permutation(segments)):
        Om, Lm = oracle.merge(O_s[order], L_s[order])
        np.testing.assert_allclose(Om, ref, rtol=1e-13, atol=1e-14)
        assert abs(Lm - sps.logsumexp(s)) < 1e-12
    # an empty part (LSE = -inf) carries weight 0
    Om, Lm = oracle.merge(np.vstack([O_s, np.full((1, 3), 123.0)]), np.append(L_s, -np.inf))
    np.testing.assert_allclose(Om, ref, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------- paged decode
def test_bsr_example_paged_equals_contiguous_exactly():
    g = gold("bsr_page_table_example.json")
    lengths, tables, ps = g["lengths"], g["tables"], g["page_size"]
    # the printed BSR arrays are the concatenated tables and their prefix counts
    assert sum(tables, []) == g["indices"]
    assert list(np.cumsum([0] + [len(t) for t in tables])) == g["indptr"]
    assert [len(t) for t in tables] == [-(-n // ps) for n in lengths]
    B, Hq, Hkv, d = 3, 4, 2, 8
    num_pages = max(g["indices"]) + 1
    table = np.full((B, max(len(t) for t in tables)), -1, np.int32)
    for r, t in enumerate(tables):
        table[r, :len(t)] = t
    q = normal_bits((B, Hq, d), 81, BF16)
    kp = normal_bits((num_pages, ps, Hkv, d), 82, BF16)
    vp = normal_bits((num_pages, ps, Hkv, d), 83, BF16)
    O, L = oracle.decode_paged(q, kp, vp, table, lengths, 0.3, BF16)
    for r in range(B):
        n = lengths[r]
        toks = np.arange(n)
        pages = table[r, toks // ps]
        kc = kp[pages, toks % ps]            # [n, Hkv, d] gathered, contiguous
        vc = vp[pages, toks % ps]
        # decode of request r = last row of a causal prefill whose last query is q_r
        qq = np.zeros((1, Hq, n, d), np.uint16)
        qq[0, :, n - 1] = q[r]
        Oc, Lc = oracle.attention(qq, np.ascontiguousarray(kc.transpose(1, 0, 2))[None],
                                  np.ascontiguousarray(vc.transpose(1, 0, 2))[None], True, 0.3, BF16)
        assert np.array_equal(O[r], Oc[0, :, n - 1])   # max difference exactly 0
        assert np.array_equal(L[r], Lc[0, :, n - 1])


def test_decode_matches_torch_sdpa_and_is_page_order_free():
    case = decode_case(5, 8, 2, 32, [1, 17, 100, 33, 64], page_size=16, seeds=(91, 92, 93))
    O, L = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                               case.ctx_lens, case.scale, BF16)
    for r in range(case.B):
        n = int(case.ctx_lens[r])
        toks = np.arange(n)
        pages = case.block_table[r, toks // 16]
        kc = bits_to_f64(case.k_pages[pages, toks % 16], BF16).transpose(1, 0, 2)[None]
        vc = bits_to_f64(case.v_pages[pages, toks % 16], BF16).transpose(1, 0, 2)[None]
        qv = bits_to_f64(case.q[r], BF16)[None, :, None, :]
        o = F.scaled_dot_product_attention(torch.from_numpy(qv), torch.from_numpy(kc),
                                           torch.from_numpy(vc), scale=case.scale, enable_gqa=True)
        np.testing.assert_allclose(O[r], o.numpy()[0, :, 0], rtol=1e-12, atol=1e-12)
        s = case.scale * np.einsum("hd,hnd->hn", bits_to_f64(case.q[r], BF16),
                                   np.repeat(kc[0], 4, axis=0))
        np.testing.assert_allclose(L[r], sps.logsumexp(s, axis=-1), rtol=1e-12, atol=1e-12)
    perm = permute_pages(case, 1234)
    O2, L2 = oracle.decode_paged(perm.q, perm.k_pages, perm.v_pages, perm.block_table,
                                 perm.ctx_lens, perm.scale, BF16)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_decode_zero_queries_count_visible_tokens():
    case = decode_case(4, 4, 1, 16, [1, 15, 16, 300], page_size=16, seeds=(94, 95, 96))
    O, L = oracle.decode_paged(np.zeros_like(case.q), case.k_pages, case.v_pages,
                               case.block_table, case.ctx_lens, case.scale, BF16)
    assert np.array_equal(np.round(np.exp(L)), np.repeat(case.ctx_lens[:, None], 4, 1).astype(float))


def test_decode_empty_context_reading():
    case = decode_case(2, 2, 1, 8, [0, 5], page_size=16, seeds=(97, 98, 99))
    O, L = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                               case.ctx_lens, case.scale, BF16)
    assert np.all(L[0] == -np.inf) and np.all(O[0] == 0.0) and np.all(np.isfinite(L[1]))


# ----------------------------------------------------------------------------- shared prefix
# [CS349D Lecture 4 notes, 4.4 and 5.3] requests that share a prefix attend to the prefix
# keys followed by their own; the cascade split is one way to compute the same thing.

def _prefix(Hkv, P, d, seed, dtype=BF16):
    return (normal_bits((Hkv, P, d), seed, dtype), normal_bits((Hkv, P, d), seed + 1, dtype))


def test_cascade_matches_torch_sdpa_over_prefix_then_own_tokens():
    case = decode_case(4, 8, 2, 32, [0, 1, 37, 64], page_size=16, seeds=(71, 72, 73))
    kpre, vpre = _prefix(2, 45, 32, 74)
    O, L = oracle.decode_cascade(case.q, kpre, vpre, case.k_pages, case.v_pages,
                                 case.block_table, case.ctx_lens, case.scale, BF16)
    for r in range(case.B):
        n = int(case.ctx_lens[r])
        toks = np.arange(n)
        pages = case.block_table[r, toks // 16]
        own_k = bits_to_f64(case.k_pages[pages, toks % 16], BF16).transpose(1, 0, 2)
        own_v = bits_to_f64(case.v_pages[pages, toks % 16], BF16).transpose(1, 0, 2)
        kc = np.concatenate([bits_to_f64(kpre, BF16), own_k], axis=1)[None]
        vc = np.concatenate([bits_to_f64(vpre, BF16), own_v], axis=1)[None]
        qv = bits_to_f64(case.q[r], BF16)[None, :, None, :]
        o = F.scaled_dot_product_attention(torch.from_numpy(qv), torch.from_numpy(kc),
                                           torch.from_numpy(vc), scale=case.scale, enable_gqa=True)
        np.testing.assert_allclose(O[r], o.numpy()[0, :, 0], rtol=1e-12, atol=1e-12)
        s = case.scale * np.einsum("hd,hnd->hn", bits_to_f64(case.q[r], BF16),
                                   np.repeat(kc[0], 4, axis=0))
        np.testing.assert_allclose(L[r], sps.logsumexp(s, axis=-1), rtol=1e-12, atol=1e-12)


def test_cascade_without_prefix_is_paged_decode():
    case = decode_case(3, 4, 4, 16, [5, 0, 40], page_size=16, seeds=(75, 76, 77))
    kpre = np.zeros((4, 0, 16), np.uint16)
    O, L = oracle.decode_cascade(case.q, kpre, kpre, case.k_pages, case.v_pages,
                                 case.block_table, case.ctx_lens, case.scale, BF16)
    O2, L2 = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                 case.ctx_lens, case.scale, BF16)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_cascade_equals_merge_of_prefix_and_own_states():
    case = decode_case(3, 6, 3, 16, [9, 1, 30], page_size=16, dtype=FP16, seeds=(78, 79, 80))
    kpre, vpre = _prefix(3, 20, 16, 81, FP16)
    O, L = oracle.decode_cascade(case.q, kpre, vpre, case.k_pages, case.v_pages,
                                 case.block_table, case.ctx_lens, case.scale, FP16)
    Oown, Lown = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                     case.ctx_lens, case.scale, FP16)
    # the prefix alone: a request with no own tokens
    nothing = np.zeros(case.B, np.int32)
    Opre, Lpre = oracle.decode_cascade(case.q, kpre, vpre, case.k_pages, case.v_pages,
                                       case.block_table, nothing, case.scale, FP16)
    for r in range(case.B):
        for h in range(case.Hq):
            Om, Lm = oracle.merge(np.stack([Opre[r, h], Oown[r, h]]), np.array([Lpre[r, h], Lown[r, h]]))
            np.testing.assert_allclose(O[r, h], Om, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(L[r, h], Lm, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- paged / varlen prefill
# [LLM Internals 10.3.8, variable-length batching; 10.3.7 block table; CS349D Lecture 4
# section 5.1, incremental prefill] new queries packed end to end by cu_seqlens_q, each
# request's cache holding its history followed by its new tokens.

def _gather_request(case, r):
    """Request r's cached K/V as contiguous fp64 [Hkv, kv_len, d] (by plain indexing)."""
    n = int(case.kv_lens[r])
    toks = np.arange(n)
    pages = case.block_table[r, toks // case.page_size]
    k = bits_to_f64(case.k_pages[pages, toks % case.page_size], case.dtype).transpose(1, 0, 2)
    v = bits_to_f64(case.v_pages[pages, toks % case.page_size], case.dtype).transpose(1, 0, 2)
    return k, v


@pytest.mark.parametrize("causal", [True, False])
def test_paged_prefill_matches_torch_sdpa_bottom_right(causal):
    # requests: a chunk after history, a whole prompt (q_len = kv_len), a decode step
    # (q_len = 1), an empty chunk, a chunk crossing page boundaries
    case = paged_prefill_case(8, 2, 16, [5, 19, 1, 0, 33], [40, 19, 23, 7, 50], dtype=BF16,
                              causal=causal, seeds=(81, 82, 83))
    O, L = oracle.prefill_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                case.cu_seqlens_q, case.kv_lens, causal, case.scale, BF16)
    for r in range(case.B):
        ql, kl = int(case.q_lens[r]), int(case.kv_lens[r])
        if ql == 0:
            continue
        k, v = _gather_request(case, r)
        rows = slice(case.cu_seqlens_q[r], case.cu_seqlens_q[r + 1])
        qv = bits_to_f64(case.q[rows], BF16).transpose(1, 0, 2)[None]      # [1, Hq, ql, d]
        # torch's own mask: query i sees key j iff j <= kl - ql + i (bottom-right)
        mask = None
        if causal:
            mask = torch.from_numpy(np.arange(kl)[None, :] <= (kl - ql + np.arange(ql))[:, None])
        o = F.scaled_dot_product_attention(torch.from_numpy(qv), torch.from_numpy(k[None]),
                                           torch.from_numpy(v[None]), attn_mask=mask,
                                           scale=case.scale, enable_gqa=True)
        np.testing.assert_allclose(O[rows], o.numpy()[0].transpose(1, 0, 2), rtol=1e-12,
                                   atol=1e-12)
        s = case.scale * np.einsum("hid,hnd->hin", qv[0], np.repeat(k, 4, axis=0))
        if causal:
            s = np.where(mask.numpy()[None], s, -np.inf)
        np.testing.assert_allclose(L[rows], sps.logsumexp(s, axis=-1).T, rtol=1e-12, atol=1e-12)


def test_paged_prefill_packing_example_and_isolation():
    # lengths 3, 5, 2 pack as [0, 3, 8, 10] [LLM Internals 10.3.8]; changing one request's
    # cache leaves the others' outputs bitwise unchanged (the sequences do not see each other)
    case = paged_prefill_case(4, 4, 8, [3, 5, 2], [3, 21, 9], dtype=FP16, seeds=(84, 85, 86))
    assert case.cu_seqlens_q.tolist() == [0, 3, 8, 10]
    O, L = oracle.prefill_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                case.cu_seqlens_q, case.kv_lens, True, case.scale, FP16)
    kp = case.k_pages.copy()
    vp = case.v_pages.copy()
    own = case.block_table[1, :2]
    kp[own] = normal_bits(kp[own].shape, 87, FP16)
    vp[own] = normal_bits(vp[own].shape, 88, FP16)
    O2, L2 = oracle.prefill_paged(case.q, kp, vp, case.block_table, case.cu_seqlens_q,
                                  case.kv_lens, True, case.scale, FP16)
    for rows in (slice(0, 3), slice(8, 10)):
        assert np.array_equal(O[rows], O2[rows]) and np.array_equal(L[rows], L2[rows])
    assert not np.array_equal(O[3:8], O2[3:8])


def test_paged_prefill_zero_queries_count_visible_keys():
    # q = 0: every score is 0, so LSE = ln(number of visible keys) = ln(kv - q_len + i + 1)
    case = paged_prefill_case(4, 2, 8, [7, 1, 16], [7, 30, 40], seeds=(89, 90, 91))
    q0 = np.zeros_like(case.q)
    _, L = oracle.prefill_paged(q0, case.k_pages, case.v_pages, case.block_table,
                                case.cu_seqlens_q, case.kv_lens, True, case.scale, BF16)
    for r in range(case.B):
        ql, kl = int(case.q_lens[r]), int(case.kv_lens[r])
        for i in range(ql):
            row = case.cu_seqlens_q[r] + i
            assert np.all(np.round(np.exp(L[row])) == kl - ql + i + 1)


def test_paged_prefill_of_a_whole_prompt_is_causal_attention():
    # q_len = kv_len: the chunk is the whole prompt, i.e. ordinary causal prefill
    N = 45
    case = paged_prefill_case(6, 3, 16, [N], [N], dtype=BF16, seeds=(92, 93, 94))
    O, L = oracle.prefill_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                case.cu_seqlens_q, case.kv_lens, True, case.scale, BF16)
    k, v = _gather_request(case, 0)
    q = case.q.transpose(1, 0, 2)[None]
    toks = np.arange(N)
    pages = case.block_table[0, toks // 16]
    kb = case.k_pages[pages, toks % 16].transpose(1, 0, 2)[None]
    vb = case.v_pages[pages, toks % 16].transpose(1, 0, 2)[None]
    Od, Ld = oracle.attention(q, kb, vb, True, case.scale, BF16)
    np.testing.assert_allclose(O, Od[0].transpose(1, 0, 2), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(L, Ld[0].T, rtol=1e-13, atol=1e-13)


def test_paged_prefill_rejects_padding_rows_and_handles_short_caches():
    # rows past the last request are not anyone's query
    case = paged_prefill_case(2, 1, 8, [2, 3], [4, 3], pad_q=2, seeds=(95, 96, 97))
    with pytest.raises(ValueError):
        oracle.prefill_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                             case.cu_seqlens_q, case.kv_lens, True, case.scale, BF16)
    O, L = oracle.prefill_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                case.cu_seqlens_q, case.kv_lens, True, case.scale, BF16,
                                rows=np.arange(5 * 2))
    assert np.all(np.isfinite(L))
    # a cache shorter than the chunk: the first new queries see no key (O = 0, LSE = -inf)
    case = paged_prefill_case(2, 1, 8, [4], [2], seeds=(98, 99, 100))
    O, L = oracle.prefill_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                case.cu_seqlens_q, case.kv_lens, True, case.scale, BF16)
    assert np.all(L[:2] == -np.inf) and np.all(O[:2] == 0.0)
    assert np.all(np.isfinite(L[2:]))


# ----------------------------------------------------------------------------- variants
# [CS349D Lecture 4 notes 5.4] logits soft-cap s -> c tanh(s / c) and a sliding window where
# each query sees its last w keys.

@pytest.mark.parametrize("window,dtype", [(1, BF16), (5, BF16), (16, FP16), (33, BF16), (200, BF16)])
def test_sliding_window_matches_torch_sdpa_with_its_own_mask(window, dtype):
    c = prefill_case(2, 4, 2, 70, 16, True, dtype, seeds=(101, 102, 103))
    O, L = oracle.attention_variant(c.q, c.k, c.v, True, window, 0.0, c.scale, dtype)
    i = np.arange(70)
    mask = torch.from_numpy((i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - window))
    q, k, v = (torch.from_numpy(bits_to_f64(x, dtype)) for x in (c.q, c.k, c.v))
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=c.scale, enable_gqa=True)
    np.testing.assert_allclose(O, o.numpy(), rtol=1e-12, atol=1e-12)
    s = c.scale * np.einsum("bhid,bhjd->bhij", q.numpy(), np.repeat(k.numpy(), 2, axis=1))
    s = np.where(mask.numpy(), s, -np.inf)
    np.testing.assert_allclose(L, sps.logsumexp(s, axis=-1), rtol=1e-12, atol=1e-12)


def test_sliding_window_closed_forms():
    c = prefill_case(1, 2, 1, 40, 8, True, BF16, seeds=(104, 105, 106))
    # a window of one key: each row returns its own V row exactly
    O, L = oracle.attention_variant(c.q, c.k, c.v, True, 1, 0.0, c.scale, BF16)
    assert np.array_equal(O[0, :, :, :], np.repeat(bits_to_f64(c.v, BF16)[0], 2, axis=0))
    # a window as long as the sequence is plain causal attention
    O2, L2 = oracle.attention_variant(c.q, c.k, c.v, True, 40, 0.0, c.scale, BF16)
    O3, L3 = oracle.attention(c.q, c.k, c.v, True, c.scale, BF16)
    np.testing.assert_allclose(O2, O3, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(L2, L3, rtol=1e-14, atol=1e-14)
    # zero queries: LSE counts the keys in the window
    q0 = np.zeros_like(c.q)
    _, L0 = oracle.attention_variant(q0, c.k, c.v, True, 7, 0.0, c.scale, BF16)
    want = np.log(np.minimum(np.arange(40) + 1, 7))
    np.testing.assert_allclose(L0[0, 0], want, rtol=0, atol=1e-14)
    with pytest.raises(ValueError):
        oracle.attention_variant(c.q, c.k, c.v, False, 7, 0.0, c.scale, BF16)


def test_softcap_tends_to_plain_attention_as_the_cap_grows():
    c = prefill_case(1, 4, 2, 50, 16, True, BF16, seeds=(107, 108, 109))
    q, k, v = (torch.from_numpy(bits_to_f64(x, BF16)) for x in (c.q, c.k, c.v))
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=c.scale,
                                       enable_gqa=True).numpy()
    O, _ = oracle.attention_variant(c.q, c.k, c.v, True, 0, 1e30, c.scale, BF16)
    np.testing.assert_allclose(O, o, rtol=1e-12, atol=1e-12)
    # c tanh(s / c) = s - s^3 / (3 c^2) + ...: the distance to plain attention falls as 1 / c^2
    e1 = np.abs(oracle.attention_variant(c.q, c.k, c.v, True, 0, 20.0, c.scale, BF16)[0] - o).max()
    e2 = np.abs(oracle.attention_variant(c.q, c.k, c.v, True, 0, 40.0, c.scale, BF16)[0] - o).max()
    assert 0.2 < e2 / e1 < 0.3, (e1, e2)


def test_softcap_bounds_the_weight_ratio_and_follows_the_scale():
    # V = identity (d = N) makes each output row the row of weights P; capped scores lie in
    # (-c, c), so no two weights differ by more than e^(2c), and large scores reach it
    N, cap = 16, 1.5
    rng = np.random.default_rng(110)
    qf = np.full((1, 1, N, N), 1.0, np.float32)
    kf = np.zeros((1, 1, N, N), np.float32)
    kf[0, 0, :, 0] = np.where(rng.random(N) < 0.5, 64.0, -64.0)   # scores +-64
    kf[0, 0, 0, 0], kf[0, 0, 1, 0] = 64.0, -64.0
    vf = np.eye(N, dtype=np.float32)[None, None]
    qb, kb, vb = (f32_to_bf16_bits(x) for x in (qf, kf, vf))
    P, _ = oracle.attention_variant(qb, kb, vb, False, 0, cap, 1.0, BF16)
    ratio = P[0, 0].max(axis=1) / P[0, 0].min(axis=1)
    assert np.all(ratio <= np.exp(2 * cap) * (1 + 1e-12)) and np.all(ratio > 0.999 * np.exp(2 * cap))
    # the cap applies to the scaled score: scale 2 on q equals q doubled (exact in bf16)
    c = prefill_case(1, 2, 2, 30, 8, True, BF16, seeds=(111, 112, 113))
    q2 = f32_to_bf16_bits(2.0 * bits_to_f64(c.q, BF16).astype(np.float32))
    Oa, La = oracle.attention_variant(c.q, c.k, c.v, True, 0, 3.0, 2.0, BF16)
    Ob, Lb = oracle.attention_variant(q2, c.k, c.v, True, 0, 3.0, 1.0, BF16)
    np.testing.assert_allclose(Oa, Ob, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(La, Lb, rtol=1e-14, atol=1e-14)
