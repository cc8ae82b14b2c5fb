"""GPU parity of attn_decode_paged against the fp64 oracle, through the C ABI binding.

Covers the handbook's context lengths (1, 17, 1000, 4096: a single token, a partial page),
GQA, both dtypes and both head sizes; split-count invariance; bit-exact block-table logic
(the same KV under an identity table and a shuffled table gives bitwise-equal output);
poisoned unused slots, unused pages and a guard page in front of the pool; the zero-query
count test; empty contexts (some, or every one); and the full-size 64-sequence workload,
compared with the oracle on every (sequence, head).  Outputs start as NaN / +inf, so any
pair left unwritten fails.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from attn_inputs import BF16, FP16, CONFIGS, config_case, decode_case, permute_pages
from tests.gpu_util import assert_parity, bits_of, from_dev_f64, to_dev

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC1
NAN_F16 = 0x7E01


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_decode(case, split, q_bits=None, k_pages=None, v_pages=None, pool_offset=0,
               want_lse=True):
    """pool_offset: number of extra (guard) pages placed in front of the pool; the table
    still indexes from the pool base."""
    import exact_attention_08_amd as attn
    kp = case.k_pages if k_pages is None else k_pages
    vp = case.v_pages if v_pages is None else v_pages
    Kall = to_dev(kp, case.dtype)
    Vall = to_dev(vp, case.dtype)
    K = Kall[pool_offset:]
    V = Vall[pool_offset:]
    q = to_dev(case.q if q_bits is None else q_bits, case.dtype)
    bt = torch.from_numpy(case.block_table).cuda()
    ctx = torch.from_numpy(case.ctx_lens).cuda()
    # outputs start as NaN / +inf: a (sequence, head) the merge never writes fails every check
    O = torch.full_like(q, float("nan"))
    LSE = (torch.full((case.B, case.Hq), float("inf"), dtype=torch.float32, device="cuda")
           if want_lse else None)
    nbytes = attn.attn_decode_paged_workspace_bytes(case.B, case.Hq, case.d, case.page_size,
                                                    case.max_pages, split)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    attn.attn_decode_paged(q, K, V, bt, ctx, O, LSE, split, ws, case.scale)
    torch.cuda.synchronize()
    return O, LSE


@pytest.mark.parametrize("ctx,Hq,Hkv,d,dtype,split", [
    ([1, 17, 1000, 4096], 32, 8, 128, BF16, 1024),     # the handbook's test lengths
    ([1, 17, 1000, 4096], 32, 8, 128, FP16, 256),
    ([5, 16, 33, 700], 8, 8, 64, BF16, 64),
    ([2047, 48, 3000], 16, 1, 128, BF16, 512),
    ([100, 1, 64, 65, 4100], 12, 4, 64, FP16, 16),
])
def test_decode_small_all_heads(ctx, Hq, Hkv, d, dtype, split):
    say(f"decode small ctx{ctx} Hq{Hq} Hkv{Hkv} d{d} dtype{dtype} split{split}")
    case = decode_case(len(ctx), Hq, Hkv, d, ctx, 16, dtype)
    O, LSE = run_decode(case, split)
    O_ref, L_ref = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                       case.ctx_lens, case.scale, dtype)
    assert_parity(from_dev_f64(O), O_ref, LSE.cpu().numpy(), L_ref, "decode")


def test_decode_split_count_invariance_and_zero_query_counts():
    ctx = [1, 17, 1000, 4096, 2500]
    case = decode_case(len(ctx), 32, 8, 128, ctx, 16, BF16, seeds=(21, 22, 23))
    O_ref, L_ref = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                       case.ctx_lens, case.scale, BF16)
    for split in (16, 64, 256, 1024, 4096, 8192):
        say(f"decode split {split}")
        O, LSE = run_decode(case, split)
        assert_parity(from_dev_f64(O), O_ref, LSE.cpu().numpy(), L_ref, f"split {split}")
        O0, L0 = run_decode(case, split, q_bits=np.zeros_like(case.q))
        cnt = np.round(np.exp(L0.cpu().numpy().astype(np.float64)))
        assert np.array_equal(cnt, np.repeat(case.ctx_lens[:, None].astype(float), 32, 1))


def test_decode_block_table_logic_is_bit_exact():
    ctx = [3, 16, 17, 999, 1024, 1025, 3333]
    ident = decode_case(len(ctx), 16, 4, 128, ctx, 16, BF16, seeds=(31, 32, 33),
                        identity_table=True)
    shuf = permute_pages(ident, 4321)
    O1, L1 = run_decode(ident, 256)
    O2, L2 = run_decode(shuf, 256)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    O3, L3 = run_decode(ident, 256)                  # determinism
    assert torch.equal(O1, O3) and torch.equal(L1, L3)


@pytest.mark.parametrize("dtype", [BF16, FP16])
def test_decode_poisoned_slots_pages_and_guard_are_never_read(dtype):
    ctx = [5, 16, 31, 1000, 77]
    case = decode_case(len(ctx), 8, 2, 64, ctx, 16, dtype, seeds=(41, 42, 43),
                       max_pages=80)
    nan = NAN_BF16 if dtype == BF16 else NAN_F16
    clean_O, clean_L = run_decode(case, 64)
    # poison: a guard page in front of the pool, slots >= ctx in every last page, and two
    # unreferenced pages at the end of the pool; unused table entries stay -1
    P = case.num_pages
    kp = np.full((P + 3, 16, case.Hkv, case.d), nan, np.uint16)
    vp = np.full_like(kp, nan)
    kp[1:P + 1] = case.k_pages
    vp[1:P + 1] = case.v_pages
    for r, n in enumerate(ctx):
        last = case.block_table[r, (n - 1) // 16]
        if n % 16:
            kp[1 + last, n % 16:] = nan
            vp[1 + last, n % 16:] = nan
    O, L = run_decode(case, 64, k_pages=kp, v_pages=vp, pool_offset=1)
    assert torch.isfinite(O.float()).all() and torch.isfinite(L).all()
    assert torch.equal(O, clean_O) and torch.equal(L, clean_L)


def test_decode_empty_context_and_no_lse():
    case = decode_case(3, 8, 2, 128, [0, 40, 0], 16, BF16, seeds=(51, 52, 53), max_pages=4)
    O, L = run_decode(case, 32)
    o = O.float().cpu().numpy()
    l = L.cpu().numpy()
    assert np.all(o[0] == 0) and np.all(o[2] == 0) and np.all(np.isneginf(l[[0, 2]]))
    O_ref, L_ref = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                       case.ctx_lens, case.scale, BF16)
    assert_parity(o[1], O_ref[1], l[1], L_ref[1], "ctx 40")
    O2, _ = run_decode(case, 32, want_lse=False)
    assert torch.equal(O, O2)


@pytest.mark.parametrize("B", [3, 100, 1100])
def test_decode_every_context_empty(B):
    """No sequence has a token: the work list is empty (for B up to 64, 1024 and beyond, the
    three ways the kernel finds an item's sequence).  Every output is O = 0, LSE = -inf, and
    a following call on the same workspace is still correct."""
    say(f"decode all-empty contexts B{B}")
    case = decode_case(B, 8, 2, 64, [0] * B, 16, BF16, seeds=(57, 58, 59), max_pages=4)
    O, L = run_decode(case, 32)
    assert torch.all(O.float() == 0) and torch.all(torch.isneginf(L))
    ctx = [0] * B
    ctx[B // 2] = 50
    case2 = decode_case(B, 8, 2, 64, ctx, 16, BF16, seeds=(57, 58, 59), max_pages=4)
    O2, L2 = run_decode(case2, 32)
    O_ref, L_ref = oracle.decode_paged(case2.q, case2.k_pages, case2.v_pages, case2.block_table,
                                       case2.ctx_lens, case2.scale, BF16)
    r = B // 2
    assert_parity(from_dev_f64(O2)[r], O_ref[r], L2.cpu().numpy()[r], L_ref[r], "one live")
    others = np.arange(B) != r
    assert torch.all(O2.float()[others] == 0)


def test_decode_named_workload_full_size_every_pair():
    name = "paged_gqa_decode_b64_ctx512_32768"
    c = CONFIGS[name]
    say(f"decode full size {name}: every (sequence, head)")
    case = config_case(name)
    O, LSE = run_decode(case, c["split_tokens"])
    O_ref, L_ref = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                       case.ctx_lens, case.scale, BF16)
    assert_parity(from_dev_f64(O), O_ref, LSE.cpu().numpy(), L_ref, name)
    # the balanced split on the same batch
    Ob, Lb = run_decode(case, 0)
    assert_parity(from_dev_f64(Ob), O_ref, Lb.cpu().numpy(), L_ref, name + " balanced")
    # zero-query count test at full size: exp(LSE) is the context length for every head
    O0, L0 = run_decode(case, c["split_tokens"], q_bits=np.zeros_like(case.q))
    cnt = np.round(np.exp(L0.cpu().numpy().astype(np.float64)))
    assert np.array_equal(cnt, np.repeat(case.ctx_lens[:, None].astype(float), case.Hq, 1))


@pytest.mark.parametrize("B,Hq,Hkv,d,dtype,split,seed", [
    (300, 8, 2, 64, BF16, 64, 41),      # more than 64 sequences: the work list from LDS tables
    (1500, 4, 1, 64, FP16, 32, 42),     # more than 1024: the work list from wave-wide scans
])
def test_decode_large_batches_use_the_general_work_list(B, Hq, Hkv, d, dtype, split, seed):
    say(f"decode large batch B{B} Hq{Hq} Hkv{Hkv} d{d} split{split}")
    ctx = np.random.default_rng(seed).integers(0, 200, B).astype(np.int32)
    case = decode_case(B, Hq, Hkv, d, ctx, 16, dtype, seeds=(seed, seed + 1, seed + 2),
                       max_pages=16)
    O, LSE = run_decode(case, split)
    O_ref, L_ref = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                       case.ctx_lens, case.scale, dtype)
    live = case.ctx_lens > 0
    assert np.all(np.isneginf(LSE.cpu().numpy()[~live]))
    assert_parity(from_dev_f64(O)[live], O_ref[live], LSE.cpu().numpy()[live], L_ref[live],
                  "decode large batch")
    # zero queries: exp(LSE) counts each sequence's tokens exactly
    O0, L0 = run_decode(case, split, q_bits=np.zeros_like(case.q))
    cnt = np.round(np.exp(L0.cpu().numpy().astype(np.float64)))
    assert np.array_equal(cnt[live], np.repeat(ctx[live, None].astype(float), Hq, 1))


def test_decode_many_calls_share_one_workspace():
    """Each call leaves the work-queue counters in its workspace's control block reset for the
    next.  150 back-to-back calls on one stream (the balanced split, whose length also lives
    in the control block, alternating with explicit splits), each split with a workspace of
    its own, and then the three splits in turn on one shared workspace: every output must
    equal the first bitwise."""
    import exact_attention_08_amd as attn
    say("decode: 150 calls on reused workspaces")
    ctx = [1, 700, 4100, 33, 2048, 5000]
    case = decode_case(len(ctx), 8, 2, 128, ctx, 16, BF16, seeds=(91, 92, 93))
    K, V = to_dev(case.k_pages, case.dtype), to_dev(case.v_pages, case.dtype)
    q = to_dev(case.q, case.dtype)
    bt = torch.from_numpy(case.block_table).cuda()
    cl = torch.from_numpy(case.ctx_lens).cuda()
    splits = (0, 256, 1024)
    ws = {s: torch.zeros(attn.attn_decode_paged_workspace_bytes(
        case.B, case.Hq, case.d, case.page_size, case.max_pages, s), dtype=torch.uint8,
        device="cuda") for s in splits}
    outs = {s: [] for s in splits}
    for i in range(150):
        s = splits[i % 3]
        O = torch.empty_like(q)
        L = torch.empty(case.B, case.Hq, dtype=torch.float32, device="cuda")
        attn.attn_decode_paged(q, K, V, bt, cl, O, L, s, ws[s], case.scale)
        outs[s].append((O, L))
    # one workspace (sized for the balanced split, the largest) for every split in turn
    shared = ws[0]
    for i in range(30):
        s = splits[i % 3]
        O = torch.empty_like(q)
        L = torch.empty(case.B, case.Hq, dtype=torch.float32, device="cuda")
        attn.attn_decode_paged(q, K, V, bt, cl, O, L, s, shared, case.scale)
        outs[s].append((O, L))
    torch.cuda.synchronize()
    for s in splits:
        O0, L0 = outs[s][0]
        for O, L in outs[s][1:]:
            assert torch.equal(O, O0) and torch.equal(L, L0), s
    O_ref, L_ref = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                       case.ctx_lens, case.scale, case.dtype)
    assert_parity(from_dev_f64(outs[0][0][0]), O_ref, outs[0][0][1].cpu().numpy(), L_ref,
                  "decode after slot wrap")
