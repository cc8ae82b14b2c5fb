"""GPU parity of attn_decode_cascade (requests sharing a prefix) against the fp64 oracle,
through the C ABI binding.

The oracle computes the definition: each request attends to the prefix keys followed by its
own paged tokens.  Covered: GQA and MHA, both dtypes and head sizes, prefixes shorter than
one tile, ragged and several chunks long; requests with no own tokens; no prefix (equal to
attn_decode_paged, bitwise); bitwise determinism; the full-size shared-prefix workload on
every (request, head).  Outputs start as NaN / +inf, so any pair left unwritten fails.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from attn_inputs import BF16, FP16, CASCADE_WORKLOADS, cascade_case, cascade_workload
from tests.gpu_util import assert_parity, from_dev_f64, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_cascade(case, split, want_lse=True):
    import exact_attention_08_amd as attn
    q = to_dev(case.q, case.dtype)
    K = to_dev(case.k_pages, case.dtype)
    V = to_dev(case.v_pages, case.dtype)
    Kp = to_dev(case.extra["k_prefix"], case.dtype)
    Vp = to_dev(case.extra["v_prefix"], case.dtype)
    bt = torch.from_numpy(case.block_table).cuda()
    ctx = torch.from_numpy(case.ctx_lens).cuda()
    # outputs start as NaN / +inf: a (request, head) the merge never writes fails every check
    O = torch.full_like(q, float("nan"))
    LSE = (torch.full((case.B, case.Hq), float("inf"), dtype=torch.float32, device="cuda")
           if want_lse else None)
    P = case.extra["k_prefix"].shape[1]
    nbytes = attn.attn_decode_cascade_workspace_bytes(case.B, case.Hq, case.d, case.page_size,
                                                      case.max_pages, split, P)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    attn.attn_decode_cascade(q, Kp, Vp, K, V, bt, ctx, O, LSE, split, ws, case.scale)
    torch.cuda.synchronize()
    return O, LSE


def oracle_cascade(case, pairs=None):
    return oracle.decode_cascade(case.q, case.extra["k_prefix"], case.extra["v_prefix"],
                                 case.k_pages, case.v_pages, case.block_table, case.ctx_lens,
                                 case.scale, case.dtype, pairs=pairs)


@pytest.mark.parametrize("B,Hq,Hkv,d,dtype,P,own,split", [
    (4, 32, 8, 128, BF16, 4096, [256, 256, 256, 256], 1024),   # the pages' demo proportions
    (5, 32, 8, 128, FP16, 1000, [1, 17, 0, 700, 2048], 256),
    (3, 8, 8, 64, BF16, 33, [5, 64, 100], 64),
    (7, 16, 1, 128, BF16, 2500, [0, 0, 3, 1024, 1025, 9, 4000], 512),
    (40, 12, 4, 64, FP16, 1, [16, 1, 30] * 13 + [7], 16),
    (2, 4, 2, 128, BF16, 3073, [31, 0], 1024),
])
def test_cascade_small_all_heads(B, Hq, Hkv, d, dtype, P, own, split):
    say(f"cascade B{B} Hq{Hq} Hkv{Hkv} d{d} dtype{dtype} prefix{P} split{split}")
    case = cascade_case(B, Hq, Hkv, d, P, own, 16, dtype)
    O, LSE = run_cascade(case, split)
    O_ref, L_ref = oracle_cascade(case)
    assert_parity(from_dev_f64(O), O_ref, LSE.cpu().numpy(), L_ref, "cascade")


def test_cascade_without_prefix_is_paged_decode_bitwise_and_deterministic():
    import exact_attention_08_amd as attn
    own = [1, 17, 1000, 4096, 0, 33]
    case = cascade_case(len(own), 32, 8, 128, 0, own, 16, BF16, seeds=(61, 62, 63))
    O, L = run_cascade(case, 256)
    q = to_dev(case.q, BF16)
    K = to_dev(case.k_pages, BF16)
    V = to_dev(case.v_pages, BF16)
    bt = torch.from_numpy(case.block_table).cuda()
    ctx = torch.from_numpy(case.ctx_lens).cuda()
    O2 = torch.empty_like(q)
    L2 = torch.empty(case.B, case.Hq, dtype=torch.float32, device="cuda")
    ws = torch.zeros(attn.attn_decode_paged_workspace_bytes(case.B, case.Hq, case.d, 16,
                                                            case.max_pages, 256),
                     dtype=torch.uint8, device="cuda")
    attn.attn_decode_paged(q, K, V, bt, ctx, O2, L2, 256, ws, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(L, L2)
    # with a prefix: two calls agree bit for bit
    case = cascade_case(len(own), 32, 8, 128, 2000, own, 16, BF16, seeds=(64, 65, 66))
    Oa, La = run_cascade(case, 256)
    Ob, Lb = run_cascade(case, 256)
    assert torch.equal(Oa, Ob) and torch.equal(La, Lb)


def test_cascade_prefix_only_and_zero_query_counts():
    own = [0, 0, 0]
    case = cascade_case(3, 8, 2, 128, 1500, own, 16, BF16, seeds=(67, 68, 69), max_pages=2)
    O, L = run_cascade(case, 32)
    O_ref, L_ref = oracle_cascade(case)
    assert_parity(from_dev_f64(O), O_ref, L.cpu().numpy(), L_ref, "prefix only")
    # zero queries: every key weighs the same, exp(LSE) counts prefix + own tokens
    own = [5, 0, 333]
    case = cascade_case(3, 8, 2, 64, 777, own, 16, FP16, seeds=(70, 71, 72))
    case.q[:] = 0
    O0, L0 = run_cascade(case, 64)
    cnt = np.round(np.exp(L0.cpu().numpy().astype(np.float64)))
    assert np.array_equal(cnt, np.repeat((np.array(own) + 777)[:, None].astype(float), 8, 1))


@pytest.mark.parametrize("name", sorted(CASCADE_WORKLOADS))
def test_cascade_named_workload_full_size_every_pair(name):
    c = CASCADE_WORKLOADS[name]
    say(f"cascade full size {name}: every (request, head)")
    case = cascade_workload(name)
    O, LSE = run_cascade(case, c["split_tokens"])
    O_ref, L_ref = oracle_cascade(case)
    assert_parity(from_dev_f64(O), O_ref, LSE.cpu().numpy(), L_ref, name)


def test_cascade_many_requests_span_several_prefix_query_tiles():
    # 200 requests x 4 heads = 800 prefix query rows: seven 128-row tiles per kv head
    say("cascade 200 requests")
    own = np.random.default_rng(81).integers(0, 300, 200)
    case = cascade_case(200, 32, 8, 128, 1000, own, 16, BF16, seeds=(82, 83, 84), max_pages=19)
    O, LSE = run_cascade(case, 0)
    O_ref, L_ref = oracle_cascade(case)
    assert_parity(from_dev_f64(O), O_ref, LSE.cpu().numpy(), L_ref, "cascade 200")
