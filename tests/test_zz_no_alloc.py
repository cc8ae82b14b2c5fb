"""GPU test of attn_decode_paged_noalloc (the decode for callers that cannot allocate), through
the C ABI binding.  Its output must equal attn_decode_paged's bit for bit (same kernels, same
split) and match the oracle; two calls in a row, the second on a smaller batch, check that
the shared scratch left by one call does not leak into the next.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from attn_inputs import BF16, FP16, decode_case
from tests.gpu_util import assert_parity, from_dev_f64, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_inputs(case):
    return (to_dev(case.q, case.dtype), to_dev(case.k_pages, case.dtype),
            to_dev(case.v_pages, case.dtype), torch.from_numpy(case.block_table).cuda(),
            torch.from_numpy(case.ctx_lens).cuda())


def with_workspace(case, split, inp):
    import exact_attention_08_amd as attn
    q, K, V, bt, ctx = inp
    O = torch.full_like(q, float("nan"))
    L = torch.full((case.B, case.Hq), float("inf"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(attn.attn_decode_paged_workspace_bytes(case.B, case.Hq, case.d, 16,
                                                            case.max_pages, split),
                     dtype=torch.uint8, device="cuda")
    attn.attn_decode_paged(q, K, V, bt, ctx, O, L, split, ws, case.scale)
    return O, L


def without_workspace(case, split, inp):
    import exact_attention_08_amd as attn
    q, K, V, bt, ctx = inp
    O = torch.full_like(q, float("nan"))
    L = torch.full((case.B, case.Hq), float("inf"), dtype=torch.float32, device="cuda")
    attn.attn_decode_paged_noalloc(q, K, V, bt, ctx, O, L, split, case.scale)
    return O, L


@pytest.mark.parametrize("split", [0, 256, 1024])
def test_noalloc_equals_workspace_call_on_two_calls_in_a_row(split):
    say(f"noalloc decode, split {split}")
    big = decode_case(24, 32, 8, 128, [1, 17, 1000, 4096, 2500, 9000] * 4, 16, BF16,
                      seeds=(101, 102, 103))
    small = decode_case(3, 16, 4, 64, [700, 0, 33], 16, FP16, seeds=(104, 105, 106))
    for case in (big, small):
        inp = dev_inputs(case)
        O1, L1 = with_workspace(case, split, inp)
        O2, L2 = without_workspace(case, split, inp)
        torch.cuda.synchronize()
        assert torch.equal(O1, O2) and torch.equal(L1, L2), f"B{case.B}"
        O_ref, L_ref = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                           case.ctx_lens, case.scale, case.dtype)
        live = case.ctx_lens > 0
        assert_parity(from_dev_f64(O2)[live], O_ref[live], L2.cpu().numpy()[live], L_ref[live],
                      f"noalloc B{case.B}")
        assert torch.all(O2.float()[torch.from_numpy(~live).cuda()] == 0)


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    import exact_attention_08_amd as attn
    say("noalloc decode: too large")
    case = decode_case(2, 8, 2, 128, [40, 50], 16, BF16, seeds=(107, 108, 109))
    q, K, V, _, ctx = dev_inputs(case)
    # a table of 60000 pages per sequence and 16-token splits: 60000 partial states of
    # 129 floats per (sequence, head), 495 MB in all, beyond the 64 MiB scratch
    bt = torch.zeros((case.B, 60000), dtype=torch.int32, device="cuda")
    O = torch.zeros_like(q)
    with pytest.raises(attn.AttnError) as e:
        attn.attn_decode_paged_noalloc(q, K, V, bt, ctx, O, None, 16, case.scale)
    assert e.value.code == -8
    assert torch.all(O == 0)   # nothing was launched
