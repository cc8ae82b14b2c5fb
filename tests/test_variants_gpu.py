"""GPU parity of attn_fwd_variant (causal sliding window, logits soft-cap) against the fp64
oracle, through the C ABI binding.

Covered: windows of 1 (each row returns its own V row), shorter than a 32-key block,
not a multiple of a block, many tiles long, and at least the sequence length (then equal to
attn_fwd bit for bit); soft-caps from strong (5) to mild (50), causal and not; both
together; both dtypes and head sizes, GQA and MHA; zero queries counting the keys in each
window exactly; a Llama-3-8B-sized case on sampled rows.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from attn_inputs import BF16, FP16, prefill_case
from tests.gpu_util import assert_parity, bits_of, from_dev_f64, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_variant(c, window, softcap, q=None):
    import exact_attention_08_amd as attn
    Q = to_dev(c.q if q is None else q, c.dtype)
    K, V = to_dev(c.k, c.dtype), to_dev(c.v, c.dtype)
    O = torch.empty_like(Q)
    L = torch.empty(c.B, c.Hq, c.N, dtype=torch.float32, device="cuda")
    attn.attn_fwd_variant(Q, K, V, O, L, c.causal, window, softcap, c.scale)
    torch.cuda.synchronize()
    return O, L


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dtype,causal,window,softcap", [
    (2, 8, 2, 700, 128, BF16, True, 256, 0.0),
    (1, 4, 4, 333, 64, FP16, True, 33, 0.0),
    (1, 8, 2, 1000, 64, BF16, True, 20, 0.0),
    (2, 4, 1, 513, 128, FP16, True, 129, 0.0),
    (2, 8, 2, 700, 128, BF16, True, 0, 30.0),
    (1, 4, 4, 300, 64, FP16, False, 0, 5.0),
    (1, 8, 8, 257, 128, BF16, False, 0, 50.0),
    (2, 8, 2, 900, 128, BF16, True, 200, 20.0),
    (1, 16, 4, 640, 64, BF16, True, 64, 10.0),
])
def test_variant_all_rows(B, Hq, Hkv, N, d, dtype, causal, window, softcap):
    say(f"variant B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} dtype{dtype} causal{causal} w{window} cap{softcap}")
    c = prefill_case(B, Hq, Hkv, N, d, causal, dtype, seeds=(121, 122, 123))
    O, L = run_variant(c, window, softcap)
    O_ref, L_ref = oracle.attention_variant(c.q, c.k, c.v, causal, window, softcap, c.scale,
                                            dtype)
    assert_parity(from_dev_f64(O), O_ref, L.cpu().numpy(), L_ref, "variant")


def test_window_closed_forms_and_long_window_equals_attn_fwd():
    import exact_attention_08_amd as attn
    say("variant: window 1, window >= N, zero-query counts")
    c = prefill_case(2, 8, 2, 300, 128, True, BF16, seeds=(124, 125, 126))
    # a window of one key: each row returns its own V row exactly
    O, L = run_variant(c, 1, 0.0)
    Vrep = np.repeat(c.v, 4, axis=1)
    assert np.array_equal(bits_of(O), Vrep)
    # a window at least the sequence length: attn_fwd bit for bit
    O2, L2 = run_variant(c, 300, 0.0)
    Q, K, V = (to_dev(x, BF16) for x in (c.q, c.k, c.v))
    O3 = torch.empty_like(Q)
    L3 = torch.empty_like(L2)
    attn.attn_fwd(Q, K, V, O3, L3, True, c.scale)
    torch.cuda.synchronize()
    assert torch.equal(O2, O3) and torch.equal(L2, L3)
    # zero queries: every visible key weighs the same; exp(LSE) counts the window
    for w in (7, 64, 100):
        _, L0 = run_variant(c, w, 0.0, q=np.zeros_like(c.q))
        cnt = np.round(np.exp(L0.cpu().numpy().astype(np.float64)))
        want = np.minimum(np.arange(300) + 1, w).astype(float)
        assert np.array_equal(cnt, np.broadcast_to(want, cnt.shape)), w


# window 4096 with soft-cap 50 is the benchmark's variant workload
@pytest.mark.parametrize("window", [1024, 4096])
def test_variant_llama3_8b_sized_sampled_rows(window):
    say(f"variant: Llama-3-8B heads, N 8192, window {window}, soft-cap 50")
    c = prefill_case(1, 32, 8, 8192, 128, True, BF16, seeds=(127, 128, 129))
    O, L = run_variant(c, window, 50.0)
    assert torch.isfinite(O.float()).all() and torch.isfinite(L).all()
    rng = np.random.default_rng(130)
    rows = np.unique(np.concatenate([
        np.array([0, 1, window - 1, window, window + 1, 8191]), rng.integers(0, 8192, 40)]))
    flat = np.array([h * 8192 + i for h in (0, 3, 4, 31) for i in rows], np.int64)
    O_ref, L_ref = oracle.attention_variant(c.q, c.k, c.v, True, window, 50.0, c.scale, BF16,
                                            rows=flat)
    idx = torch.from_numpy(flat).cuda()
    assert_parity(from_dev_f64(O.view(-1, 128)[idx]), O_ref, L.view(-1)[idx].cpu().numpy(),
                  L_ref, "llama variant")
