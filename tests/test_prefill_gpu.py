"""GPU parity of attn_fwd (prefill) against the fp64 oracle, through the C ABI binding.

Small shapes are compared element by element over every output; they span several 128-row
query tiles and 64/128-key KV tiles and end on ragged tails.  The four named workloads are
run at their full sizes in the launch configuration the benchmark times and compared on
sampled rows, plus exact properties that hold at any size (the zero-query count test).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from attn_inputs import BF16, FP16, CONFIGS, bits_to_f64, config_case, prefill_case
from tests.gpu_util import assert_parity, bits_of, from_dev_f64, tdtype, to_dev

pytestmark = pytest.mark.gpu


def run_fwd(case, q_bits=None):
    import exact_attention_08_amd as attn
    Q = to_dev(case.q if q_bits is None else q_bits, case.dtype)
    K = to_dev(case.k, case.dtype)
    V = to_dev(case.v, case.dtype)
    O = torch.empty_like(Q)
    LSE = torch.empty(case.B, case.Hq, case.N, dtype=torch.float32, device="cuda")
    attn.attn_fwd(Q, K, V, O, LSE, case.causal, case.scale)
    torch.cuda.synchronize()
    return O, LSE


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SMALL = [
    # B, Hq, Hkv, N, d, causal, dtype
    (1, 1, 1, 256, 64, False, FP16),     # the single-head fp16 workload, full size
    (1, 1, 1, 256, 64, True, FP16),
    (2, 4, 2, 1, 128, True, BF16),
    (1, 2, 1, 17, 64, True, BF16),
    (1, 2, 2, 100, 128, False, BF16),
    (1, 4, 1, 129, 128, True, BF16),
    (2, 2, 1, 255, 64, True, BF16),
    (1, 2, 2, 257, 64, False, FP16),
    (1, 8, 2, 300, 128, True, FP16),
    (2, 4, 4, 1000, 64, True, BF16),      # the handbook's ragged N=1000 test size
    (1, 8, 2, 1000, 128, False, BF16),
    (1, 4, 1, 640, 128, True, BF16),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,dtype", SMALL)
def test_prefill_small_all_elements(B, Hq, Hkv, N, d, causal, dtype):
    say(f"prefill small B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal{causal} dtype{dtype}")
    case = prefill_case(B, Hq, Hkv, N, d, causal, dtype)
    O, LSE = run_fwd(case)
    O_ref, L_ref = oracle.attention(case.q, case.k, case.v, causal, case.scale, dtype)
    assert_parity(from_dev_f64(O), O_ref, LSE.cpu().numpy(), L_ref, "prefill")


# Short sequences with more query tiles than resident workgroup slots (768 at d = 64, 512 at
# d = 128) run on the persistent grid, where one workgroup takes several items in turn.
PERSISTENT = [
    (16, 16, 16, 400, 64, True, BF16),
    (8, 16, 4, 520, 128, True, FP16),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,dtype", PERSISTENT)
def test_prefill_persistent_grid_all_elements(B, Hq, Hkv, N, d, causal, dtype):
    say(f"prefill persistent B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal{causal} dtype{dtype}")
    case = prefill_case(B, Hq, Hkv, N, d, causal, dtype, seeds=(11, 12, 13))
    O, LSE = run_fwd(case)
    O_ref, L_ref = oracle.attention(case.q, case.k, case.v, causal, case.scale, dtype)
    assert_parity(from_dev_f64(O), O_ref, LSE.cpu().numpy(), L_ref, "prefill persistent")


def test_prefill_repeated_and_concurrent_launches_agree_bitwise():
    # Back-to-back runs and runs on two streams at once (the persistent grid) give identical
    # bits: the kernel keeps no state between launches.
    import exact_attention_08_amd as attn
    say("prefill repeated/concurrent launches")
    case = prefill_case(16, 16, 16, 400, 64, True, BF16, seeds=(14, 15, 16))
    Q, K, V = (to_dev(x, case.dtype) for x in (case.q, case.k, case.v))
    outs = []
    for _ in range(3):
        O = torch.empty_like(Q)
        L = torch.empty(case.B, case.Hq, case.N, dtype=torch.float32, device="cuda")
        attn.attn_fwd(Q, K, V, O, L, case.causal, case.scale)
        outs.append((O, L))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for st in streams:
        O = torch.empty_like(Q)
        L = torch.empty(case.B, case.Hq, case.N, dtype=torch.float32, device="cuda")
        with torch.cuda.stream(st):
            attn.attn_fwd(Q, K, V, O, L, case.causal, case.scale, stream=st)
        outs.append((O, L))
    torch.cuda.synchronize()
    for O, L in outs[1:]:
        assert torch.equal(O, outs[0][0]) and torch.equal(L, outs[0][1])
    rows = np.arange(0, case.B * case.Hq * case.N, 997, dtype=np.int64)
    O_ref, L_ref = oracle.attention(case.q, case.k, case.v, True, case.scale, BF16, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    assert_parity(from_dev_f64(outs[0][0].view(-1, case.d)[idx]), O_ref,
                  outs[0][1].view(-1)[idx].cpu().numpy(), L_ref, "repeated")


@pytest.mark.parametrize("N,d,causal", [(1, 64, True), (200, 128, True), (333, 64, False),
                                        (1024, 128, True)])
def test_prefill_zero_queries_count_visible_keys(N, d, causal):
    # Q = 0: every score is exactly 0, every weight exactly 1, l an exact integer, so
    # exp(LSE) must round to the number of visible keys and O must be the mean of V.
    say(f"prefill count N{N} d{d} causal{causal}")
    case = prefill_case(1, 2, 1, N, d, causal, BF16, seeds=(5, 6, 7))
    O, LSE = run_fwd(case, q_bits=np.zeros_like(case.q))
    cnt = np.round(np.exp(LSE.cpu().numpy().astype(np.float64)))
    want = (np.arange(N) + 1.0) if causal else np.full(N, float(N))
    assert np.array_equal(cnt[0, 0], want) and np.array_equal(cnt[0, 1], want)
    O_ref, _ = oracle.attention(np.zeros_like(case.q), case.k, case.v, causal, case.scale, BF16)
    assert_parity(from_dev_f64(O), O_ref, what="uniform")


def test_prefill_causal_row0_is_v0_bitwise_and_runs_are_deterministic():
    case = prefill_case(2, 4, 2, 300, 128, True, BF16, seeds=(8, 9, 10))
    O1, L1 = run_fwd(case)
    O2, L2 = run_fwd(case)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    o = bits_of(O1)
    v = case.v
    for b in range(2):
        for h in range(4):
            assert np.array_equal(o[b, h, 0], v[b, h // 2, 0])


@pytest.mark.parametrize("name", [n for n, c in CONFIGS.items() if c["kind"] == "prefill"])
def test_prefill_named_workloads_full_size_sampled_rows(name):
    c = CONFIGS[name]
    say(f"prefill full size {name}")
    case = config_case(name)
    O, LSE = run_fwd(case)
    B, Hq, N, d = case.B, case.Hq, case.N, case.d
    rng = np.random.default_rng(2024)
    heads = sorted(h for h in {0, 1, Hq // 2, Hq - 1} if h < Hq)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, N // 2, N - 129, N - 128, N - 2, N - 1]
    rows = []
    for b in sorted({0, B - 1}):
        for h in heads:
            for i in sorted({x for x in fixed if 0 <= x < N} | set(rng.integers(0, N, 12).tolist())):
                rows.append((b * Hq + h) * N + i)
    rows = np.array(rows, dtype=np.int64)
    O_ref, L_ref = oracle.attention(case.q, case.k, case.v, case.causal, case.scale, case.dtype,
                                    rows=rows)
    idx = torch.from_numpy(rows).cuda()
    Og = from_dev_f64(O.view(-1, d)[idx])
    Lg = LSE.view(-1)[idx].cpu().numpy()
    assert_parity(Og, O_ref, Lg, L_ref, name)
    assert torch.isfinite(LSE).all()
    # the whole output is finite
    assert torch.isfinite(O.float()).all()
