"""GPU parity of attn_fwd (prefill) against the fp64 oracle, through the C ABI binding.

Every output starts as NaN (O) and +inf (LSE) before a launch, so a row that the grid never
writes fails every check.  Small shapes are compared element by element over every output;
they span several 128-row query tiles and 64/128-key KV tiles and end on ragged tails.  The
named workloads run at their full sizes in the launch configuration the benchmark times:
the single-head, GPT-2-medium and N = 8192 ones are compared with the oracle on every
element (head size 128 beyond 2048 keys runs the 64-rows-per-wave kernel, which is also
checked on every element at smaller sizes); at N = 32768 (8.8 TFLOP of fp64 for the whole output) four rows of every (head,
128-row query tile) pair are, one in each wave's 32 rows and both tile edges among them.
At full size the zero-query test also checks every row exactly: each score is 0, so
exp(LSE) must round to the number of visible keys and O must be the mean of the visible V
rows (a closed form computed here in fp64).
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
    O = torch.full_like(Q, float("nan"))
    LSE = torch.full((case.B, case.Hq, case.N), float("inf"), dtype=torch.float32, device="cuda")
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
# d = 128) run on the persistent grid, where one workgroup takes several items in turn, in
# head-major rounds and then a tail ordered by tile weight.
PERSISTENT = [
    (16, 16, 16, 400, 64, True, BF16),
    (8, 16, 4, 520, 128, True, FP16),
    # head groups not a multiple of 8 (one item list for the whole grid): two rounds (the
    # whole order sorted by tile weight), and five (head-major rounds, then the sorted tail)
    (9, 12, 3, 900, 64, True, BF16),
    (25, 16, 4, 1024, 64, True, BF16),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,dtype", PERSISTENT)
def test_prefill_persistent_grid_all_elements(B, Hq, Hkv, N, d, causal, dtype):
    say(f"prefill persistent B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal{causal} dtype{dtype}")
    case = prefill_case(B, Hq, Hkv, N, d, causal, dtype, seeds=(11, 12, 13))
    O, LSE = run_fwd(case)
    O_ref, L_ref = oracle.attention(case.q, case.k, case.v, causal, case.scale, dtype)
    assert_parity(from_dev_f64(O), O_ref, LSE.cpu().numpy(), L_ref, "prefill persistent")


# Head size 128 with more than 2048 keys and at least two 256-row items per CU runs the
# 64-rows-per-wave kernel: both dtypes, causal and not, grouped heads, N a multiple of
# neither 64 nor 256 (ragged last KV tile and query tile), several items per head group.
D128 = [
    (1, 32, 8, 4096, 128, True, BF16),
    (1, 48, 6, 3001, 128, True, FP16),
    (2, 16, 2, 4160, 128, False, BF16),
    (2, 16, 4, 4100, 128, True, FP16),
    (2, 16, 16, 4096, 128, True, BF16),   # one query head per kv head
    (4, 32, 8, 2049, 128, True, BF16),    # the last 256-row tile holds one row
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,dtype", D128)
def test_prefill_d128_kernel_all_elements(B, Hq, Hkv, N, d, causal, dtype):
    say(f"prefill d128 kernel B{B} Hq{Hq} Hkv{Hkv} N{N} causal{causal} dtype{dtype}")
    case = prefill_case(B, Hq, Hkv, N, d, causal, dtype, seeds=(21, 22, 23))
    O, LSE = run_fwd(case)
    O_ref, L_ref = oracle.attention(case.q, case.k, case.v, causal, case.scale, dtype)
    assert_parity(from_dev_f64(O), O_ref, LSE.cpu().numpy(), L_ref, "prefill d128")


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


def algorithmic_flops(c):
    f = 4.0 * c["B"] * c["Hq"] * c["N"] * c["N"] * c["d"]
    return f / 2 if c["causal"] else f


PREFILL_NAMES = [n for n, c in CONFIGS.items() if c["kind"] == "prefill"]
# up to ~0.6 TFLOP the whole output is compared (about a minute of fp64 on 16 host cores)
EVERY_ELEMENT = [n for n in PREFILL_NAMES if algorithmic_flops(CONFIGS[n]) <= 6e11]
PER_TILE = [n for n in PREFILL_NAMES if n not in EVERY_ELEMENT]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", EVERY_ELEMENT)
def test_prefill_named_workload_every_element(name):
    say(f"prefill full size, every element: {name}")
    case = config_case(name)
    O, LSE = run_fwd(case)
    Og = from_dev_f64(O)
    Lg = LSE.cpu().numpy()
    del O, LSE
    say(f"  oracle over {case.B * case.Hq * case.N} rows")
    O_ref, L_ref = oracle.attention(case.q, case.k, case.v, case.causal, case.scale, case.dtype)
    assert_parity(Og, O_ref, Lg, L_ref, name)


def tile_rows(case, seed):
    """Four rows of every (batch, head, 128-row query tile): the tile's first row (wave 0),
    a random row of wave 1 and of wave 2, and the tile's last row (wave 3); tails clipped."""
    rng = np.random.default_rng(seed)
    B, Hq, N = case.B, case.Hq, case.N
    n_t = (N + 127) // 128
    t0 = np.arange(n_t, dtype=np.int64) * 128
    rows = []
    for bh in range(B * Hq):
        picks = [t0, t0 + 32 + rng.integers(0, 32, n_t), t0 + 64 + rng.integers(0, 32, n_t),
                 t0 + 127]
        r = np.unique(np.minimum(np.concatenate(picks), N - 1))
        rows.append(bh * N + r)
    return np.concatenate(rows)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", PER_TILE)
def test_prefill_named_workload_every_query_tile(name):
    say(f"prefill full size, every query tile: {name}")
    case = config_case(name)
    O, LSE = run_fwd(case)
    # every row was written: nothing is left at the NaN / +inf it started as
    assert torch.isfinite(LSE).all()
    assert not torch.isnan(O).any()
    rows = tile_rows(case, 2024)
    say(f"  oracle over {len(rows)} rows")
    O_ref, L_ref = oracle.attention(case.q, case.k, case.v, case.causal, case.scale, case.dtype,
                                    rows=rows)
    idx = torch.from_numpy(rows).cuda()
    assert_parity(from_dev_f64(O.view(-1, case.d)[idx]), O_ref, LSE.view(-1)[idx].cpu().numpy(),
                  L_ref, name)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", [n for n in PREFILL_NAMES
                                  if CONFIGS[n]["B"] * CONFIGS[n]["N"] >= 8192])
def test_prefill_zero_queries_every_row_full_size(name):
    """Q = 0 at full size: exp(LSE) rounds to i + 1 (causal) or N for every row of every head,
    and O equals the running mean of V, computed here in fp64 by a cumulative sum."""
    say(f"prefill zero-query count, full size: {name}")
    case = config_case(name)
    B, Hq, Hkv, N, d = case.B, case.Hq, case.Hkv, case.N, case.d
    O, LSE = run_fwd(case, q_bits=np.zeros_like(case.q))
    cnt = np.round(np.exp(LSE.cpu().numpy().astype(np.float64)))
    want = (np.arange(N) + 1.0) if case.causal else np.full(N, float(N))
    bad = cnt != want[None, None, :]
    assert not bad.any(), f"{bad.sum()} rows count the wrong number of keys"
    G = Hq // Hkv
    Og = from_dev_f64(O)
    for b in range(B):
        for kvh in range(Hkv):
            v = bits_to_f64(case.v[b, kvh], case.dtype)
            if case.causal:
                mean = np.cumsum(v, axis=0) / (np.arange(N, dtype=np.float64) + 1.0)[:, None]
            else:
                mean = np.broadcast_to(v.mean(axis=0), (N, d))
            assert_parity(Og[b, kvh * G:(kvh + 1) * G], np.broadcast_to(mean, (G, N, d)),
                          what=f"{name} uniform b{b} kvh{kvh}")
