"""GPU tests of the balanced split (split_tokens = 0) and of graph capture.

The balanced split is chosen on the device from the lengths in device memory; its result
must equal, bit for bit, a call with that split given explicitly (the rule is restated
here from the header's description), and match the oracle.  Calls captured in a HIP graph
(torch.cuda.CUDAGraph) are replayed several times, with the lengths and inputs in the
captured buffers changed between replays and eager work in between; every replay must equal
the eager call on the same data bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from attn_inputs import (BF16, FP16, decode_case, log_uniform_ctx, paged_prefill_case,
                         prefill_case)
from tests.gpu_util import assert_parity, from_dev_f64, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def n_cu():
    return torch.cuda.get_device_properties(0).multi_processor_count


def balanced_split(ctx_lens, Hkv):
    per = int(np.sum(np.maximum(np.asarray(ctx_lens, np.int64), 0))) * Hkv // n_cu()
    return 256 if per <= 128 else 512 if per <= 3072 else 1024 if per <= 10240 else 2048


class Decode:
    def __init__(self, case):
        import exact_attention_08_amd as attn
        self.attn, self.c = attn, case
        self.q = to_dev(case.q, case.dtype)
        self.K = to_dev(case.k_pages, case.dtype)
        self.V = to_dev(case.v_pages, case.dtype)
        self.bt = torch.from_numpy(case.block_table).cuda()
        self.ctx = torch.from_numpy(case.ctx_lens).cuda()
        self.O = torch.empty_like(self.q)
        self.L = torch.empty(case.B, case.Hq, dtype=torch.float32, device="cuda")
        self.ws = torch.zeros(attn.attn_decode_paged_workspace_bytes(
            case.B, case.Hq, case.d, 16, case.max_pages, 0), dtype=torch.uint8, device="cuda")

    def __call__(self, split, O=None, L=None):
        self.attn.attn_decode_paged(self.q, self.K, self.V, self.bt, self.ctx,
                                    self.O if O is None else O, self.L if L is None else L,
                                    split, self.ws, self.c.scale)


@pytest.mark.parametrize("name,ctx,dtype", [
    ("one short", [2048], BF16),                                     # -> 256
    ("eight x 4096", [4096] * 8, FP16),                              # -> 512
    ("16 log-uniform", log_uniform_ctx(16, 512, 32768), BF16),       # -> 1024
    ("64 log-uniform", log_uniform_ctx(64, 512, 32768), BF16),       # -> 2048
    ("ragged", [0, 1, 17, 9000, 300, 4095], BF16),
])
def test_balanced_split_equals_the_explicit_split_bitwise(name, ctx, dtype):
    ctx = np.asarray(ctx, np.int32)
    L_exp = balanced_split(ctx, 8)
    say(f"balanced split {name}: expect {L_exp}")
    case = decode_case(len(ctx), 32, 8, 128, ctx, 16, dtype, seeds=(51, 52, 53),
                       max_pages=max(1, int((ctx.max() + 15) // 16)))
    d = Decode(case)
    d(0)
    O0, L0 = d.O.clone(), d.L.clone()
    d(L_exp)
    torch.cuda.synchronize()
    assert torch.equal(O0, d.O) and torch.equal(L0, d.L)
    if len(ctx) <= 8:
        O_ref, L_ref = oracle.decode_paged(case.q, case.k_pages, case.v_pages, case.block_table,
                                           case.ctx_lens, case.scale, dtype)
        live = case.ctx_lens > 0
        assert_parity(from_dev_f64(O0)[live], O_ref[live], L0.cpu().numpy()[live], L_ref[live],
                      name)


def test_decode_graph_replays_follow_changing_lengths():
    say("graph: balanced decode, lengths changed between replays")
    B, maxc = 16, 8192
    case = decode_case(B, 32, 8, 128, [maxc] * B, 16, BF16, seeds=(54, 55, 56))
    d = Decode(case)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d(0)
    rng = np.random.default_rng(57)
    sets = [np.full(B, maxc), rng.integers(0, maxc, B), np.full(B, 16), np.full(B, maxc),
            rng.integers(0, 64, B)]
    seen = set()
    for i, lens in enumerate(sets):
        lens = lens.astype(np.int32)
        d.ctx.copy_(torch.from_numpy(lens))
        d.q.copy_(to_dev(np.roll(case.q, i, axis=0), BF16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Og, Lg = d.O.clone(), d.L.clone()
        O2, L2 = torch.empty_like(Og), torch.empty_like(Lg)
        d(0, O2, L2)                                   # eager, same data
        O3, L3 = torch.empty_like(Og), torch.empty_like(Lg)
        L_exp = balanced_split(lens, 8)
        seen.add(L_exp)
        d(L_exp, O3, L3)                               # eager, the split given explicitly
        torch.cuda.synchronize()
        assert torch.equal(Og, O2) and torch.equal(Lg, L2), f"replay {i}"
        assert torch.equal(Og, O3) and torch.equal(Lg, L3), f"replay {i} vs split {L_exp}"
    assert seen == {256, 512, 1024}


def test_decode_graphs_on_two_streams_with_eager_calls_between():
    """The decode keeps no state outside the caller's workspace: two captured graphs (each
    with its own workspace) replayed at the same time on two streams, while more than 64
    eager calls run on a third workspace, all give the eager result bit for bit."""
    import exact_attention_08_amd as attn
    say("graph: two decode graphs on two streams, 80 eager calls in between")
    ca = decode_case(12, 32, 8, 128, log_uniform_ctx(12, 512, 16384, seed=71), 16, BF16,
                     seeds=(72, 73, 74))
    cb = decode_case(5, 16, 4, 64, [3000, 17, 0, 900, 5000], 16, FP16, seeds=(75, 76, 77))
    da, db = Decode(ca), Decode(cb)
    # eager references, each on a workspace of its own
    ref = {}
    for key, d, split in (("a", da, 0), ("b", db, 512)):
        ws = torch.zeros(attn.attn_decode_paged_workspace_bytes(
            d.c.B, d.c.Hq, d.c.d, 16, d.c.max_pages, split), dtype=torch.uint8, device="cuda")
        O, L = torch.empty_like(d.O), torch.empty_like(d.L)
        attn.attn_decode_paged(d.q, d.K, d.V, d.bt, d.ctx, O, L, split, ws, d.c.scale)
        ref[key] = (O, L, ws)
    torch.cuda.synchronize()
    graphs = {}
    for key, d, split in (("a", da, 0), ("b", db, 512)):
        if split:
            d.ws = torch.zeros(attn.attn_decode_paged_workspace_bytes(
                d.c.B, d.c.Hq, d.c.d, 16, d.c.max_pages, split), dtype=torch.uint8,
                device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            d(split)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            d(split)
        graphs[key] = g
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        da.O.zero_()
        db.O.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            graphs["a"].replay()
        with torch.cuda.stream(s2):
            graphs["b"].replay()
        eager = []
        wa = ref["a"][2]
        for i in range(80):
            O, L = torch.empty_like(da.O), torch.empty_like(da.L)
            attn.attn_decode_paged(da.q, da.K, da.V, da.bt, da.ctx, O, L, 0, wa, ca.scale)
            eager.append((O, L))
        torch.cuda.synchronize()
        assert torch.equal(da.O, ref["a"][0]) and torch.equal(da.L, ref["a"][1]), f"graph a {rep}"
        assert torch.equal(db.O, ref["b"][0]) and torch.equal(db.L, ref["b"][1]), f"graph b {rep}"
        for i, (O, L) in enumerate(eager):
            assert torch.equal(O, ref["a"][0]) and torch.equal(L, ref["a"][1]), f"eager {i}"
    for key, c in (("a", ca), ("b", cb)):
        O_ref, L_ref = oracle.decode_paged(c.q, c.k_pages, c.v_pages, c.block_table, c.ctx_lens,
                                           c.scale, c.dtype)
        live = c.ctx_lens > 0
        assert_parity(from_dev_f64(ref[key][0])[live], O_ref[live],
                      ref[key][1].cpu().numpy()[live], L_ref[live], f"graph {key}")


def test_prefill_and_paged_prefill_graph_replays_equal_eager():
    import exact_attention_08_amd as attn
    say("graph: attn_fwd and attn_prefill_paged replays")
    c = prefill_case(2, 8, 2, 700, 128, True, BF16, seeds=(58, 59, 60))
    Q, K, V = (to_dev(x, BF16) for x in (c.q, c.k, c.v))
    O = torch.empty_like(Q)
    L = torch.empty(2, 8, 700, dtype=torch.float32, device="cuda")
    p = paged_prefill_case(32, 8, 128, [100, 37, 300], [900, 37, 2000], 16, FP16, True,
                           seeds=(61, 62, 63))
    pq = to_dev(p.q, FP16)
    pk, pv = to_dev(p.k_pages, FP16), to_dev(p.v_pages, FP16)
    pbt = torch.from_numpy(p.block_table).cuda()
    pcu = torch.from_numpy(p.cu_seqlens_q).cuda()
    pkv = torch.from_numpy(p.kv_lens).cuda()
    PO = torch.empty_like(pq)
    PL = torch.empty(p.total_q, 32, dtype=torch.float32, device="cuda")

    def both(o=O, lse=L, po=PO, pl=PL):
        attn.attn_fwd(Q, K, V, o, lse, True, c.scale)
        attn.attn_prefill_paged(pq, pk, pv, pbt, pcu, pkv, po, pl, p.max_q_len, True, p.scale)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        both()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        both()
    for i in range(4):
        Q.copy_(to_dev(np.roll(c.q, i, axis=2), BF16))
        # new chunk lengths within the captured max_q_len, and new cache lengths
        qn = np.array([100, 37 - 9 * (i % 2), 300 - 50 * i], np.int32)
        cu = np.zeros(4, np.int32)
        cu[1:] = np.cumsum(qn)
        pcu.copy_(torch.from_numpy(cu))
        pkv.copy_(torch.from_numpy(np.array([900 - i, 37, 2000 - 100 * i], np.int32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Og, Lg, POg, PLg = O.clone(), L.clone(), PO.clone(), PL.clone()
        O2, L2, PO2, PL2 = (torch.empty_like(t) for t in (O, L, PO, PL))
        PO2.copy_(PO)
        PL2.copy_(PL)
        both(O2, L2, PO2, PL2)
        torch.cuda.synchronize()
        assert torch.equal(Og, O2) and torch.equal(Lg, L2), f"attn_fwd replay {i}"
        n = int(cu[-1])
        assert torch.equal(POg[:n], PO2[:n]) and torch.equal(PLg[:n], PL2[:n]), \
            f"paged prefill replay {i}"


def test_cascade_with_balanced_split_equals_the_explicit_split_bitwise():
    import exact_attention_08_amd as attn
    from attn_inputs import cascade_case
    say("balanced split in the cascade decode")
    own = [0, 300, 4096, 17, 1000, 2048, 5, 64]
    c = cascade_case(len(own), 32, 8, 128, 3000, own, 16, BF16, seeds=(131, 132, 133))
    q = to_dev(c.q, BF16)
    K, V = to_dev(c.k_pages, BF16), to_dev(c.v_pages, BF16)
    kpre, vpre = to_dev(c.extra["k_prefix"], BF16), to_dev(c.extra["v_prefix"], BF16)
    bt = torch.from_numpy(c.block_table).cuda()
    ctx = torch.from_numpy(c.ctx_lens).cuda()
    ws = torch.zeros(attn.attn_decode_cascade_workspace_bytes(c.B, 32, 128, 16, c.max_pages, 0,
                                                              3000),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for split in (0, balanced_split(own, 8)):
        O = torch.empty_like(q)
        L = torch.empty(c.B, 32, dtype=torch.float32, device="cuda")
        attn.attn_decode_cascade(q, kpre, vpre, K, V, bt, ctx, O, L, split, ws, c.scale)
        torch.cuda.synchronize()
        outs.append((O, L))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    O_ref, L_ref = oracle.decode_cascade(c.q, c.extra["k_prefix"], c.extra["v_prefix"],
                                         c.k_pages, c.v_pages, c.block_table, c.ctx_lens,
                                         c.scale, BF16)
    assert_parity(from_dev_f64(outs[0][0]), O_ref, outs[0][1].cpu().numpy(), L_ref, "cascade balanced")
