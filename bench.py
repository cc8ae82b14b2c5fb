#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  1. attn_fwd on the GPT-2-medium-shaped causal prefill (B=64, H=16, N=1024, d=64, bf16);
  2. attn_decode_paged on the paged GQA decode batch (64 sequences, Hq=32, Hkv=8, d=128,
     16-token pages, log-uniform contexts in [512, 32768], 1024-token splits, bf16).
Inputs are generated (seeded) and uploaded before the timed region.  W warm-up steps, then
exactly K timed steps bracketed by torch.cuda.synchronize().  HIP events recorded on the
stream the library launches on (torch's current stream) give each call's average duration.

Printed: one JSON line.  `value` is the prefill throughput in TFLOP/s (algorithmic FLOPs:
4*B*H*N^2*d/2 for causal); the decode half of the metric is in `decode` (algorithmic bytes:
every K/V element of every context read once, plus q, O, block table and lengths).
`roofline` covers the prefill kernel, `decode.roofline` the decode call; `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workloads.  Outside the step
(skipped with --no-extra): the Llama-3-8B prefill shapes, the shared-prefix decode
(attn_decode_cascade) next to the same requests through attn_decode_paged, and chunked
prefill over a paged cache (attn_prefill_paged), the sliding-window + soft-cap prefill
(attn_fwd_variant), and the read bandwidth a plain streaming
kernel reaches (the practical HBM ceiling).

    python bench.py [--gpus 1] [--steps 50] [--warmup 50] [--cpu-seconds 10] [--no-extra]

The GPU takes tens of milliseconds of sustained launches to reach its steady clock (a fresh
N = 8192 prefill runs ~15% slower over its first ~30 launches), so the step's warm-up runs
the --warmup steps and continues until 0.3 s of launches have passed, and the figures
outside the step warm up for 0.1 s before they are timed.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA
PREFILL = "gpt2_medium_b64_h16_n1024_d64_causal"
DECODE = "paged_gqa_decode_b64_ctx512_32768"
EXTRA = ["llama3_8b_prefill_n8192_causal", "llama3_8b_prefill_n32768_causal"]
CASCADE = "cascade_gqa_decode_b64_prefix8192_own128_4096"
PAGED_PREFILL = "chunked_prefill_b16_hist1024_16384_chunk256_2048"
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
WARM_SECONDS = 0.3             # minimum warm-up of the step (steady clock), whatever --warmup


def prefill_flops(c):
    f = 4.0 * c.B * c.Hq * c.N * c.N * c.d
    return f * 0.5 if c.causal else f


def prefill_bytes(c):
    e = 2
    return (2 * c.B * c.Hq * c.N * c.d * e          # Q read, O written
            + 2 * c.B * c.Hkv * c.N * c.d * e       # K, V read
            + c.B * c.Hq * c.N * 4)                 # LSE written


def decode_bytes(c):
    tokens = int(c.ctx_lens.astype("int64").sum())
    pages = int(((c.ctx_lens.astype("int64") + c.page_size - 1) // c.page_size).sum())
    kv = tokens * c.Hkv * c.d * 2 * 2               # K and V, bf16, each element once
    qo = 2 * c.B * c.Hq * c.d * 2                   # q read, O written
    meta = pages * 4 + c.B * 4 + c.B * c.Hq * 4     # block-table entries, lengths, LSE
    return kv + qo + meta, kv


def decode_flops(c):
    return 4.0 * c.Hq * c.d * float(c.ctx_lens.astype("int64").sum())


def cascade_bytes(c, prefix_len):
    """Algorithmic bytes of a shared-prefix decode: the prefix K/V once, every request's own
    K/V once, q read, O written, table entries, lengths and LSE."""
    own, _ = decode_bytes(c)
    return own + prefix_len * c.Hkv * c.d * 2 * 2


def paged_prefill_flops(c):
    """Algorithmic FLOPs of a paged / varlen prefill: 4 * Hq * d per visible (query, key)
    pair; causal query i of a request sees kv_len - q_len + i + 1 keys."""
    pairs = 0
    for ql, kl in zip(c.q_lens.astype("int64"), c.kv_lens.astype("int64")):
        ql, kl = int(ql), int(kl)
        pairs += ql * kl if not c.causal else ql * (kl - ql) + ql * (ql + 1) // 2
    return 4.0 * c.Hq * c.d * pairs


def warm(fn, torch, seconds=0.1, min_calls=3):
    """Untimed calls until `seconds` of sustained GPU work have passed (steady clock)."""
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def paged_prefill_figure(attn, torch, dev, log, reps=10):
    """Chunked prefill over a paged cache (PAGED_PREFILL workload).  Returns a dict for the
    JSON line."""
    from attn_inputs import paged_prefill_workload
    log(f"bench: extra figure {PAGED_PREFILL}")
    c = paged_prefill_workload(PAGED_PREFILL)
    q = to_dev(c.q, c.dtype)
    kp, vp = to_dev(c.k_pages, c.dtype), to_dev(c.v_pages, c.dtype)
    bt = torch.from_numpy(c.block_table).to(dev)
    cu = torch.from_numpy(c.cu_seqlens_q).to(dev)
    kvl = torch.from_numpy(c.kv_lens).to(dev)
    O = torch.empty_like(q)
    L = torch.empty(c.total_q, c.Hq, dtype=torch.float32, device=dev)

    def call():
        attn.attn_prefill_paged(q, kp, vp, bt, cu, kvl, O, L, c.max_q_len, c.causal, c.scale)

    warm(call, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    assert torch.isfinite(L).all(), "paged prefill produced a non-finite LSE"
    tf = paged_prefill_flops(c) / t / 1e12
    return {"workload": PAGED_PREFILL, "avg_launch_us": round(t * 1e6, 1),
            "algorithmic_flops_per_launch": paged_prefill_flops(c),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_TFLOPS, 4),
                         "kernel": "prefill_fwd_kernel<128,bf16,causal,paged>"},
            "total_q": c.total_q, "total_kv": int(c.kv_lens.astype("int64").sum())}


VARIANT = dict(name="llama3_8b_prefill_n8192_window4096_softcap50", B=1, Hq=32, Hkv=8,
               N=8192, d=128, window=4096, softcap=50.0)


def variant_flops(v):
    """Algorithmic FLOPs of causal attention with a sliding window: 4 * d per visible
    (query, key) pair; query i sees min(i + 1, window) keys."""
    i = __import__("numpy").arange(v["N"], dtype="int64")
    pairs = int(__import__("numpy").minimum(i + 1, v["window"]).sum())
    return 4.0 * v["B"] * v["Hq"] * v["d"] * pairs


def variant_figure(attn, torch, dev, log, reps=10):
    """attn_fwd_variant at Llama-3-8B heads with a 4096-key window and soft-cap 50."""
    from attn_inputs import prefill_case
    v = VARIANT
    log(f"bench: extra figure {v['name']}")
    c = prefill_case(v["B"], v["Hq"], v["Hkv"], v["N"], v["d"], True)
    Q, K, V = (to_dev(x, c.dtype) for x in (c.q, c.k, c.v))
    O = torch.empty_like(Q)
    L = torch.empty(v["B"], v["Hq"], v["N"], dtype=torch.float32, device=dev)

    def call():
        attn.attn_fwd_variant(Q, K, V, O, L, True, v["window"], v["softcap"], c.scale)

    warm(call, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    assert torch.isfinite(L).all()
    tf = variant_flops(v) / t / 1e12
    return {"workload": v["name"], "avg_launch_us": round(t * 1e6, 1),
            "algorithmic_flops_per_launch": variant_flops(v),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_TFLOPS, 4),
                         "kernel": "prefill_fwd_kernel<128,bf16,causal,window+softcap>"}}


def hbm_read_ceiling(torch, dev, log, gib=2, reps=5):
    """GB/s of a plain streaming-read kernel (libhbmprobe.so) over a 2 GiB buffer: the HBM
    bandwidth a simple kernel reaches here, as context for the decode's fraction."""
    import ctypes
    path = os.path.join(ROOT, "exact_attention_08_amd", "libhbmprobe.so")
    if not os.path.exists(path):
        log("bench: libhbmprobe.so not built; no HBM ceiling figure")
        return None
    lib = ctypes.CDLL(path)
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_void_p]
    lib.hbm_read_probe.restype = ctypes.c_int
    nbytes = gib << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count * 8
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        assert lib.hbm_read_probe(src.data_ptr(), nbytes, out.data_ptr(), blocks, st) == 0
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, out
    torch.cuda.empty_cache()
    return {"gbs": round(best, 1), "frac_of_peak": round(best / HBM_PEAK_GBS, 4),
            "kernel": "hbm_read_kernel (16-byte non-temporal loads, 8 in flight per lane)",
            "bytes": nbytes, "note": "best of 5 reads of a 2 GiB buffer"}


def cascade_figure(attn, torch, dev, log):
    """Shared-prefix decode (CASCADE workload) against the same requests through the plain
    paged decode, whose block tables all point at one shared copy of the prefix pages (what
    a paged cache with prefix sharing holds).  Returns a dict for the JSON line."""
    import numpy as np
    from attn_inputs import CASCADE_WORKLOADS, cascade_workload
    cw = CASCADE_WORKLOADS[CASCADE]
    log(f"bench: extra figure {CASCADE}")
    c = cascade_workload(CASCADE)
    P, split, page = cw["prefix_len"], cw["split_tokens"], c.page_size
    assert P % page == 0, "the plain layout below starts each request's own tokens on a page"
    q = to_dev(c.q, c.dtype)
    kpre, vpre = to_dev(c.extra["k_prefix"], c.dtype), to_dev(c.extra["v_prefix"], c.dtype)
    kp, vp = to_dev(c.k_pages, c.dtype), to_dev(c.v_pages, c.dtype)
    bt = torch.from_numpy(c.block_table).to(dev)
    ctx = torch.from_numpy(c.ctx_lens).to(dev)
    O = torch.empty_like(q)
    L = torch.empty(c.B, c.Hq, dtype=torch.float32, device=dev)
    ws = torch.zeros(attn.attn_decode_cascade_workspace_bytes(c.B, c.Hq, c.d, page, c.max_pages,
                                                              split, P),
                     dtype=torch.uint8, device=dev)
    # the plain layout: prefix pages first in the pool, shared by every request's table
    npre = (P + page - 1) // page
    kpre_pages = kpre.permute(1, 0, 2).reshape(npre, page, c.Hkv, c.d)
    vpre_pages = vpre.permute(1, 0, 2).reshape(npre, page, c.Hkv, c.d)
    kp_all = torch.cat([kpre_pages, kp]).contiguous()
    vp_all = torch.cat([vpre_pages, vp]).contiguous()
    own_t = torch.from_numpy(c.block_table.astype(np.int64))
    bt_all = torch.full((c.B, npre + c.max_pages), -1, dtype=torch.int64)
    bt_all[:, :npre] = torch.arange(npre)
    bt_all[:, npre:] = torch.where(own_t >= 0, own_t + npre, own_t)
    bt_all = bt_all.to(torch.int32).to(dev)
    ctx_all = ctx + P
    O2 = torch.empty_like(q)
    L2 = torch.empty_like(L)
    ws2 = torch.zeros(attn.attn_decode_paged_workspace_bytes(c.B, c.Hq, c.d, page, npre + c.max_pages,
                                                             split), dtype=torch.uint8, device=dev)

    def timed(fn, reps=20):
        warm(fn, torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    t_c = timed(lambda: attn.attn_decode_cascade(q, kpre, vpre, kp, vp, bt, ctx, O, L, split, ws,
                                                 c.scale))
    t_p = timed(lambda: attn.attn_decode_paged(q, kp_all, vp_all, bt_all, ctx_all, O2, L2, split,
                                               ws2, c.scale))
    diff = float((O.float() - O2.float()).abs().max())
    assert diff < 0.05 and torch.isfinite(L).all(), f"cascade and plain decode disagree ({diff})"
    b = cascade_bytes(c, P)
    gbs = b / t_c / 1e9
    out = {"workload": CASCADE, "avg_call_us": round(t_c * 1e6, 1),
           "algorithmic_bytes_per_call": b, "gbs": round(gbs, 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "kernel": "prefill_fwd_kernel(prefix chunks) + decode_split_kernel + "
                                  "decode_merge_kernel"},
           "plain_paged_decode_us": round(t_p * 1e6, 1),
           "speedup_vs_plain": round(t_p / t_c, 2),
           "max_abs_diff_vs_plain": diff}
    del q, kpre, vpre, kp, vp, kp_all, vp_all, ws, ws2
    torch.cuda.empty_cache()
    return out


def source_digest(files):
    """Digest of the kernel sources with comments and whitespace removed, so that the
    committed counter measurements stay valid across comment-only edits and are dropped
    (traffic = null) as soon as the code changes."""
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "exact_attention_08_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, only if it was
    taken on the current kernel source."""
    path = os.path.join(TRAFFIC_DIR, f"{kernel_key}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != digest:
        return None
    return t.get("bytes_per_launch")


def to_dev(bits, dtype):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == 0 else torch.float16).cuda()


def cpu_baseline(pc, dc, seconds):
    """The fp64 oracle on a bounded sample: random prefill rows, then random decode
    (sequence, head) pairs, each leg running ~`seconds` of wall time on all host cores."""
    import numpy as np
    import oracle
    threads = oracle.threads()
    rng = np.random.default_rng(99)
    # prefill leg: batches of rows until the time budget is used
    rows_done, flops, t_pre = 0, 0.0, 0.0
    while t_pre < seconds:
        rows = rng.integers(0, pc.B * pc.Hq * pc.N, 8 * threads).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attention(pc.q, pc.k, pc.v, pc.causal, pc.scale, pc.dtype, rows=rows)
        t_pre += time.perf_counter() - t0
        i = rows % pc.N
        flops += float((4.0 * pc.d * ((i + 1) if pc.causal else np.full_like(i, pc.N))).sum())
        rows_done += len(rows)
    # decode leg
    pairs_done, kv_bytes, t_dec = 0, 0.0, 0.0
    while t_dec < seconds:
        pairs = rng.integers(0, dc.B * dc.Hq, threads).astype(np.int64)
        t0 = time.perf_counter()
        oracle.decode_paged(dc.q, dc.k_pages, dc.v_pages, dc.block_table, dc.ctx_lens, dc.scale,
                            dc.dtype, pairs=pairs)
        t_dec += time.perf_counter() - t0
        # per (sequence, head) the oracle reads that head's K/V rows once
        kv_bytes += float((dc.ctx_lens[pairs // dc.Hq].astype(np.int64) * dc.d * 2 * 2).sum())
        pairs_done += len(pairs)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": flops / t_pre / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": (f"{rows_done} random query rows of the B64 H16 N1024 d64 causal prefill, "
                   f"fp64, {t_pre:.1f} s"),
        "cpu": model,
        "decode": {"value": kv_bytes / t_dec / 1e9, "unit": "GB/s",
                   "sample": (f"{pairs_done} random (sequence, head) pairs of the paged decode "
                              f"batch, fp64, {t_dec:.1f} s; bytes = that head's K/V rows")},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--warm-seconds", type=float, default=WARM_SECONDS,
                    help="minimum duration of the step warm-up (0: exactly --warmup steps, "
                         "for counter collection)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the Llama-3-8B prefill, shared-prefix decode and paged prefill "
                         "figures")
    ap.add_argument("--only", choices=["prefill", "decode", "cascade", "paged_prefill"],
                    default=None,
                    help="(profiling) run only one half of the step, or only the shared-prefix "
                         "decode or the paged prefill figure")
    ap.add_argument("--profile-prefill", default=None, metavar="CONFIG",
                    help="(profiling) only run attn_fwd on the named prefill configuration "
                         "--steps times and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: this library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_08_amd as attn
    from attn_inputs import CONFIGS, config_case

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log = lambda m: print(m, file=sys.stderr, flush=True)  # noqa: E731

    if args.profile_prefill:
        from attn_inputs import config_case as _cc
        c = _cc(args.profile_prefill)
        Qp, Kp, Vp = (to_dev(x, c.dtype) for x in (c.q, c.k, c.v))
        Op = torch.empty_like(Qp)
        Lp = torch.empty(c.B, c.Hq, c.N, dtype=torch.float32, device=dev)
        for _ in range(args.steps):
            attn.attn_fwd(Qp, Kp, Vp, Op, Lp, c.causal, c.scale)
        torch.cuda.synchronize()
        print(json.dumps({"profiled": args.profile_prefill, "launches": args.steps}), flush=True)
        return
    if args.only == "cascade":
        print(json.dumps({"cascade_decode": cascade_figure(attn, torch, dev, log)}), flush=True)
        return
    if args.only == "paged_prefill":
        print(json.dumps({"paged_prefill": paged_prefill_figure(attn, torch, dev, log, reps=20)}),
              flush=True)
        return

    log("bench: generating inputs")
    pc = config_case(PREFILL)
    dc = config_case(DECODE)
    split = CONFIGS[DECODE]["split_tokens"]
    Q, K, V = (to_dev(x, pc.dtype) for x in (pc.q, pc.k, pc.v))
    O = torch.empty_like(Q)
    LSE = torch.empty(pc.B, pc.Hq, pc.N, dtype=torch.float32, device=dev)
    q = to_dev(dc.q, dc.dtype)
    kp, vp = to_dev(dc.k_pages, dc.dtype), to_dev(dc.v_pages, dc.dtype)
    bt = torch.from_numpy(dc.block_table).to(dev)
    ctx = torch.from_numpy(dc.ctx_lens).to(dev)
    Od = torch.empty_like(q)
    Ld = torch.empty(dc.B, dc.Hq, dtype=torch.float32, device=dev)
    ws = torch.zeros(attn.attn_decode_paged_workspace_bytes(dc.B, dc.Hq, dc.d, dc.page_size,
                                                            dc.max_pages, split),
                     dtype=torch.uint8, device=dev)
    # a plain copy of known size, for calibrating HBM counters when profiled
    cal = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    cal2 = torch.empty_like(cal)
    cal2.copy_(cal)
    torch.cuda.synchronize()

    do_pre = args.only in (None, "prefill")
    do_dec = args.only in (None, "decode")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if do_pre:
            attn.attn_fwd(Q, K, V, O, LSE, pc.causal, pc.scale)
        if ev is not None:
            ev[1].record()
        if do_dec:
            attn.attn_decode_paged(q, kp, vp, bt, ctx, Od, Ld, split, ws, dc.scale)
        if ev is not None:
            ev[2].record()

    # W warm-up steps, continued until WARM_SECONDS of sustained launches have passed: the
    # GPU reaches its steady clock only after tens of milliseconds of work, so a small W
    # alone would time part of the clock ramp.
    log(f"bench: {args.warmup} warm-up steps (at least {args.warm_seconds} s)")
    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_w < args.warm_seconds:
        step()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"bench: {args.steps} timed steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_pre = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps * 1e-3   # seconds
    t_dec = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps * 1e-3
    med_pre = float(np.median([e[0].elapsed_time(e[1]) for e in events])) * 1e-3
    med_dec = float(np.median([e[1].elapsed_time(e[2]) for e in events])) * 1e-3
    assert torch.isfinite(LSE).all() and torch.isfinite(Ld).all()

    fl = prefill_flops(pc)
    pb = prefill_bytes(pc)
    db, kv_only = decode_bytes(dc)
    pre_tflops = fl / t_pre / 1e12 if do_pre else None
    dec_gbs = db / t_dec / 1e9 if do_dec else None
    # the prefill's algorithmic intensity is below the ridge (8 TB/s x time > 2.5 PF x time),
    # so its roofline is the HBM one
    pre_bound_hbm = pb / (HBM_PEAK_GBS * 1e9) > fl / (MFMA_PEAK_TFLOPS * 1e12)
    pre_digest = source_digest(["attn_fwd.hip", "attn_common.h", "attn_prefill_common.h"])
    dec_digest = source_digest(["attn_decode.hip", "attn_common.h"])
    pre_traffic = load_traffic("prefill_fwd_gpt2_medium", pre_digest)
    dec_traffic = load_traffic("decode_paged_b64", dec_digest)

    roof_pre = None
    if do_pre:
        if pre_bound_hbm:
            ach = pb / t_pre / 1e9
            roof_pre = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                        "traffic": pre_traffic, "kernel": "prefill_fwd_kernel<64,bf16,causal>",
                        "algorithmic_bytes_per_launch": pb,
                        "avg_launch_us": round(t_pre * 1e6, 2),
                        "median_launch_us": round(med_pre * 1e6, 2)}
        else:
            roof_pre = {"bound": "mfma", "achieved": round(pre_tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(pre_tflops / MFMA_PEAK_TFLOPS, 4),
                        "traffic": pre_traffic, "kernel": "prefill_fwd_kernel<64,bf16,causal>",
                        "avg_launch_us": round(t_pre * 1e6, 2),
                        "median_launch_us": round(med_pre * 1e6, 2)}
    roof_dec = None
    if do_dec:
        roof_dec = {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                    "traffic": dec_traffic,
                    "kernel": "decode_split_kernel<128,bf16> + decode_merge_kernel<128,bf16>",
                    "algorithmic_bytes_per_launch": db, "avg_launch_us": round(t_dec * 1e6, 2),
                    "median_launch_us": round(med_dec * 1e6, 2)}

    extra = {}
    if not args.no_extra and args.only is None:
        for name in EXTRA:
            log(f"bench: extra figure {name}")
            c = config_case(name)
            Qx, Kx, Vx = (to_dev(x, c.dtype) for x in (c.q, c.k, c.v))
            Ox = torch.empty_like(Qx)
            Lx = torch.empty(c.B, c.Hq, c.N, dtype=torch.float32, device=dev)
            warm(lambda: attn.attn_fwd(Qx, Kx, Vx, Ox, Lx, c.causal, c.scale), torch)
            reps = 10 if c.N <= 8192 else 4
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                attn.attn_fwd(Qx, Kx, Vx, Ox, Lx, c.causal, c.scale)
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / reps * 1e-3
            tf = prefill_flops(c) / t / 1e12
            extra[name] = {"tflops": round(tf, 2), "mfma_frac": round(tf / MFMA_PEAK_TFLOPS, 4),
                           "avg_launch_us": round(t * 1e6, 1)}
            del Qx, Kx, Vx, Ox, Lx
            torch.cuda.empty_cache()

    casc = ppre = ceil = var = None
    if not args.no_extra and args.only is None:
        casc = cascade_figure(attn, torch, dev, log)
        ppre = paged_prefill_figure(attn, torch, dev, log)
        var = variant_figure(attn, torch, dev, log)
        ceil = hbm_read_ceiling(torch, dev, log)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        cpu = cpu_baseline(pc, dc, args.cpu_seconds)

    out = {
        "metric": "prefill attn TFLOP/s (%MFMA peak); paged decode KV GB/s (%HBM peak)",
        "value": round(pre_tflops, 2) if pre_tflops is not None else None,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warmup_detail": {"steps_run": n_warm, "seconds": round(warm_s, 3),
                          "rule": f"--warmup steps, continued to at least {args.warm_seconds} s"},
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded i.i.d. N(0,1), bf16)",
        "config": {"workload": "gpt2-medium causal prefill B64 H16 N1024 d64 + paged GQA decode "
                               "B64 Hq32 Hkv8 d128 ctx log-uniform[512,32768] page16 split1024",
                   "prefill": {"B": pc.B, "H": pc.Hq, "N": pc.N, "d": pc.d, "causal": True},
                   "decode": {"B": dc.B, "Hq": dc.Hq, "Hkv": dc.Hkv, "d": dc.d,
                              "page": dc.page_size, "split_tokens": split,
                              "total_ctx_tokens": int(dc.ctx_lens.astype(np.int64).sum())},
                   "parallelism": "single GPU"},
        "mfma_frac": round(pre_tflops / MFMA_PEAK_TFLOPS, 4) if pre_tflops else None,
        "roofline": roof_pre,
        "decode": None if not do_dec else {
            "value": round(dec_gbs, 1), "unit": "GB/s",
            "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "kv_only_gbs": round(kv_only / t_dec / 1e9, 1),
            "tflops": round(decode_flops(dc) / t_dec / 1e12, 2),
            "roofline": roof_dec},
        "extra_prefill": extra or None,
        "cascade_decode": casc,
        "hbm_read_ceiling": ceil,
        "paged_prefill": ppre,
        "prefill_variant": var,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
