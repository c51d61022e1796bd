"""Benchmark of the attention hot path on one MI355X.

One step = one causal GQA prefill (B=4, S=2048, H_q=16, H_kv=8, D=128) plus
one paged single-token decode (256 sequences, H_q=16, H_kv=8, D=128,
block_size=16, seq_lens uniform in [128, 4096], permuted block tables) --
the Qwen3-0.6B-shaped workloads, both entry points of the C ABI, on synthetic
seeded inputs already resident in HBM.  ``--workload long`` swaps in the
long-context pair (prefill B=1 S=32768; decode 64 x 32768 tokens).
``--workload grpo`` times only the shared-prefix decode of forked sequences
(32 prompts of 2048 tokens, 8 samples each with U[1, 512] tokens of their
own), which the default line also carries as ``shared_prefix_decode``.

Prints one JSON line.  ``value`` is prefill TFLOP/s (exact unmasked-pair flop
count, 4*D per pair); the decode half of the metric (KV GB/s: K and V bytes
of every visible token) is in ``decode``.

Timing.  After the ``--warmup`` steps the same step keeps running until at
least one second of GPU work has passed (clocks settle; a handful of steps
is not enough), then exactly ``--steps`` steps are timed.  HIP events on the
launch stream bracket each prefill and each decode call; ``value`` uses the
median prefill duration over the timed steps, ``roofline.achieved`` the mean,
and both are in the line with the min and max.  ``pages_method`` repeats the
measurement the way the pages' benchmark harness does it: events around 200
back-to-back launches after 10 warm-up launches, median of 5 repeats.
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense fp16 MFMA
PEAK_HBM_GBS = 8000.0       # HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", choices=["qwen3", "long", "grpo"], default="qwen3")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--profile", action="store_true",
                   help="counter runs: no CPU baseline, and first a plain 512 MiB fp16 "
                        "negation (reads and writes 512 MiB) to calibrate the byte counters; "
                        "no shared-prefix leg (its kernels share names with plain decode), "
                        "and with --workload grpo only the shared-prefix calls")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the oracle sample")
    p.add_argument("--prefill-sweep", action="store_true",
                   help="instead of the step: causal head_dim-128 prefill at 256 workgroups "
                        "(S = 1024/2048/4096/8192, B = 8/4/2/1, H_q 16, H_kv 8), whose "
                        "workgroups run 18/34/66/130 64-key iterations, and the fit "
                        "time = fixed + iterations x per-iteration cost")
    p.add_argument("--operand-clock", action="store_true",
                   help="instead of the step: fp16 rates of the vendor GEMM (torch.matmul, "
                        "8192^3) and of the causal prefill (qwen3_prefill, long_prefill), "
                        "each on N(0,1) operands and on all-zero operands")
    return p.parse_args()


KERNEL_SOURCES = {
    "prefill_dual_kernel": ["attention_attn_prefill_amd/csrc/prefill_dual.hip",
                            "attention_attn_prefill_amd/csrc/gfx950_device.h",
                            "attention_attn_prefill_amd/csrc/q_norm_rope.h",
                            "attention_attn_prefill_amd/csrc/attn_internal.h"],
    "prefill_fwd_kernel": ["attention_attn_prefill_amd/csrc/prefill_fwd.hip",
                           "attention_attn_prefill_amd/csrc/q_norm_rope.h",
                           "attention_attn_prefill_amd/csrc/attn_internal.h"],
    "decode_split_kernel": ["attention_attn_prefill_amd/csrc/decode_paged.hip",
                            "attention_attn_prefill_amd/csrc/attn_internal.h"],
    "decode_balanced_kernel": ["attention_attn_prefill_amd/csrc/decode_paged.hip",
                               "attention_attn_prefill_amd/csrc/attn_internal.h"],
    "kv_append_kernel": ["attention_attn_prefill_amd/csrc/kv_append.hip",
                         "attention_attn_prefill_amd/csrc/attn_internal.h"],
    "qk_norm_rope_kernel": ["attention_attn_prefill_amd/csrc/rope_norm.hip",
                            "attention_attn_prefill_amd/csrc/attn_internal.h"],
    "prefix_chunk_kernel": ["attention_attn_prefill_amd/csrc/decode_prefix.hip",
                            "attention_attn_prefill_amd/csrc/attn_internal.h"],
}


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch (read + write) from the committed counter summary
    profiles/hbm_traffic_<workload>.md, or None when the kernel's source has
    changed since those counters were taken (or none were taken)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    entry = json.loads(m.group(1))["kernels"].get(kernel)
    if entry is None:
        return None
    h = hashlib.sha256()
    for src in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if h.hexdigest()[:16] != entry["source_sha256_16"]:
        return None
    return entry["read_bytes"] + entry["write_bytes"]


def cpu_baseline(pcfg, dcfg, q, k, v, dq, kc, vc, bt, sl, target_s):
    """The fp64 oracle on a bounded random sample of prefill rows and decode
    sequences, scaled to the metric's units."""
    import oracle
    from attention_attn_prefill_amd import workloads as W

    rng = np.random.default_rng(1234)
    n_rows_total = pcfg.B * pcfg.S_q * pcfg.H_q

    def pairs_of(rows):
        pos = (rows // pcfg.H_q) % pcfg.S_q
        return int((pos + 1).sum()) if pcfg.causal else len(rows) * pcfg.S_kv

    # calibrate on a small sample, then size the real one to ~60 % of the budget
    cal = rng.choice(n_rows_total, size=min(256, n_rows_total), replace=False).astype(np.int64)
    t = time.perf_counter()
    oracle.prefill(q, k, v, pcfg.causal, rows=cal)
    rate = pairs_of(cal) / max(time.perf_counter() - t, 1e-6)
    avg_pairs = pcfg.pairs / n_rows_total
    n = int(min(n_rows_total, max(256, 0.6 * target_s * rate / avg_pairs)))
    rows = np.sort(rng.choice(n_rows_total, size=n, replace=False)).astype(np.int64)
    t = time.perf_counter()
    oracle.prefill(q, k, v, pcfg.causal, rows=rows)
    tp = time.perf_counter() - t
    flops = 4 * pcfg.D * pairs_of(rows)

    # decode: sequences in random order until ~40 % of the budget is used
    order = rng.permutation(dcfg.num_seqs).astype(np.int64)
    picked, spent, kvb = [], 0.0, 0
    for chunk in np.array_split(order, max(1, dcfg.num_seqs // 8)):
        t = time.perf_counter()
        oracle.decode_paged(dq, kc, vc, bt, sl, seqs=chunk)
        spent += time.perf_counter() - t
        picked.extend(chunk.tolist())
        kvb += W.kv_bytes(sl[chunk], dcfg.H_kv, dcfg.D)
        if spent > 0.4 * target_s:
            break
    return {
        "value": flops / tp / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
        "nproc": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"prefill: {n} of {n_rows_total} query rows (uniform random, "
                  f"{pairs_of(rows)} unmasked pairs) in {tp:.2f} s; decode: {len(picked)} of "
                  f"{dcfg.num_seqs} sequences in {spent:.2f} s",
        "decode": {"value": kvb / spent / 1e9, "unit": "GB/s"},
    }


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def profile_kernel_us(workload: str, kernel_prefix: str):
    """Average duration (us) of a kernel in the committed kernel-trace
    summary profiles/kernel_stats_<workload>.md, or None."""
    import re
    path = os.path.join(ROOT, "profiles", f"kernel_stats_{workload}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        cells = [c.strip() for c in line.split("|")]
        # | `kernel name` | calls | average (us) | min | max | share |
        if len(cells) > 4 and re.search(r"::" + re.escape(kernel_prefix) + r"[<(]", cells[1]):
            try:
                return float(cells[3])
            except ValueError:
                return None
    return None


def stats_ms(xs):
    xs = np.asarray(xs, np.float64)
    return {"median": round(float(np.median(xs)), 5), "mean": round(float(xs.mean()), 5),
            "min": round(float(xs.min()), 5), "max": round(float(xs.max()), 5)}


def pages_method(fn, stream, iters=200, warm=10, repeats=5):
    """The pages' benchmark harness: events around `iters` back-to-back
    launches after `warm` warm-up launches; the median of `repeats` runs (ms
    per launch)."""
    import torch
    for _ in range(warm):
        fn()
    res = []
    for _ in range(repeats):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) / iters)
    return float(np.median(res)), res


def time_kv_append(pcfg, k, v, dev, stream, W, traffic_key, iters=100):
    """The prefill's K/V (B*S tokens) written into a paged cache through a
    permuted block table: HBM bytes = read + write of every row."""
    import torch

    from attention_attn_prefill_amd import attn_kv_append
    lens = [pcfg.S_kv] * pcfg.B
    bt, nb = W.paged_layout(lens, 16, (pcfg.S_kv + 15) // 16, (11, 11))
    slots = np.concatenate([bt[s, np.arange(L) // 16].astype(np.int64) * 16 + np.arange(L) % 16
                            for s, L in enumerate(lens)])
    kn = torch.from_numpy(k).to(dev).view(-1, pcfg.H_kv, pcfg.D)
    vn = torch.from_numpy(v).to(dev).view(-1, pcfg.H_kv, pcfg.D)
    kc = torch.empty((nb, pcfg.H_kv, 16, pcfg.D), dtype=torch.float16, device=dev)
    vc = torch.empty_like(kc)
    sm = torch.from_numpy(slots).to(dev)
    for _ in range(20):
        attn_kv_append(kn, vn, kc, vc, sm, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        attn_kv_append(kn, vn, kc, vc, sm, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    nbytes = 2 * 2 * kn.numel() * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"metric": "paged KV append GB/s (read + write)", "value": round(gbs, 1), "unit": "GB/s",
            "tokens": int(kn.shape[0]), "bytes": int(nbytes), "launch_ms": round(ms, 5),
            "roofline": {"bound": "hbm", "kernel": "kv_append_kernel", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic(traffic_key, "kv_append_kernel")}}


def time_qk_norm_rope(pcfg, q, k, v, dev, stream, W, traffic_key, iters=100, with_step=True):
    """The Qwen3 step between the projections and attention on the prefill's
    B*S tokens: QK RMSNorm + NeoX RoPE in place, fused with the paged append
    of the rotated K and of V (theta 1e6, positions 0..S-1 per sequence).
    Algorithmic HBM bytes: q and k read and written, v read, the cache rows
    of k and v written, one table row (cos + sin) per token, the position
    and slot of every token."""
    import torch

    from attention_attn_prefill_amd import attn_qk_norm_rope_append, attn_rope_table
    n, D = pcfg.B * pcfg.S_q, pcfg.D
    lens = [pcfg.S_kv] * pcfg.B
    bt, nb = W.paged_layout(lens, 16, (pcfg.S_kv + 15) // 16, (12, 12))
    slots = np.concatenate([bt[s, np.arange(L) // 16].astype(np.int64) * 16 + np.arange(L) % 16
                            for s, L in enumerate(lens)])
    tq = torch.from_numpy(q).to(dev).view(n, pcfg.H_q, D)
    tk = torch.from_numpy(k).to(dev).view(n, pcfg.H_kv, D)
    tv = torch.from_numpy(v).to(dev).view(n, pcfg.H_kv, D)
    kc = torch.empty((nb, pcfg.H_kv, 16, D), dtype=torch.float16, device=dev)
    vc = torch.empty_like(kc)
    sm = torch.from_numpy(slots).to(dev)
    pos = torch.arange(pcfg.S_q, dtype=torch.int32, device=dev).repeat(pcfg.B)
    rng = np.random.default_rng(13)
    qw = torch.from_numpy(rng.uniform(0.25, 2.0, D).astype(np.float16)).to(dev)
    kw = torch.from_numpy(rng.uniform(0.25, 2.0, D).astype(np.float16)).to(dev)
    max_pos = 40960
    ct = torch.empty((max_pos, D // 2), dtype=torch.float32, device=dev)
    st = torch.empty_like(ct)
    attn_rope_table(ct, st, 1e6, stream=stream)

    def run():
        attn_qk_norm_rope_append(tq, tk, tv, qw, kw, ct, st, pos, kc, vc, sm, stream=stream)

    for _ in range(20):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    row = D * 2
    nbytes = (2 * n * pcfg.H_q * row + 2 * n * pcfg.H_kv * row + n * pcfg.H_kv * row
              + 2 * n * pcfg.H_kv * row + n * D * 4 + n * 4 + n * 8)
    gbs = nbytes / (ms * 1e-3) / 1e9
    leg = {"metric": "QK-norm + RoPE + paged append GB/s", "value": round(gbs, 1), "unit": "GB/s",
           "tokens": n, "bytes": int(nbytes), "launch_ms": round(ms, 5),
           "roofline": {"bound": "hbm", "kernel": "qk_norm_rope_kernel<128,append>",
                        "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": measured_traffic(traffic_key, "qk_norm_rope_kernel")}}
    if not with_step:
        return leg
    # The whole attention step of a Qwen3 prefill layer, two ways:
    #   two-pass: norm + RoPE + append of q and k, then attn_prefill;
    #   fused: norm + RoPE + append of k only, then attn_prefill_qk_norm_rope
    #          (the queries are normalised and rotated as they are loaded).
    # The passes work in place, and repeating them would normalise and
    # rotate again on every call (the weights compound), which changes the
    # scores the prefill sees; so each part is timed on its own, the rope
    # passes on scratch copies and every prefill on inputs that were
    # normalised and rotated exactly once.
    from attention_attn_prefill_amd import attn_prefill, attn_prefill_qk_norm_rope, attn_qk_norm_rope
    shp_q, shp_k = (pcfg.B, pcfg.S_q, pcfg.H_q, D), (pcfg.B, pcfg.S_kv, pcfg.H_kv, D)
    q0 = torch.from_numpy(q).to(dev)
    k0 = torch.from_numpy(k).to(dev).view(n, pcfg.H_kv, D)
    q_rot, k_rot = q0.clone().view(n, pcfg.H_q, D), k0.clone()
    attn_qk_norm_rope(q_rot, k_rot, qw, kw, ct, st, pos, stream=stream)
    sq, sk = q0.clone().view(n, pcfg.H_q, D), k0.clone()
    to = torch.empty_like(q0)

    def timed(fn, reps=50):
        for _ in range(10):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_qk = timed(lambda: attn_qk_norm_rope_append(sq, sk, tv, qw, kw, ct, st, pos, kc, vc, sm, stream=stream))
    t_k = timed(lambda: attn_qk_norm_rope_append(None, sk, tv, None, kw, ct, st, pos, kc, vc, sm, stream=stream))
    t_pre = timed(lambda: attn_prefill(q_rot.view(shp_q), k_rot.view(shp_k), tv.view(shp_k), to,
                                       causal=pcfg.causal, stream=stream))
    # positions None: query row i of each sequence is at position i
    t_pre_rope = timed(lambda: attn_prefill_qk_norm_rope(q0, k_rot.view(shp_k), tv.view(shp_k), to, qw, ct, st,
                                                         None, causal=pcfg.causal, stream=stream))
    two_ms, fused_ms = t_qk + t_pre, t_k + t_pre_rope
    leg["attention_step"] = {
        "what": "QK-norm + RoPE + KV append + causal prefill on the same tokens (parts timed separately)",
        "two_pass_us": round(two_ms * 1e3, 2), "fused_q_on_load_us": round(fused_ms * 1e3, 2),
        "qk_append_us": round(t_qk * 1e3, 2), "k_only_append_us": round(t_k * 1e3, 2),
        "prefill_us": round(t_pre * 1e3, 2), "prefill_q_on_load_us": round(t_pre_rope * 1e3, 2),
        "speedup": round(two_ms / fused_ms, 3)}
    return leg


def time_cross_module(dev, stream, W, iters=200):
    """The cross-attention module at the pages' shape (B=4, T_q=64, T_k=128,
    dim=256, 8 heads of 32, rotary base 1e4): three launches per call.
    Algorithmic flops: the four projections (2*rows*dim*dim each) and the
    attention (4*B*H*T_q*T_k*D)."""
    import torch

    from attention_attn_prefill_amd import (attn_cross_attention, attn_cross_attention_workspace_size,
                                            attn_rope_table)
    B, T_q, T_k, dim, H = 4, 64, 128, 256, 8
    xq, xk, ws = W.cross_module_inputs(B, T_q, T_k, dim, seed=0)
    txq, txk = torch.from_numpy(xq).to(dev), torch.from_numpy(xk).to(dev)
    tws = [torch.from_numpy(w).to(dev) for w in ws]
    ct = torch.empty((T_k, dim // H // 2), dtype=torch.float32, device=dev)
    st = torch.empty_like(ct)
    attn_rope_table(ct, st, 1e4, stream=stream)
    wsb = torch.empty(attn_cross_attention_workspace_size(B, T_q, T_k, dim, H), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T_q, dim), dtype=torch.float16, device=dev)

    def run():
        attn_cross_attention(txq, txk, *tws, ct, st, out, H, wsb, stream=stream)

    for _ in range(20):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    flops = 2 * B * T_q * dim * dim * 2 + 2 * B * T_k * dim * dim * 2 + 4 * B * H * T_q * T_k * (dim // H)
    tf = flops / (ms * 1e-3) / 1e12
    return {"metric": "cross-attention module latency", "value": round(ms * 1e3, 2), "unit": "us per call",
            "higher_is_better": False, "flops": int(flops), "tflops": round(tf, 3), "launches": 3,
            "config": {"B": B, "T_q": T_q, "T_k": T_k, "dim": dim, "heads": H},
            "roofline": {"bound": "mfma", "kernel": "proj_kernel + prefill_fwd_kernel<32,noncausal>",
                         "achieved": round(tf, 3), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_FP16_TFLOPS, 5)}}


def time_shared_prefix(dev, stream, W, iters=50, shared_only=False):
    """The forked-decode workload (32 prompts of 2048 tokens, 8 samples each
    with U[1, 512] tokens of their own; H 16/8, D 128): plain paged decode
    against the shared-prefix path on the same tables.  Logical KV bytes count
    every sequence's context; unique bytes count each shared prompt once."""
    import torch

    from attention_attn_prefill_amd import (attn_decode_paged, attn_decode_paged_shared_prefix,
                                            attn_decode_paged_shared_prefix_workspace_size,
                                            attn_decode_paged_workspace_size)
    q, kc, vc, bt, sl, gs, pb = W.grpo_decode_inputs()
    c = W.GRPO_DECODE
    t = {n: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
         for n, x in (("q", q), ("kc", kc), ("vc", vc), ("bt", bt), ("sl", sl), ("gs", gs), ("pb", pb))}
    out = torch.empty_like(t["q"])
    n, Hq, Hkv, D = q.shape[0], q.shape[1], kc.shape[1], q.shape[2]
    ws_plain = torch.empty(max(16, attn_decode_paged_workspace_size(n, Hq, Hkv, D, bt.shape[1], 16)),
                           dtype=torch.uint8, device=dev)
    mgs = c["group_size"]
    ws_shared = torch.empty(attn_decode_paged_shared_prefix_workspace_size(n, Hq, Hkv, D, bt.shape[1], 16,
                                                                          len(pb), mgs),
                            dtype=torch.uint8, device=dev)

    def plain():
        attn_decode_paged(t["q"], t["kc"], t["vc"], out, t["bt"], t["sl"], workspace=ws_plain, stream=stream)

    def shared():
        attn_decode_paged_shared_prefix(t["q"], t["kc"], t["vc"], out, t["bt"], t["sl"], t["gs"], t["pb"], mgs,
                                        ws_shared, stream=stream)

    def timed(fn):
        for _ in range(10):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    ms_plain = None if shared_only else timed(plain)
    ms_shared = timed(shared)
    row = Hkv * D * 2 * 2  # K + V bytes per token
    logical = int(sl.astype(np.int64).sum()) * row
    shared_tokens = int(np.sum(pb.astype(np.int64) * 16 * (np.diff(gs) - 1)))
    unique = logical - shared_tokens * row
    return {"metric": "forked paged decode: logical KV GB/s", "value": round(logical / (ms_shared * 1e-3) / 1e9, 1),
            "unit": "GB/s", "launch_ms": round(ms_shared, 5),
            "plain_decode_ms": None if ms_plain is None else round(ms_plain, 5),
            "speedup_vs_plain_decode": None if ms_plain is None else round(ms_plain / ms_shared, 3),
            "logical_kv_bytes": logical, "unique_kv_bytes": unique,
            "config": dict(c),
            "roofline": {"bound": "hbm", "kernel": "prefix_chunk_kernel + decode_split_kernel (one split per sequence)",
                         "achieved": round(unique / (ms_shared * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s (unique bytes)",
                         "frac": round(unique / (ms_shared * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "traffic": shared_traffic(),
                         "traffic_unit": "bytes per call (HBM read + write, rocprofv3 counters, both kernels)"}}


def shared_traffic():
    """HBM bytes per shared-prefix call: prefix kernel plus shared-mode split
    kernel, from profiles/hbm_traffic_grpo.md (None if either is stale)."""
    a = measured_traffic("grpo", "prefix_chunk_kernel")
    b = measured_traffic("grpo", "decode_split_kernel")
    return None if a is None or b is None else a + b


def main_grpo(args):
    import torch

    from attention_attn_prefill_amd import workloads as W
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.profile:
        calibration_copy(dev)
    leg = time_shared_prefix(dev, stream, W, iters=args.steps, shared_only=args.profile)
    leg.update({"n_gpus": 1, "steps": args.steps, "warmup": 10, "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": "f16 (fp32 accumulate)",
                "data": "synthetic, seeded N(0,1) fp16; forked block tables (shared prompt blocks)"})
    leg["config"] = {"workload": "grpo_decode: 32 prompts x 8 samples, prompt 2048 tokens, own tokens U[1,512], "
                                 "H_q=16 H_kv=8 D=128 block_size=16", **leg["config"]}
    print(json.dumps(leg), flush=True)


def main_sweep(args):
    """Fixed and per-iteration cost of the head_dim-128 causal prefill.  At
    S = 128 n (n even) with B = 2048 / S, H_q 16 and H_kv 8 the grid is
    n/2 query-tile pairs x 8 head pairs x B = 256 workgroups, one per CU, and
    every workgroup runs 2n + 2 iterations of 64 keys (tile j of a pair has
    keys up to 128 (j + 1)).  Times are the pages' method (HIP events around
    back-to-back launches), so the fixed part includes the gap between
    launches."""
    import torch

    from attention_attn_prefill_amd import attn_prefill
    from attention_attn_prefill_amd import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = []
    for S, B in ((1024, 8), (2048, 4), (4096, 2), (8192, 1)):
        cfg = W.PrefillConfig(f"sweep_{S}", 90 + S // 1024, B, S, S, 16, 8, 128, True)
        q, k, v = (torch.from_numpy(x).to(dev) for x in W.prefill_inputs(cfg))
        o = torch.empty_like(q)
        iters = 2 * (S // 128) + 2
        fn = lambda: attn_prefill(q, k, v, o, causal=True)  # noqa: E731
        t0 = time.time()
        while time.time() - t0 < 1.0:
            fn()
        torch.cuda.synchronize()
        ms, reps = pages_method(fn, stream, iters=50, warm=args.warmup, repeats=7)
        rows.append({"S": S, "B": B, "workgroups": (S // 256) * 8 * B, "iterations_per_workgroup": iters,
                     "us": round(ms * 1e3, 2), "tflops": round(cfg.flops / ms / 1e9, 1)})
        print(f"[sweep] S={S} B={B}: {ms * 1e3:.2f} us", file=sys.stderr, flush=True)
    x = np.array([r["iterations_per_workgroup"] for r in rows], np.float64)
    y = np.array([r["us"] for r in rows], np.float64)
    c, f = np.polyfit(x, y, 1)
    print(json.dumps({"mode": "prefill_sweep", "kernel": "prefill_dual_kernel<128,causal>",
                      "method": "HIP events around 50 back-to-back launches, median of 7",
                      "rows": rows, "fit": {"fixed_us_per_workgroup": round(float(f), 2),
                                            "us_per_iteration": round(float(c), 4)}}))


def main_operand_clock(args):
    """How far the dense fp16 peak is reachable on this chip.  The peak
    assumes 2.4 GHz; under the power drawn by busy matrix cores the chip
    lowers its clock, and the draw depends on the operand bits.  The same
    launches are timed on N(0,1) operands and on all-zero operands (same
    instructions, same bytes): the vendor GEMM (torch.matmul on fp16,
    8192 x 8192 x 8192) and the causal prefill of both workloads.  Times are
    the pages' method (HIP events around back-to-back launches, median of 5)."""
    import torch

    from attention_attn_prefill_amd import attn_prefill
    from attention_attn_prefill_amd import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = []

    def timed(name, kind, fn, flops, iters):
        t0 = time.time()
        while time.time() - t0 < 1.0:
            fn()
        torch.cuda.synchronize()
        ms, _ = pages_method(fn, stream, iters=iters, warm=args.warmup, repeats=5)
        tf = flops / ms / 1e9
        rows.append({"op": name, "operands": kind, "us": round(ms * 1e3, 2), "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / PEAK_FP16_TFLOPS, 4)})
        print(f"[operand-clock] {name} {kind}: {ms * 1e3:.2f} us, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)

    n = 8192
    a = torch.from_numpy(W.normal_f16((n, n), [31, 1])).to(dev)
    b = torch.from_numpy(W.normal_f16((n, n), [31, 2])).to(dev)
    c = torch.empty((n, n), dtype=torch.float16, device=dev)
    for kind in ("normal", "zeros"):
        if kind == "zeros":
            a.zero_()
            b.zero_()
        timed("matmul_8192", kind, lambda: torch.matmul(a, b, out=c), 2.0 * n ** 3, 20)
    del a, b, c
    for name, iters in (("qwen3_prefill", 100), ("long_prefill", 5)):
        cfg = W.CONFIGS[name]
        q, k, v = (torch.from_numpy(x).to(dev) for x in W.prefill_inputs(cfg))
        o = torch.empty_like(q)
        for kind in ("normal", "zeros"):
            if kind == "zeros":
                for x in (q, k, v):
                    x.zero_()
            timed(name, kind, lambda: attn_prefill(q, k, v, o, causal=True), cfg.flops, iters)
        del q, k, v, o
    print(json.dumps({"mode": "operand_clock", "peak_tflops": PEAK_FP16_TFLOPS,
                      "method": "HIP events around back-to-back launches, median of 5", "rows": rows}))


def calibration_copy(dev):
    import torch
    src = torch.ones(256 << 20, dtype=torch.float16, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    print("[bench] calibration copy: 512 MiB read + 512 MiB written", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    if args.prefill_sweep:
        main_sweep(args)
        return
    if args.operand_clock:
        main_operand_clock(args)
        return
    if args.workload == "grpo":
        main_grpo(args)
        return

    import torch

    from attention_attn_prefill_amd import (attn_decode_paged, attn_decode_paged_workspace_size,
                                            attn_prefill)
    from attention_attn_prefill_amd import workloads as W

    pname, dname = ("qwen3_prefill", "paged_decode") if args.workload == "qwen3" else \
        ("long_prefill", "long_decode")
    pcfg, dcfg = W.CONFIGS[pname], W.CONFIGS[dname]
    print(f"[bench] generating {pname} + {dname} inputs", file=sys.stderr, flush=True)
    q, k, v = W.prefill_inputs(pcfg)
    dq, kc, vc, bt, sl = W.decode_inputs(dcfg)

    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    to = torch.empty_like(tq)
    tdq, tkc, tvc = (torch.from_numpy(x).to(dev) for x in (dq, kc, vc))
    tbt, tsl = torch.from_numpy(bt).to(dev), torch.from_numpy(sl).to(dev)
    tout = torch.empty_like(tdq)
    ws_bytes = attn_decode_paged_workspace_size(dcfg.num_seqs, dcfg.H_q, dcfg.H_kv, dcfg.D,
                                                dcfg.max_blocks_per_seq, dcfg.block_size)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    print("[bench] inputs resident in HBM", file=sys.stderr, flush=True)
    if args.profile:
        args.no_cpu_baseline = True
        calibration_copy(dev)

    def prefill():
        attn_prefill(tq, tk, tv, to, causal=pcfg.causal, stream=stream)

    def decode():
        attn_decode_paged(tdq, tkc, tvc, tout, tbt, tsl, workspace=ws, stream=stream)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        prefill()
        if ev is not None:
            ev[1].record(stream)
        decode()
        if ev is not None:
            ev[2].record(stream)

    # warm-up: the requested steps, then more until a second of GPU work has
    # passed (the clocks of a freshly idle GPU take that long to settle)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    extra_warm = 0
    while time.perf_counter() - t_warm < 1.0:
        for _ in range(4):
            step()
        extra_warm += 4
        torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    print(f"[bench] timed {args.steps} steps (after {args.warmup} + {extra_warm} warm-up steps)",
          file=sys.stderr, flush=True)

    pre = [e[0].elapsed_time(e[1]) for e in events]
    dec = [e[1].elapsed_time(e[2]) for e in events]
    pre_st, dec_st = stats_ms(pre), stats_ms(dec)
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    flops = pcfg.flops
    kvb = W.kv_bytes(sl, dcfg.H_kv, dcfg.D)
    pre_tflops = flops / (pre_st["median"] * 1e-3) / 1e12
    pre_tflops_mean = flops / (pre_st["mean"] * 1e-3) / 1e12
    dec_gbs = kvb / (dec_st["median"] * 1e-3) / 1e9
    dec_gbs_mean = kvb / (dec_st["mean"] * 1e-3) / 1e9

    # the pages' harness: 200 back-to-back launches, median of 5 repeats
    if args.profile:
        pm = None
    else:
        pm_pre, pm_pre_all = pages_method(prefill, stream)
        pm_dec, pm_dec_all = pages_method(decode, stream)
        pm = {"what": "HIP events around 200 back-to-back launches after 10 warm-up launches, median of 5 repeats",
              "prefill_ms": round(pm_pre, 5), "prefill_repeats_ms": [round(x, 5) for x in pm_pre_all],
              "prefill_tflops": round(flops / (pm_pre * 1e-3) / 1e12, 2),
              "decode_ms": round(pm_dec, 5), "decode_repeats_ms": [round(x, 5) for x in pm_dec_all],
              "decode_gbs": round(kvb / (pm_dec * 1e-3) / 1e9, 1)}

    traffic_key = f"{pname}_{dname}"
    pcfg_bytes = 2 * (q.size + k.size + v.size + q.size)
    pre_kernel = "prefill_dual_kernel" if pcfg.D == 128 else "prefill_fwd_kernel"
    # split-K over a workspace: the balanced first pass, then its merge
    split_us = profile_kernel_us(traffic_key, "decode_balanced_kernel")
    merge_us = profile_kernel_us(traffic_key, "decode_balanced_merge_kernel")
    line = {
        "metric": "prefill TFLOP/s + paged-decode KV GB/s (Qwen3-0.6B shapes), % of roofline",
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "extra_warmup_steps": extra_warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 (fp32 accumulate)",
        "data": "synthetic, seeded N(0,1) fp16; permuted block tables",
        "config": {
            "workload": f"{pname}: causal GQA prefill B={pcfg.B} S={pcfg.S_q} H_q={pcfg.H_q} "
                        f"H_kv={pcfg.H_kv} D={pcfg.D}; {dname}: paged decode "
                        f"{dcfg.num_seqs} seqs, H_q={dcfg.H_q} H_kv={dcfg.H_kv} D={dcfg.D} "
                        f"block_size={dcfg.block_size}, seq_lens U[{dcfg.len_lo},{dcfg.len_hi}]",
            "prefill_flops": flops,
            "prefill_dense_equivalent_flops": pcfg.dense_flops,
            "decode_kv_bytes": kvb,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma", "kernel": f"{pre_kernel}<{pcfg.D},causal>",
            "achieved": round(pre_tflops_mean, 2), "achieved_from": "mean launch duration over the timed steps",
            "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(pre_tflops_mean / PEAK_FP16_TFLOPS, 4),
            "frac_median": round(pre_tflops / PEAK_FP16_TFLOPS, 4),
            "traffic": measured_traffic(traffic_key, pre_kernel),
            "traffic_unit": "bytes per launch (HBM read + write, rocprofv3 counters)",
            "algorithmic_bytes": pcfg_bytes,
            "launch_ms": pre_st,
        },
        "decode": {
            "metric": "paged-decode KV GB/s", "value": round(dec_gbs, 1), "unit": "GB/s",
            "value_from": "median call duration (split + merge) over the timed steps",
            "launch_ms": dec_st,
            "split_kernel_us_profile": split_us, "merge_kernel_us_profile": merge_us,
            "split_merge_source": "profiles/kernel_stats_" + traffic_key + ".md (rocprofv3 kernel-trace averages)",
            "roofline": {
                "bound": "hbm", "kernel": "decode_balanced_kernel<2> + decode_balanced_merge_kernel",
                "achieved": round(dec_gbs_mean, 1), "achieved_from": "mean call duration",
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dec_gbs_mean / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(traffic_key, "decode_balanced_kernel"),
            },
        },
        "pages_method": pm,
    }
    line["kv_append"] = time_kv_append(pcfg, k, v, dev, stream, W, traffic_key)
    line["qk_norm_rope_append"] = time_qk_norm_rope(pcfg, q, k, v, dev, stream, W, traffic_key,
                                                    with_step=not args.profile)
    line["cross_attention_module"] = time_cross_module(dev, stream, W)
    if not args.profile:
        line["shared_prefix_decode"] = time_shared_prefix(dev, stream, W)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(pcfg, dcfg, q, k, v, dq, kc, vc, bt, sl,
                                            args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
