"""Shared helpers of the GPU parity tests: device transfer, calls through the
C-ABI binding, and the element-wise parity criterion.

Parity criterion (fp16 output against the fp64 oracle), per element:
    |gpu - ref| <= 4e-3 + 1e-2 * |ref|
"""
from __future__ import annotations

import sys

import numpy as np

ATOL = 4e-3
RTOL = 1e-2


def say(*args):
    """Name the case before the GPU runs it (flushed, so a crash still shows it)."""
    print("[case]", *args, file=sys.stderr, flush=True)


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    return t.cpu().numpy()


def gpu_prefill(q, k, v, causal: bool) -> np.ndarray:
    import torch
    from attention_attn_prefill_amd import attn_prefill
    tq, tk, tv = dev(q), dev(k), dev(v)
    to = torch.empty_like(tq)
    attn_prefill(tq, tk, tv, to, causal=causal)
    torch.cuda.synchronize()
    return host(to)


def gpu_decode(q, k_cache, v_cache, bt, seq_lens, split: bool = True) -> np.ndarray:
    import torch
    from attention_attn_prefill_amd import attn_decode_paged, attn_decode_paged_workspace_size
    tq, tk, tv = dev(q), dev(k_cache), dev(v_cache)
    tbt, tsl = dev(np.asarray(bt, np.int32)), dev(np.asarray(seq_lens, np.int32))
    out = torch.empty_like(tq)
    ws = None
    if split:
        n = attn_decode_paged_workspace_size(q.shape[0], q.shape[1], k_cache.shape[1], q.shape[2],
                                             bt.shape[1], k_cache.shape[2])
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda") if n else None
    attn_decode_paged(tq, tk, tv, out, tbt, tsl, workspace=ws)
    torch.cuda.synchronize()
    return host(out)


def assert_parity(got16: np.ndarray, ref: np.ndarray, what: str = "") -> float:
    """Element-wise parity; returns the max absolute error."""
    got = got16.astype(np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err, -1)), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
            f"worst at {idx}: gpu={got[idx]!r} ref={ref[idx]!r}; max abs err {err.max():.3e}")
    return float(err.max())
