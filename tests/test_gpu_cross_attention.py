"""The cross-attention module (projections, adjacent-pair RoPE, attention,
output projection) on the GPU against the fp64 oracle.

Criterion: the attention tolerance |gpu - ref| <= 4e-3 + 1e-2 * |ref| per
output element, and a relative Frobenius error below 2e-3.  The GPU rounds
the projected q, k, v and the attention output to fp16 (the MFMA operand
precision), four roundings of relative size 2^-11 each, plus the final
one, so the whole-tensor relative error stays near 1e-3 at most.
"""
import numpy as np
import pytest

import oracle
from attention_attn_prefill_amd import workloads as W
from gpu_helpers import assert_parity, dev, host, say

pytestmark = pytest.mark.gpu


def gpu_module(xq, xk, ws, H, base, max_pos=None, reuse=None):
    import torch
    from attention_attn_prefill_amd import (attn_cross_attention, attn_cross_attention_workspace_size,
                                            attn_rope_table)
    B, T_q, dim = xq.shape
    T_k = xk.shape[1]
    D = dim // H
    max_pos = max_pos or max(T_q, T_k)
    c = torch.empty((max_pos, D // 2), dtype=torch.float32, device="cuda")
    s = torch.empty_like(c)
    attn_rope_table(c, s, base)
    n = attn_cross_attention_workspace_size(B, T_q, T_k, dim, H)
    assert n > 0
    wsb = reuse if reuse is not None else torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.empty((B, T_q, dim), dtype=torch.float16, device="cuda")
    attn_cross_attention(dev(xq), dev(xk), *[dev(w) for w in ws], c, s, out, H, wsb)
    torch.cuda.synchronize()
    return host(out), wsb


def check(got, ref, what):
    assert_parity(got, ref, what)
    rel = np.linalg.norm(got.astype(np.float64) - ref) / np.linalg.norm(ref)
    assert rel < 2e-3, f"{what}: relative Frobenius error {rel:.2e}"


CASES = [  # B, T_q, T_k, dim, H, base
    (4, 64, 128, 256, 8, 1e4),    # the pages' shape
    (2, 5, 9, 64, 2, 1e4),        # ragged, far below one tile
    (1, 33, 100, 128, 1, 5e5),    # D = 128
    (3, 64, 64, 256, 4, 1e4),     # D = 64
    (2, 200, 77, 96, 3, 1e6),     # dim 96: three column tiles, ragged rows
    (1, 40, 33, 1024, 8, 1e4),    # wide: 32 column tiles, D = 128
    (1, 33, 20, 2048, 16, 1e4),   # wider still: K = 2048, many k-steps per wavefront
]


@pytest.mark.parametrize("B,T_q,T_k,dim,H,base", CASES)
def test_module_parity(B, T_q, T_k, dim, H, base):
    xq, xk, ws = W.cross_module_inputs(B, T_q, T_k, dim, seed=B * 1000 + T_q)
    say("cross-attention module", B, T_q, T_k, dim, H, base)
    got, _ = gpu_module(xq, xk, ws, H, base)
    check(got, oracle.cross_attention(xq, xk, *ws, H=H, base=base), "module")


def test_module_workspace_reuse_and_larger_table():
    """Two calls in a row through one workspace (the second smaller), with a
    table longer than the sequences."""
    xq, xk, ws = W.cross_module_inputs(4, 64, 128, 256, seed=7)
    say("cross-attention module, reuse")
    got1, wsb = gpu_module(xq, xk, ws, 8, 1e4, max_pos=4096)
    check(got1, oracle.cross_attention(xq, xk, *ws, H=8), "first call")
    xq2, xk2, ws2 = W.cross_module_inputs(2, 16, 40, 256, seed=8)
    got2, _ = gpu_module(xq2, xk2, ws2, 8, 1e4, max_pos=4096, reuse=wsb)
    check(got2, oracle.cross_attention(xq2, xk2, *ws2, H=8), "second call")


def test_module_identical_memory_rows():
    """Identical x_kv rows: every query sees the same value, whatever the
    weights, so out = (x W_v^T) W_o^T for every query row."""
    xq, xk, ws = W.cross_module_inputs(2, 40, 60, 128, seed=9)
    xk[:] = xk[:, :1, :]
    say("cross-attention module, identical memory rows")
    got, _ = gpu_module(xq, xk, ws, 4, 1e4)
    check(got, oracle.cross_attention(xq, xk, *ws, H=4), "identical rows")
