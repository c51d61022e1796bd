"""Paged KV append on the GPU: bit-exact against the oracle's scatter, and
end to end -- prefill K/V appended through a permuted table and decoded
gives the last row of causal prefill."""
import numpy as np
import pytest

import oracle
from attention_attn_prefill_amd import workloads as W
from gpu_helpers import assert_parity, dev, gpu_decode, gpu_prefill, host, say
from oracle_pins import _slots_for

pytestmark = pytest.mark.gpu


def _rand(shape, seed):
    return W.normal_f16(shape, (97, seed))


def gpu_append(kn, vn, kc, vc, slots):
    import torch
    from attention_attn_prefill_amd import attn_kv_append
    tkc, tvc = dev(kc), dev(vc)
    attn_kv_append(dev(kn), dev(vn), tkc, tvc, dev(np.asarray(slots, np.int64)))
    torch.cuda.synchronize()
    return host(tkc), host(tvc)


@pytest.mark.parametrize("H_kv,D,bs", [(8, 128, 16), (2, 64, 16), (4, 32, 8), (1, 128, 1)])
def test_append_bit_exact_with_padding(H_kv, D, bs):
    n = 200
    nb = max(37, (2 * n + bs - 1) // bs)  # room for every token twice over
    kc, vc = _rand((nb, H_kv, bs, D), 1), _rand((nb, H_kv, bs, D), 2)
    rng = np.random.default_rng(H_kv * 100 + D + bs)
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    slots[rng.choice(n, 17, replace=False)] = -1          # padding tokens
    slots[rng.choice(n, 3, replace=False)] = nb * bs + 9  # past the pool: skipped
    kn, vn = _rand((n, H_kv, D), 3), _rand((n, H_kv, D), 4)
    say("append", H_kv, D, bs)
    gk, gv = gpu_append(kn, vn, kc, vc, slots)
    ok, ov = kc.copy(), vc.copy()
    oracle.kv_append(kn, vn, ok, ov, slots)
    assert np.array_equal(gk.view(np.uint16), ok.view(np.uint16))
    assert np.array_equal(gv.view(np.uint16), ov.view(np.uint16))


def test_append_full_size_prefill_kv():
    """The qwen3_prefill K/V (4 x 2048 tokens, 8 kv heads) into a permuted cache."""
    cfg = W.CONFIGS["qwen3_prefill"]
    _, k, v = W.prefill_inputs(cfg)
    lens = [cfg.S_kv] * cfg.B
    bt, nb = W.paged_layout(lens, 16, cfg.S_kv // 16, (3, 3))
    slots = _slots_for(lens, bt)
    kc = np.zeros((nb, cfg.H_kv, 16, cfg.D), np.float16)
    vc = np.zeros_like(kc)
    kn = k.reshape(-1, cfg.H_kv, cfg.D)
    vn = v.reshape(-1, cfg.H_kv, cfg.D)
    say("append full size", kn.shape)
    gk, gv = gpu_append(kn, vn, kc, vc, slots)
    oracle.kv_append(kn, vn, kc, vc, slots)
    assert np.array_equal(gk.view(np.uint16), kc.view(np.uint16))
    assert np.array_equal(gv.view(np.uint16), vc.view(np.uint16))


def test_prefill_append_decode_end_to_end():
    """Prefill a batch, append its K/V to a paged cache through a permuted
    table, then decode each sequence's last query against that cache: the
    result matches the oracle and the GPU's own causal-prefill last row."""
    B, S, H_q, H_kv, D = 3, 333, 16, 8, 128
    q, k, v = _rand((B, S, H_q, D), 5), _rand((B, S, H_kv, D), 6), _rand((B, S, H_kv, D), 7)
    lens = [S] * B
    bt, nb = W.paged_layout(lens, 16, (S + 15) // 16 + 2, (4, 4))
    slots = _slots_for(lens, bt)
    kc = np.zeros((nb, H_kv, 16, D), np.float16)
    vc = np.zeros_like(kc)
    say("end to end")
    gk, gv = gpu_append(k.reshape(-1, H_kv, D), v.reshape(-1, H_kv, D), kc, vc, slots)
    sl = np.array(lens, np.int32)
    dec = gpu_decode(q[:, -1], gk, gv, bt, sl)
    ref = oracle.decode_paged(q[:, -1], gk, gv, bt, sl)
    assert_parity(dec, ref, "decode after append")
    pre = gpu_prefill(q, k, v, True)[:, -1].astype(np.float64)
    assert np.allclose(dec.astype(np.float64), pre, rtol=2e-2, atol=8e-3)
