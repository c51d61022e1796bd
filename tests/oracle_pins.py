"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` takes an oracle object (``oracle.Oracle``) and raises
``AssertionError`` when the oracle disagrees with the fact.  The pins are run
against the real oracle (``test_oracle_pins.py``) and against copies with a
planted mistake (``test_oracle_mutants.py``), which every mistake must trip.

What pins what:
  * binary16 decoding        -- numpy's own float16 conversion, all 65536 codes
  * scale 1/sqrt(D), exp sign, normalisation, LSE
                             -- two-key logistic closed form, D in {32,64,128}
  * which weight meets which value row
                             -- three/four-key one-hot closed form
  * causal extent (j <= i)   -- row 0 equals V[0] exactly; identical keys give
                                the mean of V[0..i]; future keys are ignored
  * GQA head mapping (kv head = h*H_kv // H_q, from the attention.cuh listing)
                             -- per-kv-head constant V
  * max subtraction (overflow safety)
                             -- huge logits against torch's fp64 SDPA
  * everything at once on random data
                             -- torch.nn.functional.scaled_dot_product_attention
                                in fp64 on the CPU (library special case)
  * paging                   -- decode equals the last causal-prefill row,
                                block-permutation invariance, a brute-force
                                scipy softmax over the gathered context
  * KV append                -- numpy fancy indexing; padding slots; append
                                then decode equals prefill
  * RoPE table               -- the pages' printed frequency formula (numpy
                                arange) recovered with atan2; cos^2+sin^2 = 1;
                                angle addition across positions
  * NeoX rotation            -- numpy complex multiplication; position 0 is
                                the identity; norms kept; only m - n matters
  * QK RMSNorm               -- unit mean square, scale invariance, a
                                constant-row closed form (mean, eps, weight);
                                numpy RMSNorm then rotation (the pages' order)
  * interleaved-pair rotation (the cross-attention workload's Q and K)
                             -- numpy complex multiplication of adjacent
                                pairs; position 0 is the identity; norms
                                kept; only the position offset matters
  * cross-attention module   -- torch fp64 (F.linear, complex RoPE, SDPA);
                                identical memory rows; a single key
  * forked (shared-prefix) decode -- tables sharing the prompt's blocks
                                give the same result as private copies
"""
from __future__ import annotations

import math

import numpy as np

from attention_attn_prefill_amd import workloads as W


def _rand16(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float16)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---- decoding --------------------------------------------------------------

def pin_half_decoder(ora):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([ora.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN codes decoded differently"
    assert np.array_equal(got[~nan], ref[~nan]), "binary16 decode differs from numpy"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "sign of zero"


# ---- closed forms ----------------------------------------------------------

def pin_two_key_logistic(ora):
    """Row 1 of a causal S=2 problem with q1 = 8 e0, k0 = e0, k1 = 0,
    v0 = e0, v1 = 0 puts weight sigma(8/sqrt(D)) on v0."""
    for D in (32, 64, 128):
        q = np.zeros((1, 2, 1, D), np.float16)
        k = np.zeros_like(q)
        v = np.zeros_like(q)
        q[0, 1, 0, 0] = 8.0
        k[0, 0, 0, 0] = 1.0
        v[0, 0, 0, 0] = 1.0
        o, lse = ora.prefill(q, k, v, causal=True, return_lse=True)
        s0 = 8.0 / math.sqrt(D)
        want = 1.0 / (1.0 + math.exp(-s0))
        assert abs(o[0, 1, 0, 0] - want) < 1e-15, (D, o[0, 1, 0, 0], want)
        assert np.all(o[0, 1, 0, 1:] == 0.0)
        assert abs(lse[0, 1, 0] - math.log(math.exp(s0) + 1.0)) < 1e-14
        # the same two keys through the paged decode entry
        kc = np.zeros((3, 1, 16, D), np.float16)
        vc = np.zeros_like(kc)
        kc[2, 0, 0, 0] = 1.0
        vc[2, 0, 0, 0] = 1.0
        bt = np.array([[2, -1]], np.int32)
        od, lsed = ora.decode_paged(q[:, 1], kc, vc, bt, np.array([2], np.int32),
                                    return_lse=True)
        assert abs(od[0, 0, 0] - want) < 1e-15, (D, od[0, 0, 0], want)
        assert np.all(od[0, 0, 1:] == 0.0)
        assert abs(lsed[0, 0] - math.log(math.exp(s0) + 1.0)) < 1e-14
    # sigma(8/sqrt(128)) = sigma(0.70711) = 0.66976 to five places
    q = np.zeros((1, 2, 1, 128), np.float16)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    q[0, 1, 0, 0], k[0, 0, 0, 0], v[0, 0, 0, 0] = 8.0, 1.0, 1.0
    assert abs(ora.prefill(q, k, v, True)[0, 1, 0, 0] - 0.66976) < 5e-6


def pin_onehot_distribution(ora):
    """q = c e0, k_j = a_j e0, v_j = e_j: the output's first coordinates are
    exactly the softmax weights exp(c a_j / sqrt D) / sum, in key order."""
    D = 16
    a = [0.5, -1.0, 1.5, 0.25]
    c = 4.0
    n = len(a)
    q = np.zeros((1, 1, 1, D), np.float16)
    k = np.zeros((1, n, 1, D), np.float16)
    v = np.zeros((1, n, 1, D), np.float16)
    q[0, 0, 0, 0] = c
    for j in range(n):
        k[0, j, 0, 0] = a[j]
        v[0, j, 0, j] = 1.0
    e = [math.exp(c * aj / math.sqrt(D)) for aj in a]
    want = np.array([x / sum(e) for x in e])
    o = ora.prefill(q, k, v, causal=False)
    assert np.allclose(o[0, 0, 0, :n], want, rtol=0, atol=1e-15), (o[0, 0, 0, :n], want)
    assert np.all(o[0, 0, 0, n:] == 0.0)
    # causal view of the same keys: row i sees keys 0..i only
    qc = np.zeros((1, n, 1, D), np.float16)
    qc[0, :, 0, 0] = c
    oc = ora.prefill(qc, k, v, causal=True)
    for i in range(n):
        ei = e[: i + 1]
        assert np.allclose(oc[0, i, 0, : i + 1], np.array(ei) / sum(ei), atol=1e-15)
        assert np.all(oc[0, i, 0, i + 1:] == 0.0)


# ---- causal structure --------------------------------------------------------

def pin_single_visible_key(ora):
    B, S, H_q, H_kv, D = 2, 5, 4, 2, 16
    q, k, v = _rand16((B, S, H_q, D), 1), _rand16((B, S, H_kv, D), 2), _rand16((B, S, H_kv, D), 3)
    o = ora.prefill(q, k, v, causal=True)
    for b in range(B):
        for h in range(H_q):
            g = h * H_kv // H_q
            assert np.array_equal(o[b, 0, h], _f64(v[b, 0, g])), (b, h)


def pin_identical_keys_mean(ora):
    B, S, H, D = 1, 9, 2, 32
    q = _rand16((B, S, H, D), 4)
    k = np.repeat(_rand16((B, 1, H, D), 5), S, axis=1)
    v = _rand16((B, S, H, D), 6)
    o = ora.prefill(q, k, v, causal=True)
    vd = _f64(v)
    for i in range(S):
        assert np.allclose(o[0, i], vd[0, : i + 1].mean(axis=0), rtol=0, atol=1e-14), i
    on = ora.prefill(q, k, v, causal=False)
    assert np.allclose(on[0], np.broadcast_to(vd[0].mean(axis=0), on[0].shape), atol=1e-14)


def pin_future_keys_ignored(ora):
    B, S, H, D = 1, 12, 2, 16
    q, k, v = _rand16((B, S, H, D), 7), _rand16((B, S, H, D), 8), _rand16((B, S, H, D), 9)
    o1 = ora.prefill(q, k, v, causal=True)
    i0 = 5
    k2, v2 = k.copy(), v.copy()
    k2[:, i0 + 1:] = _rand16(k2[:, i0 + 1:].shape, 10, 3.0)
    v2[:, i0 + 1:] = _rand16(v2[:, i0 + 1:].shape, 11, 3.0)
    o2 = ora.prefill(q, k2, v2, causal=True)
    assert np.array_equal(o1[:, : i0 + 1], o2[:, : i0 + 1])
    assert not np.array_equal(o1[:, i0 + 1:], o2[:, i0 + 1:])


# ---- heads -------------------------------------------------------------------

def pin_gqa_mapping(ora):
    for H_q, H_kv in ((6, 3), (8, 2), (4, 4), (4, 1)):
        B, S, D = 2, 6, 16
        q, k = _rand16((B, S, H_q, D), 12), _rand16((B, S, H_kv, D), 13)
        v = np.zeros((B, S, H_kv, D), np.float16)
        for g in range(H_kv):
            v[:, :, g, :] = g + 1
        for causal in (True, False):
            o = ora.prefill(q, k, v, causal=causal)
            for h in range(H_q):
                want = h * H_kv // H_q + 1
                assert np.allclose(o[:, :, h, :], want, rtol=0, atol=1e-13), (H_q, H_kv, h)
            # and through decode
        kc, vc, bt = W.paginate(k, v, np.full(B, S), 16, 1, (1, 2))
        od = ora.decode_paged(q[:, -1], kc, vc, bt, np.full(B, S, np.int32))
        for h in range(H_q):
            assert np.allclose(od[:, h, :], h * H_kv // H_q + 1, atol=1e-13), (H_q, H_kv, h)


# ---- algebra -----------------------------------------------------------------

def pin_linearity_in_v(ora):
    B, S, H, D = 1, 10, 2, 16
    q, k = _rand16((B, S, H, D), 14), _rand16((B, S, H, D), 15)
    n = np.random.default_rng(16).integers(-128, 129, size=(B, S, H, D))
    v = (n / 64.0).astype(np.float16)
    v2 = (2.0 * (n / 64.0) + 1.0).astype(np.float16)          # exact in binary16
    assert np.array_equal(_f64(v2), 2.0 * _f64(v) + 1.0)
    for causal in (True, False):
        o1 = ora.prefill(q, k, v, causal=causal)
        o2 = ora.prefill(q, k, v2, causal=causal)
        assert np.allclose(o2, 2.0 * o1 + 1.0, rtol=0, atol=1e-13)


def pin_values_one_gives_one(ora):
    B, S, H, D = 2, 7, 3, 32
    q, k = _rand16((B, S, H, D), 17, 2.0), _rand16((B, S, H, D), 18, 2.0)
    v = np.ones((B, S, H, D), np.float16)
    for causal in (True, False):
        o = ora.prefill(q, k, v, causal=causal)
        assert np.allclose(o, 1.0, rtol=0, atol=1e-14)


def pin_noncausal_key_permutation(ora):
    B, S_q, S_kv, H, D = 1, 3, 11, 2, 16
    q, k, v = _rand16((B, S_q, H, D), 19), _rand16((B, S_kv, H, D), 20), _rand16((B, S_kv, H, D), 21)
    perm = np.random.default_rng(22).permutation(S_kv)
    o1 = ora.prefill(q, k, v, causal=False)
    o2 = ora.prefill(q, k[:, perm], v[:, perm], causal=False)
    assert np.allclose(o1, o2, rtol=0, atol=1e-14)


# ---- library special case ------------------------------------------------------

def _torch_sdpa(q, k, v, causal):
    import torch
    H_q, H_kv = q.shape[2], k.shape[2]
    tq = torch.from_numpy(_f64(q)).permute(0, 2, 1, 3)
    tk = torch.from_numpy(_f64(k)).permute(0, 2, 1, 3).repeat_interleave(H_q // H_kv, dim=1)
    tv = torch.from_numpy(_f64(v)).permute(0, 2, 1, 3).repeat_interleave(H_q // H_kv, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    return out.permute(0, 2, 1, 3).contiguous().numpy()


def pin_matches_torch_sdpa(ora):
    cases = [
        (1, 17, 17, 4, 2, 32, True),
        (2, 33, 33, 6, 3, 64, True),
        (2, 9, 21, 4, 1, 128, False),
        (3, 16, 16, 2, 2, 16, False),
    ]
    for i, (B, S_q, S_kv, H_q, H_kv, D, causal) in enumerate(cases):
        q = _rand16((B, S_q, H_q, D), 30 + i)
        k = _rand16((B, S_kv, H_kv, D), 40 + i)
        v = _rand16((B, S_kv, H_kv, D), 50 + i)
        o = ora.prefill(q, k, v, causal=causal)
        assert np.allclose(o, _torch_sdpa(q, k, v, causal), rtol=1e-12, atol=1e-13), i
    # the pages' first unit-test shape (B=1 S=16 H 2/1), uniform inputs
    q, k, v = W.pages_prefill_case(0, 1, 16, 2, 1)
    assert np.allclose(ora.prefill(q, k, v, True), _torch_sdpa(q, k, v, True),
                       rtol=1e-12, atol=1e-13)


def pin_huge_logits(ora):
    """Logits of several hundred overflow exp() unless the row max is taken
    out first; torch's fp64 SDPA handles them, so must the oracle."""
    B, S, H, D = 1, 6, 1, 16
    q = np.zeros((B, S, H, D), np.float16)
    k = np.zeros_like(q)
    q[..., 0] = 60.0
    k[0, :, 0, 0] = np.array([60.0, 0.0, -60.0, 60.0, 10.0, 59.5])   # logits 15*k: up to 900
    v = _rand16((B, S, H, D), 60)
    for causal in (True, False):
        o = ora.prefill(q, k, v, causal=causal)
        assert np.all(np.isfinite(o))
        assert np.allclose(o, _torch_sdpa(q, k, v, causal), rtol=1e-12, atol=1e-13)


# ---- paging --------------------------------------------------------------------

def pin_decode_equals_last_causal_row(ora):
    H_q, H_kv, D, bs = 4, 2, 32, 16
    lens = [1, 15, 16, 17, 33, 50]
    T = max(lens)
    n = len(lens)
    Q, K, V = _rand16((n, T, H_q, D), 70), _rand16((n, T, H_kv, D), 71), _rand16((n, T, H_kv, D), 72)
    kc, vc, bt = W.paginate(K, V, lens, bs, 4, (3, 4))
    q_last = np.stack([Q[s, L - 1] for s, L in enumerate(lens)])
    od = ora.decode_paged(q_last, kc, vc, bt, np.array(lens, np.int32))
    for s, L in enumerate(lens):
        op = ora.prefill(Q[s:s + 1, :L], K[s:s + 1, :L], V[s:s + 1, :L], causal=True)
        assert np.allclose(od[s], op[0, L - 1], rtol=0, atol=1e-14), (s, L)


def pin_decode_block_permutation(ora):
    H_q, H_kv, D, bs = 2, 1, 16, 16
    lens = [40, 7, 64]
    T = max(lens)
    K, V = _rand16((3, T, H_kv, D), 80), _rand16((3, T, H_kv, D), 81)
    q = _rand16((3, H_q, D), 82)
    sl = np.array(lens, np.int32)
    kc1, vc1, bt1 = W.paginate(K, V, lens, bs, 5, (5, 1))
    kc2, vc2, bt2 = W.paginate(K, V, lens, bs, 5, (5, 2))
    assert not np.array_equal(bt1, bt2)
    assert np.array_equal(ora.decode_paged(q, kc1, vc1, bt1, sl), ora.decode_paged(q, kc2, vc2, bt2, sl))


def pin_decode_brute_force(ora):
    from scipy.special import softmax
    H_q, H_kv, D, bs = 2, 1, 16, 16
    lens = [19, 3]
    T = max(lens)
    K, V = _rand16((2, T, H_kv, D), 90), _rand16((2, T, H_kv, D), 91)
    q = _rand16((2, H_q, D), 92)
    kc, vc, bt = W.paginate(K, V, lens, bs, 2, (6, 1))
    od = ora.decode_paged(q, kc, vc, bt, np.array(lens, np.int32))
    for s, L in enumerate(lens):
        for h in range(H_q):
            kk, vv = _f64(K[s, :L, 0]), _f64(V[s, :L, 0])
            p = softmax(kk @ _f64(q[s, h]) / math.sqrt(D))
            assert np.allclose(od[s, h], p @ vv, rtol=0, atol=1e-14), (s, h)


def pin_decode_zero_length_row(ora):
    q = _rand16((2, 2, 16), 93)
    kc, vc = _rand16((2, 1, 16, 16), 94), _rand16((2, 1, 16, 16), 95)
    bt = np.array([[0], [1]], np.int32)
    od = ora.decode_paged(q, kc, vc, bt, np.array([0, 5], np.int32))
    assert np.all(od[0] == 0.0)
    assert np.all(np.isfinite(od[1])) and not np.all(od[1] == 0.0)


def pin_rejects_invalid(ora):
    q, k = _rand16((1, 4, 2, 16), 96), _rand16((1, 5, 2, 16), 97)
    for bad in (lambda: ora.prefill(q, k, k, causal=True),                   # causal, S_q != S_kv
                lambda: ora.prefill(_rand16((1, 4, 3, 16), 98), k, k, False),  # 3 % 2 != 0
                lambda: ora.decode_paged(_rand16((1, 2, 16), 99), _rand16((2, 1, 16, 16), 1),
                                         _rand16((2, 1, 16, 16), 2), np.array([[5]], np.int32),
                                         np.array([4], np.int32))):          # table entry out of range
        try:
            bad()
        except ValueError:
            continue
        raise AssertionError("invalid arguments were accepted")




# ---- paged KV append (write side of the cache) ---------------------------------

def _slots_for(lens, bt, block_size=16):
    """slot of every token of every sequence, in (sequence, token) order."""
    out = []
    for s, L in enumerate(lens):
        for t in range(L):
            out.append(int(bt[s, t // block_size]) * block_size + t % block_size)
    return np.array(out, np.int64)


def pin_kv_append_placement(ora):
    """Each token's rows land at [slot // 16, h, slot % 16, :]; checked against
    numpy fancy indexing on a token-major view of the cache."""
    H, D, bs, nb = 3, 16, 16, 5
    rng = np.random.default_rng(101)
    kc = _rand16((nb, H, bs, D), 102)
    vc = _rand16((nb, H, bs, D), 103)
    n = 23
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    kn, vn = _rand16((n, H, D), 104), _rand16((n, H, D), 105)
    want_k = kc.transpose(0, 2, 1, 3).reshape(nb * bs, H, D).copy()
    want_v = vc.transpose(0, 2, 1, 3).reshape(nb * bs, H, D).copy()
    want_k[slots] = kn
    want_v[slots] = vn
    got = ora.kv_append(kn, vn, kc, vc, slots)
    assert got == n
    assert np.array_equal(kc.transpose(0, 2, 1, 3).reshape(nb * bs, H, D), want_k)
    assert np.array_equal(vc.transpose(0, 2, 1, 3).reshape(nb * bs, H, D), want_v)


def pin_kv_append_skips_padding(ora):
    """Slot -1 (padding) and slots past the pool leave the cache untouched."""
    H, D, bs, nb = 2, 8, 16, 3
    kc, vc = _rand16((nb, H, bs, D), 106), _rand16((nb, H, bs, D), 107)
    k0, v0 = kc.copy(), vc.copy()
    kn, vn = _rand16((4, H, D), 108), _rand16((4, H, D), 109)
    slots = np.array([-1, nb * bs, -1, nb * bs + 5], np.int64)
    assert ora.kv_append(kn, vn, kc, vc, slots) == 0
    assert np.array_equal(kc, k0) and np.array_equal(vc, v0)
    slots[1] = 0  # one valid slot among the padding
    assert ora.kv_append(kn, vn, kc, vc, slots) == 1
    assert np.array_equal(kc[0, :, 0], kn[1]) and np.array_equal(vc[0, :, 0], vn[1])
    kc[0, :, 0], vc[0, :, 0] = k0[0, :, 0], v0[0, :, 0]
    assert np.array_equal(kc, k0) and np.array_equal(vc, v0)


def pin_append_then_decode_equals_prefill(ora):
    """Appending a sequence's K/V through a permuted table and decoding its
    last query reproduces the last row of causal prefill."""
    H_q, H_kv, D, bs = 4, 2, 32, 16
    lens = [37, 16, 5]
    T = max(lens)
    Q, K, V = _rand16((3, T, H_q, D), 110), _rand16((3, T, H_kv, D), 111), _rand16((3, T, H_kv, D), 112)
    bt, nb = W.paged_layout(lens, bs, 4, (9, 9))
    kc = np.zeros((nb, H_kv, bs, D), np.float16)
    vc = np.zeros_like(kc)
    kn = np.concatenate([K[s, :L] for s, L in enumerate(lens)])
    vn = np.concatenate([V[s, :L] for s, L in enumerate(lens)])
    assert ora.kv_append(kn, vn, kc, vc, _slots_for(lens, bt)) == sum(lens)
    q_last = np.stack([Q[s, L - 1] for s, L in enumerate(lens)])
    od = ora.decode_paged(q_last, kc, vc, bt, np.array(lens, np.int32))
    for s, L in enumerate(lens):
        op = ora.prefill(Q[s:s + 1, :L], K[s:s + 1, :L], V[s:s + 1, :L], causal=True)
        assert np.allclose(od[s], op[0, L - 1], rtol=0, atol=1e-14), (s, L)


# ---- QK-norm + NeoX RoPE ------------------------------------------------------

def _np_inv_freq(D, base):
    # the frequency as the cross-attention trace prints it: 1/(base^(arange(0,D,2)/D))
    return 1.0 / (base ** (np.arange(0, D, 2, dtype=np.float64) / D))


def _np_rotate(y, pos, base):
    """NeoX split-half rotation as a complex product: (y_i + i*y_{i+D/2}) *
    exp(i*pos*inv_freq_i), written with numpy's complex arithmetic."""
    D = y.shape[-1]
    z = y[..., : D // 2] + 1j * y[..., D // 2:]
    ang = np.asarray(pos, np.float64)[:, None, None] * _np_inv_freq(D, base)[None, None, :]
    r = z * np.exp(1j * ang)
    return np.concatenate([r.real, r.imag], axis=-1)


def pin_rope_table_frequency_and_angle_addition(ora):
    """Position 1 holds the pages' frequencies (recovered with atan2, every
    angle is below pi there); cos^2 + sin^2 = 1; and row p+q is row p turned
    by row q (the angle is linear in the position)."""
    for D, base in ((128, 1e4), (128, 1e6), (64, 5e5), (32, 1e4)):
        c, s = ora.rope_table(64, D, base)
        assert np.allclose(np.arctan2(s[1], c[1]), _np_inv_freq(D, base), rtol=1e-14, atol=0)
        assert np.allclose(c * c + s * s, 1.0, rtol=0, atol=1e-15)
        assert np.array_equal(c[0], np.ones(D // 2)) and np.array_equal(s[0], np.zeros(D // 2))
        for p_, q_ in ((3, 5), (17, 29), (1, 62)):
            zc = (c[p_] + 1j * s[p_]) * (c[q_] + 1j * s[q_])
            assert np.allclose(zc.real, c[p_ + q_], atol=1e-13) and np.allclose(zc.imag, s[p_ + q_], atol=1e-13)


def pin_rope_position_zero_is_identity(ora):
    x = _rand16((5, 3, 64), 201)
    c, s = ora.rope_table(4, 64, 1e4)
    out = ora.qk_norm_rope(x, None, np.zeros(5, np.int32), c, s)
    assert np.array_equal(out, _f64(x))


def pin_rope_matches_complex_rotation(ora):
    """Rotation only (no weight): the oracle equals the complex product at
    random positions, for D in {32, 64, 128} and two bases."""
    for D, base in ((128, 1e6), (64, 1e4), (32, 1e4)):
        x = _rand16((9, 4, D), 202 + D)
        pos = np.random.default_rng(203).integers(0, 4096, 9).astype(np.int32)
        c, s = ora.rope_table(4096, D, base)
        got = ora.qk_norm_rope(x, None, pos, c, s)
        assert np.allclose(got, _np_rotate(_f64(x), pos, base), rtol=0, atol=1e-12)


def pin_rope_preserves_norm_and_depends_on_offset_only(ora):
    """A rotation keeps every head's norm; <R(m) q, R(n) k> depends on m - n."""
    D = 128
    c, s = ora.rope_table(3000, D, 1e6)
    q, k = _rand16((1, 2, D), 204), _rand16((1, 2, D), 205)
    qr = lambda p: ora.qk_norm_rope(q, None, np.array([p], np.int32), c, s)
    kr = lambda p: ora.qk_norm_rope(k, None, np.array([p], np.int32), c, s)
    assert np.allclose(np.linalg.norm(qr(1234), axis=-1), np.linalg.norm(_f64(q), axis=-1), rtol=1e-14)
    for m, n, dlt in ((10, 3, 500), (700, 2900, -650), (0, 0, 2999)):
        a = np.sum(qr(m) * kr(n), axis=-1)
        b = np.sum(qr(m + dlt) * kr(n + dlt), axis=-1)
        assert np.allclose(a, b, rtol=1e-11, atol=1e-11), (m, n, dlt)


def pin_rmsnorm_unit_mean_square_and_scale_invariance(ora):
    """With unit weight and eps 0 the rows have mean square 1, and scaling
    the input by 2 (exact in binary16) changes nothing."""
    D = 128
    c, s = ora.rope_table(2, D, 1e4)
    x = _rand16((6, 5, D), 206)
    w = np.ones(D, np.float16)
    y = ora.qk_norm_rope(x, w, np.zeros(6, np.int32), c, s, eps=0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)
    y2 = ora.qk_norm_rope((x.astype(np.float32) * 2).astype(np.float16), w, np.zeros(6, np.int32), c, s, eps=0.0)
    assert np.allclose(y, y2, rtol=1e-15, atol=0)


def pin_rmsnorm_constant_row_closed_form(ora):
    """A row of D equal values a gives a / sqrt(a^2 + eps) * w_d (position 0),
    which pins the mean (not the sum), eps inside the root and the weight."""
    D = 64
    c, s = ora.rope_table(1, D, 1e4)
    w = _rand16((D,), 207)
    for a, eps in ((0.5, 1e-6), (0.01, 1e-3), (3.0, 0.25)):
        x = np.full((1, 1, D), a, np.float16)
        av = float(x[0, 0, 0])
        got = ora.qk_norm_rope(x, w, np.zeros(1, np.int32), c, s, eps=eps)[0, 0]
        assert np.allclose(got, av / math.sqrt(av * av + eps) * _f64(w), rtol=1e-14, atol=0), (a, eps)
    zero = ora.qk_norm_rope(np.zeros((1, 1, D), np.float16), w, np.zeros(1, np.int32), c, s, eps=1e-6)
    assert np.array_equal(zero, np.zeros((1, 1, D)))


def pin_norm_then_rope_against_numpy(ora):
    """Non-uniform weight at random positions: the oracle equals numpy's
    RMSNorm followed by the complex rotation, and differs from the opposite
    order (the pages put QK-norm before RoPE)."""
    D, eps, base = 128, 1e-6, 1e6
    x = _rand16((7, 3, D), 208, scale=2.0)
    w = (np.random.default_rng(209).uniform(0.2, 2.0, D)).astype(np.float16)
    pos = np.random.default_rng(210).integers(1, 2048, 7).astype(np.int32)
    c, s = ora.rope_table(2048, D, base)
    got = ora.qk_norm_rope(x, w, pos, c, s, eps=eps)
    xf = _f64(x)
    y = xf / np.sqrt(np.mean(xf * xf, axis=-1, keepdims=True) + eps) * _f64(w)
    assert np.allclose(got, _np_rotate(y, pos, base), rtol=0, atol=1e-12)
    r = _np_rotate(xf, pos, base)
    other = r / np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + eps) * _f64(w)
    assert not np.allclose(got, other, atol=1e-3)


def pin_rope_bad_position_gives_nan_row(ora):
    D = 32
    c, s = ora.rope_table(8, D, 1e4)
    x = _rand16((4, 2, D), 211)
    out = ora.qk_norm_rope(x, None, np.array([3, -1, 8, 7], np.int32), c, s)
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all()
    assert not np.isnan(out[0]).any() and not np.isnan(out[3]).any()


def pin_rope_rejects_invalid(ora):
    for args in ((4, 7, 1e4), (0, 8, 1e4), (4, 8, 0.0)):
        try:
            ora.rope_table(*args)
        except ValueError:
            continue
        raise AssertionError(f"rope_table accepted {args}")


# ---- cross-attention module with interleaved-pair RoPE ------------------------

def _np_rotate_adjacent(x, base):
    """Adjacent-pair rotation as a complex product: (x_{2j} + i*x_{2j+1}) *
    exp(i*t*inv_freq_j) for row t of [B, T, H, D], numpy complex arithmetic."""
    B, T, H, D = x.shape
    z = x[..., 0::2] + 1j * x[..., 1::2]
    ang = np.arange(T, dtype=np.float64)[None, :, None, None] * _np_inv_freq(D, base)[None, None, None, :]
    r = z * np.exp(1j * ang)
    out = np.empty(x.shape, np.float64)
    out[..., 0::2], out[..., 1::2] = r.real, r.imag
    return out


def pin_rope_interleaved_matches_complex_rotation(ora):
    """The cross-attention workload's rotation (adjacent pairs, base 1e4)
    equals numpy's complex product, at its own shapes and at D = 128."""
    for shape, base in (((4, 64, 8, 32), 1e4), ((4, 128, 8, 32), 1e4), ((2, 300, 2, 128), 1e6)):
        x = _rand16(shape, 230 + shape[1])
        assert np.allclose(ora.rope_interleaved(x, base), _np_rotate_adjacent(_f64(x), base), rtol=0, atol=1e-12)


def pin_rope_interleaved_identity_norm_and_offset(ora):
    """Row 0 is unrotated (bitwise); every pair keeps its length; and the dot
    product of rows m and n of two rotated tensors depends on m - n only."""
    x = _rand16((1, 96, 2, 64), 240)
    r = ora.rope_interleaved(x)
    assert np.array_equal(r[:, 0], _f64(x)[:, 0])
    pn = lambda a: np.hypot(a[..., 0::2], a[..., 1::2])
    assert np.allclose(pn(r), pn(_f64(x)), rtol=1e-14, atol=0)
    # the same vector at every position: <R(m) q, R(n) k> depends on m - n
    q = np.broadcast_to(_rand16((1, 1, 1, 64), 241), (1, 96, 1, 64)).copy()
    k = np.broadcast_to(_rand16((1, 1, 1, 64), 242), (1, 96, 1, 64)).copy()
    rq, rk = ora.rope_interleaved(q)[0, :, 0], ora.rope_interleaved(k)[0, :, 0]
    for m, n, d in ((5, 2, 40), (80, 10, -9), (0, 0, 95)):
        assert np.isclose(rq[m] @ rk[n], rq[m + d] @ rk[n + d], rtol=1e-12, atol=1e-12)


def pin_rope_interleaved_rejects_invalid(ora):
    import pytest
    with pytest.raises(ValueError):
        ora.rope_interleaved(_rand16((1, 2, 1, 7), 243))


def _module_inputs(B, T_q, T_k, dim, seed):
    rng = np.random.default_rng(seed)
    xq = rng.standard_normal((B, T_q, dim)).astype(np.float16)
    xk = rng.standard_normal((B, T_k, dim)).astype(np.float16)
    bound = 1.0 / math.sqrt(dim)
    ws = [rng.uniform(-bound, bound, (dim, dim)).astype(np.float16) for _ in range(4)]
    return xq, xk, ws


def _torch_module(xq, xk, ws, H, base):
    """The module written with torch in fp64 on the CPU: F.linear, RoPE as a
    complex product over adjacent pairs (torch.view_as_complex / torch.polar),
    scaled_dot_product_attention, F.linear."""
    import torch
    import torch.nn.functional as F
    t = lambda a: torch.from_numpy(_f64(a))
    B, T_q, dim = xq.shape
    T_k, D = xk.shape[1], dim // H
    q, k, v = F.linear(t(xq), t(ws[0])), F.linear(t(xk), t(ws[1])), F.linear(t(xk), t(ws[2]))

    def rope(x, T):
        x = x.view(B, T, H, D // 2, 2)
        freq = base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
        ang = torch.arange(T, dtype=torch.float64)[:, None] * freq[None, :]
        z = torch.view_as_complex(x.contiguous()) * torch.polar(torch.ones_like(ang), ang)[None, :, None, :]
        return torch.view_as_real(z).reshape(B, T, H, D)

    qh = rope(q, T_q).transpose(1, 2).contiguous()
    kh = rope(k, T_k).transpose(1, 2).contiguous()
    vh = v.view(B, T_k, H, D).transpose(1, 2).contiguous()
    a = F.scaled_dot_product_attention(qh, kh, vh)
    return F.linear(a.transpose(1, 2).reshape(B, T_q, dim), t(ws[3])).numpy()


def pin_cross_attention_matches_torch(ora):
    """The pages' shape (B=4, T_q=64, T_k=128, dim=256, 8 heads) and two
    others, against the torch fp64 module."""
    for (B, T_q, T_k, dim, H, base, seed) in ((4, 64, 128, 256, 8, 1e4, 301), (2, 5, 9, 64, 2, 1e4, 302),
                                              (1, 17, 3, 128, 1, 5e5, 303)):
        xq, xk, ws = _module_inputs(B, T_q, T_k, dim, seed)
        got = ora.cross_attention(xq, xk, *ws, H=H, base=base)
        assert np.allclose(got, _torch_module(xq, xk, ws, H, base), rtol=1e-12, atol=1e-13), (B, T_q, T_k, dim, H)


def pin_cross_attention_identical_memory_rows(ora):
    """Identical x_kv rows give identical value rows: every query attends to
    the same value whatever the softmax weights, so out = (x W_v^T) W_o^T."""
    B, T_q, T_k, dim, H = 2, 7, 11, 64, 4
    xq, xk, ws = _module_inputs(B, T_q, T_k, dim, 304)
    xk[:] = xk[:, :1, :]
    got = ora.cross_attention(xq, xk, *ws, H=H)
    want = (_f64(xk[:, 0]) @ _f64(ws[2]).T) @ _f64(ws[3]).T
    assert np.allclose(got, np.broadcast_to(want[:, None, :], got.shape), rtol=1e-12, atol=1e-14)


def pin_cross_attention_single_key(ora):
    """With one key the softmax is 1 and RoPE on K is the identity (pos 0)."""
    B, T_q, dim, H = 3, 6, 32, 2
    xq, xk, ws = _module_inputs(B, T_q, 1, dim, 305)
    got = ora.cross_attention(xq, xk, *ws, H=H)
    want = (_f64(xk[:, 0]) @ _f64(ws[2]).T) @ _f64(ws[3]).T
    assert np.allclose(got, np.broadcast_to(want[:, None, :], got.shape), rtol=1e-12, atol=1e-14)


def pin_decode_forked_tables_equal_private_copies(ora):
    """A fork copies table entries only: decoding sequences whose tables share
    the prompt's physical blocks equals decoding with a private copy of those
    blocks per sequence, bit for bit."""
    q, kc, vc, bt, sl, gs, pb = W.forked_decode_inputs([4, 1, 3], [48, 16, 37], [3, 0, 20, 9, 1, 30, 16, 2],
                                                       4, 2, D=32, seed=401)
    shared = ora.decode_paged(q, kc, vc, bt, sl)
    # give every sequence private copies of its group's shared blocks
    extra_k, extra_v, bt2 = [kc], [vc], bt.copy()
    nxt = kc.shape[0]
    for gi in range(len(pb)):
        for s in range(gs[gi], gs[gi + 1]):
            for b in range(pb[gi]):
                phys = bt[s, b]
                extra_k.append(kc[phys:phys + 1])
                extra_v.append(vc[phys:phys + 1])
                bt2[s, b] = nxt
                nxt += 1
    kc2, vc2 = np.concatenate(extra_k), np.concatenate(extra_v)
    private = ora.decode_paged(q, kc2, vc2, bt2, sl)
    assert np.array_equal(shared, private)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
