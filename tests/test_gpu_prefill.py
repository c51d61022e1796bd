"""Prefill parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded inputs, plus invariants checked on the GPU output itself."""
import os

import numpy as np
import pytest

import oracle
from attention_attn_prefill_amd import workloads as W
from gpu_helpers import assert_parity, gpu_prefill, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_unit_cases.txt")


def pages_cases():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if line:
            rows.append((line[0], *map(int, line[1:])))
    return rows


def _rand(shape, seed, scale=1.0):
    return W.normal_f16(shape, (99, seed)) if scale == 1.0 else \
        (W.normal_f16(shape, (99, seed)).astype(np.float32) * scale).astype(np.float16)


@pytest.mark.parametrize("name", ["tiny_causal", "cross_attn"])
def test_small_configs_full(name):
    """Every output element of the two small configurations.  The
    cross-attention core takes Q and K rotated by adjacent-pair RoPE (base
    10000, positions 0..T-1), done in fp64 by the oracle and rounded to fp16,
    so both sides see the same rotated inputs."""
    cfg = W.CONFIGS[name]
    q, k, v = W.prefill_inputs(cfg)
    if name == "cross_attn":
        q = oracle.rope_interleaved(q, 1e4).astype(np.float16)
        k = oracle.rope_interleaved(k, 1e4).astype(np.float16)
    say(name, q.shape, k.shape)
    got = gpu_prefill(q, k, v, cfg.causal)
    ref = oracle.prefill(q, k, v, cfg.causal)
    assert_parity(got, ref, name)


def test_pages_unit_cases():
    """The pages' unit-test shapes with inputs uniform in [-0.5, 0.5); their
    pass criterion was a max absolute error below 5e-3, and their kernels
    reached about 1.2e-4."""
    for case, (kind, B, S, H_q, H_kv, D) in enumerate(pages_cases()):
        if kind != "prefill":
            continue
        q, k, v = W.pages_prefill_case(case, B, S, H_q, H_kv, D)
        say("pages prefill", B, S, H_q, H_kv, D)
        err = assert_parity(gpu_prefill(q, k, v, True), oracle.prefill(q, k, v, True), "pages")
        assert err < 5e-3


EDGE = [
    # B, S_q, S_kv, H_q, H_kv, D, causal
    (1, 1, 1, 2, 1, 128, True),
    (1, 17, 17, 4, 2, 128, True),
    (2, 63, 63, 2, 2, 128, True),
    (1, 64, 64, 8, 1, 128, True),
    (1, 65, 65, 4, 4, 128, True),
    (1, 127, 127, 2, 1, 128, True),
    (1, 129, 129, 4, 2, 128, True),
    (3, 200, 200, 6, 3, 128, True),
    (1, 257, 257, 2, 1, 64, True),
    (2, 300, 300, 4, 2, 32, True),
    (1, 1, 300, 4, 2, 128, False),
    (2, 33, 100, 4, 1, 128, False),
    (1, 130, 7, 2, 2, 64, False),
    (1, 256, 64, 8, 8, 32, False),
    (1, 384, 384, 2, 1, 128, False),
    # several query-tile pairs with a ragged last tile, and an odd middle
    # tile, on two-head workgroups (each SIMD pairs the two heads' wavefronts)
    (2, 1000, 1000, 4, 2, 128, True),
    (1, 777, 777, 8, 2, 128, True),
    (1, 520, 520, 4, 2, 128, False),
    # non-causal, S_q != S_kv, two-head workgroups at D = 32 and 64
    (2, 200, 150, 4, 2, 32, False),
    (1, 300, 260, 8, 2, 64, False),
    # head_dim 128 with an odd H_q / H_kv (one head, 64 rows per wavefront,
    # 256-row query tiles): several tile pairs, a ragged last tile, an odd
    # middle tile, and a non-causal S_q != S_kv case
    (1, 1000, 1000, 4, 4, 128, True),
    (2, 700, 700, 6, 2, 128, True),
    (1, 300, 500, 3, 1, 128, False),
    # head_dim 128, two-head workgroups, non-causal with more keys than rows
    (1, 600, 900, 8, 4, 128, False),
]


@pytest.mark.parametrize("B,S_q,S_kv,H_q,H_kv,D,causal", EDGE)
def test_edge_shapes(B, S_q, S_kv, H_q, H_kv, D, causal):
    seed = hash((B, S_q, S_kv, H_q, H_kv, D, causal)) % 10000
    q = _rand((B, S_q, H_q, D), seed)
    k = _rand((B, S_kv, H_kv, D), seed + 1)
    v = _rand((B, S_kv, H_kv, D), seed + 2)
    say("edge", B, S_q, S_kv, H_q, H_kv, D, causal)
    assert_parity(gpu_prefill(q, k, v, causal), oracle.prefill(q, k, v, causal), "edge")


def test_large_logits():
    """Scores of several tens force max updates inside the running softmax."""
    B, S, H_q, H_kv, D = 1, 320, 4, 2, 128
    q = _rand((B, S, H_q, D), 11, 3.0)
    k = _rand((B, S, H_kv, D), 12, 3.0)
    v = _rand((B, S, H_kv, D), 13)
    say("large logits")
    for causal in (True, False):
        assert_parity(gpu_prefill(q, k, v, causal), oracle.prefill(q, k, v, causal), "large")


def test_large_logits_one_head_workgroups():
    """The overflow rerun on one-head (64 rows per wavefront) workgroups."""
    B, S, H_q, H_kv, D = 1, 600, 3, 1, 128
    q = _rand((B, S, H_q, D), 21, 3.0)
    k = _rand((B, S, H_kv, D), 22, 3.0)
    v = _rand((B, S, H_kv, D), 23)
    say("large logits, one-head workgroups")
    for causal in (True, False):
        assert_parity(gpu_prefill(q, k, v, causal), oracle.prefill(q, k, v, causal), "large HP1")


def test_increasing_logits():
    """Keys aligned with the query and growing along the sequence: the row
    max grows in every tile, so every tile rescales the running output."""
    B, S, H, D = 1, 512, 1, 128
    rng = np.random.default_rng(5)
    qhat = rng.standard_normal(D)
    qhat /= np.linalg.norm(qhat)
    q = np.broadcast_to((4.0 * qhat).astype(np.float16), (B, S, H, D)).copy()
    kf = (np.arange(S)[:, None] / S * 6.0) * qhat[None, :] + 0.05 * rng.standard_normal((S, D))
    k = kf.astype(np.float16).reshape(B, S, H, D)
    v = _rand((B, S, H, D), 14)
    say("increasing logits")
    assert_parity(gpu_prefill(q, k, v, True), oracle.prefill(q, k, v, True), "increasing")


@pytest.mark.timeout(300)
def test_qwen3_prefill_full_size_every_element():
    """The Qwen3-shaped prefill (B=4, S=2048, 16/8 heads, D=128, causal) at
    full size, every output element against the fp64 oracle."""
    cfg = W.CONFIGS["qwen3_prefill"]
    q, k, v = W.prefill_inputs(cfg)
    say("qwen3_prefill full size")
    got = gpu_prefill(q, k, v, True)
    ref = oracle.prefill(q, k, v, True)
    assert_parity(got, ref, "qwen3_prefill")


@pytest.mark.timeout(600)
def test_long_prefill_full_size_sampled_rows():
    cfg = W.CONFIGS["long_prefill"]
    q, k, v = W.prefill_inputs(cfg)
    say("long_prefill full size")
    got = gpu_prefill(q, k, v, True).reshape(-1, cfg.D)
    rows = W.sample_prefill_rows(cfg, 400, tile=4096)
    ref = oracle.prefill(q, k, v, True, rows=rows)
    assert_parity(got[rows], ref, "long_prefill")


def _max_s_kv(H_kv, D):
    """Largest S_kv the host accepts: K/V rows of one batch entry are addressed
    with 32-bit byte offsets, and the kernels stage up to three 64-key tiles
    past the last one, so (ceil(S_kv / 64) + 3) * 64 * H_kv * D * 2 < 2^31."""
    return (((1 << 31) - 1) // (64 * H_kv * D * 2) - 3) * 64


@pytest.mark.timeout(300)
@pytest.mark.parametrize("D,short", [(128, 5), (64, 0)])
def test_non_causal_at_the_kv_offset_limit(D, short):
    """The largest K/V that the 32-bit offsets allow (one kv head, 2.1 GB each
    of K and V): 40 query rows of two heads against every key.  Scores near 0
    for the bulk of the keys would make the output an average of millions of
    rows, near zero whatever keys were read, so eight needle keys spread over
    the whole range, the last one at the end of the buffer, score far above
    the rest (q[..., 0] = 8, the needle's k[0] = 32 down to 28.5) and carry
    graded weights.  A missed or misplaced needle moves the output by several
    percent.  Every row of two heads at the first and last four query
    positions against the oracle."""
    S_kv = _max_s_kv(1, D) - short
    B, S_q, H_q, H_kv = 1, 40, 2, 1
    q = _rand((B, S_q, H_q, D), 71)
    q[..., 0] = 8
    k = _rand((B, S_kv, H_kv, D), 72)
    k *= np.float16(0.1)
    needles = [3, 64 * 1000 + 17, S_kv // 3, S_kv // 2 + 1, S_kv - 64 * 7 - 2, S_kv - 65, S_kv - 2, S_kv - 1]
    for i, j in enumerate(needles):
        k[0, j, 0, 0] = 32.0 - 0.5 * i
    v = _rand((B, S_kv, H_kv, D), 73)
    say("kv offset limit", D, S_kv)
    got = gpu_prefill(q, k, v, False).reshape(-1, D)
    pos = np.array([0, 1, 2, 3, S_q - 4, S_q - 3, S_q - 2, S_q - 1], np.int64)
    rows = np.concatenate([pos * H_q + h for h in range(H_q)])
    ref = oracle.prefill(q, k, v, False, rows=rows)
    assert np.abs(ref).max() > 0.1  # the needles dominate
    assert_parity(got[rows], ref, f"kv offset limit D={D}")


# ---- invariants on the GPU output ------------------------------------------

def test_values_one_give_one():
    B, S, H_q, H_kv, D = 2, 200, 4, 2, 128
    q, k = _rand((B, S, H_q, D), 21, 2.0), _rand((B, S, H_kv, D), 22, 2.0)
    v = np.ones((B, S, H_kv, D), np.float16)
    for causal in (True, False):
        got = gpu_prefill(q, k, v, causal).astype(np.float64)
        assert np.allclose(got, 1.0, rtol=0, atol=ATOL_ONE)


ATOL_ONE = 2e-3  # the fp16 weights sum to 1 within rounding


def test_row0_is_v0_exactly():
    B, S, H_q, H_kv, D = 2, 150, 8, 2, 128
    q, k, v = _rand((B, S, H_q, D), 31), _rand((B, S, H_kv, D), 32), _rand((B, S, H_kv, D), 33)
    got = gpu_prefill(q, k, v, True)
    for h in range(H_q):
        assert np.array_equal(got[:, 0, h], v[:, 0, h * H_kv // H_q])


def test_future_keys_do_not_change_past_rows():
    B, S, H, D = 1, 300, 2, 128
    q, k, v = _rand((B, S, H, D), 41), _rand((B, S, H, D), 42), _rand((B, S, H, D), 43)
    o1 = gpu_prefill(q, k, v, True)
    cut = 137
    k2, v2 = k.copy(), v.copy()
    k2[:, cut + 1:] = _rand(k2[:, cut + 1:].shape, 44, 2.0)
    v2[:, cut + 1:] = _rand(v2[:, cut + 1:].shape, 45, 2.0)
    o2 = gpu_prefill(q, k2, v2, True)
    assert np.array_equal(o1[:, : cut + 1], o2[:, : cut + 1])


def test_gqa_constant_values():
    B, S, H_q, H_kv, D = 1, 130, 8, 2, 128
    q, k = _rand((B, S, H_q, D), 51), _rand((B, S, H_kv, D), 52)
    v = np.zeros((B, S, H_kv, D), np.float16)
    for g in range(H_kv):
        v[:, :, g] = g + 1
    got = gpu_prefill(q, k, v, True).astype(np.float64)
    for h in range(H_q):
        assert np.allclose(got[:, :, h], h * H_kv // H_q + 1, rtol=0, atol=4e-3)


def test_deterministic():
    B, S, H_q, H_kv, D = 1, 333, 4, 2, 128
    q, k, v = _rand((B, S, H_q, D), 61), _rand((B, S, H_kv, D), 62), _rand((B, S, H_kv, D), 63)
    assert np.array_equal(gpu_prefill(q, k, v, True), gpu_prefill(q, k, v, True))
