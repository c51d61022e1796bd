"""Paged-decode parity: the HIP path (split-K and single pass, through the C
ABI) against the fp64 oracle, plus paging invariants on the GPU output."""
import numpy as np
import pytest

import oracle
from attention_attn_prefill_amd import AttnError, ATTN_ERR_WORKSPACE
from attention_attn_prefill_amd import workloads as W
from gpu_helpers import assert_parity, dev, gpu_decode, gpu_prefill, say
from test_gpu_prefill import pages_cases

pytestmark = pytest.mark.gpu


def _rand(shape, seed):
    return W.normal_f16(shape, (98, seed))


def _paged_problem(lens, H_q, H_kv, max_bps, seed, D=128):
    n = len(lens)
    q = _rand((n, H_q, D), seed)
    T = max(max(lens), 1)
    K, V = _rand((n, T, H_kv, D), seed + 1), _rand((n, T, H_kv, D), seed + 2)
    kc, vc, bt = W.paginate(K, V, lens, 16, max_bps, (seed, 3))
    return q, kc, vc, bt, np.array(lens, np.int32), K, V


def test_pages_unit_cases():
    """The pages' decode shapes with uniform inputs and identity tables."""
    for case, (kind, B, S, H_q, H_kv, D) in enumerate(pages_cases()):
        if kind == "prefill":
            continue
        q, kc, vc, bt, sl, _, _ = W.pages_decode_case(case, B, S, H_q, H_kv, D)
        say("pages decode", B, S, H_q, H_kv)
        ref = oracle.decode_paged(q, kc, vc, bt, sl)
        for split in (True, False):
            err = assert_parity(gpu_decode(q, kc, vc, bt, sl, split), ref, "pages decode")
            assert err < 5e-3


def test_paged_decode_full():
    cfg = W.CONFIGS["paged_decode"]
    q, kc, vc, bt, sl = W.decode_inputs(cfg)
    say("paged_decode full", kc.shape)
    ref = oracle.decode_paged(q, kc, vc, bt, sl)
    assert_parity(gpu_decode(q, kc, vc, bt, sl, split=True), ref, "paged_decode split")
    assert_parity(gpu_decode(q, kc, vc, bt, sl, split=False), ref, "paged_decode single")


@pytest.mark.timeout(900)
def test_long_decode_full_size_every_sequence():
    """The long-context decode (64 sequences of 32768 tokens, split-K) at full
    size: all 64 sequences, every element, against the fp64 oracle."""
    cfg = W.CONFIGS["long_decode"]
    say("long_decode: generating 2 x 4 GiB of cache")
    q, kc, vc, bt, sl = W.decode_inputs(cfg)
    say("long_decode full size", kc.shape)
    got = gpu_decode(q, kc, vc, bt, sl, split=True)
    ref = oracle.decode_paged(q, kc, vc, bt, sl)
    assert_parity(got, ref, "long_decode")


LENS = [1, 2, 15, 16, 17, 31, 32, 33, 100, 511, 512, 513, 1000, 1024, 1500, 2049]


@pytest.mark.parametrize("H_q,H_kv", [(16, 8), (8, 8), (16, 4), (8, 1), (6, 2), (3, 1)])
def test_ragged_lengths_and_group_sizes(H_q, H_kv):
    q, kc, vc, bt, sl, _, _ = _paged_problem(LENS, H_q, H_kv, 160, H_q * 10 + H_kv)
    say("ragged", H_q, H_kv)
    ref = oracle.decode_paged(q, kc, vc, bt, sl)
    split = gpu_decode(q, kc, vc, bt, sl, split=True)
    single = gpu_decode(q, kc, vc, bt, sl, split=False)
    assert_parity(split, ref, "split")
    assert_parity(single, ref, "single")


# Split-K over a workspace cuts the (sequence, kv head, block) order into
# equal runs: with few blocks in all, runs of 16 blocks cross many short
# (sequence, kv head) segments, long sequences span several runs, and empty
# sequences (in the middle, two in a row, and last) own no blocks at all.
WALK_LENS = [0, 1, 16, 17, 0, 0, 300, 5, 4000, 33, 0, 2500, 16, 1, 48, 0]


# (6, 3): 1024 workgroups do not split evenly over 3 kv heads; the last one
# has no run
@pytest.mark.parametrize("H_q,H_kv", [(16, 8), (8, 1), (6, 2), (4, 4), (6, 3)])
def test_split_runs_walk_many_segments(H_q, H_kv):
    q, kc, vc, bt, sl, _, _ = _paged_problem(WALK_LENS, H_q, H_kv, 256, 300 + H_q * 10 + H_kv)
    say("run walk", H_q, H_kv)
    live = [i for i, L in enumerate(WALK_LENS) if L > 0]
    ref = oracle.decode_paged(q, kc, vc, bt, sl, seqs=live)
    for split in (True, False):
        got = gpu_decode(q, kc, vc, bt, sl, split)
        assert np.all(got[[i for i, L in enumerate(WALK_LENS) if L == 0]] == 0.0)
        assert_parity(got[live], ref, "run walk split" if split else "run walk single")


# Beyond 4096 sequences the balanced mode (whose per-sequence cost prefix
# lives in LDS) gives way to fixed-length splits of 128 blocks, each with its
# own partial slot, and the merge kernel for sequences longer than one split.
@pytest.mark.timeout(300)
@pytest.mark.parametrize("H_q,H_kv", [(16, 8), (8, 1)])
def test_fixed_splits_beyond_the_balanced_limit(H_q, H_kv):
    n, max_bps, D = 5000, 256, 128
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([97, H_q, H_kv])))
    lens = g.integers(1, 64, size=n, endpoint=True)
    lens[::499] = g.integers(2049, 4096, size=len(lens[::499]), endpoint=True)  # two splits each
    lens[7] = 2048  # exactly one full split
    lens = lens.astype(np.int32)
    bt, num_blocks = W.paged_layout(lens, 16, max_bps, (97, H_q, H_kv, 1))
    q = _rand((n, H_q, D), 400 + H_q + H_kv)
    kc = _rand((num_blocks, H_kv, 16, D), 401 + H_q + H_kv)
    vc = _rand((num_blocks, H_kv, 16, D), 402 + H_q + H_kv)
    say("fixed splits", n, H_q, H_kv, num_blocks)
    ref = oracle.decode_paged(q, kc, vc, bt, lens)
    for split in (True, False):
        assert_parity(gpu_decode(q, kc, vc, bt, lens, split), ref,
                      "fixed splits" if split else "fixed splits single")


def test_block_permutation_invariance_is_bitwise():
    lens = [700, 33, 1200, 16]
    n, H_q, H_kv, D = len(lens), 16, 8, 128
    q = _rand((n, H_q, D), 71)
    K, V = _rand((n, max(lens), H_kv, D), 72), _rand((n, max(lens), H_kv, D), 73)
    sl = np.array(lens, np.int32)
    kc1, vc1, bt1 = W.paginate(K, V, lens, 16, 80, (7, 1))
    kc2, vc2, bt2 = W.paginate(K, V, lens, 16, 80, (7, 2))
    say("permutation")
    for split in (True, False):
        assert np.array_equal(gpu_decode(q, kc1, vc1, bt1, sl, split),
                              gpu_decode(q, kc2, vc2, bt2, sl, split))


def test_decode_equals_last_row_of_causal_prefill():
    lens = [1, 77, 640]
    H_q, H_kv, D = 16, 8, 128
    for i, L in enumerate(lens):
        Q = _rand((1, L, H_q, D), 80 + i)
        K, V = _rand((1, L, H_kv, D), 90 + i), _rand((1, L, H_kv, D), 100 + i)
        kc, vc, bt = W.paginate(K, V, [L], 16, 64, (8, i))
        say("decode vs prefill", L)
        pre = gpu_prefill(Q, K, V, True)[0, L - 1].astype(np.float64)
        dec = gpu_decode(Q[:, L - 1], kc, vc, bt, np.array([L], np.int32))[0].astype(np.float64)
        assert np.allclose(dec, pre, rtol=2e-2, atol=8e-3)


def test_zero_length_gives_zero_row_and_bad_inputs_give_nan():
    lens = [0, 40, 40, 40, 5000]
    q, kc, vc, bt, sl, _, _ = _paged_problem([1, 40, 40, 40, 1], 4, 2, 80, 120)
    sl = np.array(lens, np.int32)       # seq 0 empty, seq 4 longer than its table (80 blocks)
    bt = bt.copy()
    bt[2, 1] = kc.shape[0]              # seq 2 points past the pool
    bt[3, 0] = -7                       # seq 3 has a negative entry
    bt[4, :] = 0
    ref = oracle.decode_paged(q, kc, vc, bt, sl, seqs=[1])  # only the valid row
    for split in (True, False):
        say("edge rows split" if split else "edge rows single")
        got = gpu_decode(q, kc, vc, bt, sl, split).astype(np.float64)
        assert np.all(got[0] == 0.0)
        assert_parity(got[1].astype(np.float16), ref[0], "valid row next to bad ones")
        assert np.all(np.isnan(got[2])) and np.all(np.isnan(got[3])) and np.all(np.isnan(got[4]))


def test_workspace_too_small_is_rejected():
    import torch
    from attention_attn_prefill_amd import attn_decode_paged
    q, kc, vc, bt, sl, _, _ = _paged_problem([600, 700], 16, 8, 64, 130)
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float16, device="cuda")
    with pytest.raises(AttnError) as e:
        attn_decode_paged(dev(q), dev(kc), dev(vc), out, dev(bt), dev(sl), workspace=ws)
    assert e.value.status == ATTN_ERR_WORKSPACE
