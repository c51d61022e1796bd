"""Paged decode of forked sequences (shared prompt blocks read once per
group) on the GPU, against the fp64 oracle's plain paged decode over the
same tables -- the cascade is an exact reordering of that sum -- and against
the GPU's own plain paged decode."""
import numpy as np
import pytest

import oracle
from attention_attn_prefill_amd import workloads as W
from gpu_helpers import assert_parity, dev, gpu_decode, host, say

pytestmark = pytest.mark.gpu


def gpu_shared(q, kc, vc, bt, sl, gs, pb, max_group_size=None):
    import torch
    from attention_attn_prefill_amd import (attn_decode_paged_shared_prefix,
                                            attn_decode_paged_shared_prefix_workspace_size)
    mgs = max_group_size or int(np.max(np.diff(gs)))
    n = attn_decode_paged_shared_prefix_workspace_size(q.shape[0], q.shape[1], kc.shape[1], q.shape[2],
                                                       bt.shape[1], kc.shape[2], len(pb), mgs)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.full(q.shape, float("nan"), dtype=torch.float16, device="cuda")
    attn_decode_paged_shared_prefix(dev(q), dev(kc), dev(vc), out, dev(bt), dev(sl), dev(gs), dev(pb), mgs, ws)
    torch.cuda.synchronize()
    return host(out)


def assert_close_to_plain(got, plain):
    """Shared-prefix and plain decode compute the same sum in fp32 with fp16
    weights and differ only in rounding: two fp16 output roundings (2^-11
    relative each) and the fp32 summation order.  Bound: 2e-4 + 2e-3 |plain|,
    far tighter than the attention tolerance, so a dropped, repeated or
    misplaced key (which moves rows by about |v| / context length) fails."""
    g, p = got.astype(np.float64), plain.astype(np.float64)
    bad = ~(np.abs(g - p) <= 2e-4 + 2e-3 * np.abs(p))
    assert not bad.any(), f"{int(bad.sum())} elements off plain decode; worst {np.abs(g - p).max():.3e}"


CASES = [  # group sizes, prompt lengths, suffix range, H_q, H_kv
    ([8] * 4, [512] * 4, (1, 200), 16, 8),        # 16 query rows per group
    ([16] * 2, [1024, 48], (0, 64), 16, 8),       # 32 rows: one full column block
    ([20, 3], [300, 900], (1, 100), 16, 8),       # 40 rows: two column blocks; partial prompt blocks
    ([4, 4, 1], [2048, 16, 0], (1, 40), 8, 8),    # ratio 1; a group without a prefix
    ([6, 2], [640, 640], (0, 0), 32, 8),          # ratio 4; sequences that are only the prompt
    ([1] * 5, [100, 200, 300, 400, 500], (5, 50), 16, 2),  # singleton groups, ratio 8
    ([8] * 4, [160] * 4, (1, 50), 16, 8),         # at most 16 blocks: one split, merged in the split kernel
    ([4] * 64, [64, 80, 128, 0] * 16, (0, 300), 16, 8),  # 2048 (sequence, kv head) pairs: one split each
]


@pytest.mark.parametrize("sizes,prompts,suf,H_q,H_kv", CASES)
def test_shared_prefix_parity(sizes, prompts, suf, H_q, H_kv):
    n = sum(sizes)
    suffix = np.random.default_rng(n + H_q).integers(suf[0], suf[1], n, endpoint=True)
    q, kc, vc, bt, sl, gs, pb = W.forked_decode_inputs(sizes, prompts, suffix, H_q, H_kv, seed=n)
    say("shared prefix", sizes, prompts, suf, H_q, H_kv)
    got = gpu_shared(q, kc, vc, bt, sl, gs, pb)
    assert_parity(got, oracle.decode_paged(q, kc, vc, bt, sl), "shared-prefix decode")
    assert_close_to_plain(got, gpu_decode(q, kc, vc, bt, sl))


@pytest.mark.parametrize("pad", [0, 40])
def test_preconditions_give_nan_or_zero_rows(pad):
    """A prefix longer than one of the group's sequences, a bad prefix table
    entry, and a zero-length sequence (prefix 0).  pad = 0: one split per
    sequence (the split kernel writes the rows); pad = 40 unused table
    columns: several splits and the merge kernel."""
    q, kc, vc, bt, sl, gs, pb = W.forked_decode_inputs([3, 3, 2], [64, 64, 32], [4, 9, 2, 1, 1, 1, 0, 5],
                                                       16, 8, seed=77)
    sl = sl.copy()
    bt = np.concatenate([bt, np.full((bt.shape[0], pad), -1, np.int32)], axis=1)
    pb = pb.copy()
    sl[1] = 40                  # group 0: sequence 1 shorter than the 4-block prefix
    bt[3:6, 1] = kc.shape[0] + 5  # group 1: an out-of-pool prefix entry (all its tables)
    pb[2] = 0                   # group 2: no shared prefix ...
    sl[6] = 0                   # ... and an empty sequence
    say("shared prefix preconditions")
    got = gpu_shared(q, kc, vc, bt, sl, gs, pb).astype(np.float64)
    assert np.isnan(got[1]).all()
    assert np.isnan(got[3:6]).all()
    assert np.array_equal(got[6], np.zeros_like(got[6]))
    ok = [0, 2, 7]
    ref = oracle.decode_paged(q[ok], kc, vc, bt[ok], sl[ok])
    assert_parity(got[ok].astype(np.float16), ref, "rows that keep the preconditions")


def test_grpo_workload_sampled():
    """The bench workload: 32 prompts of 2048 tokens, 8 samples each with
    U[1, 512] tokens of their own (256 sequences, H 16/8); 24 sampled
    sequences against the oracle, all 256 against plain GPU decode and
    against a second run of the same call."""
    q, kc, vc, bt, sl, gs, pb = W.grpo_decode_inputs()
    say("grpo shared-prefix workload")
    got = gpu_shared(q, kc, vc, bt, sl, gs, pb)
    # the same call again is bit-identical: no order or race depends on timing
    assert np.array_equal(got.view(np.uint16), gpu_shared(q, kc, vc, bt, sl, gs, pb).view(np.uint16))
    assert_close_to_plain(got, gpu_decode(q, kc, vc, bt, sl))
    pick = np.random.default_rng(5).choice(len(sl), 24, replace=False)
    assert_parity(got[pick], oracle.decode_paged(q, kc, vc, bt, sl, seqs=pick), "grpo sampled")
