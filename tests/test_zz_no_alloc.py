"""attn_decode_paged_scratch (split-K paged decode on the library's own
device array, no allocation) against attn_decode_paged given a workspace, and
against the fp64 oracle.

Two calls in a row, the second smaller (fewer sequences, narrower tables, a
different head grouping), so the second runs on an array that still holds the
first call's partials at other offsets.  The workspace handed to
attn_decode_paged is filled with NaN bytes first: a merge that read a partial
slot its split pass did not write would show as a non-finite output there.
"""
import numpy as np
import pytest

import oracle
from attention_attn_prefill_amd import AttnError, ATTN_ERR_WORKSPACE
from attention_attn_prefill_amd import workloads as W
from gpu_helpers import assert_parity, dev, host, say

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20  # ATTN_DECODE_SCRATCH_BYTES


def _problem(lens, H_q, H_kv, max_bps, seed, D=128):
    n = len(lens)
    q = W.normal_f16((n, H_q, D), (97, seed))
    T = max(lens)
    K = W.normal_f16((n, T, H_kv, D), (97, seed, 1))
    V = W.normal_f16((n, T, H_kv, D), (97, seed, 2))
    kc, vc, bt = W.paginate(K, V, lens, 16, max_bps, (97, seed, 3))
    return q, kc, vc, bt, np.array(lens, np.int32)


def _ws_size(q, kc, bt):
    from attention_attn_prefill_amd import attn_decode_paged_workspace_size
    return attn_decode_paged_workspace_size(q.shape[0], q.shape[1], kc.shape[1], q.shape[2],
                                            bt.shape[1], kc.shape[2])


def _run_both(prob, stream=None):
    """(scratch output, workspace output) of one problem, both on the GPU."""
    import torch
    from attention_attn_prefill_amd import attn_decode_paged, attn_decode_paged_scratch
    q, kc, vc, bt, sl = prob
    tq, tk, tv, tbt, tsl = dev(q), dev(kc), dev(vc), dev(bt), dev(sl)
    out_scratch = torch.empty_like(tq)
    out_ws = torch.empty_like(tq)
    n = _ws_size(q, kc, bt)
    ws = torch.full((max(n, 16),), 0xFF, dtype=torch.uint8, device="cuda")  # NaN floats
    attn_decode_paged_scratch(tq, tk, tv, out_scratch, tbt, tsl, stream=stream)
    attn_decode_paged(tq, tk, tv, out_ws, tbt, tsl, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    return host(out_scratch), host(out_ws)


def test_two_calls_in_a_row_second_smaller():
    import torch
    lens1 = [1, 16, 17, 129, 700, 1024, 1500, 2049, 3000, 4096] * 4 + [33, 4000, 2500, 16, 15, 4095, 511, 512]
    p1 = _problem(lens1, 16, 8, 256, 1)
    p2 = _problem([1, 40, 300, 1599, 1600, 77], 8, 1, 100, 2)
    for p in (p1, p2):
        n = _ws_size(p[0], p[1], p[3])
        assert 0 < n <= SCRATCH_BYTES  # both leave partials in the array
    # the second call's input is the smaller one (fewer sequences and tokens)
    assert p2[0].shape[0] < p1[0].shape[0] and int(p2[4].sum()) < int(p1[4].sum())

    say("no-alloc decode call 1", p1[0].shape, p1[3].shape)
    s1, w1 = _run_both(p1)
    side = torch.cuda.Stream()  # a stream of the current device
    say("no-alloc decode call 2 (smaller, side stream)", p2[0].shape, p2[3].shape)
    with torch.cuda.stream(side):
        s2, w2 = _run_both(p2, stream=side)

    for (s, w, p, what) in ((s1, w1, p1, "call 1"), (s2, w2, p2, "call 2")):
        ref = oracle.decode_paged(*p)
        assert_parity(w, ref, f"workspace {what}")
        assert_parity(s, ref, f"scratch {what}")
        # same kernels, same split plan: the same bits
        assert np.array_equal(s.view(np.uint16), w.view(np.uint16)), what


def test_single_split_shape_and_repeat():
    """A shape that needs no partials (one split) and a repeat of a split-K
    shape after it: both equal the workspace entry point bit for bit."""
    p_small = _problem([5, 64], 16, 8, 4, 3)
    assert _ws_size(p_small[0], p_small[1], p_small[3]) == 0
    p_split = _problem([1, 40, 300, 1599, 1600, 77], 8, 2, 100, 4)
    for p, what in ((p_small, "single split"), (p_split, "split-K"), (p_split, "split-K again")):
        say("no-alloc decode", what)
        s, w = _run_both(p)
        assert_parity(s, oracle.decode_paged(*p), what)
        assert np.array_equal(s.view(np.uint16), w.view(np.uint16)), what


def test_request_beyond_the_array_is_rejected():
    """4096 sequences with 256-block tables at H_q = 16 need 35 MB of partials
    (a slot per (sequence, kv head) and per run, 2 heads of 130 floats each):
    rejected on the host before anything is enqueued."""
    import torch
    from attention_attn_prefill_amd import attn_decode_paged_scratch
    num_seqs, H_q, H_kv, D, max_bps = 4096, 16, 8, 128, 256
    q = torch.zeros((num_seqs, H_q, D), dtype=torch.float16, device="cuda")
    kc = torch.zeros((1, H_kv, 16, D), dtype=torch.float16, device="cuda")
    bt = torch.zeros((num_seqs, max_bps), dtype=torch.int32, device="cuda")
    sl = torch.ones((num_seqs,), dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    from attention_attn_prefill_amd import attn_decode_paged_workspace_size
    assert attn_decode_paged_workspace_size(num_seqs, H_q, H_kv, D, max_bps, 16) > SCRATCH_BYTES
    with pytest.raises(AttnError) as e:
        attn_decode_paged_scratch(q, kc, kc, out, bt, sl)
    assert e.value.status == ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing ran
