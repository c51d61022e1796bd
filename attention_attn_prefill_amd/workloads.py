"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path and the fp64 oracle consume the same
binary16 arrays that it returns.

Recipe:
  * tensors: standard normal draws (NumPy ``Generator(PCG64)``, float32
    ziggurat), rounded to binary16 (round-to-nearest-even).  Each tensor has a
    ``SeedSequence([config_id, tensor_id, seed])``; large tensors are filled in
    fixed 4 Mi-element chunks, chunk c using child c of that sequence, so the
    values do not depend on the thread count.
  * paged decode: ``seq_lens`` inclusive-uniform integers (or a fixed length);
    ``num_blocks = sum(ceil(L/16))``; physical ids are a seeded permutation of
    ``0..num_blocks-1`` handed out in (sequence, logical block) order; unused
    table entries are -1.
  * the cross-attention attention core (cross_attn): normal Q/K/V from
    here; the tests rotate Q and K by adjacent-pair RoPE (base 10000,
    positions 0..T-1) with the oracle's fp64 rotation and round them to
    binary16, so both sides consume the same rotated inputs (this module
    holds no arithmetic).  The full cross-attention module draws x_q, x_kv
    and nn.Linear-style uniform weights from ``cross_module_inputs``.
  * the pages' own unit-test shapes ("Tutorial: Adding a New Kernel to
    RL.cu", test_attention.cu: the case list and the value range
    [-0.5, 0.5)) get uniform inputs from ``pages_prefill_case`` /
    ``pages_decode_case`` (this module's PCG64 draws, not the pages' own
    generator).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_CHUNK = 1 << 22


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    config_id: int
    B: int
    S_q: int
    S_kv: int
    H_q: int
    H_kv: int
    D: int
    causal: bool

    @property
    def pairs(self) -> int:
        """Unmasked (query, key) pairs: the work unit of the FLOP count."""
        if self.causal:
            return self.B * self.H_q * self.S_q * (self.S_q + 1) // 2
        return self.B * self.H_q * self.S_q * self.S_kv

    @property
    def flops(self) -> int:
        """Algorithmic flops: 2*D for Q.K plus 2*D for P.V per unmasked pair."""
        return 4 * self.D * self.pairs

    @property
    def dense_flops(self) -> int:
        """The pages' benchmark convention: 4*B*H_q*S_q*S_kv*D, mask ignored."""
        return 4 * self.B * self.H_q * self.S_q * self.S_kv * self.D


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    config_id: int
    num_seqs: int
    H_q: int
    H_kv: int
    D: int
    block_size: int
    max_blocks_per_seq: int
    len_lo: int
    len_hi: int
    extra: dict = field(default_factory=dict, compare=False)


CONFIGS = {
    "tiny_causal": PrefillConfig("tiny_causal", 1, 1, 64, 64, 2, 1, 128, True),
    "cross_attn": PrefillConfig("cross_attn", 2, 4, 64, 128, 8, 8, 32, False),
    "qwen3_prefill": PrefillConfig("qwen3_prefill", 3, 4, 2048, 2048, 16, 8, 128, True),
    "paged_decode": DecodeConfig("paged_decode", 4, 256, 16, 8, 128, 16, 256, 128, 4096),
    "long_prefill": PrefillConfig("long_prefill", 5, 1, 32768, 32768, 16, 8, 128, True),
    "long_decode": DecodeConfig("long_decode", 6, 64, 16, 8, 128, 16, 2048, 32768, 32768),
}


def normal_f16(shape, seed_words, threads: int = 16) -> np.ndarray:
    """Standard-normal binary16 array, deterministic in ``seed_words``."""
    n = int(np.prod(shape))
    out16 = np.empty(n, np.float16)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    children = np.random.SeedSequence(list(seed_words)).spawn(nchunks)

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(children[c]))
        out16[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(min(threads, nchunks)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out16.reshape(shape)


def prefill_inputs(cfg: PrefillConfig | str, seed: int = 0):
    """(q, k, v) binary16 arrays for a prefill workload."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    q = normal_f16((cfg.B, cfg.S_q, cfg.H_q, cfg.D), (cfg.config_id, 0, seed))
    k = normal_f16((cfg.B, cfg.S_kv, cfg.H_kv, cfg.D), (cfg.config_id, 1, seed))
    v = normal_f16((cfg.B, cfg.S_kv, cfg.H_kv, cfg.D), (cfg.config_id, 2, seed))
    return q, k, v


def cross_module_inputs(B: int, T_q: int, T_k: int, dim: int, seed: int = 0):
    """Inputs of the cross-attention module: x_q [B,T_q,dim] and x_kv
    [B,T_k,dim] standard normal, and four [dim,dim] weights drawn like
    nn.Linear's default initialisation, uniform in +-1/sqrt(dim), all
    binary16."""
    xq = normal_f16((B, T_q, dim), (7, 0, seed))
    xk = normal_f16((B, T_k, dim), (7, 1, seed))
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([7, 2, seed])))
    bound = 1.0 / np.sqrt(dim)
    ws = [g.uniform(-bound, bound, (dim, dim)).astype(np.float16) for _ in range(4)]
    return xq, xk, ws


def forked_decode_inputs(group_sizes, prompt_lens, suffix_lens, H_q: int, H_kv: int, D: int = 128,
                         block_size: int = 16, seed: int = 0):
    """Paged decode inputs of forked sequences (a GRPO group samples several
    completions of one prompt).  Group i has ``group_sizes[i]`` sequences
    that share a prompt of ``prompt_lens[i]`` tokens; sequence j of the
    flattened order then has ``suffix_lens[j]`` tokens of its own.

    The prompt's whole blocks are one physical copy that every table of the
    group points to (a fork copies table entries, not K/V); a partial last
    prompt block is copied into each sequence's own blocks (same prompt
    K/V).  Physical block ids are a seeded permutation.  Returns
    (q, k_cache, v_cache, block_tables, seq_lens, group_start, prefix_blocks).
    """
    group_sizes = [int(x) for x in group_sizes]
    n = sum(group_sizes)
    suffix_lens = [int(x) for x in suffix_lens]
    assert len(suffix_lens) == n and len(prompt_lens) == len(group_sizes)
    bs = block_size
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([8, seed])))
    seq_lens = []
    blocks_needed = 0
    for gi, G in enumerate(group_sizes):
        P = int(prompt_lens[gi])
        blocks_needed += P // bs
        for j in range(G):
            L = P + suffix_lens[len(seq_lens)]
            seq_lens.append(L)
            blocks_needed += (L + bs - 1) // bs - P // bs
    max_bps = max((L + bs - 1) // bs for L in seq_lens)
    perm = rng.permutation(blocks_needed).astype(np.int32)
    k_cache = normal_f16((blocks_needed, H_kv, bs, D), (8, 1, seed))
    v_cache = normal_f16((blocks_needed, H_kv, bs, D), (8, 2, seed))
    bt = np.full((n, max_bps), -1, np.int32)
    group_start = [0]
    prefix_blocks = []
    nxt = 0
    s = 0
    for gi, G in enumerate(group_sizes):
        P = int(prompt_lens[gi])
        shared = perm[nxt:nxt + P // bs]
        nxt += P // bs
        prefix_blocks.append(P // bs)
        # K/V of the partial prompt block, copied into every sequence's own block
        part_src = None
        for j in range(G):
            L = seq_lens[s]
            own = (L + bs - 1) // bs - P // bs
            ids = perm[nxt:nxt + own]
            nxt += own
            bt[s, :P // bs] = shared
            bt[s, P // bs:P // bs + own] = ids
            if P % bs and own > 0:
                if part_src is None:
                    part_src = int(ids[0])
                else:
                    k_cache[ids[0], :, :P % bs] = k_cache[part_src, :, :P % bs]
                    v_cache[ids[0], :, :P % bs] = v_cache[part_src, :, :P % bs]
            s += 1
        group_start.append(s)
    q = normal_f16((n, H_q, D), (8, 3, seed))
    return (q, k_cache, v_cache, bt, np.array(seq_lens, np.int32), np.array(group_start, np.int32),
            np.array(prefix_blocks, np.int32))


GRPO_DECODE = dict(num_groups=32, group_size=8, prompt=2048, suffix_lo=1, suffix_hi=512, H_q=16, H_kv=8)


def grpo_decode_inputs(seed: int = 0):
    """The forked-decode workload: 32 prompts of 2048 tokens, 8 samples each
    with U[1, 512] generated tokens of their own (256 sequences, H_q 16,
    H_kv 8, D 128, 16-token blocks)."""
    c = GRPO_DECODE
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([9, seed])))
    n = c["num_groups"] * c["group_size"]
    suffix = rng.integers(c["suffix_lo"], c["suffix_hi"], n, endpoint=True)
    return forked_decode_inputs([c["group_size"]] * c["num_groups"], [c["prompt"]] * c["num_groups"], suffix,
                                c["H_q"], c["H_kv"], seed=seed)


def paged_layout(seq_lens, block_size: int, max_blocks_per_seq: int, seed_words):
    """Block tables for ``seq_lens``: a seeded permutation of the physical
    blocks, assigned in (sequence, logical block) order; unused entries -1."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    nb = (np.maximum(seq_lens, 0) + block_size - 1) // block_size
    if nb.max(initial=0) > max_blocks_per_seq:
        raise ValueError("a sequence needs more blocks than the table holds")
    num_blocks = int(nb.sum())
    perm = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_words)))) \
        .permutation(max(num_blocks, 1)).astype(np.int32)
    bt = np.full((len(seq_lens), max_blocks_per_seq), -1, np.int32)
    pos = 0
    for s, n in enumerate(nb):
        bt[s, :n] = perm[pos:pos + n]
        pos += n
    return bt, max(num_blocks, 1)


def decode_inputs(cfg: DecodeConfig | str, seed: int = 0):
    """(q, k_cache, v_cache, block_tables, seq_lens) for a paged-decode workload."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.config_id, 3, seed])))
    seq_lens = g.integers(cfg.len_lo, cfg.len_hi, size=cfg.num_seqs, endpoint=True).astype(np.int32)
    bt, num_blocks = paged_layout(seq_lens, cfg.block_size, cfg.max_blocks_per_seq,
                                  (cfg.config_id, 4, seed))
    q = normal_f16((cfg.num_seqs, cfg.H_q, cfg.D), (cfg.config_id, 0, seed))
    shape = (num_blocks, cfg.H_kv, cfg.block_size, cfg.D)
    k_cache = normal_f16(shape, (cfg.config_id, 1, seed))
    v_cache = normal_f16(shape, (cfg.config_id, 2, seed))
    return q, k_cache, v_cache, bt, seq_lens


def kv_bytes(seq_lens, H_kv: int, D: int) -> int:
    """Algorithmic decode traffic: K and V bytes of every visible token."""
    return int(np.maximum(np.asarray(seq_lens, np.int64), 0).sum()) * H_kv * D * 2 * 2


# ---- inputs for the pages' own unit-test shapes ----------------------------

def uniform_f16(shape, seed_words, lo: float = -0.5, hi: float = 0.5) -> np.ndarray:
    """Uniform [lo, hi) binary16 array (PCG64, deterministic in seed_words)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_words))))
    return g.uniform(lo, hi, int(np.prod(shape))).astype(np.float16).reshape(shape)


def pages_prefill_case(case: int, B: int, S: int, H_q: int, H_kv: int, D: int = 128):
    """Q, K, V at one of the pages' prefill unit-test shapes, with values
    uniform in [-0.5, 0.5) like the pages' cases (drawn from this module's
    own PCG64 generator, seeded by the case number)."""
    q = uniform_f16((B, S, H_q, D), (10, case, 0))
    k = uniform_f16((B, S, H_kv, D), (10, case, 1))
    v = uniform_f16((B, S, H_kv, D), (10, case, 2))
    return q, k, v


def pages_decode_case(case: int, num_seqs: int, ctx: int, H_q: int, H_kv: int,
                      D: int = 128, block_size: int = 16):
    """One of the pages' decode unit-test shapes: q and a contiguous
    [num_seqs, ctx, H_kv, D] context uniform in [-0.5, 0.5), paged with the
    identity table (sequence s, logical block b -> physical s*blocks_per_seq
    + b), as the pages' decode test lays it out."""
    q = uniform_f16((num_seqs, H_q, D), (11, case, 0))
    k = uniform_f16((num_seqs, ctx, H_kv, D), (11, case, 1))
    v = uniform_f16((num_seqs, ctx, H_kv, D), (11, case, 2))
    bps = (ctx + block_size - 1) // block_size
    k_cache = np.zeros((num_seqs * bps, H_kv, block_size, D), np.float16)
    v_cache = np.zeros_like(k_cache)
    for s in range(num_seqs):
        for t in range(ctx):
            pb = s * bps + t // block_size
            k_cache[pb, :, t % block_size, :] = k[s, t]
            v_cache[pb, :, t % block_size, :] = v[s, t]
    bt = (np.arange(num_seqs)[:, None] * bps + np.arange(bps)[None, :]).astype(np.int32)
    seq_lens = np.full(num_seqs, ctx, np.int32)
    return q, k_cache, v_cache, bt, seq_lens, k, v


def paginate(k: np.ndarray, v: np.ndarray, seq_lens, block_size: int, max_blocks_per_seq: int,
             seed_words=(0, 0)):
    """Scatter contiguous per-sequence K/V [num_seqs, T, H_kv, D] into a paged
    cache with a seeded random block permutation.  Returns
    (k_cache, v_cache, block_tables)."""
    num_seqs, T, H_kv, D = k.shape
    bt, num_blocks = paged_layout(seq_lens, block_size, max_blocks_per_seq, seed_words)
    k_cache = np.zeros((num_blocks, H_kv, block_size, D), np.float16)
    v_cache = np.zeros_like(k_cache)
    for s in range(num_seqs):
        L = int(seq_lens[s])
        for lb in range((L + block_size - 1) // block_size):
            t0, t1 = lb * block_size, min(L, (lb + 1) * block_size)
            pb = bt[s, lb]
            k_cache[pb, :, : t1 - t0, :] = k[s, t0:t1].transpose(1, 0, 2)
            v_cache[pb, :, : t1 - t0, :] = v[s, t0:t1].transpose(1, 0, 2)
    return k_cache, v_cache, bt


def sample_prefill_rows(cfg: PrefillConfig, n_random: int, seed: int = 0, tile: int = 128):
    """Stratified row sample for prefill parity at full size: every (b, h) at
    the first and last rows, rows at tile boundaries, and random rows."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.config_id, 7, seed])))
    S = cfg.S_q
    pos = set(range(min(4, S))) | set(range(max(0, S - 4), S))
    for t in range(tile, S, tile):
        pos |= {t - 1, t}
    pos = np.array(sorted(pos), np.int64)
    rows = []
    for b in range(cfg.B):
        for h in range(cfg.H_q):
            rows.append((b * S + pos) * cfg.H_q + h)
    rows.append(rng.integers(0, cfg.B * S * cfg.H_q, size=n_random))
    return np.unique(np.concatenate(rows)).astype(np.int64)


def expected_pairs_decode(seq_lens) -> int:
    return int(np.maximum(np.asarray(seq_lens, np.int64), 0).sum())


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = [
    "PrefillConfig", "DecodeConfig", "CONFIGS", "normal_f16", "cross_module_inputs", "forked_decode_inputs", "grpo_decode_inputs", "GRPO_DECODE",
    "prefill_inputs", "decode_inputs", "paged_layout", "kv_bytes", "uniform_f16",
    "pages_prefill_case", "pages_decode_case", "paginate", "sample_prefill_rows",
    "expected_pairs_decode", "ceil_div",
]
