"""fp64 CPU oracle for softmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package imports
nothing from the product.

It wraps ``liboracle.so`` (``attn_oracle.c``): the plain definition of
scaled-dot-product attention, ``softmax(Q K^T / sqrt(D) + mask) V``, computed
in fp64 over the exact values of binary16 inputs.  Prefill follows the
attention.cuh / test_attention.cu listings of "Tutorial: Adding a New Kernel to
RL.cu" (layout [B,S,H,D], GQA kv head = h*H_kv//H_q, causal row i sees keys
0..i); paged decode follows the decode section of the same listing and the
"KV Cache design" section of the GRPO-CUDA project memory page; QK-norm and
the NeoX rotary embedding follow the "Qwen3" and "RoPE design" sections of the
same page.

Every function here is pinned by tests in ``tests/test_oracle_pins.py``
(closed forms, invariants, a library routine on special cases, brute force on
tiny inputs).  None is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

class Oracle:
    """ctypes front end of one build of ``attn_oracle.c``.

    The default instance loads ``liboracle.so``; the pin tests also load
    deliberately broken copies through this class to show that the pins fail.
    """

    def __init__(self, path: str | None = None):
        self._path = path
        self._lib = None

    def _load(self):
        if self._lib is not None:
            return self._lib
        path = self._path
        if path is None:
            sanitize = _build.sanitize_requested()
            path = _build.LIB_SAN if sanitize else _build.LIB
            src_mtime = os.path.getmtime(_build.SRC)
            if not os.path.exists(path) or os.path.getmtime(path) < src_mtime:
                _build.build(sanitize=sanitize)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        I64 = ctypes.c_int64
        lib.oracle_prefill.argtypes = [P, P, P, P, I, I, I, I, I, I, I, P, I64, P]
        lib.oracle_prefill.restype = I
        lib.oracle_decode_paged.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I64, P, I64, P]
        lib.oracle_decode_paged.restype = I
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = I
        lib.oracle_kv_append.argtypes = [P, P, P, P, P, I64, I, I, I, I64]
        lib.oracle_kv_append.restype = I64
        D_ = ctypes.c_double
        lib.oracle_rope_table.argtypes = [P, P, I, I, D_]
        lib.oracle_rope_table.restype = I
        lib.oracle_qk_norm_rope.argtypes = [P, P, P, P, P, I64, I, I, I, D_, P]
        lib.oracle_qk_norm_rope.restype = I
        lib.oracle_cross_attention.argtypes = [P, P, P, P, P, P, I, I, I, I, I, D_, P]
        lib.oracle_cross_attention.restype = I
        lib.oracle_rope_interleaved.argtypes = [P, I64, I64, I, I, D_, P]
        lib.oracle_rope_interleaved.restype = I
        self._lib = lib
        return lib

    def num_threads(self) -> int:
        """OpenMP threads the oracle uses (its ``cores`` figure)."""
        return self._load().oracle_num_threads()

    def half_to_double(self, bits: int) -> float:
        """The oracle's own binary16 decoder, exposed for its pin."""
        return self._load().oracle_half_to_double(int(bits) & 0xFFFF)

    def prefill(self, q, k, v, causal: bool, rows=None, return_lse: bool = False):
        """fp64 attention for Q [B,S_q,H_q,D], K/V [B,S_kv,H_kv,D] (float16).

        ``rows``: optional int64 flat row ids ``(b*S_q + i)*H_q + h``; the
        result is then ``[len(rows), D]``, else ``[B,S_q,H_q,D]``.  Returns
        float64 (and the natural-log LSE per row when ``return_lse``).
        """
        q, k, v = _f16(q), _f16(k), _f16(v)
        B, S_q, H_q, D = q.shape
        Bk, S_kv, H_kv, Dk = k.shape
        if v.shape != k.shape or Bk != B or Dk != D:
            raise ValueError("shape mismatch")
        if rows is not None:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            n_rows = rows.shape[0]
            out = np.empty((n_rows, D), np.float64)
            lse = np.empty(n_rows, np.float64) if return_lse else None
        else:
            n_rows = 0
            out = np.empty((B, S_q, H_q, D), np.float64)
            lse = np.empty((B, S_q, H_q), np.float64) if return_lse else None
        rc = self._load().oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S_q, S_kv,
                                         H_q, H_kv, D, int(bool(causal)), _ptr(rows), n_rows,
                                         _ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_prefill rejected its arguments (rc={rc})")
        return (out, lse) if return_lse else out

    def decode_paged(self, q, k_cache, v_cache, block_tables, seq_lens, seqs=None,
                     return_lse: bool = False):
        """fp64 single-token attention over a paged KV cache.

        q [num_seqs,H_q,D]; caches [num_blocks,H_kv,block_size,D] (float16);
        block_tables int32 [num_seqs,max_blocks_per_seq]; seq_lens int32
        [num_seqs].  ``seqs``: optional sequence ids; result
        ``[len(seqs),H_q,D]`` else ``[num_seqs,H_q,D]``.
        """
        q, k_cache, v_cache = _f16(q), _f16(k_cache), _f16(v_cache)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        num_seqs, H_q, D = q.shape
        num_blocks, H_kv, block_size, Dk = k_cache.shape
        if v_cache.shape != k_cache.shape or Dk != D:
            raise ValueError("shape mismatch")
        if bt.ndim != 2 or bt.shape[0] != num_seqs or sl.shape != (num_seqs,):
            raise ValueError("table shape mismatch")
        if seqs is not None:
            seqs = np.ascontiguousarray(seqs, dtype=np.int64)
            n = seqs.shape[0]
        else:
            n = num_seqs
        out = np.empty((n, H_q, D), np.float64)
        lse = np.empty((n, H_q), np.float64) if return_lse else None
        rc = self._load().oracle_decode_paged(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(sl), _ptr(out), num_seqs,
            H_q, H_kv, D, bt.shape[1], block_size, num_blocks, _ptr(seqs),
            n if seqs is not None else 0, _ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_decode_paged rejected its arguments (rc={rc})")
        return (out, lse) if return_lse else out


    def kv_append(self, k_new, v_new, k_cache, v_cache, slot_mapping):
        """Copy new K/V rows [num_tokens, H_kv, D] into the paged caches
        [num_blocks, H_kv, block_size, D] (modified in place) at
        slot_mapping (int64, block*block_size + offset; -1 skipped).
        Returns the number of tokens written."""
        k_new, v_new = _f16(k_new), _f16(v_new)
        if k_cache.dtype != np.float16 or v_cache.dtype != np.float16 or \
                not k_cache.flags.c_contiguous or not v_cache.flags.c_contiguous:
            raise TypeError("caches must be contiguous float16 arrays (updated in place)")
        sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        num_tokens, H_kv, D = k_new.shape
        num_blocks, H2, block_size, D2 = k_cache.shape
        if v_new.shape != k_new.shape or v_cache.shape != k_cache.shape or H2 != H_kv or D2 != D \
                or sm.shape != (num_tokens,):
            raise ValueError("shape mismatch")
        n = self._load().oracle_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(sm), num_tokens, H_kv, D, block_size, num_blocks)
        if n < 0:
            raise ValueError("oracle_kv_append rejected its arguments")
        return int(n)

    def rope_table(self, max_pos: int, D: int, theta: float):
        """fp64 (cos, sin) tables [max_pos, D/2] of the NeoX rotation:
        angle pos * theta^(-2i/D)."""
        cos = np.empty((max_pos, D // 2), np.float64)
        sin = np.empty((max_pos, D // 2), np.float64)
        rc = self._load().oracle_rope_table(_ptr(cos), _ptr(sin), int(max_pos), int(D), float(theta))
        if rc != 0:
            raise ValueError("oracle_rope_table rejected its arguments")
        return cos, sin

    def qk_norm_rope(self, x, weight, positions, cos, sin, eps: float = 1e-6):
        """Per-head RMSNorm (skipped when ``weight`` is None) then NeoX
        split-half rotation of x [n_tokens, H, D] (float16) at int32
        ``positions``, with fp64 tables [max_pos, D/2].  Returns float64
        [n_tokens, H, D]; rows of out-of-range positions are NaN."""
        x = _f16(x)
        n_tokens, H, D = x.shape
        w = None if weight is None else _f16(weight)
        if w is not None and w.shape != (D,):
            raise ValueError("weight must be [D]")
        pos = np.ascontiguousarray(positions, dtype=np.int32)
        cos = np.ascontiguousarray(cos, dtype=np.float64)
        sin = np.ascontiguousarray(sin, dtype=np.float64)
        if pos.shape != (n_tokens,) or cos.shape != sin.shape or cos.ndim != 2 or \
                cos.shape[1] != D // 2:
            raise ValueError("shape mismatch")
        out = np.empty((n_tokens, H, D), np.float64)
        rc = self._load().oracle_qk_norm_rope(_ptr(x), _ptr(w), _ptr(pos), _ptr(cos), _ptr(sin),
                                              n_tokens, H, D, cos.shape[0], float(eps), _ptr(out))
        if rc != 0:
            raise ValueError("oracle_qk_norm_rope rejected its arguments")
        return out

    def cross_attention(self, x_q, x_kv, w_q, w_k, w_v, w_o, H: int, base: float = 10000.0):
        """The cross-attention module with interleaved-pair RoPE: x_q
        [B,T_q,dim], x_kv [B,T_k,dim], weights [dim,dim] (nn.Linear [out,in]),
        all float16.  Returns float64 [B,T_q,dim]."""
        x_q, x_kv = _f16(x_q), _f16(x_kv)
        ws = [_f16(w) for w in (w_q, w_k, w_v, w_o)]
        B, T_q, dim = x_q.shape
        Bk, T_k, dimk = x_kv.shape
        if Bk != B or dimk != dim or any(w.shape != (dim, dim) for w in ws):
            raise ValueError("shape mismatch")
        out = np.empty((B, T_q, dim), np.float64)
        rc = self._load().oracle_cross_attention(_ptr(x_q), _ptr(x_kv), *[_ptr(w) for w in ws], B, T_q,
                                                 T_k, dim, int(H), float(base), _ptr(out))
        if rc != 0:
            raise ValueError("oracle_cross_attention rejected its arguments")
        return out


    def rope_interleaved(self, x, base: float = 10000.0):
        """Interleaved-pair rotary embedding of x [B, T, H, D] (float16): pair
        (2j, 2j+1) of row t turns by t * base^(-2j/D).  Returns float64."""
        x = _f16(x)
        B, T, H, D = x.shape
        out = np.empty((B, T, H, D), np.float64)
        rc = self._load().oracle_rope_interleaved(_ptr(x), B, T, H, D, float(base), _ptr(out))
        if rc != 0:
            raise ValueError("oracle_rope_interleaved rejected its arguments")
        return out


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.float16:
        raise TypeError("oracle inputs are binary16 (numpy float16) arrays")
    return a


default = Oracle()
num_threads = default.num_threads
half_to_double = default.half_to_double
prefill = default.prefill
decode_paged = default.decode_paged
kv_append = default.kv_append
rope_table = default.rope_table
qk_norm_rope = default.qk_norm_rope
cross_attention = default.cross_attention
rope_interleaved = default.rope_interleaved
