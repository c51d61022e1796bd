"""Thin ctypes binding of libattn.so (the C ABI in include/attn.h).

Argument marshalling only: tensor shapes become the integer arguments,
tensor storage becomes device pointers, the stream defaults to torch's current
stream.  Every step of the computation runs in the library's HIP kernels; this
module has no fallback and raises if the library cannot be loaded.
"""
from __future__ import annotations

import ctypes
import os

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_WORKSPACE = 3
ATTN_ERR_LAUNCH = 4

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {attn_status_string(status)} ({status})")


def load_library():
    """Load libattn.so (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    F, D_ = ctypes.c_float, ctypes.c_double
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = I
    lib.attn_status_string.argtypes = [I]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_prefill.argtypes = [P, P, P, P, I, I, I, I, I, I, I, P]
    lib.attn_prefill.restype = I
    lib.attn_prefill_qk_norm_rope.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.attn_prefill_qk_norm_rope.restype = I
    lib.attn_decode_paged_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.attn_decode_paged_workspace_size.restype = SZ
    lib.attn_decode_paged.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I64, P, SZ, P]
    lib.attn_decode_paged.restype = I
    lib.attn_decode_paged_scratch.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I64, P]
    lib.attn_decode_paged_scratch.restype = I
    lib.attn_kv_append.argtypes = [P, P, P, P, P, I64, I, I, I, I64, P]
    lib.attn_kv_append.restype = I
    lib.attn_rope_table.argtypes = [P, P, I, I, D_, P]
    lib.attn_rope_table.restype = I
    lib.attn_qk_norm_rope.argtypes = [P, P, P, P, P, P, P, I64, I, I, I, I, F, P]
    lib.attn_qk_norm_rope.restype = I
    lib.attn_qk_norm_rope_append.argtypes = [P, P, P, P, P, P, P, P, I64, I, I, I, I, F,
                                             P, P, P, I, I64, P]
    lib.attn_qk_norm_rope_append.restype = I
    lib.attn_cross_attention_workspace_size.argtypes = [I, I, I, I, I]
    lib.attn_cross_attention_workspace_size.restype = SZ
    lib.attn_cross_attention.argtypes = [P, P, P, P, P, P, P, P, I, P, I, I, I, I, I, P, SZ, P]
    lib.attn_cross_attention.restype = I
    lib.attn_decode_paged_shared_prefix_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
    lib.attn_decode_paged_shared_prefix_workspace_size.restype = SZ
    lib.attn_decode_paged_shared_prefix.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I64, P, P, I, I, P,
                                                    SZ, P]
    lib.attn_decode_paged_shared_prefix.restype = I
    _lib = lib
    return lib


def attn_abi_version() -> int:
    return load_library().attn_abi_version()


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_tensor(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device (cuda) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def attn_prefill(q, k, v, o, causal: bool = True, stream=None) -> None:
    """O = softmax(Q K^T / sqrt(D) + mask) V via ``attn_prefill``.

    q/o: [B, S_q, H_q, D] float16; k/v: [B, S_kv, H_kv, D] float16, all
    contiguous device tensors.  Enqueued on ``stream`` (default: current).
    """
    import torch
    B, S_q, H_q, D = q.shape
    S_kv, H_kv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, S_kv, H_kv, D) or tuple(v.shape) != tuple(k.shape) or \
            tuple(o.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, k, v, o")
    args = [_dev_tensor(x, torch.float16, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    st = load_library().attn_prefill(*args, B, S_q, S_kv, H_q, H_kv, D, int(bool(causal)),
                                     _stream_handle(stream, q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_prefill")


def attn_prefill_qk_norm_rope(q, k, v, o, q_weight, cos_table, sin_table, positions, eps: float = 1e-6,
                              causal: bool = True, stream=None) -> None:
    """Prefill with the query QK-norm + NeoX RoPE fused into the query load
    via ``attn_prefill_qk_norm_rope``: q [B,S_q,H_q,D] is read only, q_weight
    [D] fp16 or None, fp32 tables [max_pos, D/2], int32 positions [B*S_q]
    or None (row i of every sequence at position i); k must already be
    normalised and rotated."""
    import torch
    B, S_q, H_q, D = q.shape
    S_kv, H_kv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, S_kv, H_kv, D) or tuple(v.shape) != tuple(k.shape) or \
            tuple(o.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, k, v, o")
    if cos_table.dim() != 2 or cos_table.shape[1] != D // 2 or \
            tuple(sin_table.shape) != tuple(cos_table.shape) or \
            (positions is not None and positions.numel() != B * S_q):
        raise ValueError("tables must be [max_pos, head_dim/2] and positions [B*S_q] or None")
    if q_weight is not None and q_weight.numel() != D:
        raise ValueError("q_weight must have head_dim elements")
    args = [_dev_tensor(x, torch.float16, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    args += [ctypes.c_void_p(None) if q_weight is None else _dev_tensor(q_weight, torch.float16, "q_weight"),
             _dev_tensor(cos_table, torch.float32, "cos_table"), _dev_tensor(sin_table, torch.float32, "sin_table"),
             ctypes.c_void_p(None) if positions is None else _dev_tensor(positions, torch.int32, "positions")]
    st = load_library().attn_prefill_qk_norm_rope(*args, B, S_q, S_kv, H_q, H_kv, D, cos_table.shape[0],
                                                  float(eps), int(bool(causal)), _stream_handle(stream, q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_prefill_qk_norm_rope")


def attn_decode_paged_workspace_size(num_seqs: int, H_q: int, H_kv: int, head_dim: int,
                                     max_blocks_per_seq: int, block_size: int) -> int:
    return int(load_library().attn_decode_paged_workspace_size(
        num_seqs, H_q, H_kv, head_dim, max_blocks_per_seq, block_size))


def attn_decode_paged(q, k_cache, v_cache, out, block_tables, seq_lens, workspace=None,
                      stream=None) -> None:
    """Single-token attention over a paged cache via ``attn_decode_paged``.

    q/out [num_seqs, H_q, D] float16; caches [num_blocks, H_kv, block_size, D]
    float16; block_tables [num_seqs, max_blocks_per_seq] int32; seq_lens
    [num_seqs] int32; workspace: a uint8 device tensor of at least
    ``attn_decode_paged_workspace_size(...)`` bytes (split-K) or None
    (single pass).
    """
    import torch
    if workspace is None:
        ws, ws_bytes = ctypes.c_void_p(None), 0
    else:
        ws = _dev_tensor(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    st = load_library().attn_decode_paged(*_decode_args(q, k_cache, v_cache, out, block_tables, seq_lens),
                                          ws, ws_bytes, _stream_handle(stream, q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_paged")


def _decode_args(q, k_cache, v_cache, out, block_tables, seq_lens):
    import torch
    num_seqs, H_q, D = q.shape
    num_blocks, H_kv, block_size, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, caches, out")
    if block_tables.dim() != 2 or block_tables.shape[0] != num_seqs or \
            tuple(seq_lens.shape) != (num_seqs,):
        raise ValueError("block_tables / seq_lens shape mismatch")
    ptrs = [_dev_tensor(x, torch.float16, n) for x, n in
            ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out"))]
    ptrs.append(_dev_tensor(block_tables, torch.int32, "block_tables"))
    ptrs.append(_dev_tensor(seq_lens, torch.int32, "seq_lens"))
    return ptrs + [num_seqs, H_q, H_kv, D, block_tables.shape[1], block_size, num_blocks]


def attn_decode_paged_scratch(q, k_cache, v_cache, out, block_tables, seq_lens, stream=None) -> None:
    """Split-K paged decode via ``attn_decode_paged_scratch``: the arguments of
    ``attn_decode_paged`` without a workspace; the partials go to the
    library's own per-device array (ATTN_DECODE_SCRATCH_BYTES), so the call
    allocates nothing.  Calls that overlap on one device race on that array."""
    import torch
    args = _decode_args(q, k_cache, v_cache, out, block_tables, seq_lens)
    with torch.cuda.device(q.device):  # the library uses the current device's array
        st = load_library().attn_decode_paged_scratch(*args, _stream_handle(stream, q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_paged_scratch")


def attn_kv_append(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """Write new K/V rows into the paged caches via ``attn_kv_append``.

    k_new/v_new [num_tokens, H_kv, D] float16 (a [B, S, H_kv, D] prefill
    tensor is accepted and read as B*S tokens); caches
    [num_blocks, H_kv, block_size, D] float16, updated in place;
    slot_mapping [num_tokens] int64 (-1 = padding, skipped).
    """
    import torch
    H_kv, D = k_new.shape[-2], k_new.shape[-1]
    num_tokens = k_new.numel() // (H_kv * D)
    num_blocks, H2, block_size, D2 = k_cache.shape
    if tuple(v_new.shape) != tuple(k_new.shape) or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or H2 != H_kv or D2 != D or slot_mapping.numel() != num_tokens:
        raise ValueError("shape mismatch between new rows, caches and slot_mapping")
    ptrs = [_dev_tensor(x, torch.float16, n) for x, n in
            ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache"))]
    sm = _dev_tensor(slot_mapping, torch.int64, "slot_mapping")
    st = load_library().attn_kv_append(*ptrs, sm, num_tokens, H_kv, D, block_size, num_blocks,
                                       _stream_handle(stream, k_new.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_kv_append")


def attn_rope_table(cos_table, sin_table, theta: float, stream=None) -> None:
    """Fill fp32 device tables [max_pos, head_dim/2] with cos/sin of
    pos * theta^(-2i/head_dim) via ``attn_rope_table``."""
    import torch
    if cos_table.dim() != 2 or tuple(sin_table.shape) != tuple(cos_table.shape):
        raise ValueError("tables must both be [max_pos, head_dim/2]")
    c = _dev_tensor(cos_table, torch.float32, "cos_table")
    s = _dev_tensor(sin_table, torch.float32, "sin_table")
    max_pos, half = cos_table.shape
    st = load_library().attn_rope_table(c, s, max_pos, 2 * half, float(theta),
                                        _stream_handle(stream, cos_table.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_rope_table")


def _rope_args(q, k, q_weight, k_weight, cos_table, sin_table, positions):
    """Pointers and sizes of the QK-norm + RoPE entry points; q None is the
    K-only form (then q_weight must be None and H_q is passed as 1)."""
    import torch
    D, H_kv = k.shape[-1], k.shape[-2]
    if q is None:
        if q_weight is not None:
            raise ValueError("q_weight needs q")
        H_q, num_tokens = 1, k.numel() // (H_kv * D)
    else:
        H_q = q.shape[-2]
        num_tokens = q.numel() // (H_q * D)
        if q.shape[-1] != D or (q_weight is None) != (k_weight is None):
            raise ValueError("q/k head_dim differ, or only one of q_weight / k_weight is given")
    if k.numel() != num_tokens * H_kv * D or positions.numel() != num_tokens:
        raise ValueError("q, k and positions disagree on num_tokens / head_dim")
    if cos_table.dim() != 2 or cos_table.shape[1] != D // 2 or \
            tuple(sin_table.shape) != tuple(cos_table.shape):
        raise ValueError("tables must be [max_pos, head_dim/2]")
    for w in (q_weight, k_weight):
        if w is not None and w.numel() != D:
            raise ValueError("weights must have head_dim elements")
    none = ctypes.c_void_p(None)
    ptrs = [none if q is None else _dev_tensor(q, torch.float16, "q"), _dev_tensor(k, torch.float16, "k"),
            none if q_weight is None else _dev_tensor(q_weight, torch.float16, "q_weight"),
            none if k_weight is None else _dev_tensor(k_weight, torch.float16, "k_weight")]
    ptrs += [_dev_tensor(cos_table, torch.float32, "cos_table"),
             _dev_tensor(sin_table, torch.float32, "sin_table"),
             _dev_tensor(positions, torch.int32, "positions")]
    return ptrs, num_tokens, H_q, H_kv, D, cos_table.shape[0]


def attn_qk_norm_rope(q, k, q_weight, k_weight, cos_table, sin_table, positions, eps: float = 1e-6,
                      stream=None) -> None:
    """In place: per-head RMSNorm (weights [D] fp16, or both None) then the
    NeoX rotation of q [..., H_q, D] and k [..., H_kv, D] at int32 positions
    [num_tokens], via ``attn_qk_norm_rope``."""
    if q is None:
        raise ValueError("attn_qk_norm_rope needs q (the K-only form is attn_qk_norm_rope_append)")
    ptrs, n, H_q, H_kv, D, max_pos = _rope_args(q, k, q_weight, k_weight, cos_table, sin_table,
                                                positions)
    st = load_library().attn_qk_norm_rope(*ptrs, n, H_q, H_kv, D, max_pos, float(eps),
                                          _stream_handle(stream, q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_qk_norm_rope")


def attn_qk_norm_rope_append(q, k, v, q_weight, k_weight, cos_table, sin_table, positions,
                             k_cache, v_cache, slot_mapping, eps: float = 1e-6, stream=None) -> None:
    """attn_qk_norm_rope, and in the same pass the rotated k rows and the v
    rows [..., H_kv, D] go to the paged caches [num_blocks, H_kv, block_size, D]
    at int64 slot_mapping [num_tokens] (-1 skipped), via
    ``attn_qk_norm_rope_append``.  q = None (with q_weight None): keys and
    values only, for ``attn_prefill_qk_norm_rope``."""
    import torch
    ptrs, n, H_q, H_kv, D, max_pos = _rope_args(q, k, q_weight, k_weight, cos_table, sin_table,
                                                positions)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("v must have k's shape")
    num_blocks, H2, block_size, D2 = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or H2 != H_kv or D2 != D or \
            slot_mapping.numel() != n:
        raise ValueError("cache / slot_mapping shape mismatch")
    vp = _dev_tensor(v, torch.float16, "v")
    kc = _dev_tensor(k_cache, torch.float16, "k_cache")
    vc = _dev_tensor(v_cache, torch.float16, "v_cache")
    sm = _dev_tensor(slot_mapping, torch.int64, "slot_mapping")
    args = ptrs[:2] + [vp] + ptrs[2:]
    st = load_library().attn_qk_norm_rope_append(*args, n, H_q, H_kv, D, max_pos, float(eps), kc, vc,
                                                 sm, block_size, num_blocks,
                                                 _stream_handle(stream, k.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_qk_norm_rope_append")


def attn_cross_attention_workspace_size(B: int, T_q: int, T_k: int, dim: int, H: int) -> int:
    return int(load_library().attn_cross_attention_workspace_size(B, T_q, T_k, dim, H))


def attn_cross_attention(x_q, x_kv, w_q, w_k, w_v, w_o, cos_table, sin_table, out, H: int,
                         workspace, stream=None) -> None:
    """The cross-attention module with adjacent-pair RoPE via
    ``attn_cross_attention``: x_q [B,T_q,dim], x_kv [B,T_k,dim], weights
    [dim,dim] fp16 (nn.Linear [out,in]); fp32 tables [max_pos, dim/H/2];
    out [B,T_q,dim] fp16; workspace a uint8 device tensor of at least
    ``attn_cross_attention_workspace_size`` bytes."""
    import torch
    B, T_q, dim = x_q.shape
    B2, T_k, dim2 = x_kv.shape
    if B2 != B or dim2 != dim or tuple(out.shape) != tuple(x_q.shape) or \
            any(tuple(w.shape) != (dim, dim) for w in (w_q, w_k, w_v, w_o)):
        raise ValueError("shape mismatch")
    if cos_table.dim() != 2 or tuple(sin_table.shape) != tuple(cos_table.shape):
        raise ValueError("tables must be [max_pos, head_dim/2]")
    ptrs = [_dev_tensor(t, torch.float16, n) for t, n in ((x_q, "x_q"), (x_kv, "x_kv"), (w_q, "w_q"),
                                                          (w_k, "w_k"), (w_v, "w_v"), (w_o, "w_o"))]
    ptrs += [_dev_tensor(cos_table, torch.float32, "cos_table"),
             _dev_tensor(sin_table, torch.float32, "sin_table")]
    ws = _dev_tensor(workspace, torch.uint8, "workspace")
    st = load_library().attn_cross_attention(*ptrs, cos_table.shape[0], _dev_tensor(out, torch.float16, "out"),
                                             B, T_q, T_k, dim, int(H), ws, workspace.numel(),
                                             _stream_handle(stream, x_q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_cross_attention")


def attn_decode_paged_shared_prefix_workspace_size(num_seqs: int, H_q: int, H_kv: int, head_dim: int,
                                                   max_blocks_per_seq: int, block_size: int,
                                                   num_groups: int, max_group_size: int) -> int:
    return int(load_library().attn_decode_paged_shared_prefix_workspace_size(
        num_seqs, H_q, H_kv, head_dim, max_blocks_per_seq, block_size, num_groups, max_group_size))


def attn_decode_paged_shared_prefix(q, k_cache, v_cache, out, block_tables, seq_lens, group_start,
                                    prefix_blocks, max_group_size: int, workspace, stream=None) -> None:
    """Paged decode of forked sequences via ``attn_decode_paged_shared_prefix``:
    as ``attn_decode_paged``, with int32 ``group_start`` [num_groups + 1]
    (sequences group_start[i]..group_start[i+1]-1 form group i) and int32
    ``prefix_blocks`` [num_groups] (leading table entries every sequence of
    the group shares); workspace: a uint8 device tensor of at least
    ``attn_decode_paged_shared_prefix_workspace_size`` bytes."""
    import torch
    num_seqs, H_q, D = q.shape
    num_blocks, H_kv, block_size, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, caches, out")
    if block_tables.dim() != 2 or block_tables.shape[0] != num_seqs or \
            tuple(seq_lens.shape) != (num_seqs,):
        raise ValueError("block_tables / seq_lens shape mismatch")
    num_groups = prefix_blocks.numel()
    if group_start.numel() != num_groups + 1:
        raise ValueError("group_start must have num_groups + 1 entries")
    ptrs = [_dev_tensor(x, torch.float16, n) for x, n in
            ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out"))]
    ints = [_dev_tensor(x, torch.int32, n) for x, n in
            ((block_tables, "block_tables"), (seq_lens, "seq_lens"), (group_start, "group_start"),
             (prefix_blocks, "prefix_blocks"))]
    ws = _dev_tensor(workspace, torch.uint8, "workspace")
    st = load_library().attn_decode_paged_shared_prefix(
        *ptrs, ints[0], ints[1], num_seqs, H_q, H_kv, D, block_tables.shape[1], block_size, num_blocks,
        ints[2], ints[3], num_groups, int(max_group_size), ws, workspace.numel(),
        _stream_handle(stream, q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_paged_shared_prefix")
