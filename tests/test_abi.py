"""The C-ABI library on the CPU: it loads, exports every entry point that
include/attn.h declares, and rejects invalid arguments on the host, before
any HIP call (so these tests never touch a GPU)."""
import ctypes
import os
import re

import pytest

from attention_attn_prefill_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, INV, UNS, WS = (binding.ATTN_OK, binding.ATTN_ERR_INVALID_ARG,
                    binding.ATTN_ERR_UNSUPPORTED, binding.ATTN_ERR_WORKSPACE)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "attn_abi_version", "attn_status_string", "attn_prefill", "attn_prefill_qk_norm_rope",
        "attn_decode_paged_workspace_size", "attn_decode_paged", "attn_decode_paged_scratch",
        "attn_kv_append",
        "attn_rope_table", "attn_qk_norm_rope", "attn_qk_norm_rope_append",
        "attn_cross_attention_workspace_size", "attn_cross_attention",
        "attn_decode_paged_shared_prefix_workspace_size", "attn_decode_paged_shared_prefix"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_only_declared_symbols_are_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln})
    assert exported == declared_functions()


def test_status_strings(lib):
    assert binding.attn_abi_version() == 1
    names = [binding.attn_status_string(i) for i in range(5)]
    assert names == ["ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED",
                     "ATTN_ERR_WORKSPACE", "ATTN_ERR_LAUNCH"]
    assert binding.attn_status_string(99) == "ATTN_ERR_UNKNOWN"


# Fake, 16-byte aligned addresses: validation must fail before they are used.
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
NULL = ctypes.c_void_p(None)


def prefill(lib, q=P, k=P, v=P, o=P2, B=1, S_q=64, S_kv=64, H_q=2, H_kv=1, D=128, causal=1):
    return lib.attn_prefill(q, k, v, o, B, S_q, S_kv, H_q, H_kv, D, causal, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(q=NULL), INV), (dict(k=NULL), INV), (dict(v=NULL), INV), (dict(o=NULL), INV),
    (dict(B=0), INV), (dict(S_q=0, S_kv=0), INV), (dict(S_kv=-1, causal=0), INV),
    (dict(H_q=0), INV), (dict(H_kv=0), INV), (dict(H_q=3, H_kv=2), INV),
    (dict(S_q=64, S_kv=65, causal=1), INV),
    (dict(D=96), UNS), (dict(D=256), UNS), (dict(D=0), INV),
    (dict(S_q=1, S_kv=1 << 20, H_q=8, H_kv=8, causal=0), UNS),   # K of one batch entry >= 2 GiB
    # one key past the largest K/V that 32-bit offsets allow with the three
    # staged tiles past the end: (ceil(S_kv / 64) + 3) * 64 * H_kv * D * 2 >= 2^31
    # (the GPU parity test runs at the largest accepted S_kv)
    (dict(S_q=1, S_kv=8388352 + 1, H_q=2, H_kv=1, causal=0), UNS),
    (dict(S_q=1, S_kv=16776960 + 1, H_q=2, H_kv=1, D=64, causal=0), UNS),
    (dict(q=ctypes.c_void_p(0x10008)), INV), (dict(o=ctypes.c_void_p(0x20002)), INV),
])
def test_prefill_rejects(lib, kw, want):
    assert prefill(lib, **kw) == want


def decode(lib, q=P, kc=P, vc=P, out=P2, bt=P, sl=P, num_seqs=4, H_q=16, H_kv=8, D=128,
           max_bps=256, bs=16, num_blocks=100, ws=NULL, ws_bytes=0):
    return lib.attn_decode_paged(q, kc, vc, out, bt, sl, num_seqs, H_q, H_kv, D, max_bps, bs,
                                 num_blocks, ws, ws_bytes, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(q=NULL), INV), (dict(kc=NULL), INV), (dict(vc=NULL), INV), (dict(out=NULL), INV),
    (dict(bt=NULL), INV), (dict(sl=NULL), INV),
    (dict(num_seqs=0), INV), (dict(H_q=12, H_kv=8), INV), (dict(max_bps=0), INV),
    (dict(num_blocks=0), INV), (dict(D=64), UNS), (dict(bs=32), UNS),
    (dict(H_q=32, H_kv=2), UNS),
    (dict(bt=ctypes.c_void_p(0x10002)), INV), (dict(kc=ctypes.c_void_p(0x10004)), INV),
    (dict(ws=P, ws_bytes=1024), WS),
    (dict(ws=ctypes.c_void_p(0x10004), ws_bytes=1 << 30), INV),
])
def test_decode_rejects(lib, kw, want):
    assert decode(lib, **kw) == want


def decode_scratch(lib, q=P, kc=P, vc=P, out=P2, bt=P, sl=P, num_seqs=4, H_q=16, H_kv=8, D=128,
                   max_bps=256, bs=16, num_blocks=100):
    return lib.attn_decode_paged_scratch(q, kc, vc, out, bt, sl, num_seqs, H_q, H_kv, D, max_bps,
                                         bs, num_blocks, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(q=NULL), INV), (dict(out=NULL), INV), (dict(sl=NULL), INV), (dict(num_seqs=0), INV),
    (dict(H_q=12, H_kv=8), INV), (dict(num_blocks=0), INV), (dict(D=64), UNS), (dict(bs=32), UNS),
    (dict(bt=ctypes.c_void_p(0x10002)), INV),
    # partials beyond the library's 16 MiB array: 4096 sequences with
    # 256-block tables at H_q = 16 need 35 MB (a slot per (sequence, kv head)
    # and per run); 5000 sequences (fixed-length splits) need 83 MB
    (dict(num_seqs=4096, max_bps=256), WS), (dict(num_seqs=5000, max_bps=256), WS),
])
def test_decode_scratch_rejects(lib, kw, want):
    assert decode_scratch(lib, **kw) == want


def test_workspace_size(lib):
    # Split-K over a workspace runs as 1024 equal runs of the (sequence, kv
    # head, block) order: a partial slot per (sequence, kv head) and per run,
    # each with G = H_q / H_kv heads of 128 fp32 outputs + (max, sum), then
    # the block prefix (num_seqs + 1 int32)
    def balanced(num_seqs, H_q, H_kv):
        return ((num_seqs * H_kv + 1024) * (H_q // H_kv) * (128 + 2) + num_seqs + 1) * 4
    assert binding.attn_decode_paged_workspace_size(256, 16, 8, 128, 256, 16) == balanced(256, 16, 8)
    assert binding.attn_decode_paged_workspace_size(64, 16, 8, 128, 2048, 16) == balanced(64, 16, 8)
    assert binding.attn_decode_paged_workspace_size(4, 16, 8, 128, 2048, 16) == balanced(4, 16, 8)
    assert binding.attn_decode_paged_workspace_size(4096, 8, 1, 128, 256, 16) == balanced(4096, 8, 1)
    # past 4096 sequences (their prefix would not fit LDS), fixed-length
    # splits: 5000 x 8 pairs, 256-block tables, splits of 128 blocks (2 per
    # sequence), a slot per (sequence, query head, split)
    assert binding.attn_decode_paged_workspace_size(5000, 16, 8, 128, 256, 16) == \
        5000 * 16 * 2 * (128 + 2) * 4
    # the same when num_seqs * table blocks * H_kv reaches 2^31 (positions of
    # the order are 32-bit): 4096 x 8 pairs, 65536-block tables, 512 splits
    assert binding.attn_decode_paged_workspace_size(4096, 16, 8, 128, 65536, 16) == \
        4096 * 16 * 512 * (128 + 2) * 4
    # a table that fits one split: no workspace
    assert binding.attn_decode_paged_workspace_size(4, 16, 8, 128, 16, 16) == 0
    # invalid or unsupported shapes report 0
    assert binding.attn_decode_paged_workspace_size(4, 16, 8, 64, 256, 16) == 0
    assert binding.attn_decode_paged_workspace_size(0, 16, 8, 128, 256, 16) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        binding.load_library()


def append(lib, kn=P, vn=P, kc=P2, vc=P2, sm=P, n=16, H_kv=8, D=128, bs=16, nb=4):
    return lib.attn_kv_append(kn, vn, kc, vc, sm, n, H_kv, D, bs, nb, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(kn=NULL), INV), (dict(vn=NULL), INV), (dict(kc=NULL), INV), (dict(vc=NULL), INV),
    (dict(sm=NULL), INV), (dict(n=-1), INV), (dict(H_kv=0), INV), (dict(D=0), INV),
    (dict(bs=0), INV), (dict(nb=0), INV), (dict(D=36), UNS),
    (dict(kc=ctypes.c_void_p(0x20008)), INV), (dict(sm=ctypes.c_void_p(0x10004)), INV),
    (dict(n=0), OK),   # nothing to do: returns without touching the GPU
])
def test_kv_append_rejects(lib, kw, want):
    assert append(lib, **kw) == want


def rope_table(lib, c=P, s=P2, max_pos=64, D=128, theta=1e6):
    return lib.attn_rope_table(c, s, max_pos, D, theta, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(c=NULL), INV), (dict(s=NULL), INV), (dict(max_pos=0), INV), (dict(D=0), INV),
    (dict(D=7), INV), (dict(theta=0.0), INV), (dict(theta=-1.0), INV),
    (dict(c=ctypes.c_void_p(0x10004)), INV),
])
def test_rope_table_rejects(lib, kw, want):
    assert rope_table(lib, **kw) == want


def prefill_rope(lib, q=P, k=P, v=P, o=P2, qw=P, c=P, s=P2, pos=P, B=1, S_q=64, S_kv=64, H_q=2, H_kv=1,
                 D=128, max_pos=64, eps=1e-6, causal=1):
    return lib.attn_prefill_qk_norm_rope(q, k, v, o, qw, c, s, pos, B, S_q, S_kv, H_q, H_kv, D, max_pos, eps,
                                         causal, NULL)


@pytest.mark.parametrize("kw,want", [
    # the prefill's own checks come first
    (dict(q=NULL), INV), (dict(o=NULL), INV), (dict(B=0), INV), (dict(H_q=3, H_kv=2), INV),
    (dict(S_q=64, S_kv=65), INV), (dict(D=96), UNS), (dict(q=ctypes.c_void_p(0x10008)), INV),
    # then the rotation's
    (dict(c=NULL), INV), (dict(s=NULL), INV), (dict(pos=NULL, max_pos=0), INV), (dict(max_pos=0), INV),
    (dict(eps=-1e-6), INV), (dict(eps=float("nan")), INV),
    (dict(c=ctypes.c_void_p(0x10004)), INV), (dict(s=ctypes.c_void_p(0x20008)), INV),
    (dict(pos=ctypes.c_void_p(0x10002)), INV), (dict(qw=ctypes.c_void_p(0x10008)), INV),
    (dict(qw=NULL, c=NULL), INV),
])
def test_prefill_qk_norm_rope_rejects(lib, kw, want):
    assert prefill_rope(lib, **kw) == want


def qk_rope(lib, q=P, k=P2, qw=P, kw_=P2, c=P, s=P2, pos=P, n=16, H_q=16, H_kv=8, D=128,
            max_pos=64, eps=1e-6):
    return lib.attn_qk_norm_rope(q, k, qw, kw_, c, s, pos, n, H_q, H_kv, D, max_pos, eps, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(q=NULL), INV), (dict(k=NULL), INV), (dict(c=NULL), INV), (dict(s=NULL), INV),
    (dict(pos=NULL), INV), (dict(qw=NULL), INV), (dict(kw_=NULL), INV),
    (dict(n=-1), INV), (dict(H_q=0), INV), (dict(H_kv=0), INV), (dict(max_pos=0), INV),
    (dict(eps=-1e-6), INV), (dict(eps=float("nan")), INV), (dict(D=0), INV),
    (dict(D=96), UNS), (dict(D=256), UNS),
    (dict(q=ctypes.c_void_p(0x10008)), INV), (dict(pos=ctypes.c_void_p(0x10002)), INV),
    (dict(qw=ctypes.c_void_p(0x10008)), INV),
    (dict(n=0), OK), (dict(n=0, qw=NULL, kw_=NULL), OK), (dict(n=0, q=NULL, pos=NULL), OK),
    (dict(n=0, D=96), UNS), (dict(n=0, H_q=0), INV),
])
def test_qk_norm_rope_rejects(lib, kw, want):
    assert qk_rope(lib, **kw) == want


def qk_rope_append(lib, q=P, qw=P, kw_=P2, v=P, kc=P2, vc=P2, sm=P, bs=16, nb=4, n=16, D=128):
    return lib.attn_qk_norm_rope_append(q, P2, v, qw, kw_, P, P2, P, n, 16, 8, D, 64, 1e-6, kc, vc, sm,
                                        bs, nb, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(v=NULL), INV), (dict(kc=NULL), INV), (dict(vc=NULL), INV), (dict(sm=NULL), INV),
    (dict(bs=0), INV), (dict(nb=0), INV), (dict(D=64 + 8), UNS),
    (dict(sm=ctypes.c_void_p(0x10004)), INV), (dict(v=ctypes.c_void_p(0x10008)), INV),
    (dict(n=0), OK),
    # keys and values only (q NULL): q_weight must be NULL too
    (dict(q=NULL), INV), (dict(q=NULL, kw_=NULL), INV), (dict(q=NULL, qw=NULL, v=NULL), INV),
    (dict(q=NULL, qw=NULL, kw_=ctypes.c_void_p(0x20008)), INV), (dict(q=NULL, qw=NULL, n=0), OK),
])
def test_qk_norm_rope_append_rejects(lib, kw, want):
    assert qk_rope_append(lib, **kw) == want


def cross(lib, xq=P, xk=P, wq=P, wk=P, wv=P, wo=P, c=P, s=P2, max_pos=128, out=P2, B=4, T_q=64,
          T_k=128, dim=256, H=8, ws=ctypes.c_void_p(0x40000), wsb=1 << 20):
    return lib.attn_cross_attention(xq, xk, wq, wk, wv, wo, c, s, max_pos, out, B, T_q, T_k, dim, H, ws,
                                    wsb, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(xq=NULL), INV), (dict(wo=NULL), INV), (dict(c=NULL), INV), (dict(out=NULL), INV),
    (dict(B=0), INV), (dict(T_q=0), INV), (dict(T_k=-1), INV), (dict(dim=0), INV), (dict(H=0), INV),
    (dict(H=3), INV), (dict(H=16), UNS), (dict(H=1), UNS), (dict(dim=48, H=1), UNS), (dict(dim=80, H=1), UNS),
    (dict(max_pos=127), INV), (dict(xq=ctypes.c_void_p(0x10008)), INV),
    (dict(ws=NULL), WS), (dict(wsb=1000), WS), (dict(ws=ctypes.c_void_p(0x40010)), WS),
])
def test_cross_attention_rejects(lib, kw, want):
    assert cross(lib, **kw) == want


def test_cross_attention_workspace_size(lib):
    # q and the attention output 4*64*256*2 bytes each, k and v 4*128*256*2 each
    assert lib.attn_cross_attention_workspace_size(4, 64, 128, 256, 8) == 2 * 131072 + 2 * 262144
    assert lib.attn_cross_attention_workspace_size(1, 3, 5, 64, 2) == 2 * 512 + 2 * 768
    assert lib.attn_cross_attention_workspace_size(4, 64, 128, 256, 3) == 0
    assert lib.attn_cross_attention_workspace_size(4, 64, 128, 256, 16) == 0


def test_cross_attention_32bit_offset_limits(lib):
    f = lib.attn_cross_attention_workspace_size
    # dim 1024: the projections address whole 32-row tiles, so 2^20 - 32 rows
    # fit 32-bit byte offsets and 2^20 - 1 rows (rounded up to 2^20) do not
    assert f(1, (1 << 20) - 32, 64, 1024, 8) > 0
    assert f(1, (1 << 20) - 1, 64, 1024, 8) == 0
    # the attention step: whole 64-key tiles of one batch entry plus three,
    # (ceil(T_k / 64) + 3) * 64 * 1024 * 2 < 2^31, so T_k <= 16380 * 64
    assert f(1, 64, 16380 * 64, 1024, 8) > 0
    assert f(1, 64, 16380 * 64 + 1, 1024, 8) == 0


def shared(lib, q=P, kc=P, vc=P, out=P2, bt=P, sl=P, num_seqs=256, H_q=16, H_kv=8, D=128, mbs=160, bs=16,
           nb=9000, gs=P, pb=P, ng=32, mgs=8, ws=ctypes.c_void_p(0x40000), wsb=1 << 30):
    return lib.attn_decode_paged_shared_prefix(q, kc, vc, out, bt, sl, num_seqs, H_q, H_kv, D, mbs, bs, nb, gs,
                                               pb, ng, mgs, ws, wsb, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(q=NULL), INV), (dict(gs=NULL), INV), (dict(pb=NULL), INV), (dict(ng=0), INV),
    (dict(ng=257), INV), (dict(mgs=0), INV), (dict(mgs=257), INV), (dict(nb=0), INV),
    (dict(H_q=12), INV), (dict(D=64), UNS), (dict(bs=32), UNS), (dict(H_q=80, H_kv=8), UNS),
    (dict(gs=ctypes.c_void_p(0x10002)), INV),
    (dict(ws=NULL), WS), (dict(wsb=1000), WS),
])
def test_shared_prefix_rejects(lib, kw, want):
    assert shared(lib, **kw) == want


def test_shared_prefix_workspace_size(lib):
    # 256 seqs x 8 kv heads = 2048 pairs: one split per sequence, so
    # 256 x 16 heads x (prefix slots ceil(160/64) = 3 + 1 split) x 130 floats,
    # then one int32 prefix length per sequence
    n = lib.attn_decode_paged_shared_prefix_workspace_size(256, 16, 8, 128, 160, 16, 32, 8)
    assert n == 256 * 16 * (3 + 1) * 130 * 4 + 256 * 4
    # 64 x 8 = 512 pairs: the plain split rule (largest of 128/64/32/16 blocks
    # giving >= 2048 workgroups): 32 blocks, ceil(160/32) = 5 splits
    n = lib.attn_decode_paged_shared_prefix_workspace_size(64, 16, 8, 128, 160, 16, 8, 8)
    assert n == 64 * 16 * (3 + 5) * 130 * 4 + 64 * 4
    assert lib.attn_decode_paged_shared_prefix_workspace_size(256, 16, 8, 128, 160, 16, 0, 8) == 0
    assert lib.attn_decode_paged_shared_prefix_workspace_size(256, 16, 8, 64, 160, 16, 32, 8) == 0
