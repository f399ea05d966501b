"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host (no GPU needed: every call here fails validation before
anything is enqueued)."""

import ctypes
import os
import re
import subprocess

import pytest

from llama_decoder_block_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llama_block.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="library not built (run python -m llama_decoder_block_amd.build)")

FAKE = 0x10000  # 16-byte aligned, never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(llama_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("llama_rmsnorm", "llama_rope", "llama_gqa_attention", "llama_swiglu_ffn",
              "llama_block_forward"):
        assert n in names


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = binding.lib()
    for n in names:
        assert hasattr(L, n)
    assert set(binding.FUNCTIONS) == set(names)


def test_version_and_status_strings():
    L = binding.lib()
    assert L.llama_version() == 10100
    assert L.llama_status_string(0) == b"ok"
    assert L.llama_status_string(-3) == b"workspace too small"
    assert L.llama_status_string(7) == b"unknown status"


def status_and_msg(rc):
    return rc, binding.lib().llama_last_error().decode()


def test_rmsnorm_validation():
    L = binding.lib()
    rc, msg = status_and_msg(L.llama_rmsnorm(FAKE, None, FAKE, FAKE, None, 4, 0, 1e-5, 1, 0, None))
    assert rc == -1 and "d_model" in msg
    rc, _ = status_and_msg(L.llama_rmsnorm(FAKE, None, FAKE, FAKE, None, 4, 16, 1e-5, 3, 0, None))
    assert rc == -2
    rc, _ = status_and_msg(L.llama_rmsnorm(FAKE, None, None, FAKE + 64, None, 4, 16, 1e-5, 1, 0, None))
    assert rc == -1
    rc, msg = status_and_msg(L.llama_rmsnorm(FAKE, None, FAKE, FAKE, None, 4, 16, 1e-5, 1, 0, None))
    assert rc == -1 and "alias" in msg
    rc, msg = status_and_msg(L.llama_rmsnorm(FAKE + 2, None, FAKE, FAKE + 64, None, 4, 16, 1e-5, 1, 0, None))
    assert rc == -2 and "aligned" in msg
    rc, _ = status_and_msg(L.llama_rmsnorm(FAKE, None, FAKE, FAKE + 64, None, 4, 16, -1.0, 1, 0, None))
    assert rc == -1


def test_rope_validation():
    L = binding.lib()
    assert L.llama_rope(FAKE, FAKE, FAKE, 4, 8, 2, 3, 1e4, 1, None) == -1        # odd head_dim
    assert L.llama_rope(FAKE, FAKE, FAKE, 4, 8, 2, 512, 1e4, 1, None) == -2      # > 256
    assert L.llama_rope(FAKE, FAKE, None, 4, 8, 2, 128, 1e4, 1, None) == -1      # no positions
    assert L.llama_rope(FAKE, FAKE, FAKE, 4, 8, 2, 128, 0.0, 1, None) == -1      # theta
    assert L.llama_rope(None, None, FAKE, 4, 8, 2, 128, 1e4, 1, None) == -1      # nothing to do


def attn(L, **kw):
    a = dict(q=FAKE, k=FAKE + 0x100, v=FAKE + 0x200, out=FAKE + 0x300, positions=FAKE + 0x400, batch=2,
             q_len=1, kv_len=100, nq=8, nkv=2, hd=128, dt=1, ws=FAKE + 0x500, ws_bytes=1 << 30)
    a.update(kw)
    return L.llama_gqa_attention(a["q"], a["k"], a["v"], a["out"], a["positions"], a["batch"], a["q_len"],
                                 a["kv_len"], a["nq"], a["nkv"], a["hd"], a["dt"], a["ws"], a["ws_bytes"],
                                 None)


def test_attention_validation():
    L = binding.lib()
    assert attn(L, nkv=3) == -1                       # n_q % n_kv != 0
    assert attn(L, hd=127) == -1                      # odd head_dim
    assert attn(L, hd=258) == -2                      # head_dim > 256
    assert attn(L, dt=5) == -2                        # dtype code
    assert attn(L, out=FAKE) == -1                    # out aliases q
    assert attn(L, q=None) == -1
    assert attn(L, positions=None, q_len=200, kv_len=100) == -1
    need = L.llama_gqa_attention_workspace_bytes(2, 1, 100, 8, 2, 128, 1)
    assert need > 0
    assert attn(L, ws_bytes=need - 1) == -3
    assert attn(L, ws=None, ws_bytes=0) == -3
    assert "workspace" in L.llama_last_error().decode()


def test_ffn_validation():
    L = binding.lib()
    need = L.llama_swiglu_ffn_workspace_bytes(64, 4096, 14336, 1, 0)
    assert need >= 64 * 14336 * 2
    rc = L.llama_swiglu_ffn(FAKE, FAKE, FAKE, FAKE, None, FAKE + 0x100, 64, 4096, 14336, 1, 0, FAKE, need - 1,
                            None)
    assert rc == -3
    rc = L.llama_swiglu_ffn(FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 4096, 14336, 1, 0, FAKE, need, None)
    assert rc == -1  # out aliases x
    rc = L.llama_swiglu_ffn(FAKE, FAKE, FAKE, FAKE, None, FAKE + 0x100, 64, 4096, 0, 1, 0, FAKE, need, None)
    assert rc == -1


def block(L, **kw):
    w = binding.BlockWeights(*([FAKE + 0x1000 * i for i in range(1, 10)]))
    a = dict(x=FAKE, y=FAKE + 0x100, w=ctypes.byref(w), pos=FAKE + 0x200, kc=None, vc=None, cap=0, B=1, T=16,
             d=256, nq=4, nkv=2, hd=64, dff=512, theta=1e4, eps=1e-5, wdt=1, rdt=0, ws=FAKE + 0x300,
             ws_bytes=1 << 40)
    a.update(kw)
    return L.llama_block_forward(a["x"], a["y"], a["w"], a["pos"], a["kc"], a["vc"], a["cap"], a["B"], a["T"],
                                 a["d"], a["nq"], a["nkv"], a["hd"], a["dff"], a["theta"], a["eps"], a["wdt"],
                                 a["rdt"], a["ws"], a["ws_bytes"], None)


def test_block_validation():
    L = binding.lib()
    assert block(L, nkv=3) == -1
    assert block(L, kc=FAKE + 0x400, cap=0) == -1           # cache without capacity
    assert block(L, cap=64) == -1                           # capacity without cache
    assert block(L, y=FAKE) == -1                           # y aliases x
    assert block(L, pos=None) == -1
    assert block(L, w=None) == -1
    assert block(L, theta=-1.0) == -1
    assert block(L, hd=300) == -2
    w = binding.BlockWeights(*([FAKE] * 8 + [None]))
    assert block(L, w=ctypes.byref(w)) == -1
    need = L.llama_block_forward_workspace_bytes(1, 16, 256, 4, 2, 64, 512, 0, 1, 0)
    assert need > 0
    assert block(L, ws_bytes=need - 1) == -3
    # a cache removes the K/V scratch from the workspace
    assert L.llama_block_forward_workspace_bytes(1, 16, 256, 4, 2, 64, 512, 32, 1, 0) < need
    assert L.llama_block_forward_workspace_bytes(0, 16, 256, 4, 2, 64, 512, 0, 1, 0) == 0


def block_noalloc(L, **kw):
    w = binding.BlockWeights(*([FAKE + 0x1000 * i for i in range(1, 10)]))
    a = dict(x=FAKE, y=FAKE + 0x100, w=ctypes.byref(w), pos=FAKE + 0x200, kc=None, vc=None, cap=0, B=1, T=16,
             d=256, nq=4, nkv=2, hd=64, dff=512, theta=1e4, eps=1e-5, wdt=1, rdt=0)
    a.update(kw)
    return L.llama_block_forward_noalloc(a["x"], a["y"], a["w"], a["pos"], a["kc"], a["vc"], a["cap"], a["B"],
                                         a["T"], a["d"], a["nq"], a["nkv"], a["hd"], a["dff"], a["theta"], a["eps"],
                                         a["wdt"], a["rdt"], None)


def test_block_noalloc_validation_and_scratch_limit():
    """The entry point without a workspace validates like llama_block_forward
    and rejects, before touching the GPU, any call whose workspace would
    exceed the fixed scratch (LLAMA_NOALLOC_SCRATCH_BYTES)."""
    L = binding.lib()
    assert block_noalloc(L, nkv=3) == -1
    assert block_noalloc(L, cap=64) == -1
    assert block_noalloc(L, y=FAKE) == -1
    assert block_noalloc(L, hd=300) == -2
    assert block_noalloc(L, B=0) == 0
    # the Llama-3-8B prefill of 8192 tokens needs ~0.6 GB: refused
    big = L.llama_block_forward_workspace_bytes(1, 8192, 4096, 32, 8, 128, 14336, 0, 1, 0)
    assert big > binding.NOALLOC_SCRATCH_BYTES
    assert block_noalloc(L, T=8192, d=4096, nq=32, nkv=8, hd=128, dff=14336) == -3
    assert b"fixed scratch" in L.llama_last_error()
    # the 64-sequence decode step at 4097 slots fits
    dec = L.llama_block_forward_workspace_bytes(64, 1, 4096, 32, 8, 128, 14336, 4097, 1, 0)
    assert 0 < dec <= binding.NOALLOC_SCRATCH_BYTES


def test_empty_calls_are_noops():
    L = binding.lib()
    assert block(L, B=0) == 0
    assert attn(L, batch=0) == 0


def test_profile_query_unknown():
    L = binding.lib()
    assert L.llama_profile_reset() == 0
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    assert L.llama_profile_query(b"no_such_kernel", ctypes.byref(n), ctypes.byref(ms)) == -1


def test_fp8kv_validation():
    L = binding.lib()
    # append: head_dim must be 64/128/256; caches and capacity required
    assert L.llama_kv_append_fp8(FAKE, FAKE, FAKE, 2, 1, 8, 96, 1, FAKE, FAKE, FAKE, FAKE, 16, None) == -2
    assert L.llama_kv_append_fp8(FAKE, FAKE, FAKE, 2, 1, 8, 128, 1, None, FAKE, FAKE, FAKE, 16, None) == -1
    assert L.llama_kv_append_fp8(FAKE, FAKE, FAKE, 2, 1, 8, 128, 1, FAKE, FAKE, FAKE, FAKE, 0, None) == -1
    assert L.llama_kv_append_fp8(FAKE, FAKE, None, 2, 1, 8, 128, 1, FAKE, FAKE, FAKE, FAKE, 16, None) == -1
    assert L.llama_kv_append_fp8(FAKE, FAKE, FAKE, 2, 1, 8, 128, 9, FAKE, FAKE, FAKE, FAKE, 16, None) == -2

    def att(**kw):
        a = dict(q=FAKE, k=FAKE + 0x100, v=FAKE + 0x200, ks=FAKE + 0x300, vs=FAKE + 0x400, out=FAKE + 0x500,
                 pos=FAKE + 0x600, B=2, cap=100, nq=8, nkv=2, hd=128, ws=FAKE + 0x700, ws_bytes=1 << 30)
        a.update(kw)
        return L.llama_gqa_attention_fp8kv(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["out"], a["pos"], a["B"],
                                           a["cap"], a["nq"], a["nkv"], a["hd"], a["ws"], a["ws_bytes"], None)
    assert att(hd=64) == -2                 # only head_dim 128
    assert att(nq=24, nkv=2) == -2          # n_q / n_kv = 12
    assert att(nkv=3) == -1
    assert att(ks=None) == -1
    assert att(cap=0) == -1
    assert att(pos=None) == -1
    assert att(out=FAKE) == -1              # out aliases q
    assert att(k=FAKE + 0x104) == -2        # misaligned
    need = L.llama_gqa_attention_fp8kv_workspace_bytes(2, 100, 8, 2, 128)
    assert need > 0 and L.llama_gqa_attention_fp8kv_workspace_bytes(2, 100, 8, 2, 64) == 0
    assert att(ws_bytes=need - 1) == -3
    # block: the same shape limits; workspace reported for the decode step
    w = binding.BlockWeights(*([FAKE + 0x1000 * i for i in range(1, 10)]))
    need_b = L.llama_block_forward_fp8kv_workspace_bytes(4, 256, 4, 2, 128, 512, 64, 0)
    assert need_b > 0
    rc = L.llama_block_forward_fp8kv(FAKE, FAKE + 0x100, ctypes.byref(w), FAKE + 0x200, FAKE + 0x300, FAKE + 0x400,
                                     FAKE + 0x500, FAKE + 0x600, 64, 4, 256, 4, 2, 64, 512, 1e4, 1e-5, 0,
                                     FAKE + 0x700, need_b, None)
    assert rc == -2                         # head_dim 64
    rc = L.llama_block_forward_fp8kv(FAKE, FAKE + 0x100, ctypes.byref(w), FAKE + 0x200, FAKE + 0x300, FAKE + 0x400,
                                     FAKE + 0x500, FAKE + 0x600, 64, 4, 256, 4, 2, 128, 512, 1e4, 1e-5, 0,
                                     FAKE + 0x700, need_b - 1, None)
    assert rc == -3


def test_paged_validation():
    L = binding.lib()

    def att(**kw):
        a = dict(q=FAKE, kp=FAKE + 0x100, vp=FAKE + 0x200, tab=FAKE + 0x300, maxp=16, P=64, npg=100,
                 out=FAKE + 0x400, pos=FAKE + 0x500, B=2, nq=8, nkv=2, hd=128, ws=FAKE + 0x600, ws_bytes=1 << 30)
        a.update(kw)
        return L.llama_gqa_attention_paged(a["q"], a["kp"], a["vp"], a["tab"], a["maxp"], a["P"], a["npg"], a["out"],
                                           a["pos"], a["B"], a["nq"], a["nkv"], a["hd"], a["ws"], a["ws_bytes"], None)
    assert att(P=48) == -2                 # page size not a multiple of 32
    assert att(tab=None) == -1
    assert att(npg=0) == -1
    assert att(hd=64) == -2
    assert att(pos=None) == -1
    need = L.llama_gqa_attention_paged_workspace_bytes(2, 16, 64, 8, 2, 128)
    assert need > 0
    assert att(ws_bytes=need - 1) == -3
    assert L.llama_kv_append_paged(FAKE, FAKE, FAKE, FAKE, 4, 48, 2, 1, 8, 128, FAKE, FAKE, 10, None) == -2
    assert L.llama_kv_append_paged(FAKE, FAKE, FAKE, None, 4, 64, 2, 1, 8, 128, FAKE, FAKE, 10, None) == -1
    assert L.llama_kv_append_paged(FAKE, FAKE, FAKE, FAKE, 4, 64, 2, 1, 8, 12, FAKE, FAKE, 10, None) == -2


def test_lm_head_validation():
    L = binding.lib()
    need = L.llama_lm_head_argmax_workspace_bytes(64, 4096, 128256, 1, 0)
    assert need >= 64 * 128256 * 4
    assert L.llama_lm_head_argmax(FAKE, FAKE, FAKE, None, None, None, 64, 4096, 128256, 1e-5, 1, 0, FAKE, need,
                                  None) == -1                     # no token output
    assert L.llama_lm_head_argmax(FAKE, FAKE, FAKE, FAKE, None, None, 64, 4096, 0, 1e-5, 1, 0, FAKE, need,
                                  None) == -1                     # vocab 0
    assert L.llama_lm_head_argmax(FAKE, FAKE, FAKE, FAKE, None, None, 64, 4096, 128256, 1e-5, 1, 0, FAKE, need - 1,
                                  None) == -3
    assert L.llama_lm_head_argmax(FAKE, FAKE, FAKE, FAKE + 4, None, None, 64, 4096, 128256, 1e-5, 1, 0, FAKE, need,
                                  None) == -2                     # misaligned


def test_zero_widths_are_invalid():
    """Zero widths fail validation on the host; the empty-call contract (zero
    counts succeed and write nothing) is checked on the GPU."""
    L = binding.lib()
    bad = [
        L.llama_rmsnorm(FAKE, None, FAKE, FAKE + 0x100, None, 4, 0, 1e-5, 1, 0, None),
        L.llama_rope(FAKE, FAKE + 0x100, FAKE + 0x200, 4, 4, 2, 0, 1e4, 1, None),
        L.llama_gqa_attention(FAKE, FAKE + 0x100, FAKE + 0x200, FAKE + 0x300, None, 1, 4, 0, 4, 2, 64, 1, None, 0,
                              None),
        L.llama_gqa_attention(FAKE, FAKE + 0x100, FAKE + 0x200, FAKE + 0x300, None, 1, 4, 8, 0, 2, 64, 1, None, 0,
                              None),
        L.llama_swiglu_ffn(FAKE, FAKE, FAKE, FAKE, None, FAKE + 0x100, 4, 0, 64, 1, 0, None, 0, None),
        L.llama_swiglu_ffn(FAKE, FAKE, FAKE, FAKE, None, FAKE + 0x100, 4, 64, 0, 1, 0, None, 0, None),
        L.llama_lm_head_argmax(FAKE, FAKE, FAKE, FAKE + 0x100, None, None, 4, 64, 0, 1e-5, 1, 0, None, 0, None),
        L.llama_lm_head_argmax(FAKE, FAKE, FAKE, FAKE + 0x100, None, None, 4, 0, 100, 1e-5, 1, 0, None, 0, None),
    ]
    assert all(rc == -1 for rc in bad), bad
