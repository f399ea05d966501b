"""Paged KV cache on the GPU against the oracle (oracle/paged.py; layout in
include/llama_block.h).  Needs a GPU.

* the paged cache writer places every row exactly (bit-exact copies) and
  leaves every other row untouched;
* decode attention over shuffled pages matches the oracle's attention over the
  gathered cache within the bf16 attention bound, with NaN in every row it
  must not read.
"""

import numpy as np
import pytest
import torch

from oracle import paged
from llama_decoder_block_amd import binding, synth
from attn_bound import check_attention
from metrics import report, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev(t):
    return t.to(DEV)


def kernel_used(fn):
    binding.profile_reset()
    binding.profile_enable(True)
    out = fn()
    torch.cuda.synchronize()
    names = binding.profile_collect()
    binding.profile_enable(False)
    return out, [n for n in names if n.startswith("attention/")]


def shuffled_table(seed, B, max_pages, n_pages):
    g = np.random.Generator(np.random.PCG64(seed))
    return g.permutation(n_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)


def test_append_paged_places_rows():
    B, T, nkv, hd, P, max_pages, n_pages = 3, 5, 2, 128, 32, 4, 16
    k = synth.normal(300, (B, T, nkv, hd), dtype="bf16")
    v = synth.normal(301, (B, T, nkv, hd), dtype="bf16")
    table = shuffled_table(302, B, max_pages, n_pages)
    table[2, 3] = -1                                           # a hole: slots 96..127 of sequence 2
    pos = torch.tensor([[0, 31, 32, 100, 127], [64, 5, 6, 7, 200], [96, 1, 2, 3, 4]], dtype=torch.int32)
    kp = torch.full((n_pages, P, nkv, hd), 7.0, dtype=torch.bfloat16, device=DEV)
    vp = kp.clone()
    binding.kv_append_paged(dev(k), dev(v), dev(pos), dev(torch.from_numpy(table)), kp, vp)
    torch.cuda.synchronize()
    gk, gv = to64(kp), to64(vp)
    want_k = np.full(gk.shape, 7.0)
    want_v = np.full(gv.shape, 7.0)
    for b in range(B):
        for t in range(T):
            p = int(pos[b, t])
            if p >= max_pages * P:
                continue                                        # outside the table: skipped
            pg = int(table[b, p // P])
            if pg < 0:
                continue                                        # hole: skipped
            want_k[pg, p % P] = to64(k[b, t])
            want_v[pg, p % P] = to64(v[b, t])
    np.testing.assert_array_equal(gk, want_k)
    np.testing.assert_array_equal(gv, want_v)


@pytest.mark.parametrize("nq,nkv,P", [(32, 8, 64), (8, 8, 32), (32, 4, 128), (64, 8, 64)])
def test_decode_attention_paged(nq, nkv, P):
    """48 sequences with ragged visible lengths over shuffled pages of a pool
    whose other rows are NaN (one workgroup per (sequence, KV head))."""
    B, hd = 48, 128
    max_pages = -(-700 // P)
    n_pages = B * max_pages + 7
    S = max_pages * P
    k = synth.normal(310, (B, S, nkv, hd), dtype="bf16")
    v = synth.normal(311, (B, S, nkv, hd), dtype="bf16")
    lens = [700, 1, 33, 64, 65, 300, 511, 512, 513, 699, 2, 31, 32, 100, 257, 640, 7, 650, 690, 350, 128, 129, 96, 97,
            3, 63, 95, 160, 191, 224, 400, 555, 16, 17, 48, 49, 80, 81, 200, 256, 384, 448, 449, 600, 601, 666, 698, 5]
    pos = np.array([n - 1 for n in lens])
    table = shuffled_table(312, B, max_pages, n_pages)
    kc, vc = to64(k), to64(v)
    # rows after each position are never read: NaN in the pool
    kn, vn = kc.copy(), vc.copy()
    for b, p in enumerate(pos):
        kn[b, p + 1:] = np.nan
        vn[b, p + 1:] = np.nan
    kpool = torch.from_numpy(paged.scatter(kn, table, n_pages, P)).to(torch.bfloat16)
    vpool = torch.from_numpy(paged.scatter(vn, table, n_pages, P)).to(torch.bfloat16)
    q = synth.normal(313, (B, 1, nq, hd), dtype="bf16")
    out, used = kernel_used(lambda: binding.gqa_attention_paged(
        dev(q), dev(kpool), dev(vpool), dev(torch.from_numpy(table)), dev(torch.from_numpy(pos.astype(np.int32)))))
    assert used == ["attention/attn_decode_wg_paged"]
    check_attention(f"decode paged {nq}/{nkv} P{P}", out, q, kc, vc, pos[:, None], bf16_weights=False)


def test_decode_attention_paged_long_context_split():
    """Two sequences of 12000 and 5000 visible slots in pages of 256: chunks
    spread over workgroups and merged through the workspace."""
    B, nq, nkv, hd, P = 2, 32, 8, 128, 256
    max_pages = -(-12000 // P)
    n_pages = B * max_pages + 3
    S = max_pages * P
    k = synth.normal(320, (B, S, nkv, hd), dtype="bf16")
    v = synth.normal(321, (B, S, nkv, hd), dtype="bf16")
    pos = np.array([11999, 4999])
    table = shuffled_table(322, B, max_pages, n_pages)
    kc, vc = to64(k), to64(v)
    kpool = torch.from_numpy(paged.scatter(kc, table, n_pages, P)).to(torch.bfloat16)
    vpool = torch.from_numpy(paged.scatter(vc, table, n_pages, P)).to(torch.bfloat16)
    q = synth.normal(323, (B, 1, nq, hd), dtype="bf16")
    out, used = kernel_used(lambda: binding.gqa_attention_paged(
        dev(q), dev(kpool), dev(vpool), dev(torch.from_numpy(table)), dev(torch.from_numpy(pos.astype(np.int32)))))
    assert used == ["attention/attn_decode_splitk_paged"]
    check_attention("decode paged split", out, q, kc, vc, pos[:, None], bf16_weights=False)
