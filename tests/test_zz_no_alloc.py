"""llama_block_forward_noalloc (the block forward on the library's fixed
device scratch) against llama_block_forward with a caller workspace, through
the C ABI.  Needs a GPU.

Two calls in a row, the second with a smaller input, so the second runs on
scratch that still holds the first call's contents: each output (and each
updated cache) must equal the workspace entry point's bit for bit, which is
within every parity bar of the block (the two run the same kernels).
"""

import pytest
import torch

from llama_decoder_block_amd import binding, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def inputs(wl, cap):
    inp = synth.make_block_inputs(wl)
    w = {k: v.to(DEV) for k, v in inp.weights.items()}
    x, pos = inp.x.to(DEV), inp.positions.to(DEV)
    caches = None
    if cap:
        g = torch.Generator(device=DEV).manual_seed(1000 * wl.index + 77)
        shape = (wl.batch, cap, wl.n_kv, wl.head_dim)
        kc = torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)
        vc = torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)
        caches = (kc, vc)
    return x, w, pos, caches


def compare(wl, cap=0):
    x, w, pos, caches = inputs(wl, cap)
    c_ws = tuple(c.clone() for c in caches) if caches else (None, None)
    c_na = tuple(c.clone() for c in caches) if caches else (None, None)
    y_ws = binding.block_forward(x, w, pos, wl.n_q, wl.n_kv, wl.theta, wl.eps, k_cache=c_ws[0], v_cache=c_ws[1])
    y_na = torch.full_like(x, float("nan"))
    binding.block_forward_noalloc(x, w, pos, wl.n_q, wl.n_kv, wl.theta, wl.eps, k_cache=c_na[0], v_cache=c_na[1],
                                  y=y_na)
    torch.cuda.synchronize()
    assert torch.isfinite(y_na).all()
    assert torch.equal(y_na, y_ws)
    if caches:
        assert torch.equal(c_na[0], c_ws[0]) and torch.equal(c_na[1], c_ws[1])


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    """First a 64-sequence Llama-3-8B decode step against 4097-slot caches
    (the decode workload's shape, position 4096), then a smaller prefill of
    2 x 100 tokens with GQA 8/2 heads, both through the fixed scratch."""
    big = synth.workload("llama3_8b_gqa_decode")
    need = binding.lib().llama_block_forward_workspace_bytes(big.batch, 1, big.d_model, big.n_q, big.n_kv,
                                                             big.head_dim, big.d_ff, big.kv_cap, binding.BF16,
                                                             binding.F32)
    assert 0 < need <= binding.NOALLOC_SCRATCH_BYTES
    compare(big, cap=big.kv_cap)
    small = synth.workload("llama3_8b_gqa_prefill", batch=2, seq=100, d_model=512, n_q=8, n_kv=2, head_dim=128,
                           d_ff=1376)
    compare(small)
    # and a repeat of the first shape after the smaller call
    compare(big, cap=big.kv_cap)


def test_noalloc_rejects_a_call_larger_than_the_scratch():
    wl = synth.workload("llama3_8b_gqa_prefill", seq=1024)
    x, w, pos, _ = inputs(wl, 0)
    with pytest.raises(binding.LlamaError) as e:
        binding.block_forward_noalloc(x, w, pos, wl.n_q, wl.n_kv, wl.theta, wl.eps)
    assert e.value.status == -3
