"""Output layer on the GPU (final RMSNorm, linear head, argmax) against the
oracle (oracle/head.py).  Needs a GPU.

Logits are compared element by element with the storage-point oracle (the
normalized rows rounded to bf16 as the GPU stores them); the argmax is an
integer decided on the GPU's fp32 logits, so the check is that the chosen
token's oracle logit is within the logit tolerance of the oracle's maximum,
and that the tokens agree wherever the oracle's top two are further apart
than twice that tolerance.
"""

import numpy as np
import pytest
import torch

from oracle import head
from llama_decoder_block_amd import binding, synth
from metrics import report, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
LOGIT_TOL = 2e-3  # fp32 accumulation over d terms plus rare bf16 flips of the normalized row


def dev(t):
    return t.to(DEV)


def check(h, gamma, w, eps, tag):
    n, vocab = h.shape[0], w.shape[0]
    logits = torch.empty(n, vocab, dtype=torch.float32, device=DEV)
    best = torch.empty(n, dtype=torch.float32, device=DEV)
    tok = binding.lm_head_argmax(dev(h), dev(gamma), dev(w), eps, logits=logits, best=best)
    torch.cuda.synchronize()
    ref = head.lm_head_logits(to64(h), to64(gamma), to64(w), eps, bf16_storage=True)
    report(f"lm head {tag}", logits, ref)
    assert np.max(np.abs(to64(logits) - ref)) <= LOGIT_TOL
    t = tok.cpu().numpy().astype(np.int64)
    # the GPU's choice is the argmax of its own logits, exactly
    np.testing.assert_array_equal(t, head.greedy_token(to64(logits)))
    np.testing.assert_array_equal(to64(best), to64(logits)[np.arange(n), t])
    # and a valid choice for the oracle's logits
    mx = ref.max(axis=1)
    assert np.all(ref[np.arange(n), t] >= mx - 2 * LOGIT_TOL)
    srt = np.sort(ref, axis=1)
    clear = srt[:, -1] - srt[:, -2] > 4 * LOGIT_TOL
    np.testing.assert_array_equal(t[clear], head.greedy_token(ref)[clear])
    return t


@pytest.mark.parametrize("n,d,vocab", [(64, 4096, 128256), (64, 4096, 32000), (37, 4096, 32000), (5, 512, 1001),
                                        (300, 256, 4000)])
def test_lm_head_argmax(n, d, vocab):
    """64 x 4096 -> 128256 is the head of "LLaMA-3 8B 现代 LLM 架构、计算规模与能耗"
    §十 for the 64 sequences of the decode workload (the argmax over 31 full
    4096-column chunks and a partial last one of 1280); the other shapes cover ragged row counts,
    a vocabulary that is not a multiple of the chunk, and more rows than one
    skinny GEMM takes."""
    h = synth.normal(400, (n, d))
    gamma = synth.normal(401, (d,), 0.01, 1.0, dtype="bf16")
    w = synth.normal(402, (vocab, d), 0.02, dtype="bf16")
    check(h, gamma, w, 1e-5, f"{n}x{d}->{vocab}")


def test_lm_head_ties_go_to_smallest_index():
    n, d, vocab = 8, 512, 3000
    h = synth.normal(410, (n, d))
    gamma = torch.ones(d, dtype=torch.bfloat16)
    w = synth.normal(411, (vocab, d), 0.02, dtype="bf16")
    # rows 2900, 1234 and 7 identical and dominant for every token
    f = to64(h) / np.sqrt(np.mean(to64(h) ** 2, axis=1, keepdims=True))
    dom = torch.from_numpy(np.sign(f.sum(axis=0)) * 0.5).to(torch.bfloat16)
    for v in (2900, 1234, 7):
        w[v] = dom
    t = check(h, gamma, w, 1e-5, "ties")
    assert np.all(t == 7)
