"""Output layer: final RMSNorm, linear head, greedy choice.

TEST INFRASTRUCTURE ONLY (part of the oracle; see the package docstring).

[L3] §十 (output layer and sampling): after the last block, a final RMSNorm,
the linear head [d_model -> vocab] and, for greedy decoding, argmax over the
vocabulary of the last position's logits (argmax of the softmax is argmax of
the logits).  Reading: the head weight is [vocab, d_model] ([out, in], as the
block's projections); among equal logits the smallest index is chosen.
"""

import numpy as np

from .bf16 import round_bf16
from .reference import linear, rmsnorm


def lm_head_logits(h, gamma, w_head, eps, bf16_storage=False):
    """h [N, d] -> logits [N, vocab] (float64).  With ``bf16_storage`` the
    normalized rows are rounded to bf16 before the head, as the bf16 path
    stores them."""
    f = rmsnorm(np.asarray(h, dtype=np.float64), gamma, eps)
    if bf16_storage:
        f = round_bf16(f)
    return linear(f, w_head)


def greedy_token(logits):
    """argmax over the last axis; ties go to the smallest index; NaN is never
    chosen (unless a whole row is NaN, which gives 0)."""
    lg = np.asarray(logits, dtype=np.float64)
    masked = np.where(np.isnan(lg), -np.inf, lg)
    return np.argmax(masked, axis=-1)  # numpy returns the first maximal index
