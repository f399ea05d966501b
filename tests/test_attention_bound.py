"""The attention parity bound (tests/attn_bound.py) on the CPU: it admits
fp32 evaluations of the kernels' arithmetic, and it rejects plausible wrong
outputs on the same seeded inputs as the GPU tests (all zeros, one dropped
32-slot step, every eighth step dropped, an off-by-one visible length).

The fp32 evaluations follow the steps the bound is derived from: bf16 inputs,
fp32 scores, the running maximum as the row offset, exp2 in fp32, weights
rounded to bf16 (prefill) or kept in fp32 (decode), fp32 sums chunk by chunk
with the chunks merged by rescaling, one division and one rounding to bf16.  They stand in for a correct kernel; the
planted mistakes stand in for wrong ones.
"""

import math

import numpy as np
import pytest

import oracle
from attn_bound import attention_with_bound, attn_inputs
from metrics import to64

F32 = np.float32


def emulate(q, k, v, vis, bf16_weights, chunk=256):
    """fp32 attention with the kernels' arithmetic (see the module docstring):
    the visible slots in chunks of `chunk`, each chunk's (max, sum, weighted
    sum) merged into the running ones by rescaling."""
    q, k, v = to64(q).astype(F32), to64(k).astype(F32), to64(v).astype(F32)
    B, Tq, nq, hd = q.shape
    r = nq // k.shape[2]
    c = F32(F32(1.0 / math.sqrt(hd)) * F32(math.log2(math.e)))
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(B):
        for t in range(Tq):
            n = int(vis[b, t]) + 1
            for h in range(nq):
                gi = h // r
                m_run, l_run = F32(-np.inf), F32(0.0)
                o_run = np.zeros(hd, dtype=F32)
                for j0 in range(0, n, chunk):
                    kk, vv = k[b, j0:min(n, j0 + chunk), gi], v[b, j0:min(n, j0 + chunk), gi]
                    s = (kk @ q[b, t, h]).astype(F32)
                    cm = F32(s.max() * c)
                    m_new = F32(max(m_run, cm))
                    alpha = F32(np.exp2(F32(m_run - m_new))) if np.isfinite(m_run) else F32(0.0)
                    p = np.exp2((s * c - m_new).astype(F32)).astype(F32)
                    pw = oracle.round_bf16(p).astype(F32) if bf16_weights else p
                    l_run = F32(l_run * alpha + p.sum(dtype=F32))
                    o_run = (o_run * alpha + pw @ vv).astype(F32)
                    m_run = m_new
                out[b, t, h] = oracle.round_bf16((o_run / l_run).astype(F32))
    return out


def fails(got, ref, bound):
    return bool(np.any(np.abs(to64(got) - ref) > bound))


def test_bound_admits_fp32_prefill_and_decode_arithmetic():
    """Prefill-shaped (bf16 weights, 64-slot tiles) and decode-shaped (fp32
    weights, 256-slot chunks) evaluations stay inside."""
    q, k, v = attn_inputs(50, 1, 200, 200, 8, 2, 128, "bf16")
    vis = np.arange(200)[None, :]
    ref, bound = attention_with_bound(q, k, v, vis, bf16_weights=True)
    got = emulate(q, k, v, vis, True, chunk=64)
    assert not fails(got, ref, bound), np.max(np.abs(got - ref) / bound)
    # without the bf16 weight term the prefill evaluation would not fit: the
    # term is needed, not padding
    _, bound_fp32w = attention_with_bound(q, k, v, vis, bf16_weights=False)
    assert fails(got, ref, bound_fp32w)

    q, k, v = attn_inputs(90, 3, 1, 2000, 32, 8, 128, "bf16")
    vis = np.array([[1999], [700], [0]])
    ref, bound = attention_with_bound(q, k, v, vis, bf16_weights=False)
    got = emulate(q, k, v, vis, False, chunk=256)
    assert not fails(got, ref, bound), np.max(np.abs(got - ref) / bound)


@pytest.mark.parametrize("S", [32769, 131072])
def test_bound_rejects_wrong_long_context_decodes(S):
    """The inputs of the 32769- and 131072-slot decode parity tests: a correct
    fp32 evaluation passes; all zeros, one dropped 32-slot step, and every
    eighth 32-slot step dropped each fail."""
    q, k, v = attn_inputs(97, 1, 1, S, 32, 8, 128, "bf16")
    vis = np.array([[S - 1]])
    ref, bound = attention_with_bound(q, k, v, vis, bf16_weights=False)
    assert not fails(emulate(q, k, v, vis, False, chunk=2048), ref, bound)
    assert fails(np.zeros_like(ref), ref, bound)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    keep = np.ones(S, dtype=bool)
    keep[S // 2 - 32:S // 2] = False                      # one 32-slot step
    one = oracle.gqa_attention(q64, k64[:, keep], v64[:, keep], np.array([[keep.sum() - 1]]))
    assert fails(oracle.round_bf16(one), ref, bound)
    keep = np.ones(S, dtype=bool)
    for j0 in range(0, S - 32, 8 * 32):                   # every eighth step
        keep[j0:j0 + 32] = False
    eighth = oracle.gqa_attention(q64, k64[:, keep], v64[:, keep], np.array([[keep.sum() - 1]]))
    assert fails(oracle.round_bf16(eighth), ref, bound)


def test_bound_rejects_off_by_one_visible_length():
    """A decode that stops one slot short or reads one slot past the query's
    position fails on the 700-slot inputs of the per-pair decode test."""
    q, k, v = attn_inputs(95, 4, 1, 700, 32, 8, 128, "bf16")
    vis = np.array([[699], [300], [511], [64]])
    ref, bound = attention_with_bound(q, k, v, vis, bf16_weights=False)
    short = oracle.round_bf16(oracle.gqa_attention(to64(q), to64(k), to64(v), vis - 1))
    assert fails(short, ref, bound)
    vis2 = vis.copy()
    vis2[1:] += 1
    long_ = oracle.round_bf16(oracle.gqa_attention(to64(q), to64(k), to64(v), vis2))
    assert fails(long_[1:], ref[1:], bound[1:])


def test_bound_rejects_a_prefill_that_drops_the_diagonal():
    """A causal prefill whose mask hides each query's own slot (or lets it see
    the next one) fails on the flash test's inputs."""
    q, k, v = attn_inputs(50, 2, 64, 64, 8, 2, 128, "bf16")
    vis = np.broadcast_to(np.arange(64), (2, 64))
    ref, bound = attention_with_bound(q, k, v, vis, bf16_weights=True)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    vis_short = np.maximum(vis - 1, 0)
    bad = oracle.round_bf16(oracle.gqa_attention(q64, k64, v64, vis_short))
    assert fails(bad[:, 1:], ref[:, 1:], bound[:, 1:])
    vis_long = np.minimum(vis + 1, 63)
    bad = oracle.round_bf16(oracle.gqa_attention(q64, k64, v64, vis_long))
    assert fails(bad[:, :-1], ref[:, :-1], bound[:, :-1])
