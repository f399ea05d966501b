"""Per-element error bound for the bf16 attention kernels, against the exact
fp64 oracle (host-side numpy; test infrastructure).

Derived from the arithmetic the kernels perform on bf16 q, k, v (products of
two bf16 values are exact in fp32):

  1. scores s_j = q . k_j as fp32 sums of head_dim products;
  2. z_j = s_j * c - M in fp32 (c = log2(e) / sqrt(hd) rounded to fp32, M a
     row offset: any offset common to a row cancels in the normalisation),
     then the hardware exp2 (within 2 fp32 ulps); over an 8-bit cache the
     score and the weight each take one more fp32 product with a row scale;
  3. the prefill (flash) kernel rounds the unnormalised weight exp2(z_j) to
     bf16 before the weighted sum of V; the decode kernels keep it in fp32;
  4. fp32 sums over the visible slots of the weighted V rows (numerator) and
     of the unrounded weights (denominator), in the kernel's own order, with
     the partial sums of different chunks or wavefronts rescaled by a common
     factor and merged;
  5. one division and one rounding of the output to bf16.

With u = 2^-24 (fp32) and u_b = 2^-8 (bf16, 8 significant bits: an RNE
rounding changes a value by less than u_b of itself), normalised exact
weights w_j and o = sum_j w_j v_j, each output element obeys

  |o_gpu - o| <= (1 + 2 u_b) * ( u_b |o|                                  (5)
                 + [prefill] u_b sum_j w_j |v_j|                            (3)
                 + sum_j w_j eta_j (|v_j| + |o|)                           (1, 2)
                 + g(n) (sum_j w_j |v_j| + |o|) )                           (4)

where eta_j bounds the relative error of weight j from steps 1-2:
  eta_j = scale * e_s(j) + u * scale * (3 (s_max - s_j) + |s_j|) + ln2 * u * |z_j| + 6u,
  e_s(j) = g(hd) * sum_i |q_i k_ji|  (fp32 score sum), scale = 1/sqrt(hd),
and g(n) = lam * sqrt(n) * u bounds an fp32 sum of n terms relative to the
sum of their magnitudes (the numerator's error is at most g(n) sum_j p_j |v_j|,
the denominator's g(n) sum_j p_j, which reaches the output multiplied by
|o|; the merges of chunk partials add a few roundings, inside that margin).  That last form is the probabilistic rounding-error
bound of Higham and Mary ("A New Approach to Probabilistic Rounding Error
Analysis", SIAM J. Sci. Comput. 41(5), 2019): for any summation order, with
rounding errors modelled as independent and mean-zero, it holds with
probability at least 1 - 2n exp(-lam^2 (1 - u)^2 / 2); lam = 8 makes that
1 - 3e-9 at n = 131072 per element.  The deterministic form n u would be
0.8% of the output at 131072 slots, wide enough to pass an all-zero output.

The bound helper returns the oracle's output with the bound so that a test
compares element by element; `check_attention` asserts and reports the
largest error-to-bound ratio.
"""

import math

import numpy as np

import oracle
from metrics import max_abs, rel_frobenius, to64

U_F32 = 2.0 ** -24
U_BF16 = 2.0 ** -8
LAM = 8.0


def attn_inputs(seed, B, T, S, nq, nkv, hd, dtype):
    """Seeded q [B, T, nq, hd], k and v [B, S, nkv, hd] ~ N(0, 1) in `dtype`
    (the inputs of the attention parity tests)."""
    from llama_decoder_block_amd import synth
    q = synth.normal(seed, (B, T, nq, hd), dtype=dtype)
    k = synth.normal(seed + 1, (B, S, nkv, hd), dtype=dtype)
    v = synth.normal(seed + 2, (B, S, nkv, hd), dtype=dtype)
    return q, k, v


def g(n):
    """Probabilistic bound on an fp32 sum of n terms, relative to the sum of
    the magnitudes (see the module docstring)."""
    return LAM * math.sqrt(max(n, 1)) * U_F32


def attention_with_bound(q, k, v, visible_upto, bf16_weights):
    """q [B, Tq, n_q, hd]; k, v [B, S, n_kv, hd]; visible_upto [B, Tq].
    Returns (o_ref, bound), both [B, Tq, n_q, hd] float64: o_ref is the exact
    oracle (``oracle.gqa_attention``), bound the per-element bound of the
    module docstring.  ``bf16_weights``: the kernel rounds its weights to
    bf16 (the prefill kernel), else they stay fp32 (the decode kernels)."""
    q, k, v = to64(q), to64(k), to64(v)
    vis = np.asarray(visible_upto, dtype=np.int64)
    o_ref = oracle.gqa_attention(q, k, v, vis)
    B, Tq, n_q, hd = q.shape
    S, n_kv = k.shape[1], k.shape[2]
    r = n_q // n_kv
    scale = 1.0 / math.sqrt(hd)
    ghd = g(hd)
    bound = np.empty_like(o_ref)
    slots = np.arange(S)
    log2e, ln2 = math.log2(math.e), math.log(2.0)
    for b in range(B):
        mask = slots[None, :] > vis[b][:, None]                 # [Tq, S]
        n = vis[b] + 1                                          # visible slots per query
        gn = (LAM * U_F32) * np.sqrt(np.maximum(n, 1))[:, None]
        for h in range(n_q):
            gi = h // r
            kk, av = k[b, :, gi, :], np.abs(v[b, :, gi, :])
            s = np.where(mask, -np.inf, q[b, :, h, :] @ kk.T)     # unscaled scores [Tq, S]
            smax = s.max(axis=-1, keepdims=True)
            w = oracle.softmax_last(s * scale)                   # exact normalised weights
            gap = np.where(mask, 0.0, smax - s)
            e_s = ghd * (np.abs(q[b, :, h, :]) @ np.abs(kk).T)
            # |z_j| <= gap * scale * log2(e) + 9 for any row offset within 9 of the maximum
            s_abs = np.where(mask, 0.0, np.abs(s))
            eta = (scale * e_s + U_F32 * scale * (3 * gap + s_abs) + ln2 * U_F32 * (gap * scale * log2e + 9.0)
                   + 6 * U_F32)
            weta = np.where(mask, 0.0, w * eta)
            ao = np.abs(o_ref[b, :, h, :])
            A = w @ av                                            # sum_j w_j |v_j|
            terms = U_BF16 * ao + weta @ av + weta.sum(axis=-1, keepdims=True) * ao + gn * (A + ao)
            if bf16_weights:
                terms = terms + U_BF16 * A
            bound[b, :, h] = (1.0 + 2 * U_BF16) * terms
    return o_ref, bound


def check_attention(name, got, q, k, v, visible_upto, bf16_weights):
    """Asserts |got - oracle| <= bound element by element and prints the
    largest ratio of error to bound with the usual metrics."""
    o_ref, bound = attention_with_bound(q, k, v, visible_upto, bf16_weights)
    g64 = to64(got)
    err = np.abs(g64 - o_ref)
    ratio = float(np.max(err / bound))
    print(f"[{name}] max_abs={max_abs(g64, o_ref):.3e} relF={rel_frobenius(g64, o_ref):.3e} "
          f"max err/bound={ratio:.3f} (bound {bound.min():.2e}..{bound.max():.2e})", flush=True)
    assert np.all(err <= bound), f"{name}: error exceeds the bound by up to {ratio:.3f}x"
    return o_ref
