"""fp64 reference definitions of the Llama decoder block forward.

TEST INFRASTRUCTURE ONLY (see the package docstring for the page tags
[LA], [RN], [L3], [MA]).

Conventions (readings of the pages, each stated where it is used):
  * weights are stored [out, in] and a projection is ``y = x @ W.T``, as the
    nn.Linear modules of [LA] "Production PyTorch Implementation" store them;
  * Q is [B, T, n_q, hd] and K, V are [B, S, n_kv, hd] (token-major, as the
    shape walk-through of [L3] §4.2 orders them); feature index = head*hd + i;
  * a key/value slot index equals the token position; a query at position p
    sees slots 0..p (history plus itself, [L3] §九); without a cache the
    slots are this call's own tokens and query t sees tokens 0..t.
All arithmetic is float64.  With ``bf16_storage=True`` the value of every
tensor the bf16 path stores in bf16 (a, q and k after RoPE, v, o, f, the
SwiGLU product) is rounded RNE to bf16 before it is used; accumulations, the
softmax denominator and the residual stream h, y are never rounded.  On the
prefill path (more than one query token per sequence) the bf16 path also
feeds the unnormalised softmax weights to its weighted sum of V in bf16: that
rounding is modelled by :func:`bf16_prefill_weights`.
"""

import numpy as np

from .bf16 import round_bf16


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def _store(a, bf16_storage):
    return round_bf16(a) if bf16_storage else a


# ----------------------------------------------------------------------------
# RMSNorm: x * (mean(x^2) + eps)^(-1/2) * gamma over the feature axis only.
# [LA] §1 and the RMSNorm module of "Step 1"; [RN] "How it works" (eps inside
# the square root, reduction over the last axis); [L3] §四.1; [MA] RMSNorm
# equation.  [LA]'s displayed equation puts eps outside the root; every other
# statement (including [LA]'s own code) puts it inside, which is the reading.
# ----------------------------------------------------------------------------
def rmsnorm(x, gamma, eps):
    x = _as64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _as64(gamma)


# ----------------------------------------------------------------------------
# RoPE.  theta_k = theta_base^(-2k/hd) for k = 0..hd/2-1 ([LA] §3, rotation
# matrix equation; the exponent's denominator is the head dimension, as the
# frequency precompute in "Step 1" takes it).  At position m the adjacent
# pair (x_2k, x_2k+1) is multiplied by [[cos, -sin], [sin, cos]] of angle
# m*theta_k ([LA] §3; [L3] §四.3 pairs (x0,x1)...(x126,x127)).  V is not
# rotated ([L3] §4.2).
# ----------------------------------------------------------------------------
def rope_inv_freq(head_dim, theta):
    k = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * k / head_dim)


def rope(x, positions, theta):
    """Rotate ``x[..., H, hd]`` whose leading axes match ``positions``."""
    x = _as64(x)
    hd = x.shape[-1]
    pos = _as64(positions)
    ang = pos[..., None] * rope_inv_freq(hd, theta)      # [..., hd/2]
    c = np.cos(ang)[..., None, :]                          # broadcast over heads
    s = np.sin(ang)[..., None, :]
    a = x[..., 0::2]
    b = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


# ----------------------------------------------------------------------------
# Projections without bias ([LA] §2 "without bias terms"; nn.Linear(bias=False)
# in "Step 1"/"Step 2").
# ----------------------------------------------------------------------------
def linear(x, w):
    return _as64(x) @ _as64(w).T


# SiLU(z) = z * sigmoid(z) = z / (1 + e^-z)  ([LA] §2; [L3] §五; [MA] Swish).
def silu(z):
    z = _as64(z)
    return z / (1.0 + np.exp(-z))


def softmax_last(s):
    """Softmax over the last axis: subtract the max, exponentiate, normalise
    ([L3] §4.5 applies it along the token axis).  -inf entries get weight 0."""
    s = _as64(s)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# ----------------------------------------------------------------------------
# Causal grouped-query attention.  Query head h reads KV head floor(h/r),
# r = n_q/n_kv ([L3] §4.4 mapping g(h); [LA] §4 repeat_interleave).  Scores are
# q.k/sqrt(hd) ([LA] §4 GQA equation; [L3] §4.5); keys after the query's
# position are masked; softmax over keys; output is the weighted sum of V
# ([L3] §4.5); heads are concatenated in order h = 0..n_q-1 ([L3] §4.7).
# ----------------------------------------------------------------------------
def bf16_prefill_weights(s):
    """Storage-point model of the prefill path's softmax weights, for scaled
    scores ``s`` [..., S] (-inf where masked).  The softmax of [L3] §4.5
    subtracts the row maximum, exponentiates and normalises; the bf16 path
    keeps the unnormalised weights p_j = exp(s_j - max s) as a bf16 tensor for
    the weighted sum of V (A19: P is one of the tensors it stores in bf16), so
    here each p_j is rounded RNE to bf16 while the normalising sum adds the
    unrounded p_j.  The weight of the maximum is exactly 1.
    Returns (rounded weights, denominator [..., 1])."""
    s = _as64(s)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return round_bf16(e), np.sum(e, axis=-1, keepdims=True)


def gqa_attention(q, k, v, visible_upto, bf16_weights=False):
    """q [B, Tq, n_q, hd]; k, v [B, S, n_kv, hd]; visible_upto [B, Tq] int:
    query (b, t) sees key slots 0..visible_upto[b, t].  Returns [B, Tq, n_q, hd].
    ``bf16_weights`` applies :func:`bf16_prefill_weights` (storage-point
    model of the prefill path) in place of the exact softmax.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Tq, n_q, hd = q.shape
    S, n_kv = k.shape[1], k.shape[2]
    r = n_q // n_kv
    vis = np.asarray(visible_upto, dtype=np.int64)
    slots = np.arange(S)
    out = np.empty_like(q)
    scale = 1.0 / np.sqrt(hd)
    for b in range(B):
        mask = slots[None, :] > vis[b][:, None]            # [Tq, S]
        for h in range(n_q):
            g = h // r
            s = (q[b, :, h, :] @ k[b, :, g, :].T) * scale  # [Tq, S]
            s = np.where(mask, -np.inf, s)
            if bf16_weights:
                wr, den = bf16_prefill_weights(s)
                out[b, :, h, :] = (wr @ v[b, :, g, :]) / den
            else:
                out[b, :, h, :] = softmax_last(s) @ v[b, :, g, :]
    return out


# ----------------------------------------------------------------------------
# SwiGLU FFN: W_down (SiLU(W_gate x) * (W_up x))  ([LA] §2 equation and the
# SwiGLUFFN module; [L3] §五; [MA] FFN equation).
# ----------------------------------------------------------------------------
def swiglu_ffn(x, w_gate, w_up, w_down, bf16_storage=False):
    g = linear(x, w_gate)
    u = linear(x, w_up)
    m = _store(silu(g) * u, bf16_storage)
    return linear(m, w_down)


# ----------------------------------------------------------------------------
# One block: h = x + Attn(RMSNorm(x)); y = h + FFN(RMSNorm(h))
# ([LA] "Step 2" block forward; [MA] block equations; [L3] §二 data flow).
# ----------------------------------------------------------------------------
def _attention_inputs(x, w, positions, theta, eps, n_q, n_kv, bf16_storage):
    B, T, d = x.shape
    hd = w["wq"].shape[0] // n_q
    a = _store(rmsnorm(x, w["attn_norm"], eps), bf16_storage)
    q = linear(a, w["wq"]).reshape(B, T, n_q, hd)
    k = linear(a, w["wk"]).reshape(B, T, n_kv, hd)
    v = linear(a, w["wv"]).reshape(B, T, n_kv, hd)
    q = _store(rope(q, positions, theta), bf16_storage)
    k = _store(rope(k, positions, theta), bf16_storage)
    v = _store(v, bf16_storage)
    return q, k, v


def _block_tail(x_rows, o_rows, w, eps, bf16_storage):
    o_rows = _store(o_rows, bf16_storage)
    h = x_rows + linear(o_rows, w["wo"])
    f = _store(rmsnorm(h, w["ffn_norm"], eps), bf16_storage)
    y = h + swiglu_ffn(f, w["w_gate"], w["w_up"], w["w_down"], bf16_storage)
    return h, y


def block_forward(x, w, positions, theta, eps, n_q, n_kv,
                  k_cache=None, v_cache=None, bf16_storage=False,
                  return_intermediates=False):
    """Forward of one block.

    x [B, T, d]; w: dict with attn_norm, wq, wk, wv, wo, ffn_norm, w_gate,
    w_up, w_down (weights [out, in]); positions [B, T] int.
    Without caches, the K/V slots are the T tokens and query t sees 0..t.
    With caches ([B, S_cap, n_kv, hd], given post-RoPE K and plain V), the new
    rotated k and v are written at slot = position (the caches passed in are
    not modified; the updated copies are returned) and query (b, t) sees slots
    0..positions[b, t] ([L3] §七 KV cache; §九 decode attends history + self).
    Returns y, or (y, dict of intermediates) if ``return_intermediates``.
    """
    x = _as64(x)
    B, T, d = x.shape
    pos = np.asarray(positions, dtype=np.int64).reshape(B, T)
    q, k, v = _attention_inputs(x, w, pos, theta, eps, n_q, n_kv, bf16_storage)
    if k_cache is None:
        kk, vv = k, v
        vis = np.broadcast_to(np.arange(T)[None, :], (B, T))
    else:
        kk = _store(_as64(k_cache).copy(), bf16_storage)
        vv = _store(_as64(v_cache).copy(), bf16_storage)
        for b in range(B):
            kk[b, pos[b]] = k[b]
            vv[b, pos[b]] = v[b]
        vis = pos
    o = gqa_attention(q, kk, vv, vis, bf16_weights=bf16_storage and T > 1).reshape(B, T, -1)
    h, y = _block_tail(x, o, w, eps, bf16_storage)
    if not return_intermediates:
        return y
    return y, dict(q=q, k=k, v=v, o=o, h=h, k_cache=kk, v_cache=vv)


def decode_step(x, w, position, k_cache, v_cache, theta, eps, n_q, n_kv,
                bf16_storage=False):
    """One-token decode for each sequence: x [B, 1, d], position [B] int
    ([L3] §九: the new query attends the cached history plus its own key).
    Returns (y, updated k_cache, updated v_cache)."""
    pos = np.asarray(position, dtype=np.int64).reshape(-1, 1)
    y, inter = block_forward(x, w, pos, theta, eps, n_q, n_kv, k_cache, v_cache,
                             bf16_storage, return_intermediates=True)
    return y, inter["k_cache"], inter["v_cache"]


def block_forward_rows(x, w, positions, rows, theta, eps, n_q, n_kv,
                       bf16_storage=False):
    """Cache-less prefill evaluated only at the token rows ``rows`` (list of
    (b, t)).  The same definition as :func:`block_forward`: K and V are
    projected for every token that a selected row can see, the selected rows
    run attention, O, the residuals and the FFN.  Returns (y_rows, h_rows)
    with one row per entry of ``rows``."""
    x = _as64(x)
    B, T, d = x.shape
    pos = np.asarray(positions, dtype=np.int64).reshape(B, T)
    hd = w["wq"].shape[0] // n_q
    ys, hs = [], []
    for b in sorted({b for b, _ in rows}):
        ts = [t for bb, t in rows if bb == b]
        tmax = max(ts) + 1
        xb = x[b:b + 1, :tmax]
        a = _store(rmsnorm(xb, w["attn_norm"], eps), bf16_storage)
        k = linear(a, w["wk"]).reshape(1, tmax, n_kv, hd)
        v = linear(a, w["wv"]).reshape(1, tmax, n_kv, hd)
        k = _store(rope(k, pos[b:b + 1, :tmax], theta), bf16_storage)
        v = _store(v, bf16_storage)
        ti = np.asarray(ts)
        q = linear(a[:, ti], w["wq"]).reshape(1, len(ts), n_q, hd)
        q = _store(rope(q, pos[b:b + 1, ti], theta), bf16_storage)
        o = gqa_attention(q, k, v, ti[None, :], bf16_weights=bf16_storage and T > 1).reshape(1, len(ts), -1)
        h, y = _block_tail(xb[:, ti], o, w, eps, bf16_storage)
        order = {t: i for i, t in enumerate(ts)}
        for t in ts:
            ys.append(((b, t), y[0, order[t]]))
            hs.append(((b, t), h[0, order[t]]))
    ymap, hmap = dict(ys), dict(hs)
    return (np.stack([ymap[tuple(r)] for r in rows]),
            np.stack([hmap[tuple(r)] for r in rows]))
