"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a value the
pages print, a closed form, an invariant the pages state, a special case that
reduces to a library routine, or a brute-force scalar loop on tiny inputs.
Page tags: [LA] "Llama Architecture: RMSNorm, SwiGLU, RoPE, GQA, and PyTorch
Implementation"; [RN] the "RMSNorm" study note; [L3] "LLaMA-3 8B 现代 LLM 架构、
计算规模与能耗"; [MA] "LLaMA Architecture > Model Architecture".
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import bruteforce


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def rand_weights(g, d, nq, nkv, hd, dff, scale=0.3, unit_gain=False):
    w = {
        "attn_norm": np.ones(d) if unit_gain else 1.0 + 0.1 * g.standard_normal(d),
        "wq": scale * g.standard_normal((nq * hd, d)),
        "wk": scale * g.standard_normal((nkv * hd, d)),
        "wv": scale * g.standard_normal((nkv * hd, d)),
        "wo": scale * g.standard_normal((d, nq * hd)),
        "ffn_norm": np.ones(d) if unit_gain else 1.0 + 0.1 * g.standard_normal(d),
        "w_gate": scale * g.standard_normal((dff, d)),
        "w_up": scale * g.standard_normal((dff, d)),
        "w_down": scale * g.standard_normal((d, dff)),
    }
    return w


# --------------------------------------------------------------------------
# [L3] §4.3-4.6 worked example (golden file with the printed tables)
# --------------------------------------------------------------------------
def load_toy(golden_dir):
    k = np.zeros((1, 4, 2, 2))
    v = np.zeros((1, 4, 2, 2))
    q = np.zeros((1, 1, 8, 2))
    tabs = {"score": {}, "prob": {}, "out": {}}
    with open(os.path.join(golden_dir, "l3_gqa_toy_attention.txt"), encoding="utf-8") as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            tag, *vals = line.split()
            if tag in ("k", "v"):
                s, g, e0, e1 = int(vals[0]), int(vals[1]), float(vals[2]), float(vals[3])
                (k if tag == "k" else v)[0, s, g] = (e0, e1)
            elif tag == "q":
                q[0, 0, int(vals[0])] = (float(vals[1]), float(vals[2]))
            else:
                tabs[tag][int(vals[0])] = np.array([float(x) for x in vals[1:]])
    return q, k, v, tabs


def test_worked_example_outputs_match_printed_table(golden_dir):
    q, k, v, tabs = load_toy(golden_dir)
    o = oracle.gqa_attention(q, k, v, visible_upto=np.array([[3]]))
    for h in range(8):
        np.testing.assert_allclose(o[0, 0, h], tabs["out"][h], atol=5e-4)


def test_worked_example_closed_forms(golden_dir):
    # weights (e^a, 1, e^-a, 1)/(e^a + 2 + e^-a) with a = sqrt(2); outputs
    # +-tanh(1/sqrt 2) for KV head 0 and +-2 tanh(1/sqrt 2) for KV head 1.
    q, k, v, _ = load_toy(golden_dir)
    o = oracle.gqa_attention(q, k, v, visible_upto=np.array([[3]]))
    t = math.tanh(1.0 / math.sqrt(2.0))
    expect = np.array([[t, 0], [0, t], [-t, 0], [0, -t],
                       [2 * t, 0], [0, 2 * t], [-2 * t, 0], [0, -2 * t]])
    np.testing.assert_allclose(o[0, 0], expect, atol=1e-14)


def test_softmax_matches_printed_weights(golden_dir):
    _, _, _, tabs = load_toy(golden_dir)
    a = math.sqrt(2.0)
    z = math.exp(a) + 2 + math.exp(-a)
    exact = np.array([math.exp(a), 1.0, math.exp(-a), 1.0]) / z
    for h in range(8):
        p = oracle.softmax_last(tabs["score"][h])
        np.testing.assert_allclose(p, tabs["prob"][h], atol=5e-4)
    np.testing.assert_allclose(oracle.softmax_last(np.array([a, 0, -a, 0])), exact, rtol=1e-15)


def test_head_group_isolation_toy(golden_dir):
    # Q0-Q3 never read KV head 1; Q4-Q7 never read KV head 0 ([L3] §4.4)
    q, k, v, _ = load_toy(golden_dir)
    base = oracle.gqa_attention(q, k, v, np.array([[3]]))
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 1] += 0.7
    v2[0, :, 1] -= 1.3
    pert = oracle.gqa_attention(q, k2, v2, np.array([[3]]))
    np.testing.assert_array_equal(pert[0, 0, :4], base[0, 0, :4])
    assert np.all(np.abs(pert[0, 0, 4:] - base[0, 0, 4:]).max(axis=-1) > 1e-3)


# --------------------------------------------------------------------------
# RMSNorm ([LA] §1, [RN], [L3] §四.1, [MA])
# --------------------------------------------------------------------------
@pytest.mark.parametrize("c", [1.0, -3.0, 100.0, 1e-3])
def test_rmsnorm_constant_vector(c):
    eps = 1e-5
    x = np.full((3, 4096), c)
    y = oracle.rmsnorm(x, np.ones(4096), eps)
    expect = c / math.sqrt(c * c + eps)
    np.testing.assert_allclose(y, expect, rtol=1e-14)
    if c == 1.0:
        # all ones to eps: 0.999995..., and not c/(c+eps) = 0.99999000...
        assert abs(y[0, 0] - 0.9999950000374997) < 1e-15
        assert abs(y[0, 0] - 1.0 / (1.0 + eps)) > 4e-6


def test_rmsnorm_output_rms_and_row_independence():
    g = rng(1)
    eps = 1e-5
    x = g.standard_normal((5, 256)) * np.array([[0.01], [1.0], [3.0], [100.0], [1e-3]])
    y = oracle.rmsnorm(x, np.ones(256), eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)
    # row independence: each row normalised alone gives the same result
    for i in range(5):
        np.testing.assert_array_equal(oracle.rmsnorm(x[i:i + 1], np.ones(256), eps)[0], y[i])
    # the gain multiplies element-wise, no mean is removed
    gam = g.standard_normal(256)
    np.testing.assert_allclose(oracle.rmsnorm(x, gam, eps), y * gam, rtol=1e-14)
    xs = x + 5.0
    assert not np.allclose(oracle.rmsnorm(xs, np.ones(256), eps).mean(axis=1), 0.0)


def test_rmsnorm_bruteforce():
    g = rng(2)
    x = g.standard_normal(16)
    gam = g.standard_normal(16)
    np.testing.assert_allclose(oracle.rmsnorm(x[None], gam, 1e-5)[0],
                               bruteforce.rmsnorm_row(list(x), list(gam), 1e-5), rtol=1e-14)


# --------------------------------------------------------------------------
# RoPE ([LA] §3, [L3] §四.3)
# --------------------------------------------------------------------------
def test_rope_position_zero_is_identity():
    g = rng(3)
    x = g.standard_normal((1, 3, 4, 128))
    np.testing.assert_array_equal(oracle.rope(x, np.zeros((1, 3), np.int64), 5e5), x)


def test_rope_hd2_rotates_by_m_radians():
    # head_dim 2: theta_0 = base^0 = 1 for any base, so the angle is m rad and
    # (1, 0) goes to (cos m, sin m) under the page's rotation matrix.
    for base in (1e4, 5e5):
        for m in (1, 2, 7, 4096):
            out = oracle.rope(np.array([[[[1.0, 0.0]]]]), np.array([[m]]), base)
            np.testing.assert_allclose(out[0, 0, 0], [math.cos(m), math.sin(m)], atol=1e-15)
            out = oracle.rope(np.array([[[[0.0, 1.0]]]]), np.array([[m]]), base)
            np.testing.assert_allclose(out[0, 0, 0], [-math.sin(m), math.cos(m)], atol=1e-15)


def test_rope_frequencies_closed_form():
    f = oracle.rope_inv_freq(128, 1e4)
    assert f[0] == 1.0
    np.testing.assert_allclose(f[63], 1e4 ** (-126.0 / 128.0), rtol=1e-15)
    np.testing.assert_allclose(f[1], 1e4 ** (-2.0 / 128.0), rtol=1e-15)
    f5 = oracle.rope_inv_freq(128, 5e5)
    np.testing.assert_allclose(f5[32], 5e5 ** -0.5, rtol=1e-15)


def test_rope_equals_complex_multiplication():
    # multiplying x_2k + i x_2k+1 by exp(i m theta_k) (numpy complex exp)
    g = rng(4)
    hd = 128
    x = g.standard_normal((2, 5, 3, hd))
    pos = g.integers(0, 8192, size=(2, 5))
    for base in (1e4, 5e5):
        out = oracle.rope(x, pos, base)
        k = np.arange(hd // 2)
        z = x[..., 0::2] + 1j * x[..., 1::2]
        rot = np.exp(1j * pos[..., None, None] * (base ** (-2.0 * k / hd)))
        zr = z * rot
        np.testing.assert_allclose(out[..., 0::2], zr.real, atol=1e-12)
        np.testing.assert_allclose(out[..., 1::2], zr.imag, atol=1e-12)


def test_rope_preserves_pair_norms():
    g = rng(5)
    x = g.standard_normal((1, 64, 8, 128))
    pos = np.arange(64)[None] * 131
    out = oracle.rope(x, pos, 5e5)
    n_in = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n_out = out[..., 0::2] ** 2 + out[..., 1::2] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12)


@pytest.mark.parametrize("base", [1e4, 5e5])
def test_rope_dot_depends_only_on_offset(base):
    g = rng(6)
    hd = 128
    for _ in range(20):
        q = g.standard_normal(hd)
        k = g.standard_normal(hd)
        m, n = g.integers(0, 4096, size=2)
        s = int(g.integers(1, 8192 - 4096))
        def dot(mm, nn):
            qr = oracle.rope(q[None, None, None], np.array([[mm]]), base)[0, 0, 0]
            kr = oracle.rope(k[None, None, None], np.array([[nn]]), base)[0, 0, 0]
            return float(qr @ kr)
        np.testing.assert_allclose(dot(m, n), dot(m + s, n + s), rtol=1e-9, atol=1e-9)


def test_rope_composition():
    g = rng(7)
    x = g.standard_normal((1, 1, 2, 64))
    a = oracle.rope(oracle.rope(x, np.array([[300]]), 1e4), np.array([[77]]), 1e4)
    b = oracle.rope(x, np.array([[377]]), 1e4)
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_rope_bruteforce():
    g = rng(8)
    v = g.standard_normal(16)
    out = oracle.rope(v[None, None, None], np.array([[1234]]), 5e5)[0, 0, 0]
    np.testing.assert_allclose(out, bruteforce.rope_head(list(v), 1234, 5e5), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# Attention ([LA] §4, [L3] §4.4-4.7)
# --------------------------------------------------------------------------
def test_gqa_equals_mha_on_repeat_interleaved_kv():
    g = rng(9)
    B, T, nq, nkv, hd = 2, 7, 8, 2, 16
    q = g.standard_normal((B, T, nq, hd))
    k = g.standard_normal((B, T, nkv, hd))
    v = g.standard_normal((B, T, nkv, hd))
    vis = np.broadcast_to(np.arange(T), (B, T))
    gqa = oracle.gqa_attention(q, k, v, vis)
    mha = oracle.gqa_attention(q, np.repeat(k, nq // nkv, axis=2), np.repeat(v, nq // nkv, axis=2), vis)
    np.testing.assert_allclose(gqa, mha, rtol=1e-14, atol=1e-15)


def test_gqa_head_map_perturbation():
    g = rng(10)
    B, T, nq, nkv, hd = 1, 6, 12, 3, 8
    r = nq // nkv
    q = g.standard_normal((B, T, nq, hd))
    k = g.standard_normal((B, T, nkv, hd))
    v = g.standard_normal((B, T, nkv, hd))
    vis = np.arange(T)[None]
    base = oracle.gqa_attention(q, k, v, vis)
    for grp in range(nkv):
        k2 = k.copy()
        k2[:, :, grp] += 1.0
        out = oracle.gqa_attention(q, k2, v, vis)
        changed = np.abs(out - base).max(axis=(0, 1, 3)) > 0
        assert list(np.nonzero(changed)[0]) == list(range(grp * r, (grp + 1) * r))


def test_attention_first_token_sees_only_itself_and_uniform_scores():
    g = rng(11)
    B, T, nq, nkv, hd = 1, 5, 4, 2, 8
    q = g.standard_normal((B, T, nq, hd))
    k = g.standard_normal((B, T, nkv, hd))
    v = g.standard_normal((B, T, nkv, hd))
    vis = np.arange(T)[None]
    o = oracle.gqa_attention(q, k, v, vis)
    for h in range(nq):
        np.testing.assert_allclose(o[0, 0, h], v[0, 0, h // 2], rtol=1e-15)
    # q = 0: every visible key has weight 1/(t+1): o is the running mean of v
    o0 = oracle.gqa_attention(np.zeros_like(q), k, v, vis)
    for t in range(T):
        np.testing.assert_allclose(o0[0, t, 3], v[0, :t + 1, 1].mean(axis=0), rtol=1e-13)


def test_attention_softmax_against_scipy():
    from scipy.special import softmax
    g = rng(12)
    s = g.standard_normal((4, 9)) * 5
    np.testing.assert_allclose(oracle.softmax_last(s), softmax(s, axis=-1), rtol=1e-13)


# --------------------------------------------------------------------------
# SiLU and SwiGLU ([LA] §2, [L3] §五, [MA])
# --------------------------------------------------------------------------
def test_silu_closed_values_and_library():
    from scipy.special import expit
    assert oracle.silu(0.0) == 0.0
    np.testing.assert_allclose(oracle.silu(1.0), 0.7310585786300049, rtol=1e-15)
    np.testing.assert_allclose(oracle.silu(-1.0), -0.2689414213699951, rtol=1e-15)
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)


def test_swiglu_zero_gate_and_zero_down():
    g = rng(13)
    x = g.standard_normal((5, 32))
    wg = g.standard_normal((48, 32))
    wu = g.standard_normal((48, 32))
    wd = g.standard_normal((32, 48))
    assert np.all(oracle.swiglu_ffn(x, np.zeros_like(wg), wu, wd) == 0.0)
    assert np.all(oracle.swiglu_ffn(x, wg, wu, np.zeros_like(wd)) == 0.0)


def test_swiglu_diagonal_closed_form_catches_branch_swap():
    g = rng(14)
    d = 6
    x = g.standard_normal((3, d))
    a = g.uniform(0.5, 2.0, d)
    b = g.uniform(-2.0, -0.5, d)
    out = oracle.swiglu_ffn(x, np.diag(a), np.diag(b), np.eye(d))
    expect = np.empty_like(x)
    for i in range(3):
        for j in range(d):
            z = a[j] * x[i, j]
            expect[i, j] = z / (1.0 + math.exp(-z)) * (b[j] * x[i, j])
    np.testing.assert_allclose(out, expect, rtol=1e-14)
    swapped = oracle.swiglu_ffn(x, np.diag(b), np.diag(a), np.eye(d))
    assert np.abs(swapped - expect).max() > 1e-2


def test_linear_orientation_and_bruteforce():
    g = rng(15)
    x = g.standard_normal((3, 5))
    w = g.standard_normal((7, 5))       # [out, in]
    y = oracle.linear(x, w)
    assert y.shape == (3, 7)
    for i in range(3):
        np.testing.assert_allclose(y[i], bruteforce.matvec(w.tolist(), x[i].tolist()), rtol=1e-14)


# --------------------------------------------------------------------------
# Whole block ([LA] "Step 2", [MA] block equations, [L3] §二/§七/§九)
# --------------------------------------------------------------------------
TOY = dict(d=16, nq=8, nkv=2, hd=2, dff=48)


def toy_inputs(seed, B=1, T=4, unit_gain=True, scale=0.3):
    g = rng(seed)
    w = rand_weights(g, TOY["d"], TOY["nq"], TOY["nkv"], TOY["hd"], TOY["dff"], scale, unit_gain)
    x = g.standard_normal((B, T, TOY["d"]))
    pos = np.broadcast_to(np.arange(T), (B, T)).copy()
    return x, w, pos


def test_block_bruteforce_toy():
    for seed, gain in ((20, True), (21, False)):
        x, w, pos = toy_inputs(seed, B=2, T=4, unit_gain=gain)
        y = oracle.block_forward(x, w, pos, 1e4, 1e-5, 8, 2)
        yb = np.array(bruteforce.block_forward(x, w, pos, 1e4, 1e-5, 8, 2))
        np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-13)


def test_block_bruteforce_hd8_theta():
    # head_dim 8 exercises theta_base (the toy's head_dim 2 does not)
    g = rng(22)
    d, nq, nkv, hd, dff = 32, 4, 2, 8, 24
    w = rand_weights(g, d, nq, nkv, hd, dff)
    x = g.standard_normal((1, 5, d))
    pos = np.arange(5)[None] * 97 + 11
    for base in (1e4, 5e5):
        y = oracle.block_forward(x, w, pos, base, 1e-5, nq, nkv)
        yb = np.array(bruteforce.block_forward(x, w, pos, base, 1e-5, nq, nkv))
        np.testing.assert_allclose(y, yb, rtol=1e-11, atol=1e-12)


def test_block_zero_sublayers_is_identity():
    # a sublayer that outputs zeros leaves the residual stream unchanged ([MA])
    x, w, pos = toy_inputs(23, B=2, T=4, unit_gain=False)
    w0 = dict(w, wo=np.zeros_like(w["wo"]), w_down=np.zeros_like(w["w_down"]))
    y = oracle.block_forward(x, w0, pos, 1e4, 1e-5, 8, 2)
    np.testing.assert_array_equal(y, x)
    w1 = dict(w, w_down=np.zeros_like(w["w_down"]))
    y1, inter = oracle.block_forward(x, w1, pos, 1e4, 1e-5, 8, 2, return_intermediates=True)
    np.testing.assert_array_equal(y1, inter["h"])
    assert np.abs(inter["h"] - x).max() > 1e-3


def test_block_causal_future_perturbation():
    x, w, pos = toy_inputs(24, B=1, T=6, unit_gain=False)
    y = oracle.block_forward(x, w, pos, 1e4, 1e-5, 8, 2)
    for t in range(5):
        x2 = x.copy()
        x2[0, t + 1:] += 3.0
        y2 = oracle.block_forward(x2, w, pos, 1e4, 1e-5, 8, 2)
        np.testing.assert_array_equal(y2[0, :t + 1], y[0, :t + 1])
        assert np.abs(y2[0, t + 1:] - y[0, t + 1:]).max() > 1e-3


def test_prefill_then_decode_matches_longer_prefill():
    g = rng(25)
    d, nq, nkv, hd, dff = 32, 4, 2, 8, 40
    w = rand_weights(g, d, nq, nkv, hd, dff)
    B, T = 2, 6
    x = g.standard_normal((B, T + 1, d))
    pos = np.broadcast_to(np.arange(T + 1), (B, T + 1)).copy()
    full = oracle.block_forward(x, w, pos, 5e5, 1e-5, nq, nkv)
    cap = T + 3
    kc = np.zeros((B, cap, nkv, hd))
    vc = np.zeros((B, cap, nkv, hd))
    yp, inter = oracle.block_forward(x[:, :T], w, pos[:, :T], 5e5, 1e-5, nq, nkv, kc, vc,
                                     return_intermediates=True)
    np.testing.assert_allclose(yp, full[:, :T], rtol=1e-12, atol=1e-12)
    yd, kc2, vc2 = oracle.decode_step(x[:, T:T + 1], w, np.full(B, T), inter["k_cache"],
                                      inter["v_cache"], 5e5, 1e-5, nq, nkv)
    np.testing.assert_allclose(yd[:, 0], full[:, T], rtol=1e-12, atol=1e-12)
    assert np.all(kc2[:, T + 1:] == 0) and np.any(kc2[:, T] != 0)


def test_block_rows_matches_full():
    g = rng(26)
    d, nq, nkv, hd, dff = 64, 8, 2, 8, 96
    w = rand_weights(g, d, nq, nkv, hd, dff, scale=0.1)
    x = g.standard_normal((2, 9, d))
    pos = np.broadcast_to(np.arange(9), (2, 9)).copy()
    rows = [(0, 0), (1, 8), (0, 5), (1, 3)]
    for st in (False, True):
        y, inter = oracle.block_forward(x, w, pos, 1e4, 1e-5, nq, nkv, bf16_storage=st,
                                        return_intermediates=True)
        yr, hr = oracle.block_forward_rows(x, w, pos, rows, 1e4, 1e-5, nq, nkv, bf16_storage=st)
        for i, (b, t) in enumerate(rows):
            np.testing.assert_allclose(yr[i], y[b, t], rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(hr[i], inter["h"][b, t], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# bf16 rounding used by the storage-point variant (pinned to torch's cast)
# --------------------------------------------------------------------------
def test_round_bf16_against_torch_cast():
    g = rng(27)
    vals = np.concatenate([
        g.standard_normal(100000) * 10.0 ** g.integers(-40, 38, 100000),
        (1.0 + np.arange(512) / 2.0 ** 9),            # ties and near-ties around 1..2
        -(1.0 + np.arange(512) / 2.0 ** 9),
        np.array([0.0, -0.0, 3.0e38, 1e-39, 1e-44]),
    ]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    ours = oracle.round_bf16(vals)
    np.testing.assert_array_equal(ours, ref)
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 1.0            # tie to even (down)
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # tie to even (up)


# --------------------------------------------------------------------------
# storage-point model of the prefill path's softmax weights (bf16 weights,
# integer log2 offset, unrounded denominator)
# --------------------------------------------------------------------------
def attend_one(scores, v, bf16_weights):
    """One query over len(scores) keys (V rows of width <= 4) through
    oracle.gqa_attention with hd = 4: q = e_0 and k_j = 2 s_j e_0, so that
    q.k_j / sqrt(4) is exactly s_j."""
    S = len(scores)
    v = np.asarray(v, dtype=np.float64).reshape(S, -1)
    q = np.zeros((1, 1, 1, 4))
    q[..., 0] = 1.0
    k = np.zeros((1, S, 1, 4))
    k[0, :, 0, 0] = 2.0 * np.asarray(scores, dtype=np.float64)
    vv = np.zeros((1, S, 1, 4))
    vv[0, :, 0, :v.shape[1]] = v
    out = oracle.gqa_attention(q, k, vv, np.array([[S - 1]]), bf16_weights=bf16_weights)
    return out[0, 0, 0, :v.shape[1]]


def test_prefill_weights_hand_example():
    """Scores 0.3 ln 2 and -0.2 ln 2: the row maximum is the first, so the
    unnormalised weights are exp(0) = 1 and exp(-0.5 ln 2) = 2^-0.5; rounded
    to bf16 they are 1 and 0.70703125 (181/256), while the denominator keeps
    the unrounded sum 1 + 2^-0.5."""
    ln2 = math.log(2.0)
    out = attend_one([0.3 * ln2, -0.2 * ln2], [[1.0, 0.0], [0.0, 1.0]], True)
    den = 1.0 + 2.0 ** -0.5
    np.testing.assert_allclose(out, [1.0 / den, 0.70703125 / den], rtol=1e-14)
    # an integer offset ceil(max) instead of the maximum itself would round
    # 2^-0.7 and 2^-1.2 (to 158/256 and 223/512) and give other outputs
    den_c = 2.0 ** -0.7 + 2.0 ** -1.2
    assert abs(out[0] - 0.6171875 / den_c) > 1e-3
    assert abs(out[1] - 0.435546875 / den_c) > 2e-4


def test_prefill_weights_uniform_scores_give_mean():
    """Equal scores c: every weight is exp(c - c) = 1, exact in bf16, over a
    denominator of 7, so the output is exactly mean(v) whatever c is."""
    g = rng(28)
    v = g.standard_normal((7, 4))
    for c in (0.0, 2.5, -13.0, 0.3):
        np.testing.assert_allclose(attend_one([c] * 7, v, True), v.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_prefill_weights_maximum_counts_exactly_once():
    """The maximum's weight is 1 whatever its score: a row of one score s0
    and others at least 500 below it (weights exp(-500) and less, which round
    to zero in bf16 and vanish from the fp64 denominator) gives exactly v at
    the maximum's slot."""
    v = rng(32).standard_normal((5, 3))
    for s0 in (7.25, -3.5, 0.0):
        scores = [s0 - 500.0, s0 - 600.0, s0, s0 - 700.0, s0 - 800.0]
        np.testing.assert_array_equal(attend_one(scores, v, True), v[2])


def test_prefill_weights_representable_equal_exact():
    """Scores whose weights are powers of two (bf16-exact) give the exact
    softmax result."""
    g = rng(29)
    z = np.array([0.0, -1.0, -2.0, -5.0, -3.0, 1.0, -7.0])
    v = g.standard_normal((7, 4))
    got = attend_one(z * math.log(2.0), v, True)
    w = 2.0 ** z
    np.testing.assert_allclose(got, (w / w.sum()) @ v, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(got, attend_one(z * math.log(2.0), v, False), rtol=1e-13, atol=1e-15)


def test_prefill_weights_within_bf16_bound():
    """Each weight carries a relative error of at most 2^-8, so the output
    stays within 2^-8 * sum_j p_j |v_j| of the exact softmax result."""
    g = rng(30)
    for _ in range(50):
        S = int(g.integers(1, 200))
        s = g.standard_normal(S) * 4
        v = g.standard_normal((S, 3))
        got = attend_one(s, v, True)
        p = np.exp(s - s.max())
        p /= p.sum()
        exact = p @ v
        assert np.all(np.abs(got - exact) <= 2.0 ** -8 * (p @ np.abs(v)) + 1e-15)


def test_block_storage_weights_only_on_prefill_path():
    """The bf16 weight model applies to calls with more than one query token;
    a one-token call (the decode path) keeps the exact softmax."""
    g = rng(31)
    d, nq, nkv, hd, dff = 32, 4, 2, 8, 48
    w = rand_weights(g, d, nq, nkv, hd, dff, scale=0.3)
    x = g.standard_normal((1, 6, d))
    pos = np.arange(6)[None, :]
    y_st, inter = oracle.block_forward(x, w, pos, 1e4, 1e-5, nq, nkv, bf16_storage=True,
                                       return_intermediates=True)
    vis = np.broadcast_to(np.arange(6)[None, :], (1, 6))
    o_model = oracle.gqa_attention(inter["q"], inter["k"], inter["v"], vis, bf16_weights=True)
    o_exact = oracle.gqa_attention(inter["q"], inter["k"], inter["v"], vis)
    np.testing.assert_allclose(inter["o"], o_model.reshape(1, 6, -1), rtol=0, atol=0)
    assert np.abs(o_model - o_exact).max() > 0
    # one token against a cache: exact weights
    kc = np.zeros((1, 8, nkv, hd))
    vc = np.zeros((1, 8, nkv, hd))
    kc[:, :6], vc[:, :6] = inter["k"], inter["v"]
    _, i1 = oracle.block_forward(x[:, 5:6], w, pos[:, 5:6], 1e4, 1e-5, nq, nkv, kc, vc, bf16_storage=True,
                                 return_intermediates=True)
    o1 = oracle.gqa_attention(i1["q"], i1["k_cache"], i1["v_cache"], np.array([[5]]))
    np.testing.assert_allclose(i1["o"], o1.reshape(1, 1, -1), rtol=0, atol=0)


# ---------------------------------------------------------------------------
# output layer ([L3] §十): final RMSNorm, head, greedy choice
# ---------------------------------------------------------------------------
def test_greedy_token_against_scalar_loop_with_ties_and_nan():
    from oracle import head
    g = rng(60)
    lg = np.round(g.standard_normal((20, 50)) * 4) / 4       # many exact ties
    lg[3, :] = 1.0
    lg[4, 7] = np.nan
    lg[4, 9] = 100.0
    got = head.greedy_token(lg)
    for r in range(lg.shape[0]):
        best, bi = -np.inf, 0
        for c in range(lg.shape[1]):
            v = lg[r, c]
            if not np.isnan(v) and v > best:
                best, bi = v, c
        assert got[r] == bi
    assert got[3] == 0 and got[4] == 9


def test_lm_head_planted_maximum():
    # a head row aligned with the normalized row: its logit is exactly alpha,
    # far above the others, so it is chosen; the logits are RMSNorm then the
    # [out, in] product
    from oracle import head
    g = rng(61)
    d, vocab = 64, 300
    h = g.standard_normal((3, d))
    gamma = 1.0 + 0.1 * g.standard_normal(d)
    w = 0.01 * g.standard_normal((vocab, d))
    f = oracle.rmsnorm(h, gamma, 1e-5)
    for r, v in enumerate((17, 250, 3)):
        w[v] = 30.0 * f[r] / np.dot(f[r], f[r])
    lg = head.lm_head_logits(h, gamma, w, 1e-5)
    assert lg.shape == (3, vocab)
    assert np.allclose([lg[0, 17], lg[1, 250], lg[2, 3]], 30.0)
    assert list(head.greedy_token(lg)) == [17, 250, 3]
    np.testing.assert_allclose(lg, f @ w.T)
