"""Kernel-level parity of the HIP path against the CPU oracle (needs a GPU).

Every call goes through the C ABI (ctypes binding); inputs are seeded and
identical on both sides.  Bounds for bf16 outputs follow from the arithmetic:
an fp32 result rounded once to bf16 is within 2^-8 of itself (8 significant
bits); the bf16 attention outputs are held to the per-element bound of
tests/attn_bound.py (output rounding, the prefill kernel's bf16 softmax
weights, fp32 scores and sums), checked on the CPU to reject zeroed and
slot-dropping outputs on these same inputs.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from llama_decoder_block_amd import binding, synth
from attn_bound import attn_inputs, check_attention
from metrics import BF16_ULP, max_abs, max_rel_floor, rel_frobenius, report, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev(t):
    return t.to(DEV)


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d", [16, 1000, 4096, 8192])
def test_rmsnorm_f32_with_residual(d):
    x = synth.normal(11, (37, d))
    r = synth.normal(12, (37, d))
    g = synth.normal(13, (d,), 0.1, 1.0)
    s_out = torch.empty_like(x, device=DEV)
    out = binding.rmsnorm(dev(x), dev(g), 1e-5, residual=dev(r), sum_out=s_out)
    torch.cuda.synchronize()
    s64 = to64(x) + to64(r)
    ref = oracle.rmsnorm(s64, to64(g), 1e-5)
    report(f"rmsnorm f32 d={d}", out, ref)
    assert max_rel_floor(out, ref) <= 1e-4
    assert max_abs(s_out, s64) <= 1e-6 * np.abs(s64).max()


@pytest.mark.parametrize("d", [4096, 1000])
def test_rmsnorm_bf16_out(d):
    x = synth.normal(21, (300, d)) * 3.0
    g = synth.normal(22, (d,), 0.01, 1.0, dtype="bf16")
    out = binding.rmsnorm(dev(x), dev(g), 1e-5)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    ref = oracle.rmsnorm(to64(x), to64(g), 1e-5)
    err = np.abs(to64(out) - ref)
    assert np.all(err <= BF16_ULP * np.abs(ref) + 1e-6), err.max()


def test_rmsnorm_constant_rows():
    # constant rows with unit gain: every output is c/sqrt(c^2 + eps)
    c = torch.tensor([1.0, -3.0, 100.0, 1e-3]).repeat_interleave(4096).reshape(4, 4096)
    out = binding.rmsnorm(dev(c), dev(torch.ones(4096)), 1e-5)
    torch.cuda.synchronize()
    for i, cv in enumerate([1.0, -3.0, 100.0, 1e-3]):
        np.testing.assert_allclose(to64(out[i]), cv / math.sqrt(cv * cv + 1e-5), rtol=2e-6)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hd,theta", [(128, 5e5), (128, 1e4), (64, 1e4), (256, 1e4), (12, 1e4), (2, 1e4)])
@pytest.mark.parametrize("nq,nkv", [(8, 2), (32, 8), (5, 0), (0, 3)])
def test_rope(dtype, hd, theta, nq, nkv):
    """Ragged head counts (a last group of fewer than 8 heads), Q only, K only;
    head_dim 12 and 2 take the per-pair kernels for bf16."""
    n = 333
    q = synth.normal(31, (n, nq, hd), dtype=dtype) if nq else None
    k = synth.normal(32, (n, nkv, hd), dtype=dtype) if nkv else None
    pos = torch.from_numpy(np.random.Generator(np.random.PCG64(33)).integers(0, 8192, n).astype(np.int32))
    pos[:3] = torch.tensor([0, 1, 8191], dtype=torch.int32)
    qd = dev(q) if q is not None else None
    kd = dev(k) if k is not None else None
    binding.rope(qd, kd, dev(pos), theta)
    torch.cuda.synchronize()
    for src, got, name in ((q, qd, "q"), (k, kd, "k")):
        if src is None:
            continue
        ref = oracle.rope(to64(src), to64(pos), theta)
        g = to64(got)
        pn = np.sqrt(ref[..., 0::2] ** 2 + ref[..., 1::2] ** 2)
        pair_norm = np.repeat(pn, 2, axis=-1)
        if dtype == "f32":
            bound = 2e-6 * pair_norm + 1e-7
        else:
            bound = BF16_ULP * np.abs(ref) + 2e-6 * pair_norm + 1e-7
        assert np.all(np.abs(g - ref) <= bound), (name, np.max(np.abs(g - ref) - bound))
        # position 0 leaves the vector unchanged
        np.testing.assert_array_equal(to64(got[0]), to64(src[0]))


# ---------------------------------------------------------------------------
# Attention: the worked 8Q/2KV example of "LLaMA-3 8B 现代 LLM 架构、计算规模与能耗" §4.3-4.6
# ---------------------------------------------------------------------------
def toy_example():
    from test_oracle_pins import load_toy
    return load_toy(os.path.join(os.path.dirname(__file__), "golden"))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_attention_worked_example_hd2(dtype):
    q, k, v, tabs = toy_example()
    t = math.tanh(1.0 / math.sqrt(2.0))
    expect = np.array([[t, 0], [0, t], [-t, 0], [0, -t], [2 * t, 0], [0, 2 * t], [-2 * t, 0], [0, -2 * t]])
    qd = torch.tensor(q, dtype=dtype, device=DEV)
    kd = torch.tensor(k, dtype=dtype, device=DEV)
    vd = torch.tensor(v, dtype=dtype, device=DEV)
    pos = torch.tensor([[3]], dtype=torch.int32, device=DEV)
    out = binding.gqa_attention(qd, kd, vd, pos)
    torch.cuda.synchronize()
    tol = 1e-6 if dtype == torch.float32 else 2 * BF16_ULP * 2
    np.testing.assert_allclose(to64(out[0, 0]), expect, atol=tol)
    for h in range(8):
        np.testing.assert_allclose(to64(out[0, 0, h]), tabs["out"][h], atol=5e-4 + (0 if dtype == torch.float32 else tol))


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_attention_worked_example_embedded_hd128(mode):
    """The same example embedded in head_dim 128 (zeros elsewhere, q scaled by 8
    so that q.k/sqrt(128) equals the page's q.k/sqrt(2)): runs the bf16 flash
    (prefill) or split-K (decode) kernels on exactly representable inputs."""
    q, k, v, _ = toy_example()
    hd = 128
    T = 4
    Q = np.zeros((1, T, 8, hd))
    K = np.zeros((1, T, 2, hd))
    V = np.zeros((1, T, 2, hd))
    K[..., :2] = k
    V[..., :2] = v
    Q[0, 3, :, :2] = 8.0 * q[0, 0]
    Q[0, :3, :, :2] = np.random.Generator(np.random.PCG64(5)).integers(-2, 3, (3, 8, 2))
    t = math.tanh(1.0 / math.sqrt(2.0))
    expect = np.array([[t, 0], [0, t], [-t, 0], [0, -t], [2 * t, 0], [0, 2 * t], [-2 * t, 0], [0, -2 * t]])
    bf = torch.bfloat16
    if mode == "prefill":
        out = binding.gqa_attention(torch.tensor(Q, dtype=bf, device=DEV), torch.tensor(K, dtype=bf, device=DEV),
                                    torch.tensor(V, dtype=bf, device=DEV))
        got = to64(out[0, 3])
        ref_all = oracle.gqa_attention(Q, K, V, np.arange(T)[None])
        np.testing.assert_allclose(to64(out[0]), ref_all[0], atol=2 * BF16_ULP * 2)
    else:
        out = binding.gqa_attention(torch.tensor(Q[:, 3:4], dtype=bf, device=DEV),
                                    torch.tensor(K, dtype=bf, device=DEV), torch.tensor(V, dtype=bf, device=DEV),
                                    torch.tensor([[3]], dtype=torch.int32, device=DEV))
        got = to64(out[0, 0])
    torch.cuda.synchronize()
    np.testing.assert_allclose(got[:, :2], expect, atol=2 * BF16_ULP * 2)
    assert np.all(got[:, 2:] == 0)


def positions_of(pos):
    return to64(pos).astype(np.int64)


def causal(B, T):
    return np.broadcast_to(np.arange(T), (B, T))


@pytest.mark.parametrize("nq,nkv,hd", [(8, 2, 16), (4, 4, 64), (6, 3, 2)])
def test_attention_f32_prefill(nq, nkv, hd):
    B, T = 2, 70
    q, k, v = attn_inputs(40, B, T, T, nq, nkv, hd, "f32")
    out = binding.gqa_attention(dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    ref = oracle.gqa_attention(to64(q), to64(k), to64(v), causal(B, T))
    report(f"attn f32 {nq}/{nkv} hd{hd}", out, ref)
    assert max_rel_floor(out, ref) <= 1e-4


@pytest.mark.parametrize("nq,nkv", [(8, 8), (8, 4), (8, 2), (8, 1)])
@pytest.mark.parametrize("T", [200, 64])
def test_flash_bf16(nq, nkv, T):
    B, hd = 2, 128
    q, k, v = attn_inputs(50, B, T, T, nq, nkv, hd, "bf16")
    out = binding.gqa_attention(dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    check_attention(f"flash bf16 {nq}/{nkv} T={T}", out, q, k, v, causal(B, T), bf16_weights=True)


def test_flash_bf16_every_tile_written_once():
    """Workgroup numbering of the flash kernel: three sequences and four KV
    heads (12 (sequence, KV head) pairs, not a power of two) and a ragged last
    query tile.  The output starts as NaN, so a tile that no workgroup writes
    fails the bound."""
    B, T, nq, nkv, hd = 3, 200, 8, 4, 128
    q, k, v = attn_inputs(51, B, T, T, nq, nkv, hd, "bf16")
    out = torch.full((B, T, nq, hd), float("nan"), dtype=torch.bfloat16, device="cuda")
    binding.gqa_attention(dev(q), dev(k), dev(v), out=out)
    torch.cuda.synchronize()
    check_attention("flash bf16 3 sequences", out, q, k, v, causal(B, T), bf16_weights=True)


def test_flash_bf16_positions_with_cache():
    # prefill of a chunk against a longer cache: queries at positions 100..163
    B, T, S, nq, nkv, hd = 2, 64, 300, 8, 2, 128
    q, k, v = attn_inputs(60, B, T, S, nq, nkv, hd, "bf16")
    pos = (torch.arange(T, dtype=torch.int32) + 100).repeat(B, 1)
    pos[1] += 37
    out = binding.gqa_attention(dev(q), dev(k), dev(v), dev(pos))
    torch.cuda.synchronize()
    check_attention("flash bf16 positions", out, q, k, v, positions_of(pos), bf16_weights=True)


@pytest.mark.parametrize("T", [64, 1])
def test_attention_ignores_unwritten_cache_slots(T):
    """Cache slots past every query's position may hold anything (here NaN and
    inf): they get zero weight and must not reach the output (prefill of a
    chunk, T = 64, and decode, T = 1)."""
    B, S, nq, nkv, hd = 2, 300, 8, 2, 128
    q, k, v = attn_inputs(61, B, T, S, nq, nkv, hd, "bf16")
    pos = (torch.arange(T, dtype=torch.int32) + 100).repeat(B, 1)
    pos[1] += 37
    last = int(pos.max())
    kd, vd = dev(k), dev(v)
    kd[:, last + 1:] = float("nan")
    vd[:, last + 1:] = float("inf")
    vd[0, int(pos[0].max()) + 1:] = float("nan")
    out = binding.gqa_attention(dev(q), kd, vd, dev(pos))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    check_attention(f"unwritten slots T={T}", out, q, k, v, positions_of(pos), bf16_weights=T > 1)


def test_flash_gqa_equals_mha_on_repeated_kv():
    B, T, nq, nkv, hd = 1, 192, 8, 2, 128
    q, k, v = attn_inputs(70, B, T, T, nq, nkv, hd, "bf16")
    gqa = binding.gqa_attention(dev(q), dev(k), dev(v))
    kr = dev(k).repeat_interleave(nq // nkv, dim=2).contiguous()
    vr = dev(v).repeat_interleave(nq // nkv, dim=2).contiguous()
    mha = binding.gqa_attention(dev(q), kr, vr)
    torch.cuda.synchronize()
    assert torch.equal(gqa, mha)


def test_flash_causal_future_perturbation_bitwise():
    B, T, nq, nkv, hd = 1, 256, 8, 2, 128
    q, k, v = attn_inputs(80, B, T, T, nq, nkv, hd, "bf16")
    base = binding.gqa_attention(dev(q), dev(k), dev(v))
    for t in (0, 63, 64, 130, 254):
        k2, v2 = k.clone(), v.clone()
        k2[:, t + 1:] = synth.normal(81 + t, tuple(k2[:, t + 1:].shape), dtype="bf16")
        v2[:, t + 1:] = -v2[:, t + 1:] * 3
        pert = binding.gqa_attention(dev(q), dev(k2), dev(v2))
        torch.cuda.synchronize()
        assert torch.equal(pert[:, :t + 1], base[:, :t + 1])
        assert not torch.equal(pert[:, t + 1:], base[:, t + 1:])


@pytest.mark.parametrize("nq,nkv,hd", [(32, 8, 128), (8, 8, 128), (16, 8, 128), (32, 4, 128), (16, 2, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_attention(nq, nkv, hd, dtype):
    """Visible lengths 600, 257, 1, 288 and 33: full and one-slot chunks, whole
    and partial 32-slot steps."""
    B, S = 5, 600
    q, k, v = attn_inputs(90, B, 1, S, nq, nkv, hd, dtype)
    pos = torch.tensor([[599], [256], [0], [287], [32]], dtype=torch.int32)
    out = binding.gqa_attention(dev(q), dev(k), dev(v), dev(pos))
    torch.cuda.synchronize()
    if dtype == "f32":
        ref = oracle.gqa_attention(to64(q), to64(k), to64(v), positions_of(pos))
        report(f"decode {dtype} {nq}/{nkv} hd{hd}", out, ref)
        assert max_rel_floor(out, ref) <= 1e-4
    else:
        check_attention(f"decode {dtype} {nq}/{nkv} hd{hd}", out, q, k, v, positions_of(pos), bf16_weights=False)
    # one visible slot: the output is exactly that slot's V
    np.testing.assert_array_equal(to64(out[2, 0]).reshape(nkv, nq // nkv, hd),
                                  np.repeat(to64(v[2, 0])[:, None], nq // nkv, axis=1))


def decode_kernel_used(q, k, v, pos):
    binding.profile_reset()
    binding.profile_enable(True)
    out = binding.gqa_attention(dev(q), dev(k), dev(v), dev(pos))
    torch.cuda.synchronize()
    names = binding.profile_collect()
    binding.profile_enable(False)
    return out, [n for n in names if n.startswith("attention/")]


@pytest.mark.parametrize("nq,nkv", [(24, 24), (48, 24), (32, 8), (64, 8)])
def test_decode_attention_many_sequences(nq, nkv):
    """Enough (sequence, KV head) pairs for one workgroup per pair, merged in
    LDS; ragged visible lengths (1 .. S) per sequence."""
    B, S, hd = 24, 700, 128
    q, k, v = attn_inputs(95, B, 1, S, nq, nkv, hd, "bf16")
    lens = [700, 1, 33, 64, 65, 300, 511, 512, 513, 699, 2, 31, 32, 100, 257, 640, 7, 650, 690, 350, 128, 129, 96, 97]
    pos = torch.tensor([[n - 1] for n in lens], dtype=torch.int32)
    out, used = decode_kernel_used(q, k, v, pos)
    assert used == ["attention/attn_decode_wg"]
    check_attention(f"decode wg {nq}/{nkv}", out, q, k, v, positions_of(pos), bf16_weights=False)
    one = lens.index(1)
    np.testing.assert_array_equal(to64(out[one, 0]).reshape(nkv, nq // nkv, hd),
                                  np.repeat(to64(v[one, 0])[:, None], nq // nkv, axis=1))


def test_decode_attention_decode_workload_shape():
    """The Llama-3-8B decode step's attention at full size: 64 sequences, 32
    query and 8 KV heads, each query at position 4096 of a 4097-slot cache
    ("LLaMA-3 8B 现代 LLM 架构、计算规模与能耗" §九: history plus the new token),
    on the one-workgroup-per-(sequence, KV head) kernel; every output element
    against the oracle."""
    B, S, nq, nkv, hd = 64, 4097, 32, 8, 128
    q, k, v = attn_inputs(99, B, 1, S, nq, nkv, hd, "bf16")
    pos = torch.full((B, 1), S - 1, dtype=torch.int32)
    out, used = decode_kernel_used(q, k, v, pos)
    assert used == ["attention/attn_decode_wg"]
    check_attention("decode 64 x 4097 slots", out, q, k, v, positions_of(pos), bf16_weights=False)


def test_decode_attention_few_sequences_long_cache():
    """Few pairs and a long cache: chunks spread over workgroups and merged
    through the workspace."""
    B, S, nq, nkv, hd = 2, 9000, 32, 8, 128
    q, k, v = attn_inputs(96, B, 1, S, nq, nkv, hd, "bf16")
    pos = torch.tensor([[8999], [4097]], dtype=torch.int32)
    out, used = decode_kernel_used(q, k, v, pos)
    assert used == ["attention/attn_decode_splitk"]
    check_attention("decode splitk long", out, q, k, v, positions_of(pos), bf16_weights=False)


@pytest.mark.parametrize("S", [32769, 131072])
def test_decode_attention_long_context(S):
    """One sequence at the last position of a 32769- or 131072-slot cache
    (Llama-3-8B heads; the pages tabulate caches out to about 128K tokens):
    the split over workgroups with a merge through the workspace.  The bound
    rejects an all-zero output and a dropped 32-slot step on these inputs
    (tests/test_attention_bound.py)."""
    B, nq, nkv, hd = 1, 32, 8, 128
    q, k, v = attn_inputs(97, B, 1, S, nq, nkv, hd, "bf16")
    pos = torch.tensor([[S - 1]], dtype=torch.int32)
    out, used = decode_kernel_used(q, k, v, pos)
    assert used == ["attention/attn_decode_splitk"]
    check_attention(f"decode {S} slots", out, q, k, v, positions_of(pos), bf16_weights=False)


def test_chunked_prefill_against_long_cache():
    """A 256-token chunk at positions 7936..8191 attending an 8192-slot cache
    (chunked prefill): flash kernel with positions, full and partial tiles."""
    B, T, S, nq, nkv, hd = 1, 256, 8192, 32, 8, 128
    q, k, v = attn_inputs(98, B, T, S, nq, nkv, hd, "bf16")
    pos = (torch.arange(T, dtype=torch.int32) + (S - T)).reshape(1, T)
    out = binding.gqa_attention(dev(q), dev(k), dev(v), dev(pos))
    torch.cuda.synchronize()
    check_attention("chunked prefill", out, q, k, v, positions_of(pos), bf16_weights=True)


# ---------------------------------------------------------------------------
# SwiGLU FFN (GEMMs: MFMA tiles, split-K path, VALU path)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,d,dff", [(37, 64, 96), (5, 16, 48), (70, 130, 50)])
def test_swiglu_f32(n, d, dff):
    x = synth.normal(100, (n, d))
    wg = synth.normal(101, (dff, d), 0.02)
    wu = synth.normal(102, (dff, d), 0.02)
    wd = synth.normal(103, (d, dff), 0.02)
    r = synth.normal(104, (n, d))
    out = binding.swiglu_ffn(dev(x), dev(wg), dev(wu), dev(wd), residual=dev(r))
    torch.cuda.synchronize()
    ref = to64(r) + oracle.swiglu_ffn(to64(x), to64(wg), to64(wu), to64(wd))
    report(f"swiglu f32 {n}x{d}x{dff}", out, ref)
    assert max_rel_floor(out, ref) <= 1e-4


@pytest.mark.parametrize("n,d,dff", [(300, 512, 1000), (600, 512, 1000), (64, 4096, 14336), (1, 256, 64),
                                     (1024, 4096, 2048), (2048, 4096, 11008)])
def test_swiglu_bf16(n, d, dff):
    """Includes shapes with too few 256x256 tiles for the GPU, whose K is split
    over workgroups (1024 x 4096 x 2048: gate/up in 4 splits, down in 2; the
    Llama-7B FFN at 2048 tokens: down in 2)."""
    x = synth.normal(110, (n, d), dtype="bf16")
    wg = synth.normal(111, (dff, d), 0.02, dtype="bf16")
    wu = synth.normal(112, (dff, d), 0.02, dtype="bf16")
    wd = synth.normal(113, (d, dff), 0.02, dtype="bf16")
    out = binding.swiglu_ffn(dev(x), dev(wg), dev(wu), dev(wd))
    torch.cuda.synchronize()
    args = (to64(x), to64(wg), to64(wu), to64(wd))
    ref = oracle.swiglu_ffn(*args)
    ref_st = oracle.swiglu_ffn(*args, bf16_storage=True)
    report(f"swiglu bf16 {n}x{d}x{dff} (exact)", out, ref)
    report(f"swiglu bf16 {n}x{d}x{dff} (storage)", out, ref_st)
    assert rel_frobenius(out, ref) <= 1e-2
    # against the storage-point reading: fp32 accumulation differences only,
    # plus rare one-ulp flips of the bf16 product
    scale = np.abs(ref_st).max()
    assert max_abs(out, ref_st) <= 2e-2 * scale
