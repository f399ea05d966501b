"""Block-level parity of llama_block_forward against the CPU oracle (needs a GPU).

Gates (the readings of the stated tolerances):
  * fp32 path: max relative error (floored at 1e-3 of the tensor's max) <= 1e-4;
  * bf16 path: relative Frobenius error <= 1e-2 against the exact fp64 oracle,
    and max abs error <= 5e-2 against the bf16 storage-point oracle, on the
    block output y (fp32 residual stream); the same relative Frobenius gate
    on the block's whole delta y - x and on the attention sublayer's h - x
    (h from a run with W_down = 0).
"""

import numpy as np
import pytest
import torch

import oracle
from llama_decoder_block_amd import binding, synth
from fp32_emulation import SAMPLED_ROWS, block_rows32, sublayer_report
from metrics import max_abs, max_rel_floor, rel_frobenius, report, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def to_dev(inp):
    w = {k: v.to(DEV) for k, v in inp.weights.items()}
    kc = inp.k_cache.to(DEV) if inp.k_cache is not None else None
    vc = inp.v_cache.to(DEV) if inp.v_cache is not None else None
    return inp.x.to(DEV), w, inp.positions.to(DEV), kc, vc


def run_block(inp):
    wl = inp.wl
    x, w, pos, kc, vc = to_dev(inp)
    y = binding.block_forward(x, w, pos, wl.n_q, wl.n_kv, wl.theta, wl.eps, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    return y, kc, vc


def oracle_block(inp, storage=False):
    wl = inp.wl
    f = inp.as_f64()
    return oracle.block_forward(f["x"], f["w"], f["positions"], wl.theta, wl.eps, wl.n_q, wl.n_kv,
                                f.get("k_cache"), f.get("v_cache"), bf16_storage=storage,
                                return_intermediates=True)


def gpu_h(inp):
    """The GPU's residual stream after attention, h: the block run again with
    W_down = 0, where y = h + 0 exactly."""
    inp0 = synth.make_block_inputs(inp.wl)
    inp0.weights["w_down"] = torch.zeros_like(inp0.weights["w_down"])
    h, _, _ = run_block(inp0)
    return h


def check_bf16(name, y, inp):
    """y against both oracles, and the two sublayer deltas on their own: the
    residual x dominates y (|x| ~ 1 where the attention delta's rms can be
    ~0.03), so a y-level relF alone would hardly see a wrong sublayer."""
    y_ex, inter = oracle_block(inp)
    y_st, _ = oracle_block(inp, storage=True)
    report(f"{name} vs exact", y, y_ex)
    report(f"{name} vs storage", y, y_st)
    x64 = to64(inp.x)
    h = to64(gpu_h(inp))
    h_ex = inter["h"]
    report(f"{name} delta y-x", to64(y) - x64, y_ex - x64)
    report(f"{name} attention delta h-x", h - x64, h_ex - x64)
    assert rel_frobenius(y, y_ex) <= 1e-2
    assert max_abs(y, y_st) <= 5e-2
    assert rel_frobenius(to64(y) - x64, y_ex - x64) <= 1e-2
    assert rel_frobenius(h - x64, h_ex - x64) <= 1e-2


def test_toy_block_f32():
    inp = synth.make_block_inputs(synth.workload("toy_gqa_f32"))
    y, _, _ = run_block(inp)
    y_ex, _ = oracle_block(inp)
    report("toy f32", y, y_ex)
    assert max_rel_floor(y, y_ex) <= 1e-4
    f = inp.as_f64()
    wl = inp.wl
    yb = np.array(oracle.bruteforce.block_forward(f["x"], f["w"], f["positions"], wl.theta, wl.eps, wl.n_q,
                                                  wl.n_kv))
    assert max_rel_floor(y, yb) <= 1e-4


@pytest.mark.parametrize("T", [1, 7, 130])
def test_small_block_f32(T):
    wl = synth.workload("toy_gqa_f32", batch=2, seq=T, d_model=96, n_q=6, n_kv=2, head_dim=16, d_ff=200,
                        unit_gains=False)
    inp = synth.make_block_inputs(wl)
    y, _, _ = run_block(inp)
    y_ex, _ = oracle_block(inp)
    report(f"small f32 T={T}", y, y_ex)
    assert max_rel_floor(y, y_ex) <= 1e-4


def small_bf16(**kw):
    base = dict(batch=2, seq=300, d_model=512, n_q=8, n_kv=2, head_dim=128, d_ff=1376, theta=5e5)
    base.update(kw)
    return synth.workload("llama3_8b_gqa_prefill", **base)


@pytest.mark.parametrize("kw", [dict(), dict(n_kv=8), dict(seq=600, batch=1), dict(seq=33, n_kv=1),
                                dict(n_q=6, n_kv=3, head_dim=16)])
def test_small_block_bf16(kw):
    """The last case (Q/K/V segments not on 32-row boundaries, head_dim 16)
    takes the generic MFMA GEMM and the generic attention kernel."""
    inp = synth.make_block_inputs(small_bf16(**kw))
    y, _, _ = run_block(inp)
    check_bf16(f"small bf16 {kw}", y, inp)


@pytest.mark.parametrize("name,seq", [("llama3_8b_gqa_prefill", 256), ("llama7b_mha_prefill", 160),
                                      ("llama3_8b_gqa_prefill", 1100)])
def test_model_width_block_bf16(name, seq):
    inp = synth.make_block_inputs(synth.workload(name, seq=seq))
    y, _, _ = run_block(inp)
    check_bf16(f"{name} T={seq}", y, inp)


def test_block_bf16_rdtype_bf16():
    """Residual stream in bf16 as well: reported against both oracles; the
    relative Frobenius gate still holds (the max-abs gate needs an fp32 stream)."""
    inp = synth.make_block_inputs(small_bf16(seq=64))
    x, w, pos, _, _ = to_dev(inp)
    y = binding.block_forward(x.to(torch.bfloat16), w, pos, inp.wl.n_q, inp.wl.n_kv, inp.wl.theta, inp.wl.eps)
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16
    y_ex, _ = oracle_block(inp)
    report("bf16 residual", y, y_ex)
    assert rel_frobenius(y, y_ex) <= 1e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_then_decode(dtype):
    """Prefill T tokens filling a cache, then one decode step, equals the oracle's
    decode on the same cache, and matches a (T+1)-token prefill's last row."""
    B, T, cap = 2, 40, 64
    if dtype == "f32":
        wl = synth.workload("toy_gqa_f32", batch=B, seq=T + 1, d_model=64, n_q=4, n_kv=2, head_dim=16, d_ff=96,
                            unit_gains=False)
    else:
        wl = small_bf16(batch=B, seq=T + 1)
    inp = synth.make_block_inputs(wl)
    x, w, pos, _, _ = to_dev(inp)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    kc = torch.zeros(B, cap, wl.n_kv, wl.head_dim, dtype=tdt, device=DEV)
    vc = torch.zeros_like(kc)
    y_pre = binding.block_forward(x[:, :T].contiguous(), w, pos[:, :T].contiguous(), wl.n_q, wl.n_kv, wl.theta,
                                  wl.eps, k_cache=kc, v_cache=vc)
    y_dec = binding.block_forward(x[:, T:].contiguous(), w, pos[:, T:].contiguous(), wl.n_q, wl.n_kv, wl.theta,
                                  wl.eps, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    f = inp.as_f64()
    y_full = oracle.block_forward(f["x"], f["w"], f["positions"], wl.theta, wl.eps, wl.n_q, wl.n_kv)
    got = np.concatenate([to64(y_pre), to64(y_dec)], axis=1)
    report(f"prefill+decode {dtype}", got, y_full)
    if dtype == "f32":
        assert max_rel_floor(got, y_full) <= 1e-4
    else:
        y_st = oracle.block_forward(f["x"], f["w"], f["positions"], wl.theta, wl.eps, wl.n_q, wl.n_kv,
                                    bf16_storage=True)
        assert rel_frobenius(got, y_full) <= 1e-2
        assert max_abs(got, y_st) <= 5e-2
    # untouched cache slots stay zero
    assert torch.count_nonzero(kc[:, T + 1:]) == 0


def test_prefill_into_cache_sequence_bounds_inside_tiles():
    """Three 100-token sequences prefilled into caches at positions 0..99,
    30..129 and 60..159: the 300 token rows put all three sequences in the
    first 256-row GEMM tile, with sequence boundaries inside its 32-token
    blocks, so neighbouring tokens of one block have cache rows in different
    sequences.  y against both oracles, the written cache slots against the
    oracle's rotated K and plain V, and the slots no token owns still zero."""
    B, T, cap = 3, 100, 160
    wl = small_bf16(batch=B, seq=T, d_ff=1024)
    inp = synth.make_block_inputs(wl)
    inp.positions = torch.stack([torch.arange(T, dtype=torch.int32) + off for off in (0, 30, 60)])
    x, w, pos, _, _ = to_dev(inp)
    kc = torch.zeros(B, cap, wl.n_kv, wl.head_dim, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    y = binding.block_forward(x, w, pos, wl.n_q, wl.n_kv, wl.theta, wl.eps, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    f = inp.as_f64()
    z = np.zeros((B, cap, wl.n_kv, wl.head_dim))
    y_ex, inter = oracle.block_forward(f["x"], f["w"], f["positions"], wl.theta, wl.eps, wl.n_q, wl.n_kv, z, z,
                                       return_intermediates=True)
    y_st = oracle.block_forward(f["x"], f["w"], f["positions"], wl.theta, wl.eps, wl.n_q, wl.n_kv, z, z,
                                bf16_storage=True)
    report("prefill into cache, 3 x 100 tokens", y, y_ex)
    x64 = to64(inp.x)
    assert rel_frobenius(y, y_ex) <= 1e-2
    assert max_abs(y, y_st) <= 5e-2
    assert rel_frobenius(to64(y) - x64, y_ex - x64) <= 1e-2
    written = np.zeros((B, cap), dtype=bool)
    for b in range(B):
        written[b, inp.positions[b].numpy()] = True
    for got, want in ((kc, inter["k_cache"]), (vc, inter["v_cache"])):
        g = to64(got.cpu())
        assert rel_frobenius(g[written], want[written]) <= 1e-2
        assert not np.any(g[~written])


def test_decode_workload_sampled():
    """Full-size decode workload (64 sequences, cache of 4096 + 1 slots):
    all 64 outputs from the GPU, 8 sequences checked against the oracle."""
    wl = synth.workload("llama3_8b_gqa_decode")
    inp = synth.make_block_inputs(wl)
    y, kc, vc = run_block(inp)
    sel = [0, 9, 18, 27, 36, 45, 54, 63]
    f = inp.as_f64()
    sub = lambda a: a[sel]
    args = (sub(f["x"]), f["w"], sub(f["positions"]), wl.theta, wl.eps, wl.n_q, wl.n_kv,
            sub(f["k_cache"]), sub(f["v_cache"]))
    y_ex, inter = oracle.block_forward(*args, return_intermediates=True)
    y_st = oracle.block_forward(*args, bf16_storage=True)
    got = to64(y)[sel]
    h = to64(gpu_h(inp))[sel]
    x_sel = sub(f["x"])
    report("decode full vs exact", got, y_ex)
    report("decode full vs storage", got, y_st)
    report("decode full delta", got - x_sel, y_ex - x_sel)
    report("decode attention delta h-x", h - x_sel, inter["h"] - x_sel)
    assert rel_frobenius(got, y_ex) <= 1e-2
    assert max_abs(got, y_st) <= 5e-2
    assert rel_frobenius(got - x_sel, y_ex - x_sel) <= 1e-2
    assert rel_frobenius(h - x_sel, inter["h"] - x_sel) <= 1e-2
    # slot 4096 now holds the new rotated k and v; earlier slots untouched
    assert torch.equal(kc[:, :4096].cpu(), inp.k_cache[:, :4096])
    assert torch.count_nonzero(kc[:, 4096]) > 0


@pytest.mark.parametrize("d,n_q,n_kv,batch", [(1024, 8, 2, 64), (1024, 8, 2, 1), (2048, 16, 4, 33), (8192, 64, 8, 3)])
def test_decode_residual_norm_pass(d, n_q, n_kv, batch):
    """Decode rows at model widths that are multiples of 1024 (1, 2 and 8
    column chunks per lane): the O projection leaves split-K partials and one
    pass per row adds them to the residual and applies the FFN pre-norm.  The
    block output and h against both oracles, every row."""
    wl = synth.workload("llama3_8b_gqa_decode", batch=batch, d_model=d, n_q=n_q, n_kv=n_kv, head_dim=128,
                        d_ff=1536, decode_pos=70, kv_cap=96)
    inp = synth.make_block_inputs(wl)
    y, _, _ = run_block(inp)
    check_bf16(f"decode d={d} B={batch}", y, inp)


@pytest.mark.parametrize("d,n_q,n_kv,batch", [(6144, 48, 8, 40), (4096, 32, 32, 8)])
def test_decode_qkv_without_k_split(d, n_q, n_kv, batch):
    """Decode rows whose Q/K/V product has too few 64-row weight blocks to
    fill the GPU but enough 32-row ones: 40 rows of a GQA product with 8192
    weight rows (256 workgroups), and 8 rows of a multi-head one with 12288
    (384 workgroups, the target for at most 32 rows).  The product runs
    unsplit on 32-row blocks, with the rotation and the cache append in its
    own epilogue.  Block output and h against both oracles, every row, and
    the appended cache slot against the oracle's."""
    wl = synth.workload("llama3_8b_gqa_decode", batch=batch, d_model=d, n_q=n_q, n_kv=n_kv, head_dim=128,
                        d_ff=1536, decode_pos=70, kv_cap=96)
    inp = synth.make_block_inputs(wl)
    y, kc, _ = run_block(inp)
    check_bf16(f"decode QKV on 32-row blocks d={d} B={batch}", y, inp)
    _, inter = oracle_block(inp)
    new_k = to64(kc[:, 70])
    assert rel_frobenius(new_k, inter["k_cache"][:, 70]) <= 1e-2
    assert torch.equal(kc[:, 71:].cpu(), inp.k_cache[:, 71:])


def test_prefill_workload_sampled_rows():
    """Full Llama-3-8B prefill (T = 8192): sampled rows against the oracle."""
    wl = synth.workload("llama3_8b_gqa_prefill")
    inp = synth.make_block_inputs(wl)
    y, _, _ = run_block(inp)
    rows = [(0, 0), (0, 1), (0, 63), (0, 64), (0, 1000), (0, 4095), (0, 4096), (0, 8190), (0, 8191)]
    f = inp.as_f64()
    args = (f["x"], f["w"], f["positions"], rows, wl.theta, wl.eps, wl.n_q, wl.n_kv)
    y_ex, h_ex = oracle.block_forward_rows(*args)
    y_st, _ = oracle.block_forward_rows(*args, bf16_storage=True)
    got = np.stack([to64(y[b, t]) for b, t in rows])
    del y
    h_all = gpu_h(inp)
    h = np.stack([to64(h_all[b, t]) for b, t in rows])
    del h_all
    x_rows = np.stack([f["x"][b, t] for b, t in rows])
    report("prefill full vs exact", got, y_ex)
    report("prefill full vs storage", got, y_st)
    report("prefill full delta", got - x_rows, y_ex - x_rows)
    report("prefill attention delta h-x", h - x_rows, h_ex - x_rows)
    assert rel_frobenius(got, y_ex) <= 1e-2
    assert max_abs(got, y_st) <= 5e-2
    assert rel_frobenius(got - x_rows, y_ex - x_rows) <= 1e-2
    assert rel_frobenius(h - x_rows, h_ex - x_rows) <= 1e-2


def test_tp8_shard_sampled_rows():
    """One GPU's share of the Llama-3-8B prefill under 8-way tensor
    parallelism (4 query heads, 1 KV head, d_ff 1792, T = 8192): the QKV
    product (N = 768, K split over workgroups), o at K = 512 and the FFN at
    d_ff 1792, sampled rows against the oracle with the sublayer gates."""
    wl = synth.workload("llama3_8b_gqa_prefill", n_q=4, n_kv=1, d_ff=1792)
    inp = synth.make_block_inputs(wl)
    y, _, _ = run_block(inp)
    rows = [(0, 0), (0, 63), (0, 64), (0, 4095), (0, 4096), (0, 8191)]
    f = inp.as_f64()
    args = (f["x"], f["w"], f["positions"], rows, wl.theta, wl.eps, wl.n_q, wl.n_kv)
    y_ex, h_ex = oracle.block_forward_rows(*args)
    y_st, _ = oracle.block_forward_rows(*args, bf16_storage=True)
    got = np.stack([to64(y[b, t]) for b, t in rows])
    del y
    h_all = gpu_h(inp)
    h = np.stack([to64(h_all[b, t]) for b, t in rows])
    del h_all
    x_rows = np.stack([f["x"][b, t] for b, t in rows])
    report("tp8 shard vs exact", got, y_ex)
    report("tp8 shard vs storage", got, y_st)
    report("tp8 shard attention delta h-x", h - x_rows, h_ex - x_rows)
    assert rel_frobenius(got, y_ex) <= 1e-2
    assert max_abs(got, y_st) <= 5e-2
    assert rel_frobenius(got - x_rows, y_ex - x_rows) <= 1e-2
    assert rel_frobenius(h - x_rows, h_ex - x_rows) <= 1e-2


_mha_cache = {}


def mha_sampled(name):
    """GPU block output and oracle values (exact and storage-point) at the
    sampled rows of a full-size MHA prefill workload (computed once per
    workload), with the GPU's h at those rows from a second run with
    W_down = 0 (then y = h + 0 exactly) and the sublayer errors of the GPU
    path and of the fp32-accumulation emulation (tests/fp32_emulation.py)
    against the storage-point oracle."""
    if name not in _mha_cache:
        wl = synth.workload(name)
        inp = synth.make_block_inputs(wl)
        rows = SAMPLED_ROWS[name]
        y, _, _ = run_block(inp)
        got = np.stack([to64(y[b, t]) for b, t in rows])
        del y
        inp0 = synth.make_block_inputs(wl)
        inp0.weights["w_down"] = torch.zeros_like(inp0.weights["w_down"])
        h, _, _ = run_block(inp0)
        h_gpu = np.stack([to64(h[b, t]) for b, t in rows])
        del h, inp0
        torch.cuda.empty_cache()
        f = inp.as_f64()
        args = (f["x"], f["w"], f["positions"], rows, wl.theta, wl.eps, wl.n_q, wl.n_kv)
        y_ex, h_ex = oracle.block_forward_rows(*args)
        y_st, h_st = oracle.block_forward_rows(*args, bf16_storage=True)
        x_rows = np.stack([f["x"][b, t] for b, t in rows])
        report(f"{name} full vs exact", got, y_ex)
        report(f"{name} full vs storage", got, y_st)
        report(f"{name} full delta", got - x_rows, y_ex - x_rows)
        gpu_rep = sublayer_report(got, h_gpu, y_st, h_st, x_rows, f["w"], wl.eps)
        y32, h32 = block_rows32(*args)
        emu_rep = sublayer_report(y32, h32, y_st, h_st, x_rows, f["w"], wl.eps)
        for k in gpu_rep:
            print(f"[{name} sublayers] {k}: gpu {gpu_rep[k]:.4f}  fp32 emulation {emu_rep[k]:.4f}", flush=True)
        del inp, f
        _mha_cache.clear()
        _mha_cache[name] = dict(got=got, y_ex=y_ex, y_st=y_st, x_rows=x_rows, h_gpu=h_gpu, h_ex=h_ex,
                                gpu=gpu_rep, emu=emu_rep)
    return _mha_cache[name]


@pytest.mark.parametrize("name", ["llama7b_mha_prefill", "llama65b_mha_prefill"])
def test_mha_workloads_sampled_rows(name):
    """The two MHA prefill workloads at full size (Llama-7B: T = 2048, d = 4096,
    32 heads, d_ff = 11008; Llama-65B: 4 x 2048 tokens, d = 8192, 64 heads,
    d_ff = 22016), run as the block entry point runs them; sampled rows of
    every sequence against the exact oracle (relF of y, of the sublayer
    contribution y - x and of the attention sublayer h - x)."""
    r = mha_sampled(name)
    got, y_ex, x_rows = r["got"], r["y_ex"], r["x_rows"]
    assert rel_frobenius(got, y_ex) <= 1e-2
    assert rel_frobenius(got - x_rows, y_ex - x_rows) <= 1e-2
    assert rel_frobenius(r["h_gpu"] - x_rows, r["h_ex"] - x_rows) <= 1e-2
    if name == "llama7b_mha_prefill":
        assert max_abs(got, r["y_st"]) <= 5e-2


def test_mha65b_error_is_the_fp32_accumulation_floor():
    """On the Llama-65B rows the GPU's distance from the storage-point oracle
    is what any bf16 path with fp32 accumulation reaches: the fp32 emulation
    (tests/fp32_emulation.py, same storage points, float32 sums) lands within
    1.5x of it on y and on the attention sublayer h, and the GPU's FFN given
    its own h is no worse than the emulation's."""
    r = mha_sampled("llama65b_mha_prefill")
    gpu, emu = r["gpu"], r["emu"]
    assert gpu["y"] <= 1.5 * emu["y"]
    assert gpu["attention_sublayer_h"] <= 1.5 * emu["attention_sublayer_h"]
    assert gpu["ffn_sublayer_from_own_h"] <= 1.5 * emu["ffn_sublayer_from_own_h"] + 1e-3


@pytest.mark.xfail(strict=True, reason=(
    "max abs 5e-2 against the storage-point oracle is below the fp32-accumulation floor at d = 8192 / "
    "d_ff = 22016: `python tests/fp32_emulation.py llama65b_mha_prefill` (the same storage points with "
    "float32 sums) differs by 0.134 at these rows (attention sublayer h 0.016; the FFN, rms 6.3, turns "
    "h differences into bf16 flips of f and of the SwiGLU product); the GPU measures 0.149 (h 0.016)"))
def test_mha65b_max_abs_gate():
    r = mha_sampled("llama65b_mha_prefill")
    assert max_abs(r["got"], r["y_st"]) <= 5e-2


def test_decode_step_graph_replay():
    """One decode step captured in a HIP graph and replayed several times, with
    eager work and synchronisations in between: every replay gives the eager
    result bit for bit (the step only launches kernels: no memsets)."""
    B, T, cap = 4, 40, 64
    wl = small_bf16(batch=B, seq=T + 1)
    inp = synth.make_block_inputs(wl)
    x, w, pos, _, _ = to_dev(inp)
    kc = torch.zeros(B, cap, wl.n_kv, wl.head_dim, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    args = (w, wl.n_q, wl.n_kv, wl.theta, wl.eps)
    binding.block_forward(x[:, :T].contiguous(), w, pos[:, :T].contiguous(), wl.n_q, wl.n_kv, wl.theta, wl.eps,
                          k_cache=kc, v_cache=vc)
    xd, pd = x[:, T:].contiguous(), pos[:, T:].contiguous()
    need = binding.block_workspace_bytes(B, 1, wl.d_model, wl.n_q, wl.n_kv, wl.head_dim, wl.d_ff, cap,
                                         binding.BF16, binding.F32)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y_eager = torch.empty_like(xd)
    binding.block_forward(xd, w, pd, *args[1:], k_cache=kc, v_cache=vc, y=y_eager, workspace=ws)
    torch.cuda.synchronize()
    y_graph = torch.empty_like(xd)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        binding.block_forward(xd, w, pd, *args[1:], k_cache=kc, v_cache=vc, y=y_graph, workspace=ws)
    for i in range(4):
        y_graph.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph, y_eager), f"replay {i}"
        del junk


@pytest.mark.parametrize("seq", [300, 1])
def test_block_on_a_side_stream(seq):
    """The library enqueues on the caller's stream: the block run on a second
    stream (default priority) gives the default-stream result bit for bit,
    for a prefill and for a decode step against a cache."""
    if seq == 1:
        wl = synth.workload("llama3_8b_gqa_decode", batch=5, d_model=512, n_q=8, n_kv=2, head_dim=128, d_ff=1376,
                            decode_pos=70, kv_cap=96)
    else:
        wl = small_bf16(seq=seq)
    inp = synth.make_block_inputs(wl)
    x, w, pos, kc, vc = to_dev(inp)
    caches = lambda: (kc.clone() if kc is not None else None, vc.clone() if vc is not None else None)
    k0, v0 = caches()
    k1, v1 = caches()
    y0 = binding.block_forward(x, w, pos, wl.n_q, wl.n_kv, wl.theta, wl.eps, k_cache=k0, v_cache=v0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        y1 = binding.block_forward(x, w, pos, wl.n_q, wl.n_kv, wl.theta, wl.eps, k_cache=k1, v_cache=v1)
    side.synchronize()
    assert torch.equal(y0, y1)
    if k0 is not None:
        assert torch.equal(k0, k1) and torch.equal(v0, v1)
