"""Throughput of the Llama decoder-block forward on one MI355X.

Default run (python bench.py): W warm-up steps, then K timed steps of the
Llama-3-8B-shaped prefill block forward (B=1, T=8192, d=4096, 32/8 heads,
hd=128, d_ff=14336, theta=5e5, bf16 operands, fp32 residual stream), followed
by the same protocol for the Llama-3-8B-shaped decode step (64 sequences, one
token each at position 4096 against a 4097-slot bf16 KV cache).  Inputs are
seeded synthetic tensors already resident in device memory.  Prints one JSON
line (rank 0).

value      = prefill block-forward TFLOP/s (algorithmic FLOPs: linear layers
             plus causal attention pairs) over the K timed steps, which run
             back to back between two synchronizations
roofline   = the dominant kernel (fused gate/up GEMM + SiLU product):
             algorithmic FLOPs per launch / its average launch time, measured
             with HIP events recorded on the kernel's stream inside the timed
             region; traffic = its HBM bytes per launch from two rocprofv3
             counter passes (FETCH_SIZE, WRITE_SIZE) run by this script on the
             same kernel, calibrated by a plain 1 GiB copy in the same passes
mha_prefill = the Llama-7B and Llama-65B MHA prefill workloads, timed like
             the headline prefill, against their 60%-of-peak target times
tp8_shard_prefill = one GPU's share of the headline prefill under 8-way
             tensor parallelism (4 query heads, 1 KV head, d_ff 1792), the
             all-reduces left out
kernels    = every timed step of the path: launches, average time, and the
             achieved TFLOP/s (GEMMs, attention) or GB/s (norms)
decode     = the decode step (1 GiB read between steps so that weights and
             cache come from HBM), replayed from a HIP graph captured once:
             tokens/s and time per step; the per-kernel table and the decode
             attention's achieved GB/s against the HBM peak come from the same
             step run eagerly with per-kernel events (eager_ms_per_step)
cpu_baseline = the CPU oracle (numpy fp64) on a bounded sample of the same
             prefill workload: the first --cpu-tokens tokens of the sequence
"""

import argparse
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from llama_decoder_block_amd import binding, synth  # noqa: E402
from llama_decoder_block_amd import workmodel as wm  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16
HBM_PEAK_GBS = 8000.0

PREFILL = "llama3_8b_gqa_prefill"
DECODE = "llama3_8b_gqa_decode"
DOMINANT = "gate_up_silu/gemm_mfma_gate_up_silu"
DECODE_ATTN = "attention/attn_decode_wg"
PREFILL_TP8 = {"n_q": 4, "n_kv": 1, "d_ff": 1792}  # one GPU's share of 8-way tensor parallelism
MHA_TARGET_MS = {"llama7b_mha_prefill": 0.572, "llama65b_mha_prefill": 8.966}  # 60% of the bf16 MFMA peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def shape_of(wl):
    return wm.Shape(wl.d_model, wl.n_q, wl.n_kv, wl.head_dim, wl.d_ff)


def prepare(wl, dev):
    inp = synth.make_block_inputs(wl)
    w = {k: v.to(dev) for k, v in inp.weights.items()}
    x = inp.x.to(dev)
    pos = inp.positions.to(dev)
    kc = inp.k_cache.to(dev) if inp.k_cache is not None else None
    vc = inp.v_cache.to(dev) if inp.v_cache is not None else None
    kv_cap = kc.shape[1] if kc is not None else 0
    hd = wl.head_dim
    need = binding.block_workspace_bytes(wl.batch, wl.seq, wl.d_model, wl.n_q, wl.n_kv, hd, wl.d_ff, kv_cap,
                                         binding.BF16, binding.F32)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)

    def step():
        binding.block_forward(x, w, pos, wl.n_q, wl.n_kv, wl.theta, wl.eps, k_cache=kc, v_cache=vc, y=y,
                              workspace=ws)
    return step, inp


def time_steps(step, steps, warmup, flush=None):
    """W untimed steps, then K timed steps with per-kernel events on.  Each step
    is bracketed by its own pair of events; with `flush` (a callable that
    evicts the 256 MB last-level cache) the flush runs between steps,
    outside every step's events, and the total is the sum of the steps."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    binding.profile_reset()
    binding.profile_enable(True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        if flush is not None:
            flush()
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    binding.profile_enable(False)
    kernels = binding.profile_collect()
    per = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    if flush is None:
        ms = ev[0][0].elapsed_time(ev[-1][1]) / steps
    else:
        ms = sum(per) / steps
    return ms, per, kernels


def kernel_table(kernels, work):
    """avg time per launch and the achieved rate of each timed step."""
    rows = {}
    for key, (n, t) in sorted(kernels.items(), key=lambda kv: -kv[1][1]):
        avg_us = t / n * 1e3
        step_name = key.split("/")[0]
        flops, nbytes = work.get(step_name, (0, 0))
        row = {"launches": n, "avg_us": round(avg_us, 2)}
        if flops and flops / max(nbytes, 1) > 50:
            tf = flops / (avg_us * 1e-6) / 1e12
            row.update({"tflops": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        elif nbytes:
            gbs = nbytes / (avg_us * 1e-6) / 1e9
            row.update({"gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
        rows[key] = row
    return rows


def cpu_baseline(tokens):
    """The oracle (plain numpy fp64) on the first `tokens` tokens of the prefill
    workload: a causal prefix is itself a complete prefill of that length."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max((i.get("num_threads", 1) for i in pools), default=1)
        blas = ",".join(sorted({str(i.get("internal_api")) for i in pools})) or "unknown"
    except Exception:  # pragma: no cover
        threads, blas = len(os.sched_getaffinity(0)), "unknown"
    wl = synth.workload(PREFILL, seq=tokens)
    inp = synth.make_block_inputs(wl)
    f = inp.as_f64()
    t0 = time.perf_counter()
    oracle.block_forward(f["x"], f["w"], f["positions"], wl.theta, wl.eps, wl.n_q, wl.n_kv)
    dt = time.perf_counter() - t0
    flops = wm.prefill_flops(shape_of(wl), wl.batch, wl.seq)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"numpy fp64 block forward of the first {tokens} of the {synth.workload(PREFILL).seq} "
                      f"tokens of the Llama-3-8B prefill (same seeded inputs), one pass, {dt:.1f} s, BLAS {blas}"}


def device_info():
    """Agent name, compute units and peak clock from rocminfo (run before this
    process touches the GPU; a child process, never an exec)."""
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except Exception as e:  # pragma: no cover
        return {"error": f"rocminfo: {e}"}
    for blk in out.split("Agent ")[1:]:
        if not re.search(r"Device Type:\s+GPU", blk):
            continue
        def field(name):
            m = re.search(name + r":[ \t]*([^\n]*)", blk)
            return m.group(1).strip() if m and m.group(1).strip() else None
        cu, clk = field("Compute Unit"), field(r"Max Clock Freq\. \(MHz\)")
        return {"name": field("Name"),
                "compute_units": int(cu) if cu and cu.isdigit() else cu,
                "max_clock_mhz": int(clk) if clk and clk.isdigit() else clk}
    return {"error": "no GPU agent in rocminfo"}


def vendor_gemm(dev, warmup=3, reps=20):
    """Yardstick only: the vendor library's bf16 GEMM (torch.matmul, plain
    bf16 output, no epilogue) on the block's prefill shapes, M = 8192 tokens
    against [N, K] weights stored K-contiguous as the block stores them.  No
    step of the block runs through it."""
    for n, k, name in ((28672, 4096, "gate/up"), (6144, 4096, "QKV"), (4096, 4096, "o"), (4096, 14336, "down")):
        a = torch.randn(8192, k, device=dev, dtype=torch.bfloat16)
        w = torch.randn(n, k, device=dev, dtype=torch.bfloat16)
        for _ in range(warmup):
            torch.matmul(a, w.t())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, w.t())
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        log(f"[bench] vendor GEMM {name} M=8192 N={n} K={k}: {us:.1f} us = {2 * 8192 * n * k / us / 1e6:.0f} TFLOP/s")
        del a, w


def copy_bandwidth(dev, reps=10):
    """A plain 1 GiB device copy (1 GiB read + 1 GiB written), timed with
    events: the measured HBM rate, reported beside the 8 TB/s specification."""
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * src.numel() * 4 / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    log(f"[bench] device copy 1 GiB: {ms * 1e3:.1f} us = {gbs:.0f} GB/s")
    return {"bytes_per_copy": 2 * (1 << 30), "us": round(ms * 1e3, 1), "gbs": round(gbs, 1),
            "frac_of_spec": round(gbs / HBM_PEAK_GBS, 4)}


def bench_rope(wl, dev, args):
    """The standalone RoPE entry point on the prefill's Q and K
    ([T, n_q, hd] and [T, n_kv, hd] bf16, positions 0..T-1), rotated in
    place: HBM-bound, each element read and written once."""
    T, nq, nkv, hd = wl.batch * wl.seq, wl.n_q, wl.n_kv, wl.head_dim
    q = synth.normal(1000 * wl.index + 90, (T, nq, hd), dtype="bf16").to(dev)
    k = synth.normal(1000 * wl.index + 91, (T, nkv, hd), dtype="bf16").to(dev)
    pos = torch.arange(T, dtype=torch.int32, device=dev)
    # Q and K (84 MB) would fit in the 256 MB last-level cache: a 1 GiB read
    # between calls makes every call stream from HBM
    scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    ms, _, kernels = time_steps(lambda: binding.rope(q, k, pos, wl.theta), 20, args.warmup,
                                flush=lambda: scratch.sum())
    nbytes = 2 * (q.numel() + k.numel()) * q.element_size()
    n, t = kernels.get("rope", (0, 0.0))
    avg_us = t / n * 1e3 if n else ms * 1e3  # the library's own events around the launch
    gbs = nbytes / (avg_us * 1e-6) / 1e9
    log(f"[bench] standalone RoPE on Q [{T},{nq},{hd}] + K [{T},{nkv},{hd}] bf16: {ms * 1e3:.1f} us per call "
        f"= {gbs:.0f} GB/s (event-timed inside the library: {avg_us:.1f} us)")
    del q, k, pos, scratch
    torch.cuda.empty_cache()
    return {"workload": f"RoPE in place on Q [{T},{nq},{hd}] and K [{T},{nkv},{hd}] bf16, positions 0..{T - 1}, "
                        f"theta {wl.theta:g}, last-level cache flushed between calls",
            "us_per_call": round(ms * 1e3, 2), "bytes": nbytes, "bound": "hbm", "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "kernel_avg_us": round(avg_us, 2)}


def seeded_cache(shape, seed, dev):
    """bf16 K or V cache drawn on the GPU from N(0, 1) with a seeded generator."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)


def bench_chunked_prefill(wl, dev, args, history=24576):
    """A prefill chunk against an existing cache: the workload's 8192 tokens at
    positions history..history+8191, attending the `history` cached slots and
    themselves (causally), through the block entry point with the cache."""
    inp = synth.make_block_inputs(wl)
    w = {k: v.to(dev) for k, v in inp.weights.items()}
    x = inp.x.to(dev)
    B, T = wl.batch, wl.seq
    cap = history + T
    pos = (history + torch.arange(T, dtype=torch.int32)).repeat(B, 1).to(dev)
    kc = seeded_cache((B, cap, wl.n_kv, wl.head_dim), 1000 * wl.index + 60, dev)
    vc = seeded_cache((B, cap, wl.n_kv, wl.head_dim), 1000 * wl.index + 61, dev)
    need = binding.block_workspace_bytes(B, T, wl.d_model, wl.n_q, wl.n_kv, wl.head_dim, wl.d_ff, cap,
                                         binding.BF16, binding.F32)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)

    def step():
        binding.block_forward(x, w, pos, wl.n_q, wl.n_kv, wl.theta, wl.eps, k_cache=kc, v_cache=vc, y=y,
                              workspace=ws)
    ms, per, kernels = time_steps(step, args.steps, args.warmup)
    sh = shape_of(wl)
    att = wm.chunk_attention_flops(sh, B, T, history)
    flops = wm.prefill_linear_flops(sh, B * T) + att
    n_at, ms_at = kernels.get("attention/attn_flash_prefill", (0, 0.0))
    at_us = ms_at / max(n_at, 1) * 1e3
    log(f"[bench] chunked prefill ({T} tokens after {history} cached): {ms:.3f} ms/step, "
        f"{flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s; attention {at_us:.1f} us = {att / (at_us * 1e-6) / 1e12:.1f} TFLOP/s")
    out = {"workload": f"{PREFILL} tokens as one chunk at positions {history}..{cap - 1} against a bf16 cache of "
                       f"{history} earlier slots [{B},{cap},{wl.n_kv},{wl.head_dim}]",
           "ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "attention": {"avg_us": round(at_us, 2), "flops": att,
                         "tflops": round(att / (at_us * 1e-6) / 1e12, 1) if n_at else None},
           "kernels": kernel_table(kernels, wm.step_work(sh, B, T, history=history))}
    del step, w, x, kc, vc, ws, y
    torch.cuda.empty_cache()
    return out


def bench_long_decode(wd, dev, args, batch=8, position=32767):
    """The decode step for `batch` sequences at `position` (a 32K-slot cache):
    few (sequence, KV head) pairs, so decode attention splits each history
    over workgroups and merges the chunks."""
    small = synth.workload(DECODE, batch=batch, decode_pos=0, kv_cap=1)
    inp = synth.make_block_inputs(small)
    w = {k: v.to(dev) for k, v in inp.weights.items()}
    x = inp.x.to(dev)
    cap = position + 1
    kc = seeded_cache((batch, cap, wd.n_kv, wd.head_dim), 1000 * wd.index + 70, dev)
    vc = seeded_cache((batch, cap, wd.n_kv, wd.head_dim), 1000 * wd.index + 71, dev)
    pos = torch.full((batch, 1), position, dtype=torch.int32, device=dev)
    need = binding.block_workspace_bytes(batch, 1, wd.d_model, wd.n_q, wd.n_kv, wd.head_dim, wd.d_ff, cap,
                                         binding.BF16, binding.F32)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)

    def step():
        binding.block_forward(x, w, pos, wd.n_q, wd.n_kv, wd.theta, wd.eps, k_cache=kc, v_cache=vc, y=y,
                              workspace=ws)
    scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    dms, _, dk = time_steps(step, args.decode_steps, args.warmup, flush=lambda: scratch.sum())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    gms, gper, _ = time_steps(graph.replay, args.decode_steps, args.warmup, flush=lambda: scratch.sum())
    del scratch, graph
    sh = shape_of(wd)
    at_bytes = wm.decode_attention_bytes(sh, batch, cap)
    name = next((k for k in dk if k.startswith("attention/")), None)
    n_at, ms_at = dk.get(name, (0, 0.0))
    at_us = ms_at / max(n_at, 1) * 1e3
    gbs = at_bytes / (at_us * 1e-6) / 1e9 if n_at else 0.0
    log(f"[bench] long-context decode ({batch} sequences at position {position}): {gms * 1e3:.1f} us/step in a "
        f"graph; attention ({name}) {at_us:.1f} us = {gbs:.0f} GB/s")
    out = {"workload": f"{DECODE} step for {batch} sequences at position {position}, bf16 cache "
                       f"[{batch},{cap},{wd.n_kv},{wd.head_dim}], last-level cache flushed between steps",
           "ms_per_step": round(gms, 4), "tokens_per_s": round(batch / (gms * 1e-3), 1),
           "eager_ms_per_step": round(dms, 4),
           "attention": {"kernel": name, "bound": "hbm", "avg_us": round(at_us, 2), "bytes": at_bytes,
                         "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    del step, w, x, kc, vc, ws, y
    torch.cuda.empty_cache()
    return out


def bench_decode_fp8kv(wd, dev, args):
    """The decode workload against an 8-bit KV cache (E4M3 codes + one fp32
    scale per row) holding the same synthetic history, quantized on the GPU by
    the library's cache writer; timed like the bf16 decode step."""
    inp = synth.make_block_inputs(wd)
    w = {k: v.to(dev) for k, v in inp.weights.items()}
    x = inp.x.to(dev)
    pos = inp.positions.to(dev).reshape(-1)
    B, cap, nkv, hd = wd.batch, wd.kv_cap, wd.n_kv, wd.head_dim
    k8, v8, ks, vs = binding.fp8_cache(B, cap, nkv, hd, dev)
    hist = torch.arange(wd.decode_pos, dtype=torch.int32, device=dev).repeat(B, 1)
    kc, vc = inp.k_cache.to(dev), inp.v_cache.to(dev)
    binding.kv_append_fp8(kc[:, :wd.decode_pos].contiguous(), vc[:, :wd.decode_pos].contiguous(), hist,
                          k8, v8, ks, vs)
    del kc, vc
    need = binding.block_fp8kv_workspace_bytes(B, wd.d_model, wd.n_q, nkv, hd, wd.d_ff, cap, binding.F32)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)

    def step():
        binding.block_forward_fp8kv(x, w, pos, wd.n_q, nkv, wd.theta, wd.eps, k8, v8, ks, vs, y=y, workspace=ws)
    scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    dms, _, dk = time_steps(step, args.decode_steps, args.warmup, flush=lambda: scratch.sum())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    gms, gper, _ = time_steps(graph.replay, args.decode_steps, args.warmup, flush=lambda: scratch.sum())
    del scratch, graph
    shd = shape_of(wd)
    attend = wd.decode_pos + 1
    dwork = wm.step_work(shd, B, 1, attend_len=attend, kv_bytes=wm.FP8KV_BYTES_PER_ELEM)
    table = kernel_table(dk, dwork)
    name = DECODE_ATTN + "_fp8kv"
    n_at, ms_at = dk.get(name, (0, 0.0))
    at_avg = ms_at / max(n_at, 1)
    at_bytes = dwork["attention"][1]
    at_gbs = at_bytes / (at_avg * 1e-3) / 1e9 if n_at else 0.0
    log(f"[bench] decode, 8-bit KV cache: {gms * 1e3:.1f} us/step in a graph (median "
        f"{gper[len(gper) // 2] * 1e3:.1f}); eager {dms * 1e3:.1f} us/step; attention {at_avg * 1e3:.1f} us = "
        f"{at_gbs:.0f} GB/s")
    for k, row in table.items():
        log(f"[bench]   {k:40s} {row}")
    out = {
        "workload": f"{DECODE} with an 8-bit KV cache (E4M3 codes [{B},{nkv},{cap},{hd}] + fp32 row scales "
                    f"[{B},{nkv},{cap}]), same history quantized on the GPU, last-level cache flushed between steps",
        "ms_per_step": round(gms, 4),
        "ms_median": round(gper[len(gper) // 2], 4),
        "tokens_per_s": round(B / (gms * 1e-3), 1),
        "eager_ms_per_step": round(dms, 4),
        "attention": {"kernel": name, "bound": "hbm", "avg_us": round(at_avg * 1e3, 2), "bytes": at_bytes,
                      "achieved": round(at_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(at_gbs / HBM_PEAK_GBS, 4)},
        "kernels": table,
    }
    del step, w, x, k8, v8, ks, vs, ws, y
    torch.cuda.empty_cache()
    return out


def bench_paged_attention(wd, dev, args, page_size=64):
    """Decode attention alone over the same bf16 history held in a paged cache
    (pages of 64 slots, page order shuffled), against the contiguous cache's
    kernel on the same data; the last-level cache is flushed between calls."""
    inp = synth.make_block_inputs(wd)
    B, cap, nkv, hd, nq = wd.batch, wd.kv_cap, wd.n_kv, wd.head_dim, wd.n_q
    max_pages = -(-cap // page_size)
    n_pages = B * max_pages
    g = torch.Generator().manual_seed(4000 + 12)
    table = torch.randperm(n_pages, generator=g).to(torch.int32).reshape(B, max_pages)
    kc = torch.zeros(B, max_pages * page_size, nkv, hd, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kc[:, :cap], vc[:, :cap] = inp.k_cache, inp.v_cache
    kpool = torch.empty(n_pages, page_size, nkv, hd, dtype=torch.bfloat16, device=dev)
    vpool = torch.empty_like(kpool)
    flat = table.reshape(-1).to(dev).long()
    kpool[flat] = kc.reshape(n_pages, page_size, nkv, hd).to(dev)
    vpool[flat] = vc.reshape(n_pages, page_size, nkv, hd).to(dev)
    del kc, vc
    q = synth.normal(4013, (B, 1, nq, hd), dtype="bf16").to(dev)
    pos = inp.positions.reshape(-1).to(dev)
    tab = table.to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(binding.lib().llama_gqa_attention_paged_workspace_bytes(B, max_pages, page_size, nq, nkv, hd),
                     dtype=torch.uint8, device=dev)
    scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    _, _, dk = time_steps(lambda: binding.gqa_attention_paged(q, kpool, vpool, tab, pos, out=out, workspace=ws),
                          args.decode_steps, args.warmup, flush=lambda: scratch.sum())
    name = DECODE_ATTN + "_paged"
    n_at, ms_at = dk.get(name, (0, 0.0))
    at_avg = ms_at / max(n_at, 1)
    at_bytes = wm.decode_attention_bytes(shape_of(wd), B, wd.decode_pos + 1)
    at_gbs = at_bytes / (at_avg * 1e-3) / 1e9 if n_at else 0.0
    log(f"[bench] decode attention, paged cache (pages of {page_size} slots, shuffled): {at_avg * 1e3:.1f} us = "
        f"{at_gbs:.0f} GB/s")
    del scratch, kpool, vpool
    torch.cuda.empty_cache()
    return {"workload": f"{DECODE} attention over a paged bf16 cache: pages of {page_size} slots in a pool "
                        f"[{n_pages},{page_size},{nkv},{hd}], block table [{B},{max_pages}] in shuffled order",
            "kernel": name, "bound": "hbm", "avg_us": round(at_avg * 1e3, 2), "bytes": at_bytes,
            "achieved": round(at_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(at_gbs / HBM_PEAK_GBS, 4)}


def bench_lm_head(wd, dev, args, vocab=128256):
    """The output layer after the decode step ([L3] §十): final RMSNorm, the
    [4096 -> 128256] head and argmax for the 64 sequences' last positions.
    The 1.05 GB head is drawn on the GPU by torch's seeded normal generator
    (N(0, 0.02^2), rounded to bf16); the rows are the decode workload's x."""
    inp = synth.make_block_inputs(wd)
    d = wd.d_model
    g = torch.Generator(device=dev).manual_seed(4000 + 20)
    w = (torch.randn(vocab, d, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    gamma = inp.weights["ffn_norm"].to(dev)
    h = inp.x.reshape(-1, d).to(dev)
    need = binding.lib().llama_lm_head_argmax_workspace_bytes(h.shape[0], d, vocab, binding.BF16, binding.F32)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    ms, per, dk = time_steps(lambda: binding.lm_head_argmax(h, gamma, w, wd.eps, workspace=ws), args.decode_steps,
                             args.warmup, flush=lambda: scratch.sum())
    wbytes = vocab * d * 2
    rows = {}
    for key, (n, t) in sorted(dk.items(), key=lambda kv: -kv[1][1]):
        rows[key] = {"launches": n, "avg_us": round(t / n * 1e3, 2)}
    head_key = next((k for k in dk if k.startswith("lm_head")), None)
    head_us = dk[head_key][1] / dk[head_key][0] * 1e3 if head_key else 0.0
    gbs = wbytes / (head_us * 1e-6) / 1e9 if head_us else 0.0
    log(f"[bench] output layer (final norm + head {d}->{vocab} + argmax, {h.shape[0]} rows): {ms * 1e3:.1f} us; "
        f"head GEMM {head_us:.1f} us = {gbs:.0f} GB/s")
    del w, ws, scratch
    torch.cuda.empty_cache()
    return {"workload": f"final RMSNorm + head [{vocab}, {d}] bf16 + argmax for {h.shape[0]} rows, last-level cache "
                        f"flushed between calls",
            "ms_per_call": round(ms, 4), "head_kernel": head_key, "head_avg_us": round(head_us, 2),
            "head_bytes": wbytes, "head_gbs": round(gbs, 1), "head_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "kernels": rows}


# ---------------------------------------------------------------------------
# HBM bytes per launch from two rocprofv3 counter passes (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch), each scaled by the same counter's reading for
# a plain copy of known size run in the same pass.  The passes run this file
# with --traffic-pass as a child process of the profiler.
# ---------------------------------------------------------------------------
COPY_ELEMS = 1 << 28  # fp32: the calibration copy reads 1 GiB and writes 1 GiB


def traffic_pass():
    """Child of the profiler: the prefill's gate/up GEMM (with its down GEMM,
    through the FFN entry point), the standalone RoPE on the prefill's q and
    k, an RMSNorm of the prefill's fp32 rows and the calibration copy, each
    launched three times on inputs drawn on the GPU."""
    dev = "cuda:0"
    wl = synth.workload(PREFILL)
    M, d, dff, hd = wl.batch * wl.seq, wl.d_model, wl.d_ff, wl.head_dim
    g = torch.Generator(device=dev).manual_seed(1000 * wl.index + 95)
    bf = torch.bfloat16
    f = torch.randn(M, d, generator=g, device=dev).to(bf)
    wg = (torch.randn(dff, d, generator=g, device=dev) * 0.02).to(bf)
    wu = (torch.randn(dff, d, generator=g, device=dev) * 0.02).to(bf)
    wd = (torch.randn(d, dff, generator=g, device=dev) * 0.02).to(bf)
    h = torch.randn(M, d, generator=g, device=dev)
    y = torch.empty_like(h)
    q = torch.randn(M, wl.n_q, hd, generator=g, device=dev).to(bf)
    k = torch.randn(M, wl.n_kv, hd, generator=g, device=dev).to(bf)
    pos = torch.arange(M, dtype=torch.int32, device=dev)
    gamma = (1 + 0.01 * torch.randn(d, generator=g, device=dev)).to(bf)
    normed = torch.empty(M, d, dtype=bf, device=dev)
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        binding.swiglu_ffn(f, wg, wu, wd, residual=h, out=y)
        binding.rope(q, k, pos, wl.theta)
        binding.rmsnorm(h, gamma, wl.eps, out=normed)
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print("traffic pass done", flush=True)


def _counter_pass(counter, tmp):
    """One profiled child run; returns {kernel class: [KiB per dispatch]}."""
    import csv
    rocprof = "/opt/rocm/bin/rocprofv3" if os.path.exists("/opt/rocm/bin/rocprofv3") else "rocprofv3"
    out = os.path.join(tmp, counter)
    env = dict(os.environ, TMPDIR="/tmp")
    cmd = [rocprof, "--kernel-trace", "--pmc", counter, "--output-format", "csv", "-d", out, "-o", "run", "--",
           sys.executable, os.path.abspath(__file__), "--traffic-pass"]
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True, timeout=240)
    if "traffic pass done" not in r.stdout:
        raise RuntimeError(f"{counter} pass failed (rc {r.returncode}): {r.stderr[-400:]}")
    per = {}
    with open(os.path.join(out, "run_counter_collection.csv")) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            if "gemm_mfma" in name and "<true" in name:
                cls = "gate_up"
            elif "rope_heads" in name:
                cls = "rope"
            elif "rmsnorm" in name:
                cls = "rmsnorm"
            elif "neg" in name.lower():
                cls = "copy"
            else:
                continue
            per.setdefault(cls, {}).setdefault(row["Dispatch_Id"], 0.0)
            per[cls][row["Dispatch_Id"]] += float(row["Counter_Value"])
    return {c: list(v.values()) for c, v in per.items()}


def measure_traffic(algorithmic):
    """Calibrated HBM bytes per launch of the gate/up GEMM, the standalone RoPE
    and the RMSNorm: (FETCH_SIZE x fetch_scale + WRITE_SIZE x write_scale) x
    1024 with each scale = the copy's known bytes / its own counter reading.
    `algorithmic` maps the same classes to their algorithmic bytes."""
    import tempfile
    tmp = tempfile.mkdtemp(prefix="traffic_", dir="/tmp")
    fetch, write = _counter_pass("FETCH_SIZE", tmp), _counter_pass("WRITE_SIZE", tmp)
    avg = lambda xs: sum(xs) / len(xs)
    copy_bytes = COPY_ELEMS * 4
    fs = copy_bytes / (avg(fetch["copy"]) * 1024)
    ws = copy_bytes / (avg(write["copy"]) * 1024)
    out = {"fetch_scale": round(fs, 4), "write_scale": round(ws, 4)}
    for cls, alg in algorithmic.items():
        fb = avg(fetch[cls]) * 1024 * fs
        wb = avg(write[cls]) * 1024 * ws
        out[cls] = {"bytes": int(round(fb + wb)), "fetch_bytes": int(round(fb)), "write_bytes": int(round(wb)),
                    "algorithmic_bytes": int(alg), "ratio": round((fb + wb) / alg, 3)}
    log(f"[bench] HBM traffic (counter passes): {out}")
    return out


def gpu_block_inputs(wl, dev):
    """The workload's tensors drawn on the GPU (seeded torch normals with the
    workload's distributions: x ~ N(0,1), weights N(0, 0.02^2), gains
    1 + N(0, 0.01^2)), for timing only."""
    g = torch.Generator(device=dev).manual_seed(1000 * wl.index + 80)
    bf = torch.bfloat16
    d, hd, dff, nq, nkv = wl.d_model, wl.head_dim, wl.d_ff, wl.n_q, wl.n_kv
    shapes = {"wq": (nq * hd, d), "wk": (nkv * hd, d), "wv": (nkv * hd, d), "wo": (d, nq * hd),
              "w_gate": (dff, d), "w_up": (dff, d), "w_down": (d, dff)}
    w = {n: (torch.randn(sh, generator=g, device=dev) * 0.02).to(bf) for n, sh in shapes.items()}
    for n in ("attn_norm", "ffn_norm"):
        w[n] = (1 + 0.01 * torch.randn(d, generator=g, device=dev)).to(bf)
    x = torch.randn(wl.batch, wl.seq, d, generator=g, device=dev).to(bf).float()
    pos = torch.arange(wl.seq, dtype=torch.int32, device=dev).repeat(wl.batch, 1)
    return x, w, pos


def bench_mha_prefill(name, dev, args):
    """A full-size MHA prefill workload (Llama-7B: B=1 T=2048 d=4096 32 heads
    d_ff=11008; Llama-65B: B=4 T=2048 d=8192 64 heads d_ff=22016), timed like
    the headline prefill, against the 60%-of-peak target time."""
    wl = synth.workload(name)
    x, w, pos = gpu_block_inputs(wl, dev)
    need = binding.block_workspace_bytes(wl.batch, wl.seq, wl.d_model, wl.n_q, wl.n_kv, wl.head_dim, wl.d_ff, 0,
                                         binding.BF16, binding.F32)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)

    def step():
        binding.block_forward(x, w, pos, wl.n_q, wl.n_kv, wl.theta, wl.eps, y=y, workspace=ws)
    ms, per, kernels = time_steps(step, args.steps, args.warmup)
    sh = shape_of(wl)
    flops = wm.prefill_flops(sh, wl.batch, wl.seq)
    tf = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {name}: {ms:.3f} ms/step, {tf:.1f} TFLOP/s ({tf / MFMA_BF16_PEAK_TFLOPS:.1%} of peak; "
        f"target {MHA_TARGET_MS[name]} ms)")
    table = kernel_table(kernels, wm.step_work(sh, wl.batch, wl.seq))
    for k, row in table.items():
        log(f"[bench]   {k:40s} {row}")
    out = {"workload": f"{name}: B={wl.batch} T={wl.seq} d={wl.d_model} n_q={wl.n_q} n_kv={wl.n_kv} "
                       f"hd={wl.head_dim} d_ff={wl.d_ff} theta={wl.theta:g}, weights drawn on the GPU",
           "ms_per_step": round(ms, 4), "ms_median": round(per[len(per) // 2], 4), "flops": flops,
           "tflops": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
           "tokens_per_s": round(wl.batch * wl.seq / (ms * 1e-3), 1),
           "target_ms": MHA_TARGET_MS[name], "kernels": table}
    del step, x, w, pos, ws, y
    torch.cuda.empty_cache()
    return out


def bench_tp8_shard(dev, args):
    """One GPU's share of the Llama-3-8B prefill under 8-way tensor
    parallelism by KV group: the block's kernels with 4 query heads, 1 KV
    head and d_ff = 14336 / 8 = 1792 (QKV N = 768, o K = 512, gate/up
    N = 2 x 1792, down K = 1792), at T = 8192.  The two all-reduces of [8192,
    4096] that the sharded block adds (after o and after down) are not part
    of it; this times the kernels at the shard's real shapes."""
    wl = synth.workload(PREFILL, n_q=PREFILL_TP8["n_q"], n_kv=PREFILL_TP8["n_kv"], d_ff=PREFILL_TP8["d_ff"])
    x, w, pos = gpu_block_inputs(wl, dev)
    need = binding.block_workspace_bytes(wl.batch, wl.seq, wl.d_model, wl.n_q, wl.n_kv, wl.head_dim, wl.d_ff, 0,
                                         binding.BF16, binding.F32)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)

    def step():
        binding.block_forward(x, w, pos, wl.n_q, wl.n_kv, wl.theta, wl.eps, y=y, workspace=ws)
    ms, per, kernels = time_steps(step, args.steps, args.warmup)
    sh = shape_of(wl)
    flops = wm.prefill_flops(sh, wl.batch, wl.seq)
    tf = flops / (ms * 1e-3) / 1e12
    log(f"[bench] tp8 shard of {PREFILL}: {ms:.3f} ms/step, {tf:.1f} TFLOP/s ({tf / MFMA_BF16_PEAK_TFLOPS:.1%} "
        f"of peak)")
    table = kernel_table(kernels, wm.step_work(sh, wl.batch, wl.seq))
    for k, row in table.items():
        log(f"[bench]   {k:40s} {row}")
    out = {"workload": f"{PREFILL} shard of 8-way tensor parallelism: B={wl.batch} T={wl.seq} d={wl.d_model} "
                       f"n_q={wl.n_q} n_kv={wl.n_kv} hd={wl.head_dim} d_ff={wl.d_ff} theta={wl.theta:g} "
                       f"(all-reduces not included), weights drawn on the GPU",
           "ms_per_step": round(ms, 4), "ms_median": round(per[len(per) // 2], 4), "flops": flops,
           "tflops": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "kernels": table}
    del step, x, w, pos, ws, y
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (read 1 GiB, write 1 GiB) five times: the "
                         "reference reading for scaling the HBM byte counters")
    ap.add_argument("--no-traffic", action="store_true",
                    help="skip the two rocprofv3 counter passes that measure HBM bytes")
    ap.add_argument("--traffic-pass", action="store_true",
                    help="(run by the counter passes) launch the kernels whose HBM bytes are measured, then exit")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the vendor library's plain bf16 GEMM (torch.matmul) on the block's "
                         "four prefill shapes: a yardstick for the library's own GEMM kernels")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: there is no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.traffic_pass:
        traffic_pass()
        return
    device = None if (args.copy_calibration or args.vendor_gemm) else device_info()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 5 x {src.numel() * 4} bytes read and written")
        return
    if args.vendor_gemm:
        vendor_gemm(dev)
        return
    binding.lib()
    if device is not None:
        log(f"[bench] device: {device}")
    copy_bw = copy_bandwidth(dev)

    # ---------------- prefill -----------------
    wl = synth.workload(PREFILL)
    log(f"[bench] preparing {PREFILL}")
    step, _ = prepare(wl, dev)
    log(f"[bench] prefill: warmup {args.warmup}, timing {args.steps} steps")
    ms, per, kernels = time_steps(step, args.steps, args.warmup)
    sh = shape_of(wl)
    flops = wm.prefill_flops(sh, wl.batch, wl.seq)
    tflops = flops / (ms * 1e-3) / 1e12
    tok_s = wl.batch * wl.seq / (ms * 1e-3)
    work = wm.step_work(sh, wl.batch, wl.seq)
    table = kernel_table(kernels, work)
    n_dom, ms_dom = kernels.get(DOMINANT, (0, 0.0))
    dom_flops = work["gate_up_silu"][0]
    dom_avg_ms = ms_dom / max(n_dom, 1)
    dom_tflops = dom_flops / (dom_avg_ms * 1e-3) / 1e12 if n_dom else 0.0
    log(f"[bench] prefill {ms:.3f} ms/step (median {per[len(per) // 2]:.3f}, min {per[0]:.3f}), "
        f"{tflops:.1f} TFLOP/s, {tok_s / 1e6:.3f} M tok/s")
    for k, row in table.items():
        log(f"[bench]   {k:40s} {row}")
    del step
    torch.cuda.empty_cache()
    rope = bench_rope(wl, dev, args)
    chunked = bench_chunked_prefill(wl, dev, args)
    mha = {n: bench_mha_prefill(n, dev, args) for n in MHA_TARGET_MS}
    tp8 = bench_tp8_shard(dev, args)

    # ---------------- decode -----------------
    decode = None
    if not args.no_decode:
        wd = synth.workload(DECODE)
        log(f"[bench] preparing {DECODE}")
        dstep, _ = prepare(wd, dev)
        # 1 GiB read between steps so that neither weights nor cache are served
        # from the 256 MB last-level cache.  A read, not a write: written lines
        # would sit dirty in the cache and their write-back would be charged to
        # the next step.
        scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        dms, dper, dk = time_steps(dstep, args.decode_steps, args.warmup, flush=lambda: scratch.sum())
        # the same step captured once in a HIP graph and replayed: the kernels
        # run back to back without per-launch host overhead
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dstep()
        gms, gper, _ = time_steps(graph.replay, args.decode_steps, args.warmup, flush=lambda: scratch.sum())
        del scratch, graph
        shd = shape_of(wd)
        attend = wd.decode_pos + 1
        dwork = wm.step_work(shd, wd.batch, 1, attend_len=attend)
        dtable = kernel_table(dk, dwork)
        n_at, ms_at = dk.get(DECODE_ATTN, (0, 0.0))
        at_avg = ms_at / max(n_at, 1)  # split-K pass and its combine pass together
        at_bytes = dwork["attention"][1]
        at_gbs = at_bytes / (at_avg * 1e-3) / 1e9 if n_at else 0.0
        step_bytes = at_bytes + wm.decode_weight_bytes(shd)
        decode = {
            "workload": f"{DECODE}: B={wd.batch} x 1 token at position {wd.decode_pos}, KV cache "
                        f"[{wd.batch},{wd.kv_cap},{wd.n_kv},{wd.head_dim}] bf16, last-level cache flushed "
                        f"(1 GiB read) between steps",
            "ms_per_step": round(gms, 4),
            "ms_median": round(gper[len(gper) // 2], 4),
            "ms_min": round(gper[0], 4),
            "tokens_per_s": round(wd.batch / (gms * 1e-3), 1),
            "step_tflops": round(wm.decode_flops(shd, wd.batch, attend) / (gms * 1e-3) / 1e12, 3),
            "step_gbs": round(step_bytes / (gms * 1e-3) / 1e9, 1),
            "step_hbm_frac": round(step_bytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "eager_ms_per_step": round(dms, 4),
            "attention": {"kernel": DECODE_ATTN, "bound": "hbm", "avg_us": round(at_avg * 1e3, 2),
                          "bytes": at_bytes, "achieved": round(at_gbs, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(at_gbs / HBM_PEAK_GBS, 4)},
            "kernels": dtable,
        }
        log(f"[bench] decode {gms * 1e3:.1f} us/step in a graph (median {gper[len(gper) // 2] * 1e3:.1f}, "
            f"min {gper[0] * 1e3:.1f}); eager {dms * 1e3:.1f} us/step; attention {at_avg * 1e3:.1f} us = "
            f"{at_gbs:.0f} GB/s")
        for k, row in dtable.items():
            log(f"[bench]   {k:40s} {row}")
        del dstep
        torch.cuda.empty_cache()
        decode["fp8kv"] = bench_decode_fp8kv(wd, dev, args)
        decode["paged_attention"] = bench_paged_attention(wd, dev, args)
        decode["lm_head"] = bench_lm_head(wd, dev, args)
        decode["long_context"] = bench_long_decode(wd, dev, args)

    traffic = None
    if not args.no_traffic:
        T_ = wl.batch * wl.seq
        alg = {"gate_up": work["gate_up_silu"][1],
               "rope": rope["bytes"],
               "rmsnorm": T_ * wl.d_model * (4 + 2) + wl.d_model * 2}
        try:
            traffic = measure_traffic(alg)
        except Exception as e:  # the profiler is an instrument, not part of the path
            log(f"[bench] HBM traffic passes unavailable: {e}")
            traffic = {"error": str(e)[:300]}
        if "gate_up" in traffic:
            rope["traffic"] = traffic["rope"]
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_tokens} tokens")
        cpu = cpu_baseline(args.cpu_tokens)
        log(f"[bench] cpu baseline: {cpu}")

    out = {
        "metric": "block fwd TFLOP/s + tokens/s (prefill & decode), % of MFMA/HBM roofline",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_median": round(per[len(per) // 2], 4),
        "ms_min": round(per[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{PREFILL}: B={wl.batch} T={wl.seq} d={wl.d_model} n_q={wl.n_q} "
                               f"n_kv={wl.n_kv} hd={wl.head_dim} d_ff={wl.d_ff} theta={wl.theta:g}",
                   "global_batch": wl.batch, "seq_len": wl.seq, "parallelism": "single-gpu"},
        "tokens_per_s": round(tok_s, 1),
        "prefill_mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {"kernel": DOMINANT, "bound": "mfma", "achieved": round(dom_tflops, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dom_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic["gate_up"]["bytes"] if traffic and "gate_up" in traffic else None,
                     "traffic_detail": traffic.get("gate_up") if traffic else None,
                     "flops_per_launch": dom_flops, "avg_us": round(dom_avg_ms * 1e3, 2)},
        "kernels": table,
        "rope": rope,
        "rmsnorm_traffic": traffic.get("rmsnorm") if traffic else None,
        "traffic_calibration": ({k: traffic[k] for k in ("fetch_scale", "write_scale")}
                                if traffic and "fetch_scale" in traffic else None),
        "chunked_prefill": chunked,
        "mha_prefill": mha,
        "tp8_shard_prefill": tp8,
        "decode": decode,
        "device": device,
        "hbm_copy": copy_bw,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
