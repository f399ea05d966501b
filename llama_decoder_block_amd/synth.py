"""Seeded synthetic inputs with the shapes of the Llama block workloads.

This module only draws random numbers and rounds them onto the storage grid of
the workload's dtype.  It holds none of the block's arithmetic; the HIP path
and the CPU oracle both receive exactly the tensors it returns.

Recipe: numpy ``Generator(PCG64(seed))`` standard normals in float64, scaled,
then converted to the storage dtype (bfloat16 via torch's round-to-nearest-even
cast, or float32).  Seed = 1000 * workload_index + tensor_index with tensor
indices 0 x, 1 attn gain, 2 W_q, 3 W_k, 4 W_v, 5 W_o, 6 ffn gain, 7 W_gate,
8 W_up, 9 W_down, 10 K cache, 11 V cache.  Activations ~ N(0, 1), weights
~ N(0, 0.02^2), gains 1 + N(0, 0.01^2) (exactly 1 for the toy workload);
0.02 and 0.01 are read as standard deviations.  Prefill positions are
0..T-1; the decode workload places every new token at position 4096 after
4096 cached slots of N(0, 1) values.
"""

from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # seed block (1..5)
    batch: int
    seq: int              # new tokens per sequence in this call
    d_model: int
    n_q: int
    n_kv: int
    head_dim: int
    d_ff: int
    theta: float
    eps: float
    dtype: str            # "f32" or "bf16": weights and GEMM/attention operands
    unit_gains: bool = False
    decode_pos: int = -1  # >= 0: one token per sequence at this position, with a cache
    kv_cap: int = 0       # cache slots per sequence (decode)

    @property
    def n_tokens(self):
        return self.batch * self.seq

    @property
    def is_decode(self):
        return self.decode_pos >= 0


WORKLOADS = {
    w.name: w for w in [
        Workload("toy_gqa_f32", 1, 1, 4, 16, 8, 2, 2, 48, 1e4, 1e-5, "f32", unit_gains=True),
        Workload("llama7b_mha_prefill", 2, 1, 2048, 4096, 32, 32, 128, 11008, 1e4, 1e-5, "bf16"),
        Workload("llama3_8b_gqa_prefill", 3, 1, 8192, 4096, 32, 8, 128, 14336, 5e5, 1e-5, "bf16"),
        Workload("llama3_8b_gqa_decode", 4, 64, 1, 4096, 32, 8, 128, 14336, 5e5, 1e-5, "bf16",
                 decode_pos=4096, kv_cap=4097),
        Workload("llama65b_mha_prefill", 5, 4, 2048, 8192, 64, 64, 128, 22016, 1e4, 1e-5, "bf16"),
    ]
}


def workload(name, **overrides):
    """The named workload, optionally with some fields replaced (used by the
    parity tests to shorten sequences while keeping the model widths)."""
    return replace(WORKLOADS[name], **overrides)


def _draw(seed, shape, scale=1.0, offset=0.0):
    g = np.random.Generator(np.random.PCG64(seed))
    a = g.standard_normal(size=shape, dtype=np.float64)
    if scale != 1.0:
        a *= scale
    if offset != 0.0:
        a += offset
    return a


def _to_storage(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t


@dataclass
class BlockInputs:
    wl: Workload
    x: torch.Tensor                       # [B, T, d] float32 (values on the dtype grid)
    weights: dict                         # name -> torch tensor in storage dtype
    positions: torch.Tensor               # [B, T] int32
    k_cache: torch.Tensor = None          # [B, kv_cap, n_kv, hd] storage dtype
    v_cache: torch.Tensor = None
    extra: dict = field(default_factory=dict)

    def as_f64(self):
        """float64 numpy copies of every tensor (for the oracle)."""
        w = {k: v.to(torch.float64).numpy() for k, v in self.weights.items()}
        out = dict(x=self.x.to(torch.float64).numpy(), w=w,
                   positions=self.positions.numpy().astype(np.int64))
        if self.k_cache is not None:
            out["k_cache"] = self.k_cache.to(torch.float64).numpy()
            out["v_cache"] = self.v_cache.to(torch.float64).numpy()
        return out


WEIGHT_NAMES = ["attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down"]


def make_block_inputs(wl, seed_offset=0):
    """Draw every tensor of one block call for workload ``wl``."""
    base = 1000 * wl.index + seed_offset
    d, hd, dff = wl.d_model, wl.head_dim, wl.d_ff
    nq, nkv = wl.n_q, wl.n_kv
    shapes = {
        "wq": (nq * hd, d), "wk": (nkv * hd, d), "wv": (nkv * hd, d), "wo": (d, nq * hd),
        "w_gate": (dff, d), "w_up": (dff, d), "w_down": (d, dff),
    }
    tensor_index = {"attn_norm": 1, "wq": 2, "wk": 3, "wv": 4, "wo": 5, "ffn_norm": 6,
                    "w_gate": 7, "w_up": 8, "w_down": 9}
    weights = {}
    for name in WEIGHT_NAMES:
        i = tensor_index[name]
        if name in ("attn_norm", "ffn_norm"):
            if wl.unit_gains:
                a = np.ones(d)
            else:
                a = _draw(base + i, (d,), 0.01, 1.0)
        else:
            a = _draw(base + i, shapes[name], 0.02)
        weights[name] = _to_storage(a, wl.dtype)
    x = _to_storage(_draw(base + 0, (wl.batch, wl.seq, d)), wl.dtype).to(torch.float32)
    if wl.is_decode:
        positions = torch.full((wl.batch, wl.seq), wl.decode_pos, dtype=torch.int32)
        cache_shape = (wl.batch, wl.kv_cap, nkv, hd)
        kc = np.zeros(cache_shape)
        vc = np.zeros(cache_shape)
        kc[:, :wl.decode_pos] = _draw(base + 10, (wl.batch, wl.decode_pos, nkv, hd))
        vc[:, :wl.decode_pos] = _draw(base + 11, (wl.batch, wl.decode_pos, nkv, hd))
        return BlockInputs(wl, x, weights, positions,
                           _to_storage(kc, wl.dtype), _to_storage(vc, wl.dtype))
    positions = torch.arange(wl.seq, dtype=torch.int32).repeat(wl.batch, 1)
    return BlockInputs(wl, x, weights, positions)


def normal(seed, shape, scale=1.0, offset=0.0, dtype="f32"):
    """One seeded tensor on the storage grid of ``dtype`` (for kernel-level tests)."""
    return _to_storage(_draw(seed, shape, scale, offset), dtype)
