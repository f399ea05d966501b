"""Algorithmic work of one block forward: FLOPs, bytes and parameter counts.

Used by the benchmark to turn measured times into TFLOP/s, GB/s and roofline
fractions.  Conventions:
  * a matrix product of [m, k] by [k, n] costs 2*m*k*n FLOPs (the "2mnp" rule
    of "LLaMA-3 8B 现代 LLM 架构、计算规模与能耗", §八);
  * causal attention counts only visible (query, key) pairs: QK^T and PV each
    cost 2*hd per pair and head; the dense convention of that page (every pair
    of an S x S matrix) is also provided for comparison;
  * HBM bytes are the algorithmic minimum: every input read once, every output
    written once.
"""

from dataclasses import dataclass

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E


@dataclass(frozen=True)
class Shape:
    d_model: int
    n_q: int
    n_kv: int
    head_dim: int
    d_ff: int


def linear_params(s):
    """Weights of the four attention and three FFN projections."""
    attn = s.d_model * s.n_q * s.head_dim * 2 + 2 * s.d_model * s.n_kv * s.head_dim
    return attn + 3 * s.d_model * s.d_ff


def block_params(s):
    return linear_params(s) + 2 * s.d_model


def attention_params(s):
    return s.d_model * s.n_q * s.head_dim * 2 + 2 * s.d_model * s.n_kv * s.head_dim


def mlp_params(s):
    return 3 * s.d_model * s.d_ff


def prefill_linear_flops(s, n_tokens):
    return 2 * n_tokens * linear_params(s)


def causal_pairs(batch, seq):
    return batch * seq * (seq + 1) // 2


def prefill_attention_flops(s, batch, seq):
    return 4 * s.head_dim * s.n_q * causal_pairs(batch, seq)


def chunk_attention_flops(s, batch, seq, start):
    """A chunk of `seq` tokens at positions start..start+seq-1 against a cache
    holding the `start` earlier ones: token i sees start + i + 1 slots."""
    return 4 * s.head_dim * s.n_q * batch * (seq * start + seq * (seq + 1) // 2)


def dense_attention_flops(s, batch, seq):
    return 4 * s.head_dim * s.n_q * batch * seq * seq


def prefill_flops(s, batch, seq):
    return prefill_linear_flops(s, batch * seq) + prefill_attention_flops(s, batch, seq)


def decode_attention_flops(s, batch, attend_len):
    return 4 * s.head_dim * s.n_q * batch * attend_len


def decode_flops(s, batch, attend_len):
    return prefill_linear_flops(s, batch) + decode_attention_flops(s, batch, attend_len)


def kv_bytes_per_token(s, elem_bytes=2):
    return 2 * s.n_kv * s.head_dim * elem_bytes


def decode_attention_bytes(s, batch, attend_len, elem_bytes=2):
    """K and V of every visible slot read once (the query/output are negligible)."""
    return batch * attend_len * kv_bytes_per_token(s, elem_bytes)


# 8-bit KV cache: one byte per element plus one fp32 scale per row of head_dim
# elements (per slot, KV head and K or V)
FP8KV_BYTES_PER_ELEM = "fp8"


def decode_attention_bytes_fp8kv(s, batch, attend_len):
    """Codes of every visible K/V slot plus their row scales, read once."""
    return batch * attend_len * 2 * s.n_kv * (s.head_dim + 4)


def decode_weight_bytes(s, elem_bytes=2):
    return block_params(s) * elem_bytes


def gemm_flops(m, n, k):
    return 2 * m * n * k


def step_work(s, batch, seq, attend_len=None, wbytes=2, rbytes=4, kv_bytes=None, history=0):
    """Algorithmic FLOPs and HBM bytes of each step of one block forward.

    Returns {step: (flops, bytes)} keyed like the library's timing records
    (attn_norm, qkv_rope, attention, o_resid, ffn_norm, gate_up_silu,
    down_resid).  `attend_len` is None for a prefill without a cache (causal
    pairs within the sequence) and the number of visible cache slots for a
    one-token decode.  `history` (prefill only) is the number of cached slots
    before a chunk of `seq` tokens: each token also sees them, and they are
    read once.  Bytes: every weight, input and output read or written
    once; for decode attention only the K/V slots are counted (the query and
    output are 1/4000 of it).  `wbytes` / `rbytes` are the element sizes of
    the GEMM operands and of the residual stream; kv_bytes=FP8KV_BYTES_PER_ELEM
    counts the decode cache as 8-bit codes plus row scales.
    """
    m = batch * seq
    d, hd = s.d_model, s.head_dim
    nqkv = (s.n_q + 2 * s.n_kv) * hd
    nqo = s.n_q * hd
    out = {}
    norm_bytes = m * d * (rbytes + wbytes) + d * wbytes
    out["attn_norm"] = (0, norm_bytes)
    out["qkv_rope"] = (gemm_flops(m, nqkv, d), (nqkv * d + m * d + m * nqkv) * wbytes)
    if attend_len is None:
        out["attention"] = (chunk_attention_flops(s, batch, seq, history),
                            (m * (nqkv + nqo) + batch * history * 2 * s.n_kv * hd) * wbytes)
    else:
        kvb = (decode_attention_bytes_fp8kv(s, batch, attend_len) if kv_bytes == FP8KV_BYTES_PER_ELEM
               else decode_attention_bytes(s, batch, attend_len, wbytes))
        out["attention"] = (decode_attention_flops(s, batch, attend_len), kvb)
    out["o_resid"] = (gemm_flops(m, d, nqo), (d * nqo + m * nqo) * wbytes + 2 * m * d * rbytes)
    out["ffn_norm"] = (0, norm_bytes)
    out["gate_up_silu"] = (gemm_flops(m, 2 * s.d_ff, d), (2 * s.d_ff * d + m * d + m * s.d_ff) * wbytes)
    out["down_resid"] = (gemm_flops(m, d, s.d_ff), (d * s.d_ff + m * s.d_ff) * wbytes + 2 * m * d * rbytes)
    return out
