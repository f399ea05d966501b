"""The work model against the counts printed on "LLaMA-3 8B 现代 LLM 架构、计算规模与能耗"
(§六 parameter tables, §七 KV-cache sizes, §八 prefill FLOPs, §九 decode FLOPs)."""

import pytest

from llama_decoder_block_amd import workmodel as wm

L3_8B = wm.Shape(d_model=4096, n_q=32, n_kv=8, head_dim=128, d_ff=14336)


def test_parameter_counts_llama3_8b():
    assert wm.attention_params(L3_8B) == 41_943_040
    assert wm.mlp_params(L3_8B) == 176_160_768
    assert wm.block_params(L3_8B) == 218_112_000
    assert wm.linear_params(L3_8B) == 218_103_808
    mha = wm.Shape(4096, 32, 32, 128, 14336)
    assert wm.attention_params(mha) == 67_108_864


@pytest.mark.parametrize("seq,lin,att", [(128, 5.58e10, 2.68e8), (1024, 4.47e11, 1.72e10),
                                         (8192, 3.57e12, 1.10e12)])
def test_prefill_flops_table(seq, lin, att):
    assert wm.prefill_linear_flops(L3_8B, seq) == pytest.approx(lin, rel=5e-3)
    assert wm.dense_attention_flops(L3_8B, 1, seq) == pytest.approx(att, rel=5e-3)


def test_prefill_total_and_causal_count():
    total_dense = wm.prefill_linear_flops(L3_8B, 8192) + wm.dense_attention_flops(L3_8B, 1, 8192)
    assert total_dense == pytest.approx(4.67e12, rel=5e-3)
    # causal count keeps only the visible half (plus the diagonal)
    assert wm.prefill_attention_flops(L3_8B, 1, 8192) == 4 * 128 * 32 * 8192 * 8193 // 2


def test_decode_flops():
    assert wm.prefill_linear_flops(L3_8B, 1) == pytest.approx(4.36e8, rel=5e-3)
    assert wm.decode_attention_flops(L3_8B, 1, 8193) == pytest.approx(2 * 6.71e7, rel=5e-3)
    assert wm.decode_flops(L3_8B, 1, 8193) == pytest.approx(5.70e8, rel=5e-3)


def test_kv_cache_bytes():
    assert wm.kv_bytes_per_token(L3_8B) == 4096
    assert 32 * wm.kv_bytes_per_token(wm.Shape(4096, 32, 32, 128, 14336)) == 524_288
    # 8192-token context over 32 layers is 1 GiB
    assert 32 * 8192 * wm.kv_bytes_per_token(L3_8B) == 1 << 30


def test_step_work_sums_to_block_totals():
    pre = wm.step_work(L3_8B, 1, 8192)
    assert sum(f for f, _ in pre.values()) == wm.prefill_flops(L3_8B, 1, 8192)
    dec = wm.step_work(L3_8B, 64, 1, attend_len=4097)
    assert sum(f for f, _ in dec.values()) == wm.decode_flops(L3_8B, 64, 4097)
    assert dec["attention"][1] == 1_074_003_968
    # decode: the weights dominate the GEMM steps' bytes (activations add ~2%)
    wbytes = sum(dec[k][1] for k in ("qkv_rope", "o_resid", "gate_up_silu", "down_resid"))
    assert wm.decode_weight_bytes(L3_8B) < wbytes < 1.03 * wm.decode_weight_bytes(L3_8B)


def test_fp8_kv_bytes_halve_the_cache_plus_row_scales():
    # [LA] §4 memory formula with bytes_per_elem = 1, plus 4 bytes per cached row
    b16 = wm.decode_attention_bytes(L3_8B, 64, 4097)
    b8 = wm.decode_attention_bytes_fp8kv(L3_8B, 64, 4097)
    assert b8 == b16 // 2 + 64 * 4097 * 2 * 8 * 4
    w = wm.step_work(L3_8B, 64, 1, attend_len=4097, kv_bytes=wm.FP8KV_BYTES_PER_ELEM)
    assert w["attention"][1] == b8


def test_chunk_attention_flops():
    """A chunk at position 0 is a plain causal prefill; a one-token chunk at
    position p is a decode step attending p + 1 slots; two consecutive chunks
    add up to the prefill of their union."""
    s = wm.Shape(4096, 32, 8, 128, 14336)
    assert wm.chunk_attention_flops(s, 2, 8192, 0) == wm.prefill_attention_flops(s, 2, 8192)
    assert wm.chunk_attention_flops(s, 64, 1, 4096) == wm.decode_attention_flops(s, 64, 4097)
    assert (wm.chunk_attention_flops(s, 1, 3000, 0) + wm.chunk_attention_flops(s, 1, 5192, 3000)
            == wm.prefill_attention_flops(s, 1, 8192))


def test_step_work_of_a_chunk_counts_the_cached_history():
    """The attention row of a chunk after `history` cached slots carries the
    chunk's own count (each token sees the history plus the causal part of
    the chunk) and reads the history's K and V once."""
    s = wm.Shape(4096, 32, 8, 128, 14336)
    plain = wm.step_work(s, 1, 8192)
    chunk = wm.step_work(s, 1, 8192, history=24576)
    assert plain["attention"][0] == wm.prefill_attention_flops(s, 1, 8192)
    assert chunk["attention"][0] == wm.chunk_attention_flops(s, 1, 8192, 24576)
    assert chunk["attention"][1] - plain["attention"][1] == 24576 * wm.kv_bytes_per_token(s)
    for k in ("qkv_rope", "o_resid", "gate_up_silu", "down_resid"):
        assert chunk[k] == plain[k]
