"""Pins of the oracle's KV-cache variants against their definitions: the
8-bit cache model (oracle/fp8.py) against the E4M3 format and the scale
convention it states, and the paged-cache mapping (oracle/paged.py) against a
scalar loop and its inverse ([LA] "Troubleshooting Common Deployment Faults",
item 3, names both remedies; formats and layouts are readings).  Nothing here
uses a GPU."""

import numpy as np
import pytest

import oracle
from oracle import fp8


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def test_decode_known_codes():
    # values fixed by the format: bias 7, 3 mantissa bits, subnormal spacing 2**-9
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
             0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in table.items():
        assert fp8.e4m3_decode(np.uint8(c)) == v, hex(c)
    assert np.signbit(fp8.e4m3_decode(np.uint8(0x80)))
    assert np.isnan(fp8.e4m3_decode(np.uint8(0x7F))) and np.isnan(fp8.e4m3_decode(np.uint8(0xFF)))


def test_decode_grid_is_strictly_increasing_with_126_positive_values():
    pos = fp8.e4m3_decode(np.arange(0x01, 0x7F, dtype=np.uint8))
    assert len(pos) == 126
    assert np.all(np.diff(pos) > 0)
    # spacing doubles at each binade boundary: 2**-9 up to 2**-5, then 2**(e-3)
    assert np.all(np.diff(fp8.e4m3_decode(np.arange(0x00, 0x10, dtype=np.uint8))) == 2.0 ** -9)
    assert fp8.e4m3_decode(np.uint8(0x7E)) - fp8.e4m3_decode(np.uint8(0x7D)) == 32.0


def test_encode_decode_round_trip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def test_ties_go_to_even_mantissa():
    c = np.arange(0x00, 0x7E)
    mids = 0.5 * (fp8.e4m3_decode(c) + fp8.e4m3_decode(c + 1))
    want = np.where(c % 2 == 0, c, c + 1)
    assert np.array_equal(fp8.e4m3_encode(mids), want)
    assert np.array_equal(fp8.e4m3_encode(-mids), want | 0x80)


def test_nearest_rounding_bruteforce():
    grid = fp8.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    x = np.concatenate([rng(1).uniform(0, 448, 4000), rng(2).uniform(0, 0.05, 4000)])
    got = fp8.e4m3_decode(fp8.e4m3_encode(x))
    dist = np.abs(x[:, None] - grid[None, :])
    best = dist.min(axis=1)
    assert np.all(np.abs(got - x) == best)


def test_saturation_sign_and_nan():
    enc = fp8.e4m3_encode(np.array([448.0, 463.9, 1e30, -1e30, -0.0, 2.0 ** -11, -(2.0 ** -11), np.nan]))
    assert list(enc) == [0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80, 0x7F]


def test_quantize_rows_scale_and_extreme_code():
    x = rng(3).standard_normal((16, 128)).astype(np.float32).astype(np.float64)
    codes, s = fp8.quantize_rows(x)
    assert s.dtype == np.float32
    assert np.array_equal(s, (np.max(np.abs(x), axis=1).astype(np.float32) / np.float32(448)).astype(np.float32))
    # the largest magnitude of every row lands on +-448
    i = np.argmax(np.abs(x), axis=1)
    ext = codes[np.arange(16), i]
    assert np.all((ext & 0x7F) == 0x7E)


def test_quantize_rows_error_bound():
    x = (rng(4).standard_normal((64, 128)) * np.exp(rng(5).uniform(-6, 6, (64, 1)))).astype(np.float32)
    x = x.astype(np.float64)
    codes, s = fp8.quantize_rows(x)
    xh = fp8.dequantize_rows(codes, s)
    # half a step of the 3-bit mantissa, or half a subnormal step, in units of s
    # (plus the fp32 rounding of x / s)
    bound = np.abs(x) * (2.0 ** -4 + 2.0 ** -22) + s[:, None].astype(np.float64) * 2.0 ** -10
    assert np.all(np.abs(xh - x) <= bound)


def test_zero_row_stores_zero_scale_and_codes():
    x = np.zeros((2, 128))
    x[1, 5] = -0.0
    codes, s = fp8.quantize_rows(x)
    assert np.all(s == 0) and np.all(codes == 0)


def test_grid_values_with_unit_scale_are_stored_exactly():
    # rows whose maximum is 448 and whose values lie on the E4M3 grid: s = 1 and
    # the cache holds exactly the input, so attention over it is the plain one
    g = rng(6)
    grid = fp8.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    k = g.choice(grid, size=(1, 9, 2, 128)) * g.choice([-1.0, 1.0], size=(1, 9, 2, 128))
    v = g.choice(grid, size=(1, 9, 2, 128)) * g.choice([-1.0, 1.0], size=(1, 9, 2, 128))
    k[..., 0] = 448.0
    v[..., 3] = -448.0
    kc, vc, ks, vs = fp8.kv_cache_from_rows(k, v)
    assert ks.shape == (1, 2, 9) and np.all(ks == 1.0) and np.all(vs == 1.0)
    assert np.array_equal(fp8.kv_cache_values(kc, ks), k)
    assert np.array_equal(fp8.kv_cache_values(vc, vs), v)
    q = g.standard_normal((1, 1, 4, 128)) * 0.01
    vis = np.array([[8]])
    a = oracle.gqa_attention(q, fp8.kv_cache_values(kc, ks), fp8.kv_cache_values(vc, vs), vis)
    b = oracle.gqa_attention(q, k, v, vis)
    assert np.array_equal(a, b)


def test_rejects_values_fp32_cannot_hold():
    with pytest.raises(ValueError):
        fp8.quantize_rows(np.array([[1.0 + 2.0 ** -40]]))


def test_decode_step_fp8kv_reduces_to_plain_decode_for_zero_new_rows():
    # with W_k = W_v = 0 the new token's k and v are exactly zero, so its cache
    # row is scale 0 / codes 0 and the step equals the plain decode step over
    # the dequantized cache; the other slots are left as they were
    g = rng(7)
    d, nq, nkv, hd, dff, B, S = 64, 4, 2, 128, 96, 2, 9
    w = {"attn_norm": 1.0 + 0.1 * g.standard_normal(d), "wq": 0.05 * g.standard_normal((nq * hd, d)),
         "wk": np.zeros((nkv * hd, d)), "wv": np.zeros((nkv * hd, d)),
         "wo": 0.05 * g.standard_normal((d, nq * hd)), "ffn_norm": 1.0 + 0.1 * g.standard_normal(d),
         "w_gate": 0.05 * g.standard_normal((dff, d)), "w_up": 0.05 * g.standard_normal((dff, d)),
         "w_down": 0.05 * g.standard_normal((d, dff))}
    # cache rows on the E4M3 grid with maximum 448 (scale 1), so that the
    # dequantized cache is also a bf16 tensor and the plain step's bf16
    # storage point leaves it unchanged
    grid = fp8.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8)) / 64.0
    k = g.choice(grid, size=(B, S, nkv, hd)) * g.choice([-1.0, 1.0], size=(B, S, nkv, hd))
    v = g.choice(grid, size=(B, S, nkv, hd)) * g.choice([-1.0, 1.0], size=(B, S, nkv, hd))
    k[..., 0] = v[..., 1] = 7.0
    kc, vc, ks, vs = fp8.kv_cache_from_rows(k, v)
    assert np.array_equal(fp8.kv_cache_values(kc, ks), k)
    x = g.standard_normal((B, 1, d))
    pos = [3, 8]
    y, kc2, vc2, ks2, vs2 = fp8.decode_step_fp8kv(x, w, pos, kc, vc, ks, vs, 1e4, 1e-5, nq, nkv)
    kd, vd = fp8.kv_cache_values(kc, ks), fp8.kv_cache_values(vc, vs)
    y_plain = oracle.decode_step(x, w, pos, kd, vd, 1e4, 1e-5, nq, nkv, bf16_storage=True)[0]
    assert np.array_equal(y, y_plain)
    for b, p in enumerate(pos):
        assert np.all(kc2[b, :, p] == 0) and np.all(vc2[b, :, p] == 0)
        assert np.all(ks2[b, :, p] == 0) and np.all(vs2[b, :, p] == 0)
        keep = [j for j in range(S) if j != p]
        assert np.array_equal(kc2[b][:, keep], kc[b][:, keep]) and np.array_equal(ks2[b][:, keep], ks[b][:, keep])


# ---------------------------------------------------------------------------
# paged cache mapping (oracle/paged.py)
# ---------------------------------------------------------------------------
def test_paged_gather_against_scalar_mapping():
    from oracle import paged
    g = rng(8)
    P, n_pages, B, max_pages, nkv, hd = 4, 9, 2, 3, 2, 3
    pool = g.standard_normal((n_pages, P, nkv, hd))
    table = np.array([[5, 0, 7], [2, 8, 1]])
    out = paged.gather(pool, table, P)
    for b in range(B):
        for j in range(max_pages * P):
            assert np.array_equal(out[b, j], pool[table[b, j // P], j % P])


def test_paged_identity_table_and_scatter_round_trip():
    from oracle import paged
    g = rng(9)
    P, B, max_pages, nkv, hd = 8, 3, 4, 2, 16
    cache = g.standard_normal((B, max_pages * P, nkv, hd))
    ident = np.arange(B * max_pages).reshape(B, max_pages)
    pool = cache.reshape(B * max_pages, P, nkv, hd)
    assert np.array_equal(paged.gather(pool, ident, P), cache)
    perm = g.permutation(20)[:B * max_pages].reshape(B, max_pages)
    pool2 = paged.scatter(cache, perm, 20, P)
    assert np.array_equal(paged.gather(pool2, perm, P), cache)
    unused = sorted(set(range(20)) - set(perm.ravel()))
    assert np.all(np.isnan(pool2[unused]))
