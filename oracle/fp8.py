"""8-bit (FP8 E4M3) KV cache: encoding, per-row scaling and dequantization.

TEST INFRASTRUCTURE ONLY (part of the oracle; see the package docstring).

[LA] "Troubleshooting Common Deployment Faults", item 3 (out-of-memory in
long-context inference) names an 8-bit KV cache as the remedy that halves the
bytes_per_elem factor of the KV-cache memory formula in [LA] §4 ("Grouped-Query
Attention (GQA) and KV Cache Scaling").  The pages fix neither the 8-bit
format nor a scale convention, so both are readings:

* Format: OCP FP8 E4M3 -- 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits.  Exponent field 0 holds the subnormals m * 2**-9 (m = 0..7); fields
  1..15 hold (1 + m/8) * 2**(field - 7), except that field 15 with m = 7 is
  NaN (there are no infinities).  The largest finite magnitude is 448.
* Scale: one fp32 scale per (sequence, slot, KV head) row of head_dim values:
  s = max|x| / 448 (an fp32 division), each code is x / s (an fp32 division)
  rounded to the nearest E4M3 value, ties to the even mantissa, magnitudes
  beyond 448 clamped to 448, the sign kept (so -0 and negative values that
  round to zero give the code 0x80).  A row whose maximum is 0 stores scale 0
  and all-zero codes.  The stored value of a code c is s * E4M3(c).

Everything here is written from that definition with float64 arithmetic
(frexp / ldexp / rint), apart from the two fp32 divisions the scale
convention itself specifies.
"""

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6      # smallest normal magnitude is 2**-6
_SUBNORMAL_QUANTUM = -9   # subnormal spacing 2**-9
_NAN_CODE = 0x7F


def e4m3_decode(codes):
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    field = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + mant / 8.0, (field - 7).astype(np.int64))
    sub = np.ldexp(mant, _SUBNORMAL_QUANTUM)
    mag = np.where(field == 0, sub, normal)
    mag = np.where((c & 0x7F) == _NAN_CODE, np.nan, mag)
    return sign * mag


def e4m3_encode(values):
    """float64 values (normally the fp32 quotients x / s) -> uint8 codes:
    round to nearest E4M3, ties to even, clamp to +-448, keep the sign;
    NaN -> 0x7F."""
    v = np.asarray(values, dtype=np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.int64)
    nan = np.isnan(a)
    sat = ~nan & (a >= E4M3_MAX)
    rest = ~nan & ~sat
    ar = a[rest]
    # spacing of the E4M3 grid around |v|: 2**(e-3) in the binade [2**e, 2**(e+1)),
    # 2**-9 below the smallest normal 2**-6
    _, e2 = np.frexp(ar)                    # ar = f * 2**e2, 0.5 <= f < 1
    quantum_exp = np.maximum(e2 - 1 - 3, _SUBNORMAL_QUANTUM)
    units = np.rint(np.ldexp(ar, -quantum_exp))        # half to even
    r = np.ldexp(units, quantum_exp)                    # rounded magnitude
    r = np.minimum(r, E4M3_MAX)
    # bit pattern of the rounded magnitude
    codes = np.zeros(ar.shape, dtype=np.int64)
    is_sub = r < 2.0 ** _MIN_NORMAL_EXP
    codes[is_sub] = np.ldexp(r[is_sub], -_SUBNORMAL_QUANTUM).astype(np.int64)
    rn = r[~is_sub]
    _, en = np.frexp(rn)
    expo = en - 1                                        # rn = (1 + m/8) * 2**expo
    mant = (np.ldexp(rn, -expo) - 1.0) * 8.0
    codes[~is_sub] = ((expo + 7) << 3) + mant.astype(np.int64)
    out[rest] = codes
    out[sat] = 0x7E
    out[nan] = _NAN_CODE
    out = np.where(neg & ~nan, out | 0x80, out)
    return out.astype(np.uint8)


def quantize_rows(x):
    """Quantize the last axis of ``x`` (values that fp32 holds exactly, e.g.
    bf16 K or V rows) row by row.  Returns (codes uint8 [..., hd],
    scales float32 [...])."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64), equal_nan=True):
        raise ValueError("quantize_rows expects values exactly representable in fp32")
    amax = np.max(np.abs(x32), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1), scale).astype(np.float32)
    q = (x32 / safe[..., None]).astype(np.float32)
    codes = e4m3_encode(q.astype(np.float64))
    codes = np.where((scale == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes, scale


def dequantize_rows(codes, scales):
    """codes uint8 [..., hd], scales [...] -> float64 values s * E4M3(code)."""
    return np.asarray(scales, dtype=np.float64)[..., None] * e4m3_decode(codes)


def kv_cache_from_rows(k_rows, v_rows):
    """Quantize bf16-valued K / V caches [B, S, n_kv, hd] (the token-major
    layout of the bf16 caches); returns (k_codes, v_codes [B, n_kv, S, hd]
    uint8, k_scales, v_scales [B, n_kv, S] float32), the head-major layout of
    the 8-bit cache."""
    kh = np.asarray(k_rows, dtype=np.float64).transpose(0, 2, 1, 3)
    vh = np.asarray(v_rows, dtype=np.float64).transpose(0, 2, 1, 3)
    kc, ks = quantize_rows(kh)
    vc, vs = quantize_rows(vh)
    return tuple(np.ascontiguousarray(a) for a in (kc, vc, ks, vs))


def kv_cache_values(codes, scales):
    """codes [B, n_kv, S, hd] with scales [B, n_kv, S] -> float64 values in
    the token-major layout [B, S, n_kv, hd] that attention reads."""
    return dequantize_rows(codes, scales).transpose(0, 2, 1, 3)


def decode_step_fp8kv(x, w, position, k_codes, v_codes, k_scales, v_scales, theta, eps, n_q, n_kv):
    """One decode step of the block against an 8-bit cache, with the bf16
    path's storage points: the new token's rotated k and its v (rounded to
    bf16) are quantized into slot ``position[b]`` of sequence b, then query b
    attends the dequantized slots 0..position[b]; everything else is the
    plain block ([LA] "Step 2"; [L3] §七, §九).
    x [B, 1, d]; caches as in :func:`kv_cache_from_rows`.  Returns
    (y, k_codes, v_codes, k_scales, v_scales) with the updated cache copies."""
    from . import reference as ref
    x = np.asarray(x, dtype=np.float64)
    B = x.shape[0]
    pos = np.asarray(position, dtype=np.int64).reshape(B, 1)
    q, k, v = ref._attention_inputs(x, w, pos, theta, eps, n_q, n_kv, True)
    kc, vc = np.array(k_codes, copy=True), np.array(v_codes, copy=True)
    ks, vs = np.array(k_scales, copy=True), np.array(v_scales, copy=True)
    nk, sk = quantize_rows(k[:, 0])      # [B, n_kv, hd], [B, n_kv]
    nv, sv = quantize_rows(v[:, 0])
    for b in range(B):
        p = pos[b, 0]
        kc[b, :, p], vc[b, :, p] = nk[b], nv[b]
        ks[b, :, p], vs[b, :, p] = sk[b], sv[b]
    o = ref.gqa_attention(q, kv_cache_values(kc, ks), kv_cache_values(vc, vs), pos).reshape(B, 1, -1)
    _, y = ref._block_tail(x, o, w, eps, True)
    return y, kc, vc, ks, vs
