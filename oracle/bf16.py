"""Round-to-nearest-even onto the bfloat16 grid, computed in float64.

TEST INFRASTRUCTURE ONLY (part of the oracle; see the package docstring).

bfloat16 keeps float32's 8-bit exponent and 8 significant bits (7 stored).
The pages fix bf16 as the working precision of the block ([LA]
"Troubleshooting", fp16 overflow remedy; [L3] §一 weight precision) but not the
rounding mode; round-to-nearest-even is the reading used on both sides.

The rounding is done directly from float64 with frexp/rint/ldexp, so it does
not depend on any float32 or bfloat16 conversion routine.
"""

import numpy as np

_BF16_MAX = float.fromhex("0x1.fep127")  # largest finite bfloat16
_MIN_QUANTUM_EXP = -133                  # spacing of bf16 subnormals is 2**-133


def round_bf16(x):
    """Return ``x`` (float64 array-like) rounded RNE to bfloat16, as float64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0.0)
    xf = x[finite]
    _, e = np.frexp(xf)                 # xf = m * 2**e with 0.5 <= |m| < 1
    # 8 significant bits: the unit in the last place is 2**(e-8), but never
    # finer than the subnormal spacing.
    q = np.maximum(e - 8, _MIN_QUANTUM_EXP)
    scaled = np.ldexp(xf, -q)           # exact: only moves the exponent
    r = np.ldexp(np.rint(scaled), q)    # np.rint rounds half to even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[finite] = r
    return out
