"""Error metrics shared by the parity tests (host-side numpy, float64)."""

import numpy as np

BF16_ULP = 2.0 ** -8  # spacing of bf16 values in [1, 2); half of it is the RNE bound


def to64(t):
    """torch tensor (any device/dtype) or array -> float64 numpy."""
    if hasattr(t, "detach"):
        import torch
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def max_rel_floor(got, ref, floor_frac=1e-3):
    """max_i |g_i - o_i| / max(|o_i|, floor_frac * max_j |o_j|): relative error
    with a floor so that entries near zero are judged on the tensor's scale."""
    got, ref = to64(got), to64(ref)
    scale = max(np.abs(ref).max(), 1e-300)
    den = np.maximum(np.abs(ref), floor_frac * scale)
    return float(np.max(np.abs(got - ref) / den))


def rel_frobenius(got, ref):
    got, ref = to64(got), to64(ref)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(got, ref):
    return float(np.max(np.abs(to64(got) - to64(ref))))


def report(name, got, ref):
    print(f"[{name}] max_rel_floor={max_rel_floor(got, ref):.3e} relF={rel_frobenius(got, ref):.3e} "
          f"max_abs={max_abs(got, ref):.3e}", flush=True)
