"""Tolerance of the backward pass against the fp64 oracle's gradients (the target states
none for gradients; derived from the arithmetic, with u the dtype's unit roundoff:
2^-11 fp16, 2^-8 bf16).

Each gradient is a sum of products in which one 16-bit operand was rounded from fp32
just before (P for dV; dS for dQ and dK; each within u relative), O entered the row
terms D rounded to the dtype, and the result is rounded once more; fp32 accumulation
adds far less. So per gradient tensor

  - normalised: max |G_gpu - G_oracle| <= NORM_U u max |G_oracle|;
  - element-wise, on the entries that carry the tensor (|G_oracle| >= BIG_FRAC of its
    maximum): |G_gpu - G_oracle| <= REL_U u |G_oracle|.

Measured over every backward GPU test (sizes, workloads, grouped heads, unequal
lengths, random shapes, the largest key count): at most 1.7 u normalised and 4.4 u
relative on the large entries.
"""
import numpy as np

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
NORM_U = 3.0
REL_U = 8.0
BIG_FRAC = 0.25


def grad_errors(got, ref):
    """(max|d| / max|ref|, max over the big entries of |d| / |ref|)."""
    m = np.abs(ref).max() if ref.size else 0.0
    err = np.abs(got - ref)
    norm = (err.max() / m if m > 0 else err.max()) if ref.size else 0.0
    big = np.abs(ref) >= BIG_FRAC * m if m > 0 else np.zeros(ref.shape, dtype=bool)
    rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    return float(norm), rel


def check_grad(name, got, ref, dtype, label=""):
    """Assert both bounds for one gradient tensor; returns (norm, rel) in units of u."""
    assert np.all(np.isfinite(got)), f"{label}: {name} not finite"
    norm, rel = grad_errors(got, ref)
    u = U[dtype]
    assert norm <= NORM_U * u, f"{label}: {name} max|d| / max|ref| = {norm / u:.2f} u > {NORM_U} u"
    assert rel <= REL_U * u, f"{label}: {name} big-entry relative error {rel / u:.2f} u > {REL_U} u"
    return norm / u, rel / u
