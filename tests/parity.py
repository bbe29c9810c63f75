"""Comparison rule for GEMM / GEMV outputs against the float64 oracle.

Per element, with C the oracle value and C_hat the kernel's:

    |C_hat - C| <= max(2e-3 * |C|, 1e-2 * RMS(C))  [+ 0.5 ulp_bf16(C) for bf16 output]

The first two terms are the stated tolerance (relative 2e-3, or 1e-2 of the
output RMS).  A bf16 output cannot meet the relative term by itself (its own
rounding is up to 2^-9 relative), so for bf16 outputs the criterion is
applied to the value before its final rounding by allowing that rounding's
half ulp on top; the literal criterion is checked exactly with the kernel's
binary32 output mode.
"""

from dataclasses import dataclass

import numpy as np


def ulp_bf16(v):
    v = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(np.where(v == 0, 1.0, v))
    q = np.exp2(np.maximum(e - 8, -133).astype(np.float64))
    return np.where(v == 0, 2.0 ** -133, q)


@dataclass
class RuleT:
    ok: bool
    n: int
    n_fail: int
    max_rel: float
    max_abs_over_rms: float
    rel_fro: float
    frac_literal: float
    worst: tuple

    def __str__(self):
        return (f"n={self.n} fail={self.n_fail} max_rel={self.max_rel:.3e} "
                f"max_abs/rms={self.max_abs_over_rms:.3e} rel_fro={self.rel_fro:.3e} "
                f"literal_pass={self.frac_literal:.6f} worst={self.worst}")


def rule_t(got, ref, bf16_out: bool, rel=2e-3, rms_frac=1e-2) -> RuleT:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    lit = np.maximum(rel * np.abs(ref), rms_frac * rms)
    bound = lit + (0.5 * ulp_bf16(ref) if bf16_out else 0.0)
    fail = ~(err <= bound)
    nz = np.abs(ref) > 0
    max_rel = float(np.max(err[nz] / np.abs(ref[nz]))) if np.any(nz) else 0.0
    worst = ()
    if fail.any():
        i = np.unravel_index(np.argmax(np.where(fail, err - bound, -np.inf)), ref.shape)
        worst = (tuple(int(t) for t in i), float(got[i]), float(ref[i]))
    fro = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return RuleT(ok=not bool(fail.any()), n=int(ref.size), n_fail=int(fail.sum()),
                 max_rel=max_rel, max_abs_over_rms=float(err.max() / rms) if rms > 0 and err.size else 0.0,
                 rel_fro=fro, frac_literal=float(np.mean(err <= lit)) if err.size else 1.0,
                 worst=worst)
