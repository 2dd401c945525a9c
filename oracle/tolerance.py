"""Error bound for comparing a GPU result with the oracle.

TEST INFRASTRUCTURE (imported by tests/, the smoke check and the benchmark's
self-check only).

Bound per output element, with S = sum |a*b| over the terms of that element:

    |y - ref| <= 1e-4 * S + 1e-6                       (fp32 output)
    |y - ref| <= 1e-4 * S + 1e-6 + ulp_out(|y|) / 2    (bf16 / fp16 output)

The first line is the accuracy target stated for the fp32 accumulator.  A
16-bit output is the fp32 accumulator rounded to nearest-even once more, and
that rounding alone can move it by half a unit in the last place of the output
format; since rounding to nearest never leaves the binade of the rounded value
downward, ulp(|y|) is at least the ulp of the accumulator, so the second line
is the smallest bound that admits a correct fp32 accumulator.
"""
import numpy as np

REL, ABS = 1e-4, 1e-6
_FRAC_BITS = {"f32": 23, "bf16": 7, "f16": 10}
_MIN_ULP = {"f32": 2.0 ** -149, "bf16": 2.0 ** -133, "f16": 2.0 ** -24}


def half_ulp(y, out):
    """Half the spacing of `out`-format numbers at magnitude |y| (0 for f32)."""
    if out == "f32":
        return np.zeros_like(np.asarray(y, np.float64))
    a = np.abs(np.asarray(y, np.float64))
    _, e = np.frexp(a)                      # a = m * 2**e, m in [0.5, 1)
    ulp = np.ldexp(1.0, e - 1 - _FRAC_BITS[out])
    return 0.5 * np.maximum(ulp, _MIN_ULP[out])


def bound(S, y, out):
    return REL * np.asarray(S, np.float64) + ABS + half_ulp(y, out)


def check(y, ref, S, out):
    """Returns (ok, worst_ratio, worst_flat_index); ratio = |y-ref| / bound."""
    y = np.asarray(y, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    S = np.asarray(S, np.float64).ravel()
    if y.size == 0:
        return True, 0.0, -1
    err = np.abs(y - ref)
    b = bound(S, np.maximum(np.abs(y), np.abs(ref)), out)
    ratio = np.where(np.isfinite(err), err / b, np.inf)
    worst = int(np.argmax(ratio))
    return bool(np.all(ratio <= 1.0)), float(ratio[worst]), worst
