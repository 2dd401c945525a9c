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
is the smallest bound that admits a correct fp32 accumulator.  The ulp is
taken at the output |y|, not at the exact value: an output may sit one binade
above the exact value (an accumulator just below a power of two rounds up to
it), and an output below the exact value's binade is admitted only with its
own, finer, ulp.
"""
import numpy as np

REL, ABS = 1e-4, 1e-6
_FRAC_BITS = {"f32": 23, "bf16": 7, "f16": 10}
# Smallest normal magnitude of each format.  Below it (subnormals, and zero)
# the spacing of representable values stays that of the lowest normal binade:
# 2^-133 for bf16, 2^-24 for fp16.
_MIN_NORMAL = {"f32": 2.0 ** -126, "bf16": 2.0 ** -126, "f16": 2.0 ** -14}


def half_ulp(y, out):
    """Half the spacing of `out`-format numbers at magnitude |y| (0 for f32)."""
    if out == "f32":
        return np.zeros_like(np.asarray(y, np.float64))
    a = np.maximum(np.abs(np.asarray(y, np.float64)), _MIN_NORMAL[out])
    _, e = np.frexp(a)                      # a = m * 2**e, m in [0.5, 1)
    return np.ldexp(0.5, e - 1 - _FRAC_BITS[out])


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
    b = bound(S, np.abs(y), out)
    ratio = np.where(np.isfinite(err), err / b, np.inf)
    worst = int(np.argmax(ratio))
    return bool(np.all(ratio <= 1.0)), float(ratio[worst]), worst
