"""Pins for the parity comparator oracle/tolerance.py.

Every 16-bit-output parity verdict goes through tolerance.half_ulp, bound and
check, so they are pinned to the number formats' own definitions rather than
to a re-typed copy of their formulas:

* half-ulp values derived by hand from the formats: bfloat16 has 7 stored
  fraction bits and a smallest subnormal of 2^-133; IEEE binary16 has 10 and
  2^-24, and its largest finite value is 65504;
* the spacing of neighbouring representable values, obtained by stepping the
  bit pattern by one (bf16: a binary32 with the low half zero, decoded by
  numpy) or from numpy's own binary16 spacing;
* check() admits an error of bound*(1 - 1e-9) and rejects bound*(1 + 1e-9),
  rejects NaN and infinities, rejects a single bad element among many good
  ones, and takes the ulp at the output |y| (a correctly rounded output may
  sit one binade above the exact value, and one below it only with its own
  finer ulp).

Each pin takes a tolerance module (the real one, or a mutated copy) and
returns (ok, message).
"""
import numpy as np


def _close(a, b):
    return np.array_equal(np.asarray(a, np.float64), np.asarray(b, np.float64))


def pin_half_ulp_hand_values(tol):
    # (value, format, half ulp) worked out from the format definitions:
    #   bf16 at 1: ulp 2^-7 -> 2^-8;   in [128, 256): ulp 2^(7-7) = 1 -> 0.5;
    #   at 256: binade [256, 512), ulp 2 -> 1;
    #   bf16 below 2^-126 (subnormal): ulp 2^-133 -> 2^-134;
    #   fp16 at 1: ulp 2^-10 -> 2^-11;  65000 in [32768, 65536): ulp 2^(15-10) = 32 -> 16;
    #   65504 (largest finite) same binade -> 16;
    #   fp16 6e-5 < 2^-14 (subnormal): ulp 2^-24 -> 2^-25;  2^-14 itself: ulp 2^(-14-10) -> 2^-25;
    #   fp16 2^-13: ulp 2^-23 -> 2^-24;
    #   f32 output: no rounding step is added -> 0.
    cases = [(1.0, "bf16", 2.0 ** -8), (255.9, "bf16", 0.5), (256.0, "bf16", 1.0), (-256.0, "bf16", 1.0),
             (1e-39, "bf16", 2.0 ** -134), (0.0, "bf16", 2.0 ** -134),
             (1.0, "f16", 2.0 ** -11), (65000.0, "f16", 16.0), (65504.0, "f16", 16.0),
             (6e-5, "f16", 2.0 ** -25), (2.0 ** -14, "f16", 2.0 ** -25), (2.0 ** -13, "f16", 2.0 ** -24),
             (0.0, "f16", 2.0 ** -25), (3.0, "f32", 0.0), (1e30, "f32", 0.0)]
    for v, fmt, want in cases:
        got = float(tol.half_ulp(np.float64(v), fmt))
        if got != want:
            return False, f"half_ulp({v}, {fmt}) = {got!r}, want {want!r}"
    return True, ""


def _bf16_spacing(v):
    """Distance from |v| (a bf16 value) to the next larger bf16 value, by stepping its bit pattern."""
    bits = np.array([abs(v)], np.float32).view(np.uint32)[0] >> 16
    lo = np.array([np.uint32(bits) << 16], np.uint32).view(np.float32)[0]
    hi = np.array([np.uint32(bits + 1) << 16], np.uint32).view(np.float32)[0]
    return float(hi) - float(lo)


def pin_half_ulp_matches_format_spacing(tol):
    """Half the spacing of representable values, over many binades, from the formats themselves."""
    rng = np.random.default_rng(11)
    exps16 = rng.integers(-24, 16, 400)
    vals16 = np.ldexp(rng.uniform(1.0, 2.0, 400), exps16).astype(np.float16)
    vals16 = vals16[np.isfinite(vals16) & (vals16 > 0)]
    want16 = np.spacing(vals16).astype(np.float64) / 2
    got16 = tol.half_ulp(vals16.astype(np.float64), "f16")
    if not _close(got16, want16):
        i = int(np.argmax(got16 != want16))
        return False, f"f16 half_ulp({float(vals16[i])!r}) = {got16[i]!r}, want {want16[i]!r}"
    exps = rng.integers(-133, 127, 400)
    vals = np.ldexp(rng.uniform(1.0, 2.0, 400), exps).astype(np.float32)
    vals = (vals.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)  # exact bf16 values
    vals = vals[vals > 0]
    want = np.array([_bf16_spacing(float(v)) / 2 for v in vals])
    got = tol.half_ulp(vals.astype(np.float64), "bf16")
    if not _close(got, want):
        i = int(np.argmax(got != want))
        return False, f"bf16 half_ulp({float(vals[i])!r}) = {got[i]!r}, want {want[i]!r}"
    return True, ""


def pin_check_edges_of_bound(tol):
    """An error just inside the bound passes, just outside fails, for every output format, element by element.
    The values sit well inside their binades, so y and ref share the ulp on both sides of the bound."""
    cases = {"f32": (np.array([0.0, 0.75, -3.0, 100.0, 1e-4]), np.array([0.0, 1.0, 37.5, 2048.0, 1e-3])),
             "bf16": (np.array([0.75, -3.0, 100.0, 1e-4]), np.array([1.0, 37.5, 2048.0, 1e-3])),
             "f16": (np.array([0.75, -3.0, 100.0, 1e-4]), np.array([1.0, 37.5, 2048.0, 1e-3]))}
    for fmt, (ref, S) in cases.items():
        b = tol.REL * S + tol.ABS + tol.half_ulp(np.abs(ref), fmt)
        for sign in (1.0, -1.0):
            inside = ref + sign * b * (1 - 1e-9)
            outside = ref + sign * b * (1 + 1e-9)
            assert _same_binade(inside, ref, fmt) and _same_binade(outside, ref, fmt), "pin values cross a binade"
            ok_in, _, _ = tol.check(inside, ref, S, fmt)
            if not ok_in:
                return False, f"{fmt}: error of bound*(1-1e-9) rejected"
            for i in range(ref.size):
                y = ref.copy()
                y[i] = outside[i]
                ok_out, _, worst = tol.check(y, ref, S, fmt)
                if ok_out or worst != i:
                    return False, f"{fmt}: error of bound*(1+1e-9) at element {i} accepted (worst {worst})"
    # the exact constants of the accuracy target: 1e-4 * S + 1e-6
    ok, _, _ = tol.check(np.array([1.0 + 1e-4 * 10 + 1e-6 - 1e-12]), np.array([1.0]), np.array([10.0]), "f32")
    ok2, _, _ = tol.check(np.array([1.0 + 1e-4 * 10 + 1e-6 + 1e-12]), np.array([1.0]), np.array([10.0]), "f32")
    if not ok or ok2:
        return False, "f32 bound is not exactly 1e-4*S + 1e-6"
    ok3, _, _ = tol.check(np.array([1e-6 * (1 - 1e-6)]), np.array([0.0]), np.array([0.0]), "f32")
    ok4, _, _ = tol.check(np.array([1e-6 * (1 + 1e-6)]), np.array([0.0]), np.array([0.0]), "f32")
    if not ok3 or ok4:
        return False, "absolute floor 1e-6 wrong"
    return True, ""


def _same_binade(a, b, fmt):
    if fmt == "f32":
        return True
    ea = np.frexp(np.abs(np.asarray(a, np.float64)))[1]
    eb = np.frexp(np.abs(np.asarray(b, np.float64)))[1]
    return bool(np.all(ea == eb))


def pin_check_rejects_non_finite(tol):
    ref = np.array([1.0, 2.0, 3.0])
    S = np.array([1e9, 1e9, 1e9])  # a huge bound: only non-finite values can fail
    for bad in (np.nan, np.inf, -np.inf):
        for fmt in ("f32", "bf16", "f16"):
            y = ref.copy()
            y[1] = bad
            ok, _, worst = tol.check(y, ref, S, fmt)
            if ok or worst != 1:
                return False, f"{fmt}: y containing {bad} accepted (worst {worst})"
    ok, _, _ = tol.check(ref, np.array([1.0, np.nan, 3.0]), S, "f32")
    if ok:
        return False, "NaN reference accepted"
    return True, ""


def pin_check_every_element(tol):
    """One bad element among a million good ones fails, wherever it is."""
    n = 1 << 20
    ref = np.linspace(-4.0, 4.0, n)
    S = np.full(n, 10.0)
    for where in (0, n // 3, n - 1):
        y = ref.copy()
        y[where] += 0.01  # bound is 1e-3 + 1e-6
        ok, ratio, worst = tol.check(y, ref, S, "f32")
        if ok or worst != where or not (ratio > 1.0):
            return False, f"single bad element at {where} not reported (ok={ok}, worst={worst}, ratio={ratio})"
    ok, ratio, _ = tol.check(ref, ref, S, "f32")
    if not ok or ratio != 0.0:
        return False, "identical arrays not accepted with ratio 0"
    ok, _, worst = tol.check(np.array([]), np.array([]), np.array([]), "bf16")
    if not ok:
        return False, "empty arrays rejected"
    return True, ""


def pin_check_ulp_at_output_magnitude(tol):
    """The half-ulp term is taken at the output |y|.  An fp32 accumulator 257.2 (exact value 255.99, S = 14000
    so the accumulator error 1.21 is inside 1e-4*S = 1.4) rounds to the bf16 value 258 (spacing 2 in
    [256, 512)); |y - ref| = 2.01 is inside 1.4 + 1e-6 + 1 (half ulp at 258) but not inside 1.4 + 1e-6 + 0.5
    (half ulp at 255.99), so it must pass.  Conversely y = 255 for an exact 256.5 with S = 5000: every
    accumulator within 0.5 of 256.5 rounds to 256 or more, so 255 is wrong; |y - ref| = 1.5 exceeds
    0.5 + 1e-6 + 0.5 (half ulp at 255) and must fail, although it would pass with the ulp at 256.5."""
    ok, _, _ = tol.check(np.array([258.0]), np.array([255.99]), np.array([14000.0]), "bf16")
    if not ok:
        return False, "correctly rounded output one binade above the exact value rejected"
    ok, _, _ = tol.check(np.array([258.0]), np.array([255.99]), np.array([1000.0]), "bf16")
    if ok:
        return False, "error 2.01 accepted against bound 0.1 + 1"
    ok, _, _ = tol.check(np.array([255.0]), np.array([256.5]), np.array([5000.0]), "bf16")
    if ok:
        return False, "output below the exact value's binade judged with the exact value's coarser ulp"
    # fp16: exact 2047.9, accumulator 2049.2 (S = 14000 -> 1.4), rounds to 2050 (spacing 2 above 2048);
    # |y - ref| = 2.1 is inside 1.4 + 1 but not inside 1.4 + 0.5
    ok, _, _ = tol.check(np.array([2050.0]), np.array([2047.9]), np.array([14000.0]), "f16")
    if not ok:
        return False, "fp16 output one binade above the exact value rejected"
    ok, _, _ = tol.check(np.array([-2047.0]), np.array([-2048.5]), np.array([5000.0]), "f16")
    if ok:
        return False, "fp16 output below the exact value's binade judged with the coarser ulp"
    return True, ""


ALL_PINS = [pin_half_ulp_hand_values, pin_half_ulp_matches_format_spacing, pin_check_edges_of_bound,
            pin_check_rejects_non_finite, pin_check_every_element, pin_check_ulp_at_output_magnitude]
