"""The parity comparator (oracle/tolerance.py) against its pins, and planted
mistakes in copies of it, each of which must fail at least one pin.  CPU only."""
import importlib.util

import pytest

from oracle import tolerance
from tolerance_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_tolerance_pin(pin):
    ok, msg = pin(tolerance)
    assert ok, msg


MUTANTS = {
    "full_ulp": ("return np.ldexp(0.5, e - 1 - _FRAC_BITS[out])", "return np.ldexp(1.0, e - 1 - _FRAC_BITS[out])"),
    "ulp_exponent_off_by_one": ("return np.ldexp(0.5, e - 1 - _FRAC_BITS[out])",
                                "return np.ldexp(0.5, e - _FRAC_BITS[out])"),
    "bf16_fraction_bits_8": ('"bf16": 7,', '"bf16": 8,'),
    "bf16_fraction_bits_6": ('"bf16": 7,', '"bf16": 6,'),
    "f16_fraction_bits_9": ('"f16": 10}', '"f16": 9}'),
    "f16_fraction_bits_11": ('"f16": 10}', '"f16": 11}'),
    "f16_min_normal": ('"f16": 2.0 ** -14}', '"f16": 2.0 ** -15}'),
    "bf16_min_normal": ('"bf16": 2.0 ** -126,', '"bf16": 2.0 ** -125,'),
    "zero_takes_binade_of_half": ("a = np.maximum(np.abs(np.asarray(y, np.float64)), _MIN_NORMAL[out])",
                                  "a = np.abs(np.asarray(y, np.float64))"),
    "any_for_all": ("np.all(ratio <= 1.0)", "np.any(ratio <= 1.0)"),
    "ulp_from_ref_only": ("b = bound(S, np.abs(y), out)", "b = bound(S, np.abs(ref), out)"),
    "ulp_from_larger": ("b = bound(S, np.abs(y), out)", "b = bound(S, np.maximum(np.abs(y), np.abs(ref)), out)"),
    "rel_1e3": ("REL, ABS = 1e-4, 1e-6", "REL, ABS = 1e-3, 1e-6"),
    "abs_dropped": ("REL, ABS = 1e-4, 1e-6", "REL, ABS = 1e-4, 0.0"),
    "non_finite_passes": ("ratio = np.where(np.isfinite(err), err / b, np.inf)",
                          "ratio = np.where(np.isfinite(err), err / b, 0.0)"),
    "f32_gets_half_ulp": ('    if out == "f32":\n        return np.zeros_like(np.asarray(y, np.float64))\n', ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_tolerance_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(tolerance.__file__).read()
    assert src.count(old) == 1, f"mutation target for {name} not found exactly once"
    path = tmp_path / f"tol_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"tol_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in ALL_PINS:
        try:
            ok, _ = pin(mod)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin caught tolerance mutant {name}"
