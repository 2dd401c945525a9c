"""Planted mistakes in copies of the CPU oracle must each fail at least one pin.

Every mutant is a plausible slip (a transposed operand, a dropped term, a wrong
sign, an off-by-one exponent bias, a wrong padding sign, swapped filter taps, a
missing absolute value).  The mutated source is compiled on the CPU into a
temporary directory; the real oracle is never modified.
"""
import os

import pytest

import oracle
from oracle.build import SRC, build
from oracle_pins import ALL_PINS

MUTANTS = {
    "transposed_A_index": ("Ad[i * K + k] = dec(a_col_major ? A[k * lda + i] : A[i * lda + k], dtype);",
                           "Ad[i * K + k] = dec(a_col_major ? A[i * lda + k] : A[k * lda + i], dtype);"),
    "dropped_last_k": ("for (int64_t k = 0; k < K; k++) { /* i-k-j",
                       "for (int64_t k = 0; k + 1 < K; k++) { /* i-k-j"),
    "wrong_sign": ("                c[j] += prod;", "                c[j] -= prod;"),
    "bf16_shift": ("((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    "fp16_bias": ("ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    "fp16_subnormal_scale": ("ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    "conv_pad_sign": ("\n        const int64_t h = p * jb->sh - jb->ph + r * jb->dh;",
                      "\n        const int64_t h = p * jb->sh + jb->ph + r * jb->dh - 2 * jb->ph * (p > 0);"),
    "conv_swapped_rs": ("const uint16_t *wp = jb->w + ((k * jb->R + r) * jb->S + s) * jb->C;",
                        "const uint16_t *wp = jb->w + ((k * jb->R + (jb->R - 1 - r)) * jb->S + s) * jb->C;"),
    "sample_no_abs": ("            sacc += fabs(a * b);", "            sacc += a * b;"),
    "sample_B_transposed": ("jb->b_col_major ? jb->B[j * jb->ldb + k] : jb->B[k * jb->ldb + j]",
                            "jb->b_col_major ? jb->B[k * jb->ldb + j] : jb->B[j * jb->ldb + k]"),
    "conv_dilation_ignored": ("\n            const int64_t w = q * jb->sw - jb->pw + s * jb->dw;",
                              "\n            const int64_t w = q * jb->sw - jb->pw + s;"),
    # convolution gradients
    "dgrad_stride_divisibility_ignored": ("if (pnum < 0 || pnum % jb->sh != 0) continue;", "if (pnum < 0) continue;"),
    "dgrad_pad_sign": ("const int64_t pnum = h + jb->ph - r * jb->dh;", "const int64_t pnum = h - jb->ph - r * jb->dh;"),
    "dgrad_filter_flipped": ("jb->w[((k * jb->R + r) * jb->S + s) * jb->C + c]",
                             "jb->w[((k * jb->R + (jb->R - 1 - r)) * jb->S + (jb->S - 1 - s)) * jb->C + c]"),
    "dgrad_width_dilation_ignored": ("const int64_t qnum = w + jb->pw - s * jb->dw;",
                                     "const int64_t qnum = w + jb->pw - s;"),
    "dgrad_q_divided_by_sh": ("const int64_t q = qnum / jb->sw;", "const int64_t q = qnum / jb->sh;"),
    "wgrad_stride_ignored": ("\n            const int64_t h = p * jb->sh - jb->ph + r * jb->dh;",
                             "\n            const int64_t h = p - jb->ph + r * jb->dh;"),
    "wgrad_rs_decoded_swapped": ("const int64_t s = f % jb->S; f /= jb->S;\n        const int64_t r = f % jb->R; f /= jb->R;",
                                 "const int64_t r = f % jb->R; f /= jb->R;\n        const int64_t s = f % jb->S; f /= jb->S;"),
    "wgrad_dy_from_next_pixel": ("dec(jb->dy[((n * jb->P + p) * jb->Q + q) * jb->K + k], jb->dtype)",
                                 "dec(jb->dy[((n * jb->P + p) * jb->Q + (q + 1) % jb->Q) * jb->K + k], jb->dtype)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation target for {name} not found exactly once"
    msrc = tmp_path / "mutant.c"
    msrc.write_text(src.replace(old, new))
    lib = build(out=str(tmp_path / "libmutant.so"), src=str(msrc))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            ok, _ = pin(orc)
        except Exception:  # a mutant may also make an entry point reject or crash-free misbehave
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
    os.remove(lib)
