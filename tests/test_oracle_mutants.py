"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of ``oracle/oracle.c`` (on the CPU,
never on a GPU), builds it, and runs the oracle pin suite against it in a
subprocess; the suite must fail.  The mistakes are the kinds the pins are
meant to catch: a dropped term, a wrong sign, bound or index, a swapped
operand or draw, a wrong rounding rule.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from conftest import ROOT

import oracle

PIN_FILES = ["test_oracle_philox.py", "test_oracle_math.py", "test_oracle_sampler.py",
             "test_oracle_rounding.py", "test_oracle_pixels.py"]

# (name, original text, planted text)
MUTANTS = [
    ("philox_no_key_bump", "k1 += 0xBB67AE85u;", "k1 += 0u;"),
    ("philox_lo_hi_swap", "uint32_t y1 = (uint32_t)prod_b;", "uint32_t y1 = (uint32_t)(prod_b >> 32);"),
    ("stream_counter_layout", "(uint32_t)block, (uint32_t)(block >> 32), (uint32_t)n, (uint32_t)(n >> 32)",
     "(uint32_t)n, (uint32_t)(n >> 32), (uint32_t)block, (uint32_t)(block >> 32)"),
    ("u01_23_bits", "return (float)(w >> 8) * 0x1p-24f;", "return (float)(w >> 9) * 0x1p-23f;"),
    ("randint_exclusive", "(int64_t)hi - (int64_t)lo + 1", "(int64_t)hi - (int64_t)lo"),
    ("gate_not_strict", "if (or_u01(words[k++]) < erase_p) {", "if (or_u01(words[k++]) <= erase_p) {"),
    ("flip_not_strict", "p->flip = or_u01(words[k++]) < flip_p;", "p->flip = or_u01(words[k++]) <= flip_p;"),
    ("scale_ratio_words_swapped", "or_erase_dims(words[k], words[k + 1],", "or_erase_dims(words[k + 1], words[k],"),
    ("sides_swapped", "float side_h = sqrtf(erase_area * aspect);\n    float side_w = sqrtf(erase_area / aspect);",
     "float side_h = sqrtf(erase_area / aspect);\n    float side_w = sqrtf(erase_area * aspect);"),
    ("ratio_not_log_uniform", "float aspect = or_expf(log_aspect);", "float aspect = log_aspect;"),
    ("round_half_even", "float eh_f = roundf(side_h);", "float eh_f = rintf(side_h);"),
    ("accept_le_H", "eh_f < (float)H && ew_f < (float)W", "eh_f <= (float)H && ew_f < (float)W"),
    ("nine_attempts", "for (int32_t a = 0; a < 10; ++a) {", "for (int32_t a = 0; a < 9; ++a) {"),
    ("row_col_swapped", "p->i = or_randint(0, H - eh, words[k++]);\n                    p->j = or_randint(0, W - ew, words[k++]);",
     "p->j = or_randint(0, W - ew, words[k++]);\n                    p->i = or_randint(0, H - eh, words[k++]);"),
    ("flip_reverses_bytes", "uint8_t x = img[((size_t)h * (size_t)W + (size_t)src_w) * (size_t)C + (size_t)c];",
     "uint8_t x = img[((size_t)h * (size_t)W + (size_t)src_w) * (size_t)C + (size_t)(C - 1 - c)];"),
    ("erase_in_source_frame", "int in_rect = p->erase && h >= p->i && h < p->i + p->eh && w >= p->j && w < p->j + p->ew;\n            int32_t src_w = p->flip ? (W - 1 - w) : w;",
     "int32_t src_w = p->flip ? (W - 1 - w) : w;\n            int in_rect = p->erase && h >= p->i && h < p->i + p->eh && src_w >= p->j && src_w < p->j + p->ew;"),
    ("erase_one_channel", "if (in_rect) {", "if (in_rect && c == 0) {"),
    ("normalize_order", "out[o] = (float)((v - (double)mean[c]) / (double)std[c]);",
     "out[o] = (float)(v / (double)std[c] - (double)mean[c]);"),
    ("normalize_fp32_mul_sub", "double v = (double)x / 255.0;\n                    out[o] = (float)((v - (double)mean[c]) / (double)std[c]);",
     "float v = (float)x * (1.0f / (255.0f * std[c]));\n                    out[o] = v - mean[c] / std[c];"),
    ("exp_truncated", "return (float)expl((long double)L);", "return nextafterf((float)expl((long double)L), 0.0f);"),
    ("log_ratio_fp32_libm", "return (float)logl((long double)r);", "return nextafterf((float)logl((long double)r), 0.0f);"),
    # the rounding sequence of one attempt (page section 10 uniform(), section 12)
    ("fma_area_fraction", "float scale_draw = or_u01(w_scale) * scale_span;\n    float target_fraction = scale_min + scale_draw;",
     "float target_fraction = fmaf(or_u01(w_scale), scale_span, scale_min);"),
    ("fma_log_aspect", "float log_draw = or_u01(w_ratio) * log_span;\n    float log_aspect = log_rmin + log_draw;",
     "float log_aspect = fmaf(or_u01(w_ratio), log_span, log_rmin);"),
    ("sqrt_in_double", "float side_h = sqrtf(erase_area * aspect);\n    float side_w = sqrtf(erase_area / aspect);",
     "float side_h = (float)sqrt((double)erase_area * (double)aspect);\n    float side_w = (float)sqrt((double)erase_area / (double)aspect);"),
    ("lerp_two_products", "float target_fraction = scale_min + scale_draw;",
     "float target_fraction = scale_min * (1.0f - or_u01(w_scale)) + scale_max * or_u01(w_scale);\n    (void)scale_draw;"),
    ("exponent_in_extended", "float aspect = or_expf(log_aspect);",
     "float aspect = (float)expl((long double)log_rmin + (long double)or_u01(w_ratio) * ((long double)log_rmax - (long double)log_rmin));\n    (void)log_aspect;"),
]


def _build_and_run(tmpdir: str, name: str, old: str, new: str) -> tuple[str, int, str]:
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) == 1, f"{name}: anchor text must occur once"
    path = os.path.join(tmpdir, f"{name}.c")
    lib = os.path.join(tmpdir, f"lib{name}.so")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", *oracle.CFLAGS, path, "-o", lib, "-lm", "-lpthread"], check=True,
                   capture_output=True)
    env = dict(os.environ, ORACLE_LIB=lib)
    tests = [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *tests],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=600)
    return name, r.returncode, r.stdout[-600:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda m: _build_and_run(str(tmp_path), *m), MUTANTS))
    survived = [(name, out) for name, rc, out in results if rc == 0]
    assert not survived, survived
    for name, rc, out in results:
        assert rc == 1, (name, rc, out)  # a test failure, not a crash or collection error


def test_unmutated_copy_passes(tmp_path):
    name, rc, out = _build_and_run(str(tmp_path), "identity", "float or_u01(uint32_t w)",
                                   "float or_u01(uint32_t w)")
    assert rc == 0, out
