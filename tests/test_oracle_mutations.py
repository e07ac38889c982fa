"""The oracle's pins catch plausible mistakes.  CPU only.

Each case plants one mistake in a temporary copy of oracle/ftm_oracle.c: a
dropped term, a wrong scale, a swapped operand, a wrong index or a wrong
rounding rule.  The copy is built with the oracle's own compiler flags in a
temporary directory and loaded as a separate oracle module.  The pins of
tests/test_oracle_pins.py then run against it, and at least one must fail.
The committed oracle is never modified and holds no switch for any of
these mistakes.  Every planted mistake keeps all memory accesses in
bounds."""
import importlib.util
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

# (name, text in ftm_oracle.c, replacement)
MUTATIONS = [
    ("K bias dropped",
     "x[d] = P->bias ? a + act_get_f32(P->bias, bias_off + d, P->act_dt) : a;",
     "x[d] = (P->bias && which) ? a + act_get_f32(P->bias, bias_off + d, P->act_dt) : a;"),
    ("K and V bias blocks swapped",
     "const size_t bias_off = (size_t)(P->H + which * P->Hkv + j) * D;",
     "const size_t bias_off = (size_t)(P->H + (1 - which) * P->Hkv + j) * D;"),
    ("query bias dropped",
     "if (P->bias) v += (double)act_get_f32(P->bias, (size_t)h * D + d, P->act_dt);",
     "(void)0;"),
    ("query bias of the wrong head",
     "if (P->bias) v += (double)act_get_f32(P->bias, (size_t)h * D + d, P->act_dt);",
     "if (P->bias) v += (double)act_get_f32(P->bias, (size_t)j * D + d, P->act_dt);"),
    ("scale 1/D instead of 1/sqrt(D)",
     "const double inv_sqrt_d = 1.0 / sqrt((double)D);",
     "const double inv_sqrt_d = 1.0 / (double)D;"),
    ("maximum not subtracted",
     "s[i] = exp(s[i] - m);",
     "s[i] = exp(s[i]);"),
    ("weights not normalised",
     "for (int i = 0; i < L; ++i) s[i] /= z;",
     "(void)z;"),
    ("scores from V instead of K",
     "acc += qh[d] * cache_get(P->k_cache, (kv_base + i) * D + d, P->kv_dt, ks);",
     "acc += qh[d] * cache_get(P->v_cache, (kv_base + i) * D + d, P->kv_dt, ks);"),
    ("head map h mod Hkv instead of h / G",
     "const int j = h / G;",
     "const int j = h % P->Hkv;"),
    ("new row appended one position early",
     "    append_row(P, b, j, L - 1, 0);\n    append_row(P, b, j, L - 1, 1);",
     "    append_row(P, b, j, L > 1 ? L - 2 : 0, 0);\n    append_row(P, b, j, L > 1 ? L - 2 : 0, 1);"),
    ("last position left out of the attention",
     "for (int g = 0; g < G; ++g) attend_head(P, b, j * G + g, L);",
     "for (int g = 0; g < G; ++g) attend_head(P, b, j * G + g, L > 1 ? L - 1 : L);"),
    ("V scale read from the K plane",
     "vs = (double)P->kv_scales[(((size_t)1 * P->B + b) * P->Hkv + j) * P->Lmax + i];",
     "vs = (double)P->kv_scales[(((size_t)0 * P->B + b) * P->Hkv + j) * P->Lmax + i];"),
    ("INT8 scale absmax/128",
     "const float scale = amax / 127.0f;",
     "const float scale = amax / 128.0f;"),
    ("INT8 codes rounded half away from zero",
     "float c = rintf(x[d] / scale);",
     "float c = roundf(x[d] / scale);"),
    ("binary16/bfloat16 rounding truncates",
     "const double r = rint(a / spacing) * spacing;",
     "const double r = floor(a / spacing) * spacing;"),
    ("subnormal exponent off by one",
     "v = ldexp((double)f, 1 - bias - fbits);",
     "v = ldexp((double)f, -bias - fbits);"),
]


def pin_battery():
    """(name, call) pairs over the pins, cheap and broad ones first."""
    b = []
    for dt in ("f32", "f16", "bf16", "i8"):
        b.append((f"single position {dt}", lambda m, dt=dt: pins.test_single_token_output_is_v(m, dt)))
    b.append(("identical keys", pins.test_identical_keys_give_mean_of_v))
    for dt in ("f32", "f16", "bf16", "i8"):
        b.append((f"weights {dt}", lambda m, dt=dt: pins.test_weights_sum_to_one_and_vanish_past_length(m, dt)))
    b.append(("closed form", pins.test_closed_form_three_positions))
    for dt in ("f16", "i8"):
        b.append((f"grouped heads {dt}", lambda m, dt=dt: pins.test_gqa_equals_mha_with_replicated_kv(m, dt)))
    b.append(("shift invariance", pins.test_shift_invariance_needs_stable_softmax))
    b.append(("one-hot limit", pins.test_one_hot_limit))
    for dt in ("f32", "bf16", "i8"):
        b.append((f"permutation {dt}", lambda m, dt=dt: pins.test_permutation_invariance(m, dt)))
    b.append(("append only the new row", pins.test_append_touches_only_the_new_row))
    b.append(("invalid lengths", pins.test_invalid_length_gives_nan_and_no_append))
    b.append(("textbook formula", pins.test_textbook_formula_longdouble))
    b.append(("INT8 quantiser", pins.test_quantize_row_matches_torch_ops))
    for args in pins._sweep_subset():
        b.append((f"brute force {args}", lambda m, args=args: pins.test_brute_force_against_torch_float64(m, *args)))
    b.append(("binary16 decode", pins.test_f16_decode_all_patterns))
    b.append(("bfloat16 decode", pins.test_bf16_decode_all_patterns))
    for fmt in ("f16", "bf16"):
        b.append((f"{fmt} rounding", lambda m, fmt=fmt: pins.test_float_to_half_rne_matches_library(m, fmt)))
    return b


def load_variant(tmp_path, old=None, new=None):
    """The oracle module bound to a library built from a copy of the source,
    with `old` replaced by `new`."""
    src = open(oracle._SRC).read()
    if old is not None:
        assert src.count(old) == 1, f"mutation site not unique: {old}"
        src = src.replace(old, new)
    c_file = tmp_path / "ftm_oracle_variant.c"
    c_file.write_text(src)
    lib = str(tmp_path / "libftm_oracle_variant.so")
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC",
                    "-pthread", "-I", os.path.dirname(oracle._SRC), str(c_file), "-o", lib, "-lm"],
                   check=True)
    spec = importlib.util.spec_from_file_location(f"oracle_variant_{tmp_path.name}", oracle.__file__)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB = lib
    mod._lib = None
    return mod


def first_failing_pin(mod):
    for name, call in pin_battery():
        try:
            with np.errstate(all="ignore"):
                call(mod)
        except AssertionError:
            return name
    return None


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_a_pin_catches_the_planted_mistake(tmp_path, name, old, new):
    caught = first_failing_pin(load_variant(tmp_path, old, new))
    print(f"[{name}] caught by: {caught}")
    assert caught is not None, f"no pin catches: {name}"


def test_the_unmodified_copy_passes_every_pin(tmp_path):
    """The harness itself: the same build and loading path with no mistake
    planted passes the whole battery."""
    assert first_failing_pin(load_variant(tmp_path)) is None


# The paged oracle's address translation lives in oracle/__init__.py.
PAGED_MUTATIONS = [
    ("page and head axes not swapped", "        g = np.swapaxes(g, 1, 2)\n", "        pass\n"),
    ("row counted from the end of the page", "pg, row = int(tbl[b, last]), (L - 1) % P",
     "pg, row = int(tbl[b, last]), P - 1 - (L - 1) % P"),
    ("new row's page left out of the validity check", "pages_used = (L - 1) // P + 1", "pages_used = (L - 1) // P"),
    ("table columns reversed", "page_of = np.where(ok_entry, tbl, 0)", "page_of = np.where(ok_entry, tbl, 0)[:, ::-1]"),
]


def load_python_variant(tmp_path, old, new):
    """The oracle module with `old` replaced by `new` in its Python source,
    bound to the committed C library."""
    src = open(oracle.__file__).read()
    assert src.count(old) == 1, f"mutation site not unique: {old}"
    path = tmp_path / "oracle_variant.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"oracle_pyvariant_{tmp_path.name}", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB = oracle._LIB
    mod._lib = None
    return mod


def paged_battery():
    from tests import test_oracle_paged_pins as pp
    b = []
    for dt in ("f32", "f16", "bf16", "i8"):
        for P in (1, 3, 4, 16):
            b.append((f"paged {dt} P{P}", lambda m, dt=dt, P=P:
                      pp.test_paged_step_is_the_contiguous_step_on_the_described_cache(m, dt, P)))
    b.append(("identity table", pp.test_one_page_per_sequence_in_order_is_the_contiguous_layout))
    b.append(("pages outside the pool", pp.test_pages_outside_the_pool))
    return b


@pytest.mark.parametrize("name,old,new", PAGED_MUTATIONS, ids=[m[0] for m in PAGED_MUTATIONS])
def test_a_paged_pin_catches_the_planted_mistake(tmp_path, name, old, new):
    mod = load_python_variant(tmp_path, old, new)
    caught = None
    for pin, call in paged_battery():
        try:
            with np.errstate(all="ignore"):
                call(mod)
        except AssertionError:
            caught = pin
            break
    print(f"[{name}] caught by: {caught}")
    assert caught is not None, f"no paged pin catches: {name}"
