"""The CPU oracle against its pins, and mutated oracles against the same pins.

Every pin in oracle_pins.ALL_PINS must pass on the oracle.  Each mutant below
plants one plausible mistake in a copy of oracle.c (a dropped term, a wrong
sign or index, a swapped operand); at least one pin must fail on each, which
shows the pins can see that class of mistake.  Mutants are compiled and run
on the CPU only.
"""
import ctypes
import importlib
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from tests import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


MUTANTS = {
    "slot_dropped": ("int64_t slot = (int64_t)c % ORACLE_PAGE;", "int64_t slot = 0;"),
    "page_divisor": ("int64_t lp = (int64_t)c / ORACLE_PAGE;", "int64_t lp = (int64_t)c / 8;"),
    "mask_ignored": ("if (pp < 0 || pp >= n_phys_pages) return -1;",
                     "if (pp < 0 || pp >= n_phys_pages) pp = 0;"),
    "softmax_scale_dropped": ("return sm_scale * oracle_half_to_double(P->k_scales[phys]) * dot;",
                              "return oracle_half_to_double(P->k_scales[phys]) * dot;"),
    "k_scale_dropped": ("return sm_scale * oracle_half_to_double(P->k_scales[phys]) * dot;",
                        "return sm_scale * dot;"),
    "v_scale_is_k_scale": ("double w = p * oracle_half_to_double(P->v_scales[ph]);",
                           "double w = p * oracle_half_to_double(P->k_scales[ph]);"),
    "dims_reversed": ("dot += (double)qrow[d] * (double)k[d];",
                      "dot += (double)qrow[d] * (double)k[P->head_dim - 1 - d];"),
    "exp_sign": ("double p = exp(score(P, qrow, ph, sm_scale) - m);",
                 "double p = exp(m - score(P, qrow, ph, sm_scale));"),
    "lse_without_max": ("lse[k * n_rows + r] = m + log(l);", "lse[k * n_rows + r] = log(l);"),
    "no_normalisation": ("for (int64_t d = 0; d < D; ++d) o[d] /= l;\n            lse[k * n_rows + r]",
                         "(void)0;\n            lse[k * n_rows + r]"),
    "prompt_no_normalisation": ("for (int64_t d = 0; d < D; ++d) o[d] /= l;\n            lse[u]",
                                "(void)0;\n            lse[u]"),
    "merge_weight_sign": ("double w = exp(mc - M);", "double w = exp(M - mc);"),
    "merge_l_unweighted": ("L += l[u * n_chunks + c] * w;", "L += l[u * n_chunks + c];"),
    "half_bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "half_subnormal": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "wrong_query_row": ("attend_range(&P, q + (i * n_rows + r) * D, sel + i * sel_stride, 0, n_sel[i],",
                        "attend_range(&P, q + (i * n_rows + (n_rows - 1 - r)) * D, sel + i * sel_stride, 0, n_sel[i],"),
    "chunk_end_off_by_one": ("int64_t j0 = c * chunk, j1 = j0 + chunk;",
                             "int64_t j0 = c * chunk, j1 = j0 + chunk - 1;"),
    "prompt_excludes_own_cell": ("int64_t n_visible = p + 1 > 0 ? p + 1 : 0;",
                                 "int64_t n_visible = p > 0 ? p : 0;"),
    "prompt_ignores_pos0": ("int64_t p = pos0 + t;", "int64_t p = t;"),
    "prompt_head_major_rows": ("attend_range(&P, q + (t * n_qheads + h) * D, list,",
                               "attend_range(&P, q + (h * n_q + t) * D, list,"),
    "prompt_sees_one_more": ("int64_t n_visible = p + 1 > 0 ? p + 1 : 0;",
                             "int64_t n_visible = p + 2 > 0 ? p + 2 : 0;"),
    "half_truncates": ("double q = rint((2.0 * m - 1.0) * 1024.0);",
                       "double q = floor((2.0 * m - 1.0) * 1024.0);"),
    "half_bias_off": ("return sign | (uint16_t)((e + 15) << 10) | (uint16_t)q;",
                      "return sign | (uint16_t)((e + 14) << 10) | (uint16_t)q;"),
    "quant_truncates": ("q = rintf(x[d] / s);", "q = truncf(x[d] / s);"),
    "quant_no_clamp": ("if (q > 127.0f) q = 127.0f;", "(void)0;"),
    "quant_scale_128": ("float s32 = amax / 127.0f;", "float s32 = amax / 128.0f;"),
    "quant_no_saturation": ("if (s32 > 65504.0f) s32 = 65504.0f;", "(void)0;"),
    "append_ignores_pos0": ("int64_t c = pos0 + t;\n        if (c < 0 || c > INT32_MAX) continue;",
                            "int64_t c = t;\n        if (c < 0 || c > INT32_MAX) continue;"),
    "append_kv_swapped": ("quantise_row(v_new + t * head_dim, head_dim, v_codes + ph * head_dim,",
                          "quantise_row(k_new + t * head_dim, head_dim, v_codes + ph * head_dim,"),
    "append_scale_stride_ignored": ("k_scales + ph * scale_stride);", "k_scales + ph);"),
    "qsa_dead_ignored": ("if (!dead[i * max_blocks + b] && b * block_cells < (int64_t)n_visible[u]) {",
                         "if (b * block_cells < (int64_t)n_visible[u]) {"),
    "qsa_visible_off_by_one": ("if (!dead[i * max_blocks + b] && b * block_cells < (int64_t)n_visible[u]) {",
                               "if (!dead[i * max_blocks + b] && b * block_cells <= (int64_t)n_visible[u]) {"),
    "qsa_head_dropped": ("for (int64_t h = 0; h < n_heads; ++h) {", "for (int64_t h = 1; h < n_heads; ++h) {"),
    "qsa_dims_reversed": ("dot += (double)q[h * idx_dim + d] * (double)k[h * idx_dim + d];",
                          "dot += (double)q[h * idx_dim + d] * (double)k[h * idx_dim + idx_dim - 1 - d];"),
    "qsa_first_row_only": ("for (int64_t r = 0; r < n_rows; ++r) {\n                double s",
                           "for (int64_t r = 0; r < 1; ++r) {\n                double s"),
    "qsa_ties_reversed": ("return (a->b > b->b) - (a->b < b->b);", "return (a->b < b->b) - (a->b > b->b);"),
    "qsa_lowest_scores": ("if (a->c > b->c) return -1;\n    if (a->c < b->c) return 1;",
                          "if (a->c > b->c) return 1;\n    if (a->c < b->c) return -1;"),
    "qsa_extent_not_clipped": ("c < (b + 1) * block_cells && c < extent;", "c < (b + 1) * block_cells;"),
    "qsa_extent_min_of_rows": ("if ((int64_t)n_visible[i * n_rows + r] > extent) extent",
                               "if ((int64_t)n_visible[i * n_rows + r] < extent) extent"),
    "qsa_k_plus_one": ("for (int64_t j = 0; j < k_blocks && j < max_blocks", "for (int64_t j = 0; j <= k_blocks && j < max_blocks"),
    "qsa_takes_masked": ("&& rk[j].c > -INFINITY; ++j)", "; ++j)"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    path = tmp_path / f"m_{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"m_{name}.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-std=c11", str(path), "-o", str(so), "-lm"],
                   check=True)
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    so = _build_mutant(tmp_path, name, old, new)
    # load a private copy of the oracle wrapper bound to the mutant library
    spec = importlib.util.spec_from_file_location(f"oracle_mut_{name}",
                                                  os.path.join(os.path.dirname(ORACLE_SRC),
                                                               "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB = so
    mod._SRC = so  # prevent a rebuild over the mutant
    failed = []
    with np.errstate(all="ignore"):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(mod)
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
