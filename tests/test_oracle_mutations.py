"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of the oracle's C source (on the
CPU, in a temporary directory), builds it, and runs the pin suite against the
copy in a child process. The suite must fail for every planted mistake. This
checks the pins, not the oracle: the real oracle is never modified.
"""

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

MUTANTS = {
    "weights_lx_ly_swapped": ("double wy = i ? c->ly : 1.0 - c->ly;",
                              "double wy = i ? c->lx : 1.0 - c->lx;"),
    "loc_x_grad_missing_W": ("grad_loc[2 * p] = (double)W * a * dot_x;",
                             "grad_loc[2 * p] = a * dot_x;"),
    "loc_y_grad_uses_W": ("grad_loc[2 * p + 1] = (double)H * a * dot_y;",
                          "grad_loc[2 * p + 1] = (double)W * a * dot_y;"),
    "x_slope_sign_flipped": ("double sx = (1.0 - c.ly) * (a01 - a00) + c.ly * (a11 - a10);",
                             "double sx = (1.0 - c.ly) * (a00 - a01) + c.ly * (a11 - a10);"),
    "corner_transposed": ("int64_t row = start + (c->y0 + i) * W + (c->x0 + j);",
                          "int64_t row = start + (c->y0 + j) * W + (c->x0 + i);"),
    "flat_index_bounds_check": ("return yy >= 0 && yy < H && xx >= 0 && xx < W;",
                                "return yy * W + xx >= 0 && yy * W + xx < H * W;"),
    "no_half_pixel_shift": ("float xf = fmaf((float)loc_x, (float)W, -0.5f);",
                            "float xf = fmaf((float)loc_x, (float)W, 0.0f);"),
    "level_start_ignored": ("starts[l] = level_start ? level_start[l] : acc;",
                            "starts[l] = acc;"),
    "grad_value_missing_A": ("double coef = a * corner_weight(&c, i, j);",
                             "double coef = corner_weight(&c, i, j);"),
    "two_roundings_in_mapping": ("float xf = fmaf((float)loc_x, (float)W, -0.5f);",
                                 "volatile float xw = (float)loc_x * (float)W; float xf = xw - 0.5f;"),
    "grad_attn_scaled_by_A": ("grad_attn[p] = dot_s;", "grad_attn[p] = a * dot_s;"),
    "batch_offset_dropped": ("return value + ((b * S + row) * M + m) * D;",
                             "return value + ((0 * b * S + row) * M + m) * D;"),
    "forward_missing_A": ("o[d] += a * sample[d];", "o[d] += sample[d];"),
    "y_weight_from_wrong_corner": ("double sy = (1.0 - c.lx) * (a10 - a00) + c.lx * (a11 - a01);",
                                   "double sy = (1.0 - c.lx) * (a10 - a00) + c.lx * (a11 - a10);"),
    # the rounding statistics of the grad_value scatter
    "stats_abs_of_upstream_only": ("as[d] += fabs(term * g[d]);", "as[d] += term * fabs(g[d]);"),
    "stats_signed_terms": ("as[d] += fabs(term * g[d]);", "as[d] += term * g[d];"),
    "stats_count_is_a_flag": ("count[(b * S + row) * M + m] += 1;",
                              "count[(b * S + row) * M + m] = 1;"),
    "stats_corner_weight_dropped": ("double term = a * corner_weight(&c, i, j);",
                                    "double term = a;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "msda_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(src=str(mutant_src), out=str(tmp_path / "libmutant.so"))
    env = dict(os.environ, MSDA_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"


# Mistakes planted in a copy of oracle/module.py (the steps around the core);
# the copy is loaded as a module object and the module pins must fail on it.
MODULE_MUTANTS = {
    "offset_x_scaled_by_H": ("loc[:, :, :, l, :, 0] = r[:, :, None, None, 0] + off[:, :, :, l, :, 0] / W",
                             "loc[:, :, :, l, :, 0] = r[:, :, None, None, 0] + off[:, :, :, l, :, 0] / H"),
    "softmax_per_level": ("attn = softmax_lk(logits).reshape(B, Q, M, L, K)",
                          "attn = softmax_lk(logits.reshape(B, Q, M, L, K))"),
    "softmax_grad_missing_inner": ("g_logits = af * (gf - inner)", "g_logits = af * gf"),
    "grad_offset_unscaled": ("g_off[:, :, :, l, :, 1] = gl[:, :, :, l, :, 1] / H",
                             "g_off[:, :, :, l, :, 1] = gl[:, :, :, l, :, 1]"),
    "grad_ref_one_level": ("g_ref = per_level if ref_per_level else per_level.sum(axis=2)",
                           "g_ref = per_level if ref_per_level else per_level[:, :, 0]"),
    "heads_split_transposed": ("value = value.reshape(B, S, M, D)",
                               "value = value.reshape(B, S, D, M).transpose(0, 1, 3, 2).copy()"),
    "per_level_reference_ignored": ("return ref if ref.ndim == 3 else ref[:, :, l, :]",
                                    "return ref if ref.ndim == 3 else ref[:, :, 0, :]"),
    "output_proj_grad_transposed": ('grads["output_proj.weight"] = g2.T @ core.reshape(-1, core.shape[-1])',
                                    'grads["output_proj.weight"] = (g2.T @ core.reshape(-1, core.shape[-1])).T'),
    "query_grad_drops_logits": ('g_log2 @ p["attention_weights.weight"]).reshape(B, Q, C)',
                                '0 * g_log2 @ p["attention_weights.weight"]).reshape(B, Q, C)'),
}


@pytest.mark.parametrize("name", sorted(MODULE_MUTANTS))
def test_module_pins_catch_planted_mistake(name):
    import importlib.util
    import test_oracle_module_pins as pins
    src = open(os.path.join(ROOT, "oracle", "module.py")).read()
    old, new = MODULE_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    spec = importlib.util.spec_from_loader(f"oracle._mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    failed = []
    for check in pins.CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"module pins did not catch mutant {name}"
