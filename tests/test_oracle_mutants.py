"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, and runs the pins against that build in
a child process. The planted mistake must make at least one pin fail (or the
child crash). The in-tree oracle is never modified.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "oracle", "msda_oracle.c")

MUTANTS = {
    "no_half_pixel": ("fmaf(u, (float)W, -0.5f)", "fmaf(u, (float)W, 0.0f)"),
    "corner_aligned_scale": ("fmaf(u, (float)W, -0.5f)", "u * (float)(W - 1)"),
    "swapped_axes": ("*x = (double)fmaf(u, (float)W, -0.5f);\n    *y = (double)fmaf(v, (float)H, -0.5f);",
                     "*x = (double)fmaf(u, (float)H, -0.5f);\n    *y = (double)fmaf(v, (float)W, -0.5f);"),
    "swapped_x_weights": ("const double wx = dx ? fx : 1.0 - fx;", "const double wx = dx ? 1.0 - fx : fx;"),
    "swapped_y_weights": ("const double wy = dy ? fy : 1.0 - fy;", "const double wy = dy ? 1.0 - fy : fy;"),
    "bounds_off_by_one": ("(xc < (double)W)", "(xc <= (double)W - 0.0 + 0.0 && xc < (double)W + 1.0)"),
    "no_row_bound": ("&& (yc >= 0.0) ", "&& 1 "),
    "row_stride_H": ("start + (int64_t)yc * W + (int64_t)xc", "start + (int64_t)yc * (W > 1 ? W - 1 : 1) + (int64_t)xc"),
    "no_level_start": ("bilinear_corners(x, y, H, W, lsi[l], c);", "bilinear_corners(x, y, H, W, 0, c);"),
    "forward_drops_weight": ("const double t = a * c[i].w * v[d];", "const double t = c[i].w * v[d];"),
    "forward_wrong_head": ("const double *v = value + ((b * Nv + c[i].row) * M + m) * D;",
                           "const double *v = value + ((b * Nv + c[i].row) * M + (M - 1 - m)) * D;"),
    "dx_sign": ("k->dw_dx = (dx ? 1.0 : -1.0) * wy;", "k->dw_dx = (dx ? -1.0 : 1.0) * wy;"),
    "dy_uses_wrong_factor": ("k->dw_dy = (dy ? 1.0 : -1.0) * wx;", "k->dw_dy = (dy ? 1.0 : -1.0) * wy;"),
    "loc_grad_chain_H_for_x": ("grad_loc[2 * p] = a * gx * (double)W;", "grad_loc[2 * p] = a * gx * (double)H;"),
    "loc_grad_drops_A": ("grad_loc[2 * p + 1] = a * gy * (double)H;", "grad_loc[2 * p + 1] = gy * (double)H;"),
    "attn_grad_drops_g": ("ga += g[d] * s;", "ga += s;"),
    "value_grad_drops_A": ("const double t = a * c[i].w * g[d];", "const double t = c[i].w * g[d];"),
    "value_grad_wrong_corner_weight": ("const double t = a * c[i].w * g[d];", "const double t = a * c[3 - i].w * g[d];"),
    # fused front-end
    "fused_offset_x_over_H": ("loc[2 * p] = fused_coord(r[0], off[2 * p], W);",
                              "loc[2 * p] = fused_coord(r[0], off[2 * p], H);"),
    "fused_no_normalizer": ("const float quotient = off / (float)size;", "const float quotient = off + 0.0f * (float)size;"),
    "fused_softmax_per_level": ("for (int64_t j = 0; j < LK; ++j) sum += exp((double)z[j] - zmax);",
                                "for (int64_t j = 0; j < K; ++j) sum += exp((double)z[j] - zmax);"),
    "fused_logit_grad_no_jacobian": ("if (grad_logits) grad_logits[p] = a * (ga[p] - s);",
                                     "if (grad_logits) grad_logits[p] = a * ga[p];"),
    "fused_ref_grad_one_head": ("grad_ref[r] += gloc[2 * p];", "grad_ref[r] += m == 0 ? gloc[2 * p] : 0.0;"),
    "fused_offset_grad_times_W": ("grad_off[2 * p] = gloc[2 * p] / (double)W;", "grad_off[2 * p] = gloc[2 * p] * (double)W;"),
    "dcn_grid_ignores_dilation": ("const float gx = (float)(wo * sw - pw + kx * dw);",
                                  "const float gx = (float)(wo * sw - pw + kx);"),
    "dcn_stride_of_other_axis": ("const float gy = (float)(ho * sh - ph + ky * dh);",
                                 "const float gy = (float)(ho * sw - ph + ky * dh);"),
    "dcn_padding_added": ("const float gx = (float)(wo * sw - pw + kx * dw);",
                          "const float gx = (float)(wo * sw + pw + kx * dw);"),
    "dcn_kernel_index_transposed": ("const int64_t ky = k / kw, kx = k % kw;",
                                    "const int64_t kx = k / kw, ky = k % kw;"),
    "dcn_offset_axes_swapped": ("*x = (double)(float)(gx + off[0]);\n    *y = (double)(float)(gy + off[1]);",
                                "*x = (double)(float)(gx + off[1]);\n    *y = (double)(float)(gy + off[0]);"),
    "dcn_mask_ignored": ("const double term = m * c[i].w * v[d];", "const double term = c[i].w * v[d];"),
    "dcn_offset_grad_without_mask": ("grad_offset[2 * p] = m * gx;", "grad_offset[2 * p] = gx;"),
    "dcn_input_grad_wrong_group": ("const size_t base = (size_t)(((b * Nv + c[i].row) * G + g) * D);\n                            for (int64_t d = 0; d < D; ++d) {\n                                const double v = input[base + d];",
                                   "const size_t base = (size_t)(((b * Nv + c[i].row) * G + (G - 1 - g)) * D);\n                            for (int64_t d = 0; d < D; ++d) {\n                                const double v = input[base + d];"),
    # term sums S (they scale every GPU parity tolerance)
    "forward_abs_inflated": ("if (oa) oa[d] += fabs(t);", "if (oa) oa[d] += 1e6 * fabs(t);"),
    "value_grad_abs_doubled": ("if (grad_value_abs) grad_value_abs[base + d] += fabs(t);",
                               "if (grad_value_abs) grad_value_abs[base + d] += 2.0 * fabs(t);"),
    "attn_grad_abs_drops_g": ("ga_abs += fabs(g[d]) * s_abs;", "ga_abs += s_abs;"),
    "loc_grad_abs_drops_W": ("grad_loc_abs[2 * p] = fabs(a) * gx_abs * (double)W;",
                             "grad_loc_abs[2 * p] = fabs(a) * gx_abs;"),
    "loc_grad_abs_drops_A": ("grad_loc_abs[2 * p + 1] = fabs(a) * gy_abs * (double)H;",
                             "grad_loc_abs[2 * p + 1] = gy_abs * (double)H;"),
    "loc_grad_abs_signed_terms": ("dsx_abs += fabs(c[i].dw_dx * vd);", "dsx_abs += c[i].dw_dx * vd;"),
    "fused_logit_abs_drops_a": ("if (grad_logits_abs) grad_logits_abs[p] = a * (ga_abs[p] + s_abs);",
                                "if (grad_logits_abs) grad_logits_abs[p] = (ga_abs[p] + s_abs);"),
    "fused_logit_abs_no_sum": ("if (grad_logits_abs) grad_logits_abs[p] = a * (ga_abs[p] + s_abs);",
                               "if (grad_logits_abs) grad_logits_abs[p] = a * ga_abs[p];"),
    "fused_offset_abs_times_W": ("grad_off_abs[2 * p] = gloc_abs[2 * p] / (double)W;",
                                 "grad_off_abs[2 * p] = gloc_abs[2 * p] * (double)W;"),
    "fused_ref_abs_one_head": ("grad_ref_abs[r] += gloc_abs[2 * p];",
                               "grad_ref_abs[r] += m == 0 ? gloc_abs[2 * p] : 0.0;"),
    "dcn_forward_abs_inflated": ("if (oa) oa[d] += fabs(term);", "if (oa) oa[d] += 1e6 * fabs(term);"),
    "dcn_input_abs_doubled": ("if (grad_input_abs) grad_input_abs[base + d] += fabs(term);",
                              "if (grad_input_abs) grad_input_abs[base + d] += 2.0 * fabs(term);"),
    "dcn_mask_abs_drops_g": ("gm_abs += fabs(gr[d] * c[i].w * v);", "gm_abs += fabs(c[i].w * v);"),
    "dcn_offset_abs_without_mask": ("grad_offset_abs[2 * p] = fabs(m) * gx_abs;",
                                    "grad_offset_abs[2 * p] = gx_abs;"),
}

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, pins
lib = oracle.library({lib!r})
for pin in pins.ALL_PINS:
    try:
        pin(lib)
    except Exception as e:
        print("CAUGHT", pin.__name__, type(e).__name__)
        sys.exit(0)
print("SURVIVED")
sys.exit(3)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    src = open(SOURCE).read()
    assert old in src, f"mutation site for {name} not found in the oracle source"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = os.path.join(tmp, "libmutant.so")
        subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                        path, "-o", lib, "-lm"], check=True)
        child = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
        r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True,
                           timeout=300)
    # a crash (negative return code) also counts as caught
    assert r.returncode != 3, f"mutant {name} survived every pin:\n{r.stdout}\n{r.stderr}"
    assert r.returncode == 0 or r.returncode < 0, f"child failed: {r.stdout}\n{r.stderr}"
