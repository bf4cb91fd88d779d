"""Plant plausible mistakes in a copy of the oracle's C source (CPU only) and
require that at least one pin in oracle_checks.py catches each of them.

This shows the pins are strong enough that a dropped term, a wrong sign, a
wrong divisor or index, or a rounding slip anywhere in the oracle would not go
unnoticed.  The mutated copies are built in a temporary directory; the real
oracle is untouched."""
import os
import shutil

import pytest

import oracle
import oracle_checks

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("decode_bias", "e - 127 - 7", "e - 126 - 7"),
    ("decode_subnormal_quantum", "ldexp((double)f, -133)", "ldexp((double)f, -134)"),
    ("encode_ties_up", "return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    ("encode_truncate", "if (frac > 0.5) return fl + 1.0;", "if (frac > 2.0) return fl + 1.0;"),
    ("encode_subnormal_floor", "if (q < -133) q = -133;", "if (q < -140) q = -140;"),
    ("encode_no_overflow", "if (e >= 255) return", "if (e >= 256) return"),
    ("residual_subtract", "if (c->r) v += orc_bf16_decode(c->r[base + j]);",
     "if (c->r) v -= orc_bf16_decode(c->r[base + j]);"),
    ("rms_divisor", "sqrt(ss / (double)H + c->eps)", "sqrt(ss / (double)(H - 1) + c->eps)"),
    ("rms_eps_outside", "1.0 / sqrt(ss / (double)H + c->eps)",
     "1.0 / (sqrt(ss / (double)H) + c->eps)"),
    ("rms_no_weight", "s[j] * rstd * orc_bf16_decode(c->w[j])", "s[j] * rstd"),
    ("rms_weight_index", "s[j] * rstd * orc_bf16_decode(c->w[j])",
     "s[j] * rstd * orc_bf16_decode(c->w[H - 1 - j])"),
    ("rms_abs_sum", "ss += s[j] * s[j];", "ss += fabs(s[j]);"),
    ("ln_unbiased", "sq / (double)H", "sq / (double)(H - 1)"),
    ("ln_one_pass_var", "const double d = orc_bf16_decode(xr[j]) - mu;",
     "const double d = orc_bf16_decode(xr[j]);"),
    ("ln_no_bias", "+\n                              orc_bf16_decode(c->b[j]);",
     "+\n                              0.0;"),
    ("ln_mean_sign", "(orc_bf16_decode(xr[j]) - mu) * rstd", "(orc_bf16_decode(xr[j]) + mu) * rstd"),
    ("ln_mean_divisor", "const double mu = sum / (double)H;",
     "const double mu = sum / (double)(H + 1);"),
    ("lnb_drop_c1", "(g - c1 - lnb_xhat(c, i, j) * c2)", "(g - lnb_xhat(c, i, j) * c2)"),
    ("lnb_drop_c2", "(g - c1 - lnb_xhat(c, i, j) * c2)", "(g - c1)"),
    ("lnb_sign_c1", "(g - c1 - lnb_xhat(c, i, j) * c2)", "(g + c1 - lnb_xhat(c, i, j) * c2)"),
    ("lnb_no_rstd", "c->dx[i * H + j] = c->rstd[i] * (", "c->dx[i * H + j] = 1.0 * ("),
    ("lnb_g_without_w", "const double g = orc_bf16_decode(c->dy[i * H + j]) * orc_bf16_decode(c->w[j]);\n            sum_g",
     "const double g = orc_bf16_decode(c->dy[i * H + j]);\n            sum_g"),
    ("lnb_xhat_sign", "(orc_bf16_decode(c->x[i * c->hidden + j]) - c->mean[i]) * c->rstd[i]",
     "(orc_bf16_decode(c->x[i * c->hidden + j]) + c->mean[i]) * c->rstd[i]"),
    ("lnb_dweight_no_xhat", "dw += d * lnb_xhat(c, i, j);", "dw += d;"),
    ("lnb_dbias_scaled", "db += d;", "db += d * lnb_xhat(c, i, j);"),
    ("lnb_c2_divisor", "const double c2 = sum_gx / (double)H;",
     "const double c2 = sum_gx / (double)(H - 1);"),
    ("lnb_cols_skip_first_row", "for (int64_t i = 0; i < c->rows; ++i) {\n            const double d",
     "for (int64_t i = 1; i < c->rows; ++i) {\n            const double d"),
    ("rmsb_divisor", "return 1.0 / sqrt(ss / (double)c->hidden + c->eps);",
     "return 1.0 / sqrt(ss / (double)(c->hidden - 1) + c->eps);"),
    ("rmsb_drop_c", "double v = rstd * (g - xhat * cc);", "double v = rstd * g;"),
    ("rmsb_sign_c", "double v = rstd * (g - xhat * cc);", "double v = rstd * (g + xhat * cc);"),
    ("rmsb_c_divisor", "const double cc = sum_gx / (double)H;",
     "const double cc = sum_gx / (double)(H - 1);"),
    ("rmsb_dres_subtracted", "if (c->dres) v += orc_bf16_decode(c->dres[i * H + j]);",
     "if (c->dres) v -= orc_bf16_decode(c->dres[i * H + j]);"),
    ("rmsb_dw_no_rstd", "(orc_bf16_decode(c->x[i * c->hidden + j]) * c->rstd[i]);",
     "orc_bf16_decode(c->x[i * c->hidden + j]);"),
    ("rmsb_gx_no_w", "orc_bf16_decode(c->w[j]);\n            sum_gx",
     "1.0;\n            sum_gx"),
    ("rmsb_gx_no_rstd", "sum_gx += g * orc_bf16_decode(c->x[i * H + j]) * rstd;",
     "sum_gx += g * orc_bf16_decode(c->x[i * H + j]);"),
]


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def test_mutant_list_applies_cleanly():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) >= 1, f"mutant {name}: text not found in oracle.c"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(workdir, name, old, new):
    src = open(SRC).read()
    assert old in src
    d = workdir / name
    d.mkdir()
    shutil.copy(os.path.join(os.path.dirname(SRC), "oracle.h"), d / "oracle.h")
    (d / "oracle.c").write_text(src.replace(old, new))
    lib = oracle.build(sources=[str(d / "oracle.c")], out_path=str(d / "liboracle.so"))
    o = oracle.Oracle(lib)
    caught = []
    for check in oracle_checks.ALL_CHECKS:
        try:
            check(o)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin catches the planted mistake '{name}'"


# ---- the fp32-activation functions (oracle_f32.c) against oracle_checks_f32
import oracle_checks_f32  # noqa: E402

SRC_F32 = oracle.F32_SOURCE

MUTANTS_F32 = [
    ("f32_residual_subtract", "if (c->r) v += (double)c->r[base + j];",
     "if (c->r) v -= (double)c->r[base + j];"),
    ("f32_residual_biased_rounding", "c->res_out[base + j] = (float)s[j];",
     "c->res_out[base + j] = (float)(s[j] * (1.0 + 0x1p-30));"),
    ("f32_rms_eps_outside", "const double rstd = 1.0 / sqrt(ss / (double)H + c->eps);\n        if",
     "const double rstd = 1.0 / (sqrt(ss / (double)H) + c->eps);\n        if"),
    ("f32_rms_no_weight", "c->out[base + j] = s[j] * rstd * (double)c->w[j];",
     "c->out[base + j] = s[j] * rstd;"),
    ("f32_ln_unbiased", "sqrt(sq / (double)H + c->eps)", "sqrt(sq / (double)(H - 1) + c->eps)"),
    ("f32_ln_no_bias", "* (double)c->w[j] + (double)c->b[j];", "* (double)c->w[j];"),
    ("f32_ln_mean_sign", "c->y[i * H + j] = ((double)xr[j] - mu)",
     "c->y[i * H + j] = ((double)xr[j] + mu)"),
    ("f32_lnb_drop_c1", "(g - c1 - lnb32_xhat(c, i, j) * c2)", "(g - lnb32_xhat(c, i, j) * c2)"),
    ("f32_lnb_xhat_sign", "((double)c->x[i * c->hidden + j] - c->mean[i]) * c->rstd[i];",
     "((double)c->x[i * c->hidden + j] + c->mean[i]) * c->rstd[i];"),
    ("f32_lnb_dbias_scaled", "db += d;", "db += d * lnb32_xhat(c, i, j);"),
    ("f32_rmsb_drop_c", "double v = rstd * (g - xhat * cc);", "double v = rstd * g;"),
    ("f32_rmsb_dres_subtracted", "if (c->dres) v += (double)c->dres[i * H + j];",
     "if (c->dres) v -= (double)c->dres[i * H + j];"),
    ("f32_rmsb_dw_no_rstd", "((double)c->x[i * c->hidden + j] * c->rstd[i]);",
     "(double)c->x[i * c->hidden + j];"),
]


def test_f32_mutant_list_applies_cleanly():
    src = open(SRC_F32).read()
    for name, old, _ in MUTANTS_F32:
        assert src.count(old) >= 1, f"mutant {name}: text not found in oracle_f32.c"


@pytest.mark.parametrize("name,old,new", MUTANTS_F32, ids=[m[0] for m in MUTANTS_F32])
def test_f32_pins_catch_mutant(workdir, name, old, new):
    src = open(SRC_F32).read()
    d = workdir / name
    d.mkdir()
    shutil.copy(os.path.join(os.path.dirname(SRC), "oracle.h"), d / "oracle.h")
    shutil.copy(SRC, d / "oracle.c")
    (d / "oracle_f32.c").write_text(src.replace(old, new))
    lib = oracle.build(sources=[str(d / "oracle.c"), str(d / "oracle_f32.c")],
                       out_path=str(d / "liboracle.so"))
    o = oracle.Oracle(lib)
    caught = []
    for check in oracle_checks_f32.F32_CHECKS:
        try:
            check(o)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no fp32 pin catches the planted mistake '{name}'"
