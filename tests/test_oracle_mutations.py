"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them: a dropped term, a wrong sign, a wrong or
transposed index, a dropped scale, the diagonal left out, a wrong decode."""
import os
import shutil

import pytest

import oracle
from oracle import build as obuild
import pins

MUTATIONS = {
    "diagonal_excluded": ("if (t2 <= t) {", "if (t2 < t) {"),
    "key_from_query_slot": ("nh * HS + C; /* K[b][nh][t2][:] */", "nh * HS; /* K[b][nh][t2][:] */"),
    "query_row_off_by_one": ("t * C3 + nh * HS;   /* Q[b][nh][t][:] */",
                             "t * C3 + nh * HS + 1;   /* Q[b][nh][t][:] */"),
    "scale_dropped": ("orow[t2] = (float)(acc * (double)scale);", "orow[t2] = (float)acc;"),
    "scale_squared": ("return (float)(1.0 / sqrt((double)HS));", "return (float)(1.0 / (double)HS);"),
    "w_transposed": ("elem(W, dtype, n * ldw + k)", "elem(W, dtype, k * ldw + n)"),
    "gemm_first_term_dropped": ("for (int64_t k = 0; k < K; k++) {\n                double p = elem(X",
                                "for (int64_t k = 1; k < K; k++) {\n                double p = elem(X"),
    "gemm_wrong_sign": ("                acc += p;\n                asum += fabs(p);\n            }\n            Y[",
                        "                acc -= p;\n                asum += fabs(p);\n            }\n            Y["),
    "trimul_last_term_dropped": ("double acc = 0.0, asum = 0.0;\n                for (int64_t i = 0; i < HS; i++) {",
                                 "double acc = 0.0, asum = 0.0;\n                for (int64_t i = 0; i + 1 < HS; i++) {"),
    "softmax_last_term_dropped": ("double acc = 0.0, asum = 0.0;\n            for (int64_t i = 0; i < HS; i++) {",
                                  "double acc = 0.0, asum = 0.0;\n            for (int64_t i = 0; i + 1 < HS; i++) {"),
    "softmax_key_row_of_query": ("t2 * C3 + nh * HS + C;     /* K[b][nh][t2][:] */", "t * C3 + nh * HS + C;     /* K[b][nh][t2][:] */"),
    "bf16_decode_shift": ("(uint32_t)h << 16;", "(uint32_t)h << 15;"),
    "f16_decode_bias": ("expo - 25); /* (1 + frac/2^10) 2^(e-15) */", "expo - 24); /* (1 + frac/2^10) 2^(e-15) */"),
    "nan_bits": ("0x7FC00000u;", "0x7FC00001u;"),
    "tile_b_count": ("loads += (ek - sk) * (en - sn);   /* tile of B */",
                     "loads += (ek - sk) * (em - sm);   /* tile of B */"),
    "output_perturbed": ("Y[m * ldy + n] = (float)acc;", "Y[m * ldy + n] = (float)(acc * (1.0 + 0x1p-20));"),
    "bf16_ties_away": ("return (uint16_t)((u + 0x7FFFu + even) >> 16);", "return (uint16_t)((u + 0x8000u) >> 16);"),
    "f16_overflow_early": ("if (a >= 65520.0) return", "if (a > 65504.0) return"),
    "f16_subnormal_unit": ("const double q = rint(ldexp(a, 24));", "const double q = rint(ldexp(a, 23));"),
    "softmax_max_not_subtracted": ("t2 <= t; t2++) sum += exp(s[t2] - mx);", "t2 <= t; t2++) sum += exp(s[t2]);"),
    "softmax_max_is_min": ("if (s[t2] > mx) mx = s[t2];", "if (s[t2] < mx) mx = s[t2];"),
    "softmax_diagonal_excluded": ("t2 <= t; t2++) sum += exp(s[t2] - mx);", "t2 < t; t2++) sum += exp(s[t2] - mx);"),
    "softmax_log_mask_zero": ("orow[t2] = mode == 0 ? -INFINITY : 0.0;", "orow[t2] = 0.0;"),
    "softmax_scale_dropped": ("s[t2] = acc * scale;", "s[t2] = acc;"),
    "softmax_log2_sum": ("const double lse = log(sum);", "const double lse = log2(sum);"),
    "softmax_logsum_added": ("const double lp = (s[t2] - mx) - lse;", "const double lp = (s[t2] - mx) + lse;"),
    "attention_value_from_key_slot": ("t2 * C3 + 2 * C + nh * HS + i); /* V[b][nh][t2][i] */",
                                      "t2 * C3 + C + nh * HS + i); /* V[b][nh][t2][i] */"),
    "attention_diagonal_value_dropped": ("for (int64_t t2 = 0; t2 <= t; t2++) {\n                    const double p",
                                         "for (int64_t t2 = 0; t2 < t; t2++) {\n                    const double p"),
    "attention_logsum_dropped": ("const double p = exp((s[t2] - rmax) - rlog);", "const double p = exp(s[t2] - rmax);"),
    "attention_scale_dropped": ("s[t2] = scale * acc;", "s[t2] = acc;"),
    "attention_max_is_min": ("rmax = s[t2] > rmax ? s[t2] : rmax;", "rmax = s[t2] < rmax ? s[t2] : rmax;"),
    "attention_diagonal_out_of_sum": ("t2 <= t; t2++) rsum += exp(s[t2] - rmax);", "t2 < t; t2++) rsum += exp(s[t2] - rmax);"),
    "attention_key_row_of_query": ("t2 * C3 + C + nh * HS;  /* K[b][nh][t2][:] */",
                                   "t * C3 + C + nh * HS;  /* K[b][nh][t2][:] */"),
    "f16_truncates": ("double q = rint(ldexp(a, 10 - e));", "double q = floor(ldexp(a, 10 - e));"),
}


@pytest.fixture(scope="module")
def src():
    with open(obuild.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, src, name):
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    shutil.copy(os.path.join(obuild.HERE, "oracle.h"), tmp_path / "oracle.h")
    csrc = tmp_path / "oracle.c"
    csrc.write_text(src.replace(old, new))
    lib = obuild.build(src=str(csrc), out=str(tmp_path / f"lib_{name}.so"), extra=["-I", str(tmp_path)])
    bad = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(bad)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
