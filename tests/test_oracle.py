"""CPU tests: the oracle against its pins, and the pins against planted mistakes."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "li_oracle.c")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# Plausible mistakes planted in a copy of the oracle's C source: each must make
# at least one pin fail.  (old text, new text) pairs; the old text must occur.
C_MUTANTS = {
    "absorb_transposed_W": ("acc += qi[e] * W[e * r + t];", "acc += qi[e] * W[t * d + e];"),
    "absorb_wrong_query_index": ("acc += qi[e] * W[e * r + t];", "acc += qi[t % d] * W[e * r + t];"),
    "score_no_relu": ("total += w[h] * (dot > 0.0 ? dot : 0.0);\n        }\n        s[i] = total;",
                      "total += w[h] * dot;\n        }\n        s[i] = total;"),
    "score_no_head_weight": ("total += w[h] * (dot > 0.0 ? dot : 0.0);\n        }\n        s[i] = total;",
                             "total += (dot > 0.0 ? dot : 0.0);\n        }\n        s[i] = total;"),
    "score_relu_after_sum": ("total += w[h] * (dot > 0.0 ? dot : 0.0);\n        }\n        s[i] = total;",
                             "total += w[h] * dot;\n        }\n        s[i] = total > 0.0 ? total : 0.0;"),
    "score_wrong_head_index": ("dot += qt[h * r + t] * c[t];", "dot += qt[t] * c[t];"),
    "score_ignores_row_list": ("const int64_t row = rows ? (int64_t)rows[i] : i;", "const int64_t row = i;"),
    "score_dropped_last_term": ("for (int64_t t = 0; t < r; ++t)\n                dot += qt",
                                "for (int64_t t = 0; t < r - 1; ++t)\n                dot += qt"),
    "explicit_transposed_W": ("acc += W[e * r + t] * c[t];", "acc += W[t * d + e] * c[t];"),
    "topk_ascending": ("if (x->s > y->s) return -1;\n    if (x->s < y->s) return 1;",
                       "if (x->s > y->s) return 1;\n    if (x->s < y->s) return -1;"),
    "topk_tiebreak_reversed": ("return (x->p > y->p) - (x->p < y->p);", "return (x->p < y->p) - (x->p > y->p);"),
    "topk_drops_position_map": ("e[i].p = pos ? pos[i] : (int32_t)i;", "e[i].p = (int32_t)i;"),
    "e4m3_truncates": ("int m = (int)rintf(ldexpf(a, 3 - e));", "int m = (int)truncf(ldexpf(a, 3 - e));"),
    "e4m3_no_saturation": ("if (a >= 448.0f) return sign | 0x7E;", "if (a >= 480.0f) return sign | 0x7E;"),
    "e4m3_subnormal_step": ("const float n = rintf(ldexpf(a, 9));", "const float n = rintf(ldexpf(a, 8));"),
    "wht_unnormalized": ("const float k = 0.08838834764831845f;", "const float k = 1.0f;"),
    "wht_wrong_sign": ("x[j + h] = a - b;", "x[j + h] = b - a;"),
    "pow2_off_by_one": ("int e = (2.0f * f <= 1.75f) ? E - 9 : E - 8;", "int e = (2.0f * f <= 1.75f) ? E - 8 : E - 8;"),
    "fp8_score_drops_scales": ("dot += (double)qs[h * nseg + g] * (double)cs[row * nseg + g] * seg;",
                               "dot += seg;"),
    "fp8_score_relu_after_sum": ("total += w[h] * (dot > 0.0 ? dot : 0.0);\n        }\n        s[i] = total;\n    }\n}\n\n/*\n * RoPE",
                                 "total += w[h] * dot;\n        }\n        s[i] = total > 0.0 ? total : 0.0;\n    }\n}\n\n/*\n * RoPE"),
    "fp8_score_drops_bias": ("if (bias) dot += bias[h];\n            total += w[h] * (dot > 0.0 ? dot : 0.0);\n        }\n        s[i] = total;\n    }\n}\n\n/*\n * RoPE",
                             "total += w[h] * (dot > 0.0 ? dot : 0.0);\n        }\n        s[i] = total;\n    }\n}\n\n/*\n * RoPE"),
    "score_bias_after_relu": ("if (bias) dot += bias[h];\n            total += w[h] * (dot > 0.0 ? dot : 0.0);",
                              "total += w[h] * (dot > 0.0 ? dot : 0.0) + (bias ? w[h] * bias[h] : 0.0);"),
    "rope_theta_exponent": ("return pow(base, -(double)(2 * f) / (double)(2 * F));",
                            "return pow(base, -(double)f / (double)(2 * F));"),
    "rope_wrong_sign": ("x[2 * j + 1] = re * sn + im * c;", "x[2 * j + 1] = re * sn - im * c;"),
    "rope_frequency_index": ("const int64_t f = j % F;", "const int64_t f = j / S;"),
    "absorb_rope_no_conjugate": ("out[2 * (s * F + f)] = a * c + bb * e;", "out[2 * (s * F + f)] = a * c - bb * e;"),
    "absorb_rope_drops_bias": ("b[i] = acc;", "b[i] = 0.0;"),
    "absorb_rope_nope_transposed": ("acc += qi[2 * F + e] * Wn[e * r_nope + t];", "acc += qi[2 * F + e] * Wn[t * d_nope + e];"),
    "explicit_rope_no_beta": ("double acc = beta[e];", "double acc = 0.0;"),
    "explicit_rope_rotation_sign": ("key[2 * f + 1] = kr * sin(ang) + ki * cos(ang);",
                                    "key[2 * f + 1] = kr * sin(ang) - ki * cos(ang);"),
}


def _run_pins():
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    return failed


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_pins_catch_c_mutant(name, mutant_dir):
    old, new = C_MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    msrc = mutant_dir / f"{name}.c"
    msrc.write_text(src.replace(old, new, 1))
    so = mutant_dir / f"{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", str(msrc), "-o",
                           str(so), "-lm"])
    oracle.use_library(str(so))
    try:
        failed = _run_pins()
    finally:
        oracle.use_library(None)
    assert failed, f"no pin catches the planted mistake {name}"


def _mut_valid_rows_exclusive(pos, length):
    return int(max(0, min(int(pos), int(length))))


def _mut_hs_follower_full_prefix(q, W, w, latents, qseq, qpos, lens, k, M):
    res = _orig_hs(q, W, w, latents, qseq, qpos, lens, k, M)
    for l in range(1, len(q)):
        full = oracle.full_layer(q[l], W[l], w[l], latents, qseq, qpos, lens, k)
        for i, r in enumerate(res[l]):
            r.sel = full[i].sel
    return res


def _mut_hs_follower_uncapped(q, W, w, latents, qseq, qpos, lens, k, M):
    res = _orig_hs(q, W, w, latents, qseq, qpos, lens, k, M)
    for l in range(1, len(q)):
        for r in res[l]:
            r.sel = oracle.topk(r.cand_scores, len(r.cand), pos=r.cand)
    return res


_orig_hs = oracle.hs_group


def _mut_absorb_fp8_fp32_accumulation(q, W):
    """Sums the products in float32, in order, instead of rounding the exact sum once."""
    q = np.asarray(q, np.float32)
    W = np.asarray(W, np.float32)
    acc = np.zeros(q.shape[:-1] + (W.shape[1],), np.float32)
    for e in range(W.shape[0]):
        acc = (acc + q[..., e:e + 1] * W[e]).astype(np.float32)
    return oracle.quantize_rows(acc)


def _mut_absorb_fp8_truncates(q, W):
    """Rounds the exact sum toward zero instead of to nearest."""
    x = oracle.absorb(q, W)
    f = x.astype(np.float32)
    over = np.abs(f.astype(np.float64)) > np.abs(x)
    f[over] = np.nextafter(f[over], np.float32(0))
    return oracle.quantize_rows(f)


def _mut_absorb_fp8_bf16(q, W):
    """Rounds the absorbed query to bfloat16 (the plain path's precision) before quantizing."""
    from sparse_attention_token_absorb_amd import synth
    return oracle.quantize_rows(synth.round_bf16(oracle.absorb(q, W).astype(np.float32)))

PY_MUTANTS = {
    "valid_rows_exclusive": ("valid_rows", _mut_valid_rows_exclusive),
    "hs_follower_scores_full_prefix": ("hs_group", _mut_hs_follower_full_prefix),
    "hs_follower_budget_uncapped": ("hs_group", _mut_hs_follower_uncapped),
    "absorb_fp8_fp32_accumulation": ("absorb_fp8", _mut_absorb_fp8_fp32_accumulation),
    "absorb_fp8_truncates": ("absorb_fp8", _mut_absorb_fp8_truncates),
    "absorb_fp8_bf16": ("absorb_fp8", _mut_absorb_fp8_bf16),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_pins_catch_python_mutant(name, monkeypatch):
    attr, fn = PY_MUTANTS[name]
    monkeypatch.setattr(oracle, attr, fn)
    assert _run_pins(), f"no pin catches the planted mistake {name}"


def test_oracle_threads_reported():
    assert oracle.num_threads() >= 1
