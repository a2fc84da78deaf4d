"""Planted mistakes in copies of the oracle must each fail at least one pin (no GPU).

Every mutation is a plausible slip in the oracle's source: a dropped term, a wrong sign, a
wrong index, the wrong estimator, a skipped rounding. The copy is compiled with the same
flags as the real oracle and the pins run on it; the test fails if a mutant passes them all.
"""
import os
import subprocess

import pytest

from oracle import build as obuild
from oracle.oracle import Oracle
from tests import oracle_pins

MUTATIONS = [
    ("unbiased variance", "double var = q / (double)N;",
     "double var = q / (double)(N > 1 ? N - 1 : 1);"),
    ("LN eps outside sqrt", "*rstd = 1.0 / sqrt(var + eps);", "*rstd = 1.0 / (sqrt(var) + eps);"),
    ("RMS eps dropped", "*rstd = 1.0 / sqrt(ms + eps);", "*rstd = 1.0 / sqrt(ms);"),
    ("RMS mean square off by one", "double ms = q / (double)N;", "double ms = q / (double)(N + 1);"),
    ("LN mean off by one", "double mu = s / (double)N;", "double mu = s / (double)(N + 1);"),
    ("bias dropped", "xhat * w + b : xhat * w;", "xhat * w : xhat * w;"),
    ("bias sign", "xhat * w + b : xhat * w;", "xhat * w - b : xhat * w;"),
    ("weight index reversed", "double w = or_load(or_wt(dtype), W, j);",
     "double w = or_load(or_wt(dtype), W, N - 1 - j);"),
    ("LN mean-gradient term dropped", "rs[o] * (g[j] - c1 - xh[j] * c2)", "rs[o] * (g[j] - xh[j] * c2)"),
    ("LN projection sign", "rs[o] * (g[j] - c1 - xh[j] * c2)", "rs[o] * (g[j] - c1 + xh[j] * c2)"),
    ("RMS projection dropped", ": rs[o] * (g[j] - xh[j] * c2);", ": rs[o] * g[j];"),
    ("projection without xhat", "sgx += g[j] * xh[j];", "sgx += g[j];"),
    ("gradient ignores weight",
     "g[j] = or_load(or_act(dtype), dY, i * N + j) * or_load(or_wt(dtype), W, j);",
     "g[j] = or_load(or_act(dtype), dY, i * N + j);"),
    ("dY column index reversed",
     "g[j] = or_load(or_act(dtype), dY, i * N + j) * or_load(or_wt(dtype), W, j);",
     "g[j] = or_load(or_act(dtype), dY, i * N + (N - 1 - j)) * or_load(or_wt(dtype), W, j);"),
    ("dW uses raw input", "aw[j - j0] += dy * xhat;", "aw[j - j0] += dy * x;"),
    ("dB weighted by xhat", "ab[j - j0] += dy;", "ab[j - j0] += dy * xhat;"),
    ("dW skips first row",
     "for (int64_t i = r0; i < r1; ++i) {\n            int64_t o = i - r0;\n            for (int64_t j = j0;",
     "for (int64_t i = r0 + 1; i < r1; ++i) {\n            int64_t o = i - r0;\n            for (int64_t j = j0;"),
    ("incoming residual gradient dropped", "if (dH) d += or_load(or_act(dtype), dH, i * N + j);",
     "if (dH) d += 0.0;"),
    ("forward weight read as the activation type", "double w = or_load(or_wt(dtype), W, j);",
     "double w = or_load(or_act(dtype), W, j);"),
    ("backward weight read as the activation type",
     "g[j] = or_load(or_act(dtype), dY, i * N + j) * or_load(or_wt(dtype), W, j);",
     "g[j] = or_load(or_act(dtype), dY, i * N + j) * or_load(or_act(dtype), W, j);"),
    ("bias read as the activation type", "double b = B ? or_load(or_wt(dtype), B, j) : 0.0;",
     "double b = B ? or_load(or_act(dtype), B, j) : 0.0;"),
    ("residual sum not rounded",
     "if (R) v = or_round_to_dtype(dtype, or_load(dtype, R, i * N + j) + v);",
     "if (R) v = or_load(dtype, R, i * N + j) + v;"),
    ("bf16 ties away from zero", "double r = nearbyint(ldexp(a, -q));",
     "double r = round(ldexp(a, -q));"),
    ("bf16 decode shift", "uint32_t u = ((uint32_t)b) << 16;", "uint32_t u = ((uint32_t)b) << 15;"),
    ("fp16 ties away from zero", "double k = nearbyint(ldexp(a, -q));",
     "double k = round(ldexp(a, -q));"),
    ("fp16 decode exponent bias", "v = ldexp((double)(1024 + f), e - 25);",
     "v = ldexp((double)(1024 + f), e - 24);"),
    ("fp16 subnormal step", "if (q < -24) q = -24;", "if (q < -25) q = -25;"),
    ("fp16 overflow threshold", "if (out > 65504.0) out = INFINITY;",
     "if (out > 65536.0) out = INFINITY;"),
    ("fp16 read as bf16",
     "return dtype == OR_F16 ? or_f16_bits_to_double(b) : or_bf16_bits_to_double(b);",
     "return or_bf16_bits_to_double(b);"),
    ("fp16 residual rounded as bf16", "if (dtype == OR_F16) return or_round_to_f16(v);",
     "if (dtype == OR_F16) return or_round_to_bf16(v);"),
    ("fp16 mixed activations read as bf16",
     "return dtype == OR_BF16_F32W ? OR_BF16 : dtype == OR_F16_F32W ? OR_F16 : dtype;",
     "return dtype == OR_BF16_F32W ? OR_BF16 : dtype == OR_F16_F32W ? OR_BF16 : dtype;"),
    ("projection bias dropped", "out[o * Nout + j] = acc + (c ? (double)c[j] : 0.0);",
     "out[o * Nout + j] = acc;"),
    ("projection transposed", "acc += y[o * K + k] * or_load(act, L, j * K + k);",
     "acc += y[o * K + k] * or_load(act, L, k * Nout + j);"),
    ("norm beta dropped before the projection",
     "st = oracle_fwd_rows(kind, dtype, M, K, r0, r1, X, NULL, W, B, eps, y, NULL, NULL, NULL);",
     "st = oracle_fwd_rows(kind, dtype, M, K, r0, r1, X, NULL, W, NULL, eps, y, NULL, NULL, NULL);"),
    ("projection of the first row only", "acc += y[o * K + k] * or_load(act, L, j * K + k);",
     "acc += y[k] * or_load(act, L, j * K + k);"),
    ("attention scale dropped", "p[j] = scale * dot;", "p[j] = dot;"),
    ("causal window without the diagonal", "const int64_t n = causal ? i + 1 : S;",
     "const int64_t n = causal ? (i > 0 ? i : 1) : S;"),
    ("grouped heads interleaved", "const int64_t hk = h / (Hq / Hk);",
     "const int64_t hk = h % Hk;"),
    ("key norm with the query gamma and beta",
     "or_qk_row(kind, D, K, ((b * S + j) * Hk + hk) * D, Wk, Bk, eps, kn + j * D);",
     "or_qk_row(kind, D, K, ((b * S + j) * Hk + hk) * D, Wq, Bq, eps, kn + j * D);"),
    ("key norm dropped",
     "or_qk_row(kind, D, K, ((b * S + j) * Hk + hk) * D, Wk, Bk, eps, kn + j * D);",
     "or_qk_row(OR_NO_NORM, D, K, ((b * S + j) * Hk + hk) * D, Wk, Bk, eps, kn + j * D);"),
    ("query beta dropped", "or_qk_row(kind, D, Q, ((b * S + i) * Hq + h) * D, Wq, Bq, eps, qn);",
     "or_qk_row(kind, D, Q, ((b * S + i) * Hq + h) * D, Wq, NULL, eps, qn);"),
    ("keys of the first batch only",
     "or_qk_row(kind, D, K, ((b * S + j) * Hk + hk) * D, Wk, Bk, eps, kn + j * D);",
     "or_qk_row(kind, D, K, ((0 * S + j) * Hk + hk) * D, Wk, Bk, eps, kn + j * D);"),
    ("value row of the query position",
     "acc += p[j] * or_load(OR_BF16, V, ((b * S + j) * Hk + hk) * D + d);",
     "acc += p[j] * or_load(OR_BF16, V, ((b * S + i) * Hk + hk) * D + d);"),
    ("value read from the query head", "acc += p[j] * or_load(OR_BF16, V, ((b * S + j) * Hk + hk) * D + d);",
     "acc += p[j] * or_load(OR_BF16, V, ((b * S + j) * Hk + h % Hk) * D + d);"),
    ("softmax normaliser dropped", "O[(i - s0) * D + d] = acc / z;", "O[(i - s0) * D + d] = acc;"),
    ("lse without the largest logit", "if (lse) lse[i - s0] = mx + log(z);",
     "if (lse) lse[i - s0] = log(z);"),
    ("query norm weight index reversed", "double w = or_load(OR_BF16, W, d);",
     "double w = or_load(OR_BF16, W, D - 1 - d);"),
    ("QK LayerNorm bias sign", "(out[d] - mu) * rs * w + b : out[d] * rs * w;",
     "(out[d] - mu) * rs * w - b : out[d] * rs * w;"),
]


def _build_mutant(tmp_path, name, old, new):
    with open(obuild.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation %r: pattern must occur exactly once" % name
    path = os.path.join(str(tmp_path), "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(str(tmp_path), "libmutant.so")
    subprocess.run(["gcc", *obuild.CFLAGS, path, "-o", lib, "-lm"], check=True,
                   capture_output=True)
    return lib


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, name, old, new):
    orc = Oracle(_build_mutant(tmp_path, name, old, new))
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError) as e:  # a pin mismatch or a rejected result
            failures.append((pin.__name__, str(e)[:120]))
            break
    assert failures, "planted mistake %r passed every pin" % name
