"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
the pin suite catches every one of them."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle_moe.c")

MUTANTS = {
    "nibble order swapped": ("(c % 2 == 0) ? (byte & 0xFu) : (byte >> 4)", "(c % 2 == 0) ? (byte >> 4) : (byte & 0xFu)"),
    "no sign extension": ("(nib >= 8u) ? (int32_t)nib - 16 : (int32_t)nib", "(int32_t)nib"),
    "sigmoid sign": ("exp(-(double)ze)", "exp((double)ze)"),
    "bias enters weights": ("sum += (double)s[ids[j]]", "sum += (double)b[ids[j]]"),
    "ties to higher id": ("(best < 0 || b[e] > b[best])", "(best < 0 || b[e] >= b[best])"),
    "group score top-1": ("gscore[g] = b1 + b2;", "gscore[g] = b1;"),
    "group gap sign": ("group_gap = last_kept - first_dropped;", "group_gap = first_dropped - last_kept;"),
    "group gap from the best kept group": ("last_kept = gscore[best];", "if (r == 0) last_kept = gscore[best];"),
    "gate and up swapped": ("h[i] = (float)((double)g / (1.0 + exp(-(double)g)) * (double)u);",
                            "h[i] = (float)((double)u / (1.0 + exp(-(double)u)) * (double)g);"),
    "rsf on shared": ("if (shared_out) acc += (double)shared_out[(int64_t)t * H + c];",
                      "if (shared_out) acc += rsf * (double)shared_out[(int64_t)t * H + c];"),
    "dropped routed term": ("for (int32_t j = 0; j < k; ++j) {\n                int64_t p", "for (int32_t j = 0; j + 1 < k; ++j) {\n                int64_t p"),
    "up reads gate rows": ("oracle_dequant_row(qrow(up, bits, e, i, H), bits, qscale(up, e, i), H, wrow);",
                           "oracle_dequant_row(qrow(gate, bits, e, i, H), bits, qscale(up, e, i), H, wrow);"),
    "scale of row 0": ("qscale(down, e, c)", "qscale(down, e, 0)"),
    "unstable permutation": ("for (int64_t p = 0; p < P; ++p) {\n        if (ids[p] == -1) {",
                             "for (int64_t p = P - 1; p >= 0; --p) {\n        if (ids[p] == -1) {"),
    "top-p keeps the pair that reaches p exactly": ("while (keep < k && mass < p)", "while (keep < k && mass <= p)"),
    "top-p not renormalised": ("w[j] = (float)((double)s[ids[j]] / ks);", "w[j] = w[j];"),
    "top-p in selection order": ("if (w[y] > w[x] || (w[y] == w[x] && ids[y] < ids[x])) {", "if (0) {"),
    "quantiser ties away from zero": ("float v = nearbyintf(w[c] / scale);", "float v = roundf(w[c] / scale);"),
    "quantiser scale one level short": ("const float scale = amax / qmax;", "const float scale = amax / (qmax + 1.0f);"),
    "bias update sign flipped": ("if (load < total)\n            bias_out[e] = bias_in[e] + gamma;",
                                 "if (load < total)\n            bias_out[e] = bias_in[e] - gamma;"),
    "bias update moves at the mean": ("else if (load > total)", "else if (load >= total)"),
    "q8 ties away from zero": ("float t = nearbyintf(v[c] / d);", "float t = roundf(v[c] / d);"),
    "q8 scale of the next block": ("acc += (double)d[b] * (double)isum;",
                                   "acc += (double)d[(b + 1) % (n / 32)] * (double)isum;"),
    "q8 weight scale dropped": ("return (double)*qscale(m, e, r) * acc;", "return acc;"),
    "q8 blocks of 16": ("for (int32_t b = 0; b < n / 32; ++b) d[b] = q8_block(v + 32 * b, 32, q + 32 * b);",
                        "for (int32_t b = 0; b < n / 32; ++b) { d[b] = q8_block(v + 32 * b, 16, q + 32 * b); "
                        "q8_block(v + 32 * b + 16, 16, q + 32 * b + 16); }"),
    "int2 fields from the high bits": ("uint32_t f = ((uint32_t)row[c / 4] >> (2 * (c % 4))) & 3u;",
                                       "uint32_t f = ((uint32_t)row[c / 4] >> (6 - 2 * (c % 4))) & 3u;"),
    "int2 without sign": ("vals[c] = (f >= 2u) ? (int32_t)f - 4 : (int32_t)f;", "vals[c] = (int32_t)f;"),
    "int2 row length of int4": ("int64_t row_bytes = (bits == 4) ? cols / 2 : (bits == 2) ? cols / 4 : cols;",
                                "int64_t row_bytes = (bits == 4 || bits == 2) ? cols / 2 : cols;"),
    "down transposed": ("oracle_dequant_row(qrow(down, bits, e, c, I), bits, qscale(down, e, c), I, wrow);",
                        "for (int32_t i2 = 0; i2 < I; ++i2) oracle_dequant_row(qrow(down, bits, e, i2 % H, I), bits, qscale(down, e, c), 1, wrow + i2);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, f"mutation site for {name!r} not found"
    mut = src.replace(old, new)
    c = tmp_path / "oracle_mut.c"
    c.write_text(mut)
    hdr = os.path.join(ROOT, "oracle")
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-w", "-I", hdr, "-o", str(so), str(c),
                    "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(so), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", "not thread_count"],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode != 0, f"mutant {name!r} survived the pins:\n{r.stdout[-2000:]}"
