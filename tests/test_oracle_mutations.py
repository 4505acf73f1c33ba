"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake (a dropped term, a
wrong sign, a wrong index or a transposed operand), compiles the copy on the
CPU, swaps it in, and checks that at least one pin of tests/test_oracle.py
fails.  The real oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "fdllm_oracle.c")

MUTATIONS = {
    "rope_sign": ("v[i] = a * c - b * s;", "v[i] = a * c + b * s;"),
    "rope_dropped_term": ("v[i + half] = b * c + a * s;", "v[i + half] = b * c;"),
    "rope_theta_index": ("pow(base, -2.0 * (double)i / (double)dh)", "pow(base, -1.0 * (double)i / (double)dh)"),
    "weight_transposed": ("const double* w = W + (int64_t)o * d;\n            double acc = 0.0;\n            for (int k = 0; k < d; ++k) acc += w[k] * x[k];",
                          "double acc = 0.0;\n            for (int k = 0; k < d; ++k) acc += W[(int64_t)k * cols + o % cols] * x[k];"),
    "scale_missing_sqrt": ("1.0 / sqrt((double)dh)", "1.0 / (double)dh"),
    "gqa_map": ("const int g = (int)(((int64_t)h * Hkv) / H);", "const int g = h % Hkv;"),
    "vis_transposed": ("if (vis && !vis[((int64_t)b * nq + i) * nq + j]) continue;\n                    const double* kj = k + (((int64_t)b * nq + j) * Hkv + g) * dh;\n                    double s = 0.0;\n                    for (int e = 0; e < dh; ++e) s += qi[e] * kj[e];\n                    s *= scale;",
                       "if (vis && !vis[((int64_t)b * nq + j) * nq + i]) continue;\n                    const double* kj = k + (((int64_t)b * nq + j) * Hkv + g) * dh;\n                    double s = 0.0;\n                    for (int e = 0; e < dh; ++e) s += qi[e] * kj[e];\n                    s *= scale;"),
    "old_content_attended": ("if (written[(int64_t)b * N + p]) continue;\n                    double s = 0.0;\n                    for (int e = 0; e < dh; ++e) s += qi[e] * Kb[(int64_t)p * dh + e];\n                    s *= scale;",
                             "double s = 0.0;\n                    for (int e = 0; e < dh; ++e) s += qi[e] * Kb[(int64_t)p * dh + e];\n                    s *= scale;"),
    "last_occurrence_wins": ("if (pos_b[jj] == pos_b[j]) return 0;", "if (0) return 0;"),
    "bf16_truncates": ("double r = ldexp(nearbyint(ldexp(x, -q)), q);", "double r = ldexp(trunc(ldexp(x, -q)), q);"),
    "lse_log2": ("*lse = m + log(l);", "*lse = m + log2(l);"),
    "scores_without_lse": ("a += exp(s * scale - lse);", "a += exp(s * scale);"),
    "scores_last_owner": ("if (owner[pb[j]] < 0) owner[pb[j]] = j;", "owner[pb[j]] = j;"),
    "scores_vis_transposed": ("if (j >= 0 && vis && !vis[((int64_t)b * nq + i) * nq + j]) continue;",
                              "if (j >= 0 && vis && !vis[((int64_t)b * nq + j) * nq + i]) continue;"),
    "scores_unselected_rows": ("if (!sel[(int64_t)b * nq + i]) continue;", "if (0) continue;"),
}

PIN_TESTS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "test_oracle.py")


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mutated = src.replace(old, new, 1 if name != "old_content_attended" else 2)
    csrc = tmp_path / "mut.c"
    csrc.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so),
                           str(csrc), "-lm"])
    env = dict(os.environ, FDLLM_ORACLE_LIB=str(so))
    r = subprocess.run(["python", "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", PIN_TESTS],
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins did not catch mutation %s:\n%s" % (name, r.stdout[-2000:])
