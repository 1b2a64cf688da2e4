"""The oracle's pins are not vacuous: each plausible mistake, planted in a copy
of the oracle source and compiled on the CPU, must fail at least one pin.

Every mutation keeps all memory accesses in bounds; each mutant still runs in a
child process so that a crash there cannot take the test runner down.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# (name, text in rba_oracle.c, replacement)
MUTANTS = [
    ("bias dropped",
     "scores[s] = sm_scale * dot + elem(bias, bias_dtype, bias_row + d);",
     "scores[s] = sm_scale * dot + 0.0 * elem(bias, bias_dtype, bias_row + d);"),
    ("bias scaled by sm_scale",
     "scores[s] = sm_scale * dot + elem(bias, bias_dtype, bias_row + d);",
     "scores[s] = sm_scale * (dot + elem(bias, bias_dtype, bias_row + d));"),
    ("distance read from the far end of the row",
     "elem(bias, bias_dtype, bias_row + d)",
     "elem(bias, bias_dtype, bias_row + (R - 1 - d))"),
    ("clamp to the wrong bucket",
     "if (d > R - 1) d = R - 1;",
     "if (d > R - 1) d = (R > 1 ? R - 2 : 0);"),
    ("window one key too wide",
     "(W <= 0 || t - s < W)",
     "(W <= 0 || t - s <= W)"),
    ("self excluded from the causal mask",
     "int visible = (s <= t)",
     "int visible = (s < t || t == 0)"),
    ("interleaved GQA mapping",
     "h / G",
     "h % Hkv"),
    ("scale divides instead of multiplies",
     "scores[s] = sm_scale * dot",
     "scores[s] = dot / sm_scale"),
    ("value read as key",
     "dot += elem(q, dtype, q_row + i) *\n             elem(k,",
     "dot += elem(q, dtype, q_row + i) *\n             elem(v,"),
    ("lse without the max",
     "if (lse) *lse = m + log(l);",
     "if (lse) *lse = log(l);"),
    ("decode query one past the last key",
     "h / G, n - 1, n, bias,",
     "h / G, n - 2 < 0 ? 0 : n - 2, n, bias,"),
    ("history ignored: new tokens attend only to each other",
     "cu_kv[b] * (int64_t)Hkv * D, Hkv, D, h / G, pos, n, bias,",
     "(cu_kv[b] + n - L) * (int64_t)Hkv * D, Hkv, D, h / G, pos - (n - L), L, bias,"),
    ("history queries placed at the start of the sequence",
     "const int64_t pos = n - L + (tok - cu_q[b]);",
     "const int64_t pos = tok - cu_q[b];"),
    ("projection reads w transposed",
     "acc += elem(r, dtype, r_row + kk) * elem(w, dtype, (int64_t)kk * R + d);",
     "acc += elem(r, dtype, r_row + kk) * elem(w, dtype, (int64_t)d * d_rel + kk);"),
    ("projection drops its last term",
     "for (int kk = 0; kk < d_rel; ++kk)",
     "for (int kk = 0; kk < d_rel - 1; ++kk)"),
    ("projected bias row of the neighbouring head",
     "const int64_t r_row = (tok * Hq + h) * (int64_t)d_rel;",
     "const int64_t r_row = (tok * Hq + (h + 1) % Hq) * (int64_t)d_rel;"),
    ("projected rows ignore the history",
     "const int64_t pos = n - L + (tok - cu_q[b]);\n      const int64_t r_row",
     "const int64_t pos = tok - cu_q[b];\n      const int64_t r_row"),
    ("projected bias not rounded to the dtype",
     "brow[d] = round_to_dtype(acc, dtype);",
     "brow[d] = acc;"),
    ("projected bias rounded with ties away from zero",
     "const double r = nearbyint(x / ulp) * ulp;",
     "const double r = round(x / ulp) * ulp;"),
    ("projected bias rounded to one bit too many",
     "const double ulp = ldexp(1.0, e - 8);",
     "const double ulp = ldexp(1.0, e - 9);"),
    ("no max subtraction lost in normalisation",
     "for (int i = 0; i < D; ++i) out[i] /= l;",
     "for (int i = 0; i < D; ++i) out[i] /= (l + 1e-3);"),
]

_RUNNER = r"""
import json, sys
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[2])
import oracle, oracle_pins
orc = oracle.Oracle(sys.argv[3])
print(json.dumps(oracle_pins.failing_pins(orc)))
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "rba_oracle.c")).read()
    count = src.count(old)
    assert count >= 1, f"mutation site for '{name}' not found"
    mutated = src.replace(old, new)
    c_path = tmp_path / "mutant.c"
    c_path.write_text(mutated)
    lib = oracle.build(str(c_path), str(tmp_path / "libmutant.so"))
    res = subprocess.run([sys.executable, "-c", _RUNNER, ROOT, HERE, lib],
                         capture_output=True, text=True, timeout=300)
    if res.returncode != 0:
        return  # the mutant crashed: caught
    failed = json.loads(res.stdout.strip().splitlines()[-1])
    assert failed, f"no pin catches the mutant '{name}'"
