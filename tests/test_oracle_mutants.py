"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins in test_oracle_pins.py catch every one of them.

Each mutant is a one-line textual change of oracle/gdn_oracle.c, built into a
temporary shared library that the pin suite loads through
GDN_ORACLE_LIB_OVERRIDE.  The real oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTANTS = {
    "conv_taps_reversed": ("acc += w[j] * hist[j];", "acc += w[K - 2 - j] * hist[j];"),
    "conv_current_tap_wrong": ("acc += w[K - 1] * x;", "acc += w[0] * x;"),
    "no_silu_after_conv": ("static double silu(double y) { return y / (1.0 + exp(-y)); }",
                           "static double silu(double y) { return y; }"),
    "decay_dropped": ("for (int c = 0; c < dk; ++c) S[(size_t)r * dk + c] *= a;",
                      "for (int c = 0; c < dk; ++c) S[(size_t)r * dk + c] *= 1.0;"),
    "delta_sign": ("const double u = b * (yv[r] - kvmem[r]);",
                   "const double u = b * (yv[r] + kvmem[r]);"),
    "beta_dropped": ("const double u = b * (yv[r] - kvmem[r]);",
                     "const double u = (yv[r] - kvmem[r]);"),
    "kvmem_transposed": ("for (int c = 0; c < dk; ++c) acc += S[(size_t)r * dk + c] * yk[c];\n            kvmem[r] = acc;",
                         "for (int c = 0; c < dk; ++c) acc += S[(size_t)(c % dv) * dk + (r % dk)] * yk[c];\n            kvmem[r] = acc;"),
    "readout_with_key": ("acc += S[(size_t)r * dk + c] * yq[c];",
                         "acc += S[(size_t)r * dk + c] * yk[c];"),
    "readout_before_update": ("for (int r = 0; r < dv; ++r) {\n            double acc = 0.0;\n            for (int c = 0; c < dk; ++c) acc += S[(size_t)r * dk + c] * yq[c];",
                              "for (int r = 0; r < dv; ++r) {\n            double acc = 0.0;\n            for (int c = 0; c < dk; ++c) acc += (S[(size_t)r * dk + c] - b * (yv[r] - kvmem[r]) * yk[c]) * yq[c];"),
    "key_head_index": ("const int hk = h / (Hv / Hk);", "const int hk = h % Hk;"),
    "l2_without_sqrt": ("const double rq = 1.0 / sqrt(sq + d->l2_eps), rk = 1.0 / sqrt(sk + d->l2_eps);",
                        "const double rq = 1.0 / (sq + d->l2_eps), rk = 1.0 / sqrt(sk + d->l2_eps);"),
    "scale_dropped": ("for (int i = 0; i < dk; ++i) yq[i] *= d->scale;", ""),
    "rms_without_mean": ("ms /= dv;", ""),
    "gate_without_silu": ("const double gz = z ? silu(ld(z, (t * Hv + h) * dv + r, io)) : 1.0;",
                          "const double gz = z ? ld(z, (t * Hv + h) * dv + r, io) : 1.0;"),
    "conv_state_off_by_one": ("const int64_t pos = L + j;", "const int64_t pos = L + j - 1 < 0 ? 0 : L + j - 1;"),
    "initial_state_ignored": ("S[i] = ld(S0, ((int64_t)n * Hv + h) * dv * dk + i, d->state_dtype);",
                              "S[i] = 0.0 * ld(S0, ((int64_t)n * Hv + h) * dv * dk + i, d->state_dtype);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique or missing"
    mut = tmp_path / "gdn_oracle_mut.c"
    mut.write_text(src.replace(old, new))
    hdr = os.path.join(ROOT, "oracle")
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-I", hdr,
                    "-o", str(so), str(mut), "-lm"], check=True)
    env = dict(os.environ, GDN_ORACLE_LIB_OVERRIDE=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
