"""The pins have teeth: plant one plausible mistake at a time in a copy of the oracle (on the CPU) and check that
the pin suite fails for every mutant, while an unmodified copy passes."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("pred_shift_amount", "return (s >> k) | (a << (L - k));", "return (s >> k) | (a << k);"),
    ("succ_drops_new_bits", "return ((s << k) & ((1u << L) - 1u)) | b;", "return ((s << k) & ((1u << L) - 1u));"),
    ("weight_sign", "return -(d * d) / T;", "return (d * d) / T;"),
    ("weight_drops_T", "return -(d * d) / T;", "return -(d * d);"),
    ("backward_wrong_step", "x[b] = log_weight(w[t + 1], c[u], T) + bnext[u];",
     "x[b] = log_weight(w[t], c[u], T) + bnext[u];"),
    ("sigma_start_rule", "alpha[s] = (!has_sigma || (s >> k) == (sigma & gmask)) ? th : -INFINITY;",
     "alpha[s] = (!has_sigma || (s & gmask) == (sigma >> k)) ? th : -INFINITY;"),
    ("sigma_end_rule", "b[s] = (!has_sigma || s == sigma) ? 0.0 : -INFINITY;",
     "b[s] = (!has_sigma || (s >> 1) == (sigma >> 1)) ? 0.0 : -INFINITY;"),
    ("posterior_unnormalised", "acc += (double)c[s] * exp(tmp[s] - lnz);", "acc += (double)c[s] * exp(tmp[s]);"),
    ("lse_drops_max", "return mx + log(s);", "return log(s);"),
    ("grad_factor", "grad[t] = (2.0 / T) * cov;", "grad[t] = (1.0 / T) * cov;"),
    ("grad_forward_drops_history", "rt[s] = (double)g[t] * (double)c[s] + acc;", "rt[s] = (double)g[t] * (double)c[s];"),
    ("grad_backward_index", "acc += pw[b] * ((double)g[t + 1] * (double)c[u] + rbnext[u]);",
     "acc += pw[b] * ((double)g[t] * (double)c[u] + rbnext[u]);"),
    ("grad_uncentred_codeword", "cov += tmp[s] * ((double)c[s] - m0) * (rt[s] + rbcur[s] - mr);",
     "cov += tmp[s] * ((double)c[s]) * (rt[s] + rbcur[s] - mr) * 0.5;"),
    ("codebook_drops_direct_term", "gc[s] += tmp[s] * ((double)g[t] + (2.0 / T) * ((double)w[t] - (double)c[s]) * (rt[s] + rbcur[s] - mr));",
     "gc[s] += tmp[s] * ((2.0 / T) * ((double)w[t] - (double)c[s]) * (rt[s] + rbcur[s] - mr));"),
    ("codebook_residual_sign", "gc[s] += tmp[s] * ((double)g[t] + (2.0 / T) * ((double)w[t] - (double)c[s]) * (rt[s] + rbcur[s] - mr));",
     "gc[s] += tmp[s] * ((double)g[t] + (2.0 / T) * ((double)c[s] - (double)w[t]) * (rt[s] + rbcur[s] - mr));"),
    ("codebook_uncentred", "gc[s] += tmp[s] * ((double)g[t] + (2.0 / T) * ((double)w[t] - (double)c[s]) * (rt[s] + rbcur[s] - mr));",
     "gc[s] += tmp[s] * ((double)g[t] + (2.0 / T) * ((double)w[t] - (double)c[s]) * (rt[s] + rbcur[s]));"),
    ("codebook_factor", "gc[s] += tmp[s] * ((double)g[t] + (2.0 / T) * ((double)w[t] - (double)c[s]) * (rt[s] + rbcur[s] - mr));",
     "gc[s] += tmp[s] * ((double)g[t] + (1.0 / T) * ((double)w[t] - (double)c[s]) * (rt[s] + rbcur[s] - mr));"),
    ("viterbi_tie_rule", "if (v < best) { best = v; arg = a; }", "if (v <= best) { best = v; arg = a; }"),
    ("viterbi_end_tie_rule", "if (mcur[s] < mcur[s_end]) s_end = s;", "if (mcur[s] <= mcur[s_end]) s_end = s;"),
    ("viterbi_fma_order", "mcur[s] = e + best;", "mcur[s] = fmaf(d, d, best);"),
]


def _build(tmpdir, text, name):
    src = os.path.join(tmpdir, f"{name}.c")
    lib = os.path.join(tmpdir, f"lib{name}.so")
    with open(src, "w") as f:
        f.write(text)
    import oracle

    subprocess.check_call(["gcc", *oracle.GCC_FLAGS, "-o", lib, src, "-lm"])
    return lib


def _run_pins(lib):
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


@pytest.fixture(scope="module")
def original_text():
    with open(SRC) as f:
        return f.read()


def test_unmodified_copy_passes(tmp_path, original_text):
    assert _run_pins(_build(str(tmp_path), original_text, "control")) == 0


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, original_text, name, orig, bad):
    assert original_text.count(orig) >= 1, f"mutation site for {name} not found"
    text = original_text.replace(orig, bad)
    assert _run_pins(_build(str(tmp_path), text, name)) != 0, f"pins did not catch {name}"
