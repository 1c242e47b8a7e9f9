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
GC_LINE = ("gc[(size_t)s * V + v] += tmp[s] * ((double)g[t * V + v] + (2.0 / T) * (wv - cv) * "
           "(rt[s] + rbcur[s] - mr));")
MUTANTS = [
    ("pred_shift_amount", "return (s >> k) | (a << (L - k));", "return (s >> k) | (a << k);"),
    ("succ_drops_new_bits", "return ((s << k) & ((1u << L) - 1u)) | b;", "return ((s << k) & ((1u << L) - 1u));"),
    ("weight_sign", "return -e / T;", "return e / T;"),
    ("weight_drops_T", "return -e / T;", "return -e;"),
    ("weight_drops_components", "        e += d * d;", "        e = d * d;"),
    ("backward_wrong_step", "x[b] = log_weight(w + (t + 1) * V, c + (size_t)u * V, V, T) + bnext[u];",
     "x[b] = log_weight(w + t * V, c + (size_t)u * V, V, T) + bnext[u];"),
    ("sigma_start_rule", "alpha[s] = (!has_sigma || (s >> k) == (sigma & gmask)) ? th : -INFINITY;",
     "alpha[s] = (!has_sigma || (s & gmask) == (sigma >> k)) ? th : -INFINITY;"),
    ("sigma_end_rule", "b[s] = (!has_sigma || s == sigma) ? 0.0 : -INFINITY;",
     "b[s] = (!has_sigma || (s >> 1) == (sigma >> 1)) ? 0.0 : -INFINITY;"),
    ("posterior_unnormalised", "acc += (double)c[(size_t)s * V + v] * exp(tmp[s] - lnz);",
     "acc += (double)c[(size_t)s * V + v] * exp(tmp[s]);"),
    ("codebook_layout_transposed", "acc += (double)c[(size_t)s * V + v] * exp(tmp[s] - lnz);",
     "acc += (double)c[(size_t)v * S + s] * exp(tmp[s] - lnz);"),
    ("lse_drops_max", "return mx + log(s);", "return log(s);"),
    ("grad_factor", "grad[t * V + v] = (2.0 / T) * cov[v];", "grad[t * V + v] = (1.0 / T) * cov[v];"),
    ("grad_dot_drops_components", "for (int v = 0; v < V; ++v) e += (double)gt[v] * (double)cs[v];",
     "for (int v = 0; v < V; ++v) e = (double)gt[v] * (double)cs[v];"),
    ("grad_forward_drops_history", "rt[s] = dot_v(g + t * V, c + (size_t)s * V, V) + acc;",
     "rt[s] = dot_v(g + t * V, c + (size_t)s * V, V);"),
    ("grad_backward_index", "acc += pw[b] * (dot_v(g + (t + 1) * V, c + (size_t)u * V, V) + rbnext[u]);",
     "acc += pw[b] * (dot_v(g + t * V, c + (size_t)u * V, V) + rbnext[u]);"),
    ("grad_uncentred_codeword",
     "cov[v] += tmp[s] * ((double)c[(size_t)s * V + v] - m0[v]) * (rt[s] + rbcur[s] - mr);",
     "cov[v] += tmp[s] * ((double)c[(size_t)s * V + v]) * (rt[s] + rbcur[s] - mr) * 0.5;"),
    ("codebook_drops_direct_term", "GC",
     "gc[(size_t)s * V + v] += tmp[s] * ((2.0 / T) * (wv - cv) * (rt[s] + rbcur[s] - mr));"),
    ("codebook_residual_sign", "GC",
     "gc[(size_t)s * V + v] += tmp[s] * ((double)g[t * V + v] + (2.0 / T) * (cv - wv) * (rt[s] + rbcur[s] - mr));"),
    ("codebook_uncentred", "GC",
     "gc[(size_t)s * V + v] += tmp[s] * ((double)g[t * V + v] + (2.0 / T) * (wv - cv) * (rt[s] + rbcur[s]));"),
    ("codebook_factor", "GC",
     "gc[(size_t)s * V + v] += tmp[s] * ((double)g[t * V + v] + (1.0 / T) * (wv - cv) * (rt[s] + rbcur[s] - mr));"),
    ("viterbi_tie_rule", "if (v < best) { best = v; arg = a; }", "if (v <= best) { best = v; arg = a; }"),
    ("viterbi_end_tie_rule", "if (mcur[s] < mcur[s_end]) s_end = s;", "if (mcur[s] <= mcur[s_end]) s_end = s;"),
    ("viterbi_metric_in_double", "    float d = wt[0] - cs[0];\n    float e = d * d;",
     "    double d = (double)wt[0] - (double)cs[0];\n    float e = (float)(d * d);"),
    ("viterbi_components_fused", "        e = e + ev;", "        e = fmaf(dv, dv, e);"),
]
MUTANTS = [(nm, GC_LINE if o == "GC" else o, b) for nm, o, b in MUTANTS]


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
