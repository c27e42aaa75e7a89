"""The pins must catch plausible mistakes in the oracle.

Each case below plants one mistake in a copy of the oracle's C source (a
dropped term, a wrong sign or index, a transposed operand, a wrong rounding
rule), builds it, and runs the pin suites against that build in a separate
process.  The pins pass on the real oracle (the other test files), so every
mutant must make at least one of them fail (or crash)."""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pa_oracle.c")

MUTANTS = {
    "slot_offset": ("int64_t o = pos % block_size;", "int64_t o = (pos + 1) % block_size;"),
    "slot_block": ("int64_t b = pos / block_size;", "int64_t b = pos / (block_size + 1);"),
    "position_shift": ("int64_t pos = (int64_t)seq_lens[i] - c + t;",
                       "int64_t pos = (int64_t)seq_lens[i] - c + t - (t > 0);"),
    "qsl_not_cumulative": ("qsl[i + 1] = qsl[i] + num_scheduled[i];", "qsl[i + 1] = num_scheduled[i];"),
    "seq_len_drops_scheduled": ("seq_lens[i] = num_computed[i] + num_scheduled[i];",
                                "seq_lens[i] = num_computed[i];"),
    "causal_excludes_self": ("return causal ? (ti->L - ti->c + ti->t + 1) : ti->L;",
                             "return causal ? (ti->L - ti->c + ti->t) : ti->L;"),
    "causal_top_left": ("return causal ? (ti->L - ti->c + ti->t + 1) : ti->L;",
                        "return causal ? (ti->t + 1) : ti->L;"),
    "gqa_modulo": ("int64_t kvh = h / g;", "int64_t kvh = h % H;"),
    "scale_dropped": ("    s *= scale;\n", "\n"),
    "softmax_sign": ("double w = exp(scores[j - k0] - m);", "double w = exp(m - scores[j - k0]);"),
    "normaliser_dropped": ("for (int64_t e = 0; e < D; ++e) o[e] = acc[e] / l;",
                           "for (int64_t e = 0; e < D; ++e) o[e] = acc[e];"),
    "value_from_key_pool": ("acc[e] += w * pool_elem(p, p->v, kv_index(p, bt_row, j, kvh, e), p->v_scale);",
                            "acc[e] += w * pool_elem(p, p->k, kv_index(p, bt_row, j, kvh, e), p->v_scale);"),
    "write_swaps_kv": ("if (store_elem(p, p->v, di, value, in_dtype, si, p->v_scale))",
                       "if (store_elem(p, p->v, di, key, in_dtype, si, p->v_scale))"),
    "pool_layout_transposed": ("return (((size_t)block * p->block_size + off) * p->num_kv_heads + head) * p->head_dim + dim;",
                               "return (((size_t)block * p->num_kv_heads + head) * p->block_size + off) * p->head_dim + dim;"),
    "bf16_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "fp8_tie_down": ("best = (lo % 2 == 0) ? lo : hi;", "best = lo;"),
    "fp8_subnormal_exponent": ("mag = ldexp((double)m / 8.0, -6);", "mag = ldexp((double)m / 8.0, -7);"),
    "fp8_bias": ("mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "fp8_no_saturation": ("if (a >= 448.0) {\n    best = 0x7E;", "if (a >= 448.0) {\n    best = 0x7F;"),
    "fp8_multiply_scale": ("float y = x / scale;", "float y = x * scale;"),
    "fp8_scale_not_applied": ("default: return oracle_e4m3_decode(((const uint8_t *)base)[idx]) * (double)scale;",
                              "default: return oracle_e4m3_decode(((const uint8_t *)base)[idx]);"),
    "negative_slot_written": ("if (slot < 0) continue;", "if (slot < -1) continue;"),
    "merge_without_rescale": ("for (int64_t r = 0; r < R; ++r) l += exp(ms[r] - m) * ls[r];",
                              "for (int64_t r = 0; r < R; ++r) l += ls[r];"),
    "merge_drops_local_sum": ("s += exp(ms[r] - m) * ls[r] * os[r * D + e];",
                              "s += exp(ms[r] - m) * os[r * D + e];"),
}

PIN_FILES = ["tests/test_oracle_metadata.py", "tests/test_oracle_fp8.py",
             "tests/test_oracle_attention.py"]


def _run_mutant(name, td):
    old, new = MUTANTS[name]
    src = open(SRC, encoding="utf-8").read()
    if src.count(old) != 1:
        return ("site", f"mutation site for {name} not found exactly once")
    path = os.path.join(td, f"{name}.c")
    with open(path, "w", encoding="utf-8") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(td, f"lib{name}.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", lib, path,
                    "-lm"], check=True)
    env = dict(os.environ, PA_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    return (r.returncode, r.stdout[-2000:])


@pytest.fixture(scope="module")
def mutant_results():
    workers = max(2, min(8, os.cpu_count() or 2))
    with tempfile.TemporaryDirectory() as td:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            futs = {n: ex.submit(_run_mutant, n, td) for n in MUTANTS}
            return {n: f.result() for n, f in futs.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(mutant_results, name):
    rc, log = mutant_results[name]
    assert rc != "site", log
    assert rc != 0, f"mutant {name} survived the pins:\n{log}"
