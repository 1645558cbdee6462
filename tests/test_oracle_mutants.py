"""The oracle's pins are strong enough: a copy of the oracle with one plausible mistake planted
must fail tests/test_oracle.py, for every mistake below (a dropped term, a wrong sign or index, a
transposed operand, a missing rounding). Each mutant runs the pin suite in a subprocess with
the mutated package first on the import path.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    ("drop_score_scale", "/ np.sqrt(d)", "/ 1.0"),
    ("causal_off_by_one", "p = L + int(t)  ", "p = L + int(t) + 1"),
    ("gqa_head_map", "for h in range(g * G, (g + 1) * G):", "for h in range(g, Hq, Hkv):"),
    ("no_max_subtraction", "w = np.exp(s - m)", "w = np.exp(s)"),
    ("rounding_truncates", "np.rint(xs / quantum)", "np.trunc(xs / quantum)"),
    ("append_off_by_one", "cache[b, g, p:p + T, :]", "cache[b, g, p + 1:p + T + 1, :]"),
    ("query_reversed", "(K[: p + 1] @ q[b, r, h])", "(K[: p + 1] @ q[b, r, h][::-1])"),
    ("page_row_off_by_one", "pool[table[b, j // PAGE_TOKENS], :, j % PAGE_TOKENS, :]",
     "pool[table[b, j // PAGE_TOKENS], :, (j + 1) % PAGE_TOKENS, :]"),
    ("page_and_row_swapped", "pool[table[b, j // PAGE_TOKENS], :, j % PAGE_TOKENS, :]",
     "pool[table[b, j % PAGE_TOKENS], :, j // PAGE_TOKENS, :]"),
    ("rmsnorm_without_eps", "np.mean(x * x, axis=-1, keepdims=True) + eps)", "np.mean(x * x, axis=-1, keepdims=True))"),
    ("rmsnorm_sum_not_mean", "np.mean(x * x, axis=-1, keepdims=True)", "np.sum(x * x, axis=-1, keepdims=True)"),
    ("silu_sign", "return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))"),
    ("swiglu_gate_up_swapped", "return silu(gu[..., :F]) * gu[..., F:]", "return silu(gu[..., F:]) * gu[..., :F]"),
    ("stack_no_residual", 'h = round_to_dtype(h + project(o, lw["wo"]), dtype)', 'h = round_to_dtype(project(o, lw["wo"]), dtype)'),
    ("stack_activation_unrounded", "act = round_to_dtype(swiglu(gu), dtype)", "act = swiglu(gu)"),
    ("stack_wrong_norm_weight", 'rmsnorm(h, lw["g_mlp"], eps)', 'rmsnorm(h, lw["g_attn"], eps)'),
    ("rope_sin_sign", "[lo * c - hi * s, hi * c + lo * s]", "[lo * c + hi * s, hi * c - lo * s]"),
    ("rope_interleaved_pairs", "lo, hi = x[..., :half], x[..., half:]", "lo, hi = x[..., 0::2], x[..., 1::2]"),
    ("rope_frequency_exponent", "(-2.0 * np.arange(half, dtype=np.float64) / d)",
     "(-1.0 * np.arange(half, dtype=np.float64) / d)"),
    ("rope_position_off_by_one", "pos = np.asarray(past_len, dtype=np.int64)[:, None] + np.arange(T)[None, :]",
     "pos = np.asarray(past_len, dtype=np.int64)[:, None] + 1 + np.arange(T)[None, :]"),
    ("rope_query_unrotated", "q = rope(q, pos[:, ts], rope_theta)", "q = q"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    dst = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst)
    src = (dst / "__init__.py").read_text()
    assert src.count(old) >= 1, f"{name}: pattern not found"
    (dst / "__init__.py").write_text(src.replace(old, new, 1))
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]))
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"{name}: the pins did not catch it (rc {r.returncode})\n{r.stdout[-2000:]}"
