"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of oracle/rope_oracle.c (a flipped sign, a
dropped term, cos and sin swapped, an index shifted within a pair, pairs counted from 0
instead of the slice start, the two styles swapped, an mrope section boundary off by one, a
rounding slip, a broken pass-through), builds it, and runs the pin tests against it in a
child process: at least one pin must fail for every mutant.  The real oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rope_oracle.c")

# (name, text to replace, replacement, pin tests to run (-k expression))
MUTANTS = [
    ("interleave y0 sign", "float q0 = (-bb) * s0;", "float q0 = bb * s0;",
     "golden_inplace or matrices"),
    ("interleave dropped term", "float q1 = a * s1;\n            y1 = p1 + q1;",
     "float q1 = a * s1;\n            y1 = p1;", "golden_inplace or matrices"),
    ("cos and sin swapped", "float c0 = load_f32(cos_t, crow + 2 * i), c1 = load_f32(cos_t, crow + 2 * i + 1);",
     "float c0 = load_f32(sin_t, crow + 2 * i), c1 = load_f32(sin_t, crow + 2 * i + 1);",
     "golden_inplace or matrices or exact_angles"),
    ("cos index within pair", "c1 = load_f32(cos_t, crow + 2 * i + 1);", "c1 = load_f32(cos_t, crow + 2 * i);",
     "matrices"),
    ("pairs from 0 not from start", "int64_t j0 = xrow + start + 2 * i, j1 = j0 + 1;",
     "int64_t j0 = xrow + 2 * i, j1 = j0 + 1;", "golden_inplace or untouched"),
    ("broadcast operands transposed",
     "int64_t crow = ((bc * cos_t->shape[1] + sc) * cos_t->shape[2] + nc) * L;",
     "int64_t crow = ((sc * cos_t->shape[0] + bc) * cos_t->shape[2] + nc) * L;", "matrices"),
    ("NeoX partner index", "if (is_neox_style) { ja = i; jb = i + half; }",
     "if (is_neox_style) { ja = i; jb = half - 1 - i; }", "complex or golden_page or styles"),
    ("styles swapped", "if (is_neox_style) { ja = i; jb = i + half; }",
     "if (!is_neox_style) { ja = i; jb = i + half; }", "golden_page or golden_styles"),
    ("NeoX o1 sign", "float o1 = a * c - bb * s;", "float o1 = a * c + bb * s;", "golden_page or complex"),
    ("cache sin read from cos half", "cs_sin[i] = load_f32(cache, p * cache->stride[0] + half + i);",
     "cs_sin[i] = load_f32(cache, p * cache->stride[0] + i);", "complex or relative"),
    ("mrope boundary off by one", "if (i < acc) { row_sel = k; break; }",
     "if (i <= acc) { row_sel = k; break; }", "mrope or complex"),
    ("pass-through shortened", "for (int64_t j = rd; j < head_size; ++j) {",
     "for (int64_t j = rd + 1; j < head_size; ++j) {", "pass_through or golden_styles"),
    ("bf16 ties round up", "if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;",
     "if (dropped >= 0x8000u) kept += 1u;", "rounding_ties"),
    ("f16 ties round up", "if (rem > half || (rem == half && (q & 1u))) q += 1;",
     "if (rem >= half) q += 1;", "rounding_ties"),
    ("f16 subnormal quantum", "int Ec = E < -14 ? -14 : E;", "int Ec = E < -15 ? -15 : E;",
     "rounding_ties"),
    ("backward sign", "y1 = p1 - q1;", "y1 = p1 + q1;", "backward or twin"),
    ("backward uses forward's sin index", "float q0 = bb * s1;", "float q0 = bb * s0;",
     "backward or twin"),
    ("interleaved residue", "if (i % 3 == 1 && i < 3 * sec[1]) row_sel = 1;",
     "if (i % 3 == 2 && i < 3 * sec[1]) row_sel = 1;", "interleaved"),
    ("interleaved bound", "else if (i % 3 == 2 && i < 3 * sec[1]) row_sel = 2;",
     "else if (i % 3 == 2 && i < 3 * sec[1] - 3) row_sel = 2;", "interleaved"),
    ("f16 subnormal decode", "v = ldexpf((float)m, -24);", "v = ldexpf((float)m, -23);",
     "decoding"),
    ("half mode rotate sign", "const float rot = i < h ? -v[i + h] : v[i - h];",
     "const float rot = i < h ? v[i + h] : -v[i - h];", "half"),
    ("half mode partner index", "const float rot = i < h ? -v[i + h] : v[i - h];",
     "const float rot = i < h ? -v[h - 1 - i] : v[L - 1 - i];", "half"),
    ("half mode backward sign", "q = -(v[i - h] * sp);", "q = v[i - h] * sp;", "half"),
    ("half mode backward sin index", "const float sp = load_f32(sin_t, crow + i + h);",
     "const float sp = load_f32(sin_t, crow + i);", "half"),
]


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, pins, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not found exactly once: {old}"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
                    str(mutant_c), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ROPE_ORACLE_LIB=str(lib))
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", pins],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"mutant '{name}' survived the pins:\n{res.stdout[-2000:]}"
    assert "passed" in res.stdout or "failed" in res.stdout or res.returncode < 0, res.stdout[-500:]
