"""Planted mistakes: each one is a plausible error in the oracle (a wrong
nibble, bit field, index, sign, position or order), planted in a scratch copy
of oracle.c on the CPU.  The oracle's pins must turn red for every one of
them, so a mistake of that kind in the oracle itself could not have passed.

Each case copies oracle/, synth/ and the oracle tests into a temporary
directory, applies the replacement to the copy of oracle.c (the repository's
file is never touched), and runs the oracle's pin files there in a
subprocess; the case passes when at least one pin fails.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_dequant.py", "tests/test_oracle_gemv.py", "tests/test_oracle_scalars.py",
        "tests/test_oracle_layer_parts.py", "tests/test_oracle_layer.py", "tests/test_oracle_skip.py"]

# (name, [(text in oracle.c, replacement), ...])
MUTATIONS = [
    ("q4_0 nibble order",
     [("w[j] = d * (double)((qs[j] & 15) - 8);\n        w[j + 16] = d * (double)((qs[j] >> 4) - 8);",
       "w[j] = d * (double)((qs[j] >> 4) - 8);\n        w[j + 16] = d * (double)((qs[j] & 15) - 8);")]),
    ("q4_0 offset", [("w[j] = d * (double)((qs[j] & 15) - 8);", "w[j] = d * (double)((qs[j] & 15) - 7);")]),
    ("q4_k min high bits", [("*min = (sc[s + 4] >> 4) | ((sc[s] >> 6) << 4);",
                             "*min = (sc[s + 4] >> 4) | ((sc[s - 4] >> 6) << 4);")]),
    ("q4_k nibble order", [("int q = ((e / 32) % 2) ? (byte >> 4) : (byte & 15);",
                            "int q = ((e / 32) % 2) ? (byte & 15) : (byte >> 4);")]),
    ("q6_k qh shift", [("int hi = (qh[32 * n + l] >> (2 * k)) & 3;", "int hi = (qh[32 * n + l] >> (2 * (k ^ 1))) & 3;")]),
    ("q6_k scale index", [("w[e] = d * (double)sc[e / 16] * (double)(q - 32);",
                           "w[e] = d * (double)sc[(e / 16) ^ 1] * (double)(q - 32);")]),
    ("q8_0 sign", [("w[j] = d * (double)(int8_t)b[2 + j];", "w[j] = d * (double)b[2 + j];")]),
    ("gqa mapping", [("int g = h / group;", "int g = h % n_kv;")]),
    ("rope pairing",
     [("double a = p[2 * i], b = p[2 * i + 1];\n      p[2 * i] = a * c - b * s;\n      p[2 * i + 1] = a * s + b * c;",
       "double a = p[i], b = p[i + head_dim / 2];\n      p[i] = a * c - b * s;\n      p[i + head_dim / 2] = a * s + b * c;")]),
    ("rope direction", [("p[2 * i] = a * c - b * s;\n      p[2 * i + 1] = a * s + b * c;",
                         "p[2 * i] = a * c + b * s;\n      p[2 * i + 1] = -a * s + b * c;")]),
    ("query not rotated", [("or_rope(q + (int64_t)i * nq, c->n_head, hd, p, c->rope_theta);", "")]),
    ("query rotated one position on",
     [("or_rope(q + (int64_t)i * nq, c->n_head, hd, p, c->rope_theta);",
       "or_rope(q + (int64_t)i * nq, c->n_head, hd, p + 1, c->rope_theta);")]),
    ("key not rotated", [("or_rope(k, c->n_kv_head, hd, p, c->rope_theta);", "")]),
    ("new token left out of attention", [("pos + i + 1, o);", "pos + i, o);")]),
    ("attention scale", [("s[t] = dot / sqrt((double)hd);", "s[t] = dot / (double)hd;")]),
    ("swapped swiglu", [("g[r] = or_silu(g[r]) * u[r];", "g[r] = or_silu(u[r]) * g[r];")]),
    ("first residual dropped", [("for (int r = 0; r < H; ++r) xi[r] += t[r]; /* h = x + Wo o */",
                                 "for (int r = 0; r < H; ++r) xi[r] = t[r]; /* h = x + Wo o */")]),
    ("ffn norm on the layer input", [("or_rmsnorm(xi, L->ffn_norm, H, c->rms_eps, xn);", "")]),
    ("argmax tie rule", [("if (v[i] > v[best]) best = i;", "if (v[i] >= v[best]) best = i;")]),
    ("output norm bypassed", [("or_rmsnorm(x + (int64_t)i * H, m->out_norm, H, m->cfg.rms_eps, xn);",
                               "memcpy(xn, x + (int64_t)i * H, sizeof(double) * H);")]),
    ("rmsnorm gain dropped", [("out[i] = x[i] * r * (double)g[i];", "out[i] = x[i] * r;")]),
    ("rmsnorm eps outside the root", [("double r = 1.0 / sqrt(ss / (double)n + eps);",
                                       "double r = 1.0 / (sqrt(ss / (double)n) + eps);")]),
    ("f16 append rounds down", [("if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;", "")]),
]


def _run(name, reps, tmp):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    for a, b in reps:
        assert src.count(a) == 1, f"{name}: the text to replace is not in oracle.c exactly once: {a!r}"
        src = src.replace(a, b)
    d = os.path.join(tmp, name.replace(" ", "_"))
    os.makedirs(d)
    for sub in ("oracle", "synth"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(d, sub),
                        ignore=shutil.ignore_patterns("liboracle.so", "__pycache__", "*.tmp*"))
    os.makedirs(os.path.join(d, "tests", "golden"))
    helpers = ["conftest.py", "__init__.py", "blocks.py", "stack_util.py", "gpu_util.py"]
    for f in helpers + [os.path.basename(p) for p in PINS]:
        p = os.path.join(ROOT, "tests", f)
        if os.path.exists(p):
            shutil.copy(p, os.path.join(d, "tests", f))
    for f in os.listdir(os.path.join(ROOT, "tests", "golden")):
        small = os.path.getsize(os.path.join(ROOT, "tests", "golden", f)) < 1 << 20
        if (f.endswith(".json") and small) or f.endswith(".py"):
            shutil.copy(os.path.join(ROOT, "tests", "golden", f), os.path.join(d, "tests", "golden", f))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), d)
    open(os.path.join(d, "oracle", "oracle.c"), "w").write(src)
    env = dict(os.environ, OMP_NUM_THREADS="1", PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + PINS,
                       cwd=d, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-600:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        control = ex.submit(_run, "unchanged", [], str(tmp_path))
        futs = {name: ex.submit(_run, name, reps, str(tmp_path)) for name, reps in MUTATIONS}
        results = {name: f.result() for name, f in futs.items()}
        rc, out = control.result()
    assert rc == 0, f"the unchanged copy of the oracle fails its pins: {out}"
    survived = [name for name, (rc, _) in results.items() if rc == 0]
    broken = [(name, out) for name, (rc, out) in results.items() if rc not in (0, 1)]
    assert not broken, f"pin runs that did not complete: {broken}"
    assert not survived, f"planted mistakes that no pin caught: {survived}"
