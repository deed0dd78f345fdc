"""The oracle's pins catch plausible mistakes (a check of the pins, CPU only).

Each case plants one mistake in a copy of ``oracle/wide_oracle.py`` (a textual edit:
a sign, an index, a dropped term, a wrong tie rule ...), puts that copy in a scratch
directory next to copies of ``tests/`` and ``synth/``, and runs the oracle pin tests
there in a subprocess.  The pins must fail for every mistake; with the unmodified
oracle they must pass.  The edits touch only the scratch copy."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "wide_oracle.py")

# (name, text in the oracle, replacement, pin files that must catch it)
MUTATIONS = [
    ("rope sign", "x1 * c - x2 * s", "x1 * c + x2 * s", ["test_oracle_attn.py"]),
    ("rope frequency", "(-(2.0 * np.arange(half, dtype=dtype)) / hd)",
     "(-(1.0 * np.arange(half, dtype=dtype)) / hd)", ["test_oracle_attn.py"]),
    ("attention scale", "scale = 1.0 / np.sqrt(hd)", "scale = 1.0 / hd", ["test_oracle_attn.py"]),
    ("causal excludes self", "np.arange(T)[None, :] <= R[:, None]",
     "np.arange(T)[None, :] < R[:, None]", ["test_oracle_attn.py"]),
    ("phantom keys (dropped tokens stay in the softmax)",
     "allowed = causal[sel] & keep[None, :, g]", "allowed = causal[sel]",
     ["test_oracle_attn.py"]),
    ("GQA head map", "g = h // r", "g = h % n_kv", ["test_oracle_attn.py"]),
    ("decode without the new key",
     "keys = np.concatenate([Kc[b, g, :lb], K[b, g][None]], axis=0)",
     "keys = np.concatenate([Kc[b, g, :lb], 0.0 * K[b, g][None]], axis=0)",
     ["test_oracle_attn.py"]),
    ("missing silu", "H = _silu(A) * B", "H = A * B", ["test_oracle_ffn.py"]),
    ("groups interleaved instead of contiguous", "np.repeat(m, G, axis=1)",
     "np.tile(m, (1, G))", ["test_oracle_ffn.py"]),
    ("unstable partition", "order = active + inactive",
     "order = active + inactive[::-1]", ["test_oracle_reorder.py"]),
    ("big-endian bit packing", "<< np.uint64(j)\n\n    count", "<< np.uint64(63 - j)\n\n    count",
     ["test_oracle_reorder.py"]),
    ("rmsnorm without eps", "np.mean(x * x, axis=-1, keepdims=True) + eps)",
     "np.mean(x * x, axis=-1, keepdims=True))", ["test_oracle_layer.py"]),
    ("layer without the second residual", "    y = h + f\n", "    y = f\n",
     ["test_oracle_layer.py"]),
    ("router ties to the higher group", "(row[h] == row[g] and h < g)",
     "(row[h] == row[g] and h > g)", ["test_oracle_router.py"]),
]


def _scratch(tmp, name, src):
    d = os.path.join(tmp, name.replace(" ", "_").replace("(", "").replace(")", ""))
    os.makedirs(os.path.join(d, "oracle"))
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), os.path.join(d, "oracle"))
    with open(os.path.join(d, "oracle", "wide_oracle.py"), "w") as f:
        f.write(src)
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(d, "synth"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), os.path.join(d, "tests"),
                    ignore=shutil.ignore_patterns("__pycache__", "golden"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
    return d


def _pins_pass(d, files):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join("tests", f) for f in files]]
    r = subprocess.run(cmd, cwd=d, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode == 0, r.stdout[-1500:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(ORACLE).read()
    for name, old, new, _ in MUTATIONS:
        assert src.count(old) == 1, f"mutation site not unique or missing: {name}"
    files = sorted({f for m in MUTATIONS for f in m[3]})
    jobs = [("unmodified", src, files)]
    jobs += [(name, src.replace(old, new), fs) for name, old, new, fs in MUTATIONS]
    dirs = [(name, _scratch(str(tmp_path), name, s), fs) for name, s, fs in jobs]
    workers = max(1, min(4, (os.cpu_count() or 2) // 2))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: (j[0],) + _pins_pass(j[1], j[2]), dirs))
    base = results[0]
    assert base[1], f"pins fail on the unmodified oracle:\n{base[2]}"
    survivors = [name for name, ok, _ in results[1:] if ok]
    assert not survivors, f"mistakes no pin catches: {survivors}"
