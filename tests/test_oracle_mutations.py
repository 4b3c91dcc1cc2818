"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a temporary copy of one oracle C source (a unique text replacement:
a dropped scale, a mask off by one, a transposed operand, a wrong stride or decode, a missing term of
the backward, an ignored block mask), builds that copy with gcc, and runs the pin tests of that
oracle against it in a child process (FA_ORACLE_LIB names the build). The numpy parts of the oracle
(the log-space merge, the attention of T queries over a key range, the E4M3 decode) are mutated the
same way in a temporary copy of the source tree, whose own oracle package the child imports. Every
mutant must fail at least one pin; an unmutated copy passes all of them.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ORACLE = os.path.join(ROOT, "oracle")
SOURCES = ("fa_ref.c", "fa_ref_bwd.c", "fa_ref_sparse.c")

FWD_PINS = ["test_oracle_pins.py"]
BWD_PINS = ["test_oracle_bwd_pins.py"]
SPARSE_PINS = ["test_oracle_sparse_pins.py"]

# (name, file, [(old, new), ...], pin files)
MUTANTS = [
    ("fwd: scale dropped", "fa_ref.c", [("    scores[j] = scale * dot;", "    scores[j] = dot;")], FWD_PINS),
    ("fwd: causal mask one key too many", "fa_ref.c",
     [("causal ? i + 1 : T; /* visible", "causal ? (i + 2 < T ? i + 2 : T) : T; /* visible")], FWD_PINS),
    ("fwd: causal mask one key too few", "fa_ref.c",
     [("causal ? i + 1 : T; /* visible", "causal ? (i > 0 ? i : 1) : T; /* visible")], FWD_PINS),
    ("fwd: LSE in base 2", "fa_ref.c", [("*lse_out = m + log(l);", "*lse_out = m + log2(l);")], FWD_PINS),
    ("fwd: max not subtracted", "fa_ref.c",
     [("exp(scores[j] - m)", "exp(scores[j])"), ("*lse_out = m + log(l);", "*lse_out = log(l);")], FWD_PINS),
    ("fwd: max left out of the LSE", "fa_ref.c", [("*lse_out = m + log(l);", "*lse_out = log(l);")], FWD_PINS),
    ("fwd: V read transposed", "fa_ref.c",
     [("o_row[c] += e * bf16_bits_to_double(v_row[c]);", "o_row[c] += e * bf16_bits_to_double(vh[c * T + j]);")],
     FWD_PINS),
    ("fwd: K rows taken for Q", "fa_ref.c",
     [("const uint16_t* q_row = qh + i * d;", "const uint16_t* q_row = kh + i * d;")], FWD_PINS),
    ("fwd: bf16 decode off by half an ulp", "fa_ref.c",
     [("uint32_t u = (uint32_t)bits << 16;", "uint32_t u = ((uint32_t)bits << 16) | 0x8000u;")], FWD_PINS),
    ("fwd: output not normalised", "fa_ref.c",
     [("for (int64_t c = 0; c < d; ++c) o_row[c] /= l;", "for (int64_t c = 0; c < d; ++c) o_row[c] /= 1.0;")],
     FWD_PINS),
    ("fwd: head stride wrong", "fa_ref.c",
     [("      const int64_t off = head * T * d;\n      attend_one_row(q + off, k + off, v + off, T, d, causal, scale, i, scores, o + r * d, lse + r);",
       "      const int64_t off = head * (T - 1) * d;\n      attend_one_row(q + off, k + off, v + off, T, d, causal, scale, i, scores, o + r * d, lse + r);")],
     FWD_PINS),
    ("bwd: D dropped", "fa_ref_bwd.c", [("const double ds = p[j] * (dp - D);", "const double ds = p[j] * dp;")],
     BWD_PINS),
    ("bwd: scale missing on dQ", "fa_ref_bwd.c",
     [("for (int64_t c = 0; c < d; ++c) dqi[c] *= scale;", "for (int64_t c = 0; c < d; ++c) dqi[c] *= 1.0;")],
     BWD_PINS),
    ("bwd: scale missing on dK", "fa_ref_bwd.c",
     [("for (int64_t x = 0; x < T * d; ++x) dk[x] *= scale;", "for (int64_t x = 0; x < T * d; ++x) dk[x] *= 1.0;")],
     BWD_PINS),
    ("bwd: dK from K instead of Q", "fa_ref_bwd.c",
     [("dk[j * d + c] += ds * qi[c];", "dk[j * d + c] += ds * k[j * d + c];")], BWD_PINS),
    ("bwd: P not normalised", "fa_ref_bwd.c",
     [("for (int64_t j = 0; j < n_keys; ++j) p[j] /= l;", "for (int64_t j = 0; j < n_keys; ++j) p[j] /= 1.0;")],
     BWD_PINS),
    ("bwd: causal mask one key too many", "fa_ref_bwd.c",
     [("    const int64_t n_keys = causal ? i + 1 : T;\n    const double* qi",
       "    const int64_t n_keys = causal ? (i + 2 < T ? i + 2 : T) : T;\n    const double* qi")], BWD_PINS),
    ("bwd: dP from K", "fa_ref_bwd.c", [("dp += doi[c] * v[j * d + c];", "dp += doi[c] * k[j * d + c];")],
     BWD_PINS),
    ("bwd: D from V", "fa_ref_bwd.c", [("D += doi[c] * o_row[c];", "D += doi[c] * v[i * d + c];")], BWD_PINS),
    ("sparse: mask ignored", "fa_ref_sparse.c",
     [("vis[j] = mrow[j / block_n] != 0 && (!causal || j <= i);", "vis[j] = (!causal || j <= i);")], SPARSE_PINS),
    ("sparse: key block from the query block size", "fa_ref_sparse.c",
     [("vis[j] = mrow[j / block_n] != 0", "vis[j] = mrow[j / block_m] != 0")], SPARSE_PINS),
    ("sparse: causal flag ignored", "fa_ref_sparse.c",
     [("vis[j] = mrow[j / block_n] != 0 && (!causal || j <= i);", "vis[j] = mrow[j / block_n] != 0;")], SPARSE_PINS),
    ("sparse: empty row gets LSE 0", "fa_ref_sparse.c", [("lse[r] = -INFINITY;", "lse[r] = 0.0;")], SPARSE_PINS),
    ("sparse: per-head masks ignored", "fa_ref_sparse.c",
     [("(mask_heads == 1 ? 0 : head)", "(mask_heads == 1 ? 0 : 0)")], SPARSE_PINS),
]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")


def build_mutant(tmp, name, fname, edits):
    d = os.path.join(tmp, name.replace(" ", "_").replace(":", ""))
    os.makedirs(d)
    for src in SOURCES + ("fa_ref.h",):
        shutil.copy(os.path.join(ORACLE, src), d)
    path = os.path.join(d, fname)
    text = open(path).read()
    for old, new in edits:
        assert text.count(old) == 1, f"{name}: the planted edit must match exactly once: {old!r}"
        text = text.replace(old, new)
    open(path, "w").write(text)
    lib = os.path.join(d, "liboracle.so")
    r = subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", "-o", lib,
                        *[os.path.join(d, s) for s in SOURCES], "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


def run_pins(lib, pins):
    env = dict(os.environ, FA_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *[os.path.join(HERE, p) for p in pins]], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    return r.returncode, r.stdout[-800:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    libs = [(name, build_mutant(str(tmp_path), name, f, edits), pins) for name, f, edits, pins in MUTANTS]
    # control: an unmutated copy, built and run the same way, passes every pin file
    control = build_mutant(str(tmp_path), "control", "fa_ref.c", [])
    rc, out = run_pins(control, FWD_PINS + BWD_PINS + SPARSE_PINS)
    assert rc == 0, out
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda a: (a[0], *run_pins(a[1], a[2])), libs))
    survivors = [(name, out) for name, rc, out in results if rc == 0]
    for name, rc, out in results:
        print(f"[mutant] {name}: {'caught' if rc != 0 else 'SURVIVED'}", flush=True)
    assert not survivors, survivors


PY_PINS_SPLIT = ["test_oracle_splitkv_pins.py"]
PY_PINS_FP8 = ["test_oracle_fp8_pins.py"]
PY_PINS_BWD = ["test_oracle_bwd_pins.py"]
PY_MUTANTS = [
    ("merge: LSE without the max", [("lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))",
                                     "lse = np.where(empty, -np.inf, np.log(np.where(empty, 1.0, l)))")],
     PY_PINS_SPLIT),
    ("merge: weights not normalised", [("o = (w[..., None] * o_parts).sum(axis=0) / np.where(empty, 1.0, l)[..., None]",
                                        "o = (w[..., None] * o_parts).sum(axis=0)")], PY_PINS_SPLIT),
    ("cross: alignment off by one", [("visible = visible & (j <= i + (Tk - T))",
                                      "visible = visible & (j < i + (Tk - T))")], PY_PINS_SPLIT),
    ("cross: alignment dropped", [("visible = visible & (j <= i + (Tk - T))", "visible = visible & (j <= i)")],
     PY_PINS_SPLIT),
    ("cross: range end inclusive", [("visible = (j >= k_begin) & (j < k_end)", "visible = (j >= k_begin) & (j <= k_end)")],
     PY_PINS_SPLIT),
    ("cross: max not subtracted", [("e = np.exp(s - m_safe[:, None])", "e = np.exp(s)")], PY_PINS_SPLIT),
    ("cross: max left out of the LSE", [("lse[b, h] = np.where(has_key, m_safe + np.log(l_safe), -np.inf)",
                                         "lse[b, h] = np.where(has_key, np.log(l_safe), -np.inf)")], PY_PINS_SPLIT),
    ("cross: V in place of K", [("s = float(scale) * (qf @ kf.T)", "s = float(scale) * (qf @ vf.T)")], PY_PINS_SPLIT),
    ("e4m3: exponent bias 8", [("(1.0 + m / 8.0) * np.exp2(e - 7.0)", "(1.0 + m / 8.0) * np.exp2(e - 8.0)")],
     PY_PINS_FP8),
    ("e4m3: subnormal spacing 2^-10", [("np.where(e == 0, m * 2.0 ** -9,", "np.where(e == 0, m * 2.0 ** -10,")],
     PY_PINS_FP8),
    ("e4m3: NaN code missed", [("np.where((e == 15) & (m == 7), np.nan, out)", "np.where((e == 15) & (m == 6), np.nan, out)")],
     PY_PINS_FP8),
    ("fp8: v descale dropped", [("    v = e4m3_to_f64(v8) * vd\n    return attention_fwd_f64",
                                 "    v = e4m3_to_f64(v8)\n    return attention_fwd_f64")], PY_PINS_FP8),
    # the row-by-row oracles used on the full-size workloads
    ("fp8 rows: one key short", [("keys = i + 1 if causal else k.shape[0]", "keys = max(i, 1) if causal else k.shape[0]")],
     PY_PINS_FP8),
    ("fp8 rows: k descale dropped", [("e4m3_to_f64(k8[b, h]) * kd", "e4m3_to_f64(k8[b, h])")], PY_PINS_FP8),
    ("bwd rows: D dropped from dQ", [("ds = p * (V[vis] @ dO[i] - D[i])", "ds = p * (V[vis] @ dO[i])")], PY_PINS_BWD),
    ("bwd rows: key-side causal bound off by one", [("vis = idx >= j if causal else np.ones(T, dtype=bool)",
                                                     "vis = idx > j if causal else np.ones(T, dtype=bool)")],
     PY_PINS_BWD),
    ("bwd rows: scale missing on dK", [("dk[n] = scale * (ds @ Q[vis])", "dk[n] = ds @ Q[vis]")], PY_PINS_BWD),
    ("bwd rows: statistics mask off by one", [("s = np.where(idx[None, :kend] > idx[i0:i1, None], -np.inf, s)",
                                               "s = np.where(idx[None, :kend] >= idx[i0:i1, None], -np.inf, s)")],
     PY_PINS_BWD),
]


def copy_tree(dst):
    """The parts of the source tree the oracle pin tests import, with the built oracle library."""
    shutil.copytree(ORACLE, os.path.join(dst, "oracle"), ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "exact_tiled_attention_07_amd"), os.path.join(dst, "exact_tiled_attention_07_amd"),
                    ignore=shutil.ignore_patterns("__pycache__", "*.so", "csrc"))
    os.makedirs(os.path.join(dst, "tests"))
    for f in os.listdir(HERE):
        if f.endswith(".py") or f == "golden":
            src = os.path.join(HERE, f)
            (shutil.copytree if os.path.isdir(src) else shutil.copy)(src, os.path.join(dst, "tests", f))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), dst)
    if not os.path.exists(os.path.join(dst, "oracle", "liboracle.so")):
        subprocess.run([sys.executable, "-c", "import oracle; oracle.build()"], cwd=dst, check=True)


def run_pins_in_tree(root, pins):
    env = {k: v for k, v in os.environ.items() if k != "FA_ORACLE_LIB"}
    env["OMP_NUM_THREADS"] = "2"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *[os.path.join("tests", p) for p in pins]], env=env, cwd=root, capture_output=True,
                       text=True, timeout=600)
    return r.returncode, r.stdout[-800:]


def test_every_planted_mistake_in_the_numpy_oracle_fails_a_pin(tmp_path):
    control = str(tmp_path / "control")
    copy_tree(control)
    rc, out = run_pins_in_tree(control, PY_PINS_SPLIT + PY_PINS_FP8 + PY_PINS_BWD)
    assert rc == 0, out
    trees = []
    for n, (name, edits, pins) in enumerate(PY_MUTANTS):
        root = str(tmp_path / f"m{n}")
        copy_tree(root)
        path = os.path.join(root, "oracle", "__init__.py")
        text = open(path).read()
        for old, new in edits:
            assert text.count(old) == 1, f"{name}: the planted edit must match exactly once: {old!r}"
            text = text.replace(old, new)
        open(path, "w").write(text)
        trees.append((name, root, pins))
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda a: (a[0], *run_pins_in_tree(a[1], a[2])), trees))
    for name, rc, out in results:
        print(f"[mutant] {name}: {'caught' if rc != 0 else 'SURVIVED'}", flush=True)
    assert not [name for name, rc, _ in results if rc == 0]
