"""The oracle's pins catch plausible mistakes.

Each case below plants one mistake in a copy of the oracle (a dropped term, a wrong sign or
index, a reversed tie rule, a wrong head map or causal window, ...), runs the oracle's pin files
against that copy in a child process, and requires at least one pin to fail.  The unchanged copy
must pass.  Nothing here touches the oracle in the repository: the copies live in a temporary
directory, on the CPU."""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_pins.py", "tests/test_sketch_oracle.py"]

# (name, file under oracle/, function whose body is edited, old text, new text)
MUTANTS = [
    ("dropped score scale", "reference.py", "scaled_scores",
     "return (keys @ q_row) * scale", "return (keys @ q_row)"),
    ("magnitude ranking", "reference.py", "topk_positions",
     "order = np.argsort(-s32, kind=\"stable\")",
     "order = np.argsort(-np.abs(s32), kind=\"stable\")"),
    ("reversed tie rule", "reference.py", "topk_positions",
     "order = np.argsort(-s32, kind=\"stable\")",
     "order = s32.shape[0] - 1 - np.argsort(-s32[::-1], kind=\"stable\")"),
    ("float64 ranking", "reference.py", "topk_positions",
     "s32 = np.asarray(scores, dtype=np.float64).astype(np.float32)",
     "s32 = np.asarray(scores, dtype=np.float64)"),
    ("causal window one short", "reference.py", "visible_length",
     "return int(seq_len) - int(q_len) + int(t) + 1", "return int(seq_len) - int(q_len) + int(t)"),
    ("lse without the max", "reference.py", "attend",
     "float(m + math.log(l))", "float(math.log(l))"),
    ("exponent not shifted by the max", "reference.py", "attend",
     "e = np.exp(s - m)", "e = np.exp(s)"),
    ("weights not normalised", "reference.py", "attention_weights",
     "return w / w.sum()", "return w"),
    ("padding not skipped", "reference.py", "row_sparse",
     "pos = pos[pos != -1]", "pos = pos"),
    ("unweighted merge", "reference.py", "lse_merge",
     "o = sum(wi * oi for wi, (oi, _) in zip(w, live)) / w.sum()",
     "o = sum(oi for (oi, _) in live) / len(live)"),
    ("page index by remainder", "reference.py", "_rows",
     "pages = self.page_table[b, n // self.page_size]",
     "pages = self.page_table[b, n % self.page_size]"),
    ("slot by quotient", "reference.py", "_rows",
     "bits[pages, h, n % self.page_size]", "bits[pages, h, n // self.page_size]"),
    ("indexer head map hq % Hkv", "reference.py", "decode_topk",
     "h = hq // G", "h = hq % Hkv"),
    ("sparse head map hq % Hkv", "reference.py", "decode_sparse",
     "h = hq // G", "h = hq % Hkv"),
    ("sparse window ignores the token", "reference.py", "decode_sparse",
     "visible_length(cache.seq_lens[b], T, t)", "visible_length(cache.seq_lens[b], T, 0)"),
    ("sparse window ignores T", "reference.py", "decode_sparse",
     "visible_length(cache.seq_lens[b], T, t)", "visible_length(cache.seq_lens[b], 1, 0)"),
    ("dense head map hq % Hkv", "reference.py", "decode_dense",
     "h = hq // G", "h = hq % Hkv"),
    ("dense window ignores the token", "reference.py", "decode_dense",
     "visible_length(cache.seq_lens[b], T, t)", "visible_length(cache.seq_lens[b], T, 0)"),
    ("sketch scale m/128", "sketch.py", "int8_sketch",
     "m / np.float32(127.0)", "m / np.float32(128.0)"),
    ("sketch signed maximum", "sketch.py", "int8_sketch",
     "m = np.abs(x).max(axis=1)", "m = x.max(axis=1)"),
    ("sketch rounds half away from zero", "sketch.py", "int8_sketch",
     "q = np.rint(x[live] / scale[live][:, None]).astype(np.float32)",
     "r = x[live] / scale[live][:, None]; q = (np.sign(r) * np.floor(np.abs(r) + 0.5)).astype(np.float32)"),
    ("one extra candidate", "sketch.py", "sketch_candidates",
     "nc = min(int(cand_mult) * kk, visible)", "nc = min(int(cand_mult) * kk + 1, visible)"),
    ("candidates: reversed tie rule", "sketch.py", "sketch_candidates",
     "np.argsort(-approx, kind=\"stable\")[:nc]",
     "(approx.shape[0] - 1 - np.argsort(-approx[::-1], kind=\"stable\"))[:nc]"),
    ("no exact re-rank", "sketch.py", "row_topk_sketch",
     "keep = np.argsort(-s32, kind=\"stable\")[:kk]", "keep = np.arange(kk)"),
]


def _mutate(src: str, func: str, old: str, new: str) -> str:
    start = src.index(f"def {func}(")
    nxt = src.find("\ndef ", start + 1)
    nxt_cls = src.find("\nclass ", start + 1)
    ends = [e for e in (nxt, nxt_cls) if e != -1]
    end = min(ends) if ends else len(src)
    body = src[start:end]
    assert body.count(old) == 1, (func, old)
    return src[:start] + body.replace(old, new) + src[end:]


def _copy_tree(dst: str) -> None:
    for d in ("oracle", "workloads"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d),
                        ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    for f in ("conftest.py", "_util.py", "test_oracle_pins.py", "test_sketch_oracle.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), os.path.join(dst, "pytest.ini"))


def _run_pins(tmp_root: str, mutant) -> int:
    d = os.path.join(tmp_root, "case")
    _copy_tree(d)
    if mutant is not None:
        _, fname, func, old, new = mutant
        path = os.path.join(d, "oracle", fname)
        with open(path) as f:
            src = f.read()
        with open(path, "w") as f:
            f.write(_mutate(src, func, old, new))
    env = dict(os.environ)
    env.pop("PYTHONPATH", None)
    env["OMP_NUM_THREADS"] = "1"
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_FILES],
        cwd=d, env=env, capture_output=True, text=True, timeout=600,
    )
    return r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    cases = [None] + MUTANTS
    roots = []
    for i in range(len(cases)):
        p = tmp_path / f"m{i}"
        p.mkdir()
        roots.append(str(p))
    with ThreadPoolExecutor(max_workers=4) as ex:
        codes = list(ex.map(_run_pins, roots, cases))
    assert codes[0] == 0, "the unchanged oracle copy must pass its pins"
    survivors = [m[0] for m, c in zip(MUTANTS, codes[1:]) if c == 0]
    assert not survivors, f"planted mistakes no pin catches: {survivors}"
    assert all(c == 1 for c in codes[1:]), codes  # 1 = tests failed (not a crash of the runner)
