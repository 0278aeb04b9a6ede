"""The oracle's pins catch plausible mistakes: each case below plants one
single mistake in a copy of oracle/opr_oracle.py (a dropped term, a wrong
sign, index or operand, a rule of the pages misread) and runs the oracle's
CPU tests against that copy; at least one test must fail.  The copy lives in a
temporary directory with the seeded input generators, so the repository's
oracle is never touched."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in opr_oracle.py, its mutated form)
MUTATIONS = [
    ("r_out starts after h, not after t (position ids)",
     "s_rout = e_t + 1           # r_out_i starts right after t_i",
     "s_rout = e_h + 1"),
    ("next h starts after t, not after r_in (position ids)",
     "s_h = e_rin + 1            # h_{i+1} starts right after r_in_i",
     "s_h = e_t + 1"),
    ("r_out does not see t_i (visibility rule)",
     "_SAME_TURN_WHOLE = {H: (), T: (H,), RIN: (H,), ROUT: (H, T)}",
     "_SAME_TURN_WHOLE = {H: (), T: (H,), RIN: (H,), ROUT: (H,)}"),
    ("earlier reasoning visible to later turns (history set)",
     "_HISTORY_TYPES = (H, RIN)",
     "_HISTORY_TYPES = (H, RIN, T)"),
    ("causal inside a segment turned anti-causal",
     "M[rows, cols] = ki <= qi",
     "M[rows, cols] = ki >= qi"),
    ("RoPE rotation sign flipped",
     "return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)",
     "return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)"),
    ("backward without the Delta term",
     "                dS = P * (dP - delta)\n                dqr[:, h]",
     "                dS = P * dP\n                dqr[:, h]"),
    ("dQ not rotated back through RoPE",
     "            dq[b, a:e] = rope_transpose(dqr, pos, theta)",
     "            dq[b, a:e] = dqr"),
    ("GQA maps q head h to kv head h % Hkv (forward)",
     "            for h in range(Hq):\n                kv = h // g\n                S = scale * (qr[:, h] @ kr[:, kv].T)\n                S = np.where(M, S, -np.inf)\n                m = S.max",
     "            for h in range(Hq):\n                kv = h % Hkv\n                S = scale * (qr[:, h] @ kr[:, kv].T)\n                S = np.where(M, S, -np.inf)\n                m = S.max"),
    ("attn_cols: dV of listed keys from the transposed product",
     "                dV[sel, kv] += Pj.T @ dO",
     "                dV[sel, kv] += (dO.T @ Pj).T[:, ::-1]"),
    ("tile classification: a partly masked tile counted full",
     "np.where(counts == BQ * BK, FULL, PARTIAL)",
     "np.where(counts >= BQ * BK - 1, FULL, PARTIAL)"),
]

ORACLE_TESTS = ["tests/test_oracle_layout.py", "tests/test_oracle_attn.py", "tests/test_oracle_block.py"]


def _sandbox():
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    os.makedirs(os.path.join(d, "tests"))
    for f in os.listdir(os.path.join(ROOT, "tests")):
        if f.endswith(".py") and (f.startswith("test_oracle_") or f in ("conftest.py", "helpers.py")):
            shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(d, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"),
                    ignore=shutil.ignore_patterns("*.npz", "__pycache__"))
    pkg = os.path.join(d, "block_sparse_masked_opr_amd")
    os.makedirs(pkg)
    for f in ("__init__.py", "inputs.py"):
        shutil.copy(os.path.join(ROOT, "block_sparse_masked_opr_amd", f), os.path.join(pkg, f))
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    return d


def _run(d):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "-m", "not gpu", *ORACLE_TESTS], cwd=d, capture_output=True, text=True, env=env,
                          timeout=900)


def _mutated(mut):
    """Runs the oracle tests on a sandbox copy with one mutation (None: none)."""
    d = _sandbox()
    try:
        if mut is not None:
            name, old, new = mut
            path = os.path.join(d, "oracle", "opr_oracle.py")
            src = open(path).read()
            if src.count(old) != 1:
                return mut, None
            open(path, "w").write(src.replace(old, new))
        return mut, _run(d)
    finally:
        shutil.rmtree(d, ignore_errors=True)


def test_every_mutation_is_caught():
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
        results = list(ex.map(_mutated, [None] + MUTATIONS))
    (_, clean), rest = results[0], results[1:]
    assert clean.returncode == 0, "the unmutated copy fails:\n" + clean.stdout[-3000:]
    missed = []
    for (name, _old, _new), r in rest:
        if r is None:
            missed.append(f"{name}: mutation site not found exactly once")
            continue
        caught = [ln for ln in r.stdout.splitlines() if ln.startswith(("FAILED", "ERROR"))]
        print(f"{name}: caught by {caught[0] if caught else None}")
        if r.returncode == 0 or not caught:
            missed.append(name)
    assert not missed, missed
