"""The checked build (libopr_debug.so, -DOPR_DEBUG) on the GPU: on the tiny
worked example, the whole 2 x 16384 packed fwd+bwd workload and the depth
N = 8 conversation (whose history columns run cut into parts), its kernels
report no violated invariant (opr_debug_errors() == 0) and give bit-identical
O, LSE, dQ, dK and dV to the release library.  The checked library runs in a
child process (a process loads one of the two builds)."""
from __future__ import annotations

import hashlib
import json
import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
THETA = 1.0e6


def _cases():
    from block_sparse_masked_opr_amd import inputs as I
    s = I.PACKED_FWD_BWD
    depth = I.depth_conversation(8)
    return [
        ("tiny", I.tiny_rows(), 64, (1, 1, 64), 0),
        ("packed_fwd_bwd", I.packed_rows(s, I.SEEDS["packed_fwd_bwd"][0]), s.L, (s.Hq, s.Hkv, s.D),
         I.SEEDS["packed_fwd_bwd"][1]),
        ("depth8", [[depth]], I.conv_len(depth), (I.DEPTH_HEADS["Hq"], I.DEPTH_HEADS["Hkv"], I.DEPTH_HEADS["D"]),
         I.SEEDS["depth"][1]),
    ]


def _digests() -> dict:
    """Layout + forward + backward of every case with the library this
    process loaded: sha256 of each output's bytes, and the error bits."""
    from block_sparse_masked_opr_amd import binding as Bd
    from block_sparse_masked_opr_amd import inputs as I
    from tests.helpers import to_device_bf16
    dev = torch.device("cuda:0")
    out = {}
    for name, rows, L, (Hq, Hkv, D), seed in _cases():
        t = I.make_tensors(len(rows), L, Hq, Hkv, D, seed=seed)
        lay = Bd.opr_build_layout(rows, L, 128, 128, device=dev)
        q, k, v, do = (to_device_bf16(t[n], dev) for n in ("q", "k", "v", "do"))
        o, lse = Bd.opr_attn_fwd(q, k, v, lay, THETA)
        dq, dk, dv = Bd.opr_attn_bwd(q, k, v, o, lse, do, lay, THETA)
        torch.cuda.synchronize()
        res = {n: hashlib.sha256(x.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()
               for n, x in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
        res["errors"] = Bd.opr_debug_errors()
        out[name] = res
        print(f"[debug build] {name}: errors {res['errors']}", file=sys.stderr, flush=True)
    return out


def test_checked_build_matches_release():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = os.path.join(ROOT, "block_sparse_masked_opr_amd", "libopr_debug.so")
    if not os.path.exists(lib):
        pytest.fail("libopr_debug.so is not built (build(debug=True))")
    env = dict(os.environ, OPR_LIB="debug")
    code = ("import json, sys; sys.path.insert(0, %r); import tests.test_gpu_debug_build as t; "
            "print(json.dumps(t._digests()))" % ROOT)
    child = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True,
                           timeout=240)
    sys.stderr.write(child.stderr[-2000:])
    assert child.returncode == 0, child.stderr[-2000:]
    checked = json.loads(child.stdout.strip().splitlines()[-1])
    release = _digests()
    for name, res in checked.items():
        assert res["errors"] == 0, (name, res["errors"])
        assert release[name]["errors"] is None  # the release build tests nothing
        for n in ("o", "lse", "dq", "dk", "dv"):
            assert res[n] == release[name][n], (name, n)
