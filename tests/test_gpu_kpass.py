"""K-pass chunk rows on the GPU (opr_kpass_plan -> opr_build_layout -> attention).

* Rows of planned chunks, with the context copy of each chunk's last turn left
  out, through forward and backward against the fp64 oracle.
* The chunk form of Theorem 2.1 (wiki summary, "理论保证") on the kernels: the
  chunk sequences, gathered from the one-pass row's inputs, reproduce the
  one-pass outputs, and their gradients with dO on the scored rows, summed,
  reproduce the one-pass gradients.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from block_sparse_masked_opr_amd import inputs as I  # noqa: E402
from block_sparse_masked_opr_amd import sequences as S  # noqa: E402
from oracle import opr_oracle as O  # noqa: E402
from tests.helpers import assert_close  # noqa: E402
from tests.test_gpu_attn import compare_full, run_gpu  # noqa: E402


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_masked_opr_amd import binding
    return binding


def test_planned_chunk_rows(B):
    rng = np.random.default_rng(4242)
    convs = [[(int(rng.integers(8, 90)), int(rng.integers(0, 200)), *([int(rng.integers(4, 80))] * 2))
              for _ in range(int(rng.integers(2, 6)))] for _ in range(5)]
    chunks = []
    for c in convs:
        cap = max(I.conv_len(c) // 2, max(O.kpass_chunk_size(c, j, j + 1, True)[0] for j in range(len(c))))
        plan, _ = B.opr_kpass_plan(c, max_tokens=cap, tokens_weight=40.0, elide_last_rin=True)
        print(f"[kpass] {len(c)} turns, cap {cap}: chunks {[(p['first_turn'], p['n_turns']) for p in plan]}",
              flush=True)
        for p in plan:
            chunks.append(S.chunk_conversation(c, p["first_turn"], p["first_turn"] + p["n_turns"], True))
    L = max(I.conv_len(x) for x in chunks) + 70
    rows = I.pack_first_fit_decreasing(chunks, L)
    t = I.make_tensors(len(rows), L, 4, 2, 128, seed=4343)
    compare_full(f"planned chunks, {len(rows)} rows of {L}", rows, L, t, run_gpu(B, rows, L, t))


def _own_index(lay_c, lay_1):
    idx = np.empty(lay_c["type"].shape[1], dtype=np.int64)
    for j in np.unique(lay_c["turn"][0]):
        for y in range(4):
            src = np.nonzero((lay_c["turn"][0] == j) & (lay_c["type"][0] == y))[0]
            dst = np.nonzero((lay_1["turn"][0] == j) & (lay_1["type"][0] == y))[0]
            idx[src] = dst[:len(src)]
    return idx


def test_chunks_reproduce_onepass(B):
    conv = [(60, 150, 70, 70), (30, 0, 90, 90), (45, 120, 40, 40), (25, 200, 64, 64)]
    n1 = I.conv_len(conv)
    lay1 = O.layout([[conv]], n1)
    t = I.make_tensors(1, n1, 4, 2, 128, seed=5252)
    scored = (lay1["type"][0] == O.T) | (lay1["type"][0] == O.ROUT)
    t["do"][0, ~scored] = 0
    g1 = run_gpu(B, [[conv]], n1, t)
    plan, _ = B.opr_kpass_plan(conv, n_chunks=3, elide_last_rin=True)
    acc = {n: np.zeros_like(g1[n]) for n in ("dq", "dk", "dv")}
    for p in plan:
        a, b = p["first_turn"], p["first_turn"] + p["n_turns"]
        seq = S.chunk_conversation(conv, a, b, True)
        n = I.conv_len(seq)
        assert n == p["tokens"]
        layc = O.layout([[seq]], n)
        idx = _own_index(layc, lay1)
        tc = {k: np.ascontiguousarray(v[:, idx]) for k, v in t.items()}
        own = (layc["turn"][0] >= a) & ((layc["type"][0] == O.T) | (layc["type"][0] == O.ROUT))
        tc["do"][0, ~own] = 0
        gc = run_gpu(B, [[seq]], n, tc)
        print(f"[kpass] chunk [{a}, {b}) of {n} tokens vs the one-pass row", flush=True)
        assert_close("O", gc["o"][0], g1["o"][0, idx], max_abs=1e-2, mean_rel=2e-3)
        assert_close("LSE", gc["lse"][0], g1["lse"][0][:, idx], max_abs=1e-3, mean_rel=1e-5)
        for k in acc:
            np.add.at(acc[k][0], idx, gc[k][0])
    for k in acc:
        assert_close(f"sum of chunk {k}", acc[k], g1[k])
