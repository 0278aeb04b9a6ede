"""K-pass chunks and the chunk planner (CPU).

* The planner (opr_kpass_plan, host C++ in libopr) against the oracle's brute
  force over every split, whose chunk sizes are counted from the set-membership
  mask (wiki summary, "实验结果": K-Pass).
* The K-pass chunk construction and the context-copy elision against the
  one-pass definition, in fp64: every token of a chunk sequence gets exactly
  its one-pass output, and the chunks' gradients, summed, are the one-pass
  gradients (wiki summary, "理论保证", Theorem 2.1, carried to chunks).
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from block_sparse_masked_opr_amd import inputs as I
from oracle import opr_oracle as O

THETA = 1.0e6


@pytest.fixture(scope="module")
def Bd():
    from block_sparse_masked_opr_amd import binding
    return binding


def _random_conv(rng, N, lim):
    return [tuple(int(x) for x in (rng.integers(0, lim), rng.integers(0, lim), *([rng.integers(0, lim)] * 2)))
            for _ in range(N)]


def test_worked_example(Bd):
    """(h, t, r) = (8, 12, 6) x 2: the one-pass sequence has 64 tokens and 1288
    pairs (every token sees position id + 1 keys); one chunk per turn with the
    context copy of each chunk's last turn left out is exactly the N-pass
    formulation: sequences of 26 and 40 tokens, 351 + 820 = 1171 pairs."""
    conv = I.tiny_rows()[0][0]
    ch, cost = Bd.opr_kpass_plan(conv, n_chunks=1, elide_last_rin=False)
    assert [(c["tokens"], c["pairs"]) for c in ch] == [(64, 1288)] and cost == 1288
    ch, cost = Bd.opr_kpass_plan(conv, n_chunks=2, elide_last_rin=True)
    assert [(c["tokens"], c["pairs"]) for c in ch] == [(26, 351), (40, 820)] and cost == 1171
    # the one-pass sequence without its dead context copy is the cheapest plan
    ch, cost = Bd.opr_kpass_plan(conv, elide_last_rin=True)
    assert [(c["first_turn"], c["n_turns"], c["tokens"], c["pairs"]) for c in ch] == [(0, 2, 58, 1135)]


def test_chunk_per_turn_is_npass():
    """Oracle pin: one chunk per turn with elision gives the N-pass sequences
    (the oracle's own N-pass gather from the one-pass row)."""
    rng = np.random.default_rng(7)
    for _ in range(5):
        conv = _random_conv(rng, int(rng.integers(1, 6)), 20)
        n1 = I.conv_len(conv)
        if n1 == 0:
            continue
        passes = O.npass_index(O.layout([[conv]], n1), 0, 0)
        for i in range(len(conv)):
            tok, _ = O.kpass_chunk_size(conv, i, i + 1, True)
            assert tok == len(passes[i]["idx"])


@pytest.mark.parametrize("seed", range(6))
def test_plan_matches_bruteforce(Bd, seed):
    """Least cost, number of chunks (ties to fewer) and every chunk's size
    against the oracle's exhaustive search."""
    rng = np.random.default_rng(100 + seed)
    for case in range(8):
        N = int(rng.integers(1, 10))
        conv = _random_conv(rng, N, 14 if case % 2 else 40)
        elide = bool(case % 3 != 2)
        weight = [0.0, 1.0, 2.5, 37.0][case % 4]
        n_chunks = int(rng.integers(0, N + 1))
        full = I.conv_len(conv)
        cap = [0, full, max(1, full // 2), max(1, full // 3)][case % 4]
        best, arg = O.kpass_best_splits(conv, n_chunks, cap, weight, elide)
        if best == math.inf:
            with pytest.raises(Bd.OprError) as e:
                Bd.opr_kpass_plan(conv, n_chunks, cap, weight, elide)
            assert e.value.status == Bd.OPR_E_CAPACITY
            continue
        ch, cost = Bd.opr_kpass_plan(conv, n_chunks, cap, weight, elide)
        assert cost == best, (conv, n_chunks, cap, weight, elide)
        starts = [c["first_turn"] for c in ch]
        assert starts in arg
        assert len(ch) == min(len(s) for s in arg)
        assert sum(c["n_turns"] for c in ch) == N
        for c in ch:
            a, b = c["first_turn"], c["first_turn"] + c["n_turns"]
            assert (c["tokens"], c["pairs"]) == O.kpass_chunk_size(conv, a, b, elide)
            assert c["rin_elided"] == int(elide)
            assert cap == 0 or c["tokens"] <= cap


def test_plan_errors(Bd):
    conv = [(4, 5, 6, 6), (3, 2, 1, 1)]
    for args in ([], {"n_chunks": 3}, {"n_chunks": -1}, {"max_tokens": -1}, {"tokens_weight": -1.0},
                 {"tokens_weight": float("nan")}, {"tokens_weight": float("inf")}):
        c = conv if isinstance(args, dict) else args
        kw = args if isinstance(args, dict) else {}
        with pytest.raises(Bd.OprError) as e:
            Bd.opr_kpass_plan(c, **kw)
        assert e.value.status == Bd.OPR_E_INVALID
    with pytest.raises(Bd.OprError) as e:
        Bd.opr_kpass_plan([(4, -1, 6, 6)])
    assert e.value.status == Bd.OPR_E_INVALID
    # the second turn's own sequence needs 3 + 2 + 1 + (4 + 6) history = 16 tokens
    with pytest.raises(Bd.OprError) as e:
        Bd.opr_kpass_plan(conv, max_tokens=15)
    assert e.value.status == Bd.OPR_E_CAPACITY
    ch, _ = Bd.opr_kpass_plan(conv, max_tokens=16)
    assert [c["tokens"] for c in ch] == [15, 16]


def test_plan_long_conversation_and_limits(Bd):
    """Any number of chunks runs in O(N^2) time and O(N) memory: a 3000-turn
    conversation plans quickly, every chunk within the cap and the chunks
    covering the turns in order.  Requests past the documented limits are
    refused (OPR_E_UNSUPPORTED), never an exception or an allocation failure
    escaping the C ABI."""
    import time
    rng = np.random.default_rng(5)
    # short messages and responses, long reasoning: the history stays small
    conv = [(int(rng.integers(0, 4)), int(rng.integers(0, 60)), *([int(rng.integers(0, 4))] * 2)) for _ in range(3000)]
    cap = I.conv_len(conv) // 3
    t0 = time.time()
    ch, cost = Bd.opr_kpass_plan(conv, max_tokens=cap, elide_last_rin=True)
    assert time.time() - t0 < 20.0
    assert len(ch) > 1 and ch[0]["first_turn"] == 0 and sum(c["n_turns"] for c in ch) == 3000
    assert all(c["tokens"] <= cap for c in ch)
    assert all(ch[i]["first_turn"] + ch[i]["n_turns"] == ch[i + 1]["first_turn"] for i in range(len(ch) - 1))
    assert cost == sum(c["pairs"] for c in ch)          # tokens_weight 0: the cost is the pairs
    with pytest.raises(Bd.OprError) as e:
        Bd.opr_kpass_plan(conv, n_chunks=2000)           # 2000 * 3000^2 > 2^33
    assert e.value.status == Bd.OPR_E_UNSUPPORTED
    with pytest.raises(Bd.OprError) as e:
        Bd.opr_kpass_plan([(1, 1, 1, 1)] * 65537)
    assert e.value.status == Bd.OPR_E_UNSUPPORTED


def _own_index(lay_c, lay_1):
    """For each token of a chunk sequence, the one-pass token with the same
    (turn, type, offset in its segment)."""
    idx = np.empty(lay_c["type"].shape[1], dtype=np.int64)
    for j in np.unique(lay_c["turn"][0]):
        for y in range(4):
            src = np.nonzero((lay_c["turn"][0] == j) & (lay_c["type"][0] == y))[0]
            dst = np.nonzero((lay_1["turn"][0] == j) & (lay_1["type"][0] == y))[0]
            idx[src] = dst[:len(src)]
    return idx


@pytest.mark.parametrize("elide", [False, True])
def test_chunks_reproduce_onepass(elide):
    """Every token of every chunk sequence gets its one-pass output, and with
    dO on the scored rows (t and r_out) only, the chunks' dq, dk, dv summed
    onto the one-pass tokens are the one-pass gradients."""
    conv = [(9, 14, 7, 7), (5, 0, 11, 11), (12, 8, 3, 3), (4, 17, 6, 6)]
    n1 = I.conv_len(conv)
    lay1 = O.layout([[conv]], n1)
    rng = np.random.default_rng(11)
    Hq, Hkv, D = 4, 2, 16
    q = rng.standard_normal((1, n1, Hq, D))
    k = rng.standard_normal((1, n1, Hkv, D))
    v = rng.standard_normal((1, n1, Hkv, D))
    do = rng.standard_normal((1, n1, Hq, D))
    scored = (lay1["type"][0] == O.T) | (lay1["type"][0] == O.ROUT)
    do[0, ~scored] = 0.0
    o1, lse1 = O.attn_fwd(q, k, v, lay1, THETA)
    g1 = O.attn_bwd(q, k, v, do, lay1, THETA)
    for starts in ([0, 2], [0, 1, 3], [0, 1, 2, 3]):
        acc = [np.zeros_like(x) for x in g1]
        for a, b in zip(starts, starts[1:] + [len(conv)]):
            seq = O.kpass_chunk(conv, a, b, elide)
            n = sum(sum(x) for x in seq)
            layc = O.layout([[seq]], n)
            idx = _own_index(layc, lay1)
            qc, kc, vc = q[:, idx], k[:, idx], v[:, idx]
            own = (layc["turn"][0] >= a) & ((layc["type"][0] == O.T) | (layc["type"][0] == O.ROUT))
            doc = do[:, idx].copy()
            doc[0, ~own] = 0.0
            oc, lsec = O.attn_fwd(qc, kc, vc, layc, THETA)
            np.testing.assert_allclose(oc[0], o1[0, idx], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lsec[0], lse1[0][:, idx], rtol=0, atol=1e-12)
            for s, gc in zip(acc, O.attn_bwd(qc, kc, vc, doc, layc, THETA)):
                np.add.at(s[0], idx, gc[0])
        for name, s, ref in zip(("dq", "dk", "dv"), acc, g1):
            np.testing.assert_allclose(s, ref, rtol=0, atol=1e-11, err_msg=f"{name} starts={starts}")
