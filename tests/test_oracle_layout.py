"""Pins for the oracle's layout, mask and tile schedule (CPU only).

Each check ties the oracle to something outside itself: the hand-derived worked
example under tests/golden/, the position-set invariant that the N-pass
equivalence implies, brute-force tile counting, and special cases that reduce to
the textbook causal mask.
"""
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from block_sparse_masked_opr_amd import inputs as I
from oracle import opr_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_layout.txt")


def _golden():
    out = {}
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val = line.split(":", 1)
        out[key.strip()] = val.strip()
    return out


def _ints(s):
    return np.array([int(x) for x in s.split()], dtype=np.int64)


def test_tiny_golden_layout():
    g = _golden()
    lay = O.layout(I.tiny_rows(), int(g["L"]))
    np.testing.assert_array_equal(lay["type"][0], _ints(g["type"]))
    np.testing.assert_array_equal(lay["pos"][0], _ints(g["pos"]))
    np.testing.assert_array_equal(lay["turn"][0], _ints(g["turn"]))
    assert (lay["conv"][0] == 0).all()


def test_tiny_golden_pairs_and_tiles():
    g = _golden()
    lay = O.layout(I.tiny_rows(), 64)
    assert O.dense_mask(lay, 0).sum() == int(g["pairs"])
    s = O.schedule(lay, 0, 32, 32)
    np.testing.assert_array_equal(s["counts"].ravel(), _ints(g["tile32_counts"]))
    np.testing.assert_array_equal(s["tile_class"].ravel(), _ints(g["tile32_class"]))
    npairs = 0
    for p in O.npass_index(lay, 0, 0):
        n = len(p["idx"])
        npairs += n * (n + 1) // 2
    assert npairs == int(g["npass_pairs"])


# ---------------------------------------------------------------------------
# random layouts, with zero-length segments
# ---------------------------------------------------------------------------
seg = st.integers(0, 6)
turn_st = st.tuples(seg, seg, seg, seg)
conv_st = st.lists(turn_st, min_size=1, max_size=4)
row_st = st.lists(conv_st, min_size=1, max_size=3)


def _L_for(rows, extra):
    used = max(I.row_used(r) for r in rows)
    return max(1, used + extra)


@settings(max_examples=150, deadline=None)
@given(rows=st.lists(row_st, min_size=1, max_size=2), extra=st.integers(0, 9))
def test_position_set_invariant(rows, extra):
    """Each non-PAD query sees keys whose positions are exactly {0, ..., pos_q}:
    the one pass reproduces the position ids of the ordinary causal sequence
    of its N-pass pass (wiki summary, "位置 ID 策略" and "理论保证")."""
    L = _L_for(rows, extra)
    lay = O.layout(rows, L)
    for b in range(len(rows)):
        M = O.dense_mask(lay, b)
        pos = lay["pos"][b]
        typ = lay["type"][b]
        for q in range(L):
            ks = np.nonzero(M[q])[0]
            if typ[q] == O.PAD:
                assert len(ks) == 0
                assert not M[:, q].any()
                continue
            np.testing.assert_array_equal(np.sort(pos[ks]), np.arange(pos[q] + 1))
            # visible keys are earlier in the packed order and in the same conversation
            assert (ks <= q).all()
            assert (lay["conv"][b][ks] == lay["conv"][b][q]).all()


def _check_schedule(M, s, L, bq, bk):
    """Tile and 32x32 sub-block classes and lists of schedule s against direct
    pair counting in the dense mask M (rows queries, columns keys)."""
    MT, NT = -(-L // bq), -(-L // bk)
    for m in range(MT):
        lst = []
        for n in range(NT):
            cnt = int(M[m * bq:(m + 1) * bq, n * bk:(n + 1) * bk].sum())
            want = 0 if cnt == 0 else (2 if cnt == bq * bk else 1)
            assert s["tile_class"][m, n] == want
            if cnt:
                lst.append(n)
            if bq % 32 == 0 and bk % 32 == 0:
                word = int(s["sub_class"][m, n])
                for i in range(bq // 32):
                    for j in range(bk // 32):
                        q0, k0 = m * bq + 32 * i, n * bk + 32 * j
                        c = int(M[q0:q0 + 32, k0:k0 + 32].sum())
                        w = 0 if c == 0 else (2 if c == 1024 else 1)
                        assert (word >> (2 * (i * (bk // 32) + j))) & 3 == w
        assert s["q_nnz"][m] == len(lst)
        assert list(s["q_list"][m, :len(lst)]) == lst
        assert (s["q_list"][m, len(lst):] == -1).all()
    for n in range(NT):
        lst = [m for m in range(MT) if s["tile_class"][m, n] != 0]
        assert s["k_nnz"][n] == len(lst)
        assert list(s["k_list"][n, :len(lst)]) == lst
        assert (s["k_list"][n, len(lst):] == -1).all()


@settings(max_examples=100, deadline=None)
@given(rows=st.lists(row_st, min_size=1, max_size=2), extra=st.integers(0, 40),
       bq=st.sampled_from([16, 32, 64]), bk=st.sampled_from([16, 32, 64]))
def test_schedule_brute_force(rows, extra, bq, bk):
    """Tile and 32x32 sub-block classes and lists against direct pair counting."""
    L = _L_for(rows, extra)
    lay = O.layout(rows, L)
    for b in range(len(rows)):
        _check_schedule(O.dense_mask(lay, b), O.schedule(lay, b, bq, bk), L, bq, bk)


@settings(max_examples=60, deadline=None)
@given(rows=st.lists(row_st, min_size=1, max_size=2), extra=st.integers(0, 9),
       bq=st.sampled_from([1, 2, 4, 8]), bk=st.sampled_from([1, 2, 4, 8]))
def test_schedule_brute_force_small_tiles(rows, extra, bq, bk):
    """The class rule at tile sizes where tiles one pair short of full (a 2 x 2
    tile on a causal diagonal holds 3 of 4 pairs) and one pair from empty are
    common: FULL only with every pair allowed, EMPTY only with none."""
    L = _L_for(rows, extra)
    lay = O.layout(rows, L)
    for b in range(len(rows)):
        _check_schedule(O.dense_mask(lay, b), O.schedule(lay, b, bq, bk), L, bq, bk)


# ---------------------------------------------------------------------------
# attention order (a reordering of this library; the mask itself is unchanged)
# ---------------------------------------------------------------------------
def _permuted_mask(lay, b):
    """Dense mask of row b with queries and keys at their attention-order slots."""
    M = O.dense_mask(lay, b)
    slot = O.attention_order(lay, b)
    P = np.zeros_like(M)
    P[np.ix_(slot, slot)] = M
    return P


def test_tiny_golden_attention_order():
    g = _golden()
    lay = O.layout(I.tiny_rows(), 64)
    np.testing.assert_array_equal(O.attention_order(lay, 0), _ints(g["slot"]))
    s = O.schedule(lay, 0, 32, 32, order="attention")
    np.testing.assert_array_equal(s["counts"].ravel(), _ints(g["slot_tile32_counts"]))
    np.testing.assert_array_equal(s["tile_class"].ravel(), _ints(g["slot_tile32_class"]))


@settings(max_examples=150, deadline=None)
@given(rows=st.lists(row_st, min_size=1, max_size=2), extra=st.integers(0, 9))
def test_attention_order_closed_form(rows, extra):
    """A permutation inside each conversation: h and r_in tokens sit at
    conversation start + position id (their positions run 0, 1, ... without
    gaps), t and r_out follow in packed order, PAD keeps its index."""
    L = _L_for(rows, extra)
    lay = O.layout(rows, L)
    for b in range(len(rows)):
        slot = O.attention_order(lay, b)
        assert sorted(slot.tolist()) == list(range(L))
        typ, pos = lay["type"][b], lay["pos"][b]
        for c in range(O.n_convs(lay, b)):
            a, e = O.conv_range(lay, b, c)
            ty = typ[a:e]
            hist = np.nonzero((ty == O.H) | (ty == O.RIN))[0] + a
            rest = np.nonzero((ty == O.T) | (ty == O.ROUT))[0] + a
            np.testing.assert_array_equal(slot[hist], a + pos[hist])
            np.testing.assert_array_equal(slot[rest], a + len(hist) + np.arange(len(rest)))
        pad = np.nonzero(typ == O.PAD)[0]
        np.testing.assert_array_equal(slot[pad], pad)


@settings(max_examples=150, deadline=None)
@given(rows=st.lists(row_st, min_size=1, max_size=2), extra=st.integers(0, 9))
def test_slot_intervals_reproduce_mask(rows, extra):
    """In attention order every query row and every key column of the mask is
    at most two runs (no ValueError), the runs rebuild the mask exactly, and
    no query sees a key at a later slot."""
    L = _L_for(rows, extra)
    lay = O.layout(rows, L)
    for b in range(len(rows)):
        P = _permuted_mask(lay, b)
        qiv, kiv = O.slot_intervals(lay, b, row_chunk=5)
        R = np.zeros_like(P)
        C = np.zeros_like(P)
        for s_ in range(L):
            x0, x1, x2, x3 = qiv[s_]
            assert x0 <= x1 <= x2 <= x3
            R[s_, x0:x1] = True
            R[s_, x2:x3] = True
            y0, y1, y2, y3 = kiv[s_]
            assert y0 <= y1 <= y2 <= y3
            C[y0:y1, s_] = True
            C[y2:y3, s_] = True
        np.testing.assert_array_equal(R, P)
        np.testing.assert_array_equal(C, P)
        assert not np.triu(P, 1).any()


@settings(max_examples=80, deadline=None)
@given(rows=st.lists(row_st, min_size=1, max_size=2), extra=st.integers(0, 40),
       bq=st.sampled_from([16, 32, 64]), bk=st.sampled_from([16, 32, 64]))
def test_schedule_brute_force_attention_order(rows, extra, bq, bk):
    L = _L_for(rows, extra)
    lay = O.layout(rows, L)
    for b in range(len(rows)):
        _check_schedule(_permuted_mask(lay, b), O.schedule(lay, b, bq, bk, order="attention"), L, bq, bk)


def test_single_turn_is_textbook_causal():
    """One turn with no reasoning and no response is an ordinary causal sequence."""
    lay = O.layout([[[(37, 0, 0, 0)]]], 37)
    M = O.dense_mask(lay, 0)
    np.testing.assert_array_equal(M, np.tril(np.ones((37, 37), dtype=bool)))
    np.testing.assert_array_equal(lay["pos"][0], np.arange(37))


def test_rules_by_segment_tiny():
    """The four visibility rules on the worked example, segment by segment."""
    lay = O.layout(I.tiny_rows(), 64)
    M = O.dense_mask(lay, 0)
    h1, t1, i1, o1 = range(0, 8), range(8, 20), range(20, 26), range(26, 32)
    h2, t2, i2, o2 = range(32, 40), range(40, 52), range(52, 58), range(58, 64)

    def sees(q, ks):
        return all(M[q, k] for k in ks)

    def blind(q, ks):
        return not any(M[q, k] for k in ks)

    # h_2 sees H_<2 = h_1 and r_in_1, not t_1 or r_out_1
    assert sees(32, h1) and sees(32, i1) and blind(32, t1) and blind(32, o1)
    # t_2 additionally sees h_2
    assert sees(45, h2) and sees(45, h1) and sees(45, i1) and blind(45, o1)
    # r_in_2 sees h_2 but not t_2
    assert sees(55, h2) and blind(55, t2)
    # r_out_2 sees h_2 and t_2 but not r_in_2
    assert sees(60, h2) and sees(60, t2) and blind(60, i2)
    # r_out_1 sees t_1, r_in_1 does not
    assert sees(30, t1) and blind(22, t1)
    # nobody sees a later token
    assert not np.triu(M, 1).any()


@settings(max_examples=60, deadline=None)
@given(conv=st.lists(st.tuples(st.integers(1, 5), st.integers(0, 5), st.integers(0, 5)),
                     min_size=1, max_size=4))
def test_npass_sequence_positions(conv):
    """Pass i of the N-pass gathered from the packed row sits at positions 0..n-1."""
    turns = [(h, t, r, r) for (h, t, r) in conv]
    L = I.conv_len(turns)
    lay = O.layout([[turns]], L)
    for p in O.npass_index(lay, 0, 0):
        np.testing.assert_array_equal(lay["pos"][0][p["idx"]], np.arange(len(p["idx"])))


def test_useful_pairs_closed_form():
    """P = sum over non-PAD tokens of (pos + 1) (each query sees positions 0..pos)."""
    rows = I.packed_rows(I.Shape("s", 1, 2048, 1, 1, 64), 7)
    lay = O.layout(rows, 2048)
    nonpad = lay["type"] != O.PAD
    assert O.useful_pairs(lay) == int((lay["pos"][nonpad] + 1).sum())
