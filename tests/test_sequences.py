"""The product's N-pass and K-pass turn lists (block_sparse_masked_opr_amd/
sequences.py, which the GPU tests and the benchmark run through the kernels)
against the oracle's own derivation of the same sequences from the pages
(oracle.npass_index, oracle.kpass_chunk) and against the rules themselves."""
import numpy as np
from hypothesis import example, given, settings, strategies as st

from block_sparse_masked_opr_amd import inputs as I
from block_sparse_masked_opr_amd import sequences as S
from oracle import opr_oracle as O

turn = st.tuples(st.integers(0, 6), st.integers(0, 6), st.integers(0, 6))


@settings(max_examples=40, deadline=None)
@given(conv=st.lists(turn, min_size=1, max_size=5))
@example(conv=[(0, 0, 1), (0, 0, 0)])  # a trailing empty turn: its pass is the history alone
def test_npass_sequences_match_oracle_passes(conv):
    """Pass i as the product writes it has, token by token, the roles of the
    oracle's pass i gathered from the one-pass row (history h / r_in, then
    h_i, t_i, r_out_i), positions 0..n-1 and a plain causal mask."""
    conv = [(h, t, r, r) for (h, t, r) in conv]
    full = O.layout([[conv]], max(1, I.conv_len(conv)))
    passes = O.npass_index(full, 0, 0, len(conv)) if I.conv_len(conv) else []
    seqs = S.npass_conversations(conv)
    assert len(seqs) == len(conv)
    for i, seq in enumerate(seqs):
        n = I.conv_len(seq)
        if n == 0:
            continue
        lay = O.layout([[seq]], n)
        np.testing.assert_array_equal(lay["type"][0], passes[i]["role"])
        np.testing.assert_array_equal(lay["pos"][0], np.arange(n))
        np.testing.assert_array_equal(O.dense_mask(lay, 0), np.tril(np.ones((n, n), dtype=bool)))


@settings(max_examples=40, deadline=None)
@given(conv=st.lists(turn, min_size=1, max_size=6), elide=st.booleans(), data=st.data())
def test_chunk_turn_lists_match_oracle(conv, elide, data):
    conv = [(h, t, r, r) for (h, t, r) in conv]
    a = data.draw(st.integers(0, len(conv) - 1))
    b = data.draw(st.integers(a + 1, len(conv)))
    assert [tuple(x) for x in S.chunk_conversation(conv, a, b, elide)] == O.kpass_chunk(conv, a, b, elide)


def test_equal_split_bounds():
    """K equal chunks take turns [floor(kN/K), floor((k+1)N/K)); K is capped at N."""
    conv = [(1, 2, 3, 3)] * 7
    for K in (1, 2, 3, 4, 7, 9):
        chunks = S.kpass_conversations(conv, K)
        Ke = min(K, 7)
        assert len(chunks) == Ke
        for k, ch in enumerate(chunks):
            a, b = (k * 7) // Ke, ((k + 1) * 7) // Ke
            assert [tuple(x) for x in ch] == O.kpass_chunk(conv, a, b, False)


def test_kpass_rows_hold_every_chunk_once():
    """The K-pass rows pack each conversation's K chunks exactly once, within L."""
    convs = I.kpass_base_conversations(I.SEEDS["kpass"][0])
    for K in (1, 2, 4):
        rows = S.kpass_rows(K)
        want = sorted(tuple(map(tuple, ch)) for c in convs for ch in S.kpass_conversations(c, K))
        got = sorted(tuple(map(tuple, c)) for r in rows for c in r)
        assert got == want
        assert all(I.row_used(r) <= I.KPASS_ROW_LEN for r in rows)
