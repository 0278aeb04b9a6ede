"""Turn lists of the N-pass and K-pass sequences of a conversation.

The pages compare the one pass against the N-pass formulation, in which turn
i of a conversation is trained by its own causal sequence over the human
messages and responses of the earlier turns and the whole of turn i (wiki
summary, sections "问题背景" and "理论保证"), and describe the K-pass
trade-off between the two (section "实验结果", K-Pass).  These functions write
those sequences as turn lists that opr_build_layout packs like any other
conversation, so the same kernels run all three.  (The oracle derives the same
sequences on its own: oracle.npass_index, oracle.kpass_chunk.)
"""
from __future__ import annotations

from typing import List

from . import inputs
from .inputs import Conversation, KPASS_ROW_LEN, Row


def npass_conversations(conv: Conversation) -> List[Conversation]:
    """The N separate sequences of the N-pass formulation, as turn lists.

    Pass i holds the human messages and responses of the earlier turns and the
    whole of turn i: [h_1, r_1, ..., h_{i-1}, r_{i-1}, h_i, t_i, r_i].  Earlier
    turns are written (h, 0, r, 0) (response as context, no reasoning) and turn i
    as (h, t, 0, r) (reasoning and the response generated after it).
    """
    out = []
    for i in range(len(conv)):
        hist = [(h, 0, r_in, 0) for (h, _t, r_in, _r) in conv[:i]]
        h, t, _r_in, r_out = conv[i]
        out.append(hist + [(h, t, 0, r_out)])
    return out


def chunk_conversation(conv: Conversation, a: int, b: int, elide_last_rin: bool = False) -> Conversation:
    """The sequence of a K-pass chunk that trains turns [a, b) of a conversation.

    The turns before a are history written (h, 0, r_in, 0); turns a .. b-1 keep
    every segment.  With elide_last_rin, turn b-1 loses its context copy r_in
    (written (h, t, 0, r_out)), which no token of the sequence sees.
    """
    if not 0 <= a < b <= len(conv):
        raise ValueError(f"chunk [{a}, {b}) of a {len(conv)}-turn conversation")
    hist = [(h, 0, r_in, 0) for (h, _t, r_in, _r) in conv[:a]]
    own = [tuple(x) for x in conv[a:b]]
    if elide_last_rin:
        h, t, _r_in, r_out = own[-1]
        own[-1] = (h, t, 0, r_out)
    return hist + own


def kpass_conversations(conv: Conversation, K: int, elide_last_rin: bool = False) -> List[Conversation]:
    """Split a conversation into K contiguous chunks of near-equal turn count.

    Chunk k holds turns [floor(kN/K), floor((k+1)N/K)) (see chunk_conversation).
    K is capped at N.
    """
    N = len(conv)
    K = max(1, min(K, N))
    return [chunk_conversation(conv, (k * N) // K, ((k + 1) * N) // K, elide_last_rin) for k in range(K)]


def kpass_rows(K, seed: int = 401, L: int = KPASS_ROW_LEN, elide_last_rin: bool = False) -> List[Row]:
    """Rows of L tokens for K in {1, 2, 4, ...} or K == 'N' (N-pass)."""
    convs = inputs.kpass_base_conversations(seed, L=L)
    chunks = []
    for c in convs:
        chunks.extend(npass_conversations(c) if K == "N" else kpass_conversations(c, int(K), elide_last_rin))
    return inputs.pack_first_fit_decreasing(chunks, L)
