"""fp64 CPU oracle for one-pass block-sparse masked attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The library's product path never
calls it; it shares no code, table or helper with the HIP kernels.

What it computes follows the pages on One-Pass to Reason (Goru, Mehta, Jain,
arXiv 2504.18246):

* wiki summary "One-Pass to Reason: 多轮推理的高效单遍微调", sections
  "Token 复制" (token duplication), "分块稀疏注意力掩码" (block-sparse attention
  mask: the four visibility rules), "位置 ID 策略" (strategic position ids),
  "理论保证" (Theorem 2.1, one pass equals N passes) and "实现细节"
  (implementation notes: packing with the custom mask);
* raw note "One-Pass to Reason: Token Duplication and Block-Sparse Mask ...",
  sections "Core Problem" and "Method".

Plain definition used here: every token attends, with ordinary softmax
attention, to exactly the keys that the four rules allow, and RoPE is applied
at the strategic position ids.  The mask is built by set membership from the
rules (never from a simplified predicate); the N-pass brute force runs the N
separate causal sequences with positions 0..n-1.  Everything is float64 numpy.

Readings where the pages are silent (each listed in the design notes):
segment order within a turn is h, t, r_in, r_out; H_<i is the human messages
and context response copies of earlier turns of the same conversation; each
segment is causal inside itself; each packed conversation starts at position 0
and never sees another; an empty segment x "ends" at s_x + 0 - 1, so the next
start is s_x + len_x; PAD rows see nothing (O = 0, LSE = -inf, zero gradients);
RoPE is the rotate-half form with inv_freq_j = theta^(-2j/D); the softmax scale
is 1/sqrt(D); q head h reads kv head h // (Hq/Hkv).

Parity status: every function here is pinned by the CPU tests (hand-derived
worked example, invariants, library attention, finite differences and the
N-pass brute force); the tile schedule is pinned by brute-force counting.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

# token types
H, T, RIN, ROUT, PAD = 0, 1, 2, 3, 4
TYPE_NAMES = {H: "h", T: "t", RIN: "r_in", ROUT: "r_out", PAD: "pad"}


# ----------------------------------------------------------------------------
# layout: tokens and strategic position ids
# ----------------------------------------------------------------------------
def layout(rows: Sequence, L: int) -> Dict[str, np.ndarray]:
    """Per-token conversation, turn, type and position id for packed rows.

    Token duplication (wiki summary, "Token 复制"): each turn contributes the
    human message h_i, the reasoning t_i, the context copy r_in_i and the
    generation copy r_out_i, in that order; conversations follow each other in
    a row (packing, "实现细节"), the rest of the row is PAD.

    Position ids (wiki summary, "位置 ID 策略"):
      t_i and r_in_i both start right after h_i ends;
      r_out_i starts right after t_i ends;
      h_{i+1} starts right after r_in_i ends;
    the first human message of each conversation starts at 0.
    """
    B = len(rows)
    conv = np.full((B, L), -1, dtype=np.int64)
    turn = np.full((B, L), -1, dtype=np.int64)
    typ = np.full((B, L), PAD, dtype=np.int64)
    pos = np.zeros((B, L), dtype=np.int64)
    for b, convs in enumerate(rows):
        idx = 0
        for c, turns in enumerate(convs):
            s_h = 0
            for i, (h, t, r_in, r_out) in enumerate(turns):
                e_h = s_h + h - 1          # last position of h_i
                s_t = e_h + 1              # t_i starts right after h_i
                s_rin = e_h + 1            # so does r_in_i
                e_t = s_t + t - 1
                s_rout = e_t + 1           # r_out_i starts right after t_i
                e_rin = s_rin + r_in - 1
                for y, n, s in ((H, h, s_h), (T, t, s_t), (RIN, r_in, s_rin), (ROUT, r_out, s_rout)):
                    if idx + n > L:
                        raise ValueError(f"row {b}: conversations exceed L={L}")
                    sl = slice(idx, idx + n)
                    conv[b, sl] = c
                    turn[b, sl] = i
                    typ[b, sl] = y
                    pos[b, sl] = s + np.arange(n)
                    idx += n
                s_h = e_rin + 1            # h_{i+1} starts right after r_in_i
    return {"conv": conv, "turn": turn, "type": typ, "pos": pos}


def conv_range(lay, b: int, c: int) -> Tuple[int, int]:
    """Packed index range [a, a + n) of conversation c in row b (contiguous)."""
    idx = np.nonzero(lay["conv"][b] == c)[0]
    if len(idx) == 0:
        return 0, 0
    return int(idx[0]), int(idx[-1]) + 1


def n_convs(lay, b: int) -> int:
    return int(lay["conv"][b].max()) + 1


def _segments(lay, b: int, a: int, e: int):
    """Contiguous runs of equal (turn, type) inside [a, e): (turn, type, start, stop)."""
    tu = lay["turn"][b, a:e]
    ty = lay["type"][b, a:e]
    segs = []
    s = 0
    n = e - a
    while s < n:
        f = s
        while f < n and tu[f] == tu[s] and ty[f] == ty[s]:
            f += 1
        segs.append((int(tu[s]), int(ty[s]), a + s, a + f))
        s = f
    return segs


# ----------------------------------------------------------------------------
# the block-sparse mask, from the four rules
# ----------------------------------------------------------------------------
# Within its own turn a query of type y sees these whole segments
# (wiki summary, "分块稀疏注意力掩码"):
#   h_i    -> (nothing else of turn i)
#   t_i    -> h_i
#   r_in_i -> h_i
#   r_out_i-> h_i, t_i
# and its own segment causally.  Every query also sees H_<i.
_SAME_TURN_WHOLE = {H: (), T: (H,), RIN: (H,), ROUT: (H, T)}
# H_<i: the human messages and the context copies of earlier turns.
_HISTORY_TYPES = (H, RIN)


def conv_mask(lay, b: int, c: int, q0: int = 0, q1: int = None, qidx=None) -> np.ndarray:
    """Rows of conversation c's dense bool mask [nq, n] (conversation-local
    indices): the queries q0 .. q1-1, or the listed queries ``qidx``.

    Built by set membership: for each (query segment, key segment) pair the
    rules say "all", "causal" (same segment) or "none".  Conversations are
    separate blocks of the packed mask; PAD sees nothing and is never seen.
    """
    a, e = conv_range(lay, b, c)
    n = e - a
    if qidx is None:
        qidx = np.arange(q0, n if q1 is None else q1)
    qidx = np.asarray(qidx, dtype=np.int64)
    M = np.zeros((len(qidx), n), dtype=bool)
    segs = _segments(lay, b, a, e)
    for (i, y, qs, qe) in segs:
        rows = np.nonzero((qidx >= qs - a) & (qidx < qe - a))[0]
        if len(rows) == 0:
            continue
        for (j, x, ks, ke) in segs:
            cols = slice(ks - a, ke - a)
            if j < i and x in _HISTORY_TYPES:
                M[rows, cols] = True
            elif j == i and x in _SAME_TURN_WHOLE[y]:
                M[rows, cols] = True
            elif j == i and x == y:
                # causal inside the segment: key index <= query index
                qi = qidx[rows][:, None]
                ki = np.arange(ks - a, ke - a)[None, :]
                M[rows, cols] = ki <= qi
    return M


def dense_mask(lay, b: int) -> np.ndarray:
    """The whole [L, L] mask of row b (small L only)."""
    L = lay["conv"].shape[1]
    M = np.zeros((L, L), dtype=bool)
    for c in range(n_convs(lay, b)):
        a, e = conv_range(lay, b, c)
        M[a:e, a:e] = conv_mask(lay, b, c)
    return M


# ----------------------------------------------------------------------------
# tile schedule, counted from the mask
# ----------------------------------------------------------------------------
EMPTY, PARTIAL, FULL = 0, 1, 2
SUB = 32


def _group_sum(M: np.ndarray, start: int, axis: int, g: int):
    """Sum M (non-empty along ``axis``) in groups of g aligned to the absolute
    index ``start`` of its first entry; returns (first group index, sums)."""
    n = M.shape[axis]
    cuts = [0] + [k for k in range(1, n) if (start + k) % g == 0]
    return start // g, np.add.reduceat(M.astype(np.int64), cuts, axis=axis)


def schedule(lay, b: int, BQ: int, BK: int, row_chunk: int = 2048, order: str = "packed") -> Dict[str, np.ndarray]:
    """Tile classes and lists of row b for BQ x BK tiles.

    A tile is EMPTY if the mask allows none of its pairs, FULL if it allows all
    BQ*BK of them (entries beyond L count as masked), PARTIAL otherwise; the
    same rule at 32 x 32 gives the sub-block classes, packed two bits each
    (sub-block (i, j) at bit 2*(i*BK/32 + j)).  q_list[m] lists the non-empty
    k-tiles of q-tile m ascending, k_list[n] the non-empty q-tiles of k-tile n.
    order "packed" tiles the mask over the packed token order; "attention"
    tiles it over attention order (queries and keys both at their slots).
    """
    L = lay["conv"].shape[1]
    MT, NT = -(-L // BQ), -(-L // BK)
    gg = math.gcd(math.gcd(BQ, BK), SUB)   # counting granularity
    G = np.zeros((MT * BQ // gg, NT * BK // gg), dtype=np.int64)
    slot = attention_order(lay, b) if order == "attention" else np.arange(L)
    for c in range(n_convs(lay, b)):
        a, e = conv_range(lay, b, c)
        n = e - a
        inv = np.argsort(slot[a:e] - a)    # local slot -> local token
        for r0 in range(0, n, row_chunk):
            r1 = min(n, r0 + row_chunk)
            M = conv_mask(lay, b, c, qidx=inv[r0:r1])[:, inv]
            c0, Mc = _group_sum(M, a, 1, gg)
            r0g, Mrc = _group_sum(Mc, a + r0, 0, gg)
            G[r0g:r0g + Mrc.shape[0], c0:c0 + Mrc.shape[1]] += Mrc
    counts = G.reshape(MT, BQ // gg, NT, BK // gg).sum(axis=(1, 3))
    tile_class = np.where(counts == 0, EMPTY, np.where(counts == BQ * BK, FULL, PARTIAL)).astype(np.uint8)
    sub_class = np.zeros((MT, NT), dtype=np.uint64)
    if BQ % SUB == 0 and BK % SUB == 0:
        sq, sk, f = BQ // SUB, BK // SUB, SUB // gg
        Gs = G.reshape(G.shape[0] // f, f, G.shape[1] // f, f).sum(axis=(1, 3))
        sub_cls = np.where(Gs == 0, EMPTY, np.where(Gs == SUB * SUB, FULL, PARTIAL)).astype(np.uint64)
        sub_cls = sub_cls.reshape(MT, sq, NT, sk).transpose(0, 2, 1, 3)  # [MT, NT, sq, sk]
        for i in range(sq):
            for j in range(sk):
                sub_class |= sub_cls[:, :, i, j] << np.uint64(2 * (i * sk + j))
    q_nnz = np.zeros(MT, dtype=np.int64)
    q_list = np.full((MT, NT), -1, dtype=np.int64)
    for m in range(MT):
        nz = np.nonzero(counts[m] > 0)[0]
        q_nnz[m] = len(nz)
        q_list[m, :len(nz)] = nz
    k_nnz = np.zeros(NT, dtype=np.int64)
    k_list = np.full((NT, MT), -1, dtype=np.int64)
    for nn in range(NT):
        nz = np.nonzero(counts[:, nn] > 0)[0]
        k_nnz[nn] = len(nz)
        k_list[nn, :len(nz)] = nz
    return {"counts": counts, "tile_class": tile_class, "sub_class": sub_class.astype(np.uint32),
            "q_nnz": q_nnz, "q_list": q_list, "k_nnz": k_nnz, "k_list": k_list}


def useful_pairs(lay) -> int:
    """P: allowed (query, key) pairs summed over all rows, counted from the mask."""
    P = 0
    for b in range(lay["conv"].shape[0]):
        for c in range(n_convs(lay, b)):
            a, e = conv_range(lay, b, c)
            n = e - a
            for r0 in range(0, n, 2048):
                P += int(conv_mask(lay, b, c, r0, min(n, r0 + 2048)).sum())
    return P


# ----------------------------------------------------------------------------
# attention order: the same attention over reordered tokens
# ----------------------------------------------------------------------------
def attention_order(lay, b: int) -> np.ndarray:
    """Slot of every token of row b in attention order.

    Attention commutes with any reordering applied to queries and keys alike,
    so the tokens may be processed in any order.  Attention order keeps every
    conversation in its own index range and puts first the tokens that later
    turns may see (h and r_in, in packed order), then the others (t and r_out,
    in packed order); PAD tokens keep their index.  (Design choice of this
    library, not of the pages: it makes the mask of every query at most two
    runs of keys and makes it causal in slot order.)
    """
    L = lay["conv"].shape[1]
    slot = np.arange(L, dtype=np.int64)
    for c in range(n_convs(lay, b)):
        a, e = conv_range(lay, b, c)
        ty = lay["type"][b, a:e]
        first = np.nonzero((ty == H) | (ty == RIN))[0]
        second = np.nonzero((ty == T) | (ty == ROUT))[0]
        local = np.concatenate([first, second])   # slot -> token, local
        slot[a + local] = a + np.arange(e - a)
    return slot


def _runs(v: np.ndarray) -> List[Tuple[int, int]]:
    """Maximal runs [lo, hi) of True in a 1-D bool array."""
    d = np.diff(np.concatenate([[0], v.astype(np.int8), [0]]))
    return list(zip(np.nonzero(d == 1)[0].tolist(), np.nonzero(d == -1)[0].tolist()))


def _two_runs(runs: List[Tuple[int, int]], base: int) -> List[int]:
    """[lo1, hi1, lo2, hi2] of at most two runs (offset by base); a missing run
    is written [x, x) with x the end of the one before (0 for none)."""
    if len(runs) > 2:
        raise ValueError(f"{len(runs)} runs; attention order gives at most two")
    out, x = [], 0
    for k in range(2):
        if k < len(runs):
            lo, hi = runs[k][0] + base, runs[k][1] + base
            out += [lo, hi]
            x = hi
        else:
            out += [x, x]
    return out


def slot_intervals(lay, b: int, row_chunk: int = 2048) -> Tuple[np.ndarray, np.ndarray]:
    """Mask of row b in attention order as runs of slots, [L, 4] each:
    qiv[s] = the key slots that query slot s sees, kiv[s] = the query slots
    that see key slot s, each as [lo1, hi1) and [lo2, hi2) (see _two_runs).
    Read off the permuted mask row by row (queries) and column by column."""
    L = lay["conv"].shape[1]
    qiv = np.zeros((L, 4), dtype=np.int64)
    kiv = np.zeros((L, 4), dtype=np.int64)
    slot = attention_order(lay, b)
    for c in range(n_convs(lay, b)):
        a, e = conv_range(lay, b, c)
        n = e - a
        inv = np.argsort(slot[a:e] - a)
        col_runs: List[List[Tuple[int, int]]] = [[] for _ in range(n)]
        open_at = np.full(n, -1, dtype=np.int64)   # start of a column run still open
        for r0 in range(0, n, row_chunk):
            r1 = min(n, r0 + row_chunk)
            M = conv_mask(lay, b, c, qidx=inv[r0:r1])[:, inv]
            for i in range(r1 - r0):
                qiv[a + r0 + i] = _two_runs(_runs(M[i]), a)
                row = M[i]
                starts = np.nonzero(row & (open_at < 0))[0]
                ends = np.nonzero(~row & (open_at >= 0))[0]
                for k in ends.tolist():
                    col_runs[k].append((int(open_at[k]), r0 + i))
                open_at[ends] = -1
                open_at[starts] = r0 + i
        for k in np.nonzero(open_at >= 0)[0].tolist():
            col_runs[k].append((int(open_at[k]), n))
        for k in range(n):
            kiv[a + k] = _two_runs(col_runs[k], a)
    return qiv, kiv


# ----------------------------------------------------------------------------
# RoPE at the strategic positions
# ----------------------------------------------------------------------------
def rope_angles(pos: np.ndarray, D: int, theta: float) -> np.ndarray:
    """angle[..., j] = pos * theta^(-2j/D), j < D/2."""
    j = np.arange(D // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / D)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE of x [n, H, D] at positions pos [n]:
    x' = [x1 cos - x2 sin, x2 cos + x1 sin] with x1 = x[:D/2], x2 = x[D/2:]."""
    D = x.shape[-1]
    ang = rope_angles(pos, D, theta)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_transpose(g: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """R(pos)^T g: the rotation by the negated angle (gradient through RoPE)."""
    D = g.shape[-1]
    ang = rope_angles(pos, D, theta)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    g1, g2 = g[..., : D // 2], g[..., D // 2:]
    return np.concatenate([g1 * c + g2 * s, g2 * c - g1 * s], axis=-1)


# ----------------------------------------------------------------------------
# attention forward / backward
# ----------------------------------------------------------------------------
def _f64(x):
    return np.asarray(x, dtype=np.float64)


def attn_fwd(q, k, v, lay, theta: float, scale: float = None):
    """Masked GQA attention of every row.  q [B, L, Hq, D], k/v [B, L, Hkv, D].

    Returns O [B, L, Hq, D] and LSE [B, Hq, L] (natural log), float64.
    Queries are grouped by conversation: the packed mask is block diagonal.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    O = np.zeros((B, L, Hq, D))
    LSE = np.full((B, Hq, L), -np.inf)
    for b in range(B):
        for c in range(n_convs(lay, b)):
            a, e = conv_range(lay, b, c)
            if e == a:         # a conversation of empty segments: no queries, no keys
                continue
            M = conv_mask(lay, b, c)
            pos = lay["pos"][b, a:e]
            qr = rope(q[b, a:e], pos, theta)
            kr = rope(k[b, a:e], pos, theta)
            for h in range(Hq):
                kv = h // g
                S = scale * (qr[:, h] @ kr[:, kv].T)
                S = np.where(M, S, -np.inf)
                m = S.max(axis=1, keepdims=True)
                P = np.exp(S - m)
                l = P.sum(axis=1, keepdims=True)
                P = P / l
                O[b, a:e, h] = P @ v[b, a:e, kv]
                LSE[b, h, a:e] = (m + np.log(l))[:, 0]
    return O, LSE


def attn_bwd(q, k, v, do, lay, theta: float, scale: float = None, o=None):
    """Gradients of sum(O * dO) w.r.t. the pre-RoPE q, k and v, float64.

    dV = sum_group P^T dO; dP = dO V^T; dS = P (dP - Delta);
    dQ' = scale dS K'; dK' = scale sum_group dS^T Q'; dQ = R^T dQ', dK = R^T dK'.
    Delta = rowsum(P dP), which is rowsum(dO * O); with ``o`` given (the forward
    output as a backward receives it, e.g. stored in bf16), Delta = rowsum(dO * o).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    o = None if o is None else _f64(o)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for c in range(n_convs(lay, b)):
            a, e = conv_range(lay, b, c)
            if e == a:
                continue
            M = conv_mask(lay, b, c)
            pos = lay["pos"][b, a:e]
            qr = rope(q[b, a:e], pos, theta)
            kr = rope(k[b, a:e], pos, theta)
            dqr = np.zeros_like(qr)
            dkr = np.zeros_like(kr)
            for h in range(Hq):
                kv = h // g
                S = scale * (qr[:, h] @ kr[:, kv].T)
                S = np.where(M, S, -np.inf)
                P = np.exp(S - S.max(axis=1, keepdims=True))
                P = P / P.sum(axis=1, keepdims=True)
                dO = do[b, a:e, h]
                dv[b, a:e, kv] += P.T @ dO
                dP = dO @ v[b, a:e, kv].T
                delta = (P * dP).sum(axis=1, keepdims=True) if o is None else \
                    (dO * o[b, a:e, h]).sum(axis=1, keepdims=True)
                dS = P * (dP - delta)
                dqr[:, h] = scale * (dS @ kr[:, kv])
                dkr[:, kv] += scale * (dS.T @ qr[:, h])
            dq[b, a:e] = rope_transpose(dqr, pos, theta)
            dk[b, a:e] = rope_transpose(dkr, pos, theta)
    return dq, dk, dv


# ----------------------------------------------------------------------------
# N-pass brute force (Theorem 2.1)
# ----------------------------------------------------------------------------
def attn_rows(q, k, v, do, lay, b: int, rows, theta: float, scale: float = None):
    """O, LSE and dQ of the listed query rows of row b alone, in fp64.

    The definition of attn_fwd / attn_bwd restricted to some queries, for rows
    too long for the whole oracle: each query's softmax runs over the keys of
    its conversation that the mask allows, and
    dq_p = R(pos_p)^T scale * sum_k dS_pk k'_k with dS_pk = P_pk (dP_pk - Delta_p),
    dP_pk = dO_p . v_k and Delta_p = dO_p . O_p.  PAD rows get O = 0,
    LSE = -inf and dq = 0.  Returns O [n, Hq, D], LSE [n, Hq], dQ [n, Hq, D].
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    rows = np.asarray(rows, dtype=np.int64)
    Hq, D = q.shape[2], q.shape[3]
    g = Hq // k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    O = np.zeros((len(rows), Hq, D))
    LSE = np.full((len(rows), Hq), -np.inf)
    dQ = np.zeros((len(rows), Hq, D))
    conv = lay["conv"][b, rows]
    for c in np.unique(conv[conv >= 0]):
        sel = np.nonzero(conv == c)[0]
        a, e = conv_range(lay, b, int(c))
        pos = lay["pos"][b, a:e]
        M = conv_mask(lay, b, int(c), qidx=rows[sel] - a)
        kr = rope(k[b, a:e], pos, theta)
        qr = rope(q[b, rows[sel]], lay["pos"][b, rows[sel]], theta)
        dqr = np.zeros((len(sel), Hq, D))
        for h in range(Hq):
            kv = h // g
            S = np.where(M, scale * (qr[:, h] @ kr[:, kv].T), -np.inf)
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            l = P.sum(axis=1, keepdims=True)
            P = P / l
            o = P @ v[b, a:e, kv]
            O[sel, h] = o
            LSE[sel, h] = (m + np.log(l))[:, 0]
            dP = do[b, rows[sel], h] @ v[b, a:e, kv].T
            delta = (do[b, rows[sel], h] * o).sum(axis=1, keepdims=True)
            dqr[:, h] = scale * ((P * (dP - delta)) @ kr[:, kv])
        dQ[sel] = rope_transpose(dqr, lay["pos"][b, rows[sel]], theta)
    return O, LSE, dQ


def attn_cols(q, k, v, do, lay, b: int, cols, theta: float, scale: float = None, row_chunk: int = 512):
    """dK and dV of the listed key tokens of row b alone, in fp64.

    The definition of attn_bwd restricted to some keys, for rows too long for
    the whole oracle.  A key j of conversation c is seen by the queries p of c
    with M[p, j]; for each q head h of its kv group
        P_pj  = exp(scale q'_p . k'_j - LSE_p)     (LSE_p over p's whole row)
        dS_pj = P_pj (dO_p . v_j - Delta_p),        Delta_p = dO_p . O_p,
    and dv_j = sum_h sum_p P_pj dO_p, dk_j = R(pos_j)^T scale sum_h sum_p dS_pj q'_p.
    Every query row that sees a listed key is computed whole (its softmax
    needs all of its keys), row_chunk rows at a time.  PAD keys get zeros.
    Returns dK [n, Hkv, D], dV [n, Hkv, D] in the order of ``cols``.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    cols = np.asarray(cols, dtype=np.int64)
    Hq, D = q.shape[2], q.shape[3]
    Hkv = k.shape[2]
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dK = np.zeros((len(cols), Hkv, D))
    dV = np.zeros((len(cols), Hkv, D))
    conv = lay["conv"][b, cols]
    for c in np.unique(conv[conv >= 0]):
        sel = np.nonzero(conv == c)[0]
        a, e = conv_range(lay, b, int(c))
        n = e - a
        jl = cols[sel] - a                                   # conversation-local key indices
        pos = lay["pos"][b, a:e]
        kr = rope(k[b, a:e], pos, theta)
        qr = rope(q[b, a:e], pos, theta)
        # the queries that see at least one listed key
        seen = np.zeros(n, dtype=bool)
        for r0 in range(0, n, row_chunk):
            seen[r0:r0 + row_chunk] = conv_mask(lay, b, int(c), qidx=np.arange(r0, min(n, r0 + row_chunk)))[:, jl].any(axis=1)
        rows_all = np.nonzero(seen)[0]
        dkr = np.zeros((len(sel), Hkv, D))
        for r0 in range(0, len(rows_all), row_chunk):
            rows = rows_all[r0:r0 + row_chunk]
            M = conv_mask(lay, b, int(c), qidx=rows)         # [nr, n]
            for h in range(Hq):
                kv = h // g
                S = np.where(M, scale * (qr[rows, h] @ kr[:, kv].T), -np.inf)
                m = S.max(axis=1, keepdims=True)
                P = np.exp(S - m)
                P = P / P.sum(axis=1, keepdims=True)
                O = P @ v[b, a:e, kv]
                dO = do[b, a + rows, h]
                delta = (dO * O).sum(axis=1, keepdims=True)
                Pj = P[:, jl]                                # [nr, nsel]
                dPj = dO @ v[b, cols[sel], kv].T
                dSj = Pj * (dPj - delta)
                dV[sel, kv] += Pj.T @ dO
                dkr[:, kv] += scale * (dSj.T @ qr[rows, h])
        dK[sel] = rope_transpose(dkr, pos[jl], theta)
    return dK, dV


def _seg_index(lay, b, c):
    """{(turn, type): packed indices} for conversation c of row b."""
    a, e = conv_range(lay, b, c)
    out = {}
    for (i, y, s, f) in _segments(lay, b, a, e):
        out[(i, y)] = np.arange(s, f)
    return out


def npass_index(lay, b: int, c: int, n_turns: int = None) -> List[Dict[str, np.ndarray]]:
    """For each turn i, the packed rows that make up pass i of the N-pass.

    Pass i is the ordinary sequence [h_1, r_1, ..., h_{i-1}, r_{i-1}, h_i, t_i, r_i]
    in which earlier reasoning is dropped (wiki summary, "问题背景"); the context
    copy r_in_j stands for r_j of an earlier turn, the generation copy r_out_i
    for r_i of turn i.  Returns per pass: 'idx' (packed rows in sequence order)
    and 'role' (the packed type each sequence position stands for).

    Turns that hold no tokens leave no trace in the layout, so trailing ones
    are invisible to it; ``n_turns`` (the conversation's turn count) gives
    them their passes, which then hold the history alone.
    """
    seg = _seg_index(lay, b, c)
    empty = np.zeros(0, dtype=np.int64)
    N = max(i for (i, _y) in seg) + 1 if n_turns is None else n_turns
    passes = []
    for i in range(N):
        parts, roles = [], []
        for j in range(i):
            for y in (H, RIN):
                ix = seg.get((j, y), empty)
                parts.append(ix)
                roles.append(np.full(len(ix), y))
        for y in (H, T, ROUT):
            ix = seg.get((i, y), empty)
            parts.append(ix)
            roles.append(np.full(len(ix), y))
        passes.append({"idx": np.concatenate(parts).astype(np.int64),
                       "role": np.concatenate(roles).astype(np.int64)})
    return passes


def causal_attn(q, k, v, theta: float, scale: float = None):
    """Textbook causal attention of one sequence at positions 0..n-1.

    q [n, Hq, D], k/v [n, Hkv, D]; returns O [n, Hq, D], LSE [Hq, n]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, Hq, D = q.shape
    g = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    pos = np.arange(n)
    qr, kr = rope(q, pos, theta), rope(k, pos, theta)
    causal = np.tril(np.ones((n, n), dtype=bool))
    O = np.zeros((n, Hq, D))
    LSE = np.zeros((Hq, n))
    for h in range(Hq):
        S = np.where(causal, scale * (qr[:, h] @ kr[:, h // g].T), -np.inf)
        m = S.max(axis=1, keepdims=True)
        P = np.exp(S - m)
        l = P.sum(axis=1, keepdims=True)
        O[:, h] = (P / l) @ v[:, h // g]
        LSE[h] = (m + np.log(l))[:, 0]
    return O, LSE


def causal_attn_bwd(q, k, v, do, theta: float, scale: float = None):
    """Gradients of sum(O * dO) for causal_attn, w.r.t. pre-RoPE q, k, v."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n, Hq, D = q.shape
    g = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    pos = np.arange(n)
    qr, kr = rope(q, pos, theta), rope(k, pos, theta)
    causal = np.tril(np.ones((n, n), dtype=bool))
    dqr, dkr, dv = np.zeros_like(qr), np.zeros_like(kr), np.zeros_like(v)
    for h in range(Hq):
        kv = h // g
        S = np.where(causal, scale * (qr[:, h] @ kr[:, kv].T), -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P = P / P.sum(axis=1, keepdims=True)
        dv[:, kv] += P.T @ do[:, h]
        dP = do[:, h] @ v[:, kv].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dqr[:, h] = scale * (dS @ kr[:, kv])
        dkr[:, kv] += scale * (dS.T @ qr[:, h])
    return rope_transpose(dqr, pos, theta), rope_transpose(dkr, pos, theta), dv


# ----------------------------------------------------------------------------
# per-token loss (attention-only proxy for the SFT loss)
# ----------------------------------------------------------------------------
def token_ce(feats: np.ndarray, W: np.ndarray, labels: np.ndarray) -> np.ndarray:
    """Cross entropy of softmax(feats @ W) at the given labels, one value per row."""
    z = _f64(feats) @ _f64(W)
    zmax = z.max(axis=1, keepdims=True)
    lse = zmax[:, 0] + np.log(np.exp(z - zmax).sum(axis=1))
    return lse - z[np.arange(len(labels)), labels]


def loss_rows_1pass(lay, b: int) -> np.ndarray:
    """Packed rows in the 1-pass loss: reasoning and generation copies (t_i, r_out_i).

    The generation copy is the one in the loss (wiki summary, "Token 复制");
    the reasoning is generated text too, so both are scored."""
    typ = lay["type"][b]
    return np.nonzero((typ == T) | (typ == ROUT))[0]


def token_ce_grad(feats: np.ndarray, W: np.ndarray, labels: np.ndarray) -> np.ndarray:
    """Gradient of sum_p token_ce(feats, W, labels)[p] with respect to feats.

    For logits z = feats @ W, d/dz of (logsumexp(z) - z[y]) is softmax(z) minus
    the one-hot vector of y, so the gradient is (softmax(z) - onehot(y)) @ W^T,
    row by row."""
    z = _f64(feats) @ _f64(W)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    p[np.arange(len(labels)), labels] -= 1.0
    return p @ _f64(W).T


# ----------------------------------------------------------------------------
# K-pass chunks (wiki summary, "实验结果": K-Pass; "关键洞察", item 3)
# ----------------------------------------------------------------------------
def kpass_chunk(turns, a: int, b: int, elide_last_rin: bool):
    """The sequence that trains turns [a, b) of a conversation in the K-pass variant.

    The earlier turns are context only: their human message and the context copy
    of their response, no reasoning and no generation copy (the same history an
    N-pass sequence carries, "问题背景").  Turns a .. b-1 are stored in full.
    With elide_last_rin the context copy of turn b-1 is left out: only later
    turns may see a context copy, and there are none in this sequence.
    """
    seq = [(h, 0, r_in, 0) for (h, _t, r_in, _r) in turns[:a]]
    for j in range(a, b):
        h, t, r_in, r_out = turns[j]
        if elide_last_rin and j == b - 1:
            r_in = 0
        seq.append((h, t, r_in, r_out))
    return seq


def kpass_chunk_size(turns, a: int, b: int, elide_last_rin: bool) -> Tuple[int, int]:
    """(tokens, allowed pairs) of a chunk's sequence, the pairs counted from its mask."""
    seq = kpass_chunk(turns, a, b, elide_last_rin)
    n = sum(sum(x) for x in seq)
    if n == 0:
        return 0, 0
    return n, useful_pairs(layout([[seq]], n))


def kpass_best_splits(turns, n_chunks: int, max_tokens: int, weight: float, elide_last_rin: bool):
    """Every split of the turns into contiguous chunks, scored by brute force.

    A split's cost is the sum over its chunks of pairs + weight * tokens; a
    split is admissible when every chunk has at most max_tokens tokens (0: no
    cap) and, if n_chunks > 0, it has exactly n_chunks chunks.  Returns
    (least cost, the admissible splits of least cost as lists of chunk starts),
    or (inf, []) when none is admissible.  Exponential in the turn count: for
    small conversations only.
    """
    N = len(turns)
    size = {}
    best, arg = math.inf, []
    for bits in range(1 << (N - 1)):
        starts = [0] + [j for j in range(1, N) if bits >> (j - 1) & 1]
        if n_chunks > 0 and len(starts) != n_chunks:
            continue
        ends = starts[1:] + [N]
        cost, ok = 0.0, True
        for a, b in zip(starts, ends):
            if (a, b) not in size:
                size[(a, b)] = kpass_chunk_size(turns, a, b, elide_last_rin)
            tok, pairs = size[(a, b)]
            if max_tokens > 0 and tok > max_tokens:
                ok = False
                break
            cost += pairs + weight * tok
        if not ok:
            continue
        if cost < best:
            best, arg = cost, [starts]
        elif cost == best:
            arg.append(starts)
    return best, arg


# ----------------------------------------------------------------------------
# attention block around the masked attention: q/k/v projection, per-head RMS
# normalisation of q and k before RoPE (Qwen-3, the model family the pages
# train: wiki summary, "实验结果"), the masked attention, output projection
# ----------------------------------------------------------------------------
def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """g * x / sqrt(mean(x^2) + eps) over the last axis."""
    x = _f64(x)
    return _f64(g) * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rms_norm_bwd(x: np.ndarray, g: np.ndarray, dy: np.ndarray, eps: float):
    """(dx, dg) for y = rms_norm(x, g, eps) and upstream gradient dy.

    With r = (mean(x^2) + eps)^(-1/2) and D the last axis' length,
    dy_i/dx_j = g_i (r delta_ij - r^3 x_i x_j / D), so
    dx = r g dy - x r^3 mean(g dy x), and dg = sum over the other axes of dy x r."""
    x, g, dy = _f64(x), _f64(g), _f64(dy)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    dx = r * g * dy - x * r ** 3 * np.mean(g * dy * x, axis=-1, keepdims=True)
    dg = (dy * x * r).reshape(-1, x.shape[-1]).sum(axis=0)
    return dx, dg


def _split_qkv(qkv, Hq, Hkv, D):
    B, L, _ = qkv.shape
    q = qkv[..., :Hq * D].reshape(B, L, Hq, D)
    k = qkv[..., Hq * D:(Hq + Hkv) * D].reshape(B, L, Hkv, D)
    v = qkv[..., (Hq + Hkv) * D:].reshape(B, L, Hkv, D)
    return q, k, v


def block_fwd(x, w_qkv, w_o, g_q, g_k, lay, Hq: int, Hkv: int, D: int, theta: float, eps: float,
              attn=None):
    """One block: qkv = x w_qkv^T; q, k normalised per (token, head); masked
    attention at the layout's position ids (or ``attn(q, k, v)`` in its place);
    y = o w_o^T.  Returns y [B, L, d] and the intermediates."""
    x = _f64(x)
    qkv = x @ _f64(w_qkv).T
    q, k, v = _split_qkv(qkv, Hq, Hkv, D)
    qn, kn = rms_norm(q, g_q, eps), rms_norm(k, g_k, eps)
    o, lse = attn_fwd(qn, kn, v, lay, theta) if attn is None else attn(qn, kn, v)
    B, L, _ = x.shape
    y = o.reshape(B, L, Hq * D) @ _f64(w_o).T
    return y, {"qkv": qkv, "q": q, "k": k, "v": v, "qn": qn, "kn": kn, "o": o, "lse": lse}


def block_bwd(x, w_qkv, w_o, g_q, g_k, dy, lay, Hq: int, Hkv: int, D: int, theta: float, eps: float):
    """Gradients of sum(y * dy) for block_fwd: (dx, dw_qkv, dw_o, dg_q, dg_k)."""
    x, dy = _f64(x), _f64(dy)
    B, L, d = x.shape
    _, st = block_fwd(x, w_qkv, w_o, g_q, g_k, lay, Hq, Hkv, D, theta, eps)
    o2 = st["o"].reshape(B * L, Hq * D)
    dy2 = dy.reshape(B * L, d)
    do = (dy2 @ _f64(w_o)).reshape(B, L, Hq, D)
    dw_o = dy2.T @ o2
    dqn, dkn, dv = attn_bwd(st["qn"], st["kn"], st["v"], do, lay, theta)
    dq, dg_q = rms_norm_bwd(st["q"], g_q, dqn, eps)
    dk, dg_k = rms_norm_bwd(st["k"], g_k, dkn, eps)
    dqkv = np.concatenate([dq.reshape(B * L, -1), dk.reshape(B * L, -1), dv.reshape(B * L, -1)], axis=1)
    dx = (dqkv @ _f64(w_qkv)).reshape(B, L, d)
    dw_qkv = dqkv.T @ x.reshape(B * L, d)
    return dx, dw_qkv, dw_o, dg_q, dg_k
