"""Pins for the oracle's RoPE and attention forward/backward (CPU only).

* RoPE: pos 0 is the identity; it equals complex multiplication of the pair
  (x_j, x_{j+D/2}) by e^{i*angle}; it is orthogonal; scores depend only on the
  position difference; at D = 2 the angle is the position itself.
* attention: PyTorch's scaled_dot_product_attention in float64 on the CPU with
  the oracle's boolean mask, and autograd through a complex-form RoPE for the
  gradients; central finite differences of the whole oracle on a tiny case.
* Theorem 2.1 (wiki summary, "理论保证"): the one-pass rows, per-token losses and
  (scatter-added) gradients equal those of the N separate causal passes.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from block_sparse_masked_opr_amd import inputs as I
from oracle import opr_oracle as O

THETA = 1.0e6


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def test_rope_identity_at_zero():
    x = _rand((5, 3, 16), 1)
    np.testing.assert_array_equal(O.rope(x, np.zeros(5, dtype=np.int64), THETA), x)


def test_rope_is_complex_rotation():
    """Pair j is (x_j, x_{j+D/2}); RoPE multiplies x_j + i x_{j+D/2} by e^{i a_j}
    with a_j = pos * theta^(-2j/D)."""
    D = 32
    x = _rand((7, 2, D), 2)
    pos = np.array([0, 1, 5, 100, 4097, 53247, 235519])
    z = torch.complex(torch.tensor(x[..., : D // 2]), torch.tensor(x[..., D // 2:]))
    freqs = torch.tensor([THETA ** (-(2.0 * j) / D) for j in range(D // 2)], dtype=torch.float64)
    ang = torch.tensor(pos, dtype=torch.float64)[:, None] * freqs[None, :]
    zr = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    want = torch.cat([zr.real, zr.imag], dim=-1).numpy()
    np.testing.assert_allclose(O.rope(x, pos, THETA), want, rtol=0, atol=1e-12)


def test_rope_two_dims_rotates_by_position():
    x = np.array([[[1.0, 0.0]], [[1.0, 0.0]], [[0.0, 1.0]]])
    pos = np.array([1, 2, 3])
    got = O.rope(x, pos, THETA)
    np.testing.assert_allclose(got[0, 0], [math.cos(1), math.sin(1)], atol=1e-15)
    np.testing.assert_allclose(got[1, 0], [math.cos(2), math.sin(2)], atol=1e-15)
    np.testing.assert_allclose(got[2, 0], [-math.sin(3), math.cos(3)], atol=1e-15)


def test_rope_orthogonal_and_relative():
    D = 64
    x, y = _rand((1, 1, D), 3), _rand((1, 1, D), 4)
    for a, b in [(3, 1), (1000, 17), (50000, 49000)]:
        ra = O.rope(x, np.array([a]), THETA)
        rb = O.rope(y, np.array([b]), THETA)
        rd = O.rope(x, np.array([a - b]), THETA)
        assert abs(np.sum(ra * rb) - np.sum(rd * y)) < 1e-9
        np.testing.assert_allclose(np.linalg.norm(ra), np.linalg.norm(x), rtol=1e-13)
        np.testing.assert_allclose(O.rope_transpose(ra, np.array([a]), THETA), x, atol=1e-12)


# ---------------------------------------------------------------------------
# forward / backward against the library routine and finite differences
# ---------------------------------------------------------------------------
def _torch_reference(q, k, v, do, lay, theta):
    """SDPA (float64, CPU) with the oracle's boolean mask, RoPE in complex form;
    returns O, LSE and autograd gradients."""
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    freqs = torch.tensor([theta ** (-(2.0 * j) / D) for j in range(D // 2)], dtype=torch.float64)

    def rot(x, pos):
        ang = torch.tensor(pos, dtype=torch.float64)[:, None] * freqs[None, :]
        z = torch.complex(x[..., : D // 2], x[..., D // 2:]) * torch.polar(torch.ones_like(ang), ang)[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    outs, lses = [], []
    for b in range(B):
        M = torch.tensor(O.dense_mask(lay, b))
        pos = lay["pos"][b]
        qr = rot(tq[b], pos).transpose(0, 1)                       # [Hq, L, D]
        kr = rot(tk[b], pos).transpose(0, 1).repeat_interleave(Hq // Hkv, 0)
        vv = tv[b].transpose(0, 1).repeat_interleave(Hq // Hkv, 0)
        rowhas = M.any(dim=1)
        Msafe = M.clone()
        Msafe[~rowhas, 0] = True                                    # keep SDPA finite on PAD rows
        o = torch.nn.functional.scaled_dot_product_attention(qr, kr, vv, attn_mask=Msafe)
        o = torch.where(rowhas[None, :, None], o, torch.zeros_like(o))
        s = (qr @ kr.transpose(1, 2)) / math.sqrt(D)
        lse = torch.logsumexp(s.masked_fill(~M, -math.inf), dim=-1)
        outs.append(o.transpose(0, 1))
        lses.append(lse)
    Ot = torch.stack(outs)
    (Ot * torch.tensor(do)).sum().backward()
    return (Ot.detach().numpy(), torch.stack(lses).detach().numpy(),
            tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())


small_turn = st.tuples(st.integers(0, 5), st.integers(0, 5), st.integers(0, 5))


@settings(max_examples=25, deadline=None)
@given(rows=st.lists(st.lists(st.lists(small_turn, min_size=1, max_size=3), min_size=1, max_size=2),
                     min_size=1, max_size=2),
       heads=st.sampled_from([(1, 1), (2, 1), (4, 2)]), extra=st.integers(0, 5),
       seed=st.integers(0, 1000))
def test_fwd_bwd_vs_sdpa(rows, heads, extra, seed):
    rows = [[[(h, t, r, r) for (h, t, r) in c] for c in row] for row in rows]
    L = max(1, max(I.row_used(r) for r in rows) + extra)
    Hq, Hkv = heads
    D = 16
    B = len(rows)
    lay = O.layout(rows, L)
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, L, h, D)) for h in (Hq, Hkv, Hkv))
    do = rng.standard_normal((B, L, Hq, D))
    o, lse = O.attn_fwd(q, k, v, lay, THETA)
    dq, dk, dv = O.attn_bwd(q, k, v, do, lay, THETA)
    ro, rlse, rdq, rdk, rdv = _torch_reference(q, k, v, do, lay, THETA)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    finite = np.isfinite(rlse)
    np.testing.assert_array_equal(np.isfinite(lse), finite)
    np.testing.assert_allclose(lse[finite], rlse[finite], atol=1e-12)
    np.testing.assert_allclose(dq, rdq, atol=1e-11)
    np.testing.assert_allclose(dk, rdk, atol=1e-11)
    np.testing.assert_allclose(dv, rdv, atol=1e-11)


@pytest.mark.parametrize("seed", range(4))
def test_attn_rows_vs_sdpa(seed):
    """The oracle's single-row attention (O, LSE, dQ of listed queries, for
    rows too long for the whole oracle) against the torch reference on every
    row of small packed rows, PAD included."""
    rng = np.random.default_rng(900 + seed)
    rows = [[[(int(rng.integers(0, 7)), int(rng.integers(0, 9)), *([int(rng.integers(0, 6))] * 2))
              for _ in range(int(rng.integers(1, 4)))] for _ in range(int(rng.integers(1, 3)))] for _ in range(2)]
    L = max(I.row_used(r) for r in rows) + 3
    Hq, Hkv, D = 4, 2, 16
    lay = O.layout(rows, L)
    q, k, v = (rng.standard_normal((2, L, h, D)) for h in (Hq, Hkv, Hkv))
    do = rng.standard_normal((2, L, Hq, D))
    ro, rlse, rdq, _, _ = _torch_reference(q, k, v, do, lay, THETA)
    for b in range(2):
        sel = rng.permutation(L)[: L // 2 + 1]
        o, lse, dq = O.attn_rows(q, k, v, do, lay, b, sel, THETA)
        np.testing.assert_allclose(o, ro[b, sel], atol=1e-12)
        ref_lse = rlse[b][:, sel].T
        finite = np.isfinite(ref_lse)
        np.testing.assert_array_equal(np.isfinite(lse), finite)
        np.testing.assert_allclose(lse[finite], ref_lse[finite], atol=1e-12)
        np.testing.assert_allclose(dq, rdq[b, sel], atol=1e-11)


@pytest.mark.parametrize("seed", range(4))
def test_attn_cols_vs_sdpa_and_full_backward(seed):
    """The oracle's single-key gradients (dK, dV of listed keys, for rows too
    long for the whole oracle) against the torch reference (SDPA + autograd)
    and against the full-matrix backward, on listed keys of small packed rows
    (PAD keys, empty segments and several query chunks included)."""
    rng = np.random.default_rng(950 + seed)
    rows = [[[(int(rng.integers(0, 7)), int(rng.integers(0, 9)), *([int(rng.integers(0, 6))] * 2))
              for _ in range(int(rng.integers(1, 4)))] for _ in range(int(rng.integers(1, 3)))] for _ in range(2)]
    L = max(I.row_used(r) for r in rows) + 3
    Hq, Hkv, D = 4, 2, 16
    lay = O.layout(rows, L)
    q, k, v = (rng.standard_normal((2, L, h, D)) for h in (Hq, Hkv, Hkv))
    do = rng.standard_normal((2, L, Hq, D))
    _, _, _, rdk, rdv = _torch_reference(q, k, v, do, lay, THETA)
    _, fdk, fdv = O.attn_bwd(q, k, v, do, lay, THETA)
    for b in range(2):
        sel = rng.permutation(L)[: L // 2 + 1]
        dk, dv = O.attn_cols(q, k, v, do, lay, b, sel, THETA, row_chunk=int(rng.integers(1, 9)))
        np.testing.assert_allclose(dk, rdk[b, sel], atol=1e-11)
        np.testing.assert_allclose(dv, rdv[b, sel], atol=1e-11)
        np.testing.assert_allclose(dk, fdk[b, sel], atol=1e-12)
        np.testing.assert_allclose(dv, fdv[b, sel], atol=1e-12)


def test_attn_cols_invariants():
    """Properties that hold at any size: every query's probabilities sum to 1,
    so the dV of all keys sums to the sum of dO over the group's heads and the
    live queries; every query's dS sums to 0, so the rotated dK sums to 0."""
    rows = [[[(12, 20, 9, 9), (7, 15, 6, 6), (10, 4, 8, 8)]]]
    L = I.row_used(rows[0]) + 4
    Hq, Hkv, D = 4, 1, 16
    lay = O.layout(rows, L)
    rng = np.random.default_rng(77)
    q, k, v = (rng.standard_normal((1, L, h, D)) for h in (Hq, Hkv, Hkv))
    do = rng.standard_normal((1, L, Hq, D))
    dk, dv = O.attn_cols(q, k, v, do, lay, 0, np.arange(L), THETA, row_chunk=16)
    live = lay["type"][0] != O.PAD
    np.testing.assert_allclose(dv[live, 0].sum(axis=0), do[0, live].sum(axis=(0, 1)), atol=1e-10)
    dkr = O.rope(dk[live], lay["pos"][0, live], THETA)           # R(pos) dK: back in the rotated frame
    np.testing.assert_allclose(dkr.sum(axis=0), 0.0, atol=1e-10)
    assert (dk[~live] == 0).all() and (dv[~live] == 0).all()


def test_bwd_with_given_o():
    """Delta from a given forward output: with the exact O it is the default
    backward; with O rounded to bf16 only the terms through Delta move."""
    rows = [[[(6, 9, 5, 5), (4, 7, 3, 3)]]]
    L = I.row_used(rows[0]) + 2
    lay = O.layout(rows, L)
    rng = np.random.default_rng(31)
    q, k, v = (rng.standard_normal((1, L, h, 16)) for h in (4, 2, 2))
    do = rng.standard_normal((1, L, 4, 16))
    o, _ = O.attn_fwd(q, k, v, lay, THETA)
    ref = O.attn_bwd(q, k, v, do, lay, THETA)
    for a, b in zip(O.attn_bwd(q, k, v, do, lay, THETA, o=o), ref):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    ob = I.bf16_bits_to_f32(I.round_to_bf16_bits(o.astype(np.float32))).astype(np.float64)
    dq, dk, dv = O.attn_bwd(q, k, v, do, lay, THETA, o=ob)
    np.testing.assert_array_equal(dv, ref[2])          # dV does not depend on Delta
    assert 0 < np.abs(dk - ref[1]).max() < 1e-1


def test_bwd_finite_differences():
    rows = [[[(3, 2, 2, 2), (2, 3, 1, 1)], [(2, 0, 1, 1)]]]
    L = I.row_used(rows[0]) + 2
    lay = O.layout(rows, L)
    rng = np.random.default_rng(11)
    D, Hq, Hkv = 8, 2, 1
    q = rng.standard_normal((1, L, Hq, D))
    k = rng.standard_normal((1, L, Hkv, D))
    v = rng.standard_normal((1, L, Hkv, D))
    do = rng.standard_normal((1, L, Hq, D))
    dq, dk, dv = O.attn_bwd(q, k, v, do, lay, THETA)

    def f(q_, k_, v_):
        return float((O.attn_fwd(q_, k_, v_, lay, THETA)[0] * do).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 0, 0), (0, 5, 0, 3), (0, 9, x.shape[2] - 1, 7), (0, L - 3, 0, 1), (0, L - 1, 0, 2)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (f(**{a + "_": b for a, b in args_p.items()}) - f(**{a + "_": b for a, b in args_m.items()})) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7, (name, idx, fd, g[idx])


def test_pad_rows_are_zero():
    rows = [[[(3, 2, 2, 2)]]]
    L = 16
    lay = O.layout(rows, L)
    rng = np.random.default_rng(5)
    q, k, v, do = (rng.standard_normal((1, L, 1, 8)) for _ in range(4))
    o, lse = O.attn_fwd(q, k, v, lay, THETA)
    dq, dk, dv = O.attn_bwd(q, k, v, do, lay, THETA)
    assert (o[0, 9:] == 0).all() and np.isneginf(lse[0, :, 9:]).all()
    assert (dq[0, 9:] == 0).all() and (dk[0, 9:] == 0).all() and (dv[0, 9:] == 0).all()


def test_empty_conversations_change_nothing():
    """A conversation with no turns, or with only empty segments, holds no
    tokens: the row with it packed between others has exactly the outputs and
    gradients of the row without it (every conversation starts at position 0
    and sees only itself), and both agree with the torch reference."""
    a, b = [(4, 3, 2, 2), (1, 5, 3, 3)], [(2, 6, 1, 1)]
    with_empty = [[a, [], b, [(0, 0, 0, 0), (0, 0, 0, 0)], a]]
    without = [[a, b, a]]
    L = I.row_used(without[0]) + 3
    lay_e, lay_n = O.layout(with_empty, L), O.layout(without, L)
    np.testing.assert_array_equal(lay_e["pos"], lay_n["pos"])
    np.testing.assert_array_equal(lay_e["type"], lay_n["type"])
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((1, L, h, 16)) for h in (4, 2, 2))
    do = rng.standard_normal((1, L, 4, 16))
    oe, lsee = O.attn_fwd(q, k, v, lay_e, THETA)
    on, lsen = O.attn_fwd(q, k, v, lay_n, THETA)
    np.testing.assert_array_equal(oe, on)
    np.testing.assert_array_equal(lsee, lsen)
    for ge, gn in zip(O.attn_bwd(q, k, v, do, lay_e, THETA), O.attn_bwd(q, k, v, do, lay_n, THETA)):
        np.testing.assert_array_equal(ge, gn)
    ro, rlse, rdq, rdk, rdv = _torch_reference(q, k, v, do, lay_e, THETA)
    np.testing.assert_allclose(oe, ro, atol=1e-12)
    for g, r in zip(O.attn_bwd(q, k, v, do, lay_e, THETA), (rdq, rdk, rdv)):
        np.testing.assert_allclose(g, r, atol=1e-11)


def test_causal_special_case_vs_sdpa_is_causal():
    """One turn of only a human message: SDPA with is_causal=True."""
    L, D = 23, 16
    lay = O.layout([[[(L, 0, 0, 0)]]], L)
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, L, 2, D)) for _ in range(3))
    o, _ = O.attn_fwd(q, k, v, lay, THETA)
    pos = np.arange(L)
    qr = torch.tensor(O.rope(q[0], pos, THETA)).transpose(0, 1)
    kr = torch.tensor(O.rope(k[0], pos, THETA)).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(qr, kr, torch.tensor(v[0]).transpose(0, 1), is_causal=True)
    np.testing.assert_allclose(o[0], ref.transpose(0, 1).numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# Theorem 2.1: one pass equals the N separate passes
# ---------------------------------------------------------------------------
def _theorem_case(conv, Hq=2, Hkv=1, D=16, seed=0, extra=3):
    rows = [[conv]]
    L = I.row_used(rows[0]) + extra
    lay = O.layout(rows, L)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, L, Hq, D))
    k = rng.standard_normal((1, L, Hkv, D))
    v = rng.standard_normal((1, L, Hkv, D))
    return lay, q, k, v


@settings(max_examples=40, deadline=None)
@given(conv=st.lists(st.tuples(st.integers(1, 6), st.integers(0, 6), st.integers(0, 6)), min_size=1, max_size=4),
       seed=st.integers(0, 10_000))
def test_theorem_rows_equal_npass(conv, seed):
    conv = [(h, t, r, r) for (h, t, r) in conv]
    lay, q, k, v = _theorem_case(conv, seed=seed)
    o1, lse1 = O.attn_fwd(q, k, v, lay, THETA)
    for p in O.npass_index(lay, 0, 0):
        idx = p["idx"]
        on, lsen = O.causal_attn(q[0, idx], k[0, idx], v[0, idx], THETA)
        np.testing.assert_allclose(o1[0, idx], on, atol=1e-12)
        np.testing.assert_allclose(lse1[0][:, idx], lsen, atol=1e-12)


def test_theorem_tiny_loss_and_gradients():
    """Tiny workload: per-token losses on t and r_out equal the N-pass ones, and
    the N-pass gradients scatter-added onto the packed rows equal the one-pass
    gradients when each packed row's dO goes to exactly one pass occurrence."""
    rows = I.tiny_rows()
    lay = O.layout(rows, 64)
    Hq, Hkv, D = 1, 1, 64
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 64, Hq, D))
    k = rng.standard_normal((1, 64, Hkv, D))
    v = rng.standard_normal((1, 64, Hkv, D))
    o1, _ = O.attn_fwd(q, k, v, lay, THETA)
    # labels per logical token: r_in_j and r_out_j share theirs
    rng1 = np.random.default_rng(1)
    W = rng1.standard_normal((Hq * D, 32))
    logical = {}
    labels = np.zeros(64, dtype=np.int64)
    for i in range(64):
        key = (lay["turn"][0, i], "r" if lay["type"][0, i] in (O.RIN, O.ROUT) else lay["type"][0, i],
               lay["pos"][0, i])
        if key not in logical:
            logical[key] = int(rng1.integers(32))
        labels[i] = logical[key]
    rows1 = O.loss_rows_1pass(lay, 0)
    l1 = O.token_ce(o1[0, rows1].reshape(len(rows1), -1), W, labels[rows1])
    passes = O.npass_index(lay, 0, 0)
    ln_all = {}
    for p in passes:
        on, _ = O.causal_attn(q[0, p["idx"]], k[0, p["idx"]], v[0, p["idx"]], THETA)
        sel = np.nonzero((p["role"] == O.T) | (p["role"] == O.ROUT))[0]
        # t_i and r_i of pass i are scored; earlier turns are context only
        sel = sel[lay["turn"][0, p["idx"][sel]] == lay["turn"][0, p["idx"][-1]]]
        ln = O.token_ce(on[sel].reshape(len(sel), -1), W, labels[p["idx"][sel]])
        for r, val in zip(p["idx"][sel], ln):
            ln_all[int(r)] = val
    assert sorted(ln_all) == list(rows1)
    np.testing.assert_allclose(l1, [ln_all[int(r)] for r in rows1], atol=1e-12)
    assert abs(l1.sum() - sum(ln_all.values())) < 1e-10

    # gradient identity
    do = rng.standard_normal((1, 64, Hq, D))
    last_turn = lay["turn"][0].max()
    do[0, (lay["type"][0] == O.RIN) & (lay["turn"][0] == last_turn)] = 0.0  # r_in_N has no pass
    dq1, dk1, dv1 = O.attn_bwd(q, k, v, do, lay, THETA)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for i, p in enumerate(passes):
        idx, role = p["idx"], p["role"]
        tu = lay["turn"][0, idx]
        own = (tu == i) | ((role == O.RIN) & (tu == i - 1))  # turn i rows + r_in_{i-1} context
        dop = np.where(own[:, None, None], do[0, idx], 0.0)
        gq, gk, gv = O.causal_attn_bwd(q[0, idx], k[0, idx], v[0, idx], dop, THETA)
        np.add.at(dq[0], idx, gq)
        np.add.at(dk[0], idx, gk)
        np.add.at(dv[0], idx, gv)
    np.testing.assert_allclose(dq, dq1, atol=1e-12)
    np.testing.assert_allclose(dk, dk1, atol=1e-12)
    np.testing.assert_allclose(dv, dv1, atol=1e-12)


def test_kpass_with_k_equal_n_reproduces_npass_rows():
    """K = N chunks: the t and r_out rows of chunk i equal pass i of the N-pass."""
    conv = [(3, 4, 2, 2), (2, 5, 3, 3), (4, 2, 2, 2)]
    chunks = [O.kpass_chunk(conv, i, i + 1, False) for i in range(len(conv))]
    full = O.layout([[conv]], I.conv_len(conv))
    rng = np.random.default_rng(3)
    D = 16
    n1 = I.conv_len(conv)
    q, k, v = (rng.standard_normal((1, n1, 1, D)) for _ in range(3))
    passes = O.npass_index(full, 0, 0)
    for i, ch in enumerate(chunks):
        n = I.conv_len(ch)
        lay = O.layout([[ch]], n)
        # the chunk's tokens are the packed conversation's history (h, r_in) and turn i
        idx = np.concatenate([np.nonzero((full["turn"][0] < i) & np.isin(full["type"][0], [O.H, O.RIN]))[0],
                              np.nonzero(full["turn"][0] == i)[0]])
        oc, _ = O.attn_fwd(q[:, idx], k[:, idx], v[:, idx], lay, THETA)
        on, _ = O.causal_attn(q[0, passes[i]["idx"]], k[0, passes[i]["idx"]], v[0, passes[i]["idx"]], THETA)
        for y in (O.T, O.ROUT):
            rows_c = np.nonzero((lay["type"][0] == y) & (lay["turn"][0] == i))[0]
            rows_n = np.nonzero((passes[i]["role"] == y) & (full["turn"][0, passes[i]["idx"]] == i))[0]
            np.testing.assert_allclose(oc[0, rows_c], on[rows_n], atol=1e-12)


# ----------------------------------------------------------------------------
# per-token loss: gradient pins
# ----------------------------------------------------------------------------
def test_token_ce_matches_definition_and_grad_finite_differences():
    """token_ce is -log softmax(feats @ W)[label] (checked against a direct
    evaluation of the softmax), and token_ce_grad matches central finite
    differences of the summed loss."""
    rng = np.random.default_rng(11)
    n, F, V = 5, 12, 7
    feats = rng.standard_normal((n, F))
    W = rng.standard_normal((F, V)) * 0.5
    labels = rng.integers(0, V, n)
    z = feats @ W
    ref = np.array([-np.log(np.exp(z[i, labels[i]]) / np.exp(z[i]).sum()) for i in range(n)])
    np.testing.assert_allclose(O.token_ce(feats, W, labels), ref, atol=1e-12)
    g = O.token_ce_grad(feats, W, labels)
    eps = 1e-6
    for i in range(n):
        for f in range(F):
            fp, fm = feats.copy(), feats.copy()
            fp[i, f] += eps
            fm[i, f] -= eps
            num = (O.token_ce(fp, W, labels).sum() - O.token_ce(fm, W, labels).sum()) / (2 * eps)
            assert abs(num - g[i, f]) < 1e-7, (i, f, num, g[i, f])


def test_token_ce_grad_special_cases():
    """Uniform logits: the loss is log V and the gradient is (1/V - onehot) W^T.
    Softmax is shift-invariant, so adding the same column to every logit (a
    shift of W by one column broadcast over V) leaves the loss unchanged."""
    rng = np.random.default_rng(12)
    n, F, V = 4, 6, 5
    W = rng.standard_normal((F, V))
    feats = np.zeros((n, F))
    labels = np.array([0, 1, 4, 2])
    np.testing.assert_allclose(O.token_ce(feats, W, labels), np.log(V), atol=1e-12)
    onehot = np.eye(V)[labels]
    np.testing.assert_allclose(O.token_ce_grad(feats, W, labels), (1.0 / V - onehot) @ W.T, atol=1e-12)
    feats = rng.standard_normal((n, F))
    shift = rng.standard_normal((F, 1))
    np.testing.assert_allclose(O.token_ce(feats, W + shift, labels), O.token_ce(feats, W, labels), atol=1e-12)
