"""Pins of the oracle's attention block (projections, per-head RMS norm of q
and k, masked attention, output projection), on the CPU in fp64."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_sparse_masked_opr_amd import inputs as I
from oracle import opr_oracle as O

THETA = 1.0e6
EPS = 1.0e-6


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 4, 16)) * 3.0
    g = rng.uniform(0.5, 1.5, 16)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (16,), weight=torch.from_numpy(g), eps=EPS)
    np.testing.assert_allclose(O.rms_norm(x, g, EPS), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_rms_norm_scale_invariant():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 32))
    g = rng.uniform(0.5, 1.5, 32)
    np.testing.assert_allclose(O.rms_norm(37.5 * x, g, 0.0), O.rms_norm(x, g, 0.0), rtol=1e-13, atol=1e-13)
    # with g = 1 every normalised row has mean square 1 (eps = 0)
    np.testing.assert_allclose(np.mean(O.rms_norm(x, np.ones(32), 0.0) ** 2, axis=-1), 1.0, rtol=1e-13)


def test_rms_norm_bwd_matches_autograd():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 2, 16))
    g = rng.uniform(0.5, 1.5, 16)
    dy = rng.standard_normal((6, 2, 16))
    xt = torch.from_numpy(x).requires_grad_(True)
    gt = torch.from_numpy(g).requires_grad_(True)
    torch.nn.functional.rms_norm(xt, (16,), weight=gt, eps=EPS).backward(torch.from_numpy(dy))
    dx, dg = O.rms_norm_bwd(x, g, dy, EPS)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-12, atol=1e-12)


def _small_block(seed, d=24, Hq=4, Hkv=2, D=8):
    rows = [[[(3, 5, 4, 4), (2, 0, 3, 3)], [(4, 6, 2, 2)]]]
    L = I.row_used(rows[0]) + 3   # PAD tail
    rng = np.random.default_rng(seed)
    w = {"w_qkv": rng.standard_normal(((Hq + 2 * Hkv) * D, d)) / np.sqrt(d),
         "w_o": rng.standard_normal((d, Hq * D)) / np.sqrt(Hq * D),
         "g_q": rng.uniform(0.5, 1.5, D), "g_k": rng.uniform(0.5, 1.5, D)}
    x = rng.standard_normal((1, L, d))
    dy = rng.standard_normal((1, L, d))
    return rows, L, w, x, dy, (Hq, Hkv, D)


def test_block_bwd_finite_differences():
    """Every gradient of block_bwd against central differences of sum(y * dy)."""
    rows, L, w, x, dy, (Hq, Hkv, D) = _small_block(4)
    lay = O.layout(rows, L)

    def f(x_, w_):
        y, _ = O.block_fwd(x_, w_["w_qkv"], w_["w_o"], w_["g_q"], w_["g_k"], lay, Hq, Hkv, D, THETA, EPS)
        return float((y * dy).sum())

    grads = O.block_bwd(x, w["w_qkv"], w["w_o"], w["g_q"], w["g_k"], dy, lay, Hq, Hkv, D, THETA, EPS)
    rng = np.random.default_rng(5)
    h = 1e-6
    targets = [("x", None), ("w_qkv", "w_qkv"), ("w_o", "w_o"), ("g_q", "g_q"), ("g_k", "g_k")]
    for (name, key), g in zip(targets, grads):
        arr = x if key is None else w[key]
        for _ in range(12):
            ix = tuple(int(rng.integers(0, n)) for n in arr.shape)
            old = arr[ix]
            arr[ix] = old + h
            fp = f(x, w)
            arr[ix] = old - h
            fm = f(x, w)
            arr[ix] = old
            num = (fp - fm) / (2 * h)
            assert abs(num - g[ix]) <= 1e-6 * max(1.0, abs(num)), (name, ix, num, g[ix])
    # PAD rows: no output, no input gradient
    pad = lay["type"][0] == O.PAD
    y, _ = O.block_fwd(x, w["w_qkv"], w["w_o"], w["g_q"], w["g_k"], lay, Hq, Hkv, D, THETA, EPS)
    assert (y[0, pad] == 0).all() and (grads[0][0, pad] == 0).all()


def test_block_onepass_equals_npass():
    """Theorem 2.1 through the block: every op but the attention acts per
    token, so the one-pass rows equal those of the N causal passes."""
    conv = [(5, 7, 4, 4), (3, 6, 5, 5), (4, 2, 3, 3)]
    n = I.conv_len(conv)
    lay = O.layout([[conv]], n)
    rng = np.random.default_rng(6)
    Hq, Hkv, D, d = 4, 2, 8, 16
    w_qkv = rng.standard_normal(((Hq + 2 * Hkv) * D, d)) / 4
    w_o = rng.standard_normal((d, Hq * D)) / 6
    g_q, g_k = rng.uniform(0.5, 1.5, D), rng.uniform(0.5, 1.5, D)
    x = rng.standard_normal((1, n, d))
    y1, _ = O.block_fwd(x, w_qkv, w_o, g_q, g_k, lay, Hq, Hkv, D, THETA, EPS)

    def causal(q, k, v):
        o, lse = O.causal_attn(q[0], k[0], v[0], THETA)
        return o[None], lse[None]

    for p in O.npass_index(lay, 0, 0):
        yp, _ = O.block_fwd(x[:, p["idx"]], w_qkv, w_o, g_q, g_k, None, Hq, Hkv, D, THETA, EPS, attn=causal)
        np.testing.assert_allclose(yp[0], y1[0, p["idx"]], rtol=0, atol=1e-12)
