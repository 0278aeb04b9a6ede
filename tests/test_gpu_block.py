"""The attention block on the GPU (opr_block_fwd / opr_block_bwd) against the
fp64 oracle's block: hipBLASLt projections, per-head RMS norms of q and k,
the masked attention kernels, output projection, and every gradient.

Tolerances: the GPU block stores bf16 at each stage the interface fixes
(qkv, the normalised q and k, o, y; d(o), dqkv, dx), each a relative rounding
of at most 2^-9, on top of the attention kernels' own error; the oracle rounds
nothing.  Outputs are held to max |x - ref| <= 3e-2 max |ref| and
sum |x - ref| / sum |ref| <= 1e-2.  The attention inside the block is also
checked alone, from the GPU's own qkv, at the attention kernels' bar
(max-abs 2e-2, mean-rel 5e-3).
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from block_sparse_masked_opr_amd import inputs as I  # noqa: E402
from oracle import opr_oracle as O  # noqa: E402
from tests.helpers import assert_close, bf16_f64, from_device_bf16, to_device_bf16  # noqa: E402

THETA = 1.0e6
EPS = 1.0e-6


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_masked_opr_amd import binding
    return binding


def run_block(Bd, rows, L, w, t, Hq, Hkv, D):
    dev = torch.device("cuda:0")
    lay = Bd.opr_build_layout(rows, L, 128, 128, device=dev)
    wts = Bd.BlockWeights(to_device_bf16(w["w_qkv"], dev), to_device_bf16(w["w_o"], dev),
                          torch.from_numpy(w["g_q"]).to(dev), torch.from_numpy(w["g_k"]).to(dev), Hq, Hkv, D)
    x, dy = to_device_bf16(t["x"], dev), to_device_bf16(t["dy"], dev)
    y, qkv, o, lse = Bd.opr_block_fwd(x, wts, lay, THETA, eps=EPS)
    dx, dw_qkv, dw_o, dg_q, dg_k = Bd.opr_block_bwd(x, wts, lay, qkv, o, lse, dy, THETA, eps=EPS)
    torch.cuda.synchronize()
    f = lambda a: a.cpu().numpy().astype(np.float64)  # noqa: E731
    return {"y": bf16_f64(from_device_bf16(y)), "qkv": bf16_f64(from_device_bf16(qkv)),
            "o": bf16_f64(from_device_bf16(o)), "lse": f(lse), "dx": bf16_f64(from_device_bf16(dx)),
            "dw_qkv": f(dw_qkv), "dw_o": f(dw_o), "dg_q": f(dg_q), "dg_k": f(dg_k)}


def close(name, x, ref):
    assert_close(name, x, ref, max_abs=3e-2 * max(float(np.abs(ref).max()), 1e-30), mean_rel=1e-2)


BLOCK_SMALL = [
    # (label, seed, rows, extra L, Hq, Hkv, D, d_model)
    ("gqa2 d128 dm256", 11, 2, 37, 4, 2, 128, 256),
    ("mqa d64 dm128", 12, 1, 90, 4, 1, 64, 128),
    ("gqa4 d128 dm512 long turns", 13, 1, 5, 8, 2, 128, 512),
]


@pytest.mark.parametrize("case", BLOCK_SMALL, ids=[c[0] for c in BLOCK_SMALL])
def test_block_small(B, case):
    label, seed, nb, extra, Hq, Hkv, D, dm = case
    rng = np.random.default_rng(seed)
    lim = 200 if "long" in label else 60
    rows = [[[tuple([int(rng.integers(0, lim)), int(rng.integers(0, lim))] + [int(rng.integers(0, lim))] * 2)
              for _ in range(int(rng.integers(1, 4)))] for _ in range(int(rng.integers(1, 4)))] for _ in range(nb)]
    L = max(1, max(I.row_used(r) for r in rows)) + extra
    w = I.make_block_weights(dm, Hq, Hkv, D, seed=500 + seed)
    t = I.make_block_tensors(nb, L, dm, seed=600 + seed)
    print(f"[block] {label}: rows {nb} x {L}", flush=True)
    got = run_block(B, rows, L, w, t, Hq, Hkv, D)
    lay = O.layout(rows, L)
    wf = {k: bf16_f64(v) if v.dtype == np.uint16 else v.astype(np.float64) for k, v in w.items()}
    x, dy = bf16_f64(t["x"]), bf16_f64(t["dy"])
    args = (wf["w_qkv"], wf["w_o"], wf["g_q"], wf["g_k"])
    y, st = O.block_fwd(x, *args, lay, Hq, Hkv, D, THETA, EPS)
    dx, dw_qkv, dw_o, dg_q, dg_k = O.block_bwd(x, *args, dy, lay, Hq, Hkv, D, THETA, EPS)
    pad = lay["type"] == O.PAD
    live = ~pad
    assert (got["y"][pad] == 0).all() and (got["dx"][pad] == 0).all()
    close("qkv", got["qkv"], st["qkv"])
    close("o", got["o"][live], st["o"][live])
    close("lse", got["lse"].transpose(0, 2, 1)[live], st["lse"].transpose(0, 2, 1)[live])
    close("y", got["y"][live], y[live])
    close("dx", got["dx"][live], dx[live])
    close("dw_qkv", got["dw_qkv"], dw_qkv)
    close("dw_o", got["dw_o"], dw_o)
    close("dg_q", got["dg_q"], dg_q)
    close("dg_k", got["dg_k"], dg_k)
    check_attention_inside(got, lay, wf, Hq, Hkv, D, live)


def check_attention_inside(got, lay, wf, Hq, Hkv, D, live):
    """The block's attention alone, at the attention bar (max-abs 2e-2,
    mean-rel 5e-3): the oracle normalises the GPU's own bf16 qkv, rounds the
    normalised q and k to bf16 as the block stores them, and attends; so the
    stored-bf16 steps before the attention leave the comparison, and what is
    left is the attention kernels' error (plus at most one bf16 step of the
    norm's rounding on a few elements)."""
    q, k, v = O._split_qkv(got["qkv"], Hq, Hkv, D)
    rb = lambda a: bf16_f64(I.round_to_bf16_bits(np.asarray(a, dtype=np.float32)))  # noqa: E731
    qn, kn = rb(O.rms_norm(q, wf["g_q"], EPS)), rb(O.rms_norm(k, wf["g_k"], EPS))
    o, lse = O.attn_fwd(qn, kn, v, lay, THETA)
    assert_close("o (attention alone)", got["o"][live], o[live])
    assert_close("lse (attention alone)", got["lse"].transpose(0, 2, 1)[live], lse.transpose(0, 2, 1)[live])


def test_block_packed_full_size(B):
    """2 rows x 16384, 32 q / 8 kv heads, D = 128, d_model = 4096 (the Qwen-3
    width for these heads): the whole block on the GPU; the oracle recomputes
    conversation 0 of row 0 alone (every op but the attention is per token and
    conversations never see each other), checking its y, o and dx."""
    s = I.PACKED_FWD_BWD
    rows = I.packed_rows(s, I.SEEDS["packed_fwd_bwd"][0])
    dm = I.BLOCK_D_MODEL[s.Hq]
    w = I.make_block_weights(dm, s.Hq, s.Hkv, s.D, seed=701)
    t = I.make_block_tensors(s.B, s.L, dm, seed=702)
    print(f"[block] packed full size: {s.B} x {s.L}, d_model {dm}", flush=True)
    got = run_block(B, rows, s.L, w, t, s.Hq, s.Hkv, s.D)
    conv = rows[0][0]
    n = I.conv_len(conv)
    lay = O.layout([[conv]], n)
    wf = {k: bf16_f64(v) if v.dtype == np.uint16 else v.astype(np.float64) for k, v in w.items()}
    x, dy = bf16_f64(t["x"][:1, :n]), bf16_f64(t["dy"][:1, :n])
    args = (wf["w_qkv"], wf["w_o"], wf["g_q"], wf["g_k"])
    y, st = O.block_fwd(x, *args, lay, s.Hq, s.Hkv, s.D, s.theta, EPS)
    close("o (conversation 0)", got["o"][:1, :n], st["o"])
    sub = {"qkv": got["qkv"][:1, :n], "o": got["o"][:1, :n], "lse": got["lse"][:1, :, :n]}
    check_attention_inside(sub, lay, wf, s.Hq, s.Hkv, s.D, np.ones((1, n), dtype=bool))
    close("y (conversation 0)", got["y"][:1, :n], y)
    dx = O.block_bwd(x, *args, dy, lay, s.Hq, s.Hkv, s.D, s.theta, EPS)[0]
    close("dx (conversation 0)", got["dx"][:1, :n], dx)


def test_block_backward_reuse_is_identical(B):
    """opr_block_bwd given the forward's workspace (reuse_fwd_workspace) gives
    bit-identical gradients to a self-contained backward."""
    dev = torch.device("cuda:0")
    rows = [[[(40, 130, 60, 60), (25, 80, 33, 33)], [(70, 0, 45, 45)]], [[(12, 300, 90, 90)]]]
    L, Hq, Hkv, D, dm = 640, 8, 2, 128, 256
    w = I.make_block_weights(dm, Hq, Hkv, D, seed=811)
    t = I.make_block_tensors(len(rows), L, dm, seed=812)
    lay = B.opr_build_layout(rows, L, 128, 128, device=dev)
    wts = B.BlockWeights(to_device_bf16(w["w_qkv"], dev), to_device_bf16(w["w_o"], dev),
                         torch.from_numpy(w["g_q"]).to(dev), torch.from_numpy(w["g_k"]).to(dev), Hq, Hkv, D)
    x, dy = to_device_bf16(t["x"], dev), to_device_bf16(t["dy"], dev)
    ws = torch.empty(B.opr_block_workspace_size(len(rows), L, Hq, Hkv, D, dm, True), dtype=torch.uint8, device=dev)
    y, qkv, o, lse = B.opr_block_fwd(x, wts, lay, THETA, eps=EPS, workspace=ws)
    g1 = B.opr_block_bwd(x, wts, lay, qkv, o, lse, dy, THETA, eps=EPS, workspace=ws, reuse_fwd_workspace=True)
    g0 = B.opr_block_bwd(x, wts, lay, qkv, o, lse, dy, THETA, eps=EPS)
    torch.cuda.synchronize()
    print("[block] backward reuse vs self-contained", flush=True)
    for name, a, b in zip(("dx", "dw_qkv", "dw_o", "dg_q", "dg_k"), g1, g0):
        assert torch.equal(a, b), name
