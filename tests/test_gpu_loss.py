"""GPU parity of opr_token_ce (per-token cross entropy of a linear head on the
attention output, and its gradient) against the fp64 oracle, and Theorem 2.1
at the loss on the GPU.

Scored rows are the t and r_out tokens (wiki summary, "Token 复制"); labels are
drawn per logical token, so that r_in_j and r_out_j share theirs and each
N-pass sequence row carries the label of the one-pass row it stands for.

Bars: on identical inputs the loss is fp32 arithmetic on exact bf16 products,
so it must match the oracle to 1e-4 (F <= 4096 products of magnitude below 1
in fp32 accumulate far less error than that); dout is rounded to bf16 once and
is held to the acceptance bar (max |x - ref| <= 2e-2, sum|x - ref| / sum|ref|
<= 5e-3).  Rows that are not scored must be exactly 0 in both outputs.
Through the attention (Theorem 2.1 checks) every result carries the
attention's own error and is held to the acceptance bar.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from block_sparse_masked_opr_amd import inputs as I  # noqa: E402
from block_sparse_masked_opr_amd import sequences as S  # noqa: E402
from oracle import opr_oracle as O  # noqa: E402
from tests.helpers import assert_close, bf16_f64, from_device_bf16, to_device_bf16  # noqa: E402

THETA = 1.0e6
LOSS_ABS = 1e-4


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_masked_opr_amd import binding
    return binding


def logical_labels(lay, V, seed):
    """int32 [B, L] labels, one draw per logical token (row, conversation,
    turn, response-or-type, position); PAD rows get -1."""
    rng = np.random.default_rng(seed)
    Bn, L = lay["type"].shape
    out = np.full((Bn, L), -1, dtype=np.int32)
    seen = {}
    for b in range(Bn):
        for i in range(L):
            y = int(lay["type"][b, i])
            if y == O.PAD:
                continue
            kind = "r" if y in (O.RIN, O.ROUT) else y
            key = (b, int(lay["conv"][b, i]), int(lay["turn"][b, i]), kind, int(lay["pos"][b, i]))
            if key not in seen:
                seen[key] = int(rng.integers(V))
            out[b, i] = seen[key]
    return out


def bf16_tensor(x, dev):
    return to_device_bf16(I.round_to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32)), dev)


def run_ce(Bd, rows, L, o_bits, w_bits, labels, grad_scale=1.0):
    dev = torch.device("cuda:0")
    lay = Bd.opr_build_layout(rows, L, 128, 128, device=dev)
    o = to_device_bf16(o_bits, dev)
    w = to_device_bf16(w_bits, dev)
    lab = torch.from_numpy(labels).to(dev)
    loss, dout = Bd.opr_token_ce(o, w, lab, lay, grad_scale)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), from_device_bf16(dout), lay.numpy()


def check_against_oracle(name, lay, o_bits, w_bits, labels, loss, dout_bits, grad_scale=1.0, rows=None):
    """Compare loss and dout with the oracle on the given flat rows (all rows by default)."""
    Bn, L = labels.shape
    F = o_bits[0, 0].size
    typ = lay["tok_type"].reshape(-1)
    scored = (typ == O.T) | (typ == O.ROUT)
    flat = np.arange(Bn * L) if rows is None else np.asarray(rows)
    sc = flat[scored[flat]]
    un = flat[~scored[flat]]
    o64 = bf16_f64(o_bits).reshape(Bn * L, F)
    W = bf16_f64(w_bits).T  # oracle convention: z = feats @ W, W [F, V]
    lab = labels.reshape(-1)
    got_loss = loss.reshape(-1)
    got_d = bf16_f64(dout_bits).reshape(Bn * L, F)
    assert np.all(got_loss[un] == 0.0) and np.all(got_d[un] == 0.0), f"{name}: unscored rows not zero"
    ref_loss = O.token_ce(o64[sc], W, lab[sc])
    ref_d = grad_scale * O.token_ce_grad(o64[sc], W, lab[sc])
    assert_close(f"{name} loss", got_loss[sc], ref_loss, max_abs=LOSS_ABS, mean_rel=1e-5)
    assert_close(f"{name} dout", got_d[sc], ref_d)
    return len(sc), len(un)


@pytest.mark.parametrize("V", [32, 64, 128])
def test_token_ce_small(B, V):
    """Several conversations, empty segments, a ragged PAD tail and a run of
    32-row blocks with no scored row (PAD only)."""
    rows = [[[(8, 12, 6, 6), (8, 12, 6, 6)], [(5, 0, 3, 3), (7, 9, 0, 0), (3, 20, 4, 4)]],
            [[(30, 40, 20, 20)]]]
    L = 300
    Hq, D = 4, 64
    F = Hq * D
    lay0 = O.layout(rows, L)
    rng = np.random.default_rng(70 + V)
    o_bits = I.round_to_bf16_bits((0.5 * rng.standard_normal((2, L, Hq, D))).astype(np.float32))
    w_bits = I.round_to_bf16_bits((0.1 * rng.standard_normal((V, F))).astype(np.float32))
    labels = logical_labels(lay0, V, seed=V)
    print(f"[loss] small V={V}", flush=True)
    loss, dout, lay = run_ce(B, rows, L, o_bits, w_bits, labels, grad_scale=0.5)
    ns, nu = check_against_oracle(f"V={V}", lay, o_bits, w_bits, labels, loss, dout, grad_scale=0.5)
    assert ns > 0 and nu > 0


def test_token_ce_invalid_label_and_no_gradient(B):
    rows = [[[(8, 12, 6, 6), (8, 12, 6, 6)]]]
    L, F, V = 64, 64, 32
    dev = torch.device("cuda:0")
    lay = B.opr_build_layout(rows, L, 128, 128, device=dev)
    rng = np.random.default_rng(3)
    o_bits = I.round_to_bf16_bits(rng.standard_normal((1, L, F)).astype(np.float32))
    w_bits = I.round_to_bf16_bits((0.1 * rng.standard_normal((V, F))).astype(np.float32))
    labels = logical_labels(O.layout(rows, L), V, seed=1)
    typ = O.layout(rows, L)["type"][0]
    bad = int(np.nonzero(typ == O.ROUT)[0][0])
    labels[0, bad] = V  # out of range
    o, w, lab = to_device_bf16(o_bits, dev), to_device_bf16(w_bits, dev), torch.from_numpy(labels).to(dev)
    loss, dout = B.opr_token_ce(o, w, lab, lay)
    loss_only, none = B.opr_token_ce(o, w, lab, lay, with_grad=False)
    torch.cuda.synchronize()
    assert none is None
    loss, loss_only = loss.cpu().numpy(), loss_only.cpu().numpy()
    d = bf16_f64(from_device_bf16(dout))
    assert np.isnan(loss[0, bad]) and np.all(d[0, bad] == 0.0)
    ok = np.ones(L, dtype=bool)
    ok[bad] = False
    assert np.all(np.isfinite(loss[0, ok]))
    np.testing.assert_array_equal(loss[0, ok], loss_only[0, ok])


def test_token_ce_packed_full_size(B):
    """The 2 x 16384 packed workload (F = 32 x 128, V = 32) on the attention
    output of the forward, checked on sampled rows (scored and not)."""
    sh = I.PACKED_FWD_BWD
    rows = I.packed_rows(sh, I.SEEDS["packed_fwd_bwd"][0])
    t = I.make_tensors(sh.B, sh.L, sh.Hq, sh.Hkv, sh.D, seed=I.SEEDS["packed_fwd_bwd"][1], with_dout=False)
    dev = torch.device("cuda:0")
    lay = B.opr_build_layout(rows, sh.L, 128, 128, device=dev)
    q, k, v = (to_device_bf16(t[n], dev) for n in ("q", "k", "v"))
    o, _ = B.opr_attn_fwd(q, k, v, lay, THETA)
    F, V = sh.Hq * sh.D, 32
    rng = np.random.default_rng(9)
    w_bits = I.round_to_bf16_bits((rng.standard_normal((V, F)) / np.sqrt(F) * 4).astype(np.float32))
    lay_np = lay.numpy()
    laybase = {"type": lay_np["tok_type"], "conv": lay_np["tok_conv"], "turn": lay_np["tok_turn"],
               "pos": lay_np["tok_pos"]}
    labels = logical_labels(laybase, V, seed=4)
    w = to_device_bf16(w_bits, dev)
    print("[loss] packed full size", flush=True)
    loss, dout = B.opr_token_ce(o, w, torch.from_numpy(labels).to(dev), lay, 1.0)
    torch.cuda.synchronize()
    o_bits = from_device_bf16(o)
    sample = np.sort(rng.choice(sh.B * sh.L, size=2048, replace=False))
    ns, nu = check_against_oracle("packed", lay_np, o_bits, w_bits, labels, loss.cpu().numpy(),
                                  from_device_bf16(dout), rows=sample)
    assert ns > 500 and nu > 100


def _gpu_chain(Bd, rows, L, t, w_bits, labels):
    """fwd -> per-token loss and dout -> bwd, all on the GPU."""
    dev = torch.device("cuda:0")
    lay = Bd.opr_build_layout(rows, L, 128, 128, device=dev)
    q, k, v = (to_device_bf16(t[n], dev) for n in ("q", "k", "v"))
    o, lse = Bd.opr_attn_fwd(q, k, v, lay, THETA)
    loss, dout = Bd.opr_token_ce(o, to_device_bf16(w_bits, dev), torch.from_numpy(labels).to(dev), lay)
    dq, dk, dv = Bd.opr_attn_bwd(q, k, v, o, lse, dout, lay, THETA)
    torch.cuda.synchronize()
    return {"loss": loss.cpu().numpy(), "dq": dq.cpu().numpy(), "dk": dk.cpu().numpy(),
            "dv": dv.cpu().numpy(), "type": lay.numpy()["tok_type"]}


def test_theorem_loss_and_gradients_on_gpu(B):
    """Theorem 2.1 at the loss, on the GPU: the one pass and the N separate
    passes (gathered from the same tokens, run through the same kernels, with
    each pass scoring its own t_i and r_i) give every scored token the same
    loss, and the N-pass gradients scatter-added onto the packed tokens give
    the one-pass gradients; both match the oracle's one-pass chain (forward,
    loss, gradient of the summed loss, backward)."""
    conv = [(40, 130, 70, 70), (20, 90, 50, 50), (60, 30, 80, 80)]
    L1 = I.conv_len(conv)
    Hq, Hkv, D, V = 4, 2, 128, 32
    t = I.make_tensors(1, L1, Hq, Hkv, D, seed=5151, with_dout=False)
    lay1 = O.layout([[conv]], L1)
    labels1 = logical_labels(lay1, V, seed=77)
    rng = np.random.default_rng(78)
    w_bits = I.round_to_bf16_bits((rng.standard_normal((V, Hq * D)) / np.sqrt(Hq * D) * 4).astype(np.float32))
    passes = O.npass_index(lay1, 0, 0)
    idx = np.concatenate([p["idx"] for p in passes])
    np_rows = [[S.npass_conversations(conv)[i] for i in range(len(conv))]]
    tn = {n: np.ascontiguousarray(t[n][:, idx]) for n in t}
    print("[loss] theorem: one pass", flush=True)
    g1 = _gpu_chain(B, [[conv]], L1, t, w_bits, labels1)
    print("[loss] theorem: N passes", flush=True)
    gn = _gpu_chain(B, np_rows, len(idx), tn, w_bits, np.ascontiguousarray(labels1[:, idx]))

    # oracle one-pass chain
    f64 = {n: bf16_f64(t[n]).astype(np.float64) for n in t}
    ro, _ = O.attn_fwd(f64["q"], f64["k"], f64["v"], lay1, THETA)
    W = bf16_f64(w_bits).T
    sc1 = O.loss_rows_1pass(lay1, 0)
    feats = ro[0].reshape(L1, -1)
    ref_loss = O.token_ce(feats[sc1], W, labels1[0, sc1])
    ddo = np.zeros_like(feats)
    ddo[sc1] = O.token_ce_grad(feats[sc1], W, labels1[0, sc1])
    rdq, rdk, rdv = O.attn_bwd(f64["q"], f64["k"], f64["v"], ddo.reshape(1, L1, Hq, D), lay1, THETA)

    # every one-pass scored row is scored exactly once among the N passes
    scn = np.nonzero((gn["type"][0] == O.T) | (gn["type"][0] == O.ROUT))[0]
    assert sorted(idx[scn].tolist()) == sorted(sc1.tolist())
    loss_n = np.zeros(L1)
    loss_n[idx[scn]] = gn["loss"][0, scn]
    assert_close("one-pass loss vs oracle", g1["loss"][0, sc1], ref_loss)
    assert_close("N-pass loss vs oracle", loss_n[sc1], ref_loss)
    assert_close("N-pass vs one-pass loss", loss_n[sc1], g1["loss"][0, sc1], max_abs=1e-2, mean_rel=2e-3)
    assert abs(loss_n[sc1].sum() - g1["loss"][0, sc1].sum()) <= 1e-3 * abs(ref_loss.sum())
    for name, ref in (("dq", rdq), ("dk", rdk), ("dv", rdv)):
        scat = np.zeros_like(g1[name])
        np.add.at(scat[0], idx, gn[name][0])
        assert_close(f"one-pass {name}", g1[name], ref)
        assert_close(f"N-pass scattered {name}", scat, ref)
