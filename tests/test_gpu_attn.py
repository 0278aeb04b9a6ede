"""GPU parity of opr_attn_fwd / opr_attn_bwd against the fp64 oracle.

Bar: max |x - ref| <= 2e-2 and sum|x - ref| / sum|ref| <= 5e-3 for O, LSE,
dQ, dK, dV over non-PAD rows; PAD rows must be exactly O = 0, LSE = -inf and
zero gradients.  Both sides consume the same bf16 inputs (the oracle upcasts).
The gradient reference is the exact one (Delta = rowsum(P * dP) of the
oracle) wherever a kv group has at most 8 q heads.  With 16 or 32 q heads
per kv head, the bf16 rounding of o alone (the o the backward receives)
moves the summed dK by up to about 2.4e-2 through Delta = rowsum(dout * o),
so there the bar is held against the oracle's backward over its own O
rounded to bf16, and the error against the exact gradient is printed beside
it.
Full comparisons run at sizes the oracle finishes in seconds (several tiles,
ragged L, GQA 1/2/4/8/16/32, D 64 and 128, empty segments, empty rows); the
packed workloads are checked on whole sampled conversations (the mask is
block diagonal by conversation, so their rows and keys depend on nothing
else) and on every kv-head group.
"""
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from block_sparse_masked_opr_amd import inputs as I  # noqa: E402
from block_sparse_masked_opr_amd import sequences as S  # noqa: E402
from oracle import opr_oracle as O  # noqa: E402
from tests.helpers import MAX_ABS, MEAN_REL, assert_close, bf16_f64, errors, from_device_bf16, to_device_bf16  # noqa: E402

THETA = 1.0e6


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_masked_opr_amd import binding
    return binding


def run_gpu(Bd, rows, L, t, bwd=True, reuse=False, theta=None, scale=0.0):
    """Layout, forward and (optionally) backward on the GPU.  reuse: the
    backward gets the forward's workspace and reuses its state.  theta, scale:
    the RoPE base (THETA if None) and the softmax scale (0: 1/sqrt(D))."""
    theta = THETA if theta is None else theta
    dev = torch.device("cuda:0")
    lay = Bd.opr_build_layout(rows, L, 128, 128, device=dev)
    q, k, v = (to_device_bf16(t[n], dev) for n in ("q", "k", "v"))
    ws = None
    if reuse:
        ws = torch.empty(Bd.opr_attn_workspace_size(len(rows), L, q.shape[2], k.shape[2], q.shape[3], True),
                         dtype=torch.uint8, device=dev)
    o, lse = Bd.opr_attn_fwd(q, k, v, lay, theta, scale, workspace=ws)
    res = {"o": o, "lse": lse}
    if bwd:
        do = to_device_bf16(t["do"], dev)
        res["dq"], res["dk"], res["dv"] = Bd.opr_attn_bwd(q, k, v, o, lse, do, lay, theta, scale, workspace=ws,
                                                          reuse_fwd_workspace=reuse)
    torch.cuda.synchronize()
    out = {"o": bf16_f64(from_device_bf16(res["o"])), "lse": res["lse"].cpu().numpy().astype(np.float64)}
    if bwd:
        for n in ("dq", "dk", "dv"):
            out[n] = res[n].cpu().numpy().astype(np.float64)
    return out


def as_stored(o):
    """The oracle's forward output in the form the backward receives it (bf16,
    the ABI's o)."""
    return bf16_f64(I.round_to_bf16_bits(np.asarray(o, dtype=np.float32)))


EXACT_MAX_GROUP = 8  # q heads per kv head up to which dQ/dK/dV meet the bar against the exact gradient


def check_bwd(label, got, q, k, v, do, lay, o, group, sel=lambda x: x, **tol):
    """dQ, dK, dV against the exact oracle gradient (groups of up to 8 q
    heads), or, for larger groups, against the backward over the oracle's O
    rounded to bf16 with the exact errors printed.  ``sel`` picks the compared
    elements (non-PAD rows) of both sides."""
    exact = O.attn_bwd(q, k, v, do, lay, THETA)
    if group <= EXACT_MAX_GROUP:
        for n, ref in zip(("dq", "dk", "dv"), exact):
            assert_close(n, sel(got[n]), sel(ref), **tol)
        return
    stored = O.attn_bwd(q, k, v, do, lay, THETA, o=as_stored(o))
    for n, ref_e, ref_s in zip(("dq", "dk", "dv"), exact, stored):
        ma, mr = errors(sel(got[n]), sel(ref_e))
        print(f"  {n} vs exact gradient ({group} q heads per kv head, not held): max_abs={ma:.3e} mean_rel={mr:.3e}",
              flush=True)
        assert_close(n + " vs bf16-o reference", sel(got[n]), sel(ref_s), **tol)


def compare_full(label, rows, L, t, got, bwd=True):
    lay = O.layout(rows, L)
    q, k, v = (bf16_f64(t[n]) for n in ("q", "k", "v"))
    o, lse = O.attn_fwd(q, k, v, lay, THETA)
    pad = lay["type"] == O.PAD                      # [B, L]
    live = ~pad
    print(f"[attn] {label}", flush=True)
    assert (got["o"][pad] == 0).all()
    assert np.isneginf(got["lse"].transpose(0, 2, 1)[pad]).all()
    assert_close("O", got["o"][live], o[live])
    assert_close("LSE", got["lse"].transpose(0, 2, 1)[live], lse.transpose(0, 2, 1)[live])
    if bwd:
        for n in ("dq", "dk", "dv"):
            assert (got[n][pad] == 0).all(), n
        check_bwd(label, got, q, k, v, bf16_f64(t["do"]), lay, o, q.shape[2] // k.shape[2], sel=lambda x: x[live])


def test_tiny(B):
    rows = I.tiny_rows()
    t = I.make_tensors(1, 64, 1, 1, 64, seed=I.SEEDS["tiny"][1])
    compare_full("tiny", rows, 64, t, run_gpu(B, rows, 64, t))


SMALL = [
    # (label, seed, B, extra L, Hq, Hkv, D)
    ("gqa2 d128 ragged", 1, 2, 37, 4, 2, 128),
    ("mqa d64", 2, 1, 5, 8, 1, 64),
    ("mha d128 one tile", 3, 3, 0, 2, 2, 128),
    ("gqa8 d128", 4, 1, 200, 8, 1, 128),
    ("gqa4 d64 long turns", 5, 2, 1, 4, 1, 64),
    ("gqa16 d128", 6, 1, 45, 16, 1, 128),
    ("mqa32 d64 two groups", 7, 2, 3, 32, 2, 64),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small(B, case):
    label, seed, nb, extra, Hq, Hkv, D = case
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(nb):
        row = []
        for _ in range(int(rng.integers(1, 4))):
            turns = []
            for _ in range(int(rng.integers(1, 4))):
                lim = 180 if seed == 5 else 60
                h, tt, r = (int(x) for x in rng.integers(0, lim, size=3))
                turns.append((h, tt, r, r))
            row.append(turns)
        rows.append(row)
    L = max(1, max(I.row_used(r) for r in rows)) + extra
    t = I.make_tensors(nb, L, Hq, Hkv, D, seed=100 + seed)
    compare_full(label, rows, L, t, run_gpu(B, rows, L, t))


def test_empty_row_and_pad(B):
    rows = [[], [[(40, 30, 20, 20), (10, 0, 5, 5)]]]
    L = 260
    t = I.make_tensors(2, L, 2, 1, 128, seed=77)
    compare_full("empty row", rows, L, t, run_gpu(B, rows, L, t))


def test_empty_conversations(B):
    """Conversations with no turns, or with only empty segments, packed between
    others (they hold no tokens)."""
    a, b = [(40, 30, 20, 20), (10, 0, 5, 5)], [(7, 60, 33, 33)]
    rows = [[a, [], b, [(0, 0, 0, 0)]], [[(0, 0, 0, 0), (0, 0, 0, 0)], b, [], a]]
    L = max(I.row_used(r) for r in rows) + 9
    t = I.make_tensors(2, L, 4, 2, 64, seed=78)
    compare_full("empty conversations", rows, L, t, run_gpu(B, rows, L, t))


def _conv_group_errors(rows, b, c, a, e, kv, t, got, shape, bwd):
    """Errors of conversation c of row b, kv group kv, against the oracle:
    [(name, max_abs, mean_rel, held)] (held False: printed only)."""
    g = shape.Hq // shape.Hkv
    qh = list(range(kv * g, (kv + 1) * g))
    sl = {n: t[n][b:b + 1, a:e] for n in t}
    q = bf16_f64(sl["q"][:, :, qh])
    k = bf16_f64(sl["k"][:, :, [kv]])
    v = bf16_f64(sl["v"][:, :, [kv]])
    lay_c = O.layout([[rows[b][c]]], e - a)
    o, lse = O.attn_fwd(q, k, v, lay_c, THETA)
    out = [("O", *errors(got["o"][b:b + 1, a:e][:, :, qh], o), True),
           ("LSE", *errors(got["lse"][b:b + 1][:, qh, a:e], lse), True)]
    if bwd:
        do = bf16_f64(sl["do"][:, :, qh])
        sub = {"dq": got["dq"][b:b + 1, a:e][:, :, qh], "dk": got["dk"][b:b + 1, a:e][:, :, [kv]],
               "dv": got["dv"][b:b + 1, a:e][:, :, [kv]]}
        exact = O.attn_bwd(q, k, v, do, lay_c, THETA)
        held = g <= EXACT_MAX_GROUP
        refs = exact if held else O.attn_bwd(q, k, v, do, lay_c, THETA, o=as_stored(o))
        for n, ref_e, ref_h in zip(("dq", "dk", "dv"), exact, refs):
            out.append((n, *errors(sub[n], ref_h), True))
            if not held:
                out.append((n + " vs exact", *errors(sub[n], ref_e), False))
    return out


def compare_convs(label, rows, L, t, got, shape, convs_per_row=2, bwd=True):
    """Whole sampled conversations (first, last and random ones of each row),
    every kv group.  The oracle runs per (conversation, kv group) in a thread
    pool (numpy releases the interpreter lock inside its kernels)."""
    import concurrent.futures as cf
    lay = O.layout(rows, L)
    rng = np.random.default_rng(12345)
    jobs = []
    for b in range(len(rows)):
        nc = O.n_convs(lay, b)
        picks = sorted(set([0, nc - 1] + [int(x) for x in rng.integers(0, nc, size=convs_per_row)]))[:convs_per_row + 1]
        for c in picks:
            a, e = O.conv_range(lay, b, c)
            for kv in range(shape.Hkv):
                jobs.append((b, c, a, e, kv))
    workers = max(1, min(8, (os.cpu_count() or 1)))
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=max(1, (os.cpu_count() or 1) // workers)):
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            futs = [ex.submit(_conv_group_errors, rows, b, c, a, e, kv, t, got, shape, bwd) for (b, c, a, e, kv) in jobs]
            results = [f.result() for f in futs]
    failed = []
    for (b, c, a, e, kv), res in zip(jobs, results):
        print(f"[attn] {label} row {b} conv {c} tokens {e - a} kv group {kv}", flush=True)
        for n, ma, mr, held in res:
            tag = "" if held else " (printed, not held)"
            print(f"  {n}: max_abs={ma:.3e} mean_rel={mr:.3e}{tag}", flush=True)
            if held and not (ma <= MAX_ABS and mr <= MEAN_REL):
                failed.append((b, c, kv, n, ma, mr))
    assert not failed, failed


def test_packed_fwd(B):
    s = I.PACKED_FWD
    seed_len, seed_t = I.SEEDS["packed_fwd"]
    rows = I.packed_rows(s, seed_len)
    t = I.make_tensors(s.B, s.L, s.Hq, s.Hkv, s.D, seed=seed_t, with_dout=False)
    got = run_gpu(B, rows, s.L, t, bwd=False)
    compare_convs("packed_fwd", rows, s.L, t, got, s, convs_per_row=3, bwd=False)


def test_packed_fwd_bwd(B):
    s = I.PACKED_FWD_BWD
    seed_len, seed_t = I.SEEDS["packed_fwd_bwd"]
    rows = I.packed_rows(s, seed_len)
    t = I.make_tensors(s.B, s.L, s.Hq, s.Hkv, s.D, seed=seed_t)
    got = run_gpu(B, rows, s.L, t, reuse=True)  # as the benchmark runs it
    # the PAD tail of each row
    lay = O.layout(rows, s.L)
    pad = lay["type"] == O.PAD
    assert (got["o"][pad] == 0).all() and (got["dq"][pad] == 0).all()
    assert (got["dk"][pad] == 0).all() and (got["dv"][pad] == 0).all()
    compare_convs("packed_fwd_bwd", rows, s.L, t, got, s, convs_per_row=2)


def test_depth_gqa8(B):
    """Depth-sweep attention shape (64 q heads over 8 kv heads, D = 128), N = 4
    turns of (128, 1024, 256): whole conversation, two complete kv groups."""
    conv = I.depth_conversation(4)
    rows = [[conv]]
    L = I.conv_len(conv)
    s = I.Shape("depth4", 1, L, **I.DEPTH_HEADS)
    t = I.make_tensors(1, L, s.Hq, s.Hkv, s.D, seed=I.SEEDS["depth"][1])
    got = run_gpu(B, rows, L, t)
    compare_convs("depth N=4", rows, L, t, got, s, convs_per_row=0)


def test_npass_rows_match_onepass(B):
    """Theorem 2.1 on the GPU: the N-pass sequences, gathered from the one-pass
    row's tokens and run through the same kernels, reproduce the one-pass rows."""
    conv = [(40, 130, 70, 70), (20, 90, 50, 50), (60, 30, 80, 80)]
    L1 = I.conv_len(conv)
    t = I.make_tensors(1, L1, 4, 2, 128, seed=5150)
    lay1 = O.layout([[conv]], L1)
    passes = O.npass_index(lay1, 0, 0)
    np_rows = [[S.npass_conversations(conv)[i] for i in range(len(conv))]]
    Ln = sum(len(p["idx"]) for p in passes)
    idx = np.concatenate([p["idx"] for p in passes])
    tn = {n: np.ascontiguousarray(t[n][:, idx]) for n in t}
    g1 = run_gpu(B, [[conv]], L1, t)
    gn = run_gpu(B, np_rows, Ln, tn)
    # same kernels, same inputs at the same relative positions
    print("[attn] N-pass vs one-pass rows", flush=True)
    assert_close("O", gn["o"][0], g1["o"][0, idx], max_abs=1e-2, mean_rel=2e-3)


def test_scaled_inputs(B):
    """Magnitudes far from 1 (q x4, k x1/4, v x1e3, dout x1e-5): the per-block
    fp16 exponents must keep the relative error at the unscaled level."""
    rows = [[[(50, 120, 40, 40), (30, 60, 70, 70)], [(100, 0, 30, 30)]]]
    L = I.row_used(rows[0]) + 11
    t = I.make_tensors(1, L, 4, 1, 128, seed=99)
    f = {"q": 4.0, "k": 0.25, "v": 1.0e3, "do": 1.0e-5}
    ts = {n: I.round_to_bf16_bits(I.bf16_bits_to_f32(t[n]) * np.float32(f[n])) for n in t}
    got = run_gpu(B, rows, L, ts)
    lay = O.layout(rows, L)
    q, k, v, do = (bf16_f64(ts[n]) for n in ("q", "k", "v", "do"))
    o, lse = O.attn_fwd(q, k, v, lay, THETA)
    dq, dk, dv = O.attn_bwd(q, k, v, do, lay, THETA)
    live = lay["type"] != O.PAD
    print("[attn] scaled inputs", flush=True)
    # relative to the largest magnitude; O is bf16, whose rounding alone is up
    # to 2^-9 of it
    for n, x, ref in (("O", got["o"], o), ("dq", got["dq"], dq), ("dk", got["dk"], dk), ("dv", got["dv"], dv)):
        top = float(np.abs(ref[live]).max())
        assert_close(n, x[live] / top, ref[live] / top, max_abs=5e-3)
    assert_close("LSE", got["lse"].transpose(0, 2, 1)[live], lse.transpose(0, 2, 1)[live])


def test_input_range_edges(B):
    """Inputs near the ends of the stated range (largest magnitude per row or
    plane in [2^-46, 2^75)): q x 2^-40 and k x 2^40 (scores unchanged, operand
    exponents near +52 and -28), v x 2^70 (exponent near -58) and dout x 2^-44
    (near +56).  Every output is held relative to its largest magnitude, as in
    test_scaled_inputs."""
    rows = [[[(50, 120, 40, 40), (30, 60, 70, 70)], [(100, 0, 30, 30)]]]
    L = I.row_used(rows[0]) + 11
    t = I.make_tensors(1, L, 4, 1, 128, seed=98)
    f = {"q": 2.0 ** -40, "k": 2.0 ** 40, "v": 2.0 ** 70, "do": 2.0 ** -44}
    ts = {n: I.round_to_bf16_bits(I.bf16_bits_to_f32(t[n]) * np.float32(f[n])) for n in t}
    got = run_gpu(B, rows, L, ts)
    lay = O.layout(rows, L)
    q, k, v, do = (bf16_f64(ts[n]) for n in ("q", "k", "v", "do"))
    o, lse = O.attn_fwd(q, k, v, lay, THETA)
    dq, dk, dv = O.attn_bwd(q, k, v, do, lay, THETA)
    live = lay["type"] != O.PAD
    print("[attn] input range edges", flush=True)
    for n, x, ref in (("O", got["o"], o), ("dq", got["dq"], dq), ("dk", got["dk"], dk), ("dv", got["dv"], dv)):
        assert np.isfinite(x).all(), n
        top = float(np.abs(ref[live]).max())
        assert_close(n, x[live] / top, ref[live] / top, max_abs=5e-3)
    assert_close("LSE", got["lse"].transpose(0, 2, 1)[live], lse.transpose(0, 2, 1)[live])


@pytest.mark.parametrize("scale,theta", [(0.25, 1.0e4), (0.05, 5.0e5)])
def test_softmax_scale_and_rope_theta(B, scale, theta):
    """A softmax scale other than 1/sqrt(D) (0.25: scores about 2.8 times
    wider, so the running maximum is raised more often) and other RoPE bases:
    forward and backward against the oracle at the same scale and base, exact
    gradient (4 q heads per kv head).  dQ grows with the scale, so outputs are
    held as everywhere values exceed unit size: mean-rel <= 5e-3 and max-abs
    <= 2e-2 times max(1, the largest |ref|)."""
    rows = [[[(40, 150, 60, 60), (30, 100, 40, 40)], [(70, 0, 20, 20)]], [[(20, 60, 30, 30)]]]
    L = max(I.row_used(r) for r in rows) + 9
    t = I.make_tensors(len(rows), L, 8, 2, 128, seed=97)
    got = run_gpu(B, rows, L, t, theta=theta, scale=scale)
    lay = O.layout(rows, L)
    q, k, v, do = (bf16_f64(t[n]) for n in ("q", "k", "v", "do"))
    o, lse = O.attn_fwd(q, k, v, lay, theta, scale=scale)
    dq, dk, dv = O.attn_bwd(q, k, v, do, lay, theta, scale=scale)
    live = lay["type"] != O.PAD
    print(f"[attn] softmax scale {scale}, rope theta {theta:g}", flush=True)
    for n, x, ref in (("O", got["o"], o), ("dq", got["dq"], dq), ("dk", got["dk"], dk), ("dv", got["dv"], dv)):
        _assert_slices(n, x, ref, [("all", live)])
    assert_close("LSE", got["lse"].transpose(0, 2, 1)[live], lse.transpose(0, 2, 1)[live])


def _scaled(t, f):
    """bf16 inputs times per-element factors f[name] (broadcast), rounded to bf16 once."""
    out = dict(t)
    for n, fac in f.items():
        out[n] = I.round_to_bf16_bits(I.bf16_bits_to_f32(t[n]) * np.asarray(fac, dtype=np.float32))
    return out


def _assert_slices(label, got, ref, slices):
    """Per-slice bar: mean-relative error <= 5e-3 in every slice, and max-abs
    <= 2e-2 times max(1, the slice's largest |ref|) (values far above 1 are
    held relative to their magnitude, as their bf16 / fp16 rounding is)."""
    for name, sl in slices:
        x, r = got[sl], ref[sl]
        top = max(1.0, float(np.abs(r).max()) if r.size else 1.0)
        assert_close(f"{label} {name} (largest |ref| {top:.2e})", x / top, r / top, max_abs=MAX_ABS,
                     mean_rel=MEAN_REL)


def test_conversations_of_far_apart_magnitudes(B):
    """Three conversations in one row: one with q x1e-3 and dout x1e-4, one
    unscaled, one with v x1e3 and dout x1e2.  The dK/dV units of a key come
    from the queries of its own stages, so each conversation keeps its own
    precision: every conversation's O, dQ, dK and dV meet the bar on their
    own, against the exact gradient."""
    convs = [[(60, 150, 50, 50), (40, 90, 70, 70)], [(30, 200, 40, 40)], [(50, 100, 30, 30), (20, 60, 40, 40)]]
    rows = [convs]
    L = I.row_used(convs) + 19
    Hq, Hkv, D = 8, 2, 128
    t = I.make_tensors(1, L, Hq, Hkv, D, seed=2024)
    lay = O.layout(rows, L)
    fq = np.ones((1, L, 1, 1), np.float32)
    fv, fd = fq.copy(), fq.copy()
    spans = [O.conv_range(lay, 0, c) for c in range(3)]
    (a0, e0), (a1, e1), (a2, e2) = spans
    fq[:, a0:e0] = 1e-3
    fd[:, a0:e0] = 1e-4
    fv[:, a2:e2] = 1e3
    fd[:, a2:e2] = 1e2
    ts = _scaled(t, {"q": fq, "v": fv, "do": fd})
    got = run_gpu(B, rows, L, ts)
    q, k, v, do = (bf16_f64(ts[n]) for n in ("q", "k", "v", "do"))
    o, lse = O.attn_fwd(q, k, v, lay, THETA)
    dq, dk, dv = O.attn_bwd(q, k, v, do, lay, THETA)
    print("[attn] conversations of far-apart magnitudes", flush=True)
    sl = [(f"conv {c}", (0, slice(a, e))) for c, (a, e) in enumerate(spans)]
    for n, ref in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        _assert_slices(n, got[n], ref, sl)
    assert_close("LSE", got["lse"][0][:, :e2].T, lse[0][:, :e2].T)


def test_mixed_magnitudes_in_one_group(B):
    """Per-token and per-head scales inside one kv group: q x10^U[-3, 0] per
    (token, head), k x10^U[-3, 0] per token, v x10^U[-3, 3] per token and dout
    x10^U[-3, 3] per (token, head), so one 16-slot exponent tile holds values
    six decades apart.  q and k are not scaled above 1: larger scores saturate
    the softmax, where a near-tie turns any rounding of the scores into a
    large change of P (a property of the problem, not of the number format).
    Checked per q head (O, dQ) and per kv head (dK, dV) against the exact
    gradient."""
    rows = [[[(40, 160, 60, 60), (30, 120, 50, 50)], [(20, 90, 30, 30)]]]
    L = I.row_used(rows[0]) + 7
    Hq, Hkv, D = 8, 2, 128
    t = I.make_tensors(1, L, Hq, Hkv, D, seed=2025)
    rng = np.random.default_rng(2026)
    f = {"q": 10.0 ** rng.uniform(-3, 0, size=(1, L, Hq, 1)), "k": 10.0 ** rng.uniform(-3, 0, size=(1, L, 1, 1)),
         "v": 10.0 ** rng.uniform(-3, 3, size=(1, L, 1, 1)), "do": 10.0 ** rng.uniform(-3, 3, size=(1, L, Hq, 1))}
    ts = _scaled(t, f)
    got = run_gpu(B, rows, L, ts)
    lay = O.layout(rows, L)
    live = np.nonzero(lay["type"][0] != O.PAD)[0]
    q, k, v, do = (bf16_f64(ts[n]) for n in ("q", "k", "v", "do"))
    o, lse = O.attn_fwd(q, k, v, lay, THETA)
    dq, dk, dv = O.attn_bwd(q, k, v, do, lay, THETA)
    print("[attn] mixed magnitudes in one kv group", flush=True)
    for n, ref, H in (("o", o, Hq), ("dq", dq, Hq), ("dk", dk, Hkv), ("dv", dv, Hkv)):
        _assert_slices(n, got[n], ref, [(f"head {h}", (0, live, h)) for h in range(H)])


def test_backward_reuse_is_identical(B):
    """The backward reusing the forward's workspace gives bit-identical results."""
    rows = [[[(30, 200, 50, 50), (20, 90, 70, 70)], [(64, 64, 64, 64)]], [[(10, 5, 3, 3)]]]
    L = 900
    t = I.make_tensors(2, L, 8, 2, 128, seed=31)
    a = run_gpu(B, rows, L, t, reuse=False)
    r = run_gpu(B, rows, L, t, reuse=True)
    for n in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_array_equal(a[n], r[n], err_msg=n)


def test_cut_columns(B):
    """One deep conversation over a single kv head: the history k-tiles, seen by
    every later turn, have several times a workgroup's share of the stages, so
    the backward runs each as several parts whose partial dK/dV are summed in a
    fixed order.  Whole conversation against the oracle, and two backwards
    bit-identical."""
    conv = I.depth_conversation(3, h=128, t=640, r=192)
    L = I.conv_len(conv)
    t = I.make_tensors(1, L, 8, 1, 64, seed=4242)
    a = run_gpu(B, [[conv]], L, t)
    compare_full("cut columns", [[conv]], L, t, a)
    r = run_gpu(B, [[conv]], L, t)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(a[n], r[n], err_msg=n)


def _rotate(x, pos, theta):
    """Rotate-half RoPE of x [n, D] at positions pos [n] (fp64)."""
    D = x.shape[-1]
    ang = pos[:, None].astype(np.float64) * theta ** (-2.0 * np.arange(D // 2) / D)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[:, : D // 2], x[:, D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=1)


def test_long_reasoning_chunked_stage_lists(B):
    """One turn with 70,000 reasoning tokens: its last query tiles see ~549
    key tiles, more stages than one LDS stage-list chunk holds (1024 in the
    forward and dQ kernels, 512 in dK/dV), so the lists are built in several
    chunks.  O, LSE and dQ are checked on sampled rows (the deepest t and
    r_out rows, random rows, PAD rows) against the oracle row by row; dV and
    dK by properties that hold at any size: every query's probabilities sum
    to 1, so sum_k dV_k = sum over the group's heads and live queries of dO;
    every query's dS sums to 0, so the rotated dK (R(pos_k) dK_k) sums to 0."""
    conv = [(128, 70000, 64, 64)]
    n = I.conv_len(conv)
    L = n + 37
    Hq, Hkv, D = 2, 1, 128
    rows = [[conv]]
    t = I.make_tensors(1, L, Hq, Hkv, D, seed=7070)
    print(f"[attn] long reasoning: 1 x {L}", flush=True)
    got = run_gpu(B, rows, L, t)
    lay = O.layout(rows, L)
    rng = np.random.default_rng(7071)
    t_end = 128 + 70000
    sel = np.concatenate([np.arange(t_end - 64, t_end), np.arange(n - 64, n), rng.integers(0, n, 32),
                          np.arange(n, L)[:5]])
    q, k, v, do = (bf16_f64(t[name]) for name in ("q", "k", "v", "do"))
    o, lse, dq = O.attn_rows(q, k, v, do, lay, 0, sel, THETA)
    live = lay["type"][0, sel] != O.PAD
    assert (got["o"][0, sel[~live]] == 0).all() and (got["dq"][0, sel[~live]] == 0).all()
    assert_close("O (sampled rows)", got["o"][0, sel[live]], o[live])
    assert_close("LSE (sampled rows)", got["lse"][0][:, sel[live]].T, lse[live])
    assert_close("dQ (sampled rows)", got["dq"][0, sel[live]], dq[live])
    liv = lay["type"][0] != O.PAD
    sum_dv = got["dv"][0, liv, 0].sum(axis=0)
    sum_do = do[0, liv].sum(axis=(0, 1))
    # one missing query tile (128 queries x 2 heads of N(0, 1) dO) would move
    # the sum by about 16 per dimension
    tol_v = 1e-3 * np.sqrt(liv.sum() * Hq)
    print(f"  sum dV - sum dO: max {np.abs(sum_dv - sum_do).max():.3e} (tolerance {tol_v:.3e})", flush=True)
    assert np.abs(sum_dv - sum_do).max() <= tol_v
    dkr = _rotate(got["dk"][0, liv, 0], lay["pos"][0, liv], THETA)
    norm = np.sqrt((dkr ** 2).sum())
    print(f"  |sum R dK| / |R dK|: {np.abs(dkr.sum(axis=0)).max() / norm:.3e}", flush=True)
    assert np.abs(dkr.sum(axis=0)).max() <= 5e-3 * norm
