"""GPU parity of opr_build_layout: bit-exact against the oracle.

Tokens, turns, types, position ids, attention-order slots and their runs of
slots, tile classes, 32x32 sub-block classes and both tile lists in both
orders, on the worked example, random rows with empty segments, empty
conversations and empty rows, ragged L, every supported tile shape, and the
packed / depth / K-pass workloads.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from block_sparse_masked_opr_amd import inputs as I  # noqa: E402
from block_sparse_masked_opr_amd import sequences as S  # noqa: E402
from oracle import opr_oracle as O  # noqa: E402


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_masked_opr_amd import binding
    return binding


def check_layout(B, rows, L, bq, bk, label, orders=(1, 0), intervals=True):
    ref = O.layout(rows, L)
    slots = [O.attention_order(ref, b) for b in range(len(rows))]
    ivs = [O.slot_intervals(ref, b) for b in range(len(rows))] if intervals else None
    for order in orders:
        name = "attention" if order == 1 else "packed"
        print(f"[layout] {label} rows={len(rows)} L={L} tiles={bq}x{bk} order={name}", flush=True)
        lay = B.opr_build_layout(rows, L, bq, bk, order=order)
        torch.cuda.synchronize()
        got = lay.numpy()
        for f in ("conv", "turn", "type", "pos"):
            np.testing.assert_array_equal(got["tok_" + f], ref[f], err_msg=f"tok_{f} {label}")
        for b in range(len(rows)):
            np.testing.assert_array_equal(got["tok_slot"][b], slots[b], err_msg=f"tok_slot {label} b={b}")
            np.testing.assert_array_equal(got["slot_tok"][b], np.argsort(slots[b]), err_msg=f"slot_tok {label}")
            if ivs is not None:
                np.testing.assert_array_equal(got["slot_qiv"][b], ivs[b][0], err_msg=f"slot_qiv {label} b={b}")
                np.testing.assert_array_equal(got["slot_kiv"][b], ivs[b][1], err_msg=f"slot_kiv {label} b={b}")
            s = O.schedule(ref, b, bq, bk, order=name)
            for f in ("tile_class", "sub_class", "q_nnz", "q_list", "k_nnz", "k_list"):
                np.testing.assert_array_equal(got[f][b], s[f], err_msg=f"{f} {label} b={b} order={name}")
    return got


@pytest.mark.parametrize("bq,bk", [(32, 32), (64, 64), (128, 128), (32, 128), (128, 64), (64, 32)])
def test_tiny(B, bq, bk):
    check_layout(B, I.tiny_rows(), 64, bq, bk, "tiny")


def _random_rows(seed, n_rows, max_convs, max_turns, max_len):
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(n_rows):
        row = []
        for _ in range(int(rng.integers(0, max_convs + 1))):
            turns = []
            for _ in range(int(rng.integers(0, max_turns + 1))):
                h, t, r = (int(x) for x in rng.integers(0, max_len + 1, size=3))
                if rng.random() < 0.2:
                    turns.append((h, 0, r, 0))          # history-only turn
                elif rng.random() < 0.2:
                    turns.append((h, t, 0, r))          # last turn of an N-pass sequence
                else:
                    turns.append((h, t, r, r))
            row.append(turns)
        rows.append(row)
    return rows


@pytest.mark.parametrize("seed", range(6))
def test_random_rows(B, seed):
    rows = _random_rows(seed, n_rows=3, max_convs=4, max_turns=5, max_len=[3, 40, 90, 7, 150, 60][seed])
    L = max(1, max(I.row_used(r) for r in rows)) + [0, 1, 17, 130, 5, 64][seed]
    for bq, bk in [(128, 128), (32, 64), (64, 128)]:
        check_layout(B, rows, L, bq, bk, f"random seed={seed}")


def test_all_pad_row(B):
    got = check_layout(B, [[], [[(5, 3, 2, 2)]]], 200, 128, 128, "empty row")
    assert (got["tok_type"][0] == O.PAD).all() and (got["q_nnz"][0] == 0).all()


def test_packed_fwd(B):
    rows = I.packed_rows(I.PACKED_FWD, I.SEEDS["packed_fwd"][0])
    check_layout(B, rows, I.PACKED_FWD.L, 128, 128, "packed_fwd")
    check_layout(B, rows, I.PACKED_FWD.L, 64, 32, "packed_fwd")


def test_packed_fwd_bwd(B):
    rows = I.packed_rows(I.PACKED_FWD_BWD, I.SEEDS["packed_fwd_bwd"][0])
    check_layout(B, rows, I.PACKED_FWD_BWD.L, 128, 128, "packed_fwd_bwd")


@pytest.mark.parametrize("N", [2, 8, 32])
def test_depth(B, N):
    conv = I.depth_conversation(N)
    # the oracle's run extraction is quadratic in the conversation length: at
    # N = 32 (53k tokens) the runs are checked through the attention-order
    # schedule, which the device computes from them
    check_layout(B, [[conv]], I.conv_len(conv), 128, 128, f"depth 1-pass N={N}", intervals=N <= 8)
    if N <= 8:
        np_convs = S.npass_conversations(conv)
        L = sum(I.conv_len(c) for c in np_convs)
        check_layout(B, [np_convs], L, 128, 128, f"depth N-pass N={N}")


def test_kpass_rows(B):
    rows = S.kpass_rows(2)
    check_layout(B, rows, I.KPASS_ROW_LEN, 128, 128, "kpass K=2")


def test_layout_batch_sampled_rows(B):
    """64 rows x 32768 tokens (the layout's bandwidth workload): rows are built
    independently, so rows 0, 31 and 63 are checked bit-exact against the
    oracle's layout of those rows alone."""
    Bn, L = I.LAYOUT_BATCH
    rows = I.layout_batch_rows(I.SEEDS["layout_batch"][0])
    print(f"[layout] batch {Bn} x {L}", flush=True)
    lay = B.opr_build_layout(rows, L, 128, 128)
    torch.cuda.synchronize()
    got = lay.numpy()
    for b in (0, 31, Bn - 1):
        ref = O.layout([rows[b]], L)
        for f in ("conv", "turn", "type", "pos"):
            np.testing.assert_array_equal(got["tok_" + f][b], ref[f][0], err_msg=f"tok_{f} row {b}")
        np.testing.assert_array_equal(got["tok_slot"][b], O.attention_order(ref, 0), err_msg=f"tok_slot row {b}")
        s = O.schedule(ref, 0, 128, 128, order="attention")
        for f in ("tile_class", "sub_class", "q_nnz", "q_list", "k_nnz", "k_list"):
            np.testing.assert_array_equal(got[f][b], s[f], err_msg=f"{f} row {b}")


def test_pinned_host_lists_match_pageable(B):
    """Page-locked host lists are read in place by the first kernel (no copy
    on the stream); pageable ones are copied with hipMemcpyAsync.  Both give
    bit-identical layouts: random rows with empty segments and conversations,
    and 3 rows of the 64 x 32768 batch, with the turn list at a 4-byte offset
    inside its pinned allocation (not 16-byte aligned, not the allocation's
    start)."""
    import ctypes
    dev = torch.device("cuda")
    batch = I.layout_batch_rows(I.SEEDS["layout_batch"][0])
    rnd = _random_rows(77, 3, 4, 5, 60)
    cases = [("random", rnd, max(I.row_used(r) for r in rnd) + 5), ("batch rows 0-2", batch[:3], I.LAYOUT_BATCH[1])]
    for label, rows, L in cases:
        print(f"[layout] pinned host lists: {label}", flush=True)
        ref = B.opr_build_layout(rows, L).numpy()
        cpr, tpc, turns = I.flatten_rows(rows)
        cpr = np.ascontiguousarray(cpr, dtype=np.int32)
        tpc = np.ascontiguousarray(tpc, dtype=np.int32)
        tw = np.ascontiguousarray(turns, dtype=np.int32).reshape(-1)
        h_cpr = torch.from_numpy(cpr).pin_memory()
        h_tpc = torch.from_numpy(tpc).pin_memory()
        h_turns = torch.zeros(tw.size + 1, dtype=torch.int32).pin_memory()
        h_turns[1:] = torch.from_numpy(tw)
        lay = B.Layout(len(rows), L, 128, 128, dev, B.OPR_ORDER_ATTENTION)
        ws = torch.empty(B.opr_build_layout_workspace_size(len(rows), L, len(tpc), len(tw) // 4), dtype=torch.uint8,
                         device=dev)
        st = lay.c_struct()
        status = B.LIB.opr_build_layout(len(rows), L, 128, 128, h_cpr.data_ptr(), h_tpc.data_ptr(),
                                        h_turns.data_ptr() + 4, ws.data_ptr(), ws.numel(), ctypes.byref(st),
                                        torch.cuda.current_stream(dev).cuda_stream)
        assert status == 0, B.opr_status_string(status)
        torch.cuda.synchronize()
        got = lay.numpy()
        for f in ref:
            np.testing.assert_array_equal(got[f], ref[f], err_msg=f"{f} {label}")
