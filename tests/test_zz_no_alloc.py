"""opr_build_layout_noalloc (the entry point that allocates nothing: its
scratch is a fixed device array per GPU) against opr_build_layout with a
caller workspace: every output field bit-identical, on two calls in a row,
the second with a smaller input (the scratch keeps the first call's
contents), then a third in packed order."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from block_sparse_masked_opr_amd import inputs as I  # noqa: E402


@pytest.fixture(scope="module")
def Bd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_masked_opr_amd import binding
    return binding


def _same(Bd, rows, L, order):
    dev = torch.device("cuda:0")
    ref = Bd.opr_build_layout(rows, L, 128, 128, device=dev, order=order)
    got = Bd.opr_build_layout_noalloc(rows, L, 128, 128, device=dev, order=order)
    torch.cuda.synchronize()
    a, b = ref.numpy(), got.numpy()
    for f in Bd.Layout.FIELDS:
        np.testing.assert_array_equal(b[f], a[f], err_msg=f)
    print(f"[no-alloc] {len(rows)} x {L}, order {order}: all {len(Bd.Layout.FIELDS)} fields identical", flush=True)


def test_noalloc_matches_workspace_call(Bd):
    big = I.packed_rows(I.PACKED_FWD_BWD, I.SEEDS["packed_fwd_bwd"][0])          # 2 x 16384
    _same(Bd, big, I.PACKED_FWD_BWD.L, Bd.OPR_ORDER_ATTENTION)
    small = [[[(40, 30, 20, 20), (10, 0, 5, 5)], [(7, 60, 33, 33)]]]               # 1 x 300, after the big one
    _same(Bd, small, 300, Bd.OPR_ORDER_ATTENTION)
    _same(Bd, [[[(8, 12, 6, 6), (8, 12, 6, 6)]], []], 64, Bd.OPR_ORDER_PACKED)


def test_noalloc_rejects_oversized(Bd):
    """A request whose scratch exceeds the fixed size fails before any work."""
    rows = [[[(100, 100, 100, 100)]]] + [[] for _ in range(63)]
    with pytest.raises(Bd.OprError):
        Bd.opr_build_layout_noalloc(rows, 1 << 17, 128, 128, device=torch.device("cuda:0"))
