"""The C ABI on a host without a GPU: libopr.so loads, exports every entry
point that include/opr.h declares, and rejects bad arguments with the
documented status before any HIP call (fake device pointers are never touched
on these paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "opr.h")


@pytest.fixture(scope="module")
def Bd():
    import torch
    # fake device pointers must never meet a real device: these checks are for
    # hosts without a GPU (a mistake in a case would otherwise reach the GPU)
    if torch.cuda.device_count() > 0:
        pytest.skip("host-only ABI checks run where no GPU is visible")
    from block_sparse_masked_opr_amd import binding
    return binding


def declared_entry_points():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:opr_status|size_t|const char \*)\s*(opr_\w+)\(", text, re.M)))


def test_exports_every_declared_symbol(Bd):
    names = declared_entry_points()
    assert len(names) == 14, names
    lib = ctypes.CDLL(Bd._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(Bd.EXPORTED) == names


def test_checked_build_exports_and_debug_errors(Bd):
    """The checked library exports the same entry points; opr_debug_errors
    rejects a null pointer in both builds and reports a release build as
    unsupported with no bits (no HIP call on either path)."""
    bits = ctypes.c_uint32(7)
    assert Bd.LIB.opr_debug_errors(None) == Bd.OPR_E_INVALID
    assert Bd.LIB.opr_debug_errors(ctypes.byref(bits)) == Bd.OPR_E_UNSUPPORTED and bits.value == 0
    dbg = os.path.join(ROOT, "block_sparse_masked_opr_amd", "libopr_debug.so")
    if not os.path.exists(dbg):
        pytest.skip("libopr_debug.so not built")
    lib = ctypes.CDLL(dbg)
    for n in declared_entry_points():
        assert hasattr(lib, n), n
    lib.opr_debug_errors.argtypes = [ctypes.c_void_p]
    assert lib.opr_debug_errors(None) == Bd.OPR_E_INVALID


def test_status_strings(Bd):
    for s in (0, -1, -2, -3, -4):
        assert Bd.opr_status_string(s).startswith("OPR_")


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _layout_struct(Bd, null_field=None, order=1):
    lay = Bd.OprLayout(*[FAKE] * 14, order)
    if null_field:
        setattr(lay, null_field, None)
    return lay


def _build(Bd, B=1, L=64, bq=128, bk=128, cpr=(1,), tpc=(1,), turns=((8, 12, 6, 6),),
           ws_bytes=1 << 30, out=None, ws=FAKE):
    cpr_a = (ctypes.c_int32 * max(1, len(cpr)))(*cpr)
    tpc_a = (ctypes.c_int32 * max(1, len(tpc)))(*tpc)
    turns_a = (Bd.OprTurn * max(1, len(turns)))(*[Bd.OprTurn(*t) for t in turns])
    out = _layout_struct(Bd) if out is None else out
    return Bd.LIB.opr_build_layout(B, L, bq, bk, ctypes.addressof(cpr_a), ctypes.addressof(tpc_a),
                                   ctypes.addressof(turns_a), ws, ws_bytes, ctypes.byref(out), None)


def test_build_layout_errors(Bd):
    assert _build(Bd, B=0) == Bd.OPR_E_INVALID
    assert _build(Bd, L=0) == Bd.OPR_E_INVALID
    assert _build(Bd, bq=48) == Bd.OPR_E_UNSUPPORTED
    assert _build(Bd, bk=256) == Bd.OPR_E_UNSUPPORTED
    assert _build(Bd, cpr=(-1,)) == Bd.OPR_E_INVALID
    assert _build(Bd, tpc=(-2,)) == Bd.OPR_E_INVALID
    assert _build(Bd, turns=((8, -1, 6, 6),)) == Bd.OPR_E_INVALID
    assert _build(Bd, L=31) == Bd.OPR_E_CAPACITY                      # 32 tokens > L
    assert _build(Bd, L=60, cpr=(2,), tpc=(1, 2), turns=((8, 12, 6, 6), (8, 12, 6, 6), (1, 1, 1, 1))) \
        == Bd.OPR_E_CAPACITY                                          # 32 + 36 tokens > 60
    assert _build(Bd, ws_bytes=16) == Bd.OPR_E_CAPACITY
    assert _build(Bd, ws=None) == Bd.OPR_E_INVALID
    assert _build(Bd, out=_layout_struct(Bd, "q_list")) == Bd.OPR_E_INVALID
    for f in ("tok_slot", "slot_tok", "slot_qiv", "slot_kiv"):
        assert _build(Bd, out=_layout_struct(Bd, f)) == Bd.OPR_E_INVALID
    assert _build(Bd, out=_layout_struct(Bd, order=2)) == Bd.OPR_E_INVALID
    assert _build(Bd, out=_layout_struct(Bd, order=-1)) == Bd.OPR_E_INVALID
    odd = _layout_struct(Bd)
    odd.slot_kiv = FAKE + 8
    assert _build(Bd, out=odd) == Bd.OPR_E_INVALID
    assert _build(Bd, B=1 << 16, L=1 << 15, cpr=(0,) * (1 << 16)) == Bd.OPR_E_UNSUPPORTED


def _build_noalloc(Bd, B=1, L=64, bq=128, bk=128, cpr=(1,), tpc=(1,), turns=((8, 12, 6, 6),), out=None):
    cpr_a = (ctypes.c_int32 * max(1, len(cpr)))(*cpr)
    tpc_a = (ctypes.c_int32 * max(1, len(tpc)))(*tpc)
    turns_a = (Bd.OprTurn * max(1, len(turns)))(*[Bd.OprTurn(*t) for t in turns])
    out = _layout_struct(Bd) if out is None else out
    return Bd.LIB.opr_build_layout_noalloc(B, L, bq, bk, ctypes.addressof(cpr_a), ctypes.addressof(tpc_a),
                                           ctypes.addressof(turns_a), ctypes.byref(out), None)


def test_build_layout_noalloc_errors(Bd):
    """The no-allocation variant validates like opr_build_layout and rejects a
    request whose scratch would exceed OPR_LAYOUT_SCRATCH_BYTES, before any
    HIP call."""
    assert _build_noalloc(Bd, B=0) == Bd.OPR_E_INVALID
    assert _build_noalloc(Bd, bq=48) == Bd.OPR_E_UNSUPPORTED
    assert _build_noalloc(Bd, turns=((8, -1, 6, 6),)) == Bd.OPR_E_INVALID
    assert _build_noalloc(Bd, L=31) == Bd.OPR_E_CAPACITY
    assert _build_noalloc(Bd, out=_layout_struct(Bd, "k_list")) == Bd.OPR_E_INVALID
    # 64 rows x 2^17 tokens: 32 MiB of per-token turn indices alone
    big = 1 << 17
    assert Bd.opr_build_layout_workspace_size(64, big, 1, 1) > Bd.OPR_LAYOUT_SCRATCH_BYTES
    assert _build_noalloc(Bd, B=64, L=big, cpr=(1,) + (0,) * 63) == Bd.OPR_E_CAPACITY
    assert Bd.opr_build_layout_workspace_size(8, 32768, 1, 1) <= Bd.OPR_LAYOUT_SCRATCH_BYTES


def test_layout_workspace_size(Bd):
    assert Bd.opr_build_layout_workspace_size(1, 64, 1, 2) > 0
    assert Bd.opr_build_layout_workspace_size(0, 64, 1, 2) == 0
    assert Bd.opr_build_layout_workspace_size(1, 64, -1, 2) == 0


def _attn_in(Bd, **kw):
    a = dict(B=1, L=256, Hq=4, Hkv=2, D=128, softmax_scale=0.0, rope_theta=1e6,
             q=FAKE, k=FAKE, v=FAKE, layout=_layout_struct(Bd), block_q=128, block_k=128,
             timing_events=None, reuse_fwd_workspace=0)
    a.update(kw)
    return Bd.OprAttnIn(**a)


def _fwd(Bd, ws_bytes=1 << 40, o=FAKE, ws=FAKE, **kw):
    a = _attn_in(Bd, **kw)
    return Bd.LIB.opr_attn_fwd(ctypes.byref(a), o, FAKE, ws, ws_bytes, None)


def _bwd(Bd, ws_bytes=1 << 40, dq=FAKE, o=FAKE, dout=FAKE, dk=FAKE, dv=FAKE, ws=FAKE, **kw):
    a = _attn_in(Bd, **kw)
    return Bd.LIB.opr_attn_bwd(ctypes.byref(a), o, FAKE, dout, dq, dk, dv, ws, ws_bytes, None)


def test_attn_errors(Bd):
    assert Bd.LIB.opr_attn_fwd(None, FAKE, FAKE, FAKE, 1 << 40, None) == Bd.OPR_E_INVALID
    for f in (_fwd, _bwd):
        assert f(Bd, D=96) == Bd.OPR_E_UNSUPPORTED
        assert f(Bd, Hq=6, Hkv=4) == Bd.OPR_E_INVALID
        assert f(Bd, block_q=64) == Bd.OPR_E_UNSUPPORTED
        assert f(Bd, rope_theta=0.0) == Bd.OPR_E_INVALID
        assert f(Bd, softmax_scale=-1.0) == Bd.OPR_E_INVALID
        assert f(Bd, q=None) == Bd.OPR_E_INVALID
        assert f(Bd, layout=_layout_struct(Bd, "sub_class")) == Bd.OPR_E_INVALID
        assert f(Bd, layout=_layout_struct(Bd, "slot_tok")) == Bd.OPR_E_INVALID
        assert f(Bd, layout=_layout_struct(Bd, order=0)) == Bd.OPR_E_INVALID   # packed-order tiles
        odd = _layout_struct(Bd)
        odd.slot_qiv = FAKE + 4                                                # runs need 16-byte alignment
        assert f(Bd, layout=odd) == Bd.OPR_E_INVALID
        assert f(Bd, ws_bytes=1024) == Bd.OPR_E_CAPACITY
        assert f(Bd, B=0) == Bd.OPR_E_INVALID
    assert _bwd(Bd, dq=None) == Bd.OPR_E_INVALID


def test_attn_alignment(Bd):
    """The kernels read and write q, k, v, o, dout, dq, dk and dv with 16-byte
    vector accesses and carve the workspace in 256-byte aligned pieces: a
    pointer off those boundaries is rejected before any HIP call."""
    for f in (_fwd, _bwd):
        for name in ("q", "k", "v"):
            for off in (2, 4, 8):
                assert f(Bd, **{name: FAKE + off}) == Bd.OPR_E_INVALID, (f.__name__, name, off)
        assert f(Bd, o=FAKE + 8) == Bd.OPR_E_INVALID
        assert f(Bd, ws=FAKE + 16) == Bd.OPR_E_INVALID
        assert f(Bd, ws=FAKE + 128) == Bd.OPR_E_INVALID
    for name in ("dout", "dq", "dk", "dv"):
        assert _bwd(Bd, **{name: FAKE + 4}) == Bd.OPR_E_INVALID, name
    # aligned arguments pass validation and meet the workspace-size check
    assert _fwd(Bd, ws_bytes=1024) == Bd.OPR_E_CAPACITY
    assert _bwd(Bd, ws_bytes=1024) == Bd.OPR_E_CAPACITY
    assert _build(Bd, ws=FAKE + 64) == Bd.OPR_E_INVALID


def test_attn_workspace_size(Bd):
    f = Bd.opr_attn_workspace_size(2, 16384, 32, 8, 128, False)
    b = Bd.opr_attn_workspace_size(2, 16384, 32, 8, 128, True)
    assert 0 < f < b
    assert Bd.opr_attn_workspace_size(1, 100, 3, 2, 128, False) == 0
    assert Bd.opr_attn_workspace_size(1, 100, 4, 2, 80, True) == 0


def _ce(Bd, B=2, L=64, F=4096, V=32, o=FAKE, w=FAKE, labels=FAKE, typ=FAKE, gs=1.0, loss=FAKE,
        dout=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return Bd.LIB.opr_token_ce(B, L, F, V, o, w, labels, typ, gs, loss, dout, ws, ws_bytes, None)


def test_token_ce_errors(Bd):
    assert _ce(Bd, B=0) == Bd.OPR_E_INVALID
    assert _ce(Bd, L=0) == Bd.OPR_E_INVALID
    assert _ce(Bd, F=96) == Bd.OPR_E_UNSUPPORTED       # F % 64 != 0
    assert _ce(Bd, F=0) == Bd.OPR_E_UNSUPPORTED
    assert _ce(Bd, V=48) == Bd.OPR_E_UNSUPPORTED
    assert _ce(Bd, V=256) == Bd.OPR_E_UNSUPPORTED
    for arg in ("o", "w", "labels", "typ", "loss"):
        assert _ce(Bd, **{arg: None}) == Bd.OPR_E_INVALID
    assert _ce(Bd, o=FAKE + 8) == Bd.OPR_E_INVALID      # 16-byte alignment
    assert _ce(Bd, w=FAKE + 2) == Bd.OPR_E_INVALID
    assert _ce(Bd, dout=FAKE + 4) == Bd.OPR_E_INVALID
    assert _ce(Bd, gs=float("nan")) == Bd.OPR_E_INVALID
    assert _ce(Bd, ws=None) == Bd.OPR_E_INVALID         # the gradient needs the workspace
    assert _ce(Bd, ws_bytes=1024) == Bd.OPR_E_CAPACITY
    assert _ce(Bd, ws=FAKE + 8) == Bd.OPR_E_INVALID      # the workspace is written with 16-byte stores
    assert _ce(Bd, B=1 << 16, L=1 << 15) == Bd.OPR_E_UNSUPPORTED


def test_token_ce_workspace_size(Bd):
    assert Bd.opr_token_ce_workspace_size(2, 16384, 4096, 32) >= 2 * 16384 * 32 * 2
    assert Bd.opr_token_ce_workspace_size(2, 16384, 4096, 128) > Bd.opr_token_ce_workspace_size(2, 16384, 4096, 32)
    assert Bd.opr_token_ce_workspace_size(2, 16384, 4000, 32) == 0
    assert Bd.opr_token_ce_workspace_size(2, 16384, 4096, 40) == 0
    assert Bd.opr_token_ce_workspace_size(0, 16384, 4096, 32) == 0


def _block_in(Bd, **kw):
    f = dict(B=1, L=256, Hq=4, Hkv=2, D=128, d_model=256, softmax_scale=0.0, rope_theta=1.0e6, norm_eps=1e-6,
             x=FAKE, w_qkv=FAKE, w_o=FAKE, g_q=FAKE, g_k=FAKE, layout=_layout_struct(Bd), block_q=128,
             block_k=128, timing_events=None, reuse_fwd_workspace=0)
    f.update(kw)
    return Bd.OprBlockIn(**f)


def _bfwd(Bd, ws_bytes=1 << 40, y=FAKE, **kw):
    a = _block_in(Bd, **kw)
    return Bd.LIB.opr_block_fwd(ctypes.byref(a), y, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)


def _bbwd(Bd, ws_bytes=1 << 40, dx=FAKE, **kw):
    a = _block_in(Bd, **kw)
    return Bd.LIB.opr_block_bwd(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, dx, FAKE, FAKE, FAKE, FAKE, FAKE,
                                ws_bytes, None)


def test_block_errors(Bd):
    assert Bd.LIB.opr_block_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == Bd.OPR_E_INVALID
    for f in (_bfwd, _bbwd):
        assert f(Bd, d_model=100) == Bd.OPR_E_INVALID        # not a multiple of 64
        assert f(Bd, d_model=0) == Bd.OPR_E_INVALID
        assert f(Bd, norm_eps=0.0) == Bd.OPR_E_INVALID
        assert f(Bd, norm_eps=float("nan")) == Bd.OPR_E_INVALID
        assert f(Bd, D=96) == Bd.OPR_E_UNSUPPORTED
        assert f(Bd, Hq=6, Hkv=4) == Bd.OPR_E_INVALID
        for arg in ("x", "w_qkv", "w_o", "g_q", "g_k"):
            assert f(Bd, **{arg: None}) == Bd.OPR_E_INVALID
        assert f(Bd, x=FAKE + 2) == Bd.OPR_E_INVALID         # 16-byte alignment
        assert f(Bd, layout=_layout_struct(Bd, "q_list")) == Bd.OPR_E_INVALID
        assert f(Bd, layout=_layout_struct(Bd, order=0)) == Bd.OPR_E_INVALID
        assert f(Bd, block_q=64) == Bd.OPR_E_UNSUPPORTED
        assert f(Bd, ws_bytes=1024) == Bd.OPR_E_CAPACITY
    assert _bfwd(Bd, y=None) == Bd.OPR_E_INVALID
    assert _bfwd(Bd, y=FAKE + 8) == Bd.OPR_E_INVALID
    assert _bbwd(Bd, dx=None) == Bd.OPR_E_INVALID


def test_block_workspace_size(Bd):
    f = Bd.opr_block_workspace_size(2, 16384, 32, 8, 128, 4096, False)
    b = Bd.opr_block_workspace_size(2, 16384, 32, 8, 128, 4096, True)
    assert Bd.opr_attn_workspace_size(2, 16384, 32, 8, 128, False) < f < b
    assert Bd.opr_block_workspace_size(1, 100, 4, 2, 128, 100, False) == 0
    assert Bd.opr_block_workspace_size(1, 100, 4, 2, 96, 128, True) == 0
