"""ctypes binding of libopr (include/opr.h), with the same entry-point names.

Argument marshalling only: torch provides device memory and the current HIP
stream; every step of the computation runs in libopr's kernels.  Importing
this module loads libopr.so and raises if it has not been built; there is no
fallback path.  With OPR_LIB=debug in the environment it loads the checked
build, libopr_debug.so, instead (same kernels with invariant tests;
opr_debug_errors reads their error bits).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import inputs

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                         "libopr_debug.so" if os.environ.get("OPR_LIB") == "debug" else "libopr.so")

OPR_OK, OPR_E_INVALID, OPR_E_CAPACITY, OPR_E_UNSUPPORTED, OPR_E_HIP = 0, -1, -2, -3, -4
OPR_ATTN_BLOCK = 128
OPR_SUB_BLOCK = 32
OPR_ORDER_PACKED, OPR_ORDER_ATTENTION = 0, 1


class OprError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {opr_status_string(status)} ({status})")
        self.status = status


class OprTurn(ctypes.Structure):
    _fields_ = [("h", ctypes.c_int32), ("t", ctypes.c_int32),
                ("r_in", ctypes.c_int32), ("r_out", ctypes.c_int32)]


class OprLayout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "tok_conv", "tok_turn", "tok_pos", "tok_type", "tok_slot", "slot_tok", "slot_qiv",
        "slot_kiv", "tile_class", "sub_class", "q_nnz", "q_list", "k_nnz", "k_list")] + [
        ("order", ctypes.c_int32)]


class OprAttnIn(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("L", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rope_theta", ctypes.c_double),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("layout", OprLayout),
                ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("timing_events", ctypes.c_void_p), ("reuse_fwd_workspace", ctypes.c_int32)]


class OprBlockIn(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("L", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rope_theta", ctypes.c_double),
                ("norm_eps", ctypes.c_float),
                ("x", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p),
                ("g_q", ctypes.c_void_p), ("g_k", ctypes.c_void_p),
                ("layout", OprLayout),
                ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("timing_events", ctypes.c_void_p), ("reuse_fwd_workspace", ctypes.c_int32)]


class OprChunk(ctypes.Structure):
    _fields_ = [("first_turn", ctypes.c_int32), ("n_turns", ctypes.c_int32),
                ("tokens", ctypes.c_int32), ("rin_elided", ctypes.c_int32), ("pairs", ctypes.c_int64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libopr.so is not built ({_LIB_PATH}); run "
                          "`python -m block_sparse_masked_opr_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, sz, vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    lib.opr_build_layout.restype = i32
    lib.opr_build_layout.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, sz,
                                     ctypes.POINTER(OprLayout), vp]
    lib.opr_build_layout_noalloc.restype = i32
    lib.opr_build_layout_noalloc.argtypes = [i32, i32, i32, i32, vp, vp, vp, ctypes.POINTER(OprLayout), vp]
    lib.opr_build_layout_workspace_size.restype = sz
    lib.opr_build_layout_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.opr_attn_fwd.restype = i32
    lib.opr_attn_fwd.argtypes = [ctypes.POINTER(OprAttnIn), vp, vp, vp, sz, vp]
    lib.opr_attn_bwd.restype = i32
    lib.opr_attn_bwd.argtypes = [ctypes.POINTER(OprAttnIn), vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.opr_attn_workspace_size.restype = sz
    lib.opr_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    lib.opr_token_ce.restype = i32
    lib.opr_token_ce.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.opr_token_ce_workspace_size.restype = sz
    lib.opr_token_ce_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.opr_block_fwd.restype = i32
    lib.opr_block_fwd.argtypes = [ctypes.POINTER(OprBlockIn), vp, vp, vp, vp, vp, sz, vp]
    lib.opr_block_bwd.restype = i32
    lib.opr_block_bwd.argtypes = [ctypes.POINTER(OprBlockIn), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.opr_block_workspace_size.restype = sz
    lib.opr_block_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_int]
    lib.opr_kpass_plan.restype = i32
    lib.opr_kpass_plan.argtypes = [ctypes.POINTER(OprTurn), i32, i32, i32, ctypes.c_double, i32,
                                   ctypes.POINTER(OprChunk), ctypes.POINTER(i32),
                                   ctypes.POINTER(ctypes.c_double)]
    lib.opr_status_string.restype = ctypes.c_char_p
    lib.opr_status_string.argtypes = [i32]
    lib.opr_debug_errors.restype = i32
    lib.opr_debug_errors.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
    return lib


LIB = _load()

EXPORTED = ("opr_build_layout", "opr_build_layout_noalloc", "opr_build_layout_workspace_size", "opr_attn_fwd",
            "opr_attn_bwd", "opr_attn_workspace_size", "opr_token_ce", "opr_token_ce_workspace_size",
            "opr_block_fwd", "opr_block_bwd", "opr_block_workspace_size", "opr_kpass_plan",
            "opr_status_string", "opr_debug_errors")


def opr_status_string(status: int) -> str:
    return LIB.opr_status_string(int(status)).decode()


def opr_debug_errors() -> Optional[int]:
    """The current device's invariant-test bits of a checked build (then
    cleared); None for a release build, which tests nothing."""
    bits = ctypes.c_uint32(0)
    st = LIB.opr_debug_errors(ctypes.byref(bits))
    if st == OPR_E_UNSUPPORTED:
        return None
    _check(st, "opr_debug_errors")
    return int(bits.value)


def _check(status: int, what: str) -> None:
    if status != OPR_OK:
        raise OprError(status, what)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def opr_kpass_plan(conv: Sequence[Sequence[int]], n_chunks: int = 0, max_tokens: int = 0,
                   tokens_weight: float = 0.0, elide_last_rin: bool = True):
    """Chunk plan of one conversation (a list of (h, t, r_in, r_out) turns).

    Returns (chunks, cost) with chunks a list of dicts (first_turn, n_turns,
    tokens, rin_elided, pairs); raises OprError on invalid input or when no
    split meets max_tokens."""
    n = len(conv)
    arr = (OprTurn * max(n, 1))(*[OprTurn(*map(int, t)) for t in conv])
    out = (OprChunk * max(n, 1))()
    n_out = ctypes.c_int32(0)
    cost = ctypes.c_double(0.0)
    _check(LIB.opr_kpass_plan(arr, n, int(n_chunks), int(max_tokens), float(tokens_weight),
                              1 if elide_last_rin else 0, out, ctypes.byref(n_out), ctypes.byref(cost)),
           "opr_kpass_plan")
    chunks = [{f: getattr(out[i], f) for f, _ in OprChunk._fields_} for i in range(n_out.value)]
    return chunks, cost.value


def opr_build_layout_workspace_size(B: int, L: int, n_convs: int, n_turns: int) -> int:
    return int(LIB.opr_build_layout_workspace_size(B, L, n_convs, n_turns))


def opr_attn_workspace_size(B: int, L: int, Hq: int, Hkv: int, D: int, is_bwd: bool) -> int:
    return int(LIB.opr_attn_workspace_size(B, L, Hq, Hkv, D, 1 if is_bwd else 0))


class Layout:
    """Device tensors filled by opr_build_layout (int32 unless noted)."""

    FIELDS = ("tok_conv", "tok_turn", "tok_pos", "tok_type", "tok_slot", "slot_tok", "slot_qiv",
              "slot_kiv", "tile_class", "sub_class", "q_nnz", "q_list", "k_nnz", "k_list")

    def __init__(self, B: int, L: int, block_q: int, block_k: int, device, order: int = OPR_ORDER_ATTENTION):
        self.B, self.L, self.block_q, self.block_k, self.order = B, L, block_q, block_k, order
        self.MT, self.NT = -(-L // block_q), -(-L // block_k)
        e = dict(device=device)
        self.tok_conv = torch.empty((B, L), dtype=torch.int32, **e)
        self.tok_turn = torch.empty((B, L), dtype=torch.int32, **e)
        self.tok_pos = torch.empty((B, L), dtype=torch.int32, **e)
        self.tok_type = torch.empty((B, L), dtype=torch.uint8, **e)
        self.tok_slot = torch.empty((B, L), dtype=torch.int32, **e)
        self.slot_tok = torch.empty((B, L), dtype=torch.int32, **e)
        self.slot_qiv = torch.empty((B, L, 4), dtype=torch.int32, **e)
        self.slot_kiv = torch.empty((B, L, 4), dtype=torch.int32, **e)
        self.tile_class = torch.empty((B, self.MT, self.NT), dtype=torch.uint8, **e)
        # uint32 bit words, held as int32 (same bits)
        self.sub_class = torch.empty((B, self.MT, self.NT), dtype=torch.int32, **e)
        self.q_nnz = torch.empty((B, self.MT), dtype=torch.int32, **e)
        self.q_list = torch.empty((B, self.MT, self.NT), dtype=torch.int32, **e)
        self.k_nnz = torch.empty((B, self.NT), dtype=torch.int32, **e)
        self.k_list = torch.empty((B, self.NT, self.MT), dtype=torch.int32, **e)

    def c_struct(self) -> OprLayout:
        return OprLayout(*[getattr(self, f).data_ptr() for f in self.FIELDS], self.order)

    def numpy(self) -> Dict[str, np.ndarray]:
        out = {f: getattr(self, f).cpu().numpy() for f in self.FIELDS}
        out["sub_class"] = out["sub_class"].view(np.uint32)
        return out


def pinned_lists(rows: Sequence):
    """The host lists of opr_build_layout (convs per row, turns per
    conversation, turns) in page-locked memory, which the layout's first kernel
    reads in place (no copy on the stream).  Build once, pass as ``lists``."""
    cpr, tpc, turns = inputs.flatten_rows(rows)
    return tuple(torch.from_numpy(np.ascontiguousarray(x if len(x) else np.zeros(1, np.int32),
                                                       dtype=np.int32)).pin_memory()
                 for x in (cpr, tpc, turns)) + (len(tpc), len(turns))


def opr_build_layout(rows: Sequence, L: int, block_q: int = OPR_ATTN_BLOCK,
                     block_k: int = OPR_ATTN_BLOCK, device="cuda",
                     workspace: Optional[torch.Tensor] = None, out: Optional[Layout] = None,
                     order: int = OPR_ORDER_ATTENTION, lists=None) -> Layout:
    """rows: list of rows, each a list of conversations of (h, t, r_in, r_out)
    turns.  ``out``: a Layout of the same (B, L, block_q, block_k, order) to
    refill.  ``order``: OPR_ORDER_ATTENTION (what the attention calls need) or
    OPR_ORDER_PACKED (the tile schedule over the packed rows).  ``lists``: the
    rows' host lists from pinned_lists(rows), else they are flattened into
    pageable arrays here (copied with hipMemcpyAsync)."""
    device = torch.device(device)
    B = len(rows)
    if lists is not None:
        C, T = lists[3], lists[4]
    else:
        cpr, tpc, turns = inputs.flatten_rows(rows)
        C, T = len(tpc), len(turns)
    if out is not None and (out.B, out.L, out.block_q, out.block_k, out.order) == (B, L, block_q, block_k, order):
        lay = out
    else:
        lay = Layout(B, L, block_q, block_k, device, order)
    need = opr_build_layout_workspace_size(B, L, C, T)
    if need == 0:
        raise OprError(OPR_E_INVALID, "opr_build_layout_workspace_size")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if lists is not None:
        p_cpr, p_tpc, p_turns = (x.data_ptr() for x in lists[:3])
    else:
        cpr = np.ascontiguousarray(cpr, dtype=np.int32)
        tpc = np.ascontiguousarray(tpc if C else np.zeros(1, np.int32), dtype=np.int32)
        turns = np.ascontiguousarray(turns if T else np.zeros((1, 4), np.int32), dtype=np.int32)
        p_cpr, p_tpc, p_turns = cpr.ctypes.data, tpc.ctypes.data, turns.ctypes.data
    cs = lay.c_struct()
    st = LIB.opr_build_layout(B, L, block_q, block_k, p_cpr, p_tpc, p_turns, workspace.data_ptr(),
                              workspace.numel(), ctypes.byref(cs), _stream(device))
    _check(st, "opr_build_layout")
    return lay


OPR_LAYOUT_SCRATCH_BYTES = 32 << 20


def opr_build_layout_noalloc(rows: Sequence, L: int, block_q: int = OPR_ATTN_BLOCK,
                             block_k: int = OPR_ATTN_BLOCK, device="cuda", out: Optional[Layout] = None,
                             order: int = OPR_ORDER_ATTENTION) -> Layout:
    """opr_build_layout without a workspace: the library's fixed device
    scratch (OPR_LAYOUT_SCRATCH_BYTES per GPU) is used instead.  Calls that
    overlap on one GPU race on that scratch."""
    device = torch.device(device)
    B = len(rows)
    cpr, tpc, turns = inputs.flatten_rows(rows)
    C, T = len(tpc), len(turns)
    if out is not None and (out.B, out.L, out.block_q, out.block_k, out.order) == (B, L, block_q, block_k, order):
        lay = out
    else:
        lay = Layout(B, L, block_q, block_k, device, order)
    cpr = np.ascontiguousarray(cpr, dtype=np.int32)
    tpc = np.ascontiguousarray(tpc if C else np.zeros(1, np.int32), dtype=np.int32)
    turns = np.ascontiguousarray(turns if T else np.zeros((1, 4), np.int32), dtype=np.int32)
    cs = lay.c_struct()
    st = LIB.opr_build_layout_noalloc(B, L, block_q, block_k, cpr.ctypes.data, tpc.ctypes.data,
                                      turns.ctypes.data, ctypes.byref(cs), _stream(device))
    _check(st, "opr_build_layout_noalloc")
    return lay


def _attn_in(q, k, v, lay: Layout, theta: float, scale: float, events=None, reuse=False) -> OprAttnIn:
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    for name, t, H in (("q", q, Hq), ("k", k, Hkv), ("v", v, Hkv)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or tuple(t.shape) != (B, L, H, D):
            raise ValueError(f"{name} must be contiguous bfloat16 [B, L, H, D]")
    if (lay.B, lay.L) != (B, L):
        raise ValueError("layout built for a different B or L")
    return OprAttnIn(B, L, Hq, Hkv, D, float(scale), float(theta), q.data_ptr(), k.data_ptr(),
                     v.data_ptr(), lay.c_struct(), lay.block_q, lay.block_k,
                     None if events is None else ctypes.addressof(events), 1 if reuse else 0)


def opr_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lay: Layout,
                 theta: float = 1.0e6, scale: float = 0.0,
                 workspace: Optional[torch.Tensor] = None, out=None, events=None):
    """Returns (o bf16 [B, L, Hq, D], lse fp32 [B, Hq, L]).  ``events``: optional
    ctypes array of 3 hipEvent_t handles recorded around the stages."""
    a = _attn_in(q, k, v, lay, theta, scale, events)
    B, L, Hq, D = q.shape
    need = opr_attn_workspace_size(B, L, Hq, k.shape[2], D, False)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
    st = LIB.opr_attn_fwd(ctypes.byref(a), o.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                          workspace.numel(), _stream(q.device))
    _check(st, "opr_attn_fwd")
    return o, lse


def opr_attn_bwd(q, k, v, o, lse, dout, lay: Layout, theta: float = 1.0e6, scale: float = 0.0,
                 workspace: Optional[torch.Tensor] = None, out=None, events=None,
                 reuse_fwd_workspace: bool = False):
    """Returns (dq, dk, dv) fp32 with the shapes of q, k, v.  ``events``:
    optional ctypes array of 4 hipEvent_t handles recorded around the stages.
    ``reuse_fwd_workspace``: ``workspace`` is the one the matching
    opr_attn_fwd call just used (its forward state is reused)."""
    if reuse_fwd_workspace and workspace is None:
        raise ValueError("reuse_fwd_workspace needs the forward's workspace")
    a = _attn_in(q, k, v, lay, theta, scale, events, reuse_fwd_workspace)
    B, L, Hq, D = q.shape
    if dout.dtype != torch.bfloat16 or not dout.is_contiguous() or dout.shape != q.shape:
        raise ValueError("dout must be contiguous bfloat16 shaped like q")
    need = opr_attn_workspace_size(B, L, Hq, k.shape[2], D, True)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
        dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    else:
        dq, dk, dv = out
    st = LIB.opr_attn_bwd(ctypes.byref(a), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                          workspace.numel(), _stream(q.device))
    _check(st, "opr_attn_bwd")
    return dq, dk, dv


def opr_token_ce_workspace_size(B: int, L: int, F: int, V: int) -> int:
    return int(LIB.opr_token_ce_workspace_size(B, L, F, V))


def opr_token_ce(o: torch.Tensor, w: torch.Tensor, labels: torch.Tensor, lay: Layout,
                 grad_scale: float = 1.0, with_grad: bool = True,
                 workspace: Optional[torch.Tensor] = None, out=None):
    """Per-token loss of the head w (bf16 [V, F]) on o (bf16 [B, L, Hq, D] or
    [B, L, F]) at int32 labels [B, L]; scored rows are the layout's t and
    r_out tokens.  Returns (loss fp32 [B, L], dout bf16 shaped like o, or None
    without the gradient)."""
    B, L = o.shape[0], o.shape[1]
    F = o[0, 0].numel()
    V = w.shape[0]
    if o.dtype != torch.bfloat16 or not o.is_contiguous():
        raise ValueError("o must be contiguous bfloat16")
    if w.dtype != torch.bfloat16 or not w.is_contiguous() or w.dim() != 2 or w.shape[1] != F:
        raise ValueError("w must be contiguous bfloat16 [V, F]")
    if labels.dtype != torch.int32 or not labels.is_contiguous() or tuple(labels.shape) != (B, L):
        raise ValueError("labels must be contiguous int32 [B, L]")
    if (lay.B, lay.L) != (B, L):
        raise ValueError("layout and o disagree on B, L")
    if out is None:
        loss = torch.empty((B, L), dtype=torch.float32, device=o.device)
        dout = torch.empty_like(o) if with_grad else None
    else:
        loss, dout = out
    ws_ptr, ws_n = None, 0
    if dout is not None:
        need = opr_token_ce_workspace_size(B, L, F, V)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=o.device)
        ws_ptr, ws_n = workspace.data_ptr(), workspace.numel()
    st = LIB.opr_token_ce(B, L, F, V, o.data_ptr(), w.data_ptr(), labels.data_ptr(),
                          lay.tok_type.data_ptr(), float(grad_scale), loss.data_ptr(),
                          None if dout is None else dout.data_ptr(), ws_ptr, ws_n, _stream(o.device))
    _check(st, "opr_token_ce")
    return loss, dout


# ----------------------------------------------------------------------------
# attention block
# ----------------------------------------------------------------------------
def opr_block_workspace_size(B: int, L: int, Hq: int, Hkv: int, D: int, d_model: int, is_bwd: bool) -> int:
    return int(LIB.opr_block_workspace_size(B, L, Hq, Hkv, D, d_model, 1 if is_bwd else 0))


class BlockWeights:
    """Weights of one attention block: w_qkv bf16 [(Hq + 2 Hkv) D, d_model],
    w_o bf16 [d_model, Hq D], g_q and g_k fp32 [D]."""

    def __init__(self, w_qkv, w_o, g_q, g_k, Hq: int, Hkv: int, D: int):
        self.w_qkv, self.w_o, self.g_q, self.g_k = w_qkv, w_o, g_q, g_k
        self.Hq, self.Hkv, self.D = Hq, Hkv, D
        self.d_model = w_qkv.shape[1]
        if tuple(w_qkv.shape) != ((Hq + 2 * Hkv) * D, self.d_model) or tuple(w_o.shape) != (self.d_model, Hq * D):
            raise ValueError("w_qkv must be [(Hq + 2 Hkv) D, d_model] and w_o [d_model, Hq D]")
        for name, t in (("w_qkv", w_qkv), ("w_o", w_o)):
            if t.dtype != torch.bfloat16 or not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous bfloat16")
        for name, t in (("g_q", g_q), ("g_k", g_k)):
            if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (D,):
                raise ValueError(f"{name} must be contiguous float32 [D]")


def _block_in(x, wts: BlockWeights, lay: Layout, theta, scale, eps, events, reuse=False) -> OprBlockIn:
    B, L, d = x.shape
    if x.dtype != torch.bfloat16 or not x.is_contiguous() or d != wts.d_model:
        raise ValueError("x must be contiguous bfloat16 [B, L, d_model]")
    if (lay.B, lay.L) != (B, L):
        raise ValueError("layout built for a different B or L")
    return OprBlockIn(B, L, wts.Hq, wts.Hkv, wts.D, d, float(scale), float(theta), float(eps),
                      x.data_ptr(), wts.w_qkv.data_ptr(), wts.w_o.data_ptr(), wts.g_q.data_ptr(),
                      wts.g_k.data_ptr(), lay.c_struct(), lay.block_q, lay.block_k,
                      None if events is None else ctypes.addressof(events), 1 if reuse else 0)


def opr_block_fwd(x, wts: BlockWeights, lay: Layout, theta: float = 1.0e6, scale: float = 0.0,
                  eps: float = 1.0e-6, workspace: Optional[torch.Tensor] = None, out=None, events=None):
    """Returns (y bf16 [B, L, d_model], qkv bf16 [B, L, (Hq + 2 Hkv) D],
    o bf16 [B, L, Hq, D], lse fp32 [B, Hq, L]); qkv, o and lse feed
    opr_block_bwd.  ``events``: optional ctypes array of 5 hipEvent_t."""
    a = _block_in(x, wts, lay, theta, scale, eps, events)
    B, L, d = x.shape
    need = opr_block_workspace_size(B, L, wts.Hq, wts.Hkv, wts.D, d, False)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    if out is None:
        e = dict(device=x.device)
        y = torch.empty((B, L, d), dtype=torch.bfloat16, **e)
        qkv = torch.empty((B, L, (wts.Hq + 2 * wts.Hkv) * wts.D), dtype=torch.bfloat16, **e)
        o = torch.empty((B, L, wts.Hq, wts.D), dtype=torch.bfloat16, **e)
        lse = torch.empty((B, wts.Hq, L), dtype=torch.float32, **e)
    else:
        y, qkv, o, lse = out
    st = LIB.opr_block_fwd(ctypes.byref(a), y.data_ptr(), qkv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           workspace.data_ptr(), workspace.numel(), _stream(x.device))
    _check(st, "opr_block_fwd")
    return y, qkv, o, lse


def opr_block_bwd(x, wts: BlockWeights, lay: Layout, qkv, o, lse, dy, theta: float = 1.0e6, scale: float = 0.0,
                  eps: float = 1.0e-6, workspace: Optional[torch.Tensor] = None, out=None, events=None,
                  reuse_fwd_workspace: bool = False):
    """Returns (dx bf16 like x, dw_qkv fp32 like w_qkv, dw_o fp32 like w_o,
    dg_q fp32 [D], dg_k fp32 [D]).  ``events``: optional ctypes array of 6.
    ``reuse_fwd_workspace``: ``workspace`` is the one the matching
    opr_block_fwd call just used (its normalised q, k, v and attention state
    are reused)."""
    if reuse_fwd_workspace and workspace is None:
        raise ValueError("reuse_fwd_workspace needs the forward's workspace")
    a = _block_in(x, wts, lay, theta, scale, eps, events, reuse_fwd_workspace)
    B, L, d = x.shape
    if dy.dtype != torch.bfloat16 or not dy.is_contiguous() or dy.shape != x.shape:
        raise ValueError("dy must be contiguous bfloat16 shaped like x")
    need = opr_block_workspace_size(B, L, wts.Hq, wts.Hkv, wts.D, d, True)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    if out is None:
        e = dict(device=x.device)
        dx = torch.empty_like(x)
        dw_qkv = torch.empty(wts.w_qkv.shape, dtype=torch.float32, **e)
        dw_o = torch.empty(wts.w_o.shape, dtype=torch.float32, **e)
        dg_q = torch.empty((wts.D,), dtype=torch.float32, **e)
        dg_k = torch.empty((wts.D,), dtype=torch.float32, **e)
    else:
        dx, dw_qkv, dw_o, dg_q, dg_k = out
    st = LIB.opr_block_bwd(ctypes.byref(a), qkv.data_ptr(), o.data_ptr(), lse.data_ptr(), dy.data_ptr(),
                           dx.data_ptr(), dw_qkv.data_ptr(), dw_o.data_ptr(), dg_q.data_ptr(), dg_k.data_ptr(),
                           workspace.data_ptr(), workspace.numel(), _stream(x.device))
    _check(st, "opr_block_bwd")
    return dx, dw_qkv, dw_o, dg_q, dg_k
