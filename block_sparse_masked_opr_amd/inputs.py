"""Seeded synthetic inputs: conversation shapes, packed rows and tensors.

This module is shared by the HIP path's tests/bench and by the oracle's tests.
It holds no attention, mask or position arithmetic and none of the method's
sequence rules (the N-pass and K-pass turn lists are in ``sequences.py``): it
only draws segment lengths, groups conversations into rows, and draws random
tensors.  Every
consumer (the oracle, the C ABI) derives tokens, positions and masks from the
turn lists itself.

A *turn* is a 4-tuple of segment lengths ``(h, t, r_in, r_out)``: the human
message, the reasoning, the context copy of the response and the generation
copy of the response (One-Pass to Reason, "Token duplication").  In an
ordinary turn ``r_in == r_out == r`` because the response is stored twice.
A *conversation* is a list of turns; a *row* is a list of conversations packed
back to back into a sequence of ``L`` tokens (One-Pass to Reason,
implementation notes: packing with the custom mask).

The workloads mirror the pages' experiments with synthetic lengths in place of
the MathChatSync-reasoning dataset, which is not available here:

* ``tiny``    - 1 conversation, 2 turns of (h, t, r) = (8, 12, 6): 64 packed tokens.
* ``packed_fwd`` - 1 row x 8192, N~U[2,6], h~U[16,128], t~U[64,512], r~U[32,256].
* ``packed_fwd_bwd`` - 2 rows x 16384, same distributions.
* ``depth``   - one conversation of N turns (h, t, r) = (128, 1024, 256).
* ``kpass``   - conversations with N~U[4,12], h~U[32,256], t~U[256,2048],
  r~U[64,512] that fill 4 rows of 32768 tokens at K = 1 (the K-pass chunk
  sequences built from them are in ``sequences.py``).
* ``layout_batch`` - 64 rows x 32768 with the packed distributions (layout only).

Lengths use ``numpy.random.Generator(PCG64(seed))``; ``U[a, b]`` is inclusive.
Tensors are float32 ``standard_normal`` drawn in the order Q, K, V, dO, each
``[B, L, H, D]``, then rounded once to bfloat16 (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

Turn = Tuple[int, int, int, int]
Conversation = List[Turn]
Row = List[Conversation]


# ----------------------------------------------------------------------------
# workload shapes
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Shape:
    """Attention shape of a workload: rows, row length, heads and head dim."""
    name: str
    B: int
    L: int
    Hq: int
    Hkv: int
    D: int
    theta: float = 1.0e6


TINY = Shape("tiny", 1, 64, 1, 1, 64)
PACKED_FWD = Shape("packed_fwd", 1, 8192, 32, 8, 128)
PACKED_FWD_BWD = Shape("packed_fwd_bwd", 2, 16384, 32, 8, 128)
KPASS_ROW_LEN = 32768
DEPTH_HEADS = dict(Hq=64, Hkv=8, D=128)
KPASS_HEADS = dict(Hq=32, Hkv=8, D=128)

SEEDS = {
    "tiny": (None, 0),
    "packed_fwd": (101, 102),
    "packed_fwd_bwd": (201, 202),
    "depth": (None, 301),
    "kpass": (401, 402),
    "layout_batch": (501, None),
}

# the layout alone on a large batch: 64 rows of 32768 tokens, packed
# distributions (the attention workloads are too small to load the HBM)
LAYOUT_BATCH = (64, 32768)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _u(rng: np.random.Generator, lo: int, hi: int) -> int:
    """One draw from the inclusive integer range [lo, hi]."""
    return int(rng.integers(lo, hi + 1))


# ----------------------------------------------------------------------------
# conversations and rows
# ----------------------------------------------------------------------------
def sample_conversation(rng, n_rng, h_rng, t_rng, r_rng) -> Conversation:
    """N turns; each response r is stored twice (r_in = r_out = r)."""
    n = _u(rng, *n_rng)
    conv = []
    for _ in range(n):
        h = _u(rng, *h_rng)
        t = _u(rng, *t_rng)
        r = _u(rng, *r_rng)
        conv.append((h, t, r, r))
    return conv


def conv_len(conv: Conversation) -> int:
    """Packed tokens of a conversation (every stored segment counted)."""
    return int(sum(sum(turn) for turn in conv))


def conv_logical_tokens(conv: Conversation) -> int:
    """Conversation tokens h + t + r per turn, the response counted once."""
    return int(sum(h + t + max(r_in, r_out) for (h, t, r_in, r_out) in conv))


def pack_greedy(rng, B: int, L: int, sampler, max_misses: int = 16) -> List[Row]:
    """Fill B rows of L tokens: append sampled conversations while they fit;
    after ``max_misses`` consecutive draws that do not fit, the rest is PAD."""
    rows = []
    for _ in range(B):
        row, used, misses = [], 0, 0
        while misses < max_misses:
            conv = sampler(rng)
            n = conv_len(conv)
            if used + n <= L:
                row.append(conv)
                used += n
                misses = 0
            else:
                misses += 1
        rows.append(row)
    return rows


def pack_first_fit_decreasing(convs: Sequence[Conversation], L: int) -> List[Row]:
    """Pack conversations into as few rows of L tokens as first-fit-decreasing finds."""
    order = sorted(range(len(convs)), key=lambda i: -conv_len(convs[i]))
    rows: List[Row] = []
    used: List[int] = []
    for i in order:
        n = conv_len(convs[i])
        if n > L:
            raise ValueError(f"conversation of {n} tokens does not fit a row of {L}")
        for j in range(len(rows)):
            if used[j] + n <= L:
                rows[j].append(convs[i])
                used[j] += n
                break
        else:
            rows.append([convs[i]])
            used.append(n)
    return rows


def row_used(row: Row) -> int:
    return int(sum(conv_len(c) for c in row))


def tiny_rows() -> List[Row]:
    """One conversation of two turns, (h, t, r) = (8, 12, 6) each: 64 tokens."""
    return [[[(8, 12, 6, 6), (8, 12, 6, 6)]]]


def _packed_sampler(rng):
    return sample_conversation(rng, (2, 6), (16, 128), (64, 512), (32, 256))


def packed_rows(shape: Shape, seed: int) -> List[Row]:
    """Rows for the packed workloads (N~U[2,6], h~U[16,128], t~U[64,512], r~U[32,256])."""
    return pack_greedy(_rng(seed), shape.B, shape.L, _packed_sampler)


def layout_batch_rows(seed: int = 501) -> List[Row]:
    """64 rows of 32768 tokens (N~U[2,6], h~U[16,128], t~U[64,512], r~U[32,256])."""
    B, L = LAYOUT_BATCH
    return pack_greedy(_rng(seed), B, L, _packed_sampler)


def depth_conversation(N: int, h: int = 128, t: int = 1024, r: int = 256) -> Conversation:
    return [(h, t, r, r) for _ in range(N)]


def _kpass_sampler(rng):
    return sample_conversation(rng, (4, 12), (32, 256), (256, 2048), (64, 512))


def kpass_base_conversations(seed: int = 401, rows: int = 4, L: int = KPASS_ROW_LEN):
    """A fixed set of conversations that fills ``rows`` rows of L at K=1.

    Conversations longer than L are redrawn."""
    rng = _rng(seed)

    def sampler(r):
        while True:
            c = _kpass_sampler(r)
            if conv_len(c) <= L:
                return c

    packed = pack_greedy(rng, rows, L, sampler)
    return [c for row in packed for c in row]


# ----------------------------------------------------------------------------
# flattening for the C ABI: convs_per_row, turns_per_conv, turns
# ----------------------------------------------------------------------------
def flatten_rows(rows: Sequence[Row]):
    """Return int32 arrays (convs_per_row [B], turns_per_conv [C], turns [T, 4])."""
    cpr = np.array([len(r) for r in rows], dtype=np.int32)
    tpc = np.array([len(c) for r in rows for c in r], dtype=np.int32)
    turns = np.array([t for r in rows for c in r for t in c], dtype=np.int32).reshape(-1, 4)
    return cpr, tpc, turns


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------
def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def make_tensors(B, L, Hq, Hkv, D, seed, with_dout=True):
    """Q, K, V (and dO) as bfloat16 bit patterns, [B, L, H, D] each."""
    rng = _rng(seed)
    out = {}
    for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv), ("do", Hq)):
        if name == "do" and not with_dout:
            break
        x = rng.standard_normal((B, L, H, D), dtype=np.float32)
        out[name] = round_to_bf16_bits(x)
    return out


# ----------------------------------------------------------------------------
# attention block: weights and activations
# ----------------------------------------------------------------------------
# hidden sizes of the Qwen-3 models with these head counts (32 q / 8 kv heads:
# 4096; 64 q / 8 kv heads: 5120)
BLOCK_D_MODEL = {32: 4096, 64: 5120}


def make_block_weights(d_model: int, Hq: int, Hkv: int, D: int, seed: int):
    """w_qkv [(Hq + 2 Hkv) D, d_model] ~ N(0, 1/d_model) and w_o [d_model, Hq D]
    ~ N(0, 1/(Hq D)) as bfloat16 bit patterns (unit-variance projections of
    unit-variance rows); g_q, g_k ~ U[0.5, 1.5] float32 [D]."""
    rng = _rng(seed)
    w_qkv = rng.standard_normal(((Hq + 2 * Hkv) * D, d_model), dtype=np.float32) / np.float32(np.sqrt(d_model))
    w_o = rng.standard_normal((d_model, Hq * D), dtype=np.float32) / np.float32(np.sqrt(Hq * D))
    g_q = rng.uniform(0.5, 1.5, size=D).astype(np.float32)
    g_k = rng.uniform(0.5, 1.5, size=D).astype(np.float32)
    return {"w_qkv": round_to_bf16_bits(w_qkv), "w_o": round_to_bf16_bits(w_o), "g_q": g_q, "g_k": g_k}


def make_block_tensors(B: int, L: int, d_model: int, seed: int):
    """x and dy ~ N(0, 1), [B, L, d_model], as bfloat16 bit patterns."""
    rng = _rng(seed)
    return {n: round_to_bf16_bits(rng.standard_normal((B, L, d_model), dtype=np.float32)) for n in ("x", "dy")}
