"""Writes tests/golden/sampled_parity.npz: the oracle's dK and dV at sampled
keys of the two full-size backward workloads that are too large for the whole
oracle, for the GPU parity test tests/test_gpu_sampled_parity.py.

    python tests/golden/make_sampled_parity.py [--procs N]

Calls only the oracle (oracle/opr_oracle.py: layout, attention_order,
attn_cols) and the seeded input generators (block_sparse_masked_opr_amd/inputs.py,
which hold no attention arithmetic).  Each kv group's keys are computed from
the definition: every query row that sees a listed key is computed whole.

Workloads (wiki summary, section 实验结果: depth scaling and the K-pass):
* depth N = 32: one conversation of 32 turns (h, t, r) = (128, 1024, 256),
  53,248 packed tokens, 64 q / 8 kv heads, D = 128, tensor seed of the depth
  sweep.  Its early history key tiles are seen by every later turn, so the
  backward cuts their columns into parts.
* K-pass K = 1: row 0 of the 32768-token rows, 32 q / 8 kv heads, D = 128,
  tensor seed of the K-pass sweep.
Keys are picked in attention order (slots): the first and last slots of the
first tiles, tile boundaries, the end of the history and the start and end of
the reasoning / generation-copy region, and seeded random slots.  The file
also holds a fingerprint of the inputs, so that a change of the generators
shows up as a failed check rather than as a parity error.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from block_sparse_masked_opr_amd import inputs as I  # noqa: E402
from oracle import opr_oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sampled_parity.npz")
THETA = 1.0e6


def workloads():
    """(name, rows, L, Hq, Hkv, D, tensor seed, row b) of each workload."""
    depth = [[I.depth_conversation(32)]]
    # K = 1: every conversation is its own sequence, packed first-fit decreasing
    kp = I.pack_first_fit_decreasing(I.kpass_base_conversations(I.SEEDS["kpass"][0]), I.KPASS_ROW_LEN)[:1]
    return [
        ("depth32", depth, I.row_used(depth[0]), I.DEPTH_HEADS["Hq"], I.DEPTH_HEADS["Hkv"], I.DEPTH_HEADS["D"],
         I.SEEDS["depth"][1]),
        ("kpass1", kp, I.KPASS_ROW_LEN, I.KPASS_HEADS["Hq"], I.KPASS_HEADS["Hkv"], I.KPASS_HEADS["D"],
         I.SEEDS["kpass"][1]),
    ]


def key_slots(lay, L, seed):
    """Sampled key slots (attention order) of row 0: tile edges, the history's
    end, the tail's start and end, and random slots; live tokens only."""
    live = int((lay["type"][0] != O.PAD).sum())
    n1 = int(np.isin(lay["type"][0], (O.H, O.RIN)).sum())    # history slots come first
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 1023, 1024, n1 - 1, n1, n1 + 1, live - 1]
    rng = np.random.default_rng(seed)
    rand = rng.integers(0, live, size=16).tolist()
    return np.array(sorted(set(x for x in fixed + rand if 0 <= x < live)), dtype=np.int64)


def fingerprint(t):
    """Sums of the inputs' float values (bf16 bits -> float64) per tensor."""
    return np.array([float(I.bf16_bits_to_f32(t[n]).astype(np.float64).sum()) for n in ("q", "k", "v", "do")])


def group_cols(args):
    q, k, v, do, lay, cols = args
    return O.attn_cols(q, k, v, do, lay, 0, cols, THETA)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=os.cpu_count() or 1)
    a = ap.parse_args()
    out = {}
    for name, rows, L, Hq, Hkv, D, seed in workloads():
        t0 = time.time()
        lay = O.layout(rows, L)
        slot = O.attention_order(lay, 0)                       # slot of each token
        tok_of_slot = np.argsort(slot)
        slots = key_slots(lay, L, seed)
        cols = tok_of_slot[slots]                              # token index of each sampled slot
        t = I.make_tensors(1, L, Hq, Hkv, D, seed=seed)
        f = {n: I.bf16_bits_to_f32(t[n]).astype(np.float64) for n in t}
        g = Hq // Hkv
        jobs = [(f["q"][:, :, kv * g:(kv + 1) * g], f["k"][:, :, kv:kv + 1], f["v"][:, :, kv:kv + 1],
                 f["do"][:, :, kv * g:(kv + 1) * g], lay, cols) for kv in range(Hkv)]
        with cf.ProcessPoolExecutor(max_workers=min(a.procs, Hkv)) as ex:
            res = list(ex.map(group_cols, jobs))
        dk = np.concatenate([r[0] for r in res], axis=1)       # [n, Hkv, D]
        dv = np.concatenate([r[1] for r in res], axis=1)
        out[f"{name}_cols"] = cols
        out[f"{name}_slots"] = slots
        out[f"{name}_dk"] = dk.astype(np.float32)
        out[f"{name}_dv"] = dv.astype(np.float32)
        out[f"{name}_fingerprint"] = fingerprint(t)
        print(f"{name}: {len(cols)} keys, {time.time() - t0:.1f} s", flush=True)
    np.savez_compressed(OUT, **out)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
