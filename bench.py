#!/usr/bin/env python3
"""Benchmark of one-pass block-sparse masked attention on one MI355X.

A step is one pass of the whole path over one batch: opr_build_layout (tokens,
position ids, tile schedule) + opr_attn_fwd + opr_attn_bwd, on the packed
fwd+bwd workload: 2 rows x 16384 tokens of packed multi-turn conversations
(N~U[2,6] turns, h~U[16,128], t~U[64,512], r~U[32,256], responses duplicated),
32 q heads over 8 kv heads, head dim 128, RoPE theta 1e6; seeded synthetic
bf16 inputs already resident in HBM.

Prints one JSON line: useful TFLOP/s (12 * D * Hq * P, P = allowed query-key
pairs, recomputation not counted), conversation tokens/s, the roofline of the
dominant kernel (timed with HIP events on its own stream), the fp64 CPU oracle
timed on a bounded sample, and (unless --no-sweep) the one-pass vs N-pass
speedup across conversation depth and the K-pass trade-off.  Beside the
headline it also times the per-token loss step, the layout alone on 64 rows
of 32768 tokens, and (unless --no-block) the
same rows through a whole attention block (projections, q/k norms, attention;
opr_block_fwd / opr_block_bwd), and the block's one-pass vs N-pass speedup.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from block_sparse_masked_opr_amd import inputs as I  # noqa: E402  (no torch, no GPU)
from block_sparse_masked_opr_amd import sequences as S  # noqa: E402

PEAK_FP16_TFLOPS = 2500.0     # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0

CSRC = os.path.join(ROOT, "block_sparse_masked_opr_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# sources compiled into each attention kernel (a change voids its counters)
KERNEL_SOURCES = {
    "attn_fwd": ("attn_fwd.hip", "attn_common.h", "attn_sched.h"),
    "attn_dkdv": ("attn_bwd.hip", "attn_common.h", "attn_sched.h"),
    "attn_dq": ("attn_dq.hip", "attn_common.h", "attn_sched.h"),
    "layout": ("layout.hip", "opr_internal.h"),
}
# the workload each traffic summary is taken on, and its file under profiles/
TRAFFIC_WORKLOAD = {"attn_dkdv": "packed_fwd_bwd", "layout": "layout_batch"}
TRAFFIC_FILE = {"attn_dkdv": "attn_dkdv_packed_fwd_bwd_traffic.json", "layout": "layout_batch_traffic.json"}
COPY_PROBE_BYTES = 1 << 30    # bytes read (and written) per copy-probe dispatch


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(kernel):
    return os.path.join(PROFILES, TRAFFIC_FILE[kernel])


def load_traffic(kernel):
    """HBM bytes per launch of `kernel` from its committed counter summary,
    or None if there is none or the kernel's sources changed since."""
    try:
        with open(traffic_file(kernel)) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha") != source_hash(kernel):
        return None
    return d.get("bytes_per_launch")


def copy_probe(steps=5):
    """A plain device copy of COPY_PROBE_BYTES, to calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    # bytes read + bytes written: the practical HBM rate of a plain copy
    log(f"copy probe: {steps} copies of {COPY_PROBE_BYTES} bytes, {ms:.3f} ms each, "
        f"{2 * COPY_PROBE_BYTES / (ms * 1e-3) / 1e9:.0f} GB/s read + write")


def summarize_traffic(run_dir, kernel):
    """Write profiles/<kernel>_<workload>_traffic.json from four rocprofv3
    --pmc runs under run_dir: fetch/ and write/ of the benchmark (FETCH_SIZE,
    WRITE_SIZE) and copy_fetch/ and copy_write/ of --copy-probe.  Counters are
    KiB per dispatch; each is scaled by (probe bytes) / (probe counter).  For
    "layout" a launch is one opr_build_layout call: the per-dispatch averages
    of its kernels are summed."""
    import collections
    import csv
    import glob

    def per_dispatch(sub, counter, match):
        vals = collections.defaultdict(list)
        for f in glob.glob(os.path.join(run_dir, sub, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] == counter and match(row["Kernel_Name"]):
                    vals[row["Kernel_Name"]].append(float(row["Counter_Value"]))
        if not vals:
            raise SystemExit(f"no {counter} rows in {sub}")
        return sum(sum(v) / len(v) for v in vals.values())

    if kernel == "layout":
        is_kernel = lambda name: "::layout_" in name                              # noqa: E731
    else:
        is_kernel = lambda name: (kernel + "_kernel") in name                     # noqa: E731
    # the probe's copy kernel only (not the fill that initialises its source)
    is_copy = lambda name: "copy" in name.lower() and "fill" not in name.lower()  # noqa: E731
    fetch = per_dispatch("fetch", "FETCH_SIZE", is_kernel)
    write = per_dispatch("write", "WRITE_SIZE", is_kernel)
    cf = COPY_PROBE_BYTES / per_dispatch("copy_fetch", "FETCH_SIZE", is_copy)
    cw = COPY_PROBE_BYTES / per_dispatch("copy_write", "WRITE_SIZE", is_copy)
    d = {"kernel": kernel, "workload": TRAFFIC_WORKLOAD[kernel], "source_sha": source_hash(kernel),
         "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
         "copy_probe_bytes": COPY_PROBE_BYTES, "fetch_bytes_per_kib": cf, "write_bytes_per_kib": cw,
         "bytes_per_launch": round(fetch * cf + write * cw)}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(kernel), "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps(d))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self, torch):
        libdir = os.path.join(os.path.dirname(torch.__file__), "lib")
        path = os.path.join(libdir, "libamdhip64.so")
        self.hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def array(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = h
        return arr

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def free(self, arr):
        for h in arr:
            self.hip.hipEventDestroy(h)


def useful_pairs(torch, lay):
    """P = sum over non-PAD tokens of (pos + 1): every query sees positions 0..pos."""
    live = lay.tok_type != 4
    return int(((lay.tok_pos.to(torch.int64) + 1) * live).sum().item())


def device_inputs(torch, B, L, Hq, Hkv, D, seed, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    out = {}
    for n, H in (("q", Hq), ("k", Hkv), ("v", Hkv), ("do", Hq)):
        out[n] = torch.randn((B, L, H, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    return out


class Runner:
    """Buffers and calls for one workload; step() = layout + fwd + bwd."""

    def __init__(self, torch, Bd, rows, L, Hq, Hkv, D, t, dev, theta=1.0e6):
        self.torch, self.Bd, self.rows, self.L, self.theta = torch, Bd, rows, L, theta
        B = len(rows)
        self.t = t
        self.lay = Bd.opr_build_layout(rows, L, 128, 128, device=dev)
        # the host lists in pinned memory: the layout reads them in place
        self.lists = Bd.pinned_lists(rows)
        self.lws = torch.empty(Bd.opr_build_layout_workspace_size(B, L, self.lists[3], self.lists[4]),
                               dtype=torch.uint8, device=dev)
        # one workspace: the backward reuses the forward state at its start
        self.ws = torch.empty(Bd.opr_attn_workspace_size(B, L, Hq, Hkv, D, True), dtype=torch.uint8, device=dev)
        self.o = torch.empty_like(t["q"])
        self.lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
        self.dq = torch.empty(t["q"].shape, dtype=torch.float32, device=dev)
        self.dk = torch.empty(t["k"].shape, dtype=torch.float32, device=dev)
        self.dv = torch.empty(t["v"].shape, dtype=torch.float32, device=dev)

    def step(self, ev_f=None, ev_b=None):
        Bd, t = self.Bd, self.t
        Bd.opr_build_layout(self.rows, self.L, 128, 128, device=self.o.device, workspace=self.lws, out=self.lay,
                            lists=self.lists)
        Bd.opr_attn_fwd(t["q"], t["k"], t["v"], self.lay, self.theta, workspace=self.ws,
                        out=(self.o, self.lse), events=ev_f)
        Bd.opr_attn_bwd(t["q"], t["k"], t["v"], self.o, self.lse, t["do"], self.lay, self.theta,
                        workspace=self.ws, out=(self.dq, self.dk, self.dv), events=ev_b,
                        reuse_fwd_workspace=True)

    def fwd_step(self):
        Bd, t = self.Bd, self.t
        Bd.opr_build_layout(self.rows, self.L, 128, 128, device=self.o.device, workspace=self.lws, out=self.lay,
                            lists=self.lists)
        Bd.opr_attn_fwd(t["q"], t["k"], t["v"], self.lay, self.theta, workspace=self.ws, out=(self.o, self.lse))

    def time_steps(self, steps, warmup, fwd_only=False):
        torch = self.torch
        run = self.fwd_step if fwd_only else self.step
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            run()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps


class BlockRunner:
    """The attention block (hipBLASLt projections, per-head RMS norms of q and
    k, the masked attention, output projection) on seeded synthetic weights and
    rows drawn on the device; step() = layout + block fwd + block bwd."""

    FWD = ("qkv_proj", "qk_norm", "attn_fwd", "o_proj")
    BWD = ("o_proj_grad", "qk_norm_recompute", "attn_bwd", "qk_norm_grad", "qkv_proj_grad")

    def __init__(self, torch, Bd, rows, L, Hq, Hkv, D, dm, dev, seed=701, theta=1.0e6):
        self.torch, self.Bd, self.rows, self.L, self.theta = torch, Bd, rows, L, theta
        self.Hq, self.Hkv, self.D, self.dm = Hq, Hkv, D, dm
        B = len(rows)
        g = torch.Generator(device=dev)
        g.manual_seed(seed)

        def rn(shape, s):
            return (torch.randn(shape, generator=g, device=dev) * s).to(torch.bfloat16)

        self.wts = Bd.BlockWeights(rn(((Hq + 2 * Hkv) * D, dm), 1.0 / math.sqrt(dm)),
                                   rn((dm, Hq * D), 1.0 / math.sqrt(Hq * D)),
                                   torch.rand(D, generator=g, device=dev) + 0.5,
                                   torch.rand(D, generator=g, device=dev) + 0.5, Hq, Hkv, D)
        self.x, self.dy = rn((B, L, dm), 1.0), rn((B, L, dm), 1.0)
        self.lay = Bd.opr_build_layout(rows, L, 128, 128, device=dev)
        self.lists = Bd.pinned_lists(rows)
        self.lws = torch.empty(Bd.opr_build_layout_workspace_size(B, L, self.lists[3], self.lists[4]),
                               dtype=torch.uint8, device=dev)
        self.ws = torch.empty(Bd.opr_block_workspace_size(B, L, Hq, Hkv, D, dm, True), dtype=torch.uint8, device=dev)
        e = dict(device=dev)
        self.fwd_out = (torch.empty((B, L, dm), dtype=torch.bfloat16, **e),
                        torch.empty((B, L, (Hq + 2 * Hkv) * D), dtype=torch.bfloat16, **e),
                        torch.empty((B, L, Hq, D), dtype=torch.bfloat16, **e),
                        torch.empty((B, Hq, L), dtype=torch.float32, **e))
        self.bwd_out = (torch.empty_like(self.x), torch.empty(self.wts.w_qkv.shape, dtype=torch.float32, **e),
                        torch.empty(self.wts.w_o.shape, dtype=torch.float32, **e),
                        torch.empty((D,), dtype=torch.float32, **e), torch.empty((D,), dtype=torch.float32, **e))

    def step(self, ev_f=None, ev_b=None):
        Bd = self.Bd
        Bd.opr_build_layout(self.rows, self.L, 128, 128, device=self.x.device, workspace=self.lws, out=self.lay,
                            lists=self.lists)
        y, qkv, o, lse = Bd.opr_block_fwd(self.x, self.wts, self.lay, self.theta, workspace=self.ws,
                                          out=self.fwd_out, events=ev_f)
        Bd.opr_block_bwd(self.x, self.wts, self.lay, qkv, o, lse, self.dy, self.theta, workspace=self.ws,
                         out=self.bwd_out, events=ev_b, reuse_fwd_workspace=True)

    def time_steps(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            self.step()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps

    def stage_ms(self, ev, n):
        """Mean time of each stage over n steps with HIP events (recorded by the library)."""
        out = {k: 0.0 for k in self.FWD + self.BWD}
        f, b = ev.array(5), ev.array(6)
        for _ in range(n):
            self.step(f, b)
            self.torch.cuda.synchronize()
            for i, k in enumerate(self.FWD):
                out[k] += ev.ms(f[i], f[i + 1]) / n
            for i, k in enumerate(self.BWD):
                out[k] += ev.ms(b[i], b[i + 1]) / n
        ev.free(f)
        ev.free(b)
        return out

    def gemm_flops(self):
        T = self.x.shape[0] * self.x.shape[1]
        return 6.0 * T * self.dm * ((self.Hq + 2 * self.Hkv) * self.D + self.Hq * self.D)


def block_step(torch, Bd, dev, rows, shape, steps, warmup):
    """The 2 x 16384 workload through the whole attention block (d_model of
    the Qwen-3 model with these heads), fwd + bwd."""
    dm = I.BLOCK_D_MODEL[shape.Hq]
    r = BlockRunner(torch, Bd, rows, shape.L, shape.Hq, shape.Hkv, shape.D, dm, dev)
    ms = r.time_steps(steps, warmup)
    st = r.stage_ms(HipEvents(torch), 5)
    P = useful_pairs(torch, r.lay)
    gemm_ms = sum(st[k] for k in ("qkv_proj", "o_proj", "o_proj_grad", "qkv_proj_grad"))
    attn_ms = st["attn_fwd"] + st["attn_bwd"]
    conv_tokens = sum(I.conv_logical_tokens(c) for row in rows for c in row)
    out = {"workload": f"packed_fwd_bwd rows through one block, d_model {dm}", "d_model": dm, "ms": round(ms, 4),
           "tokens_per_s": round(conv_tokens / (ms * 1e-3), 1),
           "stages_ms": {k: round(v, 4) for k, v in st.items()},
           "gemm": {"ms": round(gemm_ms, 4), "tflops": round(r.gemm_flops() / (gemm_ms * 1e-3) / 1e12, 1),
                    "frac_of_bf16_peak": round(r.gemm_flops() / (gemm_ms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4)},
           "attention": {"ms": round(attn_ms, 4),
                         "useful_tflops": round(12.0 * shape.D * shape.Hq * P / (attn_ms * 1e-3) / 1e12, 1)}}
    log(f"block step {out}")
    del r
    torch.cuda.empty_cache()
    return out


def block_depth(torch, Bd, dev, Ns, steps):
    """One conversation of N turns through the block: one pass (as packed and
    without the last turn's dead context copy) against N passes."""
    Hq, Hkv, D = I.DEPTH_HEADS["Hq"], I.DEPTH_HEADS["Hkv"], I.DEPTH_HEADS["D"]
    dm = I.BLOCK_D_MODEL[Hq]
    out = []
    for N in Ns:
        conv = I.depth_conversation(N)
        rec = {"N": N, "d_model": dm}
        for kind, rows in (("one_pass", [[conv]]), ("one_pass_elided", [[S.chunk_conversation(conv, 0, N, True)]]),
                           ("n_pass", [S.npass_conversations(conv)])):
            L = I.row_used(rows[0])
            r = BlockRunner(torch, Bd, rows, L, Hq, Hkv, D, dm, dev)
            rec[kind] = {"tokens": L, "ms": round(r.time_steps(steps, 1), 4)}
            del r
            torch.cuda.empty_cache()
        rec["speedup"] = round(rec["n_pass"]["ms"] / rec["one_pass"]["ms"], 3)
        rec["speedup_elided"] = round(rec["n_pass"]["ms"] / rec["one_pass_elided"]["ms"], 3)
        log(f"block depth N={N}: {rec}")
        out.append(rec)
    return out


def packed_fwd_step(torch, Bd, dev, steps, warmup):
    """The packed forward workload (one row of 8192 tokens, 32 q / 8 kv heads,
    D = 128): layout + forward per step, useful FLOPs 4 * D * Hq * P."""
    shape = I.PACKED_FWD
    seed_len, seed_t = I.SEEDS["packed_fwd"]
    rows = I.packed_rows(shape, seed_len)
    t = device_inputs(torch, shape.B, shape.L, shape.Hq, shape.Hkv, shape.D, seed_t, dev)
    r = Runner(torch, Bd, rows, shape.L, shape.Hq, shape.Hkv, shape.D, t, dev, shape.theta)
    P = useful_pairs(torch, r.lay)
    ms = r.time_steps(steps, warmup, fwd_only=True)
    tflops = 4.0 * shape.D * shape.Hq * P / (ms * 1e-3) / 1e12
    conv_tokens = sum(I.conv_logical_tokens(c) for row in rows for c in row)
    out = {"workload": "packed_fwd: 1 row x 8192 tokens, 32 q / 8 kv heads, D=128, layout + fwd per step",
           "useful_pairs": P, "ms": round(ms, 4), "useful_tflops": round(tflops, 2),
           "frac_of_peak": round(tflops / PEAK_FP16_TFLOPS, 4),
           "tokens_per_s": round(conv_tokens / (ms * 1e-3), 1)}
    del r
    torch.cuda.empty_cache()
    return out


def layout_step(torch, Bd, dev, steps):
    """opr_build_layout alone on 64 rows x 32768 tokens (packed distributions):
    bound by HBM; algorithmic bytes = everything the layout writes (per token
    its ids, slots and runs of slots; per tile its classes and list entries).
    The time holds the copies of the host turn lists (from pinned memory) as
    well."""
    B, L = I.LAYOUT_BATCH
    rows = I.layout_batch_rows(I.SEEDS["layout_batch"][0])
    lay = Bd.opr_build_layout(rows, L, 128, 128, device=dev)
    cpr, tpc, turns = I.flatten_rows(rows)
    lws = torch.empty(Bd.opr_build_layout_workspace_size(B, L, len(tpc), len(turns)), dtype=torch.uint8, device=dev)
    st = lay.c_struct()
    # the host turn lists in pinned memory, so that their copies are asynchronous
    host = [torch.from_numpy(np.ascontiguousarray(x)).pin_memory() for x in (cpr, tpc, turns)]
    args = (B, L, 128, 128, host[0].data_ptr(), host[1].data_ptr(), host[2].data_ptr(), lws.data_ptr(), lws.numel(),
            ctypes.byref(st), torch.cuda.current_stream(dev).cuda_stream)

    def call():
        status = Bd.LIB.opr_build_layout(*args)
        if status != 0:
            raise RuntimeError(f"opr_build_layout: {Bd.opr_status_string(status)}")

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        call()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    nbytes = sum(getattr(lay, f).numel() * getattr(lay, f).element_size() for f in Bd.Layout.FIELDS)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"rows": B, "row_tokens": L, "packed_tokens": sum(I.row_used(r) for r in rows), "ms": round(ms, 4),
           "bytes_written": nbytes,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": load_traffic("layout")}}
    log(f"layout step {out}")
    return out


def loss_step(torch, Bd, r, shape, steps, dev):
    """opr_token_ce on the forward's output: per-token loss of a V = 32 head on
    the t and r_out rows and its gradient (the loss step of training); bound
    by HBM: it reads o once and writes dout once (the kernel, then the dout
    GEMM)."""
    B, L, F, V = shape.B, shape.L, shape.Hq * shape.D, 32
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    w = (torch.randn((V, F), generator=g, device=dev) / math.sqrt(F)).to(torch.bfloat16)
    labels = torch.randint(0, V, (B, L), generator=g, device=dev, dtype=torch.int32)
    ws = torch.empty(Bd.opr_token_ce_workspace_size(B, L, F, V), dtype=torch.uint8, device=dev)
    loss = torch.empty((B, L), dtype=torch.float32, device=dev)
    dout = torch.empty_like(r.o)
    for _ in range(3):
        Bd.opr_token_ce(r.o, w, labels, r.lay, 1.0, workspace=ws, out=(loss, dout))
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        Bd.opr_token_ce(r.o, w, labels, r.lay, 1.0, workspace=ws, out=(loss, dout))
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    scored = int(((r.lay.tok_type == 1) | (r.lay.tok_type == 3)).sum().item())
    # algorithmic bytes: o read and dout written (bf16), labels and types read, loss written,
    # the logit gradient g (bf16 [rows][V]) written and read back, W read by both passes
    nbytes = B * L * F * 2 * 2 + B * L * (4 + 1 + 4) + B * L * V * 2 * 2 + V * F * 2 * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "token_ce", "ms": round(ms, 4), "rows": B * L, "scored_rows": scored, "F": F, "V": V,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}}


def cpu_baseline(rows, L, shape, t_np, budget_s=10.0):
    """The fp64 oracle on a bounded sample of the workload: the conversations
    of row 0 in order, each with every q and kv head, fwd + bwd, until about
    budget_s seconds of oracle time have been spent (at least one
    conversation)."""
    from oracle import opr_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    lay = O.layout(rows, L)
    flops, dt, done, toks = 0.0, 0.0, 0, 0
    for c in range(O.n_convs(lay, 0)):
        a, e = O.conv_range(lay, 0, c)
        if e <= a:
            continue
        sub = {n: I.bf16_bits_to_f32(t_np[n][0:1, a:e]).astype(np.float64) for n in t_np}
        lay_c = O.layout([[rows[0][c]]], e - a)
        t0 = time.perf_counter()
        O.attn_fwd(sub["q"], sub["k"], sub["v"], lay_c, shape.theta)
        O.attn_bwd(sub["q"], sub["k"], sub["v"], sub["do"], lay_c, shape.theta)
        dt += time.perf_counter() - t0
        flops += 12.0 * shape.D * shape.Hq * O.useful_pairs(lay_c)
        done, toks = done + 1, toks + (e - a)
        if dt >= budget_s:
            break
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"row 0, its first {done} conversations ({toks} tokens), all {shape.Hq} q / {shape.Hkv} kv "
                      f"heads, fwd+bwd, {dt:.1f} s"}


def depth_stages(Ns, steps=10):
    """Per-stage times (HIP events recorded by the library) of the depth
    workload, one pass against the N passes, one JSON line per (N, kind)."""
    import torch
    from block_sparse_masked_opr_amd import binding as Bd
    dev = torch.device("cuda:0")
    Hq, Hkv, D = I.DEPTH_HEADS["Hq"], I.DEPTH_HEADS["Hkv"], I.DEPTH_HEADS["D"]
    names = ("fwd_prologue", "attn_fwd", "bwd_prologue", "attn_dkdv", "attn_dq")
    for N in Ns:
        conv = I.depth_conversation(N)
        for kind, rows in (("one_pass", [[conv]]), ("n_pass", [S.npass_conversations(conv)])):
            L = I.row_used(rows[0])
            t = device_inputs(torch, 1, L, Hq, Hkv, D, I.SEEDS["depth"][1], dev)
            r = Runner(torch, Bd, rows, L, Hq, Hkv, D, t, dev)
            ev = HipEvents(torch)
            evs = [(ev.array(3), ev.array(4)) for _ in range(steps)]
            for _ in range(3):
                r.step()
            torch.cuda.synchronize()
            for i in range(steps):
                r.step(*evs[i])
            torch.cuda.synchronize()
            acc = dict.fromkeys(names, 0.0)
            for f, b in evs:
                for k, (e, a, z) in zip(names, ((f, 0, 1), (f, 1, 2), (b, 0, 1), (b, 2, 3), (b, 1, 2))):
                    acc[k] += ev.ms(e[a], e[z])
                ev.free(f)
                ev.free(b)
            print(json.dumps({"N": N, "kind": kind, "tokens": L, "pairs": useful_pairs(torch, r.lay),
                              "stages_ms": {k: round(v / steps, 4) for k, v in acc.items()}}), flush=True)
            del r, t
            torch.cuda.empty_cache()


def depth_sweep(torch, Bd, dev, Ns, steps):
    """One conversation of N turns: one pass (as packed, and without the last
    turn's context copy, which nothing sees) against the N passes."""
    out = []
    Hq, Hkv, D = I.DEPTH_HEADS["Hq"], I.DEPTH_HEADS["Hkv"], I.DEPTH_HEADS["D"]
    for N in Ns:
        conv = I.depth_conversation(N)
        rec = {"N": N}
        for kind, rows in (("one_pass", [[conv]]), ("one_pass_elided", [[S.chunk_conversation(conv, 0, N, True)]]),
                           ("n_pass", [S.npass_conversations(conv)])):
            L = I.row_used(rows[0])
            t = device_inputs(torch, 1, L, Hq, Hkv, D, I.SEEDS["depth"][1], dev)
            r = Runner(torch, Bd, rows, L, Hq, Hkv, D, t, dev)
            ms = r.time_steps(steps, 1)
            P = useful_pairs(torch, r.lay)
            rec[kind] = {"tokens": L, "ms": round(ms, 4), "useful_tflops": round(12.0 * D * Hq * P / (ms * 1e-3) / 1e12, 2)}
            del r, t
            torch.cuda.empty_cache()
        rec["speedup"] = round(rec["n_pass"]["ms"] / rec["one_pass"]["ms"], 3)
        rec["speedup_elided"] = round(rec["n_pass"]["ms"] / rec["one_pass_elided"]["ms"], 3)
        log(f"depth N={N}: {rec}")
        out.append(rec)
    return out


def kpass_sweep(torch, Bd, dev, steps):
    """K-pass rows of 32768 tokens: equal-turn splits for K in {1, 2, 4} (as
    packed and with each chunk's last context copy left out), the N-pass rows,
    and planned splits (opr_kpass_plan) under the longest sequence of each
    elided equal split as the cap.  The planner's token weight is fitted from
    the equal splits' times, ms ~ a * pairs + b * tokens."""
    Hq, Hkv, D = I.KPASS_HEADS["Hq"], I.KPASS_HEADS["Hkv"], I.KPASS_HEADS["D"]
    L = I.KPASS_ROW_LEN

    def run(rec, rows):
        t = device_inputs(torch, len(rows), L, Hq, Hkv, D, I.SEEDS["kpass"][1], dev)
        r = Runner(torch, Bd, rows, L, Hq, Hkv, D, t, dev)
        ms = r.time_steps(steps, 1)
        rec.update({"rows": len(rows), "packed_tokens": sum(I.row_used(row) for row in rows),
                    "longest_sequence": max(I.conv_len(c) for row in rows for c in row),
                    "pairs": useful_pairs(torch, r.lay), "ms": round(ms, 4)})
        log(f"kpass {rec}")
        del r, t
        torch.cuda.empty_cache()
        return rec

    out = []
    for K in (1, 2, 4, "N"):
        out.append(run({"K": K, "policy": "equal", "elide_last_rin": False}, S.kpass_rows(K)))
    for K in (1, 2, 4):
        out.append(run({"K": K, "policy": "equal", "elide_last_rin": True}, S.kpass_rows(K, elide_last_rin=True)))
    eq = [x for x in out if x["policy"] == "equal"]
    A = np.array([[x["pairs"], x["packed_tokens"]] for x in eq], dtype=np.float64)
    coef, *_ = np.linalg.lstsq(A, np.array([x["ms"] for x in eq]), rcond=None)
    weight = float(max(coef[1], 0.0) / coef[0]) if coef[0] > 0 else 0.0
    convs = I.kpass_base_conversations(I.SEEDS["kpass"][0], L=L)
    for cap_of in (1, 2, 4):
        cap = next(x["longest_sequence"] for x in out if x["K"] == cap_of and x["elide_last_rin"])
        chunks = []
        for c in convs:
            plan, _ = Bd.opr_kpass_plan(c, max_tokens=cap, tokens_weight=weight, elide_last_rin=True)
            chunks += [S.chunk_conversation(c, p["first_turn"], p["first_turn"] + p["n_turns"], True) for p in plan]
        rec = {"K": None, "policy": "planned", "elide_last_rin": True, "cap": cap, "tokens_weight": round(weight, 2),
               "chunks": len(chunks)}
        out.append(run(rec, I.pack_first_fit_decreasing(chunks, L)))
    base = next(x for x in out if x["K"] == "N")["ms"]
    for x in out:
        x["speedup_vs_npass"] = round(base / x["ms"], 3)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first: the clock settles over the first few tens of steps")
    ap.add_argument("--no-sweep", action="store_true", help="skip the depth and K-pass sweeps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-block", action="store_true", help="skip the attention-block measurements")
    ap.add_argument("--sweep-steps", type=int, default=3)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--depth-stages", metavar="N", type=int, nargs="+",
                    help="only print per-stage times of the depth workload at these N (one pass and N passes)")
    ap.add_argument("--layout-only", action="store_true",
                    help="only time opr_build_layout on 64 rows x 32768 tokens and print its JSON")
    ap.add_argument("--summarize-traffic", metavar="RUN_DIR",
                    help="write the HBM traffic summary of a kernel (--traffic-kernel) from --pmc runs and exit")
    ap.add_argument("--traffic-kernel", default="attn_dkdv", choices=sorted(TRAFFIC_WORKLOAD),
                    help="the kernel that --summarize-traffic summarises (layout: one opr_build_layout call "
                         "of --layout-only)")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic, args.traffic_kernel)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the one-pass attention path runs on a single MI355X; "
              "multi-GPU sharding is a design note only (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return
    if args.depth_stages:
        depth_stages(args.depth_stages)
        return

    import torch
    from block_sparse_masked_opr_amd import binding as Bd

    dev = torch.device("cuda:0")
    if args.layout_only:
        print(json.dumps(layout_step(torch, Bd, dev, args.steps)), flush=True)
        return
    shape = I.PACKED_FWD_BWD
    seed_len, seed_t = I.SEEDS["packed_fwd_bwd"]
    rows = I.packed_rows(shape, seed_len)
    log("generating inputs ...")
    t_np = I.make_tensors(shape.B, shape.L, shape.Hq, shape.Hkv, shape.D, seed=seed_t)
    t = {n: torch.from_numpy(t_np[n].view(np.int16)).view(torch.bfloat16).to(dev) for n in t_np}
    r = Runner(torch, Bd, rows, shape.L, shape.Hq, shape.Hkv, shape.D, t, dev, shape.theta)
    P = useful_pairs(torch, r.lay)
    conv_tokens = sum(I.conv_logical_tokens(c) for row in rows for c in row)
    packed_tokens = sum(I.row_used(row) for row in rows)

    # timed region: exactly `steps` steps, HIP events per stage
    ev = HipEvents(torch)
    evs = [(ev.array(3), ev.array(4)) for _ in range(args.steps)]
    for _ in range(args.warmup):
        r.step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        r.step(*evs[i])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    stages = {"fwd_prologue": 0.0, "attn_fwd": 0.0, "bwd_prologue": 0.0, "attn_dkdv": 0.0, "attn_dq": 0.0}
    for f, b in evs:
        stages["fwd_prologue"] += ev.ms(f[0], f[1])
        stages["attn_fwd"] += ev.ms(f[1], f[2])
        stages["bwd_prologue"] += ev.ms(b[0], b[1])
        stages["attn_dq"] += ev.ms(b[1], b[2])
        stages["attn_dkdv"] += ev.ms(b[2], b[3])
    stages = {k: v / args.steps for k, v in stages.items()}
    for f, b in evs:
        ev.free(f)
        ev.free(b)
    flops = 12.0 * shape.D * shape.Hq * P
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"step {ms:.3f} ms, useful {tflops:.1f} TFLOP/s, stages (ms): "
        + ", ".join(f"{k}={v:.4f}" for k, v in stages.items()))

    # roofline of the dominant kernel: useful flops per launch / its time
    per_pair = {"attn_fwd": 4.0, "attn_dkdv": 6.0, "attn_dq": 2.0}
    dom = max(per_pair, key=lambda k: stages[k])
    achieved = per_pair[dom] * shape.D * shape.Hq * P / (stages[dom] * 1e-3) / 1e12
    traffic = load_traffic(dom)
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch", "avg_ms": round(stages[dom], 4)}

    result = {
        "metric": "masked-attn fwd+bwd useful TFLOP/s & tokens/s; 1-pass vs N-pass speedup",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "packed_fwd_bwd: 2 rows x 16384 tokens, 32 q / 8 kv heads, D=128, "
                               "layout + fwd + bwd per step",
                   "rows": shape.B, "row_tokens": shape.L, "Hq": shape.Hq, "Hkv": shape.Hkv, "D": shape.D,
                   "useful_pairs": P, "conversation_tokens": conv_tokens, "packed_tokens": packed_tokens},
        "tokens_per_s": round(conv_tokens / (ms * 1e-3), 1),
        "packed_tokens_per_s": round(packed_tokens / (ms * 1e-3), 1),
        "frac_of_peak": round(tflops / PEAK_FP16_TFLOPS, 4),
        # secondary, labelled: the FlashAttention convention counts the
        # backward as 2.5 forwards (14 * D * Hq * P for fwd + bwd)
        "tflops_fa_convention": round(14.0 * shape.D * shape.Hq * P / (ms * 1e-3) / 1e12, 2),
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "roofline": roofline,
    }
    result["loss_step"] = loss_step(torch, Bd, r, shape, args.steps, dev)
    log(f"loss step {result['loss_step']['ms']:.4f} ms, {result['loss_step']['roofline']['achieved']} GB/s")
    del r
    torch.cuda.empty_cache()
    result["layout_step"] = layout_step(torch, Bd, dev, args.steps)
    result["packed_fwd"] = packed_fwd_step(torch, Bd, dev, args.steps, args.warmup)
    log(f"packed forward {result['packed_fwd']['ms']:.4f} ms, {result['packed_fwd']['useful_tflops']} TFLOP/s")
    if not args.no_block:
        result["block_step"] = block_step(torch, Bd, dev, rows, shape, args.steps, args.warmup)
    if not args.no_sweep:
        result["depth_sweep"] = depth_sweep(torch, Bd, dev, [2, 4, 8, 16, 32], args.sweep_steps)
        result["kpass"] = kpass_sweep(torch, Bd, dev, args.sweep_steps)
        if not args.no_block:
            result["block_depth"] = block_depth(torch, Bd, dev, [2, 4, 8, 16, 32], args.sweep_steps)
    if not args.no_cpu:
        log("timing the CPU oracle on a sample ...")
        result["cpu_baseline"] = cpu_baseline(rows, shape.L, shape, t_np)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
