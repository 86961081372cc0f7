#!/usr/bin/env python3
"""Bench of the attention hot path on one MI355X.

One step is one pass of the whole hot path over one batch of each workload
the metric names ("attention TFLOP/s (bf16 fwd) at n=128 & 8192; KV-cache
decode HBM GB/s"):
  encoder_base  bf16 encoder self-attention, key padding, B32 h8 n128
  decoder_big   bf16 causal self-attention n128 + cross-attention 128->160
                with source padding, B32 h16
  long_causal   bf16 causal self-attention B1 h16 n8192
  kv_append     bf16 KV-cache append of one token per sequence at the decode
                shape (the cache update of a decode step; it writes row L-1
                with the values the cache holds there, so the decode's
                inputs do not change)
  kv_decode     bf16 KV-cache decode, B64 h16, cache 4096, L in [1, 4096]
  *_bwd         the backward pass (attn_backward, from the forward's saved
                log-sum-exp) of encoder_base, decoder_big and long_causal
                with a seeded N(0,1) dO; algorithmic flops 2.5x the
                forward's (five products per allowed pair).  Reported beside
                the forward figures, not in `value`.
  mha_proj      the multi-head projections of decoder_big's layer (d_model
                1024, h 16, B32): self-attention Q/K/V and output, cross
                attention Q (128 decoder rows), K/V (160 encoder rows) and
                output; seeded N(0, 1/d_model) weights.  Reported beside the
                attention figures, not in `value`.
Inputs are the seeded synthetic tensors of workloads.py, resident in HBM
before timing starts.  Each leg is bracketed by HIP events on the stream
the library launches on (torch's current stream); the step is bracketed by
device synchronisation.  The last step's outputs are sanity-checked against
sampled rows of the fp64 oracle at the end (outside the timed region).

value = bf16 forward TFLOP/s over the forward legs (algorithmic flops:
4 d per allowed (query, key) pair, masked pairs not counted); per-leg
TFLOP/s and GB/s, the decode GB/s and the roofline fractions are reported
beside it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
D = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# Sources of every kernel the bench launches: the traffic figures are reported
# only while these are unchanged since the counters were taken.
KERNEL_SOURCES = ["attn_fwd_bf16_pair.hip", "attn_fwd_bf16_band.hip", "attn_fwd_bf16_short.hip", "attn_fwd_bf16.hip",
                  "attn_decode.hip", "attn_cache.hip", "attn_proj.hip", "attn_bwd.hip", "common.h", "kernel_util.h"]


def kernel_source_hash() -> str:
    """Hash of the kernels' code: the sources with comments and blank space
    removed, so that a comment edit does not void the stored counters."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "head_attention_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ legs
class Leg:
    def __init__(self, name, calls=None, decode=None, append=None, proj=None, bwd=False,
                 in_value=True):
        self.name = name
        self.in_value = in_value   # a forward leg that counts towards the headline value
        self.bwd = bwd             # time attn_backward of `calls` instead of the forward
        self.proj = proj           # projection calls (list of dicts of CPU tensors)
        self.calls = calls or []   # forward calls (dicts of CPU tensors)
        self.decode = decode       # decode call (dict of CPU tensors)
        self.append = append       # cache-append call (dict of CPU tensors)
        self.flops = 0
        self.bytes = 0

    def count(self):
        """Algorithmic flops and bytes (valid Q/K/V rows read, all O rows
        written, lengths read)."""
        for c in self.calls:
            B, H, n_q, _ = c["Q"].shape
            n_k = c["K"].shape[2]
            el = c["Q"].element_size()
            pairs = workloads.allowed_pairs(c["mask"], n_q, n_k, B, c["q_lens"], c["kv_lens"],
                                            radius=c.get("radius"))
            self.flops += (10 if self.bwd else 4) * D * pairs * H
            ql = n_q * B if c["q_lens"] is None else int(c["q_lens"].sum())
            kl = n_k * B if not (c["mask"] & 1) else int(c["kv_lens"].clamp(0, n_k).sum())
            row = H * D * el
            if self.bwd:
                # read Q, O, dO (valid query rows), K, V (valid key rows) and one
                # fp32 log-sum-exp per query row; write dQ, dK, dV in full
                self.bytes += (3 * ql + 2 * kl) * row + 4 * B * H * n_q + (B * n_q + 2 * B * n_k) * row
            else:
                self.bytes += (ql + 2 * kl + B * n_q) * row
            self.bytes += 4 * B * ((c["q_lens"] is not None) + (c["kv_lens"] is not None))
        if self.decode is not None:
            d = self.decode
            B, H, _, _ = d["q"].shape
            el = d["q"].element_size()
            L = int(d["kv_lens"].sum())
            self.flops += 4 * D * L * H
            self.bytes += 2 * L * H * D * el + 2 * B * H * D * el + 4 * B
        for pc in self.proj or []:
            if pc["kind"] == "head":
                B, n, d_model = pc["X"].shape
                n_out = pc["W"].shape[0] // d_model
                self.flops += 2 * B * n * n_out * d_model * d_model
                self.bytes += 2 * (B * n * d_model * (1 + n_out) + n_out * d_model * d_model)
            else:
                B, h, n, _ = pc["O"].shape
                d_model = h * D
                self.flops += 2 * B * n * d_model * d_model
                self.bytes += 2 * (2 * B * n * d_model + d_model * d_model)
        if self.append is not None:
            a = self.append
            B, H, n_new, _ = a["Knew"].shape
            el = a["Knew"].element_size()
            # K and V rows read from the new block and written to the caches
            self.bytes += 2 * 2 * B * H * n_new * D * el + 4 * B


def make_legs():
    legs = []
    for name in ("encoder_base", "decoder_big", "long_causal"):
        legs.append(Leg(name, calls=workloads.make(name)["calls"]))
    for name in ("encoder_base", "decoder_big", "long_causal"):
        legs.append(Leg(name + "_bwd", calls=workloads.make(name)["calls"], bwd=True))
    legs.append(Leg("long_restricted", calls=workloads.make("long_restricted")["calls"], in_value=False))
    kd = workloads.make("kv_decode")
    rows = (kd["kv_lens"] - 1).long()
    bi = torch.arange(kd["q"].shape[0])
    append = {"Knew": kd["Kcache"][bi, :, rows].unsqueeze(2).contiguous(),
              "Vnew": kd["Vcache"][bi, :, rows].unsqueeze(2).contiguous(),
              "kv_lens": kd["kv_lens"]}
    legs.append(Leg("kv_append", append=append))
    legs.append(Leg("kv_decode", decode=kd))
    g = workloads.generator(1100)
    B, h, d_model, n_t, n_s = 32, 16, 1024, 128, 160
    wts = lambda rows: (torch.randn((rows, d_model), generator=g) / d_model ** 0.5).to(torch.bfloat16)
    x_dec = workloads.randn(g, (B, n_t, d_model), torch.bfloat16)
    x_enc = workloads.randn(g, (B, n_s, d_model), torch.bfloat16)
    o_self = workloads.randn(g, (B, h, n_t, D), torch.bfloat16)
    o_cross = workloads.randn(g, (B, h, n_t, D), torch.bfloat16)
    proj = [{"kind": "head", "X": x_dec, "W": wts(3 * d_model), "h": h},   # self Q, K, V
            {"kind": "out", "O": o_self, "W": wts(d_model)},               # self output
            {"kind": "head", "X": x_dec, "W": wts(d_model), "h": h},       # cross Q
            {"kind": "head", "X": x_enc, "W": wts(2 * d_model), "h": h},   # cross K, V
            {"kind": "out", "O": o_cross, "W": wts(d_model)}]              # cross output
    legs.append(Leg("mha_proj", proj=proj))
    for leg in legs:
        leg.count()
    return legs


def to_device(legs):
    import head_attention_amd as ha
    for leg in legs:
        leg.dev_calls = []
        for j, c in enumerate(leg.calls):
            dc = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in c.items()}
            dc["O"] = torch.empty_like(dc["Q"])
            if leg.bwd:
                B, H, n_q, _ = c["Q"].shape
                g = workloads.generator(1200 + j)
                dc["dO"] = workloads.randn(g, tuple(c["Q"].shape), torch.bfloat16).cuda()
                dc["lse"] = torch.empty((B, H, n_q), dtype=torch.float32, device="cuda")
                ha.forward(dc["Q"], dc["K"], dc["V"], mask_kind=dc["mask"], q_lens=dc["q_lens"],
                           kv_lens=dc["kv_lens"], scale=dc["scale"], out=dc["O"], lse=dc["lse"])
                dc["grads"] = (torch.empty_like(dc["Q"]), torch.empty_like(dc["K"]), torch.empty_like(dc["V"]))
                n_k = c["K"].shape[2]
                dc["ws"] = torch.empty(ha.backward_workspace_bytes(B, H, n_q, n_k), dtype=torch.uint8,
                                       device="cuda")
            leg.dev_calls.append(dc)
        leg.dev_proj = []
        for pc in leg.proj or []:
            dp = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in pc.items()}
            if pc["kind"] == "head":
                B, n, d_model = pc["X"].shape
                dp["outs"] = [torch.empty((B, pc["h"], n, D), dtype=torch.bfloat16, device="cuda")
                              for _ in range(pc["W"].shape[0] // d_model)]
            else:
                B, h, n, _ = pc["O"].shape
                dp["Y"] = torch.empty((B, n, h * D), dtype=torch.bfloat16, device="cuda")
            leg.dev_proj.append(dp)
        leg.dev_append = None
        if leg.append is not None:
            leg.dev_append = {k: v.cuda() for k, v in leg.append.items()}
        if leg.decode is not None:
            d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in leg.decode.items()}
            B, H, _, _ = d["q"].shape
            n_max = d["Kcache"].shape[2]
            d["O"] = torch.empty_like(d["q"])
            d["ws"] = torch.empty(ha.decode_workspace_bytes(B, H, n_max, d["q"].dtype),
                                  dtype=torch.uint8, device="cuda")
            leg.dev_decode = d
        else:
            leg.dev_decode = None


def run_leg(leg, caches=None):
    import head_attention_amd as ha
    for dp in leg.dev_proj:
        if dp["kind"] == "head":
            ha.head_projection(dp["X"], dp["W"], dp["h"], dp["outs"])
        else:
            ha.output_projection(dp["O"], dp["W"], dp["Y"])
    a = leg.dev_append
    if a is not None:
        ha.cache_append(a["Knew"], a["Vnew"], caches["Kcache"], caches["Vcache"], a["kv_lens"])
    for c in leg.dev_calls:
        if leg.bwd:
            ha.backward(c["Q"], c["K"], c["V"], c["O"], c["dO"], c["lse"], mask_kind=c["mask"],
                        q_lens=c["q_lens"], kv_lens=c["kv_lens"], scale=c["scale"], grads=c["grads"],
                        workspace=c["ws"])
            continue
        if "radius" in c:
            ha.forward_restricted(c["Q"], c["K"], c["V"], c["radius"], mask_kind=c["mask"],
                                  q_lens=c["q_lens"], kv_lens=c["kv_lens"], scale=c["scale"], out=c["O"])
            continue
        ha.forward(c["Q"], c["K"], c["V"], mask_kind=c["mask"], q_lens=c["q_lens"],
                   kv_lens=c["kv_lens"], scale=c["scale"], out=c["O"])
    d = leg.dev_decode
    if d is not None:
        ha.decode(d["q"], d["Kcache"], d["Vcache"], d["kv_lens"], scale=d["scale"], out=d["O"],
                  workspace=d["ws"])


# --------------------------------------------------------- sanity vs oracle
def sanity_check(legs):
    """Sampled rows of the last step's outputs against the fp64 oracle."""
    import oracle.attn_oracle as orc

    def np64(t):
        return t.detach().to("cpu", torch.float32).double().numpy()

    worst = 0.0
    rng = np.random.default_rng(0)
    for leg in legs:
        for c, dc in zip(leg.calls, leg.dev_calls):
            B, H, n_q, _ = c["Q"].shape
            rows = [(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(n_q)))
                    for _ in range(24)]
            ref = orc.attention(np64(c["Q"]), np64(c["K"]), np64(c["V"]), mask_kind=c["mask"],
                                q_lens=None if c["q_lens"] is None else c["q_lens"].numpy(),
                                kv_lens=None if c["kv_lens"] is None else c["kv_lens"].numpy(),
                                scale=c["scale"], rows=rows, radius=c.get("radius"))
            out = np64(dc["O"])
            worst = max(worst, max(float(np.abs(out[r] - ref[r]).max()) for r in rows))
        if leg.decode is not None:
            d = leg.decode
            pairs = [(int(rng.integers(64)), int(rng.integers(16))) for _ in range(16)]
            out = np64(leg.dev_decode["O"])
            for (b, h) in pairs:
                ref = orc.decode(np64(d["q"][b:b + 1, h:h + 1]), np64(d["Kcache"][b:b + 1, h:h + 1]),
                                 np64(d["Vcache"][b:b + 1, h:h + 1]), d["kv_lens"][b:b + 1].numpy(),
                                 scale=d["scale"])
                worst = max(worst, float(np.abs(out[b, h] - ref[0, 0]).max()))
    return worst


# ------------------------------------------------------------ CPU baseline
# Worker state for the all-core run: the long_causal tensors in fp64, set in
# the parent before the pool forks (the children read them copy-on-write).
_CPU_QKV = None


def _cpu_rows(rows):
    """One worker of the all-core run: the oracle on its share of the rows,
    one BLAS thread."""
    import oracle.attn_oracle as orc
    from threadpoolctl import threadpool_limits
    Q, K, V = _CPU_QKV
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        orc.attention(Q, K, V, mask_kind=orc.MASK_CAUSAL, scale=0.125, rows=rows)
        return time.perf_counter() - t0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_1t_s: float = 8.0, max_workers: int = 16):
    """The fp64 oracle as it stands (oracle/attn_oracle.py, untuned) on the
    long_causal workload, in the same algorithmic flop units as the GPU:
      * all cores: every query row of all 16 heads, split into interleaved
        shares over a pool of worker processes (one BLAS thread each) -- the
        host cores this process may use, at most max_workers (the CPU share
        of one GPU on these hosts);
      * one core: evenly spaced rows of every head, each with its full causal
        prefix, sized from a short probe to take about target_1t_s.
    Run before the GPU is initialised, so the pool forks a process with no
    device context."""
    import multiprocessing as mp
    import oracle.attn_oracle as orc
    from threadpoolctl import threadpool_limits
    global _CPU_QKV
    c = workloads.make("long_causal")["calls"][0]
    Q, K, V = (c[k].float().double().numpy() for k in ("Q", "K", "V"))
    H, n = Q.shape[1], Q.shape[2]
    _CPU_QKV = (Q, K, V)
    visible = len(os.sched_getaffinity(0))
    workers = max(1, min(visible, max_workers))
    model = _cpu_model()
    flops_of = lambda rows: sum(4 * D * (i + 1) for (_, _, i) in rows)

    # one core
    with threadpool_limits(limits=1):
        probe = [(0, 0, i) for i in range(n - 1, 0, -(n // 8))]
        t0 = time.perf_counter()
        orc.attention(Q, K, V, mask_kind=orc.MASK_CAUSAL, scale=0.125, rows=probe)
        per_row = (time.perf_counter() - t0) / sum(i + 1 for (_, _, i) in probe) * (n / 2)
        per_head = int(max(16, min(n, target_1t_s / max(per_row, 1e-9) / H)))
        stride = max(1, n // per_head)
        rows = [(0, h, i) for h in range(H) for i in range((stride // 2 + h) % stride, n, stride)]
        t0 = time.perf_counter()
        orc.attention(Q, K, V, mask_kind=orc.MASK_CAUSAL, scale=0.125, rows=rows)
        dt1 = time.perf_counter() - t0
    one = {
        "value": flops_of(rows) / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
        "sample": f"long_causal (B1 h16 n=8192 causal): every {stride}th query row of each head, "
                  f"{len(rows)} rows, full causal prefix each; fp64 NumPy, 1 BLAS thread; {dt1:.1f} s",
        "cpu_model": model, "host_cores_visible": visible,
    }

    # all cores: interleaved shares of every row, so each worker gets the same
    # mix of short and long causal prefixes
    all_rows = [(0, h, i) for h in range(H) for i in range(n)]
    shares = [all_rows[w::workers] for w in range(workers)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        busy = pool.map(_cpu_rows, shares)
    dtn = time.perf_counter() - t0
    _CPU_QKV = None
    allc = {
        "value": flops_of(all_rows) / dtn / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
        "sample": f"long_causal (B1 h16 n=8192 causal): all {len(all_rows)} query rows of all {H} heads, "
                  f"full causal prefix each, split over {workers} worker processes (1 BLAS thread each); "
                  f"fp64 NumPy; {dtn:.1f} s wall, {max(busy):.1f} s longest worker",
        "cpu_model": model, "host_cores_visible": visible,
    }
    return allc, one


# ------------------------------------------------------- rocprof summaries
FWD_MODES = {"0": "none", "1": "causal", "2": "band"}


def _short_kernel(name: str) -> str:
    """attn_fwd_bf16[_pair|_short]_kernel<mode> and the backward's dK/dV and dQ
    kernels (both kinds of each) -> ..._kernel<none|causal|band>;
    the projection kernel -> proj_gemm_kernel<head_out, tokens x features of
    its tile>; the bool-templated kernels -> <true|false>; other kernels of
    the library by their plain name."""
    import re
    m = re.search(r"(attn_fwd_bf16(?:_pair|_short)?_kernel|bwd_dkdv(?:_pair)?_kernel|bwd_dq(?:_pair)?_kernel)(?:<|ILi)(\d)", name)
    if m:
        return f"{m.group(1)}<{FWD_MODES[m.group(2)]}>"
    m = re.search(r"proj_gemm_kernel<(true|false), (\d), (\d), (\d)>", name) or \
        re.search(r"proj_gemm_kernelILb(\d)ELi(\d)ELi(\d)ELi(\d)E", name)
    if m:
        wm, tbw, fbw = int(m.group(2)), int(m.group(3)), int(m.group(4))
        head_out = m.group(1) in ("true", "1")
        return f"proj_gemm_kernel<{'true' if head_out else 'false'}, {32 * tbw * wm}x{32 * fbw * (8 // wm)}>"
    m = re.search(r"(attn_fwd_bf16(?:_pair|_short)?_kernel|proj_gemm_kernel|bwd_dkdv_kernel|bwd_dq_kernel)<(true|false)", name) or \
        re.search(r"(attn_fwd_bf16(?:_pair|_short)?_kernel|proj_gemm_kernel|bwd_dkdv_kernel|bwd_dq_kernel)ILb(\d)", name)
    if m:
        causal = m.group(2) in ("true", "1")
        return f"{m.group(1)}<{'true' if causal else 'false'}>"
    for key in ("attn_fwd_bf16_band_kernel", "attn_fwd_f32_kernel", "decode_partial_kernel", "decode_merge_kernel",
                "cache_append_kernel", "bwd_rowdot_kernel", "copyBuffer", "elementwise"):
        if key in name:
            return key
    return name[:60]


# Grid sizes (threads) of each leg's launches, to tell apart launches of the
# same kernel in a trace of the default bench command.
LEG_GRIDS = {("attn_fwd_bf16_short_kernel<none>", 65536): "encoder_base",
             ("attn_fwd_bf16_short_kernel<causal>", 131072): "decoder_big (causal self)",
             ("attn_fwd_bf16_short_kernel<none>", 131072): "decoder_big (cross)",
             ("attn_fwd_bf16_band_kernel", 131072): "long_restricted",
             ("cache_append_kernel", 8192): "kv_append",
             ("bwd_dkdv_pair_kernel<causal>", 262144): "long_causal_bwd",
             ("bwd_dq_pair_kernel<causal>", 524288): "long_causal_bwd",
             ("bwd_rowdot_kernel", 1048576): "long_causal_bwd",
             ("bwd_dkdv_kernel<none>", 65536): "encoder_base_bwd",
             ("bwd_dq_kernel<none>", 65536): "encoder_base_bwd",
             ("bwd_rowdot_kernel", 262144): "encoder_base_bwd",
             ("bwd_dkdv_kernel<causal>", 131072): "decoder_big_bwd (causal self)",
             ("bwd_dq_kernel<causal>", 131072): "decoder_big_bwd (causal self)",
             ("bwd_dkdv_kernel<none>", 262144): "decoder_big_bwd (cross)",
             ("bwd_dq_kernel<none>", 131072): "decoder_big_bwd (cross)",
             ("bwd_rowdot_kernel", 524288): "decoder_big_bwd (self and cross)",
             ("proj_gemm_kernel<true, 256x192>", 131072): "mha_proj (self Q, K, V)",
             ("proj_gemm_kernel<true, 128x128>", 131072): "mha_proj (cross Q)",
             ("proj_gemm_kernel<true, 320x128>", 131072): "mha_proj (cross K, V)",
             ("proj_gemm_kernel<false, 128x128>", 131072): "mha_proj (self and cross output)",
             ("attn_fwd_bf16_pair_kernel<causal>", 262144): "long_causal",
             ("decode_partial_kernel", 4194304): "kv_decode",
             ("decode_merge_kernel", 65536): "kv_decode",
             ("attn_fwd_bf16_short_kernel<none>", 256): "launch floor (1-row forward)",
             ("at::cuda::(anonymous namespace)::spin_kernel(long)", 1): "launch floor (empty kernel)",
             ("copyBuffer", 512): "bench set-up copies",
             ("attn_fwd_bf16_kernel<true>", 393216): "mid_causal_300 (B32 h16 n300)",
             ("attn_fwd_bf16_kernel<false>", 65536): "mid_cross_128_300 (B32 h8 128->300)",
             ("attn_fwd_bf16_kernel<true>", 131072): "mid_causal_500 (B8 h16 n500)"}


def summarize_trace(path: str) -> str:
    """Per (kernel, grid) launch statistics from a rocprofv3 kernel-trace CSV."""
    import csv
    import collections
    g = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        g[(_short_kernel(r["Kernel_Name"]), grid)].append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["| kernel | grid (threads) | leg | launches | avg us | min us | max us |",
             "|---|---|---|---|---|---|---|"]
    for (k, grid), v in sorted(g.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {k} | {grid} | {LEG_GRIDS.get((k, grid), '')} | {len(v)} | "
                     f"{sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(lines)


def summarize_counters(fetch_csv: str, write_csv: str, copy_mib: int, out_json: str | None):
    """Bytes per launch that miss L2 (FETCH_SIZE: reads served by the MALL or
    HBM; WRITE_SIZE: writes leaving L2), from counter runs in KiB per
    dispatch, each scaled by what the same counter reads for the plain copy
    of copy_mib MiB that bench.py --copy-probe-mib runs.  The MALL can serve
    some of these reads, so they bound HBM traffic from above."""
    import csv
    import collections

    def load(path, counter):
        g = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                g[(_short_kernel(r["Kernel_Name"]), int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in g.items()}

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    known_kib = copy_mib * 1024.0
    copy_key = max((k for k in fetch if k[0] == "copyBuffer"), key=lambda k: k[1])
    f_fetch = known_kib / fetch[copy_key]
    f_write = known_kib / write[copy_key]
    lines = [f"copy probe ({copy_mib} MiB each way, {copy_key[0]} grid {copy_key[1]}): "
             f"FETCH_SIZE {fetch[copy_key]:.1f} KiB -> scale {f_fetch:.4f}; "
             f"WRITE_SIZE {write[copy_key]:.1f} KiB -> scale {f_write:.4f}", "",
             "| kernel | grid | leg | FETCH_SIZE KiB | WRITE_SIZE KiB | read past L2 MB | written past L2 MB |",
             "|---|---|---|---|---|---|---|"]
    res = {}
    for k in sorted(fetch):
        if k[0] in ("copyBuffer", "elementwise"):
            continue
        rd = fetch[k] * f_fetch * 1024 / 1e6
        wr = write.get(k, 0.0) * f_write * 1024 / 1e6
        lines.append(f"| {k[0]} | {k[1]} | {LEG_GRIDS.get(k, '')} | {fetch[k]:.1f} | "
                     f"{write.get(k, 0.0):.1f} | {rd:.2f} | {wr:.2f} |")
        res[f"{k[0]}@{k[1]}"] = {"read_bytes": rd * 1e6, "write_bytes": wr * 1e6}
    if out_json:
        lc = res.get("attn_fwd_bf16_pair_kernel<causal>@262144")
        with open(out_json, "w") as f:
            json.dump({"kernel_source_hash": kernel_source_hash(),
                       "fetch_scale": f_fetch, "write_scale": f_write,
                       "long_causal_fwd_bytes_per_launch":
                           None if lc is None else round(lc["read_bytes"] + lc["write_bytes"]),
                       "per_kernel": res}, f, indent=1)
    return "\n".join(lines)


def summarize_pmc(csvs, trace_csv=None, n_simd: int = 1024, n_xcd: int = 8) -> str:
    """Per-kernel MFMA and VALU figures from rocprofv3 --pmc runs of the bench
    (one CSV per pass; counters averaged over a kernel's launches).

    us: average duration from a kernel-trace run of the same command when
      given (counter runs serialise dispatches), else from the counter runs.
    clock: GRBM_GUI_ACTIVE (busy GPU clocks, summed over the n_xcd XCDs) per
      XCD, less what it reads for the empty kernel the bench launches
      (torch's spin kernel: the counter window's own overhead, about 20k
      clocks), over the duration of the same counter-run dispatches.  Cycle
      fractions below are per SIMD over those cycles (n_simd SIMDs).
    mfma busy: SQ_VALU_MFMA_BUSY_CYCLES; also at the 2.4 GHz peak clock over
      the trace duration, i.e. the fraction of the bf16 MFMA peak the matrix
      cores were busy for.
    mfma TFLOP/s executed: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (padding and
      row-sum products included) over the trace duration.
    valu busy: SQ_ACTIVE_INST_VALU (quad-cycles a wave works on VALU
      instructions, summed over waves) x 4.
    co-issue: SQ_VALU_MFMA_COEXEC_CYCLES (MFMA busy while a VALU
      instruction issued).  neither ~ 1 - mfma - valu + co-issue.
    per wave: instructions issued per wave (SQ_INSTS_* over SQ_WAVES)."""
    import csv
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for path in csvs:
        for r in csv.DictReader(open(path)):
            k = (_short_kernel(r["Kernel_Name"]), int(r["Grid_Size"]))
            acc[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[k][(path, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    tdur = {}
    if trace_csv:
        g = collections.defaultdict(list)
        for r in csv.DictReader(open(trace_csv)):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            g[(_short_kernel(r["Kernel_Name"]), grid)].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        tdur = {k: sum(v) / len(v) for k, v in g.items()}
    nan = float("nan")
    empty = [k for k in acc if k[0].startswith("at::cuda::") and "GRBM_GUI_ACTIVE" in acc[k]]
    offset = (sum(acc[empty[0]]["GRBM_GUI_ACTIVE"]) / len(acc[empty[0]]["GRBM_GUI_ACTIVE"]) / n_xcd
              if empty else 0.0)
    lines = [f"clock offset (empty kernel, per XCD): {offset:.0f} GRBM clocks", "",
             "| kernel | grid | leg | us | clock GHz | mfma busy | mfma busy @2.4 GHz | mfma TFLOP/s executed | "
             "valu busy | co-issue | neither | VALU/wave | TRANS/wave | MFMA/wave |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(acc, key=lambda k: -sum(dur[k].values())):
        c = {n: sum(v) / len(v) for n, v in acc[k].items()}
        pmc_us = sum(dur[k].values()) / len(dur[k])
        us = tdur.get(k, pmc_us)
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in c or us <= 0 or pmc_us <= 0:
            continue
        if k[0].startswith("at::cuda::") or k[0] in ("copyBuffer", "elementwise"):
            continue
        if pmc_us < 5.0:  # the window overhead swamps the clock count of a launch this short
            continue
        cyc = c.get("GRBM_GUI_ACTIVE", nan) / n_xcd - offset  # clocks per XCD in the dispatch
        clk = cyc / (pmc_us * 1e3)
        per_simd = lambda n: c.get(n, nan) / n_simd / cyc
        mfma, co = per_simd("SQ_VALU_MFMA_BUSY_CYCLES"), per_simd("SQ_VALU_MFMA_COEXEC_CYCLES")
        valu = 4 * per_simd("SQ_ACTIVE_INST_VALU")
        waves = c.get("SQ_WAVES", nan)
        per_wave = lambda n: c[n] / waves if n in c and waves == waves and waves > 0 else nan
        lines.append(
            f"| {k[0]} | {k[1]} | {LEG_GRIDS.get(k, '')} | {us:.2f} | {clk:.2f} | {mfma:.3f} | "
            f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / (n_simd * us * 1e3 * 2.4):.3f} | "
            f"{c.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', 0) * 512 / (us * 1e-6) / 1e12:.1f} | "
            f"{valu:.3f} | {co:.3f} | {1 - mfma - valu + co:.3f} | "
            f"{per_wave('SQ_INSTS_VALU'):.0f} | {per_wave('SQ_INSTS_VALU_TRANS_F32'):.0f} | "
            f"{per_wave('SQ_INSTS_MFMA'):.0f} |")
    return "\n".join(lines)


# -------------------------------------------------- rooflines, device, floor
RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)  # 312.5


def roof(kernel: str, flops: int, nbytes: int, ms: float) -> dict:
    """Roofline entry of one leg: bound by whichever roof its arithmetic
    intensity (algorithmic flops per algorithmic byte) meets first -- the
    bf16 MFMA peak above the ridge, HBM below it."""
    ai = flops / nbytes
    if ai >= RIDGE_FLOP_PER_BYTE:
        achieved, peak, unit, bound = flops / (ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = nbytes / (ms * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s", "hbm"
    return {"bound": bound, "kernel": kernel, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "flop_per_byte": round(ai, 1)}


def device_info() -> dict:
    """Compute units and peak clock as the HIP runtime reports them, and the
    dense bf16 MFMA peak they imply (4096 flop per clock per CU)."""
    import ctypes
    props = torch.cuda.get_device_properties(0)
    out = {"name": props.name, "arch": getattr(props, "gcnArchName", "")}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int()
        attrs = {"clock_khz": 5, "cu": 63}  # hipDeviceAttributeClockRate, ...MultiprocessorCount
        for k, a in attrs.items():
            if hip.hipDeviceGetAttribute(ctypes.byref(v), a, 0) == 0:
                out[k] = v.value
    except OSError:
        pass
    if "cu" in out and "clock_khz" in out:
        out["max_clock_mhz"] = out.pop("clock_khz") / 1e3
        out["bf16_peak_tflops_from_device"] = round(out["cu"] * out["max_clock_mhz"] * 1e6 * 4096 / 1e12, 1)
    return out


def launch_floor(stream, reps: int = 200) -> dict:
    """Per-launch time of back-to-back launches on the bench's stream, timed
    with HIP events: an empty kernel (torch's spin kernel with 0 cycles) and
    the library's smallest forward call (one bf16 row of one head)."""
    import head_attention_amd as ha
    res = {}
    q = torch.zeros((1, 1, 1, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    tests = [("forward_1row_us", lambda: ha.forward(q, q, q, out=o))]
    if hasattr(torch.cuda, "_sleep"):
        tests.insert(0, ("empty_kernel_us", lambda: torch.cuda._sleep(0)))
    for name, fn in tests:
        for _ in range(20):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    return res


# Shapes between the short-key and the paired kernels (256 < n_k, n_q < 512),
# which run on the 4-wave kernel: the decoder of the big model at n = 300
# (causal self) and cross attention from 128 decoder rows to 300 encoder rows
# with key padding, and B8 h16 n500 causal.  Timed apart from the step.
MID_SHAPES = (("mid_causal_300", 32, 16, 300, 300, True, False),
              ("mid_cross_128_300", 32, 8, 128, 300, False, True),
              ("mid_causal_500", 8, 16, 500, 500, True, False))


def mid_shapes(stream, reps: int = 20) -> dict:
    """Back-to-back forward calls at MID_SHAPES, timed with HIP events."""
    import head_attention_amd as ha
    g = torch.Generator().manual_seed(1300)
    res = {}
    for name, B, H, nq, nk, causal, kpad in MID_SHAPES:
        Q = torch.randn((B, H, nq, 64), generator=g).to(torch.bfloat16).cuda()
        K = torch.randn((B, H, nk, 64), generator=g).to(torch.bfloat16).cuda()
        V = torch.randn((B, H, nk, 64), generator=g).to(torch.bfloat16).cuda()
        kl = torch.randint(16, nk + 1, (B,), generator=g, dtype=torch.int32) if kpad else None
        mk = ha.ATTN_MASK_CAUSAL if causal else (ha.ATTN_MASK_KEY_PADDING if kpad else ha.ATTN_MASK_NONE)
        kld = kl.cuda() if kpad else None
        out = torch.empty_like(Q)

        def call():
            ha.forward(Q, K, V, mask_kind=mk, kv_lens=kld, scale=0.125, out=out)
        for _ in range(5):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        if causal:
            pairs = B * H * nq * (nq + 1) // 2
        elif kpad:
            pairs = H * nq * int(kl.sum())
        else:
            pairs = B * H * nq * nk
        res[name] = {"shape": f"B{B} h{H} {nq}x{nk}{' causal' if causal else ''}{' key padding' if kpad else ''}",
                     "us": round(us, 2), "TFLOP/s": round(4 * 64 * pairs / (us * 1e-6) / 1e12, 2)}
    return res


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sanity", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB "
                         "(the known-size reference for HBM counter calibration)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print per-kernel launch statistics of a rocprofv3 trace and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print HBM traffic per launch from rocprofv3 --pmc runs (with "
                         "--copy-probe-mib naming the probe size) and exit")
    ap.add_argument("--traffic-json", help="with --summarize-counters: write the figures here")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="COUNTER_CSV",
                    help="print per-kernel MFMA / VALU figures from rocprofv3 --pmc runs and exit")
    ap.add_argument("--trace-csv", help="with --summarize-pmc: kernel-trace CSV for the durations")
    args = ap.parse_args()

    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc, args.trace_csv))
        return

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, args.copy_probe_mib or 1024,
                                 args.traffic_json))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this library runs on one GPU: its attention path has no "
                                   "multi-GPU mode (each GPU would run the same kernels on its "
                                   "share of heads or sequences); run with --gpus 1"}))
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()  # before the GPU is initialised (its pool forks)

    import head_attention_amd as ha
    ha.lib()  # fail loudly if the library is missing
    torch.cuda.set_device(0)
    legs = make_legs()
    to_device(legs)
    stream = torch.cuda.current_stream()
    dd = next(leg.dev_decode for leg in legs if leg.dev_decode is not None)
    caches = {"Kcache": dd["Kcache"], "Vcache": dd["Vcache"]}  # the append writes the decode's caches
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for leg in legs:
            run_leg(leg, caches)
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in legs] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        for j, leg in enumerate(legs):
            ev[s][j][0].record(stream)
            run_leg(leg, caches)
            ev[s][j][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    leg_ms = [sum(ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(args.steps)) / args.steps
              for j in range(len(legs))]
    step_ms = sum(leg_ms)
    fwd = [j for j, leg in enumerate(legs) if leg.dev_calls and not leg.bwd and leg.in_value]
    fwd_flops = sum(legs[j].flops for j in fwd)
    fwd_ms = sum(leg_ms[j] for j in fwd)
    value = fwd_flops / (fwd_ms * 1e-3) / 1e12

    per_leg = {}
    for leg, ms in zip(legs, leg_ms):
        per_leg[leg.name] = {
            "us": round(ms * 1e3, 2),
            "TFLOP/s": round(leg.flops / (ms * 1e-3) / 1e12, 2),
            "GB/s": round(leg.bytes / (ms * 1e-3) / 1e9, 1),
            "alg_flops": leg.flops,
            "alg_bytes": leg.bytes,
        }
    lc = legs[[l.name for l in legs].index("long_causal")]
    kd = legs[[l.name for l in legs].index("kv_decode")]
    lc_ms = leg_ms[legs.index(lc)]
    kd_ms = leg_ms[legs.index(kd)]
    lc_tflops = lc.flops / (lc_ms * 1e-3) / 1e12
    kd_gbps = kd.bytes / (kd_ms * 1e-3) / 1e9

    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tc = json.load(f)
        if tc.get("kernel_source_hash") == kernel_source_hash():
            traffic = tc.get("long_causal_fwd_bytes_per_launch")
    except (OSError, ValueError):
        pass

    out = {
        "metric": "attention TFLOP/s (bf16 fwd) at n=128 & 8192; KV-cache decode HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), workloads.py)",
        "config": {
            "workload": "attention hot path: encoder self-attn B32 h8 n128 key-padding + "
                        "decoder causal self n128 & cross 128->160 B32 h16 + causal self "
                        "B1 h16 n8192 + KV decode B64 h16 cache 4096; d=64",
            "value_covers": "bf16 forward legs (n=128 and n=8192)",
            "decode_GBps": round(kd_gbps, 1),
            "long_causal_TFLOPs": round(lc_tflops, 2),
            "legs": per_leg,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_bf16_pair_kernel<causal> on long_causal (B1 h16 n8192)",
            "achieved": round(lc_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(lc_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    ix = {l.name: j for j, l in enumerate(legs)}

    def leg_roof(name, kernel):
        return roof(kernel, legs[ix[name]].flops, legs[ix[name]].bytes, leg_ms[ix[name]])

    out["roofline_bwd"] = leg_roof("long_causal_bwd", "bwd_rowdot + bwd_dkdv + bwd_dq on long_causal_bwd (B1 h16 n8192)")
    out["roofline_proj"] = leg_roof("mha_proj", "proj_gemm_kernel on mha_proj (decoder_big layer projections)")
    out["roofline_restricted"] = leg_roof(
        "long_restricted", "attn_fwd_bf16_band_kernel on long_restricted (B1 h16 n8192, radius 256)")
    out["roofline_decode"] = leg_roof("kv_decode", "decode_partial_kernel + decode_merge_kernel on kv_decode")
    out["roofline_n128"] = {n: leg_roof(n, k) for n, k in (
        ("encoder_base", "attn_fwd_bf16_short_kernel<none> on encoder_base (B32 h8 n128, key padding)"),
        ("decoder_big", "attn_fwd_bf16_short_kernel<causal> + <none> on decoder_big (B32 h16, 128 self, 128->160)"))}
    out["device"] = device_info()
    out["launch_floor"] = launch_floor(stream)
    out["mid_shapes"] = mid_shapes(stream)
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib * 2 ** 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes_each_way"] = args.copy_probe_mib * 2 ** 20
    if not args.no_sanity:
        out["sanity_max_abs_err_vs_oracle"] = round(sanity_check(legs), 6)
        ap = next(leg.dev_append for leg in legs if leg.dev_append is not None)
        rows = (ap["kv_lens"] - 1).long()
        bi = torch.arange(rows.shape[0], device=rows.device)
        out["sanity_append_rows_exact"] = bool(
            torch.equal(caches["Kcache"][bi, :, rows], ap["Knew"][:, :, 0])
            and torch.equal(caches["Vcache"][bi, :, rows], ap["Vnew"][:, :, 0]))
    if cpu is not None:
        out["cpu_baseline"], out["cpu_baseline_1core"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
