"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and arranges them in the shapes of the
workloads; it holds none of the attention arithmetic, and it imports neither
the HIP binding nor the CPU oracle, so both sides (and the bench) can share it.

The pages train and evaluate on WMT14 translation data, which is not used
here.  Synthetic stand-ins keep the pages' Transformer shapes -- base model
d_model 512 / h 8 and big model d_model 1024 / h 16, d_k = d_v = 64
("[논문 리뷰]Attention Is All You Need", §3.2.2 and §6.2 Table 3 "big") -- with
iid N(0, 1) activations, the variance assumption of that page's §3.2.1
scaling argument.

Recipe (one torch CPU generator per workload, seed 1000 + workload number):
lengths are drawn first with ``torch.randint(lo, hi + 1, (B,))`` (inclusive
discrete uniform), then the tensors in the order listed, each with
``torch.randn(shape, dtype=float32)``; bf16 workloads are rounded once with
``.to(torch.bfloat16)`` (round to nearest even).  Padded rows (beyond a
sequence's length) hold real N(0, 1) draws, so masking is exercised.
"""

from __future__ import annotations

import torch

D = 64  # d_k = d_v for every workload

# name -> (number, description)
WORKLOADS = {
    "tiny_fp32": (1, "unmasked self-attention B1 h8 n16 d64, fp32, scale 1/8"),
    "encoder_base": (2, "encoder self-attention, key padding, B32 h8 n128 d64, L in [8,128], bf16"),
    "decoder_big": (3, "big decoder layer: causal self n128 + cross 128->160 keys, "
                       "source L in [16,160], B32 h16 d64, bf16"),
    "long_causal": (4, "causal self-attention B1 h16 n8192 d64, bf16"),
    "kv_decode": (5, "KV-cache decode, B64 h16, cache 4096, L in [1,4096], d64, bf16"),
    "long_restricted": (6, "restricted self-attention B1 h16 n8192 d64, radius 256 "
                           "(r = 513 keys per row), bf16"),
}

MASK_NONE, MASK_KEY_PADDING, MASK_CAUSAL, MASK_RESTRICTED = 0, 1, 2, 4


def generator(seed: int) -> torch.Generator:
    return torch.Generator("cpu").manual_seed(seed)


def randn(g: torch.Generator, shape, dtype=torch.bfloat16) -> torch.Tensor:
    """N(0,1) fp32 draw, then one rounding to `dtype` (RNE for bf16)."""
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def randint(g: torch.Generator, lo: int, hi: int, n: int) -> torch.Tensor:
    """Inclusive discrete uniform on [lo, hi], int32."""
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64).to(torch.int32)


def make(name: str) -> dict:
    """Return the CPU tensors of a named workload (see WORKLOADS).

    Each entry of the returned dict is one attention call:
      {"calls": [ {"Q","K","V","mask","q_lens","kv_lens","scale"} ... ]}
    (restricted calls also carry "radius"),
    or, for the decode workload, {"q","Kcache","Vcache","kv_lens","scale"}.
    """
    num, _ = WORKLOADS[name]
    g = generator(1000 + num)
    if name == "tiny_fp32":
        shp = (1, 8, 16, D)
        Q, K, V = (randn(g, shp, torch.float32) for _ in range(3))
        return {"calls": [dict(Q=Q, K=K, V=V, mask=MASK_NONE, q_lens=None,
                               kv_lens=None, scale=0.125)]}
    if name == "encoder_base":
        L = randint(g, 8, 128, 32)
        shp = (32, 8, 128, D)
        Q, K, V = (randn(g, shp) for _ in range(3))
        return {"calls": [dict(Q=Q, K=K, V=V, mask=MASK_KEY_PADDING, q_lens=L,
                               kv_lens=L, scale=0.125)]}
    if name == "decoder_big":
        Ls = randint(g, 16, 160, 32)
        shp = (32, 16, 128, D)
        Qs, Ks, Vs = (randn(g, shp) for _ in range(3))
        Qc = randn(g, shp)
        Ke, Ve = (randn(g, (32, 16, 160, D)) for _ in range(2))
        return {"calls": [
            dict(Q=Qs, K=Ks, V=Vs, mask=MASK_CAUSAL, q_lens=None, kv_lens=None, scale=0.125),
            dict(Q=Qc, K=Ke, V=Ve, mask=MASK_KEY_PADDING, q_lens=None, kv_lens=Ls, scale=0.125),
        ]}
    if name == "long_causal":
        shp = (1, 16, 8192, D)
        Q, K, V = (randn(g, shp) for _ in range(3))
        return {"calls": [dict(Q=Q, K=K, V=V, mask=MASK_CAUSAL, q_lens=None,
                               kv_lens=None, scale=0.125)]}
    if name == "kv_decode":
        L = randint(g, 1, 4096, 64)
        q = randn(g, (64, 16, 1, D))
        Kc = randn(g, (64, 16, 4096, D))
        Vc = randn(g, (64, 16, 4096, D))
        return dict(q=q, Kcache=Kc, Vcache=Vc, kv_lens=L, scale=0.125)
    if name == "long_restricted":
        shp = (1, 16, 8192, D)
        Q, K, V = (randn(g, shp) for _ in range(3))
        return {"calls": [dict(Q=Q, K=K, V=V, mask=MASK_RESTRICTED, q_lens=None,
                               kv_lens=None, scale=0.125, radius=256)]}
    raise KeyError(name)


def allowed_pairs(mask: int, n_q: int, n_k: int, B: int, q_lens=None, kv_lens=None,
                  radius=None) -> int:
    """Number of (query, key) pairs a call actually computes, summed over the
    batch (per head).  Counting only: rows beyond q_len and keys beyond kv_len,
    in the causal future or (restricted) farther than radius from the query
    are excluded.  Used for the flop and byte models.
    """
    total = 0
    for b in range(B):
        ql = n_q if q_lens is None else int(q_lens[b])
        kl = n_k if not (mask & MASK_KEY_PADDING) else int(kv_lens[b])
        ql = max(0, min(ql, n_q))
        kl = max(0, min(kl, n_k))
        if mask & MASK_RESTRICTED:
            # row i sees keys max(0, i - radius) .. min(i or i + radius, kl - 1)
            for i in range(ql):
                hi = min(i if mask & MASK_CAUSAL else i + radius, kl - 1)
                total += max(0, hi - max(0, i - radius) + 1)
        elif mask & MASK_CAUSAL:
            # row i sees keys j <= i and j < kl
            total += sum(min(i + 1, kl) for i in range(ql))
        else:
            total += ql * kl
    return total
