"""GPU parity of the training path: the per-row log-sum-exp the forward
returns for the backward (attn_forward_lse), and attn_backward's dQ, dK, dV
against the fp64 oracle (oracle.attention_backward, itself pinned against
torch autograd and finite differences) on the same bf16 inputs, for every
mask kind, padded query rows, cross attention with n_q != n_k, and shapes
that span several tiles with a ragged tail.

Bars.  LSE: |lse_gpu - lse_ref| <= 1e-2 on bf16 inputs (the row sum is
taken over bf16-rounded weights, a relative error of at most 2^-8, i.e.
4e-3 in the log) and <= 1e-5 on the fp32 path.  Gradients (bf16 outputs):
relative L2 error <= 2e-2 and max |err| <= 2e-2 max(1, max |ref|) per
tensor; the weights and ds are rounded to bf16 (2^-9 relative) before their
products and D = dO . O uses the bf16-rounded O, so errors of a few 1e-3
relative are expected.
"""
import zlib

import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle.attn_oracle as orc
import workloads
from gpu_util import np64, say

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def _case(name, B, H, n_q, n_k, mask, ql, kl, dtype=BF16, scale=0.125):
    g = workloads.generator(zlib.crc32(name.encode()) % 10000)
    Q, K, V = (workloads.randn(g, (B, H, n, 64), dtype) for n in (n_q, n_k, n_k))
    dO = workloads.randn(g, (B, H, n_q, 64), dtype)
    ql = None if ql is None else torch.tensor(ql, dtype=torch.int32)
    kl = None if kl is None else torch.tensor(kl, dtype=torch.int32)
    return Q, K, V, dO, ql, kl, scale


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("n_q,n_k,mask", [(128, 128, 3), (128, 160, 1), (300, 300, 2), (600, 600, 3)])
def test_forward_lse(dtype, n_q, n_k, mask):
    name = f"lse{n_q}x{n_k}m{mask}"
    kl = [n_k, n_k // 3] if mask & 1 else None
    Q, K, V, _, ql, kl, scale = _case(name, 2, 3, n_q, n_k, mask, [n_q, n_q - 7], kl, dtype)
    say(f"[forward lse {dtype} {n_q}x{n_k} mask{mask}]")
    lse = torch.empty((2, 3, n_q), dtype=torch.float32, device="cuda")
    O = ha.forward(Q.cuda(), K.cuda(), V.cuda(), mask_kind=mask, q_lens=ql.cuda(),
                   kv_lens=None if kl is None else kl.cuda(), scale=scale, lse=lse)
    O_plain = ha.forward(Q.cuda(), K.cuda(), V.cuda(), mask_kind=mask, q_lens=ql.cuda(),
                         kv_lens=None if kl is None else kl.cuda(), scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(O, O_plain)  # the lse output does not change O
    ref = orc.row_logsumexp(np64(Q), np64(K), mask_kind=mask, q_lens=ql.numpy(),
                            kv_lens=None if kl is None else kl.numpy(), scale=scale)
    got = lse.cpu().double().numpy()
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    fin = np.isfinite(ref)
    err = float(np.abs(got[fin] - ref[fin]).max())
    say(f"  lse max err {err:.3e}")
    assert err <= (1e-2 if dtype == BF16 else 1e-5)


BWD = {
    # name: (B, H, n_q, n_k, mask, q_lens, kv_lens, scale)
    "none_128": (2, 4, 128, 128, 0, None, None, 0.125),
    "kpad_128": (3, 2, 128, 128, 1, [128, 90, 17], [128, 90, 17], 0.125),
    "causal_128": (2, 4, 128, 128, 2, None, None, 0.125),
    "causal_kpad_200": (2, 2, 200, 200, 3, [200, 131], [200, 131], 0.125),
    "cross_128x160": (3, 2, 128, 160, 1, None, [160, 16, 99], 0.125),
    "causal_330": (1, 2, 330, 330, 2, None, None, 0.125),
    "none_70x257": (1, 2, 70, 257, 0, None, None, 0.125),
    "negative_scale_96": (1, 2, 96, 96, 2, None, None, -0.3),
    "one_key": (2, 1, 40, 40, 1, [40, 40], [1, 2], 0.125),
    # several ring wraps of the streamed tiles, B*h a multiple of 8 (heads
    # grouped per XCD) and not
    "causal_2000_h8": (1, 8, 2000, 2000, 2, None, None, 0.125),
    "causal_kpad_1100": (2, 4, 1100, 1100, 3, [1100, 517], [1100, 517], 0.125),
    "none_700x1300": (1, 3, 700, 1300, 0, None, None, 0.125),
    # the paired dQ kernel (n_q >= 512): sign of scale folded into Q, and
    # key padding down to one key and to one 64-key tile
    "negative_scale_causal_600": (1, 2, 600, 600, 2, None, None, -0.3),
    "kpad_600": (3, 2, 600, 600, 1, [600, 333, 515], [600, 1, 64], 0.125),
}


def _check_grad(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref)) / nref if nref > 0 else float(np.linalg.norm(got))
    bound = 2e-2 * max(1.0, float(np.abs(ref).max()))
    say(f"  {what}: max_abs={float(err.max()):.3e} (bound {bound:.2e}) rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got)), what
    assert float(err.max()) <= bound, what
    assert rel <= 2e-2, what


@pytest.mark.parametrize("cid", sorted(BWD))
def test_backward(cid):
    B, H, n_q, n_k, mask, ql, kl, scale = BWD[cid]
    Q, K, V, dO, ql, kl, scale = _case(cid, B, H, n_q, n_k, mask, ql, kl, BF16, scale)
    say(f"[backward {cid}]")
    d = lambda t: None if t is None else t.cuda()
    Qd, Kd, Vd, dOd = d(Q), d(K), d(V), d(dO)
    lse = torch.empty((B, H, n_q), dtype=torch.float32, device="cuda")
    O = ha.forward(Qd, Kd, Vd, mask_kind=mask, q_lens=d(ql), kv_lens=d(kl), scale=scale, lse=lse)
    dQ, dK, dV = ha.backward(Qd, Kd, Vd, O, dOd, lse, mask_kind=mask, q_lens=d(ql), kv_lens=d(kl),
                             scale=scale)
    dQ2, dK2, dV2 = ha.backward(Qd, Kd, Vd, O, dOd, lse, mask_kind=mask, q_lens=d(ql), kv_lens=d(kl),
                                scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(dQ, dQ2) and torch.equal(dK, dK2) and torch.equal(dV, dV2)  # deterministic
    rQ, rK, rV = orc.attention_backward(np64(Q), np64(K), np64(V), np64(dO), mask_kind=mask,
                                        q_lens=None if ql is None else ql.numpy(),
                                        kv_lens=None if kl is None else kl.numpy(), scale=scale)
    _check_grad(np64(dQ), rQ, "dQ")
    _check_grad(np64(dK), rK, "dK")
    _check_grad(np64(dV), rV, "dV")
    if ql is not None:  # padded query rows: zero dQ
        for b in range(B):
            assert torch.all(dQ[b, :, int(ql[b]):] == 0)
    if kl is not None:  # excluded keys: zero dK, dV
        for b in range(B):
            assert torch.all(dK[b, :, int(kl[b]):] == 0) and torch.all(dV[b, :, int(kl[b]):] == 0)


BWD_RESTRICTED = {
    # name: (B, H, n, radius, causal, key padding, query padding)
    "r17_pad_300": (1, 4, 300, 17, False, True, True),
    "r100_causal_700_h8": (2, 4, 700, 100, True, False, False),
    "r0_kpad_520": (1, 2, 520, 0, False, True, False),
    "r300_causal_200": (1, 2, 200, 300, True, False, True),
    "r64_1000": (1, 3, 1000, 64, False, False, False),
    "r1_causal_kpad_333": (2, 2, 333, 1, True, True, True),
}


@pytest.mark.parametrize("cid", sorted(BWD_RESTRICTED))
def test_backward_restricted(cid):
    """attn_backward_restricted against the oracle's backward over the band
    of restricted self-attention (kimjiil page §4, Table 1), from the LSE of
    attn_forward_restricted with the same radius."""
    B, H, n, radius, causal, kpad, qpad = BWD_RESTRICTED[cid]
    mask = ha.ATTN_MASK_RESTRICTED | (ha.ATTN_MASK_CAUSAL if causal else 0) | (ha.ATTN_MASK_KEY_PADDING if kpad else 0)
    ql = [n - 13 * (b + 1) for b in range(B)] if qpad else None
    kl = [max(1, n // (b + 2)) for b in range(B)] if kpad else None
    Q, K, V, dO, ql, kl, scale = _case(cid, B, H, n, n, mask, ql, kl, BF16, 0.125)
    say(f"[backward restricted {cid}] B{B} h{H} n{n} radius {radius} mask {mask}")
    d = lambda t: None if t is None else t.cuda()
    Qd, Kd, Vd, dOd = d(Q), d(K), d(V), d(dO)
    lse = torch.empty((B, H, n), dtype=torch.float32, device="cuda")
    O = ha.forward_restricted(Qd, Kd, Vd, radius, mask_kind=mask, q_lens=d(ql), kv_lens=d(kl), scale=scale,
                              lse=lse)
    grads = ha.backward(Qd, Kd, Vd, O, dOd, lse, mask_kind=mask, q_lens=d(ql), kv_lens=d(kl), scale=scale,
                        radius=radius)
    again = ha.backward(Qd, Kd, Vd, O, dOd, lse, mask_kind=mask, q_lens=d(ql), kv_lens=d(kl), scale=scale,
                        radius=radius)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(grads, again))  # deterministic
    refs = orc.attention_backward(np64(Q), np64(K), np64(V), np64(dO), mask_kind=mask,
                                  q_lens=None if ql is None else ql.numpy(),
                                  kv_lens=None if kl is None else kl.numpy(), scale=scale, radius=radius)
    for name, got, ref in zip(("dQ", "dK", "dV"), grads, refs):
        _check_grad(np64(got), ref, name)
    if kl is not None:  # keys past kv_len: zero dK, dV
        for b in range(B):
            assert torch.all(grads[1][b, :, int(kl[b]):] == 0) and torch.all(grads[2][b, :, int(kl[b]):] == 0)


def _bench_dO(c):
    """The incoming gradient the bench draws for a workload call (seeded,
    same shape as O)."""
    g = workloads.generator(1200)
    return workloads.randn(g, tuple(c["Q"].shape), torch.bfloat16)


def test_long_causal_backward_sampled():
    """The bench's long_causal backward (B1 h16 n=8192 causal) at full size
    in the launch configuration the bench times, on outputs the oracle can
    compute alone: dQ of sampled rows (row i's gradient depends only on its
    own row over keys 0..i), and dK, dV of the last 128 keys (only rows
    8064..8191 see them), each from a batch of one-row problems with key
    padding kv_len = i + 1 -- the causal row written as a padded one."""
    c = workloads.make("long_causal")["calls"][0]
    dO = _bench_dO(c)
    Qd, Kd, Vd, dOd = (t.cuda() for t in (c["Q"], c["K"], c["V"], dO))
    say("[long_causal backward] B1 h16 n8192 causal")
    lse = torch.empty((1, 16, 8192), dtype=torch.float32, device="cuda")
    O = ha.forward(Qd, Kd, Vd, mask_kind=2, scale=c["scale"], lse=lse)
    dQ, dK, dV = (np64(t) for t in ha.backward(Qd, Kd, Vd, O, dOd, lse, mask_kind=2, scale=c["scale"]))
    Q, K, V, G = (np64(t) for t in (c["Q"], c["K"], c["V"], dO))
    n = 8192
    heads = (0, 5, 15)
    tail = list(range(n - 128, n))
    rng = np.random.default_rng(12)
    picks = sorted({0, 1, 63, 64, 4095, 4096} | {int(x) for x in rng.integers(0, n - 128, 10)})
    for h in heads:
        rows = picks + tail
        # one batch entry per row i: its query, all keys, kv_len = i + 1
        Qb = Q[0, h][rows][:, None, None, :]
        Gb = G[0, h][rows][:, None, None, :]
        Kb = np.broadcast_to(K[0, h], (len(rows), 1, n, 64))
        Vb = np.broadcast_to(V[0, h], (len(rows), 1, n, 64))
        kl = np.array([i + 1 for i in rows])
        rQ, rK, rV = orc.attention_backward(Qb, Kb, Vb, Gb, mask_kind=orc.MASK_KEY_PADDING, kv_lens=kl,
                                            scale=c["scale"])
        _check_grad(dQ[0, h][rows], rQ[:, 0, 0], f"dQ head {h} ({len(rows)} rows)")
        # the tail rows are all the rows that see the last 128 keys
        nt = len(tail)
        _check_grad(dK[0, h, n - 128:], rK[-nt:, 0].sum(axis=0)[n - 128:], f"dK head {h} (last 128 keys)")
        _check_grad(dV[0, h, n - 128:], rV[-nt:, 0].sum(axis=0)[n - 128:], f"dV head {h} (last 128 keys)")


@pytest.mark.parametrize("causal", [False, True], ids=["centred", "causal"])
def test_long_restricted_backward_sampled(causal):
    """Restricted backward at the long_restricted size (B1 h16 n=8192,
    radius 256) on positions the oracle can isolate: around position j only
    positions j - 2r .. j + 2r interact with j (its own window and the
    windows of the rows that see it), so the oracle's restricted backward
    on that slice gives dQ, dK and dV of j exactly."""
    c = workloads.make("long_restricted")["calls"][0]
    r = c["radius"]
    mask = c["mask"] | (ha.ATTN_MASK_CAUSAL if causal else 0)
    dO = _bench_dO(c)
    Qd, Kd, Vd, dOd = (t.cuda() for t in (c["Q"], c["K"], c["V"], dO))
    say(f"[long_restricted backward causal={causal}] B1 h16 n8192 radius {r}")
    lse = torch.empty((1, 16, 8192), dtype=torch.float32, device="cuda")
    O = ha.forward_restricted(Qd, Kd, Vd, r, mask_kind=mask, scale=c["scale"], lse=lse)
    dQ, dK, dV = (np64(t) for t in ha.backward(Qd, Kd, Vd, O, dOd, lse, mask_kind=mask, scale=c["scale"],
                                                 radius=r))
    Q, K, V, G = (np64(t) for t in (c["Q"], c["K"], c["V"], dO))
    n = 8192
    for h, j in ((0, 0), (3, 300), (7, 4100), (15, n - 1), (9, 2 * r)):
        lo, hi = max(0, j - 2 * r), min(n, j + 2 * r + 1)
        sl = lambda x: x[:, h:h + 1, lo:hi]
        rQ, rK, rV = orc.attention_backward(sl(Q), sl(K), sl(V), sl(G), mask_kind=mask, scale=c["scale"],
                                            radius=r)
        k = j - lo
        for name, got, ref in (("dQ", dQ, rQ), ("dK", dK, rK), ("dV", dV, rV)):
            _check_grad(got[0, h, j][None], ref[0, 0, k][None], f"{name} head {h} position {j}")
