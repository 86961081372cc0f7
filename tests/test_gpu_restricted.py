"""GPU parity of restricted self-attention (attn_forward_restricted): each
query attends only to the keys within `radius` of its position (the past
half under the causal mask), against the fp64 oracle on the same inputs.

Cases reach every kernel that serves the restricted mask -- the short-key
bf16 kernel (n <= 256), the bf16 band kernel (any longer n: 512-row
workgroups whose first key tile may lie before key 0) and the fp32 path --
with radii from 0 (a row sees only itself) through windows narrower than,
equal to and wider than a 64-key tile, to radii beyond the sequence (windows
wider than a workgroup's rows); key padding and padded query rows, including
rows whose whole window lies beyond kv_len; ragged n; several workgroups per
head; B*h divisible by 8 or not.  Bars are those of the plain forward (2e-2 max abs and
1e-2 relative L2 on bf16, 1e-5 relative on fp32) and of the log-sum-exp
(1e-2 bf16, 1e-5 fp32).  The bench's long_restricted workload (B1 h16
n=8192, radius 256) is checked on sampled rows at full size.
"""
import zlib

import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle.attn_oracle as orc
import workloads
from gpu_util import check, np64, say

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
R = ha.ATTN_MASK_RESTRICTED

CASES = {
    # name: (dtype, B, H, n, radius, causal, key padding, query padding)
    "short_r0": (BF16, 2, 3, 200, 0, False, False, False),
    "short_r5_pad": (BF16, 3, 2, 200, 5, False, True, True),
    "short_r40_causal_pad": (BF16, 2, 4, 256, 40, True, True, False),
    "short_r63_causal": (BF16, 1, 8, 190, 63, True, False, True),
    "short_r300": (BF16, 1, 2, 130, 300, False, False, False),
    "band_300_r17_pad": (BF16, 2, 2, 300, 17, False, True, True),
    "band_1000_r100_causal_pad": (BF16, 1, 3, 1000, 100, True, True, True),
    "band_1000_r64": (BF16, 2, 2, 1000, 64, False, False, False),
    "band_777_r1_pad": (BF16, 1, 8, 777, 1, False, True, False),
    "band_600_r600_causal": (BF16, 1, 2, 600, 600, True, False, False),
    "band_700_r255_causal": (BF16, 1, 2, 700, 255, True, False, True),
    "band_520_r0_pad": (BF16, 2, 2, 520, 0, False, True, False),
    "band_2100_r700_pad": (BF16, 2, 4, 2100, 700, False, True, True),
    "band_1300_r257_causal": (BF16, 1, 5, 1300, 257, True, False, False),
    "band_1600_r1000": (BF16, 1, 2, 1600, 1000, False, False, False),
    "f32_200_r7_pad": (F32, 2, 2, 200, 7, False, True, True),
    "f32_700_r70_causal_pad": (F32, 1, 2, 700, 70, True, True, False),
    "f32_130_r200": (F32, 1, 3, 130, 200, False, False, False),
}


def _make(name, dtype, B, H, n, kpad, qpad):
    g = workloads.generator(zlib.crc32(name.encode()) % 10000)
    ql = workloads.randint(g, 1, n, B) if qpad else None
    kl = None
    if kpad:
        kl = workloads.randint(g, 1, n, B)
        kl[0] = max(1, n // 5)  # rows past n / 5 have windows with no valid key
    Q, K, V = (workloads.randn(g, (B, H, n, 64), dtype) for _ in range(3))
    return Q, K, V, ql, kl


def _run(Q, K, V, radius, mask, ql, kl, scale, lse=None):
    out = ha.forward_restricted(Q.cuda(), K.cuda(), V.cuda(), radius, mask_kind=mask,
                                q_lens=None if ql is None else ql.cuda(),
                                kv_lens=None if kl is None else kl.cuda(), scale=scale, lse=lse)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", sorted(CASES))
def test_restricted_parity(name):
    dtype, B, H, n, radius, causal, kpad, qpad = CASES[name]
    Q, K, V, ql, kl = _make(name, dtype, B, H, n, kpad, qpad)
    mask = R | (ha.ATTN_MASK_CAUSAL if causal else 0) | (ha.ATTN_MASK_KEY_PADDING if kpad else 0)
    say(f"[restricted {name}] B{B} h{H} n{n} radius {radius} mask {mask}")
    lse = torch.empty((B, H, n), dtype=torch.float32, device="cuda")
    out = _run(Q, K, V, radius, mask, ql, kl, 0.125, lse)
    qn = None if ql is None else ql.numpy()
    kn = None if kl is None else kl.numpy()
    ref = orc.attention(np64(Q), np64(K), np64(V), mask_kind=mask, q_lens=qn, kv_lens=kn,
                        scale=0.125, radius=radius)
    check(np64(out), ref, dtype, name)
    lref = orc.row_logsumexp(np64(Q), np64(K), mask_kind=mask, q_lens=qn, kv_lens=kn,
                             scale=0.125, radius=radius)
    got = lse.cpu().double().numpy()
    assert np.array_equal(np.isinf(got), np.isinf(lref))
    fin = np.isfinite(lref)
    if fin.any():
        err = float(np.abs(got[fin] - lref[fin]).max())
        say(f"  lse max err {err:.3e}")
        assert err <= (1e-2 if dtype == BF16 else 1e-5)
    # without the LSE output the same kernel writes the same O
    assert torch.equal(out, _run(Q, K, V, radius, mask, ql, kl, 0.125))


@pytest.mark.parametrize("dtype,n", [(BF16, 200), (BF16, 900), (F32, 300)], ids=["short", "band", "fp32"])
def test_radius_zero_returns_v(dtype, n):
    """radius 0: a row's only key is itself, so O_i = V_i exactly (its weight
    is exactly 1); rows at or past kv_len have no key and are 0."""
    Q, K, V, _, _ = _make(f"r0_{n}", dtype, 2, 2, n, False, False)
    kl = torch.tensor([n, n // 3], dtype=torch.int32)
    say(f"[radius 0 {dtype} n{n}]")
    out = _run(Q, K, V, 0, R | ha.ATTN_MASK_KEY_PADDING, None, kl, 0.125).cpu()
    assert torch.equal(out[0], V[0])
    assert torch.equal(out[1, :, :n // 3], V[1, :, :n // 3])
    assert torch.all(out[1, :, n // 3:] == 0)


def test_restricted_deterministic():
    Q, K, V, _, _ = _make("det", BF16, 1, 4, 1500, False, False)
    say("[restricted determinism n1500 radius 200]")
    a = _run(Q, K, V, 200, R, None, None, 0.125)
    b = _run(Q, K, V, 200, R, None, None, 0.125)
    assert torch.equal(a, b)


@pytest.mark.parametrize("causal", [False, True], ids=["centred", "causal"])
def test_long_restricted_sampled(causal):
    """The bench's long_restricted workload (B1 h16 n=8192, radius 256) in
    the launch configuration the bench times, and its causal variant, on
    sampled rows: both edges of the sequence, both sides of every workgroup
    and tile boundary near the window edges, and random rows of every head."""
    c = workloads.make("long_restricted")["calls"][0]
    mask = c["mask"] | (ha.ATTN_MASK_CAUSAL if causal else 0)
    radius = c["radius"]
    say(f"[long_restricted causal={causal}] Q(1,16,8192,64) radius {radius}")
    out = np64(_run(c["Q"], c["K"], c["V"], radius, mask, None, None, c["scale"]))
    rng = np.random.default_rng(6)
    n = 8192
    picks = {0, 1, 63, 64, 255, 256, 257, radius - 1, radius, radius + 1, n - radius - 1, n - radius,
             n - 257, n - 256, n - 65, n - 64, n - 2, n - 1}
    picks |= {int(x) for x in rng.integers(0, n, 24)}
    rows = [(0, h, i) for h in range(16) for i in sorted(picks) if (i + h) % 2 == 0 or h == 0]
    ref = orc.attention(np64(c["Q"]), np64(c["K"]), np64(c["V"]), mask_kind=mask,
                        scale=c["scale"], rows=rows, radius=radius)
    got = np.stack([out[r] for r in rows])
    want = np.stack([ref[r] for r in rows])
    check(got, want, BF16, f"long_restricted causal={causal} ({len(rows)} rows)")
