"""GPU tests of the KV-cache steps around attn_decode: attn_cache_append
against the oracle (bit-exact: it is a copy), and whole decode loops --
self-attention decoding token by token with appends, and cross-attention
decoding against a fixed encoder cache -- against the oracle's forward rows.
The pages fix what a cached step must compute: the same rows as recomputing
attention over the whole prefix (sj-techlog page, KV cache section; kimjiil
page §3.7); cross attention reads the encoder's K/V (kimjiil page §3.2.3).
"""
import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle.attn_oracle as orc
import workloads
from gpu_util import check, np64, say

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
DTYPES = pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])


def _rand(g, shape, dtype):
    return workloads.randn(g, shape, dtype)


@DTYPES
@pytest.mark.parametrize("n_new,lens", [
    (1, [1, 7, 4096, 2]),            # one token per step, full cache
    (3, [3, 10, 4096, 700]),         # a prefill block of 3 rows
    (2, [1, 0, 4097, 5000]),         # destinations outside the cache are skipped
])
def test_cache_append_matches_oracle(dtype, n_new, lens):
    g = workloads.generator(700 + n_new)
    B, H, n_max = 4, 3, 4096
    Kc, Vc = _rand(g, (B, H, n_max, 64), dtype), _rand(g, (B, H, n_max, 64), dtype)
    Kn, Vn = _rand(g, (B, H, n_new, 64), dtype), _rand(g, (B, H, n_new, 64), dtype)
    kl = torch.tensor(lens, dtype=torch.int32)
    say(f"[append {dtype} n_new={n_new} lens={lens}]")
    Kd, Vd = Kc.cuda(), Vc.cuda()
    ha.cache_append(Kn.cuda(), Vn.cuda(), Kd, Vd, kl.cuda())
    torch.cuda.synchronize()
    Kref, Vref = orc.cache_append(np64(Kc), np64(Vc), np64(Kn), np64(Vn), kl.numpy())
    assert np.array_equal(np64(Kd.cpu()), Kref)
    assert np.array_equal(np64(Vd.cpu()), Vref)


@DTYPES
def test_incremental_decode_equals_causal_forward(dtype):
    """Token-by-token decoding with appends reproduces the causal rows."""
    g = workloads.generator(711)
    B, H, n, n_max = 3, 4, 70, 96
    Q, K, V = (_rand(g, (B, H, n, 64), dtype) for _ in range(3))
    Qd, Kd, Vd = Q.cuda(), K.cuda(), V.cuda()
    Kc = torch.full((B, H, n_max, 64), float("nan"), dtype=dtype, device="cuda")
    Vc = torch.full((B, H, n_max, 64), float("nan"), dtype=dtype, device="cuda")
    say(f"[incremental decode {dtype}] B{B} H{H} n{n}")
    outs = []
    for t in range(n):
        kl = torch.full((B,), t + 1, dtype=torch.int32, device="cuda")
        ha.cache_append(Kd[:, :, t:t + 1].contiguous(), Vd[:, :, t:t + 1].contiguous(), Kc, Vc, kl)
        outs.append(ha.decode(Qd[:, :, t:t + 1].contiguous(), Kc, Vc, kl, scale=0.125))
    torch.cuda.synchronize()
    got = np64(torch.cat(outs, dim=2))
    ref = orc.attention(np64(Q), np64(K), np64(V), mask_kind=orc.MASK_CAUSAL, scale=0.125)
    check(got, ref, dtype, "incremental decode")
    # the cache now holds exactly the sequence's K/V
    assert torch.equal(Kc[:, :, :n], Kd) and torch.equal(Vc[:, :, :n], Vd)


@DTYPES
def test_cross_attention_decode(dtype):
    """Decoder queries against a fixed encoder cache with ragged source
    lengths (decoder_big's cross-attention shape, one step)."""
    g = workloads.generator(712)
    B, H, n_src = 32, 16, 160
    src = torch.randint(16, n_src + 1, (B,), generator=g, dtype=torch.int32)
    q = _rand(g, (B, H, 1, 64), dtype)
    Ke, Ve = _rand(g, (B, H, n_src, 64), dtype), _rand(g, (B, H, n_src, 64), dtype)
    say(f"[cross-attention decode {dtype}]")
    out = ha.decode(q.cuda(), Ke.cuda(), Ve.cuda(), src.cuda(), scale=0.125)
    torch.cuda.synchronize()
    ref = orc.attention(np64(q), np64(Ke), np64(Ve), mask_kind=orc.MASK_KEY_PADDING,
                        kv_lens=src.numpy(), scale=0.125)
    check(np64(out), ref, dtype, "cross-attention decode")
    fwd = ha.forward(q.cuda(), Ke.cuda(), Ve.cuda(), mask_kind=1, kv_lens=src.cuda(), scale=0.125)
    check(np64(fwd), ref, dtype, "cross-attention forward, n_q = 1")


def test_cache_append_kv_decode_shape():
    """The append at the decode workload's shape (B64 h16, cache 4096), in the
    launch configuration the bench times, then the decode reads it."""
    w = workloads.make("kv_decode")
    g = workloads.generator(713)
    B, H = w["q"].shape[:2]
    kn, vn = _rand(g, (B, H, 1, 64), BF16), _rand(g, (B, H, 1, 64), BF16)
    kl = w["kv_lens"]
    say("[append at kv_decode shape]")
    Kc, Vc = w["Kcache"].cuda(), w["Vcache"].cuda()
    ha.cache_append(kn.cuda(), vn.cuda(), Kc, Vc, kl.cuda())
    torch.cuda.synchronize()
    rows = (kl - 1).long()
    bi = torch.arange(B)
    Kh, Vh = Kc.cpu(), Vc.cpu()
    assert torch.equal(Kh[bi, :, rows], kn[:, :, 0])
    assert torch.equal(Vh[bi, :, rows], vn[:, :, 0])
    # every other row is untouched
    Kh[bi, :, rows] = w["Kcache"][bi, :, rows]
    Vh[bi, :, rows] = w["Vcache"][bi, :, rows]
    assert torch.equal(Kh, w["Kcache"]) and torch.equal(Vh, w["Vcache"])
