"""GPU invariants of the HIP path that hold at any size, each from the pages:

* rows of the softmax sum to 1: a ones column of V comes out as ones;
* masked keys get weight exactly 0: NaN in padded K/V rows (and in padded Q
  rows) leaves the output bit for bit unchanged, in both dtypes, forward and
  decode; finite changes to a row's causal future leave it bit for bit
  unchanged;
* one allowed key reproduces its value row exactly;
* Q = 0 gives the mean of the allowed value rows;
* jointly permuting K and V rows leaves O unchanged (order-blindness);
* repeated runs are bitwise identical (no race in LDS staging).
"""
import numpy as np
import pytest
import torch

import head_attention_amd as ha
import workloads
from gpu_util import say

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
DTYPES = pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])


def _rand(seed, shape, dtype):
    return workloads.randn(workloads.generator(seed), shape, dtype).cuda()


# Sequence lengths that reach each bf16 kernel: short key range (n_k <= 256),
# 4-wave (n_k > 256, n_q < 512) and paired (n_q >= 512).
SIZES = pytest.mark.parametrize("n", [150, 333, 520])


@DTYPES
@SIZES
@pytest.mark.parametrize("mask", [0, 1, 2, 3])
def test_ones_column_sums_to_one(dtype, mask, n):
    B, H = 3, 4
    Q, K, V = (_rand(s, (B, H, n, 64), dtype) for s in (1, 2, 3))
    V[..., 5] = 1.0
    kl = torch.tensor([n, 100, 1], dtype=torch.int32, device="cuda") if mask & 1 else None
    say(f"[ones column {dtype} mask{mask} n{n}]")
    O = ha.forward(Q, K, V, mask_kind=mask, kv_lens=kl, scale=0.125).float()
    # Every kernel sums exactly the bf16 weights it multiplies by V (fp32 sums in
    # two orders, differing by far less than half a bf16 step at 1), so the bf16
    # column is exactly 1.0.
    tol = 0.0 if dtype == BF16 else 1e-6
    assert torch.all((O[..., 5] - 1).abs() <= tol), (O[..., 5] - 1).abs().max()


@DTYPES
@pytest.mark.parametrize("n", [200, 300, 600])
@pytest.mark.parametrize("mask", [1, 3])
def test_nan_padding_is_invisible(dtype, mask, n):
    B, H = 4, 2
    Q, K, V = (_rand(s, (B, H, n, 64), dtype) for s in (4, 5, 6))
    lens = [n, 65, 1, (2 * n) // 3]
    kl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ql = kl.clone()
    say(f"[NaN padding {dtype} mask{mask} n{n}]")
    O1 = ha.forward(Q, K, V, mask_kind=mask, q_lens=ql, kv_lens=kl, scale=0.125)
    Q2, K2, V2 = Q.clone(), K.clone(), V.clone()
    for b, L in enumerate(lens):
        Q2[b, :, L:] = float("nan")
        K2[b, :, L:] = float("nan")
        V2[b, :, L:] = float("nan")
    O2 = ha.forward(Q2, K2, V2, mask_kind=mask, q_lens=ql, kv_lens=kl, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)
    for b, L in enumerate(lens):
        assert torch.all(O1[b, :, L:] == 0)


@DTYPES
def test_nan_padding_is_invisible_decode(dtype):
    B, H, n = 5, 3, 1000
    q = _rand(7, (B, H, 1, 64), dtype)
    Kc, Vc = _rand(8, (B, H, n, 64), dtype), _rand(9, (B, H, n, 64), dtype)
    lens = [1000, 1, 256, 257, 640]
    kl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    say(f"[NaN padding decode {dtype}]")
    O1 = ha.decode(q, Kc, Vc, kl, scale=0.125)
    K2, V2 = Kc.clone(), Vc.clone()
    for b, L in enumerate(lens):
        K2[b, :, L:] = float("nan")
        V2[b, :, L:] = float("nan")
    O2 = ha.decode(q, K2, V2, kl, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)


@DTYPES
@pytest.mark.parametrize("n", [200, 400, 600])
def test_causal_future_is_invisible(dtype, n):
    B, H = 2, 3
    Q, K, V = (_rand(s, (B, H, n, 64), dtype) for s in (10, 11, 12))
    say(f"[causal future {dtype} n{n}]")
    O1 = ha.forward(Q, K, V, mask_kind=2, scale=0.125)
    for i in (0, 63, 64, 127, 128, 199, 250, 511):
        if i >= n - 1:
            continue
        Q2, K2, V2 = Q.clone(), K.clone(), V.clone()
        Q2[:, :, i + 1:] = 1000.0
        K2[:, :, i + 1:] = -3000.0
        V2[:, :, i + 1:] = 5000.0
        O2 = ha.forward(Q2, K2, V2, mask_kind=2, scale=0.125)
        torch.cuda.synchronize()
        assert torch.equal(O1[:, :, :i + 1], O2[:, :, :i + 1]), i


@DTYPES
@pytest.mark.parametrize("n", [130, 300, 530])
def test_single_allowed_key_returns_its_value(dtype, n):
    B, H = 3, 2
    Q, K, V = (_rand(s, (B, H, n, 64), dtype) for s in (13, 14, 15))
    kl = torch.ones(B, dtype=torch.int32, device="cuda")
    say(f"[one key {dtype} n{n}]")
    O = ha.forward(Q, K, V, mask_kind=1, kv_lens=kl, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(O, V[:, :, :1].expand_as(O))
    Oc = ha.forward(Q, K, V, mask_kind=2, scale=0.125)
    assert torch.equal(Oc[:, :, 0], V[:, :, 0])
    Od = ha.decode(Q[:, :, :1].contiguous(), K, V, kl, scale=0.125)
    assert torch.equal(Od[:, :, 0], V[:, :, 0])


@DTYPES
def test_zero_query_gives_mean_of_values(dtype):
    B, H, n = 2, 2, 200
    K, V = _rand(16, (B, H, n, 64), dtype), _rand(17, (B, H, n, 64), dtype)
    Q = torch.zeros_like(K)
    kl = torch.tensor([200, 77], dtype=torch.int32, device="cuda")
    say(f"[zero query {dtype}]")
    O = ha.forward(Q, K, V, mask_kind=1, kv_lens=kl, scale=0.125).double()
    for b, L in enumerate((200, 77)):
        mean = V[b, :, :L].double().mean(dim=1, keepdim=True)
        tol = 2e-2 if dtype == BF16 else 1e-6
        assert (O[b] - mean).abs().max() <= tol


@DTYPES
def test_joint_key_value_permutation(dtype):
    B, H, n = 2, 2, 256
    Q, K, V = (_rand(s, (B, H, n, 64), dtype) for s in (18, 19, 20))
    p = torch.randperm(n, generator=torch.Generator().manual_seed(3)).cuda()
    say(f"[permutation {dtype}]")
    O1 = ha.forward(Q, K, V, scale=0.125).double()
    O2 = ha.forward(Q, K[:, :, p].contiguous(), V[:, :, p].contiguous(), scale=0.125).double()
    tol = 2e-2 if dtype == BF16 else 1e-6
    assert (O1 - O2).abs().max() <= tol


@pytest.mark.parametrize("which", ["forward_causal", "forward_kpad", "forward_short", "decode"])
def test_bitwise_determinism(which):
    say(f"[determinism {which}]")
    if which == "decode":
        q = _rand(21, (8, 4, 1, 64), BF16)
        Kc, Vc = _rand(22, (8, 4, 2000, 64), BF16), _rand(23, (8, 4, 2000, 64), BF16)
        kl = torch.tensor([2000, 1, 3, 999, 1024, 1025, 64, 1500], dtype=torch.int32,
                          device="cuda")
        runs = [ha.decode(q, Kc, Vc, kl, scale=0.125) for _ in range(5)]
    elif which == "forward_short":
        Q, K, V = (_rand(s, (32, 8, 128, 64), BF16) for s in (27, 28, 29))
        kl = torch.randint(8, 129, (32,), generator=torch.Generator().manual_seed(4)).to(torch.int32).cuda()
        runs = [ha.forward(Q, K, V, mask_kind=1, q_lens=kl, kv_lens=kl, scale=0.125) for _ in range(5)]
    else:
        Q, K, V = (_rand(s, (2, 8, 1024, 64), BF16) for s in (24, 25, 26))
        mask = 2 if which == "forward_causal" else 1
        kl = torch.tensor([1024, 555], dtype=torch.int32, device="cuda") if mask == 1 else None
        runs = [ha.forward(Q, K, V, mask_kind=mask, kv_lens=kl, scale=0.125) for _ in range(5)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert torch.equal(r, runs[0])
