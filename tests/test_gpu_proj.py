"""GPU parity of the multi-head projections (kimjiil page §3.2.2) against the
fp64 oracle on the same bf16 inputs, and of the whole multi-head sub-layer
(projections + attention + output projection) built from the library's
entry points.  Weights are seeded N(0, 1/d_model) draws (no trained weights
are needed: the projections are plain linear maps).  The shapes reach every
tile the launcher picks (256 x 192, 320 x 128 and 128 x 128) and every tile
order: XCD rectangles of all,
1/2, 1/4 or 1/8 of the feature blocks, a last partial group of token blocks,
and the plain order for grids the split does not divide.

Bars: the attention bars of gpu_util (max abs <= 2e-2 and relative L2 <=
1e-2), and for a projection alone the bound its arithmetic fixes: products of
bf16 values are exact, the fp32 sum of K <= 1024 terms errs by far less than
1e-4 at these scales, and the bf16 rounding of the output by at most half an
ulp, 2^-8 |y|: so |y_gpu - y_ref| <= 2^-8 |y_ref| + 1e-4 element by element.
"""
import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle.attn_oracle as orc
import workloads
from gpu_util import check, np64, say


def check_rounding(out, ref, what):
    err = np.abs(out - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4
    worst = float((err / bound).max())
    say(f"  {what}: worst error / bound = {worst:.3f}")
    assert worst <= 1.0, what

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def _weights(g, rows, d_model):
    return (torch.randn((rows, d_model), generator=g) / d_model ** 0.5).to(BF16)


@pytest.mark.parametrize("B,n,h,n_out", [
    (32, 128, 8, 3),    # Transformer-base self-attention: Q, K, V
    (32, 160, 16, 2),   # Transformer-big encoder output -> K, V of cross attention
    (3, 77, 3, 1),      # ragged tokens (M = 231) and features (N = 192)
    (1, 1, 1, 3),       # one token, one head
    (32, 128, 16, 3),   # Transformer-big self-attention Q, K, V (256 x 192 tiles)
    (41, 97, 13, 3),    # 256 x 192 tiles, ragged M = 3977, N = 2496
    (2, 128, 16, 3),    # few tokens: each XCD takes 1/8 of the feature blocks
    (8, 128, 16, 2),    # XCD rectangles of 1/4 of the feature blocks by 1/2 of the tokens
    (144, 128, 16, 1),  # 9 token blocks per XCD: a full group of 8 and a group of 1
    (32, 128, 40, 1),   # 256 x 192 tiles with a partial last feature block (N = 2560)
])
def test_head_projection(B, n, h, n_out):
    g = workloads.generator(800 + n + h)
    d = 64 * h
    X = workloads.randn(g, (B, n, d), BF16)
    W = _weights(g, n_out * d, d)
    say(f"[head projection B{B} n{n} h{h} n_out{n_out}]")
    outs = ha.head_projection(X.cuda(), W.cuda(), h)
    torch.cuda.synchronize()
    refs = orc.head_projection(np64(X), np64(W), h)
    for j, (o, r) in enumerate(zip(outs, refs)):
        check(np64(o), r, BF16, f"projection {j}")
        check_rounding(np64(o), r, f"projection {j}")


@pytest.mark.parametrize("B,n,h", [(32, 128, 8), (32, 128, 16), (3, 77, 3), (1, 1, 1),
                                   (16, 257, 38),   # ragged M = 4112, N = 2432 (not a multiple of 128)
                                   (64, 128, 32),   # M = 8192, N = 2048
                                   (16, 256, 48)])  # 256 x 192 tiles, M = 4096, N = 3072
def test_output_projection(B, n, h):
    g = workloads.generator(900 + n + h)
    d = 64 * h
    O = workloads.randn(g, (B, h, n, 64), BF16)
    Wo = _weights(g, d, d)
    say(f"[output projection B{B} n{n} h{h}]")
    Y = ha.output_projection(O.cuda(), Wo.cuda())
    torch.cuda.synchronize()
    ref = orc.output_projection(np64(O), np64(Wo))
    check(np64(Y), ref, BF16, "output projection")
    check_rounding(np64(Y), ref, "output projection")


@pytest.mark.parametrize("case", ["self_causal", "cross_kpad"])
def test_multi_head_sublayer(case):
    """Transformer-big decoder shapes (h 16, d_model 1024), two batch entries:
    causal self-attention, and cross attention from 128 queries to 160
    encoder positions with source padding."""
    g = workloads.generator(1001 if case == "self_causal" else 1002)
    B, h, d = 2, 16, 1024
    n_q, n_k = (128, 128) if case == "self_causal" else (128, 160)
    Xq = workloads.randn(g, (B, n_q, d), BF16)
    Xkv = Xq if case == "self_causal" else workloads.randn(g, (B, n_k, d), BF16)
    Wq, Wkv, Wo = _weights(g, d, d), _weights(g, 2 * d, d), _weights(g, d, d)
    src = None if case == "self_causal" else torch.tensor([160, 37], dtype=torch.int32)
    say(f"[multi-head {case}]")
    (Q,) = ha.head_projection(Xq.cuda(), Wq.cuda(), h)
    K, V = ha.head_projection(Xkv.cuda(), Wkv.cuda(), h)
    mask = ha.ATTN_MASK_CAUSAL if case == "self_causal" else ha.ATTN_MASK_KEY_PADDING
    O = ha.forward(Q, K, V, mask_kind=mask, kv_lens=None if src is None else src.cuda(), scale=0.125)
    Y = ha.output_projection(O, Wo.cuda())
    torch.cuda.synchronize()
    ref = orc.multi_head_attention(np64(Xq), np64(Xkv), np64(Wq), np64(Wkv), np64(Wo), h,
                                   mask_kind=orc.MASK_CAUSAL if src is None else orc.MASK_KEY_PADDING,
                                   kv_lens=None if src is None else src.numpy(), scale=0.125)
    check(np64(Y), ref, BF16, f"multi-head {case}")
