"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

* The five named workloads (workloads.py) in the launch configuration the
  bench times: tiny_fp32, encoder_base and decoder_big against the oracle on
  every element; long_causal on sampled rows (first/last rows of tiles, both
  sides of every boundary, random rows, every head); kv_decode on every
  (b, h) pair.
* Ragged and edge cases at sizes the oracle finishes in seconds that still
  span several tiles and a ragged tail, in both dtypes: n not a multiple of
  the tile sizes, lengths 0 / 1 / n, padded query rows, n_k = 0, negative
  and zero scale, out-of-range lengths (clamped), B*h divisible by 8 or not
  (the two workgroup orders), and shapes that reach each bf16 kernel (short
  key range, 4-wave, paired).
"""
import zlib

import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle.attn_oracle as orc
import workloads
from gpu_util import check, dev, np64, say

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def _oracle_call(c, rows=None):
    return orc.attention(np64(c["Q"]), np64(c["K"]), np64(c["V"]), mask_kind=c["mask"],
                         q_lens=None if c["q_lens"] is None else c["q_lens"].numpy(),
                         kv_lens=None if c["kv_lens"] is None else c["kv_lens"].numpy(),
                         scale=c["scale"], rows=rows)


def _gpu_call(c):
    out = ha.forward(dev(c["Q"]), dev(c["K"]), dev(c["V"]), mask_kind=c["mask"],
                     q_lens=dev(c["q_lens"]), kv_lens=dev(c["kv_lens"]), scale=c["scale"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["tiny_fp32", "encoder_base", "decoder_big"])
def test_workload_full(name):
    w = workloads.make(name)
    for k, c in enumerate(w["calls"]):
        say(f"[{name} call {k}] Q{tuple(c['Q'].shape)} K{tuple(c['K'].shape)} mask={c['mask']}")
        out = _gpu_call(c)
        ref = _oracle_call(c)
        check(np64(out), ref, c["Q"].dtype, f"{name}[{k}]")


def test_workload_long_causal_sampled():
    w = workloads.make("long_causal")
    c = w["calls"][0]
    say("[long_causal] Q(1,16,8192,64) causal")
    out = np64(_gpu_call(c))
    n = 8192
    rng = np.random.default_rng(5)
    base = [0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, 1000, 4095, 4096, 8064, 8190, 8191]
    rows = []
    for h in range(16):
        picks = set(base) | set(rng.integers(0, n, 16).tolist())
        rows += [(0, h, int(i)) for i in sorted(picks)]
    ref = _oracle_call(c, rows=rows)
    got = np.stack([out[r] for r in rows])
    exp = np.stack([ref[r] for r in rows])
    check(got, exp, BF16, f"long_causal ({len(rows)} sampled rows)")


def test_workload_kv_decode_all_pairs():
    w = workloads.make("kv_decode")
    say("[kv_decode] q(64,16,1,64) cache(64,16,4096,64)")
    out = ha.decode(dev(w["q"]), dev(w["Kcache"]), dev(w["Vcache"]), dev(w["kv_lens"]),
                    scale=w["scale"])
    torch.cuda.synchronize()
    out = np64(out)
    refs = []
    for b in range(64):
        refs.append(orc.decode(np64(w["q"][b:b + 1]), np64(w["Kcache"][b:b + 1]),
                               np64(w["Vcache"][b:b + 1]), w["kv_lens"][b:b + 1].numpy(),
                               scale=w["scale"]))
    check(out, np.concatenate(refs), BF16, "kv_decode (all 1024 pairs)")


# ----------------------------------------------------------------- ragged cases
def _case(seed, B, H, n_q, n_k, mask, dtype, q_lens=None, kv_lens=None, scale=0.125):
    g = workloads.generator(seed)
    Q = workloads.randn(g, (B, H, n_q, 64), dtype)
    K = workloads.randn(g, (B, H, n_k, 64), dtype)
    V = workloads.randn(g, (B, H, n_k, 64), dtype)
    ql = None if q_lens is None else torch.tensor(q_lens, dtype=torch.int32)
    kl = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32)
    return dict(Q=Q, K=K, V=V, mask=mask, q_lens=ql, kv_lens=kl, scale=scale)


RAGGED = {
    # id: (B, H, n_q, n_k, mask, q_lens, kv_lens, scale)
    "single_element": (1, 1, 1, 1, 0, None, None, 0.125),
    "short_q_long_k": (2, 2, 5, 70, 0, None, None, 0.125),
    "causal_200": (2, 3, 200, 200, 2, None, None, 0.125),
    "kpad_130x333": (3, 2, 130, 333, 1, [130, 7, 0], [333, 64, 1], 0.125),
    "kpad_lens_0_1": (4, 1, 65, 129, 1, [65, 65, 1, 33], [0, 1, 128, 129], 0.125),
    "causal_kpad_257": (2, 2, 257, 257, 3, [257, 100], [257, 63], 0.125),
    "xcd_order_64": (8, 1, 64, 64, 0, None, None, 0.125),
    "xcd_order_causal_300": (16, 1, 300, 300, 2, None, None, 0.125),
    "negative_scale": (2, 2, 96, 96, 2, None, None, -0.3),
    "zero_scale": (2, 2, 40, 90, 1, None, [90, 17], 0.0),
    "big_scale": (1, 2, 70, 70, 0, None, None, 2.0),
    "cross_128x160": (4, 2, 128, 160, 1, None, [16, 160, 99, 128], 0.125),
    # n_k <= 256: the short-key-range bf16 kernel (all of K/V loaded at once)
    "short_causal_256": (2, 2, 256, 256, 2, None, None, 0.125),
    "short_kpad_77x255": (3, 2, 77, 255, 1, [77, 10, 0], [255, 193, 1], 0.125),
    "short_long_q_900x256": (1, 2, 900, 256, 1, [900], [200], 0.125),
    "short_big_scale_150": (1, 2, 150, 150, 3, [150], [150], 2.0),
    "short_single_key_col_300x1": (2, 2, 300, 1, 0, None, None, 0.125),
    "short_one_tile_512x64": (1, 2, 512, 64, 0, None, None, 0.125),
    "short_k_600x5": (1, 2, 600, 5, 0, None, None, 0.125),
    # 256 < n_k, n_q < 512: the 4-wave bf16 kernel (keys streamed in tiles)
    "fourwave_causal_384": (1, 2, 384, 384, 2, None, None, 0.125),
    "fourwave_kpad_200x400": (2, 2, 200, 400, 1, [200, 50], [400, 257], 0.125),
    # n_q >= 512: the paired 8-wave bf16 kernel (256 query rows per workgroup)
    "pair_causal_1000": (1, 2, 1000, 1000, 2, None, None, 0.125),
    "pair_none_600x700": (2, 2, 600, 700, 0, None, None, 0.125),
    "pair_kpad_520x777": (3, 2, 520, 777, 1, [520, 300, 0], [777, 65, 1], 0.125),
    "pair_causal_kpad_768": (2, 2, 768, 768, 3, [768, 700], [768, 129], 0.125),
    "pair_xcd_causal_512": (8, 1, 512, 512, 2, None, None, 0.125),
    "pair_kv_257_600x257": (1, 2, 600, 257, 1, [600], [257], 0.125),
    "pair_big_scale_600": (1, 2, 600, 600, 0, None, None, 2.0),
    "pair_negative_scale_540": (1, 2, 540, 540, 2, None, None, -0.3),
    "pair_zero_scale_530x300": (2, 1, 530, 300, 1, None, [300, 44], 0.0),
}


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("cid", sorted(RAGGED))
def test_ragged(cid, dtype):
    B, H, n_q, n_k, mask, ql, kl, scale = RAGGED[cid]
    c = _case(zlib.crc32(cid.encode()) % 10000, B, H, n_q, n_k, mask, dtype, ql, kl, scale)
    say(f"[ragged {cid} {dtype}] B{B} H{H} nq{n_q} nk{n_k} mask{mask}")
    out = _gpu_call(c)
    check(np64(out), _oracle_call(c), dtype, cid)


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])
def test_no_keys_gives_zero_rows(dtype):
    say(f"[n_k=0 {dtype}]")
    Q = torch.randn(2, 3, 17, 64, device="cuda").to(dtype)
    K = torch.empty(2, 3, 0, 64, device="cuda", dtype=dtype)
    out = torch.full_like(Q, float("nan"))
    ha.forward(Q, K, K.clone(), out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    kl = torch.zeros(2, dtype=torch.int32, device="cuda")
    Kf = torch.randn(2, 3, 9, 64, device="cuda").to(dtype)
    out = torch.full_like(Q, float("nan"))
    ha.forward(Q, Kf, Kf.clone(), mask_kind=1, kv_lens=kl, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])
def test_out_of_range_lengths_are_clamped(dtype):
    """Lengths outside [0, n] are a precondition violation; the kernels clamp
    them, so they behave as 0 / n and never read outside the buffers."""
    c = _case(77, 3, 2, 50, 70, 1, dtype, q_lens=[50, 50, 50], kv_lens=[70, 70, 0])
    say(f"[clamped lengths {dtype}]")
    ref = _gpu_call(c)
    c2 = dict(c)
    c2["q_lens"] = torch.tensor([10 ** 6, 50, 50], dtype=torch.int32)
    c2["kv_lens"] = torch.tensor([10 ** 6, 70, -5], dtype=torch.int32)
    out = _gpu_call(c2)
    assert torch.equal(out, ref)


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])
def test_decode_ragged(dtype):
    B, H, n_max = 6, 3, 700
    g = workloads.generator(4242)
    q = workloads.randn(g, (B, H, 1, 64), dtype)
    Kc = workloads.randn(g, (B, H, n_max, 64), dtype)
    Vc = workloads.randn(g, (B, H, n_max, 64), dtype)
    lens = torch.tensor([0, 1, 256, 257, 700, 513], dtype=torch.int32)
    say(f"[decode ragged {dtype}] B{B} H{H} n_max{n_max}")
    out = ha.decode(dev(q), dev(Kc), dev(Vc), dev(lens), scale=0.125)
    torch.cuda.synchronize()
    ref = orc.decode(np64(q), np64(Kc), np64(Vc), lens.numpy(), scale=0.125)
    check(np64(out), ref, dtype, "decode ragged")
    assert np.all(np64(out)[0] == 0.0)  # kv_len = 0 row


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])
def test_decode_matches_forward_last_row(dtype):
    """The cached step equals the causal forward's last row (kimjiil page
    §3.7: caching changes the work, not the result) -- both on the GPU,
    within the parity bar of each against the oracle."""
    B, H, n = 3, 2, 300
    c = _case(99, B, H, n, n, 2, dtype)
    full = _gpu_call(c)
    lens = torch.tensor([n, 150, 1], dtype=torch.int32)
    q = torch.stack([c["Q"][b, :, int(lens[b]) - 1] for b in range(B)])[:, :, None].contiguous()
    say(f"[decode vs forward {dtype}]")
    out = ha.decode(dev(q), dev(c["K"]), dev(c["V"]), dev(lens), scale=0.125)
    torch.cuda.synchronize()
    got = np64(out)[:, :, 0]
    ref = np.stack([np64(full)[b, :, int(lens[b]) - 1] for b in range(B)])
    tol = 4e-2 if dtype == BF16 else 2e-6
    assert np.abs(got - ref).max() <= tol * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("mask,scale", [(0, 0.125), (2, 0.125), (0, 1.0), (1, 0.125)],
                         ids=["none", "causal", "scale1", "kpad"])
def test_logit_spikes(dtype, mask, scale):
    """Planted keys whose logits are far above the rest (exponents beyond 2^64
    at the pages' scale), late in long rows, and rows whose logits on the
    first 20 keys are far below zero (their other logits are ordinary): the
    softmax must stay stable wherever the spike lands.  Rows whose every
    logit is far below zero are covered by test_gpu_extreme.py."""
    B, H, n = 2, 2, 700
    c = _case(31337, B, H, n, n, mask, dtype, kv_lens=[700, 555] if mask & 1 else None,
              scale=scale)
    Q, K = c["Q"].float(), c["K"].float()
    for b in range(B):
        for h in range(H):
            for i, j in ((10, 400), (300, 650), (5, 64), (600, 599)):
                K[b, h, j] = 9.0 * Q[b, h, i]          # q_i . k_j = 9 |q_i|^2 ~ 576
            Q[b, h, 640:660] = -6.0 * K[b, h, :20].mean(0)  # far below zero on keys 0..19
    c["Q"], c["K"] = Q.to(dtype), K.to(dtype)
    say(f"[logit spikes {dtype} mask{mask} scale{scale}]")
    out = _gpu_call(c)
    check(np64(out), _oracle_call(c), dtype, f"spikes mask{mask} scale{scale}")
