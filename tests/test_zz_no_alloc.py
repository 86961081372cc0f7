"""attn_decode_noalloc, the decode step for callers that cannot allocate:
through the C ABI, two calls in a row (the second smaller, on the scratch the
first one left behind) against the existing attn_decode on the same inputs --
the same kernels, so the outputs must agree bit for bit -- and against the
fp64 oracle at the bf16 / fp32 parity bars."""
import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle.attn_oracle as orc
import workloads
from gpu_util import check, dev, np64, say

pytestmark = pytest.mark.gpu


def _inputs(seed, B, H, n_max, lens, dtype):
    g = workloads.generator(seed)
    q = workloads.randn(g, (B, H, 1, 64), dtype)
    Kc = workloads.randn(g, (B, H, n_max, 64), dtype)
    Vc = workloads.randn(g, (B, H, n_max, 64), dtype)
    return q, Kc, Vc, torch.tensor(lens, dtype=torch.int32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_noalloc_decode_matches_decode_twice(dtype):
    calls = [
        # a large call first (many splits per row, lengths up to the cache size) ...
        (8101, 16, 8, 3000, [3000, 1, 257, 2999, 1500, 256, 2048, 700, 1023, 2500, 3, 1800, 2222, 64, 999, 2871]),
        # ... then a smaller one, whose partials sit in scratch the first call filled
        (8102, 3, 2, 600, [600, 1, 300]),
    ]
    for seed, B, H, n_max, lens in calls:
        q, Kc, Vc, kl = _inputs(seed, B, H, n_max, lens, dtype)
        say(f"[decode_noalloc {dtype}] B{B} H{H} n_max{n_max}")
        qd, Kd, Vd, kd = dev(q), dev(Kc), dev(Vc), dev(kl)
        out = torch.full_like(qd, float("nan"))
        ha.decode_noalloc(qd, Kd, Vd, kd, scale=0.125, out=out)
        ref_gpu = ha.decode(qd, Kd, Vd, kd, scale=0.125)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_gpu), "attn_decode_noalloc differs from attn_decode"
        ref = orc.decode(np64(q), np64(Kc), np64(Vc), kl.numpy(), scale=0.125)
        check(np64(out), ref, dtype, f"decode_noalloc B{B} H{H} n_max{n_max}")


def test_noalloc_decode_full_size_workload():
    """The kv_decode workload (B 64, h 16, cache 4096) fits the scratch."""
    w = workloads.make("kv_decode")
    say("[decode_noalloc kv_decode]")
    qd, Kd, Vd, kd = dev(w["q"]), dev(w["Kcache"]), dev(w["Vcache"]), dev(w["kv_lens"])
    out = torch.empty_like(qd)
    ha.decode_noalloc(qd, Kd, Vd, kd, scale=w["scale"], out=out)
    ref_gpu = ha.decode(qd, Kd, Vd, kd, scale=w["scale"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref_gpu)


def test_noalloc_decode_rejects_oversized_layout():
    q = torch.zeros((64, 16, 1, 64), dtype=torch.bfloat16, device="cuda")
    Kc = torch.zeros((64, 16, 7937, 64), dtype=torch.bfloat16, device="cuda")
    kl = torch.ones(64, dtype=torch.int32, device="cuda")
    with pytest.raises(ha.AttnError, match="SCRATCH_LIMIT"):
        ha.decode_noalloc(q, Kc, Kc, kl)
