"""GPU parity at the full benchmark sizes, element by element: every output
of the HIP path in the launch configuration the bench times against the fp64
oracle on the same seeded inputs (no sampling).

* long_causal (B1 h16 n=8192, causal): all 131,072 rows of O;
* long_restricted (B1 h16 n=8192, radius 256), centred and causal windows:
  all rows of O;
* long_causal backward: dQ, dK and dV of two complete heads (0 and 15),
  every element, from the bench's seeded dO.

Bars as everywhere for bf16 (max-abs 2e-2 and relative L2 1e-2 on O; the
backward's 2e-2 max(1, max|ref|) and relative L2 2e-2 per gradient).  The
oracle runs single-threaded NumPy row by row, about 15-20 s for the whole
long_causal forward on the GPU machine's host.
"""
import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle.attn_oracle as orc
import workloads
from gpu_util import check, np64, say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def _oracle_full(c, mask, radius=None):
    return orc.attention(np64(c["Q"]), np64(c["K"]), np64(c["V"]), mask_kind=mask, scale=c["scale"],
                         radius=radius)


def test_long_causal_all_rows():
    c = workloads.make("long_causal")["calls"][0]
    say("[long_causal full] B1 h16 n8192 causal, all 131072 rows")
    out = ha.forward(c["Q"].cuda(), c["K"].cuda(), c["V"].cuda(), mask_kind=c["mask"], scale=c["scale"])
    torch.cuda.synchronize()
    check(np64(out), _oracle_full(c, c["mask"]), BF16, "long_causal (all rows)")


@pytest.mark.parametrize("causal", [False, True], ids=["centred", "causal"])
def test_long_restricted_all_rows(causal):
    c = workloads.make("long_restricted")["calls"][0]
    r = c["radius"]
    mask = c["mask"] | (ha.ATTN_MASK_CAUSAL if causal else 0)
    say(f"[long_restricted full causal={causal}] B1 h16 n8192 radius {r}, all rows")
    out = ha.forward_restricted(c["Q"].cuda(), c["K"].cuda(), c["V"].cuda(), r, mask_kind=mask,
                                scale=c["scale"])
    torch.cuda.synchronize()
    check(np64(out), _oracle_full(c, mask, radius=r), BF16, f"long_restricted causal={causal} (all rows)")


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


@pytest.mark.parametrize("head", [0, 15])
def test_long_causal_backward_full_head(head):
    """The bench's long_causal backward (all 16 heads on the GPU, as timed);
    every element of dQ, dK and dV of one head against the oracle's
    backward of that head."""
    c = workloads.make("long_causal")["calls"][0]
    dO = workloads.randn(workloads.generator(1200), tuple(c["Q"].shape), BF16)
    Qd, Kd, Vd, dOd = (t.cuda() for t in (c["Q"], c["K"], c["V"], dO))
    say(f"[long_causal backward full head {head}] B1 h16 n8192 causal")
    lse = torch.empty((1, 16, 8192), dtype=torch.float32, device="cuda")
    O = ha.forward(Qd, Kd, Vd, mask_kind=c["mask"], scale=c["scale"], lse=lse)
    dQ, dK, dV = (np64(t) for t in ha.backward(Qd, Kd, Vd, O, dOd, lse, mask_kind=c["mask"],
                                                 scale=c["scale"]))
    sl = lambda t: np64(t)[:, head:head + 1]
    rQ, rK, rV = orc.attention_backward(sl(c["Q"]), sl(c["K"]), sl(c["V"]), sl(dO), mask_kind=c["mask"],
                                        scale=c["scale"])
    for name, got, ref in (("dQ", dQ, rQ), ("dK", dK, rK), ("dV", dV, rV)):
        _check_grad(got[:, head:head + 1], ref, f"{name} head {head} (all 8192 rows)")
