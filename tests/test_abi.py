"""C-ABI tests that need no GPU: the library loads, exports every function
include/headattn.h declares, and rejects bad arguments with the documented
status codes before any HIP call (so nothing here launches a kernel)."""
import ctypes
import glob
import os
import re

import pytest

import head_attention_amd as ha
from head_attention_amd import attn_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULLP, SHAPE, DTYPE, MASK, LENS, SCALE, WORK, HIP, SCRATCH = range(10)
BF16, F32 = 0, 1
FAKE = 0x1000  # never dereferenced: every call below fails validation first


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w \*]*?\b(attn_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("attn_forward", "attn_forward_lse", "attn_forward_restricted",
              "attn_backward", "attn_backward_restricted", "attn_backward_workspace_bytes",
              "attn_decode", "attn_decode_noalloc", "attn_cache_append", "attn_head_projection",
              "attn_output_projection", "attn_decode_workspace_bytes",
              "attn_status_string", "attn_last_hip_error"):
        assert n in names, names


def test_library_exports_every_declared_symbol():
    L = ha.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings():
    for code in range(10):
        s = ha.status_string(code)
        assert s.startswith(ha._binding.STATUS_NAMES[code]), s
    assert "unknown" in ha.status_string(99)
    assert ha.lib().attn_last_hip_error() == b"hipSuccess"


def fwd(layout, mask=0, q=FAKE, k=FAKE, v=FAKE, o=FAKE + 64, ql=None, kl=None, scale=0.125):
    return ha.lib().attn_forward(q, k, v, layout, mask, ql, kl, scale, o, None)


def lay(B=2, h=3, nq=16, nk=16, d=64, dt=BF16):
    return attn_layout(B, h, nq, nk, d, dt)


@pytest.mark.parametrize("layout,code", [
    (lay(d=32), SHAPE), (lay(d=128), SHAPE), (lay(B=-1), SHAPE), (lay(nq=-5), SHAPE),
    (lay(dt=2), DTYPE), (lay(dt=-1), DTYPE),
    (lay(B=2 ** 30, h=2 ** 30, nq=2 ** 20), SHAPE),
    # a (b, h) slice holds at most 2^24 - 1 rows (32-bit byte ranges of 128 B rows)
    (lay(B=1, h=1, nq=2 ** 24, nk=16), SHAPE), (lay(B=1, h=1, nq=16, nk=2 ** 24), SHAPE),
    (lay(B=1, h=1, nq=2 ** 25, nk=2 ** 25), SHAPE),
])
def test_forward_bad_layout(layout, code):
    assert fwd(layout) == code


def test_forward_validation_order_and_codes():
    L = lay()
    assert fwd(L, mask=4) == MASK
    assert fwd(L, mask=-1) == MASK
    assert fwd(lay(nq=8, nk=16), mask=2) == MASK       # causal needs n_q == n_k
    assert fwd(L, mask=0, kl=FAKE) == MASK              # kv_lens without key padding
    assert fwd(L, mask=1, kl=None) == NULLP             # key padding without kv_lens
    assert fwd(L, scale=float("inf")) == SCALE
    assert fwd(L, scale=float("nan")) == SCALE
    assert fwd(L, q=None) == NULLP
    assert fwd(L, o=None) == NULLP
    assert fwd(L, k=None) == NULLP
    assert fwd(L, v=None) == NULLP
    assert fwd(L, o=FAKE) == SHAPE                      # output aliases Q
    assert fwd(lay(dt=F32), mask=3, kl=None) == NULLP


def test_forward_empty_calls_are_noops():
    # nothing to write: OK without touching any pointer or the device
    assert fwd(lay(B=0), q=None, k=None, v=None, o=None) == OK
    assert fwd(lay(h=0), q=None, k=None, v=None, o=None) == OK
    assert fwd(lay(nq=0, nk=5), q=None, k=None, v=None, o=None) == OK


def dec(layout, q=FAKE, k=FAKE, v=FAKE, kl=FAKE + 32, o=FAKE + 64, ws=FAKE + 128, wsb=None,
        scale=0.125):
    if wsb is None:
        wsb = ha.lib().attn_decode_workspace_bytes(layout)
    return ha.lib().attn_decode(q, k, v, layout, kl, scale, o, ws, wsb, None)


def test_decode_workspace_bytes():
    L = ha.lib()
    # (B*h) records per split, splits of 256 keys, record = (m, l, acc[64]) fp32
    assert L.attn_decode_workspace_bytes(attn_layout(64, 16, 1, 4096, 64, BF16)) == 64 * 16 * 16 * 66 * 4
    assert L.attn_decode_workspace_bytes(attn_layout(1, 1, 1, 257, 64, F32)) == 2 * 66 * 4
    assert L.attn_decode_workspace_bytes(attn_layout(1, 1, 1, 0, 64, F32)) == 66 * 4
    assert L.attn_decode_workspace_bytes(attn_layout(1, 1, 2, 64, 64, F32)) == 0   # n_q != 1
    assert L.attn_decode_workspace_bytes(attn_layout(1, 1, 1, 64, 32, F32)) == 0   # d != 64
    assert ha.decode_workspace_bytes(64, 16, 4096) == 64 * 16 * 16 * 66 * 4


def test_decode_validation():
    L = attn_layout(4, 2, 1, 300, 64, BF16)
    assert dec(attn_layout(4, 2, 2, 300, 64, BF16)) == SHAPE
    assert dec(attn_layout(4, 2, 1, 300, 16, BF16)) == SHAPE
    assert dec(attn_layout(1, 1, 1, 2 ** 24, 64, BF16)) == SHAPE   # cache above 2^24 - 1 rows
    assert dec(attn_layout(4, 2, 1, 300, 64, 7)) == DTYPE
    assert dec(L, scale=float("-inf")) == SCALE
    assert dec(L, q=None) == NULLP
    assert dec(L, kl=None) == NULLP
    assert dec(L, k=None) == NULLP
    assert dec(L, o=None) == NULLP
    assert dec(L, ws=None) == WORK
    assert dec(L, wsb=ha.lib().attn_decode_workspace_bytes(L) - 1) == WORK
    assert dec(L, o=FAKE) == SHAPE
    assert dec(attn_layout(0, 2, 1, 300, 64, BF16), q=None, o=None, kl=None) == OK


def dec_noalloc(layout, q=FAKE, k=FAKE, v=FAKE, kl=FAKE + 32, o=FAKE + 64, scale=0.125):
    return ha.lib().attn_decode_noalloc(q, k, v, layout, kl, scale, o, None)


def test_decode_noalloc_validation():
    """The allocation-free decode validates like attn_decode, and rejects a
    layout whose partials exceed the static scratch before any HIP call."""
    L = attn_layout(4, 2, 1, 300, 64, BF16)
    assert dec_noalloc(attn_layout(4, 2, 2, 300, 64, BF16)) == SHAPE
    assert dec_noalloc(attn_layout(4, 2, 1, 300, 16, BF16)) == SHAPE
    assert dec_noalloc(attn_layout(4, 2, 1, 300, 64, 7)) == DTYPE
    assert dec_noalloc(L, scale=float("nan")) == SCALE
    assert dec_noalloc(L, q=None) == NULLP
    assert dec_noalloc(L, kl=None) == NULLP
    assert dec_noalloc(L, o=FAKE) == SHAPE
    assert dec_noalloc(attn_layout(0, 2, 1, 300, 64, BF16), q=None, o=None, kl=None) == OK
    # 64 x 16 heads: partials fit up to n_max = 7936 (31 splits of 256 keys)
    lim = ha.DECODE_NOALLOC_MAX_BYTES
    assert ha.lib().attn_decode_workspace_bytes(attn_layout(64, 16, 1, 7936, 64, BF16)) <= lim
    assert ha.lib().attn_decode_workspace_bytes(attn_layout(64, 16, 1, 7937, 64, BF16)) > lim
    assert dec_noalloc(attn_layout(64, 16, 1, 7937, 64, BF16)) == SCRATCH
    assert dec_noalloc(attn_layout(1, 16, 1, 508161, 64, F32)) == SCRATCH
    assert "ATTN_ERR_SCRATCH_LIMIT" in ha.status_string(SCRATCH)
    hdr = open(os.path.join(ROOT, "include", "headattn.h"), encoding="utf-8").read()
    m = re.search(r"#define ATTN_DECODE_NOALLOC_MAX_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == lim


def app(layout, kn=FAKE, vn=FAKE + 32, kc=FAKE + 64, vc=FAKE + 96, kl=FAKE + 128):
    return ha.lib().attn_cache_append(kn, vn, kc, vc, layout, kl, None)


def test_cache_append_validation():
    L = attn_layout(4, 2, 1, 300, 64, BF16)
    assert app(attn_layout(4, 2, 1, 300, 16, BF16)) == SHAPE
    assert app(attn_layout(4, 2, -1, 300, 64, BF16)) == SHAPE
    assert app(attn_layout(4, 2, 1, 300, 64, 5)) == DTYPE
    for kw in ("kn", "vn", "kc", "vc", "kl"):
        assert app(L, **{kw: None}) == NULLP, kw
    assert app(L, kc=FAKE) == SHAPE        # new rows alias the cache
    assert app(L, vc=FAKE + 64) == SHAPE   # K and V caches alias
    # nothing to append: OK without touching any pointer or the device
    assert app(attn_layout(0, 2, 1, 300, 64, BF16), kn=None, vn=None, kc=None, vc=None, kl=None) == OK
    assert app(attn_layout(4, 2, 0, 300, 64, F32), kn=None, vn=None, kc=None, vc=None, kl=None) == OK


def test_projection_validation():
    L = ha.lib()
    lay_ = attn_layout(2, 8, 128, 0, 64, BF16)
    hp = lambda lay, n_out=3, x=FAKE, w=FAKE + 16, o0=FAKE + 32, o1=FAKE + 48, o2=FAKE + 64: \
        L.attn_head_projection(x, w, lay, n_out, o0, o1, o2, None)
    assert hp(attn_layout(2, 8, 128, 0, 64, F32)) == DTYPE
    assert hp(attn_layout(2, 8, 128, 0, 32, BF16)) == SHAPE
    assert hp(lay_, n_out=0) == SHAPE and hp(lay_, n_out=4) == SHAPE
    assert hp(lay_, x=None) == NULLP and hp(lay_, w=None) == NULLP
    assert hp(lay_, o2=None) == NULLP
    assert hp(lay_, o1=FAKE) == SHAPE          # output aliases X
    assert hp(lay_, o2=FAKE + 32) == SHAPE     # two outputs alias
    assert hp(attn_layout(2, 8, 1 << 24, 0, 64, BF16)) == SHAPE  # X over 2 GiB
    assert hp(attn_layout(0, 8, 128, 0, 64, BF16), x=None, w=None, o0=None, o1=None, o2=None) == OK
    op = lambda lay, o=FAKE, w=FAKE + 16, y=FAKE + 32: L.attn_output_projection(o, w, lay, y, None)
    assert op(attn_layout(2, 8, 128, 0, 64, F32)) == DTYPE
    assert op(lay_, y=None) == NULLP and op(lay_, o=None) == NULLP and op(lay_, w=None) == NULLP
    assert op(lay_, y=FAKE) == SHAPE
    assert op(attn_layout(2, 8, 0, 0, 64, BF16), o=None, w=None, y=None) == OK


def test_forward_lse_and_backward_validation():
    L = ha.lib()
    lay_ = attn_layout(2, 3, 16, 16, 64, BF16)
    # forward_lse: LSE required for a non-empty call; LSE must not alias O
    assert L.attn_forward_lse(FAKE, FAKE + 16, FAKE + 32, lay_, 0, None, None, 0.125, FAKE + 48, None, None) == NULLP
    assert L.attn_forward_lse(FAKE, FAKE + 16, FAKE + 32, lay_, 0, None, None, 0.125, FAKE + 48, FAKE + 48,
                              None) == SHAPE
    assert L.attn_forward_lse(None, None, None, attn_layout(0, 3, 16, 16, 64, BF16), 0, None, None, 0.125,
                              None, None, None) == OK
    # per (b, h): n_q rounded up to 64 rows, two fp32 values per row
    assert L.attn_backward_workspace_bytes(lay_) == 2 * 3 * 64 * 24
    assert L.attn_backward_workspace_bytes(attn_layout(1, 2, 130, 16, 64, BF16)) == 2 * 192 * 24
    assert L.attn_backward_workspace_bytes(attn_layout(1, 2, 0, 16, 64, BF16)) == 0
    assert L.attn_backward_workspace_bytes(attn_layout(2, 3, 16, 16, 32, BF16)) == 0

    def bwd(lay, mask=0, ql=None, kl=None, scale=0.125, ws_bytes=None, **ptrs):
        p = dict(q=FAKE, k=FAKE + 16, v=FAKE + 32, o=FAKE + 48, do=FAKE + 64, lse=FAKE + 80,
                 dq=FAKE + 96, dk=FAKE + 112, dv=FAKE + 128, ws=FAKE + 144)
        p.update(ptrs)
        wsb = L.attn_backward_workspace_bytes(lay) if ws_bytes is None else ws_bytes
        return L.attn_backward(p["q"], p["k"], p["v"], p["o"], p["do"], p["lse"], lay, mask, ql, kl, scale,
                               p["dq"], p["dk"], p["dv"], p["ws"], wsb, None)
    assert bwd(attn_layout(2, 3, 16, 16, 64, F32)) == DTYPE
    assert bwd(attn_layout(2, 3, 16, 16, 48, BF16)) == SHAPE
    assert bwd(lay_, mask=4) == MASK
    assert bwd(attn_layout(2, 3, 16, 20, 64, BF16), mask=2) == MASK   # causal needs n_q == n_k
    assert bwd(lay_, mask=0, kl=FAKE) == MASK                           # kv_lens without padding
    assert bwd(lay_, scale=float("nan")) == SCALE
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert bwd(lay_, **{name: None}) == NULLP, name
    assert bwd(lay_, mask=1) == NULLP                                   # padding without kv_lens
    assert bwd(lay_, ws=None) == WORK
    assert bwd(lay_, ws_bytes=L.attn_backward_workspace_bytes(lay_) - 1) == WORK
    assert bwd(lay_, dq=FAKE) == SHAPE                                  # output aliases Q
    assert bwd(lay_, dk=FAKE + 96) == SHAPE                             # dK aliases dQ
    assert bwd(attn_layout(0, 3, 16, 16, 64, BF16), q=None, k=None, v=None, o=None, do=None, lse=None,
               dq=None, dk=None, dv=None, ws=None) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from head_attention_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        _binding.lib()


def test_header_is_plain_c():
    # The header compiles as C99 with no HIP or torch headers in sight.
    import subprocess
    src = "#include \"headattn.h\"\nint main(void){attn_layout l={1,1,1,1,64,ATTN_BF16};" \
          "(void)l;return ATTN_OK;}\n"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        "-x", "c", "-", "-o", os.devnull], input=src.encode(),
                       capture_output=True)
    assert r.returncode == 0, r.stderr.decode()


def test_forward_restricted_validation():
    """Argument checks of attn_forward_restricted; every call here is
    rejected (or empty) before any launch."""
    L = ha.lib()
    lay_ = attn_layout(2, 3, 16, 16, 64, BF16)

    def rf(lay, mask=4, radius=3, ql=None, kl=None, scale=0.125, q=FAKE, k=FAKE + 16, v=FAKE + 32,
           o=FAKE + 48, lse=None):
        return L.attn_forward_restricted(q, k, v, lay, mask, ql, kl, radius, scale, o, lse, None)
    assert rf(lay_, mask=0) == MASK                                  # the restricted bit is required
    assert rf(lay_, mask=2) == MASK
    assert rf(lay_, radius=-1) == MASK
    assert rf(lay_, mask=4 | 8) == MASK                              # unknown bit
    assert rf(attn_layout(2, 3, 16, 20, 64, BF16)) == MASK           # self-attention only: n_q == n_k
    assert rf(lay_, mask=4, kl=FAKE) == MASK                         # kv_lens without padding
    assert rf(lay_, mask=5) == NULLP                                 # padding without kv_lens
    assert rf(lay_, scale=float("inf")) == SCALE
    assert rf(attn_layout(2, 3, 16, 16, 32, BF16)) == SHAPE
    assert rf(attn_layout(2, 3, 16, 16, 64, 7)) == DTYPE
    assert rf(lay_, q=None) == NULLP and rf(lay_, o=None) == NULLP and rf(lay_, k=None) == NULLP
    assert rf(lay_, o=FAKE) == SHAPE                                 # O aliases Q
    assert rf(lay_, lse=FAKE + 48) == SHAPE                          # LSE aliases O
    assert rf(attn_layout(0, 3, 16, 16, 64, BF16), q=None, k=None, v=None, o=None) == OK
    # the restricted bit is refused by the entry points without a radius
    assert L.attn_forward(FAKE, FAKE + 16, FAKE + 32, lay_, 4, None, None, 0.125, FAKE + 48, None) == MASK
    assert L.attn_forward_lse(FAKE, FAKE + 16, FAKE + 32, lay_, 6, None, None, 0.125, FAKE + 48, FAKE + 64,
                              None) == MASK


def test_backward_restricted_validation():
    """attn_backward_restricted takes the restricted mask and a radius;
    attn_backward refuses the restricted bit.  Every call is rejected before
    any launch."""
    L = ha.lib()
    lay_ = attn_layout(2, 3, 16, 16, 64, BF16)

    def rb(lay, mask=4, radius=2, kl=None, scale=0.125, ws_bytes=None, **ptrs):
        p = dict(q=FAKE, k=FAKE + 16, v=FAKE + 32, o=FAKE + 48, do=FAKE + 64, lse=FAKE + 80,
                 dq=FAKE + 96, dk=FAKE + 112, dv=FAKE + 128, ws=FAKE + 144)
        p.update(ptrs)
        wsb = L.attn_backward_workspace_bytes(lay) if ws_bytes is None else ws_bytes
        return L.attn_backward_restricted(p["q"], p["k"], p["v"], p["o"], p["do"], p["lse"], lay, mask, None, kl,
                                          radius, scale, p["dq"], p["dk"], p["dv"], p["ws"], wsb, None)
    assert rb(lay_, mask=0) == MASK
    assert rb(lay_, mask=2) == MASK
    assert rb(lay_, radius=-3) == MASK
    assert rb(attn_layout(2, 3, 16, 24, 64, BF16)) == MASK
    assert rb(attn_layout(2, 3, 16, 16, 64, F32)) == DTYPE
    assert rb(lay_, mask=5) == NULLP                       # padding without kv_lens
    assert rb(lay_, scale=float("nan")) == SCALE
    assert rb(lay_, ws=None) == WORK
    assert rb(lay_, dv=FAKE + 32) == SHAPE                  # dV aliases V
    assert rb(attn_layout(0, 3, 16, 16, 64, BF16), q=None, k=None, v=None, o=None, do=None, lse=None,
              dq=None, dk=None, dv=None, ws=None) == OK
    wsb = L.attn_backward_workspace_bytes(lay_)
    assert L.attn_backward(FAKE, FAKE + 16, FAKE + 32, FAKE + 48, FAKE + 64, FAKE + 80, lay_, 4, None, None, 0.125,
                           FAKE + 96, FAKE + 112, FAKE + 128, FAKE + 144, wsb, None) == MASK
