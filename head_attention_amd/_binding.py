"""ctypes binding of libheadattn.so: argument marshalling only.

Every step of the attention path runs in the library's HIP kernels; this
module only checks that torch tensors have the layout the C ABI documents
(contiguous [B, h, n, 64], on the GPU, matching dtypes), allocates outputs and
workspaces with torch (plumbing), passes raw device pointers plus torch's
current HIP stream, and turns a non-zero attn_status into an exception.
There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libheadattn.so")

ATTN_BF16 = 0
ATTN_F32 = 1
ATTN_MASK_NONE = 0
ATTN_MASK_KEY_PADDING = 1
ATTN_MASK_CAUSAL = 2
ATTN_MASK_RESTRICTED = 4

STATUS_NAMES = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL_POINTER", 2: "ATTN_ERR_BAD_SHAPE", 3: "ATTN_ERR_BAD_DTYPE",
    4: "ATTN_ERR_BAD_MASK", 5: "ATTN_ERR_BAD_LENGTHS", 6: "ATTN_ERR_BAD_SCALE",
    7: "ATTN_ERR_WORKSPACE", 8: "ATTN_ERR_HIP", 9: "ATTN_ERR_SCRATCH_LIMIT",
}

# Scratch that attn_decode_noalloc holds per GPU (ATTN_DECODE_NOALLOC_MAX_BYTES).
DECODE_NOALLOC_MAX_BYTES = 8 << 20


class attn_layout(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("h", ctypes.c_int32), ("n_q", ctypes.c_int32),
                ("n_k", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {status_string(status)}"
        if status == 8:
            msg += f" ({lib().attn_last_hip_error().decode()})"
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libheadattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m head_attention_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p = ctypes.c_void_p, ctypes.c_void_p
        L.attn_forward.argtypes = [vp, vp, vp, attn_layout, ctypes.c_int32, i32p, i32p,
                                   ctypes.c_float, vp, vp]
        L.attn_forward.restype = ctypes.c_int
        L.attn_decode.argtypes = [vp, vp, vp, attn_layout, i32p, ctypes.c_float, vp, vp,
                                  ctypes.c_size_t, vp]
        L.attn_decode.restype = ctypes.c_int
        L.attn_decode_noalloc.argtypes = [vp, vp, vp, attn_layout, i32p, ctypes.c_float, vp, vp]
        L.attn_decode_noalloc.restype = ctypes.c_int
        L.attn_cache_append.argtypes = [vp, vp, vp, vp, attn_layout, i32p, vp]
        L.attn_cache_append.restype = ctypes.c_int
        L.attn_head_projection.argtypes = [vp, vp, attn_layout, ctypes.c_int32, vp, vp, vp, vp]
        L.attn_head_projection.restype = ctypes.c_int
        L.attn_output_projection.argtypes = [vp, vp, attn_layout, vp, vp]
        L.attn_output_projection.restype = ctypes.c_int
        L.attn_forward_lse.argtypes = [vp, vp, vp, attn_layout, ctypes.c_int32, i32p, i32p,
                                       ctypes.c_float, vp, vp, vp]
        L.attn_forward_lse.restype = ctypes.c_int
        L.attn_forward_restricted.argtypes = [vp, vp, vp, attn_layout, ctypes.c_int32, i32p, i32p,
                                              ctypes.c_int32, ctypes.c_float, vp, vp, vp]
        L.attn_forward_restricted.restype = ctypes.c_int
        L.attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, attn_layout, ctypes.c_int32, i32p, i32p,
                                    ctypes.c_float, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.attn_backward.restype = ctypes.c_int
        L.attn_backward_restricted.argtypes = [vp, vp, vp, vp, vp, vp, attn_layout, ctypes.c_int32, i32p, i32p,
                                               ctypes.c_int32, ctypes.c_float, vp, vp, vp, vp, ctypes.c_size_t,
                                               vp]
        L.attn_backward_restricted.restype = ctypes.c_int
        L.attn_backward_workspace_bytes.argtypes = [attn_layout]
        L.attn_backward_workspace_bytes.restype = ctypes.c_size_t
        L.attn_decode_workspace_bytes.argtypes = [attn_layout]
        L.attn_decode_workspace_bytes.restype = ctypes.c_size_t
        L.attn_status_string.argtypes = [ctypes.c_int]
        L.attn_status_string.restype = ctypes.c_char_p
        L.attn_last_hip_error.argtypes = []
        L.attn_last_hip_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"attention tensors must be bfloat16 or float32, got {t.dtype}")


def _check_tensor(name: str, t: torch.Tensor, dtype, ndim: int = 4) -> None:
    # Cheap attribute reads only: this runs on every call, and at n = 128 a
    # call's Python time is comparable to the kernel's.
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _lens_ptr(name: str, t, B: int):
    if t is None:
        return None
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.int32 and t.dim() == 1
            and t.shape[0] == B and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor of shape [{B}]")
    return t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, t: torch.Tensor) -> int | None:
    """Raw HIP stream: `stream` if given, else torch's current stream on t's
    device (read without building a torch Stream object when torch offers
    that)."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(t.get_device()) or None
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream or None


def forward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, mask_kind: int = ATTN_MASK_NONE,
            q_lens: torch.Tensor | None = None, kv_lens: torch.Tensor | None = None,
            scale: float | None = None, out: torch.Tensor | None = None, stream=None,
            lse: torch.Tensor | None = None) -> torch.Tensor:
    """attn_forward: O = softmax(Q K^T * scale + M) V per (b, h), on the GPU.

    Q [B, h, n_q, 64]; K, V [B, h, n_k, 64]; all bf16 or all fp32, contiguous.
    q_lens / kv_lens: int32 GPU tensors [B] or None (see include/headattn.h).
    scale defaults to 1/sqrt(d).  Runs on torch's current stream (or `stream`).
    lse: an fp32 GPU tensor [B, h, n_q] to receive each row's log-sum-exp
    (attn_forward_lse), as attn_backward needs; None for the plain forward.
    """
    dt = Q.dtype
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_tensor(n, t, dt)
    B, H, n_q, d = Q.shape
    n_k = K.shape[2]
    if K.shape != (B, H, n_k, d) or V.shape != (B, H, n_k, d):
        raise ValueError(f"K {tuple(K.shape)} / V {tuple(V.shape)} do not match Q {tuple(Q.shape)}")
    if out is None:
        out = torch.empty_like(Q)
    else:
        _check_tensor("out", out, dt)
        if out.shape != Q.shape:
            raise ValueError("out must have Q's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    layout = attn_layout(B, H, n_q, n_k, d, _dtype_code(Q))
    if lse is None:
        st = lib().attn_forward(Q.data_ptr(), K.data_ptr(), V.data_ptr(), layout, int(mask_kind),
                                _lens_ptr("q_lens", q_lens, B), _lens_ptr("kv_lens", kv_lens, B),
                                float(scale), out.data_ptr(), _stream_handle(stream, Q))
        if st != 0:
            raise AttnError(st, "attn_forward")
        return out
    _check_tensor("lse", lse, torch.float32, 3)
    if lse.shape != (B, H, n_q):
        raise ValueError("lse must be [B, h, n_q]")
    st = lib().attn_forward_lse(Q.data_ptr(), K.data_ptr(), V.data_ptr(), layout, int(mask_kind),
                                _lens_ptr("q_lens", q_lens, B), _lens_ptr("kv_lens", kv_lens, B),
                                float(scale), out.data_ptr(), lse.data_ptr(), _stream_handle(stream, Q))
    if st != 0:
        raise AttnError(st, "attn_forward_lse")
    return out


def forward_restricted(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, radius: int,
                       mask_kind: int = ATTN_MASK_RESTRICTED, q_lens: torch.Tensor | None = None,
                       kv_lens: torch.Tensor | None = None, scale: float | None = None,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """attn_forward_restricted: restricted self-attention, query i sees keys
    i - radius .. i + radius (i - radius .. i when mask_kind has
    ATTN_MASK_CAUSAL).  mask_kind must hold ATTN_MASK_RESTRICTED; n_q == n_k.
    Tensors as for forward(); lse (fp32 [B, h, n_q]) is optional."""
    dt = Q.dtype
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_tensor(n, t, dt)
    B, H, n_q, d = Q.shape
    n_k = K.shape[2]
    if K.shape != (B, H, n_k, d) or V.shape != (B, H, n_k, d):
        raise ValueError(f"K {tuple(K.shape)} / V {tuple(V.shape)} do not match Q {tuple(Q.shape)}")
    if out is None:
        out = torch.empty_like(Q)
    else:
        _check_tensor("out", out, dt)
        if out.shape != Q.shape:
            raise ValueError("out must have Q's shape")
    lse_ptr = None
    if lse is not None:
        _check_tensor("lse", lse, torch.float32, 3)
        if lse.shape != (B, H, n_q):
            raise ValueError("lse must be [B, h, n_q]")
        lse_ptr = lse.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    layout = attn_layout(B, H, n_q, n_k, d, _dtype_code(Q))
    st = lib().attn_forward_restricted(Q.data_ptr(), K.data_ptr(), V.data_ptr(), layout, int(mask_kind),
                                       _lens_ptr("q_lens", q_lens, B), _lens_ptr("kv_lens", kv_lens, B),
                                       int(radius), float(scale), out.data_ptr(), lse_ptr,
                                       _stream_handle(stream, Q))
    if st != 0:
        raise AttnError(st, "attn_forward_restricted")
    return out


def backward_workspace_bytes(B: int, h: int, n_q: int, n_k: int, d: int = 64) -> int:
    return int(lib().attn_backward_workspace_bytes(attn_layout(B, h, n_q, n_k, d, ATTN_BF16)))


def decode_workspace_bytes(B: int, h: int, n_max: int, dtype=torch.bfloat16, d: int = 64) -> int:
    code = ATTN_BF16 if dtype == torch.bfloat16 else ATTN_F32
    return int(lib().attn_decode_workspace_bytes(attn_layout(B, h, 1, n_max, d, code)))


def decode(q: torch.Tensor, Kcache: torch.Tensor, Vcache: torch.Tensor, kv_lens: torch.Tensor,
           scale: float | None = None, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """attn_decode: one KV-cache decode step on the GPU.

    q [B, h, 1, 64]; Kcache, Vcache [B, h, n_max, 64]; kv_lens int32 GPU [B]
    counts valid cache rows including the new token.  `workspace` (a GPU
    tensor of at least decode_workspace_bytes(...) bytes) is allocated with
    torch when not given.
    """
    dt = q.dtype
    for n, t in (("q", q), ("Kcache", Kcache), ("Vcache", Vcache)):
        _check_tensor(n, t, dt)
    B, H, one, d = q.shape
    n_max = Kcache.shape[2]
    if one != 1 or tuple(Kcache.shape) != (B, H, n_max, d) or Vcache.shape != Kcache.shape:
        raise ValueError("q must be [B, h, 1, d] and the caches [B, h, n_max, d]")
    layout = attn_layout(B, H, 1, n_max, d, _dtype_code(q))
    need = int(lib().attn_decode_workspace_bytes(layout))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, dt)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().attn_decode(q.data_ptr(), Kcache.data_ptr(), Vcache.data_ptr(), layout,
                           _lens_ptr("kv_lens", kv_lens, B), float(scale), out.data_ptr(),
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           _stream_handle(stream, q))
    if st != 0:
        raise AttnError(st, "attn_decode")
    return out


def decode_noalloc(q: torch.Tensor, Kcache: torch.Tensor, Vcache: torch.Tensor, kv_lens: torch.Tensor,
                   scale: float | None = None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """attn_decode_noalloc: the decode step with its partials in the library's
    static per-GPU scratch (no workspace, no device allocation by the call).

    Arguments as for decode(); `out` is allocated with torch when not given
    (pass it to keep the whole step allocation-free).  Raises AttnError
    (ATTN_ERR_SCRATCH_LIMIT) when the layout needs more than
    DECODE_NOALLOC_MAX_BYTES of partials.  Calls on one GPU share that
    scratch: calls that could overlap must be ordered by the caller.
    """
    dt = q.dtype
    for n, t in (("q", q), ("Kcache", Kcache), ("Vcache", Vcache)):
        _check_tensor(n, t, dt)
    B, H, one, d = q.shape
    n_max = Kcache.shape[2]
    if one != 1 or tuple(Kcache.shape) != (B, H, n_max, d) or Vcache.shape != Kcache.shape:
        raise ValueError("q must be [B, h, 1, d] and the caches [B, h, n_max, d]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, dt)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().attn_decode_noalloc(q.data_ptr(), Kcache.data_ptr(), Vcache.data_ptr(),
                                   attn_layout(B, H, 1, n_max, d, _dtype_code(q)),
                                   _lens_ptr("kv_lens", kv_lens, B), float(scale), out.data_ptr(),
                                   _stream_handle(stream, q))
    if st != 0:
        raise AttnError(st, "attn_decode_noalloc")
    return out


def cache_append(Knew: torch.Tensor, Vnew: torch.Tensor, Kcache: torch.Tensor, Vcache: torch.Tensor,
                 kv_lens: torch.Tensor, stream=None) -> None:
    """attn_cache_append: write the new tokens' K/V rows into the caches.

    Knew, Vnew [B, h, n_new, 64]; Kcache, Vcache [B, h, n_max, 64] (written in
    place); kv_lens int32 GPU [B] = valid rows of each entry after the append.
    Row r of the new block lands in cache row kv_lens[b] - n_new + r; rows
    that would fall outside the cache are skipped (see include/headattn.h).
    """
    dt = Knew.dtype
    for n, t in (("Knew", Knew), ("Vnew", Vnew), ("Kcache", Kcache), ("Vcache", Vcache)):
        _check_tensor(n, t, dt)
    B, H, n_new, d = Knew.shape
    n_max = Kcache.shape[2]
    if Vnew.shape != Knew.shape or Kcache.shape != (B, H, n_max, d) or Vcache.shape != Kcache.shape:
        raise ValueError("new rows must be [B, h, n_new, d] and the caches [B, h, n_max, d]")
    layout = attn_layout(B, H, n_new, n_max, d, _dtype_code(Knew))
    st = lib().attn_cache_append(Knew.data_ptr(), Vnew.data_ptr(), Kcache.data_ptr(), Vcache.data_ptr(),
                                 layout, _lens_ptr("kv_lens", kv_lens, B), _stream_handle(stream, Knew))
    if st != 0:
        raise AttnError(st, "attn_cache_append")


def head_projection(X: torch.Tensor, W: torch.Tensor, h: int, outs=None, stream=None) -> list:
    """attn_head_projection: the multi-head input projections X W_j^T, split
    into heads.

    X [B, n, d_model] bf16 (d_model = 64 h); W [n_out * d_model, d_model] bf16
    (one block of d_model rows per projection, a linear layer's weight
    layout).  Returns n_out tensors [B, h, n, 64] (or fills `outs`).
    """
    _check_tensor("X", X, torch.bfloat16, 3)
    _check_tensor("W", W, torch.bfloat16, 2)
    B, n, d_model = X.shape
    if d_model != 64 * h or W.shape[1] != d_model or W.shape[0] % d_model != 0:
        raise ValueError(f"X {tuple(X.shape)} / W {tuple(W.shape)} do not fit h = {h} heads of 64")
    n_out = W.shape[0] // d_model
    if outs is None:
        outs = [torch.empty((B, h, n, 64), dtype=torch.bfloat16, device=X.device) for _ in range(n_out)]
    if len(outs) != n_out:
        raise ValueError(f"W holds {n_out} projections but {len(outs)} outputs were given")
    for j, o in enumerate(outs):
        _check_tensor(f"out{j}", o, torch.bfloat16)
        if o.shape != (B, h, n, 64):
            raise ValueError(f"out{j} must be [B, h, n, 64]")
    ptrs = [o.data_ptr() for o in outs] + [None] * (3 - n_out)
    st = lib().attn_head_projection(X.data_ptr(), W.data_ptr(), attn_layout(B, h, n, 0, 64, ATTN_BF16), n_out,
                                    ptrs[0], ptrs[1], ptrs[2], _stream_handle(stream, X))
    if st != 0:
        raise AttnError(st, "attn_head_projection")
    return outs


def output_projection(O: torch.Tensor, Wo: torch.Tensor, out: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """attn_output_projection: Concat(heads of O) Wo^T.

    O [B, h, n, 64] bf16 (the attention output); Wo [d_model, d_model] bf16.
    Returns Y [B, n, d_model].
    """
    _check_tensor("O", O, torch.bfloat16)
    _check_tensor("Wo", Wo, torch.bfloat16, 2)
    B, h, n, d = O.shape
    d_model = h * d
    if d != 64 or Wo.shape != (d_model, d_model):
        raise ValueError(f"O {tuple(O.shape)} / Wo {tuple(Wo.shape)} do not fit")
    if out is None:
        out = torch.empty((B, n, d_model), dtype=torch.bfloat16, device=O.device)
    _check_tensor("out", out, torch.bfloat16, 3)
    if out.shape != (B, n, d_model):
        raise ValueError("out must be [B, n, d_model]")
    st = lib().attn_output_projection(O.data_ptr(), Wo.data_ptr(), attn_layout(B, h, n, 0, 64, ATTN_BF16),
                                      out.data_ptr(), _stream_handle(stream, O))
    if st != 0:
        raise AttnError(st, "attn_output_projection")
    return out


def backward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, O: torch.Tensor, dO: torch.Tensor,
             lse: torch.Tensor, mask_kind: int = ATTN_MASK_NONE, q_lens: torch.Tensor | None = None,
             kv_lens: torch.Tensor | None = None, scale: float | None = None, grads=None,
             workspace: torch.Tensor | None = None, stream=None, radius: int | None = None):
    """attn_backward: (dQ, dK, dV) of O = softmax(Q K^T * scale + M) V given dO.

    Q, K, V, O, dO bf16 [B, h, n, 64] (the forward's tensors), lse the fp32
    [B, h, n_q] log-sum-exp from forward(..., lse=...); the mask arguments and
    scale must be those of the forward.  Returns three new tensors, or fills
    `grads` = (dQ, dK, dV).  With `radius` (and ATTN_MASK_RESTRICTED in
    mask_kind) it calls attn_backward_restricted, the backward of
    forward_restricted.
    """
    for n, t in (("Q", Q), ("K", K), ("V", V), ("O", O), ("dO", dO)):
        _check_tensor(n, t, torch.bfloat16)
    _check_tensor("lse", lse, torch.float32, 3)
    B, H, n_q, d = Q.shape
    n_k = K.shape[2]
    if K.shape != (B, H, n_k, d) or V.shape != K.shape or O.shape != Q.shape or dO.shape != Q.shape \
            or lse.shape != (B, H, n_q):
        raise ValueError("shapes do not match the forward's")
    if grads is None:
        grads = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    dQ, dK, dV = grads
    for n, t, ref in (("dQ", dQ, Q), ("dK", dK, K), ("dV", dV, V)):
        _check_tensor(n, t, torch.bfloat16)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must have the shape of its input")
    layout = attn_layout(B, H, n_q, n_k, d, ATTN_BF16)
    need = int(lib().attn_backward_workspace_bytes(layout))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    common = (Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), dO.data_ptr(), lse.data_ptr(), layout,
              int(mask_kind), _lens_ptr("q_lens", q_lens, B), _lens_ptr("kv_lens", kv_lens, B))
    tail = (float(scale), dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream_handle(stream, Q))
    if radius is None:
        st, where = lib().attn_backward(*common, *tail), "attn_backward"
    else:
        st, where = lib().attn_backward_restricted(*common, int(radius), *tail), "attn_backward_restricted"
    if st != 0:
        raise AttnError(st, where)
    return dQ, dK, dV
