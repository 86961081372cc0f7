"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutant replaces one step of the oracle with a plausible slip -- an
off-by-one mask, a transposed operand, a wrong scale, masking after the
softmax, a dropped term or sign -- and the full pin suite of test_oracle.py
is run against it.  A mutant that passes every pin would mean the pins do not
constrain that step.
"""
import math

import numpy as np
import pytest

import oracle.attn_oracle as orc
from test_oracle import PINS

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

_row = orc.attention_row
_allowed = orc.allowed_keys
_attention = orc.attention
_decode = orc.decode
_pe = orc.sinusoidal_pe
_append = orc.cache_append
_proj = orc.head_projection
_oproj = orc.output_projection
_bwd = orc.attention_backward


def _window(ok, i, j, radius):
    if radius is not None:
        ok &= np.abs(j - i) <= radius
    return ok


def m_causal_strict(i, n_k, kv_len, causal, radius=None):
    j = np.arange(n_k)
    ok = j < kv_len
    if causal:
        ok &= j < i  # off by one: excludes the diagonal
    return _window(ok, i, j, radius)


def m_padding_inclusive(i, n_k, kv_len, causal, radius=None):
    j = np.arange(n_k)
    ok = j <= kv_len  # off by one: admits the first pad
    if causal:
        ok &= j <= i
    return _window(ok, i, j, radius)


def m_causal_transposed(i, n_k, kv_len, causal, radius=None):
    j = np.arange(n_k)
    ok = j < kv_len
    if causal:
        ok &= j >= i  # upper instead of lower triangle
    return _window(ok, i, j, radius)


def _window_variant(kind):
    def allowed(i, n_k, kv_len, causal, radius=None):
        j = np.arange(n_k)
        ok = j < kv_len
        if causal:
            ok &= j <= i
        if radius is None:
            return ok
        if kind == "strict":
            ok &= np.abs(j - i) < radius  # off by one: drops both edges
        elif kind == "past_only":
            ok &= j >= i - radius  # no upper limit without the causal mask
        elif kind == "wide_past":
            ok &= (j >= i - radius - 1) & (j <= i + radius)  # one extra key behind
        elif kind == "radius_as_r":
            ok &= np.abs(j - i) <= radius // 2  # radius read as the window size r
        return ok
    return allowed


def m_bwd_ignores_radius(Q, K, V, dO, mask_kind=0, q_lens=None, kv_lens=None, scale=None, radius=None):
    return _bwd(Q, K, V, dO, mask_kind=mask_kind & ~orc.MASK_RESTRICTED, q_lens=q_lens,
                kv_lens=kv_lens, scale=scale)


def m_no_max_shift(q, K, V, allowed, scale, return_weights=False):
    q, K, V = (np.asarray(a, dtype=np.float64) for a in (q, K, V))
    idx = np.flatnonzero(allowed)
    w_full = np.zeros(K.shape[0])
    if idx.size == 0:
        out = np.zeros(V.shape[1])
        return (out, w_full) if return_weights else out
    e = np.exp(scale * (K[idx] @ q))  # no pivot: overflows for large logits
    w = e / e.sum()
    out = w @ V[idx]
    w_full[idx] = w
    return (out, w_full) if return_weights else out


def _row_variant(kind):
    def row(q, K, V, allowed, scale, return_weights=False):
        q, K, V = (np.asarray(a, dtype=np.float64) for a in (q, K, V))
        n_k = K.shape[0]
        w_full = np.zeros(n_k)
        if kind == "mask_after_softmax":
            s = scale * (K @ q)
            e = np.exp(s - s.max())
            w = e / e.sum()
            w = np.where(allowed, w, 0.0)  # zeroed after softmax, not renormalised
            out = w @ np.where(allowed[:, None], V, 0.0)
            return (out, w) if return_weights else out
        idx = np.flatnonzero(allowed)
        if idx.size == 0:
            out = np.zeros(V.shape[1])
            return (out, w_full) if return_weights else out
        s = scale * (K[idx] @ q)
        if kind == "no_normalise":
            w = np.exp(s - s.max())
        elif kind == "sign":
            e = np.exp(s.max() - s)
            w = e / e.sum()
        elif kind == "value_of_query":
            e = np.exp(s - s.max())
            w = e / e.sum()
            out = w @ K[idx]  # sums the keys instead of the values
            w_full[idx] = w
            return (out, w_full) if return_weights else out
        else:
            raise AssertionError(kind)
        out = w @ V[idx]
        w_full[idx] = w
        return (out, w_full) if return_weights else out
    return row


def m_swap_qk(Q, K, V, *a, **kw):
    # transposed operand: scores K Q^T instead of Q K^T (square cases only)
    if np.shape(Q) == np.shape(K):
        Q, K = K, Q
    return _attention(Q, K, V, *a, **kw)


def m_scale_one_over_dk(Q, K, V, mask_kind=0, q_lens=None, kv_lens=None, scale=None, **kw):
    if scale is None:
        scale = 1.0 / np.shape(Q)[-1]  # 1/d_k instead of 1/sqrt(d_k)
    return _attention(Q, K, V, mask_kind, q_lens, kv_lens, scale, **kw)


def m_ignore_q_lens(Q, K, V, mask_kind=0, q_lens=None, kv_lens=None, scale=None, **kw):
    return _attention(Q, K, V, mask_kind, None, kv_lens, scale, **kw)


def m_decode_without_new_token(q, Kc, Vc, kv_lens, scale=None, pairs=None):
    return _decode(q, Kc, Vc, np.maximum(np.asarray(kv_lens) - 1, 1), scale, pairs)


def m_append_one_row_late(Kc, Vc, Kn, Vn, kv_lens):
    # off by one: the block lands one row past where the lengths put it
    return _append(Kc, Vc, Kn, Vn, np.asarray(kv_lens) + 1)


def m_append_reversed(Kc, Vc, Kn, Vn, kv_lens):
    # the new block written in reverse row order
    return _append(Kc, Vc, np.asarray(Kn)[:, :, ::-1], np.asarray(Vn)[:, :, ::-1], kv_lens)


def m_append_k_only(Kc, Vc, Kn, Vn, kv_lens):
    # the V row never reaches the cache
    K2, _ = _append(Kc, Vc, Kn, Vn, kv_lens)
    return K2, np.array(Vc, copy=True)


def m_heads_interleaved(X, W, h):
    # head i takes every h-th feature instead of a contiguous block of d_k
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    B, n, d = X.shape
    d_k = d // h
    Y = X @ W.T
    outs = []
    for j in range(W.shape[0] // d):
        Yj = Y[:, :, j * d:(j + 1) * d].reshape(B, n, d_k, h).transpose(0, 3, 1, 2)
        outs.append(np.ascontiguousarray(Yj))
    return outs


def m_proj_untransposed(X, W, h):
    # X W instead of X W^T (square blocks only)
    W = np.asarray(W, dtype=np.float64)
    d = np.shape(X)[2]
    Wt = np.vstack([W[j * d:(j + 1) * d].T for j in range(W.shape[0] // d)])
    return _proj(X, Wt, h)


def m_concat_heads_reversed(O, Wo):
    return _oproj(np.asarray(O)[:, ::-1], Wo)


def _bwd_variant(kind):
    def bwd(Q, K, V, dO, mask_kind=0, q_lens=None, kv_lens=None, scale=None, radius=None):
        Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
        radius = radius if mask_kind & orc.MASK_RESTRICTED else None
        B, H, n_q, d = Q.shape
        n_k = K.shape[2]
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
        for b in range(B):
            kv_len = n_k if not (mask_kind & 1) else int(kv_lens[b])
            q_len = n_q if q_lens is None else int(q_lens[b])
            for h in range(H):
                for i in range(min(q_len, n_q)):
                    idx = np.flatnonzero(orc.allowed_keys(i, n_k, kv_len, bool(mask_kind & 2), radius))
                    if idx.size == 0:
                        continue
                    s = scale * (K[b, h][idx] @ Q[b, h, i])
                    e = np.exp(s - s.max())
                    w = e / e.sum()
                    dp = V[b, h][idx] @ dO[b, h, i]
                    ds = w * dp if kind == "no_rowsum" else w * (dp - (w * dp).sum())
                    dV[b, h][idx] += np.outer(w, dO[b, h, i])
                    dQ[b, h, i] += scale * (ds @ K[b, h][idx])
                    kscale = 1.0 if kind == "dk_unscaled" else scale
                    dK[b, h][idx] += kscale * np.outer(ds, Q[b, h, i])
        if kind == "dv_transposed":
            dV = dV[:, :, ::-1].copy()
        return dQ, dK, dV
    return bwd


def m_pe_swapped(pos, d_model):
    out = np.zeros(d_model)
    for dim in range(d_model):
        angle = pos / (10000.0 ** ((2 * (dim // 2)) / d_model))
        out[dim] = math.cos(angle) if dim % 2 == 0 else math.sin(angle)
    return out


def m_pe_exponent(pos, d_model):
    out = np.zeros(d_model)
    for dim in range(d_model):
        angle = pos / (10000.0 ** ((dim // 2) / d_model))  # i instead of 2i
        out[dim] = math.sin(angle) if dim % 2 == 0 else math.cos(angle)
    return out


MUTANTS = {
    "causal_excludes_diagonal": ("allowed_keys", m_causal_strict),
    "padding_admits_first_pad": ("allowed_keys", m_padding_inclusive),
    "causal_upper_triangle": ("allowed_keys", m_causal_transposed),
    "window_excludes_edges": ("allowed_keys", _window_variant("strict")),
    "window_past_only": ("allowed_keys", _window_variant("past_only")),
    "window_one_extra_past_key": ("allowed_keys", _window_variant("wide_past")),
    "window_radius_read_as_size": ("allowed_keys", _window_variant("radius_as_r")),
    "backward_ignores_radius": ("attention_backward", m_bwd_ignores_radius),
    "no_max_shift": ("attention_row", m_no_max_shift),
    "mask_after_softmax": ("attention_row", _row_variant("mask_after_softmax")),
    "no_normalisation": ("attention_row", _row_variant("no_normalise")),
    "sign_flip_in_exp": ("attention_row", _row_variant("sign")),
    "sums_keys_not_values": ("attention_row", _row_variant("value_of_query")),
    "scores_K_Qt": ("attention", m_swap_qk),
    "scale_1_over_dk": ("attention", m_scale_one_over_dk),
    "q_lens_ignored": ("attention", m_ignore_q_lens),
    "decode_drops_new_token": ("decode", m_decode_without_new_token),
    "append_one_row_late": ("cache_append", m_append_one_row_late),
    "append_block_reversed": ("cache_append", m_append_reversed),
    "append_drops_v": ("cache_append", m_append_k_only),
    "heads_interleaved": ("head_projection", m_heads_interleaved),
    "projection_untransposed": ("head_projection", m_proj_untransposed),
    "concat_heads_reversed": ("output_projection", m_concat_heads_reversed),
    "backward_drops_softmax_rowsum": ("attention_backward", _bwd_variant("no_rowsum")),
    "backward_dk_unscaled": ("attention_backward", _bwd_variant("dk_unscaled")),
    "backward_dv_keys_reversed": ("attention_backward", _bwd_variant("dv_transposed")),
    "pe_sin_cos_swapped": ("sinusoidal_pe", m_pe_swapped),
    "pe_exponent_i": ("sinusoidal_pe", m_pe_exponent),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin(orc)
        except Exception:  # AssertionError or a crash both count as caught
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
