"""Plain fp64 CPU oracle for scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check of the graft entry point
and the CPU-baseline leg of the bench use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constants) and imports nothing from
it.  Inputs are NumPy arrays; every value is widened exactly to float64 before
any arithmetic (bf16 and fp32 values are exactly representable in fp64).

Every function follows the plain definition on the pages; it is slow on
purpose and does no blocking, fusion or reordering beyond what the definition
states.  Page citations name the page title and its section:

* "[논문 리뷰]Attention Is All You Need" (kimjiil.github.io), §3.2.1 Eq. for
  Attention(Q,K,V); §3.2.2 multi-head attention (per-head projections W_i,
  Concat(head_1..head_h) W^O); §3.2.3 "Attention이 쓰이는 3곳" (masking sets illegal
  logits to -inf before softmax, weight exactly 0); §3.5 Positional Encoding;
  §3.7 KV cache note.
* "Attention Is All You Need를 지금 다시 읽는 법" (eightmm.github.io), the
  masked form Attention(Q,K,V,M) = softmax(QK^T/sqrt(d_k) + M)V.
* "Attention is all you need" (baxdailygit.github.io, sutskever_list), the
  five-step self-attention computation and its numeric simulation.
* "Attention Is All You Need 해부" (sj-techlog.pages.dev), "식 (1)의 모든
  기호" (shapes), "mask는 softmax 전에 더해야 한다", "KV cache는 추론의 같은
  계산을 반복하지 않게 한다", and the verification run "직접 검증".

Readings where the pages are silent (the same list is kept with the design
notes):
* Mask kinds are exclusion sets: a key is *allowed* iff j < kv_len[b] (key
  padding), for causal j <= i (top-left aligned, n_q == n_k), and for
  restricted self-attention |i - j| <= radius (j >= i - radius under the
  causal mask as well; n_q == n_k).  Excluded
  keys never enter the sum, so their weight is exactly 0 and their K/V
  contents (even NaN) cannot reach the output.
* A query row i >= q_len[b] (a padded query position) is written as 0.
* A row with no allowed key (kv_len == 0) is 0, never NaN.
* The pivot of the stable softmax is the max over the allowed scores, the
  same choice the verification script on the sj-techlog page makes.
* Decode: the single new query sits at position kv_len-1 and sees every one of
  the kv_len cached keys; the caller has already appended the new token's K/V.
* Restricted self-attention (kimjiil page §4, Table 1 and the note after it:
  each position looks only at its r surrounding positions, O(r n d) work)
  leaves the shape of the neighbourhood open.  Reading: a window centred on
  the query, r = 2 radius + 1 keys i - radius .. i + radius, clipped to the
  sequence; with the decoder's causal mask only its past half remains,
  i - radius .. i (radius + 1 keys).

parity pinned: every function below is checked against page values, closed
forms, invariants or an independent library routine in tests/test_oracle.py.
"""

from __future__ import annotations

import math

import numpy as np

MASK_NONE = 0
MASK_KEY_PADDING = 1
MASK_CAUSAL = 2
MASK_RESTRICTED = 4

__all__ = [
    "MASK_NONE",
    "MASK_KEY_PADDING",
    "MASK_CAUSAL",
    "MASK_RESTRICTED",
    "allowed_keys",
    "attention_row",
    "attention",
    "decode",
    "sinusoidal_pe",
    "kv_cache_scalars",
    "attention_flops",
]


def _f64(x) -> np.ndarray:
    """Exact widening to float64 (bf16/fp16/fp32 values are fp64-exact)."""
    return np.asarray(x, dtype=np.float64)


def _radius_of(mask_kind: int, radius, n_q: int, n_k: int):
    """The window radius of a call: None unless mask_kind has MASK_RESTRICTED,
    which is self-attention (n_q == n_k) and needs an integer radius >= 0."""
    if not mask_kind & MASK_RESTRICTED:
        return None
    if radius is None or int(radius) < 0:
        raise ValueError("restricted attention needs a radius >= 0")
    if n_q != n_k:
        raise ValueError("restricted self-attention needs n_q == n_k")
    return int(radius)


def allowed_keys(i: int, n_k: int, kv_len: int, causal: bool, radius=None) -> np.ndarray:
    """Boolean vector over the n_k keys: which keys query row i may attend to.

    Key padding ("pad token에 attention이 가지 않는가", sj-techlog page,
    failure section 2) excludes j >= kv_len.  The causal mask of the decoder
    self-attention (kimjiil page §3.2.3; the 4x4 table on the sj-techlog page)
    excludes j > i.  Restricted self-attention (kimjiil page §4, Table 1:
    a neighbourhood of r positions around the query) with radius w excludes
    |i - j| > w; None means unrestricted.
    """
    j = np.arange(n_k)
    ok = j < kv_len
    if causal:
        ok &= j <= i
    if radius is not None:
        ok &= np.abs(j - i) <= radius
    return ok


def attention_row(q, K, V, allowed, scale: float, return_weights: bool = False):
    """One query row of softmax(q K^T * scale + M) V, M = 0 / -inf.

    Steps in the order the pages give them (baxdailygit page, 5-step
    computation; sj-techlog page, Eq. (1) symbol table):
      1. scores s_j = scale * (q . k_j) for allowed j (dot products);
      2. masked logits are -inf *before* softmax, so they are simply left out;
      3. stable softmax: subtract the max allowed score, exponentiate,
         divide by the sum (rows sum to 1);
      4. weighted sum of the allowed value rows.
    Returns (out[d_v], weights[n_k]) when return_weights, else out.
    """
    q = _f64(q)
    K = _f64(K)
    V = _f64(V)
    idx = np.flatnonzero(allowed)
    w_full = np.zeros(K.shape[0], dtype=np.float64)
    if idx.size == 0:  # no allowed key: the row is 0, never NaN
        out = np.zeros(V.shape[1], dtype=np.float64)
        return (out, w_full) if return_weights else out
    s = scale * (K[idx] @ q)
    m = s.max()
    e = np.exp(s - m)
    w = e / e.sum()
    out = w @ V[idx]
    if return_weights:
        w_full[idx] = w
        return out, w_full
    return out


def attention(Q, K, V, mask_kind: int = MASK_NONE, q_lens=None, kv_lens=None,
              scale: float | None = None, rows=None, return_weights: bool = False,
              radius=None):
    """Multi-head scaled dot-product attention, heads batched as [B, h, n, d].

    Q: [B, h, n_q, d_k]; K: [B, h, n_k, d_k]; V: [B, h, n_k, d_v]
    (sj-techlog page, "식 (1)의 모든 기호"; each head is an independent
    Attention(QW^Q, KW^K, VW^V), kimjiil page §3.2.2).
    mask_kind: bit 1 = key padding by kv_lens[b]; bit 2 = causal (n_q == n_k);
    bit 4 = restricted to |i - j| <= radius (n_q == n_k; needs radius >= 0).
    q_lens[b]: rows i >= q_lens[b] are written as 0 (None = all rows valid).
    scale: defaults to 1/sqrt(d_k) (kimjiil page §3.2.1).
    rows: optional iterable of (b, h, i) to evaluate only those rows; then a
    dict {(b, h, i): out} is returned (used for sampled checks at full size).
    Returns O [B, h, n_q, d_v] in fp64 (and W [B, h, n_q, n_k] when
    return_weights).
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    B, H, n_q, d_k = Q.shape
    n_k = K.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    causal = bool(mask_kind & MASK_CAUSAL)
    if causal and n_q != n_k:
        raise ValueError("causal attention needs n_q == n_k")
    kpad = bool(mask_kind & MASK_KEY_PADDING)
    if kpad and kv_lens is None:
        raise ValueError("key padding needs kv_lens")
    radius = _radius_of(mask_kind, radius, n_q, n_k)

    def kv_len_of(b):
        return int(kv_lens[b]) if kpad else n_k

    def q_len_of(b):
        return n_q if q_lens is None else int(q_lens[b])

    if rows is not None:
        res = {}
        for (b, h, i) in rows:
            if i >= q_len_of(b):
                res[(b, h, i)] = np.zeros(V.shape[3])
                continue
            ok = allowed_keys(i, n_k, kv_len_of(b), causal, radius)
            res[(b, h, i)] = attention_row(Q[b, h, i], K[b, h], V[b, h], ok, scale)
        return res

    O = np.zeros((B, H, n_q, V.shape[3]), dtype=np.float64)
    W = np.zeros((B, H, n_q, n_k), dtype=np.float64) if return_weights else None
    for b in range(B):
        kv_len = kv_len_of(b)
        q_len = q_len_of(b)
        for h in range(H):
            for i in range(min(q_len, n_q)):
                ok = allowed_keys(i, n_k, kv_len, causal, radius)
                if return_weights:
                    O[b, h, i], W[b, h, i] = attention_row(
                        Q[b, h, i], K[b, h], V[b, h], ok, scale, True)
                else:
                    O[b, h, i] = attention_row(Q[b, h, i], K[b, h], V[b, h], ok, scale)
    return (O, W) if return_weights else O


def decode(q, Kcache, Vcache, kv_lens, scale: float | None = None, pairs=None):
    """One KV-cache decode step (kimjiil page §3.7; sj-techlog page, KV cache).

    q: [B, h, 1, d]; Kcache, Vcache: [B, h, n_max, d]; kv_lens[b] counts the
    valid cache rows *including* the new token, which the caller appended
    before the call.  The new query sits at position kv_len-1, so under the
    decoder's causal mask it sees all kv_len keys and nothing else.
    pairs: optional iterable of (b, h) to evaluate only those heads (a dict
    {(b, h): out[d]} is then returned).  Returns O [B, h, 1, d] in fp64.
    """
    q = _f64(q)
    Kc = _f64(Kcache) if not isinstance(Kcache, np.ndarray) or Kcache.dtype != np.float64 else Kcache
    Vc = _f64(Vcache) if not isinstance(Vcache, np.ndarray) or Vcache.dtype != np.float64 else Vcache
    B, H, _, d = q.shape
    n_max = Kc.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)

    def one(b, h):
        ok = allowed_keys(int(kv_lens[b]) - 1, n_max, int(kv_lens[b]), True)
        return attention_row(q[b, h, 0], Kc[b, h], Vc[b, h], ok, scale)

    if pairs is not None:
        return {(b, h): one(b, h) for (b, h) in pairs}
    O = np.zeros((B, H, 1, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            O[b, h, 0] = one(b, h)
    return O


def row_logsumexp(Q, K, mask_kind: int = MASK_NONE, q_lens=None, kv_lens=None, scale: float | None = None,
                  radius=None):
    """Per query row, log(sum_j exp(s_ij)) over the allowed keys (natural
    log), the normaliser of the softmax of kimjiil page §3.2.1; -inf for a
    row with no allowed key or a padded query row.  Returns [B, h, n_q]."""
    Q = _f64(Q)
    K = _f64(K)
    B, H, n_q, d = Q.shape
    n_k = K.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    causal = bool(mask_kind & MASK_CAUSAL)
    radius = _radius_of(mask_kind, radius, n_q, n_k)
    out = np.full((B, H, n_q), -np.inf)
    for b in range(B):
        kv_len = n_k if not (mask_kind & MASK_KEY_PADDING) else int(kv_lens[b])
        q_len = n_q if q_lens is None else int(q_lens[b])
        for h in range(H):
            for i in range(min(q_len, n_q)):
                idx = np.flatnonzero(allowed_keys(i, n_k, kv_len, causal, radius))
                if idx.size:
                    s = scale * (K[b, h][idx] @ Q[b, h, i])
                    m = s.max()
                    out[b, h, i] = m + math.log(np.exp(s - m).sum())
    return out


def attention_backward(Q, K, V, dO, mask_kind: int = MASK_NONE, q_lens=None, kv_lens=None,
                       scale: float | None = None, radius=None):
    """Gradients of L through O = softmax(Q K^T * scale + M) V, given dO =
    dL/dO (the training the pages describe back-propagates through this
    sub-layer; kimjiil page §3.2.1 defines the map).  Row by row, with the
    softmax weights w of row i over its allowed keys (the forward's plain
    definition):
        dV[j]  += w_ij dO_i
        dp_ij   = dO_i . V_j
        ds_ij   = w_ij (dp_ij - sum_k w_ik dp_ik)      (softmax Jacobian)
        dQ_i   += scale ds_ij K_j
        dK[j]  += scale ds_ij Q_i
    Excluded keys get no gradient; padded query rows (i >= q_len) contribute
    nothing and get dQ = 0.  Returns (dQ, dK, dV) in fp64."""
    Q, K, V, dO = (_f64(x) for x in (Q, K, V, dO))
    B, H, n_q, d = Q.shape
    n_k = K.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    causal = bool(mask_kind & MASK_CAUSAL)
    radius = _radius_of(mask_kind, radius, n_q, n_k)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        kv_len = n_k if not (mask_kind & MASK_KEY_PADDING) else int(kv_lens[b])
        q_len = n_q if q_lens is None else int(q_lens[b])
        for h in range(H):
            for i in range(min(q_len, n_q)):
                idx = np.flatnonzero(allowed_keys(i, n_k, kv_len, causal, radius))
                if idx.size == 0:
                    continue
                s = scale * (K[b, h][idx] @ Q[b, h, i])
                e = np.exp(s - s.max())
                w = e / e.sum()
                dp = V[b, h][idx] @ dO[b, h, i]
                ds = w * (dp - (w * dp).sum())
                dV[b, h][idx] += np.outer(w, dO[b, h, i])
                dQ[b, h, i] += scale * (ds @ K[b, h][idx])
                dK[b, h][idx] += scale * np.outer(ds, Q[b, h, i])
    return dQ, dK, dV


def cache_append(Kcache, Vcache, Knew, Vnew, kv_lens):
    """Append the K/V rows of new tokens to a decoder's caches (sj-techlog
    page, KV cache section: the cache holds the K, V of tokens 0..t-1 and a
    step adds the new token's K, V; kimjiil page §3.7: only the new token's
    projections are computed per step).

    Kcache, Vcache: [B, h, n_max, d]; Knew, Vnew: [B, h, n_new, d];
    kv_lens[b]: valid cache rows of entry b *after* the append (the lengths
    the following decode step reads).  New row r of entry b lands in cache
    row kv_lens[b] - n_new + r; a row that falls outside [0, n_max) is not
    written.  Returns new (Kcache, Vcache) arrays; the inputs are unchanged.
    """
    Kc = np.array(Kcache, copy=True)
    Vc = np.array(Vcache, copy=True)
    Kn = np.asarray(Knew)
    Vn = np.asarray(Vnew)
    B, H, n_max, _ = Kc.shape
    n_new = Kn.shape[2]
    for b in range(B):
        for r in range(n_new):
            row = int(kv_lens[b]) - n_new + r
            if 0 <= row < n_max:
                Kc[b, :, row] = Kn[b, :, r]
                Vc[b, :, row] = Vn[b, :, r]
    return Kc, Vc


def head_projection(X, W, h: int):
    """Multi-head input projections, split into heads (kimjiil page §3.2.2:
    head_i = Attention(Q W_i^Q, K W_i^K, V W_i^V), W_i of shape d_model x d_k
    with d_k = d_model / h; "Attention Is All You Need를 지금 다시 읽는 법",
    multi-head section).

    X: [B, n, d_model].  W: [n_out * d_model, d_model], one block of d_model
    rows per projection (Q, K, V, or any subset in that order), each row one
    output feature -- a projection is Y = X W^T, so block j's rows 64 i ..
    64 i + 63 are head i's W_i (transposed).  Returns a list of n_out arrays
    [B, h, n, d_model / h] in fp64: output head i, position t, dimension c
    is sum_k X[b, t, k] W[j * d_model + i * d_k + c, k].
    """
    X = _f64(X)
    W = _f64(W)
    B, n, d_model = X.shape
    d_k = d_model // h
    n_out = W.shape[0] // d_model
    Y = X @ W.T  # [B, n, n_out * d_model]
    outs = []
    for j in range(n_out):
        Yj = Y[:, :, j * d_model:(j + 1) * d_model].reshape(B, n, h, d_k)
        outs.append(np.ascontiguousarray(Yj.transpose(0, 2, 1, 3)))
    return outs


def output_projection(O, Wo):
    """MultiHead = Concat(head_1, ..., head_h) W^O (kimjiil page §3.2.2):
    O [B, h, n, d_k] is concatenated along the feature axis (head i fills
    features i d_k .. (i + 1) d_k - 1) and multiplied by Wo^T, Wo being
    [d_model, h d_k] with one row per output feature.  Returns [B, n, d_model]
    in fp64."""
    O = _f64(O)
    Wo = _f64(Wo)
    B, h, n, d_k = O.shape
    concat = O.transpose(0, 2, 1, 3).reshape(B, n, h * d_k)
    return concat @ Wo.T


def multi_head_attention(Xq, Xkv, Wq, Wkv, Wo, h: int, mask_kind: int = MASK_NONE, q_lens=None,
                         kv_lens=None, scale: float | None = None):
    """The pages' multi-head attention sub-layer: queries projected from Xq,
    keys and values from Xkv (the same tensor for self-attention, the encoder
    output for encoder-decoder attention, kimjiil page §3.2.3 table),
    scaled dot-product attention per head with the given mask, then the
    output projection.  Wq [d_model, d_model], Wkv [2 d_model, d_model] (K
    block then V block), Wo [d_model, d_model].  Returns [B, n_q, d_model]."""
    (Q,) = head_projection(Xq, Wq, h)
    K, V = head_projection(Xkv, Wkv, h)
    O = attention(Q, K, V, mask_kind=mask_kind, q_lens=q_lens, kv_lens=kv_lens, scale=scale)
    return output_projection(O, Wo)


def sinusoidal_pe(pos: int, d_model: int) -> np.ndarray:
    """PE(pos, 2i) = sin(pos / 10000^(2i/d_model)), PE(pos, 2i+1) = cos(same).

    kimjiil page §3.5; baxdailygit page "삼각함수 기반 위치 인코딩 수식".
    """
    out = np.zeros(d_model, dtype=np.float64)
    for dim in range(d_model):
        i = dim // 2
        angle = pos / (10000.0 ** ((2 * i) / d_model))
        out[dim] = math.sin(angle) if dim % 2 == 0 else math.cos(angle)
    return out


def kv_cache_scalars(layers: int, tokens: int, d_model: int) -> int:
    """Scalars held by a decoder KV cache: 2 (K and V) x layers x tokens x d_model.

    sj-techlog page, "KV cache는 추론의 같은 계산을 반복하지 않게 한다".
    """
    return 2 * layers * tokens * d_model


def attention_flops(n_pairs: int, d: int) -> int:
    """Algorithmic flops of attention over n_pairs allowed (query, key) pairs.

    Each allowed pair costs one d-long dot product for QK^T and one d-long
    axpy for the weighted sum of V: 2*d + 2*d flops (multiply + add each).
    The O(n^2 * d) per-layer cost of kimjiil page §4 Table 1.
    """
    return 4 * d * n_pairs
