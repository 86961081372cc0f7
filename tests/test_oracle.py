"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these checks retypes the oracle's formula: each compares it with a
value printed on a page, a closed form, an invariant the pages state, or an
independent library routine (torch's scaled_dot_product_attention in fp64).
The pins are written as functions of the oracle module so that
test_oracle_mutations.py can run them against oracles with planted mistakes.
"""
import math

import numpy as np
import pytest
import torch

import oracle.attn_oracle as orc_mod
from golden import load

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

RNG = np.random.default_rng(20260724)


def _heads(x):
    """[n, d] -> [1, 1, n, d]"""
    return np.asarray(x, dtype=np.float64)[None, None]


# ---------------------------------------------------------------- page values
def pin_p4_two_token_example(orc):
    """baxdailygit page, "셀프 어텐션 수치 계산 시뮬레이션" steps 2-5."""
    g = load("p4_two_token_example.txt")
    Q, K, V = g["Q"], g["K"], g["V"]
    O, W = orc.attention(_heads(Q), _heads(K), _heads(V), return_weights=True)
    W, O = W[0, 0], O[0, 0]
    # step 4: the weights, printed to 2 decimals
    assert np.array_equal(np.round(W, 2), g["A"]), W
    # steps 2-3 fix the scaled logits; log-weight differences recover them
    # (softmax is shift invariant): s_i1 - s_i0 = log(w_i1 / w_i0)
    diff = np.log(W[:, 1] / W[:, 0])
    page = g["scaled"][:, 1] - g["scaled"][:, 0]
    assert np.allclose(diff, page, atol=1e-3), (diff, page)
    # step 5 was computed from A rounded to 2 dp: |dZ| <= 0.005 * sum_j |V_j|
    bound = 0.005 * np.abs(V).sum(axis=0) + 5e-4
    assert np.all(np.abs(O - g["Z"]) <= bound), (O, g["Z"])
    # and the page's own step 5 is the rounded weights times V
    assert np.allclose(np.round(W, 2) @ V, g["Z"], atol=5e-4)


def pin_p5_unmasked_and_causal(orc):
    """sj-techlog page, "직접 검증": unmasked and causal 3-token run, 6 dp."""
    g = load("p5_verification_run.txt")
    q, k, v = g["q"], g["k"], g["v"]
    tol = 1e-6  # printed with round(x, 6)
    assert abs(math.sqrt(2) - g["scale_sqrt_dk"]) < tol
    O, W = orc.attention(_heads(q), _heads(k), _heads(v), return_weights=True)
    assert np.allclose(W[0, 0, 0], g["unmasked_w0"], atol=tol)
    assert np.allclose(O[0, 0, 0], g["unmasked_out0"], atol=tol)
    Oc, Wc = orc.attention(_heads(q), _heads(k), _heads(v), mask_kind=orc.MASK_CAUSAL,
                           return_weights=True)
    for i in range(3):
        assert np.allclose(Wc[0, 0, i], g[f"causal_w{i}"], atol=tol), (i, Wc[0, 0, i])
        assert np.allclose(Oc[0, 0, i], g[f"causal_out{i}"], atol=tol), (i, Oc[0, 0, i])


def pin_p5_mask_before_softmax(orc):
    """sj-techlog page: masking *after* softmax is the page's wrong variant
    (weights sum to 0.401112, output [4.011121, 0]); the oracle must reproduce
    that number from its unmasked weights and must not produce it as its
    causal answer."""
    g = load("p5_verification_run.txt")
    q, k, v = g["q"], g["k"], g["v"]
    _, W = orc.attention(_heads(q), _heads(k), _heads(v), return_weights=True)
    wrong = np.array([W[0, 0, 0, 0], 0.0, 0.0])
    assert abs(wrong.sum() - g["wrong_post_softmax_sum"]) < 1e-6
    assert np.allclose(wrong @ v, g["wrong_post_softmax_out0"], atol=1e-6)
    Oc = orc.attention(_heads(q), _heads(k), _heads(v), mask_kind=orc.MASK_CAUSAL)
    assert not np.allclose(Oc[0, 0, 0], g["wrong_post_softmax_out0"], atol=1e-2)
    assert np.array_equal(Oc[0, 0, 0], v[0])


def pin_pe_values(orc):
    """sj-techlog page "직접 검증" (6 dp) and baxdailygit page PE simulation (2 dp)."""
    g = load("p5_verification_run.txt")
    assert np.allclose(orc.sinusoidal_pe(0, 4), g["PE_pos0_d4"], atol=1e-6)
    assert np.allclose(orc.sinusoidal_pe(1, 4), g["PE_pos1_d4"], atol=1e-6)
    p = load("p4_positional_encoding.txt")
    d = int(p["d_model"])
    for pos in range(3):
        pe = orc.sinusoidal_pe(pos, d)
        assert np.allclose(pe, p[f"PE{pos}"], atol=5e-3 + 1e-12), (pos, pe)
        # embedding + PE; the page added the rounded PE, so allow its rounding
        assert np.allclose(p[f"emb{pos}"] + pe, p[f"in{pos}"], atol=5e-3 + 1e-9)


def pin_pe_rotation(orc):
    """kimjiil page §3.5 fold-out: PE_{pos+k} = M(k) PE_pos with 2x2 blocks
    [[cos wk, sin wk], [-sin wk, cos wk]] on each (sin, cos) pair, w_i =
    10000^(-2i/d_model), independent of pos."""
    d = 512
    w = 10000.0 ** (-np.arange(0, d, 2) / d)
    for k in (1, 3, 17, 250):
        c, s = np.cos(w * k), np.sin(w * k)
        for pos in (0, 5, 63, 1000):
            a = orc.sinusoidal_pe(pos, d)
            b = orc.sinusoidal_pe(pos + k, d)
            sin_p, cos_p = a[0::2], a[1::2]
            assert np.allclose(b[0::2], c * sin_p + s * cos_p, atol=1e-9)
            assert np.allclose(b[1::2], -s * sin_p + c * cos_p, atol=1e-9)


def pin_default_scale_variance(orc):
    """kimjiil page §3.2.1 fold-out: with q, k iid N(0,1), Var(q.k) = d_k and
    the 1/sqrt(d_k) scale brings the logits to variance 1.  The oracle's
    default scale is read back through its weights: for two keys,
    log(w1/w0) = s1 - s0 has variance 2 * Var(s) = 2."""
    rng = np.random.default_rng(7)
    n, d = 20000, 64
    Q = rng.standard_normal((1, 1, n, d))
    K = rng.standard_normal((1, n, 2, d))  # a fresh key pair per query row
    ratios = np.empty(n)
    for i in range(0, n, 2000):
        _, W = orc.attention(Q[:, :, i:i + 2000].transpose(0, 2, 1, 3),
                             K[:, i:i + 2000], np.zeros((1, 2000, 2, d)),
                             return_weights=True)
        ratios[i:i + 2000] = np.log(W[:, :, 0, 1] / W[:, :, 0, 0])[0]
    var = ratios.var()
    # sampling sd of the variance estimate: 2 * sqrt(2/n) ~ 0.02
    assert abs(var - 2.0) < 0.1, var


def pin_rows_sum_to_one(orc):
    """baxdailygit page step 4 / sj-techlog Eq.(1) table: each softmax row
    sums to 1, under every mask; a ones column of V gives an output of 1."""
    B, H, n, d = 3, 2, 9, 8
    Q, K, V = (RNG.standard_normal((B, H, n, d)) for _ in range(3))
    V[..., 0] = 1.0
    kv = np.array([9, 4, 1])
    for mask in (0, 1, 2, 3):
        O, W = orc.attention(Q, K, V, mask_kind=mask, kv_lens=kv, return_weights=True)
        assert np.allclose(W.sum(-1), 1.0, atol=1e-12)
        assert np.allclose(O[..., 0], 1.0, atol=1e-12)


def pin_masked_weight_exactly_zero(orc):
    """kimjiil page §3.2.3: illegal connections get -inf logits, so their
    weight after softmax is exactly 0; sj-techlog page: no weight on pads."""
    B, H, n, d = 2, 2, 7, 8
    Q, K, V = (RNG.standard_normal((B, H, n, d)) for _ in range(3))
    kv = np.array([5, 2])
    _, W = orc.attention(Q, K, V, mask_kind=3, kv_lens=kv, return_weights=True)
    for b in range(B):
        for i in range(n):
            for j in range(n):
                if j > i or j >= kv[b]:
                    assert np.all(W[b, :, i, j] == 0.0)
                else:
                    assert np.all(W[b, :, i, j] > 0.0)


def pin_causal_prefix_invariance(orc):
    """kimjiil page §3.1 (position i depends only on outputs before it) and
    sj-techlog page failure section 2: rows <= i do not change, bit for bit,
    when any Q/K/V row after i is perturbed -- even to NaN."""
    n, d = 12, 8
    Q, K, V = (RNG.standard_normal((1, 2, n, d)) for _ in range(3))
    O = orc.attention(Q, K, V, mask_kind=orc.MASK_CAUSAL)
    for i in (0, 4, 10):
        Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
        Q2[:, :, i + 1:] = 1e3 * RNG.standard_normal(Q2[:, :, i + 1:].shape)
        K2[:, :, i + 1:] = np.nan
        V2[:, :, i + 1:] = np.inf
        O2 = orc.attention(Q2, K2, V2, mask_kind=orc.MASK_CAUSAL)
        assert np.array_equal(O[:, :, :i + 1], O2[:, :, :i + 1])


def pin_padding_invariance(orc):
    """sj-techlog page: no attention to pad; K/V rows at or beyond kv_len
    (even NaN) cannot change the output; padded query rows are 0."""
    B, H, n, d = 3, 2, 10, 8
    Q, K, V = (RNG.standard_normal((B, H, n, d)) for _ in range(3))
    kv = np.array([10, 3, 7])
    ql = np.array([10, 3, 5])
    O = orc.attention(Q, K, V, mask_kind=1, kv_lens=kv, q_lens=ql)
    K2, V2 = K.copy(), V.copy()
    for b in range(B):
        K2[b, :, kv[b]:] = np.nan
        V2[b, :, kv[b]:] = np.nan
    O2 = orc.attention(Q, K2, V2, mask_kind=1, kv_lens=kv, q_lens=ql)
    assert np.array_equal(O, O2)
    for b in range(B):
        assert np.all(O[b, :, ql[b]:] == 0.0)
        assert np.all(np.abs(O[b, :, :ql[b]]).sum(-1) > 0)


def pin_permutation(orc):
    """baxdailygit page ("I love cats" / "cats love I") and sj-techlog page
    failure section 1: without positions attention is order-blind.  Jointly
    permuting Q, K, V rows permutes O's rows; permuting K, V rows together
    leaves O unchanged."""
    n, d = 11, 8
    Q, K, V = (RNG.standard_normal((1, 1, n, d)) for _ in range(3))
    O = orc.attention(Q, K, V)
    p = RNG.permutation(n)
    O2 = orc.attention(Q[:, :, p], K[:, :, p], V[:, :, p])
    assert np.allclose(O2, O[:, :, p], atol=1e-12)
    O3 = orc.attention(Q, K[:, :, p], V[:, :, p])
    assert np.allclose(O3, O, atol=1e-12)


def pin_one_hot_key(orc):
    """A single allowed key takes weight 1 (sj-techlog page: causal position 0
    sees only its own V, [10, 0]); with a dominant logit the output tends to
    that key's value row."""
    n, d = 6, 8
    Q, K, V = (RNG.standard_normal((2, 2, n, d)) for _ in range(3))
    O = orc.attention(Q, K, V, mask_kind=1, kv_lens=np.array([1, 1]))
    assert np.array_equal(O, np.broadcast_to(V[:, :, :1], O.shape))
    Oc = orc.attention(Q, K, V, mask_kind=2)
    assert np.array_equal(Oc[:, :, 0], V[:, :, 0])
    # approximate one-hot: K rows alpha * e_j, q = e_j
    Kd = np.zeros((1, 1, n, n))
    Kd[0, 0] = 60.0 * np.eye(n)
    Qd = np.eye(n)[None, None]
    Vd = RNG.standard_normal((1, 1, n, 4))
    Od = orc.attention(Qd, Kd, Vd, scale=1.0)
    assert np.allclose(Od[0, 0], Vd[0, 0], atol=1e-20 + 1e-12)


def pin_uniform_scores(orc):
    """Q = 0 makes every allowed logit equal, so O is the plain mean of the
    allowed value rows (softmax of a constant row)."""
    B, H, n, d = 2, 2, 8, 4
    K, V = (RNG.standard_normal((B, H, n, d)) for _ in range(2))
    Q = np.zeros((B, H, n, d))
    kv = np.array([8, 5])
    O = orc.attention(Q, K, V, mask_kind=3, kv_lens=kv)
    for b in range(B):
        for i in range(n):
            lim = min(i + 1, kv[b])
            assert np.allclose(O[b, :, i], V[b, :, :lim].mean(axis=1), atol=1e-12)


def pin_large_logits_stable(orc):
    """The max-shifted softmax (the verification script on the sj-techlog
    page subtracts the max finite score) stays finite for logits far beyond
    exp's range, and reaches the one-hot limit."""
    n, d = 5, 4
    Q, K, V = (RNG.standard_normal((1, 1, n, d)) for _ in range(3))
    O = orc.attention(Q, K, V, scale=1e4)
    assert np.all(np.isfinite(O))
    S = (Q[0, 0] @ K[0, 0].T)
    assert np.allclose(O[0, 0], V[0, 0][S.argmax(axis=1)], atol=1e-12)


def pin_library_crosscheck(orc):
    """Brute force on tiny inputs against an independent library routine:
    torch's scaled_dot_product_attention in float64 on the CPU with a boolean
    mask, over every mask kind and random lengths."""
    rng = np.random.default_rng(11)
    for trial in range(40):
        B, H = rng.integers(1, 4), rng.integers(1, 3)
        mask = int(rng.integers(0, 4))
        n_q = int(rng.integers(1, 9))
        n_k = n_q if mask & 2 else int(rng.integers(1, 9))
        d = int(rng.choice([1, 2, 4, 8]))
        Q = rng.standard_normal((B, H, n_q, d))
        K = rng.standard_normal((B, H, n_k, d))
        V = rng.standard_normal((B, H, n_k, int(rng.choice([1, 3, 8]))))
        kv = rng.integers(1, n_k + 1, size=B)
        ql = rng.integers(1, n_q + 1, size=B)
        scale = float(rng.choice([0.125, 1.0 / math.sqrt(d), 2.0]))
        O = orc.attention(Q, K, V, mask_kind=mask, kv_lens=kv, q_lens=ql, scale=scale)
        allowed = np.ones((B, 1, n_q, n_k), dtype=bool)
        if mask & 1:
            allowed &= (np.arange(n_k)[None, :] < kv[:, None])[:, None, None, :]
        if mask & 2:
            allowed &= np.tril(np.ones((n_q, n_k), dtype=bool))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V),
            attn_mask=torch.from_numpy(allowed), scale=scale).numpy()
        for b in range(B):
            assert np.allclose(O[b, :, :ql[b]], ref[b, :, :ql[b]], atol=1e-12), trial
            assert np.all(O[b, :, ql[b]:] == 0.0)


def pin_decode_equals_recompute(orc):
    """kimjiil page §3.7 / sj-techlog page KV cache: the cached step computes
    the same thing as recomputing the causal self-attention of the whole
    prefix; the new token's own K/V is part of the cache."""
    n, d, B, H = 10, 8, 3, 2
    Q, K, V = (RNG.standard_normal((B, H, n, d)) for _ in range(3))
    full = orc.attention(Q, K, V, mask_kind=orc.MASK_CAUSAL)
    lens = np.array([1, 6, 10])
    q = np.stack([Q[b, :, lens[b] - 1] for b in range(B)])[:, :, None]
    Kc = K.copy()
    Vc = V.copy()
    for b in range(B):  # rows past the valid length hold garbage
        Kc[b, :, lens[b]:] = 1e6
        Vc[b, :, lens[b]:] = np.nan
    out = orc.decode(q, Kc, Vc, lens)
    for b in range(B):
        assert np.allclose(out[b, :, 0], full[b, :, lens[b] - 1], atol=1e-13)


def pin_incremental_decode_equals_recompute(orc):
    """sj-techlog page, KV cache section (and kimjiil page §3.7): a decoder
    that appends each new token's K/V to its cache and attends from that
    token alone computes, step by step, the rows of causal self-attention
    over the whole sequence.  Caches start as NaN garbage; some entries are
    fed one token per step, one with a first block of 3 (a prefill), so the
    append's row placement and the decode's length rule are both pinned."""
    n, d, B, H, n_max = 9, 8, 3, 2, 12
    Q, K, V = (RNG.standard_normal((B, H, n, d)) for _ in range(3))
    full = orc.attention(Q, K, V, mask_kind=orc.MASK_CAUSAL)
    Kc = np.full((B, H, n_max, d), np.nan)
    Vc = np.full((B, H, n_max, d), np.nan)
    # entry 0 and 1: one token per step; entry 2: tokens 0-2 at once, then one per step
    for t in range(n):
        if t < 2:
            new_rows = {0: [t], 1: [t], 2: []}
        else:
            new_rows = {0: [t], 1: [t], 2: [0, 1, 2] if t == 2 else [t]}
        for b in range(B):
            rows = new_rows[b]
            if not rows:
                continue
            lens = np.zeros(B, dtype=np.int64)
            lens[b] = rows[-1] + 1
            Kn = np.zeros((B, H, len(rows), d))
            Vn = np.zeros((B, H, len(rows), d))
            Kn[b] = K[b][:, rows]
            Vn[b] = V[b][:, rows]
            Kb, Vb = orc.cache_append(Kc[b:b + 1], Vc[b:b + 1], Kn[b:b + 1], Vn[b:b + 1], lens[b:b + 1])
            Kc[b:b + 1], Vc[b:b + 1] = Kb, Vb
        lens = np.array([t + 1, t + 1, t + 1 if t >= 2 else 0])
        for b in range(B):
            if lens[b] == 0:
                continue
            out = orc.decode(Q[b:b + 1, :, t:t + 1], Kc[b:b + 1], Vc[b:b + 1], lens[b:b + 1])
            assert np.allclose(out[0, :, 0], full[b, :, t], atol=1e-13), (t, b)


def pin_cache_append_rows(orc):
    """The append writes exactly the new rows: row r of the block lands at
    cache row kv_len - n_new + r; every other cache row is unchanged, and a
    row that would fall outside [0, n_max) is not written."""
    B, H, n_max, d, n_new = 4, 2, 6, 3, 2
    Kc = RNG.standard_normal((B, H, n_max, d))
    Vc = RNG.standard_normal((B, H, n_max, d))
    Kn = RNG.standard_normal((B, H, n_new, d))
    Vn = RNG.standard_normal((B, H, n_new, d))
    lens = np.array([2, 6, 1, 7])  # 1: first new row would be row -1; 7: last would be row 6
    K2, V2 = orc.cache_append(Kc, Vc, Kn, Vn, lens)
    for b in range(B):
        for row in range(n_max):
            r = row - (lens[b] - n_new)
            if 0 <= r < n_new:
                assert np.array_equal(K2[b, :, row], Kn[b, :, r]) and np.array_equal(V2[b, :, row], Vn[b, :, r])
            else:
                assert np.array_equal(K2[b, :, row], Kc[b, :, row]) and np.array_equal(V2[b, :, row], Vc[b, :, row])
    assert np.array_equal(K2[2, :, 0], Kn[2, :, 1]) and np.array_equal(K2[3, :, 5], Kn[3, :, 0])


def pin_cross_attention_decode(orc):
    """kimjiil page §3.2.3 (encoder-decoder attention: queries from the
    decoder, keys and values from the encoder output) with §3.7's cache: a
    decode step against a fixed encoder cache is the key-padded cross
    attention of that one query, and does not depend on the cache rows past
    the source length."""
    B, H, n_src, d = 3, 2, 7, 5
    q = RNG.standard_normal((B, H, 1, d))
    Ke, Ve = RNG.standard_normal((B, H, n_src, d)), RNG.standard_normal((B, H, n_src, d))
    src = np.array([7, 1, 4])
    out = orc.decode(q, Ke, Ve, src)
    ref = orc.attention(q, Ke, Ve, mask_kind=orc.MASK_KEY_PADDING, kv_lens=src)
    assert np.allclose(out, ref, atol=1e-14)
    # one query, so the weights are softmax(K q s) over the first src rows
    for b in range(B):
        for h in range(H):
            s = Ke[b, h, :src[b]] @ q[b, h, 0] / math.sqrt(d)
            w = np.exp(s - s.max())
            assert np.allclose(out[b, h, 0], (w / w.sum()) @ Ve[b, h, :src[b]], atol=1e-13)


def pin_multi_head_vs_torch(orc):
    """kimjiil page §3.2.2 multi-head attention, end to end (input
    projections split into h heads of d_k = d_model / h, attention per head,
    concatenation, output projection) against torch's own implementation of
    the same sub-layer (torch.nn.functional.multi_head_attention_forward,
    fp64, no biases), for self-attention with key padding, causal
    self-attention, and cross attention with different query and key
    lengths."""
    rng = np.random.default_rng(77)
    B, h, d_k = 2, 4, 4
    d = h * d_k
    Wq = rng.standard_normal((d, d)) / math.sqrt(d)
    Wkv = rng.standard_normal((2 * d, d)) / math.sqrt(d)
    Wo = rng.standard_normal((d, d)) / math.sqrt(d)
    in_w = torch.from_numpy(np.concatenate([Wq, Wkv]))
    for case in ("self_kpad", "causal", "cross"):
        n_q, n_k = (5, 7) if case == "cross" else (6, 6)
        Xq = rng.standard_normal((B, n_q, d))
        Xkv = Xq if case != "cross" else rng.standard_normal((B, n_k, d))
        kv_lens = np.array([n_k, 3]) if case != "causal" else None
        mask = {"self_kpad": orc.MASK_KEY_PADDING, "causal": orc.MASK_CAUSAL,
                "cross": orc.MASK_KEY_PADDING}[case]
        got = orc.multi_head_attention(Xq, Xkv, Wq, Wkv, Wo, h, mask_kind=mask, kv_lens=kv_lens)
        kpm = None
        if kv_lens is not None:
            kpm = torch.from_numpy(np.arange(n_k)[None, :] >= kv_lens[:, None])
        am = torch.triu(torch.ones(n_q, n_k, dtype=torch.bool), 1) if case == "causal" else None
        ref, _ = torch.nn.functional.multi_head_attention_forward(
            torch.from_numpy(Xq).transpose(0, 1), torch.from_numpy(Xkv).transpose(0, 1),
            torch.from_numpy(Xkv).transpose(0, 1), d, h, in_w, None, None, None, False, 0.0,
            torch.from_numpy(Wo), None, training=False, key_padding_mask=kpm,
            need_weights=False, attn_mask=am)
        assert np.allclose(got, ref.transpose(0, 1).numpy(), atol=1e-12), case


def pin_head_split_and_concat(orc):
    """Head i of a projection uses rows i d_k .. (i + 1) d_k - 1 of its weight
    block (brute force over every output element), and the concatenation is
    the exact inverse of the split: projecting with the identity and
    concatenating with the identity returns X."""
    rng = np.random.default_rng(78)
    B, n, h, d_k = 2, 3, 3, 2
    d = h * d_k
    X = rng.standard_normal((B, n, d))
    W = rng.standard_normal((2 * d, d))
    A, C = orc.head_projection(X, W, h)
    for j, out in enumerate((A, C)):
        for b in range(B):
            for i in range(h):
                for t in range(n):
                    for c in range(d_k):
                        ref = sum(X[b, t, k] * W[j * d + i * d_k + c, k] for k in range(d))
                        assert abs(out[b, i, t, c] - ref) < 1e-12
    (I,) = orc.head_projection(X, np.eye(d), h)
    assert np.array_equal(orc.output_projection(I, np.eye(d)), X)
    # one head with identity projections is plain attention (kimjiil page §3.2.2 with h = 1)
    Y = orc.multi_head_attention(X, X, np.eye(d), np.vstack([np.eye(d), np.eye(d)]), np.eye(d), 1)
    assert np.allclose(Y, orc.attention(X[:, None], X[:, None], X[:, None])[:, 0], atol=1e-13)


def pin_backward_vs_autograd(orc):
    """The gradients of the attention map against torch autograd in fp64
    (an independent differentiation of the forward definition), for every
    mask kind, padded query rows and a row with no allowed key."""
    rng = np.random.default_rng(91)
    B, H, n, d = 3, 2, 7, 5
    scale = 0.37
    for mask in (0, 1, 2, 3):
        Q, K, V, dO = (rng.standard_normal((B, H, n, d)) for _ in range(4))
        kl = np.array([7, 3, 0]) if mask & 1 else None
        ql = np.array([7, 5, 2])
        dQ, dK, dV = orc.attention_backward(Q, K, V, dO, mask_kind=mask, q_lens=ql, kv_lens=kl, scale=scale)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (Q, K, V))
        allowed = np.zeros((B, 1, n, n), dtype=bool)
        for b in range(B):
            for i in range(n):
                allowed[b, 0, i] = orc.allowed_keys(i, n, n if kl is None else kl[b], bool(mask & 2))
        S = tq @ tk.transpose(-1, -2) * scale
        S = S.masked_fill(~torch.from_numpy(allowed), float("-inf"))
        P = torch.softmax(S, dim=-1).nan_to_num(0.0)   # rows with no key: weights 0
        O = P @ tv
        qmask = torch.from_numpy((np.arange(n)[None, :] < ql[:, None]).astype(np.float64))[:, None, :, None]
        (O * torch.from_numpy(dO) * qmask).sum().backward()
        for got, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
            assert np.allclose(got, ref.numpy(), atol=1e-12), mask


def pin_backward_finite_differences(orc):
    """Central differences of L = sum(O * dO) reproduce the analytic
    gradients (a check of the formulas that uses only the forward)."""
    rng = np.random.default_rng(92)
    B, H, n, d = 1, 1, 5, 3
    Q, K, V, dO = (rng.standard_normal((B, H, n, d)) for _ in range(4))
    dQ, dK, dV = orc.attention_backward(Q, K, V, dO, mask_kind=orc.MASK_CAUSAL, scale=0.5)
    L = lambda q, k, v: float((orc.attention(q, k, v, mask_kind=orc.MASK_CAUSAL, scale=0.5) * dO).sum())
    eps = 1e-6
    for X, G, which in ((Q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        for pos in ((0, 0, 0, 0), (0, 0, 2, 1), (0, 0, 4, 2)):
            Xp, Xm = X.copy(), X.copy()
            Xp[pos] += eps
            Xm[pos] -= eps
            args_p = [Q, K, V]
            args_m = [Q, K, V]
            args_p[which], args_m[which] = Xp, Xm
            fd = (L(*args_p) - L(*args_m)) / (2 * eps)
            assert abs(fd - G[pos]) < 1e-7, (which, pos)


def pin_backward_shift_invariance(orc):
    """Softmax ignores a constant added to every logit of a row, so adding
    one vector to every key leaves O unchanged: the key gradients of each
    (b, h) sum to zero.  Excluded keys and padded rows get exactly zero
    gradient; the value gradients of a row's keys sum to that row's dO
    (the weights sum to one)."""
    rng = np.random.default_rng(93)
    B, H, n, d = 2, 2, 6, 4
    Q, K, V, dO = (rng.standard_normal((B, H, n, d)) for _ in range(4))
    kl = np.array([6, 4])
    dQ, dK, dV = orc.attention_backward(Q, K, V, dO, mask_kind=orc.MASK_KEY_PADDING, kv_lens=kl)
    assert np.allclose(dK.sum(axis=2), 0.0, atol=1e-12)
    assert np.all(dK[1, :, 4:] == 0) and np.all(dV[1, :, 4:] == 0)
    assert np.allclose(dV.sum(axis=2), dO.sum(axis=2), atol=1e-12)
    # a single allowed key: O = V_0 exactly, so dV_0 = dO and dQ = dK = 0
    dQ1, dK1, dV1 = orc.attention_backward(Q, K, V, dO, mask_kind=orc.MASK_KEY_PADDING, kv_lens=np.array([1, 1]))
    assert np.allclose(dV1[:, :, 0], dO.sum(axis=2)) and np.all(dQ1 == 0) and np.all(dK1 == 0)


def pin_row_logsumexp(orc):
    """The log-normaliser of each row: exp(s_ij - lse_i) are the softmax
    weights (they sum to one), matching the weights of the forward."""
    rng = np.random.default_rng(94)
    Q, K, V = (rng.standard_normal((2, 2, 5, 3)) for _ in range(3))
    kl = np.array([5, 2])
    lse = orc.row_logsumexp(Q, K, mask_kind=3, kv_lens=kl, scale=0.7)
    _, W = orc.attention(Q, K, V, mask_kind=3, kv_lens=kl, scale=0.7, return_weights=True)
    for b in range(2):
        for h in range(2):
            for i in range(5):
                s = 0.7 * (K[b, h] @ Q[b, h, i])
                ok = orc.allowed_keys(i, 5, kl[b], True)
                assert np.allclose(np.where(ok, np.exp(s - lse[b, h, i]), 0.0), W[b, h, i], atol=1e-14)


def _band(n, radius, causal):
    """Allowed (query, key) pairs of restricted self-attention built with
    torch's own band routines: keys i - radius .. i + radius (kimjiil page
    §4, Table 1's neighbourhood of r = 2 radius + 1 positions), only the
    past half under the causal mask."""
    ones = torch.ones(n, n, dtype=torch.bool)
    band = torch.triu(ones, -radius) & torch.tril(ones, 0 if causal else radius)
    return band.numpy()


def pin_restricted_slices(orc):
    """Each row of restricted self-attention is plain attention of its query
    over the contiguous slice of keys around it (cut by index arithmetic,
    clipped at both ends of the sequence and at kv_len), computed by torch's
    scaled_dot_product_attention in fp64 with no mask at all."""
    rng = np.random.default_rng(95)
    B, H, n, d = 2, 2, 11, 4
    Q, K, V = (rng.standard_normal((B, H, n, d)) for _ in range(3))
    kl = np.array([11, 6])
    for causal in (False, True):
        for radius in (0, 1, 3, 10, 25):
            mask = orc.MASK_RESTRICTED | orc.MASK_KEY_PADDING | (orc.MASK_CAUSAL if causal else 0)
            O = orc.attention(Q, K, V, mask_kind=mask, kv_lens=kl, scale=0.4, radius=radius)
            for b in range(B):
                for i in range(n):
                    lo = max(0, i - radius)
                    hi = min(i + 1 if causal else i + radius + 1, kl[b])
                    if lo >= hi:
                        assert np.all(O[b, :, i] == 0.0), (causal, radius, b, i)
                        continue
                    ref = torch.nn.functional.scaled_dot_product_attention(
                        torch.from_numpy(Q[b, :, i:i + 1]), torch.from_numpy(K[b, :, lo:hi]),
                        torch.from_numpy(V[b, :, lo:hi]), scale=0.4).numpy()
                    assert np.allclose(O[b, :, i], ref[:, 0], atol=1e-12), (causal, radius, b, i)


def pin_restricted_vs_torch_band(orc):
    """Whole-matrix restricted self-attention against torch's fp64 attention
    with a boolean band mask from triu/tril, for radii from 0 to beyond the
    sequence, with and without the causal mask."""
    rng = np.random.default_rng(96)
    B, H, n, d = 1, 3, 9, 8
    Q, K, V = (rng.standard_normal((B, H, n, d)) for _ in range(3))
    for causal in (False, True):
        for radius in (0, 2, 4, 8, 100):
            mask = orc.MASK_RESTRICTED | (orc.MASK_CAUSAL if causal else 0)
            O = orc.attention(Q, K, V, mask_kind=mask, scale=0.3, radius=radius)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V),
                attn_mask=torch.from_numpy(_band(n, radius, causal)), scale=0.3).numpy()
            assert np.allclose(O, ref, atol=1e-12), (causal, radius)


def pin_restricted_closed_forms(orc):
    """kimjiil page §4, Table 1: a query sees r = 2 radius + 1 neighbours
    (radius + 1 under the causal mask), fewer only at the sequence ends.
    Radius 0 leaves each position only itself, so O = V exactly; a radius
    that spans the sequence is plain (or causal) self-attention."""
    rng = np.random.default_rng(97)
    n, d, radius = 12, 4, 3
    Q, K, V = (rng.standard_normal((1, 2, n, d)) for _ in range(3))
    for causal in (False, True):
        cm = orc.MASK_CAUSAL if causal else 0
        _, W = orc.attention(Q, K, V, mask_kind=orc.MASK_RESTRICTED | cm, radius=radius, return_weights=True)
        for i in range(n):
            want = (min(i, radius) + 1) if causal else (min(i, radius) + min(n - 1 - i, radius) + 1)
            assert np.count_nonzero(W[0, 0, i]) == want, (causal, i)
            if radius <= i <= n - 1 - radius:
                assert want == (radius + 1 if causal else 2 * radius + 1)
        O0 = orc.attention(Q, K, V, mask_kind=orc.MASK_RESTRICTED | cm, radius=0)
        assert np.array_equal(O0, V)
        full = orc.attention(Q, K, V, mask_kind=cm)
        wide = orc.attention(Q, K, V, mask_kind=orc.MASK_RESTRICTED | cm, radius=n - 1)
        assert np.allclose(full, wide, atol=1e-14)


def pin_restricted_backward_and_lse(orc):
    """Gradients and row log-normalisers under the restricted mask against
    torch autograd and torch.logsumexp in fp64, with the band built by
    torch's triu/tril."""
    rng = np.random.default_rng(98)
    B, H, n, d, scale = 1, 2, 8, 3, 0.6
    for causal in (False, True):
        for radius in (0, 1, 3):
            mask = orc.MASK_RESTRICTED | (orc.MASK_CAUSAL if causal else 0)
            Q, K, V, dO = (rng.standard_normal((B, H, n, d)) for _ in range(4))
            dQ, dK, dV = orc.attention_backward(Q, K, V, dO, mask_kind=mask, scale=scale, radius=radius)
            lse = orc.row_logsumexp(Q, K, mask_kind=mask, scale=scale, radius=radius)
            tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (Q, K, V))
            S = (tq @ tk.transpose(-1, -2) * scale).masked_fill(
                ~torch.from_numpy(_band(n, radius, causal)), float("-inf"))
            (torch.softmax(S, dim=-1) @ tv * torch.from_numpy(dO)).sum().backward()
            for got, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
                assert np.allclose(got, ref.numpy(), atol=1e-12), (causal, radius)
            assert np.allclose(lse, torch.logsumexp(S, dim=-1).detach().numpy(), atol=1e-12)


def pin_kv_cache_size(orc):
    """sj-techlog page KV cache arithmetic: 2 x 6 x 128 x 512 scalars,
    3.0 MiB in fp32 and 1.5 MiB in fp16."""
    g = load("p5_verification_run.txt")
    n = orc.kv_cache_scalars(6, 128, 512)
    assert n == int(g["kv_cache_scalars"])
    assert round(n * 4 / 2 ** 20, 3) == g["kv_cache_mib_fp32"]
    assert round(n * 2 / 2 ** 20, 3) == g["kv_cache_mib_fp16"]


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__[4:] for p in PINS])
def test_pin(pin):
    pin(orc_mod)


def test_monte_carlo_dot_product_variance():
    """kimjiil page §3.2.1 fold-out and sj-techlog page "왜 √d_k로 나누는가":
    E[q.k] = 0 and Var(q.k) = d_k for iid N(0,1) entries; after 1/sqrt(d_k)
    the variance is 1.  10^6 samples: the sd of the variance estimate is
    about 0.14 %, so +-1 % is a > 6 sigma band."""
    rng = np.random.default_rng(123)
    d = 64
    s = np.empty(10 ** 6)
    for i in range(0, 10 ** 6, 10 ** 5):
        q = rng.standard_normal((10 ** 5, d))
        k = rng.standard_normal((10 ** 5, d))
        s[i:i + 10 ** 5] = (q * k).sum(1)
    assert abs(s.mean()) < 0.05
    assert abs(s.var() / d - 1) < 0.01
    assert abs((s / math.sqrt(d)).var() - 1) < 0.01


def test_flop_model_long_causal():
    """Only allowed pairs are counted: n(n+1)/2 per head under the causal
    mask; 4 d flops per pair (kimjiil page §4 Table 1: O(n^2 d))."""
    import workloads
    pairs = workloads.allowed_pairs(2, 8192, 8192, 1)
    assert pairs == 8192 * 8193 // 2
    assert orc_mod.attention_flops(pairs * 16, 64) == 137_455_730_688


def test_pair_count_restricted():
    """The counting of the flop model for restricted self-attention agrees
    with the oracle's own masks by brute force (kimjiil page §4 Table 1:
    O(r n d) work with r = 2 radius + 1), including key padding, query
    padding and the causal half-window."""
    import workloads
    rng = np.random.default_rng(99)
    for trial in range(30):
        B, n = int(rng.integers(1, 4)), int(rng.integers(1, 40))
        radius = int(rng.integers(0, 45))
        mask = 4 | int(rng.integers(0, 4))
        kl = rng.integers(0, n + 1, size=B) if mask & 1 else None
        ql = rng.integers(0, n + 1, size=B)
        want = 0
        for b in range(B):
            for i in range(int(ql[b])):
                want += int(orc_mod.allowed_keys(i, n, n if kl is None else int(kl[b]), bool(mask & 2),
                                                 radius).sum())
        assert workloads.allowed_pairs(mask, n, n, B, ql, kl, radius=radius) == want, trial
    assert workloads.allowed_pairs(4, 8192, 8192, 1, radius=256) == 8192 * 513 - 256 * 257
