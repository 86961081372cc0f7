/*
 * headattn.h -- C ABI of the MI355X (gfx950) scaled dot-product attention
 * library libheadattn.so.
 *
 * The library computes, per batch entry b and head h,
 *     O = softmax(Q K^T * scale + M) V
 * ("[논문 리뷰]Attention Is All You Need", §3.2.1, the Attention(Q,K,V)
 * equation; the masked form with an additive M of 0 / -inf is the one on
 * "Attention Is All You Need를 지금 다시 읽는 법", computation section), for
 * the three uses the pages list (kimjiil page §3.2.3 table: encoder
 * self-attention, masked decoder self-attention, encoder-decoder attention)
 * and for one KV-cache decode step (kimjiil page §3.7; "Attention Is All You
 * Need 해부", section "KV cache는 추론의 같은 계산을 반복하지 않게 한다").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Every tensor is contiguous row-major [B, h, n, d]: Q and O use
 *   n = n_q, K and V use n = n_k.  d must be 64 (d_k = d_v = d_model / h =
 *   64, kimjiil page §3.2.2).  Element type is bf16 or fp32 (attn_dtype), the
 *   same for inputs and output.  Accumulation is always fp32.
 * Pointers.  Tensor and length pointers are DEVICE pointers (HIP device
 *   memory, or memory the device can read) owned by the caller; the library
 *   keeps no reference after the call returns.  Inputs must not alias O.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  All work is enqueued on it; calls return without synchronising,
 *   and a fault inside a kernel surfaces at the caller's next synchronisation.
 * Errors.  Arguments are validated on the host before any HIP call; on error
 *   nothing is enqueued and a non-zero attn_status is returned.  The library
 *   never aborts, prints or synchronises (except in the opt-in length check
 *   below).  ATTN_ERR_HIP means a HIP launch reported an error.
 * Lengths.  q_lens / kv_lens are device int32[B].  They are NOT read on the
 *   host: 0 <= len <= n is a precondition.  Kernels clamp every length into
 *   [0, n], so an out-of-range length never causes an out-of-bounds access.
 *   With the environment variable ATTN_CHECK=1 the entry points copy the
 *   lengths to the host (a synchronising copy on `stream`) and return
 *   ATTN_ERR_BAD_LENGTHS when one is out of range.
 * Allocation.  Entry points allocate no memory; decode's scratch is a
 *   caller-provided workspace.
 * Lengths of attn_cache_append are the one exception to clamping: a row
 *   whose destination falls outside the cache is skipped instead.
 * Empty calls.  B = 0, h = 0 or n_q = 0 is a valid call that does nothing.
 *   n_k = 0 (no keys) writes every row of O as 0; K and V may then be NULL.
 */
#ifndef HEADATTN_H
#define HEADATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O. */
typedef enum {
  ATTN_BF16 = 0, /* bfloat16 storage, bf16 MFMA products, fp32 accumulation */
  ATTN_F32 = 1   /* float32 storage and arithmetic (the fp32 check path)     */
} attn_dtype;

/* Shape of one call.  For attn_decode, n_q must be 1 and n_k is the cache
 * capacity n_max (rows per (b, h) slice of Kcache / Vcache). */
typedef struct {
  int32_t B;     /* batch entries, >= 0                 */
  int32_t h;     /* heads, >= 0                         */
  int32_t n_q;   /* query rows per (b, h), 0 .. 2^24-1  */
  int32_t n_k;   /* key/value rows per (b, h), 0 .. 2^24-1 */
  int32_t d;     /* head dimension, must be 64          */
  int32_t dtype; /* attn_dtype                          */
} attn_layout;

/* Mask kinds, bit flags; 3 = causal with key padding.
 * Key padding (kimjiil page §3.2.3; sj-techlog page failure section 2, "pad
 * token에 attention이 가지 않는가"): key j of batch entry b is excluded when
 * j >= kv_lens[b].
 * Causal (kimjiil page §3.2.3 and §3.1; sj-techlog page, section "mask는
 * softmax 전에 더해야 한다", 4x4 table): key j is excluded for query i when
 * j > i (top-left aligned; requires n_q == n_k).
 * Restricted (attn_forward_restricted only; kimjiil page §4, Table 1: each
 * position attends to a neighbourhood of r positions around it, O(r n d)
 * work): key j is excluded for query i when |i - j| > radius, so a row sees
 * r = 2 radius + 1 keys, or radius + 1 (i - radius .. i) together with
 * causal; requires n_q == n_k.
 * An excluded key gets logit -inf before the softmax: its weight is exactly 0
 * and its K/V contents (even NaN) never reach O. */
enum {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_KEY_PADDING = 1,
  ATTN_MASK_CAUSAL = 2,
  ATTN_MASK_RESTRICTED = 4
};

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL_POINTER = 1, /* a required pointer is NULL                    */
  ATTN_ERR_BAD_SHAPE = 2,    /* negative size, d != 64, n_q or n_k above
                                2^24 - 1 rows per (b, h), size overflow,
                                n_q != 1 for decode, or an input pointer
                                equal to O                                    */
  ATTN_ERR_BAD_DTYPE = 3,    /* dtype not an attn_dtype                       */
  ATTN_ERR_BAD_MASK = 4,     /* unknown bits; causal or restricted with
                                n_q != n_k; ATTN_MASK_RESTRICTED outside
                                attn_forward_restricted (or missing there);
                                radius < 0; kv_lens given without
                                ATTN_MASK_KEY_PADDING                         */
  ATTN_ERR_BAD_LENGTHS = 5,  /* (ATTN_CHECK=1 only) a length outside [0, n]   */
  ATTN_ERR_BAD_SCALE = 6,    /* scale is not finite                           */
  ATTN_ERR_WORKSPACE = 7,    /* decode workspace NULL or smaller than needed  */
  ATTN_ERR_HIP = 8,          /* a HIP runtime call failed                     */
  ATTN_ERR_SCRATCH_LIMIT = 9 /* attn_decode_noalloc: the layout needs more
                                than ATTN_DECODE_NOALLOC_MAX_BYTES of scratch */
} attn_status;

/*
 * attn_forward -- O = softmax(Q K^T * scale + M) V for every (b, h).
 *
 *   Q       [B, h, n_q, 64]  device, read
 *   K, V    [B, h, n_k, 64]  device, read
 *   layout  shapes and element type (bf16 or fp32)
 *   mask_kind  ATTN_MASK_* flags (see above)
 *   q_lens  device int32[B] or NULL.  Query rows i >= q_lens[b] of O are
 *           written as 0 (padded query positions); NULL = all n_q rows valid.
 *   kv_lens device int32[B]; required iff mask_kind has
 *           ATTN_MASK_KEY_PADDING, must be NULL otherwise.
 *   scale   multiplies Q K^T; finite.  The pages' choice is 1/sqrt(d_k) =
 *           0.125 (kimjiil page §3.2.1 variance argument); the caller passes it.
 *   O       [B, h, n_q, 64]  device, written in full (every row).
 *   stream  hipStream_t or NULL.
 * A row with no allowed key (kv_len = 0) is written as 0, never NaN.
 * Numerics: bf16 inputs are multiplied on MFMA with fp32 accumulation; the
 * softmax weights are rounded to bf16 once before the product with V; the
 * running max, running sum and output accumulator stay fp32; O is rounded
 * to bf16 (nearest even).  The fp32 path computes in fp32 throughout.
 */
attn_status attn_forward(const void* Q, const void* K, const void* V,
                         attn_layout layout, int32_t mask_kind,
                         const int32_t* q_lens, const int32_t* kv_lens,
                         float scale, void* O, void* stream);

/*
 * attn_forward_lse -- attn_forward that also writes each query row's
 * log-sum-exp, the normaliser of its softmax, which the backward pass
 * (attn_backward) uses to recompute the weights without a second forward.
 *
 *   LSE  device fp32 [B, h, n_q], written: LSE[b, h, i] = ln sum_j
 *        exp(scale q_i . k_j) over the allowed keys j (natural log); -inf
 *        for a padded query row or a row with no allowed key.
 * Every other argument, the output O and the error behaviour are those of
 * attn_forward; LSE = NULL (with a non-empty call) is ATTN_ERR_NULL_POINTER.
 */
attn_status attn_forward_lse(const void* Q, const void* K, const void* V,
                             attn_layout layout, int32_t mask_kind,
                             const int32_t* q_lens, const int32_t* kv_lens,
                             float scale, void* O, float* LSE, void* stream);

/*
 * attn_forward_restricted -- restricted self-attention (kimjiil page §4,
 * Table 1 and the note under it): attn_forward where query i attends only
 * to keys i - radius .. i + radius (i - radius .. i with ATTN_MASK_CAUSAL),
 * so the work per row is O(r d) with r = 2 radius + 1 instead of O(n d).
 *
 *   mask_kind  ATTN_MASK_RESTRICTED, optionally with ATTN_MASK_KEY_PADDING
 *              and ATTN_MASK_CAUSAL; n_q must equal n_k.
 *   radius     >= 0; a radius of n_k - 1 or more is plain (or causal)
 *              self-attention.  radius 0 gives O = V on every valid row.
 *   LSE        device fp32 [B, h, n_q] or NULL; when given, written as by
 *              attn_forward_lse (over the row's window).
 * Q, K, V, layout, q_lens, kv_lens, scale, O and stream are those of
 * attn_forward; so are the numerics and the error behaviour.  A row whose
 * window holds no valid key (key padding) is written as 0.
 */
attn_status attn_forward_restricted(const void* Q, const void* K, const void* V,
                                    attn_layout layout, int32_t mask_kind,
                                    const int32_t* q_lens, const int32_t* kv_lens,
                                    int32_t radius, float scale, void* O,
                                    float* LSE, void* stream);

/*
 * attn_decode -- one KV-cache decode step: for each (b, h) the single new
 * query attends to the kv_lens[b] valid rows of the cache, which already
 * include the new token's own K/V (the caller appends first; sj-techlog
 * page, KV cache section: "K,V = cached 0..t-1 + the new token").
 *
 *   q              [B, h, 1, 64]      device, read
 *   Kcache, Vcache [B, h, n_max, 64]  device, read; rows >= kv_lens[b] are
 *                  never used (may hold anything, including NaN)
 *   cache_layout   B, h, n_q = 1, n_k = n_max, d = 64, dtype
 *   kv_lens        device int32[B], required; kv_lens[b] = 0 gives a 0 row
 *   scale          finite
 *   O              [B, h, 1, 64]      device, written
 *   workspace      device buffer of at least
 *                  attn_decode_workspace_bytes(cache_layout) bytes, owned by
 *                  the caller; its contents on entry do not matter and are
 *                  overwritten (split partials).  Two calls that share a
 *                  workspace must be ordered (same stream).
 *   stream         hipStream_t or NULL.
 * Two kernels run on `stream`: split partials over fixed-size key chunks,
 * then a merge of the partials into O.
 */
attn_status attn_decode(const void* q, const void* Kcache, const void* Vcache,
                        attn_layout cache_layout, const int32_t* kv_lens,
                        float scale, void* O, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * attn_cache_append -- write the K/V rows of new tokens into a decoder's
 * caches: the cache update that precedes attn_decode (sj-techlog page, KV
 * cache section: a step's cache holds the K, V of tokens 0..t-1 plus the new
 * token's; kimjiil page §3.7: per step only the new token's K, V are
 * computed).  A block of n_new > 1 rows is a prefill of several tokens.
 *
 *   Knew, Vnew     [B, h, n_new, 64]  device, read
 *   Kcache, Vcache [B, h, n_max, 64]  device, written in place: only the
 *                  rows the block lands on change
 *   cache_layout   B, h, n_q = n_new (rows appended per (b, h)),
 *                  n_k = n_max, d = 64, dtype
 *   kv_lens        device int32[B], required: the valid rows of entry b
 *                  AFTER the append, i.e. the lengths the following
 *                  attn_decode reads.  Row r of the block lands in cache row
 *                  kv_lens[b] - n_new + r; a row that would fall outside
 *                  [0, n_max) is not written, so no length can cause an
 *                  out-of-bounds write.  With ATTN_CHECK=1 a length outside
 *                  [n_new, n_max] returns ATTN_ERR_BAD_LENGTHS.
 *   stream         hipStream_t or NULL.
 * A pure copy: the written cache rows are bit-identical to the new rows.
 * The new rows must not overlap the caches (ATTN_ERR_BAD_SHAPE when a base
 * pointer coincides).  n_new = 0, B = 0 or h = 0 does nothing.
 */
attn_status attn_cache_append(const void* Knew, const void* Vnew, void* Kcache,
                              void* Vcache, attn_layout cache_layout,
                              const int32_t* kv_lens, void* stream);

/*
 * attn_head_projection -- the multi-head input projections, written straight
 * into the per-head layout the attention calls read ("[논문 리뷰]Attention Is
 * All You Need", §3.2.2: head_i = Attention(Q W_i^Q, K W_i^K, V W_i^V) with
 * W_i of shape d_model x d_k, d_k = d_model / h = 64).
 *
 *   X       [B, n, d_model] bf16, device, read (d_model = 64 h)
 *   W       [n_out * d_model, d_model] bf16, device, read: n_out blocks of
 *           d_model rows, one row per output feature (a projection is
 *           Y = X W^T, the convention of a linear layer's weight), in the
 *           order the outputs are given; rows 64 i .. 64 i + 63 of a block
 *           are head i's projection
 *   layout  B, h, n_q = n (rows of X per batch entry), n_k ignored, d = 64,
 *           dtype = ATTN_BF16 (the only type of this entry point)
 *   n_out   1, 2 or 3: how many projections (Q; K and V; or Q, K and V)
 *   out0..2 [B, h, n, 64] bf16, device, written: out_j[b, i, t, c] =
 *           sum_k X[b, t, k] W[j d_model + 64 i + c, k]; unused ones NULL
 *   stream  hipStream_t or NULL.
 * fp32 accumulation, outputs rounded to bf16 (nearest even).  Self-attention
 * projects Q, K, V of one X (n_out = 3); encoder-decoder attention projects
 * Q from the decoder (n_out = 1) and K, V from the encoder output (n_out =
 * 2).  No output may alias X or W.  Every tensor must be under 2 GiB.
 */
attn_status attn_head_projection(const void* X, const void* W, attn_layout layout,
                                 int32_t n_out, void* out0, void* out1, void* out2,
                                 void* stream);

/*
 * attn_output_projection -- MultiHead = Concat(head_1, ..., head_h) W^O
 * (kimjiil page §3.2.2), reading the attention output O in its per-head
 * layout (no concatenation copy).
 *
 *   O       [B, h, n, 64] bf16, device, read (the attn_forward output)
 *   Wo      [d_model, d_model] bf16, device, read: one row per output
 *           feature; input feature 64 i + c is dimension c of head i
 *   layout  B, h, n_q = n, n_k ignored, d = 64, dtype = ATTN_BF16
 *   Y       [B, n, d_model] bf16, device, written:
 *           Y[b, t, f] = sum_{i, c} O[b, i, t, c] Wo[f, 64 i + c]
 *   stream  hipStream_t or NULL.
 * fp32 accumulation, Y rounded to bf16.  Y must not alias O or Wo.  Every
 * tensor must be under 2 GiB.
 */
attn_status attn_output_projection(const void* O, const void* Wo, attn_layout layout, void* Y,
                                   void* stream);

/*
 * attn_backward -- gradients of O = softmax(Q K^T * scale + M) V (the map of
 * "[논문 리뷰]Attention Is All You Need", §3.2.1, trained end to end in §5):
 * given dO = dL/dO, returns dL/dQ, dL/dK, dL/dV.  With the weights p_ij =
 * exp(scale q_i . k_j - LSE_i) of the allowed keys:
 *   dV_j = sum_i p_ij dO_i;   ds_ij = p_ij (dO_i . V_j - dO_i . O_i);
 *   dQ_i = scale sum_j ds_ij K_j;   dK_j = scale sum_i ds_ij Q_i.
 *
 *   Q, K, V, O, dO  bf16 device tensors, read: the forward's inputs, its
 *                   output O and the incoming gradient, all [B, h, n, 64]
 *   LSE             fp32 [B, h, n_q] from attn_forward_lse of the same call
 *   layout, mask_kind, q_lens, kv_lens, scale
 *                   exactly as given to the forward (dtype must be ATTN_BF16)
 *   dQ              [B, h, n_q, 64] bf16, written (padded rows as 0)
 *   dK, dV          [B, h, n_k, 64] bf16, written (excluded keys as 0)
 *   workspace       device buffer of at least attn_backward_workspace_bytes
 *                   (per query row, padded to a multiple of 64 rows: fp32
 *                   dO . O, then fp32 LSE log2(e), then 8 bf16 holding
 *                   -LSE / |scale| and -dO . O, each as a sum of three bf16
 *                   parts); contents on entry do not matter; calls that share
 *                   it must be ordered (same stream)
 *   stream          hipStream_t or NULL.
 * Three kernels on `stream` (row dots, key-major dK/dV, query-major dQ); no
 * atomics, so the results are bitwise reproducible.  bf16 products, fp32
 * accumulation; p and ds are rounded to bf16 once before their products.
 * Outputs must not alias inputs or each other.
 */
attn_status attn_backward(const void* Q, const void* K, const void* V, const void* O,
                          const void* dO, const float* LSE, attn_layout layout,
                          int32_t mask_kind, const int32_t* q_lens, const int32_t* kv_lens,
                          float scale, void* dQ, void* dK, void* dV, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * attn_backward_restricted -- attn_backward of attn_forward_restricted:
 * the same gradients over the band of restricted self-attention (kimjiil
 * page §4, Table 1), keys i - radius .. i + radius (i - radius .. i with
 * ATTN_MASK_CAUSAL).  mask_kind must hold ATTN_MASK_RESTRICTED, radius >= 0
 * and n_q == n_k; LSE comes from attn_forward_restricted with the same
 * radius.  Every other argument and the error behaviour are those of
 * attn_backward, which refuses ATTN_MASK_RESTRICTED.
 */
attn_status attn_backward_restricted(const void* Q, const void* K, const void* V,
                                     const void* O, const void* dO, const float* LSE,
                                     attn_layout layout, int32_t mask_kind,
                                     const int32_t* q_lens, const int32_t* kv_lens,
                                     int32_t radius, float scale, void* dQ, void* dK,
                                     void* dV, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Bytes of workspace attn_backward and attn_backward_restricted need: 24
 * bytes per query row (two fp32 values and 16 bytes of bf16 parts), rows of
 * each (b, h) rounded up to a multiple of 64; 0 if the layout is invalid.
 * Pure host arithmetic. */
size_t attn_backward_workspace_bytes(attn_layout layout);

/* Bytes of fp32 split partials attn_decode needs for this cache layout; 0 if
 * the layout is invalid.  Pure host arithmetic. */
size_t attn_decode_workspace_bytes(attn_layout cache_layout);

/* Scratch that attn_decode_noalloc holds per GPU: 8 MiB. */
#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)8 << 20)

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same computation and kernels, with the split
 * partials kept in a static device array of ATTN_DECODE_NOALLOC_MAX_BYTES
 * that each GPU the library runs on holds until the process ends.  The call
 * allocates and frees nothing; the caller still owns q, the caches, kv_lens
 * and O.
 *
 *   q, Kcache, Vcache, cache_layout, kv_lens, scale, O, stream
 *           exactly as for attn_decode.
 * Errors: those of attn_decode (never ATTN_ERR_WORKSPACE), plus
 * ATTN_ERR_SCRATCH_LIMIT when attn_decode_workspace_bytes(cache_layout)
 * exceeds ATTN_DECODE_NOALLOC_MAX_BYTES (e.g. B 64, h 16 fits up to
 * n_max = 7936; B 1, h 16 up to 508,160).  Every call on one GPU shares that
 * GPU's array, whose contents carry no meaning between calls (each call
 * writes every record it reads): calls that may overlap on one GPU -- on
 * different streams, or from different threads without ordering -- race and
 * must be serialised by the caller.  The first call on a device looks up the
 * array's device address once (thread-safe).
 */
attn_status attn_decode_noalloc(const void* q, const void* Kcache, const void* Vcache,
                                attn_layout cache_layout, const int32_t* kv_lens, float scale,
                                void* O, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_string(attn_status status);

/* Name of the HIP error behind the last ATTN_ERR_HIP returned on the calling
 * thread ("hipSuccess" if none).  Static string, never NULL. */
const char* attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HEADATTN_H */
