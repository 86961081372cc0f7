// Host entry points of libheadattn.so (the C ABI declared in
// include/headattn.h): argument validation, kernel selection and launch.
//
// Everything here is plain host code.  Validation happens before the first
// HIP call, so a bad argument is reported without touching a device; a valid
// call only enqueues work on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"
#include "headattn.h"

namespace {

using namespace headattn;

thread_local hipError_t g_last_hip = hipSuccess;

bool length_check_enabled() {
  static std::once_flag once;
  static bool enabled = false;
  std::call_once(once, [] {
    const char* v = std::getenv("ATTN_CHECK");
    enabled = v != nullptr && std::strcmp(v, "1") == 0;
  });
  return enabled;
}

constexpr int64_t kMaxGrid = 2147483647LL;

// Rows per (b, h) slice.  The bf16 kernels address a slice through buffer
// descriptors whose range and offsets are 32-bit byte counts of 128-byte
// rows, kept below 2^31: longer slices would wrap and read as zeros.
constexpr int32_t kMaxRows = (1 << 24) - 1;

// Shape checks common to every entry point.  Sizes must be non-negative and
// d must be 64; a (b, h) slice holds at most kMaxRows rows, and every element
// count must fit comfortably in int64.
attn_status check_layout(const attn_layout& L) {
  if (L.dtype != ATTN_BF16 && L.dtype != ATTN_F32) return ATTN_ERR_BAD_DTYPE;
  if (L.B < 0 || L.h < 0 || L.n_q < 0 || L.n_k < 0) return ATTN_ERR_BAD_SHAPE;
  if (L.d != kHeadDim) return ATTN_ERR_BAD_SHAPE;
  if (L.n_q > kMaxRows || L.n_k > kMaxRows) return ATTN_ERR_BAD_SHAPE;
  const long double elems_q = (long double)L.B * L.h * L.n_q * L.d;
  const long double elems_k = (long double)L.B * L.h * L.n_k * L.d;
  if (elems_q > 4.0e18L || elems_k > 4.0e18L) return ATTN_ERR_BAD_SHAPE;
  return ATTN_OK;
}

hipError_t read_lengths(const int32_t* dev, int n, hipStream_t s, std::vector<int32_t>& out) {
  out.resize(n);
  hipError_t e = hipMemcpyAsync(out.data(), dev, sizeof(int32_t) * n, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e;
}

attn_status check_lengths(const int32_t* dev, int B, int n, hipStream_t s) {
  if (!dev) return ATTN_OK;
  std::vector<int32_t> h;
  const hipError_t e = read_lengths(dev, B, s, h);
  if (e != hipSuccess) {
    g_last_hip = e;
    return ATTN_ERR_HIP;
  }
  for (int32_t v : h)
    if (v < 0 || v > n) return ATTN_ERR_BAD_LENGTHS;
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK: success";
    case ATTN_ERR_NULL_POINTER: return "ATTN_ERR_NULL_POINTER: a required pointer is NULL";
    case ATTN_ERR_BAD_SHAPE:
      return "ATTN_ERR_BAD_SHAPE: negative size, d != 64, more than 2^24 - 1 rows per (b, h), or size "
             "overflow";
    case ATTN_ERR_BAD_DTYPE: return "ATTN_ERR_BAD_DTYPE: dtype must be ATTN_BF16 or ATTN_F32";
    case ATTN_ERR_BAD_MASK:
      return "ATTN_ERR_BAD_MASK: unknown mask bits, causal or restricted with n_q != n_k, a "
             "negative radius or ATTN_MASK_RESTRICTED outside attn_forward_restricted, or kv_lens "
             "given/missing against ATTN_MASK_KEY_PADDING";
    case ATTN_ERR_BAD_LENGTHS: return "ATTN_ERR_BAD_LENGTHS: a length is outside [0, n]";
    case ATTN_ERR_BAD_SCALE: return "ATTN_ERR_BAD_SCALE: scale must be finite";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: decode workspace missing or too small";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: a HIP runtime call failed";
    case ATTN_ERR_SCRATCH_LIMIT:
      return "ATTN_ERR_SCRATCH_LIMIT: attn_decode_noalloc needs more than ATTN_DECODE_NOALLOC_MAX_BYTES "
             "of scratch for this layout (use attn_decode with a workspace)";
  }
  return "unknown attn_status";
}

const char* attn_last_hip_error(void) { return hipGetErrorName(g_last_hip); }

namespace {

// radius < 0: no restriction (mask_kind must not hold ATTN_MASK_RESTRICTED);
// radius >= 0: restricted self-attention (mask_kind must hold it).
attn_status forward_impl(const void* Q, const void* K, const void* V, attn_layout layout,
                         int32_t mask_kind, const int32_t* q_lens, const int32_t* kv_lens,
                         float scale, void* O, float* lse, int32_t radius, void* stream) {
  attn_status st = check_layout(layout);
  if (st != ATTN_OK) return st;
  if (mask_kind & ~(ATTN_MASK_KEY_PADDING | ATTN_MASK_CAUSAL | ATTN_MASK_RESTRICTED)) return ATTN_ERR_BAD_MASK;
  const bool kpad = (mask_kind & ATTN_MASK_KEY_PADDING) != 0;
  const bool causal = (mask_kind & ATTN_MASK_CAUSAL) != 0;
  const bool restricted = (mask_kind & ATTN_MASK_RESTRICTED) != 0;
  if (restricted != (radius >= 0)) return ATTN_ERR_BAD_MASK;
  if ((causal || restricted) && layout.n_q != layout.n_k) return ATTN_ERR_BAD_MASK;
  if (!kpad && kv_lens != nullptr) return ATTN_ERR_BAD_MASK;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  const bool empty_out = layout.B == 0 || layout.h == 0 || layout.n_q == 0;
  if (empty_out) return ATTN_OK;  // nothing to write
  if (!Q || !O) return ATTN_ERR_NULL_POINTER;
  if (layout.n_k > 0 && (!K || !V)) return ATTN_ERR_NULL_POINTER;
  if (kpad && !kv_lens) return ATTN_ERR_NULL_POINTER;
  if (Q == O || K == O || V == O) return ATTN_ERR_BAD_SHAPE;  // inputs must not alias O
  if (lse && (lse == O || lse == Q || lse == K || lse == V)) return ATTN_ERR_BAD_SHAPE;

  const int bm = layout.dtype == ATTN_BF16 ? 128 : 64;  // query rows per workgroup
  const int64_t blocks = (int64_t)((layout.n_q + bm - 1) / bm) * layout.h * layout.B;
  if (blocks > kMaxGrid) return ATTN_ERR_BAD_SHAPE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (length_check_enabled()) {
    if ((st = check_lengths(q_lens, layout.B, layout.n_q, s)) != ATTN_OK) return st;
    if ((st = check_lengths(kv_lens, layout.B, layout.n_k, s)) != ATTN_OK) return st;
  }

  FwdArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.q_lens = q_lens;
  a.kv_lens = kv_lens;
  a.B = layout.B;
  a.H = layout.h;
  a.n_q = layout.n_q;
  a.n_k = layout.n_k;
  a.scale = scale;
  a.causal = causal;
  a.lse = lse;
  // A radius of n_k or more already spans every key.
  a.radius = restricted ? std::min(radius, layout.n_k) : -1;
  hipError_t e;
  if (layout.dtype == ATTN_F32) e = launch_fwd_f32(a, s);
  else if (layout.n_k <= kShortMaxKeys) e = launch_fwd_bf16_short(a, s);
  else if (restricted) e = launch_fwd_bf16_band(a, s);
  else if (layout.n_q >= kPairMinRows) e = launch_fwd_bf16_pair(a, s);
  else e = launch_fwd_bf16(a, s);
  if (e != hipSuccess) {
    g_last_hip = e;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace

attn_status attn_forward(const void* Q, const void* K, const void* V, attn_layout layout,
                         int32_t mask_kind, const int32_t* q_lens, const int32_t* kv_lens,
                         float scale, void* O, void* stream) {
  return forward_impl(Q, K, V, layout, mask_kind, q_lens, kv_lens, scale, O, nullptr, -1, stream);
}

attn_status attn_forward_lse(const void* Q, const void* K, const void* V, attn_layout layout,
                             int32_t mask_kind, const int32_t* q_lens, const int32_t* kv_lens,
                             float scale, void* O, float* LSE, void* stream) {
  if (!LSE && layout.B > 0 && layout.h > 0 && layout.n_q > 0 && check_layout(layout) == ATTN_OK)
    return ATTN_ERR_NULL_POINTER;
  return forward_impl(Q, K, V, layout, mask_kind, q_lens, kv_lens, scale, O, LSE, -1, stream);
}

attn_status attn_forward_restricted(const void* Q, const void* K, const void* V, attn_layout layout,
                                    int32_t mask_kind, const int32_t* q_lens, const int32_t* kv_lens,
                                    int32_t radius, float scale, void* O, float* LSE, void* stream) {
  if (radius < 0) return ATTN_ERR_BAD_MASK;
  return forward_impl(Q, K, V, layout, mask_kind, q_lens, kv_lens, scale, O, LSE, radius, stream);
}

attn_status attn_cache_append(const void* Knew, const void* Vnew, void* Kcache, void* Vcache,
                              attn_layout L, const int32_t* kv_lens, void* stream) {
  attn_status st = check_layout(L);
  if (st != ATTN_OK) return st;
  if (L.B == 0 || L.h == 0 || L.n_q == 0) return ATTN_OK;  // nothing to append
  if (!Knew || !Vnew || !Kcache || !Vcache || !kv_lens) return ATTN_ERR_NULL_POINTER;
  if (Knew == Kcache || Knew == Vcache || Vnew == Kcache || Vnew == Vcache || Kcache == Vcache)
    return ATTN_ERR_BAD_SHAPE;
  const int row_bytes = kHeadDim * (L.dtype == ATTN_BF16 ? 2 : 4);
  const int64_t chunks = (int64_t)L.B * L.h * L.n_q * (row_bytes / 16);
  if ((chunks + 255) / 256 > kMaxGrid) return ATTN_ERR_BAD_SHAPE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (length_check_enabled()) {
    std::vector<int32_t> h;
    const hipError_t e = read_lengths(kv_lens, L.B, s, h);
    if (e != hipSuccess) {
      g_last_hip = e;
      return ATTN_ERR_HIP;
    }
    for (int32_t v : h)
      if (v < L.n_q || v > L.n_k) return ATTN_ERR_BAD_LENGTHS;
  }

  AppendArgs a;
  a.Kn = Knew;
  a.Vn = Vnew;
  a.Kc = Kcache;
  a.Vc = Vcache;
  a.kv_lens = kv_lens;
  a.B = L.B;
  a.H = L.h;
  a.n_new = L.n_q;
  a.n_max = L.n_k;
  a.row_bytes = row_bytes;
  const hipError_t e = launch_cache_append(a, s);
  if (e != hipSuccess) {
    g_last_hip = e;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status attn_head_projection(const void* X, const void* W, attn_layout L, int32_t n_out,
                                 void* out0, void* out1, void* out2, void* stream) {
  attn_status st = check_layout(L);
  if (st != ATTN_OK) return st;
  if (L.dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (n_out < 1 || n_out > 3) return ATTN_ERR_BAD_SHAPE;
  if (L.B == 0 || L.n_q == 0 || L.h == 0) return ATTN_OK;  // nothing to write
  void* outs[3] = {out0, out1, out2};
  if (!X || !W) return ATTN_ERR_NULL_POINTER;
  for (int j = 0; j < n_out; ++j) {
    if (!outs[j]) return ATTN_ERR_NULL_POINTER;
    if (outs[j] == X || outs[j] == W) return ATTN_ERR_BAD_SHAPE;
    for (int k = 0; k < j; ++k)
      if (outs[k] == outs[j]) return ATTN_ERR_BAD_SHAPE;
  }
  const int64_t d_model = (int64_t)L.h * kHeadDim;
  const int64_t M = (int64_t)L.B * L.n_q;
  const int64_t x_bytes = M * d_model * 2, w_bytes = (int64_t)n_out * d_model * d_model * 2;
  if (x_bytes >= (1LL << 31) || w_bytes >= (1LL << 31)) return ATTN_ERR_BAD_SHAPE;
  const int64_t blocks = ((n_out * d_model + 127) / 128) * ((M + 127) / 128);
  if (blocks > kMaxGrid) return ATTN_ERR_BAD_SHAPE;
  ProjArgs a;
  a.W = W;
  a.A = X;
  a.out[0] = out0;
  a.out[1] = n_out > 1 ? out1 : nullptr;
  a.out[2] = n_out > 2 ? out2 : nullptr;
  a.M = (int)M;
  a.N = (int)(n_out * d_model);
  a.K = (int)d_model;
  a.H = L.h;
  a.n_seq = L.n_q;
  a.w_bytes = (uint32_t)w_bytes;
  a.a_bytes = (uint32_t)x_bytes;
  a.xcd_fp = 0;
  const hipError_t e = launch_proj(a, true, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip = e;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

attn_status attn_output_projection(const void* O, const void* Wo, attn_layout L, void* Y, void* stream) {
  attn_status st = check_layout(L);
  if (st != ATTN_OK) return st;
  if (L.dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (L.B == 0 || L.n_q == 0 || L.h == 0) return ATTN_OK;
  if (!O || !Wo || !Y) return ATTN_ERR_NULL_POINTER;
  if (Y == O || Y == Wo) return ATTN_ERR_BAD_SHAPE;
  const int64_t d_model = (int64_t)L.h * kHeadDim;
  const int64_t M = (int64_t)L.B * L.n_q;
  const int64_t o_bytes = M * d_model * 2, w_bytes = d_model * d_model * 2;
  if (o_bytes >= (1LL << 31) || w_bytes >= (1LL << 31)) return ATTN_ERR_BAD_SHAPE;
  const int64_t blocks = ((d_model + 127) / 128) * ((M + 127) / 128);
  if (blocks > kMaxGrid) return ATTN_ERR_BAD_SHAPE;
  ProjArgs a;
  a.W = Wo;
  a.A = O;
  a.out[0] = Y;
  a.out[1] = a.out[2] = nullptr;
  a.M = (int)M;
  a.N = (int)d_model;
  a.K = (int)d_model;
  a.H = L.h;
  a.n_seq = L.n_q;
  a.w_bytes = (uint32_t)w_bytes;
  a.a_bytes = (uint32_t)o_bytes;
  a.xcd_fp = 0;
  const hipError_t e = launch_proj(a, false, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip = e;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

size_t attn_backward_workspace_bytes(attn_layout L) {
  if (check_layout(L) != ATTN_OK) return 0;
  // Per query row, rows rounded up to a multiple of 64: two fp32 values
  // and 16 bytes of bf16 parts.
  const size_t n_pad = ((size_t)L.n_q + 63) / 64 * 64;
  return (size_t)L.B * L.h * n_pad * (2 * sizeof(float) + 16);
}

namespace {

// radius < 0: no restriction (mask_kind must not hold ATTN_MASK_RESTRICTED);
// radius >= 0: restricted self-attention (mask_kind must hold it).
attn_status backward_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                          const float* LSE, attn_layout L, int32_t mask_kind, const int32_t* q_lens,
                          const int32_t* kv_lens, int32_t radius, float scale, void* dQ, void* dK,
                          void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  attn_status st = check_layout(L);
  if (st != ATTN_OK) return st;
  if (L.dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (mask_kind & ~(ATTN_MASK_KEY_PADDING | ATTN_MASK_CAUSAL | ATTN_MASK_RESTRICTED)) return ATTN_ERR_BAD_MASK;
  const bool kpad = (mask_kind & ATTN_MASK_KEY_PADDING) != 0;
  const bool causal = (mask_kind & ATTN_MASK_CAUSAL) != 0;
  const bool restricted = (mask_kind & ATTN_MASK_RESTRICTED) != 0;
  if (restricted != (radius >= 0)) return ATTN_ERR_BAD_MASK;
  if ((causal || restricted) && L.n_q != L.n_k) return ATTN_ERR_BAD_MASK;
  if (!kpad && kv_lens != nullptr) return ATTN_ERR_BAD_MASK;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  if (L.B == 0 || L.h == 0 || (L.n_q == 0 && L.n_k == 0)) return ATTN_OK;
  if (kpad && !kv_lens) return ATTN_ERR_NULL_POINTER;
  if (L.n_q > 0 && (!Q || !O || !dO || !LSE || !dQ)) return ATTN_ERR_NULL_POINTER;
  if (L.n_k > 0 && (!K || !V || !dK || !dV)) return ATTN_ERR_NULL_POINTER;
  const void* ins[6] = {Q, K, V, O, dO, LSE};
  const void* outs[3] = {dQ, dK, dV};
  for (const void* o : outs) {
    if (!o) continue;
    for (const void* in : ins)
      if (in == o) return ATTN_ERR_BAD_SHAPE;
  }
  if ((dQ && (dQ == dK || dQ == dV)) || (dK && dK == dV)) return ATTN_ERR_BAD_SHAPE;
  const size_t need = attn_backward_workspace_bytes(L);
  if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  // The kernels address the workspace with 32-bit byte offsets.
  if (need >= ((size_t)1 << 31)) return ATTN_ERR_BAD_SHAPE;
  const int64_t blocks = (int64_t)((std::max(L.n_q, L.n_k) + 127) / 128) * L.h * L.B;
  const int64_t n_pad = ((int64_t)L.n_q + 63) / 64 * 64;
  if (blocks > kMaxGrid || ((int64_t)L.B * L.h * n_pad + 31) / 32 > kMaxGrid) return ATTN_ERR_BAD_SHAPE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (length_check_enabled()) {
    if ((st = check_lengths(q_lens, L.B, L.n_q, s)) != ATTN_OK) return st;
    if ((st = check_lengths(kv_lens, L.B, L.n_k, s)) != ATTN_OK) return st;
  }
  BwdArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.dO = dO;
  a.lse = LSE;
  a.D = static_cast<float*>(workspace);
  a.L = a.D + (size_t)L.B * L.h * n_pad;
  a.LD16 = reinterpret_cast<uint4*>(a.L + (size_t)L.B * L.h * n_pad);  // 16-byte aligned: n_pad % 64 == 0
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.q_lens = q_lens;
  a.kv_lens = kv_lens;
  a.B = L.B;
  a.H = L.h;
  a.n_q = L.n_q;
  a.n_k = L.n_k;
  a.n_pad = (int)n_pad;
  a.scale = scale;
  a.causal = causal;
  a.radius = restricted ? std::min(radius, L.n_k) : -1;
  const hipError_t e = launch_backward(a, s);
  if (e != hipSuccess) {
    g_last_hip = e;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace

attn_status attn_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                          const float* LSE, attn_layout L, int32_t mask_kind, const int32_t* q_lens,
                          const int32_t* kv_lens, float scale, void* dQ, void* dK, void* dV,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(Q, K, V, O, dO, LSE, L, mask_kind, q_lens, kv_lens, -1, scale, dQ, dK, dV, workspace,
                       workspace_bytes, stream);
}

attn_status attn_backward_restricted(const void* Q, const void* K, const void* V, const void* O,
                                     const void* dO, const float* LSE, attn_layout L, int32_t mask_kind,
                                     const int32_t* q_lens, const int32_t* kv_lens, int32_t radius,
                                     float scale, void* dQ, void* dK, void* dV, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (radius < 0) return ATTN_ERR_BAD_MASK;
  return backward_impl(Q, K, V, O, dO, LSE, L, mask_kind, q_lens, kv_lens, radius, scale, dQ, dK, dV,
                       workspace, workspace_bytes, stream);
}

size_t attn_decode_workspace_bytes(attn_layout L) {
  if (check_layout(L) != ATTN_OK || L.n_q != 1) return 0;
  return (size_t)L.B * L.h * decode_splits(L.n_k) * kPartialStride * sizeof(float);
}

namespace {

// Checks shared by attn_decode and attn_decode_noalloc, before any HIP call.
attn_status check_decode(const void* q, const void* Kcache, const void* Vcache, const attn_layout& L,
                         const int32_t* kv_lens, float scale, const void* O) {
  attn_status st = check_layout(L);
  if (st != ATTN_OK) return st;
  if (L.n_q != 1) return ATTN_ERR_BAD_SHAPE;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  if (L.B == 0 || L.h == 0) return ATTN_OK;
  if (!q || !O || !kv_lens) return ATTN_ERR_NULL_POINTER;
  if (L.n_k > 0 && (!Kcache || !Vcache)) return ATTN_ERR_NULL_POINTER;
  if (q == O || Kcache == O || Vcache == O) return ATTN_ERR_BAD_SHAPE;
  const int64_t splits = decode_splits(L.n_k);
  if ((int64_t)L.B * L.h * splits > kMaxGrid || (int64_t)L.B * L.h > kMaxGrid) return ATTN_ERR_BAD_SHAPE;
  return ATTN_OK;
}

attn_status launch_decode(const void* q, const void* Kcache, const void* Vcache, const attn_layout& L,
                          const int32_t* kv_lens, float scale, void* O, float* work, hipStream_t s) {
  attn_status st;
  if (length_check_enabled()) {
    if ((st = check_lengths(kv_lens, L.B, L.n_k, s)) != ATTN_OK) return st;
  }
  DecodeArgs a;
  a.q = q;
  a.Kc = Kcache;
  a.Vc = Vcache;
  a.O = O;
  a.kv_lens = kv_lens;
  a.work = work;
  a.B = L.B;
  a.H = L.h;
  a.n_max = L.n_k;
  a.n_split = decode_splits(L.n_k);
  a.scale = scale;
  const hipError_t e = L.dtype == ATTN_BF16 ? launch_decode_bf16(a, s) : launch_decode_f32(a, s);
  if (e != hipSuccess) {
    g_last_hip = e;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace

attn_status attn_decode(const void* q, const void* Kcache, const void* Vcache, attn_layout L,
                        const int32_t* kv_lens, float scale, void* O, void* workspace,
                        size_t workspace_bytes, void* stream) {
  attn_status st = check_decode(q, Kcache, Vcache, L, kv_lens, scale, O);
  if (st != ATTN_OK || L.B == 0 || L.h == 0) return st;
  const size_t need = attn_decode_workspace_bytes(L);
  if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  return launch_decode(q, Kcache, Vcache, L, kv_lens, scale, O, static_cast<float*>(workspace),
                       static_cast<hipStream_t>(stream));
}

attn_status attn_decode_noalloc(const void* q, const void* Kcache, const void* Vcache, attn_layout L,
                                const int32_t* kv_lens, float scale, void* O, void* stream) {
  attn_status st = check_decode(q, Kcache, Vcache, L, kv_lens, scale, O);
  if (st != ATTN_OK || L.B == 0 || L.h == 0) return st;
  if (attn_decode_workspace_bytes(L) > kNoAllocScratchBytes) return ATTN_ERR_SCRATCH_LIMIT;
  float* work = nullptr;
  const hipError_t e = decode_scratch(&work);
  if (e != hipSuccess) {
    g_last_hip = e;
    return ATTN_ERR_HIP;
  }
  return launch_decode(q, Kcache, Vcache, L, kv_lens, scale, O, work, static_cast<hipStream_t>(stream));
}

}  // extern "C"
