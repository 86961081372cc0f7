// fp32 check path of attn_forward: softmax(Q K^T * scale + M) V in fp32.
//
// Definition followed: "[논문 리뷰]Attention Is All You Need", §3.2.1 (the
// Attention(Q,K,V) equation) and §3.2.3 (illegal connections get -inf logits
// before the softmax); the masked form softmax(QK^T/sqrt(d_k) + M)V of
// "Attention Is All You Need를 지금 다시 읽는 법".
//
// This path exists to check the arithmetic in fp32 (no bf16 rounding of the
// operands or of the weights), not for speed: one wave per 64 query rows,
// one query row per lane, fp32 FMA dot products on the vector ALUs, K/V
// tiles of 64 keys staged in LDS, and a per-key online softmax (running max
// m, running sum l, rescaled accumulator) in registers.  The online form is
// an exact rewrite of the row softmax: softmax is invariant to the pivot, and
// a change of pivot from m to m' rescales every earlier term by exp(m - m').
#include "common.h"

namespace headattn {
namespace {

constexpr int kRows = 64;  // query rows per workgroup (one per lane)
constexpr int kKeys = 64;  // keys per LDS tile

__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(FwdArgs a) {
  const int n_qt = (a.n_q + kRows - 1) / kRows;
  int bid = blockIdx.x;
  const int qt = bid % n_qt;
  bid /= n_qt;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int lane = threadIdx.x;
  const int i = qt * kRows + lane;

  const size_t bh = (size_t)b * a.H + h;
  const float* Q = static_cast<const float*>(a.Q) + bh * (size_t)a.n_q * kHeadDim;
  const float* K = static_cast<const float*>(a.K) + bh * (size_t)a.n_k * kHeadDim;
  const float* V = static_cast<const float*>(a.V) + bh * (size_t)a.n_k * kHeadDim;
  float* O = static_cast<float*>(a.O) + bh * (size_t)a.n_q * kHeadDim;

  const int q_len = a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q;
  const int kv_lim = a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k;
  const bool row_ok = i < q_len;  // q_len <= n_q
  // Restricted self-attention: row i sees keys i - wl .. i + wr.
  const bool band = a.radius >= 0;
  const int wl = band ? a.radius : 0;
  const int wr = band ? (a.causal ? 0 : a.radius) : 0;
  // Keys any row of this tile may attend to: [start, end).
  int end = kv_lim;
  if (a.causal) end = min(end, qt * kRows + kRows);
  if (band) end = min(end, qt * kRows + kRows + wr);
  // Whole tile padded (all rows >= q_len): nothing to compute.
  if (qt * kRows >= q_len) end = 0;
  const int start = band ? max(0, qt * kRows - wl) : 0;

  __shared__ float4 Ks[kKeys * kHeadDim / 4];
  __shared__ float4 Vs[kKeys * kHeadDim / 4];

  float q[kHeadDim], acc[kHeadDim];
#pragma unroll
  for (int e = 0; e < kHeadDim; ++e) acc[e] = 0.f;
  if (row_ok) {
    const float4* q4 = reinterpret_cast<const float4*>(Q + (size_t)i * kHeadDim);
#pragma unroll
    for (int e = 0; e < kHeadDim / 4; ++e) {
      const float4 v = q4[e];
      q[4 * e] = v.x; q[4 * e + 1] = v.y; q[4 * e + 2] = v.z; q[4 * e + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kHeadDim; ++e) q[e] = 0.f;
  }

  const float c = a.scale * kLog2e;  // logits in the log2 domain
  float m = -INFINITY, l = 0.f;

  for (int k0 = start; k0 < end; k0 += kKeys) {
    __syncthreads();  // previous tile fully consumed
    // Coalesced tile load: 64 lanes x 16 B per step, 16 steps per tensor.
    // Rows at or beyond kv_lim are zero-filled and never read from memory.
#pragma unroll 4
    for (int it = 0; it < kKeys * kHeadDim / 4 / kRows; ++it) {
      const int idx = it * kRows + lane;
      const int row = idx / (kHeadDim / 4);
      const int col = idx % (kHeadDim / 4);
      const int key = k0 + row;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (key < kv_lim) {
        kv = reinterpret_cast<const float4*>(K + (size_t)key * kHeadDim)[col];
        vv = reinterpret_cast<const float4*>(V + (size_t)key * kHeadDim)[col];
      }
      Ks[idx] = kv;
      Vs[idx] = vv;
    }
    __syncthreads();

    const int n_here = min(kKeys, end - k0);
    for (int j = 0; j < n_here; ++j) {
      const int key = k0 + j;
      const bool ok = row_ok && key < kv_lim && (!a.causal || key <= i) &&
                      (!band || (key >= i - wl && key <= i + wr));
      if (!ok) continue;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < kHeadDim / 4; ++e) {
        const float4 kk = Ks[j * (kHeadDim / 4) + e];
        dot = fmaf(q[4 * e], kk.x, dot);
        dot = fmaf(q[4 * e + 1], kk.y, dot);
        dot = fmaf(q[4 * e + 2], kk.z, dot);
        dot = fmaf(q[4 * e + 3], kk.w, dot);
      }
      const float s = dot * c;
      if (s > m) {  // new pivot: rescale what was accumulated under the old one
        const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - s);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < kHeadDim; ++e) acc[e] *= alpha;
        m = s;
      }
      const float p = __builtin_amdgcn_exp2f(s - m);
      l += p;
#pragma unroll
      for (int e = 0; e < kHeadDim / 4; ++e) {
        const float4 vv = Vs[j * (kHeadDim / 4) + e];
        acc[4 * e] = fmaf(p, vv.x, acc[4 * e]);
        acc[4 * e + 1] = fmaf(p, vv.y, acc[4 * e + 1]);
        acc[4 * e + 2] = fmaf(p, vv.z, acc[4 * e + 2]);
        acc[4 * e + 3] = fmaf(p, vv.w, acc[4 * e + 3]);
      }
    }
  }

  if (i < a.n_q) {
    // A row with no allowed key, or a padded query row, is written as 0.
    const float inv = (row_ok && l > 0.f) ? 1.f / l : 0.f;
    // Row log-sum-exp (m + log2 l) ln 2 in fp32; -inf for padded or keyless rows.
    if (a.lse) a.lse[bh * (size_t)a.n_q + i] = (row_ok && l > 0.f) ? (m + log2f(l)) * kLn2 : -INFINITY;
    float4* o4 = reinterpret_cast<float4*>(O + (size_t)i * kHeadDim);
#pragma unroll
    for (int e = 0; e < kHeadDim / 4; ++e)
      o4[e] = make_float4(acc[4 * e] * inv, acc[4 * e + 1] * inv, acc[4 * e + 2] * inv,
                          acc[4 * e + 3] * inv);
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  const int n_qt = (a.n_q + kRows - 1) / kRows;
  const long long blocks = (long long)n_qt * a.H * a.B;
  FwdArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_f32_kernel),
                         dim3((unsigned)blocks), dim3(64), kargs, 0, s);
}

}  // namespace headattn
