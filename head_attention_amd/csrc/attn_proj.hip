// Multi-head projections at the two ends of the attention sub-layer
// ("[논문 리뷰]Attention Is All You Need", §3.2.2: head_i = Attention(Q W_i^Q,
// K W_i^K, V W_i^V); MultiHead = Concat(head_1..head_h) W^O).
//
//   attn_head_projection:   Out_j[b, i, t, :] = X[b, t, :] W_j,i^T, written
//                           straight into the [B, h, n, 64] layout the
//                           attention kernels read (no split copy);
//   attn_output_projection: Y[b, t, :] = Concat_i(O[b, i, t, :]) Wo^T, reading
//                           the [B, h, n, 64] attention output in place (no
//                           concatenation copy).
//
// Both are one GEMM kernel, C^T = W A^T with W [N, K] (one row per output
// feature, k contiguous) and A [M, K] (one row per token): on
// v_mfma_f32_32x32x16_bf16 the A operand is a W fragment and the B operand
// an A fragment, both 16 contiguous bytes of a k-contiguous row, and each
// lane ends up holding four consecutive output features of one token -- one
// 8-byte store, along a head's 64 dimensions or along Y's row.
//
// Workgroup: 4 waves, a 128 (features) x 128 (tokens) tile, each wave 64 x
// 64 (2 x 2 blocks of 32 x 32).  K runs in steps of 64: W and A tiles of
// 128 x 64 bf16 reach LDS by buffer loads that write LDS directly, double
// buffered, one barrier per step; rows past the end of W or A read as zero
// through the descriptor's range check.  For the output projection a K step
// of 64 is exactly one head, so the A tile of a step is 128 rows of one
// head's [n, 64] slab: a per-row offset, no gather of single elements.
#include "common.h"

namespace headattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;
constexpr int kBN = 128;  // output features per workgroup
constexpr int kBM = 128;  // tokens per workgroup
constexpr int kBK = 64;   // k per step (= one head for the output projection)
constexpr uint32_t kRowBytes = kBK * 2;
constexpr int kTileChunks = 128 * 8;  // 16-byte chunks of a 128 x 64 tile
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit elements (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u;   // an offset the range check always rejects

__shared__ uint4 s_w[2][kTileChunks];
__shared__ uint4 s_a[2][kTileChunks];

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <bool HEAD_OUT>
__global__ __launch_bounds__(kThreads, 2) void proj_gemm_kernel(ProjArgs a) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hh = lane >> 5;
  const int wn = wave & 1;   // feature half of the tile
  const int wm = wave >> 1;  // token half of the tile

  const int n_blocks = (a.N + kBN - 1) / kBN;
  const int nb = blockIdx.x % n_blocks;
  const int mb = blockIdx.x / n_blocks;
  const int n0 = nb * kBN;
  const int m0 = mb * kBM;
  const int K = a.K;
  const int nk = K / kBK;

  // ---- fills: one instruction of the workgroup covers 32 rows of a tile;
  // lane l of wave w writes chunk 64 w + l of that quarter (row 8 w + l / 8,
  // position l % 8), which receives the row's chunk (l % 8) ^ (row % 8).
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.W), (short)0, (int)a.w_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.A), (short)0, (int)a.a_bytes, kBufferWord3);
  const int fpos = lane & 7;
  uint32_t w_off[4], a_off[4], a_step;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 32 * q + 8 * wave + (lane >> 3);
    const uint32_t chunk = 16u * (uint32_t)(fpos ^ (row & 7));
    const int n = n0 + row;
    w_off[q] = n < a.N ? (uint32_t)n * (uint32_t)K * 2u + chunk : kOutOfRange;
    const int m = m0 + row;
    if (HEAD_OUT) {
      // A = X [M, K] row-major
      a_off[q] = m < a.M ? (uint32_t)m * (uint32_t)K * 2u + chunk : kOutOfRange;
    } else {
      // A = Concat(heads of O): row m = (b, t), step s = head s of O[b, s, t, :]
      const int b = m / a.n_seq;
      const int t = m - b * a.n_seq;
      a_off[q] = m < a.M ? ((uint32_t)b * (uint32_t)a.H * (uint32_t)a.n_seq + (uint32_t)t) * kRowBytes + chunk
                         : kOutOfRange;
    }
  }
  // Byte advance of one K step along the A rows.
  a_step = HEAD_OUT ? kRowBytes : (uint32_t)a.n_seq * kRowBytes;
  auto fill = [&](int slot, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wo = w_off[q] == kOutOfRange ? kOutOfRange : w_off[q] + (uint32_t)kt * kRowBytes;
      const uint32_t ao = a_off[q] == kOutOfRange ? kOutOfRange : a_off[q] + (uint32_t)kt * a_step;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(&s_w[slot][256 * q + 64 * wave]), 16, wo, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(&s_a[slot][256 * q + 64 * wave]), 16, ao, 0, 0, 0);
    }
  };

  f32x16 acc[2][2];  // [feature block][token block]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  fill(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int slot = kt & 1;
    if (kt + 1 < nk) fill(slot ^ 1, kt + 1);
    // Fragments of k step s: lane (ln, hh) reads row 64 w + 32 blk + ln,
    // chunk 2 s + hh (d / k 16 s + 8 hh .. + 7).
    const uint4* wt = s_w[slot];
    const uint4* at = s_a[slot];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + hh;
      bf16x8 wf[2], af[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int rw_ = 64 * wn + 32 * blk + ln;
        const int ra_ = 64 * wm + 32 * blk + ln;
        wf[blk] = __builtin_bit_cast(bf16x8, wt[rw_ * 8 + (ch ^ (rw_ & 7))]);
        af[blk] = __builtin_bit_cast(bf16x8, at[ra_ * 8 + (ch ^ (ra_ & 7))]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();  // the next step's tile has landed; this step's slot is free
  }

  // ---- epilogue.  Register r of block (i, j) holds feature n0 + 64 wn +
  // 32 i + 8 (r / 4) + 4 hh + r % 4 of token m0 + 64 wm + 32 j + ln: four
  // consecutive features per 8-byte store.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + 64 * wm + 32 * j + ln;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + 64 * wn + 32 * i + 8 * g + 4 * hh;
        if (n >= a.N) continue;
        uint2 v;
        v.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
        v.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        if (HEAD_OUT) {
          // feature n = (projection p, head hd, dim c); token m = (b, t)
          const int d_model = a.H * kHeadDim;
          const int p = n / d_model;
          const int hd = (n - p * d_model) / kHeadDim;
          const int c = n % kHeadDim;
          const int b = m / a.n_seq;
          const int t = m - b * a.n_seq;
          __bf16* out = static_cast<__bf16*>(a.out[p]);
          *reinterpret_cast<uint2*>(out + (((size_t)b * a.H + hd) * a.n_seq + t) * kHeadDim + c) = v;
        } else {
          __bf16* y = static_cast<__bf16*>(a.out[0]);
          *reinterpret_cast<uint2*>(y + (size_t)m * a.N + n) = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_proj(const ProjArgs& a, bool head_out, hipStream_t s) {
  const long long blocks = (long long)((a.N + kBN - 1) / kBN) * ((a.M + kBM - 1) / kBM);
  ProjArgs args = a;
  void* kargs[] = {&args};
  const void* fn = head_out ? reinterpret_cast<const void*>(&proj_gemm_kernel<true>)
                            : reinterpret_cast<const void*>(&proj_gemm_kernel<false>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), kargs, 0, s);
}

}  // namespace headattn
