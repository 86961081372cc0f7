// bf16 forward of attn_forward on gfx950 matrix cores.
//
// Computes O = softmax(Q K^T * scale + M) V per (b, h) ("[논문 리뷰]Attention
// Is All You Need", §3.2.1 equation; masking by -inf logits before the
// softmax, §3.2.3), with key padding and the decoder's causal mask applied
// in registers, so no n x n score matrix ever leaves the register file.
//
// Workgroup: 4 waves (256 lanes) own 128 consecutive query rows of one (b, h);
// each wave owns 32 rows.  The key axis is walked in tiles of 64 keys; K and
// V tiles are staged in LDS (double buffered, one barrier per tile) from
// coalesced 16-byte global loads.
//
// Contractions (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   S^T[key, query] = K[key, :] . Q[query, :]   A = K tile (LDS), B = Q (regs)
//   O^T[d, query]  += V^T[d, key] . P^T[key, query]
//                                               A = V^T (LDS), B = P (regs)
// With S^T, each lane holds one query row (lane % 32) and 16 of its keys per
// 32x32 block, so the row max and row sum are in-lane reductions plus one
// exchange between the two half-waves that hold the same row.  P then feeds
// the second product straight from registers: the contraction order over
// keys is free, so V^T is written to LDS with its keys in exactly the order
// in which each lane's accumulator registers hold P.
//
// Softmax is the online form: a running pivot m and running sum l per row in
// fp32 registers.  This is exact up to rounding because softmax does not
// depend on the pivot; the pivot is moved only when a tile's max exceeds it by
// more than 2^8 in weight (then the accumulator and l are rescaled by
// exp(m_old - m_new)), so every weight used is at most 2^8 and fits bf16
// and fp32 comfortably.  Weights are rounded to bf16 once for the product
// with V; l sums the unrounded fp32 weights; O = acc / l is rounded to bf16.
#include "common.h"

namespace headattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr int kThreads = 64 * kWaves;

// One LDS stage: K tile [64 keys][64 d] and V^T tile [64 d][64 key slots],
// bf16, each row 128 B = 8 chunks of 16 B.  Chunks are XOR-swizzled per row
// so that 8 lanes reading the same logical chunk of 8 consecutive rows hit 8
// different chunk positions.
struct Stage {
  uint4 k[kBN * 8];
  uint4 vt[kHeadDim * 8];
};

__device__ __forceinline__ int k_swz(int key) { return key & 7; }
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

// Position of key group g (keys 4g..4g+3 of a 64-key tile) inside a V^T row.
// A lane of half-wave hh feeds the P.V product of 16-key step (blk, j) with
// the 8 keys {16j + 4hh + t, 16j + 8 + 4hh + t : t = 0..3} (+ 32 blk), which is
// how its S^T accumulator registers 8j..8j+7 are laid out.  Those 8 keys form
// one 16-byte chunk: chunk 4 blk + 2 j + hh, first half keys 16j+4hh.., second
// half keys 16j+8+4hh..
__device__ __forceinline__ int vt_chunk_of_group(int g) { return 2 * (g >> 2) + (g & 1); }
__device__ __forceinline__ int vt_half_of_group(int g) { return (g >> 1) & 1; }

__device__ __forceinline__ float half_swap_max(float x) {
  // Combine the two half-waves (lanes l and l ^ 32 hold the same query row).
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(FwdArgs a) {
  __shared__ Stage lds[2];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;  // query row within the wave / M,N index of MFMA
  const int hh = lane >> 5;  // half-wave: selects the 8-wide k block

  // ---- which (b, h, query tile) this workgroup owns.  Workgroups are handed
  // to the 8 XCDs round robin (id % 8); when B*h divides by 8, every XCD gets
  // whole heads so a head's K/V stays in one XCD's L2.  Under the causal mask
  // tiles are issued longest first (highest query tile first).
  const int n_qt = (a.n_q + kBM - 1) / kBM;
  const int HB = a.H * a.B;
  const int bid = blockIdx.x;
  int bh, rank;
  if ((HB & 7) == 0) {
    const int per = HB >> 3;
    const int slot = bid >> 3;
    rank = slot / per;
    bh = (bid & 7) * per + slot % per;
  } else {
    bh = bid % HB;
    rank = bid / HB;
  }
  const int qt = CAUSAL ? (n_qt - 1 - rank) : rank;
  const int b = bh / a.H;

  const __bf16* Q = static_cast<const __bf16*>(a.Q) + (size_t)bh * a.n_q * kHeadDim;
  const __bf16* K = static_cast<const __bf16*>(a.K) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* V = static_cast<const __bf16*>(a.V) + (size_t)bh * a.n_k * kHeadDim;
  __bf16* O = static_cast<__bf16*>(a.O) + (size_t)bh * a.n_q * kHeadDim;

  const int q_len = a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q;
  const int kv_lim = a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k;
  const int q0 = qt * kBM;
  const int qw0 = q0 + 32 * wave;  // first query row of this wave
  const int qi = qw0 + ln;         // query row of this lane

  int end = kv_lim;  // keys the workgroup needs
  if (CAUSAL) end = min(end, q0 + kBM);
  if (q0 >= q_len) end = 0;  // the whole tile is padded query rows
  const int n_tiles = (end + kBN - 1) / kBN;
  int wave_end = end;  // keys this wave needs (wave-uniform)
  if (CAUSAL) wave_end = min(wave_end, qw0 + 32);
  if (qw0 >= q_len) wave_end = 0;

  // ---- Q fragment: B operand of S^T = K Q^T (k = d).  Lane (ln, hh) holds
  // Q[qi][16 s + 8 hh + 0..7] for d-step s.  A negative scale is folded into
  // Q exactly (sign flip), so the kernel only ever sees c = |scale| log2 e.
  bf16x8 qf[4];
  {
    const uint32_t sign = a.scale < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qi < a.n_q) v = *reinterpret_cast<const uint4*>(Q + (size_t)qi * kHeadDim + 16 * s + 8 * hh);
      v.x ^= sign; v.y ^= sign; v.z ^= sign; v.w ^= sign;
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // c > 0 always: for |scale| log2 e below 2^-100 every weight is exp2 of
  // something below 2^-80 in magnitude, i.e. exactly 1.0f either way, so the
  // floor changes nothing while keeping -inf * c = -inf for masked logits.
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-100f);
  const float thr = 8.0f / c;  // pivot moves when a tile max exceeds it by this

  // ---- global -> register -> LDS staging.  Waves 2-3 carry the K tile
  // (4 x 16 B per lane, stored as is); waves 0-1 carry the V tile (4 rows x
  // 16 B per lane, transposed to 8 x 8 B on the way into LDS).  Rows at or
  // beyond kv_lim are zero-filled and never read: padded or out-of-range K/V
  // (even NaN) cannot reach the products.
  uint4 pre[4];
  const bool k_loader = tid >= 2 * 64;
  const int lu = k_loader ? tid - 128 : tid;
  const int lc = lu & 7;   // 16-byte chunk = d 8 lc .. 8 lc + 7
  const int lg = lu >> 3;  // K: row base (rows lg + 16 k); V: key group (keys 4 lg + t)

  auto gload = [&](int k0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = k_loader ? k0 + lg + 16 * t : k0 + 4 * lg + t;
      const __bf16* src = k_loader ? K : V;
      pre[t] = key < kv_lim ? *reinterpret_cast<const uint4*>(src + (size_t)key * kHeadDim + 8 * lc)
                            : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](Stage& st) {
    if (k_loader) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = lg + 16 * t;
        st.k[r * 8 + (lc ^ k_swz(r))] = pre[t];
      }
    } else {
      uint2* vt2 = reinterpret_cast<uint2*>(st.vt);
      const int ch = vt_chunk_of_group(lg);
      const int half = vt_half_of_group(lg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * lc + e;
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t word = (&pre[t].x)[e >> 1];
          w[t] = (e & 1) ? (word >> 16) : (word & 0xffffu);
        }
        const uint2 val = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
        vt2[d * 16 + (ch ^ vt_swz(d)) * 2 + half] = val;
      }
    }
  };

  f32x16 o0 = {}, o1 = {};  // O^T blocks: d 0..31 and d 32..63, column = query ln
  float m_use = -INFINITY;  // pivot (raw score units), same in both half-waves
  float l = 0.f;            // this half-wave's partial row sum

  if (n_tiles > 0) {
    gload(0);
    lstore(lds[0]);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * kBN;
    if (t + 1 < n_tiles) gload(k0 + kBN);
    const Stage& st = lds[t & 1];

    if (k0 < wave_end) {
      // ---- S^T = K Q^T: two 32-key blocks x four 16-wide d steps
      f32x16 s0 = {}, s1 = {};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ch = 2 * s + hh;
        const bf16x8 ka = __builtin_bit_cast(bf16x8, st.k[ln * 8 + (ch ^ k_swz(ln))]);
        const bf16x8 kb = __builtin_bit_cast(bf16x8, st.k[(32 + ln) * 8 + (ch ^ k_swz(32 + ln))]);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qf[s], s1, 0, 0, 0);
      }

      // ---- mask in registers (only tiles that cross a boundary).  Register
      // r of block blk holds key k0 + 32 blk + 8 (r / 4) + 4 hh + r % 4.
      const bool need_mask = (k0 + kBN > kv_lim) || (CAUSAL && k0 + kBN - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool ok0 = key < kv_lim && (!CAUSAL || key <= qi);
          const bool ok1 = key + 32 < kv_lim && (!CAUSAL || key + 32 <= qi);
          s0[r] = ok0 ? s0[r] : -INFINITY;
          s1[r] = ok1 ? s1[r] : -INFINITY;
        }
      }

      // ---- online softmax
      float tmax = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, fmaxf(s0[r], s1[r]));
      tmax = half_swap_max(tmax);
      const bool move = tmax > m_use + thr;  // also true on the first allowed tile
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        // Lanes that do not need a move keep their pivot (alpha = 1 exactly),
        // so a row's arithmetic never depends on the other rows of its wave.
        const float m_new = move ? fmaxf(m_use, tmax) : m_use;
        const float alpha = (m_use == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_use - m_new) * c);
        l *= alpha;
        o0 *= alpha;
        o1 *= alpha;
        m_use = m_new;
      }
      const float mc = (m_use == -INFINITY) ? 0.f : m_use * c;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], c, -mc));
        s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], c, -mc));
        psum += s0[r] + s1[r];
      }
      l += psum;

      // ---- O^T += V^T P^T: per 32-key block, two 16-key steps
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const f32x16& p = blk ? s1 : s0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint4 pw;
          pw.x = pack_bf16x2(p[8 * j + 0], p[8 * j + 1]);
          pw.y = pack_bf16x2(p[8 * j + 2], p[8 * j + 3]);
          pw.z = pack_bf16x2(p[8 * j + 4], p[8 * j + 5]);
          pw.w = pack_bf16x2(p[8 * j + 6], p[8 * j + 7]);
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
          const int ch = 4 * blk + 2 * j + hh;
          const bf16x8 va = __builtin_bit_cast(bf16x8, st.vt[ln * 8 + (ch ^ vt_swz(ln))]);
          const bf16x8 vb = __builtin_bit_cast(bf16x8, st.vt[(32 + ln) * 8 + (ch ^ vt_swz(32 + ln))]);
          o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o0, 0, 0, 0);
          o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, pb, o1, 0, 0, 0);
        }
      }
    }

    if (t + 1 < n_tiles) lstore(lds[(t + 1) & 1]);
    __syncthreads();
  }

  // ---- epilogue: O[qi][d] = acc / l.  Register r of block ob holds
  // d = 32 ob + 8 (r / 4) + 4 hh + r % 4: four consecutive d per group.
  const float l_row = half_swap_sum(l);
  // Padded query rows and rows with no allowed key are written as exact
  // zeros (a select, so garbage in a padded Q row cannot leak through).
  const bool live = qi < q_len && l_row > 0.f;
  const float inv = live ? 1.f / l_row : 0.f;
  if (qi < a.n_q) {
    __bf16* orow = O + (size_t)qi * kHeadDim;
#pragma unroll
    for (int ob = 0; ob < 2; ++ob) {
      const f32x16& o = ob ? o1 : o0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = live ? pack_bf16x2(o[4 * g + 0] * inv, o[4 * g + 1] * inv) : 0u;
        w.y = live ? pack_bf16x2(o[4 * g + 2] * inv, o[4 * g + 3] * inv) : 0u;
        *reinterpret_cast<uint2*>(orow + 32 * ob + 8 * g + 4 * hh) = w;
      }
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  const int n_qt = (a.n_q + kBM - 1) / kBM;
  const long long blocks = (long long)n_qt * a.H * a.B;
  FwdArgs args = a;
  void* kargs[] = {&args};
  const void* fn = a.causal ? reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<true>)
                            : reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<false>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), kargs, 0, s);
}

}  // namespace headattn
