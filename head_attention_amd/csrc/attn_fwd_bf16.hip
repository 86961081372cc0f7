// bf16 forward of attn_forward on gfx950 matrix cores.
//
// Computes O = softmax(Q K^T * scale + M) V per (b, h) ("[논문 리뷰]Attention
// Is All You Need", §3.2.1 equation; masking by -inf logits before the
// softmax, §3.2.3), with key padding and the decoder's causal mask applied
// in registers, so no n x n score matrix ever leaves the register file.
//
// Workgroup: 4 waves (256 lanes) own 128 consecutive query rows of one (b, h);
// each wave owns 32 rows.  The key axis is walked in tiles of 64 keys.  K and
// V^T tiles are staged in LDS from 16-byte buffer loads whose range check
// returns zeros for rows at or beyond the valid length, so padded K/V memory
// (even NaN) is never read.
//
// Contractions (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   S^T[key, query] = K[key, :] . Qc[query, :]   A = K tile (LDS), B = Qc (regs)
//   O^T[d, query]  += V^T[d, key] . P^T[key, query]
//                                                A = V^T tile (LDS), B = P (regs)
// With S^T each lane holds one query row (lane % 32) and 16 of its keys per
// 32x32 block, so row reductions are in-lane plus one exchange between the
// two half-waves; P feeds the second product from registers, since the
// contraction order over keys is free and V^T is written to LDS with its keys
// in the order in which each lane's accumulator registers hold P.
//
// Q enters the product exactly (the sign of scale is folded in as a sign
// flip); a weight is exp2(score * c - pivot * c) with c = |scale| * log2(e):
// one FMA and one v_exp_f32 per score.  (Prescaling Q by c in bf16 would save
// the FMA but shifts every logit by about 2^-9/sqrt(3) of the logits' spread,
// which exceeds the error budget on peaky rows.)
//
// Softmax is the online form with a lazy pivot m per row (the subtracted
// constant of a stable softmax; softmax does not depend on it, so any choice
// is exact up to rounding).  m stays 0 -- no subtraction at all -- unless a
// tile's weights would sum past 2^64 or a row's first tile underflows; then
// that row's m moves to its tile max and O and the running sum l are rescaled
// by exp2(m_old - m_new).  Weights are rounded to bf16 once; l sums those
// same bf16 weights (v_dot2 with ones), so numerator and denominator use
// identical weights; O = acc / l is rounded to bf16.
//
// Pipeline per wave: while the weights of tile t are formed and multiplied
// with V (VALU + MFMA), the scores of tile t+1 are computed (MFMA) in the same
// straight-line block, so the matrix cores have independent work during the
// softmax.  Tiles that need a mask or a pivot take a general step with
// branches.  K runs one tile ahead of V in LDS; each is double buffered, and
// one barrier per tile separates reuse.
#include <type_traits>

#include "kernel_util.h"

namespace headattn {
namespace {

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr int kThreads = 64 * kWaves;

// One LDS tile: 64 rows x 128 B as 8 chunks of 16 B.  K tiles are stored
// [key][chunk] (positions k_swz of the shared header), V^T tiles [d][chunk
// of 8 keys].  Chunks are XOR-swizzled per row so the 16 lanes the LDS
// serves together, reading one logical chunk of 16 consecutive rows, spread
// over all banks (rows r and r + 8 are 1 KB apart, on the same banks, and
// take different positions).  (Measured faster than padding the rows to
// 144 B, although padding needs fewer address registers.)
struct Tile {
  uint4 c[64 * 8];
};

__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

// Position of key group g (keys 4g..4g+3 of a tile) inside a V^T row.  A lane
// of half-wave hh feeds the P.V product of 16-key step (blk, j) with the keys
// {16j + 4hh + t, 16j + 8 + 4hh + t : t = 0..3} (+ 32 blk) -- how its S^T
// accumulator registers 8j..8j+7 are laid out -- so those 8 keys form chunk
// 4 blk + 2 j + hh of the row: first half keys 16j+4hh.., second 16j+8+4hh..
__device__ __forceinline__ int vt_chunk_of_group(int g) { return 2 * (g >> 2) + (g & 1); }
__device__ __forceinline__ int vt_half_of_group(int g) { return (g >> 1) & 1; }

__device__ __forceinline__ uint4 as_uint4(u32x4 v) { return make_uint4(v[0], v[1], v[2], v[3]); }

// Weight of a raw score s under pivot term mc = m * c.
__device__ __forceinline__ float ex2(float s, float c, float mc) {
  return __builtin_amdgcn_exp2f(fmaf(s, c, -mc));
}

// Weights of one tile: P = exp2(S - pivot), packed to bf16 pairs in the order
// the P.V product consumes them, and the sum of the packed (rounded) weights.
__device__ __forceinline__ float exp_pack_sum(const f32x16& s0, const f32x16& s1, float c, float mc,
                                              uint32_t (&pk)[16]) {
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pk[i] = pack_bf16x2(ex2(s0[2 * i], c, mc), ex2(s0[2 * i + 1], c, mc));
    pk[8 + i] = pack_bf16x2(ex2(s1[2 * i], c, mc), ex2(s1[2 * i + 1], c, mc));
    acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]), ones, acc0, false);
    acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[8 + i]), ones, acc1, false);
  }
  return acc0 + acc1;
}

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(FwdArgs a) {
  __shared__ Tile kbuf[2];
  __shared__ Tile vbuf[2];

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

  // Lengths are per batch entry, hence uniform over the workgroup; saying so
  // keeps them (and the buffer descriptors built from them) in SGPRs.
  const int q_len = __builtin_amdgcn_readfirstlane(a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q);
  const int kv_lim = __builtin_amdgcn_readfirstlane(a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k);
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
  const int wave_tiles = (wave_end + kBN - 1) / kBN;  // this wave works on tiles [0, wave_tiles)

  // Range-checked views of this (b, h)'s K and V: rows >= kv_lim read as 0.
  const uint32_t n_bytes = (uint32_t)kv_lim * kRowBytes;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(K), (short)0, (int)n_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(V), (short)0, (int)n_bytes, kBufferWord3);

  // ---- Q fragment: B operand of S^T = K Q^T (k = d).  Lane (ln, hh) holds
  // Q[qi][16 s + 8 hh + 0..7] for d-step s, with the sign of scale folded in
  // (an exact sign flip), so the kernel only sees c = |scale| * log2(e).  c is
  // floored at 2^-100: for smaller |scale| every weight is exp2 of a number
  // below 2^-80 in magnitude, i.e. exactly 1.0f either way.
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-100f);
  const uint32_t sign = a.scale < 0.f ? 0x80008000u : 0u;
  bf16x8 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (qi < a.n_q) v = *reinterpret_cast<const uint4*>(Q + (size_t)qi * kHeadDim + 16 * s + 8 * hh);
    v.x ^= sign;
    v.y ^= sign;
    v.z ^= sign;
    v.w ^= sign;
    qf[s] = __builtin_bit_cast(bf16x8, v);
  }

  // ---- global -> register -> LDS staging.  Waves 2-3 carry K tiles (4 x
  // 16 B per lane, stored as is); waves 0-1 carry V tiles (4 rows x 16 B per
  // lane, transposed to 8 x 8 B on the way into LDS).
  uint4 pre[4];
  const bool k_loader = wave >= 2;  // wave-uniform (scalar) role
  const int lu = tid & 127;
  const int lc = lu & 7;   // 16-byte chunk = d 8 lc .. 8 lc + 7
  const int lg = lu >> 3;  // K: row base (rows lg + 16 t); V: key group (keys 4 lg + t)

  auto gload = [&](int tk, int tv, bool checked = true) {  // K tile tk, V tile tv
    if (k_loader) {
      if (!checked || tk < n_tiles) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t row = (uint32_t)(tk * kBN + lg + 16 * t);
          pre[t] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rk, row * kRowBytes + 16 * lc, 0, 0));
        }
      }
    } else if (!checked || tv < n_tiles) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t row = (uint32_t)(tv * kBN + 4 * lg + t);
        pre[t] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rv, row * kRowBytes + 16 * lc, 0, 0));
      }
    }
  };
  auto lstore = [&](int tk, int tv, bool checked = true) {
    if (k_loader) {
      if (!checked || tk < n_tiles) {
        Tile& st = kbuf[tk & 1];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = lg + 16 * t;
          st.c[r * 8 + (lc ^ k_swz(r))] = pre[t];
        }
      }
    } else if (!checked || tv < n_tiles) {
      uint2* vt2 = reinterpret_cast<uint2*>(vbuf[tv & 1].c);
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
        vt2[d * 16 + (ch ^ vt_swz(d)) * 2 + half] = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
      }
    }
  };

  // Operand fragments of one tile, read from LDS well ahead of the MFMAs that
  // consume them.  K: [s] = rows ln, [4 + s] = rows 32 + ln, d-step s.
  // V^T: [2 blk + j] = rows (d) ln, [4 + 2 blk + j] = rows 32 + ln, key step (blk, j).
  auto read_k = [&](int t, bf16x8 (&ka)[8]) {
    const Tile& st = kbuf[t & 1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + hh;
      ka[s] = __builtin_bit_cast(bf16x8, st.c[ln * 8 + (ch ^ k_swz(ln))]);
      ka[4 + s] = __builtin_bit_cast(bf16x8, st.c[(32 + ln) * 8 + (ch ^ k_swz(32 + ln))]);
    }
  };
  auto read_v = [&](int t, bf16x8 (&va)[8]) {
    const Tile& vt = vbuf[t & 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = 2 * i + hh;  // = 4 blk + 2 j + hh for i = 2 blk + j
      va[i] = __builtin_bit_cast(bf16x8, vt.c[ln * 8 + (ch ^ vt_swz(ln))]);
      va[4 + i] = __builtin_bit_cast(bf16x8, vt.c[(32 + ln) * 8 + (ch ^ vt_swz(32 + ln))]);
    }
  };

  // S^T of a tile: two 32-key blocks x four 16-wide d steps.
  auto qk = [&](const bf16x8 (&ka)[8], f32x16& s0, f32x16& s1) {
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[4 + s], qf[s], s1, 0, 0, 0);
    }
  };

  f32x16 o0 = {}, o1 = {};  // O^T blocks: d 0..31 and d 32..63, column = query ln
  float mc = 0.f;           // pivot term of the exponent, m * c
  float l = 0.f;            // this half-wave's partial row sum of bf16 weights

  // O^T += V^T P^T: per 32-key block, two 16-key steps.
  auto pv = [&](const bf16x8 (&va)[8], const uint32_t (&pk)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pk[4 * i], pk[4 * i + 1], pk[4 * i + 2], pk[4 * i + 3]));
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pb, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[4 + i], pb, o1, 0, 0, 0);
    }
  };

  // Move the pivot of the rows flagged `move` (by either half-wave) to their
  // tile max (in exponent units); other rows keep theirs.  Rescales O and l
  // and recomputes this tile's weights under the pivots now in force.
  auto move_pivot = [&](bool move, const f32x16& s0, const f32x16& s1, uint32_t (&pk)[16]) -> float {
    move = half_swap_or(move);  // both half-waves of a row must agree
    float tmax = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, fmaxf(s0[r], s1[r]));
    tmax = half_swap_max(tmax);
    const float tm = tmax * c;  // tile max in exponent units
    const float m_new = (move && tm > -INFINITY) ? tm : mc;
    // Exactly 1 where unmoved.  A downward move only happens on the first
    // tile (underflow check), where O and l are still 0: keep alpha = 1 there
    // rather than scaling zeros by a possibly infinite factor.
    const float alpha = m_new > mc ? __builtin_amdgcn_exp2f(mc - m_new) : 1.f;
    l *= alpha;
    o0 *= alpha;
    o1 *= alpha;
    mc = m_new;
    return exp_pack_sum(s0, s1, c, mc, pk);
  };

  // Weights of tile t from its scores (sc0, sc1): mask (only on tiles that
  // cross the causal diagonal or the key-length boundary), exp2, bf16 pack
  // and row sums.  Returns the tile's row-sum contribution.
  auto weights = [&](int t, f32x16& sc0, f32x16& sc1, uint32_t (&pk)[16]) -> float {
    const int k0 = t * kBN;
    // Register r of block blk holds key k0 + 32 blk + 8 (r / 4) + 4 hh + r % 4;
    // the lane's allowed keys are those below `lim`, so each register is
    // one compare of a constant offset against lim - k0 - 4 hh.
    if ((k0 + kBN > kv_lim) || (CAUSAL && k0 + kBN - 1 > qw0)) {
      const int lim = (CAUSAL ? min(kv_lim, qi + 1) : kv_lim) - k0 - 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        sc0[r] = off < lim ? sc0[r] : -INFINITY;
        sc1[r] = off + 32 < lim ? sc1[r] : -INFINITY;
      }
    }
    return exp_pack_sum(sc0, sc1, c, mc, pk);
  };
  // Pivot checks on a tile's weights: a tile sum past 2^64 (also catches
  // inf), or, on a row's first tile, a row sum so small that the row could be
  // lost to underflow.  NaN (garbage in padded rows) triggers neither.
  auto check = [&](float lt, bool first, f32x16& sc0, f32x16& sc1, uint32_t (&pk)[16]) -> float {
    bool move = lt > kPivotHigh;
    if (first) move = move || half_swap_sum(lt) < kPivotLow;
    if (__builtin_amdgcn_ballot_w64(move) != 0) lt = move_pivot(move, sc0, sc1, pk);
    return lt;
  };

  // One pipeline step t (0 <= t <= n_tiles).  The matrix cores compute the
  // scores of tile t+1 (into sn) and O += P(t-1) V(t-1) (from pp, checked in
  // the previous step) while the vector ALUs form the weights of tile t (from
  // sc, into pc); then K(t+2) and V(t) are staged and one barrier closes the
  // step.  GENERAL adds the range, activity and mask checks that the first
  // and last tiles and the tiles on the causal diagonal or the key-length
  // boundary need; the fast form is straight-line code apart from a rarely
  // taken pivot move.
  auto step = [&](auto general_tag, int t, f32x16& sc0, f32x16& sc1, f32x16& sn0, f32x16& sn1,
                  uint32_t (&pc)[16], uint32_t (&pp)[16]) {
    constexpr bool GENERAL = decltype(general_tag)::value;
    gload(t + 2, t, GENERAL);
    if (GENERAL) {
      if (t + 1 < wave_tiles) {
        bf16x8 ka[8];
        read_k(t + 1, ka);
        qk(ka, sn0, sn1);
      }
      if (t >= 1 && t - 1 < wave_tiles) {
        bf16x8 va[8];
        read_v(t - 1, va);
        pv(va, pp);
      }
      if (t < wave_tiles) l += check(weights(t, sc0, sc1, pc), t == 0, sc0, sc1, pc);
    } else {
      bf16x8 ka[8], va[8];
      read_k(t + 1, ka);
      read_v(t - 1, va);
      qk(ka, sn0, sn1);
      pv(va, pp);
      const float lt = weights(t, sc0, sc1, pc);
      l += check(lt, false, sc0, sc1, pc);
    }
    lstore(t + 2, t, GENERAL);
    __syncthreads();
  };
  using General = std::integral_constant<bool, true>;
  using Fast = std::integral_constant<bool, false>;

  // Tiles [0, t_free) need no mask for any wave of the workgroup; step t is
  // fast when 1 <= t and t + 1 < t_free (tiles t-1, t, t+1 all mask-free, so
  // every active wave works on all three).
  int t_free = n_tiles;
  if (CAUSAL) t_free = min(t_free, q0 / kBN);
  t_free = min(t_free, kv_lim / kBN);
  const int fast_end = t_free - 1;  // fast steps are t in [1, fast_end)

  f32x16 sa0 = {}, sa1 = {}, sb0 = {}, sb1 = {};
  uint32_t pa[16] = {}, pb[16] = {};
  int t = 0;
  if (n_tiles > 0) {
    gload(0, n_tiles);  // K(0)
    lstore(0, n_tiles);
    gload(1, n_tiles);  // K(1)
    __syncthreads();
    if (0 < wave_tiles) {
      bf16x8 ka[8];
      read_k(0, ka);
      qk(ka, sa0, sa1);
    }
    lstore(1, n_tiles);
    __syncthreads();
    step(General(), 0, sa0, sa1, sb0, sb1, pa, pb);
    t = 1;
  }
  // After step t-1: the scores of tile t sit in (sb0, sb1) and the weights of
  // tile t-1 in pa for odd t; (sa0, sa1) and pb for even t.
#pragma nounroll
  for (; t + 1 < fast_end; t += 2) {
    step(Fast(), t, sb0, sb1, sa0, sa1, pb, pa);
    step(Fast(), t + 1, sa0, sa1, sb0, sb1, pa, pb);
  }
  if (t < fast_end) {
    step(Fast(), t, sb0, sb1, sa0, sa1, pb, pa);
    ++t;
  }
  if (t & 1) {  // once: bring tile t's scores to (sa0, sa1) and tile t-1's weights to pb
    const f32x16 x0 = sa0, x1 = sa1;
    sa0 = sb0;
    sa1 = sb1;
    sb0 = x0;
    sb1 = x1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t x = pa[i];
      pa[i] = pb[i];
      pb[i] = x;
    }
  }
#pragma nounroll
  for (; t + 1 <= n_tiles; t += 2) {
    step(General(), t, sa0, sa1, sb0, sb1, pa, pb);
    step(General(), t + 1, sb0, sb1, sa0, sa1, pb, pa);
  }
  if (n_tiles > 0 && t == n_tiles) step(General(), t, sa0, sa1, sb0, sb1, pa, pb);

  // ---- epilogue: O[qi][d] = acc / l.  Register r of block ob holds
  // d = 32 ob + 8 (r / 4) + 4 hh + r % 4: four consecutive d per group.
  // Padded query rows and rows with no allowed key are written as exact
  // zeros (a select, so garbage in a padded Q row cannot leak through).
  const float l_row = half_swap_sum(l);
  const bool live = qi < q_len && l_row > 0.f;
  const float inv = live ? 1.f / l_row : 0.f;
  // Row log-sum-exp ln(sum_j exp(s_ij)) = (m c + log2 l) ln 2; -inf for a
  // padded row or a row with no allowed key (one lane per row writes).
  if (a.lse && hh == 0 && qi < a.n_q)
    a.lse[(size_t)bh * a.n_q + qi] = live ? (mc + __builtin_amdgcn_logf(l_row)) * kLn2 : -INFINITY;
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
