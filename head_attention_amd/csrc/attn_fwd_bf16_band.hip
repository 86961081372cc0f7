// bf16 forward of restricted self-attention for long sequences (n_k > 256):
// eight independent row groups per workgroup on gfx950.
//
// Computes O = softmax(Q K^T * scale + M) V per (b, h) ("[논문 리뷰]Attention
// Is All You Need", §3.2.1 equation; masking by -inf logits before the
// softmax, §3.2.3), where M keeps only the keys of a band around each query:
// restricted self-attention (§4, Table 1 and the note under it), keys
// i - radius .. i + radius, or i - radius .. i with the causal mask.  The
// arithmetic is the paired kernel's: exact bf16 Q (sign of scale folded
// in), S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, weights
// 2^(s c - m c) rounded to bf16 once, row sums of those same weights on the
// matrix cores, fp32 accumulation.  The pipeline runs under the fixed pivot
// m = 0 and range-checks every row at the end; a row group with a row that
// fails it is recomputed in the same launch, under the moving pivot, one
// tile at a time.
//
// Workgroup: 8 waves own 512 consecutive query rows of one (b, h); wave w
// owns row group w (64 rows) outright -- no key split, no merge.  Waves w
// and w + 4 share a SIMD and run one phase apart: while one issues the
// products of its tile, the other forms the weights of its own.  A row
// group's window of keys is 64 + 2 radius wide (9 tiles of 64 at radius
// 256) and starts one tile after the previous group's, so at phase p the
// wave of row group g works on tile g + p / 2 (relative to the workgroup's
// first tile, which may lie before key 0: those keys read as zero and are
// masked).  Together the eight waves read a window of 8 consecutive K
// tiles (and 8 V tiles, one tile behind) that slides by one tile every two
// phases: K and V stream through two 9-slot rings in LDS (144 KB), one new
// tile of each every second phase, each filled four phases before its
// first use and refilled only after its last.  Q comes in through the V
// ring too, before the first V tiles: its fills run beside those of the
// first K tiles instead of ahead of them, and the waves that start one
// phase later take theirs one phase later.
//
// Against the paired kernel on this workload (512-row workgroups instead of
// 256): half the workgroups, so one dispatch round where it took two; no
// pair merge through LDS; one prologue per 512 rows; no second launch for
// the moving-pivot fallback.  Each row group's rows leave through LDS
// once the workgroup has passed its last barrier, as whole 128-byte rows.
//
// Layouts as in the paired kernel: K rows (and the staged Q rows) keep
// their 16-byte chunks XOR-swizzled by row; V stays row-major (chunks
// swizzled by 2 (row % 4)) and is read transposed with ds_read_b64_tr_b16.
// Fills are 16-byte buffer loads straight into LDS, issued from inline
// assembly; rows at or beyond the valid length, or before key 0, read as
// zero through the descriptor's range check, so padded memory is never read.
#include "kernel_util.h"

namespace headattn {
namespace {

constexpr int kThreads = 512;
constexpr int kWaveRows = 64;
constexpr int kGroups = 8;                 // row groups per workgroup
constexpr int kBM = kGroups * kWaveRows;   // 512 query rows per workgroup
constexpr int kBN = 64;                    // keys per tile
constexpr uint32_t kTileBytes = kBN * kRowBytes;
constexpr int kRing = 9;                   // slots per ring

__shared__ uint4 g_kring[kRing][512];
__shared__ uint4 g_vring[kRing][512];
// A tile of zeros: the V operand of every wave's first P.V, which has no
// weights yet (its V slot may still hold staged Q, or nothing).
__shared__ uint4 g_zero[512];

__device__ __forceinline__ uint32_t kslot_addr(int s) {
  return (uint32_t)(uintptr_t)(lds_void_t*)&g_kring[0][0] + (uint32_t)s * kTileBytes;
}
__device__ __forceinline__ uint32_t vslot_addr(int s) {
  return (uint32_t)(uintptr_t)(lds_void_t*)&g_vring[0][0] + (uint32_t)s * kTileBytes;
}

// floor(x / 64) for any sign.
__device__ __forceinline__ int floor_tiles(int x) { return x >= 0 ? x / kBN : -((kBN - 1 - x) / kBN); }

// (b, h, query tile) of workgroup bid: the 8 XCDs take workgroup ids round
// robin; when B*h divides by 8 each XCD gets whole heads, so a head's K/V
// stays in one XCD's L2.
__device__ __forceinline__ void band_tile(const FwdArgs& a, int bid, int& bh, int& qt) {
  const int HB = a.H * a.B;
  if ((HB & 7) == 0) {
    const int per = HB >> 3;
    const int slot = bid >> 3;
    qt = slot / per;
    bh = (bid & 7) * per + slot % per;
  } else {
    bh = bid % HB;
    qt = bid / HB;
  }
}

__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_band_kernel(FwdArgs a) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hh = lane >> 5;
  const int g = wave;         // row group
  const int par = wave >> 2;  // 0: products at even phases, 1: at odd ones

  int bh, qt;
  band_tile(a, blockIdx.x, bh, qt);
  const int b = bh / a.H;

  const __bf16* Q = static_cast<const __bf16*>(a.Q) + (size_t)bh * a.n_q * kHeadDim;
  const __bf16* K = static_cast<const __bf16*>(a.K) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* V = static_cast<const __bf16*>(a.V) + (size_t)bh * a.n_k * kHeadDim;
  __bf16* O = static_cast<__bf16*>(a.O) + (size_t)bh * a.n_q * kHeadDim;

  const int q_len = __builtin_amdgcn_readfirstlane(a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q);
  const int kv_lim = __builtin_amdgcn_readfirstlane(a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k);
  const int q0 = qt * kBM;
  const int qw0 = q0 + kWaveRows * g;  // first query row of this wave

  // Row i sees keys max(0, i - wl) .. min(kv_lim - 1, i + wr).  Tile T
  // (relative) holds keys 64 (t0 + T) .. + 63; row group g's window starts
  // at tile g exactly (t0 = floor((q0 - wl) / 64), possibly negative).
  const int wl = a.radius;
  const int wr = a.causal ? 0 : a.radius;
  const int t0 = floor_tiles(q0 - wl);
  int end = min(kv_lim, q0 + kBM + wr);  // keys the workgroup may use
  if (q0 >= q_len) end = 0;
  // Tiles of row group gg's window: gg .. last(gg) - 1 (none for a group
  // past q_len).
  auto window_tiles = [&](int gg) __attribute__((always_inline)) {
    const int qg = q0 + kWaveRows * gg;
    const int eg = qg >= q_len ? 0 : min(end, qg + kWaveRows + wr);
    const int last = eg > 0 ? (eg + kBN - 1) / kBN - t0 : gg;
    return max(0, last - gg);
  };
  const int cnt = window_tiles(g);
  int n_run = 0;
#pragma unroll
  for (int gg = 0; gg < kGroups; ++gg) n_run = max(n_run, window_tiles(gg));

  // Descriptors over the head's K and V up to the last key the workgroup
  // may use (a tile past it reads zeros without touching memory, and so
  // does a tile before key 0, whose offset is set past any range), and over
  // its Q up to q_len (padded query rows enter as zeros: the row-sum
  // products multiply other rows' weights by 0, which must not meet NaN).
  const uint32_t n_bytes = (uint32_t)max(0, end) * kRowBytes;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(K), (short)0, (int)n_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(V), (short)0, (int)n_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(Q), (short)0, (int)((uint32_t)q_len * kRowBytes), kBufferWord3);

  // ---- tile fills: lane l of wave w writes LDS chunk 64 w + l of the slot,
  // i.e. row 8 w + l / 8, position l % 8, which holds the row's chunk
  // (l % 8) ^ swizzle(row).
  const int frow = 8 * wave + (lane >> 3);
  const int fpos = lane & 7;
  const uint32_t koff = (uint32_t)frow * kRowBytes + 16u * (uint32_t)(fpos ^ k_swz(frow));
  const uint32_t voff = (uint32_t)frow * kRowBytes + 16u * (uint32_t)(fpos ^ (2 * (frow & 3)));
  auto tile_off = [&](int T) __attribute__((always_inline)) {
    const int t = t0 + T;
    return t >= 0 ? (uint32_t)t * kTileBytes : kOutOfRange;
  };
  auto fill_k = [&](int T) __attribute__((always_inline)) {
    lds_fill16_at(rk, kslot_addr(T % kRing) + 1024u * wave, tile_off(T) + koff);
  };
  auto fill_v = [&](int T) __attribute__((always_inline)) {
    lds_fill16_at(rv, vslot_addr(T % kRing) + 1024u * wave, tile_off(T) + voff);
  };

  // ---- Q: the wave's 64 rows are staged in V slot `wave` (laid out like a
  // K tile) and read from there into the B operand of S^T = K Q^T: for
  // query block qb and d-step s, lane (ln, hh) holds Q[qw0 + 32 qb + ln]
  // [16 s + 8 hh + 0..7], with the sign of scale folded in.  c = |scale|
  // log2(e), floored at 2^-100 (below that every weight is exactly 1.0f
  // either way).
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-100f);
  const uint32_t sign = a.scale < 0.f ? 0x80008000u : 0u;
  const int qrow = lane >> 3;  // row of the Q fill j: 8 j + qrow
  auto fill_q = [&](int j) __attribute__((always_inline)) {
    const int r = 8 * j + qrow;
    lds_fill16_at(rq, vslot_addr(wave) + 1024u * j,
                  (uint32_t)(qw0 + r) * kRowBytes + 16u * (uint32_t)(fpos ^ k_swz(r)));
  };
  bf16x8 qf[2][4];
  auto read_q = [&]() __attribute__((always_inline)) {
    const lds_uint4* qs = (const lds_uint4*)(uintptr_t)vslot_addr(wave);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int row = 32 * qb + ln;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 v = __builtin_bit_cast(uint4, qs[row * 8 + ((2 * s + hh) ^ k_swz(row))]);
        v.x ^= sign;
        v.y ^= sign;
        v.z ^= sign;
        v.w ^= sign;
        qf[qb][s] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };

  // Row sums on the matrix cores: a constant 0/1 A operand against the P
  // registers (row 0 selects the even k groups -- queries 0..15 -- and row 1
  // the odd ones); the sums land in lanes 0..15, registers 0 and 1.
  const bf16x8 sel = __builtin_bit_cast(
      bf16x8, (((lane & 15) == 0 && ((lane >> 4) & 1) == 0) || ((lane & 15) == 1 && ((lane >> 4) & 1) == 1))
                  ? make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u)
                  : make_uint4(0u, 0u, 0u, 0u));

  // Per-wave softmax state.  Accumulator register r of a 32x32 block holds
  // row/column 8 (r / 4) + 4 hh + r % 4 of the block's M side and column ln
  // of its N side.
  f32x16 o[2][2];      // O^T[d block][query block]
  f32x16 sc[2][2];     // S^T[key block][query block] of the current tile
  uint32_t pk[2][16];  // bf16 weights [query block][8 key block + pair]
  float mc[2];         // pivots (log2 domain)
  f32x4 ls[2];         // row sums
  bool seen[2];        // the row has met an allowed key
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      mc[i] = 0.f;
      ls[i] = f32x4{};
      seen[i] = false;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        o[i][j] = f32x16{};
        sc[i][j] = f32x16{};
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) pk[i][k] = 0u;
    }
  };

  // V^T fragments of one key step j (as in the paired kernel).
  auto load_v_step = [&](uint32_t vbase, auto j_tag, bf16x8 (&va)[2][4]) __attribute__((always_inline)) {
    constexpr int j = decltype(j_tag)::value;
    const lds_char* vt = (const lds_char*)(uintptr_t)vbase;
    const int gq = lane >> 4;
    const int i = lane & 15;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      s16x4 part[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int kr = 16 * j + 8 * x + 4 * (gq >> 1) + (i >> 2);
        const int h = 8 * db + 4 * (gq & 1) + (i & 3);
        const int byte = kr * (int)kRowBytes + 16 * ((h >> 1) ^ (2 * (kr & 3))) + 8 * (h & 1);
        part[x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_char*)(vt + byte));
      }
      va[db][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto load_k_step = [&](uint32_t kbase, auto s_tag, bf16x8 (&ka)[2][4]) __attribute__((always_inline)) {
    constexpr int s = decltype(s_tag)::value;
    const lds_uint4* kt = (const lds_uint4*)(uintptr_t)kbase;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = 32 * kb + ln;
      ka[kb][s] = __builtin_bit_cast(bf16x8, kt[row * 8 + ((2 * s + hh) ^ k_swz(row))]);
    }
  };
  auto pv_step = [&](auto j_tag, const bf16x8 (&va)[2][4]) __attribute__((always_inline)) {
    constexpr int j = decltype(j_tag)::value;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const bf16x8 pb = __builtin_bit_cast(
          bf16x8, make_uint4(pk[qb][4 * j], pk[qb][4 * j + 1], pk[qb][4 * j + 2], pk[qb][4 * j + 3]));
#pragma unroll
      for (int db = 0; db < 2; ++db)
        o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][j], pb, o[db][qb], 0, 0, 0);
      ls[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb, ls[qb], 0, 0, 0);
    }
  };
  auto qk_smajor = [&](const bf16x8 (&ka)[2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sc[kb][qb] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][s], qf[qb][s], s == 0 ? f32x16{} : sc[kb][qb], 0, 0, 0);
  };

  // Band mask of tile T (absolute keys k0 .. k0 + 63): a row keeps keys in
  // [max(0, qi - wl), min(kv_lim, qi + wr + 1)).  Only tiles that cross an
  // edge of some row's window, key 0 or kv_lim, take it.
  auto mask_tile = [&](int T) __attribute__((always_inline)) {
    const int k0 = (t0 + T) * kBN;
    const bool need_mask =
        k0 < 0 || k0 + kBN > kv_lim || k0 + kBN - 1 > qw0 + wr || k0 < qw0 + kWaveRows - 1 - wl;
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qi = qw0 + 32 * qb + ln;
        const int lim = min(kv_lim, qi + wr + 1) - k0 - 4 * hh;
        const int lo = max(0, qi - wl) - k0 - 4 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          sc[0][qb][r] = (off < lim && off >= lo) ? sc[0][qb][r] : -INFINITY;
          sc[1][qb][r] = (off + 32 < lim && off + 32 >= lo) ? sc[1][qb][r] : -INFINITY;
        }
      }
    }
  };
  // Weights of tile T under the fixed pivot 0: x = s c, 2^x.  The mask is
  // plain VALU arithmetic folded into the scaling: a key at offset o of the
  // tile (o = 4 hh + the register's compile-time offset) is allowed iff
  // o < hi and o >= lo, i.e. iff t_hi = (hi - 1/2 - o) 2^120 and
  // t_lo = (o - lo + 1/2) 2^120 are both positive, and x = s c + min(t_hi,
  // t_lo, 0) in one FMA: exactly s c where allowed, at most -2^119 where
  // not, whose 2^x is 0.  A lane's bound times 2^120 may round or overflow
  // to +-inf only when it lies 2^23 or more from the tile, far from every
  // offset, so the sign of t is always right.  Each bound applies only to
  // tiles that cross it: a subtract and a min per score and bound.  (A
  // compare-and-select costs two compares, a scalar AND and a select per
  // score, chained through the scalar unit: about 0.5 us per masked phase.)
  auto scale_mask = [&](int k0, auto hi_tag, auto lo_tag) __attribute__((always_inline)) {
    constexpr bool HI = decltype(hi_tag)::value, LO = decltype(lo_tag)::value;
    constexpr float kS = 0x1p120f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if constexpr (HI || LO) {
        // The row index from an opaque copy of the lane's: the bounds are
        // rebuilt here rather than hoisted and held through the loop.
        int lnm = ln;
        asm volatile("" : "+v"(lnm));
        const int qi = qw0 + 32 * qb + lnm;
        float hi = HI ? ((float)(min(kv_lim, qi + wr + 1) - k0 - 4 * hh) - 0.5f) * kS : 0.f;
        float lo = LO ? ((float)(max(0, qi - wl) - k0 - 4 * hh) - 0.5f) * kS : 0.f;
        // Opaque, so that hi - o stays a subtract of a literal instead of
        // being fused into the product above with o held in a register.
        asm volatile("" : "+v"(hi), "+v"(lo));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float o = (float)(32 * kb + 8 * (r >> 2) + (r & 3)) * kS;
            float pen = 0.f;
            if constexpr (HI) pen = fminf(pen, hi - o);
            if constexpr (LO) pen = fminf(pen, o - lo);
            sc[kb][qb][r] = fmaf(sc[kb][qb][r], c, pen);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[kb][qb][r] *= c;
      }
      exp_pack(sc[0][qb], sc[1][qb], pk[qb]);
    }
  };
  auto softmax_fixed = [&](int T) __attribute__((always_inline)) {
    const int k0 = (t0 + T) * kBN;
    const bool need_hi = k0 + kBN > kv_lim || k0 + kBN - 1 > qw0 + wr;
    const bool need_lo = k0 < 0 || k0 < qw0 + kWaveRows - 1 - wl;
    using Y = std::true_type;
    using N = std::false_type;
    if (need_hi && need_lo) {
      asm volatile("");
      scale_mask(k0, Y(), Y());
    } else if (need_hi) {
      asm volatile("");
      scale_mask(k0, Y(), N());
    } else if (need_lo) {
      asm volatile("");
      scale_mask(k0, N(), Y());
    } else {
      scale_mask(k0, N(), N());
    }
  };
  // Weights of tile T under the moving pivot (the paired kernel's): the
  // pivot moves to the row's tile max when a weight would pass 2^64, or,
  // while the row has summed nothing, fall below 2^-64; O and l are
  // rescaled by 2^(m_old - m_new).
  auto softmax = [&](int T) __attribute__((always_inline)) {
    mask_tile(T);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][qb][r] = fmaf(sc[kb][qb][r], c, -mc[qb]);
    float gap[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) gap[qb] = half_swap_max(max32(sc[0][qb], sc[1][qb]));
    bool move[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) move[qb] = gap[qb] > kPivotUp;
    if (__builtin_amdgcn_ballot_w64(!seen[0] || !seen[1]) != 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        move[qb] = move[qb] || (gap[qb] < kPivotDown && gap[qb] > -INFINITY && !seen[qb]);
        seen[qb] = seen[qb] || gap[qb] > -INFINITY;
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (__builtin_amdgcn_ballot_w64(move[qb]) != 0) {
        const float shift = move[qb] ? gap[qb] : 0.f;
        const float alpha = shift > 0.f ? __builtin_amdgcn_exp2f(-shift) : 1.f;
        const auto hi =
            __builtin_amdgcn_permlane16_swap(__float_as_uint(alpha), __float_as_uint(alpha), false, false);
        ls[qb][0] *= alpha;
        ls[qb][1] *= __uint_as_float(hi[1]);
        o[0][qb] *= alpha;
        o[1][qb] *= alpha;
        mc[qb] += shift;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[0][qb][r] -= shift;
          sc[1][qb][r] -= shift;
        }
      }
      exp_pack(sc[0][qb], sc[1][qb], pk[qb]);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // Matrix phase of local tile u (tile g + u): P.V of tile g + u - 1, then
  // (QK) S of tile g + u, as one straight block.  At u = 0 the weights are
  // zero and V is the zero tile (that V slot may not hold V yet); past the
  // window the weights are zero and the scores are never used; the last
  // phase, u = n_run, has no S.
  auto mphase = [&](int u, auto qk_tag) __attribute__((always_inline)) {
    constexpr bool QK = decltype(qk_tag)::value;
    const uint32_t vbase =
        u == 0 ? (uint32_t)(uintptr_t)(lds_void_t*)&g_zero[0] : vslot_addr((g + u + kRing - 1) % kRing);
    const uint32_t kbase = kslot_addr((g + u) % kRing);
    __builtin_amdgcn_s_setprio(1);
    bf16x8 va[2][4], ka[2][4];
    load_v_step(vbase, I0(), va);
    load_v_step(vbase, I1(), va);
    load_v_step(vbase, I2(), va);
    __builtin_amdgcn_sched_barrier(0);
    pv_step(I0(), va);
    __builtin_amdgcn_sched_barrier(0);
    load_v_step(vbase, I3(), va);
    __builtin_amdgcn_sched_barrier(0);
    pv_step(I1(), va);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (QK) {
      load_k_step(kbase, I0(), ka);
      load_k_step(kbase, I1(), ka);
    }
    __builtin_amdgcn_sched_barrier(0);
    pv_step(I2(), va);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (QK) {
      load_k_step(kbase, I2(), ka);
      load_k_step(kbase, I3(), ka);
    }
    __builtin_amdgcn_sched_barrier(0);
    pv_step(I3(), va);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (QK) qk_smajor(ka);
    __builtin_amdgcn_s_setprio(0);
  };
  // Vector phase of local tile u: its weights, or zeros past the window.
  auto vphase = [&](int u) __attribute__((always_inline)) {
    if (u < cnt) {
      softmax_fixed(g + u);
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("v_mov_b32 %0, 0" : "=v"(pk[qb][i]));
    }
  };
  // The odd phase 2k + 1 fills K of tile k + 9 (into the slot of K tile k,
  // last read at phase 2k) and V of tile k + 8 (into the slot of V tile
  // k - 1, last read at phase 2k); each is first read four phases later.
  auto fills = [&](int k) __attribute__((always_inline)) {
    fill_k(k + 9);
    fill_v(k + 8);
  };
  // End of phase: a wait for this wave's fills that the next phase reads
  // (vmcnt(N): all but the N latest have landed), then the barrier that
  // publishes them to the other waves.
  auto sync = [&](auto n_tag) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | decltype(n_tag)::value);
    barrier_lds();
  };
  using N0 = std::integral_constant<int, 0>;
  using N2 = std::integral_constant<int, 2>;
  using N4 = std::integral_constant<int, 4>;
  using N7 = std::integral_constant<int, 7>;

  // Row sums in the row layout: lane (ln, hh) takes query ln's sum from
  // lane ln % 16, register ln / 16.
  auto row_sums = [&](float (&l)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float v0 = __int_as_float(__builtin_amdgcn_ds_bpermute((lane & 15) * 4, __float_as_int(ls[qb][0])));
      const float v1 = __int_as_float(__builtin_amdgcn_ds_bpermute((lane & 15) * 4, __float_as_int(ls[qb][1])));
      l[qb] = (ln < 16) ? v0 : v1;
    }
  };
  // O = acc / l, bf16; log-sum-exp (m + log2 l) ln 2.  Padded rows and rows
  // with no allowed key are written as exact zeros (lse -inf).  pack_rows
  // forms the bf16 rows in registers (and writes the lse); store_rows sends
  // them through K slot `wave` (free once every wave has passed the last
  // barrier, and used by no other wave after it), so that each store writes
  // whole 128-byte rows, 8 lanes a row, rather than 16-byte pieces of 32
  // rows: row r's 16-byte piece c (d 8 c .. 8 c + 7) sits at position
  // c ^ (r % 8).  A wave's LDS operations complete in order, so its reads
  // see its writes.  Both rebuild their addresses from a fresh copy of the
  // lane index instead of holding them in registers through the tile loop.
  // Register r of block (db, qb) holds d = 32 db + 8 (r / 4) + 4 hh + r % 4
  // of query row qw0 + 32 qb + ln: four consecutive d, packed into w[vg]
  // with vg = 8 db + 4 qb + r / 4.
  auto pack_rows = [&](const float (&l)[2], u32x2 (&w)[16]) __attribute__((always_inline)) {
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const int ln_e = lane_e & 31;
    float inv[2];
    bool live[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qi = qw0 + 32 * qb + ln_e;
      live[qb] = qi < q_len && l[qb] > 0.f;
      inv[qb] = live[qb] ? 1.f / l[qb] : 0.f;
      if (a.lse && lane_e < 32 && qi < a.n_q)
        a.lse[(size_t)bh * a.n_q + qi] = live[qb] ? (mc[qb] + __builtin_amdgcn_logf(l[qb])) * kLn2 : -INFINITY;
    }
    static_for<16>([&](auto vg_tag) {
      constexpr int VG = decltype(vg_tag)::value;
      constexpr int DB = VG / 8, QB = (VG / 4) % 2, G = VG % 4, R = 4 * G;
      w[VG].x = live[QB] ? pack_bf16x2(o[DB][QB][R] * inv[QB], o[DB][QB][R + 1] * inv[QB]) : 0u;
      w[VG].y = live[QB] ? pack_bf16x2(o[DB][QB][R + 2] * inv[QB], o[DB][QB][R + 3] * inv[QB]) : 0u;
    });
  };
  auto store_rows = [&](const u32x2 (&w)[16]) __attribute__((always_inline)) {
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const int ln_e = lane_e & 31, hh_e = lane_e >> 5;
    lds_char* so = (lds_char*)(uintptr_t)kslot_addr(wave);
    static_for<16>([&](auto vg_tag) {
      constexpr int VG = decltype(vg_tag)::value;
      constexpr int DB = VG / 8, QB = (VG / 4) % 2, G = VG % 4;
      const int r = 32 * QB + ln_e;
      *(lds_u32x2*)(so + r * 128 + (((4 * DB + G) ^ (r & 7)) << 4) + 8 * hh_e) = w[VG];
    });
    const int q = lane_e & 7;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = 8 * it + (lane_e >> 3);
      const uint4 v = __builtin_bit_cast(uint4, *(const lds_uint4*)(so + r * 128 + ((q ^ (r & 7)) << 4)));
      if (qw0 + r < a.n_q) *reinterpret_cast<uint4*>(O + (size_t)(qw0 + r) * kHeadDim + 8 * q) = v;
    }
  };

  // ---- the fixed-pivot pass over the rings.
  reset();
  if (n_run > 0) {
    // Prologue.  K 0-3 are read at phase 0 (products of row groups 0-3), K
    // 4-7 at phase 1 (groups 4-7), V 0-3 at phase 2, V 4-7 and K 8 at phase
    // 3.  Each wave stages its Q in V slot `wave`: the waves of groups 0-3
    // ahead of their K fills (they read Q before the first barrier), those
    // of groups 4-7 behind their share of K 0-3 (they read Q during phase
    // 0, where they have no products).  V 0-3 go out after the first
    // barrier, V 4-7 after the second, each once the Q in its slot has been
    // read.  The compiler's own loads (lengths) have landed first, so that
    // it does not wait for them later with a vmcnt(0) that drains the ring.
    auto prologue = [&](auto par_tag) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par_tag)::value;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      g_zero[tid] = make_uint4(0, 0, 0, 0);
      if constexpr (PAR == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) fill_q(j);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) fill_k(t);
      if constexpr (PAR == 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j) fill_q(j);
      }
#pragma unroll
      for (int t = 4; t < 8; ++t) fill_k(t);
      if constexpr (PAR == 0) {
        __builtin_amdgcn_s_waitcnt(0x0F70 | 8);  // this wave's Q has landed
        read_q();
        __builtin_amdgcn_s_waitcnt(0x0070 | 4);  // vmcnt(4), lgkmcnt(0): K 0-3 landed, Q read
      } else {
        __builtin_amdgcn_s_waitcnt(0x0070 | 12);  // vmcnt(12), lgkmcnt(0): K 0-3 landed
      }
      barrier_lds();
#pragma unroll
      for (int t = 0; t < 4; ++t) fill_v(t);
      fill_k(8);
    };
    auto fill_v4_7 = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int t = 4; t < 8; ++t) fill_v(t);
    };
    // Phases 0 .. 2 n_run + 1: a wave's products of local tile u at phase
    // 2u + par, its weights one phase later.  The waits after phases 0 and
    // 1 cover the prologue's fills.
    if (par == 0) {
      prologue(std::integral_constant<int, 0>());
#pragma nounroll
      for (int u = 0; u < n_run; ++u) {
        mphase(u, std::true_type());
        if (u == 0) {
          __builtin_amdgcn_s_waitcnt(0x0070 | 5);  // phase 0: K 4-7 landed
          barrier_lds();
          fill_v4_7();
        } else {
          sync(N2());  // phase 2u
        }
        fills(u);
        vphase(u);
        if (u == 0) sync(N7());  // phase 1
        else sync(N4());         // phase 2u + 1
      }
      mphase(n_run, std::false_type());
      sync(N0());  // phase 2 n_run: this wave's fills have all landed
    } else {
      prologue(std::integral_constant<int, 1>());
      // Phase 0: this wave's Q, then K 4-7 landed and every Q read.
      __builtin_amdgcn_s_waitcnt(0x0F70 | 9);
      read_q();
      __builtin_amdgcn_s_waitcnt(0x0070 | 5);
      barrier_lds();
      fill_v4_7();
#pragma nounroll
      for (int u = 0; u < n_run; ++u) {
        fills(u);
        mphase(u, std::true_type());
        if (u == 0) sync(N7());  // phase 1
        else sync(N4());         // phase 2u + 1
        vphase(u);
        sync(N2());  // phase 2u + 2
      }
      mphase(n_run, std::false_type());        // phase 2 n_run + 1
      __builtin_amdgcn_s_waitcnt(0x0F70 | 0);  // every fill has landed
    }
  }

  // Range check of the fixed pivot.  Under pivot 0 every weight of a row is
  // at most its sum l, so l < 2^64 bounds every weight, partial sum and
  // product below fp32 overflow (a weight of 2^128 or more shows as l = inf,
  // NaN as a NaN sum); l >= 2^-32 puts the row's largest weight at 2^-56 or
  // more (a row has fewer than 2^24 keys), so a weight that fell into the
  // subnormal range is below 2^-70 of it and changes no result.  A row group
  // with a row that has an allowed key and fails either bound -- logits far
  // above 64 or far below -32 in log2 units -- is recomputed below; rows
  // without one (padded, kv_len = 0, an empty window) are zeros either way.
  bool ok;
  u32x2 w[16];
  {
    float l[2];
    row_sums(l);
    // The rows' bounds from a fresh copy of the lane's row index, rather
    // than values held in registers through the tile loop.
    int ln_c = ln;
    asm volatile("" : "+v"(ln_c));
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qi = qw0 + 32 * qb + ln_c;
      const int lo = max(0, qi - wl);
      const int hi = min(kv_lim, qi + wr + 1);
      const bool keys = qi < q_len && lo < hi;
      const bool in_range = l[qb] >= 0x1p-32f && l[qb] < 0x1p64f;
      bad = bad || (keys && !in_range);
    }
    ok = __builtin_amdgcn_ballot_w64(bad) == 0;
    if (ok) pack_rows(l, w);
  }
  // No wave reads a ring or has a fill in flight past this barrier.
  if (n_run > 0) barrier_lds();
  if (ok) {
    store_rows(w);
    return;
  }

  // ---- a row group that failed the range check: its window again, under
  // the moving pivot, one tile at a time through its own K and V slots
  // (slot `wave` of each ring).  Each wave fills whole tiles itself, so it
  // needs no barrier; the slots are free once every wave has passed the
  // barrier above.
  reset();
  {
    const uint32_t kdst = kslot_addr(wave), vdst = vslot_addr(wave);
#pragma nounroll
    for (int u = 0; u < cnt; ++u) {
      const int T = g + u;
      const uint32_t toff = tile_off(T);
      // Fill offsets from a fresh copy of the lane index each tile: held
      // through the pipeline they would not fit the registers.
      int lf = lane;
      asm volatile("" : "+v"(lf));
      const int frow = lf >> 3, fp = lf & 7;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * j + frow;
        const uint32_t roff = toff + (uint32_t)r * kRowBytes;
        lds_fill16_at(rk, kdst + 1024u * j, roff + 16u * (uint32_t)(fp ^ k_swz(r)));
        lds_fill16_at(rv, vdst + 1024u * j, roff + 16u * (uint32_t)(fp ^ (2 * (r & 3))));
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): both tiles have landed
      bf16x8 ka[2][4];
      load_k_step(kdst, I0(), ka);
      load_k_step(kdst, I1(), ka);
      load_k_step(kdst, I2(), ka);
      load_k_step(kdst, I3(), ka);
      qk_smajor(ka);
      softmax(T);
      bf16x8 va[2][4];
      load_v_step(vdst, I0(), va);
      load_v_step(vdst, I1(), va);
      load_v_step(vdst, I2(), va);
      load_v_step(vdst, I3(), va);
      pv_step(I0(), va);
      pv_step(I1(), va);
      pv_step(I2(), va);
      pv_step(I3(), va);
    }
    float l[2];
    row_sums(l);
    pack_rows(l, w);
    store_rows(w);
  }
}

}  // namespace

hipError_t launch_fwd_bf16_band(const FwdArgs& a, hipStream_t s) {
  const int n_qt = (a.n_q + kBM - 1) / kBM;
  const long long blocks = (long long)n_qt * a.H * a.B;
  FwdArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_bf16_band_kernel), dim3((unsigned)blocks),
                         dim3(kThreads), kargs, 0, s);
}

}  // namespace headattn
