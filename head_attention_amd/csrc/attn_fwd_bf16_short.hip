// bf16 forward of attn_forward for short key ranges (n_k <= 256): one load,
// then no barriers.
//
// Computes O = softmax(Q K^T * scale + M) V per (b, h) ("[논문 리뷰]Attention
// Is All You Need", §3.2.1 equation; masking by -inf logits before the
// softmax, §3.2.3) with the arithmetic of the other bf16 kernels: exact bf16
// Q (sign of scale folded in), S^T = K Q^T and O^T += V^T P^T on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation, weights exp2(s c - m c)
// with a lazy pivot, weights rounded to bf16 once and summed as rounded.
//
// The pages' encoder and decoder layers attend over at most a few hundred
// positions (Transformer-base/big at sentence length), where a kernel is
// bound by memory latency, not by either pipe: a (b, h) of 128 queries and
// 128 keys is 2 key tiles.  Streaming tiles through a double-buffered ring
// puts one global-memory round trip per tile on the critical path.  Here the
// workgroup (4 waves, 128 query rows, 32 per wave) instead issues every load
// it needs at once -- its Q rows into registers, all valid K and V rows
// straight into LDS (buffer loads that write LDS, range-checked so rows at
// or beyond the valid length read as zero) -- waits once, and then each wave
// walks its key tiles on its own with no further barrier: one memory round
// trip per workgroup.  K and V of up to 256 keys take 64 KB of LDS, so two
// workgroups fit a compute unit.
//
// LDS layout, per 64-key tile: K rows keep their 16-byte chunks XOR-swizzled
// by row; V stays row-major (chunks swizzled by 2 (row % 4)) and is read
// transposed with ds_read_b64_tr_b16, which hands each lane four consecutive
// keys of one d -- the A-operand order of O^T += V^T P^T, with the keys in
// the order the S accumulator registers hold them, so the weights feed the
// B operand straight from registers.
#include "kernel_util.h"

namespace headattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr int kMaxTiles = kShortMaxKeys / kBN;
constexpr uint32_t kTileChunks = kBN * 8;  // 16-byte chunks per tile

__shared__ uint4 s_k[kMaxTiles * kTileChunks];
__shared__ uint4 s_v[kMaxTiles * kTileChunks];
// Each wave's output rows on their way to memory (32 rows x 128 bytes).
__shared__ uint4 s_o[kWaves * 32 * 8];

// Weights of one tile under pivot term mc = m c: exp2(s c - mc), packed to
// bf16 pairs in the order P.V consumes them (keys 0..31 from s0, 32..63 from
// s1), and the sum of the packed (rounded) weights held by this lane.
__device__ __forceinline__ float exp_pack_sum(const f32x16& s0, const f32x16& s1, float c, float mc,
                                              uint32_t (&pk)[16]) {
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pk[i] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s0[2 * i], c, -mc)),
                        __builtin_amdgcn_exp2f(fmaf(s0[2 * i + 1], c, -mc)));
    pk[8 + i] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s1[2 * i], c, -mc)),
                            __builtin_amdgcn_exp2f(fmaf(s1[2 * i + 1], c, -mc)));
    acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]), ones, acc0, false);
    acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[8 + i]), ones, acc1, false);
  }
  return acc0 + acc1;
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_short_kernel(FwdArgs a) {
  constexpr bool CAUSAL = MODE == kModeCausal;
  constexpr bool BAND = MODE == kModeBand;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;  // query row within the wave / M,N index of MFMA
  const int hh = lane >> 5;  // half-wave: selects the 8-wide k block

  // ---- (b, h, query tile).  The 8 XCDs take workgroup ids round robin; when
  // B*h divides by 8 each XCD gets whole heads.  Longest tiles first under
  // the causal mask.
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

  const int q_len = __builtin_amdgcn_readfirstlane(a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q);
  const int kv_lim = __builtin_amdgcn_readfirstlane(a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k);
  const int q0 = qt * kBM;
  const int qw0 = q0 + 32 * wave;  // first query row of this wave
  const int qi = qw0 + ln;         // query row of this lane

  // Restricted self-attention: row i sees keys i - wl .. i + wr; a wave
  // starts at the first tile its rows' windows reach.
  const int wl = BAND ? a.radius : 0;
  const int wr = BAND ? (a.causal ? 0 : a.radius) : 0;
  int end = kv_lim;  // keys the workgroup needs (at most n_k <= 256)
  if (CAUSAL) end = min(end, q0 + kBM);
  if (BAND) end = min(end, q0 + kBM + wr);
  if (q0 >= q_len) end = 0;
  const int n_tiles = min((end + kBN - 1) / kBN, kMaxTiles);  // the host sends n_k <= 256 only
  int wave_end = min(end, kShortMaxKeys);  // keys this wave needs
  if (CAUSAL) wave_end = min(wave_end, qw0 + 32);
  if (BAND) wave_end = min(wave_end, qw0 + 32 + wr);
  if (qw0 >= q_len) wave_end = 0;
  const int wave_tiles = (wave_end + kBN - 1) / kBN;
  const int wave_first = BAND ? max(0, qw0 - wl) / kBN : 0;

  // ---- loads.  Every load is issued at once, in the order of use: each
  // wave's 32 Q rows into its own 4 KB of s_o, then the K and V tiles,
  // tile by tile.  The loop below waits for one tile at a time, so a
  // wave's products on tile t overlap the landing of the later tiles (the
  // whole chip loads at once here, and HBM is the limit of that burst).
  // The fills are issued from inline assembly (lds_fill16_at), which the
  // compiler does not track: the loop's vmcnt waits and barriers order them.
  // Q: B operand of S^T = K Q^T, lane (ln, hh) holds Q[qi][16 s + 8 hh +
  // 0..7], sign of scale folded in; c = |scale| log2(e), floored at 2^-100
  // (below that every weight is exactly 1.0f).  Rows at or beyond n_q read
  // as zeros through the descriptor's range check.
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-100f);
  const uint32_t sign = a.scale < 0.f ? 0x80008000u : 0u;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(Q), (short)0, (int)((uint32_t)a.n_q * kRowBytes), kBufferWord3);
  const uint32_t qdst = (uint32_t)(uintptr_t)(lds_void_t*)(s_o + 256 * wave);
  // K and V tiles: one instruction of the workgroup covers 32 rows of a
  // tile.  Lane l of wave w writes chunk 64 w + l of that half, i.e. row
  // 32 half + 8 w + l / 8, position l % 8, which receives the row's chunk
  // (l % 8) ^ swizzle(row).  The range check of the descriptor returns zeros
  // for rows at or beyond kv_lim, so padded K/V memory is never read.
  const uint32_t n_bytes = (uint32_t)kv_lim * kRowBytes;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(K), (short)0, (int)n_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(V), (short)0, (int)n_bytes, kBufferWord3);
  const int fpos = lane & 7;
  if (n_tiles > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * i + (lane >> 3);
      lds_fill16_at(rq, qdst + 1024u * i, (uint32_t)(qw0 + row) * kRowBytes + 16u * (uint32_t)(fpos ^ k_swz(row)));
    }
  }
  for (int t = 0; t < n_tiles; ++t) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 32 * half + 8 * wave + (lane >> 3);
      const uint32_t base = (uint32_t)(t * kBN + row) * kRowBytes;
      const uint32_t koff = base + 16u * (uint32_t)(fpos ^ k_swz(row));
      const uint32_t voff = base + 16u * (uint32_t)(fpos ^ (2 * (row & 3)));
      const uint32_t chunk0 = (uint32_t)t * kTileChunks + 256u * half + 64u * wave;
      lds_fill16_at(rk, (uint32_t)(uintptr_t)(lds_void_t*)(s_k + chunk0), koff);
      lds_fill16_at(rv, (uint32_t)(uintptr_t)(lds_void_t*)(s_v + chunk0), voff);
    }
  }
  bf16x8 qf[4];

  f32x16 o0 = {}, o1 = {};  // O^T blocks: d 0..31 and d 32..63, column = query ln
  float mc = 0.f;           // pivot term of the exponent, m * c
  float l = 0.f;            // this half-wave's partial row sum of bf16 weights

  // Band mode: whether the row has summed a nonzero weight yet (its pivot
  // may move down only before that); both half-waves of a row agree.  The
  // other modes need no flag: tile 0 holds key 0, which every row with a key
  // may see.
  bool seen = false;

  const int g = lane >> 4;
  const int i16 = lane & 15;
  for (int t = 0; t < n_tiles; ++t) {
    // Tile t has landed when at most the 4 fills of each later tile are in
    // flight; the barrier publishes every wave's share of it.  Every wave
    // passes every barrier, whether or not it needs the tile.
    const int later = n_tiles - 1 - t;
    if (later >= 3) __builtin_amdgcn_s_waitcnt(0x0070 | 12);  // vmcnt(12), lgkmcnt(0)
    else if (later == 2) __builtin_amdgcn_s_waitcnt(0x0070 | 8);
    else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0070 | 4);
    else __builtin_amdgcn_s_waitcnt(0x0070);
    barrier_lds();
    if (t == 0) {
      // This wave's own Q rows, filled ahead of tile 0.
      const lds_uint4* qs = (const lds_uint4*)(uintptr_t)qdst;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 v = __builtin_bit_cast(uint4, qs[ln * 8 + ((2 * s + hh) ^ k_swz(ln))]);
        v.x ^= sign;
        v.y ^= sign;
        v.z ^= sign;
        v.w ^= sign;
        qf[s] = __builtin_bit_cast(bf16x8, v);
      }
    }
    if (t < wave_first || t >= wave_tiles) continue;
    // S^T = K Q^T: lane (ln, hh) of key block kb reads K[64 t + 32 kb + ln]
    // [16 s + 8 hh + 0..7].
    const uint4* kt = s_k + t * kTileChunks;
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + hh;
      const bf16x8 k0 = __builtin_bit_cast(bf16x8, kt[ln * 8 + (ch ^ k_swz(ln))]);
      const bf16x8 k1 = __builtin_bit_cast(bf16x8, kt[(32 + ln) * 8 + (ch ^ k_swz(32 + ln))]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], s1, 0, 0, 0);
    }
    // V^T fragments: [d block][key step].  Key step j (16 keys) of key block
    // j / 2 takes keys 16 (j % 2) + {0..3, 8..11} + 4 hh of the block, the
    // order in which the S registers hold them.  Lane i of 16-lane group g
    // names key row kr and 8-byte chunk h; the transposed read returns to
    // lane i the 4 keys kr - i/4 .. +3 of d = dbase + i.
    const char* vt = reinterpret_cast<const char*>(s_v + t * kTileChunks);
    bf16x8 va[2][4];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s16x4 part[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int kr = 16 * j + 8 * x + 4 * (g >> 1) + (i16 >> 2);
          const int h = 8 * db + 4 * (g & 1) + (i16 & 3);
          const int byte = kr * (int)kRowBytes + 16 * ((h >> 1) ^ (2 * (kr & 3))) + 8 * (h & 1);
          part[x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vt + byte));
        }
        va[db][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }

    // Mask in registers, only on tiles that cross the causal diagonal or the
    // key-length boundary: register r of block kb holds key 64 t + 32 kb +
    // 8 (r / 4) + 4 hh + r % 4.
    const int k0 = t * kBN;
    bool need_mask = (k0 + kBN > kv_lim) || (CAUSAL && k0 + kBN - 1 > qw0);
    if (BAND) need_mask = need_mask || (k0 + kBN - 1 > qw0 + wr) || (k0 < qw0 + 31 - wl);
    if (need_mask) {
      int hi = kv_lim;  // keys below hi and at or above lo are allowed
      if (CAUSAL) hi = min(hi, qi + 1);
      if (BAND) hi = min(hi, qi + wr + 1);
      const int lim = hi - k0 - 4 * hh;
      const int lo = BAND ? qi - wl - k0 - 4 * hh : INT_MIN;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        s0[r] = (off < lim && off >= lo) ? s0[r] : -INFINITY;
        s1[r] = (off + 32 < lim && off + 32 >= lo) ? s1[r] : -INFINITY;
      }
    }
    uint32_t pk[16];
    float lt = exp_pack_sum(s0, s1, c, mc, pk);
    // Pivot checks on the tile's weights: a sum past 2^64 (also catches inf)
    // or, on the row's first tile, a row sum small enough to be lost to
    // underflow.  The row's pivot then moves to its tile max, O and l are
    // rescaled by 2^(m_old - m_new) (a downward move happens only while O
    // and l are 0: scale 1), and the tile's weights are recomputed.  NaN
    // (garbage in padded rows) triggers neither check.
    bool move = lt > kPivotHigh;
    if (!BAND && t == 0) move = move || half_swap_sum(lt) < kPivotLow;
    if (BAND && __builtin_amdgcn_ballot_w64(!seen) != 0) {
      // A row that has summed nothing yet: a sum this small would be lost
      // to underflow (all-masked tiles give 0 and a max of -inf: no move).
      const float row_lt = half_swap_sum(lt);
      move = move || (!seen && row_lt < kPivotLow);
      seen = seen || row_lt > 0.f;
    }
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      move = half_swap_or(move);  // both half-waves of a row must agree
      float tmax = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, fmaxf(s0[r], s1[r]));
      const float tm = half_swap_max(tmax) * c;  // tile max in exponent units
      const float m_new = (move && tm > -INFINITY) ? tm : mc;
      const float alpha = m_new > mc ? __builtin_amdgcn_exp2f(mc - m_new) : 1.f;
      l *= alpha;
      o0 *= alpha;
      o1 *= alpha;
      mc = m_new;
      lt = exp_pack_sum(s0, s1, c, mc, pk);
      if (BAND) seen = seen || tm > -INFINITY;  // the tile max now weighs 1
    }
    l += lt;

    // O^T += V^T P^T.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]));
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[0][j], pb, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[1][j], pb, o1, 0, 0, 0);
    }
  }

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
  // The rows go through this wave's own LDS area, so that each store
  // writes whole 128-byte rows (8 lanes a row) rather than 16-byte pieces
  // of 32 rows: row ln's 16-byte piece c (d 8 c .. 8 c + 7) sits at
  // position c ^ (ln % 8).  A wave's LDS operations complete in order, so
  // its reads see its writes.
  lds_char* so = (lds_char*)(uintptr_t)(lds_void_t*)(s_o + 256 * wave);
#pragma unroll
  for (int ob = 0; ob < 2; ++ob) {
    const f32x16& o = ob ? o1 : o0;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      u32x2 w;
      w.x = live ? pack_bf16x2(o[4 * gg + 0] * inv, o[4 * gg + 1] * inv) : 0u;
      w.y = live ? pack_bf16x2(o[4 * gg + 2] * inv, o[4 * gg + 3] * inv) : 0u;
      *(lds_u32x2*)(so + ln * 128 + (((4 * ob + gg) ^ (ln & 7)) << 4) + 8 * hh) = w;
    }
  }
  const int q = lane & 7;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = 8 * it + (lane >> 3);
    const uint4 v = __builtin_bit_cast(uint4, *(const lds_uint4*)(so + row * 128 + ((q ^ (row & 7)) << 4)));
    if (qw0 + row < a.n_q) *reinterpret_cast<uint4*>(O + (size_t)(qw0 + row) * kHeadDim + 8 * q) = v;
  }
}

}  // namespace

hipError_t launch_fwd_bf16_short(const FwdArgs& a, hipStream_t s) {
  const int n_qt = (a.n_q + kBM - 1) / kBM;
  const long long blocks = (long long)n_qt * a.H * a.B;
  FwdArgs args = a;
  void* kargs[] = {&args};
  const int mode = fwd_mode(a);
  const void* fn = mode == kModeBand     ? reinterpret_cast<const void*>(&attn_fwd_bf16_short_kernel<kModeBand>)
                   : mode == kModeCausal ? reinterpret_cast<const void*>(&attn_fwd_bf16_short_kernel<kModeCausal>)
                                         : reinterpret_cast<const void*>(&attn_fwd_bf16_short_kernel<kModeNone>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), kargs, 0, s);
}

}  // namespace headattn
