// bf16 forward of attn_forward for long sequences: paired waves on gfx950.
//
// Computes O = softmax(Q K^T * scale + M) V per (b, h) ("[논문 리뷰]Attention
// Is All You Need", §3.2.1 equation; masking by -inf logits before the
// softmax, §3.2.3): exact bf16 Q (sign of scale folded in), S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, weights exp2(s c - m c), bf16
// weights, fp32 accumulation.
//
// The pipeline forms every weight under a fixed pivot m = 0 -- one multiply
// and one exponential per score, no row maxima -- and checks at the end that
// every row's sum stayed in a range where that pivot is exact up to rounding
// (softmax does not depend on the pivot).  A row group with a row outside it
// (logits beyond about +64 or below about -32 in log2 units: rare,
// adversarial inputs) is recomputed in the same launch, one tile at a time,
// with a pivot that moves to the row maximum (the lazy pivot of the other
// bf16 kernels).
//
// Workgroup: 8 waves own 256 query rows of one (b, h).  The hardware puts
// waves w and w + 4 on the same SIMD; both take the same 64 rows (row group
// w % 4), and split the key tiles between them: wave w takes the even 64-key
// tiles, wave w + 4 the odd ones.  Each wave keeps its own online-softmax
// state (m, l, O) and the pair merges the two at the end -- the same exact
// rescale-and-add identity as the decode split merge.
//
// Per tile a wave does two phases: an MFMA phase (O += P V of its previous
// tile, then S = K Q^T of this tile: 32 matrix instructions) and a vector
// phase (mask, exp2 and bf16 pack of this tile: ~165 VALU instructions in
// the first kernel; the moving pivot adds the row max and its checks).  The
// pair runs one phase apart and a workgroup barrier closes every phase, so
// while one wave of a SIMD issues matrix instructions
// the other issues the exponentials: the two kinds of work overlap across the
// two waves instead of alternating inside one.  (Measured on MI355X: MFMA
// and fma/exp/cvt work from two waves of one SIMD overlap, while v_dot2
// waits for the matrix pipe -- so the row sums run on the matrix cores
// themselves, as 16x16x32 products of the weights with a 0/1 selector, in
// the MFMA phase: 8 small products per tile instead of 32 v_dot2.)
//
// The MFMA phase is one straight block: its LDS fragment reads go out in the
// order of use, at most 12 in flight, so each group of products waits only
// for its own fragments while the rest arrive.
//
// 64 rows per wave means each K or V fragment read from LDS feeds two query
// blocks, half the LDS traffic per flop of 32-row waves; the per-wave state
// (Q 32, S 64, P 32, O 64 VGPRs) still fits the 256 registers that two waves
// per SIMD leave each wave, because a wave's phases run in sequence and no
// state is double buffered.
//
// K and V tiles reach LDS by buffer loads that write LDS directly (no VGPR
// staging).  Every wave fills 1 KB of each tile; rows at or beyond the valid
// length (or past the last key the workgroup may use) read as zero through
// the descriptor's range check, so padded K/V memory (even NaN) is never
// read.  Tiles sit in an 8-slot ring, K five phases and V seven phases ahead
// of use; a phase ends with a wait for this wave's fills of four phases ago
// and a barrier.
//
// K rows keep their 16-byte chunks
// XOR-swizzled by row; V stays row-major (chunks swizzled by row % 4) and is
// read transposed with ds_read_b64_tr_b16, which hands each lane four
// consecutive keys of one d -- the A-operand order of O^T += V^T P^T.
#include "kernel_util.h"

namespace headattn {
namespace {

constexpr int kThreads = 512;
constexpr int kWaveRows = 64;
constexpr int kBM = 4 * kWaveRows;  // query rows per workgroup
constexpr int kBN = 64;             // keys per tile
constexpr uint32_t kTileBytes = kBN * kRowBytes;

// Ring of 8 slots, each the K and the V tile of one 64-key tile (8 KB each:
// 64 rows x 8 chunks of 16 B): K of slot s at g_ring[s], its V at
// g_ring[8 + s].  The fills are issued from inline assembly
// (lds_fill16_at), which the compiler does not track (with the builtin it
// would wait for every fill in flight before any read of the array): the
// phase loop's explicit vmcnt waits and barriers order them.
constexpr int kSlots = 8;
__shared__ uint4 g_ring[2 * kSlots][512];
// Fills run this many phases ahead: the fill at phase p is tile p + 5,
// into the slot of tile p - 3, whose V was last read at phase p - 1.
constexpr int kAhead = 5;
// Row sums and pivots of the odd-tile waves for the final merge.
__shared__ float2 g_lm[4][2][64];
// Per row group: a row failed the fixed-pivot range check.
__shared__ int g_bad[4];

// LDS byte address of ring row r (K of slot r, or V of slot r - 8), kept
// as an integer so that a slot chosen at run time costs one add.
__device__ __forceinline__ uint32_t ring_addr(int r) {
  return (uint32_t)(uintptr_t)(lds_void_t*)&g_ring[0][0] + (uint32_t)r * (512u * 16u);
}
// Tiles K0 .. K3 and V0 .. V3 as the 8 KB parts of the 64 KB merge area.
template <int S>
__device__ __forceinline__ uint4* mslot() {
  return S < 4 ? g_ring[S] : g_ring[kSlots + S - 4];
}

// (b, h, query tile) of workgroup bid: the 8 XCDs take workgroup ids round
// robin; when B*h divides by 8 each XCD gets whole heads.  Longest tiles
// first under the causal mask.
template <int MODE>
__device__ __forceinline__ void wg_tile(const FwdArgs& a, int bid, int& bh, int& qt) {
  const int n_qt = (a.n_q + kBM - 1) / kBM;
  const int HB = a.H * a.B;
  int rank;
  if ((HB & 7) == 0) {
    const int per = HB >> 3;
    const int slot = bid >> 3;
    rank = slot / per;
    bh = (bid & 7) * per + slot % per;
  } else {
    bh = bid % HB;
    rank = bid / HB;
  }
  qt = MODE == kModeCausal ? (n_qt - 1 - rank) : rank;
}

// One workgroup's computation: the weights under the fixed pivot 0, then a
// range check of every row; a row group with a row that fails it is
// recomputed under the moving pivot.
template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_pair_kernel(FwdArgs a) {
  constexpr bool CAUSAL = MODE == kModeCausal;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hh = lane >> 5;
  const int rg = wave & 3;    // row group (waves rg and rg + 4 share a SIMD)
  const int par = wave >> 2;  // parity of the tiles this wave takes

  int bh, qt;
  wg_tile<MODE>(a, blockIdx.x, bh, qt);
  const int b = bh / a.H;

  const __bf16* Q = static_cast<const __bf16*>(a.Q) + (size_t)bh * a.n_q * kHeadDim;
  const __bf16* K = static_cast<const __bf16*>(a.K) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* V = static_cast<const __bf16*>(a.V) + (size_t)bh * a.n_k * kHeadDim;
  __bf16* O = static_cast<__bf16*>(a.O) + (size_t)bh * a.n_q * kHeadDim;

  const int q_len = __builtin_amdgcn_readfirstlane(a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q);
  const int kv_lim = __builtin_amdgcn_readfirstlane(a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k);
  const int q0 = qt * kBM;
  const int qw0 = q0 + kWaveRows * rg;  // first query row of this wave

  int end = kv_lim;  // keys the workgroup needs
  if (CAUSAL) end = min(end, q0 + kBM);
  if (q0 >= q_len) end = 0;
  const int n_tiles = max(0, (end + kBN - 1) / kBN);
  int wave_end = end;  // keys this row group needs
  if (CAUSAL) wave_end = min(wave_end, qw0 + kWaveRows);
  if (qw0 >= q_len) wave_end = 0;
  const int wave_tiles = max(0, (wave_end + kBN - 1) / kBN);
  // The descriptors end at the last key the workgroup may use: the ring's
  // fills past its last tile read zeros without touching memory.
  const uint32_t n_bytes = (uint32_t)max(0, end) * kRowBytes;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(K), (short)0, (int)n_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(V), (short)0, (int)n_bytes, kBufferWord3);

  // ---- tile fills: lane l of wave w writes LDS chunk 64 w + l of the slot,
  // i.e. row 8 w + l / 8, position l % 8, which holds the row's chunk
  // (l % 8) ^ swizzle(row).
  const int frow = 8 * wave + (lane >> 3);
  const int fpos = lane & 7;
  const uint32_t koff = (uint32_t)frow * kRowBytes + 16u * (uint32_t)(fpos ^ k_swz(frow));
  const uint32_t voff = (uint32_t)frow * kRowBytes + 16u * (uint32_t)(fpos ^ (2 * (frow & 3)));
  auto fill_k = [&](auto slot_tag, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;
    lds_fill16_at(rk, ring_addr(S) + 1024u * wave, (uint32_t)t * kTileBytes + koff);
  };
  auto fill_v = [&](auto slot_tag, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;
    lds_fill16_at(rv, ring_addr(kSlots + S) + 1024u * wave, (uint32_t)t * kTileBytes + voff);
  };

  // ---- Q fragments: B operand of S^T = K Q^T for query block qb and d-step
  // s: lane (ln, hh) holds Q[qw0 + 32 qb + ln][16 s + 8 hh + 0..7], sign of
  // scale folded in; c = |scale| log2(e), floored at 2^-100 (below that
  // every weight is exactly 1.0f either way).  Q goes through LDS, filled
  // with the first tiles (see the prologue); its descriptor ends at q_len,
  // so padded query rows (i >= q_len, written as zeros) enter as zeros: the
  // row-sum products multiply other rows' weights by 0, which must not meet
  // NaN from padded memory.
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-100f);
  const uint32_t sign = a.scale < 0.f ? 0x80008000u : 0u;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(Q), (short)0, (int)((uint32_t)max(0, q_len) * kRowBytes), kBufferWord3);
  bf16x8 qf[2][4];

  // ---- per-wave softmax state.  Accumulator register r of a 32x32 block
  // holds row/column 8 (r / 4) + 4 hh + r % 4 of the block's M side and
  // column ln of its N side.
  f32x16 o[2][2];    // O^T[d block][query block]
  f32x16 sc[2][2];   // S^T[key block][query block] of the current tile
  uint32_t pk[2][16];  // bf16 weights [query block][8 key block + pair]
  float mc[2] = {0.f, 0.f};  // pivot term m * c per query block
  // Row sums of the bf16 weights, accumulated on the matrix cores: one
  // v_mfma_f32_16x16x32_bf16 per key step and query block takes the weights
  // as they sit in the P registers (B operand: lane l supplies 8 values of
  // column l % 16 in k group l / 16, i.e. of query l % 32 -- the groups of
  // odd index hold queries 16..31) against a constant 0/1 A operand whose
  // row 0 selects the even k groups and row 1 the odd ones.  Row 0 of the
  // 16 x 16 result then holds the sums of queries 0..15 and row 1 those of
  // queries 16..31: lanes 0..15, registers 0 and 1 (rows 2..15 stay 0).
  // Each product is an exact bf16 value times 1, summed in fp32.
  f32x4 ls[2] = {f32x4{}, f32x4{}};
  const bf16x8 sel = __builtin_bit_cast(
      bf16x8, (((lane & 15) == 0 && ((lane >> 4) & 1) == 0) || ((lane & 15) == 1 && ((lane >> 4) & 1) == 1))
                  ? make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u)
                  : make_uint4(0u, 0u, 0u, 0u));
  // Whether a row has summed a nonzero weight yet (the pivot may move down
  // only before that); both half-waves of a row agree.
  bool seen[2] = {false, false};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      o[i][j] = f32x16{};
      sc[i][j] = f32x16{};
    }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int i = 0; i < 16; ++i) pk[qb][i] = 0u;

  // MFMA operand fragments, read from LDS in the MFMA phase in the order
  // of use with at most 12 reads in flight, so each group of products waits
  // only for its own fragments (the LDS counter tracks 15 outstanding reads;
  // past that every wait becomes a wait for all of them).
  //
  // V^T: [d block][key step].  Key step j (16 keys) of key block kb = j / 2
  // takes, in MFMA k order, keys 16 (j % 2) + {0..3, 8..11} + 4 hh of the
  // block -- the order the S accumulators hold them in, so P feeds the B
  // operand straight from registers.  Each fragment is two transposed reads
  // of 4 keys: lane i of 16-lane group g names row (key) kr and 8-byte chunk
  // h, and the read returns to lane i the 4 keys kr - i/4 .. +3 of d = dbase
  // + i.
  auto load_v_at = [&](uint32_t vbase, auto j_tag, bf16x8 (&va)[2][4]) __attribute__((always_inline)) {
    constexpr int j = decltype(j_tag)::value;
    const lds_char* vt = (const lds_char*)(uintptr_t)vbase;
    const int g = lane >> 4;
    const int i = lane & 15;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      s16x4 part[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int kr = 16 * j + 8 * x + 4 * (g >> 1) + (i >> 2);
        const int h = 8 * db + 4 * (g & 1) + (i & 3);
        const int byte = kr * (int)kRowBytes + 16 * ((h >> 1) ^ (2 * (kr & 3))) + 8 * (h & 1);
        part[x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_char*)(vt + byte));
      }
      va[db][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // K: [key block][d-step]; lane (ln, hh) holds K[32 kb + ln][16 s + 8 hh +
  // 0..7].
  auto load_k_at = [&](uint32_t kbase, auto s_tag, bf16x8 (&ka)[2][4]) __attribute__((always_inline)) {
    constexpr int s = decltype(s_tag)::value;
    const lds_uint4* kt = (const lds_uint4*)(uintptr_t)kbase;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = 32 * kb + ln;
      ka[kb][s] = __builtin_bit_cast(bf16x8, kt[row * 8 + ((2 * s + hh) ^ k_swz(row))]);
    }
  };
  // The same from ring slot S (K) or kSlots + S (V).
  auto load_v_step = [&](auto slot_tag, auto j_tag, bf16x8 (&va)[2][4]) __attribute__((always_inline)) {
    load_v_at(ring_addr(kSlots + decltype(slot_tag)::value), j_tag, va);
  };
  auto load_k_step = [&](auto slot_tag, auto s_tag, bf16x8 (&ka)[2][4]) __attribute__((always_inline)) {
    load_k_at(ring_addr(decltype(slot_tag)::value), s_tag, ka);
  };
  // O^T += V^T P^T for key step j, and the row sums of that step's weights.
  auto pv_step = [&](auto j_tag, const bf16x8 (&va)[2][4]) __attribute__((always_inline)) {
    constexpr int j = decltype(j_tag)::value;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const bf16x8 pb = __builtin_bit_cast(
          bf16x8, make_uint4(pk[qb][4 * j], pk[qb][4 * j + 1], pk[qb][4 * j + 2], pk[qb][4 * j + 3]));
#pragma unroll
      for (int db = 0; db < 2; ++db) o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][j], pb, o[db][qb], 0, 0, 0);
      ls[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb, ls[qb], 0, 0, 0);
    }
  };
  // S^T = K Q^T: 2 key blocks x 2 query blocks x 4 d-steps, d-steps
  // outermost so four independent accumulation chains interleave.
  auto qk_smajor = [&](const bf16x8 (&ka)[2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][s], qf[qb][s], s == 0 ? f32x16{} : sc[kb][qb], 0, 0, 0);
  };

  // Weights of tile t from sc into pk.  Masks only on the tiles that cross
  // the causal diagonal or the key-length boundary.  The pivot is checked
  // first, on the tile's row max: a row's pivot moves to that max when the
  // max weight would exceed 2^64 (so tile sums stay far below fp32 range),
  // or, while the row has summed nothing, fall below 2^-64 (so its first
  // weights cannot underflow); O and l are rescaled by 2^(m_old - m_new).
  // Both half-waves of a row see the same max, pivot and sum, so they agree.
  // A fully masked row (max -inf) and NaN (garbage in padded query rows)
  // never move.
  auto softmax = [&](int t) __attribute__((always_inline)) {
    const int k0 = t * kBN;
    const bool need_mask = (k0 + kBN > kv_lim) || (CAUSAL && k0 + kBN - 1 > qw0);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qi = qw0 + 32 * qb + ln;
        int hi = kv_lim;  // keys below hi are allowed
        if (CAUSAL) hi = min(hi, qi + 1);
        const int lim = hi - k0 - 4 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          sc[0][qb][r] = off < lim ? sc[0][qb][r] : -INFINITY;
          sc[1][qb][r] = off + 32 < lim ? sc[1][qb][r] : -INFINITY;
        }
      }
    }
    // Exponents x = s c - m c in place (one FMA per score); a masked score
    // becomes -inf.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][qb][r] = fmaf(sc[kb][qb][r], c, -mc[qb]);
    float gap[2];  // the row's largest exponent in this tile
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) gap[qb] = half_swap_max(max32(sc[0][qb], sc[1][qb]));
    bool move[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) move[qb] = gap[qb] > kPivotUp;
    if (__builtin_amdgcn_ballot_w64(!seen[0] || !seen[1]) != 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        move[qb] = move[qb] || (gap[qb] < kPivotDown && gap[qb] > -INFINITY && !seen[qb]);
        seen[qb] = seen[qb] || gap[qb] > -INFINITY;  // after this tile the row holds a weight >= 2^-64
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (__builtin_amdgcn_ballot_w64(move[qb]) != 0) {
        // The pivot moves by gap: exponents shift down by it, O and l scale
        // by 2^-gap -- except on a downward move, which happens only while
        // l is 0 (nothing to rescale).
        const float shift = move[qb] ? gap[qb] : 0.f;
        const float alpha = shift > 0.f ? __builtin_amdgcn_exp2f(-shift) : 1.f;
        // Row sums: lanes 0..15 hold query n in register 0 and query n + 16
        // in register 1; the factor of query n + 16 comes from lane n + 16.
        const auto hi = __builtin_amdgcn_permlane16_swap(__float_as_uint(alpha), __float_as_uint(alpha), false, false);
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

  // Phases.  A phase p begins with this wave's share of the fills of
  // K(p + 5) and V(p + 5) into slot (p + 5) % 8 (tiles past the end read
  // real rows or zeros and are never used), and ends with a wait for this
  // wave's fills of four phases ago and a barrier, which publishes K(p + 1)
  // (and V(p - 1), filled two phases earlier still).  The slot of tile t
  // holds its K and its V; it is refilled only after the phase that last
  // read it (the P.V of tile t, at phase t + 2) has ended.
  // In the loop only the vector-role wave of each SIMD fills: 16 rows of
  // the K and V tiles each (rows 16 rg .. 16 rg + 15), issued with its
  // exponentials, while the matrix-role wave's LDS reads run undisturbed by
  // its own fill instructions.  Called in every phase, it fills only in the
  // wave's vector phases (VROLE).
  const int lrow = 16 * rg + (lane >> 3);
  const uint32_t koff_a = (uint32_t)lrow * kRowBytes + 16u * (uint32_t)(fpos ^ k_swz(lrow));
  const uint32_t koff_b = (uint32_t)(lrow + 8) * kRowBytes + 16u * (uint32_t)(fpos ^ k_swz(lrow + 8));
  const uint32_t voff_a = (uint32_t)lrow * kRowBytes + 16u * (uint32_t)(fpos ^ (2 * (lrow & 3)));
  auto fills = [&](auto j_tag, int p, auto vrole_tag) __attribute__((always_inline)) {
    constexpr int J = decltype(j_tag)::value;
    if constexpr (decltype(vrole_tag)::value) {
      constexpr int SF = (J + kAhead) % kSlots;
      const uint32_t toff = (uint32_t)(p + kAhead) * kTileBytes;
      const uint32_t kdst = ring_addr(SF) + 2048u * rg, vdst = ring_addr(kSlots + SF) + 2048u * rg;
      lds_fill16_at(rk, kdst, toff + koff_a);
      lds_fill16_at(rk, kdst + 1024u, toff + koff_b);
      lds_fill16_at(rv, vdst, toff + voff_a);
      lds_fill16_at(rv, vdst + 1024u, toff + voff_a + 1024u);
    }
  };
  auto sync = [&](auto vrole_tag) __attribute__((always_inline)) {
    // A wave fills in every second phase.  After its vector phase p, the
    // fills of phases p and p - 2 may fly (vmcnt(8)): the tile read at
    // phase p + 1 was filled at phase p - 4.  After a matrix phase,
    // vmcnt(6), which also covers the prologue: its ten fills per wave
    // (tiles 0 .. 4, filled by all waves) must land tile by tile over the
    // first phases.
    if constexpr (decltype(vrole_tag)::value) __builtin_amdgcn_s_waitcnt(0x0F70 | 8);
    else __builtin_amdgcn_s_waitcnt(0x0F70 | 6);
    barrier_lds();
  };
  // MFMA phase at phase p (slot J = p % 8): P.V of tile p - 2, then S of
  // tile p.  It runs unconditionally, so the phase is one straight block:
  // before a wave's first tile and past its last one the weights are zero
  // and the V slot holds finite values (zeroed at start, or a tile read
  // through the range check), so P.V adds exact zeros; scores of a tile
  // past the end are never turned into weights.  V reads of key steps 0-2
  // go out first, each P.V step issues the next reads before its products,
  // and the K reads go out during the last P.V steps, arriving before S
  // needs them.  All of P.V comes before any of S: the weights and V
  // fragments die before the scores are born.
  auto mphase = [&](auto j_tag) __attribute__((always_inline)) {
    constexpr int J = decltype(j_tag)::value;
    using SV = std::integral_constant<int, (J + kSlots - 2) % kSlots>;
    using SK = std::integral_constant<int, J>;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    __builtin_amdgcn_s_setprio(1);
    bf16x8 va[2][4], ka[2][4];
    load_v_step(SV(), I0(), va);
    load_v_step(SV(), I1(), va);
    load_v_step(SV(), I2(), va);
    __builtin_amdgcn_sched_barrier(0);
    pv_step(I0(), va);
    __builtin_amdgcn_sched_barrier(0);
    load_v_step(SV(), I3(), va);
    __builtin_amdgcn_sched_barrier(0);
    pv_step(I1(), va);
    __builtin_amdgcn_sched_barrier(0);
    load_k_step(SK(), I0(), ka);
    load_k_step(SK(), I1(), ka);
    __builtin_amdgcn_sched_barrier(0);
    pv_step(I2(), va);
    __builtin_amdgcn_sched_barrier(0);
    load_k_step(SK(), I2(), ka);
    load_k_step(SK(), I3(), ka);
    __builtin_amdgcn_sched_barrier(0);
    pv_step(I3(), va);
    __builtin_amdgcn_sched_barrier(0);
    qk_smajor(ka);
    __builtin_amdgcn_s_setprio(0);
  };
  // Weights of tile t under the fixed pivot 0 (the first pass): the same
  // masks, then x = s c and 2^x straight away -- no row maxima, no pivot
  // checks.  Whether the pivot was safe for every row is decided once, from
  // the row sums at the end (the range check after the loop).
  auto softmax_fixed = [&](int t) __attribute__((always_inline)) {
    const int k0 = t * kBN;
    const bool need_mask = (k0 + kBN > kv_lim) || (CAUSAL && k0 + kBN - 1 > qw0);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qi = qw0 + 32 * qb + ln;
        int hi = kv_lim;
        if (CAUSAL) hi = min(hi, qi + 1);
        const int lim = hi - k0 - 4 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          sc[0][qb][r] = off < lim ? sc[0][qb][r] : -INFINITY;
          sc[1][qb][r] = off + 32 < lim ? sc[1][qb][r] : -INFINITY;
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][qb][r] *= c;
      exp_pack(sc[0][qb], sc[1][qb], pk[qb]);
    }
  };
  // Vector phase of tile t: the weights of tile t, or zero weights for a
  // phase before this wave's first tile or past its last.
  auto vphase = [&](int t) __attribute__((always_inline)) {
    if (t >= 0 && t < wave_tiles) {
      softmax_fixed(t);
    } else {
      // Zeros written from inline assembly: a plain 0 here is a constant
      // the compiler materialises before the branch, in every phase.
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("v_mov_b32 %0, 0" : "=v"(pk[qb][i]));
    }
  };
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using J3 = std::integral_constant<int, 3>;
  using J4 = std::integral_constant<int, 4>;
  using J5 = std::integral_constant<int, 5>;
  using J6 = std::integral_constant<int, 6>;
  using J7 = std::integral_constant<int, 7>;

  if (n_tiles > 0) {
    // Prologue: this row group's 64 Q rows (the wave of parity p fills rows
    // 32 p .. 32 p + 31, in a K tile's layout) into a slot the ring first
    // fills at phase 0 or later -- K 5, 6, 7 or V 5 -- then tiles 0 .. 4 (K
    // and V) as if filled at phases -5 .. -1.  Q lands first, so the first
    // products wait for Q and tile 0 together, not one after the other.
    const uint32_t qdst = ring_addr(rg < 3 ? 5 + rg : kSlots + 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * par + 8 * i + (lane >> 3);
      lds_fill16_at(rq, qdst + 4096u * par + 1024u * i,
                    (uint32_t)(qw0 + r) * kRowBytes + 16u * (uint32_t)(fpos ^ k_swz(r)));
    }
    fill_k(J0(), 0);
    fill_v(J0(), 0);
    fill_k(J1(), 1);
    fill_v(J1(), 1);
    fill_k(J2(), 2);
    fill_v(J2(), 2);
    fill_k(J3(), 3);
    fill_v(J3(), 3);
    fill_k(J4(), 4);
    fill_v(J4(), 4);
    // The first MFMA phases of the two waves of a pair (p = 0, 1) read the
    // V tiles of slots 6 and 7 with zero weights: zero them, since 0 * NaN
    // of stale LDS contents would not be zero.
    g_ring[kSlots + 6][tid] = make_uint4(0, 0, 0, 0);
    g_ring[kSlots + 7][tid] = make_uint4(0, 0, 0, 0);
    // vmcnt(10): this wave's Q fills have landed; after the barrier, the
    // pair's.
    __builtin_amdgcn_s_waitcnt(0x0F70 | 10);
    barrier_lds();
    {
      const lds_uint4* qs = (const lds_uint4*)(uintptr_t)qdst;
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
    }
    // vmcnt(8) (tile 0 has landed), lgkmcnt(0): Q is in registers, and its
    // slots may be refilled after this barrier.
    __builtin_amdgcn_s_waitcnt(0x0070 | 8);
    barrier_lds();
    // Even-tile waves run MFMA phases at even p, odd-tile waves at odd p;
    // both run the same number of phases (and barriers).
    const int n_phases = n_tiles + 2;
    using M = std::false_type;  // matrix phase: no fills
    using F = std::true_type;   // vector phase: this wave fills
    if (par == 0) {
#pragma nounroll
      for (int p = 0; p < n_phases; p += 8) {
        mphase(J0());                            sync(M());
        fills(J1(), p + 1, F()); vphase(p);       sync(F());
        if (p + 2 >= n_phases) break;
        mphase(J2());                            sync(M());
        fills(J3(), p + 3, F()); vphase(p + 2);   sync(F());
        if (p + 4 >= n_phases) break;
        mphase(J4());                            sync(M());
        fills(J5(), p + 5, F()); vphase(p + 4);   sync(F());
        if (p + 6 >= n_phases) break;
        mphase(J6());                            sync(M());
        fills(J7(), p + 7, F()); vphase(p + 6);   sync(F());
      }
    } else {
#pragma nounroll
      for (int p = 0; p < n_phases; p += 8) {
        fills(J0(), p, F());     vphase(p - 1);   sync(F());
        mphase(J1());                            sync(M());
        if (p + 2 >= n_phases) break;
        fills(J2(), p + 2, F()); vphase(p + 1);   sync(F());
        mphase(J3());                            sync(M());
        if (p + 4 >= n_phases) break;
        fills(J4(), p + 4, F()); vphase(p + 3);   sync(F());
        mphase(J5());                            sync(M());
        if (p + 6 >= n_phases) break;
        fills(J6(), p + 6, F()); vphase(p + 5);   sync(F());
        mphase(J7());                            sync(M());
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70 | 0);  // no fill may land in the merge area
    barrier_lds();
  }

  // ---- merge the pair: the odd-tile wave hands (O, l, m) to its partner
  // through LDS.  Eight 8 KB tiles (64 KB) hold O as 16 vec4 groups
  // ([d block][query block][register / 4]) x 4 row groups x 64 lanes; group
  // vg sits in tile vg / 2, so every index is a compile-time tile.
  auto mptr = [&](auto vg_tag) __attribute__((always_inline)) -> float4* {
    constexpr int VG = decltype(vg_tag)::value;
    return reinterpret_cast<float4*>(mslot<VG / 2>()) + ((VG & 1) * 4 + rg) * 64 + lane;
  };
  // Full row sums in the row layout: lane (ln, hh) takes query ln's sum from
  // lane ln % 16, register ln / 16.
  float l[2];
  auto row_sums = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float v0 = __int_as_float(__builtin_amdgcn_ds_bpermute((lane & 15) * 4, __float_as_int(ls[qb][0])));
      const float v1 = __int_as_float(__builtin_amdgcn_ds_bpermute((lane & 15) * 4, __float_as_int(ls[qb][1])));
      l[qb] = (ln < 16) ? v0 : v1;
    }
  };
  // The odd-tile wave's (O, l, m) into the merge area.
  auto hand_over = [&]() __attribute__((always_inline)) {
    static_for<16>([&](auto vg_tag) {
      constexpr int VG = decltype(vg_tag)::value;
      constexpr int DB = VG / 8, QB = (VG / 4) % 2, R = 4 * (VG % 4);
      *mptr(vg_tag) = make_float4(o[DB][QB][R], o[DB][QB][R + 1], o[DB][QB][R + 2], o[DB][QB][R + 3]);
    });
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) g_lm[rg][qb][lane] = make_float2(l[qb], mc[qb]);
  };
  // The even-tile wave merges and stores:
  // O = (2^(mA - M) O_A + 2^(mB - M) O_B) / (2^(mA - M) l_A + 2^(mB - M) l_B)
  // with M = max(mA, mB); 2^0 = 1 exactly, and both pivots are finite.  Row
  // log-sum-exp (M + log2 l) ln 2; -inf for padded or keyless rows.
  // Register r of block (db, qb) holds d = 32 db + 8 (r / 4) + 4 hh + r % 4
  // of query row qw0 + 32 qb + ln: four consecutive d per 8-byte store;
  // padded rows and rows with no allowed key are written as exact zeros.
  // The output addresses are rebuilt from a fresh copy of the lane's row
  // index instead of being held in registers through the tile loop.
  auto merge_store = [&]() __attribute__((always_inline)) {
    float fa[2], fb[2], inv[2];
    bool live[2];
    int ln_e = ln;
    asm volatile("" : "+v"(ln_e));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float2 lm = g_lm[rg][qb][lane];
      const bool ea = l[qb] > 0.f, eb = lm.x > 0.f;
      const float M = ea ? (eb ? fmaxf(mc[qb], lm.y) : mc[qb]) : lm.y;
      fa[qb] = ea ? __builtin_amdgcn_exp2f(mc[qb] - M) : 0.f;
      fb[qb] = eb ? __builtin_amdgcn_exp2f(lm.y - M) : 0.f;
      const float l_row = fa[qb] * l[qb] + fb[qb] * lm.x;
      const int qi = qw0 + 32 * qb + ln_e;
      live[qb] = qi < q_len && l_row > 0.f;
      inv[qb] = live[qb] ? 1.f / l_row : 0.f;
      if (a.lse && hh == 0 && qi < a.n_q)
        a.lse[(size_t)bh * a.n_q + qi] = live[qb] ? (M + __builtin_amdgcn_logf(l_row)) * kLn2 : -INFINITY;
    }
    static_for<16>([&](auto vg_tag) {
      constexpr int VG = decltype(vg_tag)::value;
      constexpr int DB = VG / 8, QB = (VG / 4) % 2, G = VG % 4, R = 4 * G;
      const int qi = qw0 + 32 * QB + ln_e;
      const float4 ob = *mptr(vg_tag);
      const float x0 = (fa[QB] * o[DB][QB][R] + fb[QB] * ob.x) * inv[QB];
      const float x1 = (fa[QB] * o[DB][QB][R + 1] + fb[QB] * ob.y) * inv[QB];
      const float x2 = (fa[QB] * o[DB][QB][R + 2] + fb[QB] * ob.z) * inv[QB];
      const float x3 = (fa[QB] * o[DB][QB][R + 3] + fb[QB] * ob.w) * inv[QB];
      if (qi < a.n_q) {
        uint2 w;
        w.x = live[QB] ? pack_bf16x2(x0, x1) : 0u;
        w.y = live[QB] ? pack_bf16x2(x2, x3) : 0u;
        *reinterpret_cast<uint2*>(O + (size_t)qi * kHeadDim + 32 * DB + 8 * G + 4 * hh) = w;
      }
    });
  };

  row_sums();
  if (par == 1) hand_over();
  __syncthreads();
  if (par == 0) {
    // Range check of the fixed pivot.  Under pivot 0 every weight of a row
    // is at most its sum l, so l_A, l_B < 2^64 bounds every weight, partial
    // sum and product below fp32 overflow (a weight of 2^128 or more shows
    // as l = inf, NaN as a NaN sum).  l_A + l_B >= 2^-32 puts the row's
    // largest weight at 2^-56 or more (a row has fewer than 2^24 keys), so
    // a weight that fell into the subnormal range is below 2^-70 of it and
    // changes no result.  A row with an allowed key that fails either bound
    // -- logits far above 64 or far below -32 in log2 units -- sends its row
    // group to the moving-pivot recomputation below.  Rows without an
    // allowed key (padded, kv_len = 0) are zeros either way.  The bounds
    // come from a fresh copy of the lane's row index.
    int ln_c = ln;
    asm volatile("" : "+v"(ln_c));
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float2 lm = g_lm[rg][qb][lane];
      const int qi = qw0 + 32 * qb + ln_c;
      const bool keys = qi < q_len && kv_lim > 0;
      const bool in_range = l[qb] + lm.x >= 0x1p-32f && l[qb] < 0x1p64f && lm.x < 0x1p64f;
      bad = bad || (keys && !in_range);
    }
    // The ballot with every lane active (inside the lane-0 branch it would
    // see lane 0 alone).
    const bool group_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (lane == 0) g_bad[rg] = group_bad;
    // Stored whatever the check found: a row group that failed it stores
    // again below, over these rows (same wave, program order).  Storing
    // first lets the loop's accumulators die before the recomputation,
    // which would not fit the registers beside them.
    merge_store();
  }
  // Every verdict is in g_bad, and every merge-area read is done.
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  barrier_lds();
  if (__builtin_amdgcn_readfirstlane(g_bad[0] | g_bad[1] | g_bad[2] | g_bad[3]) == 0) return;

  // ---- some row group failed the range check: its two waves take their
  // tiles again (even, odd), under the moving pivot, one tile at a time
  // through ring slots `wave` (K) and 8 + `wave` (V), then merge as above.
  // The split, the order of the tiles and of the products, and the merge
  // are those of the pipeline, so a row whose pivot never moves gets the
  // same bits as there.  Each wave fills whole tiles itself; the
  // workgroup's barriers stay uniform (every wave passes them).
  const bool mine = __builtin_amdgcn_readfirstlane(g_bad[rg]) != 0;
  if (mine) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      mc[i] = 0.f;
      ls[i] = f32x4{};
      seen[i] = false;
#pragma unroll
      for (int j = 0; j < 2; ++j) o[i][j] = f32x16{};
    }
    const uint32_t kdst = ring_addr(wave), vdst = ring_addr(kSlots + wave);
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
#pragma nounroll
    for (int t = par; t < wave_tiles; t += 2) {
      // Fill offsets from a fresh copy of the lane index each tile: held
      // through the loop they would not fit the registers.
      int lf = lane;
      asm volatile("" : "+v"(lf));
      const int qrow = lf >> 3, fp = lf & 7;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * j + qrow;
        const uint32_t roff = (uint32_t)t * kTileBytes + (uint32_t)r * kRowBytes;
        lds_fill16_at(rk, kdst + 1024u * j, roff + 16u * (uint32_t)(fp ^ k_swz(r)));
        lds_fill16_at(rv, vdst + 1024u * j, roff + 16u * (uint32_t)(fp ^ (2 * (r & 3))));
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): both tiles have landed
      bf16x8 ka[2][4];
      load_k_at(kdst, I0(), ka);
      load_k_at(kdst, I1(), ka);
      load_k_at(kdst, I2(), ka);
      load_k_at(kdst, I3(), ka);
      qk_smajor(ka);
      softmax(t);
      bf16x8 va[2][4];
      load_v_at(vdst, I0(), va);
      load_v_at(vdst, I1(), va);
      load_v_at(vdst, I2(), va);
      load_v_at(vdst, I3(), va);
      pv_step(I0(), va);
      pv_step(I1(), va);
      pv_step(I2(), va);
      pv_step(I3(), va);
    }
    row_sums();
  }
  // The merge area overlaps the slots just used.
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  barrier_lds();
  if (mine && par == 1) hand_over();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  barrier_lds();
  if (mine && par == 0) merge_store();
}

}  // namespace

hipError_t launch_fwd_bf16_pair(const FwdArgs& a, hipStream_t s) {
  const int n_qt = (a.n_q + kBM - 1) / kBM;
  const long long blocks = (long long)n_qt * a.H * a.B;
  FwdArgs args = a;
  void* kargs[] = {&args};
  // Restricted attention runs on the band kernel.
  const int mode = fwd_mode(a);
  if (mode == kModeBand) return hipErrorInvalidValue;
  const void* fn = mode == kModeCausal ? reinterpret_cast<const void*>(&attn_fwd_bf16_pair_kernel<kModeCausal>)
                                       : reinterpret_cast<const void*>(&attn_fwd_bf16_pair_kernel<kModeNone>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), kargs, 0, s);
}

}  // namespace headattn
