// bf16 backward of attn_forward: dQ, dK, dV of O = softmax(Q K^T * scale +
// M) V given dO, from the saved per-row log-sum-exp (attn_forward_lse).  The
// pages train this sub-layer ("[논문 리뷰]Attention Is All You Need", §3.2.1
// defines the map; §5 trains the model); the gradients are those of the
// plain definition, row by row with weights p_ij = exp(s_ij - lse_i):
//   dV_j = sum_i p_ij dO_i          dp_ij = dO_i . V_j
//   ds_ij = p_ij (dp_ij - D_i),     D_i = dO_i . O_i = sum_j p_ij dp_ij
//   dQ_i = scale sum_j ds_ij K_j    dK_j = scale sum_i ds_ij Q_i
// The masks are the forward's: key padding, causal, and the band of
// restricted self-attention (§4, Table 1: keys i - radius .. i + radius, or
// i - radius .. i with the causal mask).
//
// Three kernels on the caller's stream:
//   bwd_rowdot:  per row, D_i = dO_i . O_i in fp32 and L_i = lse_i log2(e),
//                into the workspace; padded rows (and rows up to the next
//                multiple of 64) get D = 0 and L = +inf, i.e. weight 0;
//   bwd_dkdv:    key-major.  A workgroup owns 128 keys of one (b, h), 32 per
//                wave; query tiles of 64 rows (Q, dO, L, D) stream through
//                LDS.  Per tile a wave computes S = Q K^T and dP = dO V^T
//                with the keys on the lanes (its K and V fragments stay in
//                registers for the whole loop), forms P and dS in registers,
//                and accumulates dV^T += dO^T P and dK^T += Q^T dS with P and
//                dS as B operands straight from registers -- the A operands
//                dO^T and Q^T are read transposed from the tiles with
//                ds_read_b64_tr_b16, in the order the registers hold the
//                queries (the contraction order is free);
//   bwd_dq:      query-major, the forward's layout: a workgroup owns 128
//                query rows, key tiles stream through LDS, S^T = K Q^T and
//                dP^T = V dO^T put the queries on the lanes, and dQ^T +=
//                K^T dS^T takes dS^T from registers and K^T transposed from
//                the tile.  Three workgroups share a CU (at most 168 VGPRs,
//                3 x 51 KB of LDS): a third wave per SIMD covers the serial
//                chain of products and exponentials.  No atomics: every
//                output element has one owner, so the gradients are bitwise
//                reproducible.
// Long ranges (n_k >= 512 for dK/dV, n_q >= 512 for dQ; no mask or causal)
// take the paired variants instead: 8-wave workgroups, one per CU, whose
// two waves on each SIMD alternate matrix and vector phases, as in the
// paired forward (each is described at its kernel).
//
// Streaming: tiles reach LDS by buffer loads that write LDS directly, into a
// ring of three slots, two tiles ahead of use; one barrier per tile both
// publishes the tile in use and frees the slot of the tile before it.  Rows
// at or beyond a valid length read as zero through the descriptor's range
// check, so padded memory is never read.  Workgroups of one head share an
// XCD (its L2 then serves the re-reads of that head's Q, dO or K, V), and
// under the causal mask the longest ones start first.
//
// Numerics: bf16 inputs, fp32 accumulation; P and dS are rounded to bf16
// once before their products; D from the bf16 O and dO in fp32.  An
// excluded key has p = 0 and gets no gradient; padded query rows read as
// zero rows with L = +inf, so they contribute nothing.
#include <type_traits>

#include "kernel_util.h"

namespace headattn {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;   // rows per streamed tile
constexpr int kSlots = 3;   // LDS ring: the tile in use and two in flight

// A streamed 64-row tile in LDS: row-major, 16-byte chunk c of row r at
// position c ^ swz(r), swz(r) = 2 (r % 4) ^ (r / 4) % 4.  Row reads (16
// bytes per lane, lanes on consecutive rows, 16 lanes served together) and
// transposed reads (four rows from a multiple of 4, adjacent chunks) then
// spread over all banks: 16 consecutive rows of one chunk take 8 positions
// in each row parity (rows r and r + 8, 1 KB apart and so on the same
// banks, no longer share them), and a transposed read's rows take distinct
// positions.
// Measured with SQ_LDS_BANK_CONFLICT on the dK/dV and dQ kernels: with
// 2 (r % 4), the layout the transposed reads first had, every row read was
// 2-way conflicted; 2 (r % 4) + (r / 4) % 2 removed two thirds of the
// conflict cycles, and this layout the rest.
struct Tile {
  uint4 c[kTile * 8];
};

__device__ __forceinline__ int swz(int r) { return (2 * (r & 3)) ^ ((r >> 2) & 3); }

// Fill rows [r0, r0 + 64) of a [rows][64] bf16 tensor into t; rows at or
// beyond the descriptor's range read as zero.  256 threads, 2 instructions
// per wave.
__device__ __forceinline__ void fill_tile(Tile& t, __amdgpu_buffer_rsrc_t r, int r0, int wave, int lane) {
  // The tile's LDS byte address as an integer (a generic pointer here would
  // be kept in registers and converted back, with a null check, per fill).
  const uint32_t base = (uint32_t)(uintptr_t)(lds_void_t*)&t.c[0];
  const int fpos = lane & 7;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 32 * half + 8 * wave + (lane >> 3);
    const uint32_t off = (uint32_t)(r0 + row) * kRowBytes + 16u * (uint32_t)(fpos ^ swz(row));
    lds_fill16_at(r, base + 16u * (uint32_t)(256 * half + 64 * wave), off);
  }
}

// Row fragment: lane (ln, hh) gets row `row`, d 16 s + 8 hh .. + 7.
__device__ __forceinline__ bf16x8 row_frag(const Tile& t, int row, int s, int hh) {
  return __builtin_bit_cast(bf16x8, t.c[row * 8 + ((2 * s + hh) ^ swz(row))]);
}

// Transposed fragment (A operand of X^T[d][r] times registers holding rows
// in accumulator order): for d block db and 16-row step j, lane (ln, hh)
// gets d = 32 db + ln and rows 16 j + {0..3, 8..11} + 4 hh -- the rows that
// registers 8 (j % 2) .. + 7 of a 32-row accumulator block hold.  Two
// transposed reads of 4 rows each: lane i of 16-lane group g names row kr
// and 8-byte chunk h; the read returns to lane i the 4 rows kr - i/4 .. +3
// of d = dbase + i.
__device__ __forceinline__ bf16x8 tr_frag(const Tile& t, int db, int j, int lane) {
  // swz depends on the row mod 16 only, so the 16-row step j is a plain
  // offset and the per-lane part is shared by every j.
  const char* base = reinterpret_cast<const char*>(t.c) + 16 * j * (int)kRowBytes;
  const int g = lane >> 4;
  const int i = lane & 15;
  s16x4 part[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int kr = 8 * x + 4 * (g >> 1) + (i >> 2);  // row within the step
    const int h = 8 * db + 4 * (g & 1) + (i & 3);
    const int byte = kr * (int)kRowBytes + 16 * ((h >> 1) ^ swz(kr)) + 8 * (h & 1);
    part[x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + byte));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Ring slots (fills issued with lds_fill16, ordered by the ring's own
// waits).  The dK/dV kernel streams Q (a), dO (b) and L, D (ld); the dQ kernel K (a) and
// V (b).  Per ld slot: L of the tile's 64 rows in floats 0..63, D in
// 64..127; the buffer load that fills them writes 1 KB, the rest is a
// landing area.
struct Slot {
  Tile a, b;
  float4 ld[64];
};
__shared__ Slot g_s0, g_s1, g_s2;

template <int S>
__device__ __forceinline__ Slot& slot() {
  return S == 0 ? g_s0 : S == 1 ? g_s1 : g_s2;
}
template <int S>
__device__ __forceinline__ Tile& aslot() {
  return slot<S>().a;
}
template <int S>
__device__ __forceinline__ Tile& bslot() {
  return slot<S>().b;
}
template <int S>
__device__ __forceinline__ float4* ldslot() {
  return slot<S>().ld;
}

// (b, h) of a workgroup and its block index along the owned axis.  The 8
// XCDs take workgroup ids round robin; when B*h divides by 8 each XCD gets
// whole heads.  Blocks of equal rank run together, rank 0 first; `reverse`
// gives rank 0 to the last block.
__device__ __forceinline__ void bh_block(int bid, int n_blocks, int HB, bool reverse, int& bh, int& blk) {
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
  blk = reverse ? n_blocks - 1 - rank : rank;
}

// Wait until at most N of this wave's buffer loads are outstanding and all
// its LDS operations are done, then the workgroup barrier -- a bare
// s_barrier: a workgroup fence would add a wait for every fill in flight.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);  // vmcnt(N), lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

using Slot0 = std::integral_constant<int, 0>;
using Slot1 = std::integral_constant<int, 1>;
using Slot2 = std::integral_constant<int, 2>;

// x as hi + mid + lo, each rounded to the nearest bf16 (the sum is x to
// within 2^-24 |x|, about fp32's precision), packed as (hi, mid), (lo, 0).
__device__ __forceinline__ void split3_bf16(float x, uint32_t& w01, uint32_t& w23) {
  const uint32_t ph = pack_bf16x2(x, 0.f);
  const float r = x - __uint_as_float(ph << 16);
  const uint32_t pm = pack_bf16x2(r, 0.f);
  w01 = (ph & 0xFFFFu) | (pm << 16);
  w23 = pack_bf16x2(r - __uint_as_float(pm << 16), 0.f);
}

// ---------------------------------------------------------------- D, L = rowdot
__global__ __launch_bounds__(kThreads) void bwd_rowdot_kernel(BwdArgs a) {
  // 8 lanes per row, 16 bytes each: 32 rows per workgroup, over the padded
  // row range [0, n_pad) of each (b, h).
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  const int64_t rows = (int64_t)a.B * a.H * a.n_pad;
  float acc = 0.f;
  bool valid = false;
  int64_t src = 0;
  if (row < rows) {
    const int i = (int)(row % a.n_pad);
    const int64_t bh = row / a.n_pad;
    const int b = (int)(bh / a.H);
    const int q_len = a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q;
    valid = i < q_len;
    src = bh * a.n_q + i;
    if (valid) {
      const bf16x8 o = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.O) + src * kHeadDim + 8 * part);
      const bf16x8 g = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.dO) + src * kHeadDim + 8 * part);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    }
  }
  // Sum over the 8 lanes of the row (aligned groups of 8).
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && part == 0) {
    float l = INFINITY;  // weight exp2(s c - L) = 0
    if (valid) {
      const float v = a.lse[src];
      l = v == -INFINITY ? INFINITY : v * kLog2e;  // -inf: a row with no allowed key
    }
    a.D[row] = valid ? acc : 0.f;
    a.L[row] = l;
    // -L/c and -D as sums of three bf16 parts (for the paired dK/dV
    // kernel, which adds them inside its S and dP products); a row with L =
    // +inf gets -2^100, finite, so that its products with zero stay zero.
    const float c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-100f);
    const float lc = l == INFINITY ? -0x1p100f : -(l / c);
    uint32_t w[4];
    split3_bf16(lc, w[0], w[1]);
    split3_bf16(valid ? -acc : 0.f, w[2], w[3]);
    a.LD16[row] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---------------------------------------------------------------- dK, dV
template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr bool CAUSAL = MODE == kModeCausal;
  constexpr bool BAND = MODE == kModeBand;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hh = lane >> 5;

  const int n_kb = (a.n_k + 127) / 128;
  int bh, kb;
  bh_block(blockIdx.x, n_kb, a.B * a.H, false, bh, kb);
  const int b = bh / a.H;
  const int q_len = __builtin_amdgcn_readfirstlane(a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q);
  const int kv_lim = __builtin_amdgcn_readfirstlane(a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k);
  const int kb0 = kb * 128;
  const int kw0 = kb0 + 32 * wave;  // this wave's first key
  const int key = kw0 + ln;          // this lane's key
  // Restricted: query i sees keys i - wl .. i + wr, so key j is seen by
  // queries j - wr .. j + wl.
  const int wl = BAND ? a.radius : 0;
  const int wr = BAND ? (a.causal ? 0 : a.radius) : 0;

  const __bf16* Q = static_cast<const __bf16*>(a.Q) + (size_t)bh * a.n_q * kHeadDim;
  const __bf16* K = static_cast<const __bf16*>(a.K) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* V = static_cast<const __bf16*>(a.V) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* dO = static_cast<const __bf16*>(a.dO) + (size_t)bh * a.n_q * kHeadDim;

  // Query rows below q_len only: padded rows read as zeros.
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Q), (short)0, (int)((uint32_t)q_len * kRowBytes), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rdo =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(dO), (short)0, (int)((uint32_t)q_len * kRowBytes), kBufferWord3);
  // D then L, n_pad rows per (b, h) each, n_pad a multiple of 64, so a tile
  // never reaches the next head's rows.  Lanes 0..15 of wave 0 load 4 rows
  // of L each, lanes 16..31 4 rows of D; the other lanes read nothing (zeros
  // into the landing area).
  const uint32_t bhp = (uint32_t)a.B * a.H * a.n_pad;
  const __amdgpu_buffer_rsrc_t rld = __builtin_amdgcn_make_buffer_rsrc(a.D, (short)0, (int)(bhp * 8u), kBufferWord3);
  const uint32_t ld_base = lane < 16   ? (bhp + (uint32_t)bh * a.n_pad + 4u * lane) * 4u
                           : lane < 32 ? ((uint32_t)bh * a.n_pad + 4u * (lane - 16)) * 4u
                                       : kOutOfRange;

  // K and V fragments of this lane's key (B operands of S = Q K^T and
  // dP = dO V^T), for the whole loop; sign of scale folded into K.
  const uint32_t sign = a.scale < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-100f);
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;
    if (key < kv_lim) {
      kv = *reinterpret_cast<const uint4*>(K + (size_t)key * kHeadDim + 16 * s + 8 * hh);
      vv = *reinterpret_cast<const uint4*>(V + (size_t)key * kHeadDim + 16 * s + 8 * hh);
    }
    kv.x ^= sign;
    kv.y ^= sign;
    kv.z ^= sign;
    kv.w ^= sign;
    kf[s] = __builtin_bit_cast(bf16x8, kv);
    vf[s] = __builtin_bit_cast(bf16x8, vv);
  }

  f32x16 dk[2] = {f32x16{}, f32x16{}};  // dK^T [d block], column = key ln
  f32x16 dv[2] = {f32x16{}, f32x16{}};  // dV^T [d block]
  bool wave_live = kw0 < kv_lim;
  if (CAUSAL) wave_live = wave_live && kw0 < q_len;
  if (BAND) wave_live = wave_live && kw0 - wr < q_len;

  // Query tiles of the workgroup: [q_start, q_end) in steps of 64.
  int q_start = 0, q_end = q_len;
  if (CAUSAL) q_start = (kb0 / kTile) * kTile;
  if (BAND) {
    q_start = (max(0, kb0 - wr) / kTile) * kTile;
    q_end = min(q_end, kb0 + 128 + wl);
  }
  if (kb0 >= kv_lim) q_end = 0;  // no key of the block is valid: nothing to do
  const int n_tiles = q_end > q_start ? (q_end - q_start + kTile - 1) / kTile : 0;

  // Fill of tile u into slot S (= u % 3): Q and dO (2 + 2 loads per wave),
  // and from wave 0 one load of L and D.
  auto fill = [&](auto slot_tag, int u) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;
    const int q0 = q_start + u * kTile;
    fill_tile(aslot<S>(), rq, q0, wave, lane);
    fill_tile(bslot<S>(), rdo, q0, wave, lane);
    if (wave == 0) {
      const uint32_t off = ld_base == kOutOfRange ? kOutOfRange : ld_base + (uint32_t)q0 * 4u;
      lds_fill16_at(rld, (uint32_t)(uintptr_t)(lds_void_t*)ldslot<S>(), off);
    }
  };

  // One tile: S = u % 3 is its slot.  Tile u has landed (the only loads
  // allowed in flight are tile u + 1's) and every wave is done with tile
  // u - 1, whose slot tile u + 2 takes.
  auto step = [&](auto slot_tag, int u) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;
    using S2 = std::integral_constant<int, (S + 2) % kSlots>;
    if (u >= n_tiles) return;
    if (wave == 0) wait_barrier<5>();
    else wait_barrier<4>();
    fill(S2(), u + 2);

    const int q0 = q_start + u * kTile;
    // Does any query of the tile see any key of this wave?
    if (!wave_live) return;
    if (CAUSAL && q0 + kTile - 1 < kw0) return;
    if (BAND && (q0 + kTile - 1 < kw0 - wr || q0 > kw0 + 31 + wl)) return;
    const Tile& tq = aslot<S>();
    const Tile& tdo = bslot<S>();
    const float* tld = reinterpret_cast<const float*>(ldslot<S>());

    // S[q][key] and dP[q][key] for query blocks qb (32 rows each): lane
    // (ln, hh) register r holds query q0 + 32 qb + 8 (r / 4) + 4 hh + r % 4.
    f32x16 s_[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 sa = f32x16{}, pa = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(tq, 32 * qb + ln, s, hh), kf[s], sa, 0, 0, 0);
        pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(tdo, 32 * qb + ln, s, hh), vf[s], pa, 0, 0, 0);
      }
      s_[qb] = sa;
      dp[qb] = pa;
    }
    // P = exp2(s c - L) with the mask, dS = P (dP - D); both packed to
    // bf16 in the register order the k slots of the next products use.
    bool need_mask = (kw0 + 32 > kv_lim) || (CAUSAL && q0 < kw0 + 32);
    if (BAND) need_mask = need_mask || !(q0 + kTile - 1 - wl <= kw0 && kw0 + 31 <= q0 + wr);
    // Masked scores become -inf (so P = 0) in a block of their own, taken
    // only by tiles that cross an edge.  The compiler turned the test into
    // selects on every tile (inside the exponential loop, and as a separate
    // block too); the empty volatile statement keeps the block a branch.
    if (need_mask) {
      asm volatile("");
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = q0 + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
          bool ok = key < kv_lim;
          if (CAUSAL) ok = ok && key <= qi;
          if (BAND) ok = ok && key >= qi - wl && key <= qi + wr;
          s_[qb][r] = ok ? s_[qb][r] : -INFINITY;
        }
    }
    uint32_t pp[16], ps[16];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int ql = 32 * qb + 8 * gq + 4 * hh;  // first of this group's 4 queries
        const float4 l4 = *reinterpret_cast<const float4*>(&tld[ql]);
        const float4 d4 = *reinterpret_cast<const float4*>(&tld[kTile + ql]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dvv[4] = {d4.x, d4.y, d4.z, d4.w};
        float p[4], g[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * gq + e;
          // -inf for a masked key (c > 0); L = +inf gives 0 for padded rows
          const float x = fmaf(s_[qb][r], c, -lv[e]);
          p[e] = __builtin_amdgcn_exp2f(x);
          g[e] = p[e] * (dp[qb][r] - dvv[e]);
        }
        pp[8 * qb + 2 * gq] = pack_bf16x2(p[0], p[1]);
        pp[8 * qb + 2 * gq + 1] = pack_bf16x2(p[2], p[3]);
        ps[8 * qb + 2 * gq] = pack_bf16x2(g[0], g[1]);
        ps[8 * qb + 2 * gq + 1] = pack_bf16x2(g[2], g[3]);
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the tile's 4 steps of 16
    // queries: step j uses registers 8 (j % 2) .. + 7 of query block j / 2.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pp[4 * j], pp[4 * j + 1], pp[4 * j + 2], pp[4 * j + 3]));
      const bf16x8 sb = __builtin_bit_cast(bf16x8, make_uint4(ps[4 * j], ps[4 * j + 1], ps[4 * j + 2], ps[4 * j + 3]));
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(tdo, db, j, lane), pb, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(tq, db, j, lane), sb, dk[db], 0, 0, 0);
      }
    }
  };

  if (n_tiles > 0) {
    fill(Slot0(), 0);
    fill(Slot1(), 1);
    // Everything issued so far has landed: the register fragments loaded
    // above, and the first two tiles.  (The compiler does not see the fills;
    // without this wait it would re-wait for its own loads inside the loop
    // with a vmcnt(0) that also drains the ring.)
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    for (int u = 0; u < n_tiles; u += kSlots) {
      step(Slot0(), u);
      step(Slot1(), u + 1);
      step(Slot2(), u + 2);
    }
    // The last two fills (past the end: zeros, never read) land before the
    // workgroup's LDS is released.
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0)
  }

  // ---- store: register r of block db holds d = 32 db + 8 (r / 4) + 4 hh +
  // r % 4 of key ln.  The sign of scale sits in K', and Q entered the dK
  // product as is, so dK = scale * sum ds Q.
  if (key < a.n_k) {
    __bf16* dKr = static_cast<__bf16*>(a.dK) + ((size_t)bh * a.n_k + key) * kHeadDim;
    __bf16* dVr = static_cast<__bf16*>(a.dV) + ((size_t)bh * a.n_k + key) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int d = 32 * db + 8 * gg + 4 * hh;
        uint2 wk, wv;
        wk.x = pack_bf16x2(dk[db][4 * gg] * a.scale, dk[db][4 * gg + 1] * a.scale);
        wk.y = pack_bf16x2(dk[db][4 * gg + 2] * a.scale, dk[db][4 * gg + 3] * a.scale);
        wv.x = pack_bf16x2(dv[db][4 * gg], dv[db][4 * gg + 1]);
        wv.y = pack_bf16x2(dv[db][4 * gg + 2], dv[db][4 * gg + 3]);
        *reinterpret_cast<uint2*>(dKr + d) = wk;
        *reinterpret_cast<uint2*>(dVr + d) = wv;
      }
  }
}

// ---------------------------------------------------------------- dQ
template <int MODE>
__global__ __launch_bounds__(kThreads, 3) void bwd_dq_kernel(BwdArgs a) {
  constexpr bool CAUSAL = MODE == kModeCausal;
  constexpr bool BAND = MODE == kModeBand;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hh = lane >> 5;

  const int n_qb = (a.n_q + 127) / 128;
  int bh, qblk;
  bh_block(blockIdx.x, n_qb, a.B * a.H, CAUSAL, bh, qblk);
  const int b = bh / a.H;
  const int q_len = __builtin_amdgcn_readfirstlane(a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q);
  const int kv_lim = __builtin_amdgcn_readfirstlane(a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k);
  const int q0 = qblk * 128;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + ln;
  const int wl = BAND ? a.radius : 0;
  const int wr = BAND ? (a.causal ? 0 : a.radius) : 0;

  const __bf16* Q = static_cast<const __bf16*>(a.Q) + (size_t)bh * a.n_q * kHeadDim;
  const __bf16* K = static_cast<const __bf16*>(a.K) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* V = static_cast<const __bf16*>(a.V) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* dO = static_cast<const __bf16*>(a.dO) + (size_t)bh * a.n_q * kHeadDim;

  // Q and dO fragments of this lane's query (B operands of S^T = K Q^T and
  // dP^T = V dO^T), sign of scale folded into Q; zero for padded rows.
  const uint32_t sign = a.scale < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-100f);
  const bool row_live = qi < q_len;
  bf16x8 qf[4], gf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 qv = make_uint4(0, 0, 0, 0), gv = qv;
    if (row_live) {
      qv = *reinterpret_cast<const uint4*>(Q + (size_t)qi * kHeadDim + 16 * s + 8 * hh);
      gv = *reinterpret_cast<const uint4*>(dO + (size_t)qi * kHeadDim + 16 * s + 8 * hh);
    }
    qv.x ^= sign;
    qv.y ^= sign;
    qv.z ^= sign;
    qv.w ^= sign;
    qf[s] = __builtin_bit_cast(bf16x8, qv);
    gf[s] = __builtin_bit_cast(bf16x8, gv);
  }
  // L and D of this row (rows below n_pad exist for every qi < n_q).
  float lrow = INFINITY, dval = 0.f;
  if (qi < a.n_q) {
    lrow = a.L[(size_t)bh * a.n_pad + qi];
    dval = a.D[(size_t)bh * a.n_pad + qi];
  }

  f32x16 dq[2] = {f32x16{}, f32x16{}};  // dQ^T [d block], column = query ln
  // Key tiles of the workgroup: [k_start, end) in steps of 64.
  int k_start = 0, end = kv_lim;
  if (CAUSAL) end = min(end, q0 + 128);
  if (BAND) {
    k_start = (max(0, q0 - wl) / kTile) * kTile;
    end = min(end, q0 + 128 + wr);
  }
  if (q0 >= q_len) end = 0;
  const int n_tiles = end > k_start ? (end - k_start + kTile - 1) / kTile : 0;
  // The descriptors end at the last key the workgroup may use (never past
  // kv_len): the ring's fills past its last tile read zeros without touching
  // memory.
  const uint32_t k_bytes = (uint32_t)max(0, end) * kRowBytes;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(K), (short)0, (int)k_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(V), (short)0, (int)k_bytes, kBufferWord3);
  // Keys this wave needs: [wave_start, wave_end).
  int wave_start = 0, wave_end = end;
  if (CAUSAL) wave_end = min(wave_end, qw0 + 32);
  if (BAND) {
    wave_start = max(0, qw0 - wl);
    wave_end = min(wave_end, qw0 + 32 + wr);
  }
  if (qw0 >= q_len) wave_end = 0;

  // Fill of tile u into slot S (= u % 3): K and V, 2 + 2 loads per wave.
  auto fill = [&](auto slot_tag, int u) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;
    const int k0 = k_start + u * kTile;
    fill_tile(aslot<S>(), rk, k0, wave, lane);
    fill_tile(bslot<S>(), rv, k0, wave, lane);
  };

  // One tile, as in the dK/dV kernel.
  auto step = [&](auto slot_tag, int u) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;
    using S2 = std::integral_constant<int, (S + 2) % kSlots>;
    if (u >= n_tiles) return;
    wait_barrier<4>();
    fill(S2(), u + 2);

    const int k0 = k_start + u * kTile;
    if (k0 >= wave_end || k0 + kTile <= wave_start) return;
    const Tile& tk = aslot<S>();
    const Tile& tv = bslot<S>();
    // S^T[key][q], dP^T[key][q] for key blocks kb: register r holds key
    // k0 + 32 kb + 8 (r / 4) + 4 hh + r % 4 of query ln.
    f32x16 st[2], dpt[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sa = f32x16{}, pa = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(tk, 32 * kb + ln, s, hh), qf[s], sa, 0, 0, 0);
        pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(tv, 32 * kb + ln, s, hh), gf[s], pa, 0, 0, 0);
      }
      st[kb] = sa;
      dpt[kb] = pa;
    }
    bool need_mask = (k0 + kTile > kv_lim) || (CAUSAL && k0 + kTile - 1 > qw0);
    if (BAND) need_mask = need_mask || (k0 + kTile - 1 > qw0 + wr) || (k0 < qw0 + 31 - wl);
    if (need_mask) {
      // Register r of key block kb holds key k0 + 32 kb + 4 hh + off(r),
      // off(r) = 8 (r / 4) + r % 4; it is allowed when lo <= off(r) < lim.
      int hi = kv_lim;
      if (CAUSAL) hi = min(hi, qi + 1);
      if (BAND) hi = min(hi, qi + wr + 1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int base = k0 + 32 * kb + 4 * hh;
        const int lim = hi - base;
        const int lo = BAND ? qi - wl - base : INT_MIN;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          st[kb][r] = (off < lim && off >= lo) ? st[kb][r] : -INFINITY;
        }
      }
    }
    uint32_t ps[16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r2 = 0; r2 < 8; ++r2) {
        float g[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * r2 + e;
          const float x = fmaf(st[kb][r], c, -lrow);  // -inf for a masked key (c > 0)
          const float p = __builtin_amdgcn_exp2f(x);
          g[e] = p * (dpt[kb][r] - dval);
        }
        ps[8 * kb + r2] = pack_bf16x2(g[0], g[1]);
      }
    // dQ^T += K^T dS^T: step j uses registers 8 (j % 2) .. + 7 of key block j / 2.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 sb = __builtin_bit_cast(bf16x8, make_uint4(ps[4 * j], ps[4 * j + 1], ps[4 * j + 2], ps[4 * j + 3]));
#pragma unroll
      for (int db = 0; db < 2; ++db)
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(tk, db, j, lane), sb, dq[db], 0, 0, 0);
    }
  };

  if (n_tiles > 0) {
    fill(Slot0(), 0);
    fill(Slot1(), 1);
    // Everything issued so far has landed: the register fragments loaded
    // above, and the first two tiles.  (The compiler does not see the fills;
    // without this wait it would re-wait for its own loads inside the loop
    // with a vmcnt(0) that also drains the ring.)
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    for (int u = 0; u < n_tiles; u += kSlots) {
      step(Slot0(), u);
      step(Slot1(), u + 1);
      step(Slot2(), u + 2);
    }
    // The last two fills (past the end: zeros, never read) land before the
    // workgroup's LDS is released.
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0)
  }

  // dQ = scale sum ds K: the sign of scale sits in Q', not in K, so apply
  // the whole scale here.  Padded rows are written as zeros.
  if (qi < a.n_q) {
    __bf16* dQr = static_cast<__bf16*>(a.dQ) + ((size_t)bh * a.n_q + qi) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int d = 32 * db + 8 * gg + 4 * hh;
        uint2 w;
        w.x = row_live ? pack_bf16x2(dq[db][4 * gg] * a.scale, dq[db][4 * gg + 1] * a.scale) : 0u;
        w.y = row_live ? pack_bf16x2(dq[db][4 * gg + 2] * a.scale, dq[db][4 * gg + 3] * a.scale) : 0u;
        *reinterpret_cast<uint2*>(dQr + d) = w;
      }
  }
}

// ---------------------------------------------------------------- dQ, paired
// For long unmasked or causal rows: 8 waves, 128 queries (32 per wave, query
// block qb = wave % 4), the two waves of a SIMD (qb and qb + 4) taking the
// even and the odd key tiles of the same rows.  The waves of a pair
// alternate roles each phase (the paired forward's structure): at phase p
// the wave of parity p % 2 runs its matrix work -- dQ^T += K^T dS^T of tile
// p - 2, then S^T and dP^T of tile p -- while its partner forms P and dS of
// tile p - 1 on the vector unit; a workgroup barrier closes each phase.
// K and V go through an 8-slot ring exactly as K and V do in the paired
// forward (the fills of phase p are tile p + 5, into the slot of tile p - 3;
// only vector-role waves fill in the loop).  Q, dO, L and D are staged in
// slots the ring first fills at phase 0 or later.  At the end the odd-tile
// wave hands its dQ to its partner through LDS, which adds and stores.
constexpr int kPairThreads = 512;
constexpr int kPairRing = 8;
__shared__ Tile g_prk[kPairRing], g_prv[kPairRing];
__shared__ float g_pld[256];  // L of the 128 queries, then D
__shared__ uint4 g_pag[128];  // the 128 queries' -L/c and -D bf16 parts

__device__ __forceinline__ uint32_t tile_addr(const Tile& t) {
  return (uint32_t)(uintptr_t)(lds_void_t*)&t.c[0];
}

template <int MODE>
__global__ __launch_bounds__(kPairThreads, 1) void bwd_dq_pair_kernel(BwdArgs a) {
  constexpr bool CAUSAL = MODE == kModeCausal;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hh = lane >> 5;
  const int qb = wave & 3;    // query block (waves qb and qb + 4 share a SIMD)
  const int par = wave >> 2;  // parity of the key tiles this wave takes

  const int n_qb = (a.n_q + 127) / 128;
  int bh, qblk;
  bh_block(blockIdx.x, n_qb, a.B * a.H, CAUSAL, bh, qblk);
  const int b = bh / a.H;
  const int q_len = __builtin_amdgcn_readfirstlane(a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q);
  const int kv_lim = __builtin_amdgcn_readfirstlane(a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k);
  const int q0 = qblk * 128;
  const int qw0 = q0 + 32 * qb;

  const __bf16* Q = static_cast<const __bf16*>(a.Q) + (size_t)bh * a.n_q * kHeadDim;
  const __bf16* K = static_cast<const __bf16*>(a.K) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* V = static_cast<const __bf16*>(a.V) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* dO = static_cast<const __bf16*>(a.dO) + (size_t)bh * a.n_q * kHeadDim;

  int end = kv_lim;  // keys the workgroup needs
  if (CAUSAL) end = min(end, q0 + 128);
  if (q0 >= q_len) end = 0;
  const int n_tiles = max(0, (end + kTile - 1) / kTile);
  int wave_end = end;  // keys this wave's rows need
  if (CAUSAL) wave_end = min(wave_end, qw0 + 32);
  if (qw0 >= q_len) wave_end = 0;
  const int wave_tiles = max(0, (wave_end + kTile - 1) / kTile);

  // Descriptors: K and V end at the workgroup's last key (fills past its
  // last tile read zeros); Q and dO at q_len (padded rows read as zeros).
  const uint32_t k_bytes = (uint32_t)max(0, end) * kRowBytes;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(K), (short)0, (int)k_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(V), (short)0, (int)k_bytes, kBufferWord3);
  const uint32_t q_bytes = (uint32_t)max(0, q_len) * kRowBytes;
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Q), (short)0, (int)q_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rdo =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(dO), (short)0, (int)q_bytes, kBufferWord3);

  const uint32_t sign = a.scale < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-100f);

  // ---- fills.  Prologue: wave w fills rows 8 w .. 8 w + 7 of a tile (one
  // instruction); loop: the vector-role wave of query block qb fills rows
  // 16 qb .. 16 qb + 15 of K and of V (two instructions each).  Lane l
  // writes position l % 8 of its row, which receives chunk (l % 8) ^ swz(row).
  const int fpos = lane & 7;
  auto fill_rows = [&](__amdgpu_buffer_rsrc_t r, const Tile& t, int r0, int row) __attribute__((always_inline)) {
    lds_fill16_at(r, tile_addr(t) + 128u * (uint32_t)(row - (lane >> 3)),
                  (uint32_t)(r0 + row) * kRowBytes + 16u * (uint32_t)(fpos ^ swz(row)));
  };
  auto fills = [&](auto j_tag, int p, auto vrole_tag) __attribute__((always_inline)) {
    constexpr int J = decltype(j_tag)::value;
    if constexpr (decltype(vrole_tag)::value) {
      constexpr int SF = (J + 5) % kPairRing;
      const int k0 = (p + 5) * kTile;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 16 * qb + 8 * i + (lane >> 3);
        fill_rows(rk, g_prk[SF], k0, row);
        fill_rows(rv, g_prv[SF], k0, row);
      }
    }
  };
  auto sync = [&](auto vrole_tag) __attribute__((always_inline)) {
    // As in the paired forward: after a vector phase the fills of that phase
    // and of two phases earlier may fly; after a matrix phase vmcnt(6),
    // which also lets the prologue's tile fills land tile by tile.
    if constexpr (decltype(vrole_tag)::value) __builtin_amdgcn_s_waitcnt(0x0F70 | 8);
    else __builtin_amdgcn_s_waitcnt(0x0F70 | 6);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  bf16x8 qf[4], gf[4];
  float lrow = INFINITY;
  f32x16 dq[2] = {f32x16{}, f32x16{}};  // dQ^T [d block], column = query ln
  f32x16 st[2], dpt[2];                 // S^T, dP^T of the current tile [key block]
  uint32_t ps[16];                      // dS^T of the last tile, bf16 pairs
  bf16x8 dparts;  // this lane's query row: -L/c and -D as bf16 parts (k slots 0-7)
#pragma unroll
  for (int i = 0; i < 16; ++i) ps[i] = 0u;

  // Matrix phase J (phase p = 8 k + J): dQ from tile p - 2's K (slot
  // (J + 6) % 8) and the dS formed at phase p - 1, then S^T and dP^T of
  // tile p (slot J).  It runs unconditionally: before a wave's first tile
  // and past its last one dS is zero, so dQ gains exact zeros.
  auto mphase = [&](auto j_tag) __attribute__((always_inline)) {
    constexpr int J = decltype(j_tag)::value;
    constexpr int SD = (J + kPairRing - 2) % kPairRing;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 sb = __builtin_bit_cast(bf16x8, make_uint4(ps[4 * j], ps[4 * j + 1], ps[4 * j + 2], ps[4 * j + 3]));
#pragma unroll
      for (int db = 0; db < 2; ++db)
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(g_prk[SD], db, j, lane), sb, dq[db], 0, 0, 0);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sa = f32x16{}, pa = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(g_prk[J], 32 * kb + ln, s, hh), qf[s], sa, 0, 0, 0);
        pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(g_prv[J], 32 * kb + ln, s, hh), gf[s], pa, 0, 0, 0);
      }
      st[kb] = sa;
      dpt[kb] = pa;
    }
    // -D of each query into dP^T: one more k step, A ones against the three
    // D parts in the first lane half (zeros in the second), B the queries'
    // parts (ones from an opaque copy of the lane half, built here rather
    // than held through the loop).
    {
      int hh_c = hh;
      asm volatile("" : "+v"(hh_c));
      const uint32_t e3 = hh_c ? 0u : 0x3F803F80u, e1 = hh_c ? 0u : 0x3F80u;  // bf16 1.0 pairs
      const bf16x8 one_d = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, e3, e1));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dpt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(one_d, dparts, dpt[kb], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Vector phase of tile t: P = exp2(s c - L) under the mask and dS = P (dP
  // - D) (dP arrives with -D added), packed to bf16 in the k order of the dQ
  // product; zeros for a phase before this wave's first tile or past its
  // last.
  auto vphase = [&](int t) __attribute__((always_inline)) {
    if (t >= 0 && t < wave_tiles) {
      const int k0 = t * kTile;
      const bool need_mask = (k0 + kTile > kv_lim) || (CAUSAL && k0 + kTile - 1 > qw0);
      if (need_mask) {
        int lnm = ln;
        asm volatile("" : "+v"(lnm));
        const int qi = qw0 + lnm;
        int hi = kv_lim;
        if (CAUSAL) hi = min(hi, qi + 1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int lim = hi - (k0 + 32 * kb + 4 * hh);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + (r & 3);
            st[kb][r] = off < lim ? st[kb][r] : -INFINITY;
          }
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r2 = 0; r2 < 8; ++r2) {
          float g[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 2 * r2 + e;
            const float x = fmaf(st[kb][r], c, -lrow);  // -inf for a masked key (c > 0)
            const float p = __builtin_amdgcn_exp2f(x);
            g[e] = p * dpt[kb][r];
          }
          ps[8 * kb + r2] = pack_bf16x2(g[0], g[1]);
        }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) asm volatile("v_mov_b32 %0, 0" : "=v"(ps[i]));
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
    // Prologue: Q rows 0-63 into K slot 5, 64-127 into K slot 6, dO rows
    // 0-63 into K slot 7, 64-127 into V slot 5; L and D of the 128 rows
    // (wave 0: lanes 0-31 L, lanes 32-63 D, 16 bytes each) and their bf16
    // parts (wave 0, two loads); then tiles 0-4 as if filled at phases -5
    // .. -1.
    {
      const int row = 8 * wave + (lane >> 3);  // 0..63
      fill_rows(rq, g_prk[5], q0, row);
      fill_rows(rq, g_prk[6], q0 + 64, row);
      fill_rows(rdo, g_prk[7], q0, row);
      fill_rows(rdo, g_prv[5], q0 + 64, row);
      if (wave == 0) {
        const uint32_t bhp = (uint32_t)a.B * a.H * a.n_pad;
        const __amdgpu_buffer_rsrc_t rld =
            __builtin_amdgcn_make_buffer_rsrc(a.D, (short)0, (int)(bhp * 8u), kBufferWord3);
        const uint32_t first = (uint32_t)bh * a.n_pad + (uint32_t)q0 + 4u * (uint32_t)(lane & 31);
        const uint32_t off = (lane < 32 ? bhp + first : first) * 4u;
        lds_fill16_at(rld, (uint32_t)(uintptr_t)(lds_void_t*)&g_pld[0], off);
        // The 128 rows' bf16 parts (16 bytes a row), two loads.
        const __amdgpu_buffer_rsrc_t rag =
            __builtin_amdgcn_make_buffer_rsrc(a.LD16, (short)0, (int)(bhp * 16u), kBufferWord3);
        const uint32_t ag0 = ((uint32_t)bh * a.n_pad + (uint32_t)q0 + (uint32_t)lane) * 16u;
        lds_fill16_at(rag, (uint32_t)(uintptr_t)(lds_void_t*)&g_pag[0], ag0);
        lds_fill16_at(rag, (uint32_t)(uintptr_t)(lds_void_t*)&g_pag[64], ag0 + 1024u);
      }
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        fill_rows(rk, g_prk[t], t * kTile, row);
        fill_rows(rv, g_prv[t], t * kTile, row);
      }
    }
    // vmcnt(8): the staging fills and tile 0 have landed; after the
    // barrier, every wave's share of them.
    __builtin_amdgcn_s_waitcnt(0x0F70 | 8);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    {
      const Tile& tq = qb < 2 ? g_prk[5] : g_prk[6];
      const Tile& tg = qb < 2 ? g_prk[7] : g_prv[5];
      const int row = 32 * (qb & 1) + ln;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 v = __builtin_bit_cast(uint4, tq.c[row * 8 + ((2 * s + hh) ^ swz(row))]);
        v.x ^= sign;
        v.y ^= sign;
        v.z ^= sign;
        v.w ^= sign;
        qf[s] = __builtin_bit_cast(bf16x8, v);
        gf[s] = row_frag(tg, row, s, hh);
      }
      // Rows at or beyond q_len have L = +inf (P = 0) from the row kernel.
      lrow = g_pld[32 * qb + ln];
      dparts = __builtin_bit_cast(bf16x8, g_pag[32 * qb + ln]);
      if (qw0 + ln >= a.n_q) lrow = INFINITY;
    }
    // The first matrix phases of the two waves of a pair (p = 0, 1) read K
    // slots 6 and 7 for dQ with dS = 0: their contents are finite (Q, dO
    // staged there) or zero-filled tiles, so the products add exact zeros.
    // vmcnt(8) keeps tile 0 landed; lgkmcnt(0): every staged value is in
    // registers before the slots are refilled.
    __builtin_amdgcn_s_waitcnt(0x0070 | 8);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const int n_phases = n_tiles + 2;
    using M = std::false_type;
    using F = std::true_type;
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
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0): no fill lands in the hand-over area
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- the odd-tile wave hands its dQ to its partner through the ring
  // (32 floats per lane: 8 KB per wave, K slot qb), which adds and stores
  // dQ = scale sum ds K (the sign of scale sits in Q').
  float4* hand = reinterpret_cast<float4*>(&g_prk[qb].c[0]);
  if (par == 1) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        hand[(4 * db + g4) * 64 + lane] = make_float4(dq[db][4 * g4], dq[db][4 * g4 + 1], dq[db][4 * g4 + 2], dq[db][4 * g4 + 3]);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __syncthreads();
  if (par == 0) {
    int lnm = ln;
    asm volatile("" : "+v"(lnm));
    const int qi = qw0 + lnm;
    if (qi < a.n_q) {
      const bool row_live = qi < q_len;
      __bf16* dQr = static_cast<__bf16*>(a.dQ) + ((size_t)bh * a.n_q + qi) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 o = hand[(4 * db + g4) * 64 + lane];
          const int d = 32 * db + 8 * g4 + 4 * hh;
          uint2 w;
          w.x = row_live ? pack_bf16x2((dq[db][4 * g4] + o.x) * a.scale, (dq[db][4 * g4 + 1] + o.y) * a.scale) : 0u;
          w.y = row_live ? pack_bf16x2((dq[db][4 * g4 + 2] + o.z) * a.scale, (dq[db][4 * g4 + 3] + o.w) * a.scale) : 0u;
          *reinterpret_cast<uint2*>(dQr + d) = w;
        }
    }
  }
}

// ---------------------------------------------------------------- dK, dV, paired
// For long unmasked or causal key ranges: 8 waves, 256 keys (32 per wave,
// wave w owns keys kb0 + 32 w ..), the two waves of a SIMD (w and w + 4)
// on different keys and the same query tiles, one phase apart.  Per tile a
// wave runs a matrix phase -- dV^T += dO^T P and dK^T += Q^T dS of the
// previous tile, then S and dP of this tile -- and a vector phase (P and dS
// of this tile); while one wave of a SIMD issues its products the other
// forms its weights, and a workgroup barrier closes each phase.  There is
// no key split, so nothing is merged at the end.
//
// Query tiles (Q, dO, and the rows' -L/c and -D parts) stream through a
// 4-slot ring: tile t sits in slot t % 4.  Waves 0-3 run tile u's matrix
// phase at phase 2u and its vector phase at 2u + 1; waves 4-7 one phase
// later.  Tile u is last read
// at phase 2u + 3 (the products of waves 4-7), so at phase 2v the slot of
// tile v - 2 takes tile v + 2, filled by waves 4-7 (their vector phase) and
// first read at phase 2v + 4.  Only waves 4-7 fill in the loop.  The Q and
// dO tiles of all four slots lie within 64 KB, so every fragment read is
// one per-lane offset plus an immediate, whatever the slot.
constexpr int kDkvRing = 4;
constexpr int kDkvThreads = 512;
struct QdoSlot {
  Tile a, b;
};
__shared__ QdoSlot g_dr[kDkvRing];
__shared__ uint4 g_aug[kDkvRing][64];  // per tile row: -L/c and -D parts

template <int MODE>
__global__ __launch_bounds__(kDkvThreads, 1) void bwd_dkdv_pair_kernel(BwdArgs a) {
  constexpr bool CAUSAL = MODE == kModeCausal;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hh = lane >> 5;
  const int par = wave >> 2;   // 0: matrix phase first; 1: one phase later, fills
  const int fw = wave & 3;     // this wave's quarter of a fill

  const int n_kb = (a.n_k + 255) / 256;
  int bh, kb;
  bh_block(blockIdx.x, n_kb, a.B * a.H, false, bh, kb);
  const int b = bh / a.H;
  const int q_len = __builtin_amdgcn_readfirstlane(a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q);
  const int kv_lim = __builtin_amdgcn_readfirstlane(a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k);
  const int kb0 = kb * 256;
  const int kw0 = kb0 + 32 * wave;  // this wave's first key
  const int key = kw0 + ln;          // this lane's key

  const __bf16* Q = static_cast<const __bf16*>(a.Q) + (size_t)bh * a.n_q * kHeadDim;
  const __bf16* K = static_cast<const __bf16*>(a.K) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* V = static_cast<const __bf16*>(a.V) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* dO = static_cast<const __bf16*>(a.dO) + (size_t)bh * a.n_q * kHeadDim;
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Q), (short)0, (int)((uint32_t)q_len * kRowBytes), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rdo =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(dO), (short)0, (int)((uint32_t)q_len * kRowBytes), kBufferWord3);
  // The rows' -L/c and -D parts (16 bytes a row, from the row kernel):
  // lane l of the filling wave loads row q0 + l of a tile.
  const uint32_t bhp = (uint32_t)a.B * a.H * a.n_pad;
  const __amdgpu_buffer_rsrc_t raug = __builtin_amdgcn_make_buffer_rsrc(a.LD16, (short)0, (int)(bhp * 16u), kBufferWord3);
  const uint32_t aug_base = ((uint32_t)bh * a.n_pad + (uint32_t)lane) * 16u;

  const uint32_t sign = a.scale < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-100f);
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;
    if (key < kv_lim) {
      kv = *reinterpret_cast<const uint4*>(K + (size_t)key * kHeadDim + 16 * s + 8 * hh);
      vv = *reinterpret_cast<const uint4*>(V + (size_t)key * kHeadDim + 16 * s + 8 * hh);
    }
    kv.x ^= sign;
    kv.y ^= sign;
    kv.z ^= sign;
    kv.w ^= sign;
    kf[s] = __builtin_bit_cast(bf16x8, kv);
    vf[s] = __builtin_bit_cast(bf16x8, vv);
  }

  f32x16 dk[2] = {f32x16{}, f32x16{}};  // dK^T [d block], column = key ln
  f32x16 dv[2] = {f32x16{}, f32x16{}};  // dV^T [d block]
  const int q_start = CAUSAL ? kb0 : 0;
  const int q_end = kb0 >= kv_lim ? 0 : q_len;
  const int n_tiles = q_end > q_start ? (q_end - q_start + kTile - 1) / kTile : 0;

  auto fill = [&](auto slot_tag, int u) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;
    const int q0 = q_start + u * kTile;
    fill_tile(g_dr[S].a, rq, q0, fw, lane);
    fill_tile(g_dr[S].b, rdo, q0, fw, lane);
    if (fw == 0) lds_fill16_at(raug, (uint32_t)(uintptr_t)(lds_void_t*)&g_aug[S][0], aug_base + (uint32_t)q0 * 16u);
  };
  // Phase ends.  Waves 0-3 have nothing in flight in the loop; waves 4-7
  // wait at the end of their matrix phases (phase 2t - 1) until tile t has
  // landed: the tile filled after it (t + 1) may still fly, 4 loads (5 for
  // the wave that also loads the rows' parts).
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto sync_fills = [&]() __attribute__((always_inline)) {
    if (fw == 0) wait_barrier<5>();
    else wait_barrier<4>();
  };

  f32x16 s_[2], dp[2];  // S and dP of the current tile [query block]
  uint32_t pp[16], ps[16];  // P and dS of the previous tile, bf16 pairs

  // Matrix phase of tile u in slot J: products of tile u - 1 (slot J - 1),
  // then S and dP of tile u.  Every phase runs in full, also for a wave
  // none of whose keys a tile's queries see (the mask zeroes its weights):
  // the pair's partner and the barrier set the phase's length anyway, and
  // values assigned on every path keep the compiler from holding the
  // previous tile's S, dP, P and dS through the loop.  S and dP of tile
  // n_tiles (the last phase) are computed and never used.
  // The fragment reads go out one step ahead of the products that use them
  // (sched_barrier fences), so at most two steps' fragments are in flight.
  auto mphase = [&](auto j_tag, int u) __attribute__((always_inline)) {
    constexpr int J = decltype(j_tag)::value;
    constexpr int SP = (J + kDkvRing - 1) % kDkvRing;
    __builtin_amdgcn_s_setprio(1);
    // The rows' -L/c and -D parts of tile u, read first: a row's 8 parts
    // (both lane halves read them).
    bf16x8 ag[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) ag[qb] = __builtin_bit_cast(bf16x8, g_aug[J][32 * qb + ln]);
    if (u > 0) {
      const Tile& tq = g_dr[SP].a;
      const Tile& tdo = g_dr[SP].b;
      bf16x8 fo[2][2], fq[2][2];  // [step parity][d block]: dO^T and Q^T
      auto read = [&](int j) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          fo[j & 1][db] = tr_frag(tdo, db, j, lane);
          fq[j & 1][db] = tr_frag(tq, db, j, lane);
        }
      };
      read(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < 3) read(j + 1);
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pp[4 * j], pp[4 * j + 1], pp[4 * j + 2], pp[4 * j + 3]));
        const bf16x8 sb = __builtin_bit_cast(bf16x8, make_uint4(ps[4 * j], ps[4 * j + 1], ps[4 * j + 2], ps[4 * j + 3]));
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fo[j & 1][db], pb, dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[j & 1][db], sb, dk[db], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    {
      const Tile& tq = g_dr[J].a;
      const Tile& tdo = g_dr[J].b;
      bf16x8 rq_[2][2], rd_[2][2];  // [step parity][d half of the step pair]
      // A first k step of 16 puts the rows' -L/c into S and -D into dP:
      // A operand the rows' parts, B operand ones against the L parts (or
      // the D parts) in the first lane half and zeros in the second (ones
      // from an opaque copy of the lane half, so that the compiler builds
      // them here rather than holding them through the loop).
      f32x16 sa[2], pa[2];
      {
        int hh_c = hh;
        asm volatile("" : "+v"(hh_c));
        const uint32_t e3 = hh_c ? 0u : 0x3F803F80u, e1 = hh_c ? 0u : 0x3F80u;  // bf16 1.0 pairs
        const bf16x8 one_l = __builtin_bit_cast(bf16x8, make_uint4(e3, e1, 0u, 0u));
        const bf16x8 one_d = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, e3, e1));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          sa[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag[qb], one_l, f32x16{}, 0, 0, 0);
          pa[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag[qb], one_d, f32x16{}, 0, 0, 0);
        }
      }
      // Step i = 2 qb + h covers query block qb, d steps 2h and 2h + 1.
      auto read = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          rq_[i & 1][e] = row_frag(tq, 32 * (i >> 1) + ln, 2 * (i & 1) + e, hh);
          rd_[i & 1][e] = row_frag(tdo, 32 * (i >> 1) + ln, 2 * (i & 1) + e, hh);
        }
      };
      read(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < 3) read(i + 1);
        __builtin_amdgcn_sched_barrier(0);
        const int qb = i >> 1;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int st = 2 * (i & 1) + e;
          sa[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rq_[i & 1][e], kf[st], sa[qb], 0, 0, 0);
          pa[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rd_[i & 1][e], vf[st], pa[qb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      s_[0] = sa[0];
      s_[1] = sa[1];
      dp[0] = pa[0];
      dp[1] = pa[1];
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Vector phase of tile u: P = exp2(s c - L) under the mask, dS = P (dP -
  // D), both packed to bf16 in the k order of the next phase's products
  // (s and dP arrive with -L/c and -D added by the matrix phase).
  auto vphase = [&](auto j_tag, int u) __attribute__((always_inline)) {
    constexpr int J = decltype(j_tag)::value;
    const int q0 = q_start + u * kTile;
    if ((kw0 + 32 > kv_lim) || (CAUSAL && q0 < kw0 + 32)) {
      asm volatile("");
      int ln_m = ln;
      asm volatile("" : "+v"(ln_m));
      const int key_m = kw0 + ln_m;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = q0 + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
          bool ok = key_m < kv_lim;
          if (CAUSAL) ok = ok && key_m <= qi;
          s_[qb][r] = ok ? s_[qb][r] : -INFINITY;
        }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float p[4], g[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * gq + e;
          p[e] = __builtin_amdgcn_exp2f(s_[qb][r] * c);  // -inf for a masked key (c > 0)
          g[e] = p[e] * dp[qb][r];
        }
        pp[8 * qb + 2 * gq] = pack_bf16x2(p[0], p[1]);
        pp[8 * qb + 2 * gq + 1] = pack_bf16x2(p[2], p[3]);
        ps[8 * qb + 2 * gq] = pack_bf16x2(g[0], g[1]);
        ps[8 * qb + 2 * gq + 1] = pack_bf16x2(g[2], g[3]);
      }
    }
  };
  using R0 = std::integral_constant<int, 0>;
  using R1 = std::integral_constant<int, 1>;
  using R2 = std::integral_constant<int, 2>;
  using R3 = std::integral_constant<int, 3>;

  if (n_tiles > 0) {
    // Prologue: tiles 0 and 1 from waves 0-3; they and the K and V
    // fragments land before the first phase.
    if (par == 0) {
      fill(R0(), 0);
      fill(R1(), 1);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // Phases 0 .. 2 n_tiles + 1.  Waves 0-3: matrix phase of tile u at 2u
    // (u = 0 .. n_tiles, the last one only the products of tile n_tiles -
    // 1), vector phase at 2u + 1, and one closing barrier.  Waves 4-7: at
    // 2u the fill of tile u + 2 and the vector phase of tile u - 1, at
    // 2u + 1 the matrix phase of tile u.
    if (par == 0) {
#pragma nounroll
      for (int u = 0;; u += kDkvRing) {
        mphase(R0(), u);     sync(); if (u >= n_tiles) break;
        vphase(R0(), u);     sync();
        mphase(R1(), u + 1); sync(); if (u + 1 >= n_tiles) break;
        vphase(R1(), u + 1); sync();
        mphase(R2(), u + 2); sync(); if (u + 2 >= n_tiles) break;
        vphase(R2(), u + 2); sync();
        mphase(R3(), u + 3); sync(); if (u + 3 >= n_tiles) break;
        vphase(R3(), u + 3); sync();
      }
      sync();
    } else {
      auto fill_ahead = [&](auto slot_tag, int u) __attribute__((always_inline)) {
        if (u + 2 < n_tiles) fill(slot_tag, u + 2);
      };
#pragma nounroll
      for (int u = 0;; u += kDkvRing) {
        fill_ahead(R2(), u);     if (u > 0) vphase(R3(), u - 1); sync();
        mphase(R0(), u);         sync_fills(); if (u >= n_tiles) break;
        fill_ahead(R3(), u + 1); vphase(R0(), u);     sync();
        mphase(R1(), u + 1);     sync_fills(); if (u + 1 >= n_tiles) break;
        fill_ahead(R0(), u + 2); vphase(R1(), u + 1); sync();
        mphase(R2(), u + 2);     sync_fills(); if (u + 2 >= n_tiles) break;
        fill_ahead(R1(), u + 3); vphase(R2(), u + 2); sync();
        mphase(R3(), u + 3);     sync_fills(); if (u + 3 >= n_tiles) break;
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): no fill in flight at exit
  }

  // Store, as in the 4-wave kernel: dK = scale sum ds Q (sign in K').
  int ln_s = ln;
  asm volatile("" : "+v"(ln_s));
  const int key_s = kw0 + ln_s;
  if (key_s < a.n_k) {
    __bf16* dKr = static_cast<__bf16*>(a.dK) + ((size_t)bh * a.n_k + key_s) * kHeadDim;
    __bf16* dVr = static_cast<__bf16*>(a.dV) + ((size_t)bh * a.n_k + key_s) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int d = 32 * db + 8 * gg + 4 * hh;
        uint2 wk, wv;
        wk.x = pack_bf16x2(dk[db][4 * gg] * a.scale, dk[db][4 * gg + 1] * a.scale);
        wk.y = pack_bf16x2(dk[db][4 * gg + 2] * a.scale, dk[db][4 * gg + 3] * a.scale);
        wv.x = pack_bf16x2(dv[db][4 * gg], dv[db][4 * gg + 1]);
        wv.y = pack_bf16x2(dv[db][4 * gg + 2], dv[db][4 * gg + 3]);
        *reinterpret_cast<uint2*>(dKr + d) = wk;
        *reinterpret_cast<uint2*>(dVr + d) = wv;
      }
  }
}

const void* dkdv_fn(int mode) {
  return mode == kModeBand     ? reinterpret_cast<const void*>(&bwd_dkdv_kernel<kModeBand>)
         : mode == kModeCausal ? reinterpret_cast<const void*>(&bwd_dkdv_kernel<kModeCausal>)
                               : reinterpret_cast<const void*>(&bwd_dkdv_kernel<kModeNone>);
}

const void* dq_fn(int mode) {
  return mode == kModeBand     ? reinterpret_cast<const void*>(&bwd_dq_kernel<kModeBand>)
         : mode == kModeCausal ? reinterpret_cast<const void*>(&bwd_dq_kernel<kModeCausal>)
                               : reinterpret_cast<const void*>(&bwd_dq_kernel<kModeNone>);
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t s) {
  BwdArgs args = a;
  void* kargs[] = {&args};
  const int mode = a.radius >= 0 ? kModeBand : (a.causal ? kModeCausal : kModeNone);
  const int64_t rows = (int64_t)a.B * a.H * a.n_pad;
  hipError_t e = hipSuccess;
  if (rows > 0) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_rowdot_kernel), dim3((unsigned)((rows + 31) / 32)),
                        dim3(kThreads), kargs, 0, s);
    if (e != hipSuccess) return e;
  }
  if (a.n_k > 0) {
    const int64_t blocks = (int64_t)((a.n_k + 127) / 128) * a.H * a.B;
    // Long unmasked or causal key ranges: the paired dK/dV kernel (8 waves,
    // 256 keys, one workgroup per CU).
    if (mode != kModeBand && a.n_k >= 512) {
      const void* fn = mode == kModeCausal ? reinterpret_cast<const void*>(&bwd_dkdv_pair_kernel<kModeCausal>)
                                           : reinterpret_cast<const void*>(&bwd_dkdv_pair_kernel<kModeNone>);
      e = hipLaunchKernel(fn, dim3((unsigned)((int64_t)((a.n_k + 255) / 256) * a.H * a.B)), dim3(kDkvThreads), kargs,
                          0, s);
    } else {
      e = hipLaunchKernel(dkdv_fn(mode), dim3((unsigned)blocks), dim3(kThreads), kargs, 0, s);
    }
    if (e != hipSuccess) return e;
  }
  if (a.n_q == 0) return hipSuccess;
  const int64_t blocks = (int64_t)((a.n_q + 127) / 128) * a.H * a.B;
  // Long unmasked or causal rows: the paired dQ kernel (8 waves, one
  // workgroup per CU); shorter ones and restricted attention keep the
  // 4-wave kernel, three workgroups per CU.
  if (mode != kModeBand && a.n_q >= 512) {
    const void* fn = mode == kModeCausal ? reinterpret_cast<const void*>(&bwd_dq_pair_kernel<kModeCausal>)
                                         : reinterpret_cast<const void*>(&bwd_dq_pair_kernel<kModeNone>);
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kPairThreads), kargs, 0, s);
  }
  return hipLaunchKernel(dq_fn(mode), dim3((unsigned)blocks), dim3(kThreads), kargs, 0, s);
}

}  // namespace headattn
