// bf16 backward of attn_forward: dQ, dK, dV of O = softmax(Q K^T * scale +
// M) V given dO, from the saved per-row log-sum-exp (attn_forward_lse).  The
// pages train this sub-layer ("[논문 리뷰]Attention Is All You Need", §3.2.1
// defines the map; §5 trains the model); the gradients are those of the
// plain definition, row by row with weights p_ij = exp(s_ij - lse_i):
//   dV_j = sum_i p_ij dO_i          dp_ij = dO_i . V_j
//   ds_ij = p_ij (dp_ij - D_i),     D_i = dO_i . O_i = sum_j p_ij dp_ij
//   dQ_i = scale sum_j ds_ij K_j    dK_j = scale sum_i ds_ij Q_i
//
// Three kernels on the caller's stream:
//   bwd_rowdot:  D_i = dO_i . O_i in fp32 (0 for padded rows), into the
//                workspace;
//   bwd_dkdv:    key-major.  A workgroup owns 128 keys of one (b, h), 32 per
//                wave; query tiles of 64 rows (Q, dO, lse, D) stream through
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
//                the tile.  No atomics: every output element has one owner,
//                so the gradients are bitwise reproducible.
//
// Numerics: bf16 inputs, fp32 accumulation; P and dS are rounded to bf16
// once before their products; D from the bf16 O and dO in fp32.  Masks are
// the forward's (exclusion before the softmax): an excluded key has p = 0
// and gets no gradient; padded query rows (i >= q_len) read as zero rows
// and carry lse = +inf internally, so they contribute nothing.
#include "common.h"

namespace headattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int kThreads = 256;
constexpr int kTile = 64;  // rows per streamed tile
constexpr uint32_t kRowBytes = kHeadDim * 2;
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit elements (gfx9 family)

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// A streamed 64-row tile in LDS: row-major, 16-byte chunks of row r at
// position chunk ^ (2 (r % 4)) -- the layout the transposed reads below
// are laid out for.
struct Tile {
  uint4 c[kTile * 8];
};

// Fill rows [r0, r0 + 64) of a [rows][64] bf16 tensor into t; rows at or
// beyond the descriptor's range read as zero.  256 threads, 2 instructions.
__device__ __forceinline__ void fill_tile(Tile& t, __amdgpu_buffer_rsrc_t r, int r0, int wave, int lane) {
  const int fpos = lane & 7;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 32 * half + 8 * wave + (lane >> 3);
    const uint32_t off = (uint32_t)(r0 + row) * kRowBytes + 16u * (uint32_t)(fpos ^ (2 * (row & 3)));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(&t.c[256 * half + 64 * wave]), 16, off, 0, 0, 0);
  }
}

// Row fragment: lane (ln, hh) gets row `row`, d 16 s + 8 hh .. + 7.
__device__ __forceinline__ bf16x8 row_frag(const Tile& t, int row, int s, int hh) {
  return __builtin_bit_cast(bf16x8, t.c[row * 8 + ((2 * s + hh) ^ (2 * (row & 3)))]);
}

// Transposed fragment (A operand of X^T[d][r] times registers holding rows
// in accumulator order): for d block db and 16-row step j, lane (ln, hh)
// gets d = 32 db + ln and rows 16 j + {0..3, 8..11} + 4 hh -- the rows that
// registers 8 (j % 2) .. + 7 of a 32-row accumulator block hold.  Two
// transposed reads of 4 rows each: lane i of 16-lane group g names row kr
// and 8-byte chunk h; the read returns to lane i the 4 rows kr - i/4 .. +3
// of d = dbase + i.
__device__ __forceinline__ bf16x8 tr_frag(const Tile& t, int db, int j, int lane) {
  const char* base = reinterpret_cast<const char*>(t.c);
  const int g = lane >> 4;
  const int i = lane & 15;
  s16x4 part[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int kr = 16 * j + 8 * x + 4 * (g >> 1) + (i >> 2);
    const int h = 8 * db + 4 * (g & 1) + (i & 3);
    const int byte = kr * (int)kRowBytes + 16 * ((h >> 1) ^ (2 * (kr & 3))) + 8 * (h & 1);
    part[x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + byte));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// (b, h) of a workgroup and its block index along the owned axis.
__device__ __forceinline__ void bh_block(int bid, int n_blocks, int& bh, int& blk) {
  blk = bid % n_blocks;
  bh = bid / n_blocks;
}

// ---------------------------------------------------------------- D = rowdot
__global__ __launch_bounds__(kThreads) void bwd_rowdot_kernel(BwdArgs a) {
  // 8 lanes per row, 16 bytes each: 32 rows per workgroup.
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  const int64_t rows = (int64_t)a.B * a.H * a.n_q;
  float acc = 0.f;
  bool valid = false;
  if (row < rows) {
    const int i = (int)(row % a.n_q);
    const int b = (int)(row / ((int64_t)a.H * a.n_q));
    const int q_len = a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q;
    valid = i < q_len;
    if (valid) {
      const bf16x8 o = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.O) + row * kHeadDim + 8 * part);
      const bf16x8 g = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.dO) + row * kHeadDim + 8 * part);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    }
  }
  // Sum over the 8 lanes of the row (aligned groups of 8).
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && part == 0) a.D[row] = valid ? acc : 0.f;
}

// ---------------------------------------------------------------- dK, dV
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ Tile sq, sdo;
  __shared__ float s_lse[kTile], s_d[kTile];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hh = lane >> 5;

  const int n_kb = (a.n_k + 127) / 128;
  int bh, kb;
  bh_block(blockIdx.x, n_kb, bh, kb);
  const int b = bh / a.H;
  const int q_len = __builtin_amdgcn_readfirstlane(a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q);
  const int kv_lim = __builtin_amdgcn_readfirstlane(a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k);
  const int kb0 = kb * 128;
  const int kw0 = kb0 + 32 * wave;  // this wave's first key
  const int key = kw0 + ln;          // this lane's key

  const __bf16* Q = static_cast<const __bf16*>(a.Q) + (size_t)bh * a.n_q * kHeadDim;
  const __bf16* K = static_cast<const __bf16*>(a.K) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* V = static_cast<const __bf16*>(a.V) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* dO = static_cast<const __bf16*>(a.dO) + (size_t)bh * a.n_q * kHeadDim;
  const float* LSE = a.lse + (size_t)bh * a.n_q;
  const float* Dv = a.D + (size_t)bh * a.n_q;

  // Query rows below q_len only: padded rows read as zeros.
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Q), (short)0, (int)((uint32_t)q_len * kRowBytes), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rdo =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(dO), (short)0, (int)((uint32_t)q_len * kRowBytes), kBufferWord3);

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
  const bool wave_live = kw0 < kv_lim && (!CAUSAL || kw0 < q_len);

  int q_start = CAUSAL ? (kb0 / kTile) * kTile : 0;
  const int q_end = (kb0 < kv_lim) ? q_len : 0;  // no key of the block is valid: nothing to do
  for (int q0 = q_start; q0 < q_end; q0 += kTile) {
    __syncthreads();  // the previous tile is consumed
    fill_tile(sq, rq, q0, wave, lane);
    fill_tile(sdo, rdo, q0, wave, lane);
    if (tid < kTile) {
      const int i = q0 + tid;
      const float l = i < q_len ? LSE[i] : -INFINITY;
      // Padded rows and rows with no key: weight 0 through lse = +inf.
      s_lse[tid] = l == -INFINITY ? INFINITY : l * kLog2e;
      s_d[tid] = i < q_len ? Dv[i] : 0.f;
    }
    __syncthreads();
    // Does any query of the tile see any key of this wave?
    if (!wave_live || (CAUSAL && q0 + kTile - 1 < kw0)) continue;

    // S[q][key] and dP[q][key] for query blocks qb (32 rows each): lane
    // (ln, hh) register r holds query q0 + 32 qb + 8 (r / 4) + 4 hh + r % 4.
    f32x16 s_[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 sa = f32x16{}, pa = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(sq, 32 * qb + ln, s, hh), kf[s], sa, 0, 0, 0);
        pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(sdo, 32 * qb + ln, s, hh), vf[s], pa, 0, 0, 0);
      }
      s_[qb] = sa;
      dp[qb] = pa;
    }
    // P = exp2(s c - lse2) with the mask, dS = P (dP - D); both packed to
    // bf16 in the register order the k slots of the next products use.
    const bool need_mask = (kw0 + 32 > kv_lim) || (CAUSAL && q0 < kw0 + 32);
    uint32_t pp[16], ps[16];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int ql = 32 * qb + 8 * gq + 4 * hh;  // first of this group's 4 queries
        const float4 l4 = *reinterpret_cast<const float4*>(&s_lse[ql]);
        const float4 d4 = *reinterpret_cast<const float4*>(&s_d[ql]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dvv[4] = {d4.x, d4.y, d4.z, d4.w};
        float p[4], g[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * gq + e;
          float x = fmaf(s_[qb][r], c, -lv[e]);
          if (need_mask) {
            const int qi = q0 + ql + e;
            const bool ok = key < kv_lim && (!CAUSAL || key <= qi);
            x = ok ? x : -INFINITY;
          }
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
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(sdo, db, j, lane), pb, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(sq, db, j, lane), sb, dk[db], 0, 0, 0);
      }
    }
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
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  __shared__ Tile sk, sv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hh = lane >> 5;

  const int n_qb = (a.n_q + 127) / 128;
  int bh, qblk;
  bh_block(blockIdx.x, n_qb, bh, qblk);
  const int b = bh / a.H;
  const int q_len = __builtin_amdgcn_readfirstlane(a.q_lens ? clamp_len(a.q_lens[b], a.n_q) : a.n_q);
  const int kv_lim = __builtin_amdgcn_readfirstlane(a.kv_lens ? clamp_len(a.kv_lens[b], a.n_k) : a.n_k);
  const int q0 = qblk * 128;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + ln;

  const __bf16* Q = static_cast<const __bf16*>(a.Q) + (size_t)bh * a.n_q * kHeadDim;
  const __bf16* K = static_cast<const __bf16*>(a.K) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* V = static_cast<const __bf16*>(a.V) + (size_t)bh * a.n_k * kHeadDim;
  const __bf16* dO = static_cast<const __bf16*>(a.dO) + (size_t)bh * a.n_q * kHeadDim;

  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(K), (short)0, (int)((uint32_t)kv_lim * kRowBytes), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(V), (short)0, (int)((uint32_t)kv_lim * kRowBytes), kBufferWord3);

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
  float lse2 = INFINITY, dval = 0.f;
  if (row_live) {
    const float l = a.lse[(size_t)bh * a.n_q + qi];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    dval = a.D[(size_t)bh * a.n_q + qi];
  }

  f32x16 dq[2] = {f32x16{}, f32x16{}};  // dQ^T [d block], column = query ln
  int end = kv_lim;
  if (CAUSAL) end = min(end, q0 + 128);
  if (q0 >= q_len) end = 0;
  int wave_end = end;
  if (CAUSAL) wave_end = min(wave_end, qw0 + 32);
  if (qw0 >= q_len) wave_end = 0;

  for (int k0 = 0; k0 < end; k0 += kTile) {
    __syncthreads();
    fill_tile(sk, rk, k0, wave, lane);
    fill_tile(sv, rv, k0, wave, lane);
    __syncthreads();
    if (k0 >= wave_end) continue;
    // S^T[key][q], dP^T[key][q] for key blocks kb: register r holds key
    // k0 + 32 kb + 8 (r / 4) + 4 hh + r % 4 of query ln.
    f32x16 st[2], dpt[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sa = f32x16{}, pa = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(sk, 32 * kb + ln, s, hh), qf[s], sa, 0, 0, 0);
        pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(sv, 32 * kb + ln, s, hh), gf[s], pa, 0, 0, 0);
      }
      st[kb] = sa;
      dpt[kb] = pa;
    }
    const bool need_mask = (k0 + kTile > kv_lim) || (CAUSAL && k0 + kTile - 1 > qw0);
    uint32_t ps[16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r2 = 0; r2 < 8; ++r2) {
        float g[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * r2 + e;
          float x = fmaf(st[kb][r], c, -lse2);
          if (need_mask) {
            const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = kj < kv_lim && (!CAUSAL || kj <= qi);
            x = ok ? x : -INFINITY;
          }
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
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(sk, db, j, lane), sb, dq[db], 0, 0, 0);
    }
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

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t s) {
  BwdArgs args = a;
  void* kargs[] = {&args};
  const int64_t rows = (int64_t)a.B * a.H * a.n_q;
  hipError_t e = hipSuccess;
  if (rows > 0) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_rowdot_kernel), dim3((unsigned)((rows + 31) / 32)),
                        dim3(kThreads), kargs, 0, s);
    if (e != hipSuccess) return e;
  }
  if (a.n_k > 0) {
    const int64_t blocks = (int64_t)((a.n_k + 127) / 128) * a.H * a.B;
    const void* fn = a.causal ? reinterpret_cast<const void*>(&bwd_dkdv_kernel<true>)
                              : reinterpret_cast<const void*>(&bwd_dkdv_kernel<false>);
    e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), kargs, 0, s);
    if (e != hipSuccess) return e;
  }
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (int64_t)((a.n_q + 127) / 128) * a.H * a.B;
  const void* fn = a.causal ? reinterpret_cast<const void*>(&bwd_dq_kernel<true>)
                            : reinterpret_cast<const void*>(&bwd_dq_kernel<false>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), kargs, 0, s);
}

}  // namespace headattn
