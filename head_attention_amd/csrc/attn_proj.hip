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
// Both run on one GEMM kernel, C^T = W A^T with W [N, K] (one row per output
// feature, k contiguous) and A [M, K] (one row per token): on
// v_mfma_f32_32x32x16_bf16 the A operand is a W fragment and the B operand
// an A fragment, both 16 contiguous bytes of a k-contiguous row, and each
// lane ends up holding four consecutive output features of one token.
//
// One 8-wave workgroup per compute unit.  The tile is TM tokens x TN
// features, the waves on a WM x WN grid (WM WN = 8), each owning 32 TBW
// tokens x 32 FBW features: 256 x 192 (WM 4, TBW 2, FBW 3), 320 x 128 (WM 2,
// TBW 5, FBW 1) or 128 x 128 (WM 2, TBW 2, FBW 1), whichever leaves the least
// work on the busiest compute unit.  The decoder's self Q, K, V at
// 4096 x 3072 makes exactly 256 tiles of 256 x 192 and its cross K, V at
// 5120 x 2048 exactly 256 of 320 x 128, so every compute unit gets the same
// work.  Two waves per SIMD.  K runs in steps of 64 through two slots (448
// rows, 56 KB each) or three (256 rows): the W and A rows of a step reach
// LDS by buffer loads that write LDS directly, and a row's step is 128
// bytes, so every fill reads whole cache lines (64-byte steps read half
// lines, and fetched about 26 bytes per clock per compute unit here, against
// what the products need).  A step's fills go out as soon as its slot
// frees, one bare barrier per step.  Rows past the end of W or A read as
// zero through the descriptor's range check.  For the output projection a
// step is one whole head: A row m's step kt is O[b, kt, t, :], a per-row
// offset, no gather of single elements.  The output leaves through LDS in
// whole 128-byte rows.
#include <algorithm>
#include <type_traits>

#include "kernel_util.h"

namespace headattn {
namespace {

// Wait until at most N of this wave's buffer loads are outstanding and its
// LDS operations are done, then a bare workgroup barrier (a workgroup fence
// would add a wait for every fill in flight).
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);  // vmcnt(N), lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

constexpr uint32_t kStepRowBytes = 128;  // a row's k step of 64: 8 chunks of 16 bytes
// The ring: two slots of 448 rows, or three of 256 (112 KB either way at most).
__shared__ uint4 g_ring[2 * 448 * 8];

template <int ROWS>
__device__ __forceinline__ uint32_t ring_addr(int slot) {
  return (uint32_t)(uintptr_t)(lds_void_t*)&g_ring[0] + (uint32_t)slot * (ROWS * kStepRowBytes);
}

template <bool HEAD_OUT, int WM, int TBW, int FBW>
__global__ __launch_bounds__(512, 1) void proj_gemm_kernel(ProjArgs a) {
  constexpr int WN = 8 / WM;
  constexpr int TM = 32 * TBW * WM;  // tokens per workgroup
  constexpr int TN = 32 * FBW * WN;  // output features per workgroup
  constexpr int kRows = TM + TN;              // rows of a step
  constexpr int kSlots = kRows > 256 ? 2 : 3;  // ring slots
  constexpr int kFillW = TN / 8;               // fill instructions of the W rows
  constexpr int kFillPerWave = kRows / 64;     // fill instructions per wave and step
  static_assert(WM * WN == 8 && kRows % 64 == 0 && kSlots * kRows <= 2 * 448, "tile shape");
  static_assert(TN % 64 == 0, "a tile's features are whole 64-wide heads");
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hh = lane >> 5;
  const int wn = wave % WN;  // feature group of the tile
  const int wm = wave / WN;  // token group of the tile

  // Tile of this workgroup.  Workgroup ids go round robin over the 8 XCDs;
  // with xcd_fp = f each XCD owns a rectangle of f/8 of the token blocks by
  // 1/f of the feature blocks, so a tile's X rows and W rows are mostly
  // already in that XCD's L2 (the plain order sends the feature blocks of
  // one token block to different XCDs, each fetching the same X rows).
  // Inside the rectangle, groups of up to 8 token blocks walk all its
  // feature blocks, so the workgroups an XCD runs at once share X rows and
  // W rows.
  const int n_blocks = (a.N + TN - 1) / TN;
  int nb = blockIdx.x % n_blocks;
  int mb = blockIdx.x / n_blocks;
  if (a.xcd_fp > 0) {
    const int fp = a.xcd_fp;
    const int x = blockIdx.x & 7;
    const int l = blockIdx.x >> 3;
    const int nbr = n_blocks / fp;
    const int mbr = ((a.M + TM - 1) / TM) / (8 / fp);
    const int g0 = l / (8 * nbr) * 8;
    const int gs = min(8, mbr - g0);
    const int r = l - g0 * nbr;
    nb = (x % fp) * nbr + r / gs;
    mb = (x / fp) * mbr + g0 + r % gs;
  }
  const int n0 = nb * TN;
  const int m0 = mb * TM;
  const int K = a.K;
  const int nk = K / 64;

  // ---- fills.  A step's slot holds the tile's W rows (0 .. TN - 1) then
  // its A rows (TN .. TN + TM - 1), 128 B each, chunk c of row r at position
  // c ^ k_swz(r) (16-lane row reads conflict-free).  Fill instruction q
  // writes rows 8 q .. 8 q + 7 (1 KB, 8 lanes a row); wave w issues q = w,
  // w + 8, .., w + 48.  For the output projection a step is one whole head:
  // A row m's step kt is O[b, kt, t, :].
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.W), (short)0, (int)a.w_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.A), (short)0, (int)a.a_bytes, kBufferWord3);
  const int fpos = lane & 7;
  uint32_t f_off[kFillPerWave];
#pragma unroll
  for (int i = 0; i < kFillPerWave; ++i) {
    const int q = wave + 8 * i;
    const int row = 8 * q + (lane >> 3);
    const uint32_t chunk = 16u * (uint32_t)(fpos ^ k_swz(row));
    if (q < kFillW) {
      const int n = n0 + row;
      f_off[i] = n < a.N ? (uint32_t)n * (uint32_t)K * 2u + chunk : kOutOfRange;
    } else {
      const int m = m0 + row - TN;
      if (HEAD_OUT) {
        f_off[i] = m < a.M ? (uint32_t)m * (uint32_t)K * 2u + chunk : kOutOfRange;
      } else {
        const int b = m / a.n_seq;
        const int t = m - b * a.n_seq;
        f_off[i] = m < a.M ? ((uint32_t)b * (uint32_t)a.H * (uint32_t)a.n_seq + (uint32_t)t) * (kHeadDim * 2u) + chunk
                           : kOutOfRange;
      }
    }
  }
  auto fill = [&](auto slot_tag, int kt) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;
    const uint32_t base = ring_addr<kRows>(S);
    const uint32_t ws = (uint32_t)kt * 128u;
    const uint32_t as = HEAD_OUT ? (uint32_t)kt * 128u : (uint32_t)kt * (uint32_t)a.n_seq * (kHeadDim * 2u);
#pragma unroll
    for (int i = 0; i < kFillPerWave; ++i) {
      const int q = wave + 8 * i;
      const bool isw = q < kFillW;
      const uint32_t o = f_off[i] == kOutOfRange ? kOutOfRange : f_off[i] + (isw ? ws : as);
      lds_fill16_at(isw ? rw : ra, base + 1024u * (uint32_t)q, o);
    }
  };
  f32x16 acc[FBW][TBW];  // [feature block][token block]
#pragma unroll
  for (int i = 0; i < FBW; ++i)
#pragma unroll
    for (int j = 0; j < TBW; ++j) acc[i][j] = f32x16{};

  // One step: S = kt % kSlots is its slot.  The wait lands step kt (with
  // three slots step kt + 1's fills may still fly), and the barrier
  // publishes it and frees the slot of step kt - 1 (every wave is done with
  // it), which step kt + kSlots - 1 then takes.
  // Fragments of k sub-step s: lane (ln, hh) reads W row 32 (FBW wn + i) +
  // ln and A row TN + 32 (TBW wm + j) + ln, chunk 2 s + hh (k 16 s + 8 hh
  // .. + 7).
  auto step = [&](auto slot_tag, int kt) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;
    using SF = std::integral_constant<int, (S + kSlots - 1) % kSlots>;
    if (kt >= nk) return;
    wait_barrier<(kSlots - 2) * kFillPerWave>();
    fill(SF(), kt + kSlots - 1);
    const lds_uint4* t = (const lds_uint4*)(uintptr_t)ring_addr<kRows>(S);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + hh;
      bf16x8 wf[FBW], af[TBW];
#pragma unroll
      for (int i = 0; i < FBW; ++i) {
        const int r = 32 * (FBW * wn + i) + ln;
        wf[i] = __builtin_bit_cast(bf16x8, t[r * 8 + (ch ^ k_swz(r))]);
      }
#pragma unroll
      for (int j = 0; j < TBW; ++j) {
        const int r = TN + 32 * (TBW * wm + j) + ln;
        af[j] = __builtin_bit_cast(bf16x8, t[r * 8 + (ch ^ k_swz(r))]);
      }
#pragma unroll
      for (int i = 0; i < FBW; ++i)
#pragma unroll
        for (int j = 0; j < TBW; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  fill(S0(), 0);
  if constexpr (kSlots == 2) {
    for (int kt = 0; kt < nk; kt += 2) {
      step(S0(), kt);
      step(S1(), kt + 1);
    }
  } else {
    fill(S1(), 1);
    for (int kt = 0; kt < nk; kt += 3) {
      step(S0(), kt);
      step(S1(), kt + 1);
      step(S2(), kt + 2);
    }
  }
  // The fill past the end of K (out of range or never read) lands before
  // the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0)

  // ---- epilogue through LDS, so that every global store writes whole
  // 128-byte rows (8 lanes a row; 16-byte pieces at a 128-byte stride, as
  // the registers hold them, left the L2 merging partial lines).  The tile
  // is TN / 64 chunks of 64 features -- each one head of one projection
  // (heads are 64-aligned) -- by TM tokens; chunk c, token u sits at
  // c TM 128 + u 128 bytes, its 16-byte piece q (d 8 q .. 8 q + 7) at
  // position q ^ (u % 8).  Register r of block (i, j) holds feature
  // 32 (FBW wn + i) + 8 (r / 4) + 4 hh + r % 4 of token 32 (TBW wm + j) + ln
  // of the tile.
  constexpr int kChunks = TN / 64;
  barrier_lds();  // every wave is done with the ring
  {
    lds_char* st = (lds_char*)(uintptr_t)ring_addr<kRows>(0);
#pragma unroll
    for (int i = 0; i < FBW; ++i)
#pragma unroll
      for (int j = 0; j < TBW; ++j) {
        const int u = 32 * (TBW * wm + j) + ln;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int f = 32 * (FBW * wn + i) + 8 * g + 4 * hh;  // first of the lane's 4 features
          const int c = f >> 6, q = (f & 63) >> 3;
          u32x2 v;
          v.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
          v.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *(lds_u32x2*)(st + (c * TM + u) * 128 + ((q ^ (u & 7)) << 4) + (f & 4) * 2) = v;
        }
      }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  barrier_lds();
  const int d_model = a.H * kHeadDim;
  const lds_char* st = (const lds_char*)(uintptr_t)ring_addr<kRows>(0);
  const int q = lane & 7;
#pragma unroll 2
  for (int it = 0; it < kChunks * TM / 64; ++it) {
    const int row = 64 * it + 8 * wave + (lane >> 3);
    const int c = row / TM, u = row - c * TM;
    const int nf = n0 + 64 * c;  // first feature of the chunk
    const int m = m0 + u;
    const uint4 v = __builtin_bit_cast(uint4, *(const lds_uint4*)(st + row * 128 + ((q ^ (u & 7)) << 4)));
    if (nf >= a.N || m >= a.M) continue;
    __bf16* dst;
    if (HEAD_OUT) {
      const int p = nf / d_model;
      const int hd = (nf - p * d_model) / kHeadDim;
      const int b = m / a.n_seq;
      const int t = m - b * a.n_seq;
      dst = static_cast<__bf16*>(a.out[p]) + (((size_t)b * a.H + hd) * a.n_seq + t) * kHeadDim;
    } else {
      dst = static_cast<__bf16*>(a.out[0]) + (size_t)m * a.N + nf;
    }
    *reinterpret_cast<uint4*>(dst + 8 * q) = v;
  }
}

// The XCD split with the fewest L2 fills, W rows read by 8/f XCDs and X rows
// by f: f minimising w_bytes * 8/f + a_bytes * f among those that divide the
// tile grid evenly; 0 (plain order) when none does.
int xcd_split(const ProjArgs& a, long long n_blocks, long long m_blocks) {
  int best = 0;
  double best_cost = 0.0;
  for (int f = 1; f <= 8; f *= 2) {
    if (n_blocks % f != 0 || m_blocks % (8 / f) != 0) continue;
    const double cost = (double)a.w_bytes * (8 / f) + (double)a.a_bytes * f;
    if (best == 0 || cost < best_cost) {
      best = f;
      best_cost = cost;
    }
  }
  return best;
}

template <bool HEAD_OUT>
hipError_t launch_tb(const ProjArgs& a, hipStream_t s) {
  // The tile with the least work on its busiest compute unit (ties go to the
  // earlier one in this order); workgroups are spread evenly over the 256
  // compute units.
  const long long M = a.M, N = a.N;
  auto per_cu = [](long long tiles, long long outputs) { return (tiles + 255) / 256 * outputs; };
  const long long nba = (N + 191) / 192, mba = (M + 255) / 256;
  const long long nbb = (N + 127) / 128, mbb = (M + 319) / 320;
  const long long nbc = (N + 127) / 128, mbc = (M + 127) / 128;
  const long long ca = per_cu(nba * mba, 256 * 192);
  const long long cb = per_cu(nbb * mbb, 320 * 128);
  const long long cc = per_cu(nbc * mbc, 128 * 128);
  ProjArgs args = a;
  void* kargs[] = {&args};
  if (ca <= cb && ca <= cc) {
    args.xcd_fp = xcd_split(a, nba, mba);
    return hipLaunchKernel(reinterpret_cast<const void*>(&proj_gemm_kernel<HEAD_OUT, 4, 2, 3>),
                           dim3((unsigned)(nba * mba)), dim3(512), kargs, 0, s);
  }
  if (cb <= cc) {
    args.xcd_fp = xcd_split(a, nbb, mbb);
    return hipLaunchKernel(reinterpret_cast<const void*>(&proj_gemm_kernel<HEAD_OUT, 2, 5, 1>),
                           dim3((unsigned)(nbb * mbb)), dim3(512), kargs, 0, s);
  }
  args.xcd_fp = xcd_split(a, nbc, mbc);
  return hipLaunchKernel(reinterpret_cast<const void*>(&proj_gemm_kernel<HEAD_OUT, 2, 2, 1>),
                         dim3((unsigned)(nbc * mbc)), dim3(512), kargs, 0, s);
}

}  // namespace

hipError_t launch_proj(const ProjArgs& a, bool head_out, hipStream_t s) {
  return head_out ? launch_tb<true>(a, s) : launch_tb<false>(a, s);
}

}  // namespace headattn
