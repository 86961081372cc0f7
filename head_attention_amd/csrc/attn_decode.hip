// KV-cache decode step of attn_decode: one new query per (b, h) against the
// kv_len valid rows of its cache ("[논문 리뷰]Attention Is All You Need",
// §3.7: cached K/V mean only the new token's Q is computed per step;
// "Attention Is All You Need 해부", KV cache section: K,V = the cached
// 0..t-1 plus the new token's own K,V, appended by the caller).
//
// The work is a scan of the cache: every valid K and V row is read once from
// HBM, and there are only 4 d flops per key, so the kernels are built to keep
// HBM busy rather than the ALUs.  The cache axis is split into fixed chunks
// of kDecodeChunk keys, one workgroup per (b, h, chunk), so lengths from 1 to
// n_max spread evenly over the chip; chunks past kv_len exit at once.
//
// Pass 1 (partial): each wave takes 64 keys.  Lanes are grouped by 16-byte
// slices of a row: LPR lanes cover one 128 B (bf16) / 256 B (fp32) row, so a
// wave's 16-byte loads cover whole rows, and every lane issues all of its K
// and V loads before it uses any.  q.k is a slice dot product plus a
// cross-lane sum; the wave then forms its own softmax partial
//   m = max_j s_j,  l = sum_j exp2(s_j - m),  acc = sum_j exp2(s_j - m) v_j
// (s_j in the log2 domain), the workgroup merges its 4 wave partials in LDS,
// and writes one record (m, l, acc[64]) per chunk.
// Pass 2 (merge): per (b, h), M = max_s m_s and
//   O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
// Both passes are the same exact identity the online softmax uses: partial
// sums under different pivots combine after rescaling to a common pivot.
#include <mutex>

#include "kernel_util.h"

namespace headattn {
namespace {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPerLoad = 4;  // elements per 16-byte load
  __device__ static void unpack(const uint4& v, float* out) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  }
  __device__ static void store(float* dst, const float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = v[i];
  }
};
template <>
struct Elem<__bf16> {
  static constexpr int kPerLoad = 8;
  __device__ static void unpack(const uint4& v, float* out) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // bf16 -> fp32 is exact: the high 16 bits
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

constexpr int kWaveKeys = 64;  // keys per wave per chunk

// One 16-byte non-temporal load.
template <typename T>
__device__ __forceinline__ uint4 stream_load(const T* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

// Cross-lane combines on the vector ALUs (DPP and permlane swaps; no LDS
// traffic).  Each pairs every lane with one partner; repeated, they reduce
// over aligned groups of 2, 4, 8, 16, 32 and 64 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
struct Sum {
  __device__ static float op(float a, float b) { return a + b; }
};
struct Max {
  __device__ static float op(float a, float b) { return fmaxf(a, b); }
};
// Combine lane l with lane l ^ step (step = 1, 2), its mirror in its group of
// 8 (step 4), its partner 8 apart in a row of 16 (step 8), or across rows of
// 16 (step 16) or halves of the wave (step 32).
template <class Op, int STEP>
__device__ __forceinline__ float combine(float v) {
  if constexpr (STEP == 1) return Op::op(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
  if constexpr (STEP == 2) return Op::op(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
  if constexpr (STEP == 4) return Op::op(v, dpp_mov<0x141>(v));  // row_half_mirror
  if constexpr (STEP == 8) return Op::op(v, dpp_mov<0x128>(v));  // row_ror:8
  if constexpr (STEP == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    // take the two halves by value: a bit cast of a vector element lvalue
    // would read element 0 for both
    const uint32_t lo = r[0], hi = r[1];
    return Op::op(__uint_as_float(lo), __uint_as_float(hi));
  }
  if constexpr (STEP == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const uint32_t lo = r[0], hi = r[1];
    return Op::op(__uint_as_float(lo), __uint_as_float(hi));
  }
  return v;
}
// Reduce over lanes [FROM, TO) in the power-of-two ladder of steps.
template <class Op, int FROM, int TO>
__device__ __forceinline__ float reduce(float v) {
  if constexpr (FROM < TO) return reduce<Op, FROM * 2, TO>(combine<Op, FROM>(v));
  return v;
}

template <typename T>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_partial_kernel(DecodeArgs a) {
  constexpr int EPL = Elem<T>::kPerLoad;       // elements per lane slice
  constexpr int LPR = kHeadDim / EPL;          // lanes per cache row
  constexpr int KPP = 64 / LPR;                // keys per pass of a wave
  constexpr int NP = kWaveKeys / KPP;          // passes per wave

  // Split-major order: consecutive workgroups, which the dispatcher deals
  // round-robin to the 8 XCDs, take the same chunk index of different
  // (b, h).  Chunk s is valid only where kv_len > 256 s, so a (b, h)-major
  // order would hand XCD x mostly chunks x and x + 8 of every row and load
  // the XCDs unevenly under ragged lengths; this order gives every XCD the
  // same mix of heads.
  const int BH = a.B * a.H;
  const int split = blockIdx.x / BH;
  const int bh = blockIdx.x % BH;
  const int b = bh / a.H;
  const int kv_len = clamp_len(a.kv_lens[b], a.n_max);
  const int chunk0 = split * kDecodeChunk;
  if (chunk0 >= kv_len) return;  // workgroup-uniform: past the valid rows

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int sl = lane % LPR;  // slice: d = EPL*sl .. EPL*sl + EPL-1
  const int kk = lane / LPR;  // key within a pass
  const int w0 = chunk0 + wave * kWaveKeys;

  const T* q = static_cast<const T*>(a.q) + (size_t)bh * kHeadDim;
  const T* Kc = static_cast<const T*>(a.Kc) + (size_t)bh * a.n_max * kHeadDim;
  const T* Vc = static_cast<const T*>(a.Vc) + (size_t)bh * a.n_max * kHeadDim;

  // Issue every K and V load of this wave up front (2 x NP x 16 B per lane).
  // The cache is read once per step, so the loads are marked non-temporal:
  // streamed past the caches instead of evicting lines that are reused.
  uint4 kraw[NP], vraw[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int key = w0 + p * KPP + kk;
    if (key < kv_len) {
      kraw[p] = stream_load(Kc + (size_t)key * kHeadDim + EPL * sl);
      vraw[p] = stream_load(Vc + (size_t)key * kHeadDim + EPL * sl);
    } else {  // never read: padded rows may hold anything, even NaN
      kraw[p] = make_uint4(0, 0, 0, 0);
      vraw[p] = make_uint4(0, 0, 0, 0);
    }
  }
  float qv[EPL];
  Elem<T>::unpack(*reinterpret_cast<const uint4*>(q + EPL * sl), qv);

  // c > 0; see the forward kernel for why the floor changes no result.
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 0x1p-100f);
  const float sgn = a.scale < 0.f ? -1.f : 1.f;

  // Scores in the log2 domain, one per key of each pass (all LPR lanes of a
  // row end up holding the row's score).
  float s[NP];
  float mloc = -INFINITY;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float kv[EPL];
    Elem<T>::unpack(kraw[p], kv);
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) part = fmaf(qv[e], kv[e], part);
    part = reduce<Sum, 1, LPR>(part);  // dot product over the row's LPR lanes
    const int key = w0 + p * KPP + kk;
    s[p] = key < kv_len ? sgn * part * c : -INFINITY;
    mloc = fmaxf(mloc, s[p]);
  }
  mloc = reduce<Max, LPR, 64>(mloc);
  const float m = mloc;  // wave max (-inf if the wave has no valid key)

  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float lsum = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float w = __builtin_amdgcn_exp2f(s[p] - m);  // 0 for invalid keys
      float vv[EPL];
      Elem<T>::unpack(vraw[p], vv);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, vv[e], acc[e]);
      lsum += w;
    }
  }
  // Sum over the keys of the wave: the lanes with the same slice sit LPR
  // apart, and each of them saw every key of its own passes once.
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = reduce<Sum, LPR, 64>(acc[e]);
  lsum = reduce<Sum, LPR, 64>(lsum);

  // ---- merge the 4 wave partials of this chunk in LDS
  __shared__ float sm[kDecodeWaves], sl_[kDecodeWaves];
  __shared__ float sacc[kDecodeWaves][kHeadDim];
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) sacc[wave][EPL * sl + e] = acc[e];
  }
  if (lane == 0) {
    sm[wave] = m;
    sl_[wave] = lsum;
  }
  __syncthreads();
  if (wave == 0) {
    float M = sm[0];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, sm[w]);
    // M is finite: the chunk holds at least one valid key (chunk0 < kv_len).
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = sm[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[w] - M);
      L = fmaf(f, sl_[w], L);
      A = fmaf(f, sacc[w][lane], A);
    }
    float* rec = a.work + ((size_t)bh * a.n_split + split) * kPartialStride;
    rec[2 + lane] = A;
    if (lane == 0) {
      rec[0] = M;
      rec[1] = L;
    }
  }
}

template <typename T>
__device__ __forceinline__ void store_out(T* dst, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* dst, float v) { *dst = v; }
template <>
__device__ __forceinline__ void store_out<__bf16>(__bf16* dst, float v) { *dst = (__bf16)v; }

template <typename T>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int d = threadIdx.x;
  const int kv_len = clamp_len(a.kv_lens[b], a.n_max);
  const int ns = (kv_len + kDecodeChunk - 1) / kDecodeChunk;
  const float* rec = a.work + (size_t)bh * a.n_split * kPartialStride;
  // M = max of the split maxima: lane s reads m_s, then a wave max.
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int s = s0 + d;
    M = fmaxf(M, s < ns ? rec[(size_t)s * kPartialStride] : -INFINITY);
  }
  M = reduce<Max, 1, 64>(M);
  // O[d] = sum_s 2^(m_s - M) acc_s[d] / sum_s 2^(m_s - M) l_s, eight splits'
  // loads in flight at a time.
  float L = 0.f, A = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float mv[8], lv[8], av[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = s0 + i < ns;
      const float* r = rec + (size_t)(ok ? s0 + i : 0) * kPartialStride;
      mv[i] = ok ? r[0] : -INFINITY;
      lv[i] = r[1];
      av[i] = r[2 + d];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float f = mv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv[i] - M);
      L = fmaf(f, lv[i], L);
      A = fmaf(f, av[i], A);
    }
  }
  // kv_len = 0: no partials, the row is 0.
  const float out = L > 0.f ? A / L : 0.f;
  store_out<T>(static_cast<T*>(a.O) + (size_t)bh * kHeadDim + d, out);
}

template <typename T>
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  DecodeArgs args = a;
  void* kargs[] = {&args};
  const long long blocks = (long long)a.B * a.H * a.n_split;
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_partial_kernel<T>),
                                 dim3((unsigned)blocks), dim3(64 * kDecodeWaves), kargs, 0, s);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&decode_merge_kernel<T>),
                         dim3((unsigned)(a.B * a.H)), dim3(64), kargs, 0, s);
}

}  // namespace

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) { return launch_decode<float>(a, s); }
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) { return launch_decode<__bf16>(a, s); }

// ---- the partials of attn_decode_noalloc: a file-scope device array that
// each GPU holds for the life of the process, so that a call allocates
// nothing.  Host code never passes `scratch` itself to a kernel (in host code
// the name is a host-side stand-in, not a device address): the device address
// comes from hipGetSymbolAddress, once per device with that device current.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace headattn
