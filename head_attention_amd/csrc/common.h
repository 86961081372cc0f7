// Internal definitions shared by the HIP kernels and the host entry points of
// libheadattn.so.  Not part of the public ABI (that is include/headattn.h).
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <stdint.h>

namespace headattn {

constexpr int kHeadDim = 64;  // d_k = d_v = d_model / h = 64 for every call

// log2(e): the kernels evaluate exp(x) as exp2(x * log2(e)) with the
// hardware's v_exp_f32 (a base-2 exponential), folding log2(e) into the
// softmax scale once per call.
constexpr float kLog2e = 1.4426950408889634f;

// One forward call, as validated by the host entry point.
struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  const int32_t* q_lens;   // device int32[B] or nullptr (all rows valid)
  const int32_t* kv_lens;  // device int32[B] or nullptr (no key padding)
  int B, H, n_q, n_k;
  float scale;             // multiplies Q K^T; finite
  bool causal;
  float* lse;              // device fp32 [B*H*n_q] or nullptr: per-row log-sum-exp
  // Restricted self-attention: -1 = off; else row i sees only keys
  // i - radius .. i + radius (i - radius .. i with causal), 0 <= radius <= n_k.
  int radius;
};

// One 16-byte-per-lane buffer load that writes LDS directly (lane l's 16
// bytes land at lds + 16 l; offsets outside the descriptor's range read as
// zero), issued from inline assembly.  The compiler then does not track
// these asynchronous LDS writes and adds no waits of its own for them (with
// the builtin it could not tell some ring slots apart and drained the whole
// ring before their reads); the caller's explicit vmcnt waits and barriers
// order them.  Two rules follow: the compiler's own vector-memory loads must
// have landed (an explicit vmcnt(0)) before a ring runs, or it re-waits for
// them inside the ring with a vmcnt(0) that drains it; and nothing else in
// these kernels may use M0, which the compiler is not told about (checked in
// the ISA: M0 is a reserved register and cannot be named as a clobber).
__device__ __forceinline__ void lds_fill16(__amdgpu_buffer_rsrc_t rsrc, const void* lds, uint32_t voff) {
  typedef __attribute__((address_space(3))) const void lds_cvoid_t;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_cvoid_t*)lds;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(base)), "v"(voff), "s"(rsrc)
               : "memory");
}

// The same with the LDS destination given as its byte address.
__device__ __forceinline__ void lds_fill16_at(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc)
               : "memory");
}

// Position of the 16-byte chunks of row r of a K tile that is only read by
// rows (16 bytes per lane, lanes on consecutive rows): chunk c sits at
// c ^ k_swz(r), distinct over any 8 consecutive rows and, for 16
// consecutive rows, within each row parity -- so the reads spread over all
// banks whether the LDS serves 8 or 16 lanes per cycle (r % 8 alone left
// rows r and r + 8 on the same banks).
__device__ __forceinline__ int k_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Mask shapes the bf16 forward kernels are specialised for: none (key
// padding only), the causal triangle, and the band of restricted
// self-attention (keys i - radius .. i + radius, or i - radius .. i).
enum FwdMode : int { kModeNone = 0, kModeCausal = 1, kModeBand = 2 };
inline int fwd_mode(const FwdArgs& a) {
  return a.radius >= 0 ? kModeBand : (a.causal ? kModeCausal : kModeNone);
}

// ln(2): a row's log-sum-exp in natural units from its log2-domain pivot m
// and sum l is (m + log2 l) ln 2.
constexpr float kLn2 = 0.69314718055994531f;

// One decode call.
struct DecodeArgs {
  const void* q;
  const void* Kc;
  const void* Vc;
  void* O;
  const int32_t* kv_lens;  // device int32[B], required
  float* work;             // [B*H][n_split][kPartialStride] fp32 partials
  int B, H, n_max;
  int n_split;             // splits per (b, h) = ceil(n_max / kDecodeChunk)
  float scale;
};

// One KV-cache append: n_new rows per (b, h) copied into the caches.
struct AppendArgs {
  const void* Kn;
  const void* Vn;
  void* Kc;
  void* Vc;
  const int32_t* kv_lens;  // device int32[B], lengths after the append
  int B, H, n_new, n_max;
  int row_bytes;           // 64 * element size
};
hipError_t launch_cache_append(const AppendArgs& a, hipStream_t s);

// One projection GEMM: C^T = W A^T, W [N, K] and A [M, K] bf16 (A given as
// X [M, K] row-major, or as the heads of O [B, H, n_seq, 64] for the output
// projection); the output is split into heads ([B, H, n_seq, 64] per block of
// H * 64 features) or written row-major [M, N].
struct ProjArgs {
  const void* W;
  const void* A;
  void* out[3];
  int M, N, K;   // M = B * n_seq tokens, N output features, K = H * 64
  int H, n_seq;
  uint32_t w_bytes, a_bytes;
  // Tile order: 0 = feature block fastest over the whole grid; f in {1, 2,
  // 4, 8} = each of the 8 XCDs takes a rectangle of 1/f of the feature
  // blocks by f/8 of the token blocks (set by the launcher).
  int xcd_fp;
};
hipError_t launch_proj(const ProjArgs& a, bool head_out, hipStream_t s);

// One backward call (bf16): gradients of O = softmax(Q K^T scale + M) V.
struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* lse;        // [B*H*n_q] natural-log row normalisers from the forward
  float* D;                // workspace [B*H*n_pad]: dO . O per row (0 for padded rows)
  float* L;                // workspace [B*H*n_pad]: lse log2(e) per row (+inf for padded rows)
  uint4* LD16;             // workspace [B*H*n_pad]: per row 8 bf16, -L/c as the sum of three parts, 0,
                           // -D as the sum of three parts, 0 (c = |scale| log2 e; -2^100 for +inf L)
  void* dQ;
  void* dK;
  void* dV;
  const int32_t* q_lens;
  const int32_t* kv_lens;
  int B, H, n_q, n_k;
  int n_pad;               // n_q rounded up to a multiple of 64
  float scale;
  bool causal;
  int radius;              // restricted self-attention radius, -1 = off (0 <= radius <= n_k)
};
hipError_t launch_backward(const BwdArgs& a, hipStream_t s);

// Decode: keys per split (one workgroup of 4 waves x 64 keys).
constexpr int kDecodeWaves = 4;
constexpr int kDecodeChunk = 64 * kDecodeWaves;
// Partial record per split: m (max logit, log2 domain), l (sum of weights),
// acc[64] (unnormalised weighted sum of V).
constexpr int kPartialStride = 2 + kHeadDim;

// At least one split, so the merge pass always runs and writes O (a cache of
// capacity 0 gives zero rows).
inline int decode_splits(int n_max) {
  const int s = (n_max + kDecodeChunk - 1) / kDecodeChunk;
  return s > 0 ? s : 1;
}

// Launchers; each returns the hipError_t of its launch(es).
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16_pair(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16_short(const FwdArgs& a, hipStream_t s);
// Restricted self-attention with n_k > kShortMaxKeys: 512-row workgroups of
// eight row groups, each walking its own window of keys.
hipError_t launch_fwd_bf16_band(const FwdArgs& a, hipStream_t s);

// bf16 forward: calls whose key range fits LDS whole (n_k <= 256) run on the
// short-sequence kernel, which loads all of a (b, h)'s K and V at once.
constexpr int kShortMaxKeys = 256;

// bf16 forward: calls with at least this many query rows run on the paired
// 8-wave kernel (256 rows per workgroup); shorter ones on the 4-wave kernel
// (128 rows per workgroup), which leaves fewer rows idle.
constexpr int kPairMinRows = 512;
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);

// attn_decode_noalloc keeps its split partials in a static device array of
// this many bytes per GPU (the ATTN_DECODE_NOALLOC_MAX_BYTES of the header).
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
// Device address of that array on the current device (looked up once per
// device); never the array's host-side name.
hipError_t decode_scratch(float** ptr);

// Clamp a device-provided length into [0, n] so that a bad length can never
// index outside the caller's buffers.
__device__ __forceinline__ int clamp_len(int v, int n) { return v < 0 ? 0 : (v > n ? n : v); }

}  // namespace headattn
