// Issue-rate microbenchmark for the paired forward kernel on gfx950.
//
// Measures, in shader clocks per 64x64 tile per SIMD, what the paired
// kernel's work costs when its parts are put together one at a time:
//  - the matrix work of one tile (32 v_mfma_f32_32x32x16_bf16 for S and P.V,
//    8 v_mfma_f32_16x16x32_bf16 for the row sums) and its vector work (64
//    scale multiplies, 64 v_exp_f32, 32 bf16 packs), each alone;
//  - both from one wave, interleaved by the scheduler's group barriers;
//  - both from two waves of one SIMD, one kind each, free-running and with
//    a workgroup barrier per tile;
//  - then with the matrix operands read from LDS (16 transposed 8-byte and
//    8 16-byte reads per tile), with the two waves swapping roles every
//    tile, and with the ring fills (two 16-byte-per-lane buffer loads into
//    LDS per wave per tile, waited for four tiles later).
// One workgroup per compute unit (96 KB of LDS), 256 workgroups; clocks from
// s_memtime, the clock rate from s_memrealtime (100 MHz); best of three runs.
//
// Build and run (from the repository root):
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         bench_issue_rate.hip -o _build/bench_issue_rate && _build/bench_issue_rate
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
#include <algorithm>
#include <type_traits>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__shared__ float lds_pad[24 * 1024];  // 96 KB: one workgroup per compute unit
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_void_ptr() {
  return (__attribute__((address_space(3))) void*)(__attribute__((address_space(3))) float*)lds_pad;
}

struct St {
  bf16x8 a0, a1, b0, b1, sel;
  f32x16 c0, c1, c2, c3;
  f32x4 r0, r1;
  float x[64];
  uint32_t pk[32];
  float c;
};
__device__ __forceinline__ void init(St& s, const float* in, int lane) {
  for (int i = 0; i < 8; ++i) {
    s.a0[i] = (__bf16)(in[lane] * 0.001f * i); s.a1[i] = (__bf16)(in[lane + 1] * 0.001f);
    s.b0[i] = (__bf16)(in[lane + 2] * 0.001f); s.b1[i] = (__bf16)(in[lane + 3] * 0.001f * i);
    s.sel[i] = (__bf16)(lane < 2 ? 1.f : 0.f);
  }
  s.c0 = f32x16{}; s.c1 = f32x16{}; s.c2 = f32x16{}; s.c3 = f32x16{}; s.r0 = f32x4{}; s.r1 = f32x4{};
  for (int i = 0; i < 64; ++i) s.x[i] = in[lane + i] * 1e-3f;
  for (int i = 0; i < 32; ++i) s.pk[i] = 0;
  s.c = in[1] * 1e-3f + 1.0f;
}
// one tile's matrix work: 32 v_mfma_f32_32x32x16_bf16 (S and P.V) and 8
// v_mfma_f32_16x16x32_bf16 (row sums), four independent accumulation chains
__device__ __forceinline__ void mfma_tile(St& s) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    s.c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s.a0, s.b0, s.c0, 0, 0, 0);
    s.c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s.a1, s.b0, s.c1, 0, 0, 0);
    s.c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s.a0, s.b1, s.c2, 0, 0, 0);
    s.c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s.a1, s.b1, s.c3, 0, 0, 0);
    if (k & 1) {
      s.r0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s.sel, s.b0, s.r0, 0, 0, 0);
      s.r1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s.sel, s.b1, s.r1, 0, 0, 0);
    }
  }
}
// the same with its operands read from LDS as the paired kernel does: 16
// transposed 8-byte reads (V) and 8 16-byte reads (K) per tile, each read
// issued one step before the products that use it
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 s16x4_lds;
__device__ __forceinline__ void mfma_tile_lds(St& s, int lane) {
  typedef __attribute__((address_space(3))) char lds_char;
  const lds_char* base = (const lds_char*)(lds_void_ptr());
  bf16x8 va[8], ka[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_lds*)(base + 1024 * j + 8 * lane));
    s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_lds*)(base + 1024 * j + 512 + 8 * lane));
    va[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s.c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[2 * k], s.b0, s.c0, 0, 0, 0);
    s.c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[2 * k + 1], s.b0, s.c1, 0, 0, 0);
    s.c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[2 * k], s.b1, s.c2, 0, 0, 0);
    s.c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[2 * k + 1], s.b1, s.c3, 0, 0, 0);
    s.r0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s.sel, s.b0, s.r0, 0, 0, 0);
    s.r1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s.sel, s.b1, s.r1, 0, 0, 0);
    if (k == 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ka[i] = __builtin_bit_cast(bf16x8, *(const __attribute__((address_space(3))) uint4*)(base + 16384 + 1024 * i + 16 * lane));
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s.c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[2 * k], s.a0, s.c0, 0, 0, 0);
    s.c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[2 * k + 1], s.a0, s.c1, 0, 0, 0);
    s.c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[2 * k], s.a1, s.c2, 0, 0, 0);
    s.c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[2 * k + 1], s.a1, s.c3, 0, 0, 0);
  }
}
// one tile's vector work (KIND 0): 64 scale multiplies, 64 exp2, 32 bf16
// packs -- or, for KIND 1, the exp2 replaced by a multiply
template <int KIND>
__device__ __forceinline__ void valu_tile(St& s) {
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const float y = s.x[i] * s.c;
    s.x[i] = KIND == 0 ? __builtin_amdgcn_exp2f(y) : y * 0.9999f;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    f32x2 v = {s.x[2 * i], s.x[2 * i + 1]};
    s.pk[i] ^= __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
}
__device__ __forceinline__ void finish(St& s, float* out, uint64_t* cyc, uint64_t dt, uint64_t dr) {
  float acc = 0;
  for (int i = 0; i < 16; ++i) acc += s.c0[i] + s.c1[i] + s.c2[i] + s.c3[i];
  for (int i = 0; i < 4; ++i) acc += s.r0[i] + s.r1[i];
  for (int i = 0; i < 64; ++i) acc += s.x[i];
  for (int i = 0; i < 32; ++i) acc += (float)(s.pk[i] & 0xff);
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc + lds_pad[(threadIdx.x + 1) & 255];
  if ((threadIdx.x & 63) == 0) {
    cyc[2 * (blockIdx.x * 8 + (threadIdx.x >> 6))] = dt;
    cyc[2 * (blockIdx.x * 8 + (threadIdx.x >> 6)) + 1] = dr;
  }
}

// One wave per SIMD.  MODE 0: matrix only; 1: vector only; 2: both,
// interleaved one MFMA to G VALU by the scheduler's group barriers.
template <int MODE, int G, int KIND>
__global__ __launch_bounds__(256, 1) void one_wave(const float* in, float* out, uint64_t* cyc, int iters) {
  St s; init(s, in, threadIdx.x & 63);
  lds_pad[threadIdx.x] = s.c;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if (MODE != 1) mfma_tile(s);
    if (MODE != 0) valu_tile<KIND>(s);
    if (MODE == 2) {
#pragma unroll
      for (int k = 0; k < 40; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, G, 0);
      }
    }
  }
  finish(s, out, cyc, __builtin_amdgcn_s_memtime() - t0, __builtin_amdgcn_s_memrealtime() - r0);
}
// Two waves per SIMD (waves w and w + 4 share a SIMD): waves 0-3 matrix
// work, waves 4-7 vector work, free-running (SYNC 0) or with a workgroup
// barrier per tile (SYNC 1), as in the paired kernel.
template <int SYNC, int KIND>
__global__ __launch_bounds__(512, 1) void two_waves(const float* in, float* out, uint64_t* cyc, int iters) {
  const int wave = threadIdx.x >> 6;
  St s;
  init(s, in, threadIdx.x & 63);
  lds_pad[threadIdx.x & 255] = s.c;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  if (wave < 4) {
    for (int i = 0; i < 64; ++i) s.x[i] = 0.f;  // the matrix wave's vector state is dead
    for (int i = 0; i < 32; ++i) s.pk[i] = 0;
    for (int it = 0; it < iters; ++it) {
      mfma_tile(s);
      if (SYNC) __syncthreads();
    }
  } else {
    s.c0 = f32x16{}; s.c1 = f32x16{}; s.c2 = f32x16{}; s.c3 = f32x16{};  // the vector wave's matrix state is dead
    s.r0 = f32x4{}; s.r1 = f32x4{};
    for (int it = 0; it < iters; ++it) {
      valu_tile<KIND>(s);
      if (SYNC) __syncthreads();
    }
  }
  finish(s, out, cyc, __builtin_amdgcn_s_memtime() - t0, __builtin_amdgcn_s_memrealtime() - r0);
}

// two waves per SIMD with the matrix wave reading its operands from LDS,
// barrier per tile (LDS 1) ; the same with both kinds of work ping-ponging
// between the two waves every tile, as in the paired kernel (LDS 2)
template <int PP>
__global__ __launch_bounds__(512, 1) void two_waves_lds(const float* in, float* out, uint64_t* cyc, int iters) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  St s;
  init(s, in, lane);
  for (int i = threadIdx.x; i < 24 * 1024; i += 512) lds_pad[i] = in[i & 8191] * 1e-3f;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  if (!PP) {
    if (wave < 4) {
      for (int i = 0; i < 64; ++i) s.x[i] = 0.f;
      for (int i = 0; i < 32; ++i) s.pk[i] = 0;
      for (int it = 0; it < iters; ++it) { mfma_tile_lds(s, lane); __syncthreads(); }
    } else {
      s.c0 = f32x16{}; s.c1 = f32x16{}; s.c2 = f32x16{}; s.c3 = f32x16{};
      s.r0 = f32x4{}; s.r1 = f32x4{};
      for (int it = 0; it < iters; ++it) { valu_tile<0>(s); __syncthreads(); }
    }
  } else {
    const int par = wave >> 2;
    for (int it = 0; it < iters; it += 2) {
      if (par == 0) mfma_tile_lds(s, lane); else valu_tile<0>(s);
      __syncthreads();
      if (par == 1) mfma_tile_lds(s, lane); else valu_tile<0>(s);
      __syncthreads();
    }
  }
  finish(s, out, cyc, __builtin_amdgcn_s_memtime() - t0, __builtin_amdgcn_s_memrealtime() - r0);
}

// the role-swap variant plus the ring fills of the paired kernel: every wave
// issues two 16-byte-per-lane buffer loads into LDS per tile (8 KB of K and
// 8 KB of V per workgroup), into one of four 16 KB slots at 32 KB..96 KB
// that the products never read, and waits for those of four tiles ago
// (vmcnt(8)) before the barrier.  Source offsets wrap with a mask (src_bytes
// is a power of two): a modulo by the run-time size would add an integer
// division's worth of vector instructions per tile to both waves.
template <int TWO>
__global__ __launch_bounds__(512, 1) void two_waves_fill(const float* in, float* out, uint64_t* cyc, int iters,
                                                        const void* src, int src_bytes) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  St s;
  init(s, in, lane);
  for (int i = threadIdx.x; i < 8 * 1024; i += 512) lds_pad[i] = in[i & 8191] * 1e-3f;
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), (short)0, src_bytes, 0x00020000u);
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds_void_ptr() + 32768u;
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const int par = wave >> 2;
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = it + h;
      const uint32_t slot = lds0 + (uint32_t)(t & 3) * 16384u + 1024u * wave;
      const uint32_t goff = ((uint32_t)t * 16384u + 1024u * wave + 16u * lane) & ((uint32_t)src_bytes - 1u);
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" :: "s"(__builtin_amdgcn_readfirstlane(slot)), "v"(goff), "s"(rs) : "memory");
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" :: "s"(__builtin_amdgcn_readfirstlane(slot + 8192u)), "v"(goff + 8192u), "s"(rs) : "memory");
      if (par == h) mfma_tile_lds(s, lane); else valu_tile<0>(s);
      if (!TWO || h == 1) {
        __builtin_amdgcn_s_waitcnt(0x0F70 | 8);
        __syncthreads();
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  finish(s, out, cyc, __builtin_amdgcn_s_memtime() - t0, __builtin_amdgcn_s_memrealtime() - r0);
}

static const void* g_src = nullptr;
static int g_src_bytes = 0;
template <typename F>
void run(const char* name, F kern, float* din, float* dout, uint64_t* dcyc, int threads, bool fill = false) {
  const int iters = 2000, grid = 256;
  double best = 1e30, best_clk = 0;
  for (int rep = 0; rep < 4; ++rep) {
    if constexpr (std::is_same<F, void (*)(const float*, float*, uint64_t*, int, const void*, int)>::value)
      hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, 0, din, dout, dcyc, iters, g_src, g_src_bytes);
    else
      hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, 0, din, dout, dcyc, iters);
    (void)hipDeviceSynchronize();
    std::vector<uint64_t> cyc(grid * 16);
    (void)hipMemcpy(cyc.data(), dcyc, cyc.size() * 8, hipMemcpyDeviceToHost);
    double c = 0, r = 0; int n = 0;
    for (int g = 0; g < grid; ++g) for (int w = 0; w < threads / 64; ++w) { c += cyc[2 * (g * 8 + w)]; r += cyc[2 * (g * 8 + w) + 1]; ++n; }
    c /= n; r /= n;  // s_memrealtime runs at 100 MHz
    const double per = c / iters;
    if (rep > 0 && per < best) { best = per; best_clk = c / (r * 10.0) ; }
  }
  printf("%-58s %7.0f clocks per tile per SIMD (clock %.2f GHz)\n", name, best, best_clk);
}

int main() {
  float *din, *dout; uint64_t* dcyc;
  (void)hipMalloc(&din, 8192 * 4); (void)hipMalloc(&dout, 256 * 512 * 4); (void)hipMalloc(&dcyc, 256 * 16 * 8);
  std::vector<float> h(8192); for (int i = 0; i < 8192; ++i) h[i] = (float)((i * 37) % 101) / 101.f;
  (void)hipMemcpy(din, h.data(), 8192 * 4, hipMemcpyHostToDevice);
  run("one wave per SIMD: matrix work only", one_wave<0, 4, 0>, din, dout, dcyc, 256);
  run("one wave per SIMD: vector work only", one_wave<1, 4, 0>, din, dout, dcyc, 256);
  run("one wave per SIMD: vector work only, exp2 -> multiply", one_wave<1, 4, 1>, din, dout, dcyc, 256);
  run("one wave per SIMD: both, interleaved 1 MFMA : 3 VALU", one_wave<2, 3, 0>, din, dout, dcyc, 256);
  run("one wave per SIMD: both, interleaved 1 MFMA : 4 VALU", one_wave<2, 4, 0>, din, dout, dcyc, 256);
  run("one wave per SIMD: both, interleaved 1 MFMA : 5 VALU", one_wave<2, 5, 0>, din, dout, dcyc, 256);
  run("one wave per SIMD: both, 1:4, exp2 -> multiply", one_wave<2, 4, 1>, din, dout, dcyc, 256);
  run("two waves per SIMD: one matrix, one vector, free-running", two_waves<0, 0>, din, dout, dcyc, 512);
  run("two waves per SIMD: one matrix, one vector, barrier per tile", two_waves<1, 0>, din, dout, dcyc, 512);
  run("two waves per SIMD: free-running, exp2 -> multiply", two_waves<0, 1>, din, dout, dcyc, 512);
  run("two waves per SIMD: matrix operands from LDS, barrier per tile", two_waves_lds<0>, din, dout, dcyc, 512);
  run("two waves per SIMD: LDS operands, roles swap every tile", two_waves_lds<1>, din, dout, dcyc, 512);
  void* src; g_src_bytes = 64 << 20; (void)hipMalloc(&src, g_src_bytes); (void)hipMemset(src, 0, g_src_bytes); g_src = src;
  g_src_bytes = 2 << 20;
  run("two waves per SIMD: LDS operands, swap, ring fills", two_waves_fill<0>, din, dout, dcyc, 512);
  run("  ... barrier every two tiles", two_waves_fill<1>, din, dout, dcyc, 512);
  return 0;
}
