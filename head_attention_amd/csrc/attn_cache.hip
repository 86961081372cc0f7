// KV-cache append of attn_cache_append: the cache update that precedes a
// decode step ("Attention Is All You Need 해부", KV cache section: a step's
// cache holds tokens 0..t-1 plus the new token's K, V).
//
// A pure copy, bound by memory: each thread moves one 16-byte chunk of a new
// K row and the same chunk of the new V row (8 threads per bf16 row, 16 per
// fp32 row), so a wave covers 8 (bf16) or 4 (fp32) whole rows with 16-byte
// loads and stores.  Row r of the block of (b, h) lands in cache row
// kv_lens[b] - n_new + r; a destination outside [0, n_max) is skipped, so a
// bad length can never write out of bounds.
#include "common.h"

namespace headattn {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void cache_append_kernel(AppendArgs a) {
  const int chunks_per_row = a.row_bytes / 16;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.H * a.n_new * chunks_per_row;
  if (gid >= total) return;
  const int64_t row = gid / chunks_per_row;  // (b, h, r) row of the new block
  const int ch = (int)(gid - row * chunks_per_row);
  const int r = (int)(row % a.n_new);
  const int64_t bh = row / a.n_new;
  const int b = (int)(bh / a.H);
  const int64_t dst = (int64_t)a.kv_lens[b] - a.n_new + r;
  if (dst < 0 || dst >= a.n_max) return;
  const int64_t src_off = row * a.row_bytes + 16 * ch;
  const int64_t dst_off = (bh * a.n_max + dst) * a.row_bytes + 16 * ch;
  const uint4 k = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.Kn) + src_off);
  const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.Vn) + src_off);
  *reinterpret_cast<uint4*>(static_cast<char*>(a.Kc) + dst_off) = k;
  *reinterpret_cast<uint4*>(static_cast<char*>(a.Vc) + dst_off) = v;
}

}  // namespace

hipError_t launch_cache_append(const AppendArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.H * a.n_new * (a.row_bytes / 16);
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  AppendArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&cache_append_kernel), dim3((unsigned)blocks),
                         dim3(kThreads), kargs, 0, s);
}

}  // namespace headattn
