// Memory-roof probe: a plain device copy, the yardstick the state-streaming
// kernels (decode, commit) are measured against.  Each thread moves eight
// 16-byte pieces, 256 threads apart (every load instruction of a wave covers
// 1 KB of consecutive bytes), with nontemporal loads and stores as the decode
// step's state stream uses; all eight loads are issued before the first store.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kPieces = 8;

__global__ __launch_bounds__(kThreads) void kda_copy_probe_kernel(const f32x4* __restrict__ src,
                                                                  f32x4* __restrict__ dst, int64_t n4) {
  const int64_t first = int64_t(blockIdx.x) * (kThreads * kPieces);
  const int64_t base = first + threadIdx.x;
  f32x4 r[kPieces];
  if (first + kThreads * kPieces <= n4) {
    // a whole block: straight-line loads, then stores
#pragma unroll
    for (int j = 0; j < kPieces; ++j) r[j] = __builtin_nontemporal_load(src + base + int64_t(j) * kThreads);
#pragma unroll
    for (int j = 0; j < kPieces; ++j) __builtin_nontemporal_store(r[j], dst + base + int64_t(j) * kThreads);
    return;
  }
  // the partial last block
  for (int j = 0; j < kPieces; ++j) {
    const int64_t i = base + int64_t(j) * kThreads;
    if (i < n4) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
  }
}

}  // namespace

hipError_t launch_copy_probe(const float* src, float* dst, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;
  const int64_t per_block = int64_t(kThreads) * kPieces;
  const int64_t blocks = (n4 + per_block - 1) / per_block;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(kda_copy_probe_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const f32x4*>(src), reinterpret_cast<f32x4*>(dst), n4);
  return hipGetLastError();
}

}  // namespace kda
