// Roof probes, the yardsticks the hot-path kernels are measured against:
// * memory: a plain device copy.  Each thread moves eight 16-byte pieces,
//   256 threads apart (every load instruction of a wave covers 1 KB of
//   consecutive bytes), with nontemporal loads and stores as the decode step's
//   state stream uses; all eight loads are issued before the first store.
// * matrix: a loop of v_mfma_f32_16x16x32_bf16 (the prefill's product) over
//   eight independent accumulators per wave, so the matrix pipe never waits on
//   a result; the accumulators are stored at the end.
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

constexpr int kMfmaAcc = 8;  // independent accumulator chains per wave

__global__ __launch_bounds__(kThreads) void kda_mfma_probe_kernel(float* __restrict__ out, int iters) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * float((lane + e) & 7));
    b[e] = (__bf16)(0.001f * float((lane * 3 + e) & 7));
  }
  f32x4v acc[kMfmaAcc];
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j) acc[j] = f32x4v{0.f, 0.f, 0.f, 0.f};
  // four rounds per loop trip: a loop-carried chain per round let the register
  // allocator shuffle the accumulators between trips
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < kMfmaAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  f32x4v sum = acc[0];
#pragma unroll
  for (int j = 1; j < kMfmaAcc; ++j) sum += acc[j];
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  *reinterpret_cast<float4*>(out + 4 * i) = make_float4(sum[0], sum[1], sum[2], sum[3]);
}

}  // namespace

hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(kda_mfma_probe_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, out, iters);
  return hipGetLastError();
}

int64_t mfma_probe_flops(int blocks, int iters) {
  // per wave and iteration: kMfmaAcc products of 16 x 16 x 32, 2 flops each
  return int64_t(blocks) * (kThreads / 64) * ((iters + 3) / 4 * 4) * kMfmaAcc * (16 * 16 * 32 * 2);
}

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
