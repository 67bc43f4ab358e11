// Roof probes, the yardsticks the hot-path kernels are measured against:
// * memory: a plain device copy.  Each thread moves eight 16-byte pieces,
//   256 threads apart (every load instruction of a wave covers 1 KB of
//   consecutive bytes), with nontemporal loads and stores as the decode step's
//   state stream uses; all eight loads are issued before the first store.
// * memory in the decode step's pattern: the same bytes as a decode of n
//   states (each 128 x 128 fp32 read once and written once), in the decode
//   kernel's tiling and lane order but without its arithmetic, so the decode
//   can be compared with the copy rate of its own access pattern.
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

// One workgroup of four waves per (state, 64-column half), consecutive
// workgroups on the two halves of one state; wave w takes the 32-column slice
// w / 2 of its half and rows 64 (w % 2) .. 64 (w % 2) + 63; lane 8 rg + cg
// takes rows 8 rg .. 8 rg + 7 of those and columns 4 cg .. 4 cg + 3 of the
// slice, one 16-byte piece per row, so one load instruction of a wave covers
// eight 128-byte row segments.  All eight loads precede the stores; src may
// equal dst (each thread rewrites what it read).  DEP: no store is issued
// before every load of the workgroup has completed (a wait for the thread's
// loads, then a workgroup barrier), the ordering the decode step has (its
// stores need column sums over all 128 rows); otherwise each store follows
// its own load.
template <bool DEP>
__global__ __launch_bounds__(kThreads) void kda_copy_probe_state_kernel(const float* src, float* dst) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cg = lane & 7, rg = lane >> 3;
  const int64_t state = blockIdx.x >> 1;
  const int col = 64 * int(blockIdx.x & 1) + 32 * (wave >> 1) + 4 * cg;
  const int row0 = 64 * (wave & 1) + 8 * rg;
  const int64_t off = state * (128 * 128) + int64_t(row0) * 128 + col;
  const f32x4* s = reinterpret_cast<const f32x4*>(src + off);
  f32x4* d = reinterpret_cast<f32x4*>(dst + off);
  f32x4 r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = __builtin_nontemporal_load(s + i * 32);  // row stride: 32 pieces
  if constexpr (DEP) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) __builtin_nontemporal_store(r[i], d + i * 32);
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

hipError_t launch_copy_probe_state(const float* src, float* dst, int64_t n_states, bool dependent,
                                   hipStream_t stream) {
  if (n_states <= 0) return hipSuccess;
  if (dependent)
    hipLaunchKernelGGL(kda_copy_probe_state_kernel<true>, dim3(unsigned(2 * n_states)), dim3(kThreads), 0, stream,
                       src, dst);
  else
    hipLaunchKernelGGL(kda_copy_probe_state_kernel<false>, dim3(unsigned(2 * n_states)), dim3(kThreads), 0, stream,
                       src, dst);
  return hipGetLastError();
}

}  // namespace kda
