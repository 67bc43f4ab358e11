// Segment composition: the prefix scan over (M, S~) fragments.
//
// Each segment of a sequence is summarised by its transition M (the product of
// its per-token factors (I - beta k k^T) Diag(alpha)) and the state S~ it
// builds from a zero entry state; the true entry state of the next segment is
// S_in(i+1) = M(i) S_in(i) + S~(i) ("Kimi K3 的训练与 Serving Infra：KDA 换掉
// attention 后，系统要重做什么", sections 4.1-4.2, KCP).
//
// Value columns are independent (column j of S_in(i+1) uses only column j of
// S_in(i) and of S~(i)), so a workgroup owns one (head, 16-column slice) and
// runs the scan serially over segments; the current slice lives in LDS and
// each step is a 128 x 128 x 16 fp32 product with fixed summation order.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kCols = 16;           // columns per workgroup
constexpr int kThreads = 128;       // thread t: row t, all 16 columns

__global__ __launch_bounds__(kThreads) void kda_compose_kernel(const float* __restrict__ M,
                                                               const float* __restrict__ S_tilde,
                                                               const float* __restrict__ S_in0,
                                                               float* __restrict__ S_in,
                                                               float* __restrict__ S_final, int n_seg,
                                                               int H) {
  __shared__ float cur[kD][kCols + 1];
  const int slice = blockIdx.x % (kD / kCols);
  const int h = blockIdx.x / (kD / kCols);
  const int r = threadIdx.x;
  const int c0 = slice * kCols;
  const int64_t tile = int64_t(kD) * kD;

  float s[kCols];
#pragma unroll
  for (int j = 0; j < kCols; ++j) s[j] = S_in0 ? S_in0[h * tile + r * kD + c0 + j] : 0.0f;

  for (int i = 0; i < n_seg; ++i) {
    const int64_t base = (int64_t(i) * H + h) * tile;
    float* out = S_in + base + r * kD + c0;
#pragma unroll
    for (int j = 0; j < kCols; j += 4) st_f4(out + j, make_float4(s[j], s[j + 1], s[j + 2], s[j + 3]));
#pragma unroll
    for (int j = 0; j < kCols; ++j) cur[r][j] = s[j];
    __syncthreads();
    float acc[kCols];
    const float* st = S_tilde + base + r * kD + c0;
#pragma unroll
    for (int j = 0; j < kCols; j += 4) {
      const float4 w = ld_f4(st + j);
      acc[j] = w.x; acc[j + 1] = w.y; acc[j + 2] = w.z; acc[j + 3] = w.w;
    }
    const float* Mrow = M + base + int64_t(r) * kD;
    for (int c = 0; c < kD; c += 4) {
      const float4 m = ld_f4(Mrow + c);
      const float mv[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int j = 0; j < kCols; ++j) acc[j] = fmaf(mv[e], cur[c + e][j], acc[j]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kCols; ++j) s[j] = acc[j];
  }
  if (S_final) {
    float* out = S_final + h * tile + r * kD + c0;
#pragma unroll
    for (int j = 0; j < kCols; j += 4) st_f4(out + j, make_float4(s[j], s[j + 1], s[j + 2], s[j + 3]));
  }
}

}  // namespace

hipError_t launch_compose(const float* M, const float* S_tilde, const float* S_in0, float* S_in,
                          float* S_final, int n_seg, int H, hipStream_t stream) {
  const unsigned blocks = unsigned(H * (kD / kCols));
  hipLaunchKernelGGL(kda_compose_kernel, dim3(blocks), dim3(kThreads), 0, stream, M, S_tilde, S_in0,
                     S_in, S_final, n_seg, H);
  return hipGetLastError();
}

}  // namespace kda
