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
// runs the scan serially over segments.  Each step is a 128 x 128 x 16 fp32
// product on fp32 MFMA (v_mfma_f32_16x16x4_f32, exact products, fp32
// accumulation): wave w of eight computes output rows 16w .. 16w+15 as one
// 16 x 16 tile.  Lane group q takes the contraction indices k = 16j + 4q + e
// (j = 0..7, e = 0..3), so one load of the four groups covers 64 contiguous
// bytes of an M row; the running state is kept transposed in LDS.  Two
// accumulator chains per tile (even and odd e) halve the dependent MFMA
// latency; their sum is taken in a fixed order, so results are deterministic.
// The next two segments' M rows and S~ values are in flight in two further
// register sets while the current product runs (twelve loads per set and
// wave, well inside the wave's outstanding-load counter).
#include "kda_common.hpp"
#include "kda_internal.hpp"
#include "kda_mfma.hpp"

namespace kda {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kCols = 16;            // columns per workgroup
constexpr int kThreads = 512;        // 8 waves x 16 output rows

// One segment's operands as this lane uses them: eight 4-float pieces of its M
// row (its contraction indices) and the S~ values its accumulators start from.
struct SegOps {
  float4 a[8];
  float st[4];
};

__device__ __forceinline__ void load_seg(SegOps& x, const float* __restrict__ M, const float* __restrict__ S_tilde,
                                         int64_t base, int wave, int q, int n, int c0) {
  const float* arow = M + base + int64_t(wave * 16 + n) * kD + 4 * q;
#pragma unroll
  for (int s4 = 0; s4 < 8; ++s4) x.a[s4] = ld_f4(arow + 16 * s4);
  const int row = wave * 16 + 4 * q;
#pragma unroll
  for (int e = 0; e < 4; ++e) x.st[e] = S_tilde[base + int64_t(row + e) * kD + c0 + n];
}

__global__ __launch_bounds__(kThreads) void kda_compose_kernel(const float* __restrict__ M,
                                                               const float* __restrict__ S_tilde,
                                                               const float* __restrict__ S_in0,
                                                               float* __restrict__ S_in,
                                                               float* __restrict__ S_final, int n_seg,
                                                               int H) {
  // Workgroups are numbered so that the 8 slices of a head share blockIdx % 8
  // (one XCD, one L2 for the head's M): id = (h / 8) * 64 + slice * 8 + h % 8.
  const int id = blockIdx.x;
  const int slice = (id >> 3) & 7;
  const int h = (id >> 6) * 8 + (id & 7);
  if (h >= H) return;
  __shared__ __align__(16) float curT[kCols][kD + 4];  // running S_in slice, transposed: [column][row]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4;   // contraction group / output row group
  const int n = lane & 15;   // output column within the slice; A-operand row within a tile
  const int c0 = slice * kCols;
  const int64_t tile = int64_t(kD) * kD;

  // entry state of segment 0
  for (int e = tid; e < kD * kCols; e += kThreads) {
    const int r = e / kCols, c = e % kCols;
    curT[c][r] = S_in0 ? S_in0[h * tile + int64_t(r) * kD + c0 + c] : 0.0f;
  }
  __syncthreads();

  // publish S_in(i) (S_final for i == n_seg) from LDS
  auto publish = [&](int i) {
    float* dst = (i < n_seg) ? S_in + (int64_t(i) * H + h) * tile : S_final ? S_final + h * tile : nullptr;
    if (dst != nullptr) {
      for (int e = tid; e < kD * kCols / 4; e += kThreads) {
        const int r = e / (kCols / 4), c4 = 4 * (e % (kCols / 4));
        st_f4(dst + int64_t(r) * kD + c0 + c4, make_float4(curT[c4][r], curT[c4 + 1][r], curT[c4 + 2][r], curT[c4 + 3][r]));
      }
    }
  };
  // S_in(i+1) = M(i) S_in(i) + S~(i) into curT, from operands x
  auto advance = [&](const SegOps& x) {
    f32x4v acc[2];
    acc[0] = f32x4v{x.st[0], x.st[1], x.st[2], x.st[3]};
    acc[1] = f32x4v{0.f, 0.f, 0.f, 0.f};
    const float* bcol = &curT[n][4 * q];
#pragma unroll
    for (int s4 = 0; s4 < 8; ++s4) {
      const float4 b = *reinterpret_cast<const float4*>(bcol + 16 * s4);
      const float bv[4] = {b.x, b.y, b.z, b.w};
      const float av[4] = {x.a[s4].x, x.a[s4].y, x.a[s4].z, x.a[s4].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[e & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc[e & 1], 0, 0, 0);
    }
    __syncthreads();  // every wave has read S_in(i) from LDS
    {
      const int row = wave * 16 + 4 * q;
      const f32x4v v = acc[0] + acc[1];
      *reinterpret_cast<float4*>(&curT[n][row]) = make_float4(v[0], v[1], v[2], v[3]);
    }
    __syncthreads();
  };

  // Segment i's operands are loaded two segments ahead, while segments i - 2
  // and i - 1 are composed (three register sets used in turn; indices past
  // the last segment repeat it): one segment of prefetch distance left the
  // global-load latency exposed at every step.
  SegOps X0, X1, X2;
  const int last = n_seg > 0 ? n_seg - 1 : 0;
  auto seg_base = [&](int i) { return (int64_t(i <= last ? i : last) * H + h) * tile; };
  if (n_seg > 0) {
    load_seg(X0, M, S_tilde, seg_base(0), wave, q, n, c0);
    load_seg(X1, M, S_tilde, seg_base(1), wave, q, n, c0);
  }
  // The loop body is straight-line (every phase loads and composes, a phase
  // past the last segment recomputes into LDS what nobody reads), so the
  // compiler's wait counts see each set's loads issued two phases before use.
  int i = 0;
  for (; i < n_seg; i += 3) {
    publish(i);
    load_seg(X2, M, S_tilde, seg_base(i + 2), wave, q, n, c0);
    advance(X0);
    if (i + 1 <= n_seg) publish(i + 1);
    load_seg(X0, M, S_tilde, seg_base(i + 3), wave, q, n, c0);
    advance(X1);
    if (i + 2 <= n_seg) publish(i + 2);
    load_seg(X1, M, S_tilde, seg_base(i + 4), wave, q, n, c0);
    advance(X2);
  }
  if (i == n_seg) publish(n_seg);
}

// Staged variant for grids that leave CUs idle (at most one workgroup per CU:
// its LDS holds two copies of M): each segment's M is loaded with coalesced
// 16-byte loads after the current product's MFMAs were issued, written to the
// free LDS buffer while the step's products run, and read from LDS as the A
// operand in the next; the contraction slots and their order are those of
// kda_compose_kernel, so both give the same bits.  The loads leave the matrix
// section, which measured 2.0-2.1 us per step against 2.5 us (1.93 us with the
// staging ahead of the step's first barrier).
constexpr int kMLd = kD + 4;         // LDS row stride of a staged M (floats)
constexpr int kMPieces = kD * kD / 4 / kThreads;  // float4 pieces of M per thread (8)

__global__ __launch_bounds__(kThreads) void kda_compose_staged_kernel(const float* __restrict__ M,
                                                               const float* __restrict__ S_tilde,
                                                               const float* __restrict__ S_in0,
                                                               float* __restrict__ S_in,
                                                               float* __restrict__ S_final, int n_seg,
                                                               int H) {
  const int id = blockIdx.x;  // numbered as in kda_compose_kernel
  const int slice = (id >> 3) & 7;
  const int h = (id >> 6) * 8 + (id & 7);
  if (h >= H) return;
  __shared__ __align__(16) float curT[kCols][kD + 4];  // running S_in slice, transposed: [column][row]
  __shared__ __align__(16) float Ms[2][kD][kMLd];       // M of the current and the next segment

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int c0 = slice * kCols;
  const int64_t tile = int64_t(kD) * kD;
  const int last = n_seg > 0 ? n_seg - 1 : 0;
  auto seg_base = [&](int i) { return (int64_t(i <= last ? i : last) * H + h) * tile; };
  const int row = wave * 16 + 4 * q;  // this lane's output rows row .. row + 3, column c0 + n

  // M pieces: thread t takes float4 e = t + 512 j (rows 4 j .. , columns 4 (t % 32))
  float4 mr[kMPieces];
  auto load_m = [&](int i) {
    const float* src = M + seg_base(i);
#pragma unroll
    for (int j = 0; j < kMPieces; ++j) mr[j] = ld_f4(src + 4 * (tid + kThreads * j));
  };
  auto store_m = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kMPieces; ++j) {
      const int e = tid + kThreads * j;
      *reinterpret_cast<float4*>(&Ms[buf][e >> 5][4 * (e & 31)]) = mr[j];
    }
  };
  float st[4];
  auto load_st = [&](int i) {
    const int64_t b = seg_base(i);
#pragma unroll
    for (int e = 0; e < 4; ++e) st[e] = S_tilde[b + int64_t(row + e) * kD + c0 + n];
  };

  // entry state of segment 0, and M(0) into LDS
  for (int e = tid; e < kD * kCols; e += kThreads) {
    const int r = e / kCols, c = e % kCols;
    curT[c][r] = S_in0 ? S_in0[h * tile + int64_t(r) * kD + c0 + c] : 0.0f;
  }
  if (n_seg > 0) {
    load_m(0);
    store_m(0);
    load_st(0);
    load_m(1);
  }
  __syncthreads();

  auto publish = [&](int i) {
    float* dst = (i < n_seg) ? S_in + (int64_t(i) * H + h) * tile : S_final ? S_final + h * tile : nullptr;
    static_assert(kD * kCols / 4 == kThreads, "one 16-byte piece of the slice per thread");
    if (dst != nullptr) {
      const int r = tid / (kCols / 4), c4 = 4 * (tid % (kCols / 4));
      st_f4(dst + int64_t(r) * kD + c0 + c4, make_float4(curT[c4][r], curT[c4 + 1][r], curT[c4 + 2][r], curT[c4 + 3][r]));
    }
  };

  for (int i = 0; i < n_seg; ++i) {
    publish(i);
    // S_in(i+1) = M(i) S_in(i) + S~(i): A from Ms[i % 2], B from curT
    f32x4v acc[2];
    acc[0] = f32x4v{st[0], st[1], st[2], st[3]};
    acc[1] = f32x4v{0.f, 0.f, 0.f, 0.f};
    const float* arow = &Ms[i & 1][wave * 16 + n][4 * q];
    const float* bcol = &curT[n][4 * q];
#pragma unroll
    for (int s4 = 0; s4 < 8; ++s4) {
      const float4 a4 = *reinterpret_cast<const float4*>(arow + 16 * s4);
      const float4 b4 = *reinterpret_cast<const float4*>(bcol + 16 * s4);
      const float av[4] = {a4.x, a4.y, a4.z, a4.w};
      const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[e & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc[e & 1], 0, 0, 0);
    }
    // while the products run: M(i+1) (loaded during step i - 1) into the other
    // buffer (last read in step i - 1, before its closing barrier); then the
    // next loads
    store_m((i + 1) & 1);
    load_st(i + 1);
    __builtin_amdgcn_sched_barrier(0);  // S~ loads first: the next step waits only for them
    load_m(i + 2);
    __syncthreads();  // every wave has read S_in(i) and M(i), and stored its part of M(i + 1)
    {
      const f32x4v v = acc[0] + acc[1];
      *reinterpret_cast<float4*>(&curT[n][row]) = make_float4(v[0], v[1], v[2], v[3]);
    }
    __syncthreads();
  }
  publish(n_seg);
}

// Split-operand variant (bf16 inputs' precision class): the same scan with
// each step's products on bf16 MFMA (v_mfma_f32_16x16x32_bf16).  Both operands
// are split as x = hi + lo (hi = bf16(x), lo = bf16(x - hi)) and a product is
// hi*hi + hi*lo + lo*hi with fp32 accumulation, about 16 significant bits per
// operand: three 32-deep MFMAs do the work of sixteen 4-deep fp32 ones, ~5x
// the matrix rate.  M is staged through LDS as in the fp32 staged kernel, split
// into a hi and a lo plane when written there, with its global loads two steps
// ahead (two register sets); the running state is kept in fp32 (for
// the published entry states) and as hi/lo planes (the B operand).  Lane group
// q takes the contraction indices k = 32 s + 8 q + e (s = 0..3, e = 0..7), one
// 16-byte read per plane and operand.  Three accumulators (one per part, the
// S~ values in the first) are summed as acc0 + (acc1 + acc2).  A step measured
// 1.74 us against 1.93 us for the fp32 staged kernel: at this size it is bound
// by moving M (64 KB per step through the load path and LDS), not by the
// matrix rate.  LDS: 153 KB, one workgroup per CU; larger grids run in rounds.
constexpr int kHRow = (kD + 8) * 2;          // bytes per row of a bf16 plane (272: rows 4 banks apart)
constexpr int kMPlane = kD * kHRow;          // one plane of a staged M
constexpr int kBPlane = kCols * kHRow;       // one plane of the running slice, [column][row]

// One step's global operands as this thread holds them: its eight 16-byte
// pieces of the next M (staged into LDS at the end of the step) and the S~
// values its accumulators start from.
struct StepOps {
  float4 m[kMPieces];
  float st[4];
};

__global__ __launch_bounds__(kThreads) void kda_compose_split_kernel(const float* __restrict__ M,
                                                                    const float* __restrict__ S_tilde,
                                                                    const float* __restrict__ S_in0,
                                                                    float* __restrict__ S_in,
                                                                    float* __restrict__ S_final, int n_seg,
                                                                    int H) {
  const int id = blockIdx.x;  // numbered as in kda_compose_kernel
  const int slice = (id >> 3) & 7;
  const int h = (id >> 6) * 8 + (id & 7);
  if (h >= H) return;
  __shared__ __align__(16) float curT[kCols][kD + 4];  // running S_in slice, fp32, [column][row]
  __shared__ __align__(16) char curB[2 * kBPlane];     // the same as hi and lo planes
  __shared__ __align__(16) char Ms[2][2 * kMPlane];    // M of the current and the next segment, hi and lo planes

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int c0 = slice * kCols;
  const int64_t tile = int64_t(kD) * kD;
  const int last = n_seg > 0 ? n_seg - 1 : 0;
  auto seg_base = [&](int i) { return (int64_t(i <= last ? i : last) * H + h) * tile; };
  const int row = wave * 16 + 4 * q;  // this lane's output rows row .. row + 3, column c0 + n

  // step i reads S~(i) and stages M(i + 1): both are loaded two steps ahead,
  // S~ first, so that a step waits only for the loads of the step before it
  auto load_ops = [&](StepOps& x, int i) {
    const int64_t b = seg_base(i);
#pragma unroll
    for (int e = 0; e < 4; ++e) x.st[e] = S_tilde[b + int64_t(row + e) * kD + c0 + n];
    __builtin_amdgcn_sched_barrier(0);
    const float* src = M + seg_base(i + 1);
#pragma unroll
    for (int j = 0; j < kMPieces; ++j) x.m[j] = ld_f4(src + 4 * (tid + kThreads * j));
  };
  auto store_m = [&](const float4* m, int buf) {
#pragma unroll
    for (int j = 0; j < kMPieces; ++j) {
      const int e = tid + kThreads * j;
      const float v[4] = {m[j].x, m[j].y, m[j].z, m[j].w};
      PolBF16x3::store4(Ms[buf], kMPlane, (e >> 5) * kHRow + 8 * (e & 31), v);
    }
  };

  auto publish = [&](int i) {
    float* dst = (i < n_seg) ? S_in + (int64_t(i) * H + h) * tile : S_final ? S_final + h * tile : nullptr;
    if (dst != nullptr) {
      const int r = tid / (kCols / 4), c4 = 4 * (tid % (kCols / 4));
      st_f4(dst + int64_t(r) * kD + c0 + c4, make_float4(curT[c4][r], curT[c4 + 1][r], curT[c4 + 2][r], curT[c4 + 3][r]));
    }
  };
  for (int e = tid; e < kD * kCols; e += kThreads) {
    const int r = e / kCols, c = e % kCols;
    const float x = S_in0 ? S_in0[h * tile + int64_t(r) * kD + c0 + c] : 0.0f;
    curT[c][r] = x;
    PolBF16x3::store1(curB, kBPlane, c * kHRow + 2 * r, x);
  }
  // From a zero entry state the first step is S_in(1) = M(0) 0 + S~(0) = S~(0):
  // publish the zeros as S_in(0) and start from S~(0) at step 1.
  const int i0 = (S_in0 == nullptr && n_seg > 0) ? 1 : 0;
  if (i0 == 1) {
    __syncthreads();
    publish(0);
    __syncthreads();
    for (int e = tid; e < kD * kCols; e += kThreads) {
      const int r = e / kCols, c = e % kCols;
      const float x = S_tilde[seg_base(0) + int64_t(r) * kD + c0 + c];
      curT[c][r] = x;
      PolBF16x3::store1(curB, kBPlane, c * kHRow + 2 * r, x);
    }
  }
  StepOps X0, X1;
  if (n_seg > 0) {
    float4 m0[kMPieces];
    const float* src = M + seg_base(i0);
#pragma unroll
    for (int j = 0; j < kMPieces; ++j) m0[j] = ld_f4(src + 4 * (tid + kThreads * j));
    store_m(m0, i0 & 1);
    load_ops(X0, i0);
    load_ops(X1, i0 + 1);
  }
  __syncthreads();

  // S_in(i+1) = M(i) S_in(i) + S~(i), then M(i + 1) into the other buffer and
  // the operands of step i + 2 into x (indices past the last segment repeat it)
  auto step = [&](int i, StepOps& x) {
    publish(i);
    f32x4_t acc[3];
    acc[0] = f32x4_t{x.st[0], x.st[1], x.st[2], x.st[3]};
    acc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc[2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    PolBF16x3::Frag fa[4], fb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      fa[s] = PolBF16x3::load(Ms[i & 1], kMPlane, (wave * 16 + n) * kHRow + 2 * (32 * s + 8 * q));
      fb[s] = PolBF16x3::load(curB, kBPlane, n * kHRow + 2 * (32 * s + 8 * q));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int p = 0; p < 3; ++p) PolBF16x3::mma_part(acc[p], fa[s], fb[s], p);
    // while the products run: M(i + 1) into the other buffer (last read in
    // step i - 1, before its closing barrier), then step i + 2's loads
    store_m(x.m, (i + 1) & 1);
    load_ops(x, i + 2);
    __syncthreads();  // every wave has read S_in(i) and M(i), and stored its part of M(i + 1)
    {
      const f32x4_t v = acc[0] + (acc[1] + acc[2]);
      const float vv[4] = {v[0], v[1], v[2], v[3]};
      *reinterpret_cast<float4*>(&curT[n][row]) = make_float4(v[0], v[1], v[2], v[3]);
      PolBF16x3::store4(curB, kBPlane, n * kHRow + 2 * row, vv);
    }
    __syncthreads();
  };
  // unrolled by two so that the two operand sets keep fixed registers (the
  // body is straight-line; an odd count ends with one more step)
  int i = i0;
  for (; i + 1 < n_seg; i += 2) {
    step(i, X0);
    step(i + 1, X1);
  }
  if (i < n_seg) step(i, X0);
  publish(n_seg);
}

}  // namespace

hipError_t launch_compose(const float* M, const float* S_tilde, const float* S_in0, float* S_in,
                          float* S_final, int n_seg, int H, bool split_operands, hipStream_t stream) {
  const unsigned blocks = unsigned(((H + 7) / 8) * 64);
  if (split_operands)
    hipLaunchKernelGGL(kda_compose_split_kernel, dim3(blocks), dim3(kThreads), 0, stream, M, S_tilde, S_in0,
                       S_in, S_final, n_seg, H);
  else if (int64_t(blocks) <= device_cu_count())
    hipLaunchKernelGGL(kda_compose_staged_kernel, dim3(blocks), dim3(kThreads), 0, stream, M, S_tilde, S_in0,
                       S_in, S_final, n_seg, H);
  else
    hipLaunchKernelGGL(kda_compose_kernel, dim3(blocks), dim3(kThreads), 0, stream, M, S_tilde, S_in0,
                       S_in, S_final, n_seg, H);
  return hipGetLastError();
}

}  // namespace kda
