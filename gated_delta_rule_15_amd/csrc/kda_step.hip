// Decode step, draft-block verify and replay commit for the KDA recurrence.
//
// One token of the recurrence, in the gate-then-delta split given in the math
// box of "Kimi K3：架构与 SGLang Day-0 Support", section "attention 机制详解：KDA":
//     S~ = Diag(alpha) S;  r = S~^T k;  u = beta (v - r);  S <- S~ + k u^T
// and the readout o = S^T q after the write (section "linear attention" of the
// same page), computed as o = S~^T q + (q . k) u so that the state is streamed
// once.  Verify reads the committed state and never writes it; commit replays
// only the accepted prefix from that state in place ("SGLang 和 Miles 为 Kimi K3
// 提供首日支持", section "ReplaySSM：针对 KDA 状态的原始输入重放").
//
// These kernels are HBM streams of the fp32 state: a workgroup owns one
// (request, head, column slice) tile of 128 rows x COLS columns in registers;
// the column reductions r = S~^T k and s = S~^T q run in-thread over the
// thread's rows, then across lanes with wave shuffles, then across the four
// waves through 1.2 KB of LDS in a fixed order.  Decode, verify and commit call
// the same per-token routine with the same decomposition and no atomics, so a
// commit of L tokens is bit-identical to L decode steps and verify's o_t is
// bit-identical to the t-th of t decode steps.  This file is built with
// -ffp-contract=off and every multiply-add is an explicit fmaf.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int COLS>
struct TileMap {
  static constexpr int CG = COLS / 4;     // column groups of 4 columns
  static constexpr int RG = kThreads / CG; // row groups
  static constexpr int R = kD / RG;       // rows per thread
  static_assert(CG <= 64 && 64 % CG == 0, "column groups must tile a wave");
  static_assert(R % 4 == 0, "rows per thread must be a multiple of 4");
};

enum StepMode { kDecode = 0, kVerify = 1, kCommit = 2 };

struct StepArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* state_in;
  float* state_out;
  const int32_t* slots;
  const int32_t* accepted_len;
  void* o;
  int32_t N, G, H;
  float scale;
};

// Per-thread partial sums -> full column sums, identical in every thread that
// shares a column group.  red: LDS [kWaves][CG][NV].
template <int COLS, int NV>
__device__ __forceinline__ void reduce_columns(float (&x)[NV], float* red, int lane, int wave, int cg) {
  using M = TileMap<COLS>;
#pragma unroll
  for (int off = M::CG; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < NV; ++e) x[e] += __shfl_xor(x[e], off, 64);
  }
  if (lane < M::CG) {
#pragma unroll
    for (int e = 0; e < NV; ++e) red[(wave * M::CG + cg) * NV + e] = x[e];
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    float acc = red[(0 * M::CG + cg) * NV + e];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) acc += red[(w * M::CG + cg) * NV + e];
    x[e] = acc;
  }
}

// One token.  S: this thread's R x 4 state block (rows row0.., columns col..col+3).
// kk/qq/gg: the token's k, scale*q, g at this thread's rows; vv: v at its columns.
// READOUT additionally produces o at the thread's 4 columns.
template <int COLS, bool READOUT>
__device__ __forceinline__ void token_step(float (&S)[TileMap<COLS>::R][4],
                                           const float (&kk)[TileMap<COLS>::R],
                                           const float (&qq)[TileMap<COLS>::R],
                                           const float (&gg)[TileMap<COLS>::R], const float (&vv)[4],
                                           float beta, float* red, int lane, int wave, int cg,
                                           float (&o)[4]) {
  using M = TileMap<COLS>;
  constexpr int NV = READOUT ? 9 : 4;
  float acc[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int i = 0; i < M::R; ++i) {
    const float alpha = __expf(gg[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      S[i][j] = S[i][j] * alpha;                       // S~ = Diag(alpha) S (row scale)
      acc[j] = fmaf(kk[i], S[i][j], acc[j]);           // r = S~^T k
      if constexpr (READOUT) acc[4 + j] = fmaf(qq[i], S[i][j], acc[4 + j]);  // s = S~^T q
    }
    if constexpr (READOUT) acc[8] = fmaf(qq[i], kk[i], acc[8]);              // q . k
  }
  reduce_columns<COLS, NV>(acc, red, lane, wave, cg);
  float u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = beta * (vv[j] - acc[j]);
#pragma unroll
  for (int i = 0; i < M::R; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) S[i][j] = fmaf(kk[i], u[j], S[i][j]);  // S = S~ + k u^T
  }
  if constexpr (READOUT) {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = fmaf(acc[8], u[j], acc[4 + j]);  // o = s + (q.k) u
  }
}

template <int COLS, class InT, int MODE>
__global__ __launch_bounds__(kThreads) void kda_step_kernel(StepArgs a) {
  using M = TileMap<COLS>;
  constexpr int NS = kD / COLS;
  constexpr bool READOUT = (MODE != kCommit);
  __shared__ float red[2][kWaves * M::CG * 9];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cg = tid % M::CG;
  const int rg = tid / M::CG;
  const int row0 = rg * M::R;

  const int slice = blockIdx.x % NS;
  const int nh = blockIdx.x / NS;
  const int h = nh % a.H;
  const int n = nh / a.H;
  const int col = slice * COLS + cg * 4;

  int steps = a.G;
  if (MODE == kCommit) {
    const int L = a.accepted_len[n];
    steps = L < 0 ? 0 : (L > a.G ? a.G : L);
  }
  if (MODE == kDecode && a.o == nullptr) {
    // decode without readout still follows the same arithmetic for the state
  }
  const int64_t pool_row = a.slots ? int64_t(a.slots[n]) : int64_t(n);
  const int64_t tile = (pool_row * a.H + h) * int64_t(kD * kD);
  const float* Sin = a.state_in + tile;

  float S[M::R][4];
#pragma unroll
  for (int i = 0; i < M::R; ++i) {
    const float4 w = ld_f4(Sin + (row0 + i) * kD + col);
    S[i][0] = w.x; S[i][1] = w.y; S[i][2] = w.z; S[i][3] = w.w;
  }

  for (int t = 0; t < steps; ++t) {
    const int64_t tok = (int64_t(n) * a.G + t) * a.H + h;  // [N, G, H] token-head index
    const int64_t vec = tok * kD;
    float kk[M::R], qq[M::R], gg[M::R], vv[4];
#pragma unroll
    for (int i = 0; i < M::R; i += 4) {
      InT::load4(a.k, vec + row0 + i, &kk[i]);
      const float4 w = ld_f4(a.g + vec + row0 + i);
      gg[i] = w.x; gg[i + 1] = w.y; gg[i + 2] = w.z; gg[i + 3] = w.w;
      if constexpr (READOUT) {
        InT::load4(a.q, vec + row0 + i, &qq[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) qq[i + e] = qq[i + e] * a.scale;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) qq[i + e] = 0.0f;
      }
    }
    InT::load4(a.v, vec + col, vv);
    const float beta = a.beta[tok];
    float o[4];
    token_step<COLS, READOUT>(S, kk, qq, gg, vv, beta, red[t & 1], lane, wave, cg, o);
    if constexpr (READOUT) {
      if (rg == 0 && a.o != nullptr) InT::store4(a.o, vec + col, o);
    }
  }

  if constexpr (MODE != kVerify) {
    float* Sout = a.state_out + tile;
#pragma unroll
    for (int i = 0; i < M::R; ++i)
      st_f4(Sout + (row0 + i) * kD + col, make_float4(S[i][0], S[i][1], S[i][2], S[i][3]));
  }
}

template <int COLS, class InT, int MODE>
hipError_t launch_cols(const StepArgs& a, hipStream_t stream) {
  constexpr int NS = kD / COLS;
  const int64_t blocks = int64_t(a.N) * a.H * NS;
  hipLaunchKernelGGL((kda_step_kernel<COLS, InT, MODE>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <class InT, int MODE>
hipError_t launch_mode(const StepArgs& a, int cols, hipStream_t stream) {
  switch (cols) {
    case 128: return launch_cols<128, InT, MODE>(a, stream);
    case 64: return launch_cols<64, InT, MODE>(a, stream);
    default: return launch_cols<32, InT, MODE>(a, stream);
  }
}

template <int MODE>
hipError_t launch_step(const StepArgs& a, bool bf16, int cols, hipStream_t stream) {
  return bf16 ? launch_mode<BF16, MODE>(a, cols, stream) : launch_mode<F32, MODE>(a, cols, stream);
}

}  // namespace

// Column-slice width per workgroup: narrow enough that the grid has >= ~2048
// workgroups (8 per CU) so that every CU has several tiles in flight.
int step_cols_for(int64_t tiles) {
  if (tiles * 1 >= 2048) return 128;
  if (tiles * 2 >= 2048) return 64;
  return 32;
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         float* state, const int32_t* slots, int N, int H, bool bf16, float scale,
                         void* o, int cols, hipStream_t stream) {
  StepArgs a{q, k, v, g, beta, state, state, slots, nullptr, o, N, 1, H, scale};
  return launch_step<kDecode>(a, bf16, cols, stream);
}

hipError_t launch_verify(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* state, const int32_t* slots, int N, int G, int H, bool bf16,
                         float scale, void* o, int cols, hipStream_t stream) {
  StepArgs a{q, k, v, g, beta, state, nullptr, slots, nullptr, o, N, G, H, scale};
  return launch_step<kVerify>(a, bf16, cols, stream);
}

hipError_t launch_commit(const void* k, const void* v, const float* g, const float* beta,
                         const float* state_in, float* state_out, const int32_t* slots,
                         const int32_t* accepted_len, int N, int G, int H, bool bf16, int cols,
                         hipStream_t stream) {
  StepArgs a{nullptr, k, v, g, beta, state_in, state_out, slots, accepted_len, nullptr, N, G, H, 1.0f};
  return launch_step<kCommit>(a, bf16, cols, stream);
}

}  // namespace kda
