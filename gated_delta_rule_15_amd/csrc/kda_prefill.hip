// Chunk-parallel prefill of the KDA recurrence on gfx950 MFMA.
//
// Math (the update is from "Kimi K3：架构与 SGLang Day-0 Support",
// section "attention 机制详解：KDA"; the chunkwise form rescales keys by the
// inverse cumulative decay, as remarked in the same math box).  For a chunk of
// n <= 64 tokens with entry state S (128 x 128, rows = key channels) and
// b_r = sum_{s<=r} g_s per key channel:
//   Kh = K e^{b}, Kc = K e^{-b}, Qh = scale Q e^{b}, Kb = K e^{b_last - b}
//   A  = strict_lower(diag(beta) Kh Kc^T)          (n x n)
//   P  = lower(Qh Kc^T)                            (n x n)
//   T' = (I + A)^{-1} diag(beta)                   (UT / WY factor, n x n)
//   U  = T' (V - Kh S)                             (n x d_v)
//   O  = Qh S + P U                                (n x d_v)
//   S <- Diag(e^{b_last}) S + Kb^T U
// which is the WY form of the chunk's product of (I - beta k k^T) Diag(alpha)
// factors.  The transition M of a sequence is the same pass run from S = I
// with V = 0 and no outputs.
//
// Decomposition.  A workgroup (4 waves) owns one (sequence, head, column
// slice) and walks the sequence's chunks in order.  Each wave owns 16*JB
// value columns of the state, held in MFMA accumulator registers for the
// whole sequence (value columns never interact).  Per chunk:
//   stage 0  all threads: load g, k, q; cumulative sum of g per channel
//            (in-thread over 8 tokens, then across 8 lanes); build Kh, Kc,
//            Qh and Kb^T in LDS; beta and e^{b_last} in LDS.
//   stage 1  MFMA: the ten lower 16x16 tiles of A and of P.
//   stage 2  UT factor: diagonal 16x16 blocks of (I + A)^{-1} by forward
//            substitution (one wave), off-diagonal blocks level by level;
//            T' written as an MFMA operand.
//   stage 3  per wave, all on MFMA with the state never leaving registers:
//            R = V - Kh S, U = T' R, O = Qh S + P U, S = Gamma S + Kb^T U.
// MFMA operands from registers (S, R, U) are used in their accumulator
// layout: a lane holds rows {4q..4q+3} of two consecutive 16-row tiles, and
// the contraction index inside every 32-deep step is permuted to match; LDS
// operands are stored with the same permutation so each lane's 8 values are
// one contiguous 16-byte read.
//
// Precision policies.  bf16 inputs run every product on bf16 MFMA with each
// fp32-derived operand split into hi + lo bf16 halves (hi*hi + hi*lo + lo*hi,
// fp32 accumulation), which single bf16 rounding of the derived operands
// cannot meet a 2e-3 relative-L2 bar with.  fp32 inputs run the same
// dataflow on fp32 MFMA (16x16x4).
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kC = 64;        // chunk length (tokens)
constexpr int kThreads = 256; // 4 waves

// Position of logical index x inside its 32-block so that lane group q's
// eight contraction slots {4q..4q+3, 16+4q..16+4q+3} are contiguous.
__host__ __device__ constexpr int kperm(int x) {
  return (x & ~31) + (((x & 15) >> 2) << 3) + (x & 3) + (((x & 31) >> 4) << 2);
}

// ---------------------------------------------------------------------------
// Precision policies: operand storage in LDS and the 32-deep MFMA step.
// ---------------------------------------------------------------------------
struct PolBF16x3 {
  static constexpr int kPlanes = 2;  // hi plane, lo plane
  static constexpr int kElem = 2;    // bytes per element per plane
  struct Frag {
    bf16x8_t hi, lo;
  };
  __device__ __forceinline__ static void split(float x, uint32_t& hi, uint32_t& lo) {
    hi = f32_to_bf16_rne(x);
    lo = f32_to_bf16_rne(x - __uint_as_float(hi << 16));
  }
  __device__ __forceinline__ static void store4(char* base, int plane, int off, const float v[4]) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split(v[e], h[e], l[e]);
    *reinterpret_cast<uint2*>(base + off) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    *reinterpret_cast<uint2*>(base + plane + off) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
  }
  __device__ __forceinline__ static void store1(char* base, int plane, int off, float v) {
    uint32_t h, l;
    split(v, h, l);
    *reinterpret_cast<uint16_t*>(base + off) = uint16_t(h);
    *reinterpret_cast<uint16_t*>(base + plane + off) = uint16_t(l);
  }
  __device__ __forceinline__ static Frag load(const char* base, int plane, int off) {
    Frag f;
    f.hi = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(base + off));
    f.lo = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(base + plane + off));
    return f;
  }
  __device__ __forceinline__ static Frag make(const float v[8]) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split(v[e], h[e], l[e]);
    u32x4_t hw, lw;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hw[e] = h[2 * e] | (h[2 * e + 1] << 16);
      lw[e] = l[2 * e] | (l[2 * e + 1] << 16);
    }
    Frag f;
    f.hi = __builtin_bit_cast(bf16x8_t, hw);
    f.lo = __builtin_bit_cast(bf16x8_t, lw);
    return f;
  }
  __device__ __forceinline__ static void mma(f32x4_t& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
  }
};

struct PolF32 {
  static constexpr int kPlanes = 1;
  static constexpr int kElem = 4;
  struct Frag {
    float v[8];
  };
  __device__ __forceinline__ static void store4(char* base, int, int off, const float v[4]) {
    *reinterpret_cast<float4*>(base + off) = make_float4(v[0], v[1], v[2], v[3]);
  }
  __device__ __forceinline__ static void store1(char* base, int, int off, float v) {
    *reinterpret_cast<float*>(base + off) = v;
  }
  __device__ __forceinline__ static Frag load(const char* base, int, int off) {
    Frag f;
    const float4 a = *reinterpret_cast<const float4*>(base + off);
    const float4 b = *reinterpret_cast<const float4*>(base + off + 16);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
  __device__ __forceinline__ static Frag make(const float v[8]) {
    Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = v[e];
    return f;
  }
  __device__ __forceinline__ static void mma(f32x4_t& acc, const Frag& a, const Frag& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// LDS layout (bytes).  Row strides are padded so that the 16 rows read by one
// MFMA operand load fall in distinct banks.
// ---------------------------------------------------------------------------
template <class Pol>
struct Lds {
  static constexpr int E = Pol::kElem;
  static constexpr int P = Pol::kPlanes;
  static constexpr int kOpRow = kD * E + 16;              // [64 tok][128 ch]
  static constexpr int kOpPlane = kC * kOpRow;
  static constexpr int kOpBytes = P * kOpPlane;
  static constexpr int kKbRow = kC * E + 16;              // [128 ch][64 tok]
  static constexpr int kKbPlane = kD * kKbRow;
  static constexpr int kKbBytes = P * kKbPlane;
  static constexpr int kSqRow = kC * E + 16;              // [64][64] operand
  static constexpr int kSqPlane = kC * kSqRow;
  static constexpr int kSqBytes = P * kSqPlane;
  static constexpr int kAfLd = 68;                        // fp32 [64][68]
  static constexpr int kAfBytes = kC * kAfLd * 4;
  // regions
  static constexpr int kKh = 0;
  static constexpr int kKc = kKh + kOpBytes;              // Kc, later P | (A, then T')
  static constexpr int kPbuf = kKc;
  static constexpr int kAbuf = kKc + kSqBytes;            // A (fp32), then T' (operand)
  static constexpr int kKcBytes0 = kSqBytes + (kAfBytes > kSqBytes ? kAfBytes : kSqBytes);
  static constexpr int kKcBytes = kOpBytes > kKcBytes0 ? kOpBytes : kKcBytes0;
  static constexpr int kQh = kKc + kKcBytes;
  static constexpr int kKb = kQh + kOpBytes;
  static constexpr int kTf = kKb + kKbBytes;              // fp32 [64][68] UT factor
  static constexpr int kBeta = kTf + kAfBytes;            // 64 floats
  static constexpr int kGamma = kBeta + kC * 4;           // 128 floats
  static constexpr int kBytes = kGamma + kD * 4;
  static_assert(kBytes <= 160 * 1024, "LDS budget");
  static_assert(kOpRow % 16 == 0 && kKbRow % 16 == 0 && kSqRow % 16 == 0, "16-byte rows");
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* cu_seqlens;
  int32_t H;
  int32_t n_value_slices;  // 128 / (64 * JB)
  int32_t n_slices;        // value slices (+ as many transition slices)
  float scale;
  const float* initial_state;
  float* final_state;
  void* o;
  float* transition_out;
};

__device__ __constant__ const int kLowerI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__device__ __constant__ const int kLowerJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <class Pol, class InT, int JB>
__global__ __launch_bounds__(kThreads) void kda_prefill_kernel(PrefillArgs a) {
  using L = Lds<Pol>;
  using Frag = typename Pol::Frag;
  constexpr int E = L::E;
  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
  float* s_beta = reinterpret_cast<float*>(smem + L::kBeta);
  float* s_gamma = reinterpret_cast<float*>(smem + L::kGamma);
  float* s_af = reinterpret_cast<float*>(smem + L::kAbuf);
  float* s_tf = reinterpret_cast<float*>(smem + L::kTf);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lq = lane >> 4;  // lane group (contraction slots / output rows 4lq..)
  const int lj = lane & 15;  // output column / operand row within a tile

  const int slice = blockIdx.x % a.n_slices;
  const int sh = blockIdx.x / a.n_slices;
  const int h = sh % a.H;
  const int seq = sh / a.H;
  const bool is_transition = slice >= a.n_value_slices;
  const int vslice = is_transition ? slice - a.n_value_slices : slice;
  const int colw = vslice * (64 * JB) + wave * (16 * JB);  // first column of this wave
  const int64_t H = a.H;
  const int64_t tile_base = (int64_t(seq) * H + h) * (kD * kD);

  const int bos = a.cu_seqlens[seq];
  const int eos = a.cu_seqlens[seq + 1];
  const bool want_o = !is_transition && a.o != nullptr;
  float* const s_out = is_transition ? a.transition_out : a.final_state;

  // ---- entry state in accumulator layout: S[jb][ct][i] = S0[16ct+4lq+i][colw+16jb+lj]
  f32x4_t S[JB][8];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * ct + 4 * lq + i;
        const int col = colw + 16 * jb + lj;
        float x;
        if (is_transition) x = (row == col) ? 1.0f : 0.0f;
        else x = a.initial_state ? a.initial_state[tile_base + row * kD + col] : 0.0f;
        S[jb][ct][i] = x;
      }
    }
  }

  // stage-0 thread roles: 8 consecutive tokens x 4 consecutive channels
  const int tg = tid & 7;
  const int cq = tid >> 3;
  const int c0 = cq * 4;

  for (int t0 = bos; t0 < eos; t0 += kC) {
    const int n = (eos - t0) < kC ? (eos - t0) : kC;

    // ================= stage 0: decay prefix, rescaled operands =================
    {
      float gq[8][4], kq[8][4], qv[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = tg * 8 + i;
        if (r < n) {
          const int64_t base = (int64_t(t0 + r) * H + h) * kD + c0;
          const float4 gw = ld_f4(a.g + base);
          gq[i][0] = gw.x; gq[i][1] = gw.y; gq[i][2] = gw.z; gq[i][3] = gw.w;
          InT::load4(a.k, base, kq[i]);
          InT::load4(a.q, base, qv[i]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) { gq[i][e] = 0.0f; kq[i][e] = 0.0f; qv[i][e] = 0.0f; }
        }
      }
#pragma unroll
      for (int i = 1; i < 8; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) gq[i][e] += gq[i - 1][e];
      }
      float incl[4], excl[4], blast[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) incl[e] = gq[7][e];
#pragma unroll
      for (int d = 1; d < 8; d <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = __shfl_up(incl[e], d, 8);
          if (tg >= d) incl[e] += y;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y = __shfl_up(incl[e], 1, 8);
        excl[e] = (tg == 0) ? 0.0f : y;
        blast[e] = __shfl(excl[e] + gq[7][e], 7, 8);  // b at the chunk's last row
      }
      float kbv[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = tg * 8 + i;
        float kh[4], kc[4], qh[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float b = excl[e] + gq[i][e];
          const float eb = __expf(b);
          kh[e] = kq[i][e] * eb;
          kc[e] = kq[i][e] * __expf(-b);
          qh[e] = (qv[i][e] * a.scale) * eb;
          kbv[i][e] = kq[i][e] * __expf(blast[e] - b);
        }
        const int off = r * L::kOpRow + kperm(c0) * E;
        Pol::store4(smem + L::kKh, L::kOpPlane, off, kh);
        Pol::store4(smem + L::kKc, L::kOpPlane, off, kc);
        Pol::store4(smem + L::kQh, L::kOpPlane, off, qh);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = (c0 + e) * L::kKbRow;
        const float lo4[4] = {kbv[0][e], kbv[1][e], kbv[2][e], kbv[3][e]};
        const float hi4[4] = {kbv[4][e], kbv[5][e], kbv[6][e], kbv[7][e]};
        Pol::store4(smem + L::kKb, L::kKbPlane, row + kperm(8 * tg) * E, lo4);
        Pol::store4(smem + L::kKb, L::kKbPlane, row + kperm(8 * tg + 4) * E, hi4);
      }
      if (tg == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s_gamma[c0 + e] = __expf(blast[e]);
      }
      if (tid < kC) s_beta[tid] = (tid < n) ? a.beta[int64_t(t0 + tid) * H + h] : 0.0f;
    }
    // V at this wave's columns, accumulator layout (rows 16rt+4lq+i)
    float vreg[JB][4][4];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lq + i;
          vreg[jb][rt][i] = (!is_transition && r < n)
                                ? InT::load1(a.v, (int64_t(t0 + r) * H + h) * kD + colw + 16 * jb + lj)
                                : 0.0f;
        }
      }
    }
    __syncthreads();

    // ================= stage 1: lower tiles of A and P ==========================
    {
      f32x4_t acc[5];
#pragma unroll
      for (int u = 0; u < 5; ++u) {
        const int tau = wave + 4 * u;
        const bool isP = tau >= 10;
        const int lt = isP ? tau - 10 : tau;
        const int I = kLowerI[lt], J = kLowerJ[lt];
        const char* abase = smem + (isP ? L::kQh : L::kKh);
        acc[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int koff = (32 * ks + 8 * lq) * E;
          const Frag fa = Pol::load(abase, L::kOpPlane, (16 * I + lj) * L::kOpRow + koff);
          const Frag fb = Pol::load(smem + L::kKc, L::kOpPlane, (16 * J + lj) * L::kOpRow + koff);
          Pol::mma(acc[u], fa, fb);
        }
      }
      __syncthreads();  // every read of Kc is done: its region now takes P and A
#pragma unroll
      for (int u = 0; u < 5; ++u) {
        const int tau = wave + 4 * u;
        const bool isP = tau >= 10;
        const int lt = isP ? tau - 10 : tau;
        const int I = kLowerI[lt], J = kLowerJ[lt];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * I + 4 * lq + i;
          const int s = 16 * J + lj;
          if (isP) {
            Pol::store1(smem + L::kPbuf, L::kSqPlane, r * L::kSqRow + kperm(s) * E, (s <= r) ? acc[u][i] : 0.0f);
          } else {
            s_af[r * L::kAfLd + s] = (s < r) ? acc[u][i] * s_beta[r] : 0.0f;
          }
        }
      }
      // zero the upper tiles of P (read by the 32-deep steps of P U)
#pragma unroll
      for (int e = 0; e < 6; ++e) {
        const int idx = tid + kThreads * e;  // 0 .. 1535 over 6 tiles of 256
        const int ut = idx >> 8, w = idx & 255;
        const int I = (ut < 3) ? 0 : (ut < 5 ? 1 : 2);
        const int J = (ut < 3) ? ut + 1 : (ut < 5 ? ut - 1 : 3);
        const int r = 16 * I + (w >> 4), s = 16 * J + (w & 15);
        Pol::store1(smem + L::kPbuf, L::kSqPlane, r * L::kSqRow + kperm(s) * E, 0.0f);
      }
    }
    __syncthreads();

    // ================= stage 2: T = (I + A)^{-1}, T' = T diag(beta) ===============
    if (wave == 0) {
      const int I = lane >> 4, jj = lane & 15;
      const float* arow = s_af + (16 * I) * L::kAfLd + 16 * I;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == jj) ? 1.0f : 0.0f;
#pragma unroll
        for (int s = 0; s < i; ++s) acc = fmaf(-arow[i * L::kAfLd + s], x[s], acc);
        x[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) s_tf[(16 * I + i) * L::kAfLd + 16 * I + jj] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      const int strips = (4 - d) * 64;
      const int bI = (tid >> 6) + d, bJ = tid >> 6;
      const int ri = (tid & 63) >> 2, jq = (tid & 3) * 4;
      if (tid < strips) {  // X_IJ = sum_{K=J}^{I-1} A_IK T_KJ -> temp at block (J, I)
        float4 xs = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int K = bJ; K < bI; ++K) {
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            const float av = s_af[(16 * bI + ri) * L::kAfLd + 16 * K + m];
            const float4 tv = *reinterpret_cast<const float4*>(s_tf + (16 * K + m) * L::kAfLd + 16 * bJ + jq);
            xs.x = fmaf(av, tv.x, xs.x); xs.y = fmaf(av, tv.y, xs.y);
            xs.z = fmaf(av, tv.z, xs.z); xs.w = fmaf(av, tv.w, xs.w);
          }
        }
        *reinterpret_cast<float4*>(s_tf + (16 * bJ + ri) * L::kAfLd + 16 * bI + jq) = xs;
      }
      __syncthreads();
      if (tid < strips) {  // T_IJ = -T_II X_IJ
        float4 ys = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          const float tv = s_tf[(16 * bI + ri) * L::kAfLd + 16 * bI + m];
          const float4 xv = *reinterpret_cast<const float4*>(s_tf + (16 * bJ + m) * L::kAfLd + 16 * bI + jq);
          ys.x = fmaf(tv, xv.x, ys.x); ys.y = fmaf(tv, xv.y, ys.y);
          ys.z = fmaf(tv, xv.z, ys.z); ys.w = fmaf(tv, xv.w, ys.w);
        }
        *reinterpret_cast<float4*>(s_tf + (16 * bI + ri) * L::kAfLd + 16 * bJ + jq) =
            make_float4(-ys.x, -ys.y, -ys.z, -ys.w);
      }
      __syncthreads();
    }
    {  // T' = T diag(beta), lower triangle, as an MFMA operand (A region is free now)
      const int r = tid >> 2;
      const int sb = (tid & 3) * 16;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int s = sb + 4 * qd;
        float vals[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) vals[e] = (s + e <= r) ? s_tf[r * L::kAfLd + s + e] * s_beta[s + e] : 0.0f;
        Pol::store4(smem + L::kAbuf, L::kSqPlane, r * L::kSqRow + kperm(s) * E, vals);
      }
    }
    __syncthreads();

    // ================= stage 3: state pass (per wave, registers) =================
    {
      f32x4_t accR[JB][4], accO[JB][4];
      // R = V - Kh S  (accumulated as Kh S - V, negated when split)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          accR[jb][rt] = f32x4_t{-vreg[jb][rt][0], -vreg[jb][rt][1], -vreg[jb][rt][2], -vreg[jb][rt][3]};
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) accO[jb][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        Frag sf[JB];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const float v8[8] = {S[jb][2 * ks][0], S[jb][2 * ks][1], S[jb][2 * ks][2], S[jb][2 * ks][3],
                               S[jb][2 * ks + 1][0], S[jb][2 * ks + 1][1], S[jb][2 * ks + 1][2], S[jb][2 * ks + 1][3]};
          sf[jb] = Pol::make(v8);
        }
        const int koff = (32 * ks + 8 * lq) * E;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const Frag fk = Pol::load(smem + L::kKh, L::kOpPlane, (16 * rt + lj) * L::kOpRow + koff);
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) Pol::mma(accR[jb][rt], fk, sf[jb]);
          if (want_o) {
            const Frag fq = Pol::load(smem + L::kQh, L::kOpPlane, (16 * rt + lj) * L::kOpRow + koff);
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) Pol::mma(accO[jb][rt], fq, sf[jb]);
          }
        }
      }
      // U = T' R  (T' lower triangular: row tiles 0,1 need contraction tiles 0..1 only)
      Frag rf[JB][2];
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float v8[8] = {-accR[jb][2 * m][0], -accR[jb][2 * m][1], -accR[jb][2 * m][2], -accR[jb][2 * m][3],
                               -accR[jb][2 * m + 1][0], -accR[jb][2 * m + 1][1], -accR[jb][2 * m + 1][2],
                               -accR[jb][2 * m + 1][3]};
          rf[jb][m] = Pol::make(v8);
        }
      f32x4_t accU[JB][4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) accU[jb][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          if (m == 1 && rt < 2) continue;
          const Frag ft = Pol::load(smem + L::kAbuf, L::kSqPlane, (16 * rt + lj) * L::kSqRow + (32 * m + 8 * lq) * E);
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) Pol::mma(accU[jb][rt], ft, rf[jb][m]);
        }
      }
      Frag uf[JB][2];
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float v8[8] = {accU[jb][2 * m][0], accU[jb][2 * m][1], accU[jb][2 * m][2], accU[jb][2 * m][3],
                               accU[jb][2 * m + 1][0], accU[jb][2 * m + 1][1], accU[jb][2 * m + 1][2],
                               accU[jb][2 * m + 1][3]};
          uf[jb][m] = Pol::make(v8);
        }
      // O += P U, then store the chunk's outputs
      if (want_o) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            if (m == 1 && rt < 2) continue;
            const Frag fp = Pol::load(smem + L::kPbuf, L::kSqPlane, (16 * rt + lj) * L::kSqRow + (32 * m + 8 * lq) * E);
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) Pol::mma(accO[jb][rt], fp, uf[jb][m]);
          }
        }
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 16 * rt + 4 * lq + i;
              if (r < n) InT::store1(a.o, (int64_t(t0 + r) * H + h) * kD + colw + 16 * jb + lj, accO[jb][rt][i]);
            }
      }
      // S = Gamma S + Kb^T U
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const float4 gm = *reinterpret_cast<const float4*>(s_gamma + 16 * ct + 4 * lq);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          S[jb][ct][0] *= gm.x; S[jb][ct][1] *= gm.y; S[jb][ct][2] *= gm.z; S[jb][ct][3] *= gm.w;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const Frag fb = Pol::load(smem + L::kKb, L::kKbPlane, (16 * ct + lj) * L::kKbRow + (32 * m + 8 * lq) * E);
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) Pol::mma(S[jb][ct], fb, uf[jb][m]);
        }
      }
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  }

  if (s_out != nullptr) {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_out[tile_base + (16 * ct + 4 * lq + i) * kD + colw + 16 * jb + lj] = S[jb][ct][i];
  }
}

template <class Pol, class InT, int JB>
hipError_t launch_jb(const PrefillLaunch& p, hipStream_t stream) {
  PrefillArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.beta = p.beta;
  a.cu_seqlens = p.cu_seqlens;
  a.H = p.H;
  a.n_value_slices = kD / (64 * JB);
  a.n_slices = a.n_value_slices * (p.transition_out ? 2 : 1);
  a.scale = p.scale;
  a.initial_state = p.initial_state;
  a.final_state = p.final_state;
  a.o = p.o;
  a.transition_out = p.transition_out;
  const int64_t blocks = int64_t(p.num_seqs) * p.H * a.n_slices;
  hipLaunchKernelGGL((kda_prefill_kernel<Pol, InT, JB>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillLaunch& p, bool bf16, hipStream_t stream) {
  // Wider slices (all 128 columns per workgroup) when there are enough
  // (sequence, head) pairs to fill the chip; otherwise 64-column slices.
  const bool wide = int64_t(p.num_seqs) * p.H >= 256;
  if (bf16) return wide ? launch_jb<PolBF16x3, BF16, 2>(p, stream) : launch_jb<PolBF16x3, BF16, 1>(p, stream);
  return wide ? launch_jb<PolF32, F32, 2>(p, stream) : launch_jb<PolF32, F32, 1>(p, stream);
}

}  // namespace kda
