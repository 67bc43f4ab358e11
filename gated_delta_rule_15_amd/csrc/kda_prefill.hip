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
//   stage 0  all threads: the chunk's g, k, q, beta, v were prefetched into
//            registers during the previous chunk; cumulative sum of g per
//            channel (in-thread over 8 tokens, then across 8 lanes); build
//            Kh, Kc, Qh and Kb^T in LDS; beta and e^{b_last} in LDS.
//   stage 1  wave 0: the four diagonal 16x16 tiles of A on MFMA, then their
//            unit-lower-triangular inverses T_II by right-looking
//            substitution in registers; waves 1-3 meanwhile: the six
//            off-diagonal tiles of A and the ten lower tiles of P.
//   stage 2  the UT factor T = (I + A)^{-1} by 16-column blocks, one wave
//            per block: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ on MFMA with the
//            block column kept in registers; T' = T diag(beta) to LDS.
//   stage 3  per wave, all on MFMA with the state never leaving registers:
//            R = V - Kh S, U = T' R, O = Qh S + P U, S = Gamma S + Kb^T U;
//            the next chunk's inputs are fetched at its start.
// MFMA operands from registers (S, R, U, T blocks) are used in their
// accumulator layout: a lane holds rows {4q..4q+3} of two consecutive 16-row
// tiles, and the contraction index inside every 32-deep step is permuted to
// match; LDS operands are stored with the same permutation so each lane's 8
// values are one contiguous 16-byte read.
//
// Precision policies.  bf16 inputs run every product on bf16 MFMA with each
// fp32-derived operand split into hi + lo bf16 halves (hi*hi + hi*lo + lo*hi,
// fp32 accumulation); a single bf16 rounding of the derived operands misses a
// 2e-3 relative-L2 bar on the outputs.  fp32 inputs run the same dataflow on
// fp32 MFMA (16x16x4).
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kC = 64;        // chunk length (tokens)
constexpr int kThreads = 256; // 4 waves

// Position of logical index x inside its 32-block so that lane group q's
// eight contraction slots {4q..4q+3, 16+4q..16+4q+3} are contiguous.
__host__ __device__ constexpr int kperm(int x) {
  return (x & ~31) + (((x & 15) >> 2) << 3) + (x & 3) + (((x & 31) >> 4) << 2);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Precision policies: operand storage in LDS and the MFMA steps.
//   Frag   : one lane's 8 contraction slots of a 32-deep step
//   Frag16 : one lane's 4 contraction slots of a 16-deep step
//   mma_part(acc, a, b, p), p < kParts   : accumulate part p of a 32-deep step
//   mma16_part(acc, a, b, p), p < kParts16
// Issuing part p over many independent accumulators before part p+1 keeps the
// MFMA pipe busy.
// ---------------------------------------------------------------------------
struct PolBF16x3 {
  static constexpr int kPlanes = 2;  // hi plane, lo plane
  static constexpr int kElem = 2;    // bytes per element per plane
  static constexpr int kParts = 3;
  static constexpr int kParts16 = 3;
  struct Frag {
    bf16x8_t hi, lo;
  };
  struct Frag16 {
    s16x4_t hi, lo;
  };
  // x = hi + lo with hi = bf16(x), lo = bf16(x - hi): two values per call,
  // packed as two bf16 halves of a 32-bit word (v_cvt_pk_bf16_f32).
  __device__ __forceinline__ static void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const bf16x2_t h = {(__bf16)a, (__bf16)b};
    const uint32_t hw = __builtin_bit_cast(uint32_t, h);
    const float ra = a - __uint_as_float(hw << 16);
    const float rb = b - __uint_as_float(hw & 0xFFFF0000u);
    const bf16x2_t l = {(__bf16)ra, (__bf16)rb};
    hi = hw;
    lo = __builtin_bit_cast(uint32_t, l);
  }
  __device__ __forceinline__ static void store4(char* base, int plane, int off, const float v[4]) {
    uint32_t h0, l0, h1, l1;
    split2(v[0], v[1], h0, l0);
    split2(v[2], v[3], h1, l1);
    *reinterpret_cast<uint2*>(base + off) = make_uint2(h0, h1);
    *reinterpret_cast<uint2*>(base + plane + off) = make_uint2(l0, l1);
  }
  __device__ __forceinline__ static void store1(char* base, int plane, int off, float v) {
    const __bf16 h = (__bf16)v;
    const __bf16 l = (__bf16)(v - (float)h);
    *reinterpret_cast<__bf16*>(base + off) = h;
    *reinterpret_cast<__bf16*>(base + plane + off) = l;
  }
  __device__ __forceinline__ static Frag load(const char* base, int plane, int off) {
    Frag f;
    f.hi = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(base + off));
    f.lo = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(base + plane + off));
    return f;
  }
  __device__ __forceinline__ static Frag16 load16(const char* base, int plane, int off) {
    Frag16 f;
    f.hi = __builtin_bit_cast(s16x4_t, *reinterpret_cast<const u32x2_t*>(base + off));
    f.lo = __builtin_bit_cast(s16x4_t, *reinterpret_cast<const u32x2_t*>(base + plane + off));
    return f;
  }
  __device__ __forceinline__ static Frag make(const float v[8]) {
    u32x4_t hw, lw;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t h, l;
      split2(v[2 * e], v[2 * e + 1], h, l);
      hw[e] = h;
      lw[e] = l;
    }
    Frag f;
    f.hi = __builtin_bit_cast(bf16x8_t, hw);
    f.lo = __builtin_bit_cast(bf16x8_t, lw);
    return f;
  }
  __device__ __forceinline__ static Frag16 make16(const float v[4]) {
    u32x2_t hw, lw;
    uint32_t h, l;
    split2(v[0], v[1], h, l);
    hw[0] = h; lw[0] = l;
    split2(v[2], v[3], h, l);
    hw[1] = h; lw[1] = l;
    Frag16 f;
    f.hi = __builtin_bit_cast(s16x4_t, hw);
    f.lo = __builtin_bit_cast(s16x4_t, lw);
    return f;
  }
  __device__ __forceinline__ static void mma_part(f32x4_t& acc, const Frag& a, const Frag& b, int p) {
    if (p == 0) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    else if (p == 1) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    else acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void mma16_part(f32x4_t& acc, const Frag16& a, const Frag16& b, int p) {
    if (p == 0) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, acc, 0, 0, 0);
    else if (p == 1) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, acc, 0, 0, 0);
    else acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, acc, 0, 0, 0);
  }
};

struct PolF32 {
  static constexpr int kPlanes = 1;
  static constexpr int kElem = 4;
  static constexpr int kParts = 8;
  static constexpr int kParts16 = 4;
  struct Frag {
    float v[8];
  };
  struct Frag16 {
    float v[4];
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
  __device__ __forceinline__ static Frag16 load16(const char* base, int, int off) {
    Frag16 f;
    const float4 a = *reinterpret_cast<const float4*>(base + off);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    return f;
  }
  __device__ __forceinline__ static Frag make(const float v[8]) {
    Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = v[e];
    return f;
  }
  __device__ __forceinline__ static Frag16 make16(const float v[4]) {
    Frag16 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[e] = v[e];
    return f;
  }
  __device__ __forceinline__ static void mma_part(f32x4_t& acc, const Frag& a, const Frag& b, int p) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[p], b.v[p], acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void mma16_part(f32x4_t& acc, const Frag16& a, const Frag16& b, int p) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[p], b.v[p], acc, 0, 0, 0);
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
  static constexpr int kOpRow = kD * E + 16;              // [64 tok][128 ch]: Kh, Kc, Qh
  static constexpr int kOpPlane = kC * kOpRow;
  static constexpr int kOpBytes = P * kOpPlane;
  static constexpr int kKbRow = kC * E + 16;              // [128 ch][64 tok]: Kb^T
  static constexpr int kKbPlane = kD * kKbRow;
  static constexpr int kKbBytes = P * kKbPlane;
  static constexpr int kSqRow = kC * E + 16;              // [64][64] operands: A, P, T'
  static constexpr int kSqPlane = kC * kSqRow;
  static constexpr int kSqBytes = P * kSqPlane;
  static constexpr int kDgRow = E == 2 ? 40 : 80;         // [4 x 16 rows][16 cols]: T_II (natural order)
  static constexpr int kDgPlane = kC * kDgRow;
  static constexpr int kDgBytes = P * kDgPlane;
  static constexpr int kBlkLd = 20;                       // fp32 [4][16][20] blocks
  static constexpr int kBlkBytes = 4 * 16 * kBlkLd * 4;
  // regions
  static constexpr int kKh = 0;
  static constexpr int kKc = kKh + kOpBytes;              // Kc; then A (operand) | P; A's part becomes T'
  static constexpr int kKcBytes = kOpBytes > 2 * kSqBytes ? kOpBytes : 2 * kSqBytes;
  static constexpr int kAop = kKc;
  static constexpr int kPbuf = kKc + kSqBytes;
  static constexpr int kQh = kKc + kKcBytes;
  static constexpr int kKb = kQh + kOpBytes;
  static constexpr int kDg = kKb + kKbBytes;              // T_II as MFMA operands
  static constexpr int kAt = kDg + kDgBytes;              // A_II transposed, fp32: At[I][s][r]
  static constexpr int kTd = kAt + kBlkBytes;             // T_II column-major, fp32: Td[I][j][r]
  static constexpr int kBeta = kTd + kBlkBytes;           // 64 floats
  static constexpr int kGamma = kBeta + kC * 4;           // 128 floats
  static constexpr int kBytes = kGamma + kD * 4;
  static_assert(kBytes <= 160 * 1024, "LDS budget");
  static_assert(kOpRow % 16 == 0 && kKbRow % 16 == 0 && kSqRow % 16 == 0 && kDgRow % 8 == 0, "aligned rows");
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

// Stage-1 tile lists of waves 1..3, entry u of wave w packed in 5 bits as
// (is_P << 4) | (I << 2) | J; waves hold 6, 5, 5 tiles:
//   wave 1: A10 A20 A21 A30 P00 P10;  wave 2: A31 A32 P11 P20 P21;  wave 3: P22 P30 P31 P32 P33
__host__ __device__ constexpr uint32_t tile_code(int isP, int I, int J) { return uint32_t((isP << 4) | (I << 2) | J); }
__host__ __device__ constexpr uint32_t pack6(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t e, uint32_t f) {
  return a | (b << 5) | (c << 10) | (d << 15) | (e << 20) | (f << 25);
}
constexpr uint32_t kTiles1 = pack6(tile_code(0, 1, 0), tile_code(0, 2, 0), tile_code(0, 2, 1), tile_code(0, 3, 0),
                                   tile_code(1, 0, 0), tile_code(1, 1, 0));
constexpr uint32_t kTiles2 = pack6(tile_code(0, 3, 1), tile_code(0, 3, 2), tile_code(1, 1, 1), tile_code(1, 2, 0),
                                   tile_code(1, 2, 1), 0);
constexpr uint32_t kTiles3 = pack6(tile_code(1, 2, 2), tile_code(1, 3, 0), tile_code(1, 3, 1), tile_code(1, 3, 2),
                                   tile_code(1, 3, 3), 0);

// Inputs of one chunk as loaded (packed) into registers.
template <class InT, int JB>
struct ChunkIn {
  float4 g[8];
  typename InT::raw4 k[8], q[8];
  float beta;
  typename InT::raw1 v[JB][4][4];
};

template <class InT, int JB>
__device__ __forceinline__ void load_chunk(ChunkIn<InT, JB>& in, const PrefillArgs& a, int t0, int n, int h,
                                           int tg, int c0, int tid, int lq, int lj, int colw, bool load_v) {
  const int64_t H = a.H;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = tg * 8 + i;
    const int rr = r < n ? r : n - 1;  // clamp: always a valid token; zeroed later
    const int64_t base = (int64_t(t0 + rr) * H + h) * kD + c0;
    in.g[i] = ld_f4(a.g + base);
    in.k[i] = InT::load4raw(a.k, base);
    in.q[i] = InT::load4raw(a.q, base);
  }
  {
    const int rr = tid < n ? tid : n - 1;
    in.beta = (tid < kC) ? a.beta[int64_t(t0 + rr) * H + h] : 0.0f;
  }
  if (load_v) {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lq + i;
          const int rr = r < n ? r : n - 1;
          in.v[jb][rt][i] = InT::load1raw(a.v, (int64_t(t0 + rr) * H + h) * kD + colw + 16 * jb + lj);
        }
  }
}

template <class Pol, class InT, int JB>
__global__ __launch_bounds__(kThreads) void kda_prefill_kernel(PrefillArgs a) {
  using L = Lds<Pol>;
  using Frag = typename Pol::Frag;
  using Frag16 = typename Pol::Frag16;
  constexpr int E = L::E;
  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
  float* s_beta = reinterpret_cast<float*>(smem + L::kBeta);
  float* s_gamma = reinterpret_cast<float*>(smem + L::kGamma);
  float* s_at = reinterpret_cast<float*>(smem + L::kAt);
  float* s_td = reinterpret_cast<float*>(smem + L::kTd);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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
  if (is_transition) {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[jb][ct][i] = (16 * ct + 4 * lq + i == colw + 16 * jb + lj) ? 1.0f : 0.0f;
  } else if (a.initial_state != nullptr) {
    const float* src = a.initial_state + tile_base + colw + lj;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[jb][ct][i] = src[(16 * ct + 4 * lq + i) * kD + 16 * jb];
  } else {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) S[jb][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // stage-0 thread roles: 8 consecutive tokens x 4 consecutive channels
  const int tg = tid & 7;
  const int cq = tid >> 3;
  const int c0 = cq * 4;

  ChunkIn<InT, JB> in;
  if (bos < eos) load_chunk<InT, JB>(in, a, bos, (eos - bos) < kC ? (eos - bos) : kC, h, tg, c0, tid, lq, lj, colw,
                                     !is_transition);

  for (int t0 = bos; t0 < eos; t0 += kC) {
    const int n = (eos - t0) < kC ? (eos - t0) : kC;

    // ================= stage 0: decay prefix, rescaled operands =================
    float vreg[JB][4][4];
    {
      float gq[8][4], kq[8][4], qv[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = tg * 8 + i < n;
        float kk[4], qq[4];
        InT::unpack4(in.k[i], kk);
        InT::unpack4(in.q[i], qq);
        gq[i][0] = ok ? in.g[i].x : 0.0f; gq[i][1] = ok ? in.g[i].y : 0.0f;
        gq[i][2] = ok ? in.g[i].z : 0.0f; gq[i][3] = ok ? in.g[i].w : 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kq[i][e] = ok ? kk[e] : 0.0f;
          qv[i][e] = ok ? qq[e] * a.scale : 0.0f;
        }
      }
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vreg[jb][rt][i] = (!is_transition && 16 * rt + 4 * lq + i < n) ? InT::unpack1(in.v[jb][rt][i]) : 0.0f;
      if (tid < kC) s_beta[tid] = tid < n ? in.beta : 0.0f;
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
      float kbv[8][4], gam[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) gam[e] = __expf(blast[e]);
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
          qh[e] = qv[i][e] * eb;
          kbv[i][e] = kc[e] * gam[e];  // k e^{b_last - b}
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
        for (int e = 0; e < 4; ++e) s_gamma[c0 + e] = gam[e];
      }
    }
    __syncthreads();  // B1

    // ================= stage 1: A, P tiles; diagonal inverses =================
    f32x4_t acc1[6];
    if (wave == 0) {
      // diagonal tiles of A
#pragma unroll
      for (int I = 0; I < 4; ++I) acc1[I] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int koff = (32 * ks + 8 * lq) * E;
        Frag fa[4], fb[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          fa[I] = Pol::load(smem + L::kKh, L::kOpPlane, (16 * I + lj) * L::kOpRow + koff);
          fb[I] = Pol::load(smem + L::kKc, L::kOpPlane, (16 * I + lj) * L::kOpRow + koff);
        }
#pragma unroll
        for (int p = 0; p < Pol::kParts; ++p)
#pragma unroll
          for (int I = 0; I < 4; ++I) Pol::mma_part(acc1[I], fa[I], fb[I], p);
      }
      // At[I][s][r] = A[16I+r][16I+s] = beta_r * (Kh Kc^T)[r][s] for r > s
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        float4 w;
        float* wp = reinterpret_cast<float*>(&w);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * lq + i;
          wp[i] = (r > lj) ? acc1[I][i] * s_beta[16 * I + r] : 0.0f;
        }
        *reinterpret_cast<float4*>(s_at + (I * 16 + lj) * L::kBlkLd + 4 * lq) = w;
      }
      wave_sync();
      // T_II = (I + A_II)^{-1}: lane (I = lane/16, column j); right-looking substitution
      {
        const int I = lane >> 4, j = lane & 15;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == j) ? 1.0f : 0.0f;
#pragma unroll
        for (int s = 0; s < 15; ++s) {
          const float* col = s_at + (I * 16 + s) * L::kBlkLd;  // column s of A_II
          float cv[16];
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const float4 w = *reinterpret_cast<const float4*>(col + 4 * r4);
            cv[4 * r4] = w.x; cv[4 * r4 + 1] = w.y; cv[4 * r4 + 2] = w.z; cv[4 * r4 + 3] = w.w;
          }
#pragma unroll
          for (int r = s + 1; r < 16; ++r) x[r] = fmaf(-cv[r], x[s], x[r]);
        }
        // Td[I][j][r] = T_II[r][j] (column-major fp32) and T_II as an MFMA operand
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<float4*>(s_td + (I * 16 + j) * L::kBlkLd + 4 * r4) =
              make_float4(x[4 * r4], x[4 * r4 + 1], x[4 * r4 + 2], x[4 * r4 + 3]);
#pragma unroll
        for (int r = 0; r < 16; ++r) Pol::store1(smem + L::kDg, L::kDgPlane, (16 * I + r) * L::kDgRow + j * E, x[r]);
      }
    } else {
      const uint32_t tiles = wave == 1 ? kTiles1 : (wave == 2 ? kTiles2 : kTiles3);
      const int cnt = (wave == 1) ? 6 : 5;
#pragma unroll
      for (int u = 0; u < 6; ++u) acc1[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int koff = (32 * ks + 8 * lq) * E;
        Frag fa[6], fb[6];
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          if (u < cnt) {
            const uint32_t code = (tiles >> (5 * u)) & 31u;
            const char* abase = smem + ((code >> 4) ? L::kQh : L::kKh);
            fa[u] = Pol::load(abase, L::kOpPlane, (16 * int((code >> 2) & 3u) + lj) * L::kOpRow + koff);
            fb[u] = Pol::load(smem + L::kKc, L::kOpPlane, (16 * int(code & 3u) + lj) * L::kOpRow + koff);
          }
        }
#pragma unroll
        for (int p = 0; p < Pol::kParts; ++p)
#pragma unroll
          for (int u = 0; u < 6; ++u)
            if (u < cnt) Pol::mma_part(acc1[u], fa[u], fb[u], p);
      }
    }
    __syncthreads();  // B2: Kc is dead; its region takes A (operand) and P
    if (wave != 0) {
      const uint32_t tiles = wave == 1 ? kTiles1 : (wave == 2 ? kTiles2 : kTiles3);
      const int cnt = (wave == 1) ? 6 : 5;
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        if (u < cnt) {
          const uint32_t code = (tiles >> (5 * u)) & 31u;
          const bool isP = (code >> 4) != 0;
          const int I = int((code >> 2) & 3u), J = int(code & 3u);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * I + 4 * lq + i;
            const int s = 16 * J + lj;
            if (isP) Pol::store1(smem + L::kPbuf, L::kSqPlane, r * L::kSqRow + kperm(s) * E, (s <= r) ? acc1[u][i] : 0.0f);
            else Pol::store1(smem + L::kAop, L::kSqPlane, r * L::kSqRow + kperm(s) * E, acc1[u][i] * s_beta[r]);
          }
        }
      }
      // zero the upper tiles of P (read by the 32-deep steps of P U): 6 tiles x 256 over 192 threads
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int idx = (tid - 64) + 192 * e;  // 0 .. 1535
        const int ut = idx >> 8, wi = idx & 255;
        const int I = (ut < 3) ? 0 : (ut < 5 ? 1 : 2);
        const int J = (ut < 3) ? ut + 1 : (ut < 5 ? ut - 1 : 3);
        const int r = 16 * I + (wi >> 4), s = 16 * J + (wi & 15);
        Pol::store1(smem + L::kPbuf, L::kSqPlane, r * L::kSqRow + kperm(s) * E, 0.0f);
      }
    }
    __syncthreads();  // B3

    // ================= stage 2: T = (I + A)^{-1} by column blocks =================
    f32x4_t Tt[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) Tt[I] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      const int J = wave;
      {
        const float4 w = *reinterpret_cast<const float4*>(s_td + (J * 16 + lj) * L::kBlkLd + 4 * lq);
        Tt[J] = f32x4_t{w.x, w.y, w.z, w.w};  // rows 4lq.. of column lj of T_JJ
      }
#pragma unroll
      for (int I = 1; I < 4; ++I) {
        if (I > J) {
          f32x4_t X = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int K = 0; K < 3; ++K) {
            if (K >= J && K < I) {
              const Frag16 fa = Pol::load16(smem + L::kAop, L::kSqPlane,
                                            (16 * I + lj) * L::kSqRow + kperm(16 * K + 4 * lq) * E);
              const float bv[4] = {Tt[K][0], Tt[K][1], Tt[K][2], Tt[K][3]};
              const Frag16 fb = Pol::make16(bv);
#pragma unroll
              for (int p = 0; p < Pol::kParts16; ++p) Pol::mma16_part(X, fa, fb, p);
            }
          }
          const Frag16 ft = Pol::load16(smem + L::kDg, L::kDgPlane, (16 * I + lj) * L::kDgRow + 4 * lq * E);
          const float xv[4] = {X[0], X[1], X[2], X[3]};
          const Frag16 fx = Pol::make16(xv);
          f32x4_t Y = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < Pol::kParts16; ++p) Pol::mma16_part(Y, ft, fx, p);
          Tt[I] = -Y;
        }
      }
    }
    __syncthreads();  // B4: every read of A is done; its region takes T'
    {
      const int J = wave;
      const float bj = s_beta[16 * J + lj];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * I + 4 * lq + i;
          const int s = 16 * J + lj;
          const float val = (I > J || (I == J && r >= s)) ? Tt[I][i] * bj : 0.0f;
          Pol::store1(smem + L::kAop, L::kSqPlane, r * L::kSqRow + kperm(s) * E, val);
        }
      }
    }
    __syncthreads();  // B5

    // ================= stage 3: state pass (per wave, registers) =================
    {
      f32x4_t accR[JB][4], accO[JB][4];
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          accR[jb][rt] = f32x4_t{-vreg[jb][rt][0], -vreg[jb][rt][1], -vreg[jb][rt][2], -vreg[jb][rt][3]};
          accO[jb][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      // R = V - Kh S (accumulated as Kh S - V), then O = Qh S; one operand set live at a time
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1 && !want_o) break;
        const char* abase = smem + (pass == 0 ? L::kKh : L::kQh);
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
          Frag fk[4];
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) fk[rt] = Pol::load(abase, L::kOpPlane, (16 * rt + lj) * L::kOpRow + koff);
#pragma unroll
          for (int p = 0; p < Pol::kParts; ++p)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
              for (int jb = 0; jb < JB; ++jb) {
                if (pass == 0) Pol::mma_part(accR[jb][rt], fk[rt], sf[jb], p);
                else Pol::mma_part(accO[jb][rt], fk[rt], sf[jb], p);
              }
        }
      }
      {  // fetch the next chunk's inputs; they land while the rest of this chunk runs
        const int t1 = t0 + kC;
        if (t1 < eos) load_chunk<InT, JB>(in, a, t1, (eos - t1) < kC ? (eos - t1) : kC, h, tg, c0, tid, lq, lj, colw,
                                          !is_transition);
      }
      // U = T' R  (T' lower triangular: row tiles 0,1 use contraction tiles 0..1 only)
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
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) accU[jb][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      {
        Frag ft[6];  // (rt, m): (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
#pragma unroll
        for (int x = 0; x < 6; ++x) {
          const int rt = x < 2 ? x : 2 + ((x - 2) >> 1);
          const int m = x < 2 ? 0 : ((x - 2) & 1);
          ft[x] = Pol::load(smem + L::kAop, L::kSqPlane, (16 * rt + lj) * L::kSqRow + (32 * m + 8 * lq) * E);
        }
#pragma unroll
        for (int p = 0; p < Pol::kParts; ++p)
#pragma unroll
          for (int x = 0; x < 6; ++x) {
            const int rt = x < 2 ? x : 2 + ((x - 2) >> 1);
            const int m = x < 2 ? 0 : ((x - 2) & 1);
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) Pol::mma_part(accU[jb][rt], ft[x], rf[jb][m], p);
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
        Frag fp[6];
#pragma unroll
        for (int x = 0; x < 6; ++x) {
          const int rt = x < 2 ? x : 2 + ((x - 2) >> 1);
          const int m = x < 2 ? 0 : ((x - 2) & 1);
          fp[x] = Pol::load(smem + L::kPbuf, L::kSqPlane, (16 * rt + lj) * L::kSqRow + (32 * m + 8 * lq) * E);
        }
#pragma unroll
        for (int p = 0; p < Pol::kParts; ++p)
#pragma unroll
          for (int x = 0; x < 6; ++x) {
            const int rt = x < 2 ? x : 2 + ((x - 2) >> 1);
            const int m = x < 2 ? 0 : ((x - 2) & 1);
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) Pol::mma_part(accO[jb][rt], fp[x], uf[jb][m], p);
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
      // S = Gamma S + Kb^T U, in two halves of four row tiles
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        Frag fb[4][2];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int ct = 4 * half + c;
          const float4 gm = *reinterpret_cast<const float4*>(s_gamma + 16 * ct + 4 * lq);
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) {
            S[jb][ct][0] *= gm.x; S[jb][ct][1] *= gm.y; S[jb][ct][2] *= gm.z; S[jb][ct][3] *= gm.w;
          }
#pragma unroll
          for (int m = 0; m < 2; ++m)
            fb[c][m] = Pol::load(smem + L::kKb, L::kKbPlane, (16 * ct + lj) * L::kKbRow + (32 * m + 8 * lq) * E);
        }
#pragma unroll
        for (int p = 0; p < Pol::kParts; ++p)
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
              for (int jb = 0; jb < JB; ++jb) Pol::mma_part(S[jb][4 * half + c], fb[c][m], uf[jb][m], p);
      }
    }
    __syncthreads();  // B6: LDS is rewritten by the next chunk
  }

  if (s_out != nullptr) {
    float* dst = s_out + tile_base + colw + lj;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * ct + 4 * lq + i) * kD + 16 * jb] = S[jb][ct][i];
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
  // 64-column slices: two workgroups per (sequence, head) and value half.
  if (bf16) return launch_jb<PolBF16x3, BF16, 1>(p, stream);
  return launch_jb<PolF32, F32, 1>(p, stream);
}

}  // namespace kda
