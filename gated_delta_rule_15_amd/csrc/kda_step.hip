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
// These kernels are HBM streams of the fp32 state.  A workgroup of four waves
// owns one (request, head, 64-column half) of the 128 x 128 state in
// registers: waves 2s and 2s+1 hold column slice s (32 columns), rows 0..63
// and 64..127; lane = 8 * rg + cg holds 8 rows (8rg .. 8rg+7 of its wave's
// half) and columns 4cg .. 4cg+3 of the slice, so one load instruction of a
// wave covers eight full 128-byte row segments.  The column sums r = S~^T k,
// s = S~^T q and q . k run in-thread over 8 rows, then across the wave's 8 row
// groups in registers as a reduce-scatter (each 32- and 16-lane permute-swap
// and the DPP rotation by 8 lanes pairs two different values, so every sum is
// formed once, in one lane), then across the slice's two waves through LDS,
// summed in wave order, and an all-gather hands every lane of a column the
// same sums.
//
// Per-token inputs: decode loads them straight from memory; verify and commit
// stage blocks of 8 tokens in LDS (k, scale * q and alpha = exp(g) as fp32,
// v of the slice, beta) once per workgroup, so the dependent steps never wait
// on memory.  Both paths produce the same fp32 values (same conversions, same
// exp), every step runs the same code, the file is built with
// -ffp-contract=off with explicit fmaf, and nothing is atomic: a commit of L
// tokens is bit-identical to L decode steps, and verify's o_t to the t-th of t
// decode steps.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

#ifndef KDA_STEP_ROWS_PER_LANE
#define KDA_STEP_ROWS_PER_LANE 8
#endif
constexpr int kThreads = 256;
constexpr int kSliceCols = 32;                      // columns of one slice (8 column groups of 4)
constexpr int kCG = 8;                              // column groups per slice
constexpr int kR = KDA_STEP_ROWS_PER_LANE;          // rows per lane (8 or 16)
constexpr int kRowsPerWave = 8 * kR;                // 8 row groups per wave
constexpr int kWavesPerSlice = kD / kRowsPerWave;   // 2 (kR = 8) or 1 (kR = 16)
constexpr int kSlicesPerWg = (kThreads / 64) / kWavesPerSlice;
constexpr int kWgCols = kSliceCols * kSlicesPerWg;  // columns per workgroup
constexpr int kWgPerHead = kD / kWgCols;            // workgroups per (request, head)
constexpr int kBlockT = 8;                          // tokens staged per block (verify / commit)
#ifndef KDA_BLOCK_HALVES
#define KDA_BLOCK_HALVES 1
#endif
constexpr int kBlockHalves = KDA_BLOCK_HALVES;      // 64-column halves per verify / commit workgroup
static_assert(kR == 8 || kR == 16, "rows per lane");

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
  int32_t layer_wgs;  // verify: workgroups per resident layer (the CU count); 0 = no staggering
  int32_t pro_l2;     // prologue kernels: normalise q and k per token
  float pro_eps;
  int32_t pro_gate;   // prologue kernels: g holds gate logits
  float pro_gmin;
  float* record;          // verify with the prologue, or null: each step's key and log-decay as used
  const float* rec_in;    // commit from a record: keys and log-decays read from it (q, k, g unused)
};

// The raw-input record of a verify ("SGLang 和 Miles 为 Kimi K3 提供首日支持",
// section "ReplaySSM：针对 KDA 状态的原始输入重放": the verify keeps each draft
// step's inputs and the fold consumes what it kept): per (request, step, head)
// the key after the prologue's normalisation and the log-decay after the gate
// map, fp32, [N, G, H, 2, 128] (1 KB per step and head).
__device__ __forceinline__ int64_t record_offset(int n, int t, int h, const StepArgs& a) {
  return ((int64_t(n) * a.G + t) * a.H + h) * (2 * kD);
}

// Input prologue (the KDA math-details box of the Day-0 lesson page: unit keys
// for the readout identity; the log-decay bounded below by a scaled sigmoid,
// g_min = -5).  The same functions serve the decode step and the staged
// verify / commit inputs, so all three see bit-identical values.
__device__ __forceinline__ float gate_log_decay(float x, float g_min) {
  return g_min * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
__device__ __forceinline__ float inv_l2(float sum_sq, float eps) { return __builtin_amdgcn_rsqf(sum_sq + eps); }

// One token's inputs at this lane's 8 rows and 4 columns, as fp32.
struct TokenVals {
  float k[kR], qs[kR], alpha[kR], v[4];
  float beta;
  float qk;  // scale * q . k, when staged
};

// Staged inputs of up to kBlockT tokens (verify / commit).
struct __align__(16) Stage {
  float k[kBlockT][kD];
  float qs[kBlockT][kD];     // scale * q
  float alpha[kBlockT][kD];  // exp(g)
  float v[kBlockT][kWgCols * kBlockHalves];  // v of the workgroup's columns
  float beta[kBlockT];
  float qk[kBlockT];         // scale * q . k
};

// Verify stages q . k per token (formed once per workgroup instead of in
// every lane), by the same arithmetic as the in-lane form of the decode step:
// a sequential fma chain over each 8-channel group, then the groups summed
// by the same tree.  Needs 8 rows per lane.
constexpr bool kStageQK = (kR == 8);

// Cross-wave partial sums: [buffer][slice][column group][value][wave of the
// slice]; 9 values padded to 10 so that a column group's partials start on a
// 16-byte boundary.
constexpr int kRedVals = 10;
struct __align__(16) Red {
  float x[2][kSlicesPerWg][kCG][kRedVals][kWavesPerSlice];
};

// Lane exchanges for the column sums over a wave's 8 row groups (lane bits
// 3..5).  swap32 / swap16 exchange, between two registers, the upper 32 lanes
// of the first with the lower 32 lanes of the second (v_permlane32_swap), or
// the odd 16-lane rows of the first with the even rows of the second
// (v_permlane16_swap); ror8 reads lane l ^ 8 within each 16-lane row.
__device__ __forceinline__ void swap32(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ float ror8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

// Column sums of NV per-lane partials (NV = 9: r0..r3, s0..s3, q.k; NV = 8:
// r, s; NV = 4: r) over the wave's 8 row groups and then the slice's waves,
// returned in every lane of the column group.  Reduce-scatter: at each lane
// bit a swap pairs two different values, so each sum is formed once, in one
// lane (the lane whose row-group bits (b5, b4, b3) = idx bits (0, 1, 2)); q.k
// is summed by a butterfly (rows paired across bit 5, then 4, then 3).  With
// two waves per slice each lane then writes its one partial to LDS and, after
// the barrier, every lane reads both waves' partials of its column group and
// adds them in wave order; with one wave per slice an all-gather in registers
// hands every lane the sums.  need_s (wave-uniform): s and q.k are wanted in
// this wave; otherwise only r is returned.  The tree is the same for every NV
// (r's are summed identically), so decode, verify and commit agree bit for
// bit.
template <int NV>
__device__ __forceinline__ void column_sums(float (&v)[NV], float (*red)[kRedVals][kWavesPerSlice], int lane, int ws,
                                            int cg, bool need_s) {
  constexpr bool HAS_S = NV >= 8;
  constexpr bool HAS_QK = NV == 9;
  const bool b3 = (lane >> 3) & 1;
  const int idx = ((lane >> 5) & 1) | (((lane >> 4) & 1) << 1) | (int(b3) << 2);
  // bit 5: (v0, v1) (v2, v3) [(v4, v5) (v6, v7)]
  swap32(v[0], v[1]);
  swap32(v[2], v[3]);
  float z01 = v[0] + v[1], z23 = v[2] + v[3];
  float z45 = 0.0f, z67 = 0.0f, qk = 0.0f;
  if constexpr (HAS_S) {
    swap32(v[4], v[5]);
    swap32(v[6], v[7]);
    z45 = v[4] + v[5];
    z67 = v[6] + v[7];
  }
  if constexpr (HAS_QK) {
    float t = v[NV - 1];
    swap32(v[NV - 1], t);
    qk = v[NV - 1] + t;
  }
  // bit 4: (z01, z23) [(z45, z67)]
  swap16(z01, z23);
  const float w0123 = z01 + z23;
  float w4567 = 0.0f;
  if constexpr (HAS_S) {
    swap16(z45, z67);
    w4567 = z45 + z67;
  }
  if constexpr (HAS_QK) {
    float t = qk;
    swap16(qk, t);
    qk = qk + t;
  }
  // bit 3: lanes with b3 = 0 keep v[idx] of w0123, b3 = 1 of w4567 (with s)
  float f;
  if constexpr (HAS_S) {
    const float mine = b3 ? w4567 : w0123;
    const float other = b3 ? w0123 : w4567;
    f = mine + ror8(other);
  } else {
    f = w0123 + ror8(w0123);  // both b3 lanes form v[idx & 3]
  }
  if constexpr (HAS_QK) qk = qk + ror8(qk);
  if constexpr (kWavesPerSlice == 2) {
    if (HAS_S || !b3) red[cg][HAS_S ? idx : (idx & 3)][ws] = f;
    if (HAS_QK && (lane >> 3) == 0) red[cg][8][ws] = qk;
    __syncthreads();
    const float4* p = reinterpret_cast<const float4*>(&red[cg][0][0]);  // [value][wave] pairs
    const float4 r01 = p[0], r23 = p[1];
    v[0] = r01.x + r01.y;
    v[1] = r01.z + r01.w;
    v[2] = r23.x + r23.y;
    v[3] = r23.z + r23.w;
    if constexpr (HAS_S) {
      if (need_s) {
        const float4 s01 = p[2], s23 = p[3];
        v[4] = s01.x + s01.y;
        v[5] = s01.z + s01.w;
        v[6] = s23.x + s23.y;
        v[7] = s23.z + s23.w;
        if constexpr (HAS_QK) {
          const float2 qq = *reinterpret_cast<const float2*>(&red[cg][8][0]);
          v[8] = qq.x + qq.y;
        }
      }
    }
  } else {
    // all-gather: bit 3, then 4, then 5
    float g[2];
    if constexpr (HAS_S) {
      const float fp = ror8(f);
      g[0] = b3 ? fp : f;  // v[b5 + 2 b4]
      g[1] = b3 ? f : fp;  // v[b5 + 2 b4 + 4]
    } else {
      g[0] = f;
      g[1] = 0.0f;
    }
    constexpr int NG = HAS_S ? 2 : 1;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      float h0 = g[j], h2 = g[j];
      swap16(h0, h2);  // h0: b4 = 0 value, h2: b4 = 1 value
      float h1 = h0, h3 = h2;
      swap32(h0, h1);  // h0: b5 = 0, h1: b5 = 1
      swap32(h2, h3);
      v[4 * j + 0] = h0;
      v[4 * j + 1] = h1;
      v[4 * j + 2] = h2;
      v[4 * j + 3] = h3;
    }
    if constexpr (HAS_QK) v[8] = qk;
  }
}

// PRO: g may hold gate logits, and q is left unscaled (the caller normalises
// and scales it once the norms are known).
template <class InT, bool READOUT, bool PRO>
__device__ __forceinline__ void load_token(TokenVals& x, const StepArgs& a, int n, int t, int h, int row0, int col) {
  const int64_t tok = (int64_t(n) * a.G + t) * a.H + h;  // [N, G, H] token-head index
  const int64_t vec = tok * kD;
#pragma unroll
  for (int i = 0; i < kR; i += 4) {
    InT::unpack4(InT::load4raw(a.k, vec + row0 + i), &x.k[i]);
    float4 g = ld_f4(a.g + vec + row0 + i);
    if (PRO && a.pro_gate) {
      g.x = gate_log_decay(g.x, a.pro_gmin); g.y = gate_log_decay(g.y, a.pro_gmin);
      g.z = gate_log_decay(g.z, a.pro_gmin); g.w = gate_log_decay(g.w, a.pro_gmin);
    }
    x.alpha[i] = __expf(g.x); x.alpha[i + 1] = __expf(g.y); x.alpha[i + 2] = __expf(g.z); x.alpha[i + 3] = __expf(g.w);
    if constexpr (READOUT) {
      float q[4];
      InT::unpack4(InT::load4raw(a.q, vec + row0 + i), q);
#pragma unroll
      for (int e = 0; e < 4; ++e) x.qs[i + e] = PRO ? q[e] : q[e] * a.scale;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x.qs[i + e] = 0.0f;
    }
  }
  InT::unpack4(InT::load4raw(a.v, vec + col), x.v);
  x.beta = a.beta[tok];
  x.qk = 0.0f;  // formed in the step
}

__device__ __forceinline__ void read_token(TokenVals& x, const Stage& st, int t, int row0, int wcol, bool readout) {
#pragma unroll
  for (int i = 0; i < kR; i += 4) {
    const float4 k = *reinterpret_cast<const float4*>(&st.k[t][row0 + i]);
    const float4 al = *reinterpret_cast<const float4*>(&st.alpha[t][row0 + i]);
    x.k[i] = k.x; x.k[i + 1] = k.y; x.k[i + 2] = k.z; x.k[i + 3] = k.w;
    x.alpha[i] = al.x; x.alpha[i + 1] = al.y; x.alpha[i + 2] = al.z; x.alpha[i + 3] = al.w;
    if (readout) {
      const float4 q = *reinterpret_cast<const float4*>(&st.qs[t][row0 + i]);
      x.qs[i] = q.x; x.qs[i + 1] = q.y; x.qs[i + 2] = q.z; x.qs[i + 3] = q.w;
    } else {
      x.qs[i] = x.qs[i + 1] = x.qs[i + 2] = x.qs[i + 3] = 0.0f;
    }
  }
  const float4 v = *reinterpret_cast<const float4*>(&st.v[t][wcol]);
  x.v[0] = v.x; x.v[1] = v.y; x.v[2] = v.z; x.v[3] = v.w;
  x.beta = st.beta[t];
  x.qk = (readout && kStageQK) ? st.qk[t] : 0.0f;
}

// Stage tokens b0 .. b0 + kBlockT - 1 (indices past `last` repeat `last`).
// Threads of the first half own 8 channels (one group of 8 rows of the step's
// lane layout) of token tid / 16 for k, q and g, and form q . k; threads of
// the second half own v pieces u, u + 128, ... (u = tid - 128; piece p is
// column group p % (columns / 4) of token p / (columns / 4)).  Every load is
// issued before the first LDS store.
template <int XOR>
__device__ __forceinline__ float xor_lane(float x) {  // lane ^ XOR within 32 lanes (XOR < 32)
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (XOR << 10)));
}

template <class InT, bool READOUT, bool PRO, bool REC = false>
__device__ __forceinline__ void stage_block(Stage& st, const StepArgs& a, int n, int h, int col0, int b0, int last,
                                            int tid) {
  static_assert(!(REC && (READOUT || PRO)), "a record serves the commit of the plain inputs' step");
  static_assert(kBlockT * 16 == kThreads / 2, "8 channels of one token per thread in the first half");
  constexpr int kVPieces = kWgCols * kBlockHalves / 4;  // v pieces per token
  constexpr int kVRounds = (kBlockT * kVPieces + kThreads / 2 - 1) / (kThreads / 2);
  if (tid < kThreads / 2) {
    const int t = tid >> 4, c8 = 8 * (tid & 15);
    const int tt = b0 + t <= last ? b0 + t : last;
    const int64_t vec = ((int64_t(n) * a.G + tt) * a.H + h) * kD + c8;
    typename InT::raw4 k0{}, k1{};
    float4 g0, g1, kr0{}, kr1{};
    if constexpr (REC) {
      // the key and log-decay the verify used, as it recorded them
      const float* rec = a.rec_in + record_offset(n, tt, h, a) + c8;
      kr0 = ld_f4(rec);
      kr1 = ld_f4(rec + 4);
      g0 = ld_f4(rec + kD);
      g1 = ld_f4(rec + kD + 4);
    } else {
      k0 = InT::load4raw(a.k, vec);
      k1 = InT::load4raw(a.k, vec + 4);
      g0 = ld_f4(a.g + vec);
      g1 = ld_f4(a.g + vec + 4);
    }
    typename InT::raw4 q0{}, q1{};
    if constexpr (READOUT) {
      q0 = InT::load4raw(a.q, vec);
      q1 = InT::load4raw(a.q, vec + 4);
    }
    float beta = 0.0f;
    if (tid < kBlockT) beta = a.beta[(int64_t(n) * a.G + (b0 + tid <= last ? b0 + tid : last)) * a.H + h];

    float k[8];
    if constexpr (REC) {
      k[0] = kr0.x; k[1] = kr0.y; k[2] = kr0.z; k[3] = kr0.w;
      k[4] = kr1.x; k[5] = kr1.y; k[6] = kr1.z; k[7] = kr1.w;
    } else {
      InT::unpack4(k0, k);
      InT::unpack4(k1, k + 4);
    }
    float qs[8];
    if constexpr (READOUT) {
      InT::unpack4(q0, qs);
      InT::unpack4(q1, qs + 4);
    }
    if constexpr (PRO) {
      if (a.pro_gate) {
        g0.x = gate_log_decay(g0.x, a.pro_gmin); g0.y = gate_log_decay(g0.y, a.pro_gmin);
        g0.z = gate_log_decay(g0.z, a.pro_gmin); g0.w = gate_log_decay(g0.w, a.pro_gmin);
        g1.x = gate_log_decay(g1.x, a.pro_gmin); g1.y = gate_log_decay(g1.y, a.pro_gmin);
        g1.z = gate_log_decay(g1.z, a.pro_gmin); g1.w = gate_log_decay(g1.w, a.pro_gmin);
      }
      if (a.pro_l2) {
        // the decode step's norm: fma chain over the group's 8 channels, then
        // groups paired across channel-group bit 2, 1, 0, and 3 (the two waves)
        float pk = 0.0f, pq = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) pk = fmaf(k[e], k[e], pk);
        pk = pk + xor_lane<4>(pk);
        pk = pk + xor_lane<2>(pk);
        pk = pk + xor_lane<1>(pk);
        pk = pk + xor_lane<8>(pk);
        const float rk = inv_l2(pk, a.pro_eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) k[e] = k[e] * rk;
        if constexpr (READOUT) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pq = fmaf(qs[e], qs[e], pq);
          pq = pq + xor_lane<4>(pq);
          pq = pq + xor_lane<2>(pq);
          pq = pq + xor_lane<1>(pq);
          pq = pq + xor_lane<8>(pq);
          const float rq = inv_l2(pq, a.pro_eps);
#pragma unroll
          for (int e = 0; e < 8; ++e) qs[e] = qs[e] * rq;
        }
      }
    }
    if constexpr (PRO && READOUT) {
      // the record: written once per (request, step, head), by the first column half's workgroup
      if (a.record != nullptr && col0 == 0 && b0 + t <= last) {
        float* rec = a.record + record_offset(n, b0 + t, h, a) + c8;
        st_f4(rec, make_float4(k[0], k[1], k[2], k[3]));
        st_f4(rec + 4, make_float4(k[4], k[5], k[6], k[7]));
        st_f4(rec + kD, g0);
        st_f4(rec + kD + 4, g1);
      }
    }
    *reinterpret_cast<float4*>(&st.k[t][c8]) = make_float4(k[0], k[1], k[2], k[3]);
    *reinterpret_cast<float4*>(&st.k[t][c8 + 4]) = make_float4(k[4], k[5], k[6], k[7]);
    *reinterpret_cast<float4*>(&st.alpha[t][c8]) = make_float4(__expf(g0.x), __expf(g0.y), __expf(g0.z), __expf(g0.w));
    *reinterpret_cast<float4*>(&st.alpha[t][c8 + 4]) = make_float4(__expf(g1.x), __expf(g1.y), __expf(g1.z), __expf(g1.w));
    if constexpr (READOUT) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qs[e] = qs[e] * a.scale;
      *reinterpret_cast<float4*>(&st.qs[t][c8]) = make_float4(qs[0], qs[1], qs[2], qs[3]);
      *reinterpret_cast<float4*>(&st.qs[t][c8 + 4]) = make_float4(qs[4], qs[5], qs[6], qs[7]);
      if constexpr (kStageQK) {
        // the decode step's q . k: fma chain over the group's 8 channels, then
        // groups paired across channel-group bit 2, 1, 0, and 3 (the two waves)
        float p = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) p = fmaf(qs[e], k[e], p);
        p = p + xor_lane<4>(p);
        p = p + xor_lane<2>(p);
        p = p + xor_lane<1>(p);
        p = p + xor_lane<8>(p);
        if ((tid & 15) == 0) st.qk[t] = p;
      }
    }
    if (tid < kBlockT) st.beta[tid] = beta;
  } else {
    typename InT::raw4 vr[kVRounds];
#pragma unroll
    for (int j = 0; j < kVRounds; ++j) {
      const int u = tid - kThreads / 2 + j * (kThreads / 2);
      const int tv = u / kVPieces, cv = 4 * (u % kVPieces);
      const int ttv = b0 + tv <= last ? b0 + tv : last;
      if (u < kBlockT * kVPieces) vr[j] = InT::load4raw(a.v, ((int64_t(n) * a.G + ttv) * a.H + h) * kD + col0 + cv);
    }
#pragma unroll
    for (int j = 0; j < kVRounds; ++j) {
      const int u = tid - kThreads / 2 + j * (kThreads / 2);
      const int tv = u / kVPieces, cv = 4 * (u % kVPieces);
      if (u < kBlockT * kVPieces) {
        float f[4];
        InT::unpack4(vr[j], f);
        *reinterpret_cast<float4*>(&st.v[tv][cv]) = make_float4(f[0], f[1], f[2], f[3]);
      }
    }
  }
}

// One token on this lane's 8 x 4 block of S.  red: this slice's [cg][value][2]
// partials in the current buffer; ws: the wave's index within its slice.
// Returns o at the lane's 4 columns when READOUT and need_o (wave-uniform).
// QK_IN: x.qk holds the staged q . k; otherwise it is formed here.
template <bool READOUT, bool QK_IN>
__device__ __forceinline__ void token_step(float (&S)[kR][4], const TokenVals& x,
                                           float (*red)[kRedVals][kWavesPerSlice], int lane, int ws, int cg,
                                           bool need_o, float (&o)[4]) {
  static_assert(!QK_IN || READOUT, "q . k is a readout term");
  constexpr int NV = READOUT ? (QK_IN ? 8 : 9) : 4;
  float acc[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int i = 0; i < kR; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      S[i][j] = S[i][j] * x.alpha[i];                                        // S~ = Diag(alpha) S
      acc[j] = fmaf(x.k[i], S[i][j], acc[j]);                                // r = S~^T k
      if constexpr (READOUT) acc[4 + j] = fmaf(x.qs[i], S[i][j], acc[4 + j]);  // s = S~^T q
    }
    if constexpr (NV == 9) acc[8] = fmaf(x.qs[i], x.k[i], acc[8]);           // q . k
  }
  column_sums<NV>(acc, red, lane, ws, cg, need_o);
  float u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = x.beta * (x.v[j] - acc[j]);
#pragma unroll
  for (int i = 0; i < kR; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) S[i][j] = fmaf(x.k[i], u[j], S[i][j]);     // S = S~ + k u^T
  }
  if constexpr (READOUT) {
    if (need_o) {
      float qk;
      if constexpr (QK_IN) qk = x.qk;
      else qk = acc[NV - 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = fmaf(qk, u[j], acc[4 + j]);       // o = s + (q.k) u
    }
  }
}

template <bool NT>
__device__ __forceinline__ float4 ld_state(const float* p) {
  if constexpr (NT) {
    return make_float4(__builtin_nontemporal_load(p), __builtin_nontemporal_load(p + 1),
                       __builtin_nontemporal_load(p + 2), __builtin_nontemporal_load(p + 3));
  } else {
    return ld_f4(p);
  }
}

template <bool NT>
__device__ __forceinline__ void st_state(float* p, const float (&s)[4]) {
  if constexpr (NT) {
    __builtin_nontemporal_store(s[0], p);
    __builtin_nontemporal_store(s[1], p + 1);
    __builtin_nontemporal_store(s[2], p + 2);
    __builtin_nontemporal_store(s[3], p + 3);
  } else {
    st_f4(p, make_float4(s[0], s[1], s[2], s[3]));
  }
}

// Workgroup index -> work index.  REMAP: the chip's round-robin dispatch over
// its 8 XCDs then gives each XCD one contiguous eighth of the tiles.  Verify
// and commit use it (32 x 12 x 8: 21.4 -> 20.8 us); the decode step does not
// (64 x 12: 18.5 us plain, 19.4 us remapped).
template <bool REMAP>
__device__ __forceinline__ int work_index(int bid, int nblocks) {
  if (REMAP && nblocks % 8 == 0) return (bid % 8) * (nblocks / 8) + bid / 8;
  return bid;
}

// Verify / commit: a workgroup walks kBlockHalves 64-column halves of one
// (request, head), one half's token steps after the other, with every state
// load issued before the first step and the token inputs staged once.  One
// half per workgroup is the default: two (one workgroup per head) measured
// 37 us against 27 us for verify + commit of 32 x 12 x 8, because 384
// workgroups leave the chip under-occupied and each runs 16 dependent steps.
static_assert(kBlockHalves == 1 || kBlockHalves * kWgCols == kD, "halves cover the state");

template <class InT, int MODE, bool PRO, bool REC>
__global__ __launch_bounds__(kThreads) void kda_step_kernel(StepArgs a) {
  static_assert(MODE != kDecode, "decode runs kda_decode_kernel");
  constexpr bool READOUT = (MODE != kCommit);
  constexpr int NH = kBlockHalves;
  __shared__ Red red;
  __shared__ Stage st;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ws = wave % kWavesPerSlice;  // wave within its slice: rows kRowsPerWave * ws ..
  const int sl = wave / kWavesPerSlice;  // slice within the workgroup's columns
  const int cg = lane % kCG;
  const int rg = lane / kCG;
  const int row0 = ws * kRowsPerWave + rg * kR;

  const int wgs_per_head = kWgPerHead / NH;
  const int bid = work_index<true>(blockIdx.x, gridDim.x);
  const int part = bid % wgs_per_head;               // which half (NH == 1) or 0
  const int nh = bid / wgs_per_head;
  const int h = nh % a.H;
  const int n = nh / a.H;
  const int col0 = part * kWgCols * NH;              // first column of the workgroup
  const int wcol = sl * kSliceCols + cg * 4;         // column within a half

  int steps = a.G;
  if (MODE == kCommit) {
    const int L = a.accepted_len[n];
    steps = L < 0 ? 0 : (L > a.G ? a.G : L);
    if (steps == 0 && a.state_out == a.state_in) return;  // nothing accepted, in place: nothing to do
  }
  const int64_t pool_row = a.slots ? int64_t(a.slots[n]) : int64_t(n);
  const int64_t tile = (pool_row * a.H + h) * int64_t(kD * kD);
  const float* Sin = a.state_in + tile;
  if constexpr (MODE == kVerify) {
    // Workgroups of the second and third resident layers (blockIdx / CUs = 1,
    // 2) delay their state loads by ~1.3 us per layer, so that the first
    // layer's loads complete early and its token steps overlap the later
    // layers' loads; all layers otherwise wait for the whole state stream
    // before the first step (measured on 32 x 12 x 8: verify 13.0 -> 12.4 us).
    if (a.layer_wgs > 0) {
      const int layer = min(int(blockIdx.x) / a.layer_wgs, 2);
      for (int i = 0; i < layer; ++i) __builtin_amdgcn_s_sleep(48);
    }
  }

  float S[NH][kR][4];
#pragma unroll
  for (int j = 0; j < NH; ++j)
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const float4 w = ld_f4(Sin + (row0 + i) * kD + col0 + j * kWgCols + wcol);
      S[j][i][0] = w.x; S[j][i][1] = w.y; S[j][i][2] = w.z; S[j][i][3] = w.w;
    }

  const bool out_wave = (ws == 0 && a.o != nullptr);  // wave-uniform: forms o
  const bool writer = out_wave && rg == 0;
  const int last = steps > 0 ? steps - 1 : 0;
  int c = 0;  // token steps so far (alternates the reduction buffers)
  for (int b0 = 0; b0 < steps; b0 += kBlockT) {
    if (b0 > 0) __syncthreads();  // every step of the previous block has read the stage
    stage_block<InT, READOUT, PRO, REC>(st, a, n, h, col0, b0, last, tid);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NH; ++j) {
#pragma unroll
      for (int t = 0; t < kBlockT; ++t) {
        if (b0 + t < steps) {
          TokenVals x;
          float o[4];
          read_token(x, st, t, row0, j * kWgCols + wcol, READOUT);
          token_step<READOUT, READOUT && kStageQK>(S[j], x, red.x[c & 1][sl], lane, ws, cg, out_wave, o);
          ++c;
          if constexpr (READOUT) {
            if (writer)
              InT::store4(a.o, ((int64_t(n) * a.G + b0 + t) * a.H + h) * kD + col0 + j * kWgCols + wcol, o);
          }
        }
      }
    }
  }

  if constexpr (MODE != kVerify) {
    float* Sout = a.state_out + tile;
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int i = 0; i < kR; ++i) st_state<false>(Sout + (row0 + i) * kD + col0 + j * kWgCols + wcol, S[j][i]);
  }
}

#ifndef KDA_DECODE_TILES
#define KDA_DECODE_TILES 1
#endif
// Decode: each workgroup takes kDecodeTiles (request, head, 64-column half)
// tiles and issues all their loads before the first token step.  One tile per
// workgroup is fastest on the 64 x 12 step (18.6 us; 2 tiles 19.2 us, 4 tiles
// 21.2 us: fewer, longer workgroups lose more to the ramp than they gain from
// overlapping a tile's stores with the next tile's loads).
constexpr int kDecodeTiles = KDA_DECODE_TILES;

// Sum of one value over the wave's 8 row groups (lane bits 5, 4, 3), in every
// lane: the pairing column_sums applies to q . k.
__device__ __forceinline__ float rowgroup_allsum(float v) {
  float t = v;
  swap32(v, t);
  v = v + t;
  t = v;
  swap16(v, t);
  v = v + t;
  return v + ror8(v);
}

template <class InT, bool PRO>
__global__ __launch_bounds__(kThreads) void kda_decode_kernel(StepArgs a, int n_tiles) {
  static_assert(!PRO || kWavesPerSlice == 2, "prologue norms pair the slice's two waves");
  __shared__ Red red;
  __shared__ float nrm[kDecodeTiles][kSlicesPerWg][2][kWavesPerSlice];  // |k|^2, |q|^2 per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ws = wave % kWavesPerSlice;
  const int sl = wave / kWavesPerSlice;
  const int cg = lane % kCG;
  const int rg = lane / kCG;
  const int row0 = ws * kRowsPerWave + rg * kR;
  const int wcol = sl * kSliceCols + cg * 4;

  float S[kDecodeTiles][kR][4];
  TokenVals x[kDecodeTiles];
  int64_t toff[kDecodeTiles], ooff[kDecodeTiles];
  bool valid[kDecodeTiles];
  const int bid = work_index<false>(blockIdx.x, gridDim.x);
#pragma unroll
  for (int j = 0; j < kDecodeTiles; ++j) {
    const int t = bid * kDecodeTiles + j;
    valid[j] = t < n_tiles;
    const int tc = valid[j] ? t : bid * kDecodeTiles;  // a spare slot repeats the first tile, unstored
    const int half = tc % kWgPerHead;
    const int nh = tc / kWgPerHead;
    const int h = nh % a.H;
    const int n = nh / a.H;
    const int col = half * kWgCols + wcol;
    const int64_t pool_row = a.slots ? int64_t(a.slots[n]) : int64_t(n);
    toff[j] = (pool_row * a.H + h) * int64_t(kD * kD) + int64_t(row0) * kD + col;
    ooff[j] = (int64_t(n) * a.H + h) * kD + col;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const float4 w = ld_state<true>(a.state_in + toff[j] + i * kD);
      S[j][i][0] = w.x; S[j][i][1] = w.y; S[j][i][2] = w.z; S[j][i][3] = w.w;
    }
    load_token<InT, true, PRO>(x[j], a, n, 0, h, row0, col);
  }
  if constexpr (PRO) {
    // normalise k and q per token: the staged verify / commit inputs' arithmetic
    // (8-channel fma chains, groups paired across lane bits 5, 4, 3, then the
    // slice's two waves in order)
    if (a.pro_l2) {
#pragma unroll
      for (int j = 0; j < kDecodeTiles; ++j) {
        float pk = 0.0f, pq = 0.0f;
#pragma unroll
        for (int i = 0; i < kR; ++i) {
          pk = fmaf(x[j].k[i], x[j].k[i], pk);
          pq = fmaf(x[j].qs[i], x[j].qs[i], pq);
        }
        pk = rowgroup_allsum(pk);
        pq = rowgroup_allsum(pq);
        if (lane == 0) {
          nrm[j][sl][0][ws] = pk;
          nrm[j][sl][1][ws] = pq;
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kDecodeTiles; ++j) {
        const float rk = inv_l2(nrm[j][sl][0][0] + nrm[j][sl][0][1], a.pro_eps);
        const float rq = inv_l2(nrm[j][sl][1][0] + nrm[j][sl][1][1], a.pro_eps);
#pragma unroll
        for (int i = 0; i < kR; ++i) {
          x[j].k[i] = x[j].k[i] * rk;
          x[j].qs[i] = (x[j].qs[i] * rq) * a.scale;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kDecodeTiles; ++j)
#pragma unroll
        for (int i = 0; i < kR; ++i) x[j].qs[i] = x[j].qs[i] * a.scale;
    }
  }
  const bool out_wave = (ws == 0 && a.o != nullptr);  // wave-uniform: forms o
  const bool writer = out_wave && rg == 0;
#pragma unroll
  for (int j = 0; j < kDecodeTiles; ++j) {
    float o[4];
    token_step<true, false>(S[j], x[j], red.x[j & 1][sl], lane, ws, cg, out_wave, o);
    if (valid[j]) {
      if (writer) InT::store4(a.o, ooff[j], o);
#pragma unroll
      for (int i = 0; i < kR; ++i) st_state<true>(a.state_out + toff[j] + i * kD, S[j][i]);
    }
  }
}

template <int MODE, bool PRO, bool REC = false>
hipError_t launch_step_as(const StepArgs& a, bool bf16, hipStream_t stream) {
  const int64_t blocks = int64_t(a.N) * a.H * (kWgPerHead / kBlockHalves);
  if (bf16)
    hipLaunchKernelGGL((kda_step_kernel<BF16, MODE, PRO, REC>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((kda_step_kernel<F32, MODE, PRO, REC>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// The prologue's norms use the 8-rows-per-lane layout (two waves per slice).
constexpr bool kPrologueBuilt = (kWavesPerSlice == 2);

void set_prologue(StepArgs& a, const Prologue* pro) {
  a.pro_l2 = pro && pro->l2norm;
  a.pro_eps = pro ? pro->eps : 0.0f;
  a.pro_gate = pro && pro->gate;
  a.pro_gmin = pro ? pro->g_min : 0.0f;
}

template <int MODE>
hipError_t launch_step(StepArgs a, bool bf16, hipStream_t stream, const Prologue* pro) {
  if (!pro) return launch_step_as<MODE, false>(a, bf16, stream);
  if constexpr (kPrologueBuilt) {
    set_prologue(a, pro);
    return launch_step_as<MODE, true>(a, bf16, stream);
  }
  return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         float* state, const int32_t* slots, int N, int H, bool bf16, float scale, void* o,
                         hipStream_t stream, const Prologue* pro) {
  StepArgs a{q, k, v, g, beta, state, state, slots, nullptr, o, N, 1, H, scale, 0, 0, 0.0f, 0, 0.0f};
  const int n_tiles = N * H * kWgPerHead;
  const unsigned blocks = unsigned((n_tiles + kDecodeTiles - 1) / kDecodeTiles);
  if (!pro) {
    if (bf16)
      hipLaunchKernelGGL((kda_decode_kernel<BF16, false>), dim3(blocks), dim3(kThreads), 0, stream, a, n_tiles);
    else
      hipLaunchKernelGGL((kda_decode_kernel<F32, false>), dim3(blocks), dim3(kThreads), 0, stream, a, n_tiles);
    return hipGetLastError();
  }
  if constexpr (kPrologueBuilt) {
    set_prologue(a, pro);
    if (bf16)
      hipLaunchKernelGGL((kda_decode_kernel<BF16, true>), dim3(blocks), dim3(kThreads), 0, stream, a, n_tiles);
    else
      hipLaunchKernelGGL((kda_decode_kernel<F32, true>), dim3(blocks), dim3(kThreads), 0, stream, a, n_tiles);
    return hipGetLastError();
  }
  return hipErrorNotSupported;
}

hipError_t launch_verify(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* state, const int32_t* slots, int N, int G, int H, bool bf16,
                         float scale, void* o, hipStream_t stream, const Prologue* pro, float* record) {
  StepArgs a{q, k, v, g, beta, state, nullptr, slots, nullptr, o, N, G, H, scale, device_cu_count(), 0, 0.0f, 0, 0.0f};
  a.record = record;
  return launch_step<kVerify>(a, bf16, stream, pro);
}

hipError_t launch_commit(const void* k, const void* v, const float* g, const float* beta,
                         const float* state_in, float* state_out, const int32_t* slots,
                         const int32_t* accepted_len, int N, int G, int H, bool bf16, hipStream_t stream,
                         const Prologue* pro) {
  StepArgs a{nullptr, k, v, g, beta, state_in, state_out, slots, accepted_len, nullptr, N, G, H, 1.0f, 0, 0, 0.0f, 0,
             0.0f};
  return launch_step<kCommit>(a, bf16, stream, pro);
}

hipError_t launch_commit_record(const float* record, const void* v, const float* beta, const float* state_in,
                                float* state_out, const int32_t* slots, const int32_t* accepted_len, int N, int G,
                                int H, bool bf16, hipStream_t stream) {
  StepArgs a{nullptr, nullptr, v, nullptr, beta, state_in, state_out, slots, accepted_len, nullptr, N, G, H, 1.0f,
             0, 0, 0.0f, 0, 0.0f};
  a.rec_in = record;
  return launch_step_as<kCommit, false, true>(a, bf16, stream);
}

}  // namespace kda
