// Chunk-parallel prefill of the KDA recurrence on gfx950 MFMA.
//
// Math (the update is from "Kimi K3：架构与 SGLang Day-0 Support",
// section "attention 机制详解：KDA"; the chunkwise form rescales keys by the
// inverse cumulative decay, as remarked in the same math box).  For a chunk of
// n tokens with entry state S (128 x 128, rows = key channels) and
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
// with V = 0 and no outputs.  Chunks are 32 tokens here; every sequence (and
// every segment a caller cuts at a multiple of 64 tokens) starts a chunk, so
// the result is the same recurrence whatever the chunk size.
//
// Decomposition: one workgroup of 8 waves per (sequence, head, column slice),
// walking the sequence's chunks in order with the state in registers.
//   waves 0-3 (state): each owns 16*JB value columns of S in MFMA accumulator
//             registers for the whole sequence and, per chunk, computes
//             R = V - Kh S, O = Qh S + P U with U = T' R, S = Gamma S + Kb^T U.
//   waves 4-7 (prep):  build the NEXT chunk's operands: cumulative decay
//             (token pairs in-thread, then a scan over the 16 pairs), Kh, Kc, Qh,
//             Kb^T, the A and P tiles on MFMA, the 16x16 diagonal inverses of
//             I + A by right-looking substitution in registers, the
//             off-diagonal block T_10 = -T_11 A_10 T_00 on MFMA, and T'.
// Operand sets are double-buffered in LDS: in step i the prep waves write set
// i % 2 (chunk i) while the state waves read set (i - 1) % 2 (chunk i - 1).
// Each step has three workgroup barriers that both groups pass in lockstep:
//   phase A  state: Kh S, Qh S           | prep: decay scan, operands
//   phase B  state: T' R, P U, outputs   | prep: A, P tiles; diagonal inverses
//   phase C  state: Gamma S + Kb^T U     | prep: T_10, T'
// Inputs are fetched one chunk ahead into registers (prep: g, k, q, beta in
// phase B; state: v in phase C).  Two waves share each SIMD, so one wave's
// MFMA work overlaps the other's LDS and VALU work.
//
// Builds (template MODE and wave counts):
//   Fused  the decomposition above: 4 state waves of 16 or 32 columns with 8
//          or 4 prep waves; or, for states and transitions without outputs on
//          a grid that fills the device, 8 state waves (4 hold the state, 4 the
//          transition, 32 columns each) sharing 4 prep waves, so each chunk is
//          prepared once for both.
//   Prep   the split path's preparation: one workgroup per (chunk slot, head)
//          builds that chunk's operand set and writes it to the caller's
//          workspace (chunk-parallel: the sets do not depend on the state).
//   State  the split path's walk: state waves only, one workgroup per
//          (sequence, head), staging chunk c+1's set from the workspace while
//          chunk c runs (8 waves of 16 columns; 16 when the transition walks
//          beside the state).
#include "kda_common.hpp"
#include "kda_internal.hpp"
#include "kda_mfma.hpp"

namespace kda {
namespace {

constexpr int kC = 32;           // chunk length (tokens)

// SW state waves + PW prep waves (PW = 4: 4 tokens x 4 channels per prep
// thread; PW = 8: 2 tokens x 4 channels).
__host__ __device__ constexpr int prefill_threads(int sw, int pw) { return 64 * (sw + pw); }

// LDS layout.  NSETS operand sets (2: double-buffered between the prep and
// state roles, or between the state walk's staging and use; 1: the prep-only
// kernel); PREP: whether the prep scratch follows them.
template <class Pol, int NSETS = 2, bool PREP = true>
struct Lds {
  static constexpr int E = Pol::kElem;
  static constexpr int P = Pol::kPlanes;
  static constexpr int kOpRow = kD * E + 16;               // [32 tok][128 ch]: Kh, Kc, Qh
  static constexpr int kOpPlane = kC * kOpRow;
  static constexpr int kOpBytes = P * kOpPlane;
  static constexpr int kKbRow = kC * E + 16;               // [128 ch][32 tok]: Kb^T
  static constexpr int kKbPlane = kD * kKbRow;
  static constexpr int kKbBytes = P * kKbPlane;
  static constexpr int kSqRow = kC * E + 16;               // [32][32]: T', P
  static constexpr int kSqPlane = kC * kSqRow;
  static constexpr int kSqBytes = P * kSqPlane;
  static constexpr int kNatRow = 16 * E + (E == 2 ? 8 : 16);  // [rows][16], natural order: A_10
  static constexpr int kAopPlane = 16 * kNatRow;
  static constexpr int kAopBytes = P * kAopPlane;
  static constexpr int kFLd = 20;                          // fp32 [2 blocks][16][20]
  static constexpr int kFBytes = 2 * 16 * kFLd * 4;
  // one operand set (read by the state waves); Kb^T last, so that the prep
  // build, which writes it straight to the workspace, keeps only the rest; the
  // output operands (Qh, P) just before it, so that a walk without outputs
  // stages the set in two ranges, [Kh, Qh) and [Kb, end)
  static constexpr int kSetKh = 0;
  static constexpr int kSetTp = kSetKh + kOpBytes;
  static constexpr int kSetGamma = kSetTp + kSqBytes;      // e^{b_last - b_mid} per channel
  static constexpr int kSetEm = kSetGamma + kD * 4;         // e^{b_mid} per channel
  static constexpr int kSetQh = kSetEm + kD * 4;
  static constexpr int kSetP = kSetQh + kOpBytes;
  static constexpr int kSetKb = kSetP + kSqBytes;
  static constexpr int kSetBytes = kSetKb + kKbBytes;
  static constexpr int kSetInLds = NSETS == 1 ? kSetKb : kSetBytes;  // prep build: the set without Kb^T
  // prep scratch
  static constexpr int kKc = NSETS * kSetInLds;
  static constexpr int kAop = kKc + kOpBytes;              // A_10 (beta-scaled), MFMA operand
  static constexpr int kAt = kAop + kAopBytes;             // A_II transposed, fp32: At[I][s][r]
  static constexpr int kTd = kAt + kFBytes;                // T_II column-major, fp32: Td[I][j][r]
  static constexpr int kBeta = kTd + kFBytes;              // 32 floats
  static constexpr int kNrm = kBeta + kC * 4;              // prologue: [token][prep wave][k, q] sums of squares
  static constexpr int kBytes = PREP ? kNrm + kC * 8 * 2 * 4 : NSETS * kSetBytes;
  static_assert(kSetKb % 16 == 0, "aligned");
  static_assert(kBytes <= 160 * 1024, "LDS budget");
  static_assert(kOpRow % 16 == 0 && kKbRow % 16 == 0 && kSqRow % 16 == 0 && kSetBytes % 16 == 0, "aligned");
  static_assert(kNatRow % 8 == 0 && (E == 2 || kNatRow % 16 == 0), "aligned natural rows");

  // The set as a workspace holds it: the same regions in the same order, each
  // row without the 16 bytes of padding it carries in LDS (the padding only
  // spreads LDS banks; in HBM it would be 12% more bytes to write and read).
  static constexpr int kGOpRow = kD * E, kGSqRow = kC * E, kGKbRow = kC * E;
  static constexpr int kGOpBytes = P * kC * kGOpRow, kGSqBytes = P * kC * kGSqRow;
  static constexpr int kGKbPlane = kD * kGKbRow;
  static constexpr int kGKh = 0;
  static constexpr int kGTp = kGKh + kGOpBytes;
  static constexpr int kGGamma = kGTp + kGSqBytes;
  static constexpr int kGQh = kGGamma + 2 * kD * 4;        // Gamma and Em
  static constexpr int kGP = kGQh + kGOpBytes;
  static constexpr int kGKb = kGP + kGSqBytes;
  static constexpr int kGBytes = kGKb + P * kGKbPlane;
  static_assert(kGOpRow % 16 == 0 && kGSqRow % 16 == 0 && kGBytes % 16 == 0, "aligned");
  static_assert(kOpRow == kGOpRow + 16 && kSqRow == kGSqRow + 16 && kKbRow == kGKbRow + 16, "one pad piece per row");
  static_assert(kSetEm == kSetGamma + kD * 4 && kSetQh == kSetEm + kD * 4, "Gamma, Em adjacent");

  // LDS 16-byte piece of the set holding workspace piece x: a padded row of n
  // data pieces takes n + 1 pieces in LDS
  __device__ __forceinline__ static int lds_piece(int x) {
    if (x < kGTp / 16) return x + x / (kGOpRow / 16);
    if (x < kGGamma / 16) { const int r = x - kGTp / 16; return kSetTp / 16 + r + r / (kGSqRow / 16); }
    if (x < kGQh / 16) return kSetGamma / 16 + (x - kGGamma / 16);
    if (x < kGP / 16) { const int r = x - kGQh / 16; return kSetQh / 16 + r + r / (kGOpRow / 16); }
    if (x < kGKb / 16) { const int r = x - kGP / 16; return kSetP / 16 + r + r / (kGSqRow / 16); }
    const int r = x - kGKb / 16;
    return kSetKb / 16 + r + r / (kGKbRow / 16);
  }
};

// x from lane (lane - D) of the same G-lane group, 0 for the first D lanes of
// the group (G = 8 or 16; groups start at multiples of G).  A DPP row shift
// (16 lanes) moves values across the 8-lane groups of a row; those are zeroed.
template <int D, int G>
__device__ __forceinline__ float dpp_shr_in_group(float x, int idx_in_group) {
  const float y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + D, 0xF, 0xF, true));
  if constexpr (G == 16) return y;
  else return idx_in_group >= D ? y : 0.0f;
}

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* cu_seqlens;
  int32_t H;
  int32_t n_value_slices;  // 128 / (16 * JB * SW)
  int32_t n_slices;        // value slices (+ as many transition slices)
  int32_t slice_base;      // first slice this launch covers
  int32_t n_launch_slices; // slices per (sequence, head) this launch covers
  float scale;
  const float* initial_state;
  float* final_state;
  void* o;
  float* transition_out;
  float* checkpoints;       // or null: states at multiples of ckpt_interval tokens
  int32_t ckpt_interval;    // positive multiple of 64 when checkpoints is set
  const int32_t* seq_order; // or null: workgroup rank -> sequence (a permutation of 0 .. num_seqs - 1)
  int32_t num_seqs;
  int32_t pro_l2;           // prologue variant: normalise q and k per token
  float pro_eps;
  int32_t pro_gate;         // prologue variant: g holds gate logits
  float pro_gmin;
  char* ws;                 // split path: operand sets, [chunk slot][H] of one set each
  int32_t prep_outputs;     // prep build: also build the output operands (Qh, P)
};

// The split path's chunk slots: chunk j of sequence n lives in slot
// (cu[n] / 32) + n + j.  Slots of different sequences never collide (a
// sequence of L tokens has ceil(L / 32) chunks and the next one starts at
// least that many slots later) and every slot is below cu[N] / 32 + N + 1.
__host__ __device__ __forceinline__ int chunk_slot_base(int cu_n, int n) { return (cu_n >> 5) + n; }

// Roles of one prefill kernel build.
//   Fused: state and prep waves in one workgroup per (sequence, head, column
//          slice), the operand sets handed over through LDS.
//   Prep:  prep waves only, one workgroup per (chunk slot, head): builds that
//          chunk's operand set and writes it to the workspace.
//   State: state waves only, per (sequence, head, column slice): each chunk's
//          operand set is staged from the workspace into LDS one chunk ahead.
// The prep and state code is the same in every mode, so the split path (Prep,
// then State) gives the fused path's results bit for bit.
enum class Mode { Fused, Prep, State };

// Input prologue (the KDA math-details box of the Day-0 lesson page: unit keys;
// the log-decay bounded below by a scaled sigmoid, g_min = -5).
__device__ __forceinline__ float gate_log_decay(float x, float g_min) {
  return g_min * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}


// Prep-thread inputs of one chunk (TPT tokens x 4 channels), as loaded.
template <class InT, int TPT>
struct PrepIn {
  float4 g[TPT];
  typename InT::raw4 k[TPT], q[TPT];
  float beta;
};

template <class InT, int TPT>
__device__ __forceinline__ void load_prep(PrepIn<InT, TPT>& in, const PrefillArgs& a, int t0, int n, int h, int tg,
                                          int c0, int ptid, bool need_q) {
  // wave-uniform chunk base + 32-bit per-lane offsets; rows past the chunk end
  // are clamped to its last token (always valid) and masked where they are used
  const int64_t cbase = (int64_t(t0) * a.H + h) * kD;
  const int rstride = a.H * kD;
  const float* gb = a.g + cbase;
  const char* kb = reinterpret_cast<const char*>(a.k) + cbase * int64_t(sizeof(typename InT::storage));
  const char* qb = reinterpret_cast<const char*>(a.q) + cbase * int64_t(sizeof(typename InT::storage));
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int r = TPT * tg + i;
    const int off = (r < n ? r : n - 1) * rstride + c0;
    in.g[i] = ld_f4(gb + off);
    in.k[i] = InT::load4raw(kb, off);
    in.q[i] = need_q ? InT::load4raw(qb, off) : typename InT::raw4{};
  }
  in.beta = a.beta[int64_t(t0) * a.H + h + (ptid < n ? ptid : n - 1) * a.H];
}

// Sum over the lanes that differ in bits log2(NTG) .. 5 (a wave's channel
// groups), in every lane: a DPP rotation by 8 within 16-lane rows (NTG = 8),
// then the 16- and 32-lane permute-swaps.  Either shape sums 4 consecutive
// channel groups as ((c0 + c1) + (c2 + c3)); the 128-column shape then adds
// two such sums, the 64-column one leaves that to the cross-wave sum.
template <int NTG>
__device__ __forceinline__ float sum_channel_groups(float v) {
  if constexpr (NTG == 8) v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}

// Prologue norms, one chunk ahead of their use: this prep thread's sums of
// squares of k and q (TPT tokens x 4 channels), summed over the wave's channel
// groups, are written per (token, prep wave) to LDS.
template <class InT, int TPT, int NTG>
__device__ __forceinline__ void prep_prologue(const PrepIn<InT, TPT>& pin, const PrefillArgs& a, float* nrm,
                                              int lane, int tg, int pw, bool want_q) {
  if (!a.pro_l2) return;
#pragma unroll
  for (int rr = 0; rr < TPT; ++rr) {
    float kv[4], qv[4];
    InT::unpack4(pin.k[rr], kv);
    InT::unpack4(pin.q[rr], qv);
    float sk = 0.0f, sq = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sk = fmaf(kv[e], kv[e], sk);
      sq = fmaf(qv[e], qv[e], sq);
    }
    sk = sum_channel_groups<NTG>(sk);
    sq = sum_channel_groups<NTG>(sq);
    if (lane < NTG) {
      float* dst = nrm + ((TPT * tg + rr) * 8 + pw) * 2;
      dst[0] = sk;
      dst[1] = want_q ? sq : 0.0f;
    }
  }
}

// State-wave v of one chunk at this wave's columns.
//  fp32 inputs: the accumulator layout directly (rows 16rt+4lq+i, column lj).
//  bf16 inputs: lane (lq, lj) holds token 16rt+lj, columns 4lq..4lq+3 of each
//  16-column block (one 8-byte load); one bf16 MFMA against a negated
//  identity moves the block into the accumulator layout as -V, exactly.
template <class InT, int JB>
struct StateV {
  static constexpr bool kBf16 = false;
  typename InT::raw1 v[JB][2][4];
};
template <int JB>
struct StateV<BF16, JB> {
  static constexpr bool kBf16 = true;
  uint2 vb[JB][2];
};

template <class InT, int JB>
__device__ __forceinline__ void load_state_v(StateV<InT, JB>& sv, const PrefillArgs& a, int t0, int n, int h, int lq,
                                             int lj, int colw) {
  const char* vb = reinterpret_cast<const char*>(a.v) +
                   ((int64_t(t0) * a.H + h) * kD + colw) * int64_t(sizeof(typename InT::storage));
  const int rstride = a.H * kD;
  if constexpr (StateV<InT, JB>::kBf16) {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int r = 16 * rt + lj;
        sv.vb[jb][rt] = *reinterpret_cast<const uint2*>(vb + int64_t((r < n ? r : n - 1) * rstride + 16 * jb + 4 * lq) * 2);
      }
  } else {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lq + i;
          sv.v[jb][rt][i] = InT::load1raw(vb, (r < n ? r : n - 1) * rstride + 16 * jb + lj);
        }
  }
}

// WO: every workgroup of the launch writes outputs (value slices with o set);
// otherwise none does.  A compile-time property so the output products carry
// no branch inside the MFMA sequences (a runtime test there made the compiler
// move accumulators out and back around every conditional MFMA).  The prep
// build reads it from the arguments.
template <class Pol, class InT, int SW, int JB, int PW, bool CKPT, bool PRO, Mode MODE, bool WO>
__global__ __launch_bounds__(prefill_threads(SW, PW)) void kda_prefill_kernel(PrefillArgs a) {
  static_assert(!(CKPT && PRO), "checkpoints and the prologue are separate variants");
  static_assert(MODE == Mode::State ? PW == 0 : (PW == 4 || PW == 8), "prep waves");
  static_assert(MODE == Mode::Prep ? SW == 0
                                   : (SW == 4 || (MODE == Mode::State && (SW == 8 || SW == 16)) ||
                                      (MODE == Mode::Fused && SW == 8 && JB == 2)),
                "state waves");
  // Builds that hold a (sequence, head)'s state and its transition in one
  // workgroup (the first half of the state waves the state, the second half
  // the transition, all 128 columns each) serve a segmented prefill's pass 1:
  // the 16-wave state build reads each staged set once for both, the 8-wave
  // fused build prepares each chunk once for both.
  constexpr bool kBoth = (MODE == Mode::State && SW == 16) || (MODE == Mode::Fused && SW == 8);
  static_assert(!kBoth || (16 * JB * (SW / 2) == kD && !WO && !CKPT), "state and transition builds serve pass 1 only");
  static_assert(MODE == Mode::Fused || !CKPT, "checkpoints are written by the fused build");
  constexpr int PWX = PW > 0 ? PW : 8;  // (role constants of a build without prep waves are unused)
  constexpr int TPT = 16 / PWX;  // tokens per prep thread (4 or 2)
  constexpr int NTG = kC / TPT;  // token groups per channel group (8 or 16 lanes)
  using L = Lds<Pol, MODE == Mode::Prep ? 1 : 2, MODE != Mode::State>;
  using Frag = typename Pol::Frag;
  using Frag16 = typename Pol::Frag16;
  constexpr int E = L::E;
  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
  float* s_beta = reinterpret_cast<float*>(smem + L::kBeta);
  float* s_at = reinterpret_cast<float*>(smem + L::kAt);
  float* s_td = reinterpret_cast<float*>(smem + L::kTd);
  float* s_nrm = reinterpret_cast<float*>(smem + L::kNrm);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane >> 4;
  const int lj = lane & 15;
  const bool is_state = wave < SW;

  int slice, h, seq, pchunk = 0;
  if constexpr (MODE == Mode::Prep) {
    // workgroup = (chunk slot, head); the sequence holding the slot is the last
    // one whose first slot is at or below it (first slots increase with n)
    slice = 0;
    h = blockIdx.x % a.H;
    const int slot = blockIdx.x / a.H;
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (chunk_slot_base(a.cu_seqlens[mid], mid) <= slot) lo = mid;
      else hi = mid - 1;
    }
    seq = lo;
    pchunk = slot - chunk_slot_base(a.cu_seqlens[seq], seq);
    const int len = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
    if (pchunk < 0 || pchunk * kC >= len) return;  // a slot between sequences
  } else {
    slice = a.slice_base + int(blockIdx.x % unsigned(a.n_launch_slices));
    const int sh = blockIdx.x / unsigned(a.n_launch_slices);
    h = sh % a.H;
    seq = a.seq_order ? a.seq_order[sh / a.H] : sh / a.H;
  }
  if (seq < 0 || seq >= a.num_seqs) return;  // not a sequence of the batch (a bad order entry)
  const bool is_transition = kBoth ? wave >= SW / 2 : slice >= a.n_value_slices;
  const int vslice = kBoth ? 0 : (is_transition ? slice - a.n_value_slices : slice);
  const int64_t H = a.H;
  const int64_t tile_base = (int64_t(seq) * H + h) * (kD * kD);
  const int bos = a.cu_seqlens[seq];
  const int eos = a.cu_seqlens[seq + 1];
  const int nch = (eos - bos + kC - 1) / kC;
  const bool want_o = MODE == Mode::Prep ? a.prep_outputs != 0 : WO;

  // state-wave roles
  const int colw = kBoth ? (wave % (SW / 2)) * (16 * JB) : vslice * (16 * JB * SW) + (is_state ? wave : 0) * (16 * JB);
  // prep-thread roles: TPT consecutive tokens x 4 consecutive channels; the
  // NTG token groups of a channel group are NTG consecutive lanes of a DPP row
  const int ptid = tid - SW * 64;
  const int tg = ptid % NTG;
  const int c0 = (ptid / NTG) * 4;
  const int pw = wave - SW;

  f32x4_t S[JB][8];
  if (is_state) {
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
  }

  const bool ckpt_on = CKPT && !is_transition;

  // The two roles run separate loops (so each keeps only its own values in
  // registers) with the same three barriers per step.
  if constexpr (MODE != Mode::Prep) if (is_state) {
    StateV<InT, JB> sv;
    f32x4_t accR[JB][2], accO[JB][2];
    // B operand -I for the V transposition: slot e < 4 of lane group lq is
    // column 4lq + e, the other four slots are zero
    bf16x8_t neg_eye = {};
    if constexpr (StateV<InT, JB>::kBf16) {
  #pragma unroll
      for (int e = 0; e < 4; ++e) neg_eye[e] = (4 * lq + e == lj) ? (__bf16)(-1.0f) : (__bf16)(0.0f);
    }
    Frag uf[JB];
    // State build: operand sets come from the workspace, chunk c's into set
    // c % 2, loaded into registers one step ahead and written to LDS at the
    // end of the step that precedes their use
    // The set is copied through registers: seventeen 16-byte loads per thread,
    // issued at the start of the step before its use (their latency hides
    // under the step), written to LDS at that step's end, before its closing
    // barrier.  (Direct global-to-LDS loads were measured to hold the issuing
    // wave ~110 cycles each; seventeen named registers rather than an array,
    // which the compiler had placed in scratch memory.)
    // a walk without outputs skips the output operands, [Qh, Kb): piece x of
    // what it stages is piece x (below Qh) or x + kSkip16 of the set
    // (pieces of the workspace layout; each lands at its padded LDS place)
    constexpr int kSkipAt16 = WO ? L::kGBytes / 16 : L::kGQh / 16;
    constexpr int kSkip16 = WO ? 0 : (L::kGKb - L::kGQh) / 16;
    constexpr int kN16 = L::kGBytes / 16 - kSkip16;
    static_assert(MODE != Mode::State || (kN16 + 64 * SW - 1) / (64 * SW) <= 17, "seventeen staging registers");
    const int64_t slot0 = chunk_slot_base(bos, seq);
#define KDA_REP17(X) X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)
#define KDA_STG_DECL(e) uint4 stg##e;
    constexpr int kStageN = (kN16 + 64 * SW - 1) / (64 * SW);  // loads per thread
#define KDA_STG_PIECE(x) ((x) < kSkipAt16 ? (x) : (x) + kSkip16)
#define KDA_STG_LD(e) if constexpr ((e) < kStageN) stg##e = src_[KDA_STG_PIECE(tid + 64 * SW * (e) < kN16 ? tid + 64 * SW * (e) : kN16 - 1)];
#define KDA_STG_ST(e) if constexpr ((e) < kStageN) { if (tid + 64 * SW * (e) < kN16) dst_[L::lds_piece(KDA_STG_PIECE(tid + 64 * SW * (e)))] = stg##e; }
    KDA_REP17(KDA_STG_DECL)
    // (the loads are unconditional, chunk index clamped to the last chunk, so
    // the compiler's wait for the v loads before them is not widened over a
    // branch that skips them)
#define KDA_STAGE_LOAD(c)                                                                               \
    if constexpr (MODE == Mode::State) {                                                                \
      const int64_t c_ = (c) < nch ? (c) : nch - 1;                                                     \
      const uint4* src_ = reinterpret_cast<const uint4*>(a.ws + ((slot0 + c_) * H + h) * int64_t(L::kGBytes));    \
      KDA_REP17(KDA_STG_LD)                                                                             \
    }
#define KDA_STAGE_STORE(c, set)                                                                         \
    if constexpr (MODE == Mode::State) {                                                                \
      if ((c) < nch) {                                                                                  \
        uint4* dst_ = reinterpret_cast<uint4*>(smem + (set) * L::kSetBytes);                            \
        KDA_REP17(KDA_STG_ST)                                                                           \
      }                                                                                                 \
    }
    // step 0: the prep waves build chunk 0 (or chunk 0's set is staged); fetch chunk 0's v
    if (nch > 0) load_state_v<InT, JB>(sv, a, bos, eos - bos < kC ? eos - bos : kC, h, lq, lj, colw);
    if constexpr (MODE == Mode::State) {
      if (nch > 0) {
        KDA_STAGE_LOAD(0)
        KDA_STAGE_STORE(0, 0)
      }
      __syncthreads();
    } else {
      if constexpr (PRO) __syncthreads();  // the prep waves' chunk-0 norms
      __syncthreads();
      __syncthreads();
      __syncthreads();
    }
    for (int i = 1; i <= nch; ++i) {
      if constexpr (MODE == Mode::State) {
        KDA_STAGE_LOAD(i)  // chunk i's set, for set i & 1 (last read in step i - 1)
      }
      // this step consumes chunk i - 1 from operand set (i - 1) % 2
      const int ts = bos + (i - 1) * kC;
      const int ns = eos - ts < kC ? eos - ts : kC;
      const char* sset = smem + ((i + 1) & 1) * L::kSetBytes;

      // ============================== phase A ==============================
        {
  #pragma unroll
          for (int jb = 0; jb < JB; ++jb)
  #pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
              if constexpr (StateV<InT, JB>::kBf16) {
                // -V block by MFMA: A = V rows (tokens past the chunk end and
                // transition runs give zero rows), B = -I in this lane's slots
                const bool keep = !is_transition && 16 * rt + lj < ns;
                const u32x4_t aw = {keep ? sv.vb[jb][rt].x : 0u, keep ? sv.vb[jb][rt].y : 0u, 0u, 0u};
                accR[jb][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, aw), neg_eye,
                                                                     f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
              } else {
  #pragma unroll
                for (int e = 0; e < 4; ++e)
                  accR[jb][rt][e] = (!is_transition && 16 * rt + 4 * lq + e < ns) ? -InT::unpack1(sv.v[jb][rt][e]) : 0.0f;
              }
              accO[jb][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
          if constexpr (MODE == Mode::State) {  // fetch chunk i's v now that chunk i - 1's is consumed
            const int tv = bos + (i < nch ? i : nch - 1) * kC;
            load_state_v<InT, JB>(sv, a, tv, eos - tv < kC ? eos - tv : kC, h, lq, lj, colw);
          }
          // the chunk's operands are referenced at b_mid: carry S as e^{b_mid} S
          // (rows = key channels); phase C applies e^{b_last - b_mid}
          {
            const float* s_em = reinterpret_cast<const float*>(sset + L::kSetEm);
  #pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
              const float4 em = *reinterpret_cast<const float4*>(s_em + 16 * ct + 4 * lq);
  #pragma unroll
              for (int jb = 0; jb < JB; ++jb) {
                S[jb][ct][0] *= em.x; S[jb][ct][1] *= em.y; S[jb][ct][2] *= em.z; S[jb][ct][3] *= em.w;
              }
            }
          }
          // R = V - Kh S (accumulated as Kh S - V) and O = Qh S; each 32-row
          // block of S is split once and feeds both products
          // (state build: every fragment of the four steps is read up front,
          // so the LDS latency is paid once per chunk, not once per step)
          constexpr int kPre = MODE == Mode::State ? 4 : 1;
          Frag fk[kPre][2], fq[kPre][2];
  #pragma unroll
          for (int ks = 0; ks < kPre; ++ks)
  #pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
              const int off = (16 * rt + lj) * L::kOpRow + (32 * ks + 8 * lq) * E;
              fk[ks][rt] = Pol::load(sset + L::kSetKh, L::kOpPlane, off);
              if (want_o) fq[ks][rt] = Pol::load(sset + L::kSetQh, L::kOpPlane, off);
            }
  #pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            Frag sf[JB];
  #pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
              const float v8[8] = {S[jb][2 * ks][0], S[jb][2 * ks][1], S[jb][2 * ks][2], S[jb][2 * ks][3],
                                   S[jb][2 * ks + 1][0], S[jb][2 * ks + 1][1], S[jb][2 * ks + 1][2],
                                   S[jb][2 * ks + 1][3]};
              sf[jb] = Pol::make(v8);
            }
            const int kk = kPre == 4 ? ks : 0;
            if constexpr (kPre == 1) {
  #pragma unroll
              for (int rt = 0; rt < 2; ++rt) {
                const int off = (16 * rt + lj) * L::kOpRow + (32 * ks + 8 * lq) * E;
                fk[0][rt] = Pol::load(sset + L::kSetKh, L::kOpPlane, off);
                if (want_o) fq[0][rt] = Pol::load(sset + L::kSetQh, L::kOpPlane, off);
              }
            }
  #pragma unroll
            for (int p = 0; p < Pol::kParts; ++p)
  #pragma unroll
              for (int rt = 0; rt < 2; ++rt)
  #pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                  Pol::mma_part(accR[jb][rt], fk[kk][rt], sf[jb], p);
                  if (want_o) Pol::mma_part(accO[jb][rt], fq[kk][rt], sf[jb], p);
                }
          }
        }
      // (the state build's set was complete when the step began and each wave
      // works on its own columns: it needs no barrier inside the step)
      if constexpr (MODE != Mode::State) __syncthreads();
      // ============================== phase B ==============================
        {
          // U = T' R (one 32-deep step), then O += P U and the outputs
          Frag rf[JB];
  #pragma unroll
          for (int jb = 0; jb < JB; ++jb) {
            const float v8[8] = {-accR[jb][0][0], -accR[jb][0][1], -accR[jb][0][2], -accR[jb][0][3],
                                 -accR[jb][1][0], -accR[jb][1][1], -accR[jb][1][2], -accR[jb][1][3]};
            rf[jb] = Pol::make(v8);
          }
          f32x4_t accU[JB][2];
  #pragma unroll
          for (int jb = 0; jb < JB; ++jb)
  #pragma unroll
            for (int rt = 0; rt < 2; ++rt) accU[jb][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          {
            Frag ft[2];
  #pragma unroll
            for (int rt = 0; rt < 2; ++rt)
              ft[rt] = Pol::load(sset + L::kSetTp, L::kSqPlane, (16 * rt + lj) * L::kSqRow + 8 * lq * E);
  #pragma unroll
            for (int p = 0; p < Pol::kParts; ++p)
  #pragma unroll
              for (int rt = 0; rt < 2; ++rt)
  #pragma unroll
                for (int jb = 0; jb < JB; ++jb) Pol::mma_part(accU[jb][rt], ft[rt], rf[jb], p);
          }
  #pragma unroll
          for (int jb = 0; jb < JB; ++jb) {
            const float v8[8] = {accU[jb][0][0], accU[jb][0][1], accU[jb][0][2], accU[jb][0][3],
                                 accU[jb][1][0], accU[jb][1][1], accU[jb][1][2], accU[jb][1][3]};
            uf[jb] = Pol::make(v8);
          }
          if (want_o) {
            // the chunk's rows of this head as a buffer resource whose range ends
            // after row ns - 1: stores of rows past the chunk's end are dropped
            // by the range check, so none of them needs a branch
            constexpr int kEs = int(sizeof(typename InT::storage));
            const int row_bytes = int(H * kD) * kEs;
            const auto ors = buffer_rsrc(reinterpret_cast<char*>(a.o) + (int64_t(ts) * H + h) * (kD * kEs),
                                         (ns - 1) * row_bytes + kD * kEs);
            Frag fp[2];
  #pragma unroll
            for (int rt = 0; rt < 2; ++rt)
              fp[rt] = Pol::load(sset + L::kSetP, L::kSqPlane, (16 * rt + lj) * L::kSqRow + 8 * lq * E);
  #pragma unroll
            for (int p = 0; p < Pol::kParts; ++p)
  #pragma unroll
              for (int rt = 0; rt < 2; ++rt)
  #pragma unroll
                for (int jb = 0; jb < JB; ++jb) Pol::mma_part(accO[jb][rt], fp[rt], uf[jb], p);
  #pragma unroll
            for (int jb = 0; jb < JB; ++jb)
  #pragma unroll
              for (int rt = 0; rt < 2; ++rt)
  #pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int r = 16 * rt + 4 * lq + e;
                  InT::bstore1(ors, r * row_bytes + (colw + 16 * jb + lj) * kEs, accO[jb][rt][e]);
                }
          }
        }
      if constexpr (MODE != Mode::State) __syncthreads();
      // ============================== phase C ==============================
        {
          // S = Gamma S + Kb^T U, in two halves of four row tiles (one pass of
          // eight in the state build, whose registers allow it)
          const float* s_gamma = reinterpret_cast<const float*>(sset + L::kSetGamma);
          constexpr int kCt = MODE == Mode::State ? 8 : 4;
  #pragma unroll
          for (int half = 0; half < 8 / kCt; ++half) {
            Frag fb[kCt];
  #pragma unroll
            for (int c = 0; c < kCt; ++c) {
              const int ct = kCt * half + c;
              fb[c] = Pol::load(sset + L::kSetKb, L::kKbPlane, (16 * ct + lj) * L::kKbRow + 8 * lq * E);
              const float4 gm = *reinterpret_cast<const float4*>(s_gamma + 16 * ct + 4 * lq);
  #pragma unroll
              for (int jb = 0; jb < JB; ++jb) {
                S[jb][ct][0] *= gm.x; S[jb][ct][1] *= gm.y; S[jb][ct][2] *= gm.z; S[jb][ct][3] *= gm.w;
              }
            }
  #pragma unroll
            for (int p = 0; p < Pol::kParts; ++p)
  #pragma unroll
              for (int c = 0; c < kCt; ++c)
  #pragma unroll
                for (int jb = 0; jb < JB; ++jb) Pol::mma_part(S[jb][kCt * half + c], fb[c], uf[jb], p);
          }
        }
        if constexpr (MODE != Mode::State) {  // fetch chunk i's v (clamped to the last chunk; unconditional so nothing waits on it)
          const int tv = bos + (i < nch ? i : nch - 1) * kC;
          load_state_v<InT, JB>(sv, a, tv, eos - tv < kC ? eos - tv : kC, h, lq, lj, colw);
        }
        if (CKPT && ckpt_on) {  // S is now the state after the sequence's first i * kC tokens
          const int pos = i * kC;
          if (pos % a.ckpt_interval == 0 && pos < eos - bos) {
            // checkpoint rows of this sequence start after those of the earlier
            // ones: a sequence of length L stores floor((L - 1) / interval).
            // Summed here, where it is used, so that nothing stays live across
            // the step loop.
            int ckpt_base = 0;
            for (int n = 0; n < seq; ++n) {
              const int len = a.cu_seqlens[n + 1] - a.cu_seqlens[n];
              ckpt_base += len > 0 ? (len - 1) / a.ckpt_interval : 0;
            }
            const auto rs = buffer_rsrc(a.checkpoints + (int64_t(ckpt_base + pos / a.ckpt_interval - 1) * H + h) * (kD * kD),
                                        kD * kD * 4);
            const int voff = ((4 * lq) * kD + colw + lj) * 4;
  #pragma unroll
            for (int jb = 0; jb < JB; ++jb)
  #pragma unroll
              for (int ct = 0; ct < 8; ++ct)
  #pragma unroll
                for (int e = 0; e < 4; ++e)
                  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[jb][ct][e]), rs,
                                                        voff + ((16 * ct + e) * kD + 16 * jb) * 4, 0, 0);
          }
        }
      if constexpr (MODE == Mode::State) {
        KDA_STAGE_STORE(i, i & 1)
      }
      __syncthreads();
    }
  }
  if constexpr (MODE != Mode::State) if (!is_state) {
    // Prep build: one chunk, this workgroup's slot; fused: every chunk in turn
    const int c_first = MODE == Mode::Prep ? pchunk : 0;
    const int c_end = MODE == Mode::Prep ? pchunk + 1 : nch;
    PrepIn<InT, TPT> pin;
    if (nch > 0) {
      const int tf = bos + c_first * kC;
      load_prep<InT, TPT>(pin, a, tf, eos - tf < kC ? eos - tf : kC, h, tg, c0, ptid, want_o);
    }
    if constexpr (PRO) {
      if (nch > 0) prep_prologue<InT, TPT, NTG>(pin, a, s_nrm, lane, tg, pw, want_o);
      __syncthreads();
    }
    for (int i = c_first; i < c_end; ++i) {
      // this step builds chunk i into operand set i % 2 (the prep build's only set)
      const int tp = bos + i * kC;
      const int np = eos - tp < kC ? eos - tp : kC;
      char* pset = smem + (MODE == Mode::Prep ? 0 : (i & 1)) * L::kSetBytes;
      // K-bar of this chunk: computed with the other operands in phase A, split
      // and stored in phase C (the state waves first read it a step later)
      float kbv[TPT][4];

      // ============================== phase A ==============================
      {
        // decay prefix and rescaled operands of chunk i.  Rows past the chunk end
        // only need g = 0 (the prefix stops) and beta = 0 (their rows and columns
        // of A, T' vanish, so their finite k, q, v never reach a kept result).
        constexpr float kLog2e = 1.4426950408889634f;
        float gq[TPT][4], kq[TPT][4], qv[TPT][4];
  #pragma unroll
        for (int rr = 0; rr < TPT; ++rr) {
          const float gm = (TPT * tg + rr < np) ? kLog2e : 0.0f;  // log2-domain prefix
          InT::unpack4(pin.k[rr], kq[rr]);
          InT::unpack4(pin.q[rr], qv[rr]);
          float4 gr = pin.g[rr];
          if (PRO && a.pro_gate) {
            gr.x = gate_log_decay(gr.x, a.pro_gmin); gr.y = gate_log_decay(gr.y, a.pro_gmin);
            gr.z = gate_log_decay(gr.z, a.pro_gmin); gr.w = gate_log_decay(gr.w, a.pro_gmin);
          }
          gq[rr][0] = gr.x * gm; gq[rr][1] = gr.y * gm;
          gq[rr][2] = gr.z * gm; gq[rr][3] = gr.w * gm;
          if (PRO && a.pro_l2) {
            // the token's sums of squares from the prep waves' partials, in one
            // association for both shapes: 8-group sums (one wave of 4 prep
            // waves, or a pair of waves of 8) added in order
            const float* src = s_nrm + (TPT * tg + rr) * 8 * 2;
            float sk, sq;
            if constexpr (PW == 8) {
              sk = src[0] + src[2];
              sq = src[1] + src[3];
  #pragma unroll
              for (int m = 1; m < 4; ++m) {
                sk += src[4 * m] + src[4 * m + 2];
                sq += src[4 * m + 1] + src[4 * m + 3];
              }
            } else {
              sk = src[0];
              sq = src[1];
  #pragma unroll
              for (int m = 1; m < 4; ++m) {
                sk += src[2 * m];
                sq += src[2 * m + 1];
              }
            }
            const float rk = __builtin_amdgcn_rsqf(sk + a.pro_eps), rq = __builtin_amdgcn_rsqf(sq + a.pro_eps);
  #pragma unroll
            for (int e = 0; e < 4; ++e) {
              kq[rr][e] = kq[rr][e] * rk;
              qv[rr][e] = qv[rr][e] * rq;
            }
          }
        }
        if (ptid < kC) s_beta[ptid] = ptid < np ? pin.beta : 0.0f;
        // Decay prefix over the chunk's 32 tokens in one association for both
        // workgroup shapes, so that a sequence's results do not depend on the
        // launch shape: token pairs (2j, 2j+1) are summed in-thread, the 16 pair
        // sums are scanned by Hillis-Steele steps of 1, 2, 4 and 8 pairs (DPP
        // row shifts; pairs before the chunk contribute 0), and a token's
        // prefix is the exclusive pair prefix plus its own part of its pair.
        // Reference: b at the chunk's row 15 (its middle), so that every
        // rescaling exponent b - b_mid of the chunk lies within the decay of
        // 16 tokens (e^{+-80} at the lower bound g >= -5, inside fp32 range).
        static_assert(TPT == 2 || TPT == 4, "tokens per prep thread");
        // The four channels' scans run side by side (each step for all four,
        // then the eight broadcasts together), so their DPP and broadcast
        // latencies overlap; every value sees the same operations in the same
        // order as a channel-at-a-time scan.
        float bl[TPT][4], gam[4], emid[4];  // log2 cumulative decay relative to b_mid, per token
        float bmid[4], blast[4];
        if constexpr (TPT == 2) {  // one pair per lane, 16 lanes
          float p[4], y[4];
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = gq[0][e] + gq[1][e];
            y[e] = p[e];
          }
  #pragma unroll
          for (int e = 0; e < 4; ++e) y[e] += dpp_shr_in_group<1, NTG>(y[e], tg);
  #pragma unroll
          for (int e = 0; e < 4; ++e) y[e] += dpp_shr_in_group<2, NTG>(y[e], tg);
  #pragma unroll
          for (int e = 0; e < 4; ++e) y[e] += dpp_shr_in_group<4, NTG>(y[e], tg);
  #pragma unroll
          for (int e = 0; e < 4; ++e) y[e] += dpp_shr_in_group<8, NTG>(y[e], tg);
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            bmid[e] = __shfl(y[e], 7, NTG);
            blast[e] = __shfl(y[e], 15, NTG);
          }
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ex = dpp_shr_in_group<1, NTG>(y[e], tg) - bmid[e];
            bl[0][e] = ex + gq[0][e];
            bl[1][e] = ex + p[e];
          }
        } else {  // pairs 2 tg and 2 tg + 1 in this lane, 8 lanes
          float p0[4], p1[4], y0[4], y1[4];
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            p0[e] = gq[0][e] + gq[1][e];
            p1[e] = gq[2][e] + gq[3][e];
          }
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            y0[e] = p0[e] + dpp_shr_in_group<1, NTG>(p1[e], tg);
            y1[e] = p1[e] + p0[e];
          }
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t0 = dpp_shr_in_group<1, NTG>(y0[e], tg), t1 = dpp_shr_in_group<1, NTG>(y1[e], tg);
            y0[e] += t0;
            y1[e] += t1;
          }
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t0 = dpp_shr_in_group<2, NTG>(y0[e], tg), t1 = dpp_shr_in_group<2, NTG>(y1[e], tg);
            y0[e] += t0;
            y1[e] += t1;
          }
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t0 = dpp_shr_in_group<4, NTG>(y0[e], tg), t1 = dpp_shr_in_group<4, NTG>(y1[e], tg);
            y0[e] += t0;
            y1[e] += t1;
          }
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            bmid[e] = __shfl(y1[e], 3, NTG);
            blast[e] = __shfl(y1[e], 7, NTG);
          }
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ex0 = dpp_shr_in_group<1, NTG>(y1[e], tg) - bmid[e], ex1 = y0[e] - bmid[e];
            bl[0][e] = ex0 + gq[0][e];
            bl[1][e] = ex0 + p0[e];
            bl[2][e] = ex1 + gq[2][e];
            bl[3][e] = ex1 + p1[e];
          }
        }
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          gam[e] = __builtin_amdgcn_exp2f(blast[e] - bmid[e]);  // e^{b_last - b_mid}
          emid[e] = __builtin_amdgcn_exp2f(bmid[e]);            // e^{b_mid}
        }
  #pragma unroll
        for (int rr = 0; rr < TPT; ++rr) {
          const int r = TPT * tg + rr;
          float kh[4], kc[4], qh[4];
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float b = bl[rr][e];  // log2 of the cumulative decay, relative to b_mid
            const float eb = __builtin_amdgcn_exp2f(b);
            kh[e] = kq[rr][e] * eb;
            kc[e] = kq[rr][e] * __builtin_amdgcn_exp2f(-b);
            if (want_o) qh[e] = (qv[rr][e] * a.scale) * eb;
            kbv[rr][e] = kc[e] * gam[e];  // k e^{b_last - b} (the reference cancels)
          }
          const int off = r * L::kOpRow + kperm(c0) * E;
          Pol::store4(pset + L::kSetKh, L::kOpPlane, off, kh);
          Pol::store4(smem + L::kKc, L::kOpPlane, off, kc);
          if (want_o) Pol::store4(pset + L::kSetQh, L::kOpPlane, off, qh);
        }
        if (tg == 0) {
          float* g_out = reinterpret_cast<float*>(pset + L::kSetGamma);
          float* m_out = reinterpret_cast<float*>(pset + L::kSetEm);
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            g_out[c0 + e] = gam[e];
            m_out[c0 + e] = emid[e];
          }
        }
        if constexpr (MODE == Mode::Fused) {  // fetch chunk i + 1's inputs (clamped; unconditional so nothing waits on them)
          const int tn = bos + (i + 1 < nch ? i + 1 : nch - 1) * kC;
          load_prep<InT, TPT>(pin, a, tn, eos - tn < kC ? eos - tn : kC, h, tg, c0, ptid, want_o);
        }
      }
      __syncthreads();
      // ============================== phase B ==============================
      {
        if (pw < 2) {
          // diagonal tile A_II (I = pw), then T_II = (I + A_II)^{-1}
          const int I = pw;
          // the rows' beta, read before the products (a read after them waited
          // on the LDS once per row)
          float bet[4];
  #pragma unroll
          for (int e = 0; e < 4; ++e) bet[e] = s_beta[16 * I + 4 * lq + e];
          // two accumulation chains (contraction blocks 0, 1 and 2, 3), summed
          f32x4_t acc2[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  #pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
            Frag fa[2], fb[2];
  #pragma unroll
            for (int c = 0; c < 2; ++c) {
              const int koff = (32 * (2 * c + kp) + 8 * lq) * E;
              fa[c] = Pol::load(pset + L::kSetKh, L::kOpPlane, (16 * I + lj) * L::kOpRow + koff);
              fb[c] = Pol::load(smem + L::kKc, L::kOpPlane, (16 * I + lj) * L::kOpRow + koff);
            }
  #pragma unroll
            for (int p = 0; p < Pol::kParts; ++p)
  #pragma unroll
              for (int c = 0; c < 2; ++c) Pol::mma_part(acc2[c], fa[c], fb[c], p);
          }
          const f32x4_t acc = acc2[0] + acc2[1];
          {  // At[I][s][r] = A[16I+r][16I+s] = beta_r (Kh Kc^T)[r][s] for r > s
            float4 w;
            float* wp = reinterpret_cast<float*>(&w);
  #pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * lq + e;
              wp[e] = (r > lj) ? acc[e] * bet[e] : 0.0f;
            }
            *reinterpret_cast<float4*>(s_at + (I * 16 + lj) * L::kFLd + 4 * lq) = w;
          }
          wave_sync();
          // every lane solves column j = lane % 16 (four copies per wave)
          float x[16];
  #pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = (r == lj) ? 1.0f : 0.0f;
  #pragma unroll
          for (int s = 0; s < 15; ++s) {
            const float* col = s_at + (I * 16 + s) * L::kFLd;  // column s of A_II
            float cv[16];
  #pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const float4 w = *reinterpret_cast<const float4*>(col + 4 * r4);
              cv[4 * r4] = w.x; cv[4 * r4 + 1] = w.y; cv[4 * r4 + 2] = w.z; cv[4 * r4 + 3] = w.w;
            }
  #pragma unroll
            for (int r = s + 1; r < 16; ++r) x[r] = fmaf(-cv[r], x[s], x[r]);
          }
          if (lq == 0) {
  #pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
              *reinterpret_cast<float4*>(s_td + (I * 16 + lj) * L::kFLd + 4 * r4) =
                  make_float4(x[4 * r4], x[4 * r4 + 1], x[4 * r4 + 2], x[4 * r4 + 3]);
          }
        } else if (pw < 6 && (want_o || pw == 2)) {
          // the four remaining 16 x 16 tiles, one per wave (PW = 8) or two (PW = 4);
          // without outputs only the wave holding A_10 has work:
          //   tile 2: A_10 = Kh[16..31] Kc[0..15]^T (beta-scaled rows)
          //   tile 3: P_00 = Qh[0..15] Kc[0..15]^T    tile 4: P_10 = Qh[16..31] Kc[0..15]^T
          //   tile 5: P_11 = Qh[16..31] Kc[16..31]^T, and the zero upper block of P
          constexpr int NT = (PW == 8) ? 1 : 2;
          int tile[NT];
          if constexpr (PW == 8) tile[0] = pw;
          else { tile[0] = 2 * pw - 2; tile[NT - 1] = 2 * pw - 1; }
          f32x4_t acc[NT];
  #pragma unroll
          for (int u = 0; u < NT; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          float bet[4];  // beta of rows 16 + r (A_10), read before the products
  #pragma unroll
          for (int e = 0; e < 4; ++e) bet[e] = s_beta[16 + 4 * lq + e];
  #pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int koff = (32 * ks + 8 * lq) * E;
            Frag fa[NT], fb[NT];
  #pragma unroll
            for (int u = 0; u < NT; ++u) {
              const int arow = (tile[u] == 3) ? 0 : 16;
              const int brow = (tile[u] == 5) ? 16 : 0;
              fa[u] = Pol::load(pset + (tile[u] == 2 ? L::kSetKh : L::kSetQh), L::kOpPlane, (arow + lj) * L::kOpRow + koff);
              fb[u] = Pol::load(smem + L::kKc, L::kOpPlane, (brow + lj) * L::kOpRow + koff);
            }
  #pragma unroll
            for (int p = 0; p < Pol::kParts; ++p)
  #pragma unroll
              for (int u = 0; u < NT; ++u) Pol::mma_part(acc[u], fa[u], fb[u], p);
          }
  #pragma unroll
          for (int u = 0; u < NT; ++u)
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * lq + e;  // row within the 16-row tile
            const int pwt = tile[u];
            const f32x4_t& accu = acc[u];
            if (pwt == 2) {
              // A_10 (beta-scaled rows), natural order [r][s] for a 16-deep operand
              Pol::store1(smem + L::kAop, L::kAopPlane, r * L::kNatRow + lj * E, accu[e] * bet[e]);
            } else if (pwt == 3) {
              Pol::store1(pset + L::kSetP, L::kSqPlane, r * L::kSqRow + kperm(lj) * E, (lj <= r) ? accu[e] : 0.0f);
            } else if (pwt == 4) {
              Pol::store1(pset + L::kSetP, L::kSqPlane, (16 + r) * L::kSqRow + kperm(lj) * E, accu[e]);
            } else {
              Pol::store1(pset + L::kSetP, L::kSqPlane, (16 + r) * L::kSqRow + kperm(16 + lj) * E,
                          (lj <= r) ? accu[e] : 0.0f);
              Pol::store1(pset + L::kSetP, L::kSqPlane, r * L::kSqRow + kperm(16 + lj) * E, 0.0f);  // upper block
            }
          }
        }
      }
      if constexpr (MODE != Mode::State) __syncthreads();
      // ============================== phase C ==============================
      {
        if (pw == 0) {
          // T_10 = -T_11 (A_10 T_00)
          // every LDS read of the step first (T_00, A_10, T_11, beta), then the two products
          const float4 w = *reinterpret_cast<const float4*>(s_td + (0 * 16 + lj) * L::kFLd + 4 * lq);
          const float t00[4] = {w.x, w.y, w.z, w.w};  // rows 4lq.. of column lj of T_00
          const Frag16 fa = Pol::load16(smem + L::kAop, L::kAopPlane, lj * L::kNatRow + 4 * lq * E);
          // T_11 as the A operand: row lj, columns 4lq .. 4lq+3, read from its fp32 columns
          float t11[4];
  #pragma unroll
          for (int e = 0; e < 4; ++e) t11[e] = s_td[(16 + 4 * lq + e) * L::kFLd + lj];
          const float bj = s_beta[lj];
          const Frag16 fb = Pol::make16(t00);
          f32x4_t X = f32x4_t{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int p = 0; p < Pol::kParts16; ++p) Pol::mma16_part(X, fa, fb, p);
          const Frag16 ft = Pol::make16(t11);
          const float xv[4] = {X[0], X[1], X[2], X[3]};
          const Frag16 fx = Pol::make16(xv);
          f32x4_t Y = f32x4_t{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int p = 0; p < Pol::kParts16; ++p) Pol::mma16_part(Y, ft, fx, p);
  #pragma unroll
          for (int e = 0; e < 4; ++e)
            Pol::store1(pset + L::kSetTp, L::kSqPlane, (16 + 4 * lq + e) * L::kSqRow + kperm(lj) * E, -Y[e] * bj);
        } else if (pw <= 2) {
          // diagonal blocks T'_II = T_II diag(beta) (pw 1: I = 0 and the zero upper block; pw 2: I = 1)
          const int I = pw - 1;
          const float4 w = *reinterpret_cast<const float4*>(s_td + (I * 16 + lj) * L::kFLd + 4 * lq);
          const float tv[4] = {w.x, w.y, w.z, w.w};
          const float bj = s_beta[16 * I + lj];
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * lq + e;
            Pol::store1(pset + L::kSetTp, L::kSqPlane, (16 * I + r) * L::kSqRow + kperm(16 * I + lj) * E,
                        (r >= lj) ? tv[e] * bj : 0.0f);
            if (I == 0) Pol::store1(pset + L::kSetTp, L::kSqPlane, r * L::kSqRow + kperm(16 + lj) * E, 0.0f);
          }
        }
        // K-bar^T of this chunk (every prep thread, its own tokens and channels);
        // the prep build writes it straight into the chunk's workspace set
        char* kb_set = pset;
        if constexpr (MODE == Mode::Prep)
          kb_set = a.ws + ((chunk_slot_base(bos, seq) + int64_t(pchunk)) * H + h) * int64_t(L::kGBytes);
        // (in the workspace's layout: unpadded rows)
        constexpr int kKbAt = MODE == Mode::Prep ? L::kGKb : L::kSetKb;
        constexpr int kKbRowB = MODE == Mode::Prep ? L::kGKbRow : L::kKbRow;
        constexpr int kKbPlaneB = MODE == Mode::Prep ? L::kGKbPlane : L::kKbPlane;
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int off = (c0 + e) * kKbRowB + kperm(TPT * tg) * E;
          if constexpr (TPT == 4) {
            const float w4[4] = {kbv[0][e], kbv[1][e], kbv[2][e], kbv[3][e]};
            Pol::store4(kb_set + kKbAt, kKbPlaneB, off, w4);
          } else {
            Pol::store2(kb_set + kKbAt, kKbPlaneB, off, kbv[0][e], kbv[1][e]);
          }
        }
        // prologue: the next chunk's norms (its inputs arrived during this step)
        if constexpr (PRO && MODE == Mode::Fused) {
          prep_prologue<InT, TPT, NTG>(pin, a, s_nrm, lane, tg, pw, want_o);
        }
      }
      __syncthreads();
    }
    if constexpr (MODE == Mode::Prep) {
      // the chunk's operand set, as laid out in LDS, to its workspace slot
      // (all of it but Kb^T, already there), without the rows' LDS padding
      static_assert(L::kSetInLds == L::kSetKb, "the prep build keeps the set up to Kb^T in LDS");
      constexpr int kN16 = L::kGKb / 16;
      const int64_t slot = chunk_slot_base(bos, seq) + pchunk;
      uint4* dst = reinterpret_cast<uint4*>(a.ws + (slot * H + h) * int64_t(L::kGBytes));
      const uint4* src = reinterpret_cast<const uint4*>(smem);
      for (int idx = tid; idx < kN16; idx += 64 * PW) dst[idx] = src[L::lds_piece(idx)];
    } else {
      // step nch: the state waves consume the last chunk
      __syncthreads();
      __syncthreads();
      __syncthreads();
    }
  }

  if constexpr (MODE != Mode::Prep) if (is_state) {
    float* const s_out = is_transition ? a.transition_out : a.final_state;
    if (s_out != nullptr) {
      float* dst = s_out + tile_base + colw + lj;
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[(16 * ct + 4 * lq + e) * kD + 16 * jb] = S[jb][ct][e];
    }
  }
}

template <class Pol, class InT, int SW, int JB, int PW>
PrefillArgs make_args(const PrefillLaunch& p);

// Split path: the prep build over every (chunk slot, head), then the state
// build over (sequence, head, 64-column slice) reading the sets it wrote.
// The state launches of one call: value slices with outputs (WO), and value
// slices without outputs or transition slices (!WO); one launch when the
// call has only one kind.
template <class K>
hipError_t launch_slices(PrefillArgs a, const PrefillLaunch& p, K&& kernel) {
  const int nv = a.n_value_slices;
  auto go = [&](bool wo, int base, int count) {
    a.slice_base = base;
    a.n_launch_slices = count;
    kernel(wo, a, dim3(unsigned(int64_t(p.num_seqs) * p.H * count)));
    return hipGetLastError();
  };
  if (p.o == nullptr) return go(false, 0, a.n_slices);
  const hipError_t e = go(true, 0, nv);
  if (e != hipSuccess || p.transition_out == nullptr) return e;
  return go(false, nv, nv);
}

// The split path's walk: eight state waves of one 16-column tile each, so one
// workgroup holds a (sequence, head)'s 128 columns and stages each chunk's set
// once.  (Four waves of two tiles measured 8.7k cycles per chunk, four of one
// tile 5.8k but two workgroups per head, each staging the whole set.)
constexpr int kSplitJB = 1;
constexpr int kSplitSW = 8;

template <class Pol, class InT>
hipError_t launch_split(const PrefillLaunch& p, hipStream_t stream) {
  PrefillArgs a = make_args<Pol, InT, 4, 1, 8>(p);
  a.ws = static_cast<char*>(p.workspace);
  const int64_t prep_blocks = p.ws_slots * p.H;
  a.n_value_slices = 1;  // the prep build's one "slice" builds the set every slice reads
  a.n_slices = 1;
  a.slice_base = 0;
  a.n_launch_slices = 1;
  a.prep_outputs = (p.o != nullptr || p.ws_keep_output_operands) ? 1 : 0;
  if (p.ws_prepared) {
    // the sets are in the workspace already
  } else if (p.pro)
    hipLaunchKernelGGL((kda_prefill_kernel<Pol, InT, 0, 1, 8, false, true, Mode::Prep, false>),
                       dim3(unsigned(prep_blocks)), dim3(prefill_threads(0, 8)), 0, stream, a);
  else
    hipLaunchKernelGGL((kda_prefill_kernel<Pol, InT, 0, 1, 8, false, false, Mode::Prep, false>),
                       dim3(unsigned(prep_blocks)), dim3(prefill_threads(0, 8)), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.transition_out != nullptr && p.o == nullptr) {
    // states and transitions without outputs (a segmented prefill's pass 1):
    // one 16-wave workgroup per (sequence, head) reads each set once for both
    a.n_value_slices = 1;
    a.n_slices = 1;
    a.slice_base = 0;
    a.n_launch_slices = 1;
    hipLaunchKernelGGL((kda_prefill_kernel<Pol, InT, 16, 1, 0, false, false, Mode::State, false>),
                       dim3(unsigned(int64_t(p.num_seqs) * p.H)), dim3(prefill_threads(16, 0)), 0, stream, a);
    return hipGetLastError();
  }
  a.n_value_slices = kD / (16 * kSplitJB * kSplitSW);
  a.n_slices = a.n_value_slices * (p.transition_out ? 2 : 1);
  return launch_slices(a, p, [&](bool wo, const PrefillArgs& la, dim3 grid) {
    if (wo)
      hipLaunchKernelGGL((kda_prefill_kernel<Pol, InT, kSplitSW, kSplitJB, 0, false, false, Mode::State, true>), grid,
                         dim3(prefill_threads(kSplitSW, 0)), 0, stream, la);
    else
      hipLaunchKernelGGL((kda_prefill_kernel<Pol, InT, kSplitSW, kSplitJB, 0, false, false, Mode::State, false>),
                         grid, dim3(prefill_threads(kSplitSW, 0)), 0, stream, la);
  });
}

template <class Pol, class InT, int SW, int JB, int PW>
PrefillArgs make_args(const PrefillLaunch& p) {
  PrefillArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.beta = p.beta;
  a.cu_seqlens = p.cu_seqlens;
  a.seq_order = p.seq_order;
  a.num_seqs = p.num_seqs;
  a.H = p.H;
  a.n_value_slices = kD / (16 * JB * SW);
  a.n_slices = a.n_value_slices * (p.transition_out ? 2 : 1);
  a.scale = p.scale;
  a.initial_state = p.initial_state;
  a.final_state = p.final_state;
  a.o = p.o;
  a.transition_out = p.transition_out;
  a.checkpoints = p.checkpoints;
  a.ckpt_interval = p.ckpt_interval;
  a.pro_l2 = p.pro && p.pro->l2norm;
  a.pro_eps = p.pro ? p.pro->eps : 0.0f;
  a.pro_gate = p.pro && p.pro->gate;
  a.pro_gmin = p.pro ? p.pro->g_min : 0.0f;
  a.ws = nullptr;
  a.prep_outputs = 0;
  a.slice_base = 0;
  a.n_launch_slices = a.n_slices;
  return a;
}

template <class Pol, class InT, int SW, int JB, int PW, bool CKPT, bool PRO>
void launch_fused(bool wo, const PrefillArgs& a, dim3 grid, hipStream_t stream) {
  if (wo)
    hipLaunchKernelGGL((kda_prefill_kernel<Pol, InT, SW, JB, PW, CKPT, PRO, Mode::Fused, true>), grid,
                       dim3(prefill_threads(SW, PW)), 0, stream, a);
  else
    hipLaunchKernelGGL((kda_prefill_kernel<Pol, InT, SW, JB, PW, CKPT, PRO, Mode::Fused, false>), grid,
                       dim3(prefill_threads(SW, PW)), 0, stream, a);
}

template <class Pol, class InT, int SW, int JB, int PW>
hipError_t launch_cfg(const PrefillLaunch& p, hipStream_t stream) {
  PrefillArgs a = make_args<Pol, InT, SW, JB, PW>(p);
  if (p.checkpoints && p.pro) return hipErrorNotSupported;
  if constexpr (SW == 4 && JB == 2) {
    if (p.transition_out != nullptr && p.o == nullptr && p.checkpoints == nullptr && p.pro == nullptr) {
      // states and transitions without outputs (a segmented prefill's pass 1) on
      // a grid that fills the device: one workgroup per (sequence, head), its
      // prep waves preparing each chunk once for the state and the transition
      a.n_value_slices = 1;
      a.n_slices = 1;
      a.slice_base = 0;
      a.n_launch_slices = 1;
      hipLaunchKernelGGL((kda_prefill_kernel<Pol, InT, 8, 2, PW, false, false, Mode::Fused, false>),
                         dim3(unsigned(int64_t(p.num_seqs) * p.H)), dim3(prefill_threads(8, PW)), 0, stream, a);
      return hipGetLastError();
    }
  }
  return launch_slices(a, p, [&](bool wo, const PrefillArgs& la, dim3 grid) {
    if (p.checkpoints) launch_fused<Pol, InT, SW, JB, PW, true, false>(wo, la, grid, stream);
    else if (p.pro) launch_fused<Pol, InT, SW, JB, PW, false, true>(wo, la, grid, stream);
    else launch_fused<Pol, InT, SW, JB, PW, false, false>(wo, la, grid, stream);
  });
}

}  // namespace

// The split path's walk runs one workgroup per (sequence, head), two when a call asks for both
// outputs and transitions (value and transition slices launch separately); it applies while that
// grid leaves compute units idle.
bool prefill_split_applies(int64_t num_seqs, int64_t H, bool transitions, bool outputs) {
  return num_seqs * H * (transitions && outputs ? 2 : 1) < device_cu_count();
}

size_t prefill_workspace_bytes(int64_t num_seqs, int64_t t_end, int64_t H, bool bf16, bool transitions,
                               bool outputs) {
  if (num_seqs <= 0 || !prefill_split_applies(num_seqs, H, transitions, outputs)) return 0;
  const int64_t slots = (t_end >> 5) + num_seqs + 1;
  const int64_t set = bf16 ? Lds<PolBF16x3>::kGBytes : Lds<PolF32>::kGBytes;
  return size_t(slots * H * set);
}

int64_t prefill_workspace_slots(int64_t num_seqs, int64_t t_end) { return (t_end >> 5) + num_seqs + 1; }

hipError_t launch_prefill(const PrefillLaunch& p, bool bf16, hipStream_t stream) {
  // Large grids (more (sequence, head) units than half the CUs): 128 value
  // columns per workgroup (4 state waves x 32 columns, 4 prep waves), so each
  // chunk is prepared once per head.  Small grids: 64 value columns per
  // workgroup (4 state waves x 16 columns) and 8 prep waves, which shortens
  // the per-chunk critical path at the cost of preparing each chunk twice
  // (two workgroups per unit: past half the CUs they would need a second
  // round, and one round of the wide shape is faster: segmented 4096 x 12 on
  // the single-kernel passes, 256-token segments, 0.162 -> 0.138 ms);
  // with a workspace, small grids take the split path instead: every chunk is
  // prepared at once by a chunk-parallel launch, and the walk over the chunks
  // runs the state waves alone.
  const int64_t units = int64_t(p.num_seqs) * p.H * (p.transition_out ? 2 : 1);
  const bool wide = 2 * units > device_cu_count();
  if (p.workspace != nullptr && p.checkpoints == nullptr &&
      prefill_split_applies(p.num_seqs, p.H, p.transition_out != nullptr, p.o != nullptr))
    return bf16 ? launch_split<PolBF16x3, BF16>(p, stream) : launch_split<PolF32, F32>(p, stream);
  if (bf16)
    return wide ? launch_cfg<PolBF16x3, BF16, 4, 2, 4>(p, stream) : launch_cfg<PolBF16x3, BF16, 4, 1, 8>(p, stream);
  return wide ? launch_cfg<PolF32, F32, 4, 2, 4>(p, stream) : launch_cfg<PolF32, F32, 4, 1, 8>(p, stream);
}

}  // namespace kda
