// Batch-invariant row contract: one per-token computation for prefill and decode.
//
// The contract (the "Kimi K3.1 Pro" inference / zero-mismatch article,
// section 6.1 on KDA) replaces the running state by the state S_e at the
// entry of the open 16-token chunk plus that chunk's rows so far.  A token at
// position r of the chunk is computed from S_e and the earlier rows only:
//
//   b_r = b_{r-1} + g_r                       (cumulative log-decay, b_{-1} = 0)
//   a_r = S_e^T (k_r e^{b_r}),  w_r = S_e^T (q'_r e^{b_r})          (q' = scale q)
//   G_k[r,s] = sum_c k_rc k_sc e^{b_rc - b_sc},  G_q[r,s] = sum_c q'_rc k_sc e^{b_rc - b_sc}
//   u_r = beta_r ((v_r - sum_{s<r} G_k[r,s] u_s) - a_r)
//   o_r = (sum_{s<=r} G_q[r,s] u_s) + w_r
//
// and the 16th row closes the chunk: S_e <- Diag(e^{b_15}) S_e +
// sum_s (k_s e^{b_15 - b_s}) u_s^T.  This is the UT/WY chunk form of the
// update in "Kimi K3：架构与 SGLang Day-0 Support" ("attention 机制详解：KDA"),
// restated per row.
//
// Every fp32 result is produced by one fixed sequence of operations that does
// not depend on how many rows a launch takes at once: the decode (one row per
// call), the prefill (up to 16 rows of a chunk at once), the verify (a
// request's drafts, pools untouched) and the commit (its accepted prefix) run
// the same kernel body; each reduction has one association (a sequential
// fused multiply-add chain over 16 channels, then a fixed tree over the 8
// channel groups: ((p0+p4)+(p2+p6))+((p1+p5)+(p3+p7)) for the S_e products,
// ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)) for the Gram entries); the sums over
// earlier rows run in row order, with a_r and w_r added last, so the
// association depends on (r, s) only; and the file is built without
// floating-point contraction.  A token's output, the rows and the chunk-entry
// state are therefore bit-identical whichever call and batch computed them.
//
// Layout per (slot, head): S_e fp32 [128 key][128 value]; rows fp32 [16][3][128]
// (k_s, b_s, u_s of the open chunk); position int32 (rows held, 0..15).
// A workgroup (4 waves) owns one (sequence, head).  Wave w holds value columns
// 32w .. 32w+31 of S_e in registers: lane (m = lane >> 3, jq = lane & 7) holds
// key rows 16m .. 16m+15 of columns 32w + 4jq .. +3, so the 8 channel groups of
// every S_e^T x product meet inside the wave (lane bits 5, 4, 3, in that order).
// A prefill of few (sequence, head) units splits each over two or four
// workgroups (lane: two or one columns, same channel groups and tree; see SPLITW).
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kChunk = 16;
constexpr int kThreads = 256;
constexpr int kRowFloats = 3 * kD;  // k, b, u
constexpr int kRS = kD + 4;         // LDS row stride of the open rows' k and b: rows start 4 banks apart
constexpr float kLog2e = 1.4426950408889634f;

// e^x as 2^(x log2 e) on the hardware exponential: one rounding of the
// product, then v_exp_f32 (about 1 ulp).  Every path of the contract uses it.
__device__ __forceinline__ float exp_c(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Lane exchanges, all on the VALU (no LDS round trip).  swap32 / swap16
// exchange, between two registers, the upper 32 lanes of the first with the
// lower 32 lanes of the second (v_permlane32_swap), or the odd 16-lane rows of
// the first with the even rows of the second (v_permlane16_swap); dpp<CTRL>
// reads another lane through a DPP move: 0x128 lane l ^ 8 within a 16-lane row
// (row rotate by 8), 0x141 lane 7 - l within each 8 lanes (half-row mirror),
// 0xB1 lane l ^ 1 and 0x4E lane l ^ 2 (quad permutes).
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
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

struct ContractArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* cu;     // prefill: [num_seqs + 1] token offsets; null: gamma tokens per sequence (tokens n*gamma ...)
  const int32_t* slots;  // [num_seqs] or null (identity)
  float* S;              // [P, H, 128, 128]
  float* rows;           // [P, H, 16, 3, 128]
  int32_t* pos;          // [P, H]
  void* o;               // [tokens, H, 128] or null
  int num_seqs;
  int H;
  float scale;
  int gamma;              // tokens per sequence when cu is null (1: decode)
  const int32_t* counts;  // with cu null: [num_seqs] tokens to take (clamped to 0..gamma), or null (all gamma)
  int read_only;          // nonzero: outputs only, the pools are not written (verify)
  float* stash;           // verify, or null: per (sequence, head) the rows of its gamma tokens
                          // [gamma][3][128] and the entry state after a chunk closes [128][128]
  float* prep;            // split prefill, or null: prepared sets of the full chunks, [prep_windows][H][kPrepFloats]
  int prep_windows;       // 16-token windows of the packed tokens covered by prep
};

// Rows of the batch being computed (at most MR) next to the open chunk's rows.
template <int MR>
struct Lds {
  float rk[kChunk + 1][kRS];  // k_s of the open chunk (k_s e^{b_15 - b_s} while closing); last row: discard
  float rb[kChunk + 1][kRS];  // b_s; last row: discard
  float ru[kChunk][kD];  // u_s
  float sq[MR][kD];      // scale * q_r
  float kh[MR][kD];      // k_r e^{b_r}
  float qh[MR][kD];      // scale * q_r e^{b_r}
  float vv[MR][kD];      // v_r
  float aa[MR][kD];      // S_e^T k_hat
  float ww[MR][kD];      // S_e^T q_hat
  float gk[kChunk][MR];  // G_k[r, s] at [s][r - r0]
  float gq[kChunk][MR];  // G_q[r, s] at [s][r - r0]
  float bt[MR < 4 ? 4 : MR];  // beta_r
  float gam[kD];         // e^{b_15} while closing
};

// The chunk close on this lane's 16 x 4 block: S <- e^{b_last} S + sum_s kbar_s u_s^T
// over rows s = 0 .. nrows-1 in order (kbar already in rk, e^{b_last} in gam).
template <int CW>
__device__ __forceinline__ void close_block(float (&S)[16][CW], const float (*rk)[kRS], const float (*ru)[kD],
                                            const float* gam, int nrows, int c0, int j0) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float e = gam[c0 + i];
#pragma unroll
    for (int x = 0; x < CW; ++x) S[i][x] = e * S[i][x];
  }
  // row s's operands are read while row s - 1's products are formed
  auto ld_u = [&](int s) {
    if constexpr (CW == 4) return *reinterpret_cast<const float4*>(&ru[s][j0]);
    else if constexpr (CW == 2) return make_float4(ru[s][j0], ru[s][j0 + 1], 0.f, 0.f);
    else return make_float4(ru[s][j0], 0.f, 0.f, 0.f);
  };
  float4 un = ld_u(0);
  float4 kn[4];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) kn[i4] = *reinterpret_cast<const float4*>(&rk[0][c0 + 4 * i4]);
  for (int s = 0; s < nrows; ++s) {
    const float u[4] = {un.x, un.y, un.z, un.w};
    float kb[16];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      kb[4 * i4] = kn[i4].x; kb[4 * i4 + 1] = kn[i4].y; kb[4 * i4 + 2] = kn[i4].z; kb[4 * i4 + 3] = kn[i4].w;
    }
    if (s + 1 < nrows) {
      un = ld_u(s + 1);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) kn[i4] = *reinterpret_cast<const float4*>(&rk[s + 1][c0 + 4 * i4]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int x = 0; x < CW; ++x) S[i][x] = __builtin_fmaf(kb[i], u[x], S[i][x]);
  }
}

// Channel c's close factors: kbar_s = k_s e^{b_last - b_s} in place for rows 0 .. nrows-1,
// and gam = e^{b_last}.
__device__ __forceinline__ void close_factors(float (*rk)[kRS], const float (*rb)[kRS], float* gam, int nrows, int c) {
  const float bl = rb[nrows - 1][c];
  for (int s = 0; s < nrows; ++s) rk[s][c] = rk[s][c] * exp_c(bl - rb[s][c]);
  gam[c] = exp_c(bl);
}

// MR consecutive floats from LDS (16-byte aligned when MR >= 4), as wide reads.
template <int MR>
__device__ __forceinline__ void load_row(float (&dst)[MR], const float* src) {
  if constexpr (MR % 4 == 0) {
#pragma unroll
    for (int q = 0; q < MR / 4; ++q) {
      const float4 t = reinterpret_cast<const float4*>(src)[q];
      dst[4 * q] = t.x; dst[4 * q + 1] = t.y; dst[4 * q + 2] = t.z; dst[4 * q + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < MR; ++q) dst[q] = src[q];
  }
}

// One batch's inputs as this thread holds them: channel threads (tid < 128,
// channel c = tid) hold k, q and g of channel c; value threads (tid >= 128,
// column j = tid - 128) hold v of column j and beta.
template <typename InT, int MR>
struct BatchIn {
  typename InT::raw1 x0[MR];  // k (channel) / v (value)
  typename InT::raw1 x1[MR];  // q (channel)
  float f[MR];                // g (channel) / beta (value)
};

template <typename InT, int MR>
__device__ __forceinline__ void load_batch(BatchIn<InT, MR>& in, const ContractArgs& a, int h, int t0, int nr,
                                           int tid) {
  // Without branches (a branch around each load made the compiler wait for
  // every outstanding memory operation where the paths join): rows past nr
  // read row nr - 1 again, and value threads read v in place of q (unused).
  const int c = tid & (kD - 1);
  const bool ch = tid < kD;
  const int64_t head = int64_t(h) * kD + c;
  const void* p0 = ch ? a.k : a.v;
  const void* p1 = ch ? a.q : a.v;
  const float* pf = ch ? a.g + head : a.beta + h;
  const int64_t fs = ch ? int64_t(a.H) * kD : int64_t(a.H);
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    const int64_t t = t0 + (i < nr ? i : nr - 1);
    in.x0[i] = InT::load1raw(p0, t * a.H * kD + head);
    in.x1[i] = InT::load1raw(p1, t * a.H * kD + head);
    in.f[i] = pf[t * fs];
  }
}

// ---- B: cumulative decay in row order, rescaled key and query (channel
// threads), values and beta (value threads), for rows r0 .. r0 + nr - 1 of the
// open chunk.  Every row of the pass is formed, without branches: rows past
// nr are formed from stale inputs, their open-chunk row goes to the discard
// row, and nothing reads them as results.  stash_rows (verify): each row's key
// and decay, for a later commit.
template <typename InT, int MR, bool STASH>
__device__ __forceinline__ void form_rows(Lds<MR>& L, const BatchIn<InT, MR>& in, float scale, int r0, int nr,
                                          int tid, float* stash_rows) {
  if (tid < kD) {
    const int c = tid;
    float b = (r0 > 0) ? L.rb[r0 - 1][c] : 0.0f;
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      const float kk = InT::unpack1(in.x0[i]);
      const float sq = scale * InT::unpack1(in.x1[i]);
      b = b + in.f[i];
      const float e = exp_c(b);
      const int rr = (i < nr) ? r0 + i : kChunk;
      L.rk[rr][c] = kk;
      L.rb[rr][c] = b;
      if constexpr (STASH) {
        if (i < nr) {
          float* row = stash_rows + int64_t(i) * kRowFloats;
          row[c] = kk;
          row[kD + c] = b;
        }
      }
      L.sq[i][c] = sq;
      L.kh[i][c] = kk * e;
      L.qh[i][c] = sq * e;
    }
  } else {
    const int j = tid - kD;
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      L.vv[i][j] = InT::unpack1(in.x0[i]);
      if (j == 0) L.bt[i] = in.f[i];
    }
  }
}

// ---- C2: Gram entries G_k[r, s], G_q[r, s] for s <= r (rows r of the pass),
// 8 lanes per entry
template <int MR>
__device__ __forceinline__ void gram_entries(Lds<MR>& L, int r0, int nr, int tid, int lane) {
  const int ntask = nr * (r0 + 1) + nr * (nr - 1) / 2;  // sum over i of (r0 + i + 1)
  const int cm = 16 * (lane & 7);
  for (int base = 0; base < ntask; base += kThreads / 8) {
    const int task = base + (tid >> 3);
    // task -> (batch row i, earlier row s): row i owns r0 + i + 1 entries from
    // first(i) = i (r0 + 1) + i (i - 1) / 2, so i is the floor of the root of
    // first(i) = task, corrected by one either way for the rounding of the root
    int i = 0;
    if constexpr (MR > 1) {
      const int a2 = 2 * r0 + 1;
      i = int((__builtin_amdgcn_sqrtf(float(a2 * a2 + 8 * task)) - float(a2)) * 0.5f);
      if ((i + 1) * (r0 + 1) + (i + 1) * i / 2 <= task) ++i;
      if (i * (r0 + 1) + i * (i - 1) / 2 > task) --i;
      i = min(i, nr - 1);
    }
    const bool valid = task < ntask;
    const int s = valid ? task - (i * (r0 + 1) + i * (i - 1) / 2) : 0;
    const int r = r0 + i;
    float pk = 0.f, pq = 0.f;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const float4 br = *reinterpret_cast<const float4*>(&L.rb[r][cm + 4 * c4]);
      const float4 bs = *reinterpret_cast<const float4*>(&L.rb[s][cm + 4 * c4]);
      const float4 kr = *reinterpret_cast<const float4*>(&L.rk[r][cm + 4 * c4]);
      const float4 ks = *reinterpret_cast<const float4*>(&L.rk[s][cm + 4 * c4]);
      const float4 qr = *reinterpret_cast<const float4*>(&L.sq[i][cm + 4 * c4]);
      const float brv[4] = {br.x, br.y, br.z, br.w}, bsv[4] = {bs.x, bs.y, bs.z, bs.w};
      const float krv[4] = {kr.x, kr.y, kr.z, kr.w}, ksv[4] = {ks.x, ks.y, ks.z, ks.w};
      const float qrv[4] = {qr.x, qr.y, qr.z, qr.w};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const float t = ksv[cc] * exp_c(brv[cc] - bsv[cc]);
        pk = __builtin_fmaf(krv[cc], t, pk);
        pq = __builtin_fmaf(qrv[cc], t, pq);
      }
    }
    pk = pk + dpp<0xB1>(pk);  // groups g, g^1
    pq = pq + dpp<0xB1>(pq);
    pk = pk + dpp<0x4E>(pk);  // pairs {0,1} + {2,3} within a quad
    pq = pq + dpp<0x4E>(pq);
    pk = pk + dpp<0x141>(pk);  // quads {0,1} of each 8 lanes: each lane adds its mirror lane's quad sum
    pq = pq + dpp<0x141>(pq);
    if (valid && (lane & 7) == 0) {
      L.gk[s][i] = pk;
      L.gq[s][i] = pq;
    }
  }
}

// A full chunk's prepared set (a split prefill with a workspace): everything
// of a chunk that does not depend on the state, formed chunk-parallel by
// kda_contract_prep_kernel with the functions the walk uses, so its values are
// those the walk would form: [16][128] k e^{b} (kh), scale q e^{b} (qh), the
// close factors k e^{b_15 - b} (kb) and v; the Gram entries [16][16] each
// (G_k, G_q, as in Lds); beta [16]; e^{b_15} [128].
constexpr int kPrepKh = 0, kPrepQh = 16 * kD, kPrepKb = 32 * kD, kPrepV = 48 * kD, kPrepGk = 64 * kD,
              kPrepGq = kPrepGk + kChunk * kChunk, kPrepBt = kPrepGq + kChunk * kChunk, kPrepGam = kPrepBt + kChunk;
constexpr int kPrepFloats = kPrepGam + kD;  // 8,848 floats (35,392 bytes) per chunk and head
static_assert(kPrepFloats % 4 == 0, "16-byte pieces");

// A thread's part of a prepared set on its way from the workspace to LDS:
// pieces tid and tid + 256 of each of the four [16][128] tables, and at most
// one piece of the small ones.  (Fetching the next pass's set a pass ahead
// into these registers at the start of the pass before measured slower than
// at the pass's own start; fetching it just before the close, so that it is in
// flight during the close and the loop's last barrier, saves ~2 %.)
struct PrepPieces {
  float4 t[4][2];
  float4 gk, gq;  // Gram pieces (tid < 64), or beta / e^{b_15} in gk
};

__device__ __forceinline__ void fetch_prepared(PrepPieces& x, const float* set, int tid) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int e = tid + kThreads * m;
    x.t[0][m] = ld_f4(set + kPrepKh + 4 * e);
    x.t[1][m] = ld_f4(set + kPrepQh + 4 * e);
    x.t[2][m] = ld_f4(set + kPrepKb + 4 * e);
    x.t[3][m] = ld_f4(set + kPrepV + 4 * e);
  }
  constexpr int kSq = kChunk * kChunk / 4;  // 64 pieces per Gram table
  if (tid < kSq) {
    x.gk = ld_f4(set + kPrepGk + 4 * tid);
    x.gq = ld_f4(set + kPrepGq + 4 * tid);
  } else if (tid < kSq + kChunk / 4 + kD / 4) {
    x.gk = ld_f4(set + kPrepBt + 4 * (tid - kSq));  // beta and e^{b_15} are contiguous
  }
}

__device__ __forceinline__ void store_prepared(Lds<kChunk>& L, const PrepPieces& x, int tid) {
  constexpr int kRowVec = kD / 4;
  static_assert(16 * kRowVec == 2 * kThreads, "two pieces of each table per thread");
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int e = tid + kThreads * m;
    const int r = e / kRowVec, f = 4 * (e % kRowVec);
    *reinterpret_cast<float4*>(&L.kh[r][f]) = x.t[0][m];
    *reinterpret_cast<float4*>(&L.qh[r][f]) = x.t[1][m];
    *reinterpret_cast<float4*>(&L.rk[r][f]) = x.t[2][m];
    *reinterpret_cast<float4*>(&L.vv[r][f]) = x.t[3][m];
  }
  constexpr int kSq = kChunk * kChunk / 4;
  if (tid < kSq) {
    const int s = tid / (kChunk / 4), f = 4 * (tid % (kChunk / 4));
    *reinterpret_cast<float4*>(&L.gk[s][f]) = x.gk;
    *reinterpret_cast<float4*>(&L.gq[s][f]) = x.gq;
  } else if (tid < kSq + kChunk / 4) {
    *reinterpret_cast<float4*>(&L.bt[4 * (tid - kSq)]) = x.gk;
  } else if (tid < kSq + kChunk / 4 + kD / 4) {
    *reinterpret_cast<float4*>(&L.gam[4 * (tid - kSq - kChunk / 4)]) = x.gk;
  }
}

// SPLITW > 1 (prefill of small grids): SPLITW workgroups per (sequence, head),
// one per 128 / SPLITW value columns; a lane holds CW = 4 / SPLITW columns of
// its 16 key rows instead of 4, so the S_e products and the close cost CW / 4
// per lane, with the same chains and the same tree.  The Gram entries, the decay and the
// substitution are formed in each workgroup alike.  The workgroups write only
// what they own (S_e columns, the u columns of the open rows, outputs); the
// shared keys, decays and position are written by kda_contract_rows_kernel,
// launched after, so that no write can overtake a sibling's read.
template <typename InT, int MR, bool STASH, int SPLITW = 1>
__global__ __launch_bounds__(kThreads, MR == 1 ? 3 : (SPLITW > 1 ? 1 : 2)) void kda_contract_kernel(ContractArgs a) {
  static_assert(SPLITW == 1 || (MR == kChunk && !STASH), "the split serves the prefill");
  static_assert(SPLITW == 1 || SPLITW == 2 || SPLITW == 4, "split in 2 or 4");
  constexpr bool SPLIT = SPLITW > 1;
  constexpr int CW = 4 / SPLITW;          // value columns per lane
  constexpr int kSlices = SPLITW;         // workgroups per (sequence, head)
  constexpr int kSliceCols = kD / SPLITW;  // value columns per workgroup
  __shared__ __align__(16) Lds<MR> L;
  const int slice = blockIdx.x % kSlices;
  const int n = (blockIdx.x / kSlices) / a.H;
  const int h = (blockIdx.x / kSlices) % a.H;
  if (n >= a.num_seqs) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // value threads: tid >= kD; with a split the first kSliceCols of them, for this slice's columns
  const bool value_thread = tid >= kD && tid - kD < kSliceCols;
  const int jv = kSliceCols * slice + (tid - kD);  // value column of a value thread

  int tok0, count;
  if (a.cu != nullptr) {
    tok0 = a.cu[n];
    count = a.cu[n + 1] - tok0;
  } else {
    tok0 = n * a.gamma;
    count = a.counts ? min(max(a.counts[n], 0), a.gamma) : a.gamma;
  }
  if (count <= 0) return;
  const int64_t unit = int64_t(a.slots ? a.slots[n] : n) * a.H + h;
  float* Sp = a.S + unit * kD * kD;
  float* Rp = a.rows + unit * kChunk * kRowFloats;
  // stash of this (sequence, head): indexed by the sequence, not the slot
  const int64_t unit_stash = STASH ? (int64_t(n) * a.H + h) * (int64_t(a.gamma) * kRowFloats + kD * kD) : 0;
  int p = a.pos[unit] & (kChunk - 1);
  const int p_first = p;
  const int c0 = 16 * (lane >> 3);
  const int j0 = kSliceCols * slice + (kSliceCols / 4) * wave + CW * (lane & 7);

  // Loads in the order they are needed: the batch inputs and the open rows
  // first, S_e last, so that everything except the S_e products runs while
  // S_e streams in (loads complete in issue order).
  BatchIn<InT, MR> in{};  // rows past a short batch are read but unused: keep them defined
  int nr = min(min(MR, kChunk - p), count);
  load_batch<InT, MR>(in, a, h, tok0, nr, tid);
  constexpr int kRowVecs = kRowFloats / 4;
  float S[16][CW];
  if constexpr (MR <= 8) {
    // decode and draft blocks: the open rows are issued before S_e and held in registers
    constexpr int kRowIters = ((kChunk - 1) * kRowVecs + kThreads - 1) / kThreads;
    float4 rv[kRowIters];
#pragma unroll
    for (int t = 0; t < kRowIters; ++t) {
      const int e = tid + t * kThreads;
      if (e < p * kRowVecs) rv[t] = ld_f4(Rp + 4 * e);
    }
    __builtin_amdgcn_sched_barrier(0);
    // this lane's block of S_e: key rows c0 .. c0+15, value columns j0 .. j0+3
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 s4 = ld_f4(Sp + (c0 + i) * kD + j0);
      S[i][0] = s4.x; S[i][1] = s4.y; S[i][2] = s4.z; S[i][3] = s4.w;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kRowIters; ++t) {
      const int e = tid + t * kThreads;
      if (e < p * kRowVecs) {
        const int s = e / kRowVecs, f = 4 * (e % kRowVecs);
        float* dst = (f < kD) ? &L.rk[s][f] : (f < 2 * kD) ? &L.rb[s][f - kD] : &L.ru[s][f - 2 * kD];
        *reinterpret_cast<float4*>(dst) = rv[t];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (CW == 4) {
        const float4 s4 = ld_f4(Sp + (c0 + i) * kD + j0);
        S[i][0] = s4.x; S[i][1] = s4.y; S[i][2] = s4.z; S[i][3] = s4.w;
      } else {
#pragma unroll
        for (int x = 0; x < CW; ++x) S[i][x] = Sp[(c0 + i) * kD + j0 + x];
      }
    }
    for (int e = tid; e < p * kRowVecs; e += kThreads) {
      const int s = e / kRowVecs, f = 4 * (e % kRowVecs);
      const float4 x = ld_f4(Rp + 4 * e);
      float* dst = (f < kD) ? &L.rk[s][f] : (f < 2 * kD) ? &L.rb[s][f - kD] : &L.ru[s][f - 2 * kD];
      *reinterpret_cast<float4*>(dst) = x;
    }
  }
  if (p > 0) __syncthreads();

  bool closed = false;
  int done = 0;
  PrepPieces pre;  // split build: the next prepared pass's set, fetched before this pass's close
  bool have_pre = false;
  while (true) {
    const int r0 = p;
    const int t0 = tok0 + done;
    const bool closes = (r0 + nr == kChunk);
    // a split prefill's full chunk: its rows, Gram entries and close factors
    // were prepared by kda_contract_prep_kernel with the same functions
    bool prepared = false;
    if constexpr (SPLIT) {
      prepared = a.prep != nullptr && r0 == 0 && nr == kChunk && t0 / kChunk < a.prep_windows;
      if (prepared) {
        if (!have_pre) fetch_prepared(pre, a.prep + (int64_t(t0 / kChunk) * a.H + h) * kPrepFloats, tid);
        store_prepared(L, pre, tid);
        have_pre = false;
      } else {
        form_rows<InT, MR, false>(L, in, a.scale, r0, nr, tid, nullptr);
      }
    } else {
      form_rows<InT, MR, STASH>(L, in, a.scale, r0, nr, tid,
                                STASH ? a.stash + unit_stash + int64_t(done) * kRowFloats : nullptr);
    }
    __syncthreads();
    const int nr_next = min(MR, count - done - nr);  // after a close the next batch starts a chunk
    // split build (one workgroup per CU, registers to spare): the next batch's
    // inputs are issued as soon as this batch's are in LDS, a whole pass ahead
    if constexpr (SPLIT) {
      // (a prepared next pass reads its set instead: it starts a chunk after
      // this pass closes one)
      const int t_next = t0 + nr;
      const bool next_prepared = a.prep != nullptr && closes && nr_next == kChunk && t_next / kChunk < a.prep_windows;
      if (nr_next > 0 && !next_prepared) load_batch<InT, MR>(in, a, h, t_next, nr_next, tid);
    }
    // ---- C2: Gram entries (not for a prepared pass)
    if (!prepared) gram_entries<MR>(L, r0, nr, tid, lane);
    __syncthreads();
    // ---- D1: the sums over the open chunk's earlier rows (value threads), in
    // row order; u_r = beta_r ((v_r - sum_{s<r} G_k[r,s] u_s) - a_r) and
    // o_r = (sum_{s<=r} G_q[r,s] u_s) + w_r, each sum over s in ascending
    // order, so that the association depends on (r, s) only.  Partials wait
    // in vv (residuals) and sq (outputs), which are free by now.  The channel
    // threads form the close factors.
    if (value_thread) {
      const int j = jv;
      // all MR rows, also those past nr (unused, never stored as results): no
      // per-row branches in the loop
      float acc[MR], out[MR];
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        acc[i] = L.vv[i][j];
        out[i] = 0.f;
      }
#pragma unroll 2
      for (int s = 0; s < r0; ++s) {
        const float u = L.ru[s][j];
        float gk[MR], gq[MR];
        load_row<MR>(gk, L.gk[s]);
        load_row<MR>(gq, L.gq[s]);
#pragma unroll
        for (int i = 0; i < MR; ++i) {
          acc[i] = __builtin_fmaf(-gk[i], u, acc[i]);
          out[i] = __builtin_fmaf(gq[i], u, out[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        L.vv[i][j] = acc[i];
        L.sq[i][j] = out[i];
      }
    } else if (tid < kD && closes && !prepared) {
      close_factors(L.rk, L.rb, L.gam, kChunk, tid);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- C1: a = S_e^T k_hat and w = S_e^T q_hat for every batch row (wave-local);
    // the split build forms four rows per step, interleaved (rows past nr of the
    // last step are formed from stale operands into unused slots of aa and ww)
    constexpr int RB = (SPLIT && MR % 4 == 0) ? 4 : 1;
    for (int i0 = 0; i0 < nr; i0 += RB)
#pragma unroll
    for (int ii = 0; ii < RB; ++ii) {
      const int i = i0 + ii;
      float pa[CW], pw[CW];
#pragma unroll
      for (int x = 0; x < CW; ++x) pa[x] = pw[x] = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const float4 k4 = *reinterpret_cast<const float4*>(&L.kh[i][c0 + 4 * c4]);
        const float4 q4 = *reinterpret_cast<const float4*>(&L.qh[i][c0 + 4 * c4]);
        const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
        const float qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
          for (int x = 0; x < CW; ++x) {
            pa[x] = __builtin_fmaf(S[4 * c4 + cc][x], kv[cc], pa[x]);
            pw[x] = __builtin_fmaf(S[4 * c4 + cc][x], qv[cc], pw[x]);
          }
      }
      // tree over the 8 channel groups, reduce-scattered: level 1 pairs m, m^4
      // (lane bit 5) and splits a / w; level 2 pairs m, m^2 (bit 4) and splits
      // the columns in halves; level 3 pairs m, m^1 (bit 3).
      const bool b3 = lane & 8, b4 = lane & 16, b5 = lane & 32;
      if constexpr (CW == 4) {
#pragma unroll
        for (int x = 0; x < 4; ++x) swap32(pa[x], pw[x]);
        float l1[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) l1[x] = pa[x] + pw[x];  // bit 5 = 0: a, 1: w
        swap16(l1[0], l1[2]);
        swap16(l1[1], l1[3]);
        const float l2a = l1[0] + l1[2], l2b = l1[1] + l1[3];  // bit 4 = 0: columns 0, 1; 1: 2, 3
        const float mine = b3 ? l2b : l2a;
        const float other = b3 ? l2a : l2b;
        const float fin = mine + dpp<0x128>(other);
        const int col = j0 + (b4 ? 2 : 0) + (b3 ? 1 : 0);
        (b5 ? L.ww : L.aa)[i][col] = fin;
      } else if constexpr (CW == 2) {
        // two columns: level 2 splits them (bit 4 = 0: column 0, 1: column 1),
        // level 3 is a butterfly; the same pairings in the same order
        swap32(pa[0], pw[0]);
        swap32(pa[1], pw[1]);
        float l1[2] = {pa[0] + pw[0], pa[1] + pw[1]};  // bit 5 = 0: a, 1: w
        swap16(l1[0], l1[1]);
        float v = l1[0] + l1[1];
        v = v + dpp<0x128>(v);
        if (!b3) (b5 ? L.ww : L.aa)[i][j0 + (b4 ? 1 : 0)] = v;
      } else {
        // one column: the same pairings in the same order (own + partner, or
        // partner + own, which is the same sum), each level a butterfly
        swap32(pa[0], pw[0]);
        float v = pa[0] + pw[0];  // bit 5 = 0: a, 1: w
        float t = v;
        swap16(v, t);
        v = v + t;
        v = v + dpp<0x128>(v);
        if (!b3 && !b4) (b5 ? L.ww : L.aa)[i][j0] = v;
      }
    }
    __syncthreads();
    // ---- D2: the batch rows in order (value threads), each final once the
    // rows before it are in; then the outputs
    if (value_thread) {
      const int j = jv;
      // Within a step every later row of the pass is updated, also those past
      // nr (their values are unused and never stored), so the update has no
      // per-row branches; a row's arithmetic involves only the rows before it.
      float acc[MR], out[MR];
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        acc[i] = L.vv[i][j];
        out[i] = L.sq[i][j];
      }
      // u_r replaces its residual in acc; the rows are stored after the chain
#pragma unroll
      for (int is = 0; is < MR; ++is) {
        if (is < nr) {
          float gk[MR], gq[MR];
          load_row<MR>(gk, L.gk[r0 + is]);
          load_row<MR>(gq, L.gq[r0 + is]);
          const float u = L.bt[is] * (acc[is] - L.aa[is][j]);
          acc[is] = u;
#pragma unroll
          for (int i = is; i < MR; ++i) {
            if (i > is) acc[i] = __builtin_fmaf(-gk[i], u, acc[i]);
            out[i] = __builtin_fmaf(gq[i], u, out[i]);
          }
        }
      }
#pragma unroll
      for (int is = 0; is < MR; ++is) {
        if (is < nr) {
          L.ru[r0 + is][j] = acc[is];
          if constexpr (STASH) a.stash[unit_stash + int64_t(done + is) * kRowFloats + 2 * kD + j] = acc[is];
        }
      }
      if (a.o != nullptr) {
        // the pass's rows as a buffer resource ending after row nr - 1: stores of
        // rows past it are dropped by the range check, without a branch per row
        constexpr int kEs = int(sizeof(typename InT::storage));
        const int row_bytes = a.H * kD * kEs;
        const auto ors = buffer_rsrc(static_cast<char*>(a.o) + (int64_t(t0) * a.H + h) * (kD * kEs),
                                     (nr - 1) * row_bytes + kD * kEs);
#pragma unroll
        for (int i = 0; i < MR; ++i) {
          if constexpr (SPLIT) InT::bstore1(ors, i * row_bytes + j * kEs, out[i] + L.ww[i][j]);
          else if (i < nr) InT::store1(a.o, (int64_t(t0 + i) * a.H + h) * kD + j, out[i] + L.ww[i][j]);
        }
      }
    }
    // the next batch's inputs, in flight during the close
    if constexpr (!SPLIT) {
      if (nr_next > 0) load_batch<InT, MR>(in, a, h, t0 + nr, nr_next, tid);
    }
    __syncthreads();
    p += nr;
    done += nr;
    if (!closes) break;  // a batch that does not close the chunk ends the sequence
    // ---- E: close the chunk (a prepared next pass's set is fetched first, in flight during the close)
    if constexpr (SPLIT) {
      if (a.prep != nullptr && nr_next == kChunk && (t0 + nr) / kChunk < a.prep_windows) {
        fetch_prepared(pre, a.prep + (int64_t((t0 + nr) / kChunk) * a.H + h) * kPrepFloats, tid);
        have_pre = true;
      }
    }
    close_block(S, L.rk, L.ru, L.gam, kChunk, c0, j0);
    if constexpr (STASH) {  // verify: the closed entry state, for a commit that accepts past the chunk end
      float* Sx = a.stash + unit_stash + int64_t(a.gamma) * kRowFloats;
#pragma unroll
      for (int i = 0; i < 16; ++i) st_f4(Sx + (c0 + i) * kD + j0, make_float4(S[i][0], S[i][1], S[i][2], S[i][3]));
    }
    p = 0;
    closed = true;
    if (nr_next <= 0) break;
    nr = nr_next;
    __syncthreads();
  }

  // ---- write back: S_e if a chunk closed, the new open rows, the position
  if (a.read_only) return;
  if (closed) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (CW == 4) {
        st_f4(Sp + (c0 + i) * kD + j0, make_float4(S[i][0], S[i][1], S[i][2], S[i][3]));
      } else {
#pragma unroll
        for (int x = 0; x < CW; ++x) Sp[(c0 + i) * kD + j0 + x] = S[i][x];
      }
    }
  }
  const int first_new = closed ? 0 : p_first;
  if constexpr (SPLIT) {
    // this slice's u columns of the new open rows; the keys, decays and
    // position follow in kda_contract_rows_kernel
    constexpr int kVecs = kSliceCols / 4;
    for (int e = tid; e < (p - first_new) * kVecs; e += kThreads) {
      const int s = first_new + e / kVecs, f = kSliceCols * slice + 4 * (e % kVecs);
      st_f4(Rp + s * kRowFloats + 2 * kD + f, *reinterpret_cast<const float4*>(&L.ru[s][f]));
    }
  } else {
    for (int e = tid; e < (p - first_new) * (kRowFloats / 4); e += kThreads) {
      const int s = first_new + e / (kRowFloats / 4), f = 4 * (e % (kRowFloats / 4));
      const float* src = (f < kD) ? &L.rk[s][f] : (f < 2 * kD) ? &L.rb[s][f - kD] : &L.ru[s][f - 2 * kD];
      st_f4(Rp + s * kRowFloats + f, *reinterpret_cast<const float4*>(src));
    }
    if (tid == 0) a.pos[unit] = p;
  }
}

// Chunk-parallel preparation for a split prefill with a workspace: one
// workgroup per (16-token window w of the packed tokens, head) forms the
// prepared set of the full chunk that starts in tokens 16w .. 16w + 15, if
// any, with the walk's own functions (load_batch, form_rows, gram_entries,
// close_factors on the same LDS layout).  A sequence's full chunks start
// (16 - p) % 16 tokens after its start (p = rows its slot holds, read before
// the walk changes it) and every 16 tokens after that; full chunks are
// disjoint 16-token ranges, so at most one starts in a window, and the walk
// finds the chunk starting at token t in window t / 16.
template <typename InT>
__global__ __launch_bounds__(kThreads) void kda_contract_prep_kernel(ContractArgs a, int n_windows) {
  __shared__ __align__(16) Lds<kChunk> L;
  const int w = blockIdx.x % n_windows;
  const int h = blockIdx.x / n_windows;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lo = kChunk * w;
  // first sequence that ends after token lo
  int n0 = 0, n1 = a.num_seqs;
  while (n0 < n1) {
    const int m = (n0 + n1) / 2;
    if (a.cu[m + 1] > lo) n1 = m;
    else n0 = m + 1;
  }
  int start = -1;
  for (int n = n0; n < a.num_seqs && a.cu[n] < lo + kChunk && start < 0; ++n) {
    const int b0 = a.cu[n], b1 = a.cu[n + 1];
    const int64_t unit = int64_t(a.slots ? a.slots[n] : n) * a.H + h;
    const int first = b0 + ((kChunk - (a.pos[unit] & (kChunk - 1))) & (kChunk - 1));
    const int j = lo > first ? (lo - first + kChunk - 1) / kChunk : 0;
    const int c = first + kChunk * j;
    if (c < lo + kChunk && c + kChunk <= b1) start = c;
  }
  if (start < 0) return;
  BatchIn<InT, kChunk> in;
  load_batch<InT, kChunk>(in, a, h, start, kChunk, tid);
  form_rows<InT, kChunk, false>(L, in, a.scale, 0, kChunk, tid, nullptr);
  __syncthreads();
  gram_entries<kChunk>(L, 0, kChunk, tid, lane);
  __syncthreads();
  if (tid < kD) close_factors(L.rk, L.rb, L.gam, kChunk, tid);
  __syncthreads();
  float* set = a.prep + (int64_t(w) * a.H + h) * kPrepFloats;
  constexpr int kRowVec = kD / 4;
  for (int e = tid; e < 16 * kRowVec; e += kThreads) {
    const int r = e / kRowVec, f = 4 * (e % kRowVec);
    st_f4(set + kPrepKh + 4 * e, *reinterpret_cast<const float4*>(&L.kh[r][f]));
    st_f4(set + kPrepQh + 4 * e, *reinterpret_cast<const float4*>(&L.qh[r][f]));
    st_f4(set + kPrepKb + 4 * e, *reinterpret_cast<const float4*>(&L.rk[r][f]));
    st_f4(set + kPrepV + 4 * e, *reinterpret_cast<const float4*>(&L.vv[r][f]));
  }
  constexpr int kSq = kChunk * kChunk / 4;
  if (tid < kSq) {
    const int s = tid / (kChunk / 4), f = 4 * (tid % (kChunk / 4));
    st_f4(set + kPrepGk + 4 * tid, *reinterpret_cast<const float4*>(&L.gk[s][f]));
    st_f4(set + kPrepGq + 4 * tid, *reinterpret_cast<const float4*>(&L.gq[s][f]));
  } else if (tid < kSq + kChunk / 4) {
    const int e = tid - kSq;
    st_f4(set + kPrepBt + 4 * e, *reinterpret_cast<const float4*>(&L.bt[4 * e]));
  } else if (tid < kSq + kChunk / 4 + kD / 4) {
    const int e = tid - kSq - kChunk / 4;
    st_f4(set + kPrepGam + 4 * e, *reinterpret_cast<const float4*>(&L.gam[4 * e]));
  }
}

// After a split prefill: the keys and cumulative decays of the new open rows
// and the new position of each (sequence, head), formed from the inputs with
// the prefill's arithmetic (the same additions in the same order: from the
// last open row's decay, or from 0 at a chunk start).  One thread per key
// channel.
template <typename InT>
__global__ __launch_bounds__(kD) void kda_contract_rows_kernel(ContractArgs a) {
  const int n = blockIdx.x / a.H;
  const int h = blockIdx.x % a.H;
  if (n >= a.num_seqs) return;
  const int c = threadIdx.x;
  const int tok0 = a.cu[n];
  const int count = a.cu[n + 1] - tok0;
  if (count <= 0) return;
  const int64_t unit = int64_t(a.slots ? a.slots[n] : n) * a.H + h;
  float* Rp = a.rows + unit * kChunk * kRowFloats;
  const int p0 = a.pos[unit] & (kChunk - 1);
  const int total = p0 + count;
  const int pf = total & (kChunk - 1);
  const bool closed = total >= kChunk;
  const int first = closed ? 0 : p0;  // rows first .. pf-1 are new
  float b = (!closed && p0 > 0) ? Rp[(p0 - 1) * kRowFloats + kD + c] : 0.0f;
  const int t_first = tok0 + count - (pf - first);  // token of row `first`
  for (int s = first; s < pf; ++s) {
    const int64_t tok = int64_t(t_first + s - first) * a.H + h;
    b = b + a.g[tok * kD + c];
    Rp[s * kRowFloats + c] = InT::unpack1(InT::load1raw(a.k, tok * kD + c));
    Rp[s * kRowFloats + kD + c] = b;
  }
  __syncthreads();  // every thread has read the position
  if (c == 0) a.pos[unit] = pf;
}

// Commit from a verify's stash: the first L = accepted[n] (clamped to 0 .. gamma, gamma <= 16)
// draft rows of (n, h) go to the open chunk; if the accepted rows reach the chunk end, the entry
// state the verify formed at that close replaces S_e and the rows after it start the new chunk.
// Pure copies of values the verify computed with the decode's arithmetic.
__global__ __launch_bounds__(kThreads) void kda_contract_commit_stash_kernel(
    const float* __restrict__ stash, const int32_t* __restrict__ accepted, const int32_t* __restrict__ slots,
    float* __restrict__ S_pool, float* __restrict__ rows_pool, int32_t* __restrict__ pos_pool, int N, int H,
    int gamma) {
  const int n = blockIdx.x / H;
  const int h = blockIdx.x % H;
  if (n >= N) return;
  const int tid = threadIdx.x;
  const int L = min(max(accepted[n], 0), gamma);
  if (L == 0) return;
  const int64_t unit = int64_t(slots ? slots[n] : n) * H + h;
  const float* st = stash + (int64_t(n) * H + h) * (int64_t(gamma) * kRowFloats + kD * kD);
  int32_t* pp = pos_pool + unit;
  const int p = *pp & (kChunk - 1);
  float* Rp = rows_pool + unit * kChunk * kRowFloats;
  constexpr int kVecs = kRowFloats / 4;
  int first = 0, dst = p;                  // draft rows first .. L-1 go to pool rows dst ..
  // every load of a thread is issued before its first store, so the copies
  // wait for memory once rather than once per vector
  if (p + L >= kChunk) {                   // the drafts closed the chunk at draft kChunk - 1 - p
    const float* Sx = st + int64_t(gamma) * kRowFloats;
    float* Sp = S_pool + unit * kD * kD;
    constexpr int kPer = kD * kD / 4 / kThreads;
    float4 x[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) x[i] = ld_f4(Sx + 4 * (tid + i * kThreads));
#pragma unroll
    for (int i = 0; i < kPer; ++i) st_f4(Sp + 4 * (tid + i * kThreads), x[i]);
    first = kChunk - p;
    dst = 0;
  }
  constexpr int kRowIters = (kChunk * kVecs + kThreads - 1) / kThreads;  // at most 16 rows
  const int nvec = (L - first) * kVecs;
  float4 y[kRowIters];
#pragma unroll
  for (int i = 0; i < kRowIters; ++i) {
    const int e = tid + i * kThreads;
    if (e < nvec) y[i] = ld_f4(st + (first + e / kVecs) * kRowFloats + 4 * (e % kVecs));
  }
#pragma unroll
  for (int i = 0; i < kRowIters; ++i) {
    const int e = tid + i * kThreads;
    if (e < nvec) st_f4(Rp + (dst + e / kVecs) * kRowFloats + 4 * (e % kVecs), y[i]);
  }
  __syncthreads();  // every thread has read the position before it changes
  if (tid == 0) *pp = (p + L) & (kChunk - 1);
}

// The running state S_t = Diag(e^{b_p-1}) S_e + sum_{s<p} (k_s e^{b_p-1 - b_s}) u_s^T:
// the chunk close's arithmetic applied to the rows held, without changing them.
__global__ __launch_bounds__(kThreads) void kda_contract_state_kernel(const float* __restrict__ S_pool,
                                                                      const float* __restrict__ rows_pool,
                                                                      const int32_t* __restrict__ pos_pool,
                                                                      const int32_t* __restrict__ slots,
                                                                      float* __restrict__ out, int N, int H) {
  __shared__ __align__(16) float rk[kChunk][kRS];
  __shared__ __align__(16) float rb[kChunk][kRS];
  __shared__ __align__(16) float ru[kChunk][kD];
  __shared__ __align__(16) float gam[kD];
  const int n = blockIdx.x / H;
  const int h = blockIdx.x % H;
  if (n >= N) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t unit = int64_t(slots ? slots[n] : n) * H + h;
  const float* Sp = S_pool + unit * kD * kD;
  const float* Rp = rows_pool + unit * kChunk * kRowFloats;
  const int p = pos_pool[unit] & (kChunk - 1);
  const int c0 = 16 * (lane >> 3);
  const int j0 = 32 * wave + 4 * (lane & 7);
  float S[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 s4 = ld_f4(Sp + (c0 + i) * kD + j0);
    S[i][0] = s4.x; S[i][1] = s4.y; S[i][2] = s4.z; S[i][3] = s4.w;
  }
  if (p > 0) {
    for (int e = tid; e < p * (kRowFloats / 4); e += kThreads) {
      const int s = e / (kRowFloats / 4), f = 4 * (e % (kRowFloats / 4));
      const float4 x = ld_f4(Rp + s * kRowFloats + f);
      float* dst = (f < kD) ? &rk[s][f] : (f < 2 * kD) ? &rb[s][f - kD] : &ru[s][f - 2 * kD];
      *reinterpret_cast<float4*>(dst) = x;
    }
    __syncthreads();
    if (tid < kD) close_factors(rk, rb, gam, p, tid);
    __syncthreads();
    close_block(S, rk, ru, gam, p, c0, j0);
  }
  float* dst = out + int64_t(n * H + h) * kD * kD;
#pragma unroll
  for (int i = 0; i < 16; ++i) st_f4(dst + (c0 + i) * kD + j0, make_float4(S[i][0], S[i][1], S[i][2], S[i][3]));
}

template <typename InT, int MR, bool STASH = false>
hipError_t launch_as(ContractArgs a, hipStream_t stream, int split, int prep_windows = 0) {
  const unsigned blocks = unsigned(a.num_seqs) * unsigned(a.H);
  // a prefill with at most one workgroup per 4 (2) CUs splits each (sequence, head)
  // four (two) ways (unless the caller fixed the width); the split builds are
  // sized for one workgroup per CU
  if constexpr (MR == kChunk && !STASH) {
    const unsigned cus = unsigned(device_cu_count());
    if (split == 0) split = 4 * blocks <= cus ? 4 : (2 * blocks <= cus ? 2 : 1);
    if (a.cu != nullptr && !a.read_only && split > 1) {
      if (prep_windows <= 0) a.prep = nullptr;
      if (a.prep != nullptr) {
        hipLaunchKernelGGL((kda_contract_prep_kernel<InT>), dim3(unsigned(prep_windows) * unsigned(a.H)),
                           dim3(kThreads), 0, stream, a, prep_windows);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      if (split == 4)
        hipLaunchKernelGGL((kda_contract_kernel<InT, MR, false, 4>), dim3(4 * blocks), dim3(kThreads), 0, stream, a);
      else
        hipLaunchKernelGGL((kda_contract_kernel<InT, MR, false, 2>), dim3(2 * blocks), dim3(kThreads), 0, stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((kda_contract_rows_kernel<InT>), dim3(blocks), dim3(kD), 0, stream, a);
      return hipGetLastError();
    }
  }
  a.prep = nullptr;  // only the split build reads prepared sets
  hipLaunchKernelGGL((kda_contract_kernel<InT, MR, STASH>), dim3(blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_contract(const ContractLaunch& c, bool bf16, hipStream_t stream) {
  if (c.num_seqs == 0) return hipSuccess;
  ContractArgs a{c.q, c.k, c.v, c.g, c.beta, c.cu_seqlens, c.slots, c.S_pool, c.rows_pool, c.pos_pool,
                 c.o, c.num_seqs, c.H, c.scale, c.gamma, c.counts, c.read_only ? 1 : 0, c.stash,
                 c.cu_seqlens != nullptr ? static_cast<float*>(c.workspace) : nullptr,
                 int((c.T_total + kChunk - 1) / kChunk)};
  const int prep_windows = a.prep_windows;
  // Rows per pass: 1 for decode, 8 for draft blocks of up to 8 tokens, 16
  // otherwise (a row's arithmetic does not depend on it, only registers do).
  const bool block8 = c.cu_seqlens == nullptr && c.gamma <= 8;
  const int sp = c.split;
  if (c.stash != nullptr) {
    if (block8) return bf16 ? launch_as<BF16, 8, true>(a, stream, 1) : launch_as<F32, 8, true>(a, stream, 1);
    return bf16 ? launch_as<BF16, kChunk, true>(a, stream, 1) : launch_as<F32, kChunk, true>(a, stream, 1);
  }
  if (c.cu_seqlens == nullptr && c.gamma == 1)
    return bf16 ? launch_as<BF16, 1>(a, stream, 1) : launch_as<F32, 1>(a, stream, 1);
  if (block8) return bf16 ? launch_as<BF16, 8>(a, stream, 1) : launch_as<F32, 8>(a, stream, 1);
  return bf16 ? launch_as<BF16, kChunk>(a, stream, sp, prep_windows) : launch_as<F32, kChunk>(a, stream, sp, prep_windows);
}

size_t contract_prefill_workspace_bytes(int64_t T_total, int H) {
  return size_t((T_total + kChunk - 1) / kChunk) * size_t(H) * kPrepFloats * sizeof(float);
}

hipError_t launch_contract_commit_stash(const float* stash, const int32_t* accepted, const int32_t* slots,
                                        float* S_pool, float* rows_pool, int32_t* pos_pool, int N, int H, int gamma,
                                        hipStream_t stream) {
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(kda_contract_commit_stash_kernel, dim3(unsigned(N) * unsigned(H)), dim3(kThreads), 0, stream,
                     stash, accepted, slots, S_pool, rows_pool, pos_pool, N, H, gamma);
  return hipGetLastError();
}

hipError_t launch_contract_state(const float* S_pool, const float* rows_pool, const int32_t* pos_pool,
                                 const int32_t* slots, float* out, int N, int H, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(kda_contract_state_kernel, dim3(unsigned(N) * unsigned(H)), dim3(kThreads), 0, stream,
                     S_pool, rows_pool, pos_pool, slots, out, N, H);
  return hipGetLastError();
}

}  // namespace kda
