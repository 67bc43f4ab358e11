// Host-side launcher declarations shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Compute units of the current device (256 on MI355X; fewer in a partitioned
// mode).  Queried per launch, nothing cached.
int device_cu_count();

// Input prologue applied inside the kernels: per-token L2 normalisation of q
// and k (x / sqrt(sum x^2 + eps)) and gate logits x -> log-decay g_min * sigmoid(x).
struct Prologue {
  bool l2norm = false;
  float eps = 0.0f;
  bool gate = false;
  float g_min = 0.0f;
};

// ---- decode / verify / commit (kda_step.hip) ------------------------------
// pro: null for inputs used as given.
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         float* state, const int32_t* slots, int N, int H, bool bf16, float scale,
                         void* o, hipStream_t stream, const Prologue* pro = nullptr);

hipError_t launch_verify(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* state, const int32_t* slots, int N, int G, int H, bool bf16,
                         float scale, void* o, hipStream_t stream, const Prologue* pro = nullptr,
                         float* record = nullptr);

// The commit of the accepted prefix from a verify's record ([N, G, H, 2, 128] fp32 keys and
// log-decays as the prologue verify used them), v and beta as given.
hipError_t launch_commit_record(const float* record, const void* v, const float* beta, const float* state_in,
                                float* state_out, const int32_t* slots, const int32_t* accepted_len, int N, int G,
                                int H, bool bf16, hipStream_t stream);

hipError_t launch_commit(const void* k, const void* v, const float* g, const float* beta,
                         const float* state_in, float* state_out, const int32_t* slots,
                         const int32_t* accepted_len, int N, int G, int H, bool bf16, hipStream_t stream,
                         const Prologue* pro = nullptr);

// ---- segment composition (kda_compose.hip) --------------------------------
// Memory-roof probe: a nontemporal float4 copy of n floats (n a multiple of 4).
hipError_t launch_copy_probe(const float* src, float* dst, int64_t n, hipStream_t stream);
hipError_t launch_copy_probe_state(const float* src, float* dst, int64_t n_states, bool dependent,
                                   hipStream_t stream);
// Matrix-roof probe: blocks x 256 threads, each wave iters x 8 bf16 16x16x32 MFMAs; out receives
// blocks x 256 x 4 floats.  mfma_probe_flops: the flops one launch performs.
hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t stream);
int64_t mfma_probe_flops(int blocks, int iters);
// split_operands: bf16 MFMA on hi/lo split operands instead of fp32 MFMA
hipError_t launch_compose(const float* M, const float* S_tilde, const float* S_in0, float* S_in,
                          float* S_final, int n_seg, int H, bool split_operands, hipStream_t stream);

// ---- chunked prefill (kda_prefill.hip) ------------------------------------
struct PrefillLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* cu_seqlens;
  int32_t num_seqs;
  int32_t H;
  float scale;
  const float* initial_state;  // [num_seqs, H, 128, 128] or null (zeros)
  float* final_state;          // or null
  void* o;                     // or null
  float* transition_out;       // or null
  float* checkpoints = nullptr;  // or null: [n_ckpt, H, 128, 128]
  int32_t ckpt_interval = 0;     // positive multiple of 64 when checkpoints is set
  const int32_t* seq_order = nullptr;  // or null: device [num_seqs], the order sequences are started in
  const Prologue* pro = nullptr;       // or null: inputs used as given
  void* workspace = nullptr;           // or null: the split path's operand sets (prefill_workspace_bytes)
  int64_t ws_slots = 0;                // chunk slots the workspace holds (prefill_workspace_slots)
  bool ws_prepared = false;            // the workspace holds these rows' operand sets already
  bool ws_keep_output_operands = false;  // prepare the output operands even without outputs
};

hipError_t launch_prefill(const PrefillLaunch& p, bool bf16, hipStream_t stream);
// Whether a prefill grid takes the split path when it has a workspace.
bool prefill_split_applies(int64_t num_seqs, int64_t H, bool transitions, bool outputs);
// Workspace the split path needs for tokens up to t_end (cu_seqlens[num_seqs]); 0 when the grid
// would not take it.
size_t prefill_workspace_bytes(int64_t num_seqs, int64_t t_end, int64_t H, bool bf16, bool transitions,
                               bool outputs);
int64_t prefill_workspace_slots(int64_t num_seqs, int64_t t_end);

// ---- batch-invariant row contract (kda_contract.hip) ----------------------
struct ContractLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* cu_seqlens;  // prefill: [num_seqs + 1]; null: sequence n's tokens are n*gamma .. n*gamma+gamma-1
  const int32_t* slots;       // [num_seqs] or null (identity)
  float* S_pool;              // [P, H, 128, 128] chunk-entry states
  float* rows_pool;           // [P, H, 16, 3, 128] open-chunk rows
  int32_t* pos_pool;          // [P, H] rows held
  void* o;                    // or null
  int32_t num_seqs;
  int32_t H;
  float scale;
  int32_t gamma = 1;                // tokens per sequence when cu_seqlens is null (1: decode)
  const int32_t* counts = nullptr;  // with cu_seqlens null: device [num_seqs] tokens to apply (0..gamma)
  bool read_only = false;           // outputs only; the pools are not written (verify)
  float* stash = nullptr;           // verify: [num_seqs, H, gamma * 3 * 128 + 128 * 128] rows and closed state
  int32_t split = 0;                // prefill: workgroups per (sequence, head), 1, 2 or 4; 0 picks by grid size
  void* workspace = nullptr;        // prefill: contract_prefill_workspace_bytes(T_total, H) bytes, or null
  int64_t T_total = 0;              // prefill with a workspace: packed tokens (cu_seqlens[num_seqs])
};
size_t contract_prefill_workspace_bytes(int64_t T_total, int H);

hipError_t launch_contract(const ContractLaunch& c, bool bf16, hipStream_t stream);
hipError_t launch_contract_commit_stash(const float* stash, const int32_t* accepted, const int32_t* slots,
                                        float* S_pool, float* rows_pool, int32_t* pos_pool, int N, int H, int gamma,
                                        hipStream_t stream);
hipError_t launch_contract_state(const float* S_pool, const float* rows_pool, const int32_t* pos_pool,
                                 const int32_t* slots, float* out, int N, int H, hipStream_t stream);

}  // namespace kda
