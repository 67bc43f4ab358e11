// C ABI of the KDA library: argument validation and dispatch to the kernels.
// Nothing here computes the recurrence; every arithmetic step runs on the GPU.
#include "../../include/kda.h"
#include "kda_common.hpp"
#include "kda_internal.hpp"

#include <cstdint>
#include <mutex>

// Scratch of the allocation-free prefill (kda_prefill_noalloc): the split
// path's operand sets.  One copy per device, held from the library's load on
// that device until the process ends; every call on a device shares it.  Host
// code never uses this name as an address: the device address is looked up
// once per device (scratch_on_current_device) and passed to the kernels.
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool dims_ok(int32_t d_k, int32_t d_v) { return d_k == kda::kD && d_v == kda::kD; }
bool dtype_ok(kda_dtype_t d) { return d == KDA_F32 || d == KDA_BF16; }

kda_status_t hip_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// Validates a caller's prologue and converts it; false for a NULL or out-of-range one.
bool prologue_ok(const kda_prologue_t* p, kda::Prologue& out) {
  if (!p) return false;
  out.l2norm = p->l2norm_qk != 0;
  out.eps = p->l2norm_eps;
  out.gate = p->gate_logits != 0;
  out.g_min = p->g_min;
  if (out.l2norm && !(out.eps >= 0.0f && out.eps <= 3.0e38f)) return false;   // finite, >= 0 (NaN fails)
  if (out.gate && !(out.g_min < 0.0f && out.g_min >= -3.0e38f)) return false;  // finite, < 0
  return true;
}

// The device address of `scratch` on the current device, looked up with that
// device current the first time a call runs on it; nullptr if the lookup fails.
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}

}  // namespace

namespace kda {
int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}
}  // namespace kda

namespace {

kda_status_t prefill_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H,
                          int32_t d_k, int32_t d_v, kda_dtype_t dtype, float scale, const float* initial_state,
                          float* final_state, void* o, float* transition_out, int32_t ckpt_interval,
                          float* checkpoints, const int32_t* seq_order, const kda::Prologue* pro, void* stream,
                          void* workspace = nullptr, size_t workspace_bytes = 0, int32_t ws_flags = 0) {
  if (ws_flags & ~(KDA_WS_PREPARED | KDA_WS_KEEP_OUTPUT_OPERANDS)) return KDA_ERR_INVALID_ARG;
  if (num_seqs < 0 || H <= 0) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (checkpoints && (ckpt_interval <= 0 || ckpt_interval % 64 != 0)) return KDA_ERR_INVALID_ARG;
  if (num_seqs == 0) return KDA_OK;
  if (!cu_seqlens) return KDA_ERR_INVALID_ARG;
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] < 0) return KDA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < num_seqs; ++i)
      if (cu_seqlens_host[i + 1] < cu_seqlens_host[i]) return KDA_ERR_INVALID_ARG;
  }
  const bool any_tokens = !cu_seqlens_host || cu_seqlens_host[num_seqs] > cu_seqlens_host[0];
  if (any_tokens && (!q || !k || !v || !g || !beta)) return KDA_ERR_INVALID_ARG;
  if (!final_state && !o && !transition_out && !checkpoints) return KDA_OK;  // nothing requested
  kda::PrefillLaunch p{q, k, v, g, beta, cu_seqlens, num_seqs, H, scale, initial_state, final_state, o,
                       transition_out};
  p.checkpoints = checkpoints;
  p.ckpt_interval = checkpoints ? ckpt_interval : 0;
  p.seq_order = seq_order;
  p.pro = pro;
  if (workspace && !checkpoints) {
    // the split path sizes its chunk slots from the host copy of cu_seqlens
    if (!cu_seqlens_host) return KDA_ERR_INVALID_ARG;
    const int64_t t_end = cu_seqlens_host[num_seqs];
    const size_t need = kda::prefill_workspace_bytes(num_seqs, t_end, H, dtype == KDA_BF16, transition_out != nullptr,
                                                     o != nullptr);
    if (need > 0) {
      if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
      p.workspace = workspace;
      p.ws_slots = kda::prefill_workspace_slots(num_seqs, t_end);
      p.ws_prepared = (ws_flags & KDA_WS_PREPARED) != 0;
      p.ws_keep_output_operands = (ws_flags & KDA_WS_KEEP_OUTPUT_OPERANDS) != 0;
    }
  }
  return hip_status(kda::launch_prefill(p, dtype == KDA_BF16, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int kda_version(void) { return kVersion; }

kda_status_t kda_mfma_probe(float* out, int32_t blocks, int32_t iters, int64_t* flops, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out || reinterpret_cast<uintptr_t>(out) % 16 != 0) return KDA_ERR_INVALID_ARG;
  if (flops) *flops = kda::mfma_probe_flops(blocks, iters);
  return hip_status(kda::launch_mfma_probe(out, blocks, iters, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_copy_probe(const float* src, float* dst, int64_t n, void* stream) {
  if (n < 0 || (n % 4) != 0) return KDA_ERR_INVALID_ARG;
  if (n == 0) return KDA_OK;
  if (!src || !dst || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
    return KDA_ERR_INVALID_ARG;
  return hip_status(kda::launch_copy_probe(src, dst, n, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_copy_probe_state(const float* src, float* dst, int64_t n_states, int32_t dependent, void* stream) {
  // two workgroups per state: the grid stays below 2^31 workgroups
  if (n_states < 0 || n_states > (int64_t(1) << 29) || (dependent != 0 && dependent != 1)) return KDA_ERR_INVALID_ARG;
  if (n_states == 0) return KDA_OK;
  if (!src || !dst || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
    return KDA_ERR_INVALID_ARG;
  if (src != dst) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t bytes = uintptr_t(n_states) * 128 * 128 * sizeof(float);
    if (a < b + bytes && b < a + bytes) return KDA_ERR_INVALID_ARG;  // partial overlap
  }
  return hip_status(kda::launch_copy_probe_state(src, dst, n_states, dependent != 0, static_cast<hipStream_t>(stream)));
}

const char* kda_status_string(kda_status_t status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported (only d_k = d_v = 128 and dtype bf16/f32)";
    case KDA_ERR_HIP: return "HIP launch failed";
    case KDA_ERR_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

}  // extern "C"

namespace {

kda_status_t decode_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         float* state_pool, const int32_t* slots, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                         kda_dtype_t dtype, float scale, void* o, const kda::Prologue* pro, void* stream) {
  if (N < 0 || H <= 0) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !state_pool) return KDA_ERR_INVALID_ARG;
  return hip_status(kda::launch_decode(q, k, v, g, beta, state_pool, slots, N, H, dtype == KDA_BF16, scale,
                                       o, static_cast<hipStream_t>(stream), pro));
}

kda_status_t commit_impl(const void* k, const void* v, const float* g, const float* beta, float* state_pool,
                         const int32_t* slots, const int32_t* accepted_len, int32_t N, int32_t gamma1, int32_t H,
                         int32_t d_k, int32_t d_v, kda_dtype_t dtype, const kda::Prologue* pro, void* stream) {
  if (N < 0 || H <= 0 || gamma1 <= 0) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!k || !v || !g || !beta || !state_pool || !accepted_len) return KDA_ERR_INVALID_ARG;
  return hip_status(kda::launch_commit(k, v, g, beta, state_pool, state_pool, slots, accepted_len, N, gamma1,
                                       H, dtype == KDA_BF16, static_cast<hipStream_t>(stream), pro));
}

kda_status_t verify_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* state_pool, const int32_t* slots, int32_t N, int32_t gamma1, int32_t H,
                         int32_t d_k, int32_t d_v, kda_dtype_t dtype, float scale, void* o,
                         const int32_t* accepted_len, float* state_out_pool, const kda::Prologue* pro,
                         void* stream) {
  if (N < 0 || H <= 0 || gamma1 <= 0) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !state_pool || !o) return KDA_ERR_INVALID_ARG;
  if (accepted_len && !state_out_pool) return KDA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = kda::launch_verify(q, k, v, g, beta, state_pool, slots, N, gamma1, H, dtype == KDA_BF16,
                                    scale, o, s, pro);
  if (e != hipSuccess || !accepted_len) return hip_status(e);
  return hip_status(kda::launch_commit(k, v, g, beta, state_pool, state_out_pool, slots, accepted_len, N,
                                       gamma1, H, dtype == KDA_BF16, s, pro));
}

}  // namespace

extern "C" {

kda_status_t kda_decode_step(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, float* state_pool, const int32_t* slots, int32_t N,
                             int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype, float scale,
                             void* o, void* stream) {
  return decode_impl(q, k, v, g, beta, state_pool, slots, N, H, d_k, d_v, dtype, scale, o, nullptr, stream);
}

kda_status_t kda_decode_step_prologue(const void* q, const void* k, const void* v, const float* g,
                                      const float* beta, float* state_pool, const int32_t* slots, int32_t N,
                                      int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype, float scale, void* o,
                                      const kda_prologue_t* prologue, void* stream) {
  kda::Prologue pro;
  if (!prologue_ok(prologue, pro)) return KDA_ERR_INVALID_ARG;
  return decode_impl(q, k, v, g, beta, state_pool, slots, N, H, d_k, d_v, dtype, scale, o, &pro, stream);
}

kda_status_t kda_verify_commit(const void* k, const void* v, const float* g, const float* beta,
                               float* state_pool, const int32_t* slots, const int32_t* accepted_len,
                               int32_t N, int32_t gamma1, int32_t H, int32_t d_k, int32_t d_v,
                               kda_dtype_t dtype, void* stream) {
  return commit_impl(k, v, g, beta, state_pool, slots, accepted_len, N, gamma1, H, d_k, d_v, dtype, nullptr,
                     stream);
}

kda_status_t kda_verify_commit_prologue(const void* k, const void* v, const float* g, const float* beta,
                                        float* state_pool, const int32_t* slots, const int32_t* accepted_len,
                                        int32_t N, int32_t gamma1, int32_t H, int32_t d_k, int32_t d_v,
                                        kda_dtype_t dtype, const kda_prologue_t* prologue, void* stream) {
  kda::Prologue pro;
  if (!prologue_ok(prologue, pro)) return KDA_ERR_INVALID_ARG;
  return commit_impl(k, v, g, beta, state_pool, slots, accepted_len, N, gamma1, H, d_k, d_v, dtype, &pro, stream);
}

kda_status_t kda_verify_block(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const float* state_pool, const int32_t* slots,
                              int32_t N, int32_t gamma1, int32_t H, int32_t d_k, int32_t d_v,
                              kda_dtype_t dtype, float scale, void* o, const int32_t* accepted_len,
                              float* state_out_pool, void* stream) {
  return verify_impl(q, k, v, g, beta, state_pool, slots, N, gamma1, H, d_k, d_v, dtype, scale, o, accepted_len,
                     state_out_pool, nullptr, stream);
}

kda_status_t kda_verify_block_prologue(const void* q, const void* k, const void* v, const float* g,
                                       const float* beta, const float* state_pool, const int32_t* slots,
                                       int32_t N, int32_t gamma1, int32_t H, int32_t d_k, int32_t d_v,
                                       kda_dtype_t dtype, float scale, void* o, const int32_t* accepted_len,
                                       float* state_out_pool, const kda_prologue_t* prologue, void* stream) {
  kda::Prologue pro;
  if (!prologue_ok(prologue, pro)) return KDA_ERR_INVALID_ARG;
  return verify_impl(q, k, v, g, beta, state_pool, slots, N, gamma1, H, d_k, d_v, dtype, scale, o, accepted_len,
                     state_out_pool, &pro, stream);
}

kda_status_t kda_verify_block_record(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                    const float* state_pool, const int32_t* slots, int32_t N, int32_t gamma1,
                                    int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype, float scale, void* o,
                                    float* record, const kda_prologue_t* prologue, void* stream) {
  kda::Prologue pro;
  if (!prologue_ok(prologue, pro)) return KDA_ERR_INVALID_ARG;
  if (N < 0 || H <= 0 || gamma1 <= 0) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !state_pool || !o || !record) return KDA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(record) % 16 != 0) return KDA_ERR_INVALID_ARG;
  return hip_status(kda::launch_verify(q, k, v, g, beta, state_pool, slots, N, gamma1, H, dtype == KDA_BF16, scale,
                                       o, static_cast<hipStream_t>(stream), &pro, record));
}

kda_status_t kda_verify_commit_record(const float* record, const void* v, const float* beta, float* state_pool,
                                      const int32_t* slots, const int32_t* accepted_len, int32_t N, int32_t gamma1,
                                      int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype, void* stream) {
  if (N < 0 || H <= 0 || gamma1 <= 0) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!record || !v || !beta || !state_pool || !accepted_len) return KDA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(record) % 16 != 0) return KDA_ERR_INVALID_ARG;
  return hip_status(kda::launch_commit_record(record, v, beta, state_pool, state_pool, slots, accepted_len, N, gamma1,
                                              H, dtype == KDA_BF16, static_cast<hipStream_t>(stream)));
}

size_t kda_prefill_workspace_size(int32_t num_seqs, int64_t T_total, int32_t H, int32_t d_k, int32_t d_v,
                                  kda_dtype_t dtype, int32_t flags) {
  if (num_seqs <= 0 || T_total < 0 || H <= 0 || !dims_ok(d_k, d_v) || !dtype_ok(dtype)) return 0;
  if (flags & ~(KDA_PREFILL_TRANSITIONS | KDA_PREFILL_NO_OUTPUT)) return 0;
  return kda::prefill_workspace_bytes(num_seqs, T_total, H, dtype == KDA_BF16, (flags & KDA_PREFILL_TRANSITIONS) != 0,
                                      (flags & KDA_PREFILL_NO_OUTPUT) == 0);
}

kda_status_t kda_prefill_ex(const void* q, const void* k, const void* v, const float* g, const float* beta,
                            const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H,
                            int32_t d_k, int32_t d_v, kda_dtype_t dtype, float scale, const float* initial_state,
                            float* final_state, void* o, float* transition_out, const int32_t* seq_order,
                            const kda_prologue_t* prologue, void* workspace, size_t workspace_bytes,
                            int32_t ws_flags, void* stream) {
  kda::Prologue pro;
  if (prologue && !prologue_ok(prologue, pro)) return KDA_ERR_INVALID_ARG;
  return prefill_impl(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, num_seqs, H, d_k, d_v, dtype, scale,
                      initial_state, final_state, o, transition_out, 0, nullptr, seq_order, prologue ? &pro : nullptr,
                      stream, workspace, workspace_bytes, ws_flags);
}

kda_status_t kda_prefill_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs,
                                 int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype, float scale,
                                 const float* initial_state, float* final_state, void* o, float* transition_out,
                                 const int32_t* seq_order, const kda_prologue_t* prologue, void* stream) {
  kda::Prologue pro;
  if (prologue && !prologue_ok(prologue, pro)) return KDA_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (cu_seqlens_host && num_seqs > 0 && H > 0) {
    ws = scratch_on_current_device();
    if (!ws) return KDA_ERR_HIP;
  }
  return prefill_impl(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, num_seqs, H, d_k, d_v, dtype, scale,
                      initial_state, final_state, o, transition_out, 0, nullptr, seq_order, prologue ? &pro : nullptr,
                      stream, ws, ws ? kScratchBytes : 0);
}

size_t kda_prefill_noalloc_max_scratch(void) { return kScratchBytes; }

kda_status_t kda_prefill(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H, int32_t d_k,
                         int32_t d_v, kda_dtype_t dtype, float scale, const float* initial_state,
                         float* final_state, void* o, float* transition_out, void* stream) {
  return prefill_impl(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, num_seqs, H, d_k, d_v, dtype, scale,
                      initial_state, final_state, o, transition_out, 0, nullptr, nullptr, nullptr, stream);
}

kda_status_t kda_prefill_prologue(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                  int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype,
                                  float scale, const float* initial_state, float* final_state, void* o,
                                  float* transition_out, const kda_prologue_t* prologue, void* stream) {
  kda::Prologue pro;
  if (!prologue_ok(prologue, pro)) return KDA_ERR_INVALID_ARG;
  return prefill_impl(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, num_seqs, H, d_k, d_v, dtype, scale,
                      initial_state, final_state, o, transition_out, 0, nullptr, nullptr, &pro, stream);
}

kda_status_t kda_prefill_ordered(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const int32_t* cu_seqlens,
                                 const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H, int32_t d_k,
                                 int32_t d_v, kda_dtype_t dtype, float scale, const float* initial_state,
                                 float* final_state, void* o, float* transition_out, const int32_t* seq_order,
                                 void* stream) {
  if (!seq_order) return KDA_ERR_INVALID_ARG;
  return prefill_impl(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, num_seqs, H, d_k, d_v, dtype, scale,
                      initial_state, final_state, o, transition_out, 0, nullptr, seq_order, nullptr, stream);
}

kda_status_t kda_prefill_checkpointed(const void* q, const void* k, const void* v, const float* g,
                                      const float* beta, const int32_t* cu_seqlens,
                                      const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H, int32_t d_k,
                                      int32_t d_v, kda_dtype_t dtype, float scale, const float* initial_state,
                                      float* final_state, void* o, int32_t ckpt_interval, float* checkpoints,
                                      void* stream) {
  if (!checkpoints) return KDA_ERR_INVALID_ARG;
  return prefill_impl(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, num_seqs, H, d_k, d_v, dtype, scale,
                      initial_state, final_state, o, nullptr, ckpt_interval, checkpoints, nullptr, nullptr, stream);
}

int64_t kda_prefill_checkpoint_count(const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t ckpt_interval) {
  if (!cu_seqlens_host || num_seqs < 0 || ckpt_interval <= 0 || ckpt_interval % 64 != 0) return -1;
  int64_t n = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t len = int64_t(cu_seqlens_host[i + 1]) - cu_seqlens_host[i];
    if (len < 0) return -1;
    n += len > 0 ? (len - 1) / ckpt_interval : 0;
  }
  return n;
}

kda_status_t kda_compose_segments(const float* M, const float* S_tilde, const float* S_in0,
                                  float* S_in, float* S_final, int32_t n_seg, int32_t H,
                                  int32_t d_k, int32_t d_v, void* stream) {
  return kda_compose_segments_ex(M, S_tilde, S_in0, S_in, S_final, n_seg, H, d_k, d_v, 0, stream);
}

kda_status_t kda_compose_segments_ex(const float* M, const float* S_tilde, const float* S_in0,
                                     float* S_in, float* S_final, int32_t n_seg, int32_t H,
                                     int32_t d_k, int32_t d_v, int32_t flags, void* stream) {
  if (n_seg < 0 || H <= 0) return KDA_ERR_INVALID_ARG;
  if (flags & ~KDA_COMPOSE_SPLIT_BF16) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v)) return KDA_ERR_UNSUPPORTED;
  if (n_seg == 0 && !S_final) return KDA_OK;
  if ((n_seg > 0 && (!M || !S_tilde || !S_in))) return KDA_ERR_INVALID_ARG;
  return hip_status(kda::launch_compose(M, S_tilde, S_in0, S_in, S_final, n_seg, H,
                                        (flags & KDA_COMPOSE_SPLIT_BF16) != 0, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_contract_prefill(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                  int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype,
                                  float scale, float* S_pool, float* rows_pool, int32_t* pos_pool,
                                  const int32_t* slots, void* o, void* stream) {
  return kda_contract_prefill_split(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, num_seqs, H, d_k, d_v, dtype,
                                    scale, S_pool, rows_pool, pos_pool, slots, o, 0, stream);
}

kda_status_t kda_contract_prefill_split(const void* q, const void* k, const void* v, const float* g,
                                        const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                        int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype,
                                        float scale, float* S_pool, float* rows_pool, int32_t* pos_pool,
                                        const int32_t* slots, void* o, int32_t split_width, void* stream) {
  return kda_contract_prefill_ex(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, num_seqs, H, d_k, d_v, dtype, scale,
                                 S_pool, rows_pool, pos_pool, slots, o, split_width, nullptr, 0, stream);
}

size_t kda_contract_prefill_workspace_size(int64_t T_total, int32_t H) {
  if (T_total <= 0 || H <= 0) return 0;
  return kda::contract_prefill_workspace_bytes(T_total, H);
}

kda_status_t kda_contract_prefill_ex(const void* q, const void* k, const void* v, const float* g,
                                     const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                     int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype,
                                     float scale, float* S_pool, float* rows_pool, int32_t* pos_pool,
                                     const int32_t* slots, void* o, int32_t split_width, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (split_width != 0 && split_width != 1 && split_width != 2 && split_width != 4) return KDA_ERR_INVALID_ARG;
  if (num_seqs < 0 || H <= 0) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return KDA_OK;
  if (!cu_seqlens || !S_pool || !rows_pool || !pos_pool) return KDA_ERR_INVALID_ARG;
  if (workspace && !cu_seqlens_host) return KDA_ERR_INVALID_ARG;
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] < 0) return KDA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < num_seqs; ++i)
      if (cu_seqlens_host[i + 1] < cu_seqlens_host[i]) return KDA_ERR_INVALID_ARG;
  }
  const bool any_tokens = !cu_seqlens_host || cu_seqlens_host[num_seqs] > cu_seqlens_host[0];
  if (!any_tokens) return KDA_OK;
  if (!q || !k || !v || !g || !beta) return KDA_ERR_INVALID_ARG;
  kda::ContractLaunch c{q, k, v, g, beta, cu_seqlens, slots, S_pool, rows_pool, pos_pool, o, num_seqs, H, scale};
  c.split = split_width;
  if (workspace) {
    c.T_total = cu_seqlens_host[num_seqs];
    if (workspace_bytes < kda::contract_prefill_workspace_bytes(c.T_total, H)) return KDA_ERR_WORKSPACE;
    c.workspace = workspace;
  }
  return hip_status(kda::launch_contract(c, dtype == KDA_BF16, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_contract_decode(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                                 kda_dtype_t dtype, float scale, float* S_pool, float* rows_pool,
                                 int32_t* pos_pool, const int32_t* slots, void* o, void* stream) {
  if (N < 0 || H <= 0) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !S_pool || !rows_pool || !pos_pool) return KDA_ERR_INVALID_ARG;
  kda::ContractLaunch c{q, k, v, g, beta, nullptr, slots, S_pool, rows_pool, pos_pool, o, N, H, scale};
  return hip_status(kda::launch_contract(c, dtype == KDA_BF16, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_contract_verify(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, int32_t N, int32_t gamma1, int32_t H, int32_t d_k,
                                 int32_t d_v, kda_dtype_t dtype, float scale, const float* S_pool,
                                 const float* rows_pool, const int32_t* pos_pool, const int32_t* slots, void* o,
                                 float* stash, void* stream) {
  if (N < 0 || H <= 0 || gamma1 <= 0 || (stash && gamma1 > 16)) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !S_pool || !rows_pool || !pos_pool || !o) return KDA_ERR_INVALID_ARG;
  // read-only: the kernel writes only o (the pool pointers are not written through)
  kda::ContractLaunch c{q, k, v, g, beta, nullptr, slots, const_cast<float*>(S_pool), const_cast<float*>(rows_pool),
                        const_cast<int32_t*>(pos_pool), o, N, H, scale};
  c.gamma = gamma1;
  c.read_only = true;
  c.stash = stash;
  return hip_status(kda::launch_contract(c, dtype == KDA_BF16, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_contract_commit_stash(const float* stash, const int32_t* accepted_len, int32_t N, int32_t gamma1,
                                       int32_t H, int32_t d_k, int32_t d_v, float* S_pool, float* rows_pool,
                                       int32_t* pos_pool, const int32_t* slots, void* stream) {
  if (N < 0 || H <= 0 || gamma1 <= 0 || gamma1 > 16) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v)) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!stash || !accepted_len || !S_pool || !rows_pool || !pos_pool) return KDA_ERR_INVALID_ARG;
  return hip_status(kda::launch_contract_commit_stash(stash, accepted_len, slots, S_pool, rows_pool, pos_pool, N, H,
                                                      gamma1, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_contract_commit(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const int32_t* accepted_len, int32_t N, int32_t gamma1,
                                 int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype, float* S_pool,
                                 float* rows_pool, int32_t* pos_pool, const int32_t* slots, void* stream) {
  if (N < 0 || H <= 0 || gamma1 <= 0) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v) || !dtype_ok(dtype)) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!k || !v || !g || !beta || !accepted_len || !S_pool || !rows_pool || !pos_pool) return KDA_ERR_INVALID_ARG;
  // without q no outputs are formed; the kernel still reads a query, so it reads the keys
  kda::ContractLaunch c{q ? q : k, k, v, g, beta, nullptr, slots, S_pool, rows_pool, pos_pool, nullptr, N, H, 1.0f};
  c.gamma = gamma1;
  c.counts = accepted_len;
  return hip_status(kda::launch_contract(c, dtype == KDA_BF16, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_contract_state(const float* S_pool, const float* rows_pool, const int32_t* pos_pool,
                                const int32_t* slots, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                                float* state_out, void* stream) {
  if (N < 0 || H <= 0) return KDA_ERR_INVALID_ARG;
  if (!dims_ok(d_k, d_v)) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!S_pool || !rows_pool || !pos_pool || !state_out) return KDA_ERR_INVALID_ARG;
  return hip_status(kda::launch_contract_state(S_pool, rows_pool, pos_pool, slots, state_out, N, H,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"
