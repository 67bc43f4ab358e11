/*
 * kda.h — C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library.
 *
 * The recurrence, per sequence and head, token by token:
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T (scale * q_t)
 * with alpha_t = exp(g_t) per key channel (g = log-decay, g <= 0), beta_t a
 * scalar per token and head, and S a d_k x d_v fp32 matrix whose rows are key
 * channels.  Source: "Kimi K3：架构与 SGLang Day-0 Support" (yichizhang.dev),
 * section "attention 机制详解：KDA" (math-details box: the full update and its
 * gate-then-delta split), and section "attention 机制详解：linear attention"
 * (readout o = S^T q after the write).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is DEVICE memory owned by the caller, except the
 *     ones named *_host.  The library never allocates, frees or keeps memory.
 *   - Layouts are dense row-major.  q, k, g are [.., d_k]; v, o are [.., d_v];
 *     states are [.., d_k, d_v] fp32.  Only d_k = d_v = 128 is implemented.
 *   - q, k, v (and o) are bf16 (KDA_BF16) or fp32 (KDA_F32); g, beta and all
 *     states are always fp32.  bf16 outputs are rounded to nearest even.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronise the device.  Host-side argument errors are
 *     reported before anything is enqueued; KDA_ERR_HIP reports a failed launch.
 *   - Outputs must not alias inputs except where an entry point says so.
 *   - No global mutable state: calls on different streams are independent as
 *     long as their output buffers are disjoint.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent cu_seqlens_host */
  KDA_ERR_UNSUPPORTED = 2, /* d_k or d_v != 128, unknown dtype */
  KDA_ERR_HIP = 3,         /* the HIP runtime rejected a launch */
  KDA_ERR_WORKSPACE = 4    /* a workspace smaller than the call needs */
} kda_status_t;

typedef enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;

/* Library version (major * 10000 + minor * 100 + patch). */
int kda_version(void);

/* Static English text for a status code. */
const char* kda_status_string(kda_status_t status);

/*
 * kda_copy_probe — measurement probe, not part of the recurrence: copies n
 * fp32 values from src to dst (device buffers, 16-byte aligned, not
 * overlapping, n a multiple of 4) with nontemporal 16-byte loads and stores,
 * eight per thread.  It measures the memory roof that the state-streaming
 * kernels (decode, commit) are compared with.  KDA_ERR_INVALID_ARG for a
 * negative or unaligned n or misaligned pointers; n == 0 does nothing.
 */
kda_status_t kda_copy_probe(const float* src, float* dst, int64_t n, void* stream);

/*
 * kda_copy_probe_state — measurement probe, not part of the recurrence:
 * copies n_states 128 x 128 fp32 matrices (row-major, contiguous) from src to
 * dst in the access pattern of kda_decode_step's state stream (one workgroup
 * per 128 x 64 half, each wave load instruction covering eight 128-byte row
 * segments, nontemporal loads and stores, every load of a thread before its
 * stores), without the step's arithmetic: the copy rate of the decode's own
 * pattern, which the decode is compared with.  dependent = 1 also keeps the
 * decode's ordering: no store of a workgroup is issued before all of its loads
 * have completed (the step's stores need column sums over every row);
 * dependent = 0 lets each store follow its own load.  src == dst copies in
 * place (the decode updates its state in place); otherwise the ranges must not
 * overlap.  Device buffers, 16-byte aligned.  KDA_ERR_INVALID_ARG for a
 * negative count or one above 2^29, dependent not 0 or 1, misaligned or null
 * pointers, or partially overlapping ranges; 0 states do nothing.
 */
kda_status_t kda_copy_probe_state(const float* src, float* dst, int64_t n_states, int32_t dependent, void* stream);

/*
 * kda_mfma_probe — measurement probe, not part of the recurrence: blocks
 * workgroups of 256 threads, each wave issuing iters x 8 independent
 * v_mfma_f32_16x16x32_bf16 (the prefill's matrix product; iters rounded up
 * to a multiple of 4), to measure the
 * matrix roof the prefill is compared with.  out: device buffer of
 * blocks x 256 x 4 floats (16-byte aligned) receiving the accumulators (so
 * the work is kept); *flops (host, may be NULL) receives the flops of the
 * launch.  KDA_ERR_INVALID_ARG for non-positive counts or a bad buffer.
 */
kda_status_t kda_mfma_probe(float* out, int32_t blocks, int32_t iters, int64_t* flops, void* stream);

/*
 * kda_decode_step — one token per request: gate, delta write, readout, in place.
 *
 * Per request n and head h (the step is the gate-then-delta split of the KDA
 * update, section "attention 机制详解：KDA" of the Day-0 lesson page):
 *     S~ = Diag(exp g) S;  r = S~^T k;  u = beta (v - r);  S <- S~ + k u^T;  o = S^T (scale q)
 *   q, k, g : [N, H, 128]  (q, k in `dtype`; g fp32)
 *   v       : [N, H, 128]  (`dtype`)
 *   beta    : [N, H]       fp32
 *   state_pool : [P, H, 128, 128] fp32, read and overwritten IN PLACE at pool
 *                row slots[n] (slots == NULL means slots[n] = n and P >= N).
 *                Slots must be distinct; they are not range-checked on the device.
 *   o       : [N, H, 128] in `dtype`, or NULL to skip the readout.
 * N == 0 is a no-op.
 */
kda_status_t kda_decode_step(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, float* state_pool, const int32_t* slots,
                             int32_t N, int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype,
                             float scale, void* o, void* stream);

/*
 * kda_verify_block — score a block of gamma1 draft tokens per request from its
 * committed state, which is only READ (ReplaySSM: "SGLang 和 Miles 为 Kimi K3
 * 提供首日支持", section "ReplaySSM：针对 KDA 状态的原始输入重放"; and section 7
 * of "Kimi K3 的训练与 Serving Infra").
 *   q, k, g : [N, gamma1, H, 128];  v : [N, gamma1, H, 128];  beta : [N, gamma1, H]
 *   state_pool : [P, H, 128, 128] fp32, read at slots[n] (NULL = identity), never written.
 *   o       : [N, gamma1, H, 128]: o[n, t] = readout after tokens 1..t+1 of request n.
 * If accepted_len (device int32 [N], values in 1..gamma1) is non-NULL the call
 * also enqueues kda_verify_commit into state_out_pool (same slots), which may
 * be state_pool itself; the commit replays the accepted prefix from the state
 * that was verified, with the same per-token routine, so its result is
 * bit-identical to that many kda_decode_step calls.
 */
kda_status_t kda_verify_block(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const float* state_pool, const int32_t* slots,
                              int32_t N, int32_t gamma1, int32_t H, int32_t d_k, int32_t d_v,
                              kda_dtype_t dtype, float scale, void* o, const int32_t* accepted_len,
                              float* state_out_pool, void* stream);

/*
 * kda_verify_commit — the fold: advance each request's state by its accepted
 * prefix by replaying the stored raw inputs (k, v, g, beta) from the committed
 * state, in place (same page and section as kda_verify_block).  The caller
 * keeps the verify call's input buffers unchanged until this call has run, so
 * the fold consumes exactly the gates the verify consumed.
 *   k, g : [N, gamma1, H, 128];  v : [N, gamma1, H, 128];  beta : [N, gamma1, H]
 *   state_pool : [P, H, 128, 128] fp32 at slots[n] (NULL = identity), updated in place.
 *   accepted_len : device int32 [N]; entries are clamped to 0..gamma1 on the
 *                  device (0 leaves the state unchanged).
 */
kda_status_t kda_verify_commit(const void* k, const void* v, const float* g, const float* beta,
                               float* state_pool, const int32_t* slots, const int32_t* accepted_len,
                               int32_t N, int32_t gamma1, int32_t H, int32_t d_k, int32_t d_v,
                               kda_dtype_t dtype, void* stream);

/*
 * Input prologue — applied inside the kernels to the raw per-token inputs,
 * for callers that hand over unnormalised q, k and gate logits.  The KDA
 * math-details box of the Day-0 lesson page ("attention 机制详解：KDA") states
 * its readout identity for unit keys and bounds the log-decay below with a
 * scaled sigmoid (g_min = -5, so each step keeps more than e^-5 of the state).
 *   l2norm_qk   : nonzero: q <- q / sqrt(sum q^2 + l2norm_eps) and k likewise,
 *                 per token and head, in fp32 (the scale argument then
 *                 multiplies the normalised q).
 *   l2norm_eps  : finite, >= 0 (read when l2norm_qk is set); 1e-6 is usual.
 *   gate_logits : nonzero: the g buffer holds gate logits x, and the
 *                 log-decay used is g_min * sigmoid(x) (a reading of the
 *                 page's scaled sigmoid: its orientation is not printed).
 *   g_min       : finite, < 0 (read when gate_logits is set).
 * The *_prologue entry points below take the arguments of their plain
 * counterparts plus `prologue` (required); KDA_ERR_INVALID_ARG for a NULL
 * prologue or a value outside the ranges above.  A verify and the commit that
 * follows it must use the same prologue: the commit then reproduces, bit for
 * bit, the state of as many prologue decode steps.
 */
typedef struct kda_prologue {
  int32_t l2norm_qk;
  float l2norm_eps;
  int32_t gate_logits;
  float g_min;
} kda_prologue_t;

kda_status_t kda_decode_step_prologue(const void* q, const void* k, const void* v, const float* g,
                                      const float* beta, float* state_pool, const int32_t* slots, int32_t N,
                                      int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype, float scale, void* o,
                                      const kda_prologue_t* prologue, void* stream);

kda_status_t kda_verify_block_prologue(const void* q, const void* k, const void* v, const float* g,
                                       const float* beta, const float* state_pool, const int32_t* slots,
                                       int32_t N, int32_t gamma1, int32_t H, int32_t d_k, int32_t d_v,
                                       kda_dtype_t dtype, float scale, void* o, const int32_t* accepted_len,
                                       float* state_out_pool, const kda_prologue_t* prologue, void* stream);

kda_status_t kda_verify_commit_prologue(const void* k, const void* v, const float* g, const float* beta,
                                        float* state_pool, const int32_t* slots, const int32_t* accepted_len,
                                        int32_t N, int32_t gamma1, int32_t H, int32_t d_k, int32_t d_v,
                                        kda_dtype_t dtype, const kda_prologue_t* prologue, void* stream);

/*
 * The raw-input record of a verify ("SGLang 和 Miles 为 Kimi K3 提供首日支持",
 * section "ReplaySSM：针对 KDA 状态的原始输入重放": the verify keeps each draft
 * step's inputs, about 1 KB per step, instead of a state snapshot, and the
 * fold replays the accepted prefix from what it kept).
 *
 * kda_verify_block_record — kda_verify_block_prologue (no fused commit) that
 * also writes, for every request n, draft step t and head h, the key and the
 * log-decay the verify used after the prologue: record [N, gamma1, H, 2, 128]
 * fp32 (device, 16-byte aligned, caller-owned), [n, t, h, 0, :] the key
 * (normalised when l2norm_qk is set), [n, t, h, 1, :] the log-decay (mapped
 * from the logit when gate_logits is set).  record is required
 * (KDA_ERR_INVALID_ARG if NULL or misaligned); other arguments and errors as
 * kda_verify_block_prologue.
 *
 * kda_verify_commit_record — the commit of the accepted prefix that folds the
 * recorded keys and log-decays (no prologue, no recomputation) with v and
 * beta as given ([N, gamma1, H, 128] in `dtype`, [N, gamma1, H] fp32), in
 * place on state_pool; accepted_len as kda_verify_commit.  The state it
 * writes is bit-identical to kda_verify_commit_prologue's with the verify's
 * prologue, and so to as many prologue decode steps.
 */
kda_status_t kda_verify_block_record(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                    const float* state_pool, const int32_t* slots, int32_t N, int32_t gamma1,
                                    int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype, float scale, void* o,
                                    float* record, const kda_prologue_t* prologue, void* stream);

kda_status_t kda_verify_commit_record(const float* record, const void* v, const float* beta, float* state_pool,
                                      const int32_t* slots, const int32_t* accepted_len, int32_t N, int32_t gamma1,
                                      int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype, void* stream);

/*
 * kda_prefill — chunk-parallel prefill of a packed ragged batch.
 *
 * Computes, for every sequence n (tokens cu_seqlens[n] .. cu_seqlens[n+1]-1)
 * and head h, exactly the token-by-token recurrence above, from its initial
 * state, with chunks of 64 tokens that restart at every sequence start (the
 * chunkwise form rescales keys by the inverse cumulative decay, as the KDA
 * math box of the Day-0 lesson page describes).
 *   q, k, g : [T_total, H, 128];  v : [T_total, H, 128];  beta : [T_total, H]
 *   cu_seqlens      : device int32 [num_seqs + 1], non-decreasing, cu_seqlens[0] >= 0;
 *                     row n covers tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 of the
 *                     packed arrays (a row set need not start at token 0).
 *   cu_seqlens_host : optional host copy of the same array; when given it is
 *                     validated (non-negative start, non-decreasing).  The device
 *                     array is trusted to hold the same values.
 *   initial_state : [num_seqs, H, 128, 128] fp32, or NULL for zeros.
 *   final_state   : [num_seqs, H, 128, 128] fp32, or NULL; may alias initial_state.
 *   o             : [T_total, H, 128] in `dtype`, or NULL to skip outputs.
 *   transition_out: [num_seqs, H, 128, 128] fp32, or NULL.  When given, it
 *                   receives each sequence's transition M = M_T ... M_1 with
 *                   M_t = (I - beta_t k_t k_t^T) Diag(alpha_t), so that
 *                   final = M initial + S~ ("Kimi K3 的训练与 Serving Infra",
 *                   section 4.2, KCP fragments).
 * Empty sequences pass their initial state through.
 * Precondition on the gates: -5 <= g <= 0 in every channel, the lower bound
 * on log-decay that the KDA math box prints (its scaled sigmoid keeps g above
 * g_min = -5).  The chunk products rescale by exp(+-(b_r - b_s)) over at most
 * 16 tokens of cumulative decay, which stays inside fp32 range only under
 * that bound; gates below it are not checked (they live in device memory) and
 * can overflow to inf/NaN.  The row contract (kda_contract_*) has no such
 * bound.
 */
kda_status_t kda_prefill(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H, int32_t d_k,
                         int32_t d_v, kda_dtype_t dtype, float scale, const float* initial_state,
                         float* final_state, void* o, float* transition_out, void* stream);

/*
 * kda_prefill_workspace_size — bytes of device workspace kda_prefill_ex can use
 * for a call with num_seqs sequences within T_total packed tokens (every
 * cu_seqlens value <= T_total) and H heads; flags say what the call requests:
 *   KDA_PREFILL_TRANSITIONS  transition_out is given;
 *   KDA_PREFILL_NO_OUTPUT    o is NULL.
 * 0 means the call takes the single-kernel path and needs none: that is the
 * case when the split path's walk, num_seqs * H (sequence, head) workgroups
 * (twice that when both outputs and transitions are requested), already fills
 * the device's compute units.  Sizes: one operand set (58,368 bytes, for bf16
 * and fp32 inputs alike) per 32-token chunk slot and head,
 * T_total / 32 + num_seqs + 1 slots.  Returns 0 for invalid arguments
 * (unknown flag bits included).
 */
#define KDA_PREFILL_TRANSITIONS 1
#define KDA_PREFILL_NO_OUTPUT 2
size_t kda_prefill_workspace_size(int32_t num_seqs, int64_t T_total, int32_t H, int32_t d_k, int32_t d_v,
                                  kda_dtype_t dtype, int32_t flags);

/*
 * kda_prefill_ex — kda_prefill with every option: seq_order (as
 * kda_prefill_ordered, or NULL), prologue (as kda_prefill_prologue, or NULL)
 * and a caller-owned device workspace of workspace_bytes bytes (or NULL).
 *
 * With a workspace, a grid smaller than the device takes the split path
 * (the same chunk form, "Kimi K3：架构与 SGLang Day-0 Support", KDA math box;
 * the per-chunk factors do not depend on the state, so they are formed for all
 * chunks at once): one launch prepares every 32-token chunk's operands (decay
 * prefix, rescaled keys and queries, the Gram tiles and the UT factor) in
 * parallel into the workspace, then the walk over each sequence's chunks runs
 * only the state products.  Results are bit-identical to the single-kernel
 * path.  The workspace then needs cu_seqlens_host (KDA_ERR_INVALID_ARG
 * without it) and at least kda_prefill_workspace_size(...) bytes for this
 * call's cu_seqlens_host[num_seqs] (KDA_ERR_WORKSPACE if smaller).  Its
 * contents are scratch: nothing is kept between calls, and calls that share
 * a workspace must not overlap.  Without a workspace, or for grids that fill
 * the device, the call is kda_prefill's single kernel.
 */
kda_status_t kda_prefill_ex(const void* q, const void* k, const void* v, const float* g, const float* beta,
                            const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H,
                            int32_t d_k, int32_t d_v, kda_dtype_t dtype, float scale, const float* initial_state,
                            float* final_state, void* o, float* transition_out, const int32_t* seq_order,
                            const kda_prologue_t* prologue, void* workspace, size_t workspace_bytes,
                            int32_t ws_flags, void* stream);

/* ws_flags of kda_prefill_ex (0 for a self-contained call).  They let two
 * calls over the same rows share one preparation, as the two passes of a
 * segmented prefill do (their state walks differ; the chunks' operands do
 * not):
 *   KDA_WS_KEEP_OUTPUT_OPERANDS  prepare the output operands (rescaled queries,
 *                                the query-key Gram tiles) even though this
 *                                call writes no outputs, so that a later
 *                                KDA_WS_PREPARED call can;
 *   KDA_WS_PREPARED              skip the preparation: the workspace holds the
 *                                operand sets an earlier split-path call wrote
 *                                for the same q, k, g, beta, cu_seqlens,
 *                                prologue and scale (with outputs'
 *                                operands if this call writes outputs), and
 *                                nothing has overwritten it since.  The
 *                                library cannot check this precondition.
 * Both only matter on the split path; KDA_ERR_INVALID_ARG for other bits. */
#define KDA_WS_PREPARED 1
#define KDA_WS_KEEP_OUTPUT_OPERANDS 2

/*
 * kda_prefill_noalloc — kda_prefill_ex for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * device allocation): the same arguments without the workspace, which is
 * instead a scratch array the library holds on each device (allocated when
 * the library is loaded on it, kept until the process ends; its size is
 * kda_prefill_noalloc_max_scratch(), 128 MiB).  The call allocates and frees
 * nothing, host or device.  A call whose split path would need more than that
 * (more than about 128 MiB / (58,368 * H) chunk slots of 32 tokens, e.g.
 * 4,096 tokens x 12 heads uses 91 MB) returns KDA_ERR_WORKSPACE; grids that
 * fill the device, and calls without cu_seqlens_host, need no scratch and run
 * the single kernel.  Results are bit-identical to kda_prefill_ex's.
 * Every call on one device shares that device's scratch and finds the last
 * call's contents in it (nothing needs clearing: each call writes every part
 * it reads first), so calls that overlap in time on one device — on
 * different streams, or from different host threads — race; serialise them.
 * The first call on a device looks the array's address up (hipGetSymbolAddress)
 * and KDA_ERR_HIP reports a failed lookup.
 */
kda_status_t kda_prefill_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs,
                                 int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype, float scale,
                                 const float* initial_state, float* final_state, void* o, float* transition_out,
                                 const int32_t* seq_order, const kda_prologue_t* prologue, void* stream);

/* Bytes of the per-device scratch kda_prefill_noalloc uses (the largest workspace it can serve). */
size_t kda_prefill_noalloc_max_scratch(void);

/*
 * kda_prefill_prologue — kda_prefill on raw inputs: the input prologue
 * (kda_prologue_t above) is applied to q, k and g of every token before the
 * chunk computation.  Same arguments and results as kda_prefill, plus
 * `prologue` (required; KDA_ERR_INVALID_ARG for NULL or out-of-range values).
 */
kda_status_t kda_prefill_prologue(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                  int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype,
                                  float scale, const float* initial_state, float* final_state, void* o,
                                  float* transition_out, const kda_prologue_t* prologue, void* stream);

/*
 * kda_prefill_ordered — kda_prefill with a caller-chosen order in which the
 * sequences' workgroups are started.  A prefill walks each sequence's chunks
 * in order, so a batch runs as long as its last-started long sequence: with
 * more (sequence, head) units than compute units, starting the longest first
 * (as when the segments of cut sequences run beside whole ones,
 * "Kimi K3 的训练与 Serving Infra", section 4.2) shortens the tail.  Results
 * are those of kda_prefill, bit for bit, for any order.
 *   seq_order : device int32 [num_seqs], required: a permutation of
 *               0 .. num_seqs - 1; entry i is the sequence started i-th.
 *               Entries outside that range are skipped (that sequence is then
 *               not computed); a repeated entry computes its sequence twice,
 *               racing on its outputs.
 * Errors: KDA_ERR_INVALID_ARG for a NULL seq_order, otherwise as kda_prefill.
 */
kda_status_t kda_prefill_ordered(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const int32_t* cu_seqlens,
                                 const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H, int32_t d_k,
                                 int32_t d_v, kda_dtype_t dtype, float scale, const float* initial_state,
                                 float* final_state, void* o, float* transition_out, const int32_t* seq_order,
                                 void* stream);

/*
 * kda_prefill_checkpointed — kda_prefill that also stores the state at chunk
 * boundaries, for restoring a prefix later (prefix caching / copy-on-write
 * restore of a state, as the serving pages describe for KDA's fixed-size
 * state).  Same arguments and results as kda_prefill, without transitions, plus:
 *   ckpt_interval : positive multiple of 64 (checkpoints fall on chunk ends).
 *   checkpoints   : [n_ckpt, H, 128, 128] fp32, required.  For sequence n of
 *                   length L and m = 1, 2, ... with m * ckpt_interval < L, row
 *                   base(n) + m - 1 receives the state after the sequence's
 *                   first m * ckpt_interval tokens (from its initial state),
 *                   where base(n) sums floor((L' - 1) / ckpt_interval) over the
 *                   earlier sequences.  kda_prefill_checkpoint_count gives n_ckpt.
 * Errors: KDA_ERR_INVALID_ARG for a missing buffer or a bad interval, otherwise
 * as kda_prefill.
 */
kda_status_t kda_prefill_checkpointed(const void* q, const void* k, const void* v, const float* g,
                                      const float* beta, const int32_t* cu_seqlens,
                                      const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H, int32_t d_k,
                                      int32_t d_v, kda_dtype_t dtype, float scale, const float* initial_state,
                                      float* final_state, void* o, int32_t ckpt_interval, float* checkpoints,
                                      void* stream);

/*
 * kda_prefill_checkpoint_count — number of checkpoint rows kda_prefill_checkpointed
 * writes for this batch (host only; reads cu_seqlens_host [num_seqs + 1]).
 * Returns -1 for a bad interval, a NULL array or a decreasing cu_seqlens_host.
 */
int64_t kda_prefill_checkpoint_count(const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t ckpt_interval);

/*
 * kda_compose_segments — entry states of consecutive segments of one sequence
 * from their fragments ("Kimi K3 的训练与 Serving Infra", section 4.2: after
 * exchanging the fixed-size fragments, a prefix scan recovers each segment's
 * true entry state):
 *     S_in[0] = S_in0;   S_in[i+1] = M[i] S_in[i] + S~[i]
 *   M       : [n_seg, H, 128, 128] fp32 (d_k x d_k transitions)
 *   S_tilde : [n_seg, H, 128, 128] fp32 (zero-entry states)
 *   S_in0   : [H, 128, 128] fp32, or NULL for zeros; may be the same memory as S_in[0]
 *   S_in    : [n_seg, H, 128, 128] fp32 output (may not alias M or S_tilde)
 *   S_final : [H, 128, 128] fp32 output M[n-1] S_in[n-1] + S~[n-1], or NULL
 */
kda_status_t kda_compose_segments(const float* M, const float* S_tilde, const float* S_in0,
                                  float* S_in, float* S_final, int32_t n_seg, int32_t H,
                                  int32_t d_k, int32_t d_v, void* stream);

/*
 * kda_compose_segments_ex — kda_compose_segments with flags (0: the same call):
 *   KDA_COMPOSE_SPLIT_BF16  run each step's products on bf16 MFMA with both
 *                           operands split as x = hi + lo (hi = bf16(x),
 *                           lo = bf16(x - hi); hi*hi + hi*lo + lo*hi, fp32
 *                           accumulation): about 16 significant bits per
 *                           operand instead of exact fp32 products, at several
 *                           times the matrix rate.  The precision class of the
 *                           chunked prefill's own products on bf16 inputs;
 *                           results are deterministic but differ in the last
 *                           bits from the fp32 scan.
 * Errors as kda_compose_segments; KDA_ERR_INVALID_ARG for other flag bits.
 */
#define KDA_COMPOSE_SPLIT_BF16 1
kda_status_t kda_compose_segments_ex(const float* M, const float* S_tilde, const float* S_in0,
                                     float* S_in, float* S_final, int32_t n_seg, int32_t H,
                                     int32_t d_k, int32_t d_v, int32_t flags, void* stream);

/*
 * Batch-invariant row contract ("Kimi K3.1 Pro" inference / zero-mismatch
 * article, LLMNews 2026-11-05, section 6.1 on KDA): prefill and decode share
 * one per-row computation, so a token's output and the stored state are
 * bit-identical whichever call (prefill of any length, decode step) and
 * whatever batch computed it.  The state of a (slot, head) is not the running
 * S_t but the state at the entry of the open 16-token chunk plus that chunk's
 * rows; a chunk closes (folds its rows into the entry state) when its 16th
 * row is written.
 *   S_pool    : [P, H, 128, 128] fp32, chunk-entry states (rows = key channels).
 *   rows_pool : [P, H, 16, 3, 128] fp32; row s of the open chunk holds its key
 *               k_s, its cumulative log-decay b_s = g_0 + ... + g_s since the
 *               chunk entry, and its delta-write vector u_s.
 *   pos_pool  : [P, H] int32, rows held (0 .. 15); read as pos & 15.
 *   slots     : device int32 [N] (pool row of request / sequence n), or NULL
 *               for the identity.  Two entries naming one slot race.
 * A fresh state is S_pool = S0 (zeros or any initial state) and pos_pool = 0;
 * rows_pool then needs no initialisation.  The pools are updated in place.
 * Each row's arithmetic is fp32 with one fixed order of operations; the
 * results equal the recurrence up to fp32 rounding (the chunk form, restated
 * per row), not bit for bit the kda_decode_step path.
 */

/*
 * kda_contract_prefill — run each sequence's tokens (cu_seqlens as in
 * kda_prefill; optional host copy validated) through the contract from its
 * slot's state.  o: [T_total, H, 128] in `dtype`, or NULL.  Empty sequences
 * leave their state unchanged.
 * Errors: KDA_ERR_INVALID_ARG for a NULL buffer or a bad cu_seqlens_host;
 * KDA_ERR_UNSUPPORTED for d != 128 or another dtype; KDA_ERR_HIP on a launch error.
 */
kda_status_t kda_contract_prefill(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                  int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype,
                                  float scale, float* S_pool, float* rows_pool, int32_t* pos_pool,
                                  const int32_t* slots, void* o, void* stream);

/*
 * kda_contract_prefill_split — kda_contract_prefill with the number of
 * workgroups that share each (sequence, head) fixed by the caller instead of
 * picked from the grid size and the device's compute-unit count:
 * split_width 1, 2 or 4 (each workgroup then holds 128 / split_width value
 * columns of the state), or 0 for the automatic choice.  Every width gives the
 * same bits (the row arithmetic is the same); a caller fixes it to reproduce a
 * launch shape, e.g. to compare widths on a part with another CU count.
 * Errors as kda_contract_prefill, and KDA_ERR_INVALID_ARG for another width.
 */
kda_status_t kda_contract_prefill_split(const void* q, const void* k, const void* v, const float* g,
                                        const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                        int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype,
                                        float scale, float* S_pool, float* rows_pool, int32_t* pos_pool,
                                        const int32_t* slots, void* o, int32_t split_width, void* stream);

/*
 * kda_contract_prefill_ex — kda_contract_prefill_split with a caller
 * workspace for the split build (the automatic choice for grids of at most
 * half the compute units' worth of (sequence, head) units, or split_width 2 or
 * 4).  Every full 16-token chunk of the call, from the chunk grid of its
 * slot's position, depends on the inputs alone for its decays, rescaled keys
 * and queries, Gram entries and close factors; with a workspace these are
 * formed chunk-parallel by a first kernel and read by the walk instead of
 * formed inside it, with the same functions, so the results are bit-identical
 * to kda_contract_prefill's.
 *   workspace : device memory of kda_contract_prefill_workspace_size(T_total, H)
 *               bytes (T_total = cu_seqlens_host[num_seqs]), caller-owned,
 *               overwritten; or NULL for kda_contract_prefill_split's behaviour.
 *               Not read by builds other than the split one.
 * Errors as kda_contract_prefill_split; with a workspace, KDA_ERR_INVALID_ARG
 * without cu_seqlens_host and KDA_ERR_WORKSPACE when workspace_bytes is
 * smaller than the size above.
 */
size_t kda_contract_prefill_workspace_size(int64_t T_total, int32_t H);
kda_status_t kda_contract_prefill_ex(const void* q, const void* k, const void* v, const float* g,
                                     const float* beta, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                     int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype,
                                     float scale, float* S_pool, float* rows_pool, int32_t* pos_pool,
                                     const int32_t* slots, void* o, int32_t split_width, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * kda_contract_decode — one token per request (inputs laid out as for
 * kda_decode_step: q, k, g [N, H, 128], v [N, H, 128], beta [N, H]) through the
 * contract; o: [N, H, 128] in `dtype`, or NULL.  Reads the entry state and the
 * open rows, appends one row, and writes the entry state only when the row
 * closes the chunk.  Errors as kda_contract_prefill.
 */
kda_status_t kda_contract_decode(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                                 kda_dtype_t dtype, float scale, float* S_pool, float* rows_pool,
                                 int32_t* pos_pool, const int32_t* slots, void* o, void* stream);

/*
 * kda_contract_verify — score gamma1 draft tokens per request under the
 * contract, from the request's contract state, which is only READ (the
 * ReplaySSM verify of "SGLang 和 Miles 为 Kimi K3 提供首日支持", section
 * "ReplaySSM：针对 KDA 状态的原始输入重放", on the row contract of the K3.1
 * zero-mismatch article, section 6.1).
 *   q, k, g, v : [N, gamma1, H, 128];  beta : [N, gamma1, H];  o : [N, gamma1, H, 128]
 * o[n, t] is bit-identical to the output of the (t+1)-th of t+1 successive
 * kda_contract_decode calls on that state.  gamma1 >= 1 (any length; a chunk
 * that fills up on the way is closed in registers only).
 *   stash : NULL, or fp32 [N, H, gamma1 * 3 * 128 + 128 * 128] (caller-owned):
 *           receives each draft's row (k, cumulative log-decay, u) and, when
 *           the drafts fill the open chunk, the chunk-entry state after that
 *           close — what kda_contract_commit_stash needs.  Requires gamma1 <= 16.
 */
kda_status_t kda_contract_verify(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, int32_t N, int32_t gamma1, int32_t H, int32_t d_k,
                                 int32_t d_v, kda_dtype_t dtype, float scale, const float* S_pool,
                                 const float* rows_pool, const int32_t* pos_pool, const int32_t* slots, void* o,
                                 float* stash, void* stream);

/*
 * kda_contract_commit_stash — the commit of kda_contract_commit, from the stash
 * a kda_contract_verify call (same N, gamma1, H, slots, and the pools unchanged
 * since) filled: the accepted draft rows, and the closed entry state when they
 * reach the chunk end, are copied into the pools.  Bit-identical to
 * kda_contract_commit and to that many kda_contract_decode calls, without
 * re-reading the entry state or the inputs.  accepted_len: device int32 [N],
 * clamped to 0 .. gamma1.  Errors: KDA_ERR_INVALID_ARG for a NULL buffer or
 * gamma1 outside 1 .. 16; KDA_ERR_UNSUPPORTED for d != 128.
 */
kda_status_t kda_contract_commit_stash(const float* stash, const int32_t* accepted_len, int32_t N, int32_t gamma1,
                                       int32_t H, int32_t d_k, int32_t d_v, float* S_pool, float* rows_pool,
                                       int32_t* pos_pool, const int32_t* slots, void* stream);

/*
 * kda_contract_commit — apply the first accepted_len[n] of request n's gamma1
 * tokens (the inputs the verify saw, same layout) to its contract state, in
 * place; bit-identical to that many kda_contract_decode calls.  q may be NULL
 * (no outputs are formed).  accepted_len: device int32 [N], clamped to
 * 0 .. gamma1 (0 leaves the state unchanged).  Errors as kda_contract_prefill.
 */
kda_status_t kda_contract_commit(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const int32_t* accepted_len, int32_t N, int32_t gamma1,
                                 int32_t H, int32_t d_k, int32_t d_v, kda_dtype_t dtype, float* S_pool,
                                 float* rows_pool, int32_t* pos_pool, const int32_t* slots, void* stream);

/*
 * kda_contract_state — the running state S_t of N contract states:
 *   S_t = Diag(e^{b_last}) S_e + sum_{s < pos} (k_s e^{b_last - b_s}) u_s^T
 * (the chunk close applied to the rows held, which stay unchanged), into
 * state_out [N, H, 128, 128] fp32, e.g. to hand a sequence over to
 * kda_decode_step.  Errors as kda_contract_prefill.
 */
kda_status_t kda_contract_state(const float* S_pool, const float* rows_pool, const int32_t* pos_pool,
                                const int32_t* slots, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                                float* state_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
