/*
 * kda.h -- C ABI of the segmented KDA (Kimi Delta Attention) forward pass on
 * MI355X (gfx950).
 *
 * The method (sources: inclusionAI/cuLA pull request #110 "feat(cp): add
 * opt-in NVSHMEM CP state handoff", and pull request #136 "feat(kda): add
 * cuDNN concatenated-summary Kimi CP"):
 *
 *   per head, with a K x V state S (FP32, K-major "non-transposed" layout,
 *   #110 Supported configuration) and BF16 inputs (#110 Supported
 *   configuration), the gated delta rule
 *       S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *       o_t = S_t^T q_t
 *   runs over packed sequences (THD layout with cu_seqlens, #136 Summary by
 *   CodeRabbit).  The token range is cut into contiguous segments (the
 *   context-parallel shards of #136 Walkthrough, "Packed-shard planning").
 *   Each segment r yields an affine FP32 summary S_out = A_r S_in + B_r: the
 *   K x K transition A_r and the K x V update B_r (#136 Summary:
 *   preceding_transition / preceding_state_update; #110 Motivation: affine
 *   recurrence state).  An ordered FP32 scan composes them into carry-in
 *   states C_r (#136 Summary: affine summary composition in FP32), and the
 *   forward runs every segment from its carry-in, writing o and the final
 *   states (#136 Sequence Diagram: the forward consumes the gathered
 *   preceding summaries).
 *
 * Call order for one forward pass, all on one stream:
 *     kda_plan_segments        (host, once; reusable)
 *     kda_segment_summaries    (device)
 *     kda_compose_summaries    (device)
 *     kda_apply_carry          (device)
 * (or kda_forward, which enqueues the three device calls at once).  After
 * them, o and final_state hold the monolithic recurrence's results.
 *
 * Conventions shared by every entry point:
 *   - Return value: KDA_OK (0) or a negative kda_status.  Every check runs on
 *     the host before anything is enqueued; on error nothing is enqueued and
 *     no output is touched.  There is no fallback path of any kind.
 *   - Device pointers are plain device addresses owned by the caller; the
 *     library never allocates or frees device memory and keeps no global
 *     state, apart from the fixed per-GPU workspace array of
 *     kda_forward_noalloc.  Distinct plans may be used from distinct threads.
 *   - BF16 tensors are passed as their raw 16-bit patterns (uint16_t).
 *   - Tensors are dense and contiguous; every tensor pointer must be 16-byte
 *     aligned (KDA_ERR_MISALIGNED otherwise).
 *   - Shapes: T packed tokens, N sequences, S segments, H heads, K = V = 128
 *     (other K, V return KDA_ERR_UNSUPPORTED).
 *       q, k, g : [T, H, K] bf16        v : [T, H, V] bf16
 *       beta    : [T, H]    bf16
 *       o       : [T, H, V] fp32 (or bf16, see kda_o_format)
 *       final_state : [N, H, K, V] fp32
 *       initial_state : [N, H, K, V] fp32, or NULL (every sequence starts at 0)
 *       transitions : [S, H, K, K] fp32 updates / carry_in : [S, H, K, V] fp32
 *       workspace : kda_workspace_bytes(plan, H, K, V) bytes of device memory
 *   - Initial states: sequence n starts from initial_state[n] (the reading
 *     that a sequence start resets the state to the sequence's own initial
 *     state, zero when none is given).  Pass the same initial_state, or NULL
 *     to both, to kda_segment_summaries and kda_apply_carry.
 *   - Head range: each device call works on the heads [head_begin,
 *     head_begin + head_count) of tensors that hold H heads, and touches no
 *     other head's data (outputs included).  Heads are independent, so the
 *     three calls may be issued per head group, and the compose of one group
 *     may run on another stream while the next group's summaries run; the
 *     caller orders the calls of one group (summaries, compose, carry).
 *     head_begin < 0, head_count < 1 or head_begin + head_count > H gives
 *     KDA_ERR_INVALID_ARG.
 *   - Device calls are asynchronous on `stream`; launch failures are reported
 *     as KDA_ERR_HIP (kda_last_hip_error() gives the hipError_t).
 *   - Gate domain: every g <= 0, finite or -inf (exp(-inf) = 0 forgets the
 *     channel).  The chunked (anchored) form is exact only while every
 *     in-chunk decay factor of a 32-token chunk stays within 2^+-96: per
 *     channel, the decay from the chunk's start to its anchor (token 15) and
 *     from the anchor to the chunk's end both below 96 log2 units (66.5
 *     nats).  Each launch checks that on the device; a fragment with any
 *     chunk beyond it is run again from its starting state one token at a
 *     time in FP32 (the same launch, no host involvement; slower but exact
 *     for any such input).  g > 0 or NaN is outside the method's domain.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = -1,    /* null pointer, non-positive size, plan_dev missing */
  KDA_ERR_BAD_CU_SEQLENS = -2, /* cu_seqlens not 0 = c_0 < c_1 < ... (empty sequence) */
  KDA_ERR_BAD_SEGMENTS = -3,   /* num_segments outside [1, T] or bad custom bounds */
  KDA_ERR_UNSUPPORTED = -4,    /* K or V other than 128, H > 65535, T > 2^30 */
  KDA_ERR_MISALIGNED = -5,     /* a tensor pointer is not 16-byte aligned */
  KDA_ERR_HIP = -6,            /* a HIP launch failed; see kda_last_hip_error() */
  KDA_ERR_NO_MEMORY = -7,      /* host allocation for the plan failed */
  KDA_ERR_WORKSPACE_TOO_SMALL = -8, /* workspace_bytes < kda_workspace_bytes(plan, H, K, V) */
  KDA_ERR_BUFFER_TOO_SMALL = -9     /* another device buffer is smaller than its shape */
} kda_status;

/* Storage format of o (kda_apply_carry, kda_forward).  The recurrence runs in
 * FP32 either way; KDA_O_BF16 stores each element rounded to the nearest
 * bfloat16 (ties to even), which halves the output bytes.  The pages fix BF16
 * inputs and an FP32 state ([#110] Supported configuration) but not o's
 * storage. */
typedef enum kda_o_format {
  KDA_O_FP32 = 0,
  KDA_O_BF16 = 1
} kda_o_format;

/* Opaque host-side plan; immutable once built. */
typedef struct kda_plan kda_plan;

/*
 * kda_plan_segments -- contiguous segment plan over packed sequences.
 * #136 Walkthrough ("Packed-shard planning": CPU-only, balanced or custom
 * contiguous shards over the global sequence boundaries, validated).
 *
 *   cu_seqlens    host [num_seqs + 1]; must satisfy 0 = c_0 < c_1 < ... < c_N = T.
 *   num_seqs      N >= 1.
 *   num_segments  S with 1 <= S <= T.
 *   custom_bounds host [S + 1] with 0 = b_0 < ... < b_S = T, or NULL for the
 *                 balanced bounds b_r = floor(r * T / S).
 *   out           receives the plan (owned by the caller; free with
 *                 kda_plan_destroy).  Untouched on error.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_BAD_CU_SEQLENS, KDA_ERR_BAD_SEGMENTS,
 * KDA_ERR_UNSUPPORTED (T > 2^30 tokens), KDA_ERR_NO_MEMORY.
 */
int kda_plan_segments(const int32_t* cu_seqlens, int32_t num_seqs, int32_t num_segments,
                      const int32_t* custom_bounds, kda_plan** out);

/*
 * kda_plan_segments_pieces -- the same plan, with every segment cut into
 * pieces of piece_tokens tokens from its start (the last one shorter) that
 * the device calls run in parallel.  This fills the GPU where segments x
 * heads are few (#136 Walkthrough: balanced contiguous shards); every call's
 * results stay per segment (kda_segment_summaries folds the pieces'
 * summaries into the segment's, kda_apply_carry scans the pieces' carry-ins
 * from the segment's), and kda_workspace_bytes grows by 3 * P * H states of
 * 64 KiB for the pieces' summaries and carry-ins.  piece_tokens = 0 is
 * kda_plan_segments; otherwise it must be a multiple of 32
 * (KDA_ERR_BAD_SEGMENTS).  Other arguments and errors as kda_plan_segments.
 */
int kda_plan_segments_pieces(const int32_t* cu_seqlens, int32_t num_seqs, int32_t num_segments,
                             const int32_t* custom_bounds, int32_t piece_tokens, kda_plan** out);

/* The plan's piece count P (S when it has no pieces). */
int kda_plan_pieces(const kda_plan* plan, int32_t* P);

/*
 * kda_plan_blob -- the plan's canonical int32 serialisation.  The device
 * entry points read a device copy of exactly these n_int32 words
 * (`plan_dev`, n_int32 * 4 bytes).  Layout:
 *   header [T, N, S, F]
 *   seg_bounds[S+1] seg_first_seq[S] seg_last_seq[S] seg_carry_in[S]
 *   seg_transition_live[S] seg_frag_ptr[S+1]
 *   frag_seq[F] frag_begin[F] frag_end[F] frag_seg[F] frag_flags[F]
 *   seq_end_seg[N] frag_order[F]
 * A fragment is the part of one sequence inside one segment.  frag_flags bit
 * 1: first fragment of a segment that continues a sequence (it carries in);
 * bit 2: ends at its segment's end; bit 4: ends at its sequence's end.
 * frag_order lists the fragments longest first (ties by index): the device
 * calls start them in that order, so that the longest sequential chains do
 * not start last (it changes no result).  In a plan with pieces (P > S) the
 * seg_* arrays above describe the P pieces (the header holds P in place of
 * S) and the blob ends with the segments' own block:
 *   S, useg_bounds[S+1], useg_carry_in[S], useg_transition_live[S],
 *   useg_piece_ptr[S+1] (segment r owns pieces [ptr[r], ptr[r+1])).
 * `*blob` stays valid until kda_plan_destroy.
 */
int kda_plan_blob(const kda_plan* plan, const int32_t** blob, size_t* n_int32);

/* Sizes of a plan: tokens, sequences, segments, fragments (any may be NULL). */
int kda_plan_info(const kda_plan* plan, int32_t* T, int32_t* N, int32_t* S, int32_t* F);

void kda_plan_destroy(kda_plan* plan);

/*
 * kda_summary_bytes -- bytes of the FP32 summary workspace (transitions plus
 * updates) for this plan: S * H * (K*K + K*V) * 4.  At S = 64, H = 32,
 * K = V = 128 this is 256 MiB, the figure #136 Latest cuDNN compatibility
 * gives for the prepared CP64 summary workspace.  Returns 0 for a NULL plan
 * or non-positive sizes.
 */
size_t kda_summary_bytes(const kda_plan* plan, int32_t H, int32_t K, int32_t V);

/*
 * kda_workspace_bytes -- bytes of the caller-owned device workspace that
 * kda_segment_summaries fills and kda_apply_carry reads (#136 Summary by
 * CodeRabbit: a reusable workspace; #136 Latest cuDNN compatibility:
 * workspace requirements are validated up front).
 * It holds, for every fragment that ends its segment, the per-chunk factor
 * T diag(beta) of the UT form of the recurrence (T = (I + A)^{-1},
 * A_ij = beta_i k_i^T Diag(exp(G_i - G_j)) k_j for j < i inside a 32-token
 * chunk), so that the carry pass does not rebuild it.  Its contents are
 * opaque: what kda_segment_summaries writes for a head is valid for
 * kda_apply_carry on the same plan, H, head and inputs.
 * Size: (ceil(T / 32) + P) * H * 4096 bytes (P = S without pieces); with
 * pieces (kda_plan_segments_pieces) rounded up to 256 bytes and followed by
 * the pieces' transitions, updates and carry-ins, 3 * P * H * 65536 bytes.
 * Returns 0 for a NULL plan, H <= 0, or K, V other than 128.
 */
size_t kda_workspace_bytes(const kda_plan* plan, int32_t H, int32_t K, int32_t V);

/*
 * Device calls: arguments shared by kda_segment_summaries,
 * kda_compose_summaries, kda_apply_carry and kda_forward.
 *   plan, plan_dev  the host plan and the caller's device copy of its blob.
 *   H, K, V         heads held by every tensor; K = V = 128.
 *   head_begin, head_count  the heads this call works on (see above).
 *   X, X_bytes      every device buffer X comes with the number of bytes
 *                   the caller allocated at X.  The call needs, for the
 *                   plan's T, N, S and the H heads of the layout:
 *                     plan_dev        n_int32 * 4
 *                     q, k, g         T * H * K * 2      v   T * H * V * 2
 *                     beta            T * H * 2
 *                     initial_state   N * H * K * V * 4  (when not NULL)
 *                     transitions     S * H * K * K * 4
 *                     updates, carry_in  S * H * K * V * 4
 *                     o               T * H * V * 4 (FP32) or * 2 (BF16)
 *                     final_state     N * H * K * V * 4
 *                     workspace       kda_workspace_bytes(plan, H, K, V)
 *                   A smaller workspace gives KDA_ERR_WORKSPACE_TOO_SMALL,
 *                   any other smaller buffer KDA_ERR_BUFFER_TOO_SMALL; in
 *                   both cases nothing is enqueued.
 *   gate_lower_bound  the optional safe gate (#136 Summary by CodeRabbit:
 *                   optional safe-gate parameters): the recurrence runs on
 *                   max(g, gate_lower_bound) per element, in nats.  -INFINITY
 *                   leaves g as given; a bound >= -4.4 keeps every chunk in
 *                   the anchored form's range (no fragment is re-run).  NaN or
 *                   a bound > 0 gives KDA_ERR_INVALID_ARG.  Pass the same bound
 *                   to kda_segment_summaries and kda_apply_carry.
 *   stream          the HIP stream every launch of the call is enqueued on.
 * Check order: plan and dimensions, head range, o_format and gate bound,
 * null pointers, alignment, sizes.
 */

/*
 * kda_segment_summaries -- the affine summary of every segment.
 * #136 Summary (preceding_state_update / preceding_transition), #110
 * Motivation (each producer computes its affine recurrence state).
 *
 * Writes:
 *   updates[r]      = B_r, the state at the end of segment r run from zero
 *                     (reset at each sequence start inside it to that
 *                     sequence's initial state);
 *   transitions[r]  = A_r, the product of the per-token maps of segment r,
 *                     latest on the left, when segment r carries in and no
 *                     sequence starts inside it; otherwise exactly 0 (the
 *                     reset's linear part);
 *   workspace       the chunk factors of every fragment that ends its
 *                   segment (kda_workspace_bytes).
 * It reads no q and writes no o or final state: kda_apply_carry does.
 */
int kda_segment_summaries(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                          const uint16_t* k, size_t k_bytes, const uint16_t* v, size_t v_bytes,
                          const uint16_t* g, size_t g_bytes, const uint16_t* beta, size_t beta_bytes,
                          float gate_lower_bound,
                          const float* initial_state, size_t initial_state_bytes,
                          int32_t H, int32_t K, int32_t V, int32_t head_begin, int32_t head_count,
                          float* transitions, size_t transitions_bytes,
                          float* updates, size_t updates_bytes,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_compose_summaries -- ordered FP32 scan C_0 = 0, C_{r+1} = A_r C_r + B_r.
 * #136 Summary (affine summary composition in FP32), #110 Motivation (a
 * consumer assembles the state from every predecessor in one kernel).
 * carry_in[r] is the state entering segment r (all r in [0, S)).  Where the
 * plan says A_r is structurally zero the product is skipped (C_{r+1} = B_r).
 */
int kda_compose_summaries(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                          const float* transitions, size_t transitions_bytes,
                          const float* updates, size_t updates_bytes,
                          int32_t H, int32_t K, int32_t V, int32_t head_begin, int32_t head_count,
                          float* carry_in, size_t carry_in_bytes, hipStream_t stream);

/*
 * kda_apply_carry -- the forward with the carry applied: every fragment (a
 * run of one sequence's tokens inside one segment) starts from its
 * segment's carry-in C_r when it continues a sequence, else from the
 * sequence's initial state (zero when initial_state is NULL), and
 * writes its rows of o and, when it ends a sequence, that sequence's
 * final_state.  Every row of o and every final state is written here.
 * #136 Summary (the forward that consumes
 * preceding_state_update / preceding_transition), #110 Motivation (rank 1
 * consumes only the V-state it needs).
 *   o            [T, H, V] in the format o_format names (kda_o_format; other
 *                values give KDA_ERR_INVALID_ARG): FP32, or BF16 bits.
 *   workspace    the buffer kda_segment_summaries filled for the same plan,
 *                H and inputs (read only).
 */
int kda_apply_carry(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                    const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                    const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                    const uint16_t* beta, size_t beta_bytes, float gate_lower_bound,
                    const float* initial_state, size_t initial_state_bytes,
                    int32_t H, int32_t K, int32_t V, int32_t head_begin, int32_t head_count,
                    const float* carry_in, size_t carry_in_bytes,
                    void* o, size_t o_bytes, int32_t o_format,
                    float* final_state, size_t final_state_bytes,
                    const void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_forward -- one whole forward pass: kda_segment_summaries,
 * kda_compose_summaries and kda_apply_carry over the same heads, enqueued in
 * that order on `stream` (#136 Sequence Diagram: plan, summaries, composition,
 * then the forward that consumes them).  Every argument means what it means
 * for those calls; all of them are checked before the first launch, so an
 * error enqueues nothing.  Results are bitwise those of the three calls.
 */
int kda_forward(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                const uint16_t* beta, size_t beta_bytes, float gate_lower_bound,
                const float* initial_state, size_t initial_state_bytes,
                int32_t H, int32_t K, int32_t V, int32_t head_begin, int32_t head_count,
                float* transitions, size_t transitions_bytes,
                float* updates, size_t updates_bytes,
                float* carry_in, size_t carry_in_bytes,
                void* o, size_t o_bytes, int32_t o_format,
                float* final_state, size_t final_state_bytes,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_forward_noalloc -- kda_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same checks and the same kernels, with the
 * workspace taken from a fixed array inside the library instead of an
 * argument.  Each GPU the library runs on holds one such array of
 * kda_noalloc_max_workspace_bytes() bytes (64 MiB) until the process ends;
 * the first call on a device looks its address up (hipGetSymbolAddress), and
 * no call allocates or frees anything.  A plan and head count whose
 * kda_workspace_bytes exceeds that size return KDA_ERR_WORKSPACE_TOO_SMALL
 * before anything else is checked or enqueued.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (on different streams, or
 * from different threads without ordering) race on it and must not be made.
 * Results are bitwise those of kda_forward.
 */
int kda_forward_noalloc(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                        const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                        const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                        const uint16_t* beta, size_t beta_bytes, float gate_lower_bound,
                        const float* initial_state, size_t initial_state_bytes,
                        int32_t H, int32_t K, int32_t V, int32_t head_begin, int32_t head_count,
                        float* transitions, size_t transitions_bytes,
                        float* updates, size_t updates_bytes,
                        float* carry_in, size_t carry_in_bytes,
                        void* o, size_t o_bytes, int32_t o_format,
                        float* final_state, size_t final_state_bytes, hipStream_t stream);

/* Bytes of the fixed workspace array kda_forward_noalloc uses on each GPU. */
size_t kda_noalloc_max_workspace_bytes(void);

/*
 * kda_backward -- gradients of the recurrence (#110 Correctness: output and
 * Q/K/V/g/beta gradients; #136 Sequence Diagram: the backward of the CP
 * forward).  For the loss
 *     L = sum_t <o_t, d_o_t> + sum_n <final_n, d_final_n>
 * of the forward over the same plan, inputs and initial states, it writes
 *   dq, dk, dg  [T, H, K] fp32    dv [T, H, V] fp32    dbeta [T, H] fp32
 *   d_initial_state [N, H, K, V] fp32 (optional: NULL when not wanted)
 * d_o [T, H, V] fp32 is required, d_final [N, H, K, V] fp32 optional (NULL =
 * zero).  g is the log-decay as given (no safe gate).  The segments of the
 * plan run in parallel, as in the forward (#136: the backward gathers the
 * following summaries): the call recomputes the forward's transitions and
 * carry-ins, forms each carried segment's backward summary E_r (the
 * cotangent at its start due to its first fragment's own outputs), scans
 * D_{r-1} = A_r^T D_r + E_r in reverse, and then works per 32-token chunk on
 * the matrix cores: the state entering every chunk (forward from its
 * carry-in), the cotangent leaving every chunk (backward from D_r), and every
 * chunk's gradients from those two.  A (fragment, head) whose gates leave the
 * chunk form's exponent range is reversed in FP32 one token at a time
 * instead.  Workspace: kda_backward_workspace_bytes(plan, H, K, V) bytes,
 * caller-owned, contents not needed afterwards.  Arguments, sizes and errors
 * as for the forward's device calls (each buffer with its byte count).
 */
int kda_backward(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                 const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                 const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                 const uint16_t* beta, size_t beta_bytes,
                 const float* initial_state, size_t initial_state_bytes,
                 const float* d_o, size_t d_o_bytes, const float* d_final, size_t d_final_bytes,
                 int32_t H, int32_t K, int32_t V, int32_t head_begin, int32_t head_count,
                 float* dq, size_t dq_bytes, float* dk, size_t dk_bytes,
                 float* dv, size_t dv_bytes, float* dg, size_t dg_bytes,
                 float* dbeta, size_t dbeta_bytes,
                 float* d_initial_state, size_t d_initial_state_bytes,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_backward_from_forward -- kda_backward for a caller that kept the
 * forward's segment transitions A_r and carry-ins C_r (`transitions` and
 * `carry_in` [S, H, K, V] fp32 as kda_forward, or kda_segment_summaries and
 * kda_compose_summaries, wrote them for this plan, these inputs and initial
 * states, and no gate lower bound): the call reads them instead of
 * recomputing them (it skips kda_backward's first two launches) and
 * otherwise does and returns exactly what kda_backward does.  Read only;
 * the heads [head_begin, head_begin + head_count) of both must be current.
 * A plan with pieces gives KDA_ERR_UNSUPPORTED: its backward works on the
 * pieces' own transitions, which the forward folds away.  Other arguments,
 * sizes, workspace and errors as kda_backward.
 */
int kda_backward_from_forward(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                              const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                              const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                              const uint16_t* beta, size_t beta_bytes,
                              const float* initial_state, size_t initial_state_bytes,
                              const float* d_o, size_t d_o_bytes, const float* d_final, size_t d_final_bytes,
                              int32_t H, int32_t K, int32_t V, int32_t head_begin, int32_t head_count,
                              const float* transitions, size_t transitions_bytes,
                              const float* carry_in, size_t carry_in_bytes,
                              float* dq, size_t dq_bytes, float* dk, size_t dk_bytes,
                              float* dv, size_t dv_bytes, float* dg, size_t dg_bytes,
                              float* dbeta, size_t dbeta_bytes,
                              float* d_initial_state, size_t d_initial_state_bytes,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of kda_backward's workspace for H heads (each part 256-byte
 * aligned): kda_workspace_bytes(plan, H); five arrays of P * H states
 * (transitions, updates, carry-ins, backward summaries and their reverse
 * compose, per piece; P = S without pieces); (floor(T/16) + F) * H state
 * checkpoints and T * H * 1 KiB (every token's u and p) for the
 * token-by-token path; per 32-token chunk slot (ceil(T/32) + F of them) and
 * head, a state and a cotangent (64 KiB each), the chunk's T (4 KiB) and two
 * [32, V] fp32 tiles (16 KiB each); F * H path flags and the slot map (int32).
 * A state is 64 KiB.  0 for a NULL plan, H <= 0 or K, V other than 128. */
size_t kda_backward_workspace_bytes(const kda_plan* plan, int32_t H, int32_t K, int32_t V);

/* Human-readable name of a kda_status value. */
const char* kda_status_string(int status);

/* hipError_t of the last KDA_ERR_HIP returned on this thread (0 if none). */
int kda_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
