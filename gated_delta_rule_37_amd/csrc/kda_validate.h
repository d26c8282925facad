// Host-side argument validation of the C ABI's device calls (kda_validate.cpp).
// Each check returns KDA_OK or the kda_status the entry point returns; the
// checks run in the order the header of the C ABI states.
#ifndef KDA_VALIDATE_H_
#define KDA_VALIDATE_H_

#include <cstddef>
#include <cstdint>

#include "kda_internal.h"

namespace kda {

// The forward's workspace for H heads: the chunk cache (256-byte aligned),
// then, for a plan with pieces, the pieces' transitions, updates and
// carry-ins (P x H states each).
struct PieceLayout {
  size_t transitions, updates, carry, total;
};
PieceLayout piece_layout(const kda_plan* plan, int32_t H);
size_t workspace_need(const kda_plan* plan, int32_t H);

// Byte offsets of the parts of the backward's workspace for H heads (each
// 256-byte aligned): the forward's workspace, the forward's transitions,
// updates and carry-ins recomputed, the backward summaries E and their
// reverse compose D (each P x H states, per piece), the state checkpoints
// ((floor(T/16) + F) x H states) and every token's u and p
// (T x H x 2 x 128 floats) of the token-by-token path; for the chunked path
// the anchored states and cotangents of every 32-token chunk
// ((ceil(T/32) + F) x H states each), every chunk's T diag(beta)
// ((ceil(T/32) + F) x H x 4 KB), every chunk's V - Kr R and dU
// ((ceil(T/32) + F) x H x 16 KB each), the fragments' path flags (F x H
// int32) and the chunk-slot-to-fragment map (ceil(T/32) + F int32).
struct BwdLayout {
  size_t cache, transitions, updates, carry, esum, dcarry, ckpt, up, ck32, dcot, tcache, rv, du, iflag, smap, total;
};
// Chunk slots of the chunked backward: chunk c of fragment f at
// floor(begin_f / 32) + f + c, below ceil(T / 32) + F.
size_t backward_chunk_slots(const kda_plan* plan);
BwdLayout backward_layout(const kda_plan* plan, int32_t H);
size_t backward_workspace_need(const kda_plan* plan, int32_t H);

// Plan, plan_dev and dimensions (K = V = 128, 0 < H <= 65535).
int check_dims(const kda_plan* plan, const int32_t* plan_dev, int32_t H, int32_t K, int32_t V);

// The optional safe-gate lower bound: <= 0 or -inf (not NaN).
int check_gate_bound(float gate_lower_bound);

int check_summaries(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                    const uint16_t* k, size_t k_bytes, const uint16_t* v, size_t v_bytes,
                    const uint16_t* g, size_t g_bytes, const uint16_t* beta, size_t beta_bytes,
                    float gate_lower_bound, const float* initial_state, size_t initial_state_bytes, int32_t H, int32_t K,
                    int32_t V, int32_t head_begin, int32_t head_count, const float* transitions,
                    size_t transitions_bytes, const float* updates, size_t updates_bytes,
                    const void* workspace, size_t workspace_bytes);

int check_compose(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                  const float* transitions, size_t transitions_bytes, const float* updates,
                  size_t updates_bytes, int32_t H, int32_t K, int32_t V, int32_t head_begin,
                  int32_t head_count, const float* carry_in, size_t carry_in_bytes);

int check_carry(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                const uint16_t* beta, size_t beta_bytes, float gate_lower_bound,
                const float* initial_state, size_t initial_state_bytes, int32_t H, int32_t K,
                int32_t V, int32_t head_begin, int32_t head_count, const float* carry_in, size_t carry_in_bytes, const void* o,
                size_t o_bytes, int32_t o_format, const float* final_state, size_t final_state_bytes,
                const void* workspace, size_t workspace_bytes);

int check_backward(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                   const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                   const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                   const uint16_t* beta, size_t beta_bytes, const float* initial_state,
                   size_t initial_state_bytes, const float* d_o, size_t d_o_bytes, const float* d_final,
                   size_t d_final_bytes, int32_t H, int32_t K, int32_t V, int32_t head_begin,
                   int32_t head_count, const float* dq, size_t dq_bytes, const float* dk, size_t dk_bytes,
                   const float* dv, size_t dv_bytes, const float* dg, size_t dg_bytes, const float* dbeta,
                   size_t dbeta_bytes, const float* d_initial_state, size_t d_initial_state_bytes,
                   const void* workspace, size_t workspace_bytes);

}  // namespace kda

#endif  // KDA_VALIDATE_H_
