// Host-side argument validation of the C ABI's device calls (no HIP calls):
// every check a device entry point makes before it enqueues anything.  Kept
// apart from the launch code so that it also builds with a host compiler
// (the sanitizer tests build it with g++ -fsanitize=address,undefined).
#include "kda_validate.h"

#include <cstdint>
#include <initializer_list>

#include "kda.h"
#include "kda_internal.h"

namespace kda {
namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_heads(int32_t H, int32_t head_begin, int32_t head_count) {
  if (head_begin < 0 || head_count <= 0 || head_count > H - head_begin) return KDA_ERR_INVALID_ARG;
  return KDA_OK;
}

// A device buffer of the call: its address, the bytes the caller has there
// and the bytes the call needs.  `optional` buffers may be null (then the
// size is not checked).
struct Buf {
  const void* ptr;
  size_t have;
  size_t need;
  bool optional;
};

// Null pointers first, then alignment, then sizes, so that each error is
// reported the same way whichever buffer has it.
int check_buffers(std::initializer_list<Buf> bufs) {
  for (const Buf& b : bufs) {
    if (b.ptr == nullptr && !b.optional) return KDA_ERR_INVALID_ARG;
  }
  for (const Buf& b : bufs) {
    if (b.ptr != nullptr && !aligned16(b.ptr)) return KDA_ERR_MISALIGNED;
  }
  for (const Buf& b : bufs) {
    if (b.ptr != nullptr && b.have < b.need) return KDA_ERR_BUFFER_TOO_SMALL;
  }
  return KDA_OK;
}

// Byte sizes of the tensors of a plan, for H heads of K = V = 128.
struct Sizes {
  size_t plan_dev, qkg, v, beta, state_n, trans, state_s, o32, o16;
};
Sizes sizes_of(const kda_plan* plan, int32_t H) {
  const size_t T = static_cast<size_t>(plan->T), N = static_cast<size_t>(plan->N),
               S = static_cast<size_t>(plan->S), h = static_cast<size_t>(H), K = 128, V = 128;
  Sizes z;
  z.plan_dev = plan->blob.size() * sizeof(int32_t);
  z.qkg = T * h * K * 2;
  z.v = T * h * V * 2;
  z.beta = T * h * 2;
  z.state_n = N * h * K * V * 4;
  z.trans = S * h * K * K * 4;
  z.state_s = S * h * K * V * 4;
  z.o32 = T * h * V * 4;
  z.o16 = T * h * V * 2;
  return z;
}

int check_workspace(const void* ws, size_t have, const kda_plan* plan, int32_t H) {
  if (ws == nullptr) return KDA_ERR_INVALID_ARG;
  if (!aligned16(ws)) return KDA_ERR_MISALIGNED;
  if (have < workspace_need(plan, H)) return KDA_ERR_WORKSPACE_TOO_SMALL;
  return KDA_OK;
}

}  // namespace

int check_dims(const kda_plan* plan, const int32_t* plan_dev, int32_t H, int32_t K, int32_t V) {
  if (plan == nullptr || plan_dev == nullptr) return KDA_ERR_INVALID_ARG;
  if (H <= 0 || K <= 0 || V <= 0) return KDA_ERR_INVALID_ARG;
  if (K != 128 || V != 128) return KDA_ERR_UNSUPPORTED;
  if (H > 65535) return KDA_ERR_UNSUPPORTED;
  if (!aligned16(plan_dev)) return KDA_ERR_MISALIGNED;
  return KDA_OK;
}

BwdLayout backward_layout(const kda_plan* plan, int32_t H) {
  const size_t mat = size_t(128) * 128 * sizeof(float);
  const size_t seg_states = static_cast<size_t>(plan->P) * H * mat;   // the backward works on pieces
  auto aligned = [](size_t x) { return (x + 255) & ~size_t(255); };
  BwdLayout L{};
  size_t o = 0;
  L.cache = o;
  o += aligned(workspace_need(plan, H));
  L.transitions = o;
  o += seg_states;
  L.updates = o;
  o += seg_states;
  L.carry = o;
  o += seg_states;
  L.esum = o;
  o += seg_states;
  L.dcarry = o;
  o += seg_states;
  L.ckpt = o;
  o += (static_cast<size_t>(plan->T / kBwdCheckpointTokens) + static_cast<size_t>(plan->F)) * H * mat;
  L.up = o;
  o += static_cast<size_t>(plan->T) * H * 2 * 128 * sizeof(float);
  const size_t slots = backward_chunk_slots(plan);
  L.ck32 = o;
  o += slots * H * mat;
  L.dcot = o;
  o += slots * H * mat;
  L.tcache = o;
  o += slots * H * kChunkCacheBytes;
  L.rv = o;
  o += slots * H * 32 * 128 * sizeof(float);
  L.du = o;
  o += slots * H * 32 * 128 * sizeof(float);
  L.iflag = o;
  o += aligned(static_cast<size_t>(plan->F) * H * sizeof(int32_t));
  L.smap = o;
  o += aligned(slots * sizeof(int32_t));
  L.total = o;
  return L;
}

size_t backward_chunk_slots(const kda_plan* plan) {
  return (static_cast<size_t>(plan->T) + 31) / 32 + static_cast<size_t>(plan->F);
}

size_t backward_workspace_need(const kda_plan* plan, int32_t H) { return backward_layout(plan, H).total; }

PieceLayout piece_layout(const kda_plan* plan, int32_t H) {
  const size_t slots = static_cast<size_t>((plan->T + 31) / 32) + static_cast<size_t>(plan->P);
  const size_t cache = (slots * static_cast<size_t>(H) * kChunkCacheBytes + 255) & ~size_t(255);
  const size_t states = plan->pieces ? static_cast<size_t>(plan->P) * H * 128 * 128 * sizeof(float) : 0;
  PieceLayout L{};
  L.transitions = cache;
  L.updates = cache + states;
  L.carry = cache + 2 * states;
  L.total = cache + 3 * states;
  return L;
}

size_t workspace_need(const kda_plan* plan, int32_t H) { return piece_layout(plan, H).total; }

int check_gate_bound(float gate_lower_bound) {
  // NaN fails both comparisons
  return (gate_lower_bound <= 0.f) ? KDA_OK : KDA_ERR_INVALID_ARG;
}

int check_summaries(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                    const uint16_t* k, size_t k_bytes, const uint16_t* v, size_t v_bytes,
                    const uint16_t* g, size_t g_bytes, const uint16_t* beta, size_t beta_bytes,
                    float gate_lower_bound, const float* initial_state, size_t initial_state_bytes, int32_t H, int32_t K,
                    int32_t V, int32_t head_begin, int32_t head_count, const float* transitions,
                    size_t transitions_bytes, const float* updates, size_t updates_bytes,
                    const void* workspace, size_t workspace_bytes) {
  int st = check_dims(plan, plan_dev, H, K, V);
  if (st != KDA_OK) return st;
  st = check_heads(H, head_begin, head_count);
  if (st != KDA_OK) return st;
  st = check_gate_bound(gate_lower_bound);
  if (st != KDA_OK) return st;
  const Sizes z = sizes_of(plan, H);
  st = check_buffers({{plan_dev, plan_dev_bytes, z.plan_dev, false},
                      {k, k_bytes, z.qkg, false},
                      {v, v_bytes, z.v, false},
                      {g, g_bytes, z.qkg, false},
                      {beta, beta_bytes, z.beta, false},
                      {initial_state, initial_state_bytes, z.state_n, true},
                      {transitions, transitions_bytes, z.trans, false},
                      {updates, updates_bytes, z.state_s, false}});
  if (st != KDA_OK) return st;
  return check_workspace(workspace, workspace_bytes, plan, H);
}

int check_compose(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                  const float* transitions, size_t transitions_bytes, const float* updates,
                  size_t updates_bytes, int32_t H, int32_t K, int32_t V, int32_t head_begin,
                  int32_t head_count, const float* carry_in, size_t carry_in_bytes) {
  int st = check_dims(plan, plan_dev, H, K, V);
  if (st != KDA_OK) return st;
  st = check_heads(H, head_begin, head_count);
  if (st != KDA_OK) return st;
  const Sizes z = sizes_of(plan, H);
  return check_buffers({{plan_dev, plan_dev_bytes, z.plan_dev, false},
                        {transitions, transitions_bytes, z.trans, false},
                        {updates, updates_bytes, z.state_s, false},
                        {carry_in, carry_in_bytes, z.state_s, false}});
}

int check_carry(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                const uint16_t* beta, size_t beta_bytes, float gate_lower_bound,
                const float* initial_state, size_t initial_state_bytes, int32_t H, int32_t K,
                int32_t V, int32_t head_begin, int32_t head_count, const float* carry_in, size_t carry_in_bytes, const void* o,
                size_t o_bytes, int32_t o_format, const float* final_state, size_t final_state_bytes,
                const void* workspace, size_t workspace_bytes) {
  int st = check_dims(plan, plan_dev, H, K, V);
  if (st != KDA_OK) return st;
  st = check_heads(H, head_begin, head_count);
  if (st != KDA_OK) return st;
  if (o_format != KDA_O_FP32 && o_format != KDA_O_BF16) return KDA_ERR_INVALID_ARG;
  st = check_gate_bound(gate_lower_bound);
  if (st != KDA_OK) return st;
  const Sizes z = sizes_of(plan, H);
  st = check_buffers({{plan_dev, plan_dev_bytes, z.plan_dev, false},
                      {q, q_bytes, z.qkg, false},
                      {k, k_bytes, z.qkg, false},
                      {v, v_bytes, z.v, false},
                      {g, g_bytes, z.qkg, false},
                      {beta, beta_bytes, z.beta, false},
                      {initial_state, initial_state_bytes, z.state_n, true},
                      {carry_in, carry_in_bytes, z.state_s, false},
                      {o, o_bytes, o_format == KDA_O_BF16 ? z.o16 : z.o32, false},
                      {final_state, final_state_bytes, z.state_n, false}});
  if (st != KDA_OK) return st;
  return check_workspace(workspace, workspace_bytes, plan, H);
}

int check_backward(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                   const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                   const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                   const uint16_t* beta, size_t beta_bytes, const float* initial_state,
                   size_t initial_state_bytes, const float* d_o, size_t d_o_bytes, const float* d_final,
                   size_t d_final_bytes, int32_t H, int32_t K, int32_t V, int32_t head_begin,
                   int32_t head_count, const float* dq, size_t dq_bytes, const float* dk, size_t dk_bytes,
                   const float* dv, size_t dv_bytes, const float* dg, size_t dg_bytes, const float* dbeta,
                   size_t dbeta_bytes, const float* d_initial_state, size_t d_initial_state_bytes,
                   const void* workspace, size_t workspace_bytes) {
  int st = check_dims(plan, plan_dev, H, K, V);
  if (st != KDA_OK) return st;
  st = check_heads(H, head_begin, head_count);
  if (st != KDA_OK) return st;
  const Sizes z = sizes_of(plan, H);
  const size_t f32_tk = z.qkg * 2;   // [T, H, 128] fp32
  st = check_buffers({{plan_dev, plan_dev_bytes, z.plan_dev, false},
                      {q, q_bytes, z.qkg, false},
                      {k, k_bytes, z.qkg, false},
                      {v, v_bytes, z.v, false},
                      {g, g_bytes, z.qkg, false},
                      {beta, beta_bytes, z.beta, false},
                      {initial_state, initial_state_bytes, z.state_n, true},
                      {d_o, d_o_bytes, f32_tk, false},
                      {d_final, d_final_bytes, z.state_n, true},
                      {dq, dq_bytes, f32_tk, false},
                      {dk, dk_bytes, f32_tk, false},
                      {dv, dv_bytes, f32_tk, false},
                      {dg, dg_bytes, f32_tk, false},
                      {dbeta, dbeta_bytes, z.beta * 2, false},
                      {d_initial_state, d_initial_state_bytes, z.state_n, true}});
  if (st != KDA_OK) return st;
  if (workspace == nullptr) return KDA_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return KDA_ERR_MISALIGNED;
  if (workspace_bytes < backward_workspace_need(plan, H)) return KDA_ERR_WORKSPACE_TOO_SMALL;
  return KDA_OK;
}

}  // namespace kda
