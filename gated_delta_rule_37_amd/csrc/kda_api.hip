// C-ABI entry points of the segmented KDA forward pass: host-side argument
// validation and kernel launches.  Every check runs before anything is
// enqueued; an error returns a negative kda_status and enqueues nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>

#include "kda.h"
#include "kda_internal.h"
#include "kda_kernels.h"
#include "kda_validate.h"

namespace {

using kda::backward_workspace_need;
using kda::check_backward;
using kda::check_carry;
using kda::check_compose;
using kda::check_dims;
using kda::check_summaries;
using kda::workspace_need;
using kda::PieceLayout;

thread_local int g_last_hip_error = 0;

// Grid of a chunk kernel: F * hn workgroups numbered linearly (head fastest),
// laid out as x = hn * a, y = ceil(F / a) with the smallest a that keeps y
// within 65535.  x must stay within 2^31 - 1 work-items.
int chunk_grid(int32_t F, int32_t hn, int threads, dim3* grid) {
  const int64_t a = (static_cast<int64_t>(F) + 65534) / 65535;
  const int64_t x = static_cast<int64_t>(hn) * (a > 0 ? a : 1);
  if (x * threads > 2147483647LL) return KDA_ERR_UNSUPPORTED;
  *grid = dim3(static_cast<uint32_t>(x), static_cast<uint32_t>((F + x / hn - 1) / (x / hn)), 1);
  return KDA_OK;
}

int finish_launch() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return KDA_ERR_HIP;
  }
  return KDA_OK;
}

// --------------------------------------------------------------- launches
// Each takes arguments that have passed the checks above.

// The safe gate's lower bound as the kernels take it (log2 units).
void set_gate(kda::ChunkParams& p, float gate_lower_bound) {
  p.gate_floor_on = gate_lower_bound > -INFINITY ? 1 : 0;
  p.gate_floor = gate_lower_bound * 1.4426950408889634f;
}

// A scan launch (the compose kernel in one of its modes): grid of
// (chain, head) units padded to a multiple of 8, times the column blocks.
int launch_scan(void (*kernel)(kda::ComposeParams), const kda::ComposeParams& c, int chains, int column_blocks,
                hipStream_t stream) {
  const int64_t units = static_cast<int64_t>(chains) * c.hn;
  const int64_t blocks = ((units + 7) / 8) * 8 * column_blocks;
  if (blocks > 2147483647LL) return KDA_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kda::kComposeThreads), 0, stream, c);
  return finish_launch();
}

kda::ComposeParams scan_params(const kda_plan* plan, const int32_t* plan_dev, int32_t H, int32_t head_begin,
                               int32_t head_count) {
  kda::ComposeParams c{};
  c.plan = plan_dev;
  c.L = plan->layout;
  c.H = H;
  c.h0 = head_begin;
  c.hn = head_count;
  c.chains = plan->S;
  return c;
}

// Summaries into `transitions` / `updates`: per segment, or per piece with
// fold = false (the backward's own arrays).  With pieces and fold = true the
// pieces' summaries go to the workspace and are folded into the segments'.
int launch_summaries(const kda_plan* plan, const int32_t* plan_dev, const uint16_t* k,
                     const uint16_t* v, const uint16_t* g, const uint16_t* beta, float gate_lower_bound,
                     const float* initial_state, int32_t H, int32_t head_begin, int32_t head_count,
                     float* transitions, float* updates, void* workspace, hipStream_t stream, bool fold = true) {
  const bool via_pieces = plan->pieces && fold;
  const kda::PieceLayout PL = kda::piece_layout(plan, H);
  float* piece_a = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + PL.transitions);
  float* piece_b = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + PL.updates);
  kda::ChunkParams p{};
  p.plan = plan_dev;
  p.L = plan->layout;
  p.H = H;
  p.h0 = head_begin;
  p.hn = head_count;
  p.q = nullptr;
  p.k = k;
  p.v = v;
  p.g = g;
  p.beta = beta;
  p.o = nullptr;
  p.final_state = nullptr;
  p.transitions = via_pieces ? piece_a : transitions;
  p.updates = via_pieces ? piece_b : updates;
  p.carry = nullptr;
  p.init_state = initial_state;
  set_gate(p, gate_lower_bound);
  p.chunk_cache = static_cast<uint16_t*>(workspace);
  dim3 grid;
  int st = chunk_grid(plan->F, head_count, kda::kSummaryThreads, &grid);
  if (st != KDA_OK) return st;
  (void)hipGetLastError();
  hipLaunchKernelGGL(kda::kda_chunk_kernel, grid, dim3(kda::kSummaryThreads), 0, stream, p);
  st = finish_launch();
  if (st != KDA_OK || !via_pieces) return st;
  // each segment's (A_r, B_r) from its pieces'
  kda::ComposeParams c = scan_params(plan, plan_dev, H, head_begin, head_count);
  c.live_off = plan->layout.seg_transition_live;
  c.transitions = piece_a;
  c.updates = piece_b;
  c.out_a = transitions;
  c.out_b = updates;
  return launch_scan(kda::kda_fold_pieces_kernel, c, plan->S, 2 * kda::kComposeColumnBlocks, stream);
}

// The ordered scan over the segments (pieces = false) or, for the backward,
// over the pieces.
int launch_compose(const kda_plan* plan, const int32_t* plan_dev, const float* transitions,
                   const float* updates, int32_t H, int32_t head_begin, int32_t head_count,
                   float* carry_in, hipStream_t stream, bool pieces = false) {
  kda::ComposeParams c = scan_params(plan, plan_dev, H, head_begin, head_count);
  c.S = pieces ? plan->P : plan->S;
  c.live_off = pieces ? plan->layout.seg_transition_live : plan->layout.useg_transition_live;
  c.transitions = transitions;
  c.updates = updates;
  c.carry = carry_in;
  return launch_scan(kda::kda_compose_kernel, c, 1, kda::kComposeColumnBlocks, stream);
}

int launch_carry(const kda_plan* plan, const int32_t* plan_dev, const uint16_t* q, const uint16_t* k,
                 const uint16_t* v, const uint16_t* g, const uint16_t* beta, float gate_lower_bound,
                 const float* initial_state, int32_t H, int32_t head_begin, int32_t head_count,
                 const float* carry_in, void* o, int32_t o_format, float* final_state,
                 const void* workspace, hipStream_t stream, bool piece_level = false) {
  const float* carry = carry_in;
  if (plan->pieces && !piece_level) {
    // every piece's carry-in, from its segment's
    const kda::PieceLayout PL = kda::piece_layout(plan, H);
    const uint8_t* ws = static_cast<const uint8_t*>(workspace);
    kda::ComposeParams c = scan_params(plan, plan_dev, H, head_begin, head_count);
    c.live_off = plan->layout.seg_transition_live;
    c.transitions = reinterpret_cast<const float*>(ws + PL.transitions);
    c.updates = reinterpret_cast<const float*>(ws + PL.updates);
    c.carry = const_cast<float*>(reinterpret_cast<const float*>(ws + PL.carry));
    c.init = carry_in;
    const int st = launch_scan(kda::kda_piece_carry_kernel, c, plan->S, kda::kComposeColumnBlocks, stream);
    if (st != KDA_OK) return st;
    carry = c.carry;
  }
  kda::ChunkParams p{};
  p.plan = plan_dev;
  p.L = plan->layout;
  p.H = H;
  p.h0 = head_begin;
  p.hn = head_count;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.beta = beta;
  p.o = static_cast<float*>(o);
  p.o_bf16 = o_format == KDA_O_BF16 ? 1 : 0;
  p.final_state = final_state;
  p.transitions = nullptr;
  p.updates = nullptr;
  p.carry = carry;
  p.init_state = initial_state;
  set_gate(p, gate_lower_bound);
  p.chunk_cache = const_cast<uint16_t*>(static_cast<const uint16_t*>(workspace));
  dim3 grid;
  const int st = chunk_grid(plan->F, head_count, kda::kCarryThreads, &grid);
  if (st != KDA_OK) return st;
  (void)hipGetLastError();
  hipLaunchKernelGGL(kda::kda_carry_kernel, grid, dim3(kda::kCarryThreads), 0, stream, p);
  return finish_launch();
}

// ------------------------------------------------- allocation-free variant
// The workspace of kda_forward_noalloc: a fixed device array, one copy per
// GPU, kept until the process ends.  Host code never uses its name as an
// address (on the host it is only a stand-in); each device's address comes
// from hipGetSymbolAddress with that device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on each device), or a KDA status.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return KDA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      g_last_hip_error = static_cast<int>(e);
      return KDA_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" int kda_last_hip_error(void) { return g_last_hip_error; }

extern "C" size_t kda_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

extern "C" size_t kda_workspace_bytes(const kda_plan* plan, int32_t H, int32_t K, int32_t V) {
  if (plan == nullptr || H <= 0 || K != 128 || V != 128) return 0;
  return workspace_need(plan, H);
}

extern "C" int kda_segment_summaries(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                                     const uint16_t* k, size_t k_bytes, const uint16_t* v, size_t v_bytes,
                                     const uint16_t* g, size_t g_bytes, const uint16_t* beta,
                                     size_t beta_bytes, float gate_lower_bound, const float* initial_state,
                                     size_t initial_state_bytes, int32_t H, int32_t K, int32_t V,
                                     int32_t head_begin, int32_t head_count, float* transitions,
                                     size_t transitions_bytes, float* updates, size_t updates_bytes,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_summaries(plan, plan_dev, plan_dev_bytes, k, k_bytes, v, v_bytes, g, g_bytes, beta,
                                 beta_bytes, gate_lower_bound, initial_state, initial_state_bytes, H, K, V,
                                 head_begin, head_count, transitions, transitions_bytes, updates, updates_bytes,
                                 workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  return launch_summaries(plan, plan_dev, k, v, g, beta, gate_lower_bound, initial_state, H, head_begin,
                          head_count, transitions, updates, workspace, stream);
}

extern "C" int kda_compose_summaries(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                                     const float* transitions, size_t transitions_bytes,
                                     const float* updates, size_t updates_bytes, int32_t H, int32_t K,
                                     int32_t V, int32_t head_begin, int32_t head_count, float* carry_in,
                                     size_t carry_in_bytes, hipStream_t stream) {
  const int st = check_compose(plan, plan_dev, plan_dev_bytes, transitions, transitions_bytes, updates,
                               updates_bytes, H, K, V, head_begin, head_count, carry_in, carry_in_bytes);
  if (st != KDA_OK) return st;
  return launch_compose(plan, plan_dev, transitions, updates, H, head_begin, head_count, carry_in, stream);
}

extern "C" int kda_apply_carry(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                               const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                               const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                               const uint16_t* beta, size_t beta_bytes, float gate_lower_bound,
                               const float* initial_state,
                               size_t initial_state_bytes, int32_t H, int32_t K, int32_t V,
                               int32_t head_begin, int32_t head_count, const float* carry_in,
                               size_t carry_in_bytes, void* o, size_t o_bytes, int32_t o_format,
                               float* final_state, size_t final_state_bytes, const void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  const int st = check_carry(plan, plan_dev, plan_dev_bytes, q, q_bytes, k, k_bytes, v, v_bytes, g, g_bytes,
                             beta, beta_bytes, gate_lower_bound, initial_state, initial_state_bytes, H, K, V,
                             head_begin, head_count, carry_in, carry_in_bytes, o, o_bytes, o_format,
                             final_state, final_state_bytes, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  return launch_carry(plan, plan_dev, q, k, v, g, beta, gate_lower_bound, initial_state, H, head_begin,
                      head_count, carry_in, o, o_format, final_state, workspace, stream);
}

extern "C" int kda_forward(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                           const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                           const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                           const uint16_t* beta, size_t beta_bytes, float gate_lower_bound,
                           const float* initial_state,
                           size_t initial_state_bytes, int32_t H, int32_t K, int32_t V,
                           int32_t head_begin, int32_t head_count, float* transitions,
                           size_t transitions_bytes, float* updates, size_t updates_bytes,
                           float* carry_in, size_t carry_in_bytes, void* o, size_t o_bytes,
                           int32_t o_format, float* final_state, size_t final_state_bytes,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_summaries(plan, plan_dev, plan_dev_bytes, k, k_bytes, v, v_bytes, g, g_bytes, beta,
                           beta_bytes, gate_lower_bound, initial_state, initial_state_bytes, H, K, V,
                           head_begin, head_count,
                           transitions, transitions_bytes, updates, updates_bytes, workspace,
                           workspace_bytes);
  if (st != KDA_OK) return st;
  st = check_compose(plan, plan_dev, plan_dev_bytes, transitions, transitions_bytes, updates, updates_bytes,
                     H, K, V, head_begin, head_count, carry_in, carry_in_bytes);
  if (st != KDA_OK) return st;
  st = check_carry(plan, plan_dev, plan_dev_bytes, q, q_bytes, k, k_bytes, v, v_bytes, g, g_bytes, beta,
                   beta_bytes, gate_lower_bound, initial_state, initial_state_bytes, H, K, V, head_begin,
                   head_count, carry_in,
                   carry_in_bytes, o, o_bytes, o_format, final_state, final_state_bytes, workspace,
                   workspace_bytes);
  if (st != KDA_OK) return st;
  dim3 unused;
  st = chunk_grid(plan->F, head_count, kda::kSummaryThreads, &unused);
  if (st != KDA_OK) return st;
  st = launch_summaries(plan, plan_dev, k, v, g, beta, gate_lower_bound, initial_state, H, head_begin,
                        head_count, transitions, updates, workspace, stream);
  if (st != KDA_OK) return st;
  st = launch_compose(plan, plan_dev, transitions, updates, H, head_begin, head_count, carry_in, stream);
  if (st != KDA_OK) return st;
  return launch_carry(plan, plan_dev, q, k, v, g, beta, gate_lower_bound, initial_state, H, head_begin,
                      head_count, carry_in, o, o_format, final_state, workspace, stream);
}

extern "C" int kda_forward_noalloc(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                                   const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                                   const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                                   const uint16_t* beta, size_t beta_bytes, float gate_lower_bound,
                                   const float* initial_state,
                                   size_t initial_state_bytes, int32_t H, int32_t K, int32_t V,
                                   int32_t head_begin, int32_t head_count, float* transitions,
                                   size_t transitions_bytes, float* updates, size_t updates_bytes,
                                   float* carry_in, size_t carry_in_bytes, void* o, size_t o_bytes,
                                   int32_t o_format, float* final_state, size_t final_state_bytes,
                                   hipStream_t stream) {
  // The size check comes first, so that an oversized call is refused without
  // touching the device; the checks of kda_forward then see a workspace of
  // exactly the size needed.
  if (plan != nullptr && H > 0 && workspace_need(plan, H) > kScratchBytes) return KDA_ERR_WORKSPACE_TOO_SMALL;
  int st = check_dims(plan, plan_dev, H, K, V);
  if (st != KDA_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != KDA_OK) return st;
  // every chunk-cache slot the carry launch reads is written by the summaries
  // launch of the same call, so the array needs no clearing between calls
  return kda_forward(plan, plan_dev, plan_dev_bytes, q, q_bytes, k, k_bytes, v, v_bytes, g, g_bytes, beta,
                     beta_bytes, gate_lower_bound, initial_state, initial_state_bytes, H, K, V, head_begin, head_count,
                     transitions, transitions_bytes, updates, updates_bytes, carry_in, carry_in_bytes, o,
                     o_bytes, o_format, final_state, final_state_bytes, ws, kScratchBytes, stream);
}

extern "C" size_t kda_backward_workspace_bytes(const kda_plan* plan, int32_t H, int32_t K, int32_t V) {
  if (plan == nullptr || H <= 0 || K != 128 || V != 128) return 0;
  return backward_workspace_need(plan, H);
}

// kda_backward, and with `saved_transitions` / `saved_carry` non-null its
// variant that takes the forward's A_r and C_r instead of recomputing them.
int backward_impl(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes, const uint16_t* q,
                  size_t q_bytes, const uint16_t* k, size_t k_bytes, const uint16_t* v, size_t v_bytes,
                  const uint16_t* g, size_t g_bytes, const uint16_t* beta, size_t beta_bytes,
                  const float* initial_state, size_t initial_state_bytes, const float* d_o, size_t d_o_bytes,
                  const float* d_final, size_t d_final_bytes, int32_t H, int32_t K, int32_t V, int32_t head_begin,
                  int32_t head_count, float* dq, size_t dq_bytes, float* dk, size_t dk_bytes, float* dv,
                  size_t dv_bytes, float* dg, size_t dg_bytes, float* dbeta, size_t dbeta_bytes,
                  float* d_initial_state, size_t d_initial_state_bytes, const float* saved_transitions,
                  const float* saved_carry, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_backward(plan, plan_dev, plan_dev_bytes, q, q_bytes, k, k_bytes, v, v_bytes, g, g_bytes,
                                beta, beta_bytes, initial_state, initial_state_bytes, d_o, d_o_bytes, d_final,
                                d_final_bytes, H, K, V, head_begin, head_count, dq, dq_bytes, dk, dk_bytes, dv,
                                dv_bytes, dg, dg_bytes, dbeta, dbeta_bytes, d_initial_state,
                                d_initial_state_bytes, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  dim3 unused;
  st = chunk_grid(plan->F, head_count, kda::kSummaryThreads, &unused);
  if (st != KDA_OK) return st;
  const int64_t seg_blocks = static_cast<int64_t>(plan->P) * head_count;   // the backward works on pieces
  const int64_t items = static_cast<int64_t>(plan->F) * head_count;
  if (seg_blocks > 2147483647LL || items > 2147483647LL) return KDA_ERR_UNSUPPORTED;
  // the gradient launch is persistent, one workgroup per CU at most: the
  // device's CU count, before anything is enqueued
  int cus = 0;
  {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || cus <= 0) {
      g_last_hip_error = static_cast<int>(e);
      return KDA_ERR_HIP;
    }
  }
  const kda::BwdLayout W = kda::backward_layout(plan, H);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const bool saved = saved_transitions != nullptr;
  float* transitions = saved ? const_cast<float*>(saved_transitions) : reinterpret_cast<float*>(ws + W.transitions);
  float* updates = reinterpret_cast<float*>(ws + W.updates);
  float* carry = saved ? const_cast<float*>(saved_carry) : reinterpret_cast<float*>(ws + W.carry);
  float* esum = reinterpret_cast<float*>(ws + W.esum);
  float* dcarry = reinterpret_cast<float*>(ws + W.dcarry);
  // the forward's summaries and carry-ins, without the safe gate (read-only
  // from here on when the caller saved them)
  if (!saved) {
    st = launch_summaries(plan, plan_dev, k, v, g, beta, -INFINITY, initial_state, H, head_begin, head_count,
                          transitions, updates, ws + W.cache, stream, /*fold=*/false);
    if (st != KDA_OK) return st;
    st = launch_compose(plan, plan_dev, transitions, updates, H, head_begin, head_count, carry, stream,
                        /*pieces=*/true);
    if (st != KDA_OK) return st;
  }
  // the checkpoint launch: every fragment forward from its carry-in (or its
  // initial state, or zero), the anchored state entering every 32-token chunk
  // and its T diag(beta); fragments that leave the anchored form's range are
  // flagged for the token-by-token path
  const size_t slots = kda::backward_chunk_slots(plan);
  if (static_cast<int64_t>(slots) * head_count > 2147483647LL) return KDA_ERR_UNSUPPORTED;
  {
    kda::ChunkParams c{};
    c.plan = plan_dev;
    c.L = plan->layout;
    c.H = H;
    c.h0 = head_begin;
    c.hn = head_count;
    c.k = k;
    c.v = v;
    c.g = g;
    c.beta = beta;
    c.carry = carry;
    c.init_state = initial_state;
    set_gate(c, -INFINITY);
    c.chunk_cache = reinterpret_cast<uint16_t*>(ws + W.tcache);
    c.ckpt = reinterpret_cast<float*>(ws + W.ck32);
    c.item_flag = reinterpret_cast<int32_t*>(ws + W.iflag);
    c.slot_map = reinterpret_cast<int32_t*>(ws + W.smap);
    c.rv_out = reinterpret_cast<float*>(ws + W.rv);
    dim3 grid;
    st = chunk_grid(plan->F, head_count, kda::kCarryThreads, &grid);
    if (st != KDA_OK) return st;
    (void)hipGetLastError();
    hipLaunchKernelGGL(kda::kda_ckpt_kernel, grid, dim3(kda::kCarryThreads), 0, stream, c);
    st = finish_launch();
    if (st != KDA_OK) return st;
  }
  kda::BwdParams p{};
  p.plan = plan_dev;
  p.L = plan->layout;
  p.H = H;
  p.h0 = head_begin;
  p.hn = head_count;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.beta = beta;
  p.h0s = initial_state;
  p.d_o = d_o;
  p.dfinal = d_final;
  p.carry = carry;
  p.esum = esum;
  p.dcarry = dcarry;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dg = dg;
  p.dbeta = dbeta;
  p.dh0 = d_initial_state;
  p.ckpt = reinterpret_cast<float*>(ws + W.ckpt);
  p.upbuf = reinterpret_cast<float*>(ws + W.up);
  p.ck32 = reinterpret_cast<const float*>(ws + W.ck32);
  p.dcot = reinterpret_cast<float*>(ws + W.dcot);
  p.tcache = reinterpret_cast<const uint16_t*>(ws + W.tcache);
  p.iflag = reinterpret_cast<const int32_t*>(ws + W.iflag);
  p.smap = reinterpret_cast<int32_t*>(ws + W.smap);
  p.rvbuf = reinterpret_cast<const float*>(ws + W.rv);
  p.dubuf = reinterpret_cast<float*>(ws + W.du);
  p.nslots = static_cast<int32_t>(slots);
  // E_r: the chunked chain over each carried segment's first fragment, then
  // the token-by-token summaries of the flagged ones
  (void)hipGetLastError();
  hipLaunchKernelGGL(kda::kda_bwd_chain_e_kernel, dim3(static_cast<uint32_t>(seg_blocks)),
                     dim3(kda::kChainThreads), 0, stream, p);
  // many (piece, head) items: small workgroups, several per CU; few: large
  // ones, each item's chain shorter
  if (seg_blocks >= 1024) {
    hipLaunchKernelGGL(kda::kda_backward_summary_narrow_kernel, dim3(static_cast<uint32_t>(seg_blocks)),
                       dim3(kda::kBwdSummaryThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(kda::kda_backward_summary_kernel, dim3(static_cast<uint32_t>(seg_blocks)),
                       dim3(kda::kBwdThreads), 0, stream, p);
  }
  st = finish_launch();
  if (st != KDA_OK) return st;
  // D_r = the reverse scan of (A^T, E)
  kda::ComposeParams c = scan_params(plan, plan_dev, H, head_begin, head_count);
  c.S = plan->P;
  c.live_off = plan->layout.seg_transition_live;
  c.transitions = transitions;
  c.updates = esum;
  c.carry = dcarry;
  st = launch_scan(kda::kda_compose_reverse_kernel, c, 1, kda::kComposeColumnBlocks, stream);
  if (st != KDA_OK) return st;
  // the token-by-token path for the flagged fragments (the others' workgroups
  // skip them)
  const int64_t grid = items < kda::kBwdGrid ? items : kda::kBwdGrid;
  hipLaunchKernelGGL(kda::kda_backward_forward_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kda::kBwdThreads),
                     0, stream, p);
  hipLaunchKernelGGL(kda::kda_backward_fragment_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kda::kBwdThreads),
                     0, stream, p);
  // the chunked path: every fragment's cotangent chain, then every chunk's
  // gradients
  hipLaunchKernelGGL(kda::kda_bwd_chain_kernel, dim3(static_cast<uint32_t>(items)), dim3(kda::kChainThreads), 0,
                     stream, p);
  const int64_t ggrid = static_cast<int64_t>(slots) * head_count < cus ? static_cast<int64_t>(slots) * head_count : cus;
  hipLaunchKernelGGL(kda::kda_bwd_grad_kernel, dim3(static_cast<uint32_t>(ggrid)), dim3(kda::kGradThreads), 0,
                     stream, p);
  return finish_launch();
}

extern "C" int kda_backward(const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes,
                            const uint16_t* q, size_t q_bytes, const uint16_t* k, size_t k_bytes,
                            const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
                            const uint16_t* beta, size_t beta_bytes, const float* initial_state,
                            size_t initial_state_bytes, const float* d_o, size_t d_o_bytes,
                            const float* d_final, size_t d_final_bytes, int32_t H, int32_t K, int32_t V,
                            int32_t head_begin, int32_t head_count, float* dq, size_t dq_bytes, float* dk,
                            size_t dk_bytes, float* dv, size_t dv_bytes, float* dg, size_t dg_bytes,
                            float* dbeta, size_t dbeta_bytes, float* d_initial_state,
                            size_t d_initial_state_bytes, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return backward_impl(plan, plan_dev, plan_dev_bytes, q, q_bytes, k, k_bytes, v, v_bytes, g, g_bytes, beta,
                       beta_bytes, initial_state, initial_state_bytes, d_o, d_o_bytes, d_final, d_final_bytes, H, K,
                       V, head_begin, head_count, dq, dq_bytes, dk, dk_bytes, dv, dv_bytes, dg, dg_bytes, dbeta,
                       dbeta_bytes, d_initial_state, d_initial_state_bytes, nullptr, nullptr, workspace,
                       workspace_bytes, stream);
}

extern "C" int kda_backward_from_forward(
    const kda_plan* plan, const int32_t* plan_dev, size_t plan_dev_bytes, const uint16_t* q, size_t q_bytes,
    const uint16_t* k, size_t k_bytes, const uint16_t* v, size_t v_bytes, const uint16_t* g, size_t g_bytes,
    const uint16_t* beta, size_t beta_bytes, const float* initial_state, size_t initial_state_bytes,
    const float* d_o, size_t d_o_bytes, const float* d_final, size_t d_final_bytes, int32_t H, int32_t K,
    int32_t V, int32_t head_begin, int32_t head_count, const float* transitions, size_t transitions_bytes,
    const float* carry_in, size_t carry_in_bytes, float* dq, size_t dq_bytes, float* dk, size_t dk_bytes,
    float* dv, size_t dv_bytes, float* dg, size_t dg_bytes, float* dbeta, size_t dbeta_bytes,
    float* d_initial_state, size_t d_initial_state_bytes, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  int st = check_dims(plan, plan_dev, H, K, V);
  if (st != KDA_OK) return st;
  // a pieces plan's backward works on the pieces' transitions, which the
  // forward folds into its segments' and does not return
  if (plan->pieces) return KDA_ERR_UNSUPPORTED;
  // (the carry-ins stand in for the updates, which this call does not read)
  st = check_compose(plan, plan_dev, plan_dev_bytes, transitions, transitions_bytes, carry_in, carry_in_bytes, H,
                     K, V, head_begin, head_count, carry_in, carry_in_bytes);
  if (st != KDA_OK) return st;
  return backward_impl(plan, plan_dev, plan_dev_bytes, q, q_bytes, k, k_bytes, v, v_bytes, g, g_bytes, beta,
                       beta_bytes, initial_state, initial_state_bytes, d_o, d_o_bytes, d_final, d_final_bytes, H, K,
                       V, head_begin, head_count, dq, dq_bytes, dk, dk_bytes, dv, dv_bytes, dg, dg_bytes, dbeta,
                       dbeta_bytes, d_initial_state, d_initial_state_bytes, transitions, carry_in, workspace,
                       workspace_bytes, stream);
}
