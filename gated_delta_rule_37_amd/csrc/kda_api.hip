// C-ABI entry points of the segmented KDA forward pass: host-side argument
// validation and kernel launches.  Every check runs before anything is
// enqueued; an error returns a negative kda_status and enqueues nothing.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda.h"
#include "kda_internal.h"
#include "kda_kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const kda_plan* plan, const int32_t* plan_dev, int32_t H, int32_t K, int32_t V) {
  if (plan == nullptr || plan_dev == nullptr) return KDA_ERR_INVALID_ARG;
  if (H <= 0 || K <= 0 || V <= 0) return KDA_ERR_INVALID_ARG;
  if (K != 128 || V != 128) return KDA_ERR_UNSUPPORTED;
  if (H > 65535) return KDA_ERR_UNSUPPORTED;
  if (!aligned16(plan_dev)) return KDA_ERR_MISALIGNED;
  return KDA_OK;
}

int check_heads(int32_t H, int32_t head_begin, int32_t head_count) {
  if (head_begin < 0 || head_count <= 0 || head_count > H - head_begin) return KDA_ERR_INVALID_ARG;
  return KDA_OK;
}

// An optional tensor: null, or 16-byte aligned.
int check_optional(const void* p) { return p == nullptr || aligned16(p) ? KDA_OK : KDA_ERR_MISALIGNED; }

int check_tensors(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs) {
    if (p == nullptr) return KDA_ERR_INVALID_ARG;
  }
  for (const void* p : ptrs) {
    if (!aligned16(p)) return KDA_ERR_MISALIGNED;
  }
  return KDA_OK;
}

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

}  // namespace

extern "C" int kda_last_hip_error(void) { return g_last_hip_error; }

extern "C" size_t kda_chunk_cache_bytes(const kda_plan* plan, int32_t H) {
  if (plan == nullptr || H <= 0) return 0;
  const size_t slots = static_cast<size_t>((plan->T + 31) / 32) + static_cast<size_t>(plan->S);
  return slots * static_cast<size_t>(H) * kda::kChunkCacheBytes;
}

extern "C" int kda_segment_summaries(const kda_plan* plan, const int32_t* plan_dev,
                                     const uint16_t* k, const uint16_t* v, const uint16_t* g,
                                     const uint16_t* beta, const float* initial_state,
                                     int32_t H, int32_t K, int32_t V,
                                     int32_t head_begin, int32_t head_count,
                                     float* transitions, float* updates, void* chunk_cache,
                                     hipStream_t stream) {
  int st = check_dims(plan, plan_dev, H, K, V);
  if (st != KDA_OK) return st;
  st = check_heads(H, head_begin, head_count);
  if (st != KDA_OK) return st;
  st = check_tensors({k, v, g, beta, transitions, updates, chunk_cache});
  if (st != KDA_OK) return st;
  st = check_optional(initial_state);
  if (st != KDA_OK) return st;
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
  p.transitions = transitions;
  p.updates = updates;
  p.carry = nullptr;
  p.init_state = initial_state;
  p.chunk_cache = static_cast<uint16_t*>(chunk_cache);
  (void)hipGetLastError();
  dim3 grid;
  st = chunk_grid(plan->F, head_count, kda::kSummaryThreads, &grid);
  if (st != KDA_OK) return st;
  hipLaunchKernelGGL(kda::kda_chunk_kernel, grid, dim3(kda::kSummaryThreads), 0, stream, p);
  return finish_launch();
}

extern "C" int kda_compose_summaries(const kda_plan* plan, const int32_t* plan_dev,
                                     const float* transitions, const float* updates, int32_t H,
                                     int32_t K, int32_t V, int32_t head_begin, int32_t head_count,
                                     float* carry_in, hipStream_t stream) {
  int st = check_dims(plan, plan_dev, H, K, V);
  if (st != KDA_OK) return st;
  st = check_heads(H, head_begin, head_count);
  if (st != KDA_OK) return st;
  st = check_tensors({transitions, updates, carry_in});
  if (st != KDA_OK) return st;
  kda::ComposeParams p{};
  p.plan = plan_dev;
  p.L = plan->layout;
  p.H = H;
  p.h0 = head_begin;
  p.hn = head_count;
  p.S = plan->S;
  p.transitions = transitions;
  p.updates = updates;
  p.carry = carry_in;
  (void)hipGetLastError();
  // one workgroup per (head, column block), heads padded to a multiple of 8
  const int blocks = ((head_count + 7) / 8) * 8 * kda::kComposeColumnBlocks;
  hipLaunchKernelGGL(kda::kda_compose_kernel, dim3(blocks), dim3(kda::kComposeThreads), 0, stream, p);
  return finish_launch();
}

extern "C" int kda_apply_carry(const kda_plan* plan, const int32_t* plan_dev, const uint16_t* q,
                               const uint16_t* k, const uint16_t* v, const uint16_t* g,
                               const uint16_t* beta, const float* initial_state,
                               int32_t H, int32_t K, int32_t V,
                               int32_t head_begin, int32_t head_count,
                               const float* carry_in, void* o, int32_t o_format, float* final_state,
                               const void* chunk_cache, hipStream_t stream) {
  int st = check_dims(plan, plan_dev, H, K, V);
  if (st != KDA_OK) return st;
  st = check_heads(H, head_begin, head_count);
  if (st != KDA_OK) return st;
  st = check_tensors({q, k, v, g, beta, carry_in, o, final_state, chunk_cache});
  if (st != KDA_OK) return st;
  st = check_optional(initial_state);
  if (st != KDA_OK) return st;
  if (o_format != KDA_O_FP32 && o_format != KDA_O_BF16) return KDA_ERR_INVALID_ARG;
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
  p.carry = carry_in;
  p.init_state = initial_state;
  p.chunk_cache = const_cast<uint16_t*>(static_cast<const uint16_t*>(chunk_cache));
  (void)hipGetLastError();
  dim3 grid;
  st = chunk_grid(plan->F, head_count, kda::kCarryThreads, &grid);
  if (st != KDA_OK) return st;
  hipLaunchKernelGGL(kda::kda_carry_kernel, grid, dim3(kda::kCarryThreads), 0, stream, p);
  return finish_launch();
}
