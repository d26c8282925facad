// HIP backward (gradients) of the KDA recurrence on gfx950: for the loss
//     L = sum_t <o_t, do_t> + sum_n <final_n, dfinal_n>
// the gradients of q, k, v, g, beta and the initial states.  Sources:
// inclusionAI/cuLA pull request #110 "feat(cp): add opt-in NVSHMEM CP state
// handoff" (Correctness: output and Q/K/V/g/beta gradients are validated) and
// pull request #136 "feat(kda): add cuDNN concatenated-summary Kimi CP"
// (Sequence Diagram: the backward pass of the context-parallel KDA).
//
// Per token, with S~ = Diag(e^g) S_{t-1}, p = S~^T k, u = beta (v - p),
// S_t = S~ + k u^T and o_t = S_t^T q, the reverse step from dS = dL/dS_t is
//     dS  += q do^T
//     dq   = S_t do,  du = dS^T k,  dv = beta du,  dbeta = <du, v - p>
//     dp   = -beta du,  dk = dS u + S~ dp
//     dS~  = dS + k dp^T,  dg = rowsum(dS~ o S~),  dS_{t-1} = Diag(e^g) dS~.
// One workgroup runs one (sequence, head) in FP32, token by token: a forward
// sweep keeps the state at the start of every 32-token chunk, and the reverse
// sweep recomputes each chunk's per-token states from its checkpoint into a
// per-workgroup buffer before walking its tokens backwards.  The state and its
// cotangent live in LDS as 128 x 128 FP32 tiles; products over rows use one
// thread per column, products over columns one thread per row.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_internal.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int BD = 128;          // key = value dimension
constexpr int BS = BD + 1;       // LDS row stride (floats): row and column walks are conflict-free
constexpr int BCH = 32;          // tokens per checkpointed chunk
constexpr float kLog2eB = 1.4426950408889634f;

struct alignas(16) BwdSmem {
  float S[BD * BS];       // S_{t-1} (the forward sweep: the running state)
  float dS[BD * BS];      // dL/dS_t
  float q[BD], k[BD], dec[BD], v[BD], dov[BD];
  float p[BD], u[BD], du[BD], dp[BD];
  float part[2][BD];      // partial sums of the two halves
  float part2[2][BD];
  float part3[2][BD];
  float beta;
  float red[4];
};

__device__ __forceinline__ float bfv(const uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Sequence n's token range from the plan blob: its fragments are consecutive
// (frag_seq does not decrease), the first begins it and the last ends it.
__device__ __forceinline__ void seq_bounds(const BwdParams& p, const int n, int32_t& bos, int32_t& eos) {
  const int32_t F = p.plan[3];
  const int32_t* fs = p.plan + p.L.frag_seq;
  int lo = 0, hi = F;   // first f with frag_seq[f] >= n
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (fs[mid] < n) lo = mid + 1;
    else hi = mid;
  }
  int lo2 = lo, hi2 = F;   // first f with frag_seq[f] > n
  while (lo2 < hi2) {
    const int mid = (lo2 + hi2) >> 1;
    if (fs[mid] <= n) lo2 = mid + 1;
    else hi2 = mid;
  }
  bos = p.plan[p.L.frag_begin + lo];
  eos = p.plan[p.L.frag_end + lo2 - 1];
}

}  // namespace

__global__ void __launch_bounds__(kBwdThreads, 1) kda_backward_kernel(BwdParams p) {
  __shared__ BwdSmem sm;
  const int bid = blockIdx.x;
  const int n = bid / p.hn;
  const int h = p.h0 + bid % p.hn;
  const int tid = threadIdx.x;
  const int c = tid & (BD - 1);   // column (column walks) or row (row walks)
  const int half = tid >> 7;      // which 64 rows (column walks) or columns (row walks)
  const int H = p.H;
  int32_t bos, eos;
  seq_bounds(p, n, bos, eos);
  const int L = eos - bos;
  const int nchunks = (L + BCH - 1) / BCH;
  const size_t mat = static_cast<size_t>(BD) * BD;
  float* ckpt = p.ws + (static_cast<size_t>(bos / BCH + n) * H + h) * mat;   // chunk j: + j * H * mat
  float* cbuf = p.ws + p.ckpt_floats + (static_cast<size_t>(n) * H + h) * BCH * mat;

  // state tiles <-> global [128][128] (each thread 64 rows of one column)
  auto tile_to_global = [&](const float* t, float* g) {
    for (int r = 64 * half; r < 64 * half + 64; ++r) g[r * BD + c] = t[r * BS + c];
  };
  auto global_to_tile = [&](const float* g, float* t) {
    for (int r = 64 * half; r < 64 * half + 64; ++r) t[r * BS + c] = g == nullptr ? 0.f : g[r * BD + c];
  };
  // token t's vectors into LDS (threads 0..127: one element of each)
  auto load_token = [&](const int t, const bool grads) {
    if (tid < BD) {
      const size_t ik = (static_cast<size_t>(t) * H + h) * BD + tid;
      sm.k[tid] = bfv(p.k[ik]);
      sm.dec[tid] = __builtin_amdgcn_exp2f(bfv(p.g[ik]) * kLog2eB);
      sm.v[tid] = bfv(p.v[ik]);
      if (grads) {
        sm.q[tid] = bfv(p.q[ik]);
        sm.dov[tid] = p.d_o[ik];
      }
      if (tid == 0) sm.beta = bfv(p.beta[static_cast<size_t>(t) * H + h]);
    }
  };
  // p = S~^T k and u = beta (v - p), S~ = Diag(dec) S (column walk)
  auto compute_pu = [&]() {
    float acc = 0.f;
    for (int r = 64 * half; r < 64 * half + 64; ++r) acc += sm.k[r] * sm.dec[r] * sm.S[r * BS + c];
    sm.part[half][c] = acc;
    __syncthreads();
    if (tid < BD) {
      const float pp = sm.part[0][tid] + sm.part[1][tid];
      sm.p[tid] = pp;
      sm.u[tid] = sm.beta * (sm.v[tid] - pp);
    }
    __syncthreads();
  };
  // S <- S~ + k u^T (the forward update)
  auto update_S = [&]() {
    for (int r = 64 * half; r < 64 * half + 64; ++r)
      sm.S[r * BS + c] = sm.dec[r] * sm.S[r * BS + c] + sm.k[r] * sm.u[c];
  };

  // ---- forward sweep: the state at the start of every chunk
  global_to_tile(p.h0s == nullptr ? nullptr : p.h0s + (static_cast<size_t>(n) * H + h) * mat, sm.S);
  __syncthreads();
  for (int j = 0; j < nchunks; ++j) {
    tile_to_global(sm.S, ckpt + static_cast<size_t>(j) * H * mat);
    const int t1 = min(bos + (j + 1) * BCH, eos);
    for (int t = bos + j * BCH; t < t1; ++t) {
      load_token(t, false);
      __syncthreads();
      compute_pu();
      update_S();
      __syncthreads();
    }
  }

  // ---- reverse sweep
  global_to_tile(p.dfinal == nullptr ? nullptr : p.dfinal + (static_cast<size_t>(n) * H + h) * mat, sm.dS);
  __syncthreads();
  for (int j = nchunks - 1; j >= 0; --j) {
    const int t0 = bos + j * BCH;
    const int t1 = min(t0 + BCH, eos);
    // the chunk's per-token states S_{t-1}, from its checkpoint
    global_to_tile(ckpt + static_cast<size_t>(j) * H * mat, sm.S);
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
      tile_to_global(sm.S, cbuf + static_cast<size_t>(t - t0) * mat);
      load_token(t, false);
      __syncthreads();
      compute_pu();
      update_S();
      __syncthreads();
    }
    for (int t = t1 - 1; t >= t0; --t) {
      global_to_tile(cbuf + static_cast<size_t>(t - t0) * mat, sm.S);
      load_token(t, true);
      __syncthreads();
      compute_pu();
      // dS += q do^T
      for (int r = 64 * half; r < 64 * half + 64; ++r) sm.dS[r * BS + c] += sm.q[r] * sm.dov[c];
      __syncthreads();
      // du = dS^T k (column walk)
      {
        float acc = 0.f;
        for (int r = 64 * half; r < 64 * half + 64; ++r) acc += sm.dS[r * BS + c] * sm.k[r];
        sm.part[half][c] = acc;
      }
      __syncthreads();
      if (tid < BD) {
        const float d = sm.part[0][tid] + sm.part[1][tid];
        sm.du[tid] = d;
        sm.dp[tid] = -sm.beta * d;
        p.dv[(static_cast<size_t>(t) * H + h) * BD + tid] = sm.beta * d;
        // dbeta = <du, v - p>: a wave sum, then the two waves' sums
        float x = d * (sm.v[tid] - sm.p[tid]);
        for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
        if ((tid & 63) == 0) sm.red[tid >> 6] = x;
      }
      __syncthreads();
      if (tid == 0) p.dbeta[static_cast<size_t>(t) * H + h] = sm.red[0] + sm.red[1];
      // row walk: thread row c, columns [64 half, 64 half + 64)
      //   dq = S_t do, dk = dS u + S~ dp, dg = rowsum((dS + k dp^T) o S~)
      {
        const int r = c;
        const float dr = sm.dec[r], kr = sm.k[r];
        float aq = 0.f, ak = 0.f, ag = 0.f;
        for (int cc = 64 * half; cc < 64 * half + 64; ++cc) {
          const float st = dr * sm.S[r * BS + cc];          // S~
          const float ds = sm.dS[r * BS + cc];
          aq += (st + kr * sm.u[cc]) * sm.dov[cc];
          ak += ds * sm.u[cc] + st * sm.dp[cc];
          ag += (ds + kr * sm.dp[cc]) * st;
        }
        sm.part[half][r] = aq;
        sm.part2[half][r] = ak;
        sm.part3[half][r] = ag;
      }
      __syncthreads();
      if (tid < BD) {
        const size_t ik = (static_cast<size_t>(t) * H + h) * BD + tid;
        p.dq[ik] = sm.part[0][tid] + sm.part[1][tid];
        p.dk[ik] = sm.part2[0][tid] + sm.part2[1][tid];
        p.dg[ik] = sm.part3[0][tid] + sm.part3[1][tid];
      }
      // dS_{t-1} = Diag(dec) (dS + k dp^T)
      for (int r = 64 * half; r < 64 * half + 64; ++r)
        sm.dS[r * BS + c] = sm.dec[r] * (sm.dS[r * BS + c] + sm.k[r] * sm.dp[c]);
      __syncthreads();
    }
  }
  if (p.dh0 != nullptr) tile_to_global(sm.dS, p.dh0 + (static_cast<size_t>(n) * H + h) * mat);
}

}  // namespace kda
