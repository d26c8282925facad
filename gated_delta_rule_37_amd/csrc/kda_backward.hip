// HIP backward (gradients) of the KDA recurrence on gfx950: for the loss
//     L = sum_t <o_t, do_t> + sum_n <final_n, dfinal_n>
// the gradients of q, k, v, g, beta and the initial states.  Sources:
// inclusionAI/cuLA pull request #110 "feat(cp): add opt-in NVSHMEM CP state
// handoff" (Correctness: output and Q/K/V/g/beta gradients are validated) and
// pull request #136 "feat(kda): add cuDNN concatenated-summary Kimi CP"
// (Sequence Diagram: the backward gathers the following ranks' summaries).
//
// Per token, with S~ = Diag(e^g) S_{t-1}, p = S~^T k, u = beta (v - p),
// S_t = S~ + k u^T and o_t = S_t^T q, the reverse step from dS = dL/dS_t is
//     dS  += q do^T
//     dq   = S_t do,  du = dS^T k,  dv = beta du,  dbeta = <du, v - p>
//     dp   = -beta du,  dk = dS u + S~ dp
//     dS~  = dS + k dp^T,  dg = rowsum(dS~ o S~),  dS_{t-1} = Diag(e^g) dS~.
// The cotangent recursion does not involve the state, so a segment maps the
// cotangent at its end, D, to the one at its start affinely: A_r^T D + E_r.
// The segments (the pieces of a plan with pieces) therefore run in parallel,
// as in the forward:
//   kda_backward_summary_kernel   E_r: the first fragment of every carried
//                                 segment reversed from its own outputs only;
//   (reverse compose)             D_{r-1} = A_r^T D_r + E_r;
//   kda_backward_fragment_kernel  every (fragment, head): forward from its
//                                 carry-in C_r (or initial state), reverse
//                                 from D_r (and dfinal at a sequence end).
//
// Layout: a 1024-thread workgroup holds a 128 x 128 state in registers,
// thread (c, grp) = (tid % 128, tid / 128) owning column c of rows
// [16 grp, 16 grp + 16).  Sums over rows (p, du) go through one LDS exchange
// of eight partials; sums over columns (dq, dk, dg) are reduced within each
// wave by a transposing butterfly (lane-swap and DPP moves) and across the
// two waves of a row group through LDS.  The fragment kernel keeps the state
// every 16 tokens and every token's u and p in global memory (level 1); in
// the reverse it recomputes each 4-token group's first state from its
// chunk's checkpoint by update-only steps (u known, no exchange; the chunk's
// k, e^g and u held in LDS), and the group's per-token states in registers
// the same way before walking it backwards.  Recomputing costs three
// update-only steps per token; storing states every 4 tokens instead would
// write 64 KiB per group and workgroup, which the memory system cannot take
// at the rate 256 workgroups would produce it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_internal.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int BD = 128;               // key = value dimension
constexpr int NT = kBwdThreads;       // 1024
constexpr int NGRP = NT / BD;         // row groups: 8
constexpr int NR = BD / NGRP;         // rows per thread: 16
constexpr int GT = 4;                 // tokens per register group
constexpr int CK = kBwdCheckpointTokens;   // tokens per checkpoint chunk: 16
constexpr int GPC = CK / GT;          // groups per checkpoint chunk: 4
constexpr size_t MAT = static_cast<size_t>(BD) * BD;
constexpr float kLog2eB = 1.4426950408889634f;
static_assert(NR == 16 && NT == 1024, "backward layout: 16 rows per thread, 16 waves");

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// One group of up to four tokens' vectors (the reverse launch).
struct alignas(16) TokGroup {
  float k[GT][BD];
  float dec[GT][BD];   // e^g
  float q[GT][BD];
  float v[GT][BD];
  float dov[GT][BD];
  float beta[GT];
};

// The reverse launch's LDS: two token groups (by group parity), the du
// exchange (one partial per 32-row block, by exchange parity), the row sums
// (one partial per 32-column block, by token parity), dbeta's and u.do's
// column sums (one partial per 32-column block, by token parity), and one
// 16-token chunk's u and p (by token), k and e^g rows for the recompute.
struct alignas(16) RevSmem {
  TokGroup tg[2];
  float colpart[2][4][BD];
  float rowpart[2][3][4][BD];
  float red[2][2][4];
  float upc[CK][2][BD];
  float ckk[CK][BD];
  float ckd[CK][BD];
};

// The forward launch's LDS: two 16-token chunks' k, e^g, v and beta (by
// chunk parity); the current 4-token group's derived rows, with
// Gam_t = e^{g_0 + ... + g_t} (per channel, from the group's first token):
// gk_t = k_t Gam_t, kh_t = k_t e^{g_{t+1} + ... + g_{n-1}}, gamn = Gam_{n-1}
// and ap[(t-1)t/2 + j] = sum_r k_t k_j e^{g_{j+1} + ... + g_t} (j < t); and
// the exchange of four row-sum partials per row group.
struct alignas(16) FwdChunk {
  float k[CK][BD];
  float dec[CK][BD];
  float v[CK][BD];
  float beta[CK];
};
struct alignas(16) FwdGroup {
  float gk[GT][BD];
  float kh[GT][BD];
  float gamn[BD];
  float ap[8];
};
struct alignas(16) FwdSmem {
  FwdChunk ch[2];
  FwdGroup fg;
  f4 colpart4[NGRP][BD];
};

__device__ __forceinline__ f4 l4(const float* src) { return *reinterpret_cast<const f4*>(src); }

__device__ __forceinline__ float bfv(const uint32_t b) { return __uint_as_float(b << 16); }

// Raw buffer resources: a uniform base and byte count in scalar registers,
// 32-bit per-lane offsets; accesses at or past the count read zero and drop
// writes (buffer word 3 of gfx9 raw, unswizzled 32-bit access).
constexpr int kBufWord3 = 0x00020000;
using Rsrc = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ Rsrc rsrc(const void* base, const uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufWord3);
}

// A group's loads, in registers between their issue and their store to LDS
// (four dwords, whatever the role).  Waves 0-1 load k and g, waves 2-3 q and v
// (4 bf16 of each per lane), waves 4-5 d_o (4 floats), lanes 0-3 of wave 6
// beta; bits 5-6 of tid select the token m of the group, and a token past the
// group's n reads zero.
using Fetch = u4;

__device__ __forceinline__ void fetch_group(const BwdParams& p, const int h, const int t0, const int n, const int tid,
                                            const int wave, Fetch& x) {
  const int H = p.H;
  const size_t tok0 = static_cast<size_t>(t0) * H + h;
  const int m = (tid >> 5) & 3;
  if (wave < 4) {
    const uint32_t row = static_cast<uint32_t>(H) * BD * 2;
    const uint32_t nrec = (n - 1) * row + BD * 2;
    const bool kg = wave < 2;
    const Rsrc ra = rsrc((kg ? p.k : p.q) + tok0 * BD, nrec);
    const Rsrc rb = rsrc((kg ? p.g : p.v) + tok0 * BD, nrec);
    const int off = m * row + 8 * (tid & 31);
    const u2 a = __builtin_amdgcn_raw_buffer_load_b64(ra, off, 0, 0);
    const u2 b = __builtin_amdgcn_raw_buffer_load_b64(rb, off, 0, 0);
    x = u4{a[0], a[1], b[0], b[1]};
  } else if (wave < 6) {
    const uint32_t row = static_cast<uint32_t>(H) * BD * 4;
    const Rsrc rd = rsrc(p.d_o + tok0 * BD, (n - 1) * row + BD * 4);
    x = __builtin_amdgcn_raw_buffer_load_b128(rd, m * row + 16 * (tid & 31), 0, 0);
  } else if (wave == 6) {
    const uint32_t nb = (n - 1) * H * 2 + 2;
    const int lane = tid & 63;
    x[0] = __builtin_amdgcn_raw_buffer_load_b16(rsrc(p.beta + tok0, nb), lane < GT ? lane * H * 2 : nb, 0, 0);
  }
}

__device__ __forceinline__ void store_group(TokGroup& tg, const int n, const int tid, const int wave, const Fetch& x) {
  const int m = (tid >> 5) & 3;
  if (wave < 4) {
    if (m >= n) return;
    const int e = 4 * (tid & 31);
    const uint32_t wa[4] = {x[0] & 0xffffu, x[0] >> 16, x[1] & 0xffffu, x[1] >> 16};
    const uint32_t wb[4] = {x[2] & 0xffffu, x[2] >> 16, x[3] & 0xffffu, x[3] >> 16};
    if (wave < 2) {
      f4 kk, dc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kk[j] = bfv(wa[j]);
        dc[j] = __builtin_amdgcn_exp2f(bfv(wb[j]) * kLog2eB);
      }
      *reinterpret_cast<f4*>(&tg.k[m][e]) = kk;
      *reinterpret_cast<f4*>(&tg.dec[m][e]) = dc;
    } else {
      f4 qq, vv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qq[j] = bfv(wa[j]);
        vv[j] = bfv(wb[j]);
      }
      *reinterpret_cast<f4*>(&tg.q[m][e]) = qq;
      *reinterpret_cast<f4*>(&tg.v[m][e]) = vv;
    }
  } else if (wave < 6) {
    if (m < n) *reinterpret_cast<f4*>(&tg.dov[m][4 * (tid & 31)]) = __builtin_bit_cast(f4, x);
  } else if (wave == 6) {
    const int lane = tid & 63;
    if (lane < n) tg.beta[lane] = bfv(x[0]);
  }
}

// Keeps the scheduler from hoisting the LDS row loads of later steps above
// this point (with 16 waves per CU the load latency is hidden by the other
// waves; the registers are not).
__device__ __forceinline__ void slice_fence() { __builtin_amdgcn_sched_barrier(0); }

// s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maximum.  Called right
// after a state is loaded into registers that a loop then updates: the wait
// counter is in order and shared by loads and stores, and a loop whose
// registers may still hold a pending load from before it waits for every
// memory access of the wave (the loop's own prefetches and stores included)
// at their first use in each iteration.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int CTRL>
__device__ __forceinline__ float dpp(const float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Transposing butterfly: val(i) gives this lane's term of value i (16
// values, summed over the wave's 64 lanes).  Returns the full sum of value
// ridx(lane) = 8 b5 + 4 b4 + 2 b2 + b3 (b = the lane's bits); the four lanes
// that differ in bits 0-1 return the same value.  Each stage pairs lanes that
// still hold the same values and keeps half of them: lane bit 5 (rows of 32
// swapped), bit 4 (rows of 16 swapped), bit 2 (mirror within 8 lanes, which
// also flips bits 0-1), bit 3 (rotation by 8 within 16); then all-reduces
// over bits 0 and 1.  The flips generate all 64 lanes, each counted once.
// Values i and i + 8 are made together and folded at once.
__device__ __forceinline__ int ridx(const int lane) {
  return 8 * ((lane >> 5) & 1) + 4 * ((lane >> 4) & 1) + 2 * ((lane >> 2) & 1) + ((lane >> 3) & 1);
}

template <typename Val>
__device__ __forceinline__ float wave_rows_reduce(Val&& val, const int lane) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float lo = val(j), hi = val(j + 8);
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    x[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[j]), __float_as_uint(x[j + 4]), false, false);
    x[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool b2 = (lane & 4) != 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float a = x[j] + dpp<0x141>(x[j]);          // row_half_mirror
    const float b = x[j + 2] + dpp<0x141>(x[j + 2]);
    x[j] = b2 ? b : a;
  }
  const float a = x[0] + dpp<0x128>(x[0]);            // row_ror:8
  const float b = x[1] + dpp<0x128>(x[1]);
  float y = (lane & 8) ? b : a;
  y += dpp<0xB1>(y);                                  // quad_perm [1,0,3,2]
  y += dpp<0x4E>(y);                                  // quad_perm [2,3,0,1]
  return y;
}

// The thread's 16 elements of a [128][128] FP32 state at a uniform base:
// rows 16 grp + i, column c, i.e. byte offset voff + 512 i with
// voff = 4 (2048 grp + c).
__device__ __forceinline__ void load_state(const float* src, const int voff, float (&s)[NR]) {
  if (src == nullptr) {
#pragma unroll
    for (int i = 0; i < NR; ++i) s[i] = 0.f;
    return;
  }
  const Rsrc r = rsrc(src, MAT * 4);
#pragma unroll
  for (int i = 0; i < NR; ++i) s[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, i * 512, 0));
}
__device__ __forceinline__ void store_state(float* dst, const int voff, const float (&s)[NR]) {
  const Rsrc r = rsrc(dst, MAT * 4);
#pragma unroll
  for (int i = 0; i < NR; ++i) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s[i]), r, voff, i * 512, 0);
}
// Per-thread context of the forward launch: thread (c, grp) = (tid % 128,
// tid / 128) holds column c of rows [16 grp, 16 grp + 16) of the state.
struct FwdCtx {
  FwdSmem& sm;
  int tid, c, grp, lane, wave;   // grp and wave are wave-uniform
  int voff;  // byte offset of the thread's first state element, 4 (NR BD grp + c)

  __device__ FwdCtx(FwdSmem& s, const int t)
      : sm(s), tid(t), c(t & (BD - 1)), grp(__builtin_amdgcn_readfirstlane(t >> 7)), lane(t & 63),
        wave(__builtin_amdgcn_readfirstlane(t >> 6)), voff(4 * (NR * BD * (t >> 7) + (t & (BD - 1)))) {}
};

// The derived rows of the group of n tokens at token t0 of chunk cb: waves
// 0-1 one row each, wave 2 the six ap sums (two rows per lane, reduced by
// the butterfly).  Tokens t >= n count as k = 0, e^g = 1.
__device__ __forceinline__ void derive_rows(const FwdCtx& x, const FwdChunk& cb, const int t0, const int n) {
  FwdGroup& fg = x.sm.fg;
  if (x.wave < 2) {
    const int r = x.tid;
    float kv[GT], dv[GT];
#pragma unroll
    for (int t = 0; t < GT; ++t) {
      kv[t] = t < n ? cb.k[t0 + t][r] : 0.f;
      dv[t] = t < n ? cb.dec[t0 + t][r] : 1.f;
    }
    float gam = 1.f;
#pragma unroll
    for (int t = 0; t < GT; ++t) {
      gam *= dv[t];
      fg.gk[t][r] = kv[t] * gam;
    }
    fg.gamn[r] = gam;
    float suf = 1.f;
#pragma unroll
    for (int t = GT - 1; t >= 0; --t) {
      fg.kh[t][r] = kv[t] * suf;
      suf *= dv[t];
    }
  } else if (x.wave == 2) {
    float acc[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = 2 * x.lane + hh;
      float kv[GT], dv[GT];
#pragma unroll
      for (int t = 0; t < GT; ++t) {
        kv[t] = t < n ? cb.k[t0 + t][r] : 0.f;
        dv[t] = t < n ? cb.dec[t0 + t][r] : 1.f;
      }
#pragma unroll
      for (int t = 1; t < GT; ++t) {
        float d = 1.f;
#pragma unroll
        for (int j = t - 1; j >= 0; --j) {
          d *= dv[j + 1];
          acc[(t - 1) * t / 2 + j] = fmaf(kv[t] * kv[j], d, acc[(t - 1) * t / 2 + j]);
        }
      }
    }
    const float y = wave_rows_reduce([&](const int i) { return i < 6 ? acc[i] : 0.f; }, x.lane);
    const int i = ridx(x.lane);
    if ((x.lane & 3) == 0 && i < 6) fg.ap[i] = y;
  }
}

// The forward over the group (n tokens at token t0 of chunk cb) from S (its
// first state) to its last state, with every token's u and p of column c:
// one exchange for the four sums a_t = sum_r gk_t S
// (p_t = a_t + sum_{j<t} ap_tj u_j, u_t = beta_t (v_t - p_t)), then
// S <- Diag(gamn) S + sum_t kh_t u_t^T.  emit(t, u_t, p_t) for t < n;
// tokens t >= n get u = 0.
template <typename Emit>
__device__ __forceinline__ void fwd_group(FwdCtx& x, const FwdChunk& cb, const int t0, const int n, float (&s)[NR],
                                          Emit&& emit) {
  const FwdGroup& fg = x.sm.fg;
  const int r0 = NR * x.grp;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NR / 4; ++j) {
#pragma unroll
    for (int t = 0; t < GT; ++t) {
      const f4 kk = l4(&fg.gk[t][r0 + 4 * j]);
      acc[t] = fmaf(kk[0], s[4 * j], fmaf(kk[1], s[4 * j + 1], fmaf(kk[2], s[4 * j + 2], fmaf(kk[3], s[4 * j + 3], acc[t]))));
    }
  }
  x.sm.colpart4[x.grp][x.c] = acc;
  __syncthreads();
  f4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < NGRP; ++g) a += x.sm.colpart4[g][x.c];
  float u[GT];
#pragma unroll
  for (int t = 0; t < GT; ++t) {
    float pt = a[t];
#pragma unroll
    for (int j = 0; j < t; ++j) pt = fmaf(fg.ap[(t - 1) * t / 2 + j], u[j], pt);
    u[t] = t < n ? cb.beta[t0 + t] * (cb.v[t0 + t][x.c] - pt) : 0.f;
    if (t < n) emit(t, u[t], pt);
  }
#pragma unroll
  for (int j = 0; j < NR / 4; ++j) {
    const f4 gn = l4(&fg.gamn[r0 + 4 * j]);
    const f4 h0 = l4(&fg.kh[0][r0 + 4 * j]);
    const f4 h1 = l4(&fg.kh[1][r0 + 4 * j]);
    const f4 h2 = l4(&fg.kh[2][r0 + 4 * j]);
    const f4 h3 = l4(&fg.kh[3][r0 + 4 * j]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      s[4 * j + e] = fmaf(gn[e], s[4 * j + e], fmaf(h0[e], u[0], fmaf(h1[e], u[1], fmaf(h2[e], u[2], h3[e] * u[3]))));
  }
}

// A chunk's loads for the forward launch, in registers between their issue
// and their store to LDS: threads 0-511 k, 512-1023 g (token (tid / 32) % 16,
// four bf16 at 4 (tid % 32)); every thread v (token tid / 64, two bf16 at
// 2 (tid % 64)); threads 0-15 beta of token tid.  Tokens past the chunk's n
// read zero.  Every thread issues the same three loads.
__device__ __forceinline__ void fetch_chunk(const BwdParams& p, const int h, const int t0, const int n, const int tid,
                                            u4& x) {
  const uint32_t row = static_cast<uint32_t>(p.H) * BD * 2;
  const size_t tok0 = static_cast<size_t>(t0) * p.H + h;
  const uint32_t nrec = (n - 1) * row + BD * 2;
  const int m = (tid >> 5) & (CK - 1);
  const u2 a = __builtin_amdgcn_raw_buffer_load_b64(rsrc((tid >= NT / 2 ? p.g : p.k) + tok0 * BD, nrec),
                                                    m * row + 8 * (tid & 31), 0, 0);
  const uint32_t vv = __builtin_amdgcn_raw_buffer_load_b32(rsrc(p.v + tok0 * BD, nrec), (tid >> 6) * row + 4 * (tid & 63),
                                                           0, 0);
  const uint32_t nb = (n - 1) * p.H * 2 + 2;
  const uint32_t bb = __builtin_amdgcn_raw_buffer_load_b16(rsrc(p.beta + tok0, nb), tid < CK ? tid * p.H * 2 : nb, 0, 0);
  x = u4{a[0], a[1], vv, bb};
}

__device__ __forceinline__ void store_chunk(FwdChunk& cb, const int n, const int tid, const u4& x) {
  const int m = (tid >> 5) & (CK - 1);
  if (m < n) {
    const uint32_t w[4] = {x[0] & 0xffffu, x[0] >> 16, x[1] & 0xffffu, x[1] >> 16};
    f4 r;
    if (tid >= NT / 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = __builtin_amdgcn_exp2f(bfv(w[e]) * kLog2eB);
      *reinterpret_cast<f4*>(&cb.dec[m][4 * (tid & 31)]) = r;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = bfv(w[e]);
      *reinterpret_cast<f4*>(&cb.k[m][4 * (tid & 31)]) = r;
    }
  }
  const int mv = tid >> 6;
  if (mv < n) {
    cb.v[mv][2 * (tid & 63)] = bfv(x[2] & 0xffffu);
    cb.v[mv][2 * (tid & 63) + 1] = bfv(x[2] >> 16);
  }
  if (tid < n) cb.beta[tid] = bfv(x[3]);
}

// The reverse launch's layout: wave w owns the 32 x 32 block of rows from
// 32 (w / 4) and columns from 32 (w % 4); lane l of it the 4 x 4 block of
// rows R0 + i, R0 = 32 (w / 4) + 4 (l / 8), and columns C0 + j,
// C0 = 32 (w % 4) + 4 (l % 8), as s[4 i + j].  A sum over rows (du) is taken
// over the thread's four rows, the wave's eight row quads (lane swaps and a
// DPP move) and the four row blocks (LDS); a sum over columns (the rows of
// dq, dk, dg) over the thread's four columns, the wave's eight column quads
// (DPP moves) and the four column blocks (LDS).  Compared with a column of
// 16 rows per thread, three of every four additions of the per-token row
// sums happen inside the thread.
struct R4 {
  RevSmem& sm;
  int tid, lane, wave, rb, cb, R0, C0, voff;   // wave, rb and cb are wave-uniform
  int par;   // du exchange parity
  int gb;    // token-group buffer parity
  __device__ R4(RevSmem& s, const int t)
      : sm(s), tid(t), lane(t & 63), wave(__builtin_amdgcn_readfirstlane(t >> 6)), rb(wave >> 2), cb(wave & 3),
        R0(32 * rb + 4 * ((t & 63) >> 3)), C0(32 * cb + 4 * (t & 7)), voff(4 * (BD * R0 + C0)), par(0), gb(0) {}
};

// The thread's 16 elements of a row-major [128][128] FP32 state: row R0 + i
// at byte voff + 512 i, four columns per 16-byte access.
__device__ __forceinline__ void load4(const float* src, const int voff, float (&s)[16]) {
  if (src == nullptr) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
    return;
  }
  const Rsrc r = rsrc(src, MAT * 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f4 t = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 512 * i, 0));
#pragma unroll
    for (int j = 0; j < 4; ++j) s[4 * i + j] = t[j];
  }
}
__device__ __forceinline__ void add4(const float* src, const int voff, float (&s)[16]) {
  const Rsrc r = rsrc(src, MAT * 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f4 t = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 512 * i, 0));
#pragma unroll
    for (int j = 0; j < 4; ++j) s[4 * i + j] += t[j];
  }
}
__device__ __forceinline__ void store4(float* dst, const int voff, const float (&s)[16]) {
  const Rsrc r = rsrc(dst, MAT * 4);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(u4, f4{s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]}), r, voff, 512 * i, 0);
}

// S <- Diag(e^g) S + k u^T for the thread's block, from a token's k and e^g
// rows and its u (by column) in LDS.
__device__ __forceinline__ void update4(const R4& x, const float* krow, const float* drow, const float* urow,
                                        float (&s)[16]) {
  const f4 kk = l4(krow + x.R0), dc = l4(drow + x.R0), uu = l4(urow + x.C0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s[4 * i + j] = fmaf(dc[i], s[4 * i + j], kk[i] * uu[j]);
}

// Sum over the wave's eight row quads (lane bits 3-5) of four per-column
// values v[j]: returns that of j = 2 b5 + b4 (b = the lane's bits; lanes
// that differ in bit 3 agree).  Rows of 32 swapped (bit 5), rows of 16
// swapped (bit 4), rotation by 8 within 16 (bit 3).
__device__ __forceinline__ float sum_row_quads(const f4 v) {
  const auto r0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[2]), false, false);
  const auto r1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1]), __float_as_uint(v[3]), false, false);
  const float a = __uint_as_float(r0[0]) + __uint_as_float(r0[1]);
  const float b = __uint_as_float(r1[0]) + __uint_as_float(r1[1]);
  const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const float c = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
  return c + dpp<0x128>(c);   // row_ror:8
}

// Sum over the wave's eight column quads (lane bits 0-2) of four per-row
// values w[i]: returns that of i = 2 b2 + b1 (lanes that differ in bit 0
// agree).  Mirror within 8 lanes (pairs bit 2, also flips bits 0-1), then
// quad permutations for bits 1 and 0; the flips cover the eight lanes once.
__device__ __forceinline__ float sum_col_quads(const f4 w, const int lane) {
  const float a0 = w[0] + dpp<0x141>(w[0]);   // row_half_mirror
  const float a2 = w[2] + dpp<0x141>(w[2]);
  const float b0 = w[1] + dpp<0x141>(w[1]);
  const float b2 = w[3] + dpp<0x141>(w[3]);
  const bool hi2 = (lane & 4) != 0;
  const float a = hi2 ? a2 : a0;
  const float b = hi2 ? b2 : b0;
  const float ca = a + dpp<0x4E>(a);          // quad_perm [2,3,0,1]
  const float cb = b + dpp<0x4E>(b);
  const float c = (lane & 2) ? cb : ca;
  return c + dpp<0xB1>(c);                    // quad_perm [1,0,3,2]
}

// Sum of one value over the wave's eight column quads (every lane).
__device__ __forceinline__ float sum_col_quads1(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  return v + dpp<0x141>(v);
}

// The reverse step of token m (global index t) from S_{t-1} = st, with u and
// p of the thread's columns from the forward launch, in two parts around a
// pending tail: rev_begin adds q do^T and sums du over the rows (its exchange
// is the step's only barrier); rev_rest writes dv, publishes the row sums
// into rowpart[b] and red[b] and steps the cotangent back.  rev_tail (waves
// 0 and 1, one row each) turns a published token's sums into its dq, dk, dg
// and dbeta after a later barrier: the next token's exchange, or the barrier
// that ends a group.  Consecutive tokens alternate b.
__device__ __forceinline__ f4 rev_begin(R4& x, const TokGroup& tg, const int m, float (&ds)[16]) {
  const f4 qq = l4(&tg.q[m][x.R0]), kk = l4(&tg.k[m][x.R0]), dd = l4(&tg.dov[m][x.C0]);
  f4 pc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ds[4 * i + j] = fmaf(qq[i], dd[j], ds[4 * i + j]);
      pc[j] = fmaf(ds[4 * i + j], kk[i], pc[j]);
    }
  const float v = sum_row_quads(pc);
  float* cp = &x.sm.colpart[x.par][0][0];
  if ((x.lane & 8) == 0) cp[x.rb * BD + x.C0 + 2 * ((x.lane >> 5) & 1) + ((x.lane >> 4) & 1)] = v;
  __syncthreads();
  const f4 du = (l4(cp + x.C0) + l4(cp + BD + x.C0)) + (l4(cp + 2 * BD + x.C0) + l4(cp + 3 * BD + x.C0));
  x.par ^= 1;
  return du;
}

__device__ __forceinline__ void rev_rest(R4& x, const BwdParams& p, const int h, const TokGroup& tg, const int m,
                                         const int t, const float (&st)[16], float (&ds)[16], const f4 uu,
                                         const f4 pp, const f4 du, const int b) {
  const size_t tk = static_cast<size_t>(t) * p.H + h;
  const float beta = tg.beta[m];
  const f4 dd = l4(&tg.dov[m][x.C0]);
  const f4 dp = -beta * du;
  if (x.rb == 1) {   // waves 4-7, one per column block: dv, dbeta's and u.do's terms
    if (x.lane < 8)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, beta * du), rsrc(p.dv + tk * BD, BD * 4), 4 * x.C0,
                                             0, 0);
    const f4 vv = l4(&tg.v[m][x.C0]);
    float sb = 0.f, su = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sb = fmaf(du[j], vv[j] - pp[j], sb);
      su = fmaf(uu[j], dd[j], su);
    }
    sb = sum_col_quads1(sb);
    su = sum_col_quads1(su);
    if (x.lane == 0) {
      x.sm.red[b][0][x.cb] = sb;
      x.sm.red[b][1][x.cb] = su;
    }
  }
  // per row over the thread's columns: W = S do, X = S dp, Y = <S, dS>, Z = dS u;
  // the rows of dq, dk and dg need W, Z + e X and Y + k X
  const f4 kk = l4(&tg.k[m][x.R0]), ee = l4(&tg.dec[m][x.R0]);
  f4 w, q1, q2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float W = 0.f, X = 0.f, Y = 0.f, Z = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      W = fmaf(st[4 * i + j], dd[j], W);
      X = fmaf(st[4 * i + j], dp[j], X);
      Y = fmaf(st[4 * i + j], ds[4 * i + j], Y);
      Z = fmaf(ds[4 * i + j], uu[j], Z);
    }
    w[i] = W;
    q1[i] = fmaf(ee[i], X, Z);
    q2[i] = fmaf(kk[i], X, Y);
  }
  const float r0 = sum_col_quads(w, x.lane);
  const float r1 = sum_col_quads(q1, x.lane);
  const float r2 = sum_col_quads(q2, x.lane);
  if ((x.lane & 1) == 0) {
    const int row = x.R0 + 2 * ((x.lane >> 2) & 1) + ((x.lane >> 1) & 1);
    x.sm.rowpart[b][0][x.cb][row] = r0;
    x.sm.rowpart[b][1][x.cb][row] = r1;
    x.sm.rowpart[b][2][x.cb][row] = r2;
  }
  // dS_{t-1} = Diag(e^g) (dS + k dp^T)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) ds[4 * i + j] = ee[i] * fmaf(kk[i], dp[j], ds[4 * i + j]);
}

// dq = e^g (S_{t-1} do) + k (u . do), dk = dS u + e^g (S_{t-1} dp),
// dg = e^g rowsum(S_{t-1} o (dS + k dp^T)), dbeta = <du, v - p>.
__device__ __forceinline__ void rev_tail(const R4& x, const BwdParams& p, const int h, const TokGroup& tg, const int m,
                                         const int t, const int b) {
  if (x.wave >= 2) return;
  const size_t tk = static_cast<size_t>(t) * p.H + h;
  const int r = x.tid;
  const auto& rp = x.sm.rowpart[b];
  const float x1 = (rp[0][0][r] + rp[0][1][r]) + (rp[0][2][r] + rp[0][3][r]);
  const float x2 = (rp[1][0][r] + rp[1][1][r]) + (rp[1][2][r] + rp[1][3][r]);
  const float x3 = (rp[2][0][r] + rp[2][1][r]) + (rp[2][2][r] + rp[2][3][r]);
  const auto& rd = x.sm.red[b];
  const float ud = (rd[1][0] + rd[1][1]) + (rd[1][2] + rd[1][3]);
  const float dr = tg.dec[m][r], kr = tg.k[m][r];
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(fmaf(dr, x1, kr * ud)), rsrc(p.dq + tk * BD, BD * 4), 4 * r,
                                        0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x2), rsrc(p.dk + tk * BD, BD * 4), 4 * r, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dr * x3), rsrc(p.dg + tk * BD, BD * 4), 4 * r, 0, 0);
  if (r == 0) p.dbeta[tk] = (rd[0][0] + rd[0][1]) + (rd[0][2] + rd[0][3]);
}

}  // namespace

// E_r for every segment r and head: the cotangent at the start of segment r
// due to the outputs of its first fragment (and that fragment's dfinal when
// it ends a sequence) when nothing after the segment contributes.  Zero for a
// segment that does not continue a sequence.  One workgroup per (r, head).
//
// The cotangent-only step is short and its one exchange per token sets the
// pace.  With many (segment, head) items the launch uses small workgroups
// (256 threads, 64 rows of one column per thread), several per CU, whose
// chains overlap; with few, 1024-thread workgroups (16 rows per thread),
// whose chain per token is four times shorter.
namespace {
template <int ER>
struct alignas(16) ESmem {
  static constexpr int EG = BD / ER;
  float k[2][GT][BD];       // token vectors by group parity
  float dec[2][GT][BD];
  float q[2][GT][BD];
  float dov[2][GT][BD];
  float beta[2][GT];
  float colpart[2][EG][BD];
};

// Waves 0-1 load k and g (4 bf16 each), waves 2-3 q (4 bf16) and d_o (4
// floats), lanes 0-3 of wave 0 also beta; bits 5-6 of tid select the token.
struct EFetch {
  u4 a;
  f4 f;
  uint32_t beta;
};

__device__ __forceinline__ void efetch(const BwdParams& p, const int h, const int t0, const int n, const int tid,
                                       const int wave, EFetch& x) {
  if (wave >= 4) return;
  const int H = p.H;
  const size_t tok0 = static_cast<size_t>(t0) * H + h;
  const int m = (tid >> 5) & 3;
  const uint32_t row = static_cast<uint32_t>(H) * BD * 2;
  const uint32_t nrec = (n - 1) * row + BD * 2;
  const int off = m * row + 8 * (tid & 31);
  if (wave < 2) {
    const u2 a = __builtin_amdgcn_raw_buffer_load_b64(rsrc(p.k + tok0 * BD, nrec), off, 0, 0);
    const u2 b = __builtin_amdgcn_raw_buffer_load_b64(rsrc(p.g + tok0 * BD, nrec), off, 0, 0);
    x.a = u4{a[0], a[1], b[0], b[1]};
    if (wave == 0) {
      const uint32_t nb = (n - 1) * H * 2 + 2;
      const int lane = tid & 63;
      x.beta = __builtin_amdgcn_raw_buffer_load_b16(rsrc(p.beta + tok0, nb), lane < GT ? lane * H * 2 : nb, 0, 0);
    }
  } else {
    const u2 a = __builtin_amdgcn_raw_buffer_load_b64(rsrc(p.q + tok0 * BD, nrec), off, 0, 0);
    x.a = u4{a[0], a[1], 0u, 0u};
    const uint32_t rowf = static_cast<uint32_t>(H) * BD * 4;
    x.f = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(p.d_o + tok0 * BD, (n - 1) * rowf + BD * 4),
                                                                        m * rowf + 16 * (tid & 31), 0, 0));
  }
}

template <int ER>
__device__ __forceinline__ void estore(ESmem<ER>& sm, const int b, const int n, const int tid, const int wave,
                                       const EFetch& x) {
  if (wave >= 4) return;
  const int m = (tid >> 5) & 3;
  const int e = 4 * (tid & 31);
  if (wave == 0 && (tid & 63) < n) sm.beta[b][tid & 63] = bfv(x.beta);
  if (m >= n) return;
  const uint32_t wa[4] = {x.a[0] & 0xffffu, x.a[0] >> 16, x.a[1] & 0xffffu, x.a[1] >> 16};
  if (wave < 2) {
    const uint32_t wb[4] = {x.a[2] & 0xffffu, x.a[2] >> 16, x.a[3] & 0xffffu, x.a[3] >> 16};
    f4 kk, dc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kk[j] = bfv(wa[j]);
      dc[j] = __builtin_amdgcn_exp2f(bfv(wb[j]) * kLog2eB);
    }
    *reinterpret_cast<f4*>(&sm.k[b][m][e]) = kk;
    *reinterpret_cast<f4*>(&sm.dec[b][m][e]) = dc;
  } else {
    f4 qq;
#pragma unroll
    for (int j = 0; j < 4; ++j) qq[j] = bfv(wa[j]);
    *reinterpret_cast<f4*>(&sm.q[b][m][e]) = qq;
    *reinterpret_cast<f4*>(&sm.dov[b][m][e]) = x.f;
  }
}

template <int ER>
__device__ __forceinline__ void backward_summary(const BwdParams& p) {
  constexpr int EG = BD / ER;
  __shared__ ESmem<ER> sm;
  const int r = blockIdx.x / p.hn;
  const int h = p.h0 + blockIdx.x % p.hn;
  const int H = p.H;
  const int tid = threadIdx.x;
  const int c = tid & (BD - 1);
  const int grp = __builtin_amdgcn_readfirstlane(tid >> 7);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = ER * grp;
  const int voff = 4 * (ER * BD * grp + c);   // row r0 + i at + 512 i
  // the chunked launch took every segment except the carried ones whose
  // first fragment is on this path
  if (p.plan[p.L.seg_carry_in + r] == 0) return;
  if (p.iflag[static_cast<size_t>(p.plan[p.L.seg_frag_ptr + r]) * p.hn + (h - p.h0)] == 0) return;
  float ds[ER];
#pragma unroll
  for (int i = 0; i < ER; ++i) ds[i] = 0.f;
  {
    const int f = p.plan[p.L.seg_frag_ptr + r];
    const int32_t flags = p.plan[p.L.frag_flags + f];
    const int32_t seq = p.plan[p.L.frag_seq + f];
    const int32_t beg = p.plan[p.L.frag_begin + f];
    const int32_t end = p.plan[p.L.frag_end + f];
    if ((flags & kFragSeqEnd) && p.dfinal != nullptr) {
      const Rsrc rd = rsrc(p.dfinal + (static_cast<size_t>(seq) * H + h) * MAT, MAT * 4);
#pragma unroll
      for (int i = 0; i < ER; ++i) ds[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, voff, i * 512, 0));
    }
    const int ng = (end - beg + GT - 1) / GT;
    int gb = 0, par = 0;
    {
      EFetch f0;
      const int n0 = min(GT, end - beg - GT * (ng - 1));
      efetch(p, h, beg + GT * (ng - 1), n0, tid, wave, f0);
      estore(sm, 0, n0, tid, wave, f0);
    }
    for (int gi = ng - 1; gi >= 0; --gi) {
      EFetch fx;
      __syncthreads();
      const int n = min(GT, end - beg - GT * gi);
      if (gi > 0) efetch(p, h, beg + GT * (gi - 1), GT, tid, wave, fx);
#pragma unroll
      for (int m = GT - 1; m >= 0; --m) {
        if (m < n) {
          // dS += q do^T, du = dS^T k (rows), dS <- Diag(e^g) (dS + k dp^T)
          const float doc = sm.dov[gb][m][c];
          f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < ER / 4; ++j) {
            const f4 qq = l4(&sm.q[gb][m][r0 + 4 * j]);
            const f4 kk = l4(&sm.k[gb][m][r0 + 4 * j]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ds[4 * j + e] = fmaf(qq[e], doc, ds[4 * j + e]);
              acc[e] = fmaf(ds[4 * j + e], kk[e], acc[e]);
            }
          }
          sm.colpart[par][grp][c] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
          __syncthreads();
          float du = 0.f;
#pragma unroll
          for (int g2 = 0; g2 < EG; ++g2) du += sm.colpart[par][g2][c];
          par ^= 1;
          const float dp = -sm.beta[gb][m] * du;
#pragma unroll
          for (int j = 0; j < ER / 4; ++j) {
            const f4 kk = l4(&sm.k[gb][m][r0 + 4 * j]);
            const f4 dc = l4(&sm.dec[gb][m][r0 + 4 * j]);
#pragma unroll
            for (int e = 0; e < 4; ++e) ds[4 * j + e] = dc[e] * fmaf(kk[e], dp, ds[4 * j + e]);
          }
        }
      }
      if (gi > 0) estore(sm, gb ^ 1, GT, tid, wave, fx);
      gb ^= 1;
    }
  }
  const Rsrc re = rsrc(p.esum + (static_cast<size_t>(r) * H + h) * MAT, MAT * 4);
#pragma unroll
  for (int i = 0; i < ER; ++i) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ds[i]), re, voff, i * 512, 0);
}
}  // namespace

__global__ void __launch_bounds__(kBwdThreads, 4) kda_backward_summary_kernel(BwdParams p) {
  backward_summary<BD * BD / kBwdThreads>(p);
}

__global__ void __launch_bounds__(kBwdSummaryThreads) kda_backward_summary_narrow_kernel(BwdParams p) {
  backward_summary<BD * BD / kBwdSummaryThreads>(p);
}

// Per (fragment, head) item: the item's fields, its checkpoint and u/p
// addressing, and the group prefetch (shared by the two fragment launches).
struct Item {
  int32_t flags, seg, seq, beg, len, ng, nch, top, h;
  bool chunked;   // on the chunked path (not this one)
  float* ck;   // checkpoint of chunk j at ck + j H MAT
  __device__ Item(const BwdParams& p, const int item) {
    const int f = p.plan[p.L.frag_order + item / p.hn];
    h = p.h0 + item % p.hn;
    chunked = p.iflag[static_cast<size_t>(f) * p.hn + item % p.hn] == 0;
    flags = p.plan[p.L.frag_flags + f];
    seg = p.plan[p.L.frag_seg + f];
    seq = p.plan[p.L.frag_seq + f];
    beg = p.plan[p.L.frag_begin + f];
    len = p.plan[p.L.frag_end + f] - beg;
    ng = (len + GT - 1) / GT;          // 4-token groups
    nch = (len + CK - 1) / CK;         // 16-token chunks
    top = ng - GPC * (nch - 1);        // groups of the last chunk
    ck = p.ckpt + (static_cast<size_t>(beg / CK + f) * p.H + h) * MAT;
  }
  __device__ int gtokens(const int g) const { return min(GT, len - GT * g); }
  // [u | p] of token t (1 KiB per token and head)
  __device__ float* up_base(const BwdParams& p, const int t) const {
    return p.upbuf + (static_cast<size_t>(t) * p.H + h) * 2 * BD;
  }
};

// One token group: wait for its vectors, prefetch group gn's (gn < 0: none),
// run body(tg, n), then store the prefetch for the next group.
template <typename Body>
__device__ __forceinline__ void token_group(R4& x, const BwdParams& p, const Item& it, const int g, const int gn,
                                            Body&& body) {
  Fetch fx;
  __syncthreads();
  if (gn >= 0) fetch_group(p, it.h, it.beg + GT * gn, it.gtokens(gn), x.tid, x.wave, fx);
  body(x.sm.tg[x.gb], it.gtokens(g));
  if (gn >= 0) store_group(x.sm.tg[x.gb ^ 1], it.gtokens(gn), x.tid, x.wave, fx);
  x.gb ^= 1;
}

// Every (fragment, head) item, forward from the fragment's start state
// (carry-in C_r for a carried fragment, else the initial state or zero): the
// state at the start of every 16-token chunk (row-major) and every
// token's u and p, for the reverse launch.  Four tokens per exchange; a
// chunk's inputs are loaded during the chunk before it, so the launch waits
// for global memory once per chunk (the wait counter is in order: a wait
// for a load also waits for every store issued before it).  Persistent:
// workgroup b takes items b, b + grid, ... in the plan's longest-first order.
__global__ void __launch_bounds__(kBwdThreads, 1) kda_backward_forward_kernel(BwdParams p) {
  __shared__ FwdSmem sm;
  const int items = p.plan[3] * p.hn;
  FwdCtx x(sm, threadIdx.x);
  const size_t up_token = static_cast<size_t>(p.H) * 2 * BD;   // floats between tokens
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const Item it(p, item);
    if (it.chunked) continue;
    auto ctokens = [&](const int j) { return min(CK, it.len - CK * j); };
    float run[NR];
    {
      const float* s0 = nullptr;
      if (it.flags & kFragCarried) s0 = p.carry + (static_cast<size_t>(it.seg) * p.H + it.h) * MAT;
      else if (p.h0s != nullptr) s0 = p.h0s + (static_cast<size_t>(it.seq) * p.H + it.h) * MAT;
      load_state(s0, x.voff, run);
    }
    __syncthreads();   // the previous item's reads of both chunk buffers are done
    {
      u4 f0;
      fetch_chunk(p, it.h, it.beg, ctokens(0), x.tid, f0);
      store_chunk(sm.ch[0], ctokens(0), x.tid, f0);
    }
    wait_vmem();
    for (int j = 0; j < it.nch; ++j) {
      const int nj = ctokens(j);
      const FwdChunk& cb = sm.ch[j & 1];
      u4 fx;
      __syncthreads();   // chunk j's rows are in LDS; chunk j - 1's reads of the other buffer are done
      if (j + 1 < it.nch) fetch_chunk(p, it.h, it.beg + CK * (j + 1), ctokens(j + 1), x.tid, fx);
      store_state(it.ck + static_cast<size_t>(j) * p.H * MAT, x.voff, run);
      for (int gl = 0; GT * gl < nj; ++gl) {
        const int n = min(GT, nj - GT * gl);
        if (gl > 0) __syncthreads();   // every read of the previous group's derived rows is done
        derive_rows(x, cb, GT * gl, n);
        __syncthreads();
        const int t0 = it.beg + CK * j + GT * gl;
        const Rsrc ru = rsrc(it.up_base(p, t0), (n - 1) * up_token * 4 + 2 * BD * 4);
        fwd_group(x, cb, GT * gl, n, run, [&](const int m, const float u, const float pp) {
          if (x.wave < 2) {
            const int o = static_cast<int>(m * up_token * 4) + 4 * x.c;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(u), ru, o, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pp), ru, o + 4 * BD, 0, 0);
          }
        });
      }
      if (j + 1 < it.nch) store_chunk(sm.ch[(j + 1) & 1], ctokens(j + 1), x.tid, fx);
    }
  }
}

// Every (fragment, head) item, backwards from its end: the cotangent starts
// from D_r (when the fragment ends its segment) plus dfinal (when it ends its
// sequence); a fragment that starts its sequence writes what reaches that
// start to dh0.  Per 4-token group from the last: its first state is
// recomputed from its chunk's checkpoint by update-only steps with the u
// that the forward launch kept (no exchange; the chunk's k, e^g and u held
// in LDS), the state before its token m from that by m more, then the
// reverse steps.  Persistent, in the forward launch's item order.
__global__ void __launch_bounds__(kBwdThreads, 1) kda_backward_fragment_kernel(BwdParams p) {
  __shared__ RevSmem sm;
  const int items = p.plan[3] * p.hn;
  const int tid = threadIdx.x;
  R4 x(sm, tid);
  const size_t up_token = static_cast<size_t>(p.H) * 2 * BD;   // floats between tokens

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const Item it(p, item);
    if (it.chunked) continue;
    const int h = it.h;
    // Chunk j's k and e^g rows (threads 0-511 k, 512-1023 g: token
    // (tid / 32) % 16, four values each) and its tokens' u and p (64 threads
    // per token, 16 bytes each) into LDS.  Called after every read of the
    // previous chunk's rows: the next group's barrier publishes them.
    auto load_chunk = [&](const int j) {
      const int t0 = it.beg + CK * j;
      const int n = min(CK, it.len - CK * j);
      const int m = (tid >> 5) & (CK - 1);
      const bool isg = tid >= NT / 2;
      const uint32_t row = static_cast<uint32_t>(p.H) * BD * 2;
      const size_t tok0 = static_cast<size_t>(t0) * p.H + h;
      const u2 kg = __builtin_amdgcn_raw_buffer_load_b64(rsrc((isg ? p.g : p.k) + tok0 * BD, (n - 1) * row + BD * 2),
                                                         m * row + 8 * (tid & 31), 0, 0);
      const int mu = tid >> 6;
      const u4 uv = __builtin_amdgcn_raw_buffer_load_b128(
          rsrc(it.up_base(p, t0), (n - 1) * up_token * 4 + 2 * BD * 4), static_cast<int>(mu * up_token * 4) + 16 * (tid & 63),
          0, 0);
      const uint32_t w[4] = {kg[0] & 0xffffu, kg[0] >> 16, kg[1] & 0xffffu, kg[1] >> 16};
      f4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = isg ? __builtin_amdgcn_exp2f(bfv(w[e]) * kLog2eB) : bfv(w[e]);
      *reinterpret_cast<f4*>(isg ? &sm.ckd[m][4 * (tid & 31)] : &sm.ckk[m][4 * (tid & 31)]) = r;
      *reinterpret_cast<f4*>(&sm.upc[mu][0][0] + 4 * (tid & 63)) = __builtin_bit_cast(f4, uv);
    };

    float ds[16];   // the cotangent at the fragment's end
    if (it.flags & kFragSegLast) {
      load4(p.dcarry + (static_cast<size_t>(it.seg) * p.H + h) * MAT, x.voff, ds);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) ds[e] = 0.f;
    }
    if ((it.flags & kFragSeqEnd) && p.dfinal != nullptr)
      add4(p.dfinal + (static_cast<size_t>(it.seq) * p.H + h) * MAT, x.voff, ds);
    wait_vmem();
    __syncthreads();   // the previous item's reads of both token buffers and the chunk rows are done
    {
      Fetch f0;
      fetch_group(p, h, it.beg + GT * (it.ng - 1), it.gtokens(it.ng - 1), tid, x.wave, f0);
      store_group(sm.tg[x.gb], it.gtokens(it.ng - 1), tid, x.wave, f0);
    }
    load_chunk(it.nch - 1);

    float run[16];
    for (int j = it.nch - 1; j >= 0; --j) {
      const int g0 = GPC * j;
      const int g1 = g0 + (j == it.nch - 1 ? it.top : GPC);   // the chunk's groups [g0, g1)
      const float* ckj = it.ck + static_cast<size_t>(j) * p.H * MAT;
      for (int g = g1 - 1; g >= g0; --g) {
        token_group(x, p, it, g, g - 1, [&](const TokGroup& tg, const int n) {
          float w[16];
          load4(ckj, x.voff, run);
          for (int q = 0; q < GT * (g - g0); ++q) update4(x, sm.ckk[q], sm.ckd[q], sm.upc[q][0], run);
          const int t0 = it.beg + GT * g;
          const int q0 = GT * (g - g0);   // the group's first token in the chunk
#pragma unroll
          for (int e = 0; e < 16; ++e) w[e] = run[e];
#pragma unroll
          for (int m = 0; m + 1 < GT; ++m)
            if (m + 1 < n) update4(x, tg.k[m], tg.dec[m], sm.upc[q0 + m][0], w);
#pragma unroll
          for (int m = GT - 1; m >= 0; --m) {
            if (m < n) {
              if (m + 1 < n) {
#pragma unroll
                for (int e = 0; e < 16; ++e) w[e] = run[e];
#pragma unroll
                for (int q = 0; q < m; ++q) update4(x, tg.k[q], tg.dec[q], sm.upc[q0 + q][0], w);
              }
              const f4 du = rev_begin(x, tg, m, ds);
              if (m + 1 < n) rev_tail(x, p, h, tg, m + 1, t0 + m + 1, (m + 1) & 1);   // published before the barrier above
              rev_rest(x, p, h, tg, m, t0 + m, w, ds, l4(&sm.upc[q0 + m][0][x.C0]), l4(&sm.upc[q0 + m][1][x.C0]), du,
                       m & 1);
            }
          }
          __syncthreads();
          rev_tail(x, p, h, tg, 0, t0, 0);
        });
      }
      if (j > 0) load_chunk(j - 1);   // every read of chunk j's rows ended at the barrier above
    }
    if (!(it.flags & kFragCarried) && p.dh0 != nullptr)
      store4(p.dh0 + (static_cast<size_t>(it.seq) * p.H + h) * MAT, x.voff, ds);
  }
}

}  // namespace kda
