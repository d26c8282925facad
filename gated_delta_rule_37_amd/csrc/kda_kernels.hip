// HIP kernels (gfx950) of the segmented KDA forward pass.
//
// Sources: inclusionAI/cuLA pull request #110 "feat(cp): add opt-in NVSHMEM CP
// state handoff" (Motivation: affine recurrence state per producer, one merge
// kernel per consumer; Supported configuration: BF16 inputs, FP32 state,
// non-transposed state layout) and pull request #136 "feat(kda): add cuDNN
// concatenated-summary Kimi CP" (Summary: preceding_state_update /
// preceding_transition, affine composition in FP32).
//
// Per head the state S is K x V (K = V = 128), K-major.  One token applies
//     S <- (I - beta k k^T) Diag(exp g) S + beta k v^T,   o = S^T q.
// Chunked form used here (chunk of C = 32 tokens, G_i = in-chunk prefix sum of
// g up to token i, all exponent arithmetic in log2 units):
//     A[i][j] = beta_i sum_d k_id k_jd e^{G_id - G_jd}     (j < i)
//     T       = (I + A)^{-1}                              (unit lower triangular)
//     U       = T diag(beta) (V - (K o e^G) S)            (the delta-rule targets)
//     O       = (Q o e^G) S + P U,  P[i][j] = sum_d q_id k_jd e^{G_id - G_jd} (j <= i)
//     S      <- Diag(e^{G_C}) S + K^^T U,  K^[j][d] = k_jd e^{G_Cd - G_jd}
// The exponential factors are split around one anchor per chunk (token 15):
// Kr = k e^{G-a}, Kc = k e^{a-G}, Qr = q e^{G-a}, so every in-chunk pair
// (i, j) sees e^{G_i - G_j} = e^{G_i - a} e^{a - G_j} with each factor bounded
// by the decay mass of at most 16 tokens.  Then (K o e^G) S = Kr (e^a o S),
// (Q o e^G) S = Qr (e^a o S) and K^ = e^{G_C - a} o Kc.
//
// Precision: every product that feeds the state uses split bfloat16
// operands x = x_hi + x_lo on the bf16 matrix cores (three MFMAs:
// hi*hi + hi*lo + lo*hi, FP32 accumulation), which carries about 16
// significant bits per operand; raw BF16 inputs (v) are exact and need one
// split side only.  The state itself stays FP32 in accumulator registers.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_internal.h"
#include "kda_kernels.h"

namespace kda {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KD = 128;   // key dimension
constexpr int VD = 128;   // value dimension
constexpr int CH = 32;    // chunk length (tokens)
constexpr int NT = kChunkThreads;     // chunk kernel: 8 waves of 64
constexpr int NTC = kComposeThreads;  // compose kernel: 4 waves of 64
constexpr int NS = 136;   // row stride (bf16) of token-major [32][128] tiles
constexpr int TS = 40;    // row stride (bf16) of channel-major [128][32] tiles
constexpr int FS = 36;    // row stride (fp32) of the 32 x 32 triangular-solve tiles
constexpr int XS = 20;    // row stride (fp32) of the 16 x 16 off-diagonal product
constexpr float kLog2e = 1.4426950408889634f;
// Buffer resource word 3 for gfx9 raw (unswizzled, 32-bit) buffer access;
// accesses at or past num_records read zero and drop writes.
constexpr int kBufDword3 = 0x00020000;

enum Mode { kModeFwd = 0, kModeSumS = 1, kModeSumPhi = 2 };

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ void split(float x, bf16& hi, bf16& lo) {
  hi = static_cast<bf16>(x);
  lo = static_cast<bf16>(x - static_cast<float>(hi));
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// acc += a * b with split operands (hi*hi + hi*lo + lo*hi).
__device__ __forceinline__ f32x16 mfma3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                        const bf16x8& bl, f32x16 acc) {
  acc = mfma(ah, bh, acc);
  acc = mfma(ah, bl, acc);
  acc = mfma(al, bh, acc);
  return acc;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc += a * b (16x16x32) with split operands (hi*hi + hi*lo + lo*hi).
__device__ __forceinline__ f32x4 mfma16x3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                          const bf16x8& bl, f32x4 acc) {
  acc = mfma16(ah, bh, acc);
  acc = mfma16(ah, bl, acc);
  acc = mfma16(al, bh, acc);
  return acc;
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0.f;
  return z;
}

// Wait states between an MFMA that wrote t0/t1 and the permlane swaps that read
// them.  The compiler does not always pad this dependency (seen when the last
// MFMA of a chain sits in another basic block), and a swap that reads the
// registers early picks up the accumulator without its last product.  The
// swaps consume the asm's outputs, so they cannot be scheduled before it; 20
// wait states cover a 16-pass MFMA.
__device__ __forceinline__ void mfma_result_fence(f32x4& t0, f32x4& t1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(t0), "+v"(t1));
}
__device__ __forceinline__ void mfma_result_fence(f32x16& t) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(t));
}

// Two 16 x 16 accumulator tiles t0 (rows 0..15) and t1 (rows 16..31) hold, in
// lane l and register e, rows 4(l/16) + e of column l%16.  A B operand of the
// 16x16x32 MFMA needs rows 8(l/16) + 0..7 of one column per lane.  A 32-lane
// swap of (t0, t1) followed by a 16-lane swap regroups them (checked on gfx950:
// permlane32_swap(x, y) -> (x_lo|y_lo, x_hi|y_hi); permlane16_swap(x, y) ->
// (x0 y0 x2 y2, x1 y1 x3 y3) by 16-lane rows).
__device__ __forceinline__ void tiles16_to_b(const f32x4& t0, const f32x4& t1, float out[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(t0[e]), __float_as_uint(t1[e]), false, false);
    const auto q = __builtin_amdgcn_permlane16_swap(p[0], p[1], false, false);
    out[e] = __uint_as_float(q[0]);
    out[4 + e] = __uint_as_float(q[1]);
  }
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// A 32 x 32 accumulator tile holds, in lane l and register 4r+e, the element
// (row 8r + 4(l/32) + e, column l%32).  A B operand of the 32x32x16 MFMA needs
// rows 16s + 8(l/32) + 0..7 of one column per lane.  Swapping the upper half of
// register group 2s with the lower half of group 2s+1 across the two 32-lane
// halves regroups them: out[0..3] = rows 16s + 8h + 0..3, out[4..7] = the next
// four.
__device__ __forceinline__ void tile_rows_to_b(const f32x16& t, int s, float out[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t x = __float_as_uint(t[4 * (2 * s) + e]);
    const uint32_t y = __float_as_uint(t[4 * (2 * s + 1) + e]);
    const auto p = __builtin_amdgcn_permlane32_swap(x, y, false, false);
    out[e] = __uint_as_float(p[0]);
    out[4 + e] = __uint_as_float(p[1]);
  }
}

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Split two floats into packed (hi, lo) bf16 pairs: x = hi + lo to ~16 bits.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  bf16x2 h;
  h[0] = static_cast<bf16>(x0);
  h[1] = static_cast<bf16>(x1);
  bf16x2 l;
  l[0] = static_cast<bf16>(x0 - static_cast<float>(h[0]));
  l[1] = static_cast<bf16>(x1 - static_cast<float>(h[1]));
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

__device__ __forceinline__ void split8(const float x[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16 a, b;
    split(x[e], a, b);
    hi[e] = a;
    lo[e] = b;
  }
}

struct ChunkSmem {
  bf16 kr_h[CH * NS], kr_l[CH * NS];   // Kr = k e^{G-a}, token-major
  bf16 kc_h[CH * NS], kc_l[CH * NS];   // Kc = k e^{a-G}, token-major
  bf16 qr_h[CH * NS], qr_l[CH * NS];   // Qr = q e^{G-a}, token-major
  bf16 kht_h[KD * TS], kht_l[KD * TS]; // K^ = k e^{G_C - G}, channel-major
  bf16 vt[VD * TS];                    // V, channel-major (exact)
  bf16 tb_h[CH * TS], tb_l[CH * TS];   // T diag(beta), [i][j]
  bf16 p_h[CH * TS], p_l[CH * TS];     // P, [i][j]
  float at[CH * FS];                   // at[j][i] = A[i][j]
  float an[CH * FS];                   // an[i][j] = A[i][j]
  float tt[CH * FS];                   // tt[c][i] = T[i][c] (diagonal blocks)
  float tn[CH * FS];                   // tn[i][c] = T[i][c] (diagonal blocks)
  float xt[16 * XS];                   // X = A10 T00, stored xt[c][i]
  float tot[8 * KD];                   // per 4-token group gate sums
  float ea[KD];                        // e^{a}
  float gam[KD];                       // e^{G_C}
  float beta[CH];
};

struct Work {
  int mode;         // Mode, or -1 for none
  bool from_carry;  // FWD starting from carry_in[seg]
  bool zero_a;      // write a zero transition and stop
};

__device__ __forceinline__ Work decode_work(const ChunkParams& p, int32_t flags, int32_t seg) {
  Work w{-1, false, false};
  const int role = blockIdx.z;
  if (p.pass == 1) {
    if (role == 0) {
      if (flags & kFragCarried) {
        if (flags & kFragSegLast) w.mode = kModeSumS;
      } else {
        w.mode = kModeFwd;
      }
    } else if (flags & kFragSegLast) {
      if (p.plan[p.L.seg_transition_live + seg]) w.mode = kModeSumPhi;
      else w.zero_a = true;
    }
  } else {
    if (flags & kFragCarried) {
      w.mode = kModeFwd;
      w.from_carry = true;
    }
  }
  return w;
}

}  // namespace

// The body for one fragment, specialised on the mode so that the unrolled
// chunk loop carries no mode branches (branches would split it into many
// basic blocks and keep the scheduler from running operand loads ahead).
template <int MODE>
__device__ __forceinline__ void run_fragment(const ChunkParams& p, ChunkSmem& sm, const int f,
                                             const int32_t flags, const int32_t seg,
                                             const int32_t seq, const int32_t beg,
                                             const int32_t end, const bool from_carry) {
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  // wave index, made provably uniform so that wave-derived addresses and
  // buffer resources live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lm = lane & 15;   // 16x16x32 MFMA: row/column index of this lane
  const int lg = lane >> 4;   // 16x16x32 MFMA: k-group / row group of this lane
  const int H = p.H;
  constexpr int mode = MODE;
  constexpr bool fwd = MODE == kModeFwd;
  constexpr bool use_v = MODE != kModeSumPhi;
  const int col = 16 * wave + lm;

  // ---- initial state: tile dt, register e holds row 16dt + 4lg + e
  f32x4 S[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) S[dt] = zero4();
  if (mode == kModeSumPhi) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) S[dt][e] = (16 * dt + 4 * lg + e == col) ? 1.f : 0.f;
    }
  } else if (from_carry) {
    const float* src = p.carry + (static_cast<size_t>(seg) * H + h) * KD * VD + col;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) S[dt][e] = src[(16 * dt + 4 * lg + e) * VD];
    }
  }

  // P0 thread layout: wave w handles tokens 4w .. 4w+3 of the chunk, lane l
  // channels 2l and 2l+1 (so every token row is one coalesced 256-byte read).
  const int cp = lane;
  const int tg = wave;
  const int row_bytes = H * KD * 2;                       // one token of q, k, g, v
  const int in_voff = (4 * tg) * row_bytes + 4 * cp;      // this thread's first element
  const int o_row = H * VD * 4;                           // one token of o (bytes)
  const int o_voff = (4 * lg) * o_row + 4 * col;

  // raw BF16 pairs of the chunk being prefetched (registers, one chunk ahead);
  // buffer loads past the fragment's last token return zero
  uint32_t rk[4], rg[4], rq[4], rv[4];
  uint32_t rb = 0u;   // beta's raw bits: converted only when used, so that no
                      // wait on the prefetch is forced inside fetch()
  // Branch-free, so that the loads and the use of the previous chunk's
  // registers share one basic block: loads a mode does not need, and loads
  // past the fragment, get a zero-size buffer (they return zero and touch no
  // memory).
  auto fetch = [&](int cs) {
    const int nn = min(CH, end - cs);
    const size_t base = (static_cast<size_t>(min(cs, end - 1)) * H + h) * KD;
    const int nrec = nn > 0 ? (nn - 1) * row_bytes + KD * 2 : 0;
    const auto rsk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.k + base), 0, nrec, kBufDword3);
    const auto rsg = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.g + base), 0, nrec, kBufDword3);
    const auto rsq =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.q + base), 0, fwd ? nrec : 0, kBufDword3);
    const auto rsv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.v + base), 0, use_v ? nrec : 0, kBufDword3);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int off = in_voff + m * row_bytes;
      rk[m] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rsk, off, 0, 0));
      rg[m] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rsg, off, 0, 0));
      rq[m] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rsq, off, 0, 0));
      rv[m] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rsv, off, 0, 0));
    }
    // beta: wave 0's first 32 lanes read one value per token
    const int nb = (tg == 0 && nn > 0) ? (nn - 1) * H * 2 + 2 : 0;
    const auto rsb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.beta + static_cast<size_t>(min(cs, end - 1)) * H + h), 0, nb, kBufDword3);
    rb = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rsb, lane < CH ? lane * H * 2 : nb, 0, 0));
  };
  fetch(beg);

  for (int c0 = beg; c0 < end; c0 += CH) {
    const int n = min(CH, end - c0);

    // ================= P0: gate prefix and the derived operands of the chunk
    float kf[4][2], qf[4][2], G[4][2];
    uint32_t vcur[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      kf[m][0] = __uint_as_float(rk[m] << 16);
      kf[m][1] = __uint_as_float(rk[m] & 0xffff0000u);
      qf[m][0] = __uint_as_float(rq[m] << 16);
      qf[m][1] = __uint_as_float(rq[m] & 0xffff0000u);
      G[m][0] = __uint_as_float(rg[m] << 16) * kLog2e;
      G[m][1] = __uint_as_float(rg[m] & 0xffff0000u) * kLog2e;
      vcur[m] = rv[m];
    }
    if (tg == 0 && lane < CH) sm.beta[lane] = __uint_as_float(rb << 16);
    // Consume the prefetched registers before the next prefetch is issued: the
    // q/v/beta loads are conditional, so if the scheduler hoisted the new loads
    // above these uses, the inserted memory wait would have to cover the
    // shortest load path and stall on the new loads.
    __builtin_amdgcn_sched_barrier(0);
    fetch(c0 + CH);
#pragma unroll
    for (int m = 1; m < 4; ++m) {
      G[m][0] += G[m - 1][0];
      G[m][1] += G[m - 1][1];
    }
    *reinterpret_cast<float2*>(&sm.tot[tg * KD + 2 * cp]) = make_float2(G[3][0], G[3][1]);
    __syncthreads();

    // prefix of the earlier token groups, the anchor a = G at token 15 (end of
    // group 3) and G_C = G at the last token, all summed in group order
    float pre[2] = {0.f, 0.f}, a[2] = {0.f, 0.f}, gc[2] = {0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float2 tv = *reinterpret_cast<const float2*>(&sm.tot[t * KD + 2 * cp]);
      if (t == tg) { pre[0] = gc[0]; pre[1] = gc[1]; }
      if (t == 4) { a[0] = gc[0]; a[1] = gc[1]; }
      gc[0] += tv.x;
      gc[1] += tv.y;
    }
    const float shift[2] = {pre[0] - a[0], pre[1] - a[1]};
    const float ega[2] = {__builtin_amdgcn_exp2f(gc[0] - a[0]), __builtin_amdgcn_exp2f(gc[1] - a[1])};
    if (tg == 0) {
      *reinterpret_cast<float2*>(&sm.ea[2 * cp]) =
          make_float2(__builtin_amdgcn_exp2f(a[0]), __builtin_amdgcn_exp2f(a[1]));
      *reinterpret_cast<float2*>(&sm.gam[2 * cp]) =
          make_float2(__builtin_amdgcn_exp2f(gc[0]), __builtin_amdgcn_exp2f(gc[1]));
    }

    // per element: Kr = k e^{G-a}, Kc = k e^{a-G}, K^ = Kc e^{G_C-a}, Qr = q e^{G-a}
    uint32_t khh[2][2], khl[2][2];
    float kh_prev[2] = {0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float kr[2], kc[2], kh[2], qr[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float x = G[m][c] + shift[c];
        const float er = __builtin_amdgcn_exp2f(x);
        const float ec = __builtin_amdgcn_exp2f(-x);
        kr[c] = kf[m][c] * er;
        kc[c] = kf[m][c] * ec;
        kh[c] = kc[c] * ega[c];
        qr[c] = qf[m][c] * er;
      }
      const int i = 4 * tg + m;
      uint32_t hh, ll;
      split_pair(kr[0], kr[1], hh, ll);
      *reinterpret_cast<uint32_t*>(&sm.kr_h[i * NS + 2 * cp]) = hh;
      *reinterpret_cast<uint32_t*>(&sm.kr_l[i * NS + 2 * cp]) = ll;
      split_pair(kc[0], kc[1], hh, ll);
      *reinterpret_cast<uint32_t*>(&sm.kc_h[i * NS + 2 * cp]) = hh;
      *reinterpret_cast<uint32_t*>(&sm.kc_l[i * NS + 2 * cp]) = ll;
      if (fwd) {
        split_pair(qr[0], qr[1], hh, ll);
        *reinterpret_cast<uint32_t*>(&sm.qr_h[i * NS + 2 * cp]) = hh;
        *reinterpret_cast<uint32_t*>(&sm.qr_l[i * NS + 2 * cp]) = ll;
      }
      // K^ packed along tokens (channel-major layout): pairs (m-1, m)
      if (m & 1) {
        split_pair(kh_prev[0], kh[0], khh[m >> 1][0], khl[m >> 1][0]);
        split_pair(kh_prev[1], kh[1], khh[m >> 1][1], khl[m >> 1][1]);
      } else {
        kh_prev[0] = kh[0];
        kh_prev[1] = kh[1];
      }
    }
    // channel-major rows d = 2cp + c, tokens 4tg .. 4tg+3 (8 bytes each)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int d = 2 * cp + c;
      const uint32_t sel = c == 0 ? 0x05040100u : 0x07060302u;  // low / high halves
      *reinterpret_cast<uint2*>(&sm.kht_h[d * TS + 4 * tg]) = make_uint2(khh[0][c], khh[1][c]);
      *reinterpret_cast<uint2*>(&sm.kht_l[d * TS + 4 * tg]) = make_uint2(khl[0][c], khl[1][c]);
      if (use_v) {
        *reinterpret_cast<uint2*>(&sm.vt[d * TS + 4 * tg]) =
            make_uint2(__builtin_amdgcn_perm(vcur[1], vcur[0], sel), __builtin_amdgcn_perm(vcur[3], vcur[2], sel));
      }
    }
    __syncthreads();

    // ================= P1: A (waves 0, 1) and P (waves 2, 3) by 16-row blocks
    // (the all-zero block above the diagonal is not computed)
    if (wave < 2 || (wave < 4 && fwd)) {
      const int rb = wave & 1;                  // row block: rows 16rb .. 16rb+15
      const bool is_a = wave < 2;
      const bf16* xh = is_a ? sm.kr_h : sm.qr_h;
      const bf16* xl = is_a ? sm.kr_l : sm.qr_l;
      f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
      for (int kk = 0; kk < KD / 32; ++kk) {
        const int aoff = (16 * rb + lm) * NS + 32 * kk + 8 * lg;
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&xh[aoff]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&xl[aoff]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          if (ct > rb) continue;
          const int boff = (16 * ct + lm) * NS + 32 * kk + 8 * lg;
          acc[ct] = mfma16x3(ah, al, *reinterpret_cast<const bf16x8*>(&sm.kc_h[boff]),
                             *reinterpret_cast<const bf16x8*>(&sm.kc_l[boff]), acc[ct]);
        }
      }
      mfma_result_fence(acc[0], acc[1]);
      // tile ct holds rows i = 16rb + 4lg + e of column j = 16ct + lm
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int j = 16 * ct + lm;
        const int i0 = 16 * rb + 4 * lg;
        if (is_a) {
          if (ct > rb) continue;
          float4 v4;
          float* vp = reinterpret_cast<float*>(&v4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            const float x = (j < i) ? sm.beta[i] * acc[ct][e] : 0.f;
            vp[e] = x;
            sm.an[i * FS + j] = x;
          }
          *reinterpret_cast<float4*>(&sm.at[j * FS + i0]) = v4;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            const float x = (ct <= rb && j <= i) ? acc[ct][e] : 0.f;
            bf16 hh, ll;
            split(x, hh, ll);
            sm.p_h[i * TS + j] = hh;
            sm.p_l[i * TS + j] = ll;
          }
        }
      }
    }
    __syncthreads();

    // Y = Kr (e^a o S) and O = Qr (e^a o S), this wave's 16 columns; the
    // state is scaled and split into B operands one 32-row k-step at a time
    f32x4 Y[2] = {zero4(), zero4()};
    f32x4 O[2] = {zero4(), zero4()};
    auto state_products = [&]() {
#pragma unroll
      for (int kk = 0; kk < KD / 32; ++kk) {
        float x[8];
        tiles16_to_b(S[2 * kk], S[2 * kk + 1], x);
        const float4 e0 = *reinterpret_cast<const float4*>(&sm.ea[32 * kk + 8 * lg]);
        const float4 e1 = *reinterpret_cast<const float4*>(&sm.ea[32 * kk + 8 * lg + 4]);
        x[0] *= e0.x; x[1] *= e0.y; x[2] *= e0.z; x[3] *= e0.w;
        x[4] *= e1.x; x[5] *= e1.y; x[6] *= e1.z; x[7] *= e1.w;
        bf16x8 sbh, sbl;
        split8(x, sbh, sbl);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const int off = (16 * rt + lm) * NS + 32 * kk + 8 * lg;
          Y[rt] = mfma16x3(*reinterpret_cast<const bf16x8*>(&sm.kr_h[off]),
                           *reinterpret_cast<const bf16x8*>(&sm.kr_l[off]), sbh, sbl, Y[rt]);
          if (fwd) {
            O[rt] = mfma16x3(*reinterpret_cast<const bf16x8*>(&sm.qr_h[off]),
                             *reinterpret_cast<const bf16x8*>(&sm.qr_l[off]), sbh, sbl, O[rt]);
          }
        }
      }
    };

    // ================= P2: diagonal blocks of T (wave 0), state products (rest)
    if (wave == 0) {
      if (lane < 32) {
        const int b = lane >> 4;   // diagonal block
        const int c = lane & 15;   // column of the block solved by this lane
        const int base = 16 * b;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const float* arow = &sm.at[(base + jj) * FS + base];
#pragma unroll
          for (int q4 = jj / 4; q4 < 4; ++q4) {
            const float4 t4 = *reinterpret_cast<const float4*>(&arow[4 * q4]);
            const float av[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * q4 + e;
              if (i > jj) x[i] -= av[e] * x[jj];
            }
          }
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          *reinterpret_cast<float4*>(&sm.tt[(base + c) * FS + base + 4 * q4]) =
              make_float4(x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.tn[(base + i) * FS + base + c] = x[i];
      }
    } else {
      state_products();
    }
    __syncthreads();

    // ================= P2b: T10 = -T11 A10 T00 and T diag(beta) (wave 5);
    // wave 0's state products meanwhile.  Wave 5 exchanges X through LDS with
    // itself only, and a wave's LDS accesses complete in order, so no barrier
    // is needed between writing X and reading it back.
    if (wave == 5) {
      // lane: column tc of the block, rows ti = 4qq + (lane / 16), qq = 0..3.
      // Every operand row is loaded whole with independent 16-byte reads.
      const int tc = lane & 15;
      const int tr = lane >> 4;
      float tcol[16];   // T00[:, tc] (row tc of tt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 v4 = *reinterpret_cast<const float4*>(&sm.tt[tc * FS + 4 * q4]);
        tcol[4 * q4] = v4.x; tcol[4 * q4 + 1] = v4.y; tcol[4 * q4 + 2] = v4.z; tcol[4 * q4 + 3] = v4.w;
      }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int ti = 4 * qq + tr;
        float arow[16];   // A10[ti, :]
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v4 = *reinterpret_cast<const float4*>(&sm.an[(16 + ti) * FS + 4 * q4]);
          arow[4 * q4] = v4.x; arow[4 * q4 + 1] = v4.y; arow[4 * q4 + 2] = v4.z; arow[4 * q4 + 3] = v4.w;
        }
        float xs = 0.f;
#pragma unroll
        for (int kx = 0; kx < 16; ++kx) xs += arow[kx] * tcol[kx];
        sm.xt[tc * XS + ti] = xs;   // X = A10 T00, stored by column
      }
      // the wave's own LDS writes complete in order before its later reads
      float xcol[16];   // X[:, tc]
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 v4 = *reinterpret_cast<const float4*>(&sm.xt[tc * XS + 4 * q4]);
        xcol[4 * q4] = v4.x; xcol[4 * q4 + 1] = v4.y; xcol[4 * q4 + 2] = v4.z; xcol[4 * q4 + 3] = v4.w;
      }
      const float b0 = sm.beta[tc];
      const float b1 = sm.beta[16 + tc];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int ti = 4 * qq + tr;
        float trow[16];   // T11[ti, :]
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v4 = *reinterpret_cast<const float4*>(&sm.tn[(16 + ti) * FS + 16 + 4 * q4]);
          trow[4 * q4] = v4.x; trow[4 * q4 + 1] = v4.y; trow[4 * q4 + 2] = v4.z; trow[4 * q4 + 3] = v4.w;
        }
        float t10 = 0.f;
#pragma unroll
        for (int kx = 0; kx < 16; ++kx) t10 -= trow[kx] * xcol[kx];
        bf16 hh, ll;
        split(sm.tn[ti * FS + tc] * b0, hh, ll);
        sm.tb_h[ti * TS + tc] = hh;
        sm.tb_l[ti * TS + tc] = ll;
        split(trow[tc] * b1, hh, ll);
        sm.tb_h[(16 + ti) * TS + 16 + tc] = hh;
        sm.tb_l[(16 + ti) * TS + 16 + tc] = ll;
        split(t10 * b0, hh, ll);
        sm.tb_h[(16 + ti) * TS + tc] = hh;
        sm.tb_l[(16 + ti) * TS + tc] = ll;
        sm.tb_h[ti * TS + 16 + tc] = static_cast<bf16>(0.f);
        sm.tb_l[ti * TS + 16 + tc] = static_cast<bf16>(0.f);
      }
    } else if (wave == 0) {
      state_products();
    }
    __syncthreads();

    // ================= P3: U = T diag(beta) (V - Y), O += P U, state update
    // Land the next chunk's prefetch here, most of a chunk after it was issued:
    // the empty asm takes the registers as operands, so the memory wait is
    // placed before it and none is left for the next chunk's first use.
    asm volatile("" : "+v"(rk[0]), "+v"(rk[1]), "+v"(rk[2]), "+v"(rk[3]), "+v"(rg[0]), "+v"(rg[1]),
                 "+v"(rg[2]), "+v"(rg[3]), "+v"(rq[0]), "+v"(rq[1]), "+v"(rq[2]), "+v"(rq[3]),
                 "+v"(rv[0]), "+v"(rv[1]), "+v"(rv[2]), "+v"(rv[3]), "+v"(rb));
    f32x4 U[2] = {zero4(), zero4()};
    {
      f32x4 D[2];
      mfma_result_fence(Y[0], Y[1]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        float vv[4] = {0.f, 0.f, 0.f, 0.f};
        if (use_v) {
          const uint2 v2 = *reinterpret_cast<const uint2*>(&sm.vt[col * TS + 16 * rt + 4 * lg]);
          vv[0] = __uint_as_float(v2.x << 16);
          vv[1] = __uint_as_float(v2.x & 0xffff0000u);
          vv[2] = __uint_as_float(v2.y << 16);
          vv[3] = __uint_as_float(v2.y & 0xffff0000u);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) D[rt][e] = vv[e] - Y[rt][e];
      }
      float x[8];
      tiles16_to_b(D[0], D[1], x);
      bf16x8 dbh, dbl;
      split8(x, dbh, dbl);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int off = (16 * rt + lm) * TS + 8 * lg;
        U[rt] = mfma16x3(*reinterpret_cast<const bf16x8*>(&sm.tb_h[off]),
                         *reinterpret_cast<const bf16x8*>(&sm.tb_l[off]), dbh, dbl, U[rt]);
      }
    }
    bf16x8 ubh, ubl;
    {
      float x[8];
      mfma_result_fence(U[0], U[1]);
      tiles16_to_b(U[0], U[1], x);
      split8(x, ubh, ubl);
    }
    if (fwd) {
      // rows past the fragment's end fall outside the buffer and are dropped
      const auto rso = __builtin_amdgcn_make_buffer_rsrc(
          p.o + (static_cast<size_t>(c0) * H + h) * VD, 0, (n - 1) * o_row + 4 * VD, kBufDword3);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int off = (16 * rt + lm) * TS + 8 * lg;
        O[rt] = mfma16x3(*reinterpret_cast<const bf16x8*>(&sm.p_h[off]),
                         *reinterpret_cast<const bf16x8*>(&sm.p_l[off]), ubh, ubl, O[rt]);
      }
      mfma_result_fence(O[0], O[1]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // (an element of an ext_vector goes through a scalar first:
          // __builtin_bit_cast on the element reads element 0)
          const float ov = O[rt][e];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(ov), rso, o_voff + (16 * rt + e) * o_row,
                                                0, 0);
        }
      }
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const float4 e4 = *reinterpret_cast<const float4*>(&sm.gam[16 * dt + 4 * lg]);
      S[dt][0] *= e4.x;
      S[dt][1] *= e4.y;
      S[dt][2] *= e4.z;
      S[dt][3] *= e4.w;
      const int off = (16 * dt + lm) * TS + 8 * lg;
      S[dt] = mfma16x3(*reinterpret_cast<const bf16x8*>(&sm.kht_h[off]),
                       *reinterpret_cast<const bf16x8*>(&sm.kht_l[off]), ubh, ubl, S[dt]);
    }
    // The next chunk's first barrier orders its LDS writes after every read
    // of this chunk: before that barrier it writes only tot and beta, which
    // P3 does not read.  The state tiles are read next at least a P0 and two
    // barriers later, far past the MFMA result latency.
  }

  // ---- the fragment's final state
  float* dst0 = nullptr;
  float* dst1 = nullptr;
  if (mode == kModeSumPhi) {
    dst0 = p.transitions + (static_cast<size_t>(seg) * H + h) * KD * KD;
  } else if (mode == kModeSumS) {
    dst0 = p.updates + (static_cast<size_t>(seg) * H + h) * KD * VD;
  } else {
    if (flags & kFragSeqEnd) dst0 = p.final_state + (static_cast<size_t>(seq) * H + h) * KD * VD;
    if (p.pass == 1 && (flags & kFragSegLast))
      dst1 = p.updates + (static_cast<size_t>(seg) * H + h) * KD * VD;
  }
#pragma unroll
  for (int dt = 0; dt < 8; dt += 2) mfma_result_fence(S[dt], S[dt + 1]);
  if (dst0) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst0[(16 * dt + 4 * lg + e) * VD + col] = S[dt][e];
  }
  if (dst1) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst1[(16 * dt + 4 * lg + e) * VD + col] = S[dt][e];
  }
}


// One workgroup runs one fragment (a run of tokens of one sequence inside one
// segment) of one head, chunk after chunk, holding the state in registers.
// Eight waves; wave w owns state columns [16w, 16w + 16) as eight 16 x 16 FP32
// accumulator tiles.
//
// Per chunk:
//   P0  (all)      load (prefetched one chunk ahead), gate prefix, Kr, Kc, Qr
//                  (token-major) and K^, V (channel-major) into LDS
//   P1  (waves 0-3) A = beta o (Kr Kc^T) and P = Qr Kc^T, 16 x 16 tiles
//   P2  wave 0 lanes 0-31: diagonal 16 x 16 blocks of T = (I + A)^{-1};
//       every other wave meanwhile: Y = Kr (e^a o S) and O = Qr (e^a o S)
//   P2b wave 5: off-diagonal block of T and T diag(beta); wave 0: its Y, O
//   P3  (all)      U = T diag(beta) (V - Y), O += P U, S <- e^{G_C} o S + K^^T U
// using W S = T diag(beta) (K o e^G) S, K o e^G = e^a o Kr, Q o e^G = e^a o Qr.
__global__ void __launch_bounds__(NT, 1) kda_chunk_kernel(ChunkParams p) {
  __shared__ ChunkSmem sm;
  const int f = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int H = p.H;

  const int32_t flags = p.plan[p.L.frag_flags + f];
  const int32_t seg = p.plan[p.L.frag_seg + f];
  const int32_t seq = p.plan[p.L.frag_seq + f];
  const int32_t beg = p.plan[p.L.frag_begin + f];
  const int32_t end = p.plan[p.L.frag_end + f];
  const Work work = decode_work(p, flags, seg);

  if (work.zero_a) {
    float4* dst = reinterpret_cast<float4*>(p.transitions + (static_cast<size_t>(seg) * H + h) * KD * KD);
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = tid; i < KD * KD / 4; i += NT) dst[i] = z;
    return;
  }
  if (work.mode == kModeFwd) {
    run_fragment<kModeFwd>(p, sm, f, flags, seg, seq, beg, end, work.from_carry);
  } else if (work.mode == kModeSumS) {
    run_fragment<kModeSumS>(p, sm, f, flags, seg, seq, beg, end, work.from_carry);
  } else if (work.mode == kModeSumPhi) {
    run_fragment<kModeSumPhi>(p, sm, f, flags, seg, seq, beg, end, work.from_carry);
  }
}

// Ordered scan C_0 = 0, C_{r+1} = A_r C_r + B_r for one head and one block of
// 32 state columns.  Wave w computes rows [32w, 32w + 32); the current carry
// is shared through LDS as split B operands.
__global__ void __launch_bounds__(NTC, 1) kda_compose_kernel(ComposeParams p) {
  __shared__ bf16x8 cbh[8][64];
  __shared__ bf16x8 cbl[8][64];
  const int h = blockIdx.x;
  const int cb = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int lh = lane >> 5;
  const int H = p.H;
  const int col = 32 * cb + ln;

  f32x16 cur = zero16();
  for (int r = 0; r < p.S; ++r) {
    float* cdst = p.carry + (static_cast<size_t>(r) * H + h) * KD * VD;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 0; e < 4; ++e) cdst[(32 * wave + 8 * q + 4 * lh + e) * VD + col] = cur[4 * q + e];
    }
    if (r == p.S - 1) break;
    const float* bsrc = p.updates + (static_cast<size_t>(r) * H + h) * KD * VD;
    f32x16 nxt;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 0; e < 4; ++e) nxt[4 * q + e] = bsrc[(32 * wave + 8 * q + 4 * lh + e) * VD + col];
    }
    if (p.plan[p.L.seg_transition_live + r]) {
      mfma_result_fence(cur);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float x[8];
        tile_rows_to_b(cur, s, x);
        split8(x, cbh[2 * wave + s][lane], cbl[2 * wave + s][lane]);
      }
      __syncthreads();
      const float* arow = p.transitions + ((static_cast<size_t>(r) * H + h) * KD + 32 * wave + ln) * KD;
#pragma unroll
      for (int kk = 0; kk < KD / 16; ++kk) {
        const float4 x0 = *reinterpret_cast<const float4*>(&arow[16 * kk + 8 * lh]);
        const float4 x1 = *reinterpret_cast<const float4*>(&arow[16 * kk + 8 * lh + 4]);
        const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        bf16x8 ah, al;
        split8(xv, ah, al);
        nxt = mfma3(ah, al, cbh[kk][lane], cbl[kk][lane], nxt);
      }
      __syncthreads();
    }
    cur = nxt;
  }
}

}  // namespace kda
