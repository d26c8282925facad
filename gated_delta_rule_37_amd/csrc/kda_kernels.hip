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
//     W       = T diag(beta) (K o e^G)                    U~ = T diag(beta) V
//     U       = U~ - W S
//     O       = (Q o e^G) S + P U,  P[i][j] = sum_d q_id k_jd e^{G_id - G_jd} (j <= i)
//     S      <- Diag(e^{G_C}) S + K^^T U,  K^[j][d] = k_jd e^{G_Cd - G_jd}
// The exponential factors are split around one anchor per chunk (token 15):
// Kr = k e^{G-a}, Kc = k e^{a-G}, Qr = q e^{G-a}, so every in-chunk pair
// (i, j) sees e^{G_i - G_j} = e^{G_i - a} e^{a - G_j} with each factor bounded
// by the decay mass of at most 16 tokens.  Then W = e^a o (T diag(beta) Kr)
// (column scaling), K^ = e^{G_C - a} o Kc, and the state update becomes
//     S <- e^{G_C - a} o (e^a o S + Kc^T U)              (row scalings).
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
constexpr int NT = 256;   // threads per workgroup (4 waves of 64)
constexpr int NS = 136;   // row stride (bf16) of token-major [32][128] tiles
constexpr int TS = 40;    // row stride (bf16) of channel-major [128][32] tiles
constexpr int FS = 36;    // row stride (fp32) of the 32 x 32 triangular-solve tiles
constexpr float kLog2e = 1.4426950408889634f;

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
  bf16 kr_h[CH * NS], kr_l[CH * NS];   // Kr, token-major; holds -W after the A product
  bf16 kc_h[CH * NS], kc_l[CH * NS];   // Kc, token-major
  bf16 qr_h[CH * NS], qr_l[CH * NS];   // Qr, token-major
  bf16 qg_h[CH * NS], qg_l[CH * NS];   // Q o e^G, token-major
  bf16 krt_h[KD * TS], krt_l[KD * TS]; // Kr, channel-major
  bf16 kct_h[KD * TS], kct_l[KD * TS]; // Kc, channel-major
  bf16 vt[VD * TS];                    // V, channel-major (exact)
  bf16 tb_h[CH * TS], tb_l[CH * TS];   // T diag(beta), [i][j]
  bf16 p_h[CH * TS], p_l[CH * TS];     // P, [i][j]
  float at[CH * FS];                   // at[j][i] = A[i][j]
  float an[CH * FS];                   // an[i][j] = A[i][j]
  float tt[CH * FS];                   // tt[c][i] = T[i][c] (diagonal blocks)
  float tn[CH * FS];                   // tn[i][c] = T[i][c] (diagonal blocks)
  float xt[16 * 17];                   // X = A10 T00, stored xt[c][i]
  float tot[8 * KD];                   // per 4-token group gate sums
  float ea[KD];                        // e^{a}
  float ega[KD];                       // e^{G_C - a}
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

// One workgroup runs one fragment (a run of tokens of one sequence inside one
// segment) of one head, chunk after chunk, holding the state in registers.
// Wave w owns state columns [32w, 32w + 32).
__global__ void __launch_bounds__(NT, 1) kda_chunk_kernel(ChunkParams p) {
  __shared__ ChunkSmem sm;
  const int f = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 31;   // MFMA row/column index of this lane
  const int lh = lane >> 5;   // MFMA half (k-group) of this lane
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
  if (work.mode < 0) return;
  const int mode = work.mode;
  const bool fwd = mode == kModeFwd;
  const bool use_v = mode != kModeSumPhi;

  // ---- initial state: accumulator tile dt holds rows 32dt + 8r + 4lh + e
  f32x16 S[4];
  const int col = 32 * wave + ln;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 32 * dt + 8 * r + 4 * lh + e;
        float x = 0.f;
        if (mode == kModeSumPhi) x = (d == col) ? 1.f : 0.f;
        else if (work.from_carry)
          x = p.carry[((static_cast<size_t>(seg) * H + h) * KD + d) * VD + col];
        S[dt][4 * r + e] = x;
      }
    }
  }

  const int cg = tid & 31;   // channel group: channels 4cg .. 4cg+3
  const int tg = tid >> 5;   // token group: tokens 4tg .. 4tg+3 of the chunk

  for (int c0 = beg; c0 < end; c0 += CH) {
    const int n = min(CH, end - c0);

    // ================= P0: load the chunk, gate prefix, derived operands
    float kf[4][4], qf[4][4], G[4][4];
    uint16_t vb[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = 4 * tg + m;
      uint2 kk = make_uint2(0, 0), qq = make_uint2(0, 0), gg = make_uint2(0, 0),
            vv = make_uint2(0, 0);
      if (i < n) {
        const size_t row = (static_cast<size_t>(c0 + i) * H + h) * KD + 4 * cg;
        kk = *reinterpret_cast<const uint2*>(p.k + row);
        gg = *reinterpret_cast<const uint2*>(p.g + row);
        if (fwd) qq = *reinterpret_cast<const uint2*>(p.q + row);
        if (use_v) vv = *reinterpret_cast<const uint2*>(p.v + row);
      }
      const uint16_t ks[4] = {static_cast<uint16_t>(kk.x & 0xffff), static_cast<uint16_t>(kk.x >> 16),
                              static_cast<uint16_t>(kk.y & 0xffff), static_cast<uint16_t>(kk.y >> 16)};
      const uint16_t qs[4] = {static_cast<uint16_t>(qq.x & 0xffff), static_cast<uint16_t>(qq.x >> 16),
                              static_cast<uint16_t>(qq.y & 0xffff), static_cast<uint16_t>(qq.y >> 16)};
      const uint16_t gs[4] = {static_cast<uint16_t>(gg.x & 0xffff), static_cast<uint16_t>(gg.x >> 16),
                              static_cast<uint16_t>(gg.y & 0xffff), static_cast<uint16_t>(gg.y >> 16)};
      vb[m][0] = static_cast<uint16_t>(vv.x & 0xffff);
      vb[m][1] = static_cast<uint16_t>(vv.x >> 16);
      vb[m][2] = static_cast<uint16_t>(vv.y & 0xffff);
      vb[m][3] = static_cast<uint16_t>(vv.y >> 16);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kf[m][c] = bf2f(ks[c]);
        qf[m][c] = bf2f(qs[c]);
        G[m][c] = bf2f(gs[c]) * kLog2e;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      G[1][c] += G[0][c];
      G[2][c] += G[1][c];
      G[3][c] += G[2][c];
    }
    *reinterpret_cast<float4*>(&sm.tot[tg * KD + 4 * cg]) = make_float4(G[3][0], G[3][1], G[3][2], G[3][3]);
    if (tid < CH) {
      sm.beta[tid] = (tid < n) ? bf2f(p.beta[static_cast<size_t>(c0 + tid) * H + h]) : 0.f;
    }
    __syncthreads();

    float pre[4] = {0.f, 0.f, 0.f, 0.f}, a[4], gc[4];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float4 v4 = *reinterpret_cast<const float4*>(&sm.tot[t * KD + 4 * cg]);
      const float vals[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (t < tg) pre[c] += vals[c];
      }
    }
    // anchor a = G at token 15 and G_C = G at the chunk's last token, summed
    // in the same order as the per-thread prefixes
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) s += sm.tot[t * KD + 4 * cg + c];
      a[c] = s;
#pragma unroll
      for (int t = 4; t < 8; ++t) s += sm.tot[t * KD + 4 * cg + c];
      gc[c] = s;
    }
    float eac[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      eac[c] = exp2f(a[c]);
#pragma unroll
      for (int m = 0; m < 4; ++m) G[m][c] += pre[c];
    }
    if (tg == 0) {
      *reinterpret_cast<float4*>(&sm.ea[4 * cg]) = make_float4(eac[0], eac[1], eac[2], eac[3]);
      *reinterpret_cast<float4*>(&sm.ega[4 * cg]) =
          make_float4(exp2f(gc[0] - a[0]), exp2f(gc[1] - a[1]), exp2f(gc[2] - a[2]), exp2f(gc[3] - a[3]));
    }

    bf16 krh[4][4], krl[4][4], kch[4][4], kcl[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      bf16x4 w_krh, w_krl, w_kch, w_kcl, w_qrh, w_qrl, w_qgh, w_qgl;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float x = G[m][c] - a[c];
        const float er = exp2f(x);
        const float ec = exp2f(-x);
        split(kf[m][c] * er, krh[m][c], krl[m][c]);
        split(kf[m][c] * ec, kch[m][c], kcl[m][c]);
        w_krh[c] = krh[m][c];
        w_krl[c] = krl[m][c];
        w_kch[c] = kch[m][c];
        w_kcl[c] = kcl[m][c];
        if (fwd) {
          const float qr = qf[m][c] * er;
          bf16 hh, ll;
          split(qr, hh, ll);
          w_qrh[c] = hh;
          w_qrl[c] = ll;
          split(qr * eac[c], hh, ll);
          w_qgh[c] = hh;
          w_qgl[c] = ll;
        }
      }
      const int i = 4 * tg + m;
      *reinterpret_cast<bf16x4*>(&sm.kr_h[i * NS + 4 * cg]) = w_krh;
      *reinterpret_cast<bf16x4*>(&sm.kr_l[i * NS + 4 * cg]) = w_krl;
      *reinterpret_cast<bf16x4*>(&sm.kc_h[i * NS + 4 * cg]) = w_kch;
      *reinterpret_cast<bf16x4*>(&sm.kc_l[i * NS + 4 * cg]) = w_kcl;
      if (fwd) {
        *reinterpret_cast<bf16x4*>(&sm.qr_h[i * NS + 4 * cg]) = w_qrh;
        *reinterpret_cast<bf16x4*>(&sm.qr_l[i * NS + 4 * cg]) = w_qrl;
        *reinterpret_cast<bf16x4*>(&sm.qg_h[i * NS + 4 * cg]) = w_qgh;
        *reinterpret_cast<bf16x4*>(&sm.qg_l[i * NS + 4 * cg]) = w_qgl;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = 4 * cg + c;
      bf16x4 t_krh, t_krl, t_kch, t_kcl, t_v;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        t_krh[m] = krh[m][c];
        t_krl[m] = krl[m][c];
        t_kch[m] = kch[m][c];
        t_kcl[m] = kcl[m][c];
        t_v[m] = __builtin_bit_cast(bf16, vb[m][c]);
      }
      *reinterpret_cast<bf16x4*>(&sm.krt_h[d * TS + 4 * tg]) = t_krh;
      *reinterpret_cast<bf16x4*>(&sm.krt_l[d * TS + 4 * tg]) = t_krl;
      *reinterpret_cast<bf16x4*>(&sm.kct_h[d * TS + 4 * tg]) = t_kch;
      *reinterpret_cast<bf16x4*>(&sm.kct_l[d * TS + 4 * tg]) = t_kcl;
      if (use_v) *reinterpret_cast<bf16x4*>(&sm.vt[d * TS + 4 * tg]) = t_v;
    }
    __syncthreads();

    // ================= P1: A = beta (Kr Kc^T) (wave 0) and P = Qr Kc^T (wave 1)
    if (wave == 0 || (wave == 1 && fwd)) {
      const bf16* xh = wave == 0 ? sm.kr_h : sm.qr_h;
      const bf16* xl = wave == 0 ? sm.kr_l : sm.qr_l;
      f32x16 acc = zero16();
#pragma unroll
      for (int kk = 0; kk < KD / 16; ++kk) {
        const int off = ln * NS + 16 * kk + 8 * lh;
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&xh[off]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&xl[off]);
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&sm.kc_h[off]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&sm.kc_l[off]);
        acc = mfma3(ah, al, bh, bl, acc);
      }
      // lane holds rows i = 8r + 4lh + e of column j = ln
      const int j = ln;
      if (wave == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float4 v4;
          float* vp = reinterpret_cast<float*>(&v4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 8 * r + 4 * lh + e;
            const float x = (j < i) ? sm.beta[i] * acc[4 * r + e] : 0.f;
            vp[e] = x;
            sm.an[i * FS + j] = x;
          }
          *reinterpret_cast<float4*>(&sm.at[j * FS + 8 * r + 4 * lh]) = v4;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 8 * r + 4 * lh + e;
            const float x = (j <= i) ? acc[4 * r + e] : 0.f;
            bf16 hh, ll;
            split(x, hh, ll);
            sm.p_h[i * TS + j] = hh;
            sm.p_l[i * TS + j] = ll;
          }
        }
      }
    }

    // every wave: its state columns as split B operands (rows of S = k index)
    bf16x8 sbh[8], sbl[8];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float x[8];
        tile_rows_to_b(S[dt], s, x);
        split8(x, sbh[2 * dt + s], sbl[2 * dt + s]);
      }
    }
    __syncthreads();

    // ================= P2: T = (I + A)^{-1} by 16 x 16 blocks
    if (wave == 0 && lane < 32) {
      const int b = lane >> 4;   // diagonal block
      const int c = lane & 15;   // column of the block solved by this lane
      const int base = 16 * b;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const float* arow = &sm.at[(base + jj) * FS + base];
        float av[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 t4 = *reinterpret_cast<const float4*>(&arow[4 * q4]);
          av[4 * q4 + 0] = t4.x;
          av[4 * q4 + 1] = t4.y;
          av[4 * q4 + 2] = t4.z;
          av[4 * q4 + 3] = t4.w;
        }
#pragma unroll
        for (int i = jj + 1; i < 16; ++i) x[i] -= av[i] * x[jj];
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        *reinterpret_cast<float4*>(&sm.tt[(base + c) * FS + base + 4 * q4]) =
            make_float4(x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.tn[(base + i) * FS + base + c] = x[i];
    }
    __syncthreads();
    const int ti = tid >> 4;   // row within a 16 x 16 block
    const int tc = tid & 15;   // column within a 16 x 16 block
    {
      float xs = 0.f;
#pragma unroll
      for (int kx = 0; kx < 16; ++kx) xs += sm.an[(16 + ti) * FS + kx] * sm.tt[tc * FS + kx];
      sm.xt[tc * 17 + ti] = xs;
    }
    __syncthreads();
    {
      float t10 = 0.f;
#pragma unroll
      for (int kx = 0; kx < 16; ++kx) t10 -= sm.tn[(16 + ti) * FS + 16 + kx] * sm.xt[tc * 17 + kx];
      const float b0 = sm.beta[tc];
      const float b1 = sm.beta[16 + tc];
      bf16 hh, ll;
      split(sm.tn[ti * FS + tc] * b0, hh, ll);
      sm.tb_h[ti * TS + tc] = hh;
      sm.tb_l[ti * TS + tc] = ll;
      split(sm.tn[(16 + ti) * FS + 16 + tc] * b1, hh, ll);
      sm.tb_h[(16 + ti) * TS + 16 + tc] = hh;
      sm.tb_l[(16 + ti) * TS + 16 + tc] = ll;
      split(t10 * b0, hh, ll);
      sm.tb_h[(16 + ti) * TS + tc] = hh;
      sm.tb_l[(16 + ti) * TS + tc] = ll;
      sm.tb_h[ti * TS + 16 + tc] = static_cast<bf16>(0.f);
      sm.tb_l[ti * TS + 16 + tc] = static_cast<bf16>(0.f);
    }
    __syncthreads();

    // ================= P3: -W (token-major, into kr_*) and U~ = T diag(beta) V
    {
      f32x16 acc = zero16();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int aoff = (32 * wave + ln) * TS + 16 * s + 8 * lh;
        const int boff = ln * TS + 16 * s + 8 * lh;
        acc = mfma3(*reinterpret_cast<const bf16x8*>(&sm.krt_h[aoff]),
                    *reinterpret_cast<const bf16x8*>(&sm.krt_l[aoff]),
                    *reinterpret_cast<const bf16x8*>(&sm.tb_h[boff]),
                    *reinterpret_cast<const bf16x8*>(&sm.tb_l[boff]), acc);
      }
      // acc: W^T rows d = 32 wave + 8r + 4lh + e, column i = ln
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = 32 * wave + 8 * r + 4 * lh;
        const float4 e4 = *reinterpret_cast<const float4*>(&sm.ea[d0]);
        const float ev[4] = {e4.x, e4.y, e4.z, e4.w};
        bf16x4 wh, wl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16 hh, ll;
          split(-ev[e] * acc[4 * r + e], hh, ll);
          wh[e] = hh;
          wl[e] = ll;
        }
        *reinterpret_cast<bf16x4*>(&sm.kr_h[ln * NS + d0]) = wh;
        *reinterpret_cast<bf16x4*>(&sm.kr_l[ln * NS + d0]) = wl;
      }
    }
    f32x16 U = zero16();
    if (use_v) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int aoff = ln * TS + 16 * s + 8 * lh;
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&sm.vt[(32 * wave + ln) * TS + 16 * s + 8 * lh]);
        U = mfma(*reinterpret_cast<const bf16x8*>(&sm.tb_h[aoff]), bv, U);
        U = mfma(*reinterpret_cast<const bf16x8*>(&sm.tb_l[aoff]), bv, U);
      }
    }
    __syncthreads();

    // ================= P4: U -= W S, O = Qg S + P U, S <- e^{G_C-a}(e^a S + Kc^T U)
#pragma unroll
    for (int kk = 0; kk < KD / 16; ++kk) {
      const int off = ln * NS + 16 * kk + 8 * lh;
      U = mfma3(*reinterpret_cast<const bf16x8*>(&sm.kr_h[off]),
                *reinterpret_cast<const bf16x8*>(&sm.kr_l[off]), sbh[kk], sbl[kk], U);
    }
    f32x16 O = zero16();
    if (fwd) {
#pragma unroll
      for (int kk = 0; kk < KD / 16; ++kk) {
        const int off = ln * NS + 16 * kk + 8 * lh;
        O = mfma3(*reinterpret_cast<const bf16x8*>(&sm.qg_h[off]),
                  *reinterpret_cast<const bf16x8*>(&sm.qg_l[off]), sbh[kk], sbl[kk], O);
      }
    }
    bf16x8 ubh[2], ubl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float x[8];
      tile_rows_to_b(U, s, x);
      split8(x, ubh[s], ubl[s]);
    }
    if (fwd) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int off = ln * TS + 16 * s + 8 * lh;
        O = mfma3(*reinterpret_cast<const bf16x8*>(&sm.p_h[off]),
                  *reinterpret_cast<const bf16x8*>(&sm.p_l[off]), ubh[s], ubl[s], O);
      }
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float4 e4 = *reinterpret_cast<const float4*>(&sm.ea[32 * dt + 8 * r + 4 * lh]);
        S[dt][4 * r + 0] *= e4.x;
        S[dt][4 * r + 1] *= e4.y;
        S[dt][4 * r + 2] *= e4.z;
        S[dt][4 * r + 3] *= e4.w;
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int off = (32 * dt + ln) * TS + 16 * s + 8 * lh;
        S[dt] = mfma3(*reinterpret_cast<const bf16x8*>(&sm.kct_h[off]),
                      *reinterpret_cast<const bf16x8*>(&sm.kct_l[off]), ubh[s], ubl[s], S[dt]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float4 e4 = *reinterpret_cast<const float4*>(&sm.ega[32 * dt + 8 * r + 4 * lh]);
        S[dt][4 * r + 0] *= e4.x;
        S[dt][4 * r + 1] *= e4.y;
        S[dt][4 * r + 2] *= e4.z;
        S[dt][4 * r + 3] *= e4.w;
      }
    }
    if (fwd) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 8 * r + 4 * lh + e;
          if (i < n) p.o[(static_cast<size_t>(c0 + i) * H + h) * VD + col] = O[4 * r + e];
        }
      }
    }
    __syncthreads();
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
  for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 32 * dt + 8 * r + 4 * lh + e;
        if (dst0) dst0[d * VD + col] = S[dt][4 * r + e];
        if (dst1) dst1[d * VD + col] = S[dt][4 * r + e];
      }
    }
  }
}

// Ordered scan C_0 = 0, C_{r+1} = A_r C_r + B_r for one head and one block of
// 32 state columns.  Wave w computes rows [32w, 32w + 32); the current carry
// is shared through LDS as split B operands.
__global__ void __launch_bounds__(NT, 1) kda_compose_kernel(ComposeParams p) {
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
