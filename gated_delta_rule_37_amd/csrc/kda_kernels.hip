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

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_kernels.h"

namespace kda {
namespace {


constexpr int KD = 128;   // key dimension
constexpr int VD = 128;   // value dimension
constexpr int CH = 32;    // chunk length (tokens)
constexpr int NOWN = 4;               // waves per role: owners (32 columns each), helpers (32 channels each)
// summaries kernel: owners of S (waves 0-3) and of the transition (4-7), helpers 8-11
static_assert(4 * NOWN * 64 == kSummaryThreads, "summaries kernel wave roles");
static_assert(3 * NOWN * 64 == kCarryThreads, "carry kernel: owners, operand helpers, T helpers");
constexpr int NS = 152;   // row stride (bf16) of token-major [32][128] tiles (conflict-free row and transposed reads)
constexpr int TS = 40;    // row stride (bf16) of channel-major [128][32] tiles
constexpr int FS = 36;    // row stride (fp32) of the 32 x 32 triangular-solve tiles
constexpr int XS = 20;    // row stride (fp32) of the 16 x 16 off-diagonal product
constexpr float kLog2e = 1.4426950408889634f;
// Largest in-chunk factor exponent (log2 units) of the anchored chunk form.
// A fragment with a chunk where some channel's decay between a token and the
// anchor (or from the chunk start to the anchor) exceeds it is run again
// token by token (see pipe_owner).
constexpr float kFactorMax = 96.f;
// Floor of the per-token log2 decay in the token-by-token re-run: 2^-300
// times any finite FP32 value is below the smallest FP32 denormal, so the
// floor changes no FP32 product.
constexpr float kGateFloor = -300.f;
// Buffer resource word 3 for gfx9 raw (unswizzled, 32-bit) buffer access;
// accesses at or past num_records read zero and drop writes.
constexpr int kBufDword3 = 0x00020000;
// Cache policy of the o stores (and the checkpoint launch's states and
// V - Kr R tiles): non-temporal (nt).  They are written once per launch and
// read by nothing in it; streaming them past the caches leaves them to the
// inputs and the chunk cache (the carry launch ~1% faster).
constexpr int kStreamAux = 2;

enum Mode { kModeFwd = 0, kModeSumS = 1, kModeSumPhi = 2, kModeCkpt = 3 };


// What one workgroup of the summaries launch does with its fragment.  Only
// the last fragment of each segment runs there: its state from zero is B_r
// (waves 0-3); waves 4-7 build A_r from the identity when the fragment carries
// in (no sequence starts inside the segment), and otherwise write the zero
// transition (the reset's linear part).  Every fragment's o and final state
// come from the carry launch.
struct Work {
  bool run;
  bool phi;
};
__device__ __forceinline__ Work decode_summary(const ChunkParams& p, int32_t flags, int32_t seg) {
  Work w{false, false};
  if (flags & kFragSegLast) {
    w.run = true;
    w.phi = (flags & kFragCarried) && p.plan[p.L.seg_transition_live + seg];
  }
  return w;
}


// 16 bytes of a token-major tile row for st4, halves exchanged when the row
// is stored that way (hi_rows)
__device__ __forceinline__ u32x4 sw_rows(const int hi_rows, const uint32_t (&w)[4]) {
  return hi_rows ? u32x4{w[2], w[3], w[0], w[1]} : u32x4{w[0], w[1], w[2], w[3]};
}
__device__ __forceinline__ u32x4 sw_rows(const int hi_rows, const u32x4& w) {
  return hi_rows ? u32x4{w[2], w[3], w[0], w[1]} : w;
}

}  // namespace


// 16 x 16 tile of X Kc^T over the 128 channels: rows 16rb .. 16rb+15 of X
// (Kr or Qr) against rows 16ct .. 16ct+15 of Kc, split operands.  Lane l
// receives rows 16rb + 4(l/16) + e, e = 0..3, of column 16ct + l%16.  Where
// both row blocks are stored alike the order of the eight channels inside a
// lane's 16 bytes cancels out of the dot product; SWAP serves rb = 1, ct = 0
// in the exchanged-half layout.
template <bool SWAP = false>
__device__ __forceinline__ f32x4 tile16(const bf16* xh, const bf16* xl, const bf16* ch, const bf16* cl,
                                        const int rb, const int ct, const int lm, const int lg) {
  f32x4 acc = zero4();
#pragma unroll
  for (int kk = 0; kk < KD / 32; ++kk) {
    const int aoff = (16 * rb + lm) * NS + 32 * kk + 8 * lg;
    const int boff = (16 * ct + lm) * NS + 32 * kk + 8 * lg;
    bf16x8 ah, al;
    if (SWAP) {
      // the A rows are stored with exchanged halves and the Kc rows are not:
      // read A back in channel order
      ah = ld_halves_swapped(&xh[aoff]);
      al = ld_halves_swapped(&xl[aoff]);
    } else {
      ah = *reinterpret_cast<const bf16x8*>(&xh[aoff]);
      al = *reinterpret_cast<const bf16x8*>(&xl[aoff]);
    }
    acc = mfma16x3(ah, al, *reinterpret_cast<const bf16x8*>(&ch[boff]), *reinterpret_cast<const bf16x8*>(&cl[boff]), acc);
  }
  mfma_result_fence(acc);
  return acc;
}

// Diagonal block rb of A = beta o (Kr Kc^T) and the inverse of that block of
// I + A.  The block goes to LDS transposed (an[16rb + j][16rb + i] = A_ij,
// one 16-byte store per lane), and the wave reads its own columns back
// without a barrier (its LDS accesses complete in order).  Lanes c = 0..15
// then solve for one line of the inverse each (lanes 16..63 repeat them):
//   rb = 0: column c of T00 by forward substitution, right-looking
//           (x_j final, then x_i -= A_ij x_j for i > j), stored by column:
//           tt[c][i] = T00[i][c];
//   rb = 1: row c of T11, i.e. column c of (I + A11^T)^{-1}, by back
//           substitution, y_i = [i == c] - sum_{j>i} A_ji y_j, stored by row:
//           tn[16 + c][16 + i] = T11[c][i].
// The merge reads T00 by columns and T11 by rows only.
__device__ __forceinline__ void a_diag_solve(const bf16* krh, const bf16* krl, const bf16* kch, const bf16* kcl,
                                             const float* beta, float* an, float* tt, float* tn, const int rb,
                                             const int lane_s) {
  const int lm = lane_s & 15;
  const int lg = lane_s >> 4;
  const f32x4 acc = tile16(krh, krl, kch, kcl, rb, rb, lm, lg);
  const f32x4 brow = ld4(&beta[16 * rb + 4 * lg]);
  const int base = 16 * rb;
  {
    // lane (lg, lm) holds A[4lg + e][lm], e = 0..3: column lm, four rows
    f32x4 col;
#pragma unroll
    for (int e = 0; e < 4; ++e) col[e] = (lm < 4 * lg + e) ? brow[e] * acc[e] : 0.f;
    st4(&an[(base + lm) * FS + base + 4 * lg], col);
  }
  wave_lds_order();
  const int c = lm;
  float x[16];
  if (rb == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
      // column j of A, rows j+1 .. 15
#pragma unroll
      for (int q4 = (j + 1) / 4; q4 < 4; ++q4) {
        const f32x4 a = ld4(&an[(base + j) * FS + base + 4 * q4]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * q4 + e > j) x[4 * q4 + e] -= a[e] * x[j];
      }
    }
    if (lane_s < 16) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        st4(&tt[c * FS + 4 * q4], f32x4{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]});
    }
  } else {
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      float yi = (i == c) ? 1.f : 0.f;
      // column i of A, rows i+1 .. 15
#pragma unroll
      for (int q4 = (i + 1) / 4; q4 < 4; ++q4) {
        const f32x4 a = ld4(&an[(base + i) * FS + base + 4 * q4]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * q4 + e > i) yi -= a[e] * x[4 * q4 + e];
      }
      x[i] = yi;
    }
    if (lane_s < 16) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        st4(&tn[(base + c) * FS + base + 4 * q4], f32x4{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]});
    }
  }
}

// A10 = beta o (Kr Kc^T), rows 16..31 and columns 0..15, into an.
template <bool SWZ>
__device__ __forceinline__ void a_offdiag(const bf16* krh, const bf16* krl, const bf16* kch, const bf16* kcl,
                                          const float* beta, float* an, const int lane_s) {
  const int lm = lane_s & 15;
  const int lg = lane_s >> 4;
  const f32x4 acc = tile16<SWZ>(krh, krl, kch, kcl, 1, 0, lm, lg);
  const f32x4 brow = ld4(&beta[16 + 4 * lg]);
#pragma unroll
  for (int e = 0; e < 4; ++e) an[(16 + 4 * lg + e) * FS + lm] = brow[e] * acc[e];
}

// One 16 x 16 block (rbp, ctp) of P, ctp <= rbp, as split bf16 (entries above
// the diagonal zero; columns in k-slot order); block (0, 0) also writes the
// zero block (0, 1).
__device__ __forceinline__ void p_store(const f32x4& acc, const int rbp, const int ctp, bf16* ph, bf16* pl,
                                        const int lane_s) {
  const int lm = lane_s & 15;
  const int lg = lane_s >> 4;
  const int j = 16 * ctp + lm;
  const int jp = 16 * ctp + kslot_col(lm);   // stored column of j
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 16 * rbp + 4 * lg + e;
    bf16 hh, ll;
    split(j <= i ? acc[e] : 0.f, hh, ll);
    ph[i * TS + jp] = hh;
    pl[i * TS + jp] = ll;
    if (rbp == 0) {
      ph[i * TS + 16 + kslot_col(lm)] = static_cast<bf16>(0.f);
      pl[i * TS + 16 + kslot_col(lm)] = static_cast<bf16>(0.f);
    }
  }
}

// T10 = -T11 A10 T00 and T diag(beta) (T itself with UNSC) as split bf16
// (columns in k-slot order), for the columns
// tc = 4q .. 4q+3 (q = 0..3), lane (row ti, column tc); X = A10 T00 goes
// through LDS inside the wave, which needs no barrier.
template <bool UNSC = false>
__device__ __forceinline__ void t_merge(const float* an, const float* tt, const float* tn, float* xt,
                                        const float* beta, bf16* tbh, bf16* tbl, const int q, const int lane_s) {
  const int ti = lane_s & 15;
  const int tc = 4 * q + (lane_s >> 4);
  f32x4 u[4], w[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    u[q4] = ld4(&an[(16 + ti) * FS + 4 * q4]);   // A10[ti, :]
    w[q4] = ld4(&tt[tc * FS + 4 * q4]);          // T00[:, tc]
  }
  float xs = 0.f;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
    xs += u[q4][0] * w[q4][0] + u[q4][1] * w[q4][1] + u[q4][2] * w[q4][2] + u[q4][3] * w[q4][3];
  xt[tc * XS + ti] = xs;   // X = A10 T00, stored by column
  const float t00 = tt[tc * FS + ti];               // T00[ti][tc]
  const float t11 = tn[(16 + ti) * FS + 16 + tc];    // T11[ti][tc]
  const float b0 = UNSC ? 1.f : beta[tc];
  const float b1 = UNSC ? 1.f : beta[16 + tc];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) u[q4] = ld4(&tn[(16 + ti) * FS + 16 + 4 * q4]);   // T11[ti, :]
  wave_lds_order();
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) w[q4] = ld4(&xt[tc * XS + 4 * q4]);   // X[:, tc]
  float t10 = 0.f;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
    t10 -= u[q4][0] * w[q4][0] + u[q4][1] * w[q4][1] + u[q4][2] * w[q4][2] + u[q4][3] * w[q4][3];
  const int cp = kslot_col(tc);   // stored column of tc (and of 16 + tc)
  bf16 hh, ll;
  split(t00 * b0, hh, ll);
  tbh[ti * TS + cp] = hh;
  tbl[ti * TS + cp] = ll;
  split(t11 * b1, hh, ll);
  tbh[(16 + ti) * TS + 16 + cp] = hh;
  tbl[(16 + ti) * TS + 16 + cp] = ll;
  split(t10 * b0, hh, ll);
  tbh[(16 + ti) * TS + cp] = hh;
  tbl[(16 + ti) * TS + cp] = ll;
  tbh[ti * TS + 16 + cp] = static_cast<bf16>(0.f);
  tbl[ti * TS + 16 + cp] = static_cast<bf16>(0.f);
}

// Chunk-kernel workgroups are numbered linearly, x fastest: id = rank * hn +
// head.  The heads of one fragment are adjacent and the fragments come in the
// plan's launch order (longest first).  The host spreads the ids over x and y
// only when y alone would exceed its limit; ids past the end do nothing.
__device__ __forceinline__ uint64_t block_linear() {
  return static_cast<uint64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
}
__device__ __forceinline__ int block_head(const ChunkParams& p) {
  return p.h0 + static_cast<int>(block_linear() % static_cast<uint64_t>(p.hn));
}
__device__ __forceinline__ int64_t block_rank(const ChunkParams& p) {
  return static_cast<int64_t>(block_linear() / static_cast<uint64_t>(p.hn));
}

// Chunk cache transfer of T diag(beta) (4 KB per chunk and head): the 256
// lanes of four waves (index 0..255 = 64 wave + lane) each move 16 bytes,
// lane i taking half i/128 (hi, lo), row (i/4) % 32 and quarter i % 4.
__device__ __forceinline__ size_t cache_elem(const ChunkParams& p, const int h, const int32_t seg, const int32_t beg,
                                             const int it, const int i) {
  const int which = i >> 7;
  const int row = (i >> 2) & 31;
  const int q = i & 3;
  return (static_cast<size_t>(chunk_cache_slot(seg, beg, it)) * p.H + h) * (kChunkCacheBytes / 2) +
         which * (CH * CH) + row * CH + 8 * q;
}
__device__ __forceinline__ int cache_lds(const int i) { return ((i >> 2) & 31) * TS + 8 * (i & 3); }

// ===========================================================================
// Both sequential kernels run each fragment as a two-step pipeline of wave
// roles, so that the operands and the UT transform of later chunks are built
// while the owners work on the current one:
//
//   owners                 step 2n: products of chunk n
//                          step 2n+1: finish chunk n
//   operand helpers        steps 2m-3, 2m-2: operands of chunk m
//   T helpers              steps 2m-1, 2m: A, T diag(beta), P of chunk m
//
// A fragment of nc chunks takes the steps -3 .. 2nc-1, each ending with a
// workgroup barrier (every wave executes 2nc + 3 of them).  Kr, Qr, Kc, V,
// fac and beta are double-buffered by chunk parity; T diag(beta), P and the
// solve scratch are single.  Who writes what, and when (m = chunk):
//   Kr, Qr, fac, beta (m)  step 2m-3   last readers of chunk m-2: step 2m-3
//                                      at the latest (fac), else 2m-4
//   Kc, V (m)              step 2m-2   last reader of chunk m-2:  step 2m-3
//   an, tt, tn (m)         step 2m-1   last reader of chunk m-1:  step 2m-2
//   T diag(beta), P (m)    step 2m     last reader of chunk m-1:  step 2m-1
// fac(m) re-anchors the state for chunk m; the owners apply it at the end of
// finish(m-1) (and fac(0) before the first chunk).  fac spans the decay of
// up to 32 tokens; where one FP32 factor would underflow it is split into a
// normal factor and a power of two (fexp, flagged per operand helper in
// fsplit), which the owners apply with ldexp on those rows only.
// ===========================================================================
// Token-major tiles in the carry launch hold rows 16 .. 31 with the two 8-byte
// halves of every 16-byte group exchanged (element c at c ^ 4).  At this row
// stride rows r and r + 16 fall on the same banks, so the owners' 8-byte reads
// of 32 rows met two to a bank; exchanged, they cover all 64 banks once.  The
// summaries launch keeps the plain layout: there the T helpers' off-diagonal
// block of A, which pays for the exchange with twice the reads, is on the
// longest chain of its step.
struct alignas(16) PipeSmem {
  bf16 kr_h[2][CH * NS], kr_l[2][CH * NS];    // Kr = k e^{G-a}, token-major
  bf16 qr_h[2][CH * NS], qr_l[2][CH * NS];    // Qr = q e^{G-a}, token-major
  bf16 kc_h[2][CH * NS], kc_l[2][CH * NS];    // Kc = k e^{a-G}, token-major
  bf16 vv[2][CH * NS];                        // V, token-major (exact)
  bf16 tb_h[CH * TS], tb_l[CH * TS];          // T diag(beta), [i][j]
  bf16 p_h[CH * TS], p_l[CH * TS];            // P, [i][j]
  float an[CH * FS];                          // A10 by rows, diagonal blocks transposed
  float tt[CH * FS];                          // tt[c][i] = T00[i][c]
  float tn[CH * FS];                          // tn[16 + i][16 + c] = T11[i][c]
  float xt[16 * XS];                          // X = A10 T00, stored xt[c][i]
  float fac[2][KD];                           // state rescale before chunk m
  float beta[2][CH];
  alignas(16) int16_t fexp[2][KD];            // power-of-two part of fac (0: none)
  int32_t fsplit[2][NOWN];                    // per operand helper: some fac split
  alignas(16) int32_t rerun[NOWN];            // per operand helper: some chunk beyond the anchored form
};

// Whether the fragment is run again token by token: the OR of the operand
// helpers' flags, uniform over the wave.  The helpers write them in step
// 2nc-3; every wave reads them after its last pipeline barrier.
__device__ __forceinline__ bool fragment_rerun(const PipeSmem& sm) {
  const u32x4 f = *reinterpret_cast<const u32x4*>(&sm.rerun[0]);
  return __builtin_amdgcn_readfirstlane(f[0] | f[1] | f[2] | f[3]) != 0;
}

// In the token-by-token re-run the operand buffers of parity b hold FP32
// rows of 32 tokens: k in kr_h (tokens 0..15) and kr_l (16..31), q in
// qr_h / qr_l and the per-token decay 2^l in kc_h / kc_l, each [16][128].
__device__ __forceinline__ float* tok_rows(bf16* lo_half, bf16* hi_half, const int t) {
  return reinterpret_cast<float*>(t < 16 ? lo_half : hi_half) + (t & 15) * KD;
}
typedef const volatile __attribute__((address_space(3))) f32x4 lds_f32x4;
// a 16-byte LDS read the compiler neither merges with nor hoists over another
__device__ __forceinline__ f32x4 ld4v(const float* p) { return *(lds_f32x4*)(const_cast<float*>(p)); }

// Owner wave ow: the state columns [32ow, 32ow + 32) as four 32 x 32 FP32
// accumulator tiles R[dt] (rows 32dt + 8r + 4(l/32) + e in lane l, register
// 4r + e; column 32ow + l%32).  R is the state scaled by the anchor of the
// chunk it enters, e^{a} o S, which is the operand Kr and Qr multiply; one
// update is
//     S_new = Diag(e^{G_C}) S + K^^T U = Diag(e^{G_C - a}) (R + Kc^T U)
// and fac = e^{a_next + G_C - a} re-anchors it for the next chunk
// (e^{G_C - a} after the last one, which leaves S itself).  Modes:
//   kModeFwd    from the carry-in, the sequence's initial state or zero (init):
//               o and, at a sequence end, the final state
//   kModeSumS   from the sequence's initial state or zero (init), no o: B_r
//   kModeSumPhi from the identity with V = 0, no o: A_r
//   kModeCkpt   from the carry-in, the sequence's initial state or zero, no o:
//               R entering every chunk n, at checkpoint slot ck0 + n
// init points at the starting state's [K, V] matrix for this head, or is null.
template <int MODE>
__device__ __forceinline__ void pipe_owner(const ChunkParams& p, PipeSmem& sm, const int h, const int ow,
                                           const int32_t flags,
                                           const int32_t seg, const int32_t seq, const int32_t beg,
                                           const int32_t end, const float* init, const int64_t ck0 = 0) {
  constexpr bool fwd = MODE == kModeFwd;
  constexpr bool use_v = MODE != kModeSumPhi;
  const int H = p.H;
  const int lane = threadIdx.x & 63;
  const int lh = lane >> 5;
  const int col = 32 * ow + (lane & 31);
  const int nc = (end - beg + CH - 1) / CH;
  const int o_row = H * VD * 4;   // one token of o (bytes)

  f32x16 R[4];
  // the starting state (unanchored): identity, the given state or zero
  auto load_start = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) R[dt] = zero16();
    if (MODE == kModeSumPhi) {
      // the diagonal element of column col sits in tile col/32, register
      // 4((col%32)/8) + col%4, of the lanes with l/32 = (col/4)%2
      const int ln_s = opaque(lane) & 31;
      const bool own = ((ln_s >> 2) & 1) == (lane >> 5);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          R[dt][i] = (own && dt == ow && i == 4 * (ln_s >> 3) + (ln_s & 3)) ? 1.f : 0.f;
    } else if (init != nullptr) {
      const float* src = init + col;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) R[dt][4 * r + e] = src[(32 * dt + 8 * r + 4 * lh + e) * VD];
    }
  };
  load_start();
  f32x16 Y = zero16(), O = zero16();

  // A operands of k-step kk (channels 16kk .. 16kk+15, k-slot order)
  // per-lane LDS element offsets, fixed for the whole fragment
  constexpr bool xrows = fwd;   // rows 16 .. 31 stored with exchanged halves
  const int prod_off = (lane & 31) * NS + 4 * ((lane >> 5) ^ (xrows ? (lane >> 4) & 1 : 0));   // A operand rows of Kr, Qr
  const int tr_off = (4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * NS + 16 * ((lane >> 4) & 1) +
                     4 * ((lane & 15) & 3);                     // transposed reads of V, Kc
  const int tr_sw = xrows ? tr_off ^ 4 : tr_off;              // the same in rows 16 .. 31
  const int tb_off = (lane & 31) * TS + 8 * (lane >> 5);    // rows of T diag(beta), P
  auto load_ops = [&](bf16x8 (&o)[4], const int b, const int kk) {
    o[0] = ld_kslots_at(&sm.kr_h[b][prod_off + 16 * kk]);
    o[1] = ld_kslots_at(&sm.kr_l[b][prod_off + 16 * kk]);
    if (fwd) {
      o[2] = ld_kslots_at(&sm.qr_h[b][prod_off + 16 * kk]);
      o[3] = ld_kslots_at(&sm.qr_l[b][prod_off + 16 * kk]);
    }
  };
  auto load_fac = [&](f32x4 (&f)[4], const int b, const int dt, const int lh) {
#pragma unroll
    for (int r = 0; r < 4; ++r) f[r] = ld4(&sm.fac[b][32 * dt + 8 * r + 4 * lh]);
  };
  auto rescale = [&](const int dt, const f32x4 (&f)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) R[dt][4 * r + e] *= f[r][e];
  };
  // the power-of-two part of fac, on the rare chunks where some channel has it
  // (rows 32dt .. 32dt+31 are operand helper dt's channels, so its flag
  // covers tile dt)
  auto rescale_exp = [&](const int b, const int lh) {
    const u32x4 fl = *reinterpret_cast<const u32x4*>(&sm.fsplit[b][0]);
    if (__builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3]) == 0) return;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      if (__builtin_amdgcn_readfirstlane(fl[dt]) == 0) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          R[dt][4 * r + e] = __builtin_ldexpf(R[dt][4 * r + e], sm.fexp[b][32 * dt + 8 * r + 4 * lh + e]);
    }
  };

  f32x4 bkeep[4];   // kModeCkpt: beta of chunk n's tokens 8r + 4lh + 0..3
  // step 2n: Y = Kr R and O = Qr R (R already anchored for chunk n), operand
  // loads one k-step ahead
  auto products = [&](const int n) __attribute__((always_inline)) {
    const int b = n & 1;
    if (MODE == kModeCkpt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) bkeep[r] = ld4(&sm.beta[b][8 * r + 4 * lh]);
    }
    Y = zero16();
    if (fwd) O = zero16();
    bf16x8 opa[2][4];
    load_ops(opa[0], b, 0);
#pragma unroll
    for (int kk = 0; kk < KD / 16; ++kk) {
      if (kk + 1 < KD / 16) load_ops(opa[(kk + 1) & 1], b, kk + 1);
      float x[8];
      tile_kslots(R[kk >> 1], kk & 1, x);
      bf16x8 bh, bl;
      split8(x, bh, bl);
      const bf16x8(&o)[4] = opa[kk & 1];
      Y = mfma3(o[0], o[1], bh, bl, Y);
      if (fwd) O = mfma3(o[2], o[3], bh, bl, O);
    }
  };

  // step 2n+1: D = V - Y, U = T diag(beta) D, O += P U, store o, R += Kc^T U
  auto finish = [&](const int n) __attribute__((always_inline)) {
    const int b = n & 1;
    const int c0 = beg + n * CH;
    const int nn = min(CH, end - c0);
    mfma_result_fence(Y);
    f32x16 D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float vv[4] = {0.f, 0.f, 0.f, 0.f};
      if (use_v) {
        // V[8r + 4lh + e][col], e = 0..3, from the token-major copy
        const s16x4 v4 = lds_read_tr(&sm.vv[b][(r >= 2 ? tr_sw : tr_off) + 8 * r * NS + 32 * ow]);
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = bf2f(static_cast<uint16_t>(v4[e]));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) D[4 * r + e] = vv[e] - Y[4 * r + e];
    }
    if (MODE == kModeCkpt) {
      // V - Kr R of the chunk for the backward's gradient launch, [token][V]
      const auto rsv = __builtin_amdgcn_make_buffer_rsrc(p.rv_out + (static_cast<size_t>(ck0 + n) * H + h) * CH * VD, 0,
                                                         CH * VD * 4, kBufDword3);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(D[4 * r + e]), rsv, 4 * (4 * lh * VD + col),
                                                4 * (8 * r + e) * VD, kStreamAux);
      // the T helpers leave T unscaled in this mode (the cache keeps T for
      // the backward): U = T diag(beta) D, with beta read in products(n)
      // (the operand helpers rewrite this buffer in step 2n+1)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) D[4 * r + e] *= bkeep[r][e];
    }
    // D and U feed the next products as B operands in k-slot order (tokens):
    // T diag(beta) and P are stored in that column order, Kc^T is read in it
    bf16x8 dh[2], dl[2];
    tile_kslots_split(D, dh, dl);
    f32x16 U = zero16();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int off = tb_off + 16 * s;   // columns stored in k-slot order
      U = mfma3(*reinterpret_cast<const bf16x8*>(&sm.tb_h[off]), *reinterpret_cast<const bf16x8*>(&sm.tb_l[off]),
                dh[s], dl[s], U);
    }
    mfma_result_fence(U);
    bf16x8 ubh[2], ubl[2];
    tile_kslots_split(U, ubh, ubl);
    if (fwd) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int off = tb_off + 16 * s;
        O = mfma3(*reinterpret_cast<const bf16x8*>(&sm.p_h[off]), *reinterpret_cast<const bf16x8*>(&sm.p_l[off]),
                  ubh[s], ubl[s], O);
      }
    }
    // R += Kc^T U: the A operand (row = channel 32dt + l%32, k slots = tokens
    // 16s + 4(l/32) + 0..3 and 16s + 8 + 4(l/32) + 0..3) is read as column
    // fragments of the token-major Kc
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int off = (s ? tr_sw : tr_off) + 16 * s * NS + 32 * dt;
        const bf16x8 ah = join8(lds_read_tr(&sm.kc_h[b][off]), lds_read_tr(&sm.kc_h[b][off + 8 * NS]));
        const bf16x8 al = join8(lds_read_tr(&sm.kc_l[b][off]), lds_read_tr(&sm.kc_l[b][off + 8 * NS]));
        R[dt] = mfma3(ah, al, ubh[s], ubl[s], R[dt]);
      }
    }
    // re-anchor for chunk n+1 (after the last chunk: e^{G_C - a}, which
    // leaves S itself)
    mfma_result_fence(R[0], R[1], R[2], R[3]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x4 f[4];
      load_fac(f, (n + 1) & 1, dt, lh);
      rescale(dt, f);
    }
    if (fwd) {
      mfma_result_fence(O);
      // rows past the fragment's end fall outside the buffer and are dropped
      if (p.o_bf16) {
        // BF16 o: the FP32 result rounded to nearest even
        const int ob_row = o_row / 2;
        const auto rso = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<uint16_t*>(p.o) + (static_cast<size_t>(c0) * H + h) * VD, 0,
            (nn - 1) * ob_row + 2 * VD, kBufDword3);
        const int o_voff = 4 * lh * ob_row + 2 * col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16 ob = static_cast<bf16>(O[4 * r + e]);
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, ob), rso, o_voff,
                                                  (8 * r + e) * ob_row, kStreamAux);
          }
        }
      } else {
        const auto rso = __builtin_amdgcn_make_buffer_rsrc(p.o + (static_cast<size_t>(c0) * H + h) * VD, 0,
                                                           (nn - 1) * o_row + 4 * VD, kBufDword3);
        const int o_voff = 4 * lh * o_row + 4 * col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ov = O[4 * r + e];
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(ov), rso, o_voff, (8 * r + e) * o_row, kStreamAux);
          }
        }
      }
    }
    // last, so that the rare branch does not cut the step's code in two
    rescale_exp((n + 1) & 1, lh);
  };

  // Block n of the re-run, one token at a time in FP32:
  //     R <- 2^l o R;  u = beta (v - R^T k);  R <- R + k u^T;  o = R^T q,
  // with R the state itself.  A lane holds 64 rows of its column; the other
  // 64 are in lane l ^ 32, so each dot product over the rows is the lane's
  // part plus its partner's (summed in the same order in both lanes).
  auto token_steps = [&](const int n) __attribute__((always_inline)) {
    const int b = n & 1;
    const int c0 = beg + n * CH;
    const int nn = min(CH, end - c0);
    const int lane_r = opaque(lane);
    const int lhr = lane_r >> 5;
    const int colr = 32 * ow + (lane_r & 31);
    auto halves = [](const float x) {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    };
    for (int t = 0; t < nn; ++t) {
      const float* kt = tok_rows(sm.kr_h[b], sm.kr_l[b], t);
      const float* dct = tok_rows(sm.kc_h[b], sm.kc_l[b], t);
      float part[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        part[dt] = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 32 * dt + 8 * r + 4 * lhr;
          const f32x4 dv = ld4v(dct + row);
          const f32x4 kv = ld4v(kt + row);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            R[dt][4 * r + e] *= dv[e];
            part[dt] = __builtin_fmaf(kv[e], R[dt][4 * r + e], part[dt]);
          }
        }
      }
      const float kS = halves((part[0] + part[1]) + (part[2] + part[3]));
      float vt = 0.f;
      if (use_v) vt = bf2f(__builtin_bit_cast(uint16_t, sm.vv[b][t * NS + ((fwd && t >= 16) ? (colr ^ 4) : colr)]));
      const float u = sm.beta[b][t] * (vt - kS);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4 kv = ld4v(kt + 32 * dt + 8 * r + 4 * lhr);
#pragma unroll
          for (int e = 0; e < 4; ++e) R[dt][4 * r + e] = __builtin_fmaf(kv[e], u, R[dt][4 * r + e]);
        }
      }
      if (fwd) {
        const float* qt = tok_rows(sm.qr_h[b], sm.qr_l[b], t);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          part[dt] = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const f32x4 qv = ld4v(qt + 32 * dt + 8 * r + 4 * lhr);
#pragma unroll
            for (int e = 0; e < 4; ++e) part[dt] = __builtin_fmaf(qv[e], R[dt][4 * r + e], part[dt]);
          }
        }
        const float ov = halves((part[0] + part[1]) + (part[2] + part[3]));
        if (lhr == 0) {
          const size_t oi = (static_cast<size_t>(c0 + t) * H + h) * VD + colr;
          if (p.o_bf16) reinterpret_cast<bf16*>(p.o)[oi] = static_cast<bf16>(ov);
          else p.o[oi] = ov;
        }
      }
    }
  };

  // the anchored state entering chunk n, row-major [K][V] (one column per
  // lane, 32 lanes to a 128-byte row piece)
  auto store_ckpt = [&](const int n) __attribute__((always_inline)) {
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(p.ckpt + (static_cast<size_t>(ck0 + n) * H + h) * KD * VD, 0,
                                                      KD * VD * 4, kBufDword3);
    const int voff = 4 * (4 * lh * VD + col);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(R[dt][4 * r + e]), rs, voff,
                                                4 * (32 * dt + 8 * r + e) * VD, kStreamAux);
  };

  block_sync();   // steps -3 .. -1: the helpers fill the pipeline
  block_sync();
  block_sync();
  {
    // anchor the starting state for chunk 0
    const int lh2 = opaque(lane) >> 5;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x4 f[4];
      load_fac(f, 0, dt, lh2);
      rescale(dt, f);
    }
    rescale_exp(0, lh2);
  }
  for (int n = 0; n < nc; ++n) {
    if (MODE == kModeCkpt) store_ckpt(n);
    products(n);
    block_sync();
    finish(n);
    block_sync();
  }
  if (MODE == kModeCkpt && ow == 0 && lane == 0)
    p.item_flag[static_cast<size_t>(ck0 - beg / CH) * p.hn + (h - p.h0)] = fragment_rerun(sm) ? 1 : 0;
  if (fragment_rerun(sm)) {
    // Some chunk's in-chunk factors left the range the anchored form keeps
    // finite and accurate, so its results for this fragment are discarded:
    // the fragment runs again from its starting state, one token at a time
    // in FP32.  The operand helpers stage each 32-token block as FP32 rows
    // (two barriers per block, in every wave).
    load_start();
    for (int n = 0; n < nc; ++n) {
      block_sync();
      token_steps(n);
      block_sync();
    }
  }
  const int lane_e = opaque(lane);
  const int lh_e = lane_e >> 5;
  const int col_e = 32 * ow + (lane_e & 31);
  float* dst = nullptr;
  if (MODE == kModeSumPhi) dst = p.transitions + (static_cast<size_t>(seg) * H + h) * KD * KD;
  else if (MODE == kModeSumS) dst = p.updates + (static_cast<size_t>(seg) * H + h) * KD * VD;
  else if (MODE == kModeFwd && (flags & kFragSeqEnd)) dst = p.final_state + (static_cast<size_t>(seq) * H + h) * KD * VD;
  if (dst) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(32 * dt + 8 * r + 4 * lh_e + e) * (MODE == kModeSumPhi ? KD : VD) + col_e] =
            R[dt][4 * r + e];
  }
}

// Operand helper oh (0..3) of the pipeline: channels [32oh, 32oh + 32); lane
// l holds octet 32oh + 8(l/16) of the tokens l%16 and 16 + l%16.  Part 1 of
// chunk m (step 2m-3): land the inputs loaded two steps earlier, issue the
// next chunk's loads, gate prefix, fac, beta, Kr and (with o) Qr; Kc and V
// stay in registers until part 2 (step 2m-2), when the owners are done with
// chunk m-2's.
template <int MODE>
__device__ __forceinline__ void pipe_ophelper(const ChunkParams& p, PipeSmem& sm, const int h, const int oh, const int32_t beg,
                                              const int32_t end) {
  constexpr bool fwd = MODE == kModeFwd;
  const int H = p.H;
  const int lane = threadIdx.x & 63;
  const int tk = lane & 15;                    // tokens tk and 16 + tk
  const int c8 = 32 * oh + 8 * (lane >> 4);    // first of this lane's eight channels
  const int nc = (end - beg + CH - 1) / CH;
  const int row_bytes = H * KD * 2;
  const int in_voff = tk * row_bytes + 2 * c8;

  u32x4 rk[2], rg[2], rq[2], rv[2];
  uint32_t rb = 0u;
  auto fetch = [&](int cs) {
    const int nn = min(CH, end - cs);
    const size_t base = (static_cast<size_t>(min(cs, end - 1)) * H + h) * KD;
    const int nrec = nn > 0 ? (nn - 1) * row_bytes + KD * 2 : 0;
    const auto rsk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.k + base), 0, nrec, kBufDword3);
    const auto rsg = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.g + base), 0, nrec, kBufDword3);
    const auto rsq = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.q + base), 0, nrec, kBufDword3);
    const auto rsv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.v + base), 0, nrec, kBufDword3);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int off = in_voff + 16 * j * row_bytes;
      rk[j] = __builtin_amdgcn_raw_buffer_load_b128(rsk, off, 0, 0);
      rg[j] = __builtin_amdgcn_raw_buffer_load_b128(rsg, off, 0, 0);
      if (fwd) rq[j] = __builtin_amdgcn_raw_buffer_load_b128(rsq, off, 0, 0);
      if (fwd) rv[j] = __builtin_amdgcn_raw_buffer_load_b128(rsv, off, 0, 0);
    }
    const int nb = (oh == 0 && nn > 0) ? (nn - 1) * H * 2 + 2 : 0;
    const auto rsb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.beta + static_cast<size_t>(min(cs, end - 1)) * H + h), 0, nb, kBufDword3);
    rb = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rsb, lane < CH ? lane * H * 2 : nb, 0, 0));
  };
  // The summaries launch loads v in part 2, right after storing the previous
  // chunk's v to LDS, and pins k's unpacked values before the next loads:
  // both loads then land in registers that are already free, with no copies
  // at the loop's back edge (which would wait for them one step early).
  auto fetch_v = [&](int cs) {
    const int nn = min(CH, end - cs);
    const size_t base = (static_cast<size_t>(min(cs, end - 1)) * H + h) * KD;
    const int nrec = nn > 0 ? (nn - 1) * row_bytes + KD * 2 : 0;
    const auto rsv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.v + base), 0, nrec, kBufDword3);
#pragma unroll
    for (int j = 0; j < 2; ++j) rv[j] = __builtin_amdgcn_raw_buffer_load_b128(rsv, in_voff + 16 * j * row_bytes, 0, 0);
  };
  fetch(beg);
  if (!fwd) fetch_v(beg);

  // fac = 2^t for this lane's eight channels (t in log2 units), written by
  // the lanes with tk = 0.  Where 2^t would leave the FP32 normal range (the
  // decay of the 32 tokens between two anchors beyond ~83 nats), it is
  // stored as 2^(t - e) with an integer e < 0 in fexp, applied by ldexp; the
  // wave's flag tells the owners whether any channel needs it.
  auto store_fac = [&](const int b, const float (&t)[8]) {
    float tmin = t[0];
#pragma unroll
    for (int c = 1; c < 8; ++c) tmin = fminf(tmin, t[c]);
    const bool split = __builtin_amdgcn_ballot_w64(tk == 0 && tmin < -120.f) != 0;
    float fv[8];
    if (split) {
      uint32_t ev[4] = {0u, 0u, 0u, 0u};   // eight int16 exponents, two per word
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int e = t[c] < -120.f ? static_cast<int>(floorf(t[c])) + 60 : 0;
        ev[c >> 1] |= (static_cast<uint32_t>(e) & 0xffffu) << (16 * (c & 1));
        fv[c] = __builtin_amdgcn_exp2f(t[c] - static_cast<float>(e));
      }
      // the owners read these only for the rows of a helper that set its flag
      if (tk == 0) *reinterpret_cast<u32x4*>(&sm.fexp[b][c8]) = u32x4{ev[0], ev[1], ev[2], ev[3]};
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) fv[c] = __builtin_amdgcn_exp2f(t[c]);
    }
    if (tk == 0) {
      st4(&sm.fac[b][c8], f32x4{fv[0], fv[1], fv[2], fv[3]});
      st4(&sm.fac[b][c8 + 4], f32x4{fv[4], fv[5], fv[6], fv[7]});
    }
    if (lane == 0) sm.fsplit[b][oh] = split ? 1 : 0;
  };

  float dprev[8];   // (G_C - a) of the previous chunk, log2 units
#pragma unroll
  for (int c = 0; c < 8; ++c) dprev[c] = 0.f;
  bool rerun_w = false;   // some chunk is beyond the anchored form (this wave's channels)

  for (int m = 0; m < nc; ++m) {
    const int b = m & 1;
    uint32_t kch[2][4], kcl[2][4];
    u32x4 vkeep[2];
    // ---- part 1 (step 2m-3); in the carry launch this is the longest
    // chain of its step, so it goes ahead of the (younger) T helpers
    if (fwd) __builtin_amdgcn_s_setprio(2);
    {
      float kf[2][8], qf[2][8], G[2][8];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          kf[j][2 * w] = __uint_as_float(rk[j][w] << 16);
          kf[j][2 * w + 1] = __uint_as_float(rk[j][w] & 0xffff0000u);
          if (fwd) {
            qf[j][2 * w] = __uint_as_float(rq[j][w] << 16);
            qf[j][2 * w + 1] = __uint_as_float(rq[j][w] & 0xffff0000u);
          }
          G[j][2 * w] = __uint_as_float(rg[j][w] << 16) * kLog2e;
          G[j][2 * w + 1] = __uint_as_float(rg[j][w] & 0xffff0000u) * kLog2e;
        }
        if (fwd) vkeep[j] = rv[j];
        if (!fwd) {
#pragma unroll
          for (int c = 0; c < 8; ++c) asm volatile("" : "+v"(kf[j][c]));
        }
      }
      if (p.gate_floor_on) {
        // the optional safe gate: every log-decay at least the lower bound
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int c = 0; c < 8; ++c) G[j][c] = fmaxf(G[j][c], p.gate_floor);
      }
      if (oh == 0 && lane < CH) sm.beta[b][lane] = __uint_as_float(rb << 16);
      __builtin_amdgcn_sched_barrier(0);
      fetch(beg + (m + 1) * CH);

      scan_stage<0x111, 2>(G);   // row_shr:1
      scan_stage<0x112, 2>(G);   // row_shr:2
      scan_stage<0x114, 2>(G);   // row_shr:4
      scan_stage<0x118, 2>(G);   // row_shr:8
      float a[8], gc[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        a[c] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(G[0][c]), 0x1F0));
        gc[c] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(G[1][c]), 0x1F0));
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        G[1][c] += a[c];
        gc[c] += a[c];
      }
      {
        float t[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) t[c] = a[c] + dprev[c];
        store_fac(b, t);
      }
      // The anchored form keeps every in-chunk factor 2^(G_i - a) within
      // 2^+-kFactorMax when the anchor's decay a and the anchor-to-end decay
      // G_C - a both stay above -kFactorMax (g <= 0: the extremes are token
      // 0, at most -a, and token 31).  Beyond that on any channel of any
      // chunk the fragment's results are discarded and it runs again.
      float dmin = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        dprev[c] = gc[c] - a[c];
        dmin = fminf(dmin, fminf(a[c], dprev[c]));
      }
      rerun_w |= __builtin_amdgcn_ballot_w64(!(dmin >= -kFactorMax)) != 0;

#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t krh[4], krl[4], qrh[4], qrl[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float kr[2], kc[2], qr[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const float x = G[j][2 * w + c] - a[2 * w + c];
            const float er = __builtin_amdgcn_exp2f(x);
            const float ec = __builtin_amdgcn_exp2f(-x);
            kr[c] = kf[j][2 * w + c] * er;
            kc[c] = kf[j][2 * w + c] * ec;
            if (fwd) qr[c] = qf[j][2 * w + c] * er;
          }
          split_pair_dead(kr[0], kr[1], krh[w], krl[w]);
          split_pair_dead(kc[0], kc[1], kch[j][w], kcl[j][w]);
          if (fwd) split_pair_dead(qr[0], qr[1], qrh[w], qrl[w]);
        }
        const int off = (tk + 16 * j) * NS + c8;
        // rows 16 .. 31 with exchanged halves in the carry launch
        st4(&sm.kr_h[b][off], sw_rows(fwd && j, krh));
        st4(&sm.kr_l[b][off], sw_rows(fwd && j, krl));
        if (fwd) {
          st4(&sm.qr_h[b][off], sw_rows(j, qrh));
          st4(&sm.qr_l[b][off], sw_rows(j, qrl));
        }
      }
    }
    block_sync();
    if (fwd) __builtin_amdgcn_s_setprio(0);
    // ---- part 2 (step 2m-2)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int off = (tk + 16 * j) * NS + c8;
      st4(&sm.kc_h[b][off], sw_rows(fwd && j, kch[j]));
      st4(&sm.kc_l[b][off], sw_rows(fwd && j, kcl[j]));
      st4(&sm.vv[b][off], sw_rows(fwd && j, fwd ? vkeep[j] : rv[j]));
    }
    if (!fwd) fetch_v(beg + (m + 1) * CH);
    block_sync();
  }
  // step 2nc-3: R *= e^{G_C - a} after the last chunk turns R back into S
  store_fac(nc & 1, dprev);
  if (lane == 0) sm.rerun[oh] = rerun_w ? 1 : 0;
  block_sync();
  block_sync();   // steps 2nc-2, 2nc-1
  block_sync();
  if (fragment_rerun(sm)) {
    // The token-by-token re-run: block m's k, q and per-token decay as FP32
    // rows, v and beta as in the pipeline, then the owners' turn.
    for (int m = 0; m < nc; ++m) {
      const int b = m & 1;
      fetch(beg + m * CH);
      if (!fwd) fetch_v(beg + m * CH);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float kx[8], dx[8], qx[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          kx[2 * w] = __uint_as_float(rk[j][w] << 16);
          kx[2 * w + 1] = __uint_as_float(rk[j][w] & 0xffff0000u);
          // (gate_floor is -inf when the safe gate is off)
          dx[2 * w] = __builtin_amdgcn_exp2f(
              fmaxf(fmaxf(__uint_as_float(rg[j][w] << 16) * kLog2e, p.gate_floor), kGateFloor));
          dx[2 * w + 1] = __builtin_amdgcn_exp2f(
              fmaxf(fmaxf(__uint_as_float(rg[j][w] & 0xffff0000u) * kLog2e, p.gate_floor), kGateFloor));
          qx[2 * w] = __uint_as_float(rq[j][w] << 16);
          qx[2 * w + 1] = __uint_as_float(rq[j][w] & 0xffff0000u);
        }
        float* kd = tok_rows(sm.kr_h[b], sm.kr_l[b], tk + 16 * j) + c8;
        float* dd = tok_rows(sm.kc_h[b], sm.kc_l[b], tk + 16 * j) + c8;
        st4(kd, f32x4{kx[0], kx[1], kx[2], kx[3]});
        st4(kd + 4, f32x4{kx[4], kx[5], kx[6], kx[7]});
        st4(dd, f32x4{dx[0], dx[1], dx[2], dx[3]});
        st4(dd + 4, f32x4{dx[4], dx[5], dx[6], dx[7]});
        if (fwd) {
          float* qd = tok_rows(sm.qr_h[b], sm.qr_l[b], tk + 16 * j) + c8;
          st4(qd, f32x4{qx[0], qx[1], qx[2], qx[3]});
          st4(qd + 4, f32x4{qx[4], qx[5], qx[6], qx[7]});
        }
        st4(&sm.vv[b][(tk + 16 * j) * NS + c8], sw_rows(fwd && j, rv[j]));
      }
      if (oh == 0 && lane < CH) sm.beta[b][lane] = __uint_as_float(rb << 16);
      block_sync();
      block_sync();
    }
  }
}

// T helper th (0..3) of the pipeline.  Part 1 of chunk m (step 2m-1) computes
// the diagonal blocks of A and their inverses (th 0, 1) and A10 (th 2), and
// part 2 (step 2m) merges them into T diag(beta), four columns per helper.
// The summaries launch (FILL) also copies each chunk's T diag(beta) into the
// chunk cache during the next chunk's part 1, while it is still in LDS.  The
// carry launch instead loads it from the cache in part 1 and stores it to LDS
// in part 2 for every fragment that the summaries launch ran (those that end
// their segment).  It also computes the three blocks of P in part 1 and
// stores them in part 2: one block on each of th 0-2 where T diag(beta) comes
// from the cache, all three on th 3 where th 0-2 build it.
template <bool FILL, bool UNSC = false>
__device__ __forceinline__ void pipe_thelper(const ChunkParams& p, PipeSmem& sm, const int h, const int th,
                                             const int32_t flags,
                                             const int32_t seg, const int32_t beg, const int32_t end) {
  const int lane = threadIdx.x & 63;
  const int nc = (end - beg + CH - 1) / CH;
  const bool cached = !FILL && (flags & kFragSegLast) != 0;
  const int ci = 64 * th + lane;   // this lane's 16 bytes of a cached chunk
  auto to_cache = [&](const int m) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(&((ci >> 7) ? sm.tb_l : sm.tb_h)[cache_lds(ci)]);
    *reinterpret_cast<u32x4*>(p.chunk_cache + cache_elem(p, h, seg, beg, m, ci)) = v;
  };
  block_sync();   // steps -3, -2: the operands of chunk 0 are being built
  block_sync();
  for (int m = 0; m < nc; ++m) {
    const int b = m & 1;
    f32x4 pacc[3];
    u32x4 tbv;
    // the solves are the longest chain of the summaries launch's step 2m-1;
    // without a raised priority the T helpers, the youngest waves, lose
    // every issue slot to the others
    if (FILL) __builtin_amdgcn_s_setprio(3);
    {
      const int lane_s = opaque(lane);
      if (FILL && m > 0) to_cache(m - 1);
      if (cached) {
        tbv = *reinterpret_cast<const u32x4*>(p.chunk_cache + cache_elem(p, h, seg, beg, m, ci));
      } else if (th < 2) {
        a_diag_solve(sm.kr_h[b], sm.kr_l[b], sm.kc_h[b], sm.kc_l[b], sm.beta[b], sm.an, sm.tt, sm.tn, th, lane_s);
      } else if (th == 2) {
        a_offdiag<!FILL>(sm.kr_h[b], sm.kr_l[b], sm.kc_h[b], sm.kc_l[b], sm.beta[b], sm.an, lane_s);
      }
      if (!FILL) {
        const int lm = lane_s & 15;
        const int lg = lane_s >> 4;
        if (cached) {
          // T helpers 0-2 are free here: one P block each
          if (th == 1) pacc[0] = tile16<true>(sm.qr_h[b], sm.qr_l[b], sm.kc_h[b], sm.kc_l[b], 1, 0, lm, lg);
          else if (th < 3) pacc[0] = tile16(sm.qr_h[b], sm.qr_l[b], sm.kc_h[b], sm.kc_l[b], th > 0, th > 1, lm, lg);
        } else if (th == 3) {
          pacc[0] = tile16(sm.qr_h[b], sm.qr_l[b], sm.kc_h[b], sm.kc_l[b], 0, 0, lm, lg);
          pacc[1] = tile16<true>(sm.qr_h[b], sm.qr_l[b], sm.kc_h[b], sm.kc_l[b], 1, 0, lm, lg);
          pacc[2] = tile16(sm.qr_h[b], sm.qr_l[b], sm.kc_h[b], sm.kc_l[b], 1, 1, lm, lg);
        }
      }
    }
    block_sync();
    if (FILL) __builtin_amdgcn_s_setprio(0);
    {
      const int lane_s = opaque(lane);
      if (cached) st4(&((ci >> 7) ? sm.tb_l : sm.tb_h)[cache_lds(ci)], tbv);
      else t_merge<UNSC>(sm.an, sm.tt, sm.tn, sm.xt, sm.beta[b], sm.tb_h, sm.tb_l, th, lane_s);
      if (!FILL) {
        if (cached) {
          if (th < 3) p_store(pacc[0], th > 0, th > 1, sm.p_h, sm.p_l, lane_s);
        } else if (th == 3) {
          p_store(pacc[0], 0, 0, sm.p_h, sm.p_l, lane_s);
          p_store(pacc[1], 1, 0, sm.p_h, sm.p_l, lane_s);
          p_store(pacc[2], 1, 1, sm.p_h, sm.p_l, lane_s);
        }
      }
    }
    block_sync();
  }
  if (FILL) to_cache(nc - 1);
  block_sync();   // step 2nc-1
  if (fragment_rerun(sm)) {
    for (int m = 0; m < 2 * nc; ++m) block_sync();   // the re-run's barriers
  }
}

// Helper wave with nothing to compute: keeps the barrier count of a fragment
// (including the re-run's, when some chunk is beyond the anchored form).
__device__ __forceinline__ void pipe_idle(const PipeSmem& sm, const int32_t beg, const int32_t end) {
  const int nc = (end - beg + CH - 1) / CH;
  for (int i = 0; i < 2 * nc + 3; ++i) block_sync();
  if (fragment_rerun(sm)) {
    for (int m = 0; m < 2 * nc; ++m) block_sync();
  }
}

// The state a fragment starts from, for this head: the carry-in C_r where it
// continues a sequence across its segment's start (carry launch; the
// summaries launch runs B_r from zero there), else it starts a sequence and
// begins at that sequence's initial state, if any.
__device__ __forceinline__ const float* start_state(const ChunkParams& p, const int h_, const int32_t flags,
                                                    const int32_t seg,
                                                    const int32_t seq, const bool carry_launch) {
  const size_t h = static_cast<size_t>(h_);
  if ((flags & kFragCarried) != 0)
    return carry_launch ? p.carry + (static_cast<size_t>(seg) * p.H + h) * KD * VD : nullptr;
  return p.init_state != nullptr ? p.init_state + (static_cast<size_t>(seq) * p.H + h) * KD * VD : nullptr;
}

// Summaries launch: one workgroup per fragment that ends its segment and
// head.  Waves 0-3 own the update B_r (the fragment from a zero state),
// waves 4-7 the transition A_r (from the identity with V = 0) when the
// segment's sequence runs through it, else they write A_r = 0; waves 8-11
// are the operand helpers and 12-15 the T helpers, shared by both states.
__global__ void __launch_bounds__(kSummaryThreads, 1) kda_chunk_kernel(ChunkParams p) {
  __shared__ PipeSmem sm;
  const int64_t rank = block_rank(p);
  if (rank >= p.plan[3]) return;   // padding of the grid (header word 3 is F)
  const int f = p.plan[p.L.frag_order + static_cast<int>(rank)];
  const int h = block_head(p);
  const int tid = threadIdx.x;
  const int32_t flags = p.plan[p.L.frag_flags + f];
  const int32_t seg = p.plan[p.L.frag_seg + f];
  const Work work = decode_summary(p, flags, seg);
  if (!work.run) return;
  const int32_t seq = p.plan[p.L.frag_seq + f];
  const int32_t beg = p.plan[p.L.frag_begin + f];
  const int32_t end = p.plan[p.L.frag_end + f];
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave < NOWN) {
    pipe_owner<kModeSumS>(p, sm, h, wave, flags, seg, seq, beg, end, start_state(p, h, flags, seg, seq, false));
  } else if (wave < 2 * NOWN) {
    if (work.phi) {
      pipe_owner<kModeSumPhi>(p, sm, h, wave - NOWN, flags, seg, seq, beg, end, nullptr);
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(p.transitions + (static_cast<size_t>(seg) * p.H + h) * KD * KD);
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      for (int i = tid - NOWN * 64; i < KD * KD / 4; i += NOWN * 64) dst[i] = z;
      pipe_idle(sm, beg, end);
    }
  } else if (wave < 3 * NOWN) {
    pipe_ophelper<kModeSumS>(p, sm, h, wave - 2 * NOWN, beg, end);
  } else {
    pipe_thelper<true>(p, sm, h, wave - 3 * NOWN, flags, seg, beg, end);
  }
}

// Carry launch: every fragment runs with the forward body (o and, where a
// sequence ends, the final state), from its segment's carry-in C_r when it
// continues a sequence, else from its sequence's initial state (or zero).
__global__ void __launch_bounds__(kCarryThreads, 1) kda_carry_kernel(ChunkParams p) {
  __shared__ PipeSmem sm;
  const int64_t rank = block_rank(p);
  if (rank >= p.plan[3]) return;   // padding of the grid (header word 3 is F)
  const int f = p.plan[p.L.frag_order + static_cast<int>(rank)];
  const int h = block_head(p);
  const int tid = threadIdx.x;
  const int32_t flags = p.plan[p.L.frag_flags + f];
  const int32_t seg = p.plan[p.L.frag_seg + f];
  const int32_t seq = p.plan[p.L.frag_seq + f];
  const int32_t beg = p.plan[p.L.frag_begin + f];
  const int32_t end = p.plan[p.L.frag_end + f];
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave < NOWN) pipe_owner<kModeFwd>(p, sm, h, wave, flags, seg, seq, beg, end, start_state(p, h, flags, seg, seq, true));
  else if (wave < 2 * NOWN) pipe_ophelper<kModeFwd>(p, sm, h, wave - NOWN, beg, end);
  else pipe_thelper<false>(p, sm, h, wave - 2 * NOWN, flags, seg, beg, end);
}

// Checkpoint launch of the chunked backward: every fragment, forward from its
// segment's carry-in (or its sequence's initial state, or zero) without o,
// storing the anchored state entering each chunk, V - Kr R and T (without
// diag(beta)) of each chunk at slot floor(begin / 32) + f + chunk (the fragment index f in
// place of the segment's: every fragment gets its own slots), and whether the
// fragment left the anchored form's range.  Waves as in the carry launch.
__global__ void __launch_bounds__(kCarryThreads, 1) kda_ckpt_kernel(ChunkParams p) {
  __shared__ PipeSmem sm;
  const int64_t rank = block_rank(p);
  if (rank >= p.plan[3]) return;   // padding of the grid (header word 3 is F)
  const int f = p.plan[p.L.frag_order + static_cast<int>(rank)];
  const int h = block_head(p);
  const int tid = threadIdx.x;
  const int32_t flags = p.plan[p.L.frag_flags + f];
  const int32_t seg = p.plan[p.L.frag_seg + f];
  const int32_t seq = p.plan[p.L.frag_seq + f];
  const int32_t beg = p.plan[p.L.frag_begin + f];
  const int32_t end = p.plan[p.L.frag_end + f];
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (h == p.h0 && wave == 2 * NOWN) {
    // the slot map: this fragment's chunks, then the unused slot (if any)
    // before the next fragment's first
    const int32_t s0 = beg / CH + f;
    const int32_t nc = (end - beg + CH - 1) / CH;
    const int32_t F = p.plan[3];
    const int32_t s1 = f + 1 < F ? p.plan[p.L.frag_begin + f + 1] / CH + f + 1 : (p.plan[0] + CH - 1) / CH + F;
    for (int32_t s = s0 + (tid & 63); s < s1; s += 64) p.slot_map[s] = s - s0 < nc ? f : -1;
  }
  if (wave < NOWN)
    pipe_owner<kModeCkpt>(p, sm, h, wave, flags, seg, seq, beg, end, start_state(p, h, flags, seg, seq, true),
                          static_cast<int64_t>(beg / CH) + f);
  else if (wave < 2 * NOWN) pipe_ophelper<kModeSumS>(p, sm, h, wave - NOWN, beg, end);
  else pipe_thelper<true, true>(p, sm, h, wave - 2 * NOWN, flags, f, beg, end);
}

}  // namespace kda
