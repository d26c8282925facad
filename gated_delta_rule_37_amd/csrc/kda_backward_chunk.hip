// Chunked backward of the KDA recurrence on the bf16 matrix cores (gfx950).
//
// Sources: inclusionAI/cuLA pull request #110 "feat(cp): add opt-in NVSHMEM CP
// state handoff" (Correctness: output and Q/K/V/g/beta gradients) and pull
// request #136 "feat(kda): add cuDNN concatenated-summary Kimi CP" (Sequence
// Diagram: the backward gathers the following ranks' summaries).  The pages
// give no formulas; the chunk form below is derived from the recurrence.
//
// Per chunk of C = 32 tokens (a ragged last chunk is padded with zero
// tokens), with G the in-chunk prefix of g, a = G_15 the anchor and
// Gc = G_31 (log2 units on the device):
//     Kr = k e^{G-a},  Kc = k e^{a-G},  Qr = q e^{G-a}
//     A' = strict_lower(Kr Kc^T),  T = (I + diag(beta) A')^-1,  P = lower_incl(Qr Kc^T)
// The checkpoint launch (kda_ckpt_kernel) stores R_c = e^{a} o S_c, the state
// entering chunk c with its rows scaled by the anchor, and T diag(beta).
// Pass 2 (kda_bwd_chain_kernel) runs each fragment's cotangent backwards in
// the same anchored frame:
//     D_c = fac_c o Delta_{c+1}         (fac_c = e^{a_{c+1} + Gc_c - a_c}; at the
//                                        fragment's end e^{Gc - a} o dS_end)
//     dU  = P^T dO + Kc D_c,  dR = diag(beta) T^T dU
//     Delta_c = D_c + Qr^T dO - Kr^T dR,   dS_start = e^{a_0} o Delta_0
// and stores every D_c and dU.  Pass 3 (kda_bwd_grad_kernel) takes every
// chunk on its own from R_c, D_c, dU and the checkpoint launch's V - Kr R_c:
//     W = Kr R,  X = diag(beta)(V - W),  U = T X,  dU = P^T dO + Kc D
//     dX = T^T dU,  dv = dR = diag(beta) dX,  dA = strict_lower(-dX U^T)
//     dbeta = rowsum(dX o (V - W)) + rowsum(dA o A'),  dA' = diag(beta) dA
//     dP = lower_incl(dO U^T)
//     dq = (dO R^T + dP Kc) o e^{G-a}
//     dk = (-dR R^T + dA' Kc) o e^{G-a} + (dP^T Qr + dA'^T Kr + U D^T) o e^{a-G}
//     dG = q o dq + k o (dk_d - dk_i - dk_h),  dG_31 += colsum(k o dk_h) + rowsum(D o R)
//     dg = the reverse in-chunk prefix sum of dG (natural units)
// with dk_d, dk_i, dk_h the three terms of dk.  Every product is split bf16
// (hi*hi + hi*lo + lo*hi) with FP32 accumulation, as in the forward.  A
// fragment whose chunks leave the anchored form's range (flagged by the
// checkpoint launch) takes the token-by-token kernels instead.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int KD = 128;
constexpr int VD = 128;
constexpr int CH = 32;
constexpr int NB = 136;   // row stride (bf16) of the gradient launch's token-major [32][128] planes
constexpr int NC = 152;   // the chain launch's (conflict-free transposed reads; more LDS)
// Cache policy of stores that nothing in the same launch reads back (the
// cotangents, dU and the gradients): non-temporal, leaving the caches to the
// launch's own inputs.
constexpr int kWriteOnce = 2;
constexpr int TB = 40;    // row stride (bf16) of the 32 x 32 matrices (columns in k-slot order)
constexpr int FS = 36;    // row stride (fp32) of the 16 x 16 solve tiles
constexpr int AS = 33;    // row stride (fp32) of A'
constexpr int GS = 132;   // row stride (fp32) of the G - a plane
constexpr float kLog2eC = 1.4426950408889634f;
constexpr int kW3 = 0x00020000;   // raw buffer resource word 3 (gfx9): reads past the count give 0
constexpr size_t MATF = static_cast<size_t>(KD) * VD;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t res(const void* base, const uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kW3);
}

// Column fragment of a token-major plane: lane l receives column c0 + l % 32,
// tokens 16s + 4(l/32) + 0..3 and 16s + 8 + 4(l/32) + 0..3 (the k-slot order
// of k-step s), by two transposed reads.
template <int S = NB>
__device__ __forceinline__ int tr_base(const int lane) {
  return (4 * (lane >> 5) + ((lane & 15) >> 2)) * S + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
}
template <int S = NB>
__device__ __forceinline__ bf16x8 colfrag(const bf16* plane, const int s, const int c0, const int trb) {
  const bf16* p = plane + trb + 16 * s * S + c0;
  return join8(lds_read_tr(p), lds_read_tr(p + 8 * S));
}
// Row fragment: row l % 32, columns 16kk + 4(l/32) + 0..3 and 16kk + 8 +
// 4(l/32) + 0..3 (the same k-slot order over the 128 channels).
__device__ __forceinline__ bf16x8 rowfrag(const bf16* plane, const int kk, const int pro) {
  return ld_kslots_at(plane + pro + 16 * kk);
}
// Row l % 32 of a 32 x 32 matrix stored with its columns in k-slot order:
// the k-slots of k-step s in one 16-byte read.
__device__ __forceinline__ bf16x8 smallrow(const bf16* m, const int s, const int tbo) {
  return *reinterpret_cast<const bf16x8*>(m + tbo + 16 * s);
}

// k-slot position of token t inside its 16-token group (bits 2 and 3 swapped)
__device__ __forceinline__ int kpos(const int t) { return kslot_col(t); }

// Stores of a 32 x 32 accumulator tile (lane l: column j = l % 32, rows
// i = 8r + 4(l/32) + e in register 4r + e) as split bf16:
//   store_t: dst[j][kpos(i)] (the transposed matrix, columns in k-slot order;
//            four consecutive positions per r, one 8-byte store each);
//   store_n: dst[i][kpos(j)] (two-byte stores).
__device__ __forceinline__ void store_t(const f32x16& t, bf16* dh, bf16* dl, const int lane) {
  const int j = lane & 31;
  const int lh = lane >> 5;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t h0, l0, h1, l1;
    split_pair(t[4 * r], t[4 * r + 1], h0, l0);
    split_pair(t[4 * r + 2], t[4 * r + 3], h1, l1);
    const int pos = j * TB + 16 * (r >> 1) + 8 * lh + 4 * (r & 1);
    *reinterpret_cast<uint2*>(dh + pos) = make_uint2(h0, h1);
    *reinterpret_cast<uint2*>(dl + pos) = make_uint2(l0, l1);
  }
}
__device__ __forceinline__ void store_n(const f32x16& t, bf16* dh, bf16* dl, const int lane) {
  const int j = lane & 31;
  const int lh = lane >> 5;
  const int pj = kpos(j);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf16 hh, ll;
      split(t[4 * r + e], hh, ll);
      dh[(8 * r + 4 * lh + e) * TB + pj] = hh;
      dl[(8 * r + 4 * lh + e) * TB + pj] = ll;
    }
}
// A tile with rows = channels c0 + 8r + 4(l/32) + e and column = token l % 32
// into a token-major plane (row = token): four consecutive channels per r.
__device__ __forceinline__ void store_plane_t(const f32x16& t, bf16* ph, bf16* pl, const int c0, const int lane) {
  const int i = lane & 31;
  const int lh = lane >> 5;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t h0, l0, h1, l1;
    split_pair(t[4 * r], t[4 * r + 1], h0, l0);
    split_pair(t[4 * r + 2], t[4 * r + 3], h1, l1);
    const int pos = i * NB + c0 + 8 * r + 4 * lh;
    *reinterpret_cast<uint2*>(ph + pos) = make_uint2(h0, h1);
    *reinterpret_cast<uint2*>(pl + pos) = make_uint2(l0, l1);
  }
}

// 16 x 16 block (rb, ct) of X C^T over the 128 channels (16x16x32 MFMAs):
// lane l gets rows 16rb + 4(l/16) + e, e = 0..3, of column 16ct + l % 16.
template <int S = NB>
__device__ __forceinline__ f32x4 tile16c(const bf16* xh, const bf16* xl, const bf16* ch, const bf16* cl, const int rb,
                                         const int ct, const int lane) {
  const int lm = lane & 15;
  const int lg = lane >> 4;
  f32x4 acc = zero4();
#pragma unroll
  for (int kk = 0; kk < KD / 32; ++kk) {
    const int ao = (16 * rb + lm) * S + 32 * kk + 8 * lg;
    const int bo = (16 * ct + lm) * S + 32 * kk + 8 * lg;
    acc = mfma16x3(*reinterpret_cast<const bf16x8*>(xh + ao), *reinterpret_cast<const bf16x8*>(xl + ao),
                   *reinterpret_cast<const bf16x8*>(ch + bo), *reinterpret_cast<const bf16x8*>(cl + bo), acc);
  }
  mfma_result_fence(acc);
  return acc;
}

// ---------------------------------------------------------------------------
// One chunk's inputs for an operand builder (4 waves, wave ob = 0..3): lane l
// holds channels c8 .. c8+7 (c8 = 32 ob + 8(l/16)) of tokens l % 16 and
// 16 + l % 16: k, g, q as bf16 and dO as FP32.  Loads past the chunk's n
// tokens return zero.
struct ChunkIn {
  u32x4 k[2], g[2], q[2];
  f32x4 d[2][2];
};

__device__ __forceinline__ void fetch_chunk(const BwdParams& p, const int h, const int c0, const int n, const int ob,
                                            const int lane, ChunkIn& x) {
  const int H = p.H;
  const int tk = lane & 15;
  const int c8 = 32 * ob + 8 * (lane >> 4);
  const size_t base = (static_cast<size_t>(c0) * H + h) * KD;
  const uint32_t row = static_cast<uint32_t>(H) * KD * 2;
  const uint32_t nrec = (n - 1) * row + KD * 2;
  const auto rk = res(p.k + base, nrec);
  const auto rg = res(p.g + base, nrec);
  const auto rq = res(p.q + base, nrec);
  const uint32_t rowf = static_cast<uint32_t>(H) * VD * 4;
  const auto rd = res(p.d_o + base, (n - 1) * rowf + VD * 4);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int off = (tk + 16 * j) * row + 2 * c8;
    x.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    x.g[j] = __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0);
    x.q[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      x.d[j][hf] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, (tk + 16 * j) * rowf + 4 * (c8 + 4 * hf), 0, 0));
  }
}

struct Planes {
  bf16 *krh, *krl, *kch, *kcl, *qrh, *qrl, *doh, *dol;
};

// The chunk's Kr, Kc, Qr and dO as split bf16 token-major planes, and (gl
// non-null) G - a per token and channel; a and gc (= G_31) of the lane's
// eight channels in log2 units.  The in-chunk prefix runs across the 16
// lanes of a DPP row (4 row shifts); the anchor and G_31 are the rows' last
// lanes.
// Kr's two 16-byte row pieces of the lane (tokens l % 16 and 16 + l % 16),
// hi and lo, for a builder that stores them a step later.
struct KrHeld {
  u32x4 h[2], l[2];
};
template <int S = NB>
__device__ __forceinline__ void store_kr(const KrHeld& k, bf16* krh, bf16* krl, const int ob, const int lane) {
  const int tk = lane & 15;
  const int c8 = 32 * ob + 8 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    st4(krh + (tk + 16 * j) * S + c8, k.h[j]);
    st4(krl + (tk + 16 * j) * S + c8, k.l[j]);
  }
}
template <int S = NB>
__device__ __forceinline__ void build_chunk(const ChunkIn& x, const Planes& P, float* gl, const int ob, const int lane,
                                            float (&a)[8], float (&gc)[8], KrHeld* held = nullptr) {
  const int tk = lane & 15;
  const int c8 = 32 * ob + 8 * (lane >> 4);
  float kf[2][8], qf[2][8], G[2][8];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      kf[j][2 * w] = __uint_as_float(x.k[j][w] << 16);
      kf[j][2 * w + 1] = __uint_as_float(x.k[j][w] & 0xffff0000u);
      qf[j][2 * w] = __uint_as_float(x.q[j][w] << 16);
      qf[j][2 * w + 1] = __uint_as_float(x.q[j][w] & 0xffff0000u);
      G[j][2 * w] = __uint_as_float(x.g[j][w] << 16) * kLog2eC;
      G[j][2 * w + 1] = __uint_as_float(x.g[j][w] & 0xffff0000u) * kLog2eC;
    }
  scan_stage<0x111, 2>(G);   // row_shr:1
  scan_stage<0x112, 2>(G);   // row_shr:2
  scan_stage<0x114, 2>(G);   // row_shr:4
  scan_stage<0x118, 2>(G);   // row_shr:8
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    a[c] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(G[0][c]), 0x1F0));
    gc[c] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(G[1][c]), 0x1F0)) + a[c];
    G[1][c] += a[c];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t krh[4], krl[4], kch[4], kcl[4], qrh[4], qrl[4], dh[4], dl[4];
    float xs[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float kr[2], kc[2], qr[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float xx = G[j][2 * w + c] - a[2 * w + c];
        xs[2 * w + c] = xx;
        const float er = __builtin_amdgcn_exp2f(xx);
        const float ec = __builtin_amdgcn_exp2f(-xx);
        kr[c] = kf[j][2 * w + c] * er;
        kc[c] = kf[j][2 * w + c] * ec;
        qr[c] = qf[j][2 * w + c] * er;
      }
      split_pair_dead(kr[0], kr[1], krh[w], krl[w]);
      split_pair_dead(kc[0], kc[1], kch[w], kcl[w]);
      split_pair_dead(qr[0], qr[1], qrh[w], qrl[w]);
      const f32x4& dv = x.d[j][w >> 1];
      split_pair(dv[2 * (w & 1)], dv[2 * (w & 1) + 1], dh[w], dl[w]);
    }
    const int off = (tk + 16 * j) * S + c8;
    if (held != nullptr) {
      held->h[j] = u32x4{krh[0], krh[1], krh[2], krh[3]};
      held->l[j] = u32x4{krl[0], krl[1], krl[2], krl[3]};
    } else {
      st4(P.krh + off, u32x4{krh[0], krh[1], krh[2], krh[3]});
      st4(P.krl + off, u32x4{krl[0], krl[1], krl[2], krl[3]});
    }
    st4(P.kch + off, u32x4{kch[0], kch[1], kch[2], kch[3]});
    st4(P.kcl + off, u32x4{kcl[0], kcl[1], kcl[2], kcl[3]});
    st4(P.qrh + off, u32x4{qrh[0], qrh[1], qrh[2], qrh[3]});
    st4(P.qrl + off, u32x4{qrl[0], qrl[1], qrl[2], qrl[3]});
    st4(P.doh + off, u32x4{dh[0], dh[1], dh[2], dh[3]});
    st4(P.dol + off, u32x4{dl[0], dl[1], dl[2], dl[3]});
    if (gl != nullptr) {
      st4(gl + (tk + 16 * j) * GS + c8, f32x4{xs[0], xs[1], xs[2], xs[3]});
      st4(gl + (tk + 16 * j) * GS + c8 + 4, f32x4{xs[4], xs[5], xs[6], xs[7]});
    }
  }
}

// ===========================================================================
// Pass 2: the cotangent chain of one fragment, chunks from the last.  Twelve
// waves in three roles, as in the forward's pipeline:
//   owners (0-3)           the anchored cotangent Delta, columns [32w, 32w+32)
//                          as four 32 x 32 FP32 accumulator tiles (rows =
//                          channels 32dt + 8r + 4(l/32) + e)
//   operand builders (4-7) Kr, Kc, Qr, dO and fac of a chunk
//   T helpers (8-11)       P^T from Kr, Kc planes; T transposed from the
//                          checkpoint launch's cache
// With m the position of chunk c = nc-1-m in that order, each step ending
// with a barrier:
//   step 2m     builders: chunk m's planes and fac into buffer m & 1 (its Kr
//               into the single Kr plane at step 2m+2, after the owners'
//               last read of chunk m-1's)
//   step 2m+1   T helpers: P(m)^T, and the cache load of T(m)
//   step 2m+2   T helpers: T(m)^T;  owners: D = fac o Delta, store D,
//               dU = Kc D + P^T dO
//   step 2m+3   owners: dR = diag(beta) T^T dU, Delta = D + Qr^T dO - Kr^T dR
//   step 2nc    builders: e^{a_0} (the last rescale) into buffer nc & 1
// (every wave takes 2nc + 2 barriers).  The planes are double-buffered by m
// except Kr; P^T and T diag(beta)^T are single (each written one step after
// its last reader).  Rows are 152 elements apart, which keeps the transposed
// reads free of bank conflicts.
// ===========================================================================
struct alignas(16) ChainSmem {
  bf16 kr_h[CH * NC], kr_l[CH * NC];   // single: stored a step after the others
  bf16 kc_h[2][CH * NC], kc_l[2][CH * NC];
  bf16 qr_h[2][CH * NC], qr_l[2][CH * NC];
  bf16 do_h[2][CH * NC], do_l[2][CH * NC];
  bf16 pt_h[CH * TB], pt_l[CH * TB];   // P^T, columns in k-slot order
  bf16 tt_h[CH * TB], tt_l[CH * TB];   // T^T, columns in k-slot order
  float beta[2][CH];
  float fac[2][KD];
  alignas(16) int16_t fexp[2][KD];     // power-of-two part of fac (0: none)
  int32_t fsplit[2][4];                // per builder: some channel has one
};

__device__ __forceinline__ Planes chain_planes(ChainSmem& sm, const int b) {
  return Planes{sm.kr_h, sm.kr_l, sm.kc_h[b], sm.kc_l[b], sm.qr_h[b], sm.qr_l[b], sm.do_h[b], sm.do_l[b]};
}

// fac = 2^t for the lane's eight channels (lanes with l % 16 = 0 write).
// Where 2^t would leave the FP32 normal range it is stored as 2^(t - e) with
// an integer exponent e applied by ldexp, and the builder's flag is set.
__device__ __forceinline__ void put_fac(ChainSmem& sm, const int b, const int ob, const int lane, const float (&t)[8]) {
  const int tk = lane & 15;
  const int c8 = 32 * ob + 8 * (lane >> 4);
  float tmin = t[0];
#pragma unroll
  for (int c = 1; c < 8; ++c) tmin = fminf(tmin, t[c]);
  const bool sp = __builtin_amdgcn_ballot_w64(tk == 0 && tmin < -120.f) != 0;
  float fv[8];
  uint32_t ev[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int e = (sp && t[c] < -120.f) ? static_cast<int>(floorf(t[c])) + 60 : 0;
    ev[c >> 1] |= (static_cast<uint32_t>(e) & 0xffffu) << (16 * (c & 1));
    fv[c] = __builtin_amdgcn_exp2f(t[c] - static_cast<float>(e));
  }
  if (tk == 0) {
    st4(&sm.fac[b][c8], f32x4{fv[0], fv[1], fv[2], fv[3]});
    st4(&sm.fac[b][c8 + 4], f32x4{fv[4], fv[5], fv[6], fv[7]});
    *reinterpret_cast<u32x4*>(&sm.fexp[b][c8]) = u32x4{ev[0], ev[1], ev[2], ev[3]};
  }
  if (lane == 0) sm.fsplit[b][ob] = sp ? 1 : 0;
}

// The power-of-two part of fac, on the rare chunks where some channel has it
// (rows 32dt .. 32dt+31 are builder dt's channels, so its flag covers tile
// dt); the normal part is applied separately.  The two factors commute.
__device__ __forceinline__ void rescale_exp4(f32x16 (&D)[4], const ChainSmem& sm, const int b, const int lh) {
  const u32x4 fl = *reinterpret_cast<const u32x4*>(&sm.fsplit[b][0]);
  if (__builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3]) == 0) return;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    if (__builtin_amdgcn_readfirstlane(fl[dt]) == 0) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        D[dt][4 * r + e] = __builtin_ldexpf(D[dt][4 * r + e], sm.fexp[b][32 * dt + 8 * r + 4 * lh + e]);
  }
}

// Owner ow: the cotangent from the fragment's end back to its start.
template <bool E>
__device__ __forceinline__ void chain_owner(const BwdParams& p, ChainSmem& sm, const int h, const int ow, const int nc,
                                            const int64_t ck0, const float* end1, const float* end2, float* out) {
  const int H = p.H;
  const int lane = threadIdx.x & 63;
  const int lh = lane >> 5;
  const int col = 32 * ow + (lane & 31);
  f32x16 Dl[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) Dl[dt] = zero16();
  // the cotangent at the fragment's end (row 32dt + 8r + 4lh + e, column col)
  const int voff = 4 * (4 * lh * VD + col);
  auto add_end = [&](const float* src) {
    const auto rs = res(src, MATF * 4);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Dl[dt][4 * r + e] += __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(rs, voff, 4 * (32 * dt + 8 * r + e) * VD, 0));
  };
  if (end1 != nullptr) add_end(end1);
  if (end2 != nullptr) add_end(end2);
  const int pro = (lane & 31) * NC + 4 * lh;
  const int trb = tr_base<NC>(lane);
  const int tbo = (lane & 31) * TB + 8 * lh;
  __syncthreads();   // steps 0, 1
  __syncthreads();
  for (int m = 0; m < nc; ++m) {
    const int b = m & 1;
    const int c = nc - 1 - m;
    // ---- step 2m+2: per 32-row tile, D = fac o Delta (stored), then its
    // two k-steps of Kc D
    rescale_exp4(Dl, sm, b, lh);
    const auto rsd = res(p.dcot + (static_cast<size_t>(ck0 + c) * H + h) * MATF, MATF * 4);
    f32x16 Y = zero16();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 fv = ld4(&sm.fac[b][32 * dt + 8 * r + 4 * lh]);
#pragma unroll
        for (int e = 0; e < 4; ++e) Dl[dt][4 * r + e] *= fv[e];
      }
      if (!E) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(Dl[dt][4 * r + e]), rsd, voff,
                                                  4 * (32 * dt + 8 * r + e) * VD, kWriteOnce);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int kk = 2 * dt + s2;
        float xv[8];
        tile_kslots(Dl[dt], s2, xv);
        bf16x8 bh, bl;
        split8(xv, bh, bl);
        Y = mfma3(rowfrag(sm.kc_h[b], kk, pro), rowfrag(sm.kc_l[b], kk, pro), bh, bl, Y);
      }
    }
    bf16x8 doh[2], dol[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      doh[s] = colfrag<NC>(sm.do_h[b], s, 32 * ow, trb);
      dol[s] = colfrag<NC>(sm.do_l[b], s, 32 * ow, trb);
      Y = mfma3(smallrow(sm.pt_h, s, tbo), smallrow(sm.pt_l, s, tbo), doh[s], dol[s], Y);
    }
    __syncthreads();
    // ---- step 2m+3
    mfma_result_fence(Y);
    if (!E) {
      // dU for the gradient launch, [token][V]
      const auto rsu = res(p.dubuf + (static_cast<size_t>(ck0 + c) * H + h) * CH * VD, CH * VD * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(Y[4 * r + e]), rsu, voff, 4 * (8 * r + e) * VD,
                                                kWriteOnce);
    }
    bf16x8 uh[2], ul[2];
    tile_kslots_split(Y, uh, ul);
    f32x16 dR = zero16();
#pragma unroll
    for (int s = 0; s < 2; ++s) dR = mfma3(smallrow(sm.tt_h, s, tbo), smallrow(sm.tt_l, s, tbo), uh[s], ul[s], dR);
    mfma_result_fence(dR);
    // dR = diag(beta) T^T dU, negated for Delta -= Kr^T dR
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 bv = ld4(&sm.beta[b][8 * r + 4 * lh]);
#pragma unroll
      for (int e = 0; e < 4; ++e) dR[4 * r + e] *= -bv[e];
    }
    bf16x8 rh[2], rl[2];
    tile_kslots_split(dR, rh, rl);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        Dl[dt] = mfma3(colfrag<NC>(sm.qr_h[b], s, 32 * dt, trb), colfrag<NC>(sm.qr_l[b], s, 32 * dt, trb), doh[s], dol[s],
                       Dl[dt]);
        Dl[dt] = mfma3(colfrag<NC>(sm.kr_h, s, 32 * dt, trb), colfrag<NC>(sm.kr_l, s, 32 * dt, trb), rh[s], rl[s],
                       Dl[dt]);
      }
    }
    mfma_result_fence(Dl[0], Dl[1], Dl[2], Dl[3]);
    __syncthreads();
  }
  // the start of the fragment: dS = e^{a_0} o Delta_0
  rescale_exp4(Dl, sm, nc & 1, lh);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 fv = ld4(&sm.fac[nc & 1][32 * dt + 8 * r + 4 * lh]);
#pragma unroll
      for (int e = 0; e < 4; ++e) Dl[dt][4 * r + e] *= fv[e];
    }
  if (out != nullptr) {
    const auto rs = res(out, MATF * 4);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(Dl[dt][4 * r + e]), rs, voff,
                                                4 * (32 * dt + 8 * r + e) * VD, 0);
  }
}

__device__ __forceinline__ void chain_builder(const BwdParams& p, ChainSmem& sm, const int h, const int ob,
                                              const int beg, const int end, const int nc) {
  const int lane = threadIdx.x & 63;
  auto ntok = [&](const int c) { return min(CH, end - beg - CH * c); };
  ChunkIn x;
  fetch_chunk(p, h, beg + CH * (nc - 1), ntok(nc - 1), ob, lane, x);
  float anext[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) anext[c] = 0.f;
  KrHeld kr;   // chunk m's Kr, stored at step 2m+2 (the owners read the
               // previous chunk's until the end of step 2m+1)
  for (int m = 0; m < nc; ++m) {
    const int b = m & 1;
    const int c = nc - 1 - m;
    if (m > 0) store_kr<NC>(kr, sm.kr_h, sm.kr_l, ob, lane);
    if (ob == 0 && lane < CH) {
      const int n = ntok(c);
      const auto rb = res(p.beta + static_cast<size_t>(beg + CH * c) * p.H + h, (n - 1) * p.H * 2 + 2);
      sm.beta[b][lane] = __uint_as_float(
          static_cast<uint32_t>(static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rb, lane * p.H * 2, 0, 0)))
          << 16);
    }
    float a[8], gc[8];
    build_chunk<NC>(x, chain_planes(sm, b), nullptr, ob, lane, a, gc, &kr);
    if (c > 0) fetch_chunk(p, h, beg + CH * (c - 1), ntok(c - 1), ob, lane, x);
    float t[8];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      t[cc] = anext[cc] + (gc[cc] - a[cc]);
      anext[cc] = a[cc];
    }
    put_fac(sm, b, ob, lane, t);
    __syncthreads();   // step 2m
    __syncthreads();   // step 2m+1
  }
  store_kr<NC>(kr, sm.kr_h, sm.kr_l, ob, lane);   // the last chunk's, at step 2nc
  put_fac(sm, nc & 1, ob, lane, anext);   // e^{a_0}
  __syncthreads();   // step 2nc
  __syncthreads();   // step 2nc+1
}

__device__ __forceinline__ void chain_thelper(const BwdParams& p, ChainSmem& sm, const int h, const int th,
                                              const int nc, const int64_t ck0) {
  const int lane = threadIdx.x & 63;
  const int ci = 64 * th + lane;   // this lane's 16 bytes of a cached T diag(beta)
  const int which = ci >> 7;
  const int ti = (ci >> 2) & 31;
  const int tq = ci & 3;
  __syncthreads();   // step 0
  for (int m = 0; m < nc; ++m) {
    const int b = m & 1;
    const int c = nc - 1 - m;
    // ---- step 2m+1: P^T, cache load
    const u32x4 tv = *reinterpret_cast<const u32x4*>(
        p.tcache + (static_cast<size_t>(ck0 + c) * p.H + h) * (kChunkCacheBytes / 2) + which * (CH * CH) + ti * CH +
        8 * tq);
    const int lm = lane & 15;
    const int lg = lane >> 4;
    if (th < 3) {
      const int rb = th > 0;
      const int ct = th > 1;
      const f32x4 acc = tile16c<NC>(sm.qr_h[b], sm.qr_l[b], sm.kc_h[b], sm.kc_l[b], rb, ct, lane);
      // P[i][j], i = 16rb + 4lg + e, j = 16ct + lm, kept where j <= i, to
      // P^T[j][kpos(i)]
      uint32_t hv[2], lv[2];
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[e] = (16 * ct + lm <= 16 * rb + 4 * lg + e) ? acc[e] : 0.f;
      split_pair(pv[0], pv[1], hv[0], lv[0]);
      split_pair(pv[2], pv[3], hv[1], lv[1]);
      const int pos = (16 * ct + lm) * TB + 16 * rb + kpos(4 * lg);
      *reinterpret_cast<uint2*>(sm.pt_h + pos) = make_uint2(hv[0], hv[1]);
      *reinterpret_cast<uint2*>(sm.pt_l + pos) = make_uint2(lv[0], lv[1]);
    } else {
      // P^T rows 16..31, columns (tokens) 0..15: zero
      const int pos = (16 + lm) * TB + 4 * lg;
      *reinterpret_cast<uint2*>(sm.pt_h + pos) = make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(sm.pt_l + pos) = make_uint2(0u, 0u);
    }
    __syncthreads();
    // ---- step 2m+2: T^T[j][kpos(i)] = T[i][j]; the cache row holds column
    // j = kpos(8 tq + x) at position 8 tq + x
    {
      bf16* dst = which ? sm.tt_l : sm.tt_h;
      const int pi = kpos(ti);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dst[kpos(8 * tq + 2 * w) * TB + pi] = __builtin_bit_cast(bf16, static_cast<uint16_t>(tv[w] & 0xffffu));
        dst[kpos(8 * tq + 2 * w + 1) * TB + pi] = __builtin_bit_cast(bf16, static_cast<uint16_t>(tv[w] >> 16));
      }
    }
    __syncthreads();
  }
  __syncthreads();   // step 2nc+1
}

template <bool E>
__device__ __forceinline__ void chain_run(const BwdParams& p, const int f, const int hi, const int r_e) {
  __shared__ ChainSmem sm;
  const int h = p.h0 + hi;
  const int32_t flags = p.plan[p.L.frag_flags + f];
  const int32_t seg = p.plan[p.L.frag_seg + f];
  const int32_t seq = p.plan[p.L.frag_seq + f];
  const int32_t beg = p.plan[p.L.frag_begin + f];
  const int32_t end = p.plan[p.L.frag_end + f];
  const int nc = (end - beg + CH - 1) / CH;
  const int64_t ck0 = static_cast<int64_t>(beg / CH) + f;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  if (wave < 4) {
    const float* end1 = nullptr;
    const float* end2 = nullptr;
    float* out = nullptr;
    if (!E && (flags & kFragSegLast)) end1 = p.dcarry + (static_cast<size_t>(seg) * p.H + h) * MATF;
    if ((flags & kFragSeqEnd) && p.dfinal != nullptr) end2 = p.dfinal + (static_cast<size_t>(seq) * p.H + h) * MATF;
    if (E) out = p.esum + (static_cast<size_t>(r_e) * p.H + h) * MATF;
    else if (!(flags & kFragCarried) && p.dh0 != nullptr) out = p.dh0 + (static_cast<size_t>(seq) * p.H + h) * MATF;
    chain_owner<E>(p, sm, h, wave, nc, ck0, end1, end2, out);
  } else if (wave < 8) {
    chain_builder(p, sm, h, wave - 4, beg, end, nc);
  } else {
    chain_thelper(p, sm, h, wave - 8, nc, ck0);
  }
}

// ===========================================================================
// Pass 3: one chunk's gradients from R_c and D_c (their row fragments), the
// checkpoint launch's V - Kr R_c and the chain launch's dU.  Sixteen waves in
// four roles, each running its own sequence of the same seven barriers (no
// role's registers stay live in another's branch):
//   phase  waves 0-3           waves 4-7           waves 8-11          waves 12-15
//   0                                              Kr, Kc, Qr, dO       V - W and dU
//                                                  planes, G - a, beta  (value block w)
//   1      R's row fragments   D's row fragments   A' (8), P^T (9)
//          (channel block w)   (channel block w)
//   2                                              T and T^T
//   3                                                                   U^T -> U plane,
//                                                                       dX, dX^T -> dX
//                                                                       plane, dv
//   4                                              dP (8); dA, dA' (9)  rowsum(dX o (V-W))
//   5      dO R^T + dP Kc,     U D^T + dP^T Qr                          rowsum(D o R),
//          -dR R^T + dA' Kc    + dA'^T Kr -> LDS                        dbeta (12)
//   6      dq, dk, dg
// The row fragments (the only large reads) are issued after phase 0, so the
// inputs the operand build waits on go first and the fragments have four
// phases to arrive.
// ===========================================================================
constexpr int XWS = 33;   // row stride (fp32) of the phase-5 exchange tiles

struct alignas(16) GradSmem {
  bf16 kr_h[CH * NB], kr_l[CH * NB];
  bf16 kc_h[CH * NB], kc_l[CH * NB];
  bf16 qr_h[CH * NB], qr_l[CH * NB];
  bf16 do_h[CH * NB], do_l[CH * NB];
  bf16 u_h[CH * NB], u_l[CH * NB];
  bf16 dx_h[CH * NB], dx_l[CH * NB];
  // 32 x 32 matrices, columns in k-slot order: T[i][kpos(j)], T^T, P^T
  // (phases 1-3), then dP, dP^T, dA', dA'^T (phases 4-5)
  union {
    struct {
      bf16 t_h[CH * TB], t_l[CH * TB], tt_h[CH * TB], tt_l[CH * TB], pt_h[CH * TB], pt_l[CH * TB];
    } a;
    struct {
      bf16 dp_h[CH * TB], dp_l[CH * TB], dpt_h[CH * TB], dpt_l[CH * TB];
      bf16 da_h[CH * TB], da_l[CH * TB], dat_h[CH * TB], dat_l[CH * TB];
    } b;
  } m;
  // A' (phases 1-4), then the exchange (phase 5)
  union {
    struct {
      float ap[CH * AS];    // A' (strictly lower)
    } s;
    struct {
      float xw[4][CH * XWS];   // (dk_i + dk_h)[token][channel] per channel block
      float kh[4][CH];         // colsum(k o dk_h) per channel block
    } x;
  } e;
  float gl[CH * GS];                     // G - a (log2 units)
  float beta[CH];
  float red[4][CH];                      // rowsum(dX o (V - W)) per value block
  float red2[CH];                        // rowsum(dA o A')
  float rs[KD];                          // rowsum(D o R)
};

// Rows 8r + 4(l/32) + e (r, e = 0..3) of a [tokens][H][128] FP32 tensor at
// token c0, column col, for tokens below n (others dropped).
__device__ __forceinline__ void store_rows(float* base, const int H, const int n, const int col, const int lane,
                                           const f32x16& t) {
  const uint32_t rowf = static_cast<uint32_t>(H) * 128 * 4;
  const auto rs = res(base, (n - 1) * rowf + 128 * 4);
  const int voff = static_cast<int>(4 * (lane >> 5) * rowf + 4 * col);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(t[4 * r + e]), rs, voff, static_cast<int>((8 * r + e) * rowf),
                                            kWriteOnce);
}

// Row fragments of a state (channel row, all 128 values in k-slot order):
// x[8ks + j] = S[row][16ks + 4(l/32) + j'].
__device__ __forceinline__ void load_rowfrags(const float* S, const int row, const int lane, float (&x)[64]) {
  const auto rs = res(S, MATF * 4);
  const int roff = 4 * (row * VD + 4 * (lane >> 5));
#pragma unroll
  for (int ks = 0; ks < VD / 16; ++ks) {
    const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, roff, 64 * ks, 0));
    const f32x4 b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, roff, 64 * ks + 32, 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * ks + e] = a[e];
      x[8 * ks + 4 + e] = b[e];
    }
  }
}
// acc += A B over the 128 channels (or values) with A's rows from a
// token-major plane pair and B from eight k-steps of fragments in registers.
__device__ __forceinline__ f32x16 prod_frags(const bf16* ah, const bf16* al, const float (&x)[64], const int pro,
                                             f32x16 acc) {
#pragma unroll
  for (int kk = 0; kk < KD / 16; ++kk) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = x[8 * kk + j];
    bf16x8 bh, bl;
    split8<true>(v, bh, bl);
    acc = mfma3(rowfrag(ah, kk, pro), rowfrag(al, kk, pro), bh, bl, acc);
  }
  return acc;
}
// The tile rows (tokens 8r + 4(l/32) + e, k-slot order of k-steps 0, 1) of
// column c0 + l % 32 of a split token-major plane, as FP32.
__device__ __forceinline__ void plane_col(const bf16* ph, const bf16* pl, const int c0, const int trb, float (&x)[16]) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const bf16x8 h = colfrag(ph, s, c0, trb);
    const bf16x8 l = colfrag(pl, s, c0, trb);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[8 * s + j] = static_cast<float>(h[j]) + static_cast<float>(l[j]);
  }
}

// One chunk of the gradient launch: its fields, shared by the wave roles.
struct GradCtx {
  int64_t slot;
  int H, h, c0, n, lane, lh, wave, w4, pro, trb, tbo;
  uint32_t rowb;   // one token of a bf16 [T, H, 128] tensor
  const float* Rg;
  const float* Dg;
};

// Waves 0-3 (channel block w), one chunk.
__device__ __forceinline__ void grad_role_a(const BwdParams& p, GradSmem& sm, const GradCtx& x) {
  const int lane = x.lane, lh = x.lh, w = x.w4;
  float fr[64];
  __syncthreads();   // phase 0
  // ---- phases 1-4 (three barriers): R's row fragments, in flight until phase
  // 5 (issued a chunk earlier they were slower: the phase-5 re-read of R and D
  // for rowsum(D o R) then misses L2)
  load_rowfrags(x.Rg, 32 * w + (lane & 31), lane, fr);
  for (int i = 0; i < 3; ++i) __syncthreads();
  // ---- phase 5: dO R^T + dP Kc and -dR R^T + dA' Kc for channel block w
  // (one split of each R fragment serves both products)
  f32x16 vq = zero16(), vd = zero16();
#pragma unroll
  for (int kk = 0; kk < VD / 16; ++kk) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = fr[8 * kk + j];
    bf16x8 bh, bl;
    split8<true>(v, bh, bl);
    vq = mfma3(rowfrag(sm.do_h, kk, x.pro), rowfrag(sm.do_l, kk, x.pro), bh, bl, vq);
    vd = mfma3(rowfrag(sm.dx_h, kk, x.pro), rowfrag(sm.dx_l, kk, x.pro), bh, bl, vd);
  }
  mfma_result_fence(vd);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) vd[4 * r + e] *= -sm.beta[8 * r + 4 * lh + e];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const bf16x8 kch = colfrag(sm.kc_h, s, 32 * w, x.trb), kcl = colfrag(sm.kc_l, s, 32 * w, x.trb);
    vq = mfma3(smallrow(sm.m.b.dp_h, s, x.tbo), smallrow(sm.m.b.dp_l, s, x.tbo), kch, kcl, vq);
    vd = mfma3(smallrow(sm.m.b.da_h, s, x.tbo), smallrow(sm.m.b.da_l, s, x.tbo), kch, kcl, vd);
  }
  mfma_result_fence(vq);
  mfma_result_fence(vd);
  __syncthreads();
  // ---- phase 6: dq, dk, dg
  const int col = 32 * w + (lane & 31);
  float kr[16], qr[16];
  plane_col(sm.kr_h, sm.kr_l, 32 * w, x.trb, kr);
  plane_col(sm.qr_h, sm.qr_l, 32 * w, x.trb, qr);
  f32x16 dk, dG;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 8 * r + 4 * lh + e;
      const int q = 4 * r + e;
      const float xg = sm.gl[i * GS + col];
      const float ega = __builtin_amdgcn_exp2f(xg);
      const float eag = __builtin_amdgcn_exp2f(-xg);
      vq[q] *= ega;
      vd[q] *= ega;
      const float w1 = sm.e.x.xw[w][i * XWS + (lane & 31)];
      dk[q] = vd[q] + w1;
      // q = Qr e^{a-G}, k = Kr e^{a-G}
      dG[q] = qr[q] * eag * vq[q] + kr[q] * eag * (vd[q] - w1);
    }
  // the chunk-end term, on token 31 (lane half 1, register 15)
  if (lh == 1) dG[15] += sm.e.x.kh[w][lane & 31] + sm.rs[col];
  // dg_t = sum of dG over tokens t .. 31 of the chunk (dG is the gradient of
  // the prefix G in natural units: every factor above is a product)
  float gs[4], ps[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) gs[r] = (dG[4 * r] + dG[4 * r + 1]) + (dG[4 * r + 2] + dG[4 * r + 3]);
#pragma unroll
  for (int r = 0; r < 4; ++r) ps[r] = __shfl_xor(gs[r], 32);
  f32x16 dg;
  float after = 0.f;   // sum of the groups after group (r, lh)
#pragma unroll
  for (int r = 3; r >= 0; --r) {
    float run = after + (lh == 0 ? ps[r] : 0.f);
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      run += dG[4 * r + e];
      dg[4 * r + e] = run;
    }
    after += gs[r] + ps[r];
  }
  const size_t ob = (static_cast<size_t>(x.c0) * x.H + x.h) * KD;
  store_rows(p.dq + ob, x.H, x.n, col, lane, vq);
  store_rows(p.dk + ob, x.H, x.n, col, lane, dk);
  store_rows(p.dg + ob, x.H, x.n, col, lane, dg);
}

// Waves 4-7 (channel block w), one chunk.
__device__ __forceinline__ void grad_role_b(const BwdParams& p, GradSmem& sm, const GradCtx& x) {
  const int lane = x.lane, lh = x.lh, w = x.w4;
  float fr[64];
  __syncthreads();   // phase 0
  // ---- phases 1-4 (three barriers): D's row fragments, in flight until phase 5
  load_rowfrags(x.Dg, 32 * w + (lane & 31), lane, fr);
  for (int i = 0; i < 3; ++i) __syncthreads();
  // ---- phase 5: (U D^T + dP^T Qr + dA'^T Kr) e^{a-G} to the exchange, with
  // colsum(k o U D^T e^{a-G})
  const int col = 32 * w + (lane & 31);
  f32x16 Dkh = prod_frags(sm.u_h, sm.u_l, fr, x.pro, zero16());
  f32x16 Dki = zero16();
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    Dki = mfma3(smallrow(sm.m.b.dpt_h, s, x.tbo), smallrow(sm.m.b.dpt_l, s, x.tbo), colfrag(sm.qr_h, s, 32 * w, x.trb),
                colfrag(sm.qr_l, s, 32 * w, x.trb), Dki);
    Dki = mfma3(smallrow(sm.m.b.dat_h, s, x.tbo), smallrow(sm.m.b.dat_l, s, x.tbo), colfrag(sm.kr_h, s, 32 * w, x.trb),
                colfrag(sm.kr_l, s, 32 * w, x.trb), Dki);
  }
  float kr[16];
  plane_col(sm.kr_h, sm.kr_l, 32 * w, x.trb, kr);
  mfma_result_fence(Dkh);
  mfma_result_fence(Dki);
  float ks = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 8 * r + 4 * lh + e;
      const float eag = __builtin_amdgcn_exp2f(-sm.gl[i * GS + col]);
      const float vh = Dkh[4 * r + e] * eag;
      sm.e.x.xw[w][i * XWS + (lane & 31)] = vh + Dki[4 * r + e] * eag;
      ks = fmaf(kr[4 * r + e] * eag, vh, ks);   // k = Kr e^{a-G}
    }
  ks += __shfl_xor(ks, 32);
  if (lh == 0) sm.e.x.kh[w][lane & 31] = ks;
  __syncthreads();
}

// Waves 8-11, one chunk: the operands and the copies of T (phase 0), A' and
// P^T (phase 1), dP and dA (phase 4); in phase 5 the next chunk's inputs are
// fetched into `in` (held across its barriers to its phase 0).
struct GradPre {
  ChunkIn in;
  u32x4 t;      // 16 bytes of the chunk's cached T
  float beta;   // wave 8, lanes below 32
};

__device__ __forceinline__ void grad_prefetch_c(const BwdParams& p, const GradCtx& x, GradPre& pre) {
  fetch_chunk(p, x.h, x.c0, x.n, x.w4, x.lane, pre.in);
  const uint16_t* tc = p.tcache + (static_cast<size_t>(x.slot) * x.H + x.h) * (kChunkCacheBytes / 2);
  const int ci = x.lane + 64 * x.w4;
  pre.t = *reinterpret_cast<const u32x4*>(tc + (ci >> 7) * (CH * CH) + ((ci >> 2) & 31) * CH + 8 * (ci & 3));
  pre.beta = 0.f;
  if (x.wave == 8 && x.lane < CH) {
    const auto rb = res(p.beta + static_cast<size_t>(x.c0) * x.H + x.h, (x.n - 1) * x.H * 2 + 2);
    pre.beta = __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(
                                   __builtin_amdgcn_raw_buffer_load_b16(rb, x.lane * x.H * 2, 0, 0)))
                               << 16);
  }
}

__device__ __forceinline__ void grad_role_c(const BwdParams& p, GradSmem& sm, const GradCtx& x, const GradCtx& xn,
                                            GradPre& pre) {
  const int lane = x.lane, lh = x.lh, wave = x.wave, w = x.w4;
  // ---- phase 0: Kr, Kc, Qr, dO planes and G - a; beta; T and T^T (a cache
  // row holds column j = kpos(p) at position p)
  {
    if (wave == 8 && lane < CH) sm.beta[lane] = pre.beta;
    float a[8], gc[8];
    build_chunk(pre.in, Planes{sm.kr_h, sm.kr_l, sm.kc_h, sm.kc_l, sm.qr_h, sm.qr_l, sm.do_h, sm.do_l}, sm.gl, w,
                lane, a, gc);
    const int ci = lane + 64 * w;
    const int which = ci >> 7;
    const int ti = (ci >> 2) & 31;
    const int tq = ci & 3;
    const u32x4 tv = pre.t;
    bf16* tn = which ? sm.m.a.t_l : sm.m.a.t_h;
    bf16* tt = which ? sm.m.a.tt_l : sm.m.a.tt_h;
    *reinterpret_cast<u32x4*>(tn + ti * TB + 8 * tq) = tv;
    const int pi = kpos(ti);
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      tt[kpos(8 * tq + 2 * w2) * TB + pi] = __builtin_bit_cast(bf16, static_cast<uint16_t>(tv[w2] & 0xffffu));
      tt[kpos(8 * tq + 2 * w2 + 1) * TB + pi] = __builtin_bit_cast(bf16, static_cast<uint16_t>(tv[w2] >> 16));
    }
  }
  __syncthreads();
  // ---- phase 1: A' = Kr Kc^T (strictly lower, FP32) (wave 8) or P = Qr Kc^T
  // -> P^T (wave 9)
  if (wave == 8 || wave == 9) {
    f32x16 acc = zero16();
    const bf16* xh = wave == 8 ? sm.kr_h : sm.qr_h;
    const bf16* xl = wave == 8 ? sm.kr_l : sm.qr_l;
#pragma unroll
    for (int kk = 0; kk < KD / 16; ++kk)
      acc = mfma3(rowfrag(xh, kk, x.pro), rowfrag(xl, kk, x.pro), rowfrag(sm.kc_h, kk, x.pro),
                  rowfrag(sm.kc_l, kk, x.pro), acc);
    mfma_result_fence(acc);
    const int j = lane & 31;
    if (wave == 8) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 8 * r + 4 * lh + e;
          sm.e.s.ap[i * AS + j] = j < i ? acc[4 * r + e] : 0.f;
        }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j > 8 * r + 4 * lh + e) acc[4 * r + e] = 0.f;
      store_t(acc, sm.m.a.pt_h, sm.m.a.pt_l, lane);
    }
  }
  __syncthreads();
  __syncthreads();   // phase 3
  // ---- phase 4: dP = lower_incl(dO U^T) (wave 8);  dA^T = strict_upper(-U dX^T)
  // (rows j, columns i: token i's sums over j stay in its lane and its
  // partner's), rowsum(dA o A'), dA' = diag(beta) dA (wave 9)
  if (wave == 8 || wave == 9) {
    f32x16 acc = zero16();
    const bf16* ah = wave == 8 ? sm.do_h : sm.u_h;
    const bf16* al = wave == 8 ? sm.do_l : sm.u_l;
    const bf16* bh = wave == 8 ? sm.u_h : sm.dx_h;
    const bf16* bl = wave == 8 ? sm.u_l : sm.dx_l;
#pragma unroll
    for (int kk = 0; kk < VD / 16; ++kk)
      acc = mfma3(rowfrag(ah, kk, x.pro), rowfrag(al, kk, x.pro), rowfrag(bh, kk, x.pro), rowfrag(bl, kk, x.pro), acc);
    mfma_result_fence(acc);
    const int cl = lane & 31;
    if (wave == 8) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (cl > 8 * r + 4 * lh + e) acc[4 * r + e] = 0.f;
      store_n(acc, sm.m.b.dp_h, sm.m.b.dp_l, lane);
      store_t(acc, sm.m.b.dpt_h, sm.m.b.dpt_l, lane);
    } else {
      // acc[j][i] = (U dX^T)[j][i] = (dX U^T)[i][j]; this lane's column is i
      const int i = cl;
      const float bi = sm.beta[i];
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 8 * r + 4 * lh + e;
          const float da = j < i ? -acc[4 * r + e] : 0.f;
          part = fmaf(da, sm.e.s.ap[i * AS + j], part);
          acc[4 * r + e] = bi * da;
        }
      part += __shfl_xor(part, 32);
      if (lh == 0) sm.red2[i] = part;
      // acc holds dA'^T [j][i]: its rows to dat, its transpose to da
      store_n(acc, sm.m.b.dat_h, sm.m.b.dat_l, lane);
      store_t(acc, sm.m.b.da_h, sm.m.b.da_l, lane);
    }
  }
  __syncthreads();
  // ---- phase 5: the next chunk's inputs (this chunk's again after the last
  // one: an unconditional fetch lets the old values die here)
  grad_prefetch_c(p, xn, pre);
  __syncthreads();   // phase 5
}

// V - W and dU of a chunk at the tile's rows (token 8r + 4lh + e, value
// 32w + l % 32), and V - W transposed (value 32w + 8r + 4lh + e, token l % 32).
struct GradPreD {
  f32x16 rv, du, rvt;
};

__device__ __forceinline__ void grad_prefetch_d(const BwdParams& p, const GradCtx& x, GradPreD& pre) {
  const int lane = x.lane, lh = x.lh, w = x.w4;
  const int col = 32 * w + (lane & 31);
  const auto rs1 = res(p.rvbuf + (static_cast<size_t>(x.slot) * x.H + x.h) * CH * VD, CH * VD * 4);
  const auto rs2 = res(p.dubuf + (static_cast<size_t>(x.slot) * x.H + x.h) * CH * VD, CH * VD * 4);
  const int voff = 4 * (4 * lh * VD + col);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pre.rv[4 * r + e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs1, voff, 4 * (8 * r + e) * VD, 0));
      pre.du[4 * r + e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs2, voff, 4 * (8 * r + e) * VD, 0));
    }
  const int toff = 4 * ((lane & 31) * VD + 32 * w + 4 * lh);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const f32x4 v4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs1, toff, 32 * r, 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) pre.rvt[4 * r + e] = v4[e];
  }
}

// Waves 12-15 (value block w), one chunk: U^T, dX, dX^T and dv (phase 3),
// rowsum(dX o (V - W)) and rowsum(D o R) (phase 4), dbeta (phase 5); in
// phase 6 the next chunk's V - W and dU are fetched into `pre`.
__device__ __forceinline__ void grad_role_d(const BwdParams& p, GradSmem& sm, const GradCtx& x, const GradCtx& xn,
                                            GradPreD& pre) {
  const int lane = x.lane, lh = x.lh, w = x.w4;
  const int col = 32 * w + (lane & 31);
  const f32x16 rv = pre.rv, du = pre.du, rvt = pre.rvt;
  __syncthreads();
  __syncthreads();   // phase 1
  // ---- phase 3: X = diag(beta)(V - W), U^T = X^T T^T -> U plane;
  // dX = T^T dU, dX^T = dU^T T -> dX plane;  dv = diag(beta) dX
  {
    f32x16 X;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) X[4 * r + e] = sm.beta[8 * r + 4 * lh + e] * rv[4 * r + e];
    bf16x8 xh[2], xl[2];
    tile_kslots_split(X, xh, xl);
    f32x16 UT = zero16();
#pragma unroll
    for (int s = 0; s < 2; ++s)
      UT = mfma3(xh[s], xl[s], smallrow(sm.m.a.t_h, s, x.tbo), smallrow(sm.m.a.t_l, s, x.tbo), UT);
    mfma_result_fence(UT);
    store_plane_t(UT, sm.u_h, sm.u_l, 32 * w, lane);
  }
  f32x16 dXT = zero16();
  {
    bf16x8 uh[2], ul[2];
    tile_kslots_split(du, uh, ul);
    f32x16 dX = zero16();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      dX = mfma3(smallrow(sm.m.a.tt_h, s, x.tbo), smallrow(sm.m.a.tt_l, s, x.tbo), uh[s], ul[s], dX);
      dXT = mfma3(uh[s], ul[s], smallrow(sm.m.a.tt_h, s, x.tbo), smallrow(sm.m.a.tt_l, s, x.tbo), dXT);
    }
    mfma_result_fence(dX);
    mfma_result_fence(dXT);
    store_plane_t(dXT, sm.dx_h, sm.dx_l, 32 * w, lane);
    f32x16 dv;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) dv[4 * r + e] = sm.beta[8 * r + 4 * lh + e] * dX[4 * r + e];
    store_rows(p.dv + (static_cast<size_t>(x.c0) * x.H + x.h) * VD, x.H, x.n, col, lane, dv);
  }
  __syncthreads();
  // ---- phase 4: rowsum(dX o (V - W)) over value block w, from the
  // transposed tiles (token l % 32: the lane's 16 values and its partner's)
  {
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) part = fmaf(dXT[q], rvt[q], part);
    part += __shfl_xor(part, 32);
    if (lh == 0) sm.red[w][lane & 31] = part;
  }
  // rowsum(D o R) for the channels of block w (read in phase 6; row
  // 32w + l % 32, the lane's half of the values, in two passes of 32): R and
  // D were fetched in phase 1 by waves 0-7, so these reads find them in L2
  {
    const int row = 32 * w + (lane & 31);
    const auto rr = res(x.Rg, MATF * 4);
    const auto rd = res(x.Dg, MATF * 4);
    const int roff = 4 * (row * VD + 4 * lh);
    float s = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4 a[8], b[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int o = 256 * half + 64 * q;
        a[2 * q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, roff, o, 0));
        a[2 * q + 1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, roff, o + 32, 0));
        b[2 * q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, roff, o, 0));
        b[2 * q + 1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, roff, o + 32, 0));
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(a[q][e], b[q][e], s);
    }
    s += __shfl_xor(s, 32);
    if (lh == 0) sm.rs[row] = s;
  }
  __syncthreads();
  // ---- phase 5: dbeta
  if (x.wave == 12 && lane < CH) {
    const float db = sm.red2[lane] + ((sm.red[0][lane] + sm.red[1][lane]) + (sm.red[2][lane] + sm.red[3][lane]));
    const auto rb = res(p.dbeta + static_cast<size_t>(x.c0) * x.H + x.h, (x.n - 1) * x.H * 4 + 4);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(db), rb, lane * x.H * 4, 0, 0);
  }
  __syncthreads();
  // ---- phase 6: the next chunk's V - W and dU (see grad_role_c)
  grad_prefetch_d(p, xn, pre);
}

// The next chunk item at or after `it` (stepping by the grid) that is on the
// chunked path: item = slot * hn + head offset; `total` when none is left.
__device__ __forceinline__ int grad_next(const BwdParams& p, int it, const int total) {
  for (; it < total; it += static_cast<int>(gridDim.x)) {
    const int slot = it / p.hn;
    const int f = p.smap[slot];
    if (f >= 0 && p.iflag[static_cast<size_t>(f) * p.hn + (it - slot * p.hn)] == 0) return it;
  }
  return total;
}

__device__ __forceinline__ void grad_ctx(const BwdParams& p, const int it, GradCtx& x) {
  const int slot = it / p.hn;
  const int f = p.smap[slot];
  x.slot = slot;
  x.h = p.h0 + (it - slot * p.hn);
  const int32_t beg = p.plan[p.L.frag_begin + f];
  const int32_t end = p.plan[p.L.frag_end + f];
  x.c0 = beg + CH * (slot - (beg / CH + f));
  x.n = min(CH, end - x.c0);
  x.Rg = p.ck32 + (static_cast<size_t>(slot) * x.H + x.h) * MATF;
  x.Dg = p.dcot + (static_cast<size_t>(slot) * x.H + x.h) * MATF;
}

// Persistent: each workgroup (one per CU) walks the items it + k * grid; the
// operand waves and the V - W / dU waves fetch the next item's inputs during
// the current one's last phases.  Every wave walks the same items and takes
// the same six barriers per item, the last of which keeps the next item's
// phase-0 writes behind this item's phase-6 reads.
// The lane's fields of an item's context, from a value the compiler cannot
// see through: so the per-lane LDS addresses of every phase are recomputed in
// each item instead of being hoisted out of the item loop and kept live
// (which spilled).
__device__ __forceinline__ void grad_lane(GradCtx& x) {
  const int tid = opaque(static_cast<int>(threadIdx.x));
  x.lane = tid & 63;
  x.lh = x.lane >> 5;
  x.pro = (x.lane & 31) * NB + 4 * x.lh;
  x.trb = tr_base(x.lane);
  x.tbo = (x.lane & 31) * TB + 8 * x.lh;
}

// Persistent: each workgroup (one per CU) walks the items it + k * grid; the
// operand waves and the V - W / dU waves fetch the next item's inputs during
// the current one's last phases.  Every wave walks the same items and takes
// the same six barriers per item, the last of which keeps the next item's
// phase-0 writes behind this item's phase-6 reads.
__device__ __forceinline__ void grad_chunks(const BwdParams& p) {
  __shared__ GradSmem sm;
  const int total = p.nslots * p.hn;
  GradCtx x, xn;
  x.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  x.w4 = x.wave & 3;
  x.H = p.H;
  x.rowb = static_cast<uint32_t>(x.H) * 128 * 2;
  grad_lane(x);
  xn = x;
  int it = grad_next(p, static_cast<int>(blockIdx.x), total);
  if (it >= total) return;
  grad_ctx(p, it, x);
  if (x.wave < 8) {
    while (true) {
      grad_lane(x);
      if (x.wave < 4) grad_role_a(p, sm, x);
      else grad_role_b(p, sm, x);
      __syncthreads();
      it = grad_next(p, it + static_cast<int>(gridDim.x), total);
      if (it >= total) break;
      grad_ctx(p, it, x);
    }
  } else if (x.wave < 12) {
    GradPre pre;
    grad_prefetch_c(p, x, pre);
    while (true) {
      const int nx = grad_next(p, it + static_cast<int>(gridDim.x), total);
      grad_ctx(p, nx < total ? nx : it, xn);
      grad_lane(x);
      grad_lane(xn);
      grad_role_c(p, sm, x, xn, pre);
      __syncthreads();
      if (nx >= total) break;
      it = nx;
      x = xn;
    }
  } else {
    GradPreD pre;
    grad_prefetch_d(p, x, pre);
    while (true) {
      const int nx = grad_next(p, it + static_cast<int>(gridDim.x), total);
      grad_ctx(p, nx < total ? nx : it, xn);
      grad_lane(x);
      grad_lane(xn);
      grad_role_d(p, sm, x, xn, pre);
      __syncthreads();
      if (nx >= total) break;
      it = nx;
      x = xn;
    }
  }
}

}  // namespace

// E_r per (piece r, head): the first fragment of a segment that continues a
// sequence, reversed from its dfinal (at a sequence end) or zero with the
// cotangent only; zero for a segment that starts its sequence.  Fragments on
// the token-by-token path are left to kda_backward_summary_kernel.
__global__ void __launch_bounds__(kChainThreads, 1) kda_bwd_chain_e_kernel(BwdParams p) {
  const int r = blockIdx.x / p.hn;
  const int hi = blockIdx.x % p.hn;
  const int h = p.h0 + hi;
  if (p.plan[p.L.seg_carry_in + r] == 0) {
    f32x4* dst = reinterpret_cast<f32x4*>(p.esum + (static_cast<size_t>(r) * p.H + h) * MATF);
    for (int i = threadIdx.x; i < static_cast<int>(MATF / 4); i += kChainThreads) dst[i] = zero4();
    return;
  }
  const int f = p.plan[p.L.seg_frag_ptr + r];
  if (p.iflag[static_cast<size_t>(f) * p.hn + hi] != 0) return;
  chain_run<true>(p, f, hi, r);
}

// Every (fragment, head) on the chunked path, in the plan's launch order:
// the cotangent from D_r (at a segment end) plus dfinal (at a sequence end)
// back to the fragment's start, storing every chunk's D_c; dh0 where the
// fragment starts its sequence.
__global__ void __launch_bounds__(kChainThreads, 1) kda_bwd_chain_kernel(BwdParams p) {
  const int rank = blockIdx.x / p.hn;
  const int hi = blockIdx.x % p.hn;
  const int f = p.plan[p.L.frag_order + rank];
  if (p.iflag[static_cast<size_t>(f) * p.hn + hi] != 0) return;
  chain_run<false>(p, f, hi, 0);
}

// Every chunk slot and head: that chunk's gradients (slots of no fragment,
// and fragments on the token-by-token path, are skipped); a persistent grid
// of at most one workgroup per CU.
__global__ void __launch_bounds__(kGradThreads, 1) kda_bwd_grad_kernel(BwdParams p) { grad_chunks(p); }

}  // namespace kda
