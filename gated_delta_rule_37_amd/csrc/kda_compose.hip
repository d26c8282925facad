// HIP kernels (gfx950) of the ordered FP32 scan over segment summaries.
//
// Sources: inclusionAI/cuLA pull request #136 "feat(kda): add cuDNN
// concatenated-summary Kimi CP" (Summary: each rank's preceding transition
// and update compose affinely, in FP32, into the state a rank starts from;
// Sequence Diagram: the backward gathers the following ranks' summaries).
//
// A segment maps the state at its start to the state at its end affinely,
// S_end = A_r S_start + B_r.  The carry into segment r+1 is therefore
// C_{r+1} = A_r C_r + B_r from C_0 = 0 (or a sequence's initial state),
// one 128 x 128 by 128 x 128 FP32 product per step, in segment order.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_internal.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int KD = 128;   // key dimension
constexpr int VD = 128;   // value dimension
// Buffer resource word 3 for gfx9 raw (unswizzled, 32-bit) buffer access.
constexpr int kBufDword3 = 0x00020000;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte LDS accesses through the native vector type (HIP's float4 struct
// is split into pairs of 8-byte accesses)
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, const f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0.f;
  return z;
}

}  // namespace

// Ordered scan C_0 = 0, C_{r+1} = A_r C_r + B_r on FP32 matrix cores, for one
// head and one block of 16 state columns (the columns of C never mix, so each
// block scans on its own).  Wave w computes rows [16w, 16w + 16) as one
// 16 x 16 tile (v_mfma_f32_16x16x4_f32; lane l, register i holds row
// 16w + 4(l/16) + i, column l%16).  The k slots are permuted so that each
// operand is contiguous: MFMA s = 4q + e, k slot j = l/16 stands for
// k = 32j + 4(q xor (j & 1)) + e, so a lane's A operand over the whole
// product is A_r[16w + l%16][32j .. 32j + 31] and its B operand
// C_r[32j .. 32j + 31][col], in 16-byte blocks.
//
// Moving A_r (64 KB per step and workgroup) costs more than the products.
// Each wave loads only the part of A_r its own tile multiplies (its 16 rows,
// two whole rows per wave instruction), kComposeRing steps ahead into a
// ring of register buffers (the step loop is unrolled over the ring, so no
// buffer is copied), and turns it into the operand layout through an LDS
// region of its own with padded rows.  No other wave touches that region,
// so the wave stores step r+1's A and reads its operand back in the middle
// of step r's products, off the scan's chain: the chain per step is the
// carry's transposed store, one barrier, the carry's operand reads and the
// products.  The carry tile alternates by step parity.  The column blocks of
// a head are numbered onto one XCD (workgroups are dealt to the eight XCDs
// in turn), where they share its L2 copy of A_r.
//
// Global accesses go through buffer resources built in scalar registers
// from each step's matrices, with lane offsets fixed for the whole scan: no
// per-lane address is computed into a register that a load in flight still
// owns (the compiler would make such a write wait for that load).
// Row strides of the LDS tiles.  A stride of 34 16-byte units (34 = 2 mod
// 16) with the k-block order of kblk below makes every 16-byte access of the
// scan conflict-free: the A stores, the operand reads and the transposed
// carry stores.  (A 16-byte LDS access is served in four 16-lane passes:
// lanes {0-3, 12-15, 20-27}, {4-11, 16-19, 28-31} and the same + 32; the
// 16 lanes of a pass must touch 16 different 4-bank units.)
constexpr int kAtStride = KD + 8;   // floats per row of a wave's A_r region
constexpr int kCtStride = KD + 8;   // floats per column of the transposed carry tile
constexpr int kComposeRing = 3;     // operand ring: A_r is loaded kComposeRing - 1 steps before its store to LDS
constexpr int kComposeWaves = kComposeThreads / 64;
constexpr int kAPieces = KD * KD / 4 / kComposeThreads;   // 16-byte pieces of A_r per lane
constexpr int kARegion = 16 * kAtStride;                 // floats per wave's A_r region
constexpr int kBtStride = kComposeColumns + 4;           // floats per row of a wave's B_r rows
static_assert(kComposeWaves * 16 == KD, "compose: one 16-row tile per wave");
static_assert(kAPieces == 8, "compose: a wave's 16 rows (or columns) of A_r are 8 pieces per lane");
static_assert(KD * 16 + 4 * 16 <= kARegion, "compose: the reverse layout fits a wave's region");

struct alignas(16) ComposeSmem {
  float at[kComposeWaves][kARegion];            // each wave's part of A_r
  float ct[2][kComposeColumns * kCtStride];     // C_r[:, block] transposed, by step parity
  float bt[kComposeWaves][16 * kBtStride];       // each wave's 16 rows of B_r[:, block]
};

// The same scan serves four uses (MODE):
//  kScanCompose  the forward's C_0 = 0, C_{r+1} = A_r C_r + B_r over the
//                segments (or, for the backward, over the pieces);
//  kScanReverse  the backward's D_{S-1} = 0, D_{r-1} = A_r^T D_r + E_r: step s
//                stands for segment S-1-s, and a wave's operand is the block
//                of 16 columns of A_r (its rows of A_r^T);
//  kScanFold     per segment, its pieces' summaries folded into the
//                segment's own: X <- A'_i X (+ B'_i) from X = [I | 0] over
//                the pieces in order, one chain per (segment, head) and 16
//                column blocks (8 of A_r, 8 of B_r); only the end is written;
//  kScanPieces   per segment, every piece's carry-in: X = C_r (zero for a
//                segment that does not continue a sequence), written at each
//                piece, then X <- A'_i X + B'_i.
// A transition that is structurally zero (its flag clear) is skipped.
enum ScanMode { kScanCompose = 0, kScanReverse = 1, kScanFold = 2, kScanPieces = 3 };

template <int MODE>
__device__ __forceinline__ void compose_scan(const ComposeParams& p, ComposeSmem& sm) {
  constexpr bool REV = MODE == kScanReverse;
  constexpr bool CHAINS = MODE == kScanFold || MODE == kScanPieces;
  constexpr int NCB = MODE == kScanFold ? 2 * kComposeColumnBlocks : kComposeColumnBlocks;
  const int H = p.H;
  const int xcd = blockIdx.x % 8;
  const int kq = blockIdx.x / 8;
  const int cb = kq % NCB;
  const int unit = xcd + 8 * (kq / NCB);   // (chain, head), its column blocks on one XCD
  if (unit >= (CHAINS ? p.chains : 1) * p.hn) return;
  const int chain = CHAINS ? unit / p.hn : 0;
  const int h = p.h0 + unit % p.hn;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lc = lane & 15;    // column within the block (and row within the tile for A)
  const int lj = lane >> 4;    // k slot
  // MFMA 4q + e, k slot lj, stands for k = kblk(q) + e: the slots of lanes
  // 16-31 and 48-63 take their 4-k blocks in another order than those of
  // lanes 0-15 and 32-47 (any order serves, as long as A and C agree)
  auto kblk = [&](const int q) { return 32 * lj + 4 * (q ^ (lj & 1)); };
  const bool bpart = MODE == kScanFold && cb >= kComposeColumnBlocks;   // a column block of B_r
  const int col = kComposeColumns * (bpart ? cb - kComposeColumnBlocks : cb) + lc;
  const int row0 = 16 * wave;
  float* const region = sm.at[wave];

  // the chain: steps over the segments, or over one segment's pieces
  int base = 0, S = p.S;
  if (CHAINS) {
    base = p.plan[p.L.useg_piece_ptr + chain];
    const int len = p.plan[p.L.useg_piece_ptr + chain + 1] - base;
    S = MODE == kScanFold ? len + 1 : len;   // a fold applies every piece, then writes
  }
  auto seg_of = [&](const int r) { return REV ? S - 1 - r : base + r; };
  // this wave's part of A_r, coalesced.  Forward: piece u is row
  // 16w + 2u + lane/32, floats 4(lane % 32) .. (two whole rows per wave
  // instruction).  Reverse: piece u is row 16u + lane/4, floats
  // 16w + 4(lane % 4) .. (sixteen 64-byte row pieces per instruction).
  const int a_off = REV ? (lane >> 2) * KD + row0 + 4 * (lane & 3) : (row0 + (lane >> 5)) * KD + 4 * (lane & 31);
  constexpr int a_step = REV ? 16 * KD : 2 * KD;
  // B_r: the wave's 16 rows of the column block, one 16-byte piece per lane
  // (row 16w + lane/4, columns 4(lane % 4) ..), staged through the wave's
  // own rows of bt like A_r (a fold's column block of A_r loads it too and
  // adds zero instead)
  const int b_off = (row0 + (lane >> 2)) * VD + kComposeColumns * (bpart ? cb - kComposeColumnBlocks : cb) + 4 * (lane & 3);
  auto load_a = [&](const int r, f32x4 (&a)[kAPieces + 1]) {
    const size_t m = static_cast<size_t>(seg_of(r)) * H + h;
    const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.transitions + m * KD * KD), 0,
                                                      KD * KD * 4, kBufDword3);
    const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.updates + m * KD * VD), 0,
                                                      KD * VD * 4, kBufDword3);
#pragma unroll
    for (int u = 0; u < kAPieces; ++u)
      a[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, 4 * (a_off + u * a_step), 0, 0));
    a[kAPieces] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, 4 * b_off, 0, 0));
  };
  // into the wave's region.  Forward: row-major 16 x kAtStride.  Reverse:
  // k-major, 16 floats per k, with a 16-float skew per 32 k so that the
  // lanes' scalar reads of one k slot fall into distinct banks.
  const int st_off = REV ? (lane >> 2) * 16 + 4 * (lane & 3) : (lane >> 5) * kAtStride + 4 * (lane & 31);
  auto store_a = [&](const f32x4 (&a)[kAPieces + 1]) {
#pragma unroll
    for (int u = 0; u < kAPieces; ++u) {
      const int o = REV ? u * 256 + (u >> 1) * 16 : u * 2 * kAtStride;
      st4(&region[st_off + o], a[u]);
    }
    st4(&sm.bt[wave][(lane >> 2) * kBtStride + 4 * (lane & 3)], a[kAPieces]);
  };
  auto read_b = [&]() {
    f32x4 bv;
#pragma unroll
    for (int i = 0; i < 4; ++i) bv[i] = sm.bt[wave][(4 * lj + i) * kBtStride + lc];
    return bv;
  };
  auto read_a = [&](f32x4 (&aop)[8], const int q0, const int q1) {
#pragma unroll
    for (int q = q0; q < q1; ++q) {
      if (REV) {
#pragma unroll
        for (int e = 0; e < 4; ++e) aop[q][e] = region[(kblk(q) + e) * 16 + 16 * lj + lc];
      } else {
        aop[q] = ld4(&region[lc * kAtStride + kblk(q)]);
      }
    }
  };
  // this lane's four entries of a carry, as byte offsets in its matrix
  const int c_off = 4 * ((row0 + 4 * lj) * VD + col);
  // where step r's value goes: the carry of that segment or piece, or for a
  // fold (last step only) the segment's transition or update
  auto dest = [&](const int r) -> float* {
    if (MODE == kScanFold) return (bpart ? p.out_b : p.out_a) + (static_cast<size_t>(chain) * H + h) * KD * VD;
    return p.carry + (static_cast<size_t>(seg_of(r)) * H + h) * KD * VD;
  };

  // transition flags of steps [lbase, lbase + 64) as a wave-wide bit mask.
  // (A plan read inside the loop would be a vector load whose wait also
  // drains the prefetches and the carry stores in flight.)
  uint64_t lmask = 0;
  int lbase = -64;
  auto live_at = [&](const int r) {
    if (r - lbase >= 64) {
      lbase = r & ~63;
      const int idx = lbase + lane;
      // forward: A_idx is applied for idx < S-1; reverse: A_{S-1-idx}^T for
      // 1 <= idx < S-1 (D_{S-1} is zero, so A_{S-1} is never read)
      const bool f = idx < S - 1 && (!REV || idx >= 1) && p.plan[p.live_off + seg_of(idx)] != 0;
      lmask = __builtin_amdgcn_ballot_w64(f);
    }
    return ((lmask >> (r - lbase)) & 1ull) != 0;
  };

  // ring slot t % kComposeRing holds step t's A_r and B_r pieces from the
  // load until their store to LDS during step t-1 (every loaded register
  // has that one consumer), and its flag until its use.  aop and bcur hold
  // the operands of the step whose products run next: each half of aop is
  // read back for step t+1 as soon as step t's products have consumed it.
  //
  // Every step issues the same global accesses whatever its flags (four
  // carry stores, then B and A of step t + kComposeRing, clamped to the
  // last step), so the compiler's wait counts are exact and each wait lets
  // the later steps' loads stay in flight; with loads under conditions it
  // has to wait for all but the newest few.
  f32x4 a_ring[kComposeRing][kAPieces + 1];
  f32x4 aop[8];
  f32x4 bcur;
  bool lv[kComposeRing];
  f32x4 cur = zero4();
  if (MODE == kScanFold && !bpart) {
#pragma unroll
    for (int i = 0; i < 4; ++i) cur[i] = row0 + 4 * lj + i == col ? 1.f : 0.f;   // the identity
  } else if (MODE == kScanPieces && p.plan[p.L.useg_carry_in + chain] != 0) {
    const float* csrc = p.init + (static_cast<size_t>(chain) * H + h) * KD * VD;
#pragma unroll
    for (int i = 0; i < 4; ++i) cur[i] = csrc[(row0 + 4 * lj + i) * VD + col];
  }
  if (S < 2) {   // no step applies a transition: the start is the one value
    if (S == 1) {
      float* cdst = dest(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) cdst[(row0 + 4 * lj + i) * VD + col] = cur[i];
    }
    return;
  }
#pragma unroll
  for (int d = 0; d < kComposeRing; ++d) {
    lv[d] = live_at(d);
    load_a(d < S - 1 ? d : S - 2, a_ring[d]);
  }
  store_a(a_ring[0]);
  read_a(aop, 0, 8);
  bcur = read_b();
  for (int r0 = 0;; r0 += kComposeRing) {
#pragma unroll
    for (int ph = 0; ph < kComposeRing; ++ph) {
      const int r = r0 + ph;            // r % kComposeRing == ph
      {
        // a fold writes its one destination at every step; the last write,
        // step S-1's, stays
        const auto rc = __builtin_amdgcn_make_buffer_rsrc(dest(r), 0, KD * VD * 4, kBufDword3);
#pragma unroll
        for (int i = 0; i < 4; ++i) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(cur[i]), rc, c_off + 4 * i * VD, 0, 0);
      }
      if (r == S - 1) return;
      const int buf = r & 1;
      const int p1 = (ph + 1) % kComposeRing;
      const bool live = lv[ph];
      // step r + kComposeRing's operands into the slot whose A and B went to
      // LDS during step r-1: issued first, they have the whole step to land
      {
        const int rn = r + kComposeRing;
        const int rc = rn < S - 1 ? rn : S - 2;
        lv[ph] = live_at(rn);
        load_a(rc, a_ring[ph]);
      }
      // the carry, transposed into LDS: column lc, rows row0 + 4lj + 0..3
      st4(&sm.ct[buf][lc * kCtStride + row0 + 4 * lj], cur);
      // the carry reached LDS; the barrier also ends step r-1's reads of the
      // other parity's tile, which step r+1 refills
      __syncthreads();
      f32x4 bop[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) bop[q] = ld4(&sm.ct[buf][lc * kCtStride + kblk(q)]);
      // four independent accumulator chains (k slot e of every MFMA group),
      // summed at the end: the MFMAs issue back to back instead of each
      // waiting for the previous one's result.  Step r+1's A goes through the
      // wave's region between the two halves of the products.
      // (a fold's column block of A_r adds no B)
      const f32x4 b0 = MODE == kScanFold && !bpart ? zero4() : bcur;
      f32x4 acc[4] = {b0, zero4(), zero4(), zero4()};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop[q][e], bop[q][e], acc[e], 0, 0, 0);
      store_a(a_ring[p1]);
      read_a(aop, 0, 4);
#pragma unroll
      for (int q = 4; q < 8; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop[q][e], bop[q][e], acc[e], 0, 0, 0);
      read_a(aop, 4, 8);
      bcur = read_b();
      // the products run whatever the flag (the loop has no branch for the
      // compiler to merge wait counts over); a transition that is
      // structurally zero is dropped here, whatever its buffer holds
      const f32x4 prod = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      f32x4 nxt;
#pragma unroll
      for (int i = 0; i < 4; ++i) nxt[i] = live ? prod[i] : b0[i];
      cur = nxt;
    }
  }
}

__global__ void __launch_bounds__(kComposeThreads, 1) kda_compose_kernel(ComposeParams p) {
  __shared__ ComposeSmem sm;
  compose_scan<kScanCompose>(p, sm);
}

__global__ void __launch_bounds__(kComposeThreads, 1) kda_compose_reverse_kernel(ComposeParams p) {
  __shared__ ComposeSmem sm;
  compose_scan<kScanReverse>(p, sm);
}

__global__ void __launch_bounds__(kComposeThreads, 1) kda_fold_pieces_kernel(ComposeParams p) {
  __shared__ ComposeSmem sm;
  compose_scan<kScanFold>(p, sm);
}

__global__ void __launch_bounds__(kComposeThreads, 1) kda_piece_carry_kernel(ComposeParams p) {
  __shared__ ComposeSmem sm;
  compose_scan<kScanPieces>(p, sm);
}

}  // namespace kda
