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
// block scans on its own).  Sixteen waves: wave w computes the partial
// product of row tile t = w % 8 (rows [16t, 16t + 16)) over the k half
// h = w / 8 (k in [64h, 64h + 64)), one 16 x 16 tile (v_mfma_f32_16x16x4_f32;
// lane l, register i holds row 16t + 4(l/16) + i, column l%16), 16 MFMAs a
// step.  Two waves per row tile give each SIMD four waves, whose LDS
// traffic, barrier waits and chain tails overlap each other's products.
// The k slots are permuted: MFMA 4q + e, k slot j = l/16 stands for
// k = 64h + 16j + 4(q xor (j & 1)) + e, so each lane's operands are 16-byte
// blocks.
//
// A step's carry is held as the two waves' partial sums: each wave stores
// its partial, transposed, into its half's copy of the carry tile; after the
// step's one barrier the waves read the sum of both copies as their B
// operand, and both waves of a row tile store the full carry (the same
// values) to global memory.  A transition that is structurally zero is
// dropped by a select (the k-half-0 wave keeps B_r, the other zero).
//
// Each wave loads only the block of A_r its products use (its 16 rows by
// its 64 k; the reverse scan's wave the block of A_r^T, i.e. 64 rows by 16
// columns of A_r), kComposeRing steps ahead into a ring of register
// buffers (the step loop is unrolled over the ring, so no buffer is
// copied), and turns it into the operand layout through an LDS region no
// other wave touches: it stores step r+1's block and reads it back in the
// middle of step r's products, off the scan's chain.  The forward region
// has 64-float rows whose 16-byte slots are XOR-swizzled by the row, which
// with the k order above makes its stores and operand reads conflict-free
// (a 16-byte LDS access is served in four 16-lane passes: lanes
// {0-3, 12-15, 20-27}, {4-11, 16-19, 28-31} and the same + 32; the 16 lanes
// of a pass must touch 16 different 4-bank units).  Global accesses go
// through buffer resources built in scalar registers with fixed lane
// offsets, and every step issues the same accesses whatever its flags, so
// the compiler's wait counts are exact.  The column blocks of a head are
// numbered onto one XCD (workgroups are dealt to the eight XCDs in turn),
// where they share its L2 copy of A_r.
constexpr int kCtStride = KD + 8;   // floats per column of a carry-tile copy (34 16-byte units)
constexpr int kComposeRing = 2;     // operand ring: a block is loaded kComposeRing - 1 steps before its store to LDS
constexpr int kComposeWaves = kComposeThreads / 64;
constexpr int kKHalf = KD / 2;                                 // k per wave
constexpr int kAPieces = 16 * kKHalf / 4 / 64;                 // 16-byte pieces of a wave's A block per lane
constexpr int kARegion = 16 * kKHalf + 4 * 16;                 // floats per wave's region (reverse: skewed)
constexpr int kBtStride = kComposeColumns + 4;                 // floats per row of a wave's B_r rows
static_assert(kComposeWaves == 16 && kAPieces == 4, "compose: 8 row tiles x 2 k halves, 4 pieces per lane");

struct alignas(16) ComposeSmem {
  float at[kComposeWaves][kARegion];                     // each wave's block of A_r
  float ct[2][2][kComposeColumns * kCtStride];           // partial carries, by step parity and k half
  float bt[kComposeWaves / 2][16 * kBtStride];           // each row tile's 16 rows of B_r[:, block]
};

// The same scan serves four uses (MODE):
//  kScanCompose  the forward's C_0 = 0, C_{r+1} = A_r C_r + B_r over the
//                segments (or, for the backward, over the pieces);
//  kScanReverse  the backward's D_{S-1} = 0, D_{r-1} = A_r^T D_r + E_r: step s
//                stands for segment S-1-s;
//  kScanFold     per segment, its pieces' summaries folded into the
//                segment's own: X <- A'_i X (+ B'_i) from X = [I | 0] over
//                the pieces in order, one chain per (segment, head) and 16
//                column blocks (8 of A_r, 8 of B_r); only the end is kept;
//  kScanPieces   per segment, every piece's carry-in: X = C_r (zero for a
//                segment that does not continue a sequence), written at each
//                piece, then X <- A'_i X + B'_i.
// A transition that is structurally zero (its flag clear) is dropped.
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
  const int tile = wave & 7;   // row tile
  const int kh = wave >> 3;    // k half
  const int lc = lane & 15;    // column within the block (and row within the tile for A)
  const int lj = lane >> 4;    // k slot
  // MFMA 4q + e, k slot lj, stands for k = 64 kh + kblk(q) + e
  auto kblk = [&](const int q) { return 16 * lj + 4 * (q ^ (lj & 1)); };
  const bool bpart = MODE == kScanFold && cb >= kComposeColumnBlocks;   // a column block of B_r
  const int col0 = kComposeColumns * (bpart ? cb - kComposeColumnBlocks : cb);
  const int col = col0 + lc;
  const int row0 = 16 * tile;
  float* const region = sm.at[wave];

  // the chain: steps over the segments, or over one segment's pieces
  int base = 0, S = p.S;
  if (CHAINS) {
    base = p.plan[p.L.useg_piece_ptr + chain];
    const int len = p.plan[p.L.useg_piece_ptr + chain + 1] - base;
    S = MODE == kScanFold ? len + 1 : len;   // a fold applies every piece, then writes
  }
  auto seg_of = [&](const int r) { return REV ? S - 1 - r : base + r; };
  // Piece u < 4 of a step's slot, as a byte offset in A_r: forward, row
  // 16t + 4u + lane/16, floats 64kh + 4(lane % 16) .. (four 256-byte row
  // pieces per wave instruction); reverse, row 64kh + 16u + lane/4, floats
  // 16t + 4(lane % 4) .. (sixteen 64-byte row pieces).  Piece 4: B_r[16t +
  // lane/4][col0 + 4(lane % 4) ..], the row tile's rows of the column block.
  const int a_off = 4 * (REV ? (kKHalf * kh + (lane >> 2)) * KD + row0 + 4 * (lane & 3)
                             : (row0 + (lane >> 4)) * KD + kKHalf * kh + 4 * (lane & 15));
  constexpr int a_step = 4 * (REV ? 16 * KD : 4 * KD);
  const int b_off = 4 * ((row0 + (lane >> 2)) * VD + col0 + 4 * (lane & 3));
  auto load_step = [&](const int r, f32x4 (&a)[kAPieces + 1]) {
    const size_t m = static_cast<size_t>(seg_of(r)) * H + h;
    const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.transitions + m * KD * KD), 0,
                                                      KD * KD * 4, kBufDword3);
    const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.updates + m * KD * VD), 0,
                                                      KD * VD * 4, kBufDword3);
#pragma unroll
    for (int u = 0; u < kAPieces; ++u)
      a[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, a_off + u * a_step, 0, 0));
    a[kAPieces] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, b_off, 0, 0));
  };
  // The wave's block into its region, and its operand back.  Forward: row
  // i of the tile at 64 i, its 16-byte slot s holding k-block s xor
  // (2i % 16).  Reverse: k-major, 16 floats per k, with a 16-float skew per
  // 16 k (the lanes' scalar reads of one k slot then fall into distinct
  // banks).
  auto store_at = [&](const f32x4 (&a)[kAPieces + 1]) {
#pragma unroll
    for (int u = 0; u < kAPieces; ++u) {
      if (REV) {
        const int kl = 16 * u + (lane >> 2);
        st4(&region[kl * 16 + 16 * u + 4 * (lane & 3)], a[u]);
      } else {
        const int i = 4 * u + (lane >> 4);
        st4(&region[64 * i + 4 * ((lane & 15) ^ ((2 * i) & 15))], a[u]);
      }
    }
  };
  auto read_at = [&](f32x4 (&aop)[kAPieces], const int q0, const int q1) {
#pragma unroll
    for (int q = q0; q < q1; ++q) {
      if (REV) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kl = kblk(q) + e;
          aop[q][e] = region[kl * 16 + 16 * (kl >> 4) + lc];
        }
      } else {
        aop[q] = ld4(&region[64 * lc + 4 * ((kblk(q) >> 2) ^ ((2 * lc) & 15))]);
      }
    }
  };
  // B_r through the row tile's rows of bt into the accumulator layout (both
  // waves of the tile store the same values)
  auto store_b = [&](const f32x4& b) { st4(&sm.bt[tile][(lane >> 2) * kBtStride + 4 * (lane & 3)], b); };
  auto read_b = [&]() {
    f32x4 bv;
#pragma unroll
    for (int i = 0; i < 4; ++i) bv[i] = sm.bt[tile][(4 * lj + i) * kBtStride + lc];
    return bv;
  };
  // this lane's four entries of a carry, as byte offsets in its matrix
  const int c_off = 4 * ((row0 + 4 * lj) * VD + col);
  // where step r's value goes: the carry of that segment or piece, or for a
  // fold the segment's transition or update
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

  // this wave's partial of the running value (the k-half-1 wave starts at 0)
  f32x4 part = zero4();
  if (kh == 0) {
    if (MODE == kScanFold && !bpart) {
#pragma unroll
      for (int i = 0; i < 4; ++i) part[i] = row0 + 4 * lj + i == col ? 1.f : 0.f;   // the identity
    } else if (MODE == kScanPieces && p.plan[p.L.useg_carry_in + chain] != 0) {
      const float* csrc = p.init + (static_cast<size_t>(chain) * H + h) * KD * VD;
#pragma unroll
      for (int i = 0; i < 4; ++i) part[i] = csrc[(row0 + 4 * lj + i) * VD + col];
    }
  }
  if (S < 2) {   // no step applies a transition: the start is the one value
    if (S == 1 && kh == 0) {
      float* cdst = dest(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) cdst[(row0 + 4 * lj + i) * VD + col] = part[i];
    }
    return;
  }

  // ring slot t % kComposeRing holds step t's pieces from the load until
  // their store to LDS during step t-1, and lv its flag until its use; aop
  // and bcur hold the operands of the step whose products run next
  f32x4 ring[kComposeRing][kAPieces + 1];
  f32x4 aop[kAPieces];
  f32x4 bcur;
  bool lv[kComposeRing];
#pragma unroll
  for (int d = 0; d < kComposeRing; ++d) {
    lv[d] = live_at(d);
    load_step(d < S - 1 ? d : S - 2, ring[d]);
  }
  store_at(ring[0]);
  store_b(ring[0][kAPieces]);
  read_at(aop, 0, kAPieces);
  bcur = read_b();
  const int ct_own = lc * kCtStride + row0 + 4 * lj;   // this lane's entries in a carry-tile copy
  for (int r0 = 0;; r0 += kComposeRing) {
#pragma unroll
    for (int ph = 0; ph < kComposeRing; ++ph) {
      const int r = r0 + ph;            // r % kComposeRing == ph
      const int buf = r & 1;
      const int p1 = (ph + 1) % kComposeRing;
      const bool live = lv[ph];
      // step r + kComposeRing's pieces into the slot step r-1 has used up,
      // issued first so that they have the whole step to land (the last
      // steps load the last transition again, unused)
      {
        const int rn = r + kComposeRing;
        lv[ph] = live_at(rn);
        load_step(rn < S - 1 ? rn : S - 2, ring[ph]);
      }
      // this wave's partial of C_r, transposed into its half's copy
      st4(&sm.ct[buf][kh][ct_own], part);
      // both partials reached LDS; the barrier also ends step r-1's reads of
      // the other parity's copies, which step r+1 refills
      __syncthreads();
      {
        // C_r in full, stored by both waves of the row tile
        const f32x4 other = ld4(&sm.ct[buf][kh ^ 1][ct_own]);
        const auto rc = __builtin_amdgcn_make_buffer_rsrc(dest(r), 0, KD * VD * 4, kBufDword3);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(part[i] + other[i]), rc, c_off + 4 * i * VD, 0, 0);
      }
      if (r == S - 1) return;
      f32x4 bop[kAPieces];
#pragma unroll
      for (int q = 0; q < kAPieces; ++q) {
        const int o = lc * kCtStride + kKHalf * kh + kblk(q);
        bop[q] = ld4(&sm.ct[buf][0][o]) + ld4(&sm.ct[buf][1][o]);
      }
      // four independent accumulator chains (k slot e of every MFMA group),
      // summed at the end; step r+1's operands go through LDS between the
      // two halves of the products
      const f32x4 b0 = kh == 0 && !(MODE == kScanFold && !bpart) ? bcur : zero4();
      f32x4 acc[4] = {b0, zero4(), zero4(), zero4()};
#pragma unroll
      for (int q = 0; q < kAPieces / 2; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop[q][e], bop[q][e], acc[e], 0, 0, 0);
      store_at(ring[p1]);
      store_b(ring[p1][kAPieces]);
      read_at(aop, 0, kAPieces / 2);
#pragma unroll
      for (int q = kAPieces / 2; q < kAPieces; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop[q][e], bop[q][e], acc[e], 0, 0, 0);
      read_at(aop, kAPieces / 2, kAPieces);
      bcur = read_b();
      // the products run whatever the flag (the loop has no branch for the
      // compiler to merge wait counts over); a transition that is
      // structurally zero is dropped here, whatever its buffer holds
      const f32x4 prod = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) part[i] = live ? prod[i] : b0[i];
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
