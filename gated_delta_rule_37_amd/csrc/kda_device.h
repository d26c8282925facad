// Device helpers shared by the chunk kernels of the forward pass and the
// chunked backward (gfx950): bf16 types, split-bf16 operands on the bf16
// matrix cores, the k-slot operand order of accumulator tiles, and the LDS
// transpose read.
#ifndef KDA_DEVICE_H_
#define KDA_DEVICE_H_

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kda {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte LDS accesses through native vector types (HIP's float4/uint4
// structs are split into pairs of 8-byte accesses)
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, const f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void st4(bf16* p, const u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

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
__device__ __forceinline__ void mfma_result_fence(f32x4& t) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(t));
}
__device__ __forceinline__ void mfma_result_fence(f32x16& t0, f32x16& t1, f32x16& t2, f32x16& t3) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(t0), "+v"(t1), "+v"(t2), "+v"(t3));
}
__device__ __forceinline__ void mfma_result_fence(f32x16& t) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(t));
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (round to nearest even), x0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1) {
  const f32x2 v = {x0, x1};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Split two floats into packed (hi, lo) bf16 pairs: x = hi + lo to ~16 bits.
// hi is unpacked with integer ops (bf16 is the upper half of a float), so a
// pair costs two conversions, two bit operations and two subtractions.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(x0, x1);
  lo = pack_bf16(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u));
}

// The same split for inputs that are dead afterwards, one instruction
// cheaper per element: v_dot2c_f32_bf16 adds the exact bf16 products
// h.e * m.e to x in place, and with m = (-1, 0) or (0, -1) the result x - h.e
// is representable, hence exact (checked bitwise on gfx950 against the
// subtraction above).  The multipliers go through an SGPR because the
// compiler would otherwise encode them as the inline constant -1.0, which the
// instruction reads as the 32-bit float, not as a bf16 pair.
__device__ __forceinline__ bf16x2 sgpr_bf16x2(uint32_t bits) {
  asm("" : "+s"(bits));
  return __builtin_bit_cast(bf16x2, bits);
}
__device__ __forceinline__ void split_pair_dead(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const f32x2 v = {x0, x1};
  const bf16x2 h = __builtin_convertvector(v, bf16x2);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = pack_bf16(__builtin_amdgcn_fdot2_f32_bf16(h, sgpr_bf16x2(0x0000bf80u), x0, false),
                 __builtin_amdgcn_fdot2_f32_bf16(h, sgpr_bf16x2(0xbf800000u), x1, false));
}

template <bool DEAD = false>
__device__ __forceinline__ void split8(const float x[8], bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t a, b;
    if (DEAD) split_pair_dead(x[2 * w], x[2 * w + 1], a, b);
    else split_pair(x[2 * w], x[2 * w + 1], a, b);
    h[w] = a;
    l[w] = b;
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// Returns x unchanged, but the compiler cannot see through it: lane indices
// taken through it at each step make the step recompute its LDS addresses
// (one add each) instead of keeping dozens of them live across the chunk loop.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Workgroup barrier for the two wave roles.  Owners and helpers run separate
// loops (so that neither holds the other's registers), and both execute the
// same sequence of barriers: s_barrier counts arriving waves, wherever they
// are in the program.
__device__ __forceinline__ void block_sync() { __syncthreads(); }

// Orders a wave's own LDS writes before its later reads of other lanes'
// values (LDS accesses of one wave complete in program order; this keeps the
// compiler from moving the reads up).
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

// k-slot order used with accumulator tiles as B operands.  A 32 x 32 tile t
// (rows 16s .. 16s+15 of it feeding k-step s) becomes a B operand without any
// cross-lane move when the k slot (l/32, j) of the MFMA stands for row
// 16s + 4(l/32) + j (j < 4) or 16s + 8 + 4(l/32) + j - 4 (j >= 4): those are
// the lane's own registers 8s + j and 8s + 4 + j - 4.  The dot product does
// not depend on the order of k, so the A operand only has to take its k
// columns in the same order: two 8-byte pieces, at columns 16s + 4(l/32) and
// 16s + 8 + 4(l/32).
__device__ __forceinline__ void tile_kslots(const f32x16& t, const int s, float out[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[j] = t[8 * s + j];
    out[4 + j] = t[8 * s + 4 + j];
  }
}
__device__ __forceinline__ void tile_kslots_split(const f32x16& t, bf16x8 bh[2], bf16x8 bl[2]) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float x[8];
    tile_kslots(t, s, x);
    split8<true>(x, bh[s], bl[s]);
  }
}
// A operand in k-slot order from a row-major bf16 matrix at p = row + c
// (c = 16s + 4(l/32) for k-step s): p[0..3] and p[8..11], as two 8-byte reads.
// They are volatile LDS loads, which keeps the compiler from fusing them into
// one ds_read2_b64 (four times as slow on gfx950) while a fixed per-lane base
// with immediate offsets still serves every k-step.
typedef const volatile __attribute__((address_space(3))) bf16x4 lds_bf16x4;
__device__ __forceinline__ bf16x8 ld_kslots_at(const bf16* p) {
  const bf16x4 a = *(lds_bf16x4*)(const_cast<bf16*>(p));
  const bf16x4 b = *(lds_bf16x4*)(const_cast<bf16*>(p + 8));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// The same 16 bytes with the two 8-byte halves exchanged (two 8-byte reads,
// high half first), for rows stored with their halves exchanged.
__device__ __forceinline__ bf16x8 ld_halves_swapped(const bf16* p) {
  const bf16x4 a = *(lds_bf16x4*)(const_cast<bf16*>(p + 4));
  const bf16x4 b = *(lds_bf16x4*)(const_cast<bf16*>(p));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Matrices whose columns only ever feed k-slot A operands (T diag(beta) and P,
// columns = tokens) are stored with the columns in k-slot order, so that
// the operand is one contiguous 16-byte read at 16s + 8(l/32): column t of
// each 16-column group sits at position t with bits 2 and 3 swapped.
__device__ __forceinline__ int kslot_col(const int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

// Transposed LDS read (gfx950 ds_read_b64_tr_b16): within each group of 16
// lanes, lane i receives element i%4 of the 8-byte chunks addressed by lanes
// i/4, i/4 + 4, i/4 + 8 and i/4 + 12 (checked on gfx950).  Pointing lane s at
// row r0 + s/4, columns c0 + 4(s%4) of a row-major bf16 matrix therefore gives
// lane i the column c0 + i, rows r0 .. r0+3: a column fragment of a matrix
// stored by rows.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ s16x4 lds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<bf16*>(p)));
}
__device__ __forceinline__ bf16x8 join8(const s16x4 a, const s16x4 b) {
  const s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// One step of an inclusive scan across each 16-lane row: x += (x of the lane
// CTRL's row shift away; zero past the row's start).
template <int CTRL, int TPL>
__device__ __forceinline__ void scan_stage(float (&G)[TPL][8]) {
#pragma unroll
  for (int j = 0; j < TPL; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c)
      G[j][c] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(G[j][c]), CTRL, 0xf, 0xf, true));
}

}  // namespace kda

#endif  // KDA_DEVICE_H_
