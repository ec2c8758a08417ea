// Bit-plane -> code rebuild used by the VMM kernels (pure integer logic, so it
// also runs on the host for checks).
//
// Store convention (one 32-column word of one row tile): w[p] holds bit 7-p
// of the 8-bit codes; column 4m + j of the word sits at bit 8j + m.  The
// rebuild produces d[m] (m = 0..7) whose byte j is the code of column 4m + j
// with its low 8 - B bits cleared, i.e. the B most significant planes put back
// in place (GRINQH paper, section 3.3: truncation keeps the most significant
// segments; Appendix C.1: codes are rebuilt with OR and SHIFT only).
//
// Inside every byte lane the planes form an 8 x 8 bit matrix (row = plane,
// column = m); the rebuild is its transpose, done with three block-swap
// stages.  Planes at or beyond B are compile-time zeros, so the compiler drops
// the work they would cost.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grinqh {

// Swap the off-diagonal k x k blocks of each byte-lane bit matrix held by
// rows lo (upper) and hi (lower).  M selects the low k bits of every 2k-bit
// field.
template <int k, uint32_t M>
__host__ __device__ inline void swap_blocks(uint32_t& lo, uint32_t& hi) {
  const uint32_t nlo = (lo & M) | ((hi << k) & ~M);
  const uint32_t nhi = ((lo >> k) & M) | (hi & ~M);
  lo = nlo;
  hi = nhi;
}

// (a & m) | (b & ~m) as one v_bfi_b32 on the device.
__host__ __device__ inline uint32_t bit_select(uint32_t m, uint32_t a, uint32_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(m), "v"(a), "v"(b));
  return r;
#else
  return (a & m) | (b & ~m);
#endif
}

// swap_blocks when one side is known to be zero at compile time (LZ: lo is
// zero, HZ: hi is zero); the full case is one shift and one bit select per
// output.
template <int k, uint32_t M, bool LZ, bool HZ>
__host__ __device__ inline void swap_blocks_z(uint32_t& lo, uint32_t& hi) {
  if constexpr (LZ && HZ) {
  } else if constexpr (LZ) {
    lo = (hi << k) & ~M;
    hi = hi & ~M;
  } else if constexpr (HZ) {
    hi = (lo >> k) & M;
    lo = lo & M;
  } else {
    const uint32_t nlo = bit_select(M, lo, hi << k);
    hi = bit_select(M, lo >> k, hi);
    lo = nlo;
  }
}

// Which of v[0..7] are still zero after each stage, for B planes.
__host__ __device__ constexpr bool zero0(int B, int r) { return 7 - r >= B; }
__host__ __device__ constexpr bool zero1(int B, int r) { return zero0(B, r & 3) && zero0(B, (r & 3) + 4); }
__host__ __device__ constexpr bool zero2(int B, int r) {
  return zero1(B, r & 5) && zero1(B, (r & 5) + 2);
}

template <int B>
__host__ __device__ inline void planes_to_codes(const uint32_t (&w)[8], uint32_t (&d)[8]) {
  // v[r] = plane 7 - r, so that after the transpose bit r of a code byte is
  // code bit r.
  uint32_t v[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) v[r] = (7 - r < B) ? w[7 - r] : 0u;
  if constexpr (B <= 1) {
    // one plane: plain shifts and masks, which the compiler folds well (from
    // two planes on, the zero-aware stages below take fewer instructions)
#pragma unroll
    for (int r = 0; r < 4; ++r) swap_blocks<4, 0x0F0F0F0Fu>(v[r], v[r + 4]);
#pragma unroll
    for (int r = 0; r < 8; r += 4) {
      swap_blocks<2, 0x33333333u>(v[r], v[r + 2]);
      swap_blocks<2, 0x33333333u>(v[r + 1], v[r + 3]);
    }
#pragma unroll
    for (int r = 0; r < 8; r += 2) swap_blocks<1, 0x55555555u>(v[r], v[r + 1]);
  } else {
    swap_blocks_z<4, 0x0F0F0F0Fu, zero0(B, 0), zero0(B, 4)>(v[0], v[4]);
    swap_blocks_z<4, 0x0F0F0F0Fu, zero0(B, 1), zero0(B, 5)>(v[1], v[5]);
    swap_blocks_z<4, 0x0F0F0F0Fu, zero0(B, 2), zero0(B, 6)>(v[2], v[6]);
    swap_blocks_z<4, 0x0F0F0F0Fu, zero0(B, 3), zero0(B, 7)>(v[3], v[7]);
    swap_blocks_z<2, 0x33333333u, zero1(B, 0), zero1(B, 2)>(v[0], v[2]);
    swap_blocks_z<2, 0x33333333u, zero1(B, 1), zero1(B, 3)>(v[1], v[3]);
    swap_blocks_z<2, 0x33333333u, zero1(B, 4), zero1(B, 6)>(v[4], v[6]);
    swap_blocks_z<2, 0x33333333u, zero1(B, 5), zero1(B, 7)>(v[5], v[7]);
    swap_blocks_z<1, 0x55555555u, zero2(B, 0), zero2(B, 1)>(v[0], v[1]);
    swap_blocks_z<1, 0x55555555u, zero2(B, 2), zero2(B, 3)>(v[2], v[3]);
    swap_blocks_z<1, 0x55555555u, zero2(B, 4), zero2(B, 5)>(v[4], v[5]);
    swap_blocks_z<1, 0x55555555u, zero2(B, 6), zero2(B, 7)>(v[6], v[7]);
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) d[m] = v[m];
}

// Runtime bit width -> specialised rebuild (b = 0 gives all zeros).
__host__ __device__ inline void planes_to_codes_rt(int b, const uint32_t (&w)[8], uint32_t (&d)[8]) {
  switch (b) {
    case 1: planes_to_codes<1>(w, d); break;
    case 2: planes_to_codes<2>(w, d); break;
    case 3: planes_to_codes<3>(w, d); break;
    case 4: planes_to_codes<4>(w, d); break;
    case 5: planes_to_codes<5>(w, d); break;
    case 6: planes_to_codes<6>(w, d); break;
    case 7: planes_to_codes<7>(w, d); break;
    case 8: planes_to_codes<8>(w, d); break;
    default:
#pragma unroll
      for (int m = 0; m < 8; ++m) d[m] = 0u;
      break;
  }
}

}  // namespace grinqh
