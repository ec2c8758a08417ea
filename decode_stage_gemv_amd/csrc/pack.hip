// Offline packing of b_max-bit codes into the MSB-first 1-bit-plane store
// (GRINQH paper, section 3.3 "Storage Layout and Weight Loading"; Appendix
// C.1 "Bit-packing" and "Grouping").  Also the workspace fill kernel.
#include "common.hpp"

namespace grinqh {

// One thread builds the b_max plane words of one (row, 32-column word).
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, int64_t K,
                                                   int64_t N, int bmax, uint8_t* __restrict__ planes) {
  const int64_t Np = padded_cols(N);
  const int64_t words_per_row = Np / 32;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= K * words_per_row) return;
  const int64_t i = gid / words_per_row;
  const int64_t cw = gid - i * words_per_row;
  const int64_t t = cw / kWordsPerTile;
  const int64_t w = cw - t * kWordsPerTile;
  const int64_t ct = (Np - t * kTile) < kTile ? (Np - t * kTile) : kTile;

  // d[m] holds the codes of columns 4m .. 4m + 3 of this word, byte j = column 4m + j.
  const uint8_t* row = codes + i * N;
  const int64_t c0 = cw * 32;
  uint32_t d[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = c0 + 4 * m + j;
      const uint32_t code = col < N ? row[col] : 0u;
      v |= code << (8 * j);
    }
    d[m] = v;
  }
  // Plane p word: bit 8j + m = bit (b_max - 1 - p) of byte j of d[m].
  uint8_t* base = planes + store_offset(t * K * kTile + i * ct, bmax) + 4 * w;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    if (p < bmax) {
      const int bit = bmax - 1 - p;
      uint32_t word = 0;
#pragma unroll
      for (int m = 0; m < 8; ++m) word |= ((d[m] >> bit) & 0x01010101u) << m;
      *reinterpret_cast<uint32_t*>(base + p * (ct / 8)) = word;
    }
  }
}

int launch_pack(const uint8_t* codes, int64_t K, int64_t N, int bmax, uint8_t* planes, hipStream_t s) {
  const int64_t total = K * (padded_cols(N) / 32);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, K, N, bmax, planes);
  return check_launch("grinqh_pack");
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint8_t* __restrict__ p, int64_t bytes) {
  const int64_t words = bytes / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < words; k += stride)
    reinterpret_cast<uint32_t*>(p)[k] = 0u;
  const int64_t tail = bytes - words * 4;
  if (blockIdx.x == 0 && (int64_t)threadIdx.x < tail) p[words * 4 + threadIdx.x] = 0;
}

int launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
  if (reinterpret_cast<uintptr_t>(ptr) % 4 != 0) return fail(GRINQH_EINVAL, "workspace must be 4-byte aligned");
  int64_t blocks = ((int64_t)bytes / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<uint8_t*>(ptr), (int64_t)bytes);
  return check_launch("grinqh_workspace_init");
}

}  // namespace grinqh
