// Unpacking the bit-plane store at full width into dense fp16 weights (GRINQH
// paper, section 4 "Prefill vs. Decoding Evaluation": for prefill the weights
// are unpacked at full b_max precision and multiplied densely; section 3.3:
// w = s q + z with nothing truncated at b = b_max).
//
// Output layout ("B-fragment order"): element (k, n) of the dense K x N matrix
// sits at ((k / 8) N_pad + n) 8 + k % 8, i.e. eight consecutive rows of one
// column form one 16-byte fragment and the fragments of one 8-row block run
// along the columns.  This is the order in which a 32 x 32 x 16 fp16 matrix
// instruction takes its B operand (one fragment per lane), so the GEMM reads
// it straight into registers.  Rows past K (up to K rounded up to 64) and
// columns past N are zero.
//
// Work split: thread (row pair r, plane word w) loads the b_max plane words of
// rows 2r and 2r + 1 for columns 32 w .. 32 w + 31 (rows of the last 8-row
// blocks that lie past K, up to the padded row count, are written as zero),
// rebuilds the codes with the
// bit transpose of bitplane.hpp, and writes one dword (the two rows as an fp16
// pair, w = s q + z rounded once by a packed fused multiply-add) per column.
// The 64 threads of a wave cover 4 row pairs x 16 words, so each store
// instruction writes whole 16-byte fragments.
#include "bitplane.hpp"
#include "common.hpp"

namespace grinqh {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

struct UnpackArgs {
  const uint8_t* planes;
  const uint16_t* scales;
  const uint16_t* zeros;
  uint32_t* out;          // dwords: ((k / 8) N_pad + n) 4 + (k % 8) / 2
  int64_t K, N;
  int bmax;
};

}  // namespace

int64_t unpack_dense_bytes(int64_t K, int64_t N) { return dense_rows(K) * padded_cols(N) * 2; }

template <int BMAX>
__global__ __launch_bounds__(256) void unpack_kernel(UnpackArgs a) {
  const int64_t K = a.K, N = a.N;
  const int64_t Np = padded_cols(N);
  const int64_t words = Np / 32;
  const int64_t pairs = dense_rows(K) / 2;               // row pairs up to the padded row count
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t wq = (words + 15) / 16;                  // 16-word groups per row
  const int64_t grp = t >> 6;
  const int64_t rp = 4 * (grp / wq) + (t & 3);           // row pair
  const int64_t w = 16 * (grp % wq) + ((t >> 2) & 15);   // plane word (32 columns)
  if (rp >= pairs || w >= words) return;

  const int64_t t0 = w / kWordsPerTile * kTile;          // store tile of this word
  const int64_t ct = (Np - t0) < kTile ? (Np - t0) : kTile;
  const int64_t pb = ct / 8;
  const int64_t wt = w - t0 / 32;                        // word within the tile
  uint32_t w1[8], w2[8];
  const int64_t r1 = 2 * rp, r2 = 2 * rp + 1;
  uint32_t* dst = a.out + ((r1 / 8) * Np + 32 * w) * 4 + (rp & 3);
  if (r1 >= K) {                                         // both rows past K: zero fill of the last block
#pragma unroll
    for (int c = 0; c < 32; ++c) dst[c * 4] = 0u;
    return;
  }
  const bool ok2 = r2 < K;
  const uint8_t* b1 = a.planes + store_offset(t0 * K + r1 * ct, BMAX) + 4 * wt;
  const uint8_t* b2 = a.planes + store_offset(t0 * K + (ok2 ? r2 : r1) * ct, BMAX) + 4 * wt;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    w1[p] = p < BMAX ? *reinterpret_cast<const uint32_t*>(b1 + p * pb) : 0u;
    w2[p] = p < BMAX ? *reinterpret_cast<const uint32_t*>(b2 + p * pb) : 0u;
  }
  // scale and zero of the 32 columns (group of the two rows), clamped to N
  const int64_t g = r1 / kGroup;
  uint16_t sc[32], zr[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    int64_t n = 32 * w + c;
    n = n < N ? n : N - 1;
    sc[c] = a.scales[g * N + n];
    zr[c] = a.zeros[g * N + n];
  }
  uint32_t d1[8], d2[8];
  planes_to_codes<BMAX>(w1, d1);
  planes_to_codes<BMAX>(w2, d2);
  constexpr int kSh = 8 - BMAX;                          // codes come back as q 2^(8 - b_max)
  constexpr uint32_t kKeep = 0x01010101u * (0xFFu >> kSh);
  if constexpr (kSh > 0) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      d1[m] = (d1[m] >> kSh) & kKeep;
      d2[m] = (d2[m] >> kSh) & kKeep;
    }
  }
  const uint32_t hi_mask = ok2 ? 0xFFFFFFFFu : 0x0000FFFFu;   // a row past K is zero
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 4 * m + j;
      // [row 2r code, 0x64, row 2r+1 code, 0x64] = fp16 (1024 + c1, 1024 + c2)
      const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24);
      const uint32_t pr = __builtin_amdgcn_perm(d2[m], d1[m], sel) | 0x64006400u;
      const half2_t q = __builtin_bit_cast(half2_t, pr) - (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
      const _Float16 s = __builtin_bit_cast(_Float16, sc[c]);
      const _Float16 z = __builtin_bit_cast(_Float16, zr[c]);
      const half2_t v = __builtin_elementwise_fma(q, (half2_t){s, s}, (half2_t){z, z});
      uint32_t out = __builtin_bit_cast(uint32_t, v) & hi_mask;
      if (32 * w + c >= N) out = 0u;                     // padding column
      dst[c * 4] = out;
    }
  }
}

int launch_unpack_dense(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros, int64_t K,
                        int64_t N, int bmax, void* out, hipStream_t s) {
  UnpackArgs a{planes, scales, zeros, reinterpret_cast<uint32_t*>(out), K, N, bmax};
  const int64_t words = padded_cols(N) / 32;
  const int64_t threads = dense_rows(K) / 8 * 64 * ((words + 15) / 16);   // a wave per 8-row block x 16 words
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return fail(GRINQH_EINVAL, "K x N too large for one unpack launch");
  const dim3 grid((unsigned)blocks), block(256);
  switch (bmax) {
    case 1: hipLaunchKernelGGL(unpack_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(unpack_kernel<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(unpack_kernel<3>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(unpack_kernel<4>, grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL(unpack_kernel<5>, grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL(unpack_kernel<6>, grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL(unpack_kernel<7>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(unpack_kernel<8>, grid, block, 0, s, a); break;
  }
  return check_launch("grinqh_unpack_dense");
}

}  // namespace grinqh
