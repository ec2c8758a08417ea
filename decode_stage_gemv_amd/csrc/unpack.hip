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
// Work split: a wave owns one 8-row block x 512 columns (16 plane words).
// Phase 1: thread (row pair r of the block, plane word w) loads the b_max plane
// words of its two rows, rebuilds the codes with the bit transpose of
// bitplane.hpp and writes them as exact fp16 integers, the two rows as one
// dword per column, into the wave's LDS slice in fragment order (columns
// XOR-swizzled within their 32-column word so that the writes spread over
// the banks).  Phase 2: lane l reads back whole 16-byte fragments (columns l,
// l + 64, ...), turns the eight codes into w = s q + z with packed fp16 fused
// multiply-adds (one rounding; s and z are shared by the fragment's rows) and
// stores them, so that each store instruction writes 1 KB of contiguous
// output.
#include "bitplane.hpp"
#include "common.hpp"

namespace grinqh {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kUWords = 16;                      // plane words (32 columns each) per wave
constexpr int kUCols = 32 * kUWords;             // 512 columns per wave
constexpr int kUWaves = 4;

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
__global__ __launch_bounds__(64 * kUWaves) void unpack_kernel(UnpackArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t s_f[kUWaves][kUCols * 4];
  const int64_t K = a.K, N = a.N;
  const int64_t Np = padded_cols(N);
  const int64_t words = Np / 32;
  const int64_t wq = (words + kUWords - 1) / kUWords;     // 16-word groups per row
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * kUWaves + wv;  // wave of the grid
  const int64_t kb = gw / wq;                             // 8-row block
  const int64_t n0 = (gw % wq) * kUCols;                  // first column of the wave
  uint32_t* f = s_f[wv];
  const bool live = kb < dense_rows(K) / 8;               // always true for the launcher's grid

  // ---- phase 1: codes of rows 8 kb + 2 pi, + 1 for columns of word wi
  {
    const int pi = lane & 3, wi = lane >> 2;
    const int64_t w = n0 / 32 + wi;
    const int64_t r1 = 8 * kb + 2 * pi, r2 = r1 + 1;
    uint32_t w1[8], w2[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) w1[p] = w2[p] = 0u;
    if (live && w < words && r1 < K) {
      const int64_t t0 = w / kWordsPerTile * kTile;         // store tile of this word
      const int64_t ct = (Np - t0) < kTile ? (Np - t0) : kTile;
      const int64_t pb = ct / 8;
      const int64_t wt = w - t0 / 32;                       // word within the tile
      const uint8_t* b1 = a.planes + store_offset(t0 * K + r1 * ct, BMAX) + 4 * wt;
      const uint8_t* b2 = a.planes + store_offset(t0 * K + (r2 < K ? r2 : r1) * ct, BMAX) + 4 * wt;
#pragma unroll
      for (int p = 0; p < BMAX; ++p) {
        w1[p] = *reinterpret_cast<const uint32_t*>(b1 + p * pb);
        w2[p] = *reinterpret_cast<const uint32_t*>(b2 + p * pb);
      }
    }
    uint32_t d1[8], d2[8];
    planes_to_codes<BMAX>(w1, d1);
    planes_to_codes<BMAX>(w2, d2);
    constexpr int kSh = 8 - BMAX;                           // codes come back as q 2^(8 - b_max)
    constexpr uint32_t kKeep = 0x01010101u * (0xFFu >> kSh);
    if constexpr (kSh > 0) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        d1[m] = (d1[m] >> kSh) & kKeep;
        d2[m] = (d2[m] >> kSh) & kKeep;
      }
    }
    uint32_t* dst = f + 32 * wi * 4 + pi;
    const int sw = wi & 7;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // [row 2r code, 0x64, row 2r+1 code, 0x64] = fp16 (1024 + c1, 1024 + c2)
        const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24);
        const uint32_t pr = __builtin_amdgcn_perm(d2[m], d1[m], sel) | 0x64006400u;
        const half2_t q = __builtin_bit_cast(half2_t, pr) - (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
        dst[((4 * m + j) ^ sw) * 4] = __builtin_bit_cast(uint32_t, q);
      }
    }
  }
  __syncthreads();

  // ---- phase 2: lane l dequantises and stores fragments of columns l + 64 i
  const int64_t g = 8 * kb / kGroup;
  const int kvalid = (int)(K - 8 * kb);                    // rows of this block below K (uniform)
#pragma unroll
  for (int i = 0; i < kUCols / 64; ++i) {
    const int col = 64 * i + lane;
    const int64_t n = n0 + col;
    if (!live || n >= Np) continue;
    const int wi = col >> 5;
    uint32_t q[4], o[4];
    __builtin_memcpy(q, &f[(32 * wi + ((col & 31) ^ (wi & 7))) * 4], 16);
    if (n < N) {
      const _Float16 sv = __builtin_bit_cast(_Float16, a.scales[g * N + n]);
      const _Float16 zv = __builtin_bit_cast(_Float16, a.zeros[g * N + n]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, q[e]),
                                                                      (half2_t){sv, sv}, (half2_t){zv, zv}));
      if (kvalid < 8) {                                     // last block: rows past K are zero
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (2 * e >= kvalid) o[e] = 0u;
          else if (2 * e + 1 >= kvalid) o[e] &= 0xFFFFu;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = 0u;                // padding column
    }
    __builtin_memcpy(&a.out[(kb * Np + n) * 4], o, 16);
  }
}

int launch_unpack_dense(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros, int64_t K,
                        int64_t N, int bmax, void* out, hipStream_t s) {
  UnpackArgs a{planes, scales, zeros, reinterpret_cast<uint32_t*>(out), K, N, bmax};
  const int64_t words = padded_cols(N) / 32;
  const int64_t waves = dense_rows(K) / 8 * ((words + kUWords - 1) / kUWords);   // 8-row block x 16 words each
  const int64_t blocks = (waves + kUWaves - 1) / kUWaves;
  if (blocks > 0x7FFFFFFF) return fail(GRINQH_EINVAL, "K x N too large for one unpack launch");
  const dim3 grid((unsigned)blocks), block(64 * kUWaves);
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
