// Decode-stage VMM for nested non-uniform weights reconstructed from look-up
// tables (GRINQH paper, section 3.3 "Storage Layout and Weight Loading":
// k-means style nested codes in the same bit-plane store; "Weight
// Reconstruction and Bias Correction": with tables the nested levels are
// already centred, so no midpoint term; Appendix E.2).
//
//   y[j] += sum over rows with b_i > 0 of x_i * T_{b_i}[j][q_ij >> (b_max - b_i)]
//
// with one fp16 table per output column j and bit width b (2^b entries).
//
// Work split.  A workgroup owns 128 columns (four plane words of one store
// tile) and a range of rows.  It first copies the tables of the widths in use
// for its columns into LDS (row p of width b's table holds entry p of all 128
// columns, in a word-interleaved order and with a padded stride so that the
// lanes' random lookups spread over the banks), and the rows' activations and
// widths (assignment of section 3.1, fused).  Then each lane takes one row
// and one plane word (32 columns) at a time: it loads only the top b planes
// of that row (section 3.3), rebuilds the 32 codes with the bit transpose of
// bitplane.hpp, and for each column looks the weight up in LDS and adds
// x_i * w into an fp32 accumulator for that column.  Rows of width 0 load
// nothing.  The next chunk's plane words are in flight while a chunk is
// processed.  At the end the lanes that share a word are reduced with
// shuffles, the waves in LDS, and the sums are added into y with fp32
// atomics (so y accumulates, as the accumulating uniform entry point does).
#include "bitplane.hpp"
#include "common.hpp"

namespace grinqh {

namespace {

constexpr int kLCols = 128;                 // columns per workgroup
constexpr int kLWords = kLCols / 32;        // plane words per row
constexpr int kLWaves = 8;
constexpr int kLThreads = 64 * kLWaves;
constexpr int kLRowsPerPass = kLThreads / kLWords;   // rows processed per pass (128)
constexpr int kLStride = kLCols + 2;        // halves per LDS table row (padded)
constexpr int kLMaxRows = 2048;             // rows per workgroup
constexpr int kLTargetWGs = 512;

struct LutArgs {
  const uint8_t* planes;
  const uint16_t* lut;
  const uint16_t* x;
  float* y;
  float* clear;
  int64_t K, N;
  int bmax, rows, n_ct;
  int lut_halves;          // LDS halves taken by the tables
  int toff[9];             // LDS offset (halves) of width b's table; -1 if not in use
  AssignParams ap;
};

// LDS position of column c (0..127) inside a table row: word-interleaved, so
// that the lanes of one wave (different words, same column within the word)
// hit consecutive halves.
__device__ inline int lut_pos(int c) { return (c & 31) * kLWords + (c >> 5); }

}  // namespace

int lut_smem_bytes(const LutArgs& a) { return a.lut_halves * 2 + a.rows * 2 + a.rows + 16; }

__global__ __launch_bounds__(kLThreads) void vmm_lut_kernel(LutArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t s_dyn[];
  uint16_t* s_lut = s_dyn;
  uint16_t* s_xv = s_dyn + a.lut_halves;
  uint8_t* s_b = reinterpret_cast<uint8_t*>(s_xv + a.rows);
  __shared__ float s_red[kLWaves][kLCols];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = a.K, N = a.N;
  const int cti = blockIdx.x % a.n_ct;
  const int split = blockIdx.x / a.n_ct;
  const int64_t n0 = (int64_t)cti * kLCols;
  const int64_t k0 = (int64_t)split * a.rows;
  const int nrows = (int)((K - k0) < a.rows ? (K - k0) : a.rows);
  const int64_t t0 = n0 / kTile * kTile;
  const int64_t Np = padded_cols(N);
  const int ct = (int)((Np - t0) < kTile ? (Np - t0) : kTile);
  const int pb = ct / 8;
  const int bmax = a.bmax;
  const int word0 = (int)(n0 - t0) / 32;

  // ---- tables of the widths in use -> LDS
  for (int b = 1; b <= bmax; ++b) {
    const int off = a.toff[b];
    if (off < 0) continue;
    const int nb = 1 << b;
    const uint16_t* src = a.lut + N * (int64_t)(nb - 2) + n0 * nb;   // column n0's table of width b
    for (int e = tid; e < kLCols * nb; e += kLThreads) {
      const int c = e >> b, p = e & (nb - 1);
      const uint16_t v = n0 + c < N ? src[e] : (uint16_t)0;
      s_lut[off + p * kLStride + lut_pos(c)] = v;
    }
  }
  // ---- activations and widths of this workgroup's rows
  const AssignRegs ar = load_assign_regs(a.ap);
  for (int r = tid; r < nrows; r += kLThreads) {
    const uint16_t xv = a.x[k0 + r];
    s_xv[r] = xv;
    s_b[r] = (uint8_t)bits_of(xv, ar);
  }
  __syncthreads();

  // ---- rows: lane = (row slot rs, word wl); pass q covers rows q*128 .. +127
  const int wl = tid & (kLWords - 1);
  const int rs = tid >> 2;
  const int passes = (nrows + kLRowsPerPass - 1) / kLRowsPerPass;
  const uint8_t* wbase = a.planes + 4 * (word0 + wl);
  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.0f;

  // plane words of the lane's row in pass q (planes past its width are 0)
  auto load_pass = [&](int q, uint32_t (&w)[8], int& b, uint16_t& xv) {
    const int r = q * kLRowsPerPass + rs;
    b = r < nrows ? s_b[r] : 0;
    xv = r < nrows ? s_xv[r] : (uint16_t)0;
    const uint8_t* base = wbase + store_offset(t0 * K + (k0 + (r < nrows ? r : 0)) * ct, bmax);
#pragma unroll
    for (int p = 0; p < 8; ++p) w[p] = p < b ? *reinterpret_cast<const uint32_t*>(base + p * pb) : 0u;
  };

  uint32_t wc[8];
  int bc;
  uint16_t xc;
  if (passes > 0) load_pass(0, wc, bc, xc);
  for (int q = 0; q < passes; ++q) {
    uint32_t wn[8];
    int bn = 0;
    uint16_t xn = 0;
    if (q + 1 < passes) load_pass(q + 1, wn, bn, xn);
    if (bc > 0) {
      uint32_t d[8];
      planes_to_codes<8>(wc, d);   // plane p at code bit 7 - p: q 2^(8 - b_max) with low bits cleared
      const int shift = 8 - bc;    // prefix = top bc bits of the 8-bit field
      const uint16_t* tab = s_lut + a.toff[bc];
      const float xf = half_bits_to_float(xc);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 4 * m + j;                       // column within the word
          const uint32_t code = (d[m] >> (8 * j)) & 0xFFu;
          const uint32_t p = code >> shift;
          const uint16_t wv = tab[p * kLStride + c * kLWords + wl];
          acc[c] += xf * half_bits_to_float(wv);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) wc[p] = wn[p];
    bc = bn;
    xc = xn;
  }

  // ---- reduce: lanes sharing a word (lane bits 2..5), then the waves
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    float v = acc[c];
    v += __shfl_xor(v, 4, 64);
    v += __shfl_xor(v, 8, 64);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    acc[c] = v;
  }
  if (lane < kLWords) {
#pragma unroll
    for (int c = 0; c < 32; ++c) s_red[wid][32 * lane + c] = acc[c];
  }
  __syncthreads();
  if (tid < kLCols) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kLWaves; ++w) v += s_red[w][tid];
    const int64_t n = n0 + tid;
    if (n < N) {
      if (nrows > 0) __hip_atomic_fetch_add(a.y + n, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (a.clear && split == 0) a.clear[n] = 0.0f;
    }
  }
}

int launch_vmm_lut(const uint8_t* planes, const uint16_t* lut, const uint16_t* x, int64_t K, int64_t N,
                   int bmax, const AssignParams& ap, float* y, float* clear, hipStream_t s) {
  LutArgs a{};
  a.planes = planes; a.lut = lut; a.x = x; a.y = y; a.clear = clear;
  a.K = K; a.N = N; a.bmax = bmax; a.ap = ap;
  // widths in use: the levels the assignment can produce
  bool used[9] = {false};
  for (int t = 0; t <= ap.n; ++t) used[ap.lv[t]] = true;
  int off = 0;
  for (int b = 0; b <= 8; ++b) a.toff[b] = -1;
  for (int b = 1; b <= bmax; ++b)
    if (used[b]) {
      a.toff[b] = off;
      off += (1 << b) * kLStride;
    }
  a.lut_halves = (off + 7) / 8 * 8;
  a.n_ct = (int)(padded_cols(N) / kLCols);
  int64_t splits = (K + kLMaxRows - 1) / kLMaxRows;
  const int64_t want = (kLTargetWGs + a.n_ct - 1) / a.n_ct;
  if (want > splits) splits = want;
  if (splits > (K + 63) / 64) splits = (K + 63) / 64;
  if (splits < 1) splits = 1;
  int64_t rows = (K + splits - 1) / splits;
  rows = (rows + 7) / 8 * 8;
  splits = (K + rows - 1) / rows;
  a.rows = (int)rows;
  if ((int64_t)a.n_ct * splits > 0x7FFFFFFF)
    return fail(GRINQH_EINVAL, "%lld workgroups: more than one launch handles", (long long)(a.n_ct * splits));
  const int smem = lut_smem_bytes(a);
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(vmm_lut_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 140 * 1024);
    if (e != hipSuccess) return fail(GRINQH_EDEVICE, "grinqh_decode_vmm_lut: %s", hipGetErrorString(e));
    attr_set = true;
  }
  hipLaunchKernelGGL(vmm_lut_kernel, dim3((unsigned)(a.n_ct * splits)), dim3(kLThreads), smem, s, a);
  return check_launch("grinqh_decode_vmm_lut");
}

}  // namespace grinqh
