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
// for its columns into LDS (column c's 2^b entries at c (2^b + 2) + 16 (c / 32)
// halves: a copy of contiguous runs, and the padding spreads the lanes'
// random lookups over the banks), computes the rows' widths (assignment of
// section 3.1, fused) and lists the rows of non-zero width (rows of width 0
// are never touched again).  Then each lane takes one listed row and one
// plane word (32 columns) at a time: it loads only the top b planes of that
// row (section 3.3), rebuilds the 32 codes with the bit transpose of
// bitplane.hpp, and for each column looks the weight up in LDS and adds
// x_i * w into an fp32 accumulator for that column.  The next chunk's plane
// words are in flight while a chunk is processed.  At the end the lanes that share a word are reduced with
// shuffles, the waves in LDS, and the sums are added into y with fp32
// atomics (so y accumulates, as the accumulating uniform entry point does).
#include <type_traits>

#include "bitplane.hpp"
#include "common.hpp"

namespace grinqh {

namespace {

constexpr int kLCols = 128;                 // columns per workgroup
constexpr int kLWords = kLCols / 32;        // plane words per row
constexpr int kLWaves = 8;
constexpr int kLThreads = 64 * kLWaves;
constexpr int kLRowsPerPass = kLThreads / kLWords;   // rows processed per pass (128)
constexpr int kLMaxRows = 2048;             // rows per workgroup
constexpr int kLTargetWGs = 512;            // two resident workgroups per CU

struct LutArgs {
  const uint8_t* planes;
  const uint16_t* lut;
  const uint16_t* x;
  float* y;
  float* clear;
  int64_t K, N;
  int bmax, rows, n_ct;
  int lut_halves;          // LDS halves taken by the tables (at least the reduction buffer)
  int toff[9];             // LDS offset (halves) of width b's table; -1 if not in use
  int nused;               // widths in use
  int used[8];             // those widths, ascending
  AssignParams ap;
};

constexpr int kLRedFloats = kLWaves * kLCols;   // wave reduction buffer, aliased on the tables

}  // namespace

// LDS: tables, then x (fp16) and the list of active rows (u16 offsets) and
// widths (u8) of the workgroup's rows, and a counter.
int lut_smem_bytes(const LutArgs& a) { return a.lut_halves * 2 + a.rows * 2 + a.rows * 2 + a.rows + 16; }

// LDS position (halves) of entry p of column c in a width-b table block.
__device__ inline int lut_at(int c, int p, int stride) { return c * stride + 16 * (c >> 5) + p; }

// LDS use allows at most two workgroups (four waves per SIMD) per CU; saying
// so lets the compiler keep all 32 table lookups of a word in flight.
__global__ __launch_bounds__(kLThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void vmm_lut_kernel(LutArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t s_dyn[];
  uint16_t* s_lut = s_dyn;
  uint16_t* s_xv = s_dyn + a.lut_halves;
  uint16_t* s_act = s_xv + a.rows;                            // active rows, in no particular order
  uint8_t* s_b = reinterpret_cast<uint8_t*>(s_act + a.rows);
  __shared__ int s_nact;
  float* s_red = reinterpret_cast<float*>(s_dyn);   // after the row loop the tables are dead

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

  // ---- tables of the widths in use -> LDS, one width after another: the
  // 128 columns' tables of width b are one contiguous run in global memory,
  // copied with loads of up to 16 bytes, all loads of a round issued before
  // its stores.
  if (tid == 0) s_nact = 0;
  {
    const int cols = (int)((N - n0) < kLCols ? (N - n0) : kLCols);      // columns that exist
    for (int u = 0; u < a.nused; ++u) {
      const int b = a.used[u];
      const int nb = 1 << b, stride = nb + 2;
      const uint16_t* src = a.lut + N * (int64_t)(nb - 2) + n0 * nb;
      uint16_t* dst = s_lut + a.toff[b];
      // halves per load: 8 (16 bytes) or 4 when the run is aligned for it
      // (its start depends on N), else 2
      const uintptr_t at = reinterpret_cast<uintptr_t>(src);
      const int ch = (nb >= 8 && at % 16 == 0) ? 8 : (nb >= 4 && at % 8 == 0) ? 4 : 2;
      auto copy = [&](auto tag) {
        constexpr int kCh = decltype(tag)::value;        // halves per load
        using V = typename std::conditional<kCh == 8, uint4, typename std::conditional<kCh == 4, uint2, uint32_t>::type>::type;
        const V* vs = reinterpret_cast<const V*>(src);
        const int total = cols * nb / kCh;             // loads
        for (int e0 = 0; e0 < total; e0 += 4 * kLThreads) {
          V v[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int e = e0 + k * kLThreads + tid;
            v[k] = vs[e < total ? e : 0];
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int e = e0 + k * kLThreads + tid;
            if (e < total) {
              const int h = e * kCh;                   // first half of this load in the run
              uint32_t w[4];
              __builtin_memcpy(w, &v[k], sizeof(V));
              uint32_t* d = reinterpret_cast<uint32_t*>(dst + lut_at(h >> b, h & (nb - 1), stride));
#pragma unroll
              for (int q = 0; q < kCh / 2; ++q) d[q] = w[q];
            }
          }
        }
      };
      if (ch == 8) copy(std::integral_constant<int, 8>());
      else if (ch == 4) copy(std::integral_constant<int, 4>());
      else copy(std::integral_constant<int, 2>());
    }
  }
  // ---- activations and widths of this workgroup's rows
  const AssignRegs ar = load_assign_regs(a.ap);
  __syncthreads();                 // s_nact cleared
  for (int r = tid; r < nrows; r += kLThreads) {
    const uint16_t xv = a.x[k0 + r];
    const uint32_t b = bits_of(xv, ar);
    s_xv[r] = xv;
    s_b[r] = (uint8_t)b;
    if (b > 0) s_act[atomicAdd(&s_nact, 1)] = (uint16_t)r;
  }
  __syncthreads();
  const int nact = s_nact;

  // ---- rows: lane = (row slot rs, word wl); pass q covers rows q*128 .. +127
  const int wl = tid & (kLWords - 1);
  const int rs = tid >> 2;
  const int passes = (nact + kLRowsPerPass - 1) / kLRowsPerPass;
  const uint8_t* wbase = a.planes + 4 * (word0 + wl);
  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.0f;

  // plane words of the lane's row in pass q (planes past its width are 0)
  auto load_pass = [&](int q, uint32_t (&w)[8], int& b, uint16_t& xv) {
    const int slot = q * kLRowsPerPass + rs;
    const int r = slot < nact ? s_act[slot] : 0;
    b = slot < nact ? s_b[r] : 0;
    xv = slot < nact ? s_xv[r] : (uint16_t)0;
    const uint8_t* base = wbase + store_offset(t0 * K + (k0 + r) * ct, bmax);
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
      const uint32_t shift = 8u - (uint32_t)bc;          // prefix = top bc bits of each code byte
      const uint32_t stride = (1u << bc) + 2u;           // halves per column table in LDS
      const uint16_t* tab = s_lut + a.toff[bc] + lut_at(32 * wl, 0, (int)stride);
      const float xf = half_bits_to_float(xc);
      uint16_t wv[32];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 4 * m + j;                       // column within the word
          const uint32_t p = __builtin_amdgcn_ubfe(d[m], 8u * j + shift, (uint32_t)bc);
          wv[c] = tab[(uint32_t)c * stride + p];
        }
      }
#pragma unroll
      for (int c = 0; c < 32; ++c) acc[c] = __builtin_fmaf(xf, half_bits_to_float(wv[c]), acc[c]);
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
  __syncthreads();                 // every wave is done with the tables
  if (lane < kLWords) {
#pragma unroll
    for (int c = 0; c < 32; ++c) s_red[wid * kLCols + 32 * lane + c] = acc[c];
  }
  __syncthreads();
  if (tid < kLCols) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kLWaves; ++w) v += s_red[w * kLCols + tid];
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
  a.nused = 0;
  for (int b = 1; b <= bmax; ++b)
    if (used[b]) {
      a.toff[b] = off;
      a.used[a.nused++] = b;
      off += ((1 << b) + 2) * kLCols + 16 * kLWords;
    }
  for (int u = a.nused; u < 8; ++u) a.used[u] = 8;
  if (off < 2 * kLRedFloats) off = 2 * kLRedFloats;
  a.lut_halves = (off + 7) / 8 * 8;
  a.n_ct = (int)(padded_cols(N) / kLCols);
  // as many row splits as fit in one round of resident workgroups (two per
  // CU), at least enough to keep every split within kLMaxRows rows
  int64_t splits = kLTargetWGs / a.n_ct;
  if (splits > (K + 63) / 64) splits = (K + 63) / 64;
  if (splits < (K + kLMaxRows - 1) / kLMaxRows) splits = (K + kLMaxRows - 1) / kLMaxRows;
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
