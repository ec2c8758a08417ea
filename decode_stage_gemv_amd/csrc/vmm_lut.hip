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
// section 3.1, fused) and lists the rows of non-zero width grouped by width,
// each width's run padded to a multiple of 32 (rows of width 0 are never
// touched again).  A run of 32 listed rows of one width is a "unit"; a wave
// takes units in turn, lane (row pair, plane word) loading only the top b
// planes of its two rows (section 3.3), rebuilding their codes with the bit
// transpose of bitplane.hpp specialised for b, looking up both rows' weights
// of each of its 32 columns in LDS (constant table strides for b) and adding
// x1 w1 + x2 w2 with one fp16 dot into the column's fp32 accumulator.  The
// next unit's plane words are in flight while a unit is processed.
// Workgroups that share a store tile are numbered onto one XCD (its eight
// 128-column slices read the same plane lines, its row splits the same
// tables).  At the end the lanes that share a word are reduced with lane
// swaps and row rotations in registers, the waves in LDS, and the sums are
// added into y with fp32 atomics (so y accumulates, as the accumulating
// uniform entry point does).
#include <atomic>
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
constexpr int kLMaxDynLds = 160 * 1024 - 1024;   // gfx950: 160 KB of LDS per workgroup, less the static part
constexpr int kLSlices = kTile / kLCols;    // 128-column slices per store tile (8)
constexpr int kLXCDs = 8;                   // MI355X

struct LutArgs {
  const uint8_t* planes;
  const uint16_t* lut;
  const uint16_t* x;
  float* y;
  float* clear;
  int64_t K, N;
  int bmax, rows, n_ct;
  int splits;              // row splits
  int lut_halves;          // LDS halves taken by the tables (at least the reduction buffer)
  int toff[9];             // LDS offset (halves) of width b's table; -1 if not in use
  int nused;               // widths in use
  int used[8];             // those widths, ascending
  int lut_bytes;           // size of the table buffer (< 2^31)
  AssignParams ap;
};

constexpr int kLRedFloats = kLWaves * kLCols;   // wave reduction buffer, aliased on the tables
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kLOutOfRange = 0x7FFFFF00u;  // buffer offset past every range used here
constexpr int kLRsrcWord3 = 0x00020000;         // raw 32-bit buffer, gfx9 family

// Raw buffer descriptor from values that are the same in every lane (the
// read-first-lane keeps the compiler from treating it as divergent).
__device__ inline __amdgpu_buffer_rsrc_t lut_rsrc(const void* base, int64_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, n,
                                           kLRsrcWord3);
}

}  // namespace

// LDS: tables, then x (fp16) and the list of active rows (u16 offsets) of
// the workgroup's rows.
// The row list holds each width's rows in a run padded to a multiple of 32
// entries (at most 31 padding entries for each of the 8 widths).
constexpr int kLListPad = 8 * 32;
int lut_smem_bytes(const LutArgs& a) {
  return a.lut_halves * 2 + a.rows * 2 + (a.rows + kLListPad) * 2;
}

// Cross-lane sums without LDS traffic.  lut_halves_sum: lanes l < 32 get
// a(l) + a(l + 32), lanes l >= 32 get b(l - 32) + b(l) (one swap of a's upper
// half with b's lower half).  lut_rows_sum: with rows of 16 lanes, rows 0
// and 2 get a's row plus the next row of a, rows 1 and 3 get b's previous
// row plus its own (one swap of a's odd rows with b's even rows).  Swapped
// values pass through plain integers: a vector element inside a bit cast is
// mistranslated by the compiler.
__device__ inline float lut_halves_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const uint32_t lo = r[0], hi = r[1];
  return __uint_as_float(lo) + __uint_as_float(hi);
}
__device__ inline float lut_rows_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const uint32_t lo = r[0], hi = r[1];
  return __uint_as_float(lo) + __uint_as_float(hi);
}
// The value of the lane kR places further on within its 16-lane row.
template <int kR>
__device__ inline float lut_row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + kR, 0xF, 0xF, false));
}

// LDS position (halves) of entry p of column c in a width-b table block.
__device__ inline int lut_at(int c, int p, int stride) { return c * stride + 16 * (c >> 5) + p; }

// LDS use allows at most two workgroups (four waves per SIMD) per CU; saying
// so lets the compiler keep all 32 table lookups of a word in flight.
__global__ __launch_bounds__(kLThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void vmm_lut_kernel(const uint16_t* __restrict__ xp, const uint16_t* __restrict__ lutp,
                    const uint8_t* __restrict__ planesp, int Ki, int Ni, int rows, int splits, int n_ct,
                    int lut_bytes, int used_mask, int bmax, LutArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t s_dyn[];
  uint16_t* s_lut = s_dyn;
  uint16_t* s_xv = s_dyn + a.lut_halves;
  uint16_t* s_act = s_xv + rows;                              // active rows by width (see below)
  __shared__ int s_cnt[9], s_cur[9];
  float* s_red = reinterpret_cast<float*>(s_dyn);   // after the row loop the tables are dead

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = Ki, N = Ni;
  // workgroup -> (store tile, row split, 128-column slice), slices fastest,
  // then splits: the eight slices of a store tile read the same 128-byte
  // plane lines (16 bytes each) and the splits of a tile the same tables, so
  // consecutive entries of this order are placed on one XCD (hardware
  // workgroup ids go round-robin over the 8 XCDs) and share its L2
  int L = blockIdx.x;
  const int T = (n_ct + kLSlices - 1) / kLSlices * kLSlices * splits;   // the grid (as launched)
  if (T % kLXCDs == 0) L = (L % kLXCDs) * (T / kLXCDs) + L / kLXCDs;
  const int sub = L % kLSlices;
  const int split = (L / kLSlices) % splits;
  const int cti = (L / kLSlices / splits) * kLSlices + sub;
  if (cti >= n_ct) return;         // a slice past a narrow last tile
  const int64_t n0 = (int64_t)cti * kLCols;
  const int64_t k0 = (int64_t)split * rows;
  const int nrows = (int)((K - k0) < rows ? (K - k0) : rows);
  const int64_t t0 = n0 / kTile * kTile;
  const int64_t Np = padded_cols(N);
  const int ct = (int)((Np - t0) < kTile ? (Np - t0) : kTile);
  const int pb = ct / 8;
  const int word0 = (int)(n0 - t0) / 32;

  // ---- tables of the widths in use -> LDS: the 128 columns' tables of
  // width b are one contiguous run in global memory (4-byte aligned: every
  // table has an even number of entries), copied in 16-byte chunks.
  if (tid < 9) {
    s_cnt[tid] = 0;
    s_cur[tid] = 0;
  }
  // the activations of this thread's rows first, so that their latency
  // passes under the table copy (rows past the range are clamped, unused)
  constexpr int kLRowIters = kLMaxRows / kLThreads;
  uint16_t xpre[kLRowIters];
#pragma unroll
  for (int k = 0; k < kLRowIters; ++k) {
    const int r = tid + k * kLThreads;
    xpre[k] = 0;
    if (k * kLThreads < nrows) xpre[k] = xp[k0 + (r < nrows ? r : 0)];   // no load for a slice past the rows
  }
  {
    // Every width's chunks of this thread are loaded before any is stored
    // (one memory latency for the whole copy).  The widths are unrolled at
    // compile time, so shifts and strides are constants; width b takes
    // max(1, 16 2^b / 512) chunks of 16 bytes per thread, a width not in use
    // issues no loads, and chunks past the buffer read out of range (zero,
    // no traffic).  The full 128 columns are copied even where fewer exist:
    // tables of columns past N feed outputs that are never stored.
    const __amdgpu_buffer_rsrc_t lrs = lut_rsrc(lutp, lut_bytes);
    u32x4_t c1[1], c2[1], c3[1], c4[1], c5[1], c6[2], c7[4], c8[8];
    auto load_w = [&](auto bw, auto& v) {
      constexpr int B = decltype(bw)::value;
      constexpr int kChunks = 16 << B;
      constexpr int kSlots = sizeof(v) / sizeof(v[0]);
      const bool used = (used_mask >> B) & 1;
      if (!used) return;           // no load instructions for a width not in use
      // wave-uniform, in scalar registers (the buffer is below 2^31 bytes):
      // a per-lane 64-bit multiply-add here reads an undefined upper half
      // that the compiler may place in an activation load's register, and
      // then waits for that load
      const uint32_t run = __builtin_amdgcn_readfirstlane(
          2u * ((uint32_t)N * ((1u << B) - 2u) + (uint32_t)n0 * (1u << B)));
#pragma unroll
      for (int k = 0; k < kSlots; ++k) {
        const int e = k * kLThreads + tid;
        const uint32_t off = (used && e < kChunks) ? run + 16u * (uint32_t)e : kLOutOfRange;
        v[k] = __builtin_amdgcn_raw_buffer_load_b128(lrs, (int)off, 0, 0);
      }
    };
    auto store_w = [&](auto bw, const auto& v) {
      constexpr int B = decltype(bw)::value;
      constexpr int kChunks = 16 << B;
      constexpr int kSlots = sizeof(v) / sizeof(v[0]);
      constexpr int nb = 1 << B;
      if (a.toff[B] < 0) return;
      uint16_t* dst = s_lut + a.toff[B];
#pragma unroll
      for (int k = 0; k < kSlots; ++k) {
        const int e = k * kLThreads + tid;
        if (e < kChunks) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int h = 8 * e + 2 * q;                   // half of the run
            *reinterpret_cast<uint32_t*>(dst + lut_at(h >> B, h & (nb - 1), nb + 2)) = v[k][q];
          }
        }
      }
    };
    load_w(std::integral_constant<int, 8>(), c8);
    load_w(std::integral_constant<int, 7>(), c7);
    load_w(std::integral_constant<int, 6>(), c6);
    load_w(std::integral_constant<int, 5>(), c5);
    load_w(std::integral_constant<int, 4>(), c4);
    load_w(std::integral_constant<int, 3>(), c3);
    load_w(std::integral_constant<int, 2>(), c2);
    load_w(std::integral_constant<int, 1>(), c1);
    // compiler barrier: otherwise the loads of a width sink into the branch
    // that stores them and are issued only after the earlier widths' stores
    // (one more memory latency)
    asm volatile("" ::: "memory");
    store_w(std::integral_constant<int, 8>(), c8);
    store_w(std::integral_constant<int, 7>(), c7);
    store_w(std::integral_constant<int, 6>(), c6);
    store_w(std::integral_constant<int, 5>(), c5);
    store_w(std::integral_constant<int, 4>(), c4);
    store_w(std::integral_constant<int, 3>(), c3);
    store_w(std::integral_constant<int, 2>(), c2);
    store_w(std::integral_constant<int, 1>(), c1);
  }
  // ---- activations and widths of this workgroup's rows; the active rows
  // are listed by width: width b's rows fill entries 32 ub[b] .. of the list
  // (in no particular order), padded with 0xFFFF up to 32 ub[b + 1], so that
  // every run of 32 entries (a "unit") holds rows of one width
  const AssignRegs ar = load_assign_regs(a.ap);
  __syncthreads();                 // counters cleared
  // widths of this thread's rows (0 past the range), kept in registers
  uint32_t bk[kLRowIters];
#pragma unroll
  for (int k = 0; k < kLRowIters; ++k) {
    const int r = tid + k * kLThreads;
    bk[k] = 0;
    if (r < nrows) {
      bk[k] = bits_of(xpre[k], ar);
      s_xv[r] = xpre[k];
    }
  }
  // count the rows of each width, then each wave takes the units' starts
  // from the counts (no per-row widths in LDS: that space would keep the
  // largest tables from fitting two workgroups per CU)
#pragma unroll
  for (int k = 0; k < kLRowIters; ++k)
    if (bk[k] > 0) atomicAdd(&s_cnt[bk[k]], 1);
  __syncthreads();
  int ub[10];                      // first unit of each width (wave-uniform)
  {
    int u = 0;
#pragma unroll
    for (int v = 1; v <= 8; ++v) {
      ub[v] = u;
      u += (__builtin_amdgcn_readfirstlane(s_cnt[v]) + 31) >> 5;
    }
    ub[9] = u;
  }
  // place every row of non-zero width in its width's run
#pragma unroll
  for (int k = 0; k < kLRowIters; ++k) {
    const uint32_t b = bk[k];
    if (b > 0) {
      int first = 0;
#pragma unroll
      for (int v = 1; v <= 8; ++v) first = b == (uint32_t)v ? ub[v] : first;
      s_act[32 * first + atomicAdd(&s_cur[b], 1)] = (uint16_t)(tid + k * kLThreads);
    }
  }
  // pad each width's run to whole units: wave w pads width w + 1
  static_assert(kLWaves >= 8, "one wave per width");
#pragma unroll
  for (int v = 1; v <= 8; ++v) {
    if (wid + 1 != v) continue;
    const int e = __builtin_amdgcn_readfirstlane(s_cnt[v]) + lane;
    if (lane < 32 && e < 32 * (ub[v + 1] - ub[v])) s_act[32 * ub[v] + e] = 0xFFFFu;
  }
  __syncthreads();
  const int units = ub[9];

  // ---- units: lane = (row pair ps, word wl); a wave takes units wid,
  // wid + 8, ...; all 32 rows of a unit have one width, so the rebuild and
  // the table strides are specialised for it
  const int wl = tid & (kLWords - 1);
  const int ps = lane >> 2;        // row pair of the unit: entries 2 ps, 2 ps + 1
  // buffer over this workgroup's row tiles: row r at r rstride, plane p at
  // scalar offset p pb, this lane's word at 4 (word0 + wl)
  const uint32_t rstride = (uint32_t)(pb * bmax);
  const __amdgpu_buffer_rsrc_t prs =
      lut_rsrc(planesp + store_offset(t0 * K + k0 * ct, bmax), (int64_t)(nrows > 0 ? nrows : 1) * rstride);
  const uint32_t woff = 4u * (uint32_t)(word0 + wl);
  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.0f;

  // plane words of the lane's two rows in unit u, the unit's width and the
  // rows' activations as an fp16 pair.  A unit issues 8 loads (planes 0..3)
  // or, above width 4, 16; within those, planes past the width, padding rows
  // and units past the end use an out-of-range offset (reads 0, moves no
  // bytes), so the loads take at most one branch and the next unit's loads
  // stay in flight while one is processed.
  struct Unit {
    uint32_t w1[8], w2[8];
    uint32_t xw;
    int b;
  };
  auto load_unit = [&](int u, Unit& t) {
    int b = 0;
#pragma unroll
    for (int v = 1; v <= 8; ++v) b = (u >= ub[v] && u < ub[v + 1]) ? v : b;
    t.b = b;
    const int uu = u < units ? u : 0;
    const uint32_t e1 = b > 0 ? s_act[32 * uu + 2 * ps] : 0xFFFFu;
    const uint32_t e2 = b > 0 ? s_act[32 * uu + 2 * ps + 1] : 0xFFFFu;
    const uint32_t x1 = e1 != 0xFFFFu ? s_xv[e1] : 0u;
    const uint32_t x2 = e2 != 0xFFFFu ? s_xv[e2] : 0u;
    t.xw = x1 | (x2 << 16);
    const uint32_t v1 = e1 != 0xFFFFu ? e1 * rstride + woff : kLOutOfRange;
    const uint32_t v2 = e2 != 0xFFFFu ? e2 * rstride + woff : kLOutOfRange;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      t.w1[p] = __builtin_amdgcn_raw_buffer_load_b32(prs, (int)(p < b ? v1 : kLOutOfRange), p < bmax ? p * pb : 0, 0);
      t.w2[p] = __builtin_amdgcn_raw_buffer_load_b32(prs, (int)(p < b ? v2 : kLOutOfRange), p < bmax ? p * pb : 0, 0);
    }
    if (b > 4) {   // planes 4..7 only for the wide units (fewer memory instructions)
#pragma unroll
      for (int p = 4; p < 8; ++p) {
        t.w1[p] = __builtin_amdgcn_raw_buffer_load_b32(prs, (int)(p < b ? v1 : kLOutOfRange), p < bmax ? p * pb : 0, 0);
        t.w2[p] = __builtin_amdgcn_raw_buffer_load_b32(prs, (int)(p < b ? v2 : kLOutOfRange), p < bmax ? p * pb : 0, 0);
      }
    }
  };
  // one unit of width B: rebuild the two rows' codes, look both weights of
  // each column up (table index = the code's top B bits), and add
  // x1 w1 + x2 w2 with one fp16 dot into the column's fp32 accumulator
  auto process = [&](const Unit& t, auto bw, uint32_t (&wv)[32]) {
    constexpr int B = decltype(bw)::value;
    constexpr int kStride = (1 << B) + 2;                // halves per column table in LDS
    uint32_t d1[8], d2[8];
    planes_to_codes<B>(t.w1, d1);                        // plane p at code bit 7 - p
    planes_to_codes<B>(t.w2, d2);
    const char* tb = reinterpret_cast<const char*>(s_lut + a.toff[B] + lut_at(32 * wl, 0, kStride));
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 4 * m + j;                         // column within the word
        // byte offset 2 p of table entry p: bits 7 - B .. 7 of the code byte
        // (bit 7 - B is zero after the rebuild)
        uint32_t o1, o2;
        if constexpr (B < 8) {
          o1 = __builtin_amdgcn_ubfe(d1[m], 8u * j + 7u - B, B + 1u);
          o2 = __builtin_amdgcn_ubfe(d2[m], 8u * j + 7u - B, B + 1u);
        } else {
          o1 = __builtin_amdgcn_ubfe(d1[m], 8u * j, 8u) << 1;
          o2 = __builtin_amdgcn_ubfe(d2[m], 8u * j, 8u) << 1;
        }
        const _Float16 lo = *reinterpret_cast<const _Float16*>(tb + 2 * c * kStride + o1);
        const _Float16 hi = *reinterpret_cast<const _Float16*>(tb + 2 * c * kStride + o2);
        wv[c] = __builtin_bit_cast(uint32_t, (half2_t){lo, hi});
      }
    }
  };
  // the width-specialised part only produces the weight pairs; the dots
  // into the accumulators are one piece of code after the switch (inside
  // every case they made the compiler copy each accumulator per dot)
  auto process_rt = [&](const Unit& t) {
    uint32_t wv[32];
    switch (t.b) {
      case 1: process(t, std::integral_constant<int, 1>(), wv); break;
      case 2: process(t, std::integral_constant<int, 2>(), wv); break;
      case 3: process(t, std::integral_constant<int, 3>(), wv); break;
      case 4: process(t, std::integral_constant<int, 4>(), wv); break;
      case 5: process(t, std::integral_constant<int, 5>(), wv); break;
      case 6: process(t, std::integral_constant<int, 6>(), wv); break;
      case 7: process(t, std::integral_constant<int, 7>(), wv); break;
      case 8: process(t, std::integral_constant<int, 8>(), wv); break;
      default: return;
    }
    const half2_t xh = __builtin_bit_cast(half2_t, t.xw);
#pragma unroll
    for (int c = 0; c < 32; ++c) acc[c] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, wv[c]), xh, acc[c], false);
  };


  // two register sets in turn (no copies between them: a register copy of
  // a loaded value would wait for the load), the next unit always in flight
  Unit tA, tB;
  load_unit(wid, tA);
  for (int u = wid; u < units; u += 2 * kLWaves) {
    load_unit(u + kLWaves, tB);                          // past the end: nothing moves
    process_rt(tA);
    load_unit(u + 2 * kLWaves, tA);
    process_rt(tB);
  }

  // ---- reduce over the lanes that share a word (lane bits 2..5), in
  // registers: a lane-half swap sums accumulator pairs (2q, 2q + 1) over
  // bit 5, a row swap sums those pairs over bit 4, and two rotations inside
  // each 16-lane row sum over bits 3 and 2.  Value r then holds, in row rho
  // (lanes 16 rho ..), column 4 r + {0, 2, 1, 3}[rho] of word lane & 3;
  // lanes 0..3 of each row write it, then the waves are reduced in LDS
  float h32[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) h32[q] = lut_halves_sum(acc[2 * q], acc[2 * q + 1]);
  float r16[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float v = lut_rows_sum(h32[2 * r], h32[2 * r + 1]);
    v += lut_row_ror<8>(v);
    v += lut_row_ror<4>(v);
    r16[r] = v;
  }
  __syncthreads();                 // every wave is done with the tables
  if ((lane & 15) < kLWords) {
    const int rho = lane >> 4;
    const int cofs = ((rho & 1) << 1) | (rho >> 1);
    float* dst = s_red + wid * kLCols + 32 * (lane & 3) + cofs;
#pragma unroll
    for (int r = 0; r < 8; ++r) dst[4 * r] = r16[r];
  }
  __syncthreads();
  if (tid < kLCols) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kLWaves; ++w) v += s_red[w * kLCols + tid];
    const int64_t n = n0 + tid;
    if (n < N) {
      if (nrows > 0) __hip_atomic_fetch_add(a.y + n, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // device scope: written through, no dirty line left for the kernel's end
      if (a.clear && split == 0) __hip_atomic_store(a.clear + n, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

int launch_vmm_lut(const uint8_t* planes, const uint16_t* lut, const uint16_t* x, int64_t K, int64_t N,
                   int bmax, const AssignParams& ap, float* y, float* clear, hipStream_t s) {
  if (reinterpret_cast<uintptr_t>(lut) % 4 != 0)
    return fail(GRINQH_EINVAL, "grinqh_decode_vmm_lut: the table buffer must be 4-byte aligned");
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
  const int64_t lut_bytes = N * ((int64_t(1) << (bmax + 1)) - 2) * 2;
  if (lut_bytes >= (int64_t(1) << 31))
    return fail(GRINQH_EINVAL, "grinqh_decode_vmm_lut: tables of %lld bytes (at most 2^31 - 1)", (long long)lut_bytes);
  a.lut_bytes = (int)lut_bytes;
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
  a.splits = (int)splits;
  const int64_t wgs = (a.n_ct + kLSlices - 1) / kLSlices * kLSlices * splits;
  if (wgs > 0x7FFFFFFF)
    return fail(GRINQH_EINVAL, "%lld workgroups: more than one launch handles", (long long)wgs);
  const int smem = lut_smem_bytes(a);
  if (smem > kLMaxDynLds)
    return fail(GRINQH_EINVAL, "grinqh_decode_vmm_lut: %d bytes of LDS needed (tables of the levels in use and "
                               "%d rows), at most %d", smem, a.rows, kLMaxDynLds);
  // the kernel may take more than the default dynamic LDS: raised once per
  // device (idempotent, so two threads racing to do it is harmless)
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(GRINQH_EDEVICE, "grinqh_decode_vmm_lut: no device");
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (!(attr_done.load(std::memory_order_acquire) & bit)) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(vmm_lut_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLMaxDynLds);
    if (e != hipSuccess) return fail(GRINQH_EDEVICE, "grinqh_decode_vmm_lut: %s", hipGetErrorString(e));
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  int used_mask = 0;
  for (int b = 1; b <= 8; ++b) used_mask |= a.toff[b] >= 0 ? 1 << b : 0;
  hipLaunchKernelGGL(vmm_lut_kernel, dim3((unsigned)wgs), dim3(kLThreads), smem, s, a.x, a.lut, a.planes, (int)K,
                     (int)N, a.rows, a.splits, a.n_ct, a.lut_bytes, used_mask, bmax, a);
  return check_launch("grinqh_decode_vmm_lut");
}

}  // namespace grinqh
