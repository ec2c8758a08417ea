// Internal helpers shared by the GRINQH HIP sources (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grinqh.h"

namespace grinqh {

constexpr int kGroup = GRINQH_GROUP;
constexpr int kTile = GRINQH_TILE;
constexpr int kWordsPerTile = kTile / 32;
constexpr int kMaxThresholds = GRINQH_MAX_THRESHOLDS;

// Thresholds and levels travel as a kernel argument (a few SGPR loads).
struct AssignParams {
  float th[kMaxThresholds];          // slots past n: +inf
  uint32_t lv[kMaxThresholds + 1];   // slots past n: levels[n]; 32-bit for scalar loads
  int n;
};

__host__ __device__ inline int64_t padded_cols(int64_t N) { return (N + 127) / 128 * 128; }
__host__ __device__ inline int64_t n_tiles(int64_t N) { return (padded_cols(N) + kTile - 1) / kTile; }
__host__ __device__ inline int64_t n_groups(int64_t K) { return (K + kGroup - 1) / kGroup; }
// Byte offset in a b_max-bit store of a position that an 8-plane store has at
// `off8` (row tile starts: every row tile is b_max / 8 as long).  off8 is a
// multiple of 128 there, so the result is exact.
__host__ __device__ inline int64_t store_offset(int64_t off8, int bmax) { return off8 / 8 * bmax; }

__device__ inline float half_bits_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Thresholds and level steps held in wave-uniform registers (read once per
// kernel): step[t] = levels[t + 1] - levels[t].
struct AssignRegs {
  float th[kMaxThresholds];
  int step[kMaxThresholds];
  int lv0;
  uint32_t lvb[2];   // levels[0..7], one per byte
  uint32_t lv8;      // levels[8]
  int n;             // thresholds in use
};

__device__ inline AssignRegs load_assign_regs(const AssignParams& ap) {
  AssignRegs r;
#pragma unroll
  for (int t = 0; t < kMaxThresholds; ++t) {
    r.th[t] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, ap.th[t])));
    r.step[t] = __builtin_amdgcn_readfirstlane((int)ap.lv[t + 1] - (int)ap.lv[t]);
  }
  r.lv0 = __builtin_amdgcn_readfirstlane((int)ap.lv[0]);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    r.lvb[h] = __builtin_amdgcn_readfirstlane(ap.lv[4 * h] | (ap.lv[4 * h + 1] << 8) | (ap.lv[4 * h + 2] << 16) |
                                              (ap.lv[4 * h + 3] << 24));
  r.lv8 = __builtin_amdgcn_readfirstlane(ap.lv[kMaxThresholds]);
  r.n = __builtin_amdgcn_readfirstlane(ap.n);
  return r;
}

// b = levels[#thresholds reached] for two rows at once (the thresholds do
// not decrease, so the reached ones are a prefix).  Only the n thresholds in
// use are compared, behind a wave-uniform test: past them every slot holds
// +inf, which only |x| = +inf reaches, and levels[c] = levels[n] for every
// such count c anyway.  The level is one byte select from the packed level
// table.  (The assignment kernel's width_of adds the level steps of the
// reached thresholds instead, over the first NT slots only.)
__device__ inline void bits_of2(uint16_t xh0, uint16_t xh1, const AssignRegs& r, uint32_t& b0, uint32_t& b1) {
  const float a0 = __builtin_fabsf(half_bits_to_float(xh0));
  const float a1 = __builtin_fabsf(half_bits_to_float(xh1));
  uint32_t c0 = 0, c1 = 0;
#pragma unroll
  for (int t = 0; t < kMaxThresholds; ++t) {
    if (t < r.n) {   // wave-uniform
      c0 += a0 >= r.th[t] ? 1u : 0u;
      c1 += a1 >= r.th[t] ? 1u : 0u;
    }
  }
  // levels[c]: byte c of the packed table (selectors 0..3 pick the second
  // operand's bytes, 4..7 the first's), levels[8] past it
  const uint32_t l0 = __builtin_amdgcn_perm(r.lvb[1], r.lvb[0], c0) & 0xFFu;
  const uint32_t l1 = __builtin_amdgcn_perm(r.lvb[1], r.lvb[0], c1) & 0xFFu;
  b0 = c0 < kMaxThresholds ? l0 : r.lv8;
  b1 = c1 < kMaxThresholds ? l1 : r.lv8;
}

// The same for one row.
__device__ inline uint32_t bits_of(uint16_t xh, const AssignRegs& r) {
  const float ax = __builtin_fabsf(half_bits_to_float(xh));
  uint32_t c = 0;
#pragma unroll
  for (int t = 0; t < kMaxThresholds; ++t) {
    if (t < r.n) c += ax >= r.th[t] ? 1u : 0u;   // wave-uniform test
  }
  const uint32_t b = __builtin_amdgcn_perm(r.lvb[1], r.lvb[0], c) & 0xFFu;
  return c < kMaxThresholds ? b : r.lv8;
}

// Host-side status plumbing and argument checks (api.hip).
int fail(int status, const char* fmt, ...);
int check_launch(const char* what);
void clear_error();
int check_layer(const void* planes, const void* scales, const void* zeros, const void* x, const void* y,
                int64_t K, int64_t N, int b_max);
int check_assign_params(const float* thresholds, const uint8_t* levels, int n, int max_level, AssignParams* ap);

// Workspace geometry used by the VMM kernels and grinqh_workspace_bytes.
struct VmmGeometry {
  int64_t rows_per_split;  // K rows of one sub-item (64 or 128)
  int64_t subs;            // sub-items per workgroup (1, 2, 4 or 8)
  int64_t waves;           // waves per workgroup (8 or 16)
  int64_t splits;          // ceil(K / (rows_per_split subs)): items along K
  int64_t tiles;           // column tiles
  int64_t partial_floats;  // splits * N_pad when splits > 1, else 0
  int64_t counter_offset;  // byte offset of the per-tile counters
  int64_t words_offset;    // byte offset of the column words (2 N_pad of 8 bytes)
  int64_t bytes;           // total workspace bytes
};
VmmGeometry vmm_geometry(int64_t K, int64_t N);

// One member of a grouped launch: an independent decode step with its own
// store, activation, thresholds and output, sharing K and b_max with the
// other members; `first` is its first workgroup in the grid.
struct VmmMember {
  const uint8_t* planes;
  const uint16_t* scales;
  const uint16_t* zeros;
  const uint16_t* x;
  float* y;
  float* clear;
  int N, tiles, first;
  AssignParams ap;
};

struct VmmGroup {
  int count;
  VmmMember m[GRINQH_MAX_GROUP];
};

// A grouped accumulating launch (members filled in except tiles and first).
int launch_vmm_group(int count, VmmMember* members, int64_t K, int bmax, hipStream_t s);

// Launchers (one per .hip file).
int launch_pack(const uint8_t* codes, int64_t K, int64_t N, int bmax, uint8_t* planes, hipStream_t s);
int launch_calibrate(const uint16_t* calib, int64_t V, int64_t K, const double* cuts, int n,
                     float* thresholds, hipStream_t s);
int launch_assign(const uint16_t* x, int64_t K, const AssignParams& ap, uint8_t* bits,
                  int32_t* active_idx, int32_t* n_active, hipStream_t s);
int launch_vmm_list(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                    const uint16_t* x, const uint8_t* bits, const int32_t* active_idx,
                    const int32_t* n_active, int64_t K, int64_t N, int bmax, float* y, void* ws,
                    hipStream_t s);
int launch_vmm_fused(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                     const uint16_t* x, int64_t K, int64_t N, int bmax, const AssignParams& ap,
                     float* y, void* ws, hipStream_t s);
// The fused split-K VMM with the partial rows and tile counters given apart
// (the allocation-free entry point keeps them in a fixed device array).
int launch_vmm_fused_split(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                           const uint16_t* x, int64_t K, int64_t N, int bmax, const AssignParams& ap,
                           float* y, float* partials, unsigned* counters, unsigned long long* words,
                           int64_t max_cols, hipStream_t s);
int noalloc_scratch(int64_t partial_bytes, int64_t tiles, int64_t cols, float** partials, unsigned** counters,
                    unsigned long long** words, int64_t* max_cols);
int launch_vmm_accumulate(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                          const uint16_t* x, int64_t K, int64_t N, int bmax, const AssignParams& ap,
                          float* y, float* clear, hipStream_t s);
int launch_prefill(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros, const uint16_t* X,
                   int64_t M, int64_t K, int64_t N, int bmax, float* Y, hipStream_t s);
int launch_vmm_lut(const uint8_t* planes, const uint16_t* lut, const uint16_t* x, int64_t K, int64_t N,
                   int bmax, const AssignParams& ap, float* y, float* clear, hipStream_t s);
// rows of the unpacked dense weights: K padded to a multiple of 64 (one
// K-step of the dense GEMM) so that the GEMM's loads need no bounds checks
__host__ __device__ inline int64_t dense_rows(int64_t K) { return (K + 63) / 64 * 64; }
int64_t unpack_dense_bytes(int64_t K, int64_t N);
int launch_unpack_dense(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros, int64_t K,
                        int64_t N, int bmax, void* out, hipStream_t s);
int launch_dense_gemm(const uint16_t* X, const void* W, int64_t M, int64_t K, int64_t N, float* Y, hipStream_t s);
int launch_fill_zero(void* ptr, size_t bytes, hipStream_t s);

}  // namespace grinqh
