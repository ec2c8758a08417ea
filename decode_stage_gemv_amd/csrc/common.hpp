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
};

__device__ inline AssignRegs load_assign_regs(const AssignParams& ap) {
  AssignRegs r;
#pragma unroll
  for (int t = 0; t < kMaxThresholds; ++t) {
    r.th[t] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, ap.th[t])));
    r.step[t] = __builtin_amdgcn_readfirstlane((int)ap.lv[t + 1] - (int)ap.lv[t]);
  }
  r.lv0 = __builtin_amdgcn_readfirstlane((int)ap.lv[0]);
  return r;
}

// b = levels[#thresholds reached].  With non-decreasing thresholds the
// reached ones are a prefix, so b = levels[0] plus the steps of the reached
// thresholds (a sum, so no table lookup).  Slots past n hold +inf and a zero
// step (set by the host), so all slots are compared.
__device__ inline uint32_t bits_of(uint16_t xh, const AssignRegs& r) {
  const float ax = __builtin_fabsf(half_bits_to_float(xh));
  int b = r.lv0;
#pragma unroll
  for (int t = 0; t < kMaxThresholds; ++t) b += ax >= r.th[t] ? r.step[t] : 0;
  return (uint32_t)b;
}

// Host-side status plumbing (api.hip).
int fail(int status, const char* fmt, ...);
int check_launch(const char* what);

// Workspace geometry used by the VMM kernels and grinqh_workspace_bytes.
struct VmmGeometry {
  int64_t rows_per_split;  // K rows handled by one workgroup (64 or 128)
  int64_t waves;           // waves per workgroup (4 or 8)
  int64_t splits;          // ceil(K / rows_per_split)
  int64_t tiles;           // column tiles
  int64_t partial_floats;  // splits * N_pad when splits > 1, else 0
  int64_t counter_offset;  // byte offset of the per-tile counters
  int64_t bytes;           // total workspace bytes
};
VmmGeometry vmm_geometry(int64_t K, int64_t N);

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
