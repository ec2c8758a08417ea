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
  float th[kMaxThresholds];
  uint32_t lv[kMaxThresholds + 1];   // 32-bit so the kernel reads them with scalar loads
  int n;
};

__host__ __device__ inline int64_t padded_cols(int64_t N) { return (N + 127) / 128 * 128; }
__host__ __device__ inline int64_t n_tiles(int64_t N) { return (padded_cols(N) + kTile - 1) / kTile; }
__host__ __device__ inline int64_t n_groups(int64_t K) { return (K + kGroup - 1) / kGroup; }

__device__ inline float half_bits_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Level index for one activation: number of thresholds |x| reaches (fp32).
__device__ inline int level_of(uint16_t xh, const AssignParams& ap) {
  const float ax = __builtin_fabsf(half_bits_to_float(xh));
  int k = 0;
#pragma unroll
  for (int t = 0; t < kMaxThresholds; ++t) k += (t < ap.n && ax >= ap.th[t]) ? 1 : 0;
  return k;
}

// b_i = levels[k] with compile-time indices only (thresholds are non-decreasing,
// so k thresholds reached means the first k).
__device__ inline uint32_t level_bits(int k, const AssignParams& ap) {
  uint32_t b = ap.lv[0];
#pragma unroll
  for (int t = 1; t <= kMaxThresholds; ++t) b = (k >= t) ? (uint32_t)ap.lv[t] : b;
  return b;
}

// Thresholds and levels held in wave-uniform registers (read once per kernel).
struct AssignRegs {
  float th[kMaxThresholds];
  uint32_t lv[kMaxThresholds + 1];
  int n;
};

__device__ inline AssignRegs load_assign_regs(const AssignParams& ap) {
  AssignRegs r;
#pragma unroll
  for (int t = 0; t < kMaxThresholds; ++t)
    r.th[t] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, ap.th[t])));
#pragma unroll
  for (int t = 0; t <= kMaxThresholds; ++t) r.lv[t] = __builtin_amdgcn_readfirstlane(ap.lv[t]);
  r.n = __builtin_amdgcn_readfirstlane(ap.n);
  return r;
}

// b = levels[#thresholds reached]; with non-decreasing thresholds the reached
// ones are a prefix, so the last one reached names the level.
__device__ inline uint32_t bits_of(uint16_t xh, const AssignRegs& r) {
  const float ax = __builtin_fabsf(half_bits_to_float(xh));
  uint32_t b = r.lv[0];
#pragma unroll
  for (int t = 0; t < kMaxThresholds; ++t) b = (t < r.n && ax >= r.th[t]) ? r.lv[t + 1] : b;
  return b;
}

// Host-side status plumbing (api.hip).
int fail(int status, const char* fmt, ...);
int check_launch(const char* what);

// Workspace geometry used by the VMM kernels and grinqh_workspace_bytes.
struct VmmGeometry {
  int64_t rows_per_split;  // K rows handled by one workgroup
  int64_t splits;          // ceil(K / rows_per_split)
  int64_t tiles;           // column tiles
  int64_t partial_floats;  // splits * N_pad when splits > 1, else 0
  int64_t counter_offset;  // byte offset of the per-tile counters
  int64_t bytes;           // total workspace bytes
};
VmmGeometry vmm_geometry(int64_t K, int64_t N);

// Launchers (one per .hip file).
int launch_pack(const uint8_t* codes, int64_t K, int64_t N, uint8_t* planes, hipStream_t s);
int launch_calibrate(const uint16_t* calib, int64_t V, int64_t K, const double* cuts, int n,
                     float* thresholds, hipStream_t s);
int launch_assign(const uint16_t* x, int64_t K, const AssignParams& ap, uint8_t* bits,
                  int32_t* active_idx, int32_t* n_active, hipStream_t s);
int launch_vmm_list(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                    const uint16_t* x, const uint8_t* bits, const int32_t* active_idx,
                    const int32_t* n_active, int64_t K, int64_t N, float* y, void* ws,
                    hipStream_t s);
int launch_vmm_fused(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                     const uint16_t* x, int64_t K, int64_t N, const AssignParams& ap, float* y,
                     void* ws, hipStream_t s);
int launch_vmm_accumulate(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                          const uint16_t* x, int64_t K, int64_t N, const AssignParams& ap, float* y,
                          float* clear, hipStream_t s);
int launch_fill_zero(void* ptr, size_t bytes, hipStream_t s);

}  // namespace grinqh
