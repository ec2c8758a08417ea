// Offline threshold calibration by percentile mapping (GRINQH paper, section
// 3.2 "Threshold Calibration"; Appendix A.1 eq. (2)).
//
// theta_k = mean over calibration vectors v of Q(|v|, c_k), Q the linear-
// interpolation quantile at position c_k (K - 1).  Order statistics come from
// a two-pass radix select on the 15-bit magnitude of each fp16 value (for
// non-negative fp16 the bit pattern orders like the value), so they are exact.
// One workgroup per threshold walks the vectors in order and accumulates the
// mean in fp64, so the result does not depend on the launch shape.
#include <math.h>

#include "common.hpp"

namespace grinqh {

constexpr int kCalThreads = 256;

struct CutParams {
  double c[kMaxThresholds];
};

// Inclusive block scan of one value per thread (256 threads, 4 waves).
__device__ inline int64_t block_inclusive_scan(int64_t v, int64_t* wave_sums) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) wave_sums[wid] = v;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wid; ++w) before += wave_sums[w];
  __syncthreads();
  return v + before;
}

// Rank r (0-based) order statistic of the magnitudes of v[0..K).
__device__ uint16_t select_rank(const uint16_t* __restrict__ v, int64_t K, int64_t r,
                                unsigned* hist, int64_t* wave_sums, int* s_bin, int64_t* s_rem) {
  int prefix_hi = -1;  // high byte once known
  for (int pass = 0; pass < 2; ++pass) {
    hist[threadIdx.x] = 0;
    __syncthreads();
    for (int64_t k = threadIdx.x; k < K; k += kCalThreads) {
      const uint32_t key = v[k] & 0x7FFFu;
      if (pass == 0) {
        atomicAdd(&hist[key >> 8], 1u);
      } else if ((int)(key >> 8) == prefix_hi) {
        atomicAdd(&hist[key & 0xFFu], 1u);
      }
    }
    __syncthreads();
    const int64_t cnt = hist[threadIdx.x];
    const int64_t incl = block_inclusive_scan(cnt, wave_sums);
    const int64_t excl = incl - cnt;
    if (cnt > 0 && excl <= r && r < incl) {
      *s_bin = threadIdx.x;
      *s_rem = r - excl;
    }
    __syncthreads();
    if (pass == 0) prefix_hi = *s_bin;
    r = *s_rem;
    __syncthreads();
  }
  return (uint16_t)((prefix_hi << 8) | *s_bin);
}

__global__ __launch_bounds__(kCalThreads) void calibrate_kernel(const uint16_t* __restrict__ calib,
                                                                int64_t V, int64_t K, CutParams cp,
                                                                float* __restrict__ thresholds) {
#pragma clang fp contract(off)
  __shared__ unsigned hist[256];
  __shared__ int64_t wave_sums[4];
  __shared__ int s_bin;
  __shared__ int64_t s_rem;
  const int k = blockIdx.x;
  const double c = cp.c[k];
  if (c <= 0.0 || c >= 1.0) {
    if (threadIdx.x == 0) thresholds[k] = c <= 0.0 ? 0.0f : __builtin_inff();
    return;
  }
  const double h = c * (double)(K - 1);
  int64_t lo = (int64_t)floor(h);
  if (lo < 0) lo = 0;
  if (lo > K - 1) lo = K - 1;
  const int64_t hi = lo + 1 < K ? lo + 1 : K - 1;
  const double frac = h - (double)lo;
  double total = 0.0;
  for (int64_t vi = 0; vi < V; ++vi) {
    const uint16_t* vec = calib + vi * K;
    const uint16_t klo = select_rank(vec, K, lo, hist, wave_sums, &s_bin, &s_rem);
    const uint16_t khi = hi == lo ? klo : select_rank(vec, K, hi, hist, wave_sums, &s_bin, &s_rem);
    const double a_lo = (double)half_bits_to_float(klo);
    const double a_hi = (double)half_bits_to_float(khi);
    const double diff = a_hi - a_lo;
    const double step = frac * diff;
    const double q = a_lo + step;
    total = total + q;
  }
  if (threadIdx.x == 0) thresholds[k] = (float)(total / (double)V);
}

int launch_calibrate(const uint16_t* calib, int64_t V, int64_t K, const double* cuts, int n,
                     float* thresholds, hipStream_t s) {
  CutParams cp;
  for (int k = 0; k < kMaxThresholds; ++k) cp.c[k] = k < n ? cuts[k] : 0.0;
  hipLaunchKernelGGL(calibrate_kernel, dim3(n), dim3(kCalThreads), 0, s, calib, V, K, cp, thresholds);
  return check_launch("grinqh_calibrate");
}

}  // namespace grinqh
