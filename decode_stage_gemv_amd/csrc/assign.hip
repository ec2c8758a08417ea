// Dynamic precision assignment and active-row selection (GRINQH paper,
// section 3.1 "Dynamic Precision Assignment").
//
// One workgroup of 1024 threads walks x in chunks of 16 Ki elements; each
// thread owns 16 consecutive rows of a chunk, so a block-wide exclusive scan of
// per-thread counts gives every active row its ascending slot directly.
#include "common.hpp"

namespace grinqh {

// Inclusive prefix sum over the 64 lanes without LDS traffic: shifts by 1,
// 2, 4, 8 lanes inside each 16-lane row (lanes shifted in from outside the
// row read 0), then each row adds the totals of the rows below it.
__device__ inline int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  const int lane = threadIdx.x & 63;
  const int t0 = __builtin_amdgcn_readlane(v, 15);   // row totals
  const int t1 = __builtin_amdgcn_readlane(v, 31);
  const int t2 = __builtin_amdgcn_readlane(v, 47);
  v += lane >= 16 ? t0 : 0;
  v += lane >= 32 ? t1 : 0;
  v += lane >= 48 ? t2 : 0;
  return v;
}

constexpr int kAssignThreads = 1024;
constexpr int kAssignPerThread = 16;

__global__ __launch_bounds__(kAssignThreads) void assign_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                                AssignParams ap, uint8_t* __restrict__ bits,
                                                                int32_t* __restrict__ active_idx,
                                                                int32_t* __restrict__ n_active) {
  __shared__ int wave_tot[kAssignThreads / 64];
  const AssignRegs ar = load_assign_regs(ap);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  int base = 0;
  for (int64_t c0 = 0; c0 < K; c0 += (int64_t)kAssignThreads * kAssignPerThread) {
    const int64_t e0 = c0 + (int64_t)tid * kAssignPerThread;
    uint32_t b[kAssignPerThread];
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < kAssignPerThread; ++e) {
      const int64_t i = e0 + e;
      b[e] = 0;
      if (i < K) b[e] = bits_of(x[i], ar);
      cnt += b[e] > 0 ? 1 : 0;
    }
#pragma unroll
    for (int e = 0; e < kAssignPerThread; ++e) {
      const int64_t i = e0 + e;
      if (i < K) bits[i] = (uint8_t)b[e];
    }
    const int incl = wave_inclusive_sum(cnt);
    if (lane == 63) wave_tot[wid] = incl;
    __syncthreads();
    int before = 0, chunk_total = 0;
#pragma unroll
    for (int w = 0; w < kAssignThreads / 64; ++w) {
      const int v = wave_tot[w];
      before += w < wid ? v : 0;
      chunk_total += v;
    }
    int pos = base + before + incl - cnt;
#pragma unroll
    for (int e = 0; e < kAssignPerThread; ++e) {
      if (b[e] > 0) active_idx[pos++] = (int32_t)(e0 + e);
    }
    base += chunk_total;
    __syncthreads();
  }
  if (tid == 0) *n_active = base;
}

int launch_assign(const uint16_t* x, int64_t K, const AssignParams& ap, uint8_t* bits,
                  int32_t* active_idx, int32_t* n_active, hipStream_t s) {
  hipLaunchKernelGGL(assign_kernel, dim3(1), dim3(kAssignThreads), 0, s, x, K, ap, bits, active_idx, n_active);
  return check_launch("grinqh_assign_bits");
}

}  // namespace grinqh
