// Dynamic precision assignment and active-row selection (GRINQH paper,
// section 3.1 "Dynamic Precision Assignment").
//
// One workgroup of 1024 threads.  Rows are read in passes of 4096: thread t
// owns rows 4t .. 4t + 3 of a pass (one 8-byte load of four fp16 values, so a
// wave's load covers 512 contiguous bytes), and up to eight passes (32768
// rows) are loaded before any is used.  Each row's width is the level of the
// number of thresholds |x| reaches, compared in fp32 against exactly the n
// thresholds given (a kernel per n, so no compare is spent on unused slots).
// The ascending list position of an active row is
//   (active rows of earlier passes) + (of earlier threads in this pass)
//   + (of earlier rows of this thread),
// from one wave scan per pass (DPP row shifts) and one exchange of the wave
// totals of all passes through LDS, so a super-chunk of eight passes costs a
// single barrier.  Widths are stored as one 4-byte word per thread and pass.
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
constexpr int kAssignWaves = kAssignThreads / 64;
constexpr int kRowsPerThread = 4;
constexpr int kPassRows = kAssignThreads * kRowsPerThread;   // 4096
constexpr int kPasses = 8;                                   // passes per super-chunk
constexpr int64_t kChunkRows = (int64_t)kPassRows * kPasses;  // 32768

// Width of one row against the first NT thresholds (fp32 compare; NaN reaches
// none, +inf reaches all).
template <int NT>
__device__ inline uint32_t width_of(uint16_t xh, const AssignRegs& r) {
  const float ax = __builtin_fabsf(half_bits_to_float(xh));
  int b = r.lv0;
#pragma unroll
  for (int t = 0; t < NT; ++t) b += ax >= r.th[t] ? r.step[t] : 0;
  return (uint32_t)b;
}

// kAligned: x is 8-byte aligned, so four rows come in one 8-byte load.
template <int NT, bool kAligned>
__global__ __launch_bounds__(kAssignThreads) void assign_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                                AssignParams ap, uint8_t* __restrict__ bits,
                                                                int32_t* __restrict__ active_idx,
                                                                int32_t* __restrict__ n_active) {
  __shared__ int wave_tot[kPasses][kAssignWaves];
  const AssignRegs ar = load_assign_regs(ap);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  int base = 0;   // active rows before this super-chunk
  for (int64_t c0 = 0; c0 < K; c0 += kChunkRows) {
    // passes of this super-chunk that hold rows (uniform: no work for the rest)
    const int64_t left = (K - c0 + kPassRows - 1) / kPassRows;
    const int npass = left < kPasses ? (int)left : kPasses;
    // ---- loads of every pass first (rows past K read as 0 and are dropped)
    uint32_t xv[kPasses][2];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int64_t i0 = c0 + (int64_t)p * kPassRows + kRowsPerThread * tid;
      xv[p][0] = xv[p][1] = 0;
      if (p >= npass) continue;
      if (kAligned && i0 + kRowsPerThread <= K) {
        const uint2 q = *reinterpret_cast<const uint2*>(x + i0);
        xv[p][0] = q.x;
        xv[p][1] = q.y;
      } else {
#pragma unroll
        for (int e = 0; e < kRowsPerThread; ++e)
          if (i0 + e < K) xv[p][e >> 1] |= (uint32_t)x[i0 + e] << (16 * (e & 1));
      }
    }
    // ---- widths, per-thread counts, wave scans (one per pass)
    uint32_t wb[kPasses];   // the thread's four widths of a pass, one per byte
    int cnt[kPasses], incl[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int64_t i0 = c0 + (int64_t)p * kPassRows + kRowsPerThread * tid;
      wb[p] = 0;
      cnt[p] = 0;
      incl[p] = 0;
      if (p >= npass) continue;
#pragma unroll
      for (int e = 0; e < kRowsPerThread; ++e) {
        const uint32_t b = i0 + e < K ? width_of<NT>((uint16_t)(xv[p][e >> 1] >> (16 * (e & 1))), ar) : 0u;
        wb[p] |= b << (8 * e);
        cnt[p] += b > 0 ? 1 : 0;
      }
      incl[p] = wave_inclusive_sum(cnt[p]);
      if (lane == 63) wave_tot[p][wid] = incl[p];
    }
    __syncthreads();
    // ---- positions: earlier passes, then earlier waves of this pass, then
    // earlier threads of this wave
    int pass_base = base;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      if (p >= npass) break;
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kAssignWaves; ++w) {
        const int v = wave_tot[p][w];
        before += w < wid ? v : 0;
        total += v;
      }
      const int64_t i0 = c0 + (int64_t)p * kPassRows + kRowsPerThread * tid;
      if (kAligned && i0 + kRowsPerThread <= K) {
        *reinterpret_cast<uint32_t*>(bits + i0) = wb[p];
      } else {
#pragma unroll
        for (int e = 0; e < kRowsPerThread; ++e)
          if (i0 + e < K) bits[i0 + e] = (uint8_t)(wb[p] >> (8 * e));
      }
      int pos = pass_base + before + incl[p] - cnt[p];
#pragma unroll
      for (int e = 0; e < kRowsPerThread; ++e)
        if ((wb[p] >> (8 * e)) & 0xFFu) active_idx[pos++] = (int32_t)(i0 + e);
      pass_base += total;
    }
    base = pass_base;
    __syncthreads();   // wave_tot is reused by the next super-chunk
  }
  if (tid == 0) *n_active = base;
}

template <bool kAligned>
static void launch_n(int n, const uint16_t* x, int64_t K, const AssignParams& ap, uint8_t* bits,
                     int32_t* active_idx, int32_t* n_active, hipStream_t s) {
#define GRINQH_ASSIGN(NT)                                                                                      \
  hipLaunchKernelGGL((assign_kernel<NT, kAligned>), dim3(1), dim3(kAssignThreads), 0, s, x, K, ap, bits, \
                     active_idx, n_active)
  switch (n) {
    case 0: GRINQH_ASSIGN(0); break;
    case 1: GRINQH_ASSIGN(1); break;
    case 2: GRINQH_ASSIGN(2); break;
    case 3: GRINQH_ASSIGN(3); break;
    case 4: GRINQH_ASSIGN(4); break;
    case 5: GRINQH_ASSIGN(5); break;
    case 6: GRINQH_ASSIGN(6); break;
    case 7: GRINQH_ASSIGN(7); break;
    default: GRINQH_ASSIGN(8); break;
  }
#undef GRINQH_ASSIGN
}

int launch_assign(const uint16_t* x, int64_t K, const AssignParams& ap, uint8_t* bits,
                  int32_t* active_idx, int32_t* n_active, hipStream_t s) {
  // the 8-byte loads and 4-byte width stores need both buffers 8- and 4-byte aligned
  const bool aligned = reinterpret_cast<uintptr_t>(x) % 8 == 0 && reinterpret_cast<uintptr_t>(bits) % 4 == 0;
  if (aligned)
    launch_n<true>(ap.n, x, K, ap, bits, active_idx, n_active, s);
  else
    launch_n<false>(ap.n, x, K, ap, bits, active_idx, n_active, s);
  return check_launch("grinqh_assign_bits");
}

}  // namespace grinqh
