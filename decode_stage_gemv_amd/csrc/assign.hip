// Dynamic precision assignment and active-row selection (GRINQH paper,
// section 3.1 "Dynamic Precision Assignment").
//
// Each row's width is the level of the number of thresholds |x_i| reaches
// (an fp32 compare against the n thresholds); the active rows (width > 0)
// are listed in ascending order.
//
// Chunked kernel (K up to kChunkedMaxRows): one 512-thread workgroup per
// 2048-row chunk.  A workgroup needs the number of active rows before its
// chunk to know where its part of the list starts; it counts them itself
// from x (no communication between workgroups, no workspace, no waits).  The
// count does not need the widths, only whether a row is active, which is a
// function of |x| with at most n + 2 switch points over the 15-bit magnitude
// a = bits(x) & 0x7fff (NaN patterns sit above +inf).  With the switch points
// B_k (host-computed), a row is active iff an odd number of them are <= a.
// Two rows share one 32-bit word and a packed 16-bit subtraction of B_k
// leaves that comparison in bit 15 of each half (see active_in_word), so the
// count costs about 2 VALU operations per row: two subtractions, one
// three-input xor/and and one bit count per word.  The chunk's own rows take
// the fp32 compares, a wave scan and one exchange of wave totals, and their
// list entries go out through LDS as contiguous stores.
//
// Long inputs (K > kChunkedMaxRows, far above decode sizes) take a single
// workgroup that walks K in 32768-row super-chunks, so the redundant prefix
// counts stay bounded.
#include <math.h>
#include <algorithm>

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

// ---------------------------------------------------------------- chunked

constexpr int kMaxSwitches = kMaxThresholds + 2;                      // even
constexpr int kChunkThreads = 512;
constexpr int kChunkWaves = kChunkThreads / 64;
constexpr int kChunkRowsPerThread = 4;                                // one 8-byte load
constexpr int kChunkRows = kChunkThreads * kChunkRowsPerThread;       // 2048
constexpr int kGroupsPerChunk = kChunkRows / 8;                       // 16-byte groups
constexpr int64_t kChunkedMaxRows = int64_t(1) << 17;                 // at most 64 chunks
constexpr int kMaxBatch = 16;                                         // prefix loads in flight

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

// Switch points of the activity function, each as B | B << 16 (both halves);
// slots past the count hold 0x8000, which no magnitude reaches.
struct ActivitySwitches {
  uint32_t b[kMaxSwitches];
};

// Active rows among the two fp16 values h = s 0x8000 + a of w.  Per half,
// (h - B) mod 2^16 has bit 15 equal to [a >= B] xor (not s) for B <= 0x8000,
// so over an even number NS of switch points the sign terms cancel and the
// xor of the bit-15s is the parity of the points reached: the activity.
template <int NS>
__device__ inline int active_in_word(uint32_t w, const ActivitySwitches& sw) {
  static_assert(NS % 2 == 0, "the sign terms cancel only in pairs");
  uint32_t f = 0;
#pragma unroll
  for (int k = 0; k < NS; ++k)
    f ^= __builtin_bit_cast(uint32_t, __builtin_bit_cast(ushort2_t, w) - __builtin_bit_cast(ushort2_t, sw.b[k]));
  return __builtin_popcount(f & 0x80008000u);
}

template <int NS>
__device__ inline int active_in_group(uint4 q, const ActivitySwitches& sw) {
  return active_in_word<NS>(q.x, sw) + active_in_word<NS>(q.y, sw) + active_in_word<NS>(q.z, sw) +
         active_in_word<NS>(q.w, sw);
}

// Eight rows from 16-byte group gi (all below K).
template <bool kAligned>
__device__ inline uint4 load_group(const uint16_t* __restrict__ x, int64_t gi) {
  if (kAligned) return reinterpret_cast<const uint4*>(x)[gi];
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e >> 1] |= (uint32_t)x[8 * gi + e] << (16 * (e & 1));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Four rows i0 .. i0 + 3; with kWhole all are below K, else those at or past
// K read as 0 (element loads from clamped indexes, no branches, so the loads
// are in flight together).
template <bool kAligned>
__device__ inline uint2 load_own(const uint16_t* __restrict__ x, int64_t i0, int64_t K, bool whole) {
  if (kAligned && whole) return *reinterpret_cast<const uint2*>(x + i0);
  uint32_t w[2] = {0, 0};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool in = whole || i0 + e < K;
    const uint32_t v = x[in ? i0 + e : K - 1];
    w[e >> 1] |= (in ? v : 0u) << (16 * (e & 1));
  }
  return make_uint2(w[0], w[1]);
}

// kAligned: x 16-byte and bits 4-byte aligned.  kBatch: prefix loads per
// thread issued together (the host sizes it to the grid).
template <int NT, int NS, int kBatch, bool kAligned>
__global__ __launch_bounds__(kChunkThreads) void assign_chunked_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                                       AssignParams ap, ActivitySwitches sw,
                                                                       uint8_t* __restrict__ bits,
                                                                       int32_t* __restrict__ active_idx,
                                                                       int32_t* __restrict__ n_active) {
  __shared__ int s_tot[2][kChunkWaves];        // [0]: rows before the chunk, [1]: the chunk's rows
  __shared__ int32_t s_idx[kChunkRows + 64];   // + one spare slot per lane
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int chunk = blockIdx.x;
  const int64_t i0 = (int64_t)chunk * kChunkRows + kChunkRowsPerThread * tid;
  // every chunk but the last is whole (a uniform condition)
  const bool whole = (int64_t)(chunk + 1) * kChunkRows <= K;
  const uint2 own = load_own<kAligned>(x, i0, K, whole);

  // ---- active rows before the chunk: its chunk * 256 groups of 8 rows, one
  // 16-byte load each, lane-contiguous over the workgroup.  A batch of loads
  // goes out with no branch between them (indexes past the end clamp to the
  // last group and their counts are dropped), so it costs one round trip.
  const int64_t groups = (int64_t)chunk * kGroupsPerChunk;
  const int per_thread = (chunk + 1) / 2;   // ceil(groups / kChunkThreads)
  int before_cnt = 0;
  for (int k0 = 0; k0 < per_thread; k0 += kBatch) {
    uint4 q[kBatch];
    bool ok[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t gi = (int64_t)(k0 + u) * kChunkThreads + tid;
      ok[u] = gi < groups;
      q[u] = load_group<kAligned>(x, ok[u] ? gi : groups - 1);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int n = active_in_group<NS>(q[u], sw);
      before_cnt += ok[u] ? n : 0;
    }
  }

  // ---- the chunk's own rows: widths (fp32 compares) and list positions
  const AssignRegs ar = load_assign_regs(ap);
  const int64_t left = K - i0;
  const int valid = whole ? kChunkRowsPerThread : (int)(left < 0 ? 0 : left < 4 ? left : 4);
  uint32_t wb = 0;   // four widths, one per byte
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < kChunkRowsPerThread; ++e) {
    const uint32_t pair = e < 2 ? own.x : own.y;   // rows (0, 1) and (2, 3)
    uint32_t b = width_of<NT>((uint16_t)(e & 1 ? pair >> 16 : pair), ar);
    b = e < valid ? b : 0u;
    wb |= b << (8 * e);
    cnt += b > 0 ? 1 : 0;
  }
  const int incl = wave_inclusive_sum(cnt);
  const int wave_before = __builtin_amdgcn_readlane(wave_inclusive_sum(before_cnt), 63);
  if (lane == 63) {
    s_tot[0][wid] = wave_before;
    s_tot[1][wid] = incl;
  }
  if (kAligned && whole) {
    *reinterpret_cast<uint32_t*>(bits + i0) = wb;
  } else {
#pragma unroll
    for (int e = 0; e < kChunkRowsPerThread; ++e)
      if (e < valid) bits[i0 + e] = (uint8_t)(wb >> (8 * e));
  }
  __syncthreads();
  int base = 0, wave_off = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kChunkWaves; ++w) {
    base += s_tot[0][w];
    wave_off += w < wid ? s_tot[1][w] : 0;
    total += s_tot[1][w];
  }
  // positions inside the chunk's part of the list; an inactive row writes to
  // a spare slot of its lane instead (no branch)
  int pos = wave_off + incl - cnt;
#pragma unroll
  for (int e = 0; e < kChunkRowsPerThread; ++e) {
    const bool act = ((wb >> (8 * e)) & 0xFFu) != 0;
    s_idx[act ? pos : kChunkRows + lane] = (int32_t)(i0 + e);
    pos += act ? 1 : 0;
  }
  __syncthreads();
  for (int i = tid; i < total; i += kChunkThreads) active_idx[base + i] = s_idx[i];
  if (chunk == (int)gridDim.x - 1 && tid == 0) *n_active = base + total;
}

// ------------------------------------------------------- one workgroup (long K)

constexpr int kLongThreads = 1024;
constexpr int kLongWaves = kLongThreads / 64;
constexpr int kLongRowsPerThread = 4;
constexpr int kPassRows = kLongThreads * kLongRowsPerThread;   // 4096
constexpr int kPasses = 8;                                     // passes per super-chunk
constexpr int64_t kSuperRows = (int64_t)kPassRows * kPasses;   // 32768

// Thread t owns rows 4t .. 4t + 3 of a 4096-row pass (one 8-byte load); the
// eight passes of a super-chunk are loaded first, scanned per wave, and
// placed with one exchange of all wave totals (one barrier per super-chunk).
// kAligned: x 8-byte and bits 4-byte aligned.
template <int NT, bool kAligned>
__global__ __launch_bounds__(kLongThreads) void assign_long_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                                   AssignParams ap, uint8_t* __restrict__ bits,
                                                                   int32_t* __restrict__ active_idx,
                                                                   int32_t* __restrict__ n_active) {
  __shared__ int wave_tot[kPasses][kLongWaves];
  const AssignRegs ar = load_assign_regs(ap);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  int base = 0;   // active rows before this super-chunk
  for (int64_t c0 = 0; c0 < K; c0 += kSuperRows) {
    const int64_t left = (K - c0 + kPassRows - 1) / kPassRows;
    const int npass = left < kPasses ? (int)left : kPasses;
    uint32_t xv[kPasses][2];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int64_t i0 = c0 + (int64_t)p * kPassRows + kLongRowsPerThread * tid;
      xv[p][0] = xv[p][1] = 0;
      if (p >= npass) continue;
      if (kAligned && i0 + kLongRowsPerThread <= K) {
        const uint2 q = *reinterpret_cast<const uint2*>(x + i0);
        xv[p][0] = q.x;
        xv[p][1] = q.y;
      } else {
#pragma unroll
        for (int e = 0; e < kLongRowsPerThread; ++e)
          if (i0 + e < K) xv[p][e >> 1] |= (uint32_t)x[i0 + e] << (16 * (e & 1));
      }
    }
    uint32_t wb[kPasses];
    int cnt[kPasses], incl[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int64_t i0 = c0 + (int64_t)p * kPassRows + kLongRowsPerThread * tid;
      wb[p] = 0;
      cnt[p] = 0;
      incl[p] = 0;
      if (p >= npass) continue;
#pragma unroll
      for (int e = 0; e < kLongRowsPerThread; ++e) {
        const uint32_t b = i0 + e < K ? width_of<NT>((uint16_t)(xv[p][e >> 1] >> (16 * (e & 1))), ar) : 0u;
        wb[p] |= b << (8 * e);
        cnt[p] += b > 0 ? 1 : 0;
      }
      incl[p] = wave_inclusive_sum(cnt[p]);
      if (lane == 63) wave_tot[p][wid] = incl[p];
    }
    __syncthreads();
    int pass_base = base;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      if (p >= npass) break;
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kLongWaves; ++w) {
        const int v = wave_tot[p][w];
        before += w < wid ? v : 0;
        total += v;
      }
      const int64_t i0 = c0 + (int64_t)p * kPassRows + kLongRowsPerThread * tid;
      if (kAligned && i0 + kLongRowsPerThread <= K) {
        *reinterpret_cast<uint32_t*>(bits + i0) = wb[p];
      } else {
#pragma unroll
        for (int e = 0; e < kLongRowsPerThread; ++e)
          if (i0 + e < K) bits[i0 + e] = (uint8_t)(wb[p] >> (8 * e));
      }
      int pos = pass_base + before + incl[p] - cnt[p];
#pragma unroll
      for (int e = 0; e < kLongRowsPerThread; ++e)
        if ((wb[p] >> (8 * e)) & 0xFFu) active_idx[pos++] = (int32_t)(i0 + e);
      pass_base += total;
    }
    base = pass_base;
    __syncthreads();   // wave_tot is reused by the next super-chunk
  }
  if (tid == 0) *n_active = base;
}

// ------------------------------------------------------------------ host side

// fp16 bit pattern (sign cleared) to its value.
static double half_magnitude(uint32_t a) {
  const int e = (int)(a >> 10) & 31;
  const int m = (int)(a & 1023);
  if (e == 31) return m ? NAN : INFINITY;
  return e == 0 ? ldexp((double)m, -24) : ldexp((double)(m + 1024), e - 25);
}

// Smallest finite-or-infinite magnitude pattern a in [0, 0x7c00] whose value
// is >= th (th >= 0, not NaN; +inf reaches th = +inf).
static uint32_t first_reaching(float th) {
  uint32_t lo = 0, hi = 0x7C00;   // half_magnitude(0x7c00) = +inf >= th
  while (lo < hi) {
    const uint32_t mid = (lo + hi) / 2;
    if (half_magnitude(mid) >= (double)th) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Switch points of "row active" over the magnitude pattern a in [0, 0x7fff]:
// a row of magnitude a < 0x7c01 reaches the thresholds whose first reaching
// pattern is <= a and is active iff that count's level is > 0; NaN patterns
// (a >= 0x7c01) reach none.
static int activity_switches(const AssignParams& ap, ActivitySwitches* sw) {
  uint32_t reach[kMaxThresholds];
  for (int t = 0; t < ap.n; ++t) reach[t] = first_reaching(ap.th[t]);
  auto active_at = [&](uint32_t a) {
    if (a > 0x7C00) return ap.lv[0] > 0;
    int c = 0;
    for (int t = 0; t < ap.n; ++t) c += a >= reach[t] ? 1 : 0;
    return ap.lv[c] > 0;
  };
  uint32_t cand[kMaxThresholds + 2];
  int nc = 0;
  cand[nc++] = 0;
  for (int t = 0; t < ap.n; ++t) cand[nc++] = reach[t];
  cand[nc++] = 0x7C01;
  std::sort(cand, cand + nc);
  int ns = 0;
  bool prev = false;   // below a = 0 nothing is active
  for (int i = 0; i < nc; ++i) {
    if (i > 0 && cand[i] == cand[i - 1]) continue;
    const bool cur = active_at(cand[i]);
    if (cur != prev) sw->b[ns++] = cand[i] | (cand[i] << 16);
    prev = cur;
  }
  for (int k = ns; k < kMaxSwitches; ++k) sw->b[k] = 0x80008000u;
  return ns;
}

template <int NT, int NS>
static void launch_chunked(bool aligned, const uint16_t* x, int64_t K, const AssignParams& ap,
                           const ActivitySwitches& sw, uint8_t* bits, int32_t* active_idx, int32_t* n_active,
                           hipStream_t s) {
  const int64_t chunks = (K + kChunkRows - 1) / kChunkRows;
  const int64_t per_thread = chunks / 2;   // prefix loads per thread of the last chunk
  const dim3 grid((unsigned)chunks), block(kChunkThreads);
#define GRINQH_CHUNKED(B, A) \
  hipLaunchKernelGGL((assign_chunked_kernel<NT, NS, B, A>), grid, block, 0, s, x, K, ap, sw, bits, active_idx, n_active)
  if constexpr (NS > 2) {   // level tables with several active bands: rare, one load at a time
    if (aligned) GRINQH_CHUNKED(1, true);
    else GRINQH_CHUNKED(1, false);
  } else {
    if (!aligned) GRINQH_CHUNKED(1, false);
    else if (per_thread <= 1) GRINQH_CHUNKED(1, true);
    else if (per_thread <= 2) GRINQH_CHUNKED(2, true);
    else if (per_thread <= 4) GRINQH_CHUNKED(4, true);
    else if (per_thread <= 8) GRINQH_CHUNKED(8, true);
    else GRINQH_CHUNKED(kMaxBatch, true);
  }
#undef GRINQH_CHUNKED
}

template <int NT>
static void launch_nt(const uint16_t* x, int64_t K, const AssignParams& ap, uint8_t* bits, int32_t* active_idx,
                      int32_t* n_active, hipStream_t s) {
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x), ba = reinterpret_cast<uintptr_t>(bits);
  if (K <= kChunkedMaxRows) {
    ActivitySwitches sw;
    const bool aligned = xa % 16 == 0 && ba % 4 == 0;
    if (activity_switches(ap, &sw) <= 2)
      launch_chunked<NT, 2>(aligned, x, K, ap, sw, bits, active_idx, n_active, s);
    else
      launch_chunked<NT, kMaxSwitches>(aligned, x, K, ap, sw, bits, active_idx, n_active, s);
  } else if (xa % 8 == 0 && ba % 4 == 0) {
    hipLaunchKernelGGL((assign_long_kernel<NT, true>), dim3(1), dim3(kLongThreads), 0, s, x, K, ap, bits,
                       active_idx, n_active);
  } else {
    hipLaunchKernelGGL((assign_long_kernel<NT, false>), dim3(1), dim3(kLongThreads), 0, s, x, K, ap, bits,
                       active_idx, n_active);
  }
}

int launch_assign(const uint16_t* x, int64_t K, const AssignParams& ap, uint8_t* bits,
                  int32_t* active_idx, int32_t* n_active, hipStream_t s) {
  switch (ap.n) {
    case 0: launch_nt<0>(x, K, ap, bits, active_idx, n_active, s); break;
    case 1: launch_nt<1>(x, K, ap, bits, active_idx, n_active, s); break;
    case 2: launch_nt<2>(x, K, ap, bits, active_idx, n_active, s); break;
    case 3: launch_nt<3>(x, K, ap, bits, active_idx, n_active, s); break;
    case 4: launch_nt<4>(x, K, ap, bits, active_idx, n_active, s); break;
    case 5: launch_nt<5>(x, K, ap, bits, active_idx, n_active, s); break;
    case 6: launch_nt<6>(x, K, ap, bits, active_idx, n_active, s); break;
    case 7: launch_nt<7>(x, K, ap, bits, active_idx, n_active, s); break;
    default: launch_nt<8>(x, K, ap, bits, active_idx, n_active, s); break;
  }
  return check_launch("grinqh_assign_bits");
}

}  // namespace grinqh
