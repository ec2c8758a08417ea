// Decode-stage VMM over the bit-plane store (GRINQH paper, section 3.3
// "Weight Reconstruction and Bias Correction"; Appendix C.1).
//
// Work split.  A workgroup owns one column tile (<= 1024 columns, one row
// tile of the store per row) and one 128-row group of K, so every row it
// touches shares one (scale, zero) row.  Its active rows are sorted by bit
// width and taken two at a time; each 32-lane group of the workgroup owns a
// stream of row pairs, and lane l of a group owns plane word l (32 columns).
//
// Per row pair and lane: the b planes of each row are fetched with buffer
// loads whose offset is pushed out of range for planes the row does not need
// (they return 0 and move no data), so every iteration issues the same number
// of loads and the next pair's loads are in flight while the current pair is
// computed.  The codes come back from the planes through a bit-transpose
// network specialised for b (bitplane.hpp); byte j of code word m from the two
// rows is paired into one fp16x2 operand (the code as an fp16 subnormal,
// c * 2^-24) and v_dot2 multiplies it by the pair's fp16 activations, adding
// into an fp32 accumulator: one dot per two weights.  With the group factored
// out,
//   sum_i x_i (s r_ij + z) = s (A_j + H) + z X,
//   A_j = sum_i x_i (q_ij with low 8-b_i bits cleared),
//   H = sum_i x_i phi_i,  X = sum_i x_i,
// so the scale and zero are applied once per column per workgroup.
//
// Reduction across workgroups of a tile (split K): each workgroup writes one
// partial row; the last to arrive (per-tile counter) adds them in split order
// and writes y, so y does not depend on scheduling.
#include <stdlib.h>

#include "bitplane.hpp"
#include "common.hpp"

namespace grinqh {

constexpr int kVmmThreads = 512;
constexpr int kWaves = kVmmThreads / 64;
constexpr int kLaneGroups = kVmmThreads / 32;
constexpr int kRowsPerWG = kGroup;
constexpr uint32_t kOutOfRange = 0x7FFFFF00u;   // buffer offset beyond any tile block
constexpr uint32_t kRsrcWord3 = 0x00020000u;    // raw 32-bit buffer, gfx9 family

constexpr int kScopeDevice = 16;              // cache-policy bits: sc1 = device scope

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

VmmGeometry vmm_geometry(int64_t K, int64_t N) {
  VmmGeometry g;
  g.rows_per_split = kRowsPerWG;
  g.splits = (K + kRowsPerWG - 1) / kRowsPerWG;
  g.tiles = n_tiles(N);
  g.partial_floats = g.splits > 1 ? g.splits * padded_cols(N) : 0;
  g.counter_offset = (g.partial_floats * 4 + 255) / 256 * 256;
  g.bytes = g.splits > 1 ? g.counter_offset + g.tiles * 4 : 0;
  return g;
}

struct VmmArgs {
  const uint8_t* planes;
  const uint16_t* scales;
  const uint16_t* zeros;
  const uint16_t* x;
  const uint8_t* bits;
  const int32_t* active_idx;
  const int32_t* n_active;
  float* y;
  float* clear;
  float* partials;
  unsigned* counters;
  int64_t K, N;
  int splits, tiles;
  AssignParams ap;
};

// First position p in [0, n) with idx[p] >= key (n if none); one full wave.
__device__ int64_t wave_lower_bound(const int32_t* __restrict__ idx, int64_t n, int64_t key) {
  const int lane = threadIdx.x & 63;
  int64_t lo = 0, hi = n;
  while (hi > lo) {
    const int64_t span = hi - lo;
    if (span <= 64) {
      const bool pred = lane < span ? (idx[lo + lane] >= key) : true;
      const uint64_t m = __ballot(pred);
      return lo + (__ffsll((unsigned long long)m) - 1);
    }
    const int64_t q = lo + ((int64_t)(lane + 1) * span) / 65;
    const bool pred = idx[q] >= key;
    const uint64_t m = __ballot(pred);
    if (m == 0) {
      lo = __shfl(q, 63, 64) + 1;
    } else {
      const int f = __ffsll((unsigned long long)m) - 1;
      const int64_t qf = __shfl(q, f, 64);
      const int64_t qp = __shfl(q, f > 0 ? f - 1 : 0, 64);
      hi = qf;
      if (f > 0) lo = qp + 1;
    }
  }
  return lo;
}

// One row pair's plane words and activations.
struct PairRegs {
  uint32_t w1[8], w2[8];
  uint32_t xp;     // fp16 x of row 1 (low half) and row 2 (high half)
  int b1, b2;
};

__device__ inline void issue_pair(__amdgpu_buffer_rsrc_t rsrc, int q, int npairs, int m,
                                  const int* s_row, const int* s_bits, const uint16_t* s_xh,
                                  int ct, uint32_t lane_off, bool lane_ok, PairRegs& r) {
  int r1 = 0, r2 = 0, b1 = 0, b2 = 0;
  uint32_t x1 = 0, x2 = 0;
  if (q < npairs) {
    const int e1 = 2 * q, e2 = 2 * q + 1;
    r1 = s_row[e1];
    b1 = s_bits[e1];
    x1 = s_xh[e1];
    if (e2 < m) {
      r2 = s_row[e2];
      b2 = s_bits[e2];
      x2 = s_xh[e2];
    }
  }
  if (!lane_ok) b1 = b2 = 0;
  const uint32_t ps = (uint32_t)ct / 8;
  const uint32_t base1 = (uint32_t)r1 * (uint32_t)ct + lane_off;
  const uint32_t base2 = (uint32_t)r2 * (uint32_t)ct + lane_off;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t o1 = p < b1 ? base1 + (uint32_t)p * ps : kOutOfRange;
    const uint32_t o2 = p < b2 ? base2 + (uint32_t)p * ps : kOutOfRange;
    r.w1[p] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)o1, 0, 0);
    r.w2[p] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)o2, 0, 0);
  }
  r.xp = x1 | (x2 << 16);
  r.b1 = b1;
  r.b2 = b2;
}

__device__ inline void compute_pair(const PairRegs& r, float (&acc)[32]) {
  if ((r.b1 | r.b2) == 0) return;
  uint32_t d1[8], d2[8];
  planes_to_codes_rt(r.b1, r.w1, d1);
  planes_to_codes_rt(r.b2, r.w2, d2);
  const half2_t xv = __builtin_bit_cast(half2_t, r.xp);
#pragma unroll
  for (int mm = 0; mm < 8; ++mm) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // bytes: [row1 code, 0, row2 code, 0] -> two fp16 subnormals c * 2^-24
      const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24);
      const uint32_t pr = __builtin_amdgcn_perm(d2[mm], d1[mm], sel);
      acc[4 * mm + j] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pr), xv, acc[4 * mm + j], false);
    }
  }
}

// Output modes.
enum : int {
  kOutSplitK = 0,     // partial rows + last-arriving workgroup adds them in split order
  kOutAccumulate = 1  // fp32 device-scope atomic adds into y (y += x W)
};

template <bool kFused, int kOut>
__global__ __launch_bounds__(kVmmThreads) void vmm_kernel(VmmArgs a) {
  __shared__ int s_row[kRowsPerWG];
  __shared__ int s_bits[kRowsPerWG];
  __shared__ uint16_t s_xh[kRowsPerWG];
  __shared__ int s_cnt[2][9];
  __shared__ int s_m;
  __shared__ int s_p0;
  __shared__ float s_hx[2][2];
  __shared__ int s_last;
  __shared__ float s_red[kLaneGroups * 32 * 33];

  const int tile = blockIdx.x % a.tiles;
  const int split = blockIdx.x / a.tiles;
  const int64_t k0 = (int64_t)split * kRowsPerWG;
  const int64_t k1 = (k0 + kRowsPerWG) < a.K ? (k0 + kRowsPerWG) : a.K;
  const int64_t Np = padded_cols(a.N);
  const int64_t t0 = (int64_t)tile * kTile;
  const int ct = (int)((Np - t0) < kTile ? (Np - t0) : kTile);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t g = split;   // one 128-row group per workgroup

  // ---- scale and zero of this thread's two output columns (tid, tid + 512),
  // fetched now so their latency hides behind the rest of the work
  uint16_t sc[2] = {0, 0}, zr[2] = {0, 0};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int col = tid + u * kVmmThreads;
    if (col < ct && t0 + col < a.N) {
      sc[u] = a.scales[g * a.N + t0 + col];
      zr[u] = a.zeros[g * a.N + t0 + col];
    }
  }
  if constexpr (kOut == kOutAccumulate) {
    // the caller's next output buffer, zeroed once per column (split 0 only)
    if (a.clear && split == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int col = tid + u * kVmmThreads;
        if (col < ct && t0 + col < a.N) a.clear[t0 + col] = 0.0f;
      }
    }
  }

  // ---- gather this group's candidate rows: thread t < 128 holds one
  if constexpr (!kFused) {
    if (wid == 0) {
      const int64_t n = *a.n_active;
      const int64_t p0 = wave_lower_bound(a.active_idx, n, k0);
      const int64_t p1 = wave_lower_bound(a.active_idx, n, k1);
      int m = (int)(p1 - p0);
      m = m < 0 ? 0 : (m > kRowsPerWG ? kRowsPerWG : m);
      if (lane == 0) {
        s_m = m;
        s_p0 = (int)p0;
      }
    }
    __syncthreads();
  }
  uint32_t b = 0;
  uint16_t xh = 0;
  int rloc = 0;
  if (wid < 2) {
    if constexpr (kFused) {
      rloc = tid;
      if (k0 + tid < k1) {
        xh = a.x[k0 + tid];
        b = level_bits(level_of(xh, a.ap), a.ap);
      }
    } else {
      if (tid < s_m) {
        const int64_t i = a.active_idx[s_p0 + tid];
        if (i >= k0 && i < k1) {   // a well-formed list always is
          rloc = (int)(i - k0);
          b = a.bits[i];
          b = b > 8u ? 8u : b;
          xh = a.x[i];
        }
      }
    }
  }

  // ---- stable counting sort of active rows by bit width (1..8)
  uint64_t my_mask = 0;
  if (wid < 2) {
#pragma unroll
    for (int v = 1; v <= 8; ++v) {
      const uint64_t mv = __ballot(b == (uint32_t)v);
      if (lane == 0) s_cnt[wid][v] = __popcll(mv);
      if (b == (uint32_t)v) my_mask = mv;
    }
    // H = sum x phi and X = sum x over active rows (fixed butterfly order)
    const float xf = half_bits_to_float(xh);
    float h = (b > 0 && b < 8) ? xf * (float)(1 << (7 - (b > 0 ? b : 1))) : 0.0f;
    float xs = b > 0 ? xf : 0.0f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      h += __shfl_xor(h, off, 64);
      xs += __shfl_xor(xs, off, 64);
    }
    if (lane == 0) {
      s_hx[wid][0] = h;
      s_hx[wid][1] = xs;
    }
  }
  __syncthreads();
  if (wid < 2 && b > 0) {
    int pos = (wid == 1) ? s_cnt[0][b] : 0;
    for (int v = 1; v < (int)b; ++v) pos += s_cnt[0][v] + s_cnt[1][v];
    pos += __popcll(my_mask & ((1ull << lane) - 1ull));
    s_row[pos] = rloc;
    s_bits[pos] = (int)b;
    s_xh[pos] = xh;
  }
  if (tid == 0) {
    int m = 0;
    for (int v = 1; v <= 8; ++v) m += s_cnt[0][v] + s_cnt[1][v];
    s_m = m;
  }
  __syncthreads();
  const int m = s_m;

  // ---- stream row pairs: lane group lg takes pairs lg, lg + 16, lg + 32,
  // lg + 48 (at most 64 pairs per group), three in flight at a time
  const int lg = tid >> 5;
  const int ll = tid & 31;
  const bool lane_ok = ll < ct / 32;
  // Descriptor over this group's row tiles only: row r of the group starts at r * ct.
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.planes + t0 * a.K + k0 * ct), (short)0, (int)((k1 - k0) * ct), (int)kRsrcWord3);
  const uint32_t lane_off = 4u * (uint32_t)ll;
  const int npairs = (m + 1) / 2;
  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.0f;
  {
    PairRegs p0, p1, p2;
    issue_pair(rsrc, lg, npairs, m, s_row, s_bits, s_xh, ct, lane_off, lane_ok, p0);
    issue_pair(rsrc, lg + kLaneGroups, npairs, m, s_row, s_bits, s_xh, ct, lane_off, lane_ok, p1);
    issue_pair(rsrc, lg + 2 * kLaneGroups, npairs, m, s_row, s_bits, s_xh, ct, lane_off, lane_ok, p2);
    compute_pair(p0, acc);
    issue_pair(rsrc, lg + 3 * kLaneGroups, npairs, m, s_row, s_bits, s_xh, ct, lane_off, lane_ok, p0);
    compute_pair(p1, acc);
    compute_pair(p2, acc);
    compute_pair(p0, acc);
  }

  // ---- reduce the 16 lane groups in LDS (row stride 33 keeps both the
  // writes and the column-wise reads free of bank conflicts).  A half-wave
  // swap (v_permlane32_swap) would halve this, but this toolchain drops one of
  // the swap's two results, so it is not used.
  {
    float* dst = s_red + (lg * 32 + ll) * 33;
#pragma unroll
    for (int c = 0; c < 32; ++c) dst[c] = acc[c];
  }
  __syncthreads();
  const float H = s_hx[0][0] + s_hx[1][0];
  const float X = s_hx[0][1] + s_hx[1][1];
  float val[2] = {0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int col = tid + u * kVmmThreads;
    if (m > 0 && col < ct && t0 + col < a.N) {
      float A = 0.0f;
#pragma unroll
      for (int h = 0; h < kLaneGroups; ++h) A += s_red[(h * 32 + (col >> 5)) * 33 + (col & 31)];
      A *= 16777216.0f;   // codes entered as c * 2^-24
      val[u] = half_bits_to_float(sc[u]) * (A + H) + half_bits_to_float(zr[u]) * X;
    }
  }

  if constexpr (kOut == kOutAccumulate) {
    if (m > 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int col = tid + u * kVmmThreads;
        if (col < ct && t0 + col < a.N)
          __hip_atomic_fetch_add(a.y + t0 + col, val[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  } else {
    if (a.splits == 1) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int col = tid + u * kVmmThreads;
        if (col < ct && t0 + col < a.N) a.y[t0 + col] = val[u];
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int col = tid + u * kVmmThreads;
      // device-scope store: written through to the point where every XCD sees it
      if (col < ct)
        __hip_atomic_store(a.partials + (int64_t)split * Np + t0 + col, val[u], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- the last workgroup of the tile adds the partial rows in split
    // order.  No cache-wide fence: each wave waits until its device-scope
    // stores are acknowledged, the barrier makes that true for the whole
    // workgroup, and only then is the tile counter bumped; the workgroup that
    // sees the final count reads the partial rows with device-scope loads.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (old == (unsigned)(a.splits - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.partials + t0), (short)0, (int)(a.splits * Np * 4), (int)kRsrcWord3);
    const uint32_t row_bytes = (uint32_t)(Np * 4);
    float sum[2] = {0.0f, 0.0f};
    // 32 splits per round, all loads of a round in flight together; splits
    // past the end read as zero (out-of-range offsets)
    for (int sp0 = 0; sp0 < a.splits; sp0 += 32) {
      uint32_t v[32][2];
#pragma unroll
      for (int u = 0; u < 32; ++u)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int col = tid + e * kVmmThreads;
          const bool ok = sp0 + u < a.splits && col < ct;
          const uint32_t off = ok ? (uint32_t)(sp0 + u) * row_bytes + 4u * (uint32_t)col : kOutOfRange;
          v[u][e] = __builtin_amdgcn_raw_buffer_load_b32(prs, (int)off, 0, kScopeDevice);
        }
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        sum[0] += __builtin_bit_cast(float, v[u][0]);
        sum[1] += __builtin_bit_cast(float, v[u][1]);
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int col = tid + e * kVmmThreads;
      if (col < ct && t0 + col < a.N) a.y[t0 + col] = sum[e];
    }
    if (tid == 0) __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

static int launch_vmm(bool fused, int out_mode, VmmArgs& a, void* ws, hipStream_t s) {
  const VmmGeometry g = vmm_geometry(a.K, a.N);
  if (g.partial_floats * 4 >= (int64_t)kOutOfRange)
    return fail(GRINQH_EINVAL, "K x N too large for one split-K workspace (%lld partial floats)",
                (long long)g.partial_floats);
  a.splits = (int)g.splits;
  a.tiles = (int)g.tiles;
  a.partials = reinterpret_cast<float*>(ws);
  a.counters = g.bytes > 0 && ws ? reinterpret_cast<unsigned*>(reinterpret_cast<char*>(ws) + g.counter_offset) : nullptr;
  const dim3 grid((unsigned)(g.splits * g.tiles));
  const dim3 block(kVmmThreads);
  if (out_mode == kOutAccumulate) {
    if (fused)
      hipLaunchKernelGGL((vmm_kernel<true, kOutAccumulate>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((vmm_kernel<false, kOutAccumulate>), grid, block, 0, s, a);
  } else {
    if (fused)
      hipLaunchKernelGGL((vmm_kernel<true, kOutSplitK>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((vmm_kernel<false, kOutSplitK>), grid, block, 0, s, a);
  }
  return check_launch(out_mode == kOutAccumulate ? "grinqh_decode_vmm_accumulate"
                                                 : (fused ? "grinqh_decode_vmm" : "grinqh_vmm"));
}

int launch_vmm_list(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                    const uint16_t* x, const uint8_t* bits, const int32_t* active_idx,
                    const int32_t* n_active, int64_t K, int64_t N, float* y, void* ws,
                    hipStream_t s) {
  VmmArgs a{};
  a.planes = planes; a.scales = scales; a.zeros = zeros; a.x = x;
  a.bits = bits; a.active_idx = active_idx; a.n_active = n_active;
  a.y = y; a.K = K; a.N = N;
  return launch_vmm(false, kOutSplitK, a, ws, s);
}

int launch_vmm_fused(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                     const uint16_t* x, int64_t K, int64_t N, const AssignParams& ap, float* y,
                     void* ws, hipStream_t s) {
  VmmArgs a{};
  a.planes = planes; a.scales = scales; a.zeros = zeros; a.x = x;
  a.y = y; a.K = K; a.N = N; a.ap = ap;
  return launch_vmm(true, kOutSplitK, a, ws, s);
}

int launch_vmm_accumulate(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                          const uint16_t* x, int64_t K, int64_t N, const AssignParams& ap, float* y,
                          float* clear, hipStream_t s) {
  VmmArgs a{};
  a.planes = planes; a.scales = scales; a.zeros = zeros; a.x = x;
  a.y = y; a.clear = clear; a.K = K; a.N = N; a.ap = ap;
  return launch_vmm(true, kOutAccumulate, a, nullptr, s);
}

}  // namespace grinqh
