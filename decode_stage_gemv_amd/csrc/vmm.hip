// Decode-stage VMM over the bit-plane store (GRINQH paper, section 3.3
// "Weight Reconstruction and Bias Correction"; Appendix C.1).
//
// Work split: a workgroup owns one column tile (<= 1024 columns) and one
// 128-row group of K, so every row it touches shares one (scale, zero) row.
// Its 8 half-waves (32 lanes each) take the group's active rows in turn; a
// lane owns one 32-column plane word, loads only the b_i planes a row needs
// and rebuilds the 32 truncated codes with rotate/AND-OR.  With the group
// factored out,
//   sum_i x_i (s r_ij + z) = s (A_j + H) + z X,
//   A_j = sum_i x_i (q_ij with low 8-b_i bits cleared),
//   H = sum_i x_i phi_i,  X = sum_i x_i,
// so the per-weight work is one convert and one FMA.  Half-wave partials
// meet in LDS; workgroups of the same tile meet through a workspace of
// partial rows, and the last one to arrive (per-tile counter) adds them in a
// fixed order, so y does not depend on scheduling.
#include "common.hpp"

namespace grinqh {

constexpr int kVmmThreads = 256;
constexpr int kHalfWaves = kVmmThreads / 32;
constexpr int kRowsPerWG = kGroup;

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
  float* partials;
  unsigned* counters;
  int64_t K, N;
  int splits, tiles;
  AssignParams ap;
};

__device__ inline uint32_t rotr(uint32_t w, int s) { return __builtin_amdgcn_alignbit(w, w, s); }

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

template <bool kFused>
__global__ __launch_bounds__(kVmmThreads) void vmm_group_kernel(VmmArgs a) {
  __shared__ int s_row[kRowsPerWG];
  __shared__ int s_bits[kRowsPerWG];
  __shared__ float s_x[kRowsPerWG];
  __shared__ int s_wcount[2];
  __shared__ int s_m;
  __shared__ float s_hx[4][2];
  __shared__ int s_last;
  __shared__ float s_red[kHalfWaves * kTile];

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

  // ---- active rows of [k0, k1), ascending, into LDS
  if constexpr (kFused) {
    uint32_t b = 0;
    float xf = 0.0f;
    int before = 0;
    if (wid < 2) {
      const int64_t i = k0 + tid;
      if (i < k1) {
        const uint16_t xh = a.x[i];
        b = level_bits(level_of(xh, a.ap), a.ap);
        xf = half_bits_to_float(xh);
      }
      const uint64_t mask = __ballot(b > 0);
      before = __popcll(mask & ((1ull << lane) - 1ull));
      if (lane == 0) s_wcount[wid] = __popcll(mask);
    }
    __syncthreads();
    if (wid < 2 && b > 0) {
      const int pos = (wid == 1 ? s_wcount[0] : 0) + before;
      s_row[pos] = tid;
      s_bits[pos] = (int)b;
      s_x[pos] = xf;
    }
    if (tid == 0) s_m = s_wcount[0] + s_wcount[1];
  } else {
    if (wid == 0) {
      const int64_t n = *a.n_active;
      const int64_t p0 = wave_lower_bound(a.active_idx, n, k0);
      const int64_t p1 = wave_lower_bound(a.active_idx, n, k1);
      int m = (int)(p1 - p0);
      m = m < 0 ? 0 : (m > kRowsPerWG ? kRowsPerWG : m);
      for (int r = lane; r < m; r += 64) {
        const int64_t i = a.active_idx[p0 + r];
        const bool inside = i >= k0 && i < k1;   // a well-formed list always is
        uint32_t b = inside ? a.bits[i] : 0u;
        b = b > 8u ? 8u : b;
        s_row[r] = inside ? (int)(i - k0) : 0;
        s_bits[r] = (int)b;
        s_x[r] = inside ? half_bits_to_float(a.x[i]) : 0.0f;
      }
      if (lane == 0) s_m = m;
    }
  }
  __syncthreads();
  const int m = s_m;

  // ---- H = sum x phi and X = sum x over the active rows (fixed order)
  {
    float h = 0.0f, xs = 0.0f;
    if (tid < m) {
      const int b = s_bits[tid];
      const float xf = s_x[tid];
      if (b > 0) {
        xs = xf;
        h = b < 8 ? xf * (float)(1 << (7 - b)) : 0.0f;
      }
    }
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

  // ---- plane streaming, rebuild, FMA
  const int hw = tid >> 5;
  const int hl = tid & 31;
  const bool col_ok = hl < ct / 32;
  const uint8_t* tile_base = a.planes + t0 * a.K;
  const int plane_stride = ct / 8;
  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.0f;

  for (int e = hw; e < m; e += kHalfWaves) {
    const int r = s_row[e];
    const int b = s_bits[e];
    const float xf = s_x[e];
    const uint8_t* rowp = tile_base + (k0 + r) * ct + 4 * hl;
    uint32_t w[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      w[p] = 0u;
      if (p < b && col_ok) w[p] = *reinterpret_cast<const uint32_t*>(rowp + p * plane_stride);
    }
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
      uint32_t d = 0u;
#pragma unroll
      for (int p = 0; p < 8; ++p) d |= rotr(w[p], (mm + p - 7) & 31) & (0x01010101u << (7 - p));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[4 * mm + j] += xf * (float)((d >> (8 * j)) & 0xFFu);
    }
  }

  // ---- reduce half-waves, dequantise with the group's scale and zero
#pragma unroll
  for (int c = 0; c < 32; ++c) s_red[hw * kTile + hl * 32 + c] = acc[c];
  __syncthreads();
  const float H = s_hx[0][0] + s_hx[1][0] + s_hx[2][0] + s_hx[3][0];
  const float X = s_hx[0][1] + s_hx[1][1] + s_hx[2][1] + s_hx[3][1];
  const int64_t g = k0 / kGroup;
  for (int col = tid; col < ct; col += kVmmThreads) {
    const int64_t gc = t0 + col;
    float val = 0.0f;
    if (m > 0 && gc < a.N) {
      float A = 0.0f;
#pragma unroll
      for (int h = 0; h < kHalfWaves; ++h) A += s_red[h * kTile + col];
      const float s = half_bits_to_float(a.scales[g * a.N + gc]);
      const float z = half_bits_to_float(a.zeros[g * a.N + gc]);
      val = s * (A + H) + z * X;
    }
    if (a.splits == 1) {
      if (gc < a.N) a.y[gc] = val;
    } else {
      a.partials[(int64_t)split * Np + gc] = val;
    }
  }
  if (a.splits == 1) return;

  // ---- last workgroup of the tile adds the partial rows in split order
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned old = atomicAdd(&a.counters[tile], 1u);
    s_last = (old == (unsigned)(a.splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int col = tid; col < ct; col += kVmmThreads) {
    const int64_t gc = t0 + col;
    if (gc >= a.N) continue;
    float sum = 0.0f;
    for (int sp = 0; sp < a.splits; ++sp) sum += a.partials[(int64_t)sp * Np + gc];
    a.y[gc] = sum;
  }
  if (tid == 0) a.counters[tile] = 0u;
}

static int launch_vmm(bool fused, VmmArgs& a, void* ws, hipStream_t s) {
  const VmmGeometry g = vmm_geometry(a.K, a.N);
  a.splits = (int)g.splits;
  a.tiles = (int)g.tiles;
  a.partials = reinterpret_cast<float*>(ws);
  a.counters = g.bytes > 0 ? reinterpret_cast<unsigned*>(reinterpret_cast<char*>(ws) + g.counter_offset) : nullptr;
  const int64_t grid = g.splits * g.tiles;
  if (fused)
    hipLaunchKernelGGL(vmm_group_kernel<true>, dim3((unsigned)grid), dim3(kVmmThreads), 0, s, a);
  else
    hipLaunchKernelGGL(vmm_group_kernel<false>, dim3((unsigned)grid), dim3(kVmmThreads), 0, s, a);
  return check_launch(fused ? "grinqh_decode_vmm" : "grinqh_vmm");
}

int launch_vmm_list(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                    const uint16_t* x, const uint8_t* bits, const int32_t* active_idx,
                    const int32_t* n_active, int64_t K, int64_t N, float* y, void* ws,
                    hipStream_t s) {
  VmmArgs a{};
  a.planes = planes; a.scales = scales; a.zeros = zeros; a.x = x;
  a.bits = bits; a.active_idx = active_idx; a.n_active = n_active;
  a.y = y; a.K = K; a.N = N;
  return launch_vmm(false, a, ws, s);
}

int launch_vmm_fused(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                     const uint16_t* x, int64_t K, int64_t N, const AssignParams& ap, float* y,
                     void* ws, hipStream_t s) {
  VmmArgs a{};
  a.planes = planes; a.scales = scales; a.zeros = zeros; a.x = x;
  a.y = y; a.K = K; a.N = N; a.ap = ap;
  return launch_vmm(true, a, ws, s);
}

}  // namespace grinqh
