// Decode-stage VMM over the bit-plane store (GRINQH paper, section 3.3
// "Weight Reconstruction and Bias Correction"; Appendix C.1).
//
// Work split.  A workgroup owns one column tile (one row tile of the store
// per row, ct <= 1024 columns) and one 128-row group of K, so every row it
// touches shares one (scale, zero) row.
//
// Staging.  The group's active rows are sorted by bit width; row e gets b_e
// consecutive "plane slots" (one slot = one plane of the row tile, ct / 8
// bytes), so the workgroup's whole working set is sum_e b_e slots.  The slots
// stream into a four-chunk LDS ring (128 slots per chunk) with direct-to-LDS
// 16-byte buffer loads: lane L of a load instruction fetches one 16-byte piece
// of one slot, found through a slot -> row table, so each instruction moves
// 1 KB of needed bytes and nothing else.  Every wave issues the same number of
// load instructions per chunk, so the loads of three chunks stay in flight
// while the current one is computed.
//
// Compute.  Row pairs are formed from consecutive sorted rows; a 32-lane group
// owns a pair, lane l owns 32 columns (one plane word).  The codes come back
// from the planes through a bit-transpose network (bitplane.hpp); byte j of
// code word m from the two rows is paired into one fp16x2 operand (the code as
// an fp16 subnormal, c * 2^-24) and v_dot2 multiplies it by the pair's fp16
// activations into an fp32 accumulator: one dot per two weights.  With the
// group factored out,
//   sum_i x_i (s r_ij + z) = s (A_j + H) + z X,
//   A_j = sum_i x_i (q_ij with low 8-b_i bits cleared),
//   H = sum_i x_i phi_i,  X = sum_i x_i,
// so scale and zero are applied once per column per workgroup.
//
// Output.  Split-K mode writes one partial row per workgroup; the last one to
// arrive (per-tile counter) adds them in split order, so y does not depend on
// scheduling.  Accumulate mode adds into y with fp32 device-scope atomics.
#include "bitplane.hpp"
#include "common.hpp"

namespace grinqh {

constexpr int kVmmThreads = 512;                 // 8 waves
constexpr int kLaneGroups = kVmmThreads / 32;    // 16 groups of 32 lanes
constexpr int kRowsPerWG = kGroup;               // one scale group per workgroup
constexpr int kChunkSlots = 128;                 // plane slots per staging chunk
constexpr int kRingChunks = 4;
constexpr int kRingSlots = kChunkSlots * kRingChunks;
constexpr int kMaxSlots = kRowsPerWG * 8;
constexpr int kMaxChunks = kMaxSlots / kChunkSlots;
constexpr int kInstPerWave = 2;                  // 8 waves x 2 x 1 KB = one 128-slot chunk of 128-byte planes
constexpr int kRingBytes = kRingSlots * 128;     // 64 KB
constexpr int kTrashBytes = 1024;                // target of load slots a chunk does not need
constexpr int kRedStride = 33;                   // LDS row stride of the lane-group reduction
constexpr int kBigWords = kLaneGroups * 32 * kRedStride;   // reduction area; the ring + trash fit inside
static_assert((kRingBytes + kTrashBytes) / 4 <= kBigWords, "ring must fit in the shared area");
constexpr uint32_t kOutOfRange = 0x7FFFFF00u;    // buffer offset beyond any range used here
constexpr uint32_t kRsrcWord3 = 0x00020000u;     // raw 32-bit buffer, gfx9 family
constexpr int kScopeDevice = 16;                 // cache-policy bits: sc1 = device scope
// s_waitcnt immediates (gfx9 encoding): vmcnt in bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]; all-ones fields mean "do not wait".
constexpr int kWaitVm4 = 0x0F70 | (2 * kInstPerWave);   // vmcnt(4) only
constexpr int kWaitVm0 = 0x0F70;                         // vmcnt(0) only

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// One 16-byte-per-lane direct-to-LDS buffer load: lane L's piece lands at
// dst + 16 L (dst must be wave-uniform).  Written as inline asm so that the
// compiler does not treat every later LDS read as dependent on it (it would
// wait for all outstanding loads); the staging loop waits for exactly the
// chunk it needs with s_waitcnt.  The instruction has no result register, and
// its address register is read when it issues.
__device__ inline void lds_load16(const u32x4& rsrc, void* dst, uint32_t voff) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)dst);
  uint32_t saved_m0;
  // M0 carries the LDS base; it is saved and restored around the load.
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory");
}

// phi * x for one row: the midpoint term of section 3.3 (0 at b = 8 and for no row).
__device__ inline float phi_x(int b, float x) {
  return (b > 0 && b < 8) ? x * __builtin_bit_cast(float, (uint32_t)(127 + 7 - b) << 23) : 0.0f;
}

// Rebuild two rows' codes.  The bit widths branch on scalar values when the
// whole wave agrees (the usual case: rows are sorted by width) and fall back
// to the full 8-plane network otherwise (planes a row does not have are 0).
__device__ inline void rebuild_pair(int b1, int b2, const uint32_t (&w1)[8], const uint32_t (&w2)[8],
                                    uint32_t (&d1)[8], uint32_t (&d2)[8]) {
  const int u1 = __builtin_amdgcn_readfirstlane(b1);
  const int u2 = __builtin_amdgcn_readfirstlane(b2);
  if (__ballot(b1 != u1 || b2 != u2) == 0) {
    planes_to_codes_rt(u1, w1, d1);
    planes_to_codes_rt(u2, w2, d2);
  } else {
    planes_to_codes<8>(w1, d1);
    planes_to_codes<8>(w2, d2);
  }
}

// acc[4m + j] += x1 * row1 code + x2 * row2 code for the 32 columns of a lane:
// bytes [row1 code, 0, row2 code, 0] form two fp16 subnormals c * 2^-24.
__device__ inline void dot_pair(const uint32_t (&d1)[8], const uint32_t (&d2)[8], half2_t xv, float (&acc)[32]) {
#pragma unroll
  for (int mm = 0; mm < 8; ++mm) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t sel = (uint32_t)jj | (0x0Cu << 8) | ((uint32_t)(4 + jj) << 16) | (0x0Cu << 24);
      const uint32_t pr = __builtin_amdgcn_perm(d2[mm], d1[mm], sel);
      acc[4 * mm + jj] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pr), xv, acc[4 * mm + jj], false);
    }
  }
}

// Both rows have B planes at 128-byte slots starting at r1 / r2 (this lane's
// word already added): B LDS reads each with immediate offsets, then the
// B-specialised rebuild.
template <int B>
__device__ inline void pair_fast(const uint8_t* r1, const uint8_t* r2, half2_t xv, float (&acc)[32]) {
  uint32_t w1[8], w2[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    w1[p] = p < B ? *reinterpret_cast<const uint32_t*>(r1 + p * 128) : 0u;
    w2[p] = p < B ? *reinterpret_cast<const uint32_t*>(r2 + p * 128) : 0u;
  }
  uint32_t d1[8], d2[8];
  planes_to_codes<B>(w1, d1);
  planes_to_codes<B>(w2, d2);
  dot_pair(d1, d2, xv, acc);
}

// Output modes.
enum : int {
  kOutSplitK = 0,     // partial rows + last-arriving workgroup adds them in split order
  kOutAccumulate = 1  // fp32 device-scope atomic adds into y (y += x W)
};

template <bool kFused, int kOut>
__global__ __launch_bounds__(kVmmThreads) void vmm_kernel(VmmArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t s_big[kBigWords];   // staging ring | reduction
  __shared__ uint32_t s_slot_off[kMaxSlots];  // plane slot -> byte offset of that plane in the group's row tiles
  __shared__ int16_t s_row[kRowsPerWG];       // sorted row -> row within the group
  __shared__ uint8_t s_b[kRowsPerWG];
  __shared__ uint16_t s_xh[kRowsPerWG];
  __shared__ uint16_t s_slot0[kRowsPerWG];    // first plane slot of a sorted row
  __shared__ int s_cnt[2][9];
  __shared__ int s_qs[kMaxChunks + 2];        // first pair of each chunk
  __shared__ int s_m, s_p0, s_stot, s_last;
  __shared__ float s_hx[kLaneGroups][2];

  const AssignRegs ar = load_assign_regs(a.ap);   // scalar registers, read before any global load
  const int tile = blockIdx.x % a.tiles;
  const int split = blockIdx.x / a.tiles;
  const int64_t k0 = (int64_t)split * kRowsPerWG;
  const int64_t k1 = (k0 + kRowsPerWG) < a.K ? (k0 + kRowsPerWG) : a.K;
  const int64_t Np = padded_cols(a.N);
  const int64_t t0 = (int64_t)tile * kTile;
  const int ct = (int)((Np - t0) < kTile ? (Np - t0) : kTile);   // multiple of 128
  const int pb = ct / 8;                                          // bytes per plane slot, multiple of 16
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t g = split;

  // ---- activation first, then scale and zero of this thread's two output
  // columns (tid, tid + 512).  All loads are unconditional (clamped index,
  // validity applied later) so nothing waits on them before it is needed.
  uint32_t b = 0;
  uint16_t xh = 0;
  int rloc = 0;
  uint16_t xr = 0;
  if constexpr (kFused) {
    // every thread loads (waves 2..7 repeat rows 0..127): no branch around the load
    const int64_t i = k0 + (tid & (kRowsPerWG - 1));
    xr = a.x[i < k1 ? i : k1 - 1];
  }
  uint16_t sc[2], zr[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    int col = tid + u * kVmmThreads;
    col = col < ct ? col : ct - 1;
    int64_t gc = t0 + col;
    gc = gc < a.N ? gc : a.N - 1;
    sc[u] = a.scales[g * a.N + gc];
    zr[u] = a.zeros[g * a.N + gc];
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

  if constexpr (kFused) {
    if (wid < 2) {
      rloc = tid;
      if (k0 + tid < k1) {
        xh = xr;
        b = bits_of(xh, ar);
      }
    }
  } else {
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
    if (wid < 2 && tid < s_m) {
      const int64_t i = a.active_idx[s_p0 + tid];
      if (i >= k0 && i < k1) {   // a well-formed list always is
        rloc = (int)(i - k0);
        b = a.bits[i];
        b = b > 8u ? 8u : b;
        xh = a.x[i];
      }
    }
  }

  // ---- stable counting sort of active rows by bit width (1..8); a row's
  // plane slots follow from the bucket sizes, no scan needed
  uint64_t my_mask = 0;
  if (wid < 2) {
#pragma unroll
    for (int v = 1; v <= 8; ++v) {
      const uint64_t mv = __ballot(b == (uint32_t)v);
      if (lane == 0) s_cnt[wid][v] = __popcll(mv);
      if (b == (uint32_t)v) my_mask = mv;
    }
  }
  __syncthreads();
  if (wid < 2 && b > 0) {
    int row_base = 0, slot_base = 0;
#pragma unroll
    for (int v = 1; v < 8; ++v) {
      const int c = s_cnt[0][v] + s_cnt[1][v];
      row_base += v < (int)b ? c : 0;
      slot_base += v < (int)b ? v * c : 0;
    }
    const int rank = ((wid == 1) ? s_cnt[0][b] : 0) + __popcll(my_mask & ((1ull << lane) - 1ull));
    const int pos = row_base + rank;
    const int slot0 = slot_base + rank * (int)b;
    s_row[pos] = (int16_t)rloc;
    s_b[pos] = (uint8_t)b;
    s_xh[pos] = xh;
    s_slot0[pos] = (uint16_t)slot0;
#pragma unroll
    for (int p = 0; p < 8; ++p)
      if (p < (int)b) s_slot_off[slot0 + p] = (uint32_t)rloc * (uint32_t)ct + (uint32_t)(p * pb);
  }
  if (tid == 0) {
    int m = 0, stot = 0;
#pragma unroll
    for (int v = 1; v <= 8; ++v) {
      const int c = s_cnt[0][v] + s_cnt[1][v];
      m += c;
      stot += v * c;
    }
    s_m = m;
    s_stot = stot;
  }
  __syncthreads();
  const int m = s_m;
  const int stot = s_stot;
  const int npairs = (m + 1) / 2;
  const int nchunks = (stot + kChunkSlots - 1) / kChunkSlots;

  // ---- pair q is ready once the chunk holding its last slot has landed
  if (wid == 0) {
    int rc = kMaxChunks + 1;
    if (lane < npairs) {
      const int e = (2 * lane + 1 < m) ? 2 * lane + 1 : m - 1;
      rc = ((int)s_slot0[e] + (int)s_b[e] - 1) / kChunkSlots;
    }
#pragma unroll
    for (int c = 0; c <= kMaxChunks; ++c) {
      const int n_before = __popcll(__ballot(rc < c));
      if (lane == 0) s_qs[c] = n_before;
    }
  }

  // ---- staging: each wave issues kInstPerWave 1 KB direct-to-LDS loads per chunk
  // buffer descriptor over this group's row tiles (base, stride 0, size, format word)
  u32x4 rsrc;
  {
    const uint64_t base = (uint64_t)(uintptr_t)(a.planes + t0 * a.K + k0 * ct);
    rsrc.x = __builtin_amdgcn_readfirstlane((uint32_t)base);
    rsrc.y = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32) & 0xFFFFu);
    rsrc.z = __builtin_amdgcn_readfirstlane((uint32_t)((k1 - k0) * ct));
    rsrc.w = kRsrcWord3;
  }
  uint8_t* const ring = reinterpret_cast<uint8_t*>(s_big);
  uint8_t* const trash = ring + kRingBytes;
  const int pps = pb / 16;                 // 16-byte pieces per slot (1..8)
  // floor(n / pps) = (n * magic) >> 16 exactly for n < 8192, pps <= 8
  const uint32_t pps_magic = (0x10000u + (uint32_t)pps - 1u) / (uint32_t)pps;
  const int chunk_bytes = kChunkSlots * pb;
  __syncthreads();   // s_qs, slot table, row tables visible

  auto issue_chunk = [&](int c) {
#pragma unroll
    for (int i = 0; i < kInstPerWave; ++i) {
      const int j = kInstPerWave * wid + i;               // instruction slot within the chunk
      const bool inst_ok = c < nchunks && j * 1024 < chunk_bytes;
      const int piece = j * 64 + lane;                    // 16-byte piece within the chunk
      const int sl = (int)(((uint32_t)piece * pps_magic) >> 16);   // slot within the chunk
      const int s = c * kChunkSlots + sl;                           // plane slot
      const bool ok = inst_ok && s < stot;
      const uint32_t off = ok ? s_slot_off[s] + (uint32_t)((piece - sl * pps) * 16) : kOutOfRange;
      uint8_t* dst = inst_ok ? ring + (c % kRingChunks) * chunk_bytes + j * 1024 : trash;
      lds_load16(rsrc, dst, off);
    }
  };

  const int lg = tid >> 5;
  const int ll = tid & 31;
  const bool lane_ok = ll < ct / 32;
  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.0f;
  float h_acc = 0.0f, x_acc = 0.0f;   // this lane group's share of H and X

  const bool full_tile = ct == kTile;
  issue_chunk(0);
  issue_chunk(1);
  issue_chunk(2);
  for (int c = 0; c < nchunks; ++c) {
    // this wave's loads of chunk c are done once at most two later chunks'
    // loads are outstanding; the barrier makes that true for every wave
    __builtin_amdgcn_s_waitcnt(kWaitVm4);
    __syncthreads();
    for (int q = s_qs[c] + lg; q < s_qs[c + 1]; q += kLaneGroups) {
      const int e1 = 2 * q, e2 = 2 * q + 1;
      const int b1 = s_b[e1];
      const int b2 = e2 < m ? (int)s_b[e2] : 0;
      const uint32_t x1h = s_xh[e1], x2h = e2 < m ? (uint32_t)s_xh[e2] : 0u;
      const int sl1 = s_slot0[e1] % kRingSlots, sl2 = e2 < m ? (int)s_slot0[e2] % kRingSlots : 0;
      const float x1 = half_bits_to_float((uint16_t)x1h), x2 = half_bits_to_float((uint16_t)x2h);
      h_acc += phi_x(b1, x1) + phi_x(b2, x2);
      x_acc += x1 + (b2 > 0 ? x2 : 0.0f);
      const half2_t xv = __builtin_bit_cast(half2_t, x1h | (x2h << 16));
      // Fast path: the whole wave has one width B for both rows, the tile is a
      // full 1024 columns and neither row wraps around the ring end.
      const int ub = __builtin_amdgcn_readfirstlane(b1);
      const bool fast = __ballot(!(full_tile && b1 == ub && b2 == ub && sl1 + ub <= kRingSlots &&
                                   sl2 + ub <= kRingSlots)) == 0;
      if (fast) {
        const uint8_t* r1 = ring + sl1 * 128 + 4 * ll;
        const uint8_t* r2 = ring + sl2 * 128 + 4 * ll;
        switch (ub) {
          case 1: pair_fast<1>(r1, r2, xv, acc); break;
          case 2: pair_fast<2>(r1, r2, xv, acc); break;
          case 3: pair_fast<3>(r1, r2, xv, acc); break;
          case 4: pair_fast<4>(r1, r2, xv, acc); break;
          case 5: pair_fast<5>(r1, r2, xv, acc); break;
          case 6: pair_fast<6>(r1, r2, xv, acc); break;
          case 7: pair_fast<7>(r1, r2, xv, acc); break;
          default: pair_fast<8>(r1, r2, xv, acc); break;
        }
      } else {
        uint32_t w1[8], w2[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          w1[p] = (p < b1 && lane_ok) ? *reinterpret_cast<const uint32_t*>(ring + ((sl1 + p) % kRingSlots) * pb + 4 * ll) : 0u;
          w2[p] = (p < b2 && lane_ok) ? *reinterpret_cast<const uint32_t*>(ring + ((sl2 + p) % kRingSlots) * pb + 4 * ll) : 0u;
        }
        uint32_t d1[8], d2[8];
        rebuild_pair(b1, b2, w1, w2, d1, d2);
        dot_pair(d1, d2, xv, acc);
      }
    }
    __syncthreads();          // chunk c - 1 is no longer read: its ring place can be refilled
    issue_chunk(c + 3);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // trailing (empty) loads landed before the LDS is reused
  __syncthreads();

  // ---- reduce the 16 lane groups in LDS (row stride 33 keeps both the
  // writes and the column-wise reads free of bank conflicts)
  float* red = reinterpret_cast<float*>(s_big);
  {
    float* dst = red + (lg * 32 + ll) * kRedStride;
#pragma unroll
    for (int c = 0; c < 32; ++c) dst[c] = acc[c];
    if (ll == 0) {
      s_hx[lg][0] = h_acc;
      s_hx[lg][1] = x_acc;
    }
  }
  __syncthreads();
  float H = 0.0f, X = 0.0f;
#pragma unroll
  for (int h = 0; h < kLaneGroups; ++h) {
    H += s_hx[h][0];
    X += s_hx[h][1];
  }
  float val[2] = {0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int col = tid + u * kVmmThreads;
    if (m > 0 && col < ct && t0 + col < a.N) {
      float A = 0.0f;
#pragma unroll
      for (int h = 0; h < kLaneGroups; ++h) A += red[(h * 32 + (col >> 5)) * kRedStride + (col & 31)];
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
