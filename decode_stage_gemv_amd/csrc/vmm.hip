// Decode-stage VMM over the bit-plane store (GRINQH paper, section 3.3
// "Weight Reconstruction and Bias Correction"; Appendix C.1).
//
// Work split.  A workgroup owns one column tile (one row tile of the store
// per row, ct <= 1024 columns) and one item of 128 (or 64) rows inside one
// 128-row group of K, so every row it touches shares one (scale, zero) row.
//
// Row order.  Every wave sees all rows of the group (two per lane) and
// buckets the active ones by bit width b with ballots, in registers.  Each
// bucket is cut into "couples" of four rows of one width (the last couple of
// a bucket is padded with empty rows: x = 0, no bytes).  A couple is two row
// pairs; the two 32-lane halves of a wave take one pair each, lane l owning
// 32 columns (one plane word of each row), so the bit width is the same for
// the whole wave.  Couple k belongs to wave k mod W, W the workgroup's
// waves (8, 4 or 2; its "records", in order).
//
// Loads.  A lane loads its pair's plane words straight into registers with
// 4-byte buffer loads: planes p < b come from the row tile; a record is 8
// loads (planes 0..3) or, above width 4, 16, and within those the loads of
// planes p >= b repeat plane 0 (a cache hit that the width-specialised
// rebuild ignores); padding rows use an out-of-range voffset, which returns
// 0 and moves no bytes.  Only the top b planes of a row are fetched from
// memory.  Three records are in
// flight per wave; a wave waits only for its own loads and never for another
// wave until the final reduction.
//
// Compute.  The codes come back from the planes through a bit-transpose
// network (bitplane.hpp); byte j of code word m from the two rows of a pair
// is paired into one fp16x2 operand (the code as an fp16 subnormal,
// c * 2^-24) and v_dot2 multiplies it by the pair's fp16 activations into an
// fp32 accumulator: one dot per two weights.  With the group factored out,
//   sum_i x_i (s r_ij + z) = s (A_j + H) + z X,
//   A_j = sum_i x_i (q_ij with low 8-b_i bits cleared),
//   H = sum_i x_i phi_i,  X = sum_i x_i,
// so scale and zero are applied once per column per workgroup, and H and X
// are plain sums over the group's active rows.  A store of b_max < 8 bits has
// b_max planes per row: the network puts plane p at code bit 7 - p as always,
// so codes come out as q 2^(8 - b_max) and the scale is s 2^(b_max - 8).
//
// Output.  Split-K mode writes one partial row per workgroup; the last one to
// arrive (per-tile counter) adds them in split order, so y does not depend on
// scheduling.  Accumulate mode adds into y with fp32 device-scope atomics.
#include "bitplane.hpp"
#include "common.hpp"

namespace grinqh {

constexpr int kMaxRows = kGroup;                 // rows of one workgroup: 128 or 64, within one scale group
constexpr int kMaxCouples = kMaxRows / 4 + 6;    // sum over 8 widths of ceil(c_v / 4) <= (128 + 8 * 3) / 4
constexpr int kRedStride = 33;                   // LDS row stride of the wave reduction
// Launch shape.  The grid is (row item, column tile) pairs.  Small layers
// use 64-row items so that more workgroups share the CUs; workgroups have 8
// waves while two fit per CU, 4 waves up to one round of 16 waves per CU,
// and 2 waves beyond that, so that the largest layers still run in one
// round (each wave then takes more records, in a rolled loop).
constexpr int kTargetCUs = 256;                  // MI355X
constexpr uint32_t kOutOfRange = 0x7FFFFF00u;    // buffer offset beyond any range used here
constexpr int kRsrcWord3 = 0x00020000;           // raw 32-bit buffer, gfx9 family
constexpr int kScopeDevice = 16;                 // cache-policy bits: sc1 = device scope
// s_waitcnt immediates (gfx9 encoding): vmcnt in bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]; all-ones fields mean "do not wait".
constexpr int kWaitVm0 = 0x0F70;                 // vmcnt(0) only

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

VmmGeometry vmm_geometry(int64_t K, int64_t N) {
  VmmGeometry g;
  g.tiles = n_tiles(N);
  g.rows_per_split = n_groups(K) * g.tiles < kTargetCUs ? 64 : 128;
  g.splits = (K + g.rows_per_split - 1) / g.rows_per_split;
  // waves per workgroup: 8 while the workgroups fit two per CU, then 4, and
  // 2 once 4-wave workgroups would need a second round (at four waves per
  // SIMD a round holds 16 waves per CU): every extra round repeats the
  // whole latency chain of a workgroup (activations, planes, reduction)
  const int64_t wgs = g.splits * g.tiles;
  g.waves = wgs > 4 * kTargetCUs ? 2 : (wgs > 2 * kTargetCUs ? 4 : 8);
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
  int splits, tiles, rows;
  int bmax;   // planes per row of the store (1..8)
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

// phi * x for one row: the midpoint term of section 3.3 in 8-bit code units,
// 2^(7 - b) (0 at b = b_max, where nothing is truncated, and for no row).
__device__ inline float phi_x(int b, int bmax, float x) {
  return (b > 0 && b < bmax) ? x * __builtin_bit_cast(float, (uint32_t)(127 + 7 - b) << 23) : 0.0f;
}

// Lanes l < 32 get a(l) + a(l + 32), lanes l >= 32 get b(l - 32) + b(l): one
// swap of the upper half of a with the lower half of b (the swapped values
// pass through plain integers: a vector element inside a bit cast is
// mistranslated by the compiler).
__device__ inline float halves_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const uint32_t lo = r[0], hi = r[1];
  return __uint_as_float(lo) + __uint_as_float(hi);
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

// One record in flight: the lane's plane words of its pair (planes the rows
// do not have are 0) and the pair's activations.
struct RecordRegs {
  uint32_t w1[8], w2[8];
};

// Issue the loads of record j of this wave (width b; b = 0 for a record the
// wave does not have) into r.  The record's row sources (byte offsets of the
// row tiles within the group's block, out of range for padding rows) come
// from the wave's LDS table.  Lane l of a pair loads plane word l of planes
// p < b of both rows (plane p at scalar offset p pb from the row tile).  A
// record issues 8 loads (planes 0..3 of both rows) or, for b > 4, 16: few
// shapes of load count keep the compiler's wait counts close to exact (a
// branch per plane made them wait for nearly everything), and the second
// half is skipped for the narrow widths that carry most rows; every vector
// memory instruction costs issue time on the CU even when it moves nothing.
// Within a half, the loads of planes p >= b repeat plane 0 (a cache hit;
// compute_record ignores them), and a padding row or a record the wave does
// not have uses an out-of-range voffset, which returns 0 and moves no bytes
// (only the voffset takes part in the range check).
// lane_off is 4 l for the lanes of a word the tile has (4 l < pb) and
// kOutOfRange for the others, so that a narrow last tile never reads past
// its own row tiles: the scalar plane offset is not range-checked.
template <int kMaxRecords>
__device__ inline void load_record(RecordRegs& r, __amdgpu_buffer_rsrc_t rsrc, const uint32_t* src,
                                   int j, int b, int pb, uint32_t lane_off) {
  const int h = (threadIdx.x >> 5) & 1;
  const int jj = j < kMaxRecords ? j : kMaxRecords - 1;   // table index (unused when b = 0)
  const uint32_t s1 = b > 0 ? src[4 * jj + 2 * h] : kOutOfRange;
  const uint32_t s2 = b > 0 ? src[4 * jj + 2 * h + 1] : kOutOfRange;
  // s < 2^17 and kOutOfRange < 2^31, so the sums do not wrap
  const uint32_t v1 = s1 == kOutOfRange ? kOutOfRange : s1 + lane_off;
  const uint32_t v2 = s2 == kOutOfRange ? kOutOfRange : s2 + lane_off;
#pragma unroll
  for (int p = 0; p < 4; ++p)
    r.w1[p] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)v1, p < b ? p * pb : 0, 0);
#pragma unroll
  for (int p = 0; p < 4; ++p)
    r.w2[p] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)v2, p < b ? p * pb : 0, 0);
  if (b > 4) {
#pragma unroll
    for (int p = 4; p < 8; ++p)
      r.w1[p] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)v1, p < b ? p * pb : 0, 0);
#pragma unroll
    for (int p = 4; p < 8; ++p)
      r.w2[p] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)v2, p < b ? p * pb : 0, 0);
  }
}

// Rebuild and accumulate one record (width b >= 1, wave-uniform): the
// network for exactly b planes, so planes at or past b are never read.
template <int B>
__device__ inline void rebuild_pair(const RecordRegs& r, uint32_t (&d1)[8], uint32_t (&d2)[8]) {
  planes_to_codes<B>(r.w1, d1);
  planes_to_codes<B>(r.w2, d2);
}

__device__ inline void compute_record(const RecordRegs& r, int b, uint32_t xw, float (&acc)[32]) {
  uint32_t d1[8], d2[8];
  switch (b) {
    case 1: rebuild_pair<1>(r, d1, d2); break;
    case 2: rebuild_pair<2>(r, d1, d2); break;
    case 3: rebuild_pair<3>(r, d1, d2); break;
    case 4: rebuild_pair<4>(r, d1, d2); break;
    case 5: rebuild_pair<5>(r, d1, d2); break;
    case 6: rebuild_pair<6>(r, d1, d2); break;
    case 7: rebuild_pair<7>(r, d1, d2); break;
    default: rebuild_pair<8>(r, d1, d2); break;
  }
  dot_pair(d1, d2, __builtin_bit_cast(half2_t, xw), acc);
}

// Output modes.
enum : int {
  kOutSplitK = 0,     // partial rows + last-arriving workgroup adds them in split order
  kOutAccumulate = 1  // fp32 device-scope atomic adds into y (y += x W)
};

// Everything the prologue needs before its first loads (the activation,
// plane, scale and zero pointers and the shape) comes first as plain
// scalars: the build asks for the first nine arguments to be preloaded into
// scalar registers, so the activation and scale loads issue at once instead
// of after a fetch of the argument block, and that fetch (thresholds,
// levels) completes while the activations are in flight.
template <bool kFused, int kOut, int kWaves>
__global__ __launch_bounds__(64 * kWaves) void vmm_kernel(const uint16_t* __restrict__ x,
                                                          const uint8_t* __restrict__ planes,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ zeros, int K, int N,
                                                          int tiles, int rows, int bmax, VmmArgs a) {
  constexpr int kVmmThreads = 64 * kWaves;
  constexpr int kCols = kTile / kVmmThreads;        // output columns per thread in the epilogue
  constexpr int kMaxRecords = (kMaxCouples + kWaves - 1) / kWaves;
  constexpr int kRedWords = kWaves * 32 * kRedStride;
  __shared__ float s_red[kRedWords];                      // wave reduction
  __shared__ uint32_t s_src[kWaves][kMaxRecords * 4];     // per wave: record row -> source byte offset
  __shared__ uint32_t s_cx[kWaves][kMaxRecords * 2];      // per wave: record pair -> fp16 x of its rows
  __shared__ float s_hx[2];
  __shared__ int s_last;
  // 2-wave workgroups: each thread has 8 epilogue columns, whose scales and
  // zeros are parked in LDS during the record loop (registers are short)
  constexpr bool kParkScales = kWaves == 2;
  __shared__ uint32_t s_scz[kParkScales ? kTile : 1];

  // workgroup = (column tile, 128-row group), tiles fastest (K, N < 2^31)
  const int tile = blockIdx.x % tiles;
  const int split = blockIdx.x / tiles;
  const int k0 = split * rows;
  const int k1 = (k0 + rows) < K ? (k0 + rows) : K;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int64_t g = k0 / kGroup;                // scale group

  // ---- every wave sees all rows of the group, two per lane (lane and lane
  // + 64): activation loads first, then scale and zero of this thread's two
  // output columns (tid, tid + 512).  Loads are unconditional (clamped
  // index, validity applied later) so nothing waits on them early.
  uint32_t bq[2] = {0u, 0u};   // bit width of the lane's two rows
  uint16_t xq[2] = {0, 0};     // their fp16 activations
  int rq[2] = {0, 0};          // their rows within the group
  if constexpr (kFused) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t i = k0 + lane + 64 * e;
      xq[e] = x[i < k1 ? i : k1 - 1];
      rq[e] = lane + 64 * e;
    }
  }
  // keep the activation loads ahead of everything else: they need only the
  // preloaded arguments, and waits count loads in issue order
  __builtin_amdgcn_sched_barrier(0);
  const AssignRegs ar = load_assign_regs(a.ap);   // scalar registers
  const int Np = (N + 127) & ~127;
  const int t0 = tile * kTile;
  const int ct = (Np - t0) < kTile ? (Np - t0) : kTile;   // multiple of 128
  const int pb = ct / 8;                                  // bytes per plane, multiple of 16
  const int rstride = pb * bmax;                          // bytes per row tile
  uint16_t sc[kCols], zr[kCols];
#pragma unroll
  for (int u = 0; u < kCols; ++u) {
    int col = tid + u * kVmmThreads;
    col = col < ct ? col : ct - 1;
    int gc = t0 + col;
    gc = gc < N ? gc : N - 1;
    sc[u] = scales[g * N + gc];
    zr[u] = zeros[g * N + gc];
  }

  if constexpr (kFused) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
      if (k0 + rq[e] < k1) bq[e] = bits_of(xq[e], ar);
  } else {
    // the listed rows of this group: positions [p0, p1) of the list, the
    // two searches in two waves at once (each is a chain of dependent loads)
    __shared__ int s_p[2];
    if (wid < 2) {
      const int64_t n = *a.n_active;
      const int64_t p = wave_lower_bound(a.active_idx, n, wid == 0 ? k0 : k1);
      if (lane == 0) s_p[wid] = (int)p;
    }
    __syncthreads();
    const int p0 = s_p[0];
    int m = s_p[1] - p0;
    m = m < 0 ? 0 : (m > kMaxRows ? kMaxRows : m);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int q = lane + 64 * e;
      if (q < m) {
        const int64_t i = a.active_idx[p0 + q];
        if (i >= k0 && i < k1) {   // a well-formed list always is
          rq[e] = (int)(i - k0);
          uint32_t bb = a.bits[i];
          bq[e] = bb > (uint32_t)bmax ? (uint32_t)bmax : bb;
          xq[e] = x[i];
        }
      }
    }
  }

  // ---- bucket the rows by width with ballots (every wave, no LDS): rows of
  // width v, in lane order (first set, then second set), get ranks 0, 1, ...;
  // rank r of width v -> couple cb_v + r / 4, place r % 4
  int cnt[9];
  uint64_t msk[2][9];
#pragma unroll
  for (int v = 1; v <= 8; ++v) {
    msk[0][v] = __ballot(bq[0] == (uint32_t)v);
    msk[1][v] = __ballot(bq[1] == (uint32_t)v);
    cnt[v] = __popcll(msk[0][v]) + __popcll(msk[1][v]);
  }
  int cbv[10];   // first couple of each width; cbv[9] = number of couples
  cbv[0] = 0;
  cbv[1] = 0;
#pragma unroll
  for (int v = 1; v <= 8; ++v) cbv[v + 1] = cbv[v] + ((cnt[v] + 3) >> 2);
  const int ncp = cbv[9];
  const int nrec = ncp > wid ? (ncp - wid + kWaves - 1) / kWaves : 0;   // this wave's couples

  if (wid == kWaves - 1) {
    // H = sum x phi and X = sum x over the group's active rows (the last
    // wave has the fewest records, so this stays off the longest path)
    float hs = 0.0f, xs = 0.0f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float xf = bq[e] > 0 ? half_bits_to_float(xq[e]) : 0.0f;
      hs += phi_x((int)bq[e], bmax, xf);
      xs += xf;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      hs += __shfl_xor(hs, off, 64);
      xs += __shfl_xor(xs, off, 64);
    }
    if (lane == 0) {
      s_hx[0] = hs;
      s_hx[1] = xs;
    }
  }

  // ---- this wave's records: every lane writes the source offset and x of
  // its own rows that fall into one of them; lanes 0..3 mark padding rows
  uint32_t* const src = s_src[wid];
  uint32_t* const cx = s_cx[wid];
  // lane j < kMaxRecords describes record j (couple wid + 8 j): its width
  // (0 if the wave has no such record) and, for a width's last couple, the
  // padding places, all in vector registers at once
  int rec_w = 0;
  {
    const int k = wid + kWaves * lane;
    if (lane < kMaxRecords && k < ncp) {
      int v = 1;
#pragma unroll
      for (int u = 2; u <= 8; ++u) v += k >= cbv[u] ? 1 : 0;
      int cv = 0, cbs = 0;
#pragma unroll
      for (int u = 1; u <= 8; ++u) {
        cv = u == v ? cnt[u] : cv;
        cbs = u == v ? cbv[u] : cbs;
      }
      const int nreal = cv - 4 * (k - cbs);        // rows present in this couple (>= 1)
      for (int t = nreal; t < 4; ++t) {
        src[4 * lane + t] = kOutOfRange;
        reinterpret_cast<uint16_t*>(cx)[4 * lane + t] = 0;
      }
      rec_w = v;
    }
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t b = bq[e];
    if (b > 0) {
      int rank = 0, cb = 0;
#pragma unroll
      for (int v = 1; v <= 8; ++v) {
        if (b == (uint32_t)v) {
          rank = (e == 1 ? __popcll(msk[0][v]) : 0) +
                 (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(msk[e][v] >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)msk[e][v], 0u));
          cb = cbv[v];
        }
      }
      const int k = cb + (rank >> 2);
      if ((k & (kWaves - 1)) == wid) {
        const int j = k / kWaves;
        src[4 * j + (rank & 3)] = (uint32_t)rq[e] * (uint32_t)rstride;
        reinterpret_cast<uint16_t*>(cx)[4 * j + (rank & 3)] = xq[e];
      }
    }
  }

  // buffer descriptor over this group's row tiles of the tile block
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(planes + store_offset((int64_t)t0 * K + (int64_t)k0 * ct, bmax)), (short)0,
      (k1 - k0) * rstride, kRsrcWord3);

  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.0f;
  // the prologue's own loads (x, scale, zero) have landed long ago; from here
  // on vmcnt counts only record loads
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if constexpr (kParkScales) {
#pragma unroll
    for (int u = 0; u < kCols; ++u) s_scz[tid + u * kVmmThreads] = (uint32_t)sc[u] | ((uint32_t)zr[u] << 16);
  }
  {
    // Three records in flight.  The record sequence is unrolled (8- and
    // 4-wave workgroups: at most 5 and 10 records a wave) or rolled over
    // rounds of three (2-wave workgroups) so that the load order is static:
    // record j + 3 is issued into the registers of record j right after j is
    // consumed, and the compiler's wait counts let j + 1 and j + 2 stay
    // outstanding.  Records past nrec load nothing (width 0) and are not
    // computed.
    const int h = (tid >> 5) & 1;
    const uint32_t lane_off = 4 * (tid & 31) < pb ? 4u * (uint32_t)(tid & 31) : kOutOfRange;
    auto width = [&](int j) { return j < kMaxRecords ? __builtin_amdgcn_readlane(rec_w, j) : 0; };
    RecordRegs rr[3];
    int bw[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      bw[j] = width(j);
      load_record<kMaxRecords>(rr[j], rsrc, src, j, bw[j], pb, lane_off);
    }
    if constexpr (kMaxRecords <= 12) {
#pragma unroll
      for (int j = 0; j < kMaxRecords; ++j) {
        if (j < nrec) compute_record(rr[j % 3], bw[j % 3], cx[2 * j + h], acc);
        if (j + 3 < kMaxRecords) {
          bw[j % 3] = width(j + 3);
          load_record<kMaxRecords>(rr[j % 3], rsrc, src, j + 3, bw[j % 3], pb, lane_off);
        }
      }
    } else {
      // too many records to unroll (2-wave workgroups): a rolled loop over
      // rounds of three, the three register sets in fixed roles, so that the
      // load order and the wait counts stay static; records past the wave's
      // last load nothing (width 0)
      for (int j0 = 0; j0 < nrec; j0 += 3) {
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const int j = j0 + q;
          if (j < nrec) compute_record(rr[q], bw[q], cx[2 * j + h], acc);
          bw[q] = width(j + 3);
          load_record<kMaxRecords>(rr[q], rsrc, src, j + 3, bw[q], pb, lane_off);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  // ---- the two halves of a wave hold the same columns (different pairs):
  // one lane-half swap per two accumulators leaves column 2c + h of the
  // lane's word, summed over both halves, in half h; then reduce the waves
  // in LDS (row stride 33 keeps both the writes and the column-wise reads
  // free of bank conflicts)
  const int m = ncp;   // couples (0: no active row)
  float* red = s_red;
  {
    const int hh = lane >> 5;
    float* dst = red + (wid * 32 + (lane & 31)) * kRedStride + hh;
#pragma unroll
    for (int c = 0; c < 16; ++c) dst[2 * c] = halves_sum(acc[2 * c], acc[2 * c + 1]);
  }
  __syncthreads();
  const float H = s_hx[0];
  const float X = s_hx[1];
  // codes entered as c 2^-24 and stand at q 2^(8 - b_max)
  const float afac = __builtin_bit_cast(float, (uint32_t)(127 + 24) << 23);
  const float sfac = __builtin_bit_cast(float, (uint32_t)(127 + bmax - 8) << 23);
  float val[kCols];
#pragma unroll
  for (int u = 0; u < kCols; ++u) {
    val[u] = 0.0f;
    const int col = tid + u * kVmmThreads;
    if (m > 0 && col < ct && t0 + col < N) {
      float A = 0.0f;
#pragma unroll
      for (int h = 0; h < kWaves; ++h) A += red[(h * 32 + (col >> 5)) * kRedStride + (col & 31)];
      uint16_t su = sc[u], zu = zr[u];
      if constexpr (kParkScales) {
        const uint32_t p = s_scz[col];
        su = (uint16_t)(p & 0xFFFFu);
        zu = (uint16_t)(p >> 16);
      }
      val[u] = (half_bits_to_float(su) * sfac) * (A * afac + H) + half_bits_to_float(zu) * X;
    }
  }

  if constexpr (kOut == kOutAccumulate) {
    if (m > 0) {
#pragma unroll
      for (int u = 0; u < kCols; ++u) {
        const int col = tid + u * kVmmThreads;
        if (col < ct && t0 + col < N)
          __hip_atomic_fetch_add(a.y + t0 + col, val[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // the caller's next output buffer, zeroed once per column (split 0 only)
    if (a.clear && split == 0) {
#pragma unroll
      for (int u = 0; u < kCols; ++u) {
        const int col = tid + u * kVmmThreads;
        if (col < ct && t0 + col < N) a.clear[t0 + col] = 0.0f;
      }
    }
    return;
  } else {
    if (a.splits == 1) {
#pragma unroll
      for (int u = 0; u < kCols; ++u) {
        const int col = tid + u * kVmmThreads;
        if (col < ct && t0 + col < N) a.y[t0 + col] = val[u];
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < kCols; ++u) {
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
    float sum[kCols];
#pragma unroll
    for (int e = 0; e < kCols; ++e) sum[e] = 0.0f;
    constexpr int kRound = 64 / kCols;   // splits per round (loads in flight per thread: 64)
    // kRound splits per round, all loads of a round in flight together;
    // splits past the end read as zero (out-of-range offsets); the sum runs
    // in split order
    for (int sp0 = 0; sp0 < a.splits; sp0 += kRound) {
      uint32_t v[kRound][kCols];
#pragma unroll
      for (int u = 0; u < kRound; ++u)
#pragma unroll
        for (int e = 0; e < kCols; ++e) {
          const int col = tid + e * kVmmThreads;
          const bool ok = sp0 + u < a.splits && col < ct;
          const uint32_t off = ok ? (uint32_t)(sp0 + u) * row_bytes + 4u * (uint32_t)col : kOutOfRange;
          v[u][e] = __builtin_amdgcn_raw_buffer_load_b32(prs, (int)off, 0, kScopeDevice);
        }
#pragma unroll
      for (int u = 0; u < kRound; ++u)
#pragma unroll
        for (int e = 0; e < kCols; ++e) sum[e] += __builtin_bit_cast(float, v[u][e]);
    }
#pragma unroll
    for (int e = 0; e < kCols; ++e) {
      const int col = tid + e * kVmmThreads;
      if (col < ct && t0 + col < N) a.y[t0 + col] = sum[e];
    }
    if (tid == 0) __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int kWaves>
static void launch_shape(bool fused, int out_mode, dim3 grid, const VmmArgs& a, hipStream_t s) {
  const dim3 block(64 * kWaves);
#define GRINQH_VMM_LAUNCH(F, O)                                                                              \
  hipLaunchKernelGGL((vmm_kernel<F, O, kWaves>), grid, block, 0, s, a.x, a.planes, a.scales, a.zeros, (int)a.K, \
                     (int)a.N, a.tiles, a.rows, a.bmax, a)
  if (out_mode == kOutAccumulate) {
    if (fused)
      GRINQH_VMM_LAUNCH(true, kOutAccumulate);
    else
      GRINQH_VMM_LAUNCH(false, kOutAccumulate);
  } else {
    if (fused)
      GRINQH_VMM_LAUNCH(true, kOutSplitK);
    else
      GRINQH_VMM_LAUNCH(false, kOutSplitK);
  }
#undef GRINQH_VMM_LAUNCH
}

static int launch_vmm(bool fused, int out_mode, VmmArgs& a, void* ws, hipStream_t s) {
  const VmmGeometry g = vmm_geometry(a.K, a.N);
  if (g.splits * g.tiles > 0x7FFFFFFF)
    return fail(GRINQH_EINVAL, "%lld workgroups: more than one launch handles", (long long)(g.splits * g.tiles));
  if (g.partial_floats * 4 >= (int64_t)kOutOfRange)
    return fail(GRINQH_EINVAL, "K x N too large for one split-K workspace (%lld partial floats)",
                (long long)g.partial_floats);
  a.splits = (int)g.splits;
  a.tiles = (int)g.tiles;
  a.rows = (int)g.rows_per_split;
  a.partials = reinterpret_cast<float*>(ws);
  a.counters = g.bytes > 0 && ws ? reinterpret_cast<unsigned*>(reinterpret_cast<char*>(ws) + g.counter_offset) : nullptr;
  const dim3 grid((unsigned)(g.splits * g.tiles));
  if (g.waves == 2)
    launch_shape<2>(fused, out_mode, grid, a, s);
  else if (g.waves == 4)
    launch_shape<4>(fused, out_mode, grid, a, s);
  else
    launch_shape<8>(fused, out_mode, grid, a, s);
  return check_launch(out_mode == kOutAccumulate ? "grinqh_decode_vmm_accumulate"
                                                 : (fused ? "grinqh_decode_vmm" : "grinqh_vmm"));
}

int launch_vmm_list(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                    const uint16_t* x, const uint8_t* bits, const int32_t* active_idx,
                    const int32_t* n_active, int64_t K, int64_t N, int bmax, float* y, void* ws,
                    hipStream_t s) {
  VmmArgs a{};
  a.planes = planes; a.scales = scales; a.zeros = zeros; a.x = x;
  a.bits = bits; a.active_idx = active_idx; a.n_active = n_active;
  a.y = y; a.K = K; a.N = N; a.bmax = bmax;
  return launch_vmm(false, kOutSplitK, a, ws, s);
}

int launch_vmm_fused(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                     const uint16_t* x, int64_t K, int64_t N, int bmax, const AssignParams& ap,
                     float* y, void* ws, hipStream_t s) {
  VmmArgs a{};
  a.planes = planes; a.scales = scales; a.zeros = zeros; a.x = x;
  a.y = y; a.K = K; a.N = N; a.bmax = bmax; a.ap = ap;
  return launch_vmm(true, kOutSplitK, a, ws, s);
}

int launch_vmm_accumulate(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                          const uint16_t* x, int64_t K, int64_t N, int bmax, const AssignParams& ap,
                          float* y, float* clear, hipStream_t s) {
  VmmArgs a{};
  a.planes = planes; a.scales = scales; a.zeros = zeros; a.x = x;
  a.y = y; a.clear = clear; a.K = K; a.N = N; a.bmax = bmax; a.ap = ap;
  return launch_vmm(true, kOutAccumulate, a, nullptr, s);
}

}  // namespace grinqh
