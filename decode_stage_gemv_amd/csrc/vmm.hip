// Decode-stage VMM over the bit-plane store (GRINQH paper, section 3.3
// "Weight Reconstruction and Bias Correction"; Appendix C.1).
//
// Work split.  A workgroup owns one column tile (one row tile of the store
// per row, ct <= 1024 columns) and S consecutive sub-items of K: a sub-item is
// 128 (or 64) rows inside one 128-row group, so every row it touches shares
// one (scale, zero) row.  Large layers use 16-wave workgroups holding S = 2, 4
// or 8 sub-items (8, 4 or 2 waves each), one workgroup per CU: the sub-items
// run side by side and the epilogue adds their results, each with its own
// scale and zero, into one output per column.  Where that would leave CUs
// idle, 4-wave workgroups of one 128-row sub-item share the CUs, and small
// layers use 8-wave workgroups of one 64-row sub-item (choose_shape).
//
// Row order.  Every wave sees all rows of its sub-item (two per lane, one in
// the 64-row sub-items of the small-layer shape) and
// buckets the active ones by bit width b with ballots, in registers.  Each
// bucket is cut into "couples" of four rows of one width (the last couple of
// a bucket is padded with empty rows: x = 0, no bytes).  A couple is two row
// pairs; the two 32-lane halves of a wave take one pair each, lane l owning
// 32 columns (one plane word of each row), so the bit width is the same for
// the whole wave.  Couple k belongs to the sub-item's wave whose turn is
// k mod W, W its waves (8, 4 or 2; its "records", in order); the turns start
// at a different wave in each sub-item of a workgroup, so the waves that get
// one couple more sit on different SIMDs.
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
constexpr int kRedStride = 33;                   // LDS row stride of the wave reduction
// Launch shape.  The grid is (item, column tile) pairs; an item is S
// sub-items of R rows (R = 128, or 64 on small layers).  The shapes are
// 16-wave workgroups with S = 1, 2, 4 or 8 (a sub-item then has 16, 8, 4 or
// 2 waves, each taking more records, in a rolled loop at 2 waves), 4-wave
// workgroups with one 128-row sub-item (several per CU, for layers whose
// 16-wave grid would leave CUs idle), and 8-wave workgroups with one 64-row
// sub-item (small layers); choose_shape picks one per layer.  One workgroup
// per CU keeps a CU's loads and arithmetic in one schedule, and the
// sub-items' output rows are added before they leave the workgroup.
constexpr int kTargetCUs = 256;                  // MI355X
constexpr uint32_t kOutOfRange = 0x7FFFFF00u;    // buffer offset beyond any range used here
constexpr int kRsrcWord3 = 0x00020000;           // raw 32-bit buffer, gfx9 family
constexpr int kScopeDevice = 16;                 // cache-policy bits: sc1 = device scope
// s_waitcnt immediates (gfx9 encoding): vmcnt in bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]; all-ones fields mean "do not wait".
constexpr int kWaitVm0 = 0x0F70;                 // vmcnt(0) only
// Fixed-point split-K reduction: at most 64 splits (one bit each in the
// 64-bit mask of float partials; the arrival count takes 7 bits), partials
// below 2^22 in magnitude go as integers in units of 2^-20 (their rounding,
// at most 2^-21 each, is the only difference from an exact sum), offset by
// 2^42 so that every added value lies in [0, 2^43]: 64 of them stay below
// 2^50, the top of the value field.
constexpr int kFixedMaxSplits = 64;
constexpr int kFixedFrac = 20;
constexpr int kFixedOffsetBit = 42;
constexpr float kFixedLimit = 4194304.0f;        // 2^22

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Timeline build (GRINQH_TIMELINE defined, libgrinqh_timeline.so): wave 0 of
// each workgroup (or every wave, for the per-wave slots) records the 100 MHz
// constant clock at fixed points of a plain launch into a device array, which
// grinqh_timeline_read copies out; the ordinary build compiles none of it.
// The empty asm statements keep the compiler from moving a stamp across the
// memory operations around it.
#ifdef GRINQH_TIMELINE
constexpr int kTimelineWGs = GRINQH_TIMELINE_WORKGROUPS;
constexpr int kTimelineSlots = GRINQH_TIMELINE_SLOTS;
__device__ unsigned long long g_timeline[kTimelineWGs * kTimelineSlots];
#define GRINQH_STAMP(slot, cond)                                                             \
  do {                                                                                       \
    asm volatile("" ::: "memory");                                                           \
    if ((cond) && blockIdx.x < (unsigned)kTimelineWGs)                                       \
      g_timeline[(size_t)blockIdx.x * kTimelineSlots + (slot)] = __builtin_amdgcn_s_memrealtime(); \
    asm volatile("" ::: "memory");                                                           \
  } while (0)
#else
#define GRINQH_STAMP(slot, cond) \
  do {                           \
  } while (0)
#endif

// The shape of one workgroup: waves, sub-items and rows per sub-item.
struct VmmShape {
  int waves, subs, rows;
};

// Rows of a sub-item of each shape: 64 in the 8-wave single-item shape (small
// layers), 128 in the others.  A grouped launch's kernel takes it from here
// rather than from an argument.
__host__ __device__ constexpr int group_rows(int waves, int subs) { return waves == 8 && subs == 1 ? 64 : 128; }

// Pick the workgroup shape whose busiest CU holds the fewest rows, among
// shapes whose whole grid is resident at once (at most 16 waves per CU, the
// kernels' occupancy); ties go to the larger workgroup (one schedule per
// CU).  Measured per layer on MI355X: 128-row sub-items beat 64-row ones
// except on small layers, where a 64-row item doubles the workgroups.  The
// set of shapes is kept small on purpose: a decode pass alternates layers,
// and each kernel is tens of KB of code, so layers that share a kernel find
// its code still in the instruction cache.
static VmmShape choose_shape(int64_t K, int64_t N) {
  static const VmmShape kShapes[] = {{16, 2, 128}, {16, 4, 128}, {16, 8, 128}, {4, 1, 128}, {8, 1, 64}};
  const int64_t tiles = n_tiles(N);
  VmmShape best = {16, 8, 128};   // layers too large for one round
  int64_t best_rows = -1;
  for (const VmmShape& c : kShapes) {
    const int64_t wgs = (K + (int64_t)c.rows * c.subs - 1) / ((int64_t)c.rows * c.subs) * tiles;
    const int64_t per_cu = (wgs + kTargetCUs - 1) / kTargetCUs;
    if (per_cu * c.waves > 16) continue;
    const int64_t rows = per_cu * c.subs * c.rows;
    if (best_rows < 0 || rows < best_rows || (rows == best_rows && c.waves > best.waves)) {
      best = c;
      best_rows = rows;
    }
  }
  return best;
}

VmmGeometry vmm_geometry(int64_t K, int64_t N) {
  VmmGeometry g;
  g.tiles = n_tiles(N);
  const VmmShape sh = choose_shape(K, N);
  g.rows_per_split = sh.rows;
  g.subs = sh.subs;
  g.waves = sh.waves;
  const int64_t item = g.rows_per_split * g.subs;
  g.splits = (K + item - 1) / item;
  g.partial_floats = g.splits > 1 ? g.splits * padded_cols(N) : 0;
  g.counter_offset = (g.partial_floats * 4 + 255) / 256 * 256;
  g.words_offset = (g.counter_offset + g.tiles * 4 + 255) / 256 * 256;
  g.bytes = g.splits > 1 ? g.words_offset + 2 * padded_cols(N) * 8 : 0;
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
  unsigned long long* acc_words;    // split-K, up to kFixedMaxSplits: one word per column
  unsigned long long* mask_words;   // ... and one mask of the splits that sent a float partial
  int64_t K, N;
  int splits, tiles, rows;
  int bmax;   // planes per row of the store (1..8)
  AssignParams ap;
  VmmGroup group;   // grouped launches only
};

// First position p in [0, n) with idx[p] >= key (n if none); one full wave.
// The first probe reads the 64 entries around `hint` (where the key would
// sit if the listed rows were spread evenly over [0, K)): for a list of that
// kind it nearly always brackets the key, one round trip instead of two or
// three; otherwise it still narrows the range and the search goes on.
__device__ int64_t wave_lower_bound(const int32_t* __restrict__ idx, int64_t n, int64_t key, int64_t hint) {
  const int lane = threadIdx.x & 63;
  int64_t lo = 0, hi = n;
  if (n > 64) {
    int64_t base = hint - 32;
    base = base < 0 ? 0 : (base > n - 64 ? n - 64 : base);
    const uint64_t m = __ballot(idx[base + lane] >= key);
    if (m == 0) {
      lo = base + 64;   // every probed entry is below the key
    } else if (m & 1ull) {
      hi = base;        // the first probed entry already reaches it: p <= base
    } else {
      return base + (__ffsll((unsigned long long)m) - 1);
    }
  }
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

// v moved by one DPP control (rows past row_mask, and lanes shifted in from
// outside a row, read 0).
template <int kCtrl, int kRowMask>
__device__ inline float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, true));
}

// Sum of v over the wave, in every lane: inclusive sums inside each 16-lane
// row (shifts by 1, 2, 4, 8), row 15's total into rows 1 and 3, row 31's
// into rows 2 and 3, then lane 63's value read out.
__device__ inline float wave_total(float v) {
  v += dpp_f32<0x111, 0xF>(v);   // row_shr:1
  v += dpp_f32<0x112, 0xF>(v);   // row_shr:2
  v += dpp_f32<0x114, 0xF>(v);   // row_shr:4
  v += dpp_f32<0x118, 0xF>(v);   // row_shr:8
  v += dpp_f32<0x142, 0xA>(v);   // row_bcast:15
  v += dpp_f32<0x143, 0xC>(v);   // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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
// levels) completes while the activations are in flight.  kMulti: a grouped
// launch, where the same leading arguments carry the members' activation
// pointers and workgroup ranges instead, so a workgroup finds its member and
// starts its activation loads from registers; the member's other pointers,
// shape and thresholds follow from the argument block (a few scalar loads).
template <bool kFused, int kOut, int kWaves, int kSubs, bool kMulti = false>
__global__ __launch_bounds__(64 * kWaves) void vmm_kernel(const uint16_t* __restrict__ x_arg,
                                                          const uint8_t* __restrict__ planes_arg,
                                                          const uint16_t* __restrict__ scales_arg,
                                                          const uint16_t* __restrict__ zeros_arg, int K, int N_arg,
                                                          int tiles_arg, int rows, int bmax, VmmArgs a) {
  static_assert(!kMulti || (kFused && kOut == kOutAccumulate), "grouped launches accumulate");
  constexpr int kVmmThreads = 64 * kWaves;
  constexpr int kSubWaves = kWaves / kSubs;         // waves per sub-item
  constexpr int kCols = kTile / kVmmThreads;        // output columns per thread in the epilogue
  // couples of a sub-item: at most rows / 4 + 6 (sum over 8 widths of ceil(c_v / 4))
  constexpr int kMaxRecords = (group_rows(kWaves, kSubs) / 4 + 6 + kSubWaves - 1) / kSubWaves;
  constexpr int kRedWords = kWaves * 32 * kRedStride;
  constexpr int kGroupRows = group_rows(kWaves, kSubs);   // a grouped launch's sub-item rows
  __shared__ float s_red[kRedWords];                      // wave reduction
  __shared__ uint32_t s_src[kWaves][kMaxRecords * 4];     // per wave: record row -> source byte offset
  __shared__ uint32_t s_cx[kWaves][kMaxRecords * 2];      // per wave: record pair -> fp16 x of its rows
  __shared__ float s_hx[kSubs][2];                        // per sub-item: H and X
  __shared__ int s_ncp[kSubs];                            // per sub-item: couples (0: no active row)
  __shared__ int s_last;
  // more than two sub-items: each thread's scales and zeros (one pair per
  // sub-item and column) are parked in LDS during the record loop (registers
  // are short)
  constexpr bool kParkScales = kSubs > 2;
  __shared__ uint32_t s_scz[kParkScales ? kSubs * kTile : 1];

  const uint16_t* __restrict__ x = x_arg;
  const uint8_t* __restrict__ planes = planes_arg;
  const uint16_t* __restrict__ scales = scales_arg;
  const uint16_t* __restrict__ zeros = zeros_arg;
  int N = N_arg, tiles = tiles_arg;
  float* out = a.y;
  float* clear = a.clear;
  AssignParams apm;
  const AssignParams* ap = &a.ap;
  int bid = blockIdx.x;
  int tile, split;
  if constexpr (kMulti) {
    // Grouped launch: the preloaded leading arguments carry every member's
    // activation pointer (x_arg, planes_arg, scales_arg, zeros_arg: members
    // 0..3) and the first workgroup of members 1..3 (N_arg, tiles_arg, rows;
    // past the grid for absent members), so the member and its activations
    // need no memory access.  Inside a member the workgroups run split
    // fastest, so its rows do not depend on its tile count; the member's
    // other fields (scalar loads) arrive while the activations load.
    const int m = (bid >= N_arg ? 1 : 0) + (bid >= tiles_arg ? 1 : 0) + (bid >= rows ? 1 : 0);
    bid -= m == 0 ? 0 : (m == 1 ? N_arg : (m == 2 ? tiles_arg : rows));
    x = m == 0 ? x_arg
               : (m == 1 ? reinterpret_cast<const uint16_t*>(planes_arg) : (m == 2 ? scales_arg : zeros_arg));
    rows = kGroupRows;
    constexpr int kItem = kGroupRows * kSubs;
    const int splits = (K + kItem - 1) / kItem;
    split = bid % splits;
    tile = bid / splits;
    const VmmMember& mb = a.group.m[m];
    planes = mb.planes;
    scales = mb.scales;
    zeros = mb.zeros;
    N = mb.N;
    tiles = mb.tiles;
    out = mb.y;
    clear = mb.clear;
    apm = mb.ap;
    ap = &apm;
  } else {
    // workgroup = (column tile, item of kSubs sub-items), tiles fastest (K, N < 2^31)
    tile = bid % tiles;
    split = bid / tiles;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  if constexpr (!kMulti) GRINQH_STAMP(0, tid == 0);   // timeline: start
  const int sub = wid / kSubWaves;              // this wave's sub-item
  const int swid = wid - sub * kSubWaves;       // the wave's index within it
  const int kitem = split * rows * kSubs;       // first row of the item
  // this wave's sub-item: rows [k0, k1), empty past K
  const int k0 = kitem + sub * rows < K ? kitem + sub * rows : K;
  const int k1 = (k0 + rows) < K ? (k0 + rows) : K;
  const int64_t G = (K + kGroup - 1) / kGroup;
  const int64_t g = k0 / kGroup < G ? k0 / kGroup : G - 1;   // its scale group (clamped when empty)

  // ---- every wave sees all rows of the group, two per lane (lane and lane
  // + 64): activation loads first, then scale and zero of this thread's two
  // output columns (tid, tid + 512).  Loads are unconditional (clamped
  // index, validity applied later) so nothing waits on them early.
  // rows per lane: two for 128-row sub-items, one for 64-row ones (whose
  // second set would always be empty: no loads, compares or ballots for it)
  constexpr int kRPL = group_rows(kWaves, kSubs) / 64;
  uint32_t bq[2] = {0u, 0u};   // bit width of the lane's rows
  uint16_t xq[2] = {0, 0};     // their fp16 activations
  int rq[2] = {0, 0};          // their rows within the group
  if constexpr (kFused) {
#pragma unroll
    for (int e = 0; e < kRPL; ++e) {
      const int64_t i = k0 + lane + 64 * e;
      xq[e] = x[i < k1 ? i : (k1 > k0 ? k1 - 1 : K - 1)];
      rq[e] = lane + 64 * e;
    }
  }
  // keep the activation loads ahead of everything else: they need only the
  // preloaded arguments, and waits count loads in issue order
  __builtin_amdgcn_sched_barrier(0);
  const AssignRegs ar = load_assign_regs(*ap);   // scalar registers
  const int Np = (N + 127) & ~127;
  const int t0 = tile * kTile;
  const int ct = (Np - t0) < kTile ? (Np - t0) : kTile;   // multiple of 128
  const int pb = ct / 8;                                  // bytes per plane, multiple of 16
  const int rstride = pb * bmax;                          // bytes per row tile
  // scale and zero of every sub-item for this thread's epilogue columns
  uint16_t sc[kSubs][kCols], zr[kSubs][kCols];
#pragma unroll
  for (int si = 0; si < kSubs; ++si) {
    int64_t gs = (int64_t)(kitem + si * rows) / kGroup;
    gs = gs < G ? gs : G - 1;
#pragma unroll
    for (int u = 0; u < kCols; ++u) {
      int col = tid + u * kVmmThreads;
      col = col < ct ? col : ct - 1;
      int gc = t0 + col;
      gc = gc < N ? gc : N - 1;
      sc[si][u] = scales[gs * N + gc];
      zr[si][u] = zeros[gs * N + gc];
    }
  }
  if constexpr (kOut == kOutAccumulate) {
    // the caller's next output buffer, zeroed once per column (split 0 only)
    if (clear && split == 0) {
#pragma unroll
      for (int u = 0; u < kCols; ++u) {
        const int col = tid + u * kVmmThreads;
        // device scope: written through to the level every XCD reads, so
        // the line is not left dirty in this XCD's L2 for the end of the
        // kernel to write back (measured 0.05-0.45 us faster per launch)
        if (col < ct && t0 + col < N)
          __hip_atomic_store(clear + t0 + col, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  if constexpr (kFused) {
    // both rows' activations were loaded from clamped indexes: widths of
    // rows past the sub-item are dropped afterwards
    uint32_t b0, b1 = 0;
    if constexpr (kRPL == 2)
      bits_of2(xq[0], xq[1], ar, b0, b1);
    else
      b0 = bits_of(xq[0], ar);
    bq[0] = k0 + rq[0] < k1 ? b0 : 0u;
    bq[1] = kRPL == 2 && k0 + rq[1] < k1 ? b1 : 0u;
#ifdef GRINQH_TIMELINE
    asm volatile("" ::"v"(bq[0]), "v"(bq[1]));
#endif
    if constexpr (!kMulti) GRINQH_STAMP(1, tid == 0);   // timeline: widths known
  } else {
    // the listed rows of this group: positions [p0, p1) of the list, the
    // two searches in two waves at once (each is a chain of dependent loads)
    __shared__ int s_p[kSubs][2];
    if (swid < 2) {
      // a count outside [0, K] (not from a well-formed list) is clamped, so
      // the searches stay inside the K entries the list buffer must hold
      int64_t n = *a.n_active;
      n = n < 0 ? 0 : (n > a.K ? a.K : n);
      const int64_t key = swid == 0 ? k0 : k1;
      const int64_t p = wave_lower_bound(a.active_idx, n, key, key * n / a.K);
      if (lane == 0) s_p[sub][swid] = (int)p;
    }
    __syncthreads();
    const int p0 = s_p[sub][0];
    int m = s_p[sub][1] - p0;
    m = m < 0 ? 0 : (m > kMaxRows ? kMaxRows : m);
#pragma unroll
    for (int e = 0; e < kRPL; ++e) {
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
    msk[1][v] = kRPL == 2 ? __ballot(bq[1] == (uint32_t)v) : 0ull;
    cnt[v] = __popcll(msk[0][v]) + __popcll(msk[1][v]);
  }
  int cbv[10];   // first couple of each width; cbv[9] = number of couples
  cbv[0] = 0;
  cbv[1] = 0;
#pragma unroll
  for (int v = 1; v <= 8; ++v) cbv[v + 1] = cbv[v] + ((cnt[v] + 3) >> 2);
  const int ncp = cbv[9];
#ifdef GRINQH_TIMELINE
  asm volatile("" ::"s"(ncp));
#endif
  if constexpr (!kMulti) GRINQH_STAMP(2, tid == 0);   // timeline: buckets counted
  // Couples go to the sub-item's waves in turn.  Wave w runs on SIMD w mod 4,
  // and the waves that get one couple more are the first turns, so each
  // sub-item starts its turns on a different SIMD: rot is the wave (within
  // the sub-item) that takes turn 0.
  int rot = 0;
  if constexpr (kSubs == 2) rot = 2 * sub;              // 8 waves each: turn 0 on SIMD 0, 2
  else if constexpr (kSubs == 4) rot = sub;             // 4 waves each: SIMD 0, 1, 2, 3
  else if constexpr (kSubs == 8) rot = (sub >> 1) & 1;  // 2 waves each, on SIMDs 2s mod 4 and + 1
  const int cw = (swid + kSubWaves - rot) & (kSubWaves - 1);   // the wave's turn
  const int nrec = ncp > cw ? (ncp - cw + kSubWaves - 1) / kSubWaves : 0;   // this wave's couples

  if (cw == kSubWaves - 1) {
    // H = sum x phi and X = sum x over the sub-item's active rows (the last
    // turn has the fewest records, so this stays off the longest path)
    float hs = 0.0f, xs = 0.0f;
#pragma unroll
    for (int e = 0; e < kRPL; ++e) {
      const float xf = bq[e] > 0 ? half_bits_to_float(xq[e]) : 0.0f;
      hs += phi_x((int)bq[e], bmax, xf);
      xs += xf;
    }
    hs = wave_total(hs);
    xs = wave_total(xs);
    if (lane == 0) {
      s_hx[sub][0] = hs;
      s_hx[sub][1] = xs;
      s_ncp[sub] = ncp;
    }
  }

  // ---- this wave's records: every slot of the wave's table starts as a
  // padding row (out-of-range source, x = 0), then every lane writes the
  // source offset and x of its own rows that fall into one of the records
  // over it (one wave's LDS writes land in program order)
  uint32_t* const src = s_src[wid];
  uint32_t* const cx = s_cx[wid];
#pragma unroll
  for (int i = 0; i < kMaxRecords * 4; i += 64)
    if (i + lane < kMaxRecords * 4) src[i + lane] = kOutOfRange;
#pragma unroll
  for (int i = 0; i < kMaxRecords * 4; i += 64)   // as halves: the rows' writes below are halves too
    if (i + lane < kMaxRecords * 4) reinterpret_cast<uint16_t*>(cx)[i + lane] = 0;
  // lane j < kMaxRecords holds the width of record j (couple cw + W j; 0 if
  // the wave has no such record)
  int rec_w = 0;
  {
    const int k = cw + kSubWaves * lane;
    if (lane < kMaxRecords && k < ncp) {
      int v = 1;
#pragma unroll
      for (int u = 2; u <= 8; ++u) v += k >= cbv[u] ? 1 : 0;
      rec_w = v;
    }
  }
#pragma unroll
  for (int e = 0; e < kRPL; ++e) {
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
      if ((k & (kSubWaves - 1)) == cw) {
        const int j = k / kSubWaves;
        src[4 * j + (rank & 3)] = (uint32_t)rq[e] * (uint32_t)rstride;
        reinterpret_cast<uint16_t*>(cx)[4 * j + (rank & 3)] = xq[e];
      }
    }
  }

  // The record tables were written above by whichever lanes own the rows and
  // are read below by the other lanes of the same wave: a wave-scope fence
  // orders the LDS writes before the reads, and the wave barrier keeps the
  // compiler from moving either across this point.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if constexpr (!kMulti) GRINQH_STAMP(3, tid == 0);   // timeline: record tables written

  // buffer descriptor over this sub-item's row tiles of the tile block
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(planes + store_offset((int64_t)t0 * K + (int64_t)k0 * ct, bmax)), (short)0,
      (k1 - k0) * rstride, kRsrcWord3);

  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.0f;
  // The scale and zero loads may still be in flight (a cold group's come from
  // HBM): the record loads issue behind them without waiting, and the
  // compiler's counts wait for them only where they are used.  Parking them
  // in LDS uses them here.
  if constexpr (kParkScales) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
    for (int si = 0; si < kSubs; ++si)
#pragma unroll
      for (int u = 0; u < kCols; ++u)
        s_scz[si * kTile + tid + u * kVmmThreads] = (uint32_t)sc[si][u] | ((uint32_t)zr[si][u] << 16);
  }
  {
    // Three records in flight.  The record sequence is unrolled (8-wave
    // sub-items: at most 5 records a wave) or rolled over rounds of three
    // (sub-items of 4 or 2 waves: up to 10 or 19 records) so that the load
    // order is static:
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
    if constexpr (!kMulti) GRINQH_STAMP(4, tid == 0);   // timeline: first three records issued
    if constexpr (kMaxRecords <= 5) {
#pragma unroll
      for (int j = 0; j < kMaxRecords; ++j) {
        if (j < nrec) compute_record(rr[j % 3], bw[j % 3], cx[2 * j + h], acc);
        if (j + 3 < kMaxRecords) {
          bw[j % 3] = width(j + 3);
          load_record<kMaxRecords>(rr[j % 3], rsrc, src, j + 3, bw[j % 3], pb, lane_off);
        }
      }
    } else {
      // a rolled loop over rounds of three, the three register sets in fixed
      // roles, so that the load order and the wait counts stay static;
      // records past the wave's last load nothing (width 0).  Unrolled, each
      // record slot is a copy of the rebuild for every width (about 5 KB of
      // code): ten slots made a 55 KB kernel whose instruction fetches cost
      // more than the loop when layers alternate
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
#ifdef GRINQH_TIMELINE
  asm volatile("" ::"v"(acc[0]), "v"(acc[15]), "v"(acc[31]));
#endif
  if constexpr (!kMulti) GRINQH_STAMP(8 + wid, lane == 0);   // timeline: this wave's records done
  // ---- the two halves of a wave hold the same columns (different pairs):
  // one lane-half swap per two accumulators leaves column 2c + h of the
  // lane's word, summed over both halves, in half h; then reduce the waves
  // in LDS (row stride 33 keeps both the writes and the column-wise reads
  // free of bank conflicts)
  float* red = s_red;
  {
    const int hh = lane >> 5;
    float* dst = red + (wid * 32 + (lane & 31)) * kRedStride + hh;
#pragma unroll
    for (int c = 0; c < 16; ++c) dst[2 * c] = halves_sum(acc[2 * c], acc[2 * c + 1]);
  }
  __syncthreads();
  if constexpr (!kMulti) GRINQH_STAMP(5, tid == 0);   // timeline: waves reduced
  // codes entered as c 2^-24 and stand at q 2^(8 - b_max)
  const float afac = __builtin_bit_cast(float, (uint32_t)(127 + 24) << 23);
  const float sfac = __builtin_bit_cast(float, (uint32_t)(127 + bmax - 8) << 23);
  // sub-items with an active row (the epilogue adds only those)
  int mall = 0;
#pragma unroll
  for (int si = 0; si < kSubs; ++si) mall += s_ncp[si];
  const int m = mall;
  // per column: the sum over sub-items of s (A + H) + z X, each sub-item's
  // A summed over its waves, in wave order
  float val[kCols];
#pragma unroll
  for (int u = 0; u < kCols; ++u) {
    val[u] = 0.0f;
    const int col = tid + u * kVmmThreads;
    if (col < ct && t0 + col < N) {
#pragma unroll
      for (int si = 0; si < kSubs; ++si) {
        if (s_ncp[si] > 0) {
          float A = 0.0f;
#pragma unroll
          for (int h = 0; h < kSubWaves; ++h)
            A += red[((si * kSubWaves + h) * 32 + (col >> 5)) * kRedStride + (col & 31)];
          uint16_t su = sc[si][u], zu = zr[si][u];
          if constexpr (kParkScales) {
            const uint32_t p = s_scz[si * kTile + col];
            su = (uint16_t)(p & 0xFFFFu);
            zu = (uint16_t)(p >> 16);
          }
          val[u] += (half_bits_to_float(su) * sfac) * (A * afac + s_hx[si][0]) + half_bits_to_float(zu) * s_hx[si][1];
        }
      }
    }
  }

  if constexpr (kOut == kOutAccumulate) {
    if (m > 0) {
#pragma unroll
      for (int u = 0; u < kCols; ++u) {
        const int col = tid + u * kVmmThreads;
        if (col < ct && t0 + col < N)
          __hip_atomic_fetch_add(out + t0 + col, val[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#ifdef GRINQH_TIMELINE
    if constexpr (!kMulti) {
      GRINQH_STAMP(6, tid == 0);   // timeline: atomics issued
      __builtin_amdgcn_s_waitcnt(0);
      GRINQH_STAMP(7, tid == 0);   // timeline: atomics acknowledged
    }
#endif
    return;
  } else {
    if (a.splits == 1) {
#pragma unroll
      for (int u = 0; u < kCols; ++u) {
        const int col = tid + u * kVmmThreads;
        if (col < ct && t0 + col < N)   // device scope: no dirty line left for the kernel's end
          __hip_atomic_store(out + t0 + col, val[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
    if (a.splits <= kFixedMaxSplits) {
      // ---- exact, order-free accumulation (up to kFixedMaxSplits splits).
      // Every workgroup adds its partial sum p of a column, as the integer
      // round(p 2^kFixedFrac) offset by 2^kFixedOffsetBit, into the column's
      // 64-bit word with one device-scope atomic that also counts its
      // arrival (bits 57..63) and returns the old word.  Integer addition
      // does not depend on the order of the adds, so the total does not
      // depend on scheduling, and the thread whose add completes the count
      // turns the total into y and clears the word for the next call: one
      // round trip.  A partial too large for the fixed-point range, or not
      // finite, goes instead as a float to its slot of the partial rows
      // (acknowledged), then as the split's bit in the column's mask word
      // (acknowledged), and its add carries only the arrival and a count of
      // such partials (bits 50..56); the last thread then adds those floats
      // to the converted total in split order.  Each word holds at most
      // kFixedMaxSplits offset values of at most 2^(kFixedOffsetBit + 1), so
      // the value field (bits 0..49) never carries into the counts, and the
      // split's mask bit (1 << split) stays inside the 64-bit mask.
#pragma unroll
      for (int u = 0; u < kCols; ++u) {
        const int col = tid + u * kVmmThreads;
        if (col >= ct) continue;
        const int64_t j = t0 + col;
        const float pv = val[u];
        unsigned long long add = 1ull << 57;
        if (__builtin_fabsf(pv) < kFixedLimit) {
          const float sc = pv * __builtin_bit_cast(float, (uint32_t)(127 + kFixedFrac) << 23);   // exact
          add += (unsigned long long)((long long)__builtin_rintf(sc) + (1ll << kFixedOffsetBit));
        } else {
          __hip_atomic_store(a.partials + (int64_t)split * Np + j, pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_s_waitcnt(0);
          const unsigned long long prev =
              __hip_atomic_fetch_or(a.mask_words + j, 1ull << split, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          asm volatile("" ::"v"(prev));   // the OR has returned before the add below
          add += 1ull << 50;
        }
        const unsigned long long old =
            __hip_atomic_fetch_add(a.acc_words + j, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int)(old >> 57) == a.splits - 1) {
          const unsigned long long tot = old + add;
          const int nfloat = (int)((tot >> 50) & 127u);
          const long long vsum = (long long)(tot & ((1ull << 50) - 1)) -
                                 (long long)(a.splits - nfloat) * (1ll << kFixedOffsetBit);
          float yv = (float)((double)vsum * __builtin_bit_cast(double, (uint64_t)(1023 - kFixedFrac) << 52));
          if (nfloat > 0) {
            const unsigned long long m = __hip_atomic_load(a.mask_words + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int sp = 0; sp < a.splits; ++sp)
              if ((m >> sp) & 1ull)
                yv += __hip_atomic_load(a.partials + (int64_t)sp * Np + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.mask_words + j, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          __hip_atomic_store(a.acc_words + j, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (j < N) __hip_atomic_store(out + j, yv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#ifdef GRINQH_TIMELINE
      __builtin_amdgcn_s_waitcnt(0);
      GRINQH_STAMP(6, tid == 0);   // timeline: column words added (and, where last, y written)
#endif
      return;
    }
    // ---- more splits: partial rows, and the last workgroup of the tile adds
    // them in split order
#pragma unroll
    for (int u = 0; u < kCols; ++u) {
      const int col = tid + u * kVmmThreads;
      // device-scope store: written through to the point where every XCD sees it
      if (col < ct)
        __hip_atomic_store(a.partials + (int64_t)split * Np + t0 + col, val[u], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- the last workgroup of the tile adds the partial rows in split
    // order.  Ordering argument (no cache-wide fence, which would write back
    // and invalidate the whole L2 of every XCD):
    //  1. the partial stores above are device-scope: they go through the
    //     XCD's L2 to the level that every XCD reads, and the wait below
    //     returns only once the memory system has acknowledged each of them;
    //  2. the barrier makes (1) hold for every wave of the workgroup before
    //     thread 0 bumps the tile counter (a device-scope atomic, performed
    //     at that same level), so a count of c means c workgroups' partials
    //     are already visible there;
    //  3. the workgroup that reads the final count learns it through LDS
    //     after a second barrier, so its partial loads are issued only after
    //     the atomic returned, and they are device-scope loads, which miss the
    //     XCD's own L2 and read that level.
    // Relaxed atomics plus acknowledged stores and this control dependence
    // give the order an acquire/release pair would give at agent scope.
    __builtin_amdgcn_s_waitcnt(0);
    GRINQH_STAMP(6, tid == 0);   // timeline: partial row stored and acknowledged
    __syncthreads();
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (old == (unsigned)(a.splits - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    // thread t < 256 adds columns 4t .. 4t + 3 with 16-byte loads (the
    // partial rows are 16-byte aligned: N_pad is a multiple of 128), kRound
    // splits per round with all loads of a round in flight together; splits
    // past the end and columns past the tile read as zero (out-of-range
    // offsets); the sum runs in split order
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.partials + t0), (short)0, (int)(a.splits * Np * 4), (int)kRsrcWord3);
    const uint32_t row_bytes = (uint32_t)(Np * 4);
    if (tid < kTile / 4) {
      const int c4 = 4 * tid;
      float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      constexpr int kRound = 16;
      for (int sp0 = 0; sp0 < a.splits; sp0 += kRound) {
        uint32_t v[kRound][4];
#pragma unroll
        for (int u = 0; u < kRound; ++u) {
          const bool ok = sp0 + u < a.splits && c4 < ct;
          const uint32_t off = ok ? (uint32_t)(sp0 + u) * row_bytes + 4u * (uint32_t)c4 : kOutOfRange;
          const auto q = __builtin_amdgcn_raw_buffer_load_b128(prs, (int)off, 0, kScopeDevice);
          v[u][0] = q[0];
          v[u][1] = q[1];
          v[u][2] = q[2];
          v[u][3] = q[3];
        }
#pragma unroll
        for (int u = 0; u < kRound; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) sum[e] += __builtin_bit_cast(float, v[u][e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)   // device scope: no dirty line left for the kernel's end
        if (c4 + e < ct && t0 + c4 + e < N)
          __hip_atomic_store(out + t0 + c4 + e, sum[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#ifdef GRINQH_TIMELINE
    __builtin_amdgcn_s_waitcnt(0);
    GRINQH_STAMP(7, tid == 0);   // timeline: the tile's sum written (last workgroup only)
#endif
  }
}

}  // namespace grinqh

// The timeline reader (declared in grinqh.h).
extern "C" int grinqh_timeline_read(uint64_t* stamps, int64_t count) {
#ifdef GRINQH_TIMELINE
  grinqh::clear_error();
  if (!stamps || count < 0 || count > (int64_t)grinqh::kTimelineWGs * grinqh::kTimelineSlots)
    return grinqh::fail(GRINQH_EINVAL, "grinqh_timeline_read: NULL buffer or count %lld outside [0, %d]",
                        (long long)count, grinqh::kTimelineWGs * grinqh::kTimelineSlots);
  if (count == 0) return GRINQH_OK;
  const hipError_t e = hipMemcpyFromSymbol(stamps, HIP_SYMBOL(grinqh::g_timeline), sizeof(uint64_t) * (size_t)count,
                                           0, hipMemcpyDeviceToHost);
  if (e != hipSuccess)
    return grinqh::fail(GRINQH_EDEVICE, "grinqh_timeline_read: %s", hipGetErrorString(e));
  return GRINQH_OK;
#else
  (void)stamps;
  (void)count;
  return grinqh::fail(GRINQH_ENOSYS, "grinqh_timeline_read: this library was built without the timeline");
#endif
}

namespace grinqh {

// The caller's workspace: partial rows first, the per-tile counters after
// them, then the column words (one accumulator and one mask per padded column).
static float* ws_partials(void* ws) { return reinterpret_cast<float*>(ws); }
static unsigned long long* ws_words(void* ws, int64_t K, int64_t N) {
  const VmmGeometry g = vmm_geometry(K, N);
  return g.bytes > 0 && ws ? reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(ws) + g.words_offset)
                           : nullptr;
}
static unsigned* ws_counters(void* ws, int64_t K, int64_t N) {
  const VmmGeometry g = vmm_geometry(K, N);
  return g.bytes > 0 && ws ? reinterpret_cast<unsigned*>(reinterpret_cast<char*>(ws) + g.counter_offset) : nullptr;
}

template <int kWaves, int kSubs>
static void launch_shape(bool fused, int out_mode, dim3 grid, const VmmArgs& a, hipStream_t s, bool multi = false) {
  const dim3 block(64 * kWaves);
  if (multi) {
    hipLaunchKernelGGL((vmm_kernel<true, kOutAccumulate, kWaves, kSubs, true>), grid, block, 0, s, a.x, a.planes,
                       a.scales, a.zeros, (int)a.K, (int)a.N, a.tiles, a.rows, a.bmax, a);
    return;
  }
#define GRINQH_VMM_LAUNCH(F, O)                                                                          \
  hipLaunchKernelGGL((vmm_kernel<F, O, kWaves, kSubs>), grid, block, 0, s, a.x, a.planes, a.scales, a.zeros, \
                     (int)a.K, (int)a.N, a.tiles, a.rows, a.bmax, a)
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

static bool dispatch_shape(int waves, int subs, bool fused, int out_mode, dim3 grid, const VmmArgs& a,
                           hipStream_t s, bool multi) {
  switch (waves * 16 + subs) {
    case 16 * 16 + 8: launch_shape<16, 8>(fused, out_mode, grid, a, s, multi); return true;
    case 16 * 16 + 4: launch_shape<16, 4>(fused, out_mode, grid, a, s, multi); return true;
    case 16 * 16 + 2: launch_shape<16, 2>(fused, out_mode, grid, a, s, multi); return true;
    case 8 * 16 + 1: launch_shape<8, 1>(fused, out_mode, grid, a, s, multi); return true;
    case 4 * 16 + 1: launch_shape<4, 1>(fused, out_mode, grid, a, s, multi); return true;
    default: return false;
  }
}

// partials/counters: the split-K workspace (both NULL in accumulate mode).
// words: the column accumulators, then (max_cols entries on) the column masks.
static int launch_vmm(bool fused, int out_mode, VmmArgs& a, float* partials, unsigned* counters,
                      unsigned long long* words, int64_t max_cols, hipStream_t s) {
  const VmmGeometry g = vmm_geometry(a.K, a.N);
  if (g.splits * g.tiles > 0x7FFFFFFF)
    return fail(GRINQH_EINVAL, "%lld workgroups: more than one launch handles", (long long)(g.splits * g.tiles));
  if (g.partial_floats * 4 >= (int64_t)kOutOfRange)
    return fail(GRINQH_EINVAL, "K x N too large for one split-K workspace (%lld partial floats)",
                (long long)g.partial_floats);
  a.splits = (int)g.splits;
  a.tiles = (int)g.tiles;
  a.rows = (int)g.rows_per_split;
  a.partials = partials;
  a.counters = counters;
  a.acc_words = words;
  a.mask_words = words ? words + max_cols : nullptr;
  const dim3 grid((unsigned)(g.splits * g.tiles));
  if (!dispatch_shape((int)g.waves, (int)g.subs, fused, out_mode, grid, a, s, false))
    return fail(GRINQH_EINVAL, "no kernel for %lld waves x %lld sub-items", (long long)g.waves, (long long)g.subs);
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
  return launch_vmm(false, kOutSplitK, a, ws_partials(ws), ws_counters(ws, K, N), ws_words(ws, K, N), padded_cols(N), s);
}

int launch_vmm_fused(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                     const uint16_t* x, int64_t K, int64_t N, int bmax, const AssignParams& ap,
                     float* y, void* ws, hipStream_t s) {
  VmmArgs a{};
  a.planes = planes; a.scales = scales; a.zeros = zeros; a.x = x;
  a.y = y; a.K = K; a.N = N; a.bmax = bmax; a.ap = ap;
  return launch_vmm(true, kOutSplitK, a, ws_partials(ws), ws_counters(ws, K, N), ws_words(ws, K, N), padded_cols(N), s);
}

int launch_vmm_fused_split(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                           const uint16_t* x, int64_t K, int64_t N, int bmax, const AssignParams& ap,
                           float* y, float* partials, unsigned* counters, unsigned long long* words,
                           int64_t max_cols, hipStream_t s) {
  VmmArgs a{};
  a.planes = planes; a.scales = scales; a.zeros = zeros; a.x = x;
  a.y = y; a.K = K; a.N = N; a.bmax = bmax; a.ap = ap;
  return launch_vmm(true, kOutSplitK, a, partials, counters, words, max_cols, s);
}

// Several independent accumulating decode steps in one grid: the members'
// workgroups follow each other (member m from members[m].first), all with
// the shape chosen for K and the members' column tiles together.
int launch_vmm_group(int count, VmmMember* members, int64_t K, int bmax, hipStream_t s) {
  int64_t tiles_total = 0;
  for (int m = 0; m < count; ++m) tiles_total += n_tiles(members[m].N);
  const VmmShape sh = choose_shape(K, tiles_total * kTile);
  const int64_t item = (int64_t)sh.rows * sh.subs;
  const int64_t splits = (K + item - 1) / item;
  VmmArgs a{};
  a.K = K;
  a.bmax = bmax;
  a.rows = sh.rows;
  a.splits = (int)splits;
  a.group.count = count;
  int64_t first = 0;
  for (int m = 0; m < count; ++m) {
    members[m].tiles = (int)n_tiles(members[m].N);
    members[m].first = (int)first;
    first += splits * members[m].tiles;
    if (first > 0x7FFFFFFF) return fail(GRINQH_EINVAL, "%lld workgroups: more than one launch handles", (long long)first);
    a.group.m[m] = members[m];
  }
  if (sh.rows != group_rows(sh.waves, sh.subs))
    return fail(GRINQH_EINVAL, "internal: shape %d x %d x %d has no grouped kernel", sh.waves, sh.subs, sh.rows);
  // the preloaded scalar arguments of a grouped launch: the members'
  // activation pointers, then the first workgroup of members 1..3 (INT_MAX
  // for absent members)
  a.x = members[0].x;
  a.planes = reinterpret_cast<const uint8_t*>(members[count > 1 ? 1 : 0].x);
  a.scales = members[count > 2 ? 2 : 0].x;
  a.zeros = members[count > 3 ? 3 : 0].x;
  a.N = count > 1 ? members[1].first : 0x7FFFFFFF;
  a.tiles = count > 2 ? members[2].first : 0x7FFFFFFF;
  a.rows = count > 3 ? members[3].first : 0x7FFFFFFF;
  a.y = members[0].y;
  if (!dispatch_shape(sh.waves, sh.subs, true, kOutAccumulate, dim3((unsigned)first), a, s, true))
    return fail(GRINQH_EINVAL, "no kernel for %d waves x %d sub-items", sh.waves, sh.subs);
  return check_launch("grinqh_decode_vmm_accumulate_group");
}

int launch_vmm_accumulate(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                          const uint16_t* x, int64_t K, int64_t N, int bmax, const AssignParams& ap,
                          float* y, float* clear, hipStream_t s) {
  VmmArgs a{};
  a.planes = planes; a.scales = scales; a.zeros = zeros; a.x = x;
  a.y = y; a.clear = clear; a.K = K; a.N = N; a.bmax = bmax; a.ap = ap;
  return launch_vmm(true, kOutAccumulate, a, nullptr, nullptr, nullptr, 0, s);
}

}  // namespace grinqh
