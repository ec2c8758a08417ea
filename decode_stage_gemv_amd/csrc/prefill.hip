// Dense prefill over the bit-plane store (GRINQH paper, section 3: the
// prefill stage loads weights at one fixed precision; section 4 "Prefill vs.
// Decoding Evaluation": the kernel unpacks the weights at full b_max
// precision and runs a dense matrix-matrix product; section 5 "End-to-end
// Measurements").
//
//   Y[m][n] = sum_k X[m][k] (s[g][n] q[k][n] + z[g][n]),  g = k / 128,
//
// for a batch of M token activations, every row read at its full width.
//
// Work split.  A workgroup (8 waves) owns 256 tokens x 256 columns (a quarter
// of a 1024-column store tile); wave (r, c) of the 2 x 4 wave grid owns 128
// tokens x 64 columns as 4 x 2 blocks of 32 x 32 accumulated in fp32 by
// v_mfma_f32_32x32x16_f16.  K is walked 64 rows per step.  Unpacking costs
// vector-ALU work per weight while the matrix work per weight grows with the
// tokens sharing it, hence the square tile: 256 tokens share every weight.
//
// Per step, for the next step while the matrix cores run this one:
//   1. X[m0 .. m0+255][k0 .. k0+63] (fp16) goes to LDS (rows padded by 16
//      bytes so that the A-fragment reads are conflict-free).
//   2. Thread (row, plane word, half) loads the b_max plane words of its row
//      and rebuilds the row's 32 codes (bit transpose of bitplane.hpp); the
//      two threads of a row pair swap codes with a lane permute, and each
//      writes 16 columns of the pair to LDS as exact fp16 integers (1024 + c
//      from a byte permute and an OR, then - 1024), the pair in one dword.
//      The B operand of the MFMA wants eight consecutive k of one column per
//      lane, so codes are stored column-major in 16-byte fragments of eight
//      rows; inside each 32-column word the column is XOR-swizzled by the
//      word index, so writes spread over the banks and fragment reads are
//      conflict-free.  The step's scale and zero of every column go to LDS.
//   3. A lane dequantises each B fragment after reading it: w = s q + z
//      with one packed fp16 fused multiply-add per two weights (one rounding
//      to fp16, the same weights as the unpacked path).  Within a step the
//      fragments of the next 16 rows are read while the MFMAs of the current
//      ones issue.
//   X, B and the scales are double-buffered in LDS (one barrier per step);
//   the step after next is loaded into registers meanwhile, and the two
//   waves sharing a SIMD do the matrix and the unpack halves of a step in
//   opposite order.  All global loads are unconditional buffer loads: rows
//   past K, tokens past M and words past a narrow tile read zero through
//   out-of-range offsets, and the prefetch past the last step repeats it, so
//   the compiler's wait counts stay exact.
// Workgroups sharing a column strip are numbered onto one XCD (consecutive
// workgroup ids go to different XCDs), where they read its planes through
// one L2.
#include "bitplane.hpp"
#include "common.hpp"

namespace grinqh {

namespace {

constexpr int kPM = 256;                // tokens per workgroup tile
constexpr int kPN = 256;                // columns per workgroup tile (a quarter of a store tile)
constexpr int kPK = 64;                 // rows per step
constexpr int kPWaves = 8;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kXPitch = kPK + 8;        // halves per LDS row of the X tile
constexpr int kXChunks = kPM * kPK / 8 / kPThreads;   // 16-byte X chunks per thread per step (4)
constexpr int kFragRows = kPK / 8;      // B fragment rows (of 8 k) per step
constexpr int kQuarters = kTile / kPN;  // workgroup tiles per store tile
constexpr int kXCDs = 8;                // MI355X
constexpr uint32_t kOOR = 0x7FFFFF00u;  // buffer offset past every range used here
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family
constexpr int kDppSwapPairs = 0xB1;     // quad_perm [1, 0, 3, 2]: exchange with the neighbouring lane

// Raw buffer descriptor from values that are the same in every lane; the
// read-first-lane makes that visible to the compiler, which otherwise may
// treat the descriptor as divergent and loop over the lanes at every load.
__device__ inline __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, n,
                                           kRsrcWord3);
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct PrefillArgs {
  const uint8_t* planes;
  const uint16_t* scales;
  const uint16_t* zeros;
  const uint16_t* X;
  float* Y;
  int64_t M, K, N;
  int m_tiles, n_tiles;   // token tiles, 256-column tiles (four per store tile)
};

// One step's global data for this thread (raw).  X chunks are 8 halves
// each: four dwords (VEC) or one half per register.
template <bool VEC>
struct StepRegs {
  uint32_t x[kXChunks][VEC ? 4 : 8];
  uint32_t w[8];             // plane words of the thread's row (planes >= b_max: 0)
  uint32_t sz;               // scale (low half) and zero (high half) of column tid % 256
};

}  // namespace

// VEC: K a multiple of 8 and X 16-byte aligned, so each 8-half X chunk is one
// 16-byte load; otherwise eight 2-byte loads.
template <int BMAX, bool VEC>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_x[2][kPM * kXPitch];
  __shared__ __attribute__((aligned(16))) uint32_t s_w[2][kFragRows * kPN * 4];
  __shared__ uint32_t s_sz[2][kPN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wid >> 2, wc = wid & 3;
  const int64_t M = a.M, N = a.N;
  const int K = (int)a.K;                               // < 2^21 (checked by the launcher)
  const int64_t Np = padded_cols(N);

  // workgroup -> (column strip, token tile); ids that share an XCD (id mod 8)
  // take consecutive entries of the strip-major order
  const int T = a.m_tiles * a.n_tiles;
  int L = blockIdx.x;
  if (T % kXCDs == 0) L = (L % kXCDs) * (T / kXCDs) + L / kXCDs;
  const int64_t n0 = (int64_t)(L / a.m_tiles) * kPN;
  const int64_t m0 = (int64_t)(L % a.m_tiles) * kPM;
  const int64_t t0 = n0 / kTile * kTile;                // store tile
  const int ct = (int)((Np - t0) < kTile ? (Np - t0) : kTile);
  const int c0 = (int)(n0 - t0);                        // first column of this quarter in the tile
  if (c0 >= ct) return;                                 // the quarter lies past a narrow last tile
  const int pb = __builtin_amdgcn_readfirstlane(ct / 8);   // uniform: used as a scalar offset
  const int steps = (K + kPK - 1) / kPK;
  const int last = steps - 1;

  // plane words: buffer over the store tile (row tiles of BMAX planes)
  const uint32_t rstride = (uint32_t)(pb * BMAX);
  const __amdgpu_buffer_rsrc_t prs = uniform_rsrc(a.planes + store_offset(t0 * K, BMAX), (int64_t)K * rstride);
  // unpack unit: row 2 up + uh of the step, plane word uw of this quarter;
  // up = row pair (fragment row up / 4, dword up % 4 of the fragment)
  const int uh = tid & 1;
  const int uw = (tid >> 1) & 7;
  const int up = tid >> 4;
  const int word = c0 / 32 + uw;
  const uint32_t wbyte = word < ct / 32 ? 4u * (uint32_t)word : kOOR;
  // X: buffer over this tile's tokens; chunk c of this thread is token
  // (tid + 512 c) / 8, halves 8 ((tid + 512 c) % 8) .. + 7 of the step
  const int64_t mrows = (M - m0) < kPM ? (M - m0) : kPM;
  const __amdgpu_buffer_rsrc_t xrs = uniform_rsrc(a.X + m0 * K, mrows * K * 2);
  // column whose scale and zero this thread stages (clamped to N)
  int64_t scol = n0 + (tid & (kPN - 1));
  scol = scol < N ? scol : N - 1;

  constexpr int kXRegs = VEC ? 4 : 8;
  auto load_step = [&](int st, StepRegs<VEC>& r) {
    const int k0 = st * kPK;
#pragma unroll
    for (int c = 0; c < kXChunks; ++c) {
      const int q = tid + c * kPThreads;
      const int k = k0 + 8 * (q & 7);
      const uint32_t rowb = (uint32_t)(q >> 3) * (uint32_t)K * 2u;
      if constexpr (VEC) {
        const uint32_t off = k < K ? rowb + (uint32_t)(2 * k) : kOOR;
        const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)off, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) r.x[c][e] = t[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t off = k + e < K ? rowb + (uint32_t)(2 * (k + e)) : kOOR;
          r.x[c][e] = __builtin_amdgcn_raw_buffer_load_b16(xrs, (int)off, 0, 0);
        }
      }
    }
    const int row = k0 + 2 * up + uh;
    const uint32_t off = (row < K && wbyte != kOOR) ? (uint32_t)row * rstride + wbyte : kOOR;
#pragma unroll
    for (int p = 0; p < 8; ++p)
      r.w[p] = p < BMAX ? __builtin_amdgcn_raw_buffer_load_b32(prs, (int)off, p * pb, 0) : 0u;
    const int64_t g = k0 / kGroup;
    r.sz = (uint32_t)a.scales[g * N + scol] | ((uint32_t)a.zeros[g * N + scol] << 16);
  };

  constexpr int kSh = 8 - BMAX;                              // codes come back as q 2^(8 - b_max)
  constexpr uint32_t kKeep = 0x01010101u * (0xFFu >> kSh);
  // per j: byte selectors that put this row's code in its half of the pair
  // (row 2 up in the low half, 2 up + 1 in the high half) and the partner's
  // code in the other; v_perm takes bytes 0..3 from its second operand
  // (this lane) and 4..7 from its first (the partner)
  uint32_t psel[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    psel[j] = uh == 0 ? ((uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24))
                      : ((uint32_t)(4 + j) | (0x0Cu << 8) | ((uint32_t)j << 16) | (0x0Cu << 24));
  // one step's X, codes and scales into LDS buffer buf
  auto write_step = [&](int buf, const StepRegs<VEC>& r) {
#pragma unroll
    for (int c = 0; c < kXChunks; ++c) {
      const int q = tid + c * kPThreads;
      uint32_t d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (VEC) d[e] = r.x[c][e];
        else d[e] = (r.x[c][2 * e] & 0xFFFFu) | (r.x[c][2 * e + 1] << 16);
      }
      __builtin_memcpy(&s_x[buf][(q >> 3) * kXPitch + 8 * (q & 7)], d, 16);
    }
    uint32_t dm[8];
    planes_to_codes<BMAX>(r.w, dm);
    if constexpr (kSh > 0) {
#pragma unroll
      for (int m = 0; m < 8; ++m) dm[m] = (dm[m] >> kSh) & kKeep;
    }
    // this thread writes columns 16 uh .. 16 uh + 15 of the word (code words
    // 4 uh .. 4 uh + 3) for both rows of the pair
    uint32_t* dst = s_w[buf] + ((up >> 2) * kPN + 32 * uw) * 4 + (up & 3);
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const uint32_t lo = dm[mm], hi = dm[4 + mm];
      // the partner needs the half this thread does not write, and vice versa
      const uint32_t give = uh == 0 ? hi : lo;
      const uint32_t keep = uh == 0 ? lo : hi;
      const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)give, kDppSwapPairs, 0xF, 0xF, false);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = 16 * uh + 4 * mm + j;            // column within the word
        const uint32_t pr = __builtin_amdgcn_perm(got, keep, psel[j]) | 0x64006400u;
        const half2_t cv = __builtin_bit_cast(half2_t, pr) - (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
        dst[(col ^ uw) * 4] = __builtin_bit_cast(uint32_t, cv);
      }
    }
    if (tid < kPN) s_sz[buf][tid] = r.sz;
  };

  float16_t acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.0f;

  // MFMAs of one step from LDS buffer buf.  With 16-byte X loads the
  // sub-steps are pipelined: while the MFMAs of sub-step s16 issue, the
  // fragments of s16 + 1 are read from LDS (each A fragment right behind the
  // two MFMAs that last use the registers it replaces) and its weights are
  // dequantised afterwards, so the LDS latency hides behind matrix work
  // instead of stalling every sub-step.  The 2-byte X form holds twice the X
  // registers and has no room for a second set of fragments: it reads each
  // sub-step's fragments after the previous sub-step's MFMAs.
  constexpr bool kPipe = VEC;
  auto read_b = [&](int buf, int s16, uint32_t (&raw)[2][4]) {
    const int kb = 2 * s16 + (lane >> 5);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int wi = 2 * wc + cb;                        // 32-column word of the quarter
      __builtin_memcpy(raw[cb], &s_w[buf][(kb * kPN + 32 * wi + ((lane & 31) ^ wi)) * 4], 16);
    }
  };
  auto read_a = [&](int buf, int s16, int rb, half8_t& af) {
    const int row = 128 * wr + 32 * rb + (lane & 31);
    __builtin_memcpy(&af, &s_x[buf][row * kXPitch + 16 * s16 + 8 * (lane >> 5)], 16);
  };
  // w = s q + z on both halves of every dword (the raw words are copied
  // through plain arrays: taking elements of a loaded vector inside a bit
  // cast made this compiler read only the first dword)
  auto dequant = [&](const uint32_t (&raw)[2][4], const uint32_t (&s2)[2], const uint32_t (&z2)[2],
                     half8_t (&bf)[2]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        wv[e] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, raw[cb][e]),
                                                                       __builtin_bit_cast(half2_t, s2[cb]),
                                                                       __builtin_bit_cast(half2_t, z2[cb])));
      __builtin_memcpy(&bf[cb], wv, 16);
    }
  };
  auto mfma_step = [&](int buf) {
    uint32_t s2[2], z2[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const uint32_t sz = s_sz[buf][64 * wc + 32 * cb + (lane & 31)];
      s2[cb] = (sz & 0xFFFFu) * 0x00010001u;
      z2[cb] = (sz >> 16) * 0x00010001u;
    }
    half8_t af[4], bf[2];
    uint32_t raw[2][4];
    read_b(buf, 0, raw);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) read_a(buf, 0, rb, af[rb]);
    dequant(raw, s2, z2, bf);
#pragma unroll
    for (int s16 = 0; s16 < kPK / 16; ++s16) {
      const bool more = s16 + 1 < kPK / 16;
      if (kPipe && more) read_b(buf, s16 + 1, raw);
      __builtin_amdgcn_sched_barrier(0);
      // the wave issuing MFMAs goes first while it does (the other wave on
      // the SIMD is loading or unpacking): keeps the matrix core fed
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[rb], bf[cb], acc[rb][cb], 0, 0, 0);
        if (kPipe && more) read_a(buf, s16 + 1, rb, af[rb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      if (more) {
        if constexpr (!kPipe) {
          read_b(buf, s16 + 1, raw);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) read_a(buf, s16 + 1, rb, af[rb]);
        }
        dequant(raw, s2, z2, bf);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- software pipeline.  Everything is double-buffered in LDS: during
  // step st a wave runs the MFMAs of st and writes the X, codes and scales
  // of st + 1 into the other buffers; the two waves that share a SIMD (w and
  // w + 4) do the two halves in opposite order, so one's vector-ALU work
  // overlaps the other's matrix work.  The data of st + 2 is loaded into
  // registers meanwhile.
  StepRegs<VEC> r;
  load_step(0, r);
  write_step(0, r);
  load_step(last < 1 ? last : 1, r);
  __syncthreads();
  const bool matrix_first = wid >= kPWaves / 2;
  for (int st = 0; st < steps; ++st) {
    if (matrix_first) mfma_step(st & 1);
    if (st < last) write_step((st + 1) & 1, r);
    load_step(st + 2 < last ? st + 2 : last, r);   // past the end: repeats the last step, unused
    if (!matrix_first) mfma_step(st & 1);
    __syncthreads();
  }

  // ---- output: lane holds column (lane & 31) of each block, rows
  // 8 (v / 4) + 4 (lane / 32) + v % 4
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int64_t n = n0 + 64 * wc + 32 * cb + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + 128 * wr + 32 * rb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M && n < N) a.Y[m * N + n] = acc[rb][cb][v];
      }
    }
}

int launch_prefill(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros, const uint16_t* X,
                   int64_t M, int64_t K, int64_t N, int bmax, float* Y, hipStream_t s) {
  // buffer ranges: one store tile (K 1024 b_max / 8 bytes) and one token
  // tile of X (256 K 2 bytes) must stay below 2^31 bytes
  if (K >= (int64_t(1) << 21))
    return fail(GRINQH_EINVAL, "K = %lld: the prefill handles K < 2^21", (long long)K);
  const int64_t mt = (M + kPM - 1) / kPM;
  const int64_t nq = kQuarters * n_tiles(N);
  if (mt * nq > 0x7FFFFFFF) return fail(GRINQH_EINVAL, "M x N needs more than 2^31 workgroups");
  PrefillArgs a{planes, scales, zeros, X, Y, M, K, N, (int)mt, (int)nq};
  const dim3 grid((unsigned)(mt * nq)), block(kPThreads);
  const bool vec = K % 8 == 0 && reinterpret_cast<uintptr_t>(X) % 16 == 0;
  switch (bmax * 2 + (vec ? 1 : 0)) {
#define GRINQH_PREFILL_CASE(B)                                                        \
  case 2 * B: hipLaunchKernelGGL((prefill_kernel<B, false>), grid, block, 0, s, a); break; \
  case 2 * B + 1: hipLaunchKernelGGL((prefill_kernel<B, true>), grid, block, 0, s, a); break;
    GRINQH_PREFILL_CASE(1)
    GRINQH_PREFILL_CASE(2)
    GRINQH_PREFILL_CASE(3)
    GRINQH_PREFILL_CASE(4)
    GRINQH_PREFILL_CASE(5)
    GRINQH_PREFILL_CASE(6)
    GRINQH_PREFILL_CASE(7)
    GRINQH_PREFILL_CASE(8)
#undef GRINQH_PREFILL_CASE
    default: return fail(GRINQH_EINVAL, "b_max = %d outside 1..8", bmax);
  }
  return check_launch("grinqh_prefill");
}

}  // namespace grinqh
