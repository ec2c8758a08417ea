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
// Work split.  A workgroup (8 waves) owns 128 tokens x one 512-column half of
// a 1024-column store tile (half of every 128-byte plane line it reads; the
// workgroup of the other half usually runs on the same XCD).  Wave w owns
// columns 64 w .. 64 w + 63 of the half for all 128 tokens, as 4 x 2 blocks of
// 32 x 32 accumulated in fp32 by v_mfma_f32_32x32x16_f16, so every weight is
// dequantised by exactly one wave.  K is walked 64 rows per step.  Unpacking
// costs vector-ALU work per weight while the matrix work per weight grows
// with the tokens sharing it, hence the tall tile.
//
// Per step:
//   1. X[m0 .. m0+127][k0 .. k0+63] (fp16) goes to LDS, rows padded by 16
//      bytes so that the A-fragment reads are conflict-free.
//   2. Thread (row pair r, plane word w) rebuilds the codes of its two rows x
//      32 columns from their b_max plane words (the bit transpose of
//      bitplane.hpp, specialised for b_max) and writes them to LDS as exact
//      fp16 integers, the two rows of a pair in one dword.  The B operand of
//      the MFMA wants eight consecutive k of one column per lane, so codes
//      are stored column-major in 16-byte fragments of eight rows; inside
//      each 32-column block the column is XOR-swizzled by the block index,
//      which makes the writes and the fragment reads conflict-free.
//   3. Each lane dequantises its B fragments right after reading them:
//      w = s q + z with one packed fp16 fused multiply-add per two weights
//      (one rounding to fp16); s and z are constant along a fragment.
//   4. B is double-buffered in LDS: while a wave runs the MFMAs of one step
//      it also rebuilds the codes of the next, and the two waves sharing a
//      SIMD do the two in opposite order so that vector-ALU and matrix work
//      overlap.  The step after that is loaded into registers meanwhile.
//      Plane and X loads are buffer loads: rows past K, tokens past M, words
//      past a narrow tile and columns past K read as zero through
//      out-of-range offsets, and the plane index is a scalar offset.
// Workgroups are numbered so that the ones sharing a column half land on the
// same XCD (consecutive workgroup ids go to different XCDs), where they read
// its planes through one L2.
#include "bitplane.hpp"
#include "common.hpp"

namespace grinqh {

namespace {

constexpr int kPM = 128;                // tokens per workgroup tile
constexpr int kPN = kTile / 2;          // columns per workgroup tile: half a store tile
constexpr int kPK = 64;                 // rows per step
constexpr int kPWaves = 8;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kXPitch = kPK + 8;        // halves per LDS row of the X tile
constexpr int kXChunks = kPM * kPK / 8 / kPThreads;   // 16-byte X chunks per thread per step (2)
constexpr int kFragRows = kPK / 8;      // B fragment rows (of 8 k) per step
constexpr int kXCDs = 8;                // MI355X
constexpr uint32_t kOOR = 0x7FFFFF00u;  // buffer offset past every range used here
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family

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
  int m_tiles, halves;   // token tiles, 512-column halves of the store tiles
};

// One step's global data for this thread (raw; see the buffer-load notes).
// X chunks are 8 halves each: four dwords (VEC) or one half per register.
template <bool VEC>
struct StepRegs {
  uint32_t x[kXChunks][VEC ? 4 : 8];
  uint32_t w1[8], w2[8];     // plane words of the thread's two rows
  uint16_t s[2], z[2];       // scale and zero of the lane's two B-fragment columns
};

}  // namespace

// VEC: K a multiple of 8 and X 16-byte aligned, so each 8-half X chunk is one
// 16-byte load; otherwise eight 2-byte loads.  All global loads are
// unconditional (past the end they read zero or repeat the last step), so
// that the compiler's wait counts stay exact instead of draining every load
// in flight at the loop head.
template <int BMAX, bool VEC>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kPM * kXPitch];
  __shared__ __attribute__((aligned(16))) uint32_t s_w[2][kFragRows * kPN * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t M = a.M, N = a.N;
  const int K = (int)a.K;                               // < 2^21 (checked by the launcher)

  // workgroup -> (token tile, column half); ids that share an XCD (id mod 8)
  // take consecutive entries of the column-half-major order
  const int T = a.m_tiles * a.halves;
  int L = blockIdx.x;
  if (T % kXCDs == 0) L = (L % kXCDs) * (T / kXCDs) + L / kXCDs;
  const int half = L / a.m_tiles;
  const int64_t m0 = (int64_t)(L % a.m_tiles) * kPM;
  const int64_t t0 = (int64_t)(half >> 1) * kTile;      // store tile
  const int64_t Np = padded_cols(N);
  const int ct = (int)((Np - t0) < kTile ? (Np - t0) : kTile);
  const int pb = __builtin_amdgcn_readfirstlane(ct / 8);   // uniform: used as a scalar offset
  const int c0 = (half & 1) * kPN;                      // first column of this half in the tile
  if (c0 >= ct) return;                                 // the half lies past a narrow last tile
  const int steps = (K + kPK - 1) / kPK;

  // plane words: buffer over the store tile (row tiles of BMAX planes)
  const uint32_t rstride = (uint32_t)(pb * BMAX);
  const __amdgpu_buffer_rsrc_t prs = uniform_rsrc(a.planes + store_offset(t0 * K, BMAX), (int64_t)K * rstride);
  // unpack unit: plane word uw (of this half) of rows 2 ur, 2 ur + 1 of the step
  const int uw = tid & 15;
  const int ur = tid >> 4;
  const int word = c0 / 32 + uw;
  const uint32_t wbyte = word < ct / 32 ? 4u * (uint32_t)word : kOOR;
  // X: buffer over this tile's tokens; chunk c of this thread is token
  // (tid + 512 c) / 8, halves 8 ((tid + 512 c) % 8) .. + 7 of the step
  const int64_t mrows = (M - m0) < kPM ? (M - m0) : kPM;
  const __amdgpu_buffer_rsrc_t xrs = uniform_rsrc(a.X + m0 * K, mrows * K * 2);
  // B-fragment columns of this lane (one per column block cb)
  int ncol[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int64_t n = t0 + c0 + 64 * wid + 32 * cb + (lane & 31);
    ncol[cb] = (int)(n < N ? n : N - 1);
  }

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
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = k0 + 2 * ur + e;
      const uint32_t off = row < K ? (uint32_t)row * rstride + wbyte : kOOR;
      uint32_t* w = e == 0 ? r.w1 : r.w2;
#pragma unroll
      for (int p = 0; p < BMAX; ++p) w[p] = __builtin_amdgcn_raw_buffer_load_b32(prs, (int)off, p * pb, 0);
#pragma unroll
      for (int p = BMAX; p < 8; ++p) w[p] = 0u;
    }
    const int64_t g = k0 / kGroup;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      r.s[cb] = a.scales[g * N + ncol[cb]];
      r.z[cb] = a.zeros[g * N + ncol[cb]];
    }
  };

  constexpr int kSh = 8 - BMAX;                              // codes come back as q 2^(8 - b_max)
  constexpr uint32_t kKeep = 0x01010101u * (0xFFu >> kSh);
  // rebuilt codes of one step (plane words in r) into B buffer dst
  auto unpack = [&](const StepRegs<VEC>& r, uint32_t* buf) {
    uint32_t d1[8], d2[8];
    planes_to_codes<BMAX>(r.w1, d1);
    planes_to_codes<BMAX>(r.w2, d2);
    if constexpr (kSh > 0) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        d1[m] = (d1[m] >> kSh) & kKeep;
        d2[m] = (d2[m] >> kSh) & kKeep;
      }
    }
    uint32_t* dst = buf + ((ur >> 2) * kPN + 32 * uw) * 4 + (ur & 3);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // [row 2r code, 0x64, row 2r+1 code, 0x64] = fp16 (1024 + c1, 1024 + c2)
        const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24);
        const uint32_t pr = __builtin_amdgcn_perm(d2[m], d1[m], sel) | 0x64006400u;
        const half2_t c = __builtin_bit_cast(half2_t, pr) - (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
        const int col = 4 * m + j;
        dst[(col ^ uw) * 4] = __builtin_bit_cast(uint32_t, c);
      }
    }
  };
  auto write_x = [&](const uint32_t (&x)[kXChunks][VEC ? 4 : 8]) {
#pragma unroll
    for (int c = 0; c < kXChunks; ++c) {
      const int q = tid + c * kPThreads;
      uint32_t d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (VEC) d[e] = x[c][e];
        else d[e] = (x[c][2 * e] & 0xFFFFu) | (x[c][2 * e + 1] << 16);
      }
      __builtin_memcpy(&s_x[(q >> 3) * kXPitch + 8 * (q & 7)], d, 16);
    }
  };

  float16_t acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.0f;

  // MFMAs of one step from B buffer buf; s2, z2: scale and zero pairs
  auto mfma_step = [&](const uint32_t* buf, const uint32_t (&s2)[2], const uint32_t (&z2)[2]) {
#pragma unroll
    for (int s16 = 0; s16 < kPK / 16; ++s16) {
      half8_t af[4], bf[2];
      const int kb = 2 * s16 + (lane >> 5);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int blk = 2 * wid + cb;   // 32-column block of the half
        // copied into plain arrays: taking elements of a loaded vector inside
        // a bit cast made this compiler read only the first dword
        uint32_t raw[4], wv[4];
        __builtin_memcpy(raw, &buf[(kb * kPN + 32 * blk + ((lane & 31) ^ blk)) * 4], 16);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          wv[e] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
                                                   __builtin_bit_cast(half2_t, raw[e]),
                                                   __builtin_bit_cast(half2_t, s2[cb]),
                                                   __builtin_bit_cast(half2_t, z2[cb])));
        __builtin_memcpy(&bf[cb], wv, 16);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int row = 32 * rb + (lane & 31);
        __builtin_memcpy(&af[rb], &s_x[row * kXPitch + 16 * s16 + 8 * (lane >> 5)], 16);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[rb], bf[cb], acc[rb][cb], 0, 0, 0);
    }
  };

  // ---- software pipeline.  B is double-buffered: during step st every wave
  // runs the MFMAs of step st and rebuilds the codes of step st + 1 into the
  // other buffer.  The two waves that share a SIMD (w and w + 4) do the two
  // halves in opposite order, so one's vector-ALU work overlaps the other's
  // matrix work.  X is single-buffered and rewritten between two barriers.
  StepRegs<VEC> r;
  constexpr int kXRegs = VEC ? 4 : 8;
  const int last = steps - 1;
  uint32_t s2[2], z2[2], xn[kXChunks][kXRegs];
  load_step(0, r);
  unpack(r, s_w[0]);
  write_x(r.x);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    s2[cb] = (uint32_t)r.s[cb] * 0x00010001u;
    z2[cb] = (uint32_t)r.z[cb] * 0x00010001u;
  }
  load_step(last < 1 ? last : 1, r);
  __syncthreads();
  const bool matrix_first = wid >= kPWaves / 2;
  for (int st = 0; st < steps; ++st) {
    const bool more = st + 1 < steps;
    const uint32_t* cur = s_w[st & 1];
    uint32_t* nxt = s_w[(st + 1) & 1];
    if (matrix_first) mfma_step(cur, s2, z2);
    if (more) {
      unpack(r, nxt);
#pragma unroll
      for (int c = 0; c < kXChunks; ++c)
#pragma unroll
        for (int e = 0; e < kXRegs; ++e) xn[c][e] = r.x[c][e];
    }
    uint32_t s2n[2], z2n[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      s2n[cb] = (uint32_t)r.s[cb] * 0x00010001u;
      z2n[cb] = (uint32_t)r.z[cb] * 0x00010001u;
    }
    load_step(st + 2 < last ? st + 2 : last, r);   // past the end: repeats the last step, unused
    if (!matrix_first) mfma_step(cur, s2, z2);
    __syncthreads();                 // MFMAs of st done with X; codes of st + 1 written
    if (more) write_x(xn);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      s2[cb] = s2n[cb];
      z2[cb] = z2n[cb];
    }
    __syncthreads();                 // X of st + 1 visible
  }

  // ---- output: lane holds column (lane & 31) of each block, rows
  // 8 (v / 4) + 4 (lane / 32) + v % 4
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int64_t n = t0 + c0 + 64 * wid + 32 * cb + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + 32 * rb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M && n < N) a.Y[m * N + n] = acc[rb][cb][v];
      }
    }
}

int launch_prefill(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros, const uint16_t* X,
                   int64_t M, int64_t K, int64_t N, int bmax, float* Y, hipStream_t s) {
  // buffer ranges: one store tile (K 1024 b_max / 8 bytes) and one token
  // tile of X (128 K 2 bytes) must stay below 2^31 bytes
  if (K >= (int64_t(1) << 21))
    return fail(GRINQH_EINVAL, "K = %lld: the prefill handles K < 2^21", (long long)K);
  const int64_t mt = (M + kPM - 1) / kPM;
  const int64_t nh = 2 * n_tiles(N);
  if (mt * nh > 0x7FFFFFFF) return fail(GRINQH_EINVAL, "M x N needs more than 2^31 workgroups");
  PrefillArgs a{planes, scales, zeros, X, Y, M, K, N, (int)mt, (int)nh};
  const dim3 grid((unsigned)(mt * nh)), block(kPThreads);
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
