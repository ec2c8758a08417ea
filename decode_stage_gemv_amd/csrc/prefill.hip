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
// Work split.  A workgroup (4 waves) owns a 128-token x 128-column tile of Y
// and walks K one scale group (128 rows) at a time; wave (r, c) of the 2 x 2
// wave grid owns a 64 x 64 quarter as 2 x 2 blocks of 32 x 32, accumulated
// in fp32 by v_mfma_f32_32x32x16_f16.  The 128 columns lie inside one
// 1024-column tile of the store.
//
// Per group:
//   1. X[m0 .. m0+127][k0 .. k0+127] (fp16) goes to LDS, rows padded by 16
//      bytes so the A-fragment reads are conflict-free.
//   2. Each thread rebuilds the codes of two rows x 32 columns from their
//      b_max plane words (the bit transpose of bitplane.hpp) and writes them
//      to LDS as exact fp16 integers, the two rows of a pair in one dword:
//      the B operand of the MFMA wants eight consecutive k of one column per
//      lane, so the codes are stored column-major in 16-byte fragments of
//      eight rows, with the column index XOR-swizzled by the fragment row so
//      that both the writes and the reads are free of bank conflicts.
//   3. Each lane dequantises its B fragments right after reading them:
//      w = s q + z with one packed fp16 fused multiply-add per two weights
//      (one rounding to fp16), s and z being constant along a fragment.
//   4. While the MFMAs of this group run, the loads of the next group's X,
//      plane words, scales and zeros are already in flight (registers).
#include "bitplane.hpp"
#include "common.hpp"

namespace grinqh {

namespace {

constexpr int kPM = 128;                // tokens per workgroup tile
constexpr int kPN = 128;                // columns per workgroup tile
constexpr int kPK = kGroup;             // rows per step: one scale group
constexpr int kPThreads = 256;          // 4 waves
constexpr int kXPitch = kPK + 8;        // halves per LDS row of the X tile
constexpr int kXChunks = kPM * kPK / 8 / kPThreads;   // 16-byte X chunks per thread per step (8)
constexpr int kFragRows = 8;            // rows per B fragment
constexpr int kFrags = kPK / kFragRows; // fragment rows per step (16)

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
  int bmax;
};

// Registers holding one step's global data for this thread.  Loads are
// issued unconditionally from in-bounds addresses; what lies outside the
// matrices is masked only when the data is consumed, so nothing waits for a
// load before the next step.
struct StepRegs {
  u32x4_t x[kXChunks];      // X chunks (8 halves each)
  uint32_t xok;             // bit u: chunk u lies inside X
  uint32_t w1[8], w2[8];    // plane words of the thread's two rows (raw)
  bool ok1, ok2;            // the two rows exist (row < K)
  uint16_t s[2], z[2];      // scale and zero of the lane's two B-fragment columns
};

// Eight halves X[m][k .. k+7].  The address is clamped into the matrix;
// `ok` says whether the chunk is real (the caller masks it later).  `aligned`
// (K a multiple of 8, uniform) allows one 16-byte load per chunk; otherwise
// the halves are loaded one by one and masked here (zeros outside X).
__device__ inline u32x4_t load_x_chunk(const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t m,
                                       int64_t k, bool aligned, bool& ok) {
  const bool row_ok = m < M;
  const int64_t mc = row_ok ? m : M - 1;
  const uint16_t* row = X + mc * K;
  u32x4_t v;
  if (aligned) {
    ok = row_ok && k < K;
    v = *reinterpret_cast<const u32x4_t*>(row + (ok ? k : 0));
  } else {
    ok = true;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = row_ok && k + e < K;
      const uint32_t val = row[ok ? k + e : 0];
      h[e] = ok ? val : 0u;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = h[2 * e] | (h[2 * e + 1] << 16);
  }
  return v;
}

}  // namespace

__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kPM * kXPitch];
  __shared__ __attribute__((aligned(16))) uint32_t s_w[kFrags * kPN * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wid >> 1, wc = wid & 1;
  const int64_t M = a.M, K = a.K, N = a.N;
  const int64_t n0 = (int64_t)blockIdx.x * kPN;
  const int64_t m0 = (int64_t)blockIdx.y * kPM;
  const int64_t Np = padded_cols(N);
  const int64_t t0 = n0 / kTile * kTile;                  // 1024-column tile of the store
  const int ct = (int)((Np - t0) < kTile ? (Np - t0) : kTile);
  const int pb = ct / 8;
  const int word0 = (int)(n0 - t0) / 32;                  // first plane word of this column tile
  const int bmax = a.bmax;
  const int G = (int)n_groups(K);

  // unpack unit of this thread: rows 2p, 2p + 1 of the step, plane word `uw`
  const int up = tid & 63;
  const int uw = tid >> 6;
  // B-fragment columns of this lane (one per column block cb)
  int ncol[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int64_t n = n0 + 64 * wc + 32 * cb + (lane & 31);
    ncol[cb] = (int)(n < N ? n : N - 1);
  }

  const bool x_aligned = (K & 7) == 0;
  auto load_step = [&](int g, StepRegs& r) {
    const int64_t k0 = (int64_t)g * kPK;
    r.xok = 0u;
#pragma unroll
    for (int u = 0; u < kXChunks; ++u) {
      const int q = tid + u * kPThreads;
      bool ok;
      r.x[u] = load_x_chunk(a.X, M, K, m0 + (q >> 4), k0 + 8 * (q & 15), x_aligned, ok);
      r.xok |= ok ? (1u << u) : 0u;
    }
    // plane words: every load is in bounds (rows past K read row K - 1,
    // planes past b_max read plane 0); masked when rebuilt
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t row = k0 + 2 * up + e;
      const bool ok = row < K;
      uint32_t* w = e == 0 ? r.w1 : r.w2;
      (e == 0 ? r.ok1 : r.ok2) = ok;
      const uint8_t* base = a.planes + store_offset(t0 * K + (ok ? row : K - 1) * ct, bmax) + 4 * (word0 + uw);
#pragma unroll
      for (int p = 0; p < 8; ++p) w[p] = *reinterpret_cast<const uint32_t*>(base + (p < bmax ? p : 0) * pb);
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      r.s[cb] = a.scales[(int64_t)g * N + ncol[cb]];
      r.z[cb] = a.zeros[(int64_t)g * N + ncol[cb]];
    }
  };

  float16_t acc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.0f;

  const int sh = 8 - bmax;                                   // codes come back as q 2^(8 - b_max)
  const uint32_t keep = 0x01010101u * (0xFFu >> sh);
  StepRegs cur;
  load_step(0, cur);
  for (int g = 0; g < G; ++g) {
    // ---- X tile and rebuilt codes of this step into LDS
#pragma unroll
    for (int u = 0; u < kXChunks; ++u) {
      const int q = tid + u * kPThreads;
      u32x4_t v = cur.x[u];
      const bool ok = (cur.xok >> u) & 1u;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = ok ? v[e] : 0u;
      *reinterpret_cast<u32x4_t*>(&s_x[(q >> 4) * kXPitch + 8 * (q & 15)]) = v;
    }
    {
      uint32_t w1[8], w2[8], d1[8], d2[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        w1[p] = (cur.ok1 && p < bmax) ? cur.w1[p] : 0u;
        w2[p] = (cur.ok2 && p < bmax) ? cur.w2[p] : 0u;
      }
      planes_to_codes<8>(w1, d1);
      planes_to_codes<8>(w2, d2);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        d1[m] = (d1[m] >> sh) & keep;
        d2[m] = (d2[m] >> sh) & keep;
      }
      const int kb = up >> 2, rr = up & 3;
      uint32_t* dst = s_w + (kb * kPN + 32 * uw) * 4 + rr;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // [row 2p code, 0x64, row 2p+1 code, 0x64] = fp16 (1024 + c1, 1024 + c2)
          const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24);
          const uint32_t pr = __builtin_amdgcn_perm(d2[m], d1[m], sel) | 0x64006400u;
          const half2_t c = __builtin_bit_cast(half2_t, pr) - (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
          const int col = 4 * m + j;
          dst[(col ^ kb) * 4] = __builtin_bit_cast(uint32_t, c);
        }
      }
    }
    // scale and zero of this step, duplicated into both halves
    uint32_t s2[2], z2[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      s2[cb] = (uint32_t)cur.s[cb] * 0x00010001u;
      z2[cb] = (uint32_t)cur.z[cb] * 0x00010001u;
    }
    __syncthreads();
    if (g + 1 < G) load_step(g + 1, cur);

    // ---- MFMAs over the step: 8 sub-steps of 16 rows
#pragma unroll
    for (int s16 = 0; s16 < kPK / 16; ++s16) {
      half8_t af[2], bf[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = 64 * wr + 32 * rb + (lane & 31);
        af[rb] = *reinterpret_cast<const half8_t*>(&s_x[row * kXPitch + 16 * s16 + 8 * (lane >> 5)]);
      }
      const int kb = 2 * s16 + (lane >> 5);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int nl = 64 * wc + 32 * cb;
        // copied into a plain array: taking elements of the loaded vector
        // inside a bit cast made this compiler read only the first dword
        uint32_t raw[4], wv[4];
        __builtin_memcpy(raw, &s_w[(kb * kPN + nl + ((lane & 31) ^ kb)) * 4], 16);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          wv[e] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
                                                   __builtin_bit_cast(half2_t, raw[e]),
                                                   __builtin_bit_cast(half2_t, s2[cb]),
                                                   __builtin_bit_cast(half2_t, z2[cb])));
        __builtin_memcpy(&bf[cb], wv, 16);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[rb], bf[cb], acc[rb][cb], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- output: lane holds column (lane & 31) of each block, rows
  // 8 (v / 4) + 4 (lane / 32) + v % 4
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int64_t n = n0 + 64 * wc + 32 * cb + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + 64 * wr + 32 * rb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M && n < N) a.Y[m * N + n] = acc[rb][cb][v];
      }
    }
}

int launch_prefill(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros, const uint16_t* X,
                   int64_t M, int64_t K, int64_t N, int bmax, float* Y, hipStream_t s) {
  const int64_t mt = (M + kPM - 1) / kPM;
  const int64_t nt = (padded_cols(N) + kPN - 1) / kPN;
  if (mt > 65535) return fail(GRINQH_EINVAL, "M = %lld: more than %d token tiles", (long long)M, 65535 * kPM);
  PrefillArgs a{planes, scales, zeros, X, Y, M, K, N, bmax};
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)nt, (unsigned)mt), dim3(kPThreads), 0, s, a);
  return check_launch("grinqh_prefill");
}

}  // namespace grinqh
