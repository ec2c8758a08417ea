// Dense fp16 GEMM over weights unpacked into B-fragment order (unpack.hip):
// the matrix half of the prefill path that unpacks once and multiplies
// densely (GRINQH paper, section 4 "Prefill vs. Decoding Evaluation").
//
//   Y[m][n] = sum_k X[m][k] W[k][n],  X fp16 [M][K], W fp16 in fragment order,
//   Y fp32 [M][N], products summed in fp32 by v_mfma_f32_32x32x16_f16.
//
// Work split.  A workgroup (8 waves) owns a 256-token x 256-column tile of Y;
// wave (r, c) of the 2 x 4 wave grid owns 128 tokens x 64 columns as 4 x 2
// blocks of 32 x 32.  K is walked 64 rows per step.  X goes through LDS
// (double-buffered, rows padded by 16 bytes so that the A-fragment reads are
// conflict-free, one barrier per step).  The B fragments need no LDS: in
// fragment order each lane's 16 bytes are contiguous with its neighbours',
// so a wave loads them straight into registers, each sub-step's fragments
// reloaded for the next step right after its MFMAs.  Workgroups
// that share a column strip are numbered onto one XCD (consecutive ids go to
// different XCDs) so that they read the strip through one L2.
#include "common.hpp"

namespace grinqh {

namespace {

constexpr int kGM = 256;                // tokens per workgroup tile
constexpr int kGN = 256;                // columns per workgroup tile
constexpr int kGK = 64;                 // rows per step
constexpr int kGThreads = 512;
constexpr int kGPitch = kGK + 8;        // halves per LDS row of the X tile
constexpr int kGXChunks = kGM * kGK / 8 / kGThreads;   // 16-byte X chunks per thread per step (4)
constexpr int kXCDs = 8;                // MI355X
constexpr uint32_t kOOR = 0x7FFFFF00u;
constexpr int kRsrcWord3 = 0x00020000;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const uint16_t* X;
  const uint32_t* W;      // fragment order, dwords
  float* Y;
  int64_t M, K, N;
  int m_tiles, n_tiles;
};

__device__ inline __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, n,
                                           kRsrcWord3);
}

// B fragments of one step for this lane: [k16 sub-step][column block][4 dwords]
struct BRegs {
  uint32_t v[kGK / 16][2][4];
};

}  // namespace

// VEC: K a multiple of 8 and X 16-byte aligned, so each 8-half X chunk is one
// 16-byte load; otherwise eight 2-byte loads.  Every load is unconditional
// (buffer loads past the tile read zero, the weights are padded to a whole
// number of steps, the prefetch past the last step re-reads that step), so
// that the compiler's wait counts stay exact and loads stay in flight across
// a step.
template <bool VEC>
__global__ __launch_bounds__(kGThreads) void dense_gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_x[2][kGM * kGPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wid >> 2, wc = wid & 3;
  const int64_t M = a.M, N = a.N;
  const int K = (int)a.K;
  const int64_t Np = padded_cols(N);

  const int T = a.m_tiles * a.n_tiles;
  int L = blockIdx.x;
  if (T % kXCDs == 0) L = (L % kXCDs) * (T / kXCDs) + L / kXCDs;
  const int64_t n0 = (int64_t)(L / a.m_tiles) * kGN;
  const int64_t m0 = (int64_t)(L % a.m_tiles) * kGM;
  const int steps = (K + kGK - 1) / kGK;   // the weights hold 64 steps' rows exactly

  // X: buffer over this tile's tokens; chunk c of this thread is token
  // (tid + 512 c) / 8, halves 8 ((tid + 512 c) % 8) .. + 7 of the step
  const int64_t mrows = (M - m0) < kGM ? (M - m0) : kGM;
  const __amdgpu_buffer_rsrc_t xrs = uniform_rsrc(a.X + m0 * K, mrows * K * 2);
  // W: this lane's column in each block cb (clamped to the padded width: a
  // 256-column tile can reach 128 columns past it; those outputs are not
  // stored)
  const uint32_t* wcol[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int64_t n = n0 + 64 * wc + 32 * cb + (lane & 31);
    wcol[cb] = a.W + (n < Np ? n : Np - 1) * 4;
  }

  constexpr int kXRegs = VEC ? 4 : 8;      // dwords (VEC) or halves (one per register) per chunk
  auto load_x = [&](int st, uint32_t (&x)[kGXChunks][kXRegs]) {
    const int k0 = st * kGK;
#pragma unroll
    for (int c = 0; c < kGXChunks; ++c) {
      const int q = tid + c * kGThreads;
      const int k = k0 + 8 * (q & 7);
      const uint32_t rowb = (uint32_t)(q >> 3) * (uint32_t)K * 2u;
      if constexpr (VEC) {
        const uint32_t off = k < K ? rowb + (uint32_t)(2 * k) : kOOR;
        const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)off, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[c][e] = t[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t off = k + e < K ? rowb + (uint32_t)(2 * (k + e)) : kOOR;
          x[c][e] = __builtin_amdgcn_raw_buffer_load_b16(xrs, (int)off, 0, 0);
        }
      }
    }
  };
  auto write_x = [&](int buf, const uint32_t (&x)[kGXChunks][kXRegs]) {
#pragma unroll
    for (int c = 0; c < kGXChunks; ++c) {
      const int q = tid + c * kGThreads;
      uint32_t d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (VEC) d[e] = x[c][e];
        else d[e] = (x[c][2 * e] & 0xFFFFu) | (x[c][2 * e + 1] << 16);
      }
      __builtin_memcpy(&s_x[buf][(q >> 3) * kGPitch + 8 * (q & 7)], d, 16);
    }
  };
  auto load_b16 = [&](int st, int s16, uint32_t (&v)[2][4]) {
    const int64_t kb = (int64_t)st * (kGK / 8) + 2 * s16 + (lane >> 5);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const uint4 t = *reinterpret_cast<const uint4*>(wcol[cb] + kb * Np * 4);
      v[cb][0] = t.x;
      v[cb][1] = t.y;
      v[cb][2] = t.z;
      v[cb][3] = t.w;
    }
  };

  float16_t acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.0f;

  // MFMAs of one step from LDS buffer buf and the B fragments in b; right
  // after a sub-step's MFMAs its fragments are reloaded for step nst (one
  // step ahead, one register set)
  // The scheduling barriers keep each sub-step's reloads right behind its
  // MFMAs (left alone, the compiler sinks them to the end of the step, where
  // the next step's first MFMAs would wait for them).
  BRegs b;
  auto read_a = [&](int buf, int s16, half8_t (&af)[4]) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int row = 128 * wr + 32 * rb + (lane & 31);
      __builtin_memcpy(&af[rb], &s_x[buf][row * kGPitch + 16 * s16 + 8 * (lane >> 5)], 16);
    }
  };
  auto mfma_step = [&](int buf, int nst) {
    half8_t af[2][4];
    read_a(buf, 0, af[0]);
#pragma unroll
    for (int s16 = 0; s16 < kGK / 16; ++s16) {
      if (s16 + 1 < kGK / 16) read_a(buf, s16 + 1, af[(s16 + 1) & 1]);
      half8_t bf[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) __builtin_memcpy(&bf[cb], b.v[s16][cb], 16);
      // the wave issuing MFMAs goes first while it does (the other wave on
      // the SIMD is loading or unpacking): keeps the matrix core fed
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[s16 & 1][rb], bf[cb], acc[rb][cb], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
      load_b16(nst, s16, b.v[s16]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline: X of step st + 1 is in registers while step st runs and is
  // written to the other LDS buffer before the step's MFMAs, so one barrier
  // per step suffices; B of step st + 1 is loaded during step st.  Past the
  // last step the loads repeat the last step (never used).
  // The prologue issues its loads in the loop's order (X before B) so that
  // the wait counts at the loop head come out the same from both edges.
  const int last = steps - 1;
  uint32_t xr[kGXChunks][kXRegs];
  load_x(0, xr);
  write_x(0, xr);
  load_x(last < 1 ? last : 1, xr);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s16 = 0; s16 < kGK / 16; ++s16) load_b16(0, s16, b.v[s16]);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  for (int st = 0; st < steps; ++st) {
    write_x((st + 1) & 1, xr);
    load_x(st + 2 < last ? st + 2 : last, xr);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(st & 1, st + 1 < last ? st + 1 : last);
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

int launch_dense_gemm(const uint16_t* X, const void* W, int64_t M, int64_t K, int64_t N, float* Y, hipStream_t s) {
  if (K >= (int64_t(1) << 21))
    return fail(GRINQH_EINVAL, "K = %lld: the dense GEMM handles K < 2^21", (long long)K);
  const int64_t mt = (M + kGM - 1) / kGM;
  const int64_t nt = (padded_cols(N) + kGN - 1) / kGN;
  if (mt * nt > 0x7FFFFFFF) return fail(GRINQH_EINVAL, "M x N needs more than 2^31 workgroups");
  GemmArgs a{X, reinterpret_cast<const uint32_t*>(W), Y, M, K, N, (int)mt, (int)nt};
  if (K % 8 == 0 && reinterpret_cast<uintptr_t>(X) % 16 == 0)
    hipLaunchKernelGGL(dense_gemm_kernel<true>, dim3((unsigned)(mt * nt)), dim3(kGThreads), 0, s, a);
  else
    hipLaunchKernelGGL(dense_gemm_kernel<false>, dim3((unsigned)(mt * nt)), dim3(kGThreads), 0, s, a);
  return check_launch("grinqh_dense_gemm");
}

}  // namespace grinqh
