// C-ABI entry points: host-side validation, then one launcher per call.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.hpp"

namespace grinqh {

static thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_last_error[0] = 0; }

// [a, a + na) and [b, b + nb) share a byte.
static bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// A buffer the call zeroes while it reads x and adds into y may overlap
// neither (its writes land while other workgroups still read x).
static int check_clear(const float* clear, const float* y, const uint16_t* x, int64_t K, int64_t N) {
  if (!clear) return GRINQH_OK;
  if (overlaps(clear, (uint64_t)N * 4, y, (uint64_t)N * 4)) return fail(GRINQH_EINVAL, "clear overlaps y");
  if (overlaps(clear, (uint64_t)N * 4, x, (uint64_t)K * 2)) return fail(GRINQH_EINVAL, "clear overlaps x");
  return GRINQH_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GRINQH_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return GRINQH_OK;
}

static inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// max_level: the widest level allowed (8, or the store's b_max for the fused VMM).
int check_assign_params(const float* thresholds, const uint8_t* levels, int n, int max_level,
                               AssignParams* ap) {
  if (n < 0 || n > kMaxThresholds) return fail(GRINQH_EINVAL, "n = %d thresholds, expected 0..%d", n, kMaxThresholds);
  if (n > 0 && !thresholds) return fail(GRINQH_EINVAL, "thresholds is NULL");
  if (!levels) return fail(GRINQH_EINVAL, "levels is NULL");
  memset(ap, 0, sizeof(*ap));
  ap->n = n;
  for (int t = 0; t < n; ++t) {
    const float v = thresholds[t];
    if (isnan(v) || v < 0.0f) return fail(GRINQH_EINVAL, "threshold %d is %g (must be >= 0, not NaN)", t, (double)v);
    if (t > 0 && v < thresholds[t - 1]) return fail(GRINQH_EINVAL, "thresholds decrease at index %d", t);
    ap->th[t] = v;
  }
  for (int t = 0; t <= n; ++t) {
    if (levels[t] > max_level)
      return fail(GRINQH_EINVAL, "level %d is %u (must be 0..%d)", t, (unsigned)levels[t], max_level);
    ap->lv[t] = levels[t];
  }
  // Unused slots: thresholds +inf and levels[n] repeated, so the kernels
  // compare against all kMaxThresholds slots without looking at n (a finite
  // |x| never reaches +inf; +inf reaches every slot and still gets levels[n]).
  for (int t = n; t < kMaxThresholds; ++t) {
    ap->th[t] = INFINITY;
    ap->lv[t + 1] = levels[n];
  }
  return GRINQH_OK;
}

static int check_shape(int64_t K, int64_t N, int b_max) {
  if (K <= 0 || N <= 0) return fail(GRINQH_EINVAL, "K = %lld, N = %lld must be positive", (long long)K, (long long)N);
  if (K >= (int64_t(1) << 31) || N >= (int64_t(1) << 31)) return fail(GRINQH_EINVAL, "K or N too large");
  if (b_max < 1 || b_max > GRINQH_MAX_BITS) return fail(GRINQH_EINVAL, "b_max = %d, expected 1..8", b_max);
  if (K * padded_cols(N) >= (int64_t(1) << 40)) return fail(GRINQH_EINVAL, "store larger than 2^40 bytes");
  return GRINQH_OK;
}

int check_layer(const void* planes, const void* scales, const void* zeros, const void* x,
                       const void* y, int64_t K, int64_t N, int b_max) {
  if (!planes || !scales || !zeros || !x || !y) return fail(GRINQH_EINVAL, "NULL data pointer");
  return check_shape(K, N, b_max);
}

static int check_vmm_common(const void* planes, const void* scales, const void* zeros, const void* x,
                            const void* y, int64_t K, int64_t N, int b_max, const void* ws, size_t ws_bytes) {
  const int st = check_layer(planes, scales, zeros, x, y, K, N, b_max);
  if (st != GRINQH_OK) return st;
  const VmmGeometry g = vmm_geometry(K, N);
  if (!ws && g.bytes > 0) return fail(GRINQH_EINVAL, "workspace is NULL");
  if ((int64_t)ws_bytes < g.bytes)
    return fail(GRINQH_EINVAL, "workspace has %zu bytes, needs %lld", ws_bytes, (long long)g.bytes);
  return GRINQH_OK;
}

}  // namespace grinqh

using namespace grinqh;

extern "C" {

int grinqh_layout_version(void) { return 4; }

const char* grinqh_status_string(int status) {
  switch (status) {
    case GRINQH_OK: return "ok";
    case GRINQH_EINVAL: return "invalid argument";
    case GRINQH_EDEVICE: return "device error";
    case GRINQH_ENOSYS: return "not implemented";
    default: return "unknown status";
  }
}

const char* grinqh_last_error(void) { return g_last_error; }

int64_t grinqh_planes_bytes(int64_t K, int64_t N, int b_max) {
  if (K <= 0 || N <= 0 || b_max < 1 || b_max > GRINQH_MAX_BITS) return -1;
  return K * padded_cols(N) / 8 * b_max;
}

int64_t grinqh_workspace_bytes(int64_t K, int64_t N) {
  if (K <= 0 || N <= 0) return -1;
  return vmm_geometry(K, N).bytes;
}

int grinqh_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!workspace && workspace_bytes) return fail(GRINQH_EINVAL, "workspace is NULL");
  if (workspace_bytes == 0) return GRINQH_OK;
  return launch_fill_zero(workspace, workspace_bytes, as_stream(stream));
}

int grinqh_pack(const uint8_t* codes, int64_t K, int64_t N, int b_max, uint8_t* planes, void* stream) {
  g_last_error[0] = 0;
  if (!codes || !planes) return fail(GRINQH_EINVAL, "NULL pointer");
  const int st = check_shape(K, N, b_max);
  if (st != GRINQH_OK) return st;
  return launch_pack(codes, K, N, b_max, planes, as_stream(stream));
}

int grinqh_calibrate(const uint16_t* calib, int64_t V, int64_t K, const double* P, int n_levels,
                     float* thresholds, void* stream) {
  g_last_error[0] = 0;
  if (!calib || !P || (!thresholds && n_levels > 1)) return fail(GRINQH_EINVAL, "NULL pointer");
  if (V <= 0 || K <= 0) return fail(GRINQH_EINVAL, "V = %lld, K = %lld must be positive", (long long)V, (long long)K);
  if (V >= (int64_t(1) << 31) || K >= (int64_t(1) << 31)) return fail(GRINQH_EINVAL, "V or K too large");
  if (n_levels < 1 || n_levels > kMaxThresholds + 1) return fail(GRINQH_EINVAL, "n_levels = %d, expected 1..9", n_levels);
  double cuts[kMaxThresholds];
  double acc = 0.0;
  for (int k = 0; k < n_levels; ++k) {
    if (!isfinite(P[k]) || P[k] < 0.0) return fail(GRINQH_EINVAL, "P[%d] = %g must be finite and >= 0", k, P[k]);
  }
  // c_k = p_0 + ... + p_{k-1}, accumulated left to right.
  for (int k = 1; k < n_levels; ++k) {
    acc = acc + P[k - 1];
    cuts[k - 1] = acc;
  }
  if (n_levels == 1) return GRINQH_OK;
  return launch_calibrate(calib, V, K, cuts, n_levels - 1, thresholds, as_stream(stream));
}

int grinqh_assign_bits(const uint16_t* x, int64_t K, const float* thresholds, const uint8_t* levels,
                       int n, uint8_t* bits, int32_t* active_idx, int32_t* n_active, void* stream) {
  g_last_error[0] = 0;
  if (!x || !bits || !active_idx || !n_active) return fail(GRINQH_EINVAL, "NULL pointer");
  if (K <= 0 || K >= (int64_t(1) << 31)) return fail(GRINQH_EINVAL, "K = %lld out of range", (long long)K);
  AssignParams ap;
  int st = check_assign_params(thresholds, levels, n, GRINQH_MAX_BITS, &ap);
  if (st != GRINQH_OK) return st;
  return launch_assign(x, K, ap, bits, active_idx, n_active, as_stream(stream));
}

int grinqh_vmm(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
               const uint16_t* x, const uint8_t* bits, const int32_t* active_idx,
               const int32_t* n_active, int64_t K, int64_t N, int b_max, float* y,
               void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  int st = check_vmm_common(planes, scales, zeros, x, y, K, N, b_max, workspace, workspace_bytes);
  if (st != GRINQH_OK) return st;
  if (!bits || !active_idx || !n_active) return fail(GRINQH_EINVAL, "NULL assignment pointer");
  return launch_vmm_list(planes, scales, zeros, x, bits, active_idx, n_active, K, N, b_max, y, workspace,
                         as_stream(stream));
}

int grinqh_decode_vmm(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                      const uint16_t* x, int64_t K, int64_t N, int b_max,
                      const float* thresholds, const uint8_t* levels, int n, float* y,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  int st = check_vmm_common(planes, scales, zeros, x, y, K, N, b_max, workspace, workspace_bytes);
  if (st != GRINQH_OK) return st;
  AssignParams ap;
  st = check_assign_params(thresholds, levels, n, b_max, &ap);
  if (st != GRINQH_OK) return st;
  return launch_vmm_fused(planes, scales, zeros, x, K, N, b_max, ap, y, workspace, as_stream(stream));
}

int grinqh_decode_vmm_accumulate(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                                 const uint16_t* x, int64_t K, int64_t N, int b_max,
                                 const float* thresholds, const uint8_t* levels, int n,
                                 float* y, float* clear, void* stream) {
  g_last_error[0] = 0;
  int st = check_layer(planes, scales, zeros, x, y, K, N, b_max);
  if (st == GRINQH_OK) st = check_clear(clear, y, x, K, N);
  if (st != GRINQH_OK) return st;
  AssignParams ap;
  st = check_assign_params(thresholds, levels, n, b_max, &ap);
  if (st != GRINQH_OK) return st;
  return launch_vmm_accumulate(planes, scales, zeros, x, K, N, b_max, ap, y, clear, as_stream(stream));
}

int grinqh_decode_vmm_accumulate_group(int count, const uint8_t* const* planes, const uint16_t* const* scales,
                                       const uint16_t* const* zeros, const uint16_t* const* x, int64_t K,
                                       const int64_t* N, int b_max, const float* const* thresholds,
                                       const uint8_t* const* levels, const int* n, float* const* y,
                                       float* const* clear, void* stream) {
  g_last_error[0] = 0;
  if (count < 1 || count > GRINQH_MAX_GROUP)
    return fail(GRINQH_EINVAL, "count = %d members, expected 1..%d", count, GRINQH_MAX_GROUP);
  if (!planes || !scales || !zeros || !x || !N || !thresholds || !levels || !n || !y)
    return fail(GRINQH_EINVAL, "NULL member array");
  VmmMember mem[GRINQH_MAX_GROUP];
  for (int m = 0; m < count; ++m) {
    int st = check_layer(planes[m], scales[m], zeros[m], x[m], y[m], K, N[m], b_max);
    if (st == GRINQH_OK) st = check_assign_params(thresholds[m], levels[m], n[m], b_max, &mem[m].ap);
    if (st != GRINQH_OK) {
      char why[sizeof(g_last_error)];
      snprintf(why, sizeof(why), "%s", g_last_error);
      return fail(st, "member %d: %s", m, why);
    }
    float* c = clear ? clear[m] : nullptr;
    if (c) {
      for (int k = 0; k < count; ++k) {
        if (overlaps(c, (uint64_t)N[m] * 4, y[k], (uint64_t)N[k] * 4))
          return fail(GRINQH_EINVAL, "member %d: clear overlaps the y of member %d", m, k);
        if (overlaps(c, (uint64_t)N[m] * 4, x[k], (uint64_t)K * 2))
          return fail(GRINQH_EINVAL, "member %d: clear overlaps the x of member %d", m, k);
      }
    }
    mem[m].planes = planes[m];
    mem[m].scales = scales[m];
    mem[m].zeros = zeros[m];
    mem[m].x = x[m];
    mem[m].y = y[m];
    mem[m].clear = c;
    mem[m].N = (int)N[m];
  }
  return launch_vmm_group(count, mem, K, b_max, as_stream(stream));
}

int64_t grinqh_lut_entries(int64_t N, int b_max) {
  if (N <= 0 || b_max < 1 || b_max > GRINQH_MAX_BITS) return -1;
  return N * ((int64_t(1) << (b_max + 1)) - 2);
}

int grinqh_decode_vmm_lut(const uint8_t* planes, const uint16_t* lut, const uint16_t* x, int64_t K, int64_t N,
                          int b_max, const float* thresholds, const uint8_t* levels, int n, float* y,
                          float* clear, void* stream) {
  g_last_error[0] = 0;
  if (!lut) return fail(GRINQH_EINVAL, "NULL data pointer");
  int st = check_layer(planes, lut, lut, x, y, K, N, b_max);
  if (st == GRINQH_OK) st = check_clear(clear, y, x, K, N);
  if (st != GRINQH_OK) return st;
  AssignParams ap;
  st = check_assign_params(thresholds, levels, n, b_max, &ap);
  if (st != GRINQH_OK) return st;
  return launch_vmm_lut(planes, lut, x, K, N, b_max, ap, y, clear, as_stream(stream));
}

int64_t grinqh_dense_bytes(int64_t K, int64_t N) {
  if (K <= 0 || N <= 0) return -1;
  return unpack_dense_bytes(K, N);
}

int grinqh_unpack_dense(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros, int64_t K,
                        int64_t N, int b_max, void* dense, size_t dense_bytes, void* stream) {
  g_last_error[0] = 0;
  int st = check_layer(planes, scales, zeros, dense, dense, K, N, b_max);
  if (st != GRINQH_OK) return st;
  if ((int64_t)dense_bytes < unpack_dense_bytes(K, N))
    return fail(GRINQH_EINVAL, "dense buffer has %zu bytes, needs %lld", dense_bytes, (long long)unpack_dense_bytes(K, N));
  if (reinterpret_cast<uintptr_t>(dense) % 16 != 0) return fail(GRINQH_EINVAL, "dense buffer must be 16-byte aligned");
  return launch_unpack_dense(planes, scales, zeros, K, N, b_max, dense, as_stream(stream));
}

int grinqh_dense_gemm(const uint16_t* X, const void* dense, int64_t M, int64_t K, int64_t N, float* Y, void* stream) {
  g_last_error[0] = 0;
  if (!X || !dense || !Y) return fail(GRINQH_EINVAL, "NULL data pointer");
  if (M <= 0 || M >= (int64_t(1) << 31)) return fail(GRINQH_EINVAL, "M = %lld out of range", (long long)M);
  int st = check_shape(K, N, 8);
  if (st != GRINQH_OK) return st;
  if (reinterpret_cast<uintptr_t>(dense) % 16 != 0) return fail(GRINQH_EINVAL, "dense buffer must be 16-byte aligned");
  return launch_dense_gemm(X, dense, M, K, N, Y, as_stream(stream));
}

int grinqh_prefill(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                   const uint16_t* X, int64_t M, int64_t K, int64_t N, int b_max, float* Y, void* stream) {
  g_last_error[0] = 0;
  int st = check_layer(planes, scales, zeros, X, Y, K, N, b_max);
  if (st != GRINQH_OK) return st;
  if (M <= 0 || M >= (int64_t(1) << 31)) return fail(GRINQH_EINVAL, "M = %lld out of range", (long long)M);
  return launch_prefill(planes, scales, zeros, X, M, K, N, b_max, Y, as_stream(stream));
}

}  // extern "C"
