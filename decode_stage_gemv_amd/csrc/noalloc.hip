// Allocation-free form of the fused decode step (grinqh_decode_vmm_noalloc).
//
// grinqh_decode_vmm needs a caller-provided workspace for its split-K partial
// rows and per-tile counters.  Callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc) use
// this entry point instead: the workspace is a file-scope device array of a
// fixed size, one copy per GPU for the life of the process.  The kernels are
// the ones grinqh_decode_vmm launches; only where the workspace comes from
// differs.
#include <mutex>

#include "common.hpp"

namespace grinqh {

// Layout of the array: the tile counters and the column words (accumulators,
// then masks) at fixed places at the front, so that every layer shape finds
// them where every earlier call, of any shape, left zeros; the split-K
// partial rows after them.
constexpr size_t kScratchBytes = GRINQH_NOALLOC_SCRATCH_BYTES;
constexpr size_t kCounterBytes = 64 * 1024;   // up to 16384 column tiles
constexpr int64_t kMaxWordCols = 262144;      // column words for N up to 262144
constexpr size_t kWordBytes = 2 * kMaxWordCols * 8;
constexpr size_t kPartialBytes = kScratchBytes - kCounterBytes - kWordBytes;

// Zero-initialised when the code object is loaded.  The counters and column
// words must be zero when a call starts: a completed call leaves every
// counter and word it used at zero again (the last workgroup of a tile, or
// the last add to a column, resets it), and the partial rows are always
// written before they are read.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};   // device address of `scratch` on each GPU
}  // namespace

// The device address of this GPU's copy of `scratch`.  Host code never uses
// the array's own name as an address (on the host it is only a stand-in
// symbol); the address comes from the runtime, once per device, with that
// device current.
static int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GRINQH_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(GRINQH_EDEVICE, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GRINQH_EDEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return GRINQH_OK;
}

int noalloc_scratch(int64_t partial_bytes, int64_t tiles, int64_t cols, float** partials, unsigned** counters,
                    unsigned long long** words, int64_t* max_cols) {
  if (partial_bytes > (int64_t)kPartialBytes)
    return fail(GRINQH_EINVAL,
                "layer needs %lld bytes of split-K partials; the allocation-free entry point holds %zu",
                (long long)partial_bytes, kPartialBytes);
  if (tiles * 4 > (int64_t)kCounterBytes)
    return fail(GRINQH_EINVAL, "%lld column tiles; the allocation-free entry point holds %zu",
                (long long)tiles, kCounterBytes / 4);
  if (cols > kMaxWordCols)
    return fail(GRINQH_EINVAL, "%lld padded columns; the allocation-free entry point holds %lld",
                (long long)cols, (long long)kMaxWordCols);
  void* base = nullptr;
  const int st = scratch_address(&base);
  if (st != GRINQH_OK) return st;
  *counters = reinterpret_cast<unsigned*>(base);
  *words = reinterpret_cast<unsigned long long*>(reinterpret_cast<uint8_t*>(base) + kCounterBytes);
  *max_cols = kMaxWordCols;
  *partials = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(base) + kCounterBytes + kWordBytes);
  return GRINQH_OK;
}

}  // namespace grinqh

using namespace grinqh;

extern "C" int grinqh_decode_vmm_noalloc(const uint8_t* planes, const uint16_t* scales, const uint16_t* zeros,
                                         const uint16_t* x, int64_t K, int64_t N, int b_max,
                                         const float* thresholds, const uint8_t* levels, int n, float* y,
                                         void* stream) {
  clear_error();
  int st = check_layer(planes, scales, zeros, x, y, K, N, b_max);
  if (st != GRINQH_OK) return st;
  AssignParams ap;
  st = check_assign_params(thresholds, levels, n, b_max, &ap);
  if (st != GRINQH_OK) return st;
  const VmmGeometry g = vmm_geometry(K, N);
  float* partials = nullptr;
  unsigned* counters = nullptr;
  unsigned long long* words = nullptr;
  int64_t max_cols = 0;
  st = noalloc_scratch(g.partial_floats * 4, g.tiles, padded_cols(N), &partials, &counters, &words, &max_cols);
  if (st != GRINQH_OK) return st;
  return launch_vmm_fused_split(planes, scales, zeros, x, K, N, b_max, ap, y, partials, counters, words, max_cols,
                                reinterpret_cast<hipStream_t>(stream));
}
