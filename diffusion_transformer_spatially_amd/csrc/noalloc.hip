// Allocation-free form of the sensitive-row FFN (safe_rows_ffn_noalloc), for callers that cannot allocate
// device memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
// bf16 hidden activation between the two products, which safe_rows_ffn takes from a caller workspace,
// lives here in a file-scope device array of fixed size; the kernels are those of safe_rows_ffn.
//
// Each GPU the library runs on holds its own copy of the array (allocated with the code object) until the
// process ends.  Its device address is looked up once per device, with that device current, on the first
// call made there, and kept; the array's name itself is only a host-side stand-in and is never passed to
// a kernel.  Every call on a GPU shares that GPU's array: calls that overlap on one GPU (two streams, two
// threads) race on it.  Nothing in the array needs to start at zero: the first product writes every
// hidden row the second product reads for a row that is written out.
#include <mutex>

#include "common.hpp"

namespace safe {

constexpr size_t kFfnScratchBytes = static_cast<size_t>(32) << 20;  // 32 MiB: B * k * F * 2 bytes at most
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kFfnScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of this GPU's scratch array (looked up once per device).
static hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace safe

extern "C" size_t safe_rows_ffn_noalloc_max_bytes(void) { return safe::kFfnScratchBytes; }

extern "C" safe_status safe_rows_ffn_noalloc(const void* x, const int32_t* rows, int32_t k, int32_t B, int32_t N,
                                             int32_t D, int32_t F, const void* w1, const float* b1, const void* w2,
                                             const float* b2, void* cache, hipStream_t stream) {
  if (B < 1 || N < 1 || D < 1 || F < 1) return SAFE_ERR_SHAPE;
  if (k < 0 || k > N) return SAFE_ERR_RANGE;
  if (k == 0) return SAFE_OK;
  if (safe_rows_ffn_workspace_bytes(B, k, F) > safe::kFfnScratchBytes) return SAFE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (safe::scratch_address(&ws) != hipSuccess) return SAFE_ERR_HIP;
  return safe_rows_ffn(x, rows, k, B, N, D, F, w1, b1, w2, b2, cache, ws, safe::kFfnScratchBytes, stream);
}
