// kvc_compress_event_noalloc: the whole event with its scratch memory in a
// file-scope device array instead of a caller-supplied workspace, for callers
// that cannot allocate (code under HIP graph capture, serving loops that
// forbid allocation).  Each GPU the library runs on holds its own copy of the
// array from module load until the process ends.
#include <mutex>

#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr size_t kScratchBytes = KVC_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size must keep the 256-byte alignment");

// Device-side scratch.  In host code this name is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device the work of `stream` runs on.
hipError_t stream_device(hipStream_t stream, int* dev) {
  if (stream == nullptr) return hipGetDevice(dev);
  return hipStreamGetDevice(stream, dev);
}

// Device address of the scratch array on device `dev`, looked up once with
// that device current.  Returns nullptr on failure.
void* scratch_on(int dev) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev]) return g_scratch[dev];
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || ptr == nullptr) return nullptr;
  g_scratch[dev] = ptr;
  return ptr;
}

}  // namespace
}  // namespace kvc

extern "C" int kvc_compress_event_noalloc(const kvc_params* p, const void* q_win, const void* k,
                                          const void* v, const uint64_t* credit_in, void* k_out,
                                          void* v_out, uint64_t* credit_out, int32_t* kept_out,
                                          float* u_out, void* stream) {
  const int rc = kvc_check_params(p);
  if (rc != KVC_OK) return rc;
  if (p->n_heads == 0) return KVC_OK;
  if (kvc_workspace_bytes(p) > kvc::kScratchBytes) return KVC_ESCRATCH;
  int dev = -1;
  if (kvc::stream_device(hipStream_t(stream), &dev) != hipSuccess || dev < 0 ||
      dev >= kvc::kMaxDevices)
    return KVC_EDEVICE;
  void* ws = kvc::scratch_on(dev);
  if (ws == nullptr) return KVC_EDEVICE;
  return kvc_compress_event(p, q_win, k, v, credit_in, k_out, v_out, credit_out, kept_out, u_out,
                            ws, kvc::kScratchBytes, stream);
}
