// nq_lrb_linear_noalloc: the layer with its workspace in a fixed device array
// of the library, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable: every GPU the library runs on
// gets its own copy when the code object is loaded there, and keeps it until
// the process ends.  Host code never uses the array's name as an address (in
// host code it names a host-side stand-in); the device address of each GPU's
// copy is looked up once per device with hipGetSymbolAddress and kept.
#include <mutex>

#include "nq_internal.h"

namespace nq {
namespace {

static __device__ __align__(256) unsigned char scratch[NQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up on the
// first call on each device, with that device current).
nq_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "nq_lrb_linear_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("nq_lrb_linear_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    return NQ_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "nq_lrb_linear_noalloc: hipGetSymbolAddress");
    if (!p) {
      set_error("nq_lrb_linear_noalloc: no device address for the scratch array");
      return NQ_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NQ_OK;
}

}  // namespace
}  // namespace nq

using namespace nq;

extern "C" nq_status nq_lrb_linear_noalloc(const nq_lrb* L, const void* x, nq_dtype x_dtype, int64_t T, float* y,
                                           void* stream) {
  clear_error();
  const char* who = "nq_lrb_linear_noalloc";
  nq_status st = check_lrb(who, L);
  if (st != NQ_OK) return st;
  if ((st = check_io(who, L, x, x_dtype, T, y)) != NQ_OK) return st;
  const size_t need = linear_workspace(*L, T);
  if (need > (size_t)NQ_NOALLOC_SCRATCH_BYTES) {
    set_error("%s: this call needs %zu bytes of workspace, above the fixed %zu-byte scratch; use nq_lrb_linear "
              "with a caller workspace",
              who, need, (size_t)NQ_NOALLOC_SCRATCH_BYTES);
    return NQ_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != NQ_OK) return st;
  // the decode regime keeps its counters in the stream's counter slot (or
  // clears them in the array with a fill kernel); the GEMM regime writes every
  // workspace value before reading it
  return hip_status(launch_linear(*L, x, x_dtype, T, y, ws, (hipStream_t)stream), "nq_lrb_linear_noalloc launch");
}
