// wsg_argmax for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// span keys of its first launch go to a library-owned device array instead
// of a caller workspace.  The kernels are wsg_argmax's own.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy from the moment the code object is loaded until
// the process ends.  Host code never passes the array's name to a kernel
// (on the host that name is a stand-in, not a device address): the first
// call on each device looks up that device's address with
// hipGetSymbolAddress and keeps it.
#include <mutex>

#include "../../include/wsg.h"
#include "argmax.hpp"
#include "status.hpp"

namespace wsg {

namespace {

// 16384 keys (128 KiB): one key per 4096 logits and row, e.g. 431 rows of a
// 151936-entry vocabulary.
constexpr int kScratchKeys = 16384;
__device__ __align__(256) unsigned long long scratch[kScratchKeys];

constexpr int kMaxDevices = 64;
unsigned long long* g_scratch[kMaxDevices];   // per device, from hipGetSymbolAddress
std::mutex g_scratch_mu;

// The current device's copy of the scratch array (looked up once per device).
wsg_status scratch_on_current_device(unsigned long long** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WSG_ERR_HIP, "wsg_argmax_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(WSG_ERR_UNSUPPORTED, "wsg_argmax_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(WSG_ERR_HIP, "wsg_argmax_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch[dev] = static_cast<unsigned long long*>(p);
  }
  *out = g_scratch[dev];
  return WSG_OK;
}

}  // namespace

}  // namespace wsg

using namespace wsg;

extern "C" wsg_status wsg_argmax_noalloc(int32_t dtype, int32_t rows, int32_t n, const void* d_logits,
                                         int32_t* d_out, void* hip_stream) {
  clear_error();
  wsg_status st = argmax_check("wsg_argmax_noalloc", dtype, rows, n, d_logits, d_out);
  if (st != WSG_OK) return st;
  const size_t keys = argmax_keys(rows, n);
  if (keys > (size_t)kScratchKeys)
    return fail(WSG_ERR_INVALID_ARG,
                "wsg_argmax_noalloc: %d rows of %d logits need %zu span keys, more than the %d-key scratch "
                "(at most rows * ceil(n / 4096) = %d)",
                rows, n, keys, kScratchKeys, kScratchKeys);
  unsigned long long* ptr = nullptr;
  st = scratch_on_current_device(&ptr);
  if (st != WSG_OK) return st;
  (void)hipGetLastError();
  // Every key the second launch reads is written by the first in the same
  // call, so nothing in the array has to start at zero.
  argmax_rows(dtype, rows, n, d_logits, d_out, ptr, static_cast<hipStream_t>(hip_stream));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WSG_ERR_HIP, "wsg_argmax_noalloc: kernel launch failed: %s", hipGetErrorString(e));
  return WSG_OK;
}
