// Host-side launchers of the stand-alone GEMV family (arguments already
// validated by the C ABI layer).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wsg {

// dtype 0 = FP32 weights/activations, 1 = FP16; R in {1,2,4,8}; T in {1,2};
// grid 0 = one row group per wave; flags bit 0 = non-temporal weight loads.
void gemv_dispatch(int dtype, int M, int K, int T, int R, int grid, int flags, const void* W,
                   const void* X, float* Y, hipStream_t s);

void gemv_q4_dispatch(int M, int K, int T, int R, int grid, int flags, const uint32_t* Wq,
                      const void* S, const void* X, float* Y, hipStream_t s);

// Read-only streaming reference: bytes % 16 == 0, bytes >= 16.
void stream_read_dispatch(const void* buf, int64_t bytes, float* out, hipStream_t s);

}  // namespace wsg
