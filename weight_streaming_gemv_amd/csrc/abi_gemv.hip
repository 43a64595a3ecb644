// C ABI of the stand-alone GEMV family: argument validation, then launch.
#include "../../include/wsg.h"
#include "gemv.hpp"
#include "prefill.hpp"
#include "status.hpp"

using namespace wsg;

namespace {

bool valid_rows(int32_t& r) {
  if (r == 0) r = 1;   // cold-tuned default: one row per wave
  return r == 1 || r == 2 || r == 4 || r == 8;
}

wsg_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WSG_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return WSG_OK;
}

}  // namespace

extern "C" wsg_status wsg_gemv_ex(int32_t w_dtype, int32_t M, int32_t K, int32_t T, int32_t rows_per_wave,
                                  int32_t grid_blocks, int32_t flags, const void* d_W, const void* d_X,
                                  float* d_Y, void* hip_stream) {
  clear_error();
  if (w_dtype != WSG_F32 && w_dtype != WSG_F16) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv: bad dtype %d", w_dtype);
  if (M < 1 || K < 1) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv: M=%d K=%d must be >= 1", M, K);
  if (T < 1 || T > 2) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv: T=%d must be 1 or 2", T);
  // default shape for FP32 rows of 3072: two waves per row (one wave cannot
  // keep such a row's loads in flight)
  if (rows_per_wave == 0 && w_dtype == WSG_F32 && K == 3072) flags |= WSG_GEMV_SPLIT2;
  if (!valid_rows(rows_per_wave)) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv: rows_per_wave must be 1, 2, 4 or 8");
  if (grid_blocks < 0) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv: grid_blocks < 0");
  if (flags & ~(WSG_GEMV_NONTEMPORAL | WSG_GEMV_SPLIT2)) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv: unknown flags 0x%x", flags);
  if ((flags & WSG_GEMV_SPLIT2) &&
      (w_dtype != WSG_F32 || rows_per_wave != 1 || (K != 1024 && K != 2048 && K != 3072)))
    return fail(WSG_ERR_INVALID_ARG,
                "wsg_gemv: WSG_GEMV_SPLIT2 needs FP32 weights, one row per wave and K of 1024, 2048 or 3072 "
                "(dtype=%d rows_per_wave=%d K=%d)", w_dtype, rows_per_wave, K);
  if (!d_W || !d_X || !d_Y) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv: null pointer");
  if (((uintptr_t)d_W | (uintptr_t)d_X) & 15) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv: W and X must be 16-byte aligned");
  if ((int64_t)M * K > (int64_t)1 << 40) return fail(WSG_ERR_UNSUPPORTED, "wsg_gemv: matrix too large");
  gemv_dispatch(w_dtype, M, K, T, rows_per_wave, grid_blocks, flags, d_W, d_X, d_Y,
                static_cast<hipStream_t>(hip_stream));
  return check_launch("wsg_gemv");
}

extern "C" wsg_status wsg_gemv(int32_t w_dtype, int32_t M, int32_t K, int32_t T, int32_t rows_per_wave,
                               const void* d_W, const void* d_X, float* d_Y, void* hip_stream) {
  return wsg_gemv_ex(w_dtype, M, K, T, rows_per_wave, 0, 0, d_W, d_X, d_Y, hip_stream);
}

extern "C" wsg_status wsg_gemv_q4g64_ex(int32_t M, int32_t K, int32_t T, int32_t rows_per_wave,
                                        int32_t grid_blocks, int32_t flags, const uint32_t* d_Wq,
                                        const void* d_scales, const void* d_X, float* d_Y, void* hip_stream) {
  clear_error();
  if (M < 1 || K < 64 || K % 64 != 0) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv_q4g64: need M >= 1 and K a positive multiple of 64 (M=%d K=%d)", M, K);
  if (T < 1 || T > 2) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv_q4g64: T=%d must be 1 or 2", T);
  if (!valid_rows(rows_per_wave)) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv_q4g64: rows_per_wave must be 1, 2, 4 or 8");
  if (grid_blocks < 0) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv_q4g64: grid_blocks < 0");
  if (flags & ~WSG_GEMV_NONTEMPORAL) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv_q4g64: unknown flags 0x%x", flags);
  if (!d_Wq || !d_scales || !d_X || !d_Y) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv_q4g64: null pointer");
  if (((uintptr_t)d_Wq | (uintptr_t)d_X) & 15) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv_q4g64: Wq and X must be 16-byte aligned");
  if (((uintptr_t)d_scales) & 1) return fail(WSG_ERR_INVALID_ARG, "wsg_gemv_q4g64: scales must be 2-byte aligned");
  gemv_q4_dispatch(M, K, T, rows_per_wave, grid_blocks, flags, d_Wq, d_scales, d_X, d_Y,
                   static_cast<hipStream_t>(hip_stream));
  return check_launch("wsg_gemv_q4g64");
}

extern "C" wsg_status wsg_gemv_q4g64(int32_t M, int32_t K, int32_t T, int32_t rows_per_wave,
                                     const uint32_t* d_Wq, const void* d_scales, const void* d_X, float* d_Y,
                                     void* hip_stream) {
  return wsg_gemv_q4g64_ex(M, K, T, rows_per_wave, 0, 0, d_Wq, d_scales, d_X, d_Y, hip_stream);
}

extern "C" wsg_status wsg_gemm_nt_f32(int32_t M, int32_t N, int32_t K, const float* d_A, const float* d_B, float* d_C,
                                     int32_t accumulate, void* hip_stream) {
  clear_error();
  if (M < 1 || N < 64 || N % 64 != 0 || K < 32 || K % 32 != 0)
    return fail(WSG_ERR_INVALID_ARG, "wsg_gemm_nt_f32: need M >= 1, N %% 64 == 0, K %% 32 == 0 (M=%d N=%d K=%d)", M, N, K);
  if (accumulate != 0 && accumulate != 1) return fail(WSG_ERR_INVALID_ARG, "wsg_gemm_nt_f32: accumulate must be 0 or 1");
  if (!d_A || !d_B || !d_C) return fail(WSG_ERR_INVALID_ARG, "wsg_gemm_nt_f32: null pointer");
  if (((uintptr_t)d_A | (uintptr_t)d_B | (uintptr_t)d_C) & 15)
    return fail(WSG_ERR_INVALID_ARG, "wsg_gemm_nt_f32: pointers must be 16-byte aligned");
  (void)hipGetLastError();
  if (!gemm_nt_f32(d_A, d_B, d_C, M, N, K, accumulate == 1, static_cast<hipStream_t>(hip_stream)))
    return fail(WSG_ERR_UNSUPPORTED, "wsg_gemm_nt_f32: shape not supported");
  return check_launch("wsg_gemm_nt_f32");
}

extern "C" wsg_status wsg_gemm_swiglu_f32(int32_t M, int32_t I, int32_t K, const float* d_A, const float* d_Wgu,
                                         float* d_ACT, void* hip_stream) {
  clear_error();
  if (M < 1 || I < 32 || I % 32 != 0 || K < 32 || K % 32 != 0)
    return fail(WSG_ERR_INVALID_ARG, "wsg_gemm_swiglu_f32: need M >= 1, I %% 32 == 0, K %% 32 == 0 (M=%d I=%d K=%d)", M, I,
                K);
  if (!d_A || !d_Wgu || !d_ACT) return fail(WSG_ERR_INVALID_ARG, "wsg_gemm_swiglu_f32: null pointer");
  if (((uintptr_t)d_A | (uintptr_t)d_Wgu | (uintptr_t)d_ACT) & 15)
    return fail(WSG_ERR_INVALID_ARG, "wsg_gemm_swiglu_f32: pointers must be 16-byte aligned");
  (void)hipGetLastError();
  if (!gemm_swiglu_f32(d_A, d_Wgu, d_ACT, M, I, K, static_cast<hipStream_t>(hip_stream)))
    return fail(WSG_ERR_UNSUPPORTED, "wsg_gemm_swiglu_f32: shape not supported");
  return check_launch("wsg_gemm_swiglu_f32");
}

extern "C" wsg_status wsg_stream_read(const void* d_buf, int64_t bytes, float* d_out, void* hip_stream) {
  clear_error();
  if (!d_buf || !d_out) return fail(WSG_ERR_INVALID_ARG, "wsg_stream_read: null pointer");
  if (bytes < 16 || bytes % 16 != 0) return fail(WSG_ERR_INVALID_ARG, "wsg_stream_read: bytes must be a positive multiple of 16");
  if ((uintptr_t)d_buf & 15) return fail(WSG_ERR_INVALID_ARG, "wsg_stream_read: buffer must be 16-byte aligned");
  if (bytes / (16 * 4096) > (int64_t)0x7fffffff) return fail(WSG_ERR_UNSUPPORTED, "wsg_stream_read: buffer too large");
  stream_read_dispatch(d_buf, bytes, d_out, static_cast<hipStream_t>(hip_stream));
  return check_launch("wsg_stream_read");
}
