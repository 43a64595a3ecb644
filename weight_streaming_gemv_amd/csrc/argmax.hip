// Greedy selection over stand-alone logit vectors (Megakernels, "GPU-wide
// end-to-end generation": the next token is chosen on the GPU by two
// argmax kernels, ties going to the lowest token id).  The keys are the
// ones the decode head writes (argmax_key in common.hpp), so this path and
// the decode step order equal logits the same way.
//
//   k_span_keys   block (b, r): the largest key of logits [b*4096, (b+1)*4096)
//                 of row r (16 coalesced loads per thread, all issued first)
//   k_keys_token  one block per row: the largest of the row's span keys,
//                 decoded to its index
#include "../../include/wsg.h"
#include "argmax.hpp"
#include "common.hpp"
#include "status.hpp"

namespace wsg {

namespace {

constexpr int kSpanThreads = 256;
constexpr int kSpanPerThread = kArgmaxSpan / kSpanThreads;

template <typename TS>
__global__ __launch_bounds__(kSpanThreads) void k_span_keys(const TS* __restrict__ logits, int n, int nb,
                                                            unsigned long long* __restrict__ keys) {
  __shared__ unsigned long long s_best[kSpanThreads / kWave];
  const int b = blockIdx.x, r = blockIdx.y;
  const TS* row = logits + (size_t)r * n;
  const int base = b * kArgmaxSpan + (int)threadIdx.x;
  // Indices past the row are clamped to its last element: a repeated key
  // cannot change a maximum, so no branch separates the loads.
  int idx[kSpanPerThread];
  TS v[kSpanPerThread];
#pragma unroll
  for (int u = 0; u < kSpanPerThread; ++u) {
    idx[u] = min(base + u * kSpanThreads, n - 1);
    v[u] = row[idx[u]];
  }
  unsigned long long best = 0;
#pragma unroll
  for (int u = 0; u < kSpanPerThread; ++u) {
    const unsigned long long k = argmax_key(Store<TS>::to_f(v[u]), idx[u]);
    best = k > best ? k : best;
  }
  best = wave_max_u64(best);
  if (lane_id() == 0) s_best[wave_id()] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = s_best[0];
#pragma unroll
    for (int w = 1; w < kSpanThreads / kWave; ++w) m = s_best[w] > m ? s_best[w] : m;
    keys[(size_t)r * nb + b] = m;
  }
}

__global__ __launch_bounds__(kSpanThreads) void k_keys_token(const unsigned long long* __restrict__ keys, int nb,
                                                             int32_t* __restrict__ out) {
  __shared__ unsigned long long s_best[kSpanThreads / kWave];
  const int r = blockIdx.x;
  unsigned long long best = 0;
  for (int i = threadIdx.x; i < nb; i += kSpanThreads) {
    const unsigned long long k = keys[(size_t)r * nb + i];
    best = k > best ? k : best;
  }
  best = wave_max_u64(best);
  if (lane_id() == 0) s_best[wave_id()] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = s_best[0];
#pragma unroll
    for (int w = 1; w < kSpanThreads / kWave; ++w) m = s_best[w] > m ? s_best[w] : m;
    out[r] = argmax_key_index(m);
  }
}

}  // namespace

void argmax_rows(int dtype, int rows, int n, const void* logits, int32_t* out, unsigned long long* keys,
                 hipStream_t s) {
  const int nb = (int)argmax_keys(1, n);
  if (dtype == WSG_F16)
    hipLaunchKernelGGL(k_span_keys<__half>, dim3(nb, rows), dim3(kSpanThreads), 0, s,
                       static_cast<const __half*>(logits), n, nb, keys);
  else
    hipLaunchKernelGGL(k_span_keys<float>, dim3(nb, rows), dim3(kSpanThreads), 0, s,
                       static_cast<const float*>(logits), n, nb, keys);
  hipLaunchKernelGGL(k_keys_token, dim3(rows), dim3(kSpanThreads), 0, s, keys, nb, out);
}

// Argument checks shared by the argmax entry points.
wsg_status argmax_check(const char* fn, int32_t dtype, int32_t rows, int32_t n, const void* d_logits,
                        const int32_t* d_out) {
  if (dtype != WSG_F32 && dtype != WSG_F16) return fail(WSG_ERR_INVALID_ARG, "%s: bad dtype %d", fn, dtype);
  if (rows < 1 || rows > 65535) return fail(WSG_ERR_INVALID_ARG, "%s: rows=%d outside [1, 65535]", fn, rows);
  if (n < 1 || n > kArgmaxMaxN) return fail(WSG_ERR_INVALID_ARG, "%s: n=%d outside [1, 2^30]", fn, n);
  if (!d_logits || !d_out) return fail(WSG_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (((uintptr_t)d_logits & (dtype == WSG_F16 ? 1 : 3)) || ((uintptr_t)d_out & 3))
    return fail(WSG_ERR_INVALID_ARG, "%s: logits and out must be aligned to their element size", fn);
  return WSG_OK;
}

}  // namespace wsg

using namespace wsg;

extern "C" wsg_status wsg_argmax_workspace_bytes(int32_t rows, int32_t n, size_t* bytes) {
  clear_error();
  if (rows < 1 || rows > 65535 || n < 1 || n > kArgmaxMaxN || !bytes)
    return fail(WSG_ERR_INVALID_ARG, "wsg_argmax_workspace_bytes: need 1 <= rows <= 65535, 1 <= n <= 2^30, bytes not NULL");
  *bytes = argmax_keys(rows, n) * sizeof(unsigned long long);
  return WSG_OK;
}

extern "C" wsg_status wsg_argmax(int32_t dtype, int32_t rows, int32_t n, const void* d_logits, int32_t* d_out,
                                 void* d_workspace, size_t ws_bytes, void* hip_stream) {
  clear_error();
  const wsg_status st = argmax_check("wsg_argmax", dtype, rows, n, d_logits, d_out);
  if (st != WSG_OK) return st;
  const size_t need = argmax_keys(rows, n) * sizeof(unsigned long long);
  if (!d_workspace) return fail(WSG_ERR_INVALID_ARG, "wsg_argmax: workspace is NULL");
  if ((uintptr_t)d_workspace & 7) return fail(WSG_ERR_INVALID_ARG, "wsg_argmax: workspace must be 8-byte aligned");
  if (ws_bytes < need) return fail(WSG_ERR_INVALID_ARG, "wsg_argmax: workspace has %zu bytes, need %zu", ws_bytes, need);
  (void)hipGetLastError();
  argmax_rows(dtype, rows, n, d_logits, d_out, static_cast<unsigned long long*>(d_workspace),
              static_cast<hipStream_t>(hip_stream));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WSG_ERR_HIP, "wsg_argmax: kernel launch failed: %s", hipGetErrorString(e));
  return WSG_OK;
}
