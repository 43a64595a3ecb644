// Chunked prefill: several consecutive prompt rows of one request per
// chunk, batched projections, causal attention over the whole prefix
// (Megakernels, "Chunked prefill for long prompts").
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/wsg.h"
#include "decode.hpp"

namespace wsg {

// Byte offsets (inside the workspace) of the chunk scratch for C rows.
struct PrefillLayout {
  int rows = 0;
  size_t x = 0, a = 0, qkv = 0, o = 0, act = 0, part = 0, total = 0;
};

PrefillLayout prefill_layout(int rows, int H, int I, int Q, int KV, size_t es, size_t base);

struct PrefillCtx {
  DecodeArgs args;
  DecodeShape shape;
  const LayerPtrs* layers;
  int n_layers;
  uint8_t* ws;
  PrefillLayout pf;
  int chunk;
};

PrefillCtx prefill_ctx(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs* layers, int n_layers,
                       uint8_t* ws, const PrefillLayout& pf, int chunk);

// Run rows [p0, p0 + n) through every layer in chunks of c.chunk rows (K/V
// written to the cache; the last layer stops after its K/V write).  With
// to_head the last row alone also completes the last layer and its final
// residual goes to the decode residual buffer c.args.x, and the device
// position is set to p0 + n - 1 for the head and argmax that follow;
// otherwise it is set to p0 + n.  Asynchronous on s.
wsg_status run_prefill_chunks(const PrefillCtx& c, int p0, int n, bool to_head, hipStream_t s);

// C[M x N] (+)= A[M x K] . B[N x K]^T on FP32 MFMA (N % 64 == 0, K % 32 == 0).
bool gemm_nt_f32(const float* A, const float* B, float* C, int M, int N, int K, bool accumulate, hipStream_t s);
// ACT[M x I] = silu(A . Wg^T) * (A . Wu^T), Wgu = [Wg; Wu] packed [2I x K].
bool gemm_swiglu_f32(const float* A, const float* Wgu, float* ACT, int M, int I, int K, hipStream_t s);

}  // namespace wsg
