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
  size_t x = 0, a = 0, qkv = 0, o = 0, act = 0, gu = 0, total = 0;
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

// Run rows [p0, p0 + n) through every layer (K/V written to the cache; no
// head).  Asynchronous on s.  Advances the device position by n.
wsg_status run_prefill_chunks(const PrefillCtx& c, int p0, int n, hipStream_t s);

}  // namespace wsg
