// Chunked prefill (batched projections on MFMA, causal prefix attention).
#include "prefill.hpp"
#include "status.hpp"

namespace wsg {

namespace {
size_t al(size_t v) { return (v + 255) & ~size_t(255); }
}  // namespace

PrefillLayout prefill_layout(int rows, int H, int I, int Q, int KV, size_t es, size_t base) {
  PrefillLayout p;
  p.rows = rows;
  if (rows <= 0) return p;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = base + off; off = al(off + bytes); return o; };
  p.x = take((size_t)rows * H * es);
  p.a = take((size_t)rows * H * es);
  p.qkv = take((size_t)rows * (Q + 2 * KV) * es);
  p.o = take((size_t)rows * Q * es);
  p.act = take((size_t)rows * I * es);
  p.gu = take((size_t)rows * 2 * I * es);
  p.total = off;
  return p;
}

PrefillCtx prefill_ctx(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs* layers, int n_layers,
                       uint8_t* ws, const PrefillLayout& pf, int chunk) {
  PrefillCtx c;
  c.args = a; c.shape = sh; c.layers = layers; c.n_layers = n_layers; c.ws = ws; c.pf = pf; c.chunk = chunk;
  return c;
}

wsg_status run_prefill_chunks(const PrefillCtx&, int, int, hipStream_t) {
  return fail(WSG_ERR_UNSUPPORTED, "chunked prefill is not built yet; create the model with prefill_chunk = 0");
}

}  // namespace wsg
