// Runtime of the decode engine: packed-weight and workspace layouts, model
// creation, the ordered stage plan per token (captured once into HIP graphs
// and replayed), prefill and step, and the C ABI around them.
//
// The host packs weights and precomputes the rotary table once, outside
// any timed region, and runs no layer arithmetic (Megakernels, "What runs
// in the DSL").  Per token the host launches one graph and reads back the
// 4-byte token id, the only synchronisation (Megakernels, "GPU-wide
// end-to-end generation").
#include <math.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "../../include/wsg.h"
#include "decode.hpp"
#include "prefill.hpp"
#include "status.hpp"

namespace wsg {

thread_local char g_last_error[512];

namespace {

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct Dims {
  int L, H, I, nq, nkv, D, V, cap, chunk, Q, KV, G;
  size_t es;   // storage element bytes
  bool pack;   // lossless packed copies of the decode matrices
  bool q4;     // int4 group-64 decode matrices
};

Dims dims_of(const wsg_config& c) {
  Dims d;
  d.L = c.n_layers; d.H = c.hidden; d.I = c.intermediate; d.nq = c.n_q_heads; d.nkv = c.n_kv_heads;
  d.D = c.head_dim; d.V = c.vocab; d.cap = c.max_context; d.chunk = c.prefill_chunk;
  d.Q = d.nq * d.D; d.KV = d.nkv * d.D; d.G = d.nkv > 0 ? d.nq / d.nkv : 0;
  d.es = c.dtype == WSG_F16 ? 2 : 4;
  d.pack = c.lossless_pack != 0;
  d.q4 = c.weight_format == WSG_W_Q4G64;
  return d;
}

// Bytes of one packed int4 row of width k: k/8 words, then k/64 FP16 scales.
size_t q4_row_bytes(int k) { return (size_t)k / 2 + (size_t)k / 32; }

bool dim_ok(int v, int dtype) {
  if (dtype == WSG_F32 && v == 256) return true;
  return v == 512 || v == 1024 || v == 2048 || v == 3072;
}

wsg_status validate_config(const wsg_config* c) {
  if (!c) return fail(WSG_ERR_INVALID_ARG, "config is NULL");
  if (c->dtype != WSG_F32 && c->dtype != WSG_F16) return fail(WSG_ERR_INVALID_ARG, "dtype %d", c->dtype);
  if (c->n_layers < 1 || c->vocab < 1 || c->max_context < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1)
    return fail(WSG_ERR_INVALID_ARG, "sizes must be positive");
  if (c->prefill_chunk < 0 || c->prefill_chunk > 4096) return fail(WSG_ERR_INVALID_ARG, "prefill_chunk must be in [0, 4096]");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f)) return fail(WSG_ERR_INVALID_ARG, "rms_eps and rope_theta must be > 0");
  if (c->head_dim != 128) return fail(WSG_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", c->head_dim);
  if (c->n_q_heads % c->n_kv_heads != 0) return fail(WSG_ERR_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads");
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4) return fail(WSG_ERR_UNSUPPORTED, "query group size %d not in {1,2,4}", G);
  if (!dim_ok(c->hidden, c->dtype) || !dim_ok(c->intermediate, c->dtype) ||
      !dim_ok(c->n_q_heads * c->head_dim, c->dtype))
    return fail(WSG_ERR_UNSUPPORTED, "hidden/intermediate/query width must be in {512,1024,2048,3072}%s",
                c->dtype == WSG_F32 ? " or 256" : "");
  if ((int64_t)c->max_context > (1 << 20)) return fail(WSG_ERR_UNSUPPORTED, "max_context too large");
  if (c->lossless_pack != 0 && c->lossless_pack != 1) return fail(WSG_ERR_INVALID_ARG, "lossless_pack must be 0 or 1");
  if (c->lossless_pack && c->dtype != WSG_F32)
    return fail(WSG_ERR_UNSUPPORTED, "lossless packing applies to FP32 models");
  if (c->prefill_chunk > 0 && (c->dtype != WSG_F32 || G > 2))
    return fail(WSG_ERR_UNSUPPORTED, "chunked prefill needs FP32 storage and a query group of 1 or 2");
  if (c->weight_format != WSG_W_DENSE && c->weight_format != WSG_W_Q4G64)
    return fail(WSG_ERR_INVALID_ARG, "weight_format %d", c->weight_format);
  if (c->weight_format == WSG_W_Q4G64) {
    if (c->dtype != WSG_F16) return fail(WSG_ERR_UNSUPPORTED, "int4 weights need FP16 storage");
    if (c->hidden % 1024 || c->intermediate % 1024 || (c->n_q_heads * c->head_dim) % 1024)
      return fail(WSG_ERR_UNSUPPORTED, "int4 weights need hidden, intermediate and query widths that are multiples of 1024");
    if (c->lossless_pack) return fail(WSG_ERR_UNSUPPORTED, "lossless packing applies to dense FP32 models");
  }
  return WSG_OK;
}

// ------------------------------------------------------------ layouts
struct LayerOff {
  size_t in_norm, post_norm, q_norm, k_norm, wqkv, wo, wgu, wd;
  size_t wqkv_p = 0, wo_p = 0, wgu_p = 0, wd_p = 0;   // packed copies (lossless_pack)
};
struct PackedLayout {
  size_t embed = 0, final_norm = 0, total = 0;
  size_t hdr = 0, embed_p = 0;   // lossless_pack: flag header, packed embedding
  std::vector<LayerOff> layers;
};

// Flag header of the packed copies: magic, count, then one byte per decode
// matrix (embedding, then per layer W_qkv, W_o, W_gu, W_d): 1 = packed copy
// present and verified.
constexpr uint32_t kPackMagic = 0x50475357u;
int pack_count(const Dims& d) { return 1 + 4 * d.L; }

PackedLayout packed_layout(const Dims& d) {
  PackedLayout p;
  size_t off = 0;
  auto take = [&](size_t elems) { const size_t o = off; off = align256(off + elems * d.es); return o; };
  auto take_bytes = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  // a decode matrix [rows][k]: dense elements or int4 rows
  auto take_mat = [&](size_t rows, int k) { return d.q4 ? take_bytes(rows * q4_row_bytes(k)) : take(rows * k); };
  p.embed = take_mat(d.V, d.H);
  p.final_norm = take(d.H);
  for (int l = 0; l < d.L; ++l) {
    LayerOff lo;
    lo.in_norm = take(d.H);
    lo.post_norm = take(d.H);
    lo.q_norm = take(d.D);
    lo.k_norm = take(d.D);
    lo.wqkv = take_mat(d.Q + 2 * d.KV, d.H);
    lo.wo = take_mat(d.H, d.Q);
    lo.wgu = take_mat(2 * d.I, d.H);
    lo.wd = take_mat(d.H, d.I);
    p.layers.push_back(lo);
  }
  if (d.pack) {
    p.hdr = take_bytes(8 + pack_count(d));
    p.embed_p = take_bytes((size_t)d.V * d.H * 2);
    for (LayerOff& lo : p.layers) {
      lo.wqkv_p = take_bytes((size_t)(d.Q + 2 * d.KV) * d.H * 2);
      lo.wo_p = take_bytes((size_t)d.H * d.Q * 2);
      lo.wgu_p = take_bytes((size_t)2 * d.I * d.H * 2);
      lo.wd_p = take_bytes((size_t)d.H * d.I * 2);
    }
  }
  p.total = off;
  return p;
}

// Lossless packed copy of elems FP32 values at src into dst (elems 16-bit
// halves): 1 = written and verified, 0 = not eligible (odd count, a
// non-finite value or nonzero low 16 bits), -1 = verification mismatch.
int pack_lossless(const uint8_t* src_bytes, uint8_t* dst_bytes, size_t elems) {
  if (elems % 2 != 0) return 0;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(src_bytes);
  for (size_t i = 0; i < elems; ++i)
    if ((src[i] & 0xFFFFu) != 0 || ((src[i] >> 23) & 0xFFu) == 0xFFu) return 0;
  uint16_t* dst = reinterpret_cast<uint16_t*>(dst_bytes);
  for (size_t i = 0; i < elems; ++i) dst[i] = (uint16_t)(src[i] >> 16);
  for (size_t i = 0; i < elems; ++i)
    if (((uint32_t)dst[i] << 16) != src[i]) return -1;
  return 1;
}

// Decode attention splits the keys into ranges of a fixed size per captured
// graph (so a block's key range does not depend on the position read on
// the device): at least attn_chunk(d) keys (64, or more so that the whole
// capacity needs at most 128 splits), and longer ranges for longer contexts
// (attn_chunk_for).
constexpr int kMaxAttnSplits = 128;

int attn_chunk(const Dims& d) {
  int c = (d.cap + kMaxAttnSplits - 1) / kMaxAttnSplits;
  c = (c + 15) & ~15;
  return c < 64 ? 64 : c;
}

int attn_split_cap(const Dims& d) {
  const int need = (d.cap + attn_chunk(d) - 1) / attn_chunk(d);
  int s = 1;
  while (s < need) s <<= 1;
  return s;
}

struct WsLayout {
  size_t kv = 0, rope_cos = 0, rope_sin = 0, rope_cur = 0, x = 0, x2 = 0, qkv = 0, o = 0, act = 0, logits = 0;
  size_t opart = 0, dpart = 0, attn_part = 0, am_part = 0, ctrl = 0, ids = 0, total = 0;
  PrefillLayout pf;
  int attn_splits_cap = 1;
  int opart_slots = 0;
};

WsLayout ws_layout(const Dims& d) {
  WsLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  w.kv = take((size_t)d.L * 2 * d.nkv * d.cap * d.D * d.es);
  w.rope_cos = take((size_t)d.cap * (d.D / 2) * 4);
  w.rope_sin = take((size_t)d.cap * (d.D / 2) * 4);
  // per-row buffers: kMaxTokens rows (a two-token step)
  const size_t T = kMaxTokens;
  w.rope_cur = take(T * d.D * 4);
  w.x = take(T * d.H * d.es);
  w.x2 = take(T * d.H * d.es);
  w.qkv = take(T * (d.Q + 2 * d.KV) * d.es);
  w.o = take(T * d.Q * d.es);
  w.act = take(T * d.I * d.es);
  w.logits = take(T * d.V * d.es);
  w.opart_slots = std::max(d.nkv, attn_o_part_slots(d.H, d.nkv, 1));
  w.opart = take(T * w.opart_slots * d.H * 4);
  w.dpart = take(T * kMaxDownSplit * d.H * 4);
  w.attn_splits_cap = attn_split_cap(d);
  w.attn_part = take(T * d.nkv * w.attn_splits_cap * d.G * kAttnPartStride * 4);
  w.am_part = take(T * kHeadMaxBlocks * 8);
  w.ctrl = take((size_t)kCtrlWords * 4);
  w.ids = take((size_t)(d.cap + 1) * 4);
  const size_t pf_base = off;
  w.pf = prefill_layout(d.chunk, d.H, d.I, d.Q, d.KV, d.es, pf_base);
  off = align256(pf_base + w.pf.total);
  w.total = off;
  return w;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace
}  // namespace wsg

using namespace wsg;

struct wsg_model {
  wsg_config cfg;
  Dims d;
  hipStream_t stream = nullptr;
  bool own_stream = false;
  const uint8_t* packed = nullptr;
  uint8_t* ws = nullptr;
  PackedLayout pl;
  WsLayout wl;
  DecodeArgs args;
  DecodeShape shape;    // launch shape of single-token steps
  DecodeShape shape2;   // launch shape of two-token steps
  std::vector<LayerPtrs> layers;
  int32_t pos = 0;
  bool has_output = false;
  int32_t* pin = nullptr;          // pinned staging of ids copied in: [1..]
  int32_t* mail = nullptr;         // pinned mailbox the argmax launch writes (MailWord layout)
  bool use_graph = true;
  // a captured step graph; a graph captured while a per-layer stage was timed
  // holds event-record nodes around that stage's launches (n_events events of
  // ev, bracketing launches that stream `bytes` weight bytes in all)
  struct CachedGraph { hipGraphExec_t exec; uint64_t last_use; int n_events; int64_t bytes; };
  std::map<uint64_t, CachedGraph> graphs;   // key: graph_key(splits, chunk, tokens, mode, advance)
  uint64_t graph_uses = 0;
  int timed_stage = -1;
  std::vector<hipEvent_t> ev;
  int ev_used = 0;
  int64_t timed_bytes_per_launch_sum = 0;
  int n_packed = 0;   // decode matrices with a lossless packed copy
  double acc_ms = 0;
  int64_t acc_launches = 0, acc_bytes = 0;
  int prefill_rows = 0;
  bool event_error = false;
  bool capturing = false;
  int skip_stage = -1;   // a stage kind enqueue_body leaves out (stage timing by difference)
  char event_msg[160] = {0};
};

namespace {

// Weight bytes one launch of a stage streams for layer l (the head: the
// embedding); packed copies count half.
int64_t stage_bytes(const wsg_model* m, int stage, int l) {
  const Dims& d = m->d;
  const LayerPtrs* L = l >= 0 && l < (int)m->layers.size() ? &m->layers[l] : nullptr;
  // [rows][k]: int4 rows, the packed copy, or dense elements
  auto b = [&](int64_t rows, int k, const void* packed) {
    if (d.q4) return rows * (int64_t)q4_row_bytes(k);
    return packed ? rows * k * 2 : rows * k * (int64_t)d.es;
  };
  switch (stage) {
    case WSG_STAGE_QKV: return b(d.Q + 2 * d.KV, d.H, L ? L->wqkv_p : nullptr);
    case WSG_STAGE_O: return b(d.H, d.Q, L ? L->wo_p : nullptr);
    case WSG_STAGE_GATEUP: return b(2 * d.I, d.H, L ? L->wgu_p : nullptr);
    case WSG_STAGE_DOWN: return b(d.H, d.I, L ? L->wd_p : nullptr);
    case WSG_STAGE_HEAD: return b(d.V, d.H, m->args.embed_p);
    default: return 0;
  }
}

// Events bracket launches of the timed stage kind.  While a step graph is
// captured, an event recorded on the stream becomes a node whose event has no
// usable timestamps on this platform, so the event is added as an explicit
// event-record node after the capture's current leaves instead, and the
// captured work continues from that node; such nodes time correctly on replay.
bool record_event(wsg_model* m, hipEvent_t e) {
  hipError_t r;
  const char* what = "hipEventRecord";
  if (m->capturing) {
    hipStreamCaptureStatus cs;
    unsigned long long id = 0;
    hipGraph_t g = nullptr;
    const hipGraphNode_t* deps = nullptr;
    size_t nd = 0;
    hipGraphNode_t node = nullptr;
    r = hipStreamGetCaptureInfo_v2(m->stream, &cs, &id, &g, &deps, &nd);
    what = "hipStreamGetCaptureInfo_v2";
    if (r == hipSuccess) { r = hipGraphAddEventRecordNode(&node, g, deps, nd, e); what = "hipGraphAddEventRecordNode"; }
    if (r == hipSuccess) {
      r = hipStreamUpdateCaptureDependencies(m->stream, &node, 1, hipStreamSetCaptureDependencies);
      what = "hipStreamUpdateCaptureDependencies";
    }
  } else {
    r = hipEventRecord(e, m->stream);
  }
  if (r != hipSuccess) {
    snprintf(m->event_msg, sizeof(m->event_msg), "%s: %s", what, hipGetErrorString(r));
    m->event_error = true;
    return false;
  }
  return true;
}

template <typename F>
bool timed(wsg_model* m, int stage, int64_t bytes, F&& launch) {
  if (stage == m->skip_stage) return true;
  const bool t = (m->timed_stage == stage) && (m->ev_used + 2 <= (int)m->ev.size());
  if (t) record_event(m, m->ev[m->ev_used]);
  const bool ok = launch();
  if (t) {
    record_event(m, m->ev[m->ev_used + 1]);
    m->ev_used += 2;
    m->timed_bytes_per_launch_sum += bytes;
  }
  return ok;
}

DecodeShape shape_for(const wsg_model* m, int tokens) {
  DecodeShape sh = tokens == 2 ? m->shape2 : m->shape;
  sh.tokens = tokens;
  return sh;
}

// How a layer runs attention and the output projection.
enum AttnMode : int {
  kAttnSeparate = 0,   // split-K attention, merge launch, output GEMV
  kAttnFused = 1,      // short contexts: attention fused with the KV-head-split output GEMV
  kAttnMergeO = 2,     // longer contexts: split-K attention, then the merge fused with that GEMV
};

// K slices of the down projection for a step of `tokens` rows: the launch
// shape's, where the weights are dense, the slice width holds whole lane
// vectors (256 FP32 or 512 FP16 elements) and a row group is 1 or 2 rows;
// else 1.
int down_split(const wsg_model* m, const DecodeShape& sh) {
  const int S = sh.split_down;
  if (S <= 1 || m->d.q4 || m->d.I % S || (sh.rows_down != 1 && sh.rows_down != 2)) return 1;
  const int vec = m->d.es == 2 ? 512 : 256;
  return (m->d.I / S) % vec == 0 ? S : 1;
}

// All layers of one step of `tokens` rows; the last down projection
// advances the position when no head follows (prompt rows before the
// last).  With a split down projection, every layer but the last writes K
// slices that the next layer's QKV launch sums; the last writes x itself,
// for the head.
bool enqueue_body(wsg_model* m, int splits, int chunk, int mode, bool advance, int tokens) {
  DecodeShape sh = shape_for(m, tokens);
  sh.attn_splits = splits;
  sh.attn_chunk = chunk;
  const hipStream_t s = m->stream;
  const int L = m->d.L;
  const int S = down_split(m, sh);
  for (int l = 0; l < L; ++l) {
    const LayerPtrs& lp = m->layers[l];
    const DecodeArgs& a = m->args;
    const int npd = (l > 0 && S > 1) ? S : 0;
    if (!timed(m, WSG_STAGE_QKV, stage_bytes(m, WSG_STAGE_QKV, l),
               [&] { return launch_qkv(a, sh, lp, l == 0, npd, s); }))
      return false;
    if (mode == kAttnFused) {
      if (!timed(m, WSG_STAGE_ATTN, stage_bytes(m, WSG_STAGE_O, l), [&] { return launch_attn_o(a, sh, lp, s); }))
        return false;
    } else if (mode == kAttnMergeO) {
      if (!timed(m, WSG_STAGE_ATTN, 0, [&] { return launch_attn(a, sh, lp, false, s); })) return false;
      if (!timed(m, WSG_STAGE_O, stage_bytes(m, WSG_STAGE_O, l), [&] { return launch_merge_o(a, sh, lp, s); }))
        return false;
    } else {
      if (!timed(m, WSG_STAGE_ATTN, 0, [&] {
            return launch_attn(a, sh, lp, true, s) && (splits == 1 || launch_attn_merge(a, sh, s));
          }))
        return false;
      if (!timed(m, WSG_STAGE_O, stage_bytes(m, WSG_STAGE_O, l), [&] { return launch_o(a, sh, lp, s); })) return false;
    }
    if (!timed(m, WSG_STAGE_GATEUP, stage_bytes(m, WSG_STAGE_GATEUP, l),
               [&] { return launch_gateup(a, sh, lp, mode != kAttnSeparate, s); }))
      return false;
    if (!timed(m, WSG_STAGE_DOWN, stage_bytes(m, WSG_STAGE_DOWN, l), [&] {
          return (S > 1 && l < L - 1) ? launch_down_split(a, sh, lp, S, s)
                                      : launch_down(a, sh, lp, advance && l == L - 1, s);
        }))
      return false;
  }
  return true;
}

bool enqueue_head(wsg_model* m, int tokens) { return launch_head(m->args, shape_for(m, tokens), m->stream); }
bool enqueue_argmax(wsg_model* m, int tokens) { return launch_argmax(m->args, shape_for(m, tokens), m->stream); }

// Contexts up to kFuseMaxKeys keys run attention fused with the output
// projection (each of a KV head's 32 blocks reads that head's K/V prefix;
// beyond this length the split-K path's parallelism over keys wins).
constexpr int kFuseMaxKeys = 128;

int attn_mode(const wsg_model* m, int n_keys, int tokens) {
  const DecodeShape sh = shape_for(m, tokens);
  // the KV-head-split output GEMV: enabled, its partials fit the gate/up
  // prologue, and (int4) whole 8-byte loads per lane
  const bool split_o = sh.fuse_attn_o && attn_o_part_slots(m->d.H, m->d.nkv, tokens) > 0 &&
                       !(m->d.q4 && m->d.G == 1 && sh.rows_attn_o == 4);
  if (!split_o) return kAttnSeparate;
  return n_keys <= kFuseMaxKeys ? kAttnFused : kAttnMergeO;
}

// Keys per split-K attention block for n_keys: the model's minimum, or more
// so that about kAttnTargetBlocks blocks (over all KV heads) cover the
// context, in multiples of 16 keys.  Every block has a fixed overhead (its
// query, the merge of its 16 key-rows, its partial state, and one more
// state for the merge launch to read), so fewer, longer blocks win once
// there are enough of them to keep the memory system busy; a sweep of
// fixed sizes on the 8-KV-head model at 1.1k / 2.1k / 4.2k keys was best
// at 64 / 96 / 192 keys, i.e. 20-24 splits per head.  Since the merge launch
// got cheaper, a target of one block per CU (256: 27-32 splits per head)
// measured 0.6 % faster per token than 192 at 4.1-4.4k keys; 160 was slower,
// and 320 (more blocks than CUs) 5 % slower, as were 384 or 512 before.
constexpr int kAttnTargetBlocks = 256;

// The size is taken from a ladder with four steps per doubling (64, 80, 96,
// 112, 128, 160, ...: 16 * {4,5,6,7} * 2^e), so a long generation passes
// through few (splits, chunk) graphs.
int attn_chunk_for(const wsg_model* m, int n_keys) {
  const int per_head = std::max(1, kAttnTargetBlocks / m->d.nkv);
  const int need = std::max(m->shape.attn_chunk, ceil_div(n_keys, per_head));
  int c = 64;
  for (int e = 0; c < need; ++e) {
    const int base = 64 << (e / 4);            // 64 * 2^(e/4) ...
    c = base + (base / 4) * (e % 4 + 1);       // ... times 5/4, 6/4, 7/4, 8/4
  }
  return c;
}

// Attention blocks per KV head: exactly the splits the context needs (one
// captured graph per (splits, chunk) pair).  With chunk >= attn_chunk(d)
// this is at most attn_split_cap(d).
int splits_for(int n_keys, int chunk) { return ceil_div(n_keys, chunk); }

// Graphs are destroyed only once the stream has finished any replay of them.
void drop_graphs(wsg_model* m) {
  if (m->graphs.empty()) return;
  if (m->stream) (void)hipStreamSynchronize(m->stream);
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second.exec);
  m->graphs.clear();
}

// At most kMaxGraphs captured step graphs are kept; the least recently used
// one makes room (a generation moves through a few (splits, chunk) pairs at
// a time).
constexpr size_t kMaxGraphs = 64;

// Capture (once) and return the graph for `key`, built by `enqueue`.
template <typename F>
wsg_status graph_for(wsg_model* m, uint64_t key, F&& enqueue, hipGraphExec_t* out) {
  auto it = m->graphs.find(key);
  if (it != m->graphs.end()) {
    it->second.last_use = ++m->graph_uses;
    *out = it->second.exec;
    m->ev_used = it->second.n_events;
    m->timed_bytes_per_launch_sum = it->second.bytes;
    return WSG_OK;
  }
  if (m->graphs.size() >= kMaxGraphs) {
    auto lru = m->graphs.begin();
    for (auto i = m->graphs.begin(); i != m->graphs.end(); ++i)
      if (i->second.last_use < lru->second.last_use) lru = i;
    WSG_HIP_CHECK(hipStreamSynchronize(m->stream));   // it may still be replaying
    (void)hipGraphExecDestroy(lru->second.exec);
    m->graphs.erase(lru);
  }
  WSG_HIP_CHECK(hipStreamBeginCapture(m->stream, hipStreamCaptureModeThreadLocal));
  m->capturing = true;
  m->ev_used = 0;
  m->timed_bytes_per_launch_sum = 0;
  const bool ok = enqueue();
  m->capturing = false;
  hipGraph_t g = nullptr;
  const hipError_t ec = hipStreamEndCapture(m->stream, &g);
  if (!ok) { if (g) (void)hipGraphDestroy(g); return fail(WSG_ERR_UNSUPPORTED, "no compiled kernel for this shape"); }
  if (ec != hipSuccess) return fail(WSG_ERR_HIP, "graph capture: %s", hipGetErrorString(ec));
  hipGraphExec_t ex = nullptr;
  const hipError_t ei = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (ei != hipSuccess) return fail(WSG_ERR_HIP, "graph instantiate: %s", hipGetErrorString(ei));
  if (m->event_error) {
    (void)hipGraphExecDestroy(ex);
    m->event_error = false;
    return fail(WSG_ERR_HIP, "timing event in a captured graph: %s", m->event_msg);
  }
  m->graphs.emplace(key, wsg_model::CachedGraph{ex, ++m->graph_uses, m->ev_used, m->timed_bytes_per_launch_sum});
  *out = ex;
  return WSG_OK;
}


// timed: the per-layer stage whose launches the graph brackets with event
// nodes (-1: none).
uint64_t graph_key(int splits, int chunk, int tokens, int mode, bool advance, int timed) {
  const uint64_t k = ((((uint64_t)chunk << 20 | (uint64_t)splits) * 2 + (tokens - 1)) * 3 + mode) * 2 + (advance ? 1 : 0);
  return k * 8 + (uint64_t)(timed + 1);
}

// The final norm + vocabulary head and the argmax over the residual rows in
// args.x.  They are single launches, issued directly (a graph saves nothing
// for one kernel), so stream events can bracket the head.
wsg_status run_head(wsg_model* m, int tokens) {
  const bool t = m->timed_stage == WSG_STAGE_HEAD;
  if (t) record_event(m, m->ev[0]);
  if (!enqueue_head(m, tokens)) return fail(WSG_ERR_UNSUPPORTED, "no compiled head kernel for this shape");
  if (t) {
    record_event(m, m->ev[1]);
    m->ev_used = 2;
    m->timed_bytes_per_launch_sum = stage_bytes(m, WSG_STAGE_HEAD, -1);
  }
  if (!enqueue_argmax(m, tokens)) return fail(WSG_ERR_UNSUPPORTED, "argmax launch");
  return WSG_OK;
}

// Enqueue one step of `tokens` rows at the current device position (n_keys
// = the last row's position + 1): the layer body and, if `head`, the head
// (final norm, vocabulary GEMV, argmax).
wsg_status run_forward(wsg_model* m, bool head, int n_keys, int tokens = 1) {
  const int chunk = attn_chunk_for(m, n_keys);
  const int splits = splits_for(n_keys, chunk);
  const int mode = attn_mode(m, n_keys, tokens);
  const bool advance = !head;
  (void)hipGetLastError();   // errors of earlier calls were reported by those calls
  m->ev_used = 0;
  m->timed_bytes_per_launch_sum = 0;
  if (!m->use_graph) {
    if (!enqueue_body(m, splits, chunk, mode, advance, tokens))
      return fail(WSG_ERR_UNSUPPORTED, "no compiled kernel for this shape");
  } else {
    hipGraphExec_t body = nullptr;
    const int tstage = m->timed_stage == WSG_STAGE_HEAD ? -1 : m->timed_stage;
    const wsg_status st = graph_for(m, graph_key(splits, chunk, tokens, mode, advance, tstage),
                                    [&] { return enqueue_body(m, splits, chunk, mode, advance, tokens); }, &body);
    if (st != WSG_OK) return st;
    WSG_HIP_CHECK(hipGraphLaunch(body, m->stream));
  }
  if (head) {
    const wsg_status st = run_head(m, tokens);
    if (st != WSG_OK) return st;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WSG_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return WSG_OK;
}

wsg_status collect_timing(wsg_model* m) {
  if (m->event_error) { m->event_error = false; return fail(WSG_ERR_HIP, "recording a timing event failed: %s", m->event_msg); }
  if (m->timed_stage < 0 || m->ev_used == 0) return WSG_OK;
  for (int i = 0; i + 1 < m->ev_used; i += 2) {
    float ms = 0.f;
    WSG_HIP_CHECK(hipEventElapsedTime(&ms, m->ev[i], m->ev[i + 1]));
    m->acc_ms += ms;
    m->acc_launches += 1;
  }
  m->acc_bytes += m->timed_bytes_per_launch_sum;
  m->ev_used = 0;
  return WSG_OK;
}

// The argmax launch writes its tokens straight into the pinned mailbox, so
// reading a step's token is a wait for the stream and a host load.
wsg_status read_token(wsg_model* m, int32_t* out_token) {
  WSG_HIP_CHECK(hipStreamSynchronize(m->stream));
  const wsg_status st = collect_timing(m);
  if (st != WSG_OK) return st;
  if (out_token) *out_token = reinterpret_cast<volatile int32_t*>(m->mail)[kMailOutTok];
  return WSG_OK;
}

// The per-row tokens of the last step (`rows` words from kMailRowTok).
wsg_status read_row_tokens(wsg_model* m, int rows, int32_t* out) {
  WSG_HIP_CHECK(hipStreamSynchronize(m->stream));
  const wsg_status st = collect_timing(m);
  if (st != WSG_OK) return st;
  for (int i = 0; i < rows; ++i) out[i] = reinterpret_cast<volatile int32_t*>(m->mail)[kMailRowTok + i];
  return WSG_OK;
}

// A call that fails after it enqueued work may have moved the device
// position (prefill chunks and the argmax launch advance it); put it back to
// the host's value, which the failed call leaves unchanged (best effort: after
// a HIP error the stream may refuse this launch too).  Returns st.
wsg_status restore_pos(wsg_model* m, wsg_status st) {
  if (st != WSG_OK) {
    launch_set_pos(m->args.ctrl, m->pos, m->stream);
    (void)hipGetLastError();
  }
  return st;
}

void fill_rope(const wsg_config& c, std::vector<float>& cs, std::vector<float>& sn) {
  const int half = c.head_dim / 2;
  cs.resize((size_t)c.max_context * half);
  sn.resize(cs.size());
  for (int i = 0; i < half; ++i) {
    const double inv_freq = pow((double)c.rope_theta, -2.0 * i / (double)c.head_dim);
    for (int p = 0; p < c.max_context; ++p) {
      const double a = (double)p * inv_freq;
      cs[(size_t)p * half + i] = (float)cos(a);
      sn[(size_t)p * half + i] = (float)sin(a);
    }
  }
}

}  // namespace

// ======================================================================= ABI
extern "C" {

const char* wsg_last_error(void) { return g_last_error; }
const char* wsg_version(void) { return "wsg 0.1 gfx950"; }

wsg_status wsg_packed_weight_bytes(const wsg_config* cfg, size_t* bytes) {
  clear_error();
  const wsg_status st = validate_config(cfg);
  if (st != WSG_OK) return st;
  if (!bytes) return fail(WSG_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = packed_layout(dims_of(*cfg)).total;
  return WSG_OK;
}

wsg_status wsg_workspace_bytes(const wsg_config* cfg, size_t* bytes) {
  clear_error();
  const wsg_status st = validate_config(cfg);
  if (st != WSG_OK) return st;
  if (!bytes) return fail(WSG_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ws_layout(dims_of(*cfg)).total;
  return WSG_OK;
}

wsg_status wsg_pack_weights(const wsg_config* cfg, const wsg_host_weights* w, void* host_out, size_t out_bytes) {
  clear_error();
  wsg_status st = validate_config(cfg);
  if (st != WSG_OK) return st;
  if (!w || !host_out) return fail(WSG_ERR_INVALID_ARG, "weights or output is NULL");
  if (cfg->weight_format != WSG_W_DENSE)
    return fail(WSG_ERR_INVALID_ARG, "int4 models are packed by wsg_pack_weights_q4");
  const Dims d = dims_of(*cfg);
  const PackedLayout p = packed_layout(d);
  if (out_bytes < p.total) return fail(WSG_ERR_INVALID_ARG, "output has %zu bytes, need %zu", out_bytes, p.total);
  if (!w->embed || !w->final_norm || !w->in_norm || !w->wq || !w->wk || !w->wv || !w->q_norm || !w->k_norm ||
      !w->wo || !w->post_norm || !w->wg || !w->wu || !w->wd)
    return fail(WSG_ERR_INVALID_ARG, "a weight pointer is NULL");
  for (int l = 0; l < d.L; ++l)
    if (!w->in_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->q_norm[l] || !w->k_norm[l] || !w->wo[l] ||
        !w->post_norm[l] || !w->wg[l] || !w->wu[l] || !w->wd[l])
      return fail(WSG_ERR_INVALID_ARG, "layer %d has a NULL weight pointer", l);
  uint8_t* out = static_cast<uint8_t*>(host_out);
  memset(out, 0, p.total);
  const size_t es = d.es;
  auto put = [&](size_t off, const void* src, size_t elems) { memcpy(out + off, src, elems * es); };
  put(p.embed, w->embed, (size_t)d.V * d.H);
  put(p.final_norm, w->final_norm, d.H);
  for (int l = 0; l < d.L; ++l) {
    const LayerOff& lo = p.layers[l];
    put(lo.in_norm, w->in_norm[l], d.H);
    put(lo.post_norm, w->post_norm[l], d.H);
    put(lo.q_norm, w->q_norm[l], d.D);
    put(lo.k_norm, w->k_norm[l], d.D);
    put(lo.wqkv, w->wq[l], (size_t)d.Q * d.H);
    put(lo.wqkv + (size_t)d.Q * d.H * es, w->wk[l], (size_t)d.KV * d.H);
    put(lo.wqkv + (size_t)(d.Q + d.KV) * d.H * es, w->wv[l], (size_t)d.KV * d.H);
    put(lo.wo, w->wo[l], (size_t)d.H * d.Q);
    put(lo.wgu, w->wg[l], (size_t)d.I * d.H);
    put(lo.wgu + (size_t)d.I * d.H * es, w->wu[l], (size_t)d.I * d.H);
    put(lo.wd, w->wd[l], (size_t)d.H * d.I);
  }
  if (d.pack) {
    uint32_t* hdr = reinterpret_cast<uint32_t*>(out + p.hdr);
    uint8_t* flags = out + p.hdr + 8;
    hdr[0] = kPackMagic;
    hdr[1] = (uint32_t)pack_count(d);
    int idx = 0;
    auto pack = [&](size_t src, size_t dst, size_t elems) {
      const int r = pack_lossless(out + src, out + dst, elems);
      if (r < 0) return false;
      if (r == 0) memset(out + dst, 0, elems * 2);
      flags[idx++] = (uint8_t)r;
      return true;
    };
    bool ok = pack(p.embed, p.embed_p, (size_t)d.V * d.H);
    for (int l = 0; l < d.L && ok; ++l) {
      const LayerOff& lo = p.layers[l];
      ok = pack(lo.wqkv, lo.wqkv_p, (size_t)(d.Q + 2 * d.KV) * d.H) && pack(lo.wo, lo.wo_p, (size_t)d.H * d.Q) &&
           pack(lo.wgu, lo.wgu_p, (size_t)2 * d.I * d.H) && pack(lo.wd, lo.wd_p, (size_t)d.H * d.I);
    }
    if (!ok) return fail(WSG_ERR_STATE, "lossless packed copy failed its bitwise verification");
  }
  return WSG_OK;
}

wsg_status wsg_pack_weights_q4(const wsg_config* cfg, const wsg_host_weights* norms, const wsg_host_q4_weights* q,
                               void* host_out, size_t out_bytes) {
  clear_error();
  wsg_status st = validate_config(cfg);
  if (st != WSG_OK) return st;
  if (cfg->weight_format != WSG_W_Q4G64) return fail(WSG_ERR_INVALID_ARG, "config is not an int4 model");
  if (!norms || !q || !host_out) return fail(WSG_ERR_INVALID_ARG, "weights or output is NULL");
  const Dims d = dims_of(*cfg);
  const PackedLayout p = packed_layout(d);
  if (out_bytes < p.total) return fail(WSG_ERR_INVALID_ARG, "output has %zu bytes, need %zu", out_bytes, p.total);
  if (!norms->final_norm || !norms->in_norm || !norms->post_norm || !norms->q_norm || !norms->k_norm)
    return fail(WSG_ERR_INVALID_ARG, "a norm gain pointer is NULL");
  if (!q->embed.words || !q->embed.scales || !q->wq || !q->wk || !q->wv || !q->wo || !q->wg || !q->wu || !q->wd)
    return fail(WSG_ERR_INVALID_ARG, "an int4 matrix pointer is NULL");
  for (int l = 0; l < d.L; ++l) {
    if (!norms->in_norm[l] || !norms->post_norm[l] || !norms->q_norm[l] || !norms->k_norm[l])
      return fail(WSG_ERR_INVALID_ARG, "layer %d has a NULL norm gain pointer", l);
    for (const wsg_q4_matrix* mt : {&q->wq[l], &q->wk[l], &q->wv[l], &q->wo[l], &q->wg[l], &q->wu[l], &q->wd[l]})
      if (!mt->words || !mt->scales) return fail(WSG_ERR_INVALID_ARG, "layer %d has a NULL int4 matrix pointer", l);
  }
  uint8_t* out = static_cast<uint8_t*>(host_out);
  memset(out, 0, p.total);
  auto put = [&](size_t off, const void* src, size_t elems) { memcpy(out + off, src, elems * d.es); };
  // rows [row0, row0 + rows) of a packed int4 matrix of width k from m
  auto put_q4 = [&](size_t off, size_t row0, const wsg_q4_matrix& mt, size_t rows, int k) {
    const size_t rb = q4_row_bytes(k);
    for (size_t r = 0; r < rows; ++r) {
      uint8_t* dst = out + off + (row0 + r) * rb;
      memcpy(dst, mt.words + r * (k / 8), (size_t)k / 2);
      memcpy(dst + k / 2, mt.scales + r * (k / 64), (size_t)k / 32);
    }
  };
  put_q4(p.embed, 0, q->embed, d.V, d.H);
  put(p.final_norm, norms->final_norm, d.H);
  for (int l = 0; l < d.L; ++l) {
    const LayerOff& lo = p.layers[l];
    put(lo.in_norm, norms->in_norm[l], d.H);
    put(lo.post_norm, norms->post_norm[l], d.H);
    put(lo.q_norm, norms->q_norm[l], d.D);
    put(lo.k_norm, norms->k_norm[l], d.D);
    put_q4(lo.wqkv, 0, q->wq[l], d.Q, d.H);
    put_q4(lo.wqkv, d.Q, q->wk[l], d.KV, d.H);
    put_q4(lo.wqkv, d.Q + d.KV, q->wv[l], d.KV, d.H);
    put_q4(lo.wo, 0, q->wo[l], d.H, d.Q);
    put_q4(lo.wgu, 0, q->wg[l], d.I, d.H);
    put_q4(lo.wgu, d.I, q->wu[l], d.I, d.H);
    put_q4(lo.wd, 0, q->wd[l], d.H, d.I);
  }
  return WSG_OK;
}

wsg_status wsg_model_create(const wsg_config* cfg, const void* d_packed, size_t packed_bytes, void* d_workspace,
                            size_t ws_bytes, void* hip_stream, wsg_model** out) {
  clear_error();
  wsg_status st = validate_config(cfg);
  if (st != WSG_OK) return st;
  if (!d_packed || !d_workspace || !out) return fail(WSG_ERR_INVALID_ARG, "NULL pointer");
  if (((uintptr_t)d_packed | (uintptr_t)d_workspace) & 255)
    return fail(WSG_ERR_INVALID_ARG, "packed weights and workspace must be 256-byte aligned");
  const Dims d = dims_of(*cfg);
  PackedLayout pl = packed_layout(d);
  WsLayout wl = ws_layout(d);
  if (packed_bytes < pl.total) return fail(WSG_ERR_INVALID_ARG, "packed buffer has %zu bytes, need %zu", packed_bytes, pl.total);
  if (ws_bytes < wl.total) return fail(WSG_ERR_INVALID_ARG, "workspace has %zu bytes, need %zu", ws_bytes, wl.total);

  wsg_model* m = new wsg_model();
  m->cfg = *cfg;
  m->d = d;
  m->packed = static_cast<const uint8_t*>(d_packed);
  m->ws = static_cast<uint8_t*>(d_workspace);
  m->pl = pl;
  m->wl = wl;
  m->prefill_rows = cfg->prefill_chunk;
  auto fail_free = [&](wsg_status code) { wsg_model_destroy(m); return code; };

  if (hip_stream) {
    m->stream = static_cast<hipStream_t>(hip_stream);
  } else {
    if (hipStreamCreateWithFlags(&m->stream, hipStreamNonBlocking) != hipSuccess)
      return fail_free(fail(WSG_ERR_HIP, "hipStreamCreate failed"));
    m->own_stream = true;
  }
  if (hipHostMalloc((void**)&m->pin, (size_t)(d.cap + 2) * sizeof(int32_t), hipHostMallocDefault) != hipSuccess)
    return fail_free(fail(WSG_ERR_HIP, "hipHostMalloc failed"));
  void* mail_dev = nullptr;
  if (hipHostMalloc((void**)&m->mail, (size_t)(kMailHist + d.cap + 1) * sizeof(int32_t), hipHostMallocMapped) !=
          hipSuccess ||
      hipHostGetDevicePointer(&mail_dev, m->mail, 0) != hipSuccess)
    return fail_free(fail(WSG_ERR_HIP, "hipHostMalloc / hipHostGetDevicePointer (token mailbox) failed"));
  memset(m->mail, 0, (size_t)(kMailHist + d.cap + 1) * sizeof(int32_t));
  m->ev.resize(2 * (d.L + 1));
  for (auto& e : m->ev)
    if (hipEventCreate(&e) != hipSuccess) { e = nullptr; return fail_free(fail(WSG_ERR_HIP, "hipEventCreate failed")); }

  DecodeArgs& a = m->args;
  a.dtype = cfg->dtype;
  a.wfmt = d.q4 ? kWeightsQ4 : kWeightsDense;
  a.hidden = d.H; a.inter = d.I; a.n_q = d.nq; a.n_kv = d.nkv; a.head_dim = d.D; a.vocab = d.V; a.cap = d.cap;
  a.eps = cfg->rms_eps;
  a.embed = m->packed + pl.embed;
  a.embed_p = nullptr;
  a.final_norm = m->packed + pl.final_norm;
  a.rope_cos = reinterpret_cast<const float*>(m->ws + wl.rope_cos);
  a.rope_sin = reinterpret_cast<const float*>(m->ws + wl.rope_sin);
  a.rope_cur = reinterpret_cast<float*>(m->ws + wl.rope_cur);
  a.opart = reinterpret_cast<float*>(m->ws + wl.opart);
  a.dpart = reinterpret_cast<float*>(m->ws + wl.dpart);
  a.x = m->ws + wl.x; a.x2 = m->ws + wl.x2; a.qkv = m->ws + wl.qkv; a.o = m->ws + wl.o; a.act = m->ws + wl.act;
  a.logits = m->ws + wl.logits;
  a.attn_part = reinterpret_cast<float*>(m->ws + wl.attn_part);
  a.attn_part_splits = wl.attn_splits_cap;
  a.am_part = reinterpret_cast<unsigned long long*>(m->ws + wl.am_part);
  a.ctrl = reinterpret_cast<int32_t*>(m->ws + wl.ctrl);
  a.ids = reinterpret_cast<int32_t*>(m->ws + wl.ids);
  a.mail = static_cast<int32_t*>(mail_dev);
  const size_t kv_layer = (size_t)2 * d.nkv * d.cap * d.D * d.es;
  for (int l = 0; l < d.L; ++l) {
    const LayerOff& lo = pl.layers[l];
    LayerPtrs lp;
    lp.wqkv = m->packed + lo.wqkv; lp.wo = m->packed + lo.wo; lp.wgu = m->packed + lo.wgu; lp.wd = m->packed + lo.wd;
    lp.in_norm = m->packed + lo.in_norm; lp.post_norm = m->packed + lo.post_norm;
    lp.q_norm = m->packed + lo.q_norm; lp.k_norm = m->packed + lo.k_norm;
    lp.k_cache = m->ws + wl.kv + l * kv_layer;
    lp.v_cache = m->ws + wl.kv + l * kv_layer + kv_layer / 2;
    m->layers.push_back(lp);
  }
  if (d.pack) {
    // which decode matrices have a verified packed copy (header written by
    // wsg_pack_weights)
    std::vector<uint8_t> hdr(8 + pack_count(d));
    if (hipMemcpyAsync(hdr.data(), m->packed + pl.hdr, hdr.size(), hipMemcpyDeviceToHost, m->stream) != hipSuccess ||
        hipStreamSynchronize(m->stream) != hipSuccess)
      return fail_free(fail(WSG_ERR_HIP, "reading the packed-weight header failed"));
    uint32_t magic, count;
    memcpy(&magic, hdr.data(), 4);
    memcpy(&count, hdr.data() + 4, 4);
    if (magic != kPackMagic || (int)count != pack_count(d))
      return fail_free(fail(WSG_ERR_INVALID_ARG, "packed weights lack the lossless-copy header (pack with lossless_pack = 1)"));
    const uint8_t* f = hdr.data() + 8;
    for (int i = 0; i < pack_count(d); ++i)
      if (f[i] > 1) return fail_free(fail(WSG_ERR_INVALID_ARG, "corrupt packed-weight header"));
    if (f[0]) a.embed_p = m->packed + pl.embed_p;
    for (int l = 0; l < d.L; ++l) {
      const LayerOff& lo = pl.layers[l];
      LayerPtrs& lp = m->layers[l];
      if (f[1 + 4 * l]) lp.wqkv_p = m->packed + lo.wqkv_p;
      if (f[2 + 4 * l]) lp.wo_p = m->packed + lo.wo_p;
      if (f[3 + 4 * l]) lp.wgu_p = m->packed + lo.wgu_p;
      if (f[4 + 4 * l]) lp.wd_p = m->packed + lo.wd_p;
    }
    for (int i = 0; i < pack_count(d); ++i) m->n_packed += f[i];
  }
  DecodeShape& sh = m->shape;
  sh.rows_qkv = sh.rows_o = sh.rows_gu = sh.rows_down = 1;
  sh.grid_qkv = sh.grid_o = sh.grid_gu = sh.grid_down = 0;
  int cus = 0;
  {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 0;
  }
  if (cus > 0 && !d.q4) {
    // FP32, packed and FP16 weights: QKV on 3 blocks per CU and gate/up on
    // 2, looping over their row groups, instead of one-shot grids (4 and 3
    // per CU at the 0.6B shape): fewer waves repeat the norm prologue (the
    // residual, the attention partials and the gain, read from L2 by every
    // wave), and the second row group's weights are loaded while the first
    // is reduced (28-layer sweeps, interleaved rounds: FP32 1415 against
    // 1384 tokens/s over 640..896 / 448..768 blocks, neighbouring sizes
    // slower; FP16 1918 against 1877)
    sh.grid_qkv = 3 * cus;
    sh.grid_gu = 2 * cus;
  }
  // head: two rows per wave on the one-shot grid (18992 workgroups for the
  // 151936-row vocabulary): with non-temporal weight loads the best of rows
  // 1/2/4 x 4/8 waves x grids 4096..one-shot; each wave's activation and
  // norm prologue then serves 8 KiB of weights
  sh.rows_head = 2;
  sh.grid_head = 0;
  sh.head_waves = 4;
  sh.attn_splits = 1;
  sh.attn_chunk = attn_chunk(d);
  sh.fuse_attn_o = 1;
  sh.rows_attn_o = 8;
  // Two-token steps: four vocabulary rows per wave.  Each wave reads both
  // activation rows once (from L2) for all of its rows; at one row per wave
  // those reads double the L2 traffic of the weights they serve, and the
  // argmax would reduce four times as many block keys.
  m->shape2 = sh;
  m->shape2.rows_head = 4;
  // Gate/up and QKV loop on 256 and 512 blocks: a wave that serves two
  // activation rows streams its weights long enough to cover the per-wave
  // prologue (28-layer kernel-trace sweep: 858 against 881 us per step at
  // the one-shot grids; one-token steps keep the one-shot grids)
  m->shape2.grid_gu = 256;
  m->shape2.grid_qkv = 512;
  if (d.es == 2 && !d.q4) {
    // FP16 rows are 2 KiB: the head loops its two rows per wave over 8192
    // workgroups, so each wave's activation and norm prologue serves more
    // than one row pair (kernel-trace sweep of rows 1/2/4 x 4/8 waves x
    // grids 2048..one-shot: 49 against 62 us on the one-shot grid)
    for (DecodeShape* s : {&m->shape, &m->shape2}) s->grid_head = 8192;
  }
  if (d.pack) {
    // packed rows are 2 KiB like FP16 rows: the one-token head loops its two
    // rows per wave over 4096 workgroups (28-layer sweep of 4096 / 8192 /
    // 12288 / one-shot: 1875 / 1865 / 1847 / 1816 tokens/s)
    m->shape.grid_head = 4096;
  }
  if (d.q4) {
    // int4 rows are short (544 bytes at width 1024): the head loops over
    // four rows per wave on 2048 blocks, so each wave's activation and norm
    // prologue serves many rows (the one-shot grid reads more activation
    // bytes from L2 than weight bytes from HBM)
    for (DecodeShape* s : {&m->shape, &m->shape2}) {
      s->rows_head = 4;
      s->grid_head = 2048;
      // likewise fewer, longer waves for gate/up (whose prologue sums the
      // attention partials) and QKV (kernel-trace sweep of rows and grids)
      s->rows_gu = 4;
      s->rows_qkv = 2;
    }
  }

  std::vector<float> cs, sn;
  fill_rope(*cfg, cs, sn);
  if (hipMemcpyAsync(m->ws + wl.rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, m->stream) != hipSuccess ||
      hipMemcpyAsync(m->ws + wl.rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, m->stream) != hipSuccess ||
      hipMemsetAsync(m->ws + wl.ctrl, 0, (size_t)kCtrlWords * 4, m->stream) != hipSuccess ||
      hipMemsetAsync(m->ws + wl.ids, 0, (size_t)(d.cap + 1) * 4, m->stream) != hipSuccess ||
      // partial slots past the KV head count are summed as zeros
      hipMemsetAsync(m->ws + wl.opart, 0, (size_t)kMaxTokens * wl.opart_slots * d.H * 4, m->stream) != hipSuccess ||
      hipStreamSynchronize(m->stream) != hipSuccess)
    return fail_free(fail(WSG_ERR_HIP, "uploading the rotary table failed"));
  // graphs need a capturable (non-null) stream
  m->use_graph = (m->stream != nullptr);
  *out = m;
  return WSG_OK;
}

void wsg_model_destroy(wsg_model* m) {
  if (!m) return;
  if (m->stream) (void)hipStreamSynchronize(m->stream);
  drop_graphs(m);
  for (auto e : m->ev) if (e) (void)hipEventDestroy(e);
  if (m->pin) (void)hipHostFree(m->pin);
  if (m->mail) (void)hipHostFree(m->mail);
  if (m->own_stream && m->stream) (void)hipStreamDestroy(m->stream);
  delete m;
}

wsg_status wsg_reset_cache(wsg_model* m) {
  clear_error();
  if (!m) return fail(WSG_ERR_INVALID_ARG, "model is NULL");
  (void)hipGetLastError();   // errors of earlier calls were reported by those calls
  launch_set_pos(m->args.ctrl, 0, m->stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WSG_ERR_HIP, "reset: %s", hipGetErrorString(e));
  m->pos = 0;
  m->has_output = false;
  return WSG_OK;
}

int32_t wsg_position(const wsg_model* m) { return m ? m->pos : -1; }

wsg_status wsg_rewind(wsg_model* m, int32_t pos) {
  clear_error();
  if (!m) return fail(WSG_ERR_INVALID_ARG, "model is NULL");
  if (pos < 0) return fail(WSG_ERR_INVALID_ARG, "pos=%d must be >= 0", pos);
  if (pos > m->pos) return fail(WSG_ERR_OUT_OF_RANGE, "pos=%d is past the current position %d", pos, m->pos);
  if (pos == m->pos) return WSG_OK;
  (void)hipGetLastError();
  launch_set_pos(m->args.ctrl, pos, m->stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WSG_ERR_HIP, "rewind: %s", hipGetErrorString(e));
  m->pos = pos;
  m->has_output = true;   // the token history holds the token of slot pos
  return WSG_OK;
}

wsg_status wsg_prefill(wsg_model* m, const int32_t* host_ids, int32_t n, int32_t* out_token, const void** out_logits) {
  clear_error();
  if (!m || !host_ids) return fail(WSG_ERR_INVALID_ARG, "NULL pointer");
  if (n < 1) return fail(WSG_ERR_INVALID_ARG, "n=%d must be >= 1", n);
  if ((int64_t)m->pos + n > m->d.cap)
    return fail(WSG_ERR_OUT_OF_RANGE, "position %d + %d rows exceeds max_context %d", m->pos, n, m->d.cap);
  for (int i = 0; i < n; ++i)
    if (host_ids[i] < 0 || host_ids[i] >= m->d.V)
      return fail(WSG_ERR_OUT_OF_RANGE, "token id %d at index %d outside [0, %d)", host_ids[i], i, m->d.V);
  memcpy(m->pin + 1, host_ids, (size_t)n * sizeof(int32_t));
  WSG_HIP_CHECK(hipMemcpyAsync(m->args.ids + m->pos, m->pin + 1, (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice,
                               m->stream));
  const int p0 = m->pos;
  int done = 0;
  if (m->prefill_rows > 0 && n > 1) {
    // chunked path for every row; the last row alone completes the last
    // layer and reaches the head
    PrefillCtx pc = prefill_ctx(m->args, m->shape, m->layers.data(), m->d.L, m->ws, m->wl.pf, m->prefill_rows);
    (void)hipGetLastError();   // errors of earlier calls were reported by those calls
    m->ev_used = 0;
    m->timed_bytes_per_launch_sum = 0;
    wsg_status st = run_prefill_chunks(pc, p0, n, true, m->stream);
    if (st == WSG_OK) st = run_head(m, 1);
    if (st != WSG_OK) return restore_pos(m, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return restore_pos(m, fail(WSG_ERR_HIP, "kernel launch: %s", hipGetErrorString(e)));
    done = n;
  }
  // Rows without the chunked path: two at a time through the two-row
  // body (each weight vector read once for both rows), the last row alone
  // so that it reaches the head.
  int r = done;
  for (; r + 2 <= n - 1; r += 2) {
    const wsg_status st = run_forward(m, false, p0 + r + 2, 2);
    if (st != WSG_OK) return restore_pos(m, st);
  }
  for (; r < n; ++r) {
    const bool last = (r == n - 1);
    const wsg_status st = run_forward(m, last, p0 + r + 1);
    if (st != WSG_OK) return restore_pos(m, st);
  }
  const wsg_status st = read_token(m, out_token);
  if (st != WSG_OK) return restore_pos(m, st);
  m->pos = p0 + n;
  m->has_output = true;
  if (out_logits) *out_logits = m->args.logits;
  return WSG_OK;
}

wsg_status wsg_step(wsg_model* m, int32_t in_token, int32_t* out_token, const void** out_logits) {
  clear_error();
  if (!m) return fail(WSG_ERR_INVALID_ARG, "model is NULL");
  if (in_token >= m->d.V) return fail(WSG_ERR_OUT_OF_RANGE, "token id %d >= vocab %d", in_token, m->d.V);
  if (in_token < 0 && !m->has_output) return fail(WSG_ERR_STATE, "no previous output token; pass in_token or prefill first");
  if (m->pos >= m->d.cap) return fail(WSG_ERR_OUT_OF_RANGE, "cache full (max_context %d)", m->d.cap);
  if (in_token >= 0) {
    m->pin[1] = in_token;
    WSG_HIP_CHECK(hipMemcpyAsync(m->args.ids + m->pos, m->pin + 1, sizeof(int32_t), hipMemcpyHostToDevice, m->stream));
  }
  wsg_status st = run_forward(m, true, m->pos + 1);
  if (st != WSG_OK) return restore_pos(m, st);
  st = read_token(m, out_token);
  if (st != WSG_OK) return restore_pos(m, st);
  m->pos += 1;
  m->has_output = true;
  if (out_logits) *out_logits = m->args.logits;
  return WSG_OK;
}

wsg_status wsg_generate(wsg_model* m, int32_t n, int32_t* out_tokens) {
  clear_error();
  if (!m) return fail(WSG_ERR_INVALID_ARG, "model is NULL");
  if (n < 0) return fail(WSG_ERR_INVALID_ARG, "n=%d must be >= 0", n);
  if (n == 0) return WSG_OK;
  if (!out_tokens) return fail(WSG_ERR_INVALID_ARG, "out_tokens is NULL");
  if (!m->has_output) return fail(WSG_ERR_STATE, "no previous output token; prefill first");
  if ((int64_t)m->pos + n > m->d.cap)
    return fail(WSG_ERR_OUT_OF_RANGE, "position %d + %d steps exceeds max_context %d", m->pos, n, m->d.cap);
  if (m->timed_stage >= 0)
    return fail(WSG_ERR_STATE, "stage timing brackets single steps: use wsg_step while WSG_OPT_TIMED_STAGE is set");
  // Every step reads its input token from the device history and writes
  // the next one there (and to the mailbox), so the steps are enqueued
  // back to back and the host waits once.
  for (int t = 0; t < n; ++t) {
    const wsg_status st = run_forward(m, true, m->pos + t + 1);
    if (st != WSG_OK) return restore_pos(m, st);
  }
  const wsg_status st = read_token(m, nullptr);
  if (st != WSG_OK) return restore_pos(m, st);
  const volatile int32_t* hist = m->mail + kMailHist;
  for (int t = 0; t < n; ++t) out_tokens[t] = hist[m->pos + 1 + t];
  m->pos += n;
  return WSG_OK;
}

wsg_status wsg_step2(wsg_model* m, int32_t in_token, int32_t draft, int32_t out_tokens[2], int32_t* n_emitted,
                     const void** out_logits) {
  clear_error();
  if (!m || !out_tokens || !n_emitted) return fail(WSG_ERR_INVALID_ARG, "NULL pointer");
  if (in_token >= m->d.V) return fail(WSG_ERR_OUT_OF_RANGE, "token id %d >= vocab %d", in_token, m->d.V);
  if (draft < 0 || draft >= m->d.V) return fail(WSG_ERR_OUT_OF_RANGE, "draft id %d outside [0, %d)", draft, m->d.V);
  if (in_token < 0 && !m->has_output) return fail(WSG_ERR_STATE, "no previous output token; pass in_token or prefill first");
  if ((int64_t)m->pos + 2 > m->d.cap)
    return fail(WSG_ERR_OUT_OF_RANGE, "position %d + 2 rows exceeds max_context %d", m->pos, m->d.cap);
  m->pin[1] = in_token;
  m->pin[2] = draft;
  if (in_token >= 0)
    WSG_HIP_CHECK(hipMemcpyAsync(m->args.ids + m->pos, m->pin + 1, 2 * sizeof(int32_t), hipMemcpyHostToDevice, m->stream));
  else
    WSG_HIP_CHECK(hipMemcpyAsync(m->args.ids + m->pos + 1, m->pin + 2, sizeof(int32_t), hipMemcpyHostToDevice, m->stream));
  wsg_status st = run_forward(m, true, m->pos + 2, 2);
  if (st != WSG_OK) return restore_pos(m, st);
  int32_t tok[2];
  st = read_row_tokens(m, 2, tok);
  if (st != WSG_OK) return restore_pos(m, st);
  // the argmax kernel applied the same acceptance rule to the device position
  const int emitted = tok[0] == draft ? 2 : 1;
  out_tokens[0] = tok[0];
  out_tokens[1] = tok[1];
  *n_emitted = emitted;
  m->pos += emitted;
  m->has_output = true;
  if (out_logits) *out_logits = m->args.logits;
  return WSG_OK;
}

wsg_status wsg_kv_view(const wsg_model* m, int32_t layer, const void** d_k, const void** d_v, int32_t* valid_len,
                       int64_t strides[3]) {
  clear_error();
  if (!m || !d_k || !d_v || !valid_len) return fail(WSG_ERR_INVALID_ARG, "NULL pointer");
  if (layer < 0 || layer >= m->d.L) return fail(WSG_ERR_OUT_OF_RANGE, "layer %d outside [0, %d)", layer, m->d.L);
  *d_k = m->layers[layer].k_cache;
  *d_v = m->layers[layer].v_cache;
  *valid_len = m->pos;
  if (strides) {
    strides[0] = (int64_t)m->d.cap * m->d.D;   // KV head
    strides[1] = m->d.D;                       // position
    strides[2] = 1;                            // dim
  }
  return WSG_OK;
}

wsg_status wsg_set_prefill_chunk(wsg_model* m, int32_t rows) {
  clear_error();
  if (!m) return fail(WSG_ERR_INVALID_ARG, "model is NULL");
  if (rows < 1 || rows > m->cfg.prefill_chunk)
    return fail(WSG_ERR_INVALID_ARG, "chunk rows %d outside [1, %d]", rows, m->cfg.prefill_chunk);
  m->prefill_rows = rows;
  return WSG_OK;
}

wsg_status wsg_set_option(wsg_model* m, int32_t option, int32_t value) {
  clear_error();
  if (!m) return fail(WSG_ERR_INVALID_ARG, "model is NULL");
  switch (option) {
    case WSG_OPT_USE_GRAPH:
      if (value != 0 && value != 1) return fail(WSG_ERR_INVALID_ARG, "use_graph must be 0 or 1");
      if (value == 1 && m->stream == nullptr) return fail(WSG_ERR_STATE, "graphs need a non-null stream");
      m->use_graph = value == 1;
      return WSG_OK;
    case WSG_OPT_TIMED_STAGE:
      if (value < -1 || value > WSG_STAGE_HEAD) return fail(WSG_ERR_INVALID_ARG, "stage %d", value);
      m->timed_stage = value;
      m->acc_ms = 0; m->acc_launches = 0; m->acc_bytes = 0;
      return WSG_OK;
    default:
      break;
  }
  // launch-shape options: of single-token steps, or with
  // WSG_OPT_FOR_TWO_TOKEN of two-token steps
  DecodeShape& sh = (option & WSG_OPT_FOR_TWO_TOKEN) ? m->shape2 : m->shape;
  const int opt = option & ~WSG_OPT_FOR_TWO_TOKEN;
  int* target = nullptr;
  switch (opt) {
    case WSG_OPT_FUSE_ATTN_O:
      if (value != 0 && value != 1) return fail(WSG_ERR_INVALID_ARG, "fuse_attn_o must be 0 or 1");
      target = &sh.fuse_attn_o;
      break;
    case WSG_OPT_ROWS_ATTN_O:
      if (value != 4 && value != 8) return fail(WSG_ERR_INVALID_ARG, "attention/output rows per wave must be 4 or 8");
      target = &sh.rows_attn_o;
      break;
    case WSG_OPT_HEAD_WAVES:
      if (value != 4 && value != 8 && value != 16) return fail(WSG_ERR_INVALID_ARG, "head waves must be 4, 8 or 16");
      target = &sh.head_waves;
      break;
    case WSG_OPT_SPLIT_DOWN:
      if (value != 1 && value != 2 && value != 4) return fail(WSG_ERR_INVALID_ARG, "down K slices must be 1, 2 or 4");
      target = &sh.split_down;
      break;
    default:
      if (opt >= WSG_OPT_ROWS_QKV && opt <= WSG_OPT_ROWS_HEAD) {
        if (value != 1 && value != 2 && value != 4) return fail(WSG_ERR_INVALID_ARG, "rows per wave must be 1, 2 or 4");
        int* rows[] = {&sh.rows_qkv, &sh.rows_o, &sh.rows_gu, &sh.rows_down, &sh.rows_head};
        target = rows[opt - WSG_OPT_ROWS_QKV];
      } else if (opt >= WSG_OPT_GRID_QKV && opt <= WSG_OPT_GRID_HEAD) {
        if (value < 0 || value > (1 << 20)) return fail(WSG_ERR_INVALID_ARG, "grid must be in [0, 2^20]");
        int* grids[] = {&sh.grid_qkv, &sh.grid_o, &sh.grid_gu, &sh.grid_down, &sh.grid_head};
        target = grids[opt - WSG_OPT_GRID_QKV];
      }
      break;
  }
  if (!target) return fail(WSG_ERR_INVALID_ARG, "unknown option %d", option);
  *target = value;
  drop_graphs(m);
  return WSG_OK;
}

wsg_status wsg_weight_storage(const wsg_model* m, int32_t* packed_matrices, int32_t* decode_matrices,
                              int64_t* decode_weight_bytes) {
  clear_error();
  if (!m || !packed_matrices || !decode_matrices || !decode_weight_bytes)
    return fail(WSG_ERR_INVALID_ARG, "NULL pointer");
  *packed_matrices = m->n_packed;
  *decode_matrices = pack_count(m->d);
  int64_t b = stage_bytes(m, WSG_STAGE_HEAD, -1);
  for (int l = 0; l < m->d.L; ++l)
    b += stage_bytes(m, WSG_STAGE_QKV, l) + stage_bytes(m, WSG_STAGE_O, l) + stage_bytes(m, WSG_STAGE_GATEUP, l) +
         stage_bytes(m, WSG_STAGE_DOWN, l);
  *decode_weight_bytes = b;
  return WSG_OK;
}

wsg_status wsg_time_stage(wsg_model* m, int32_t stage, int32_t reps, double* us_per_launch, int64_t* bytes_per_launch) {
  clear_error();
  if (!m || !us_per_launch || !bytes_per_launch) return fail(WSG_ERR_INVALID_ARG, "NULL pointer");
  if (stage < WSG_STAGE_QKV || stage > WSG_STAGE_DOWN)
    return fail(WSG_ERR_INVALID_ARG, "stage %d is not a per-layer stage", stage);
  if (reps < 1 || reps > 10000) return fail(WSG_ERR_INVALID_ARG, "reps=%d outside [1, 10000]", reps);
  if (!m->has_output || m->pos >= m->d.cap)
    return fail(WSG_ERR_STATE, "time a stage between steps: after a prefill, with a free cache slot");
  if (m->stream == nullptr) return fail(WSG_ERR_STATE, "stage timing needs a non-null stream");
  // the layer body the next one-token step would run, at its context
  const int n_keys = m->pos + 1;
  const int chunk = attn_chunk_for(m, n_keys);
  const int splits = splits_for(n_keys, chunk);
  const int mode = attn_mode(m, n_keys, 1);
  if (stage == WSG_STAGE_O && mode == kAttnFused)
    return fail(WSG_ERR_UNSUPPORTED, "the output projection runs inside the attention launch at this context");
  const hipStream_t s = m->stream;
  const int saved_timed = m->timed_stage;
  m->timed_stage = -1;
  hipGraphExec_t ex[2] = {nullptr, nullptr};
  wsg_status st = WSG_OK;
  (void)hipGetLastError();
  for (int k = 0; k < 2 && st == WSG_OK; ++k) {   // 0: every stage, 1: all but `stage`
    m->skip_stage = k == 0 ? -1 : stage;
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) { st = fail(WSG_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e)); break; }
    m->capturing = true;
    const bool ok = enqueue_body(m, splits, chunk, mode, false, 1);
    m->capturing = false;
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(s, &g);
    if (!ok) st = fail(WSG_ERR_UNSUPPORTED, "no compiled kernel for this shape");
    else if (e != hipSuccess) st = fail(WSG_ERR_HIP, "graph capture: %s", hipGetErrorString(e));
    else if ((e = hipGraphInstantiate(&ex[k], g, nullptr, nullptr, 0)) != hipSuccess)
      st = fail(WSG_ERR_HIP, "graph instantiate: %s", hipGetErrorString(e));
    if (g) (void)hipGraphDestroy(g);
  }
  m->skip_stage = -1;
  m->timed_stage = saved_timed;
  m->ev_used = 0;
  // alternate the two graphs, each replay between its own pair of events;
  // the median over the repetitions of (with - without) resists a stray
  // slow replay
  std::vector<double> diff;
  hipError_t e = hipSuccess;
  if (st == WSG_OK) {
    e = hipGraphLaunch(ex[0], s);   // warm-up
    if (e == hipSuccess) e = hipGraphLaunch(ex[1], s);
    for (int r = 0; r < reps && e == hipSuccess; ++r) {
      double t[2] = {0.0, 0.0};
      for (int k = 0; k < 2 && e == hipSuccess; ++k) {
        e = hipEventRecord(m->ev[0], s);
        if (e == hipSuccess) e = hipGraphLaunch(ex[k], s);
        if (e == hipSuccess) e = hipEventRecord(m->ev[1], s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, m->ev[0], m->ev[1]);
        t[k] = ms;
      }
      diff.push_back(t[0] - t[1]);
    }
    if (e != hipSuccess) st = fail(WSG_ERR_HIP, "stage timing: %s", hipGetErrorString(e));
  }
  for (auto x : ex)
    if (x) (void)hipGraphExecDestroy(x);
  if (st != WSG_OK) return st;
  const int L = m->d.L;
  std::sort(diff.begin(), diff.end());
  const size_t n = diff.size();
  const double med = n % 2 ? diff[n / 2] : 0.5 * (diff[n / 2 - 1] + diff[n / 2]);
  *us_per_launch = med * 1e3 / L;
  int64_t bytes = 0;
  for (int l = 0; l < L; ++l) {
    if (stage == WSG_STAGE_ATTN)   // the cached keys and values it reads (+ W_o when fused)
      bytes += (int64_t)2 * m->d.nkv * n_keys * m->d.D * (int64_t)m->d.es +
               (mode == kAttnFused ? stage_bytes(m, WSG_STAGE_O, l) : 0);
    else
      bytes += stage_bytes(m, stage, l);
  }
  *bytes_per_launch = bytes / L;
  return WSG_OK;
}

wsg_status wsg_describe(const wsg_model* m, char* buf, size_t n, size_t* needed) {
  clear_error();
  if (!m || !needed) return fail(WSG_ERR_INVALID_ARG, "NULL pointer");
  std::string j = "{";
  char t[256];
  auto shape_json = [&](const char* name, const DecodeShape& sh) {
    snprintf(t, sizeof(t),
             "\"%s\": {\"rows_per_wave\": {\"qkv\": %d, \"o\": %d, \"gateup\": %d, \"down\": %d, \"head\": %d}, ",
             name, sh.rows_qkv, sh.rows_o, sh.rows_gu, sh.rows_down, sh.rows_head);
    j += t;
    snprintf(t, sizeof(t),
             "\"grid_blocks\": {\"qkv\": %d, \"o\": %d, \"gateup\": %d, \"down\": %d, \"head\": %d}, ",
             sh.grid_qkv, sh.grid_o, sh.grid_gu, sh.grid_down, head_blocks(m->args, sh));
    j += t;
    snprintf(t, sizeof(t), "\"head_waves\": %d, \"fuse_attn_o\": %d, \"rows_attn_o\": %d, \"down_k_slices\": %d}, ",
             sh.head_waves, sh.fuse_attn_o, sh.rows_attn_o, down_split(m, sh));
    j += t;
  };
  shape_json("one_token", shape_for(m, 1));
  shape_json("two_token", shape_for(m, 2));
  snprintf(t, sizeof(t), "\"attention\": {\"fused_max_keys\": %d, \"target_blocks\": %d, \"min_split_keys\": %d, ",
           kFuseMaxKeys, kAttnTargetBlocks, attn_chunk(m->d));
  j += t;
  j += "\"at_keys\": [";
  const int probes[] = {1, 48, 129, 1100, 2100, 4200, 4700, 5119};
  bool first = true;
  for (int k : probes) {
    if (k > m->d.cap) continue;
    const int c = attn_chunk_for(m, k);
    snprintf(t, sizeof(t), "%s{\"keys\": %d, \"mode\": \"%s\", \"splits\": %d, \"keys_per_split\": %d}",
             first ? "" : ", ", k, attn_mode(m, k, 1) == kAttnFused ? "fused" : (attn_mode(m, k, 1) == kAttnMergeO ? "split+merge_o" : "separate"),
             splits_for(k, c), c);
    j += t;
    first = false;
  }
  j += "]}, ";
  snprintf(t, sizeof(t), "\"prefill_chunk\": %d, \"graphs\": %s, \"weights_packed\": %d, \"version\": \"%s\"}",
           m->prefill_rows, m->use_graph ? "true" : "false", m->n_packed, wsg_version());
  j += t;
  *needed = j.size() + 1;
  if (buf && n > 0) {
    const size_t c = std::min(n - 1, j.size());
    memcpy(buf, j.data(), c);
    buf[c] = 0;
  }
  return WSG_OK;
}

wsg_status wsg_stage_time(wsg_model* m, double* total_ms, int64_t* launches, int64_t* bytes) {
  clear_error();
  if (!m || !total_ms || !launches || !bytes) return fail(WSG_ERR_INVALID_ARG, "NULL pointer");
  *total_ms = m->acc_ms; *launches = m->acc_launches; *bytes = m->acc_bytes;
  m->acc_ms = 0; m->acc_launches = 0; m->acc_bytes = 0;
  return WSG_OK;
}

}  // extern "C"
