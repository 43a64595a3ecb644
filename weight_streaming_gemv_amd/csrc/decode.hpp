// Launch interface of the decode-step kernels (one token through one layer,
// and the vocabulary head).  Arguments are validated by the runtime.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wsg {

// Control words in the workspace (int32 each).
enum CtrlWord : int {
  kCtrlPos = 0,          // current position p (tokens already in the cache)
  kCtrlOutTok = 1,       // last emitted greedy token
  kCtrlRowTok = 2,       // [kMaxTokens] greedy token of each row of the last step
  kCtrlWords = 64
};

// Words of the pinned host mailbox the argmax launch writes besides the
// control words, so that the host reads a step's tokens straight from host
// memory once the stream has synchronised (no device-to-host copy launch).
enum MailWord : int {
  kMailOutTok = 0,       // last emitted greedy token
  kMailRowTok = 1,       // [kMaxTokens] greedy token of each row of the last step
  kMailHist = 4,         // [cap + 1] host copy of every history entry the argmax writes
};

// The head kernel runs at most kHeadMaxBlocks blocks (one argmax key each;
// one row per wave for the 151936-row vocabulary would be 37984 blocks, the
// default two rows per wave 18992); a multiple of 2048 (the argmax block
// reads key pairs).
constexpr int kHeadMaxBlocks = 40960;

// Floats per split-K attention partial state (per row, KV head, split and
// query head of the group): max, sum, two pad words, 128 accumulators.
constexpr int kAttnPartStride = 132;

// Query rows one decode step can carry: 1 (a decode step) or 2 (a
// two-token step: the last token and a draft of the next).  Per-row
// activation buffers below hold kMaxTokens rows.
constexpr int kMaxTokens = 2;

// Largest number of K slices of the split down projection.
constexpr int kMaxDownSplit = 4;

// The per-row buffers rope_cur [kMaxTokens][128] FP32, x and x2
// [kMaxTokens][hidden] and qkv follow each other in the workspace, each
// starting on a 256-byte boundary; the fused attention launch finds x and
// qkv from rope_cur with these offsets (the runtime checks its layout
// against them before that launch).
__host__ __device__ constexpr size_t row_buffer_bytes(size_t bytes) { return (bytes + 255) & ~size_t(255); }
__host__ __device__ constexpr size_t row_block_x_offset() { return row_buffer_bytes(kMaxTokens * 128 * 4); }
__host__ __device__ constexpr size_t row_block_qkv_offset(int hidden, int elem_bytes) {
  return row_block_x_offset() + 2 * row_buffer_bytes((size_t)kMaxTokens * hidden * elem_bytes);
}

struct LayerPtrs {
  const void* wqkv;     // [(Q + 2 KV)][H]
  const void* wo;       // [H][Q]
  const void* wgu;      // [2 I][H]  gate rows then up rows
  const void* wd;       // [H][I]
  const void* in_norm;  // [H]
  const void* post_norm;
  const void* q_norm;   // [D]
  const void* k_norm;
  void* k_cache;        // [n_kv][cap][D]
  void* v_cache;
  // Lossless packed copies (two exact FP32 values with zero low halves per
  // 32-bit word) read by the decode kernels; nullptr = read the FP32 matrix.
  const void* wqkv_p = nullptr;
  const void* wo_p = nullptr;
  const void* wgu_p = nullptr;
  const void* wd_p = nullptr;
};

// Weight formats of the decode matrices.
constexpr int kWeightsDense = 0;   // the storage dtype (plus lossless packed copies)
constexpr int kWeightsQ4 = 1;      // int4 group-64 rows (FP16 models): words then FP16 scales per row

struct DecodeArgs {
  int dtype;            // 0 FP32, 1 FP16 storage
  int wfmt = kWeightsDense;   // weight format of every decode matrix and the embedding
  int hidden, inter, n_q, n_kv, head_dim, vocab, cap;
  float eps;
  const void* embed;    // [V][H]
  const void* embed_p;  // packed copy of embed for the head, or nullptr
  const void* final_norm;
  const float* rope_cos;  // [cap][D/2]
  const float* rope_sin;
  // Per-row buffers hold kMaxTokens rows; row t of a step is at position p + t.
  float* rope_cur;      // [rows][D]: cos then sin of each row's position (written by layer 0's qkv)
  void* x;              // residual [rows][H]: layer input / down-projection output
  void* x2;             // residual [rows][H]: output-projection output / MLP input
  void* qkv;            // [rows][Q + 2 KV]
  void* o;              // [rows][Q]
  void* act;            // [rows][I]
  void* logits;         // [rows][V]
  float* opart;         // [rows][slots][H] FP32 output-projection partials of the fused attention launch
  float* dpart;         // [rows][kMaxDownSplit][H] FP32 split-K slices of the down projection
  float* attn_part;     // [rows][n_kv][splits][G] split-K partial states
  int attn_part_splits; // capacity in splits per KV head
  unsigned long long* am_part;  // per-block argmax keys of the head: row t's at [t * head blocks]
                                //   (capacity kMaxTokens * kHeadMaxBlocks)
  int32_t* ctrl;
  int32_t* ids;         // token history [cap + 1]
  int32_t* mail;        // pinned host mailbox (device-visible address): MailWord layout
};

// Grid shapes chosen by the runtime.
struct DecodeShape {
  int rows_qkv, rows_o, rows_gu, rows_down, rows_head;   // rows per wave
  int grid_qkv, grid_o, grid_gu, grid_down, grid_head;   // blocks (0 = one row group per wave)
  int attn_splits;                                       // split-K blocks per KV head (grid.x)
  int attn_chunk;                                        // keys per split (a multiple of 16, >= 64)
  int head_waves;                                        // waves per head block (4, 8 or 16)
  int fuse_attn_o;                                       // short contexts: fused attention + output GEMV;
                                                         // longer ones: merge fused with the output GEMV
  int rows_attn_o;                                       // W_o rows per wave in the fused launch (4 or 8)
  int split_down = 1;                                    // K slices of the down projection of every layer
                                                         // but the last (1: one launch writes x)
  int tokens = 1;                                        // query rows of the step (1 or kMaxTokens)
};

// Stage launches; each returns false if the shape is not compiled in.
// npd > 0: the residual is the sum of the previous layer's npd split-K down
// slices in a.dpart (written back to a.x by the launch); 0: read a.x.
bool launch_qkv(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool first_layer, int npd,
                hipStream_t s);
// The down projection split over K into S (2 or 4) FP32 slices in a.dpart
// (the first carrying the residual a.x2), for the next layer's QKV launch.
bool launch_down_split(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, int S, hipStream_t s);
// direct: a context within one split writes o itself (else every split
// writes its partial state).
bool launch_attn(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool direct, hipStream_t s);
// Combines the split-K partial states (needed when sh.attn_splits > 1).
bool launch_attn_merge(const DecodeArgs& a, const DecodeShape& sh, hipStream_t s);
bool launch_o(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, hipStream_t s);
// Short contexts: attention fused with the output GEMV, which writes
// per-KV-head partials into opart instead of x2.
bool launch_attn_o(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, hipStream_t s);
// Longer contexts: the split-K merge fused with the output GEMV split by KV
// head, writing opart like launch_attn_o (after launch_attn with direct =
// false); same shapes as launch_attn_o.
bool launch_merge_o(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, hipStream_t s);
// Partial slots per row (>= n_kv; slots past n_kv must hold zeros) the
// gate/up prologue sums after a fused launch of `tokens` rows, or 0 if the
// shape cannot be fused.  The slot count is the same for every row count
// that can be fused.
int attn_o_part_slots(int hidden, int n_kv, int tokens);
// from_parts: x2 is the sum of the opart partials (written back to x2).
bool launch_gateup(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool from_parts, hipStream_t s);
bool launch_down(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool advance_pos, hipStream_t s);
// Final RMSNorm + vocabulary GEMV with one argmax key per block and row;
// then the one-block argmax (ties to the lowest id) writes each row's token
// into ctrl, the emitted tokens into the token history, and advances the
// position (a two-token step: by one or two, as its draft is rejected or
// accepted).
bool launch_head(const DecodeArgs& a, const DecodeShape& sh, hipStream_t s);
bool launch_argmax(const DecodeArgs& a, const DecodeShape& sh, hipStream_t s);
bool launch_set_pos(int32_t* ctrl, int pos, hipStream_t s);

// Blocks the head launch uses for a given shape (for sizing am_part).
int head_blocks(const DecodeArgs& a, const DecodeShape& sh);

}  // namespace wsg
