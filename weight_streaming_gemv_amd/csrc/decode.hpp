// Launch interface of the decode-step kernels (one token through one layer,
// and the vocabulary head).  Arguments are validated by the runtime.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wsg {

// Control words in the workspace (int32 each).
enum CtrlWord : int {
  kCtrlPos = 0,          // current position p (tokens already in the cache)
  kCtrlOutTok = 1,       // last greedy token
  kCtrlWords = 64
};

// The head kernel runs at most kHeadMaxBlocks blocks (one argmax key each;
// one row per wave for the 151936-row vocabulary is 37984 blocks); a
// multiple of 2048 (the argmax block reads key pairs).
constexpr int kHeadMaxBlocks = 40960;

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

struct DecodeArgs {
  int dtype;            // 0 FP32, 1 FP16 storage
  int hidden, inter, n_q, n_kv, head_dim, vocab, cap;
  float eps;
  const void* embed;    // [V][H]
  const void* embed_p;  // packed copy of embed for the head, or nullptr
  const void* final_norm;
  const float* rope_cos;  // [cap][D/2]
  const float* rope_sin;
  float* rope_cur;      // [D]: cos then sin of the current position (written by layer 0's qkv)
  void* x;              // residual [H]: layer input / down-projection output
  void* x2;             // residual [H]: output-projection output / MLP input
  void* qkv;            // [Q + 2 KV]
  void* o;              // [Q]
  void* act;            // [I]
  void* logits;         // [V]
  float* opart;         // [slots][H] FP32 output-projection partials of the fused attention launch
  float* attn_part;     // split-K partial states
  int attn_part_splits; // capacity in splits per KV head
  unsigned long long* am_part;  // [kHeadMaxBlocks] per-block argmax keys of the head
  int32_t* ctrl;
  int32_t* ids;         // token history [cap + 1]
};

// Grid shapes chosen by the runtime.
struct DecodeShape {
  int rows_qkv, rows_o, rows_gu, rows_down, rows_head;   // rows per wave
  int grid_qkv, grid_o, grid_gu, grid_down, grid_head;   // blocks (0 = one row group per wave)
  int attn_splits;                                       // split-K blocks per KV head (grid.x)
  int attn_chunk;                                        // keys per split (a multiple of 16, >= 64)
  int head_waves;                                        // waves per head block (4, 8 or 16)
  int fuse_attn_o;                                       // short contexts: fused attention + output GEMV
  int rows_attn_o;                                       // W_o rows per wave in the fused launch (4 or 8)
};

// Stage launches; each returns false if the shape is not compiled in.
bool launch_qkv(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool first_layer, hipStream_t s);
bool launch_attn(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, hipStream_t s);
// Combines the split-K partial states (needed when sh.attn_splits > 1).
bool launch_attn_merge(const DecodeArgs& a, const DecodeShape& sh, hipStream_t s);
bool launch_o(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, hipStream_t s);
// Short contexts: attention fused with the output GEMV, which writes
// per-KV-head partials into opart instead of x2.
bool launch_attn_o(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, hipStream_t s);
// Partial slots (>= n_kv; slots past n_kv must hold zeros) the gate/up
// prologue sums after a fused launch, or 0 if the shape cannot be fused.
int attn_o_part_slots(int hidden, int n_kv);
// from_parts: x2 is the sum of the opart partials (written back to x2).
bool launch_gateup(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool from_parts, hipStream_t s);
bool launch_down(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool advance_pos, hipStream_t s);
// Final RMSNorm + vocabulary GEMV with one argmax key per block; then the
// one-block argmax (ties to the lowest id) writes the token into ctrl and
// the token history and advances the position.
bool launch_head(const DecodeArgs& a, const DecodeShape& sh, hipStream_t s);
bool launch_argmax(const DecodeArgs& a, const DecodeShape& sh, hipStream_t s);
bool launch_set_pos(int32_t* ctrl, int pos, hipStream_t s);

// Blocks the head launch uses for a given shape (for sizing am_part).
int head_blocks(const DecodeArgs& a, const DecodeShape& sh);

}  // namespace wsg
