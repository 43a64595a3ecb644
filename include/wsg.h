/*
 * wsg.h -- C ABI of the MI355X (gfx950) weight-streaming decode library.
 *
 * The library runs the batch-one token-to-logits decode step of a
 * Qwen3-0.6B-shaped decoder (Megakernels, "What runs in the DSL" and
 * "GPU-wide end-to-end generation") and the weight-streaming GEMV family it
 * is built from (Our Kernel Benchmark Was Measuring the System Cache,
 * "Summary" and "Why it mattered").
 *
 * Conventions for every entry point:
 *   - plain C types only; pointers named d_* are HIP device pointers, all
 *     other pointers are host pointers;
 *   - every call validates its arguments before it enqueues any GPU work;
 *     on an error nothing is enqueued, model state is unchanged, the call
 *     returns a negative wsg_status and wsg_last_error() describes it;
 *   - device memory is owned by the caller (the library borrows it); the
 *     library owns only the opaque wsg_model host object, its HIP graphs
 *     (one per attention split shape a step has needed, at most 64 kept),
 *     events and a small pinned host staging buffer;
 *   - "hip_stream" is a hipStream_t passed as void*; NULL selects a stream
 *     the library creates for the model (required for graph replay when the
 *     caller has no non-default stream).
 */
#ifndef WSG_H
#define WSG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WSG_OK = 0,
  WSG_ERR_INVALID_ARG = -1,   /* null pointer, bad size, bad enum value   */
  WSG_ERR_OUT_OF_RANGE = -2,  /* token id or position outside its range   */
  WSG_ERR_STATE = -3,         /* call not valid in the model's state      */
  WSG_ERR_HIP = -4,           /* a HIP runtime call failed                */
  WSG_ERR_UNSUPPORTED = -5    /* valid, but a shape no compiled kernel takes */
} wsg_status;

/* Storage dtype of weights, KV cache, logits and stage outputs.  Reductions
 * always accumulate in FP32 (Megakernels, "What runs in the DSL"). */
typedef enum { WSG_F32 = 0, WSG_F16 = 1 } wsg_dtype;

/* Format of the decode matrices (W_qkv, W_o, W_gu, W_d and the tied
 * embedding/vocabulary matrix).  WSG_W_DENSE: the storage dtype.
 * WSG_W_Q4G64: symmetric int4 weights in groups of 64 along K with one FP16
 * scale per group ("Our Kernel Benchmark Was Measuring the System Cache",
 * "Summary": 4-bit decode matrix-vector products), weight = q * s; needs
 * dtype WSG_F16 (activations, KV cache and logits in FP16, FP32
 * accumulation), hidden, intermediate and n_q_heads*head_dim multiples of
 * 1024, prefill_chunk 0 and lossless_pack 0.  The embedding gather
 * dequantises its row and rounds it to FP16; the head multiplies by the
 * exact q * s. */
typedef enum { WSG_W_DENSE = 0, WSG_W_Q4G64 = 1 } wsg_weight_format;

/* Decoder geometry and run limits.
 *   head_dim must be 128; hidden, intermediate and n_q_heads*head_dim must
 *   each be one of 512, 1024, 2048, 3072 (256 is also accepted for FP32);
 *   n_q_heads must be a multiple of n_kv_heads with a group size of 1, 2
 *   or 4.  max_context is the KV capacity in
 *   positions.  prefill_chunk is the largest number of prompt rows one
 *   prefill chunk may hold (0 = prompt rows through the decode forward).  */
typedef struct {
  int32_t n_layers, hidden, intermediate, n_q_heads, n_kv_heads, head_dim, vocab;
  int32_t max_context;
  int32_t prefill_chunk;
  float rms_eps;      /* RMSNorm epsilon, inside the square root */
  float rope_theta;   /* RoPE base; pair i turns by p * theta^(-2i/head_dim) */
  int32_t dtype;      /* wsg_dtype */
  int32_t lossless_pack;  /* 1: lossless packed copies of the decode weights (FP32 only, see below) */
  int32_t weight_format;  /* wsg_weight_format */
} wsg_config;

/* Host-side unpacked weights, element type = cfg.dtype (float32, or IEEE
 * binary16 bit patterns).  All matrices are row-major [out][in].  The
 * per-layer members point to arrays of n_layers pointers.
 *   embed [vocab][hidden] (also the tied vocabulary head), final_norm [hidden];
 *   per layer: in_norm [hidden], wq [n_q*hd][hidden], wk [n_kv*hd][hidden],
 *   wv [n_kv*hd][hidden], q_norm [hd], k_norm [hd], wo [hidden][n_q*hd],
 *   post_norm [hidden], wg [intermediate][hidden], wu [intermediate][hidden],
 *   wd [hidden][intermediate].                                            */
typedef struct {
  const void* embed;
  const void* final_norm;
  const void* const* in_norm;
  const void* const* wq;
  const void* const* wk;
  const void* const* wv;
  const void* const* q_norm;
  const void* const* k_norm;
  const void* const* wo;
  const void* const* post_norm;
  const void* const* wg;
  const void* const* wu;
  const void* const* wd;
} wsg_host_weights;

/* Host-side int4 matrix [rows][K]: words [rows][K/8] (nibble j of word w
 * holds k = 8w + j, low nibble first, two's complement in [-8, 7]) and
 * scales [rows][K/64] (IEEE binary16 bit patterns), both row-major. */
typedef struct {
  const uint32_t* words;
  const uint16_t* scales;
} wsg_q4_matrix;

/* Host-side int4 decode matrices of a WSG_W_Q4G64 model: the embedding
 * [vocab][hidden] (also the tied head) and per layer (arrays of n_layers):
 * wq [n_q*hd][hidden], wk and wv [n_kv*hd][hidden], wo [hidden][n_q*hd],
 * wg and wu [intermediate][hidden], wd [hidden][intermediate]. */
typedef struct {
  wsg_q4_matrix embed;
  const wsg_q4_matrix* wq;
  const wsg_q4_matrix* wk;
  const wsg_q4_matrix* wv;
  const wsg_q4_matrix* wo;
  const wsg_q4_matrix* wg;
  const wsg_q4_matrix* wu;
  const wsg_q4_matrix* wd;
} wsg_host_q4_weights;

/* Lossless decode-weight storage (Megakernels, "Lossless decode-weight
 * storage"): with cfg.lossless_pack = 1 (FP32 models), wsg_pack_weights also
 * writes a packed copy of each decode matrix (the embedding, read by the
 * vocabulary head, and per layer W_qkv, W_o, W_gu, W_d) whose values are
 * all finite with zero low 16 bits and whose element count is even: two
 * values per 32-bit word (element 2i in the low half, its high 16 bits
 * stored).  Each copy is verified bitwise by reconstruction; a mismatch
 * fails the call (WSG_ERR_STATE).  Matrices that do not qualify keep FP32
 * storage only.  The decode kernels read the packed copies and rebuild each
 * FP32 value exactly before the same FP32 products, in the same order, so
 * results are bit-identical to the unpacked model; prefill, activations,
 * cache and accumulation stay FP32, and the FP32 matrices stay in the image
 * (the packed copies are an addition). */
typedef struct wsg_model wsg_model;   /* opaque; one model per stream and host thread */

/* Size in bytes of the packed weight image for cfg (host and device copies
 * have the same layout).  Packing happens once on the host, outside any
 * timed region (Megakernels, "What runs in the DSL": the host packs the
 * weights and precomputes rotary constants but runs no layer arithmetic). */
wsg_status wsg_packed_weight_bytes(const wsg_config* cfg, size_t* bytes);

/* Copy the host weights into the packed layout at host_out (out_bytes must
 * be at least wsg_packed_weight_bytes).  Fuses Wq/Wk/Wv into one
 * [(n_q+2 n_kv) hd][hidden] matrix and Wg/Wu into one [2 I][hidden] matrix;
 * values are copied bit for bit.  Dense models only (WSG_W_Q4G64 configs
 * are packed by wsg_pack_weights_q4: WSG_ERR_INVALID_ARG here). */
wsg_status wsg_pack_weights(const wsg_config* cfg, const wsg_host_weights* w,
                            void* host_out, size_t out_bytes);

/* Packed image of a WSG_W_Q4G64 model: the norm gains (FP16) come from
 * `norms` (its embedding and matrix pointers are ignored and may be NULL),
 * the decode matrices from `q`.  Each packed matrix row holds the row's
 * K/8 words followed by its K/64 scales (row i of W_qkv is row i of
 * [wq; wk; wv], of W_gu row i of [wg; wu]); values are copied bit for bit.
 * Errors: a NULL pointer, out_bytes too small (WSG_ERR_INVALID_ARG), a
 * config that is not WSG_W_Q4G64 (WSG_ERR_INVALID_ARG). */
wsg_status wsg_pack_weights_q4(const wsg_config* cfg, const wsg_host_weights* norms,
                               const wsg_host_q4_weights* q, void* host_out, size_t out_bytes);

/* Size in bytes of the device workspace for cfg: KV cache
 * [n_layers][2][n_kv][max_context][head_dim], rotary table, stage buffers,
 * prefill chunk scratch, token history and control words.  (Library
 * plumbing: no passage of the pages defines it.)  Errors: an invalid config,
 * a NULL bytes (WSG_ERR_INVALID_ARG / WSG_ERR_UNSUPPORTED). */
wsg_status wsg_workspace_bytes(const wsg_config* cfg, size_t* bytes);

/* Create a model over caller-owned device buffers: d_packed (a device copy
 * of the packed image) and d_workspace (at least wsg_workspace_bytes,
 * 256-byte aligned).  Both must stay allocated until wsg_model_destroy.
 * Builds and uploads the rotary table (synchronously, on hip_stream; the
 * host precomputes the rotary constants, Megakernels, "What runs in the
 * DSL") and clears the control words.  The cache starts empty (position 0).
 * The model object itself is library plumbing (no defining passage).
 * Errors: an invalid config, NULL or misaligned buffers, buffers smaller
 * than required (WSG_ERR_INVALID_ARG), a HIP failure (WSG_ERR_HIP; nothing
 * is left allocated). */
wsg_status wsg_model_create(const wsg_config* cfg, const void* d_packed, size_t packed_bytes,
                            void* d_workspace, size_t ws_bytes, void* hip_stream, wsg_model** out);

/* Wait for the model stream, then release the library-owned host objects
 * (graphs, events, pinned staging, an own stream); the caller's device
 * buffers are untouched.  NULL is ignored.  (Library plumbing: no defining
 * passage.) */
void wsg_model_destroy(wsg_model* m);

/* Empty the KV cache: valid length 0.  Stale slots are never read, since
 * attention only reads positions 0..p (Megakernels, "Matrix-tiled
 * attention": logical extents exclude future cache slots).  Enqueues a
 * small device update on the model stream. */
wsg_status wsg_reset_cache(wsg_model* m);

/* Run prompt tokens host_ids[0..n) at positions pos..pos+n-1 and return the
 * greedy token of the last row in *out_token (lowest id among maximal
 * logits).  Only the last row reaches the final norm and vocabulary head
 * (Benchmark methodology, "Long-document chunked prefill").  Rows go through
 * the chunked path when cfg.prefill_chunk > 0 (chunk size set by
 * wsg_set_prefill_chunk), else through the decode forward, two rows per
 * forward before the last (the two-row forward of wsg_step2, without its
 * head) and the last row alone.  *out_logits (if
 * out_logits is not NULL) receives a device pointer to the last row's
 * logits [vocab] in the storage dtype, valid until the next call.  Blocks
 * until the token id is on the host.  Errors: n < 1, any id outside
 * [0, vocab), pos + n > max_context. */
wsg_status wsg_prefill(wsg_model* m, const int32_t* host_ids, int32_t n,
                       int32_t* out_token, const void** out_logits);

/* One decode step at position pos: consumes in_token (or, if in_token < 0,
 * the previous greedy output, which never leaves the device), appends its
 * K/V to the cache and returns the next greedy token.  The 4-byte token id
 * is the only data that reaches the host (Megakernels, "GPU-wide end-to-end
 * generation"): the argmax launch stores it in pinned host memory and the
 * call waits for the model stream.  Errors: in_token >= vocab; in_token < 0
 * with no previous output (WSG_ERR_STATE); pos == max_context. */
wsg_status wsg_step(wsg_model* m, int32_t in_token, int32_t* out_token, const void** out_logits);

/* n greedy decode steps in a row, each consuming the previous one's token
 * (the first: the last greedy output), with one wait at the end: the token
 * is chosen on the GPU and the device keeps the token history, so no step
 * waits for the host (Megakernels, "GPU-wide end-to-end generation": the
 * loop needs no host round trip per token).  Writes the n tokens to
 * out_tokens[0..n) (host memory) and leaves the position at pos + n; the
 * result equals n calls of wsg_step(m, -1, ...).  There is no stop token:
 * callers that stop early (an end-of-sequence id) use wsg_step, or rewind
 * past the tokens they drop.  n = 0 does nothing.  Errors: n < 0 or a NULL
 * out_tokens with n > 0 (WSG_ERR_INVALID_ARG); no previous output
 * (WSG_ERR_STATE); pos + n > max_context (WSG_ERR_OUT_OF_RANGE); stage
 * timing enabled (WSG_OPT_TIMED_STAGE >= 0, WSG_ERR_STATE: it brackets
 * single steps).  A failure part-way leaves the position at pos. */
wsg_status wsg_generate(wsg_model* m, int32_t n, int32_t* out_tokens);

/* Two-token step: the verify pass of greedy speculative decoding, in which
 * each weight matrix is streamed once for two input vectors ("Our Kernel
 * Benchmark Was Measuring the System Cache", "Why it mattered, concretely":
 * the two-token matvec variant serving the speculative pass).  Row 0
 * consumes in_token (or, if in_token < 0, the previous greedy output) at
 * position pos; row 1 consumes `draft`, a guess of row 0's greedy token, at
 * pos + 1.  Both rows' K/V are appended in the one pass, and each row's
 * greedy token is returned: out_tokens[0] follows row 0, out_tokens[1]
 * follows row 1.  The draft is accepted when it equals out_tokens[0]; then
 * both tokens are emitted (*n_emitted = 2, position pos + 2), else only
 * out_tokens[0] is (*n_emitted = 1, position pos + 1; slot pos + 1 still
 * holds the rejected draft's K/V until the next call rewrites it, and
 * out_tokens[1] is meaningless).  The same rule is applied on the device,
 * so a following wsg_step or wsg_step2 with in_token < 0 continues from the
 * last emitted token.  Every emitted token equals what the same number of
 * wsg_step calls would produce, up to floating-point rounding.
 * *out_logits (if not NULL) receives a device pointer to both rows' logits,
 * [2][vocab] in the storage dtype, valid until the next call.  Blocks until
 * the two token ids (8 bytes, stored by the argmax launch in pinned host
 * memory) are on the host.  Errors: a NULL out_tokens or
 * n_emitted (WSG_ERR_INVALID_ARG); in_token >= vocab or draft outside
 * [0, vocab) (WSG_ERR_OUT_OF_RANGE); in_token < 0 with no previous output
 * (WSG_ERR_STATE); pos + 2 > max_context (WSG_ERR_OUT_OF_RANGE). */
wsg_status wsg_step2(wsg_model* m, int32_t in_token, int32_t draft, int32_t out_tokens[2], int32_t* n_emitted,
                     const void** out_logits);

/* Current position (number of valid KV entries; Benchmark methodology,
 * "Long-document chunked prefill": a 4096-token prompt and 1024 outputs
 * leave 5119).  -1 for a NULL model. */
int32_t wsg_position(const wsg_model* m);

/* Truncate the sequence to its first pos tokens (0 <= pos <= position):
 * cache slots from pos on become invalid (they are rewritten before they are
 * read again).  The token history is kept, so wsg_step(m, -1, ...) then
 * re-processes the token recorded at slot pos; pass in_token to process
 * another one.  Used to repeat one forward at a fixed cache slot
 * (Megakernels, "Fixed-context methodology": each trial repeats one token at
 * a fixed slot) and to drop rejected tokens.  Asynchronous on the model
 * stream.  Errors: pos < 0 (WSG_ERR_INVALID_ARG), pos > position
 * (WSG_ERR_OUT_OF_RANGE). */
wsg_status wsg_rewind(wsg_model* m, int32_t pos);

/* Device pointers to layer `layer`'s K and V cache blocks, each laid out
 * [n_kv][max_context][head_dim] in the storage dtype, the valid length, and
 * (if strides is not NULL) the element strides of those three axes.  For
 * validation (Benchmark methodology, "Long-document chunked prefill": every
 * valid KV entry is checked); the memory belongs to the workspace.  Errors:
 * NULL arguments (WSG_ERR_INVALID_ARG), a layer outside [0, n_layers)
 * (WSG_ERR_OUT_OF_RANGE). */
wsg_status wsg_kv_view(const wsg_model* m, int32_t layer, const void** d_k, const void** d_v,
                       int32_t* valid_len, int64_t strides[3]);

/* Rows per prefill chunk for later wsg_prefill calls: 1 <= rows <=
 * cfg.prefill_chunk (Benchmark methodology, "Long-document chunked
 * prefill": candidate chunk sizes are a run-time choice). */
wsg_status wsg_set_prefill_chunk(wsg_model* m, int32_t rows);

/* Options: WSG_OPT_USE_GRAPH (1 = replay captured HIP graphs, the default;
 * 0 = launch every kernel directly), WSG_OPT_TIMED_STAGE (record HIP events
 * on the model stream around every launch of one stage kind, see
 * wsg_stage_time; -1 = off).  The head is a direct launch after the layer
 * graph, bracketed by stream events.  A per-layer stage in graph mode is
 * timed by step graphs captured with explicit event-record nodes around that
 * stage's launches (kept apart from the untimed graphs); each such node
 * lengthens the step by several microseconds on this platform, but the time
 * between the two nodes of a pair is the launch's own.  In direct-launch mode
 * each bracketing event adds its own overhead to short kernels. */
enum { WSG_OPT_USE_GRAPH = 1, WSG_OPT_TIMED_STAGE = 2 };
/* WSG_OPT_FUSE_ATTN_O: 1 (default) = for contexts of up to 128 keys, each
 * layer runs attention and the output projection as one launch
 * (the projection split by KV head into FP32 partials that the gate/up
 * launch sums in a fixed order); that launch is timed as WSG_STAGE_ATTN and
 * counts the output-projection weight bytes.  0 = separate attention and
 * output-projection launches at every context length.
 * WSG_OPT_ROWS_ATTN_O: output-projection rows per wave in the fused launch
 * (4 or 8, default 8). */
enum { WSG_OPT_FUSE_ATTN_O = 3, WSG_OPT_ROWS_ATTN_O = 15 };
/* WSG_OPT_HEAD_WAVES: waves per workgroup of the head launch (4, 8 or 16,
 * default 4); each workgroup writes one argmax key, so larger workgroups
 * leave fewer keys for the final argmax launch. */
enum { WSG_OPT_HEAD_WAVES = 16 };
/* WSG_OPT_SPLIT_DOWN: K slices of the down projection (1, 2 or 4).  With 2
 * or 4, every layer but the last writes that many FP32 slices of
 * W_d . act (the first plus the residual), which the next layer's QKV
 * launch adds up in slice order before its norm (more, shorter waves for
 * the 1024-row projection); it applies to dense weights whose slice width
 * holds whole lane vectors (256 FP32 / 512 FP16 elements) with 1 or 2 rows
 * per wave, else the projection runs whole. */
enum { WSG_OPT_SPLIT_DOWN = 17 };
/* Launch shape of the decode GEMV stages (tuning): rows per wave (1, 2 or
 * 4) and blocks of 256 threads (0 = one row group per wave; fewer blocks
 * loop over row groups; the head is capped at 40960 blocks).  Defaults:
 * 1 row per wave, one-shot grids. */
enum { WSG_OPT_ROWS_QKV = 10, WSG_OPT_ROWS_O = 11, WSG_OPT_ROWS_GATEUP = 12, WSG_OPT_ROWS_DOWN = 13,
       WSG_OPT_ROWS_HEAD = 14, WSG_OPT_GRID_QKV = 20, WSG_OPT_GRID_O = 21, WSG_OPT_GRID_GATEUP = 22,
       WSG_OPT_GRID_DOWN = 23, WSG_OPT_GRID_HEAD = 24 };
/* OR WSG_OPT_FOR_TWO_TOKEN into any of the launch-shape options above
 * (WSG_OPT_FUSE_ATTN_O, WSG_OPT_ROWS_ATTN_O, WSG_OPT_HEAD_WAVES, WSG_OPT_SPLIT_DOWN,
 * WSG_OPT_ROWS_*, WSG_OPT_GRID_*) to set it for two-token steps (wsg_step2) instead of
 * single-token ones: the two kinds of step keep separate launch shapes.
 * Two-token defaults: as above, except 4 head rows per wave. */
enum { WSG_OPT_FOR_TWO_TOKEN = 0x100 };
/* Stage kinds for WSG_OPT_TIMED_STAGE.  HEAD = final RMSNorm + vocabulary
 * GEMV + greedy argmax (one launch). */
enum { WSG_STAGE_QKV = 0, WSG_STAGE_ATTN = 1, WSG_STAGE_O = 2, WSG_STAGE_GATEUP = 3,
       WSG_STAGE_DOWN = 4, WSG_STAGE_HEAD = 5 };
wsg_status wsg_set_option(wsg_model* m, int32_t option, int32_t value);

/* Accumulated device time (HIP events, on the model stream) of the timed
 * stage since the option was set or last read, the number of launches it
 * covers, and the algorithmic weight bytes those launches streamed.  Resets
 * the accumulators. */
wsg_status wsg_stage_time(wsg_model* m, double* total_ms, int64_t* launches, int64_t* bytes);

/* Device time one launch of a per-layer decode stage (WSG_STAGE_QKV, _ATTN,
 * _O, _GATEUP or _DOWN) adds to a step, at the model's shapes and the context
 * of its next one-token step: the layer body of that step (all stages of all
 * layers, as one HIP graph) and the same body without the stage's launches
 * are replayed alternately `reps` times each, every replay between two events
 * on the model stream, and the median over the repetitions of (replay with
 * the stage - replay without it) is divided by n_layers.  An event pair
 * around a single launch would add its own dispatch cost to kernels of a few
 * microseconds; whole replays spread it.  For a stage of a few microseconds
 * in a model of few layers the result is noisy (it can come out negative at
 * small reps).
 * *bytes_per_launch receives the algorithmic bytes of one launch: its
 * weights, and for the attention stage the keys and values of the context
 * (plus the output-projection weights when it is fused with attention).  For
 * the roofline of a stage (Megakernels, "GPU-wide end-to-end generation": the
 * stages of a forward are ordered launches).  What the replays leave in the
 * stage buffers and in the next cache slot is rewritten by the next step
 * before it is read; the valid cache prefix, the position and the last
 * logits are untouched.  Blocks until done.  Errors: WSG_ERR_INVALID_ARG
 * (stage, reps outside [1, 10000], NULL), WSG_ERR_STATE (no prefill yet or a
 * full cache), WSG_ERR_UNSUPPORTED (WSG_STAGE_O at a context where it runs
 * inside the attention launch). */
wsg_status wsg_time_stage(wsg_model* m, int32_t stage, int32_t reps, double* us_per_launch, int64_t* bytes_per_launch);

/* Stand-alone GEMV, Y[t][m] = sum_k W[m][k] X[t][k] for t < T, with FP32
 * accumulation (Megakernels, "GPU-wide end-to-end generation": one wave
 * per group of output rows; Our Kernel Benchmark Was Measuring the System
 * Cache, "Why it mattered": rows per wave and the two-token variant).
 *   w_dtype WSG_F32: d_W float [M][K], d_X float [T][K];
 *   w_dtype WSG_F16: d_W half [M][K],  d_X half [T][K];
 *   d_Y float [T][M].  1 <= T <= 2; rows_per_wave in {1,2,4,8}, 0 = default
 *   (one row per wave; FP32 rows of K = 3072: one row per two waves, as
 *   WSG_GEMV_SPLIT2 below).
 *   M >= 1, K >= 1, any sizes; d_W and d_X 16-byte aligned.
 * Asynchronous on hip_stream. */
wsg_status wsg_gemv(int32_t w_dtype, int32_t M, int32_t K, int32_t T, int32_t rows_per_wave,
                    const void* d_W, const void* d_X, float* d_Y, void* hip_stream);

/* wsg_gemv with an explicit launch shape: grid_blocks of 256 threads
 * (0 = one row group per wave, no grid-stride loop) and flags, OR-ed:
 *   WSG_GEMV_NONTEMPORAL: weight loads bypass cache allocation;
 *   WSG_GEMV_SPLIT2: each output row is computed by two waves of a
 *     workgroup, each streaming one half of the row, and their two FP32
 *     sums are added once (half 0 first); for long rows, whose single wave
 *     cannot keep a whole row's loads in registers.  FP32 weights,
 *     rows_per_wave 1 (or 0), K of 1024, 2048 or 3072; grid_blocks counts
 *     workgroups of two rows (0 = one per row pair).
 * Other flag bits, or WSG_GEMV_SPLIT2 outside those shapes, return
 * WSG_ERR_INVALID_ARG. */
enum { WSG_GEMV_NONTEMPORAL = 1, WSG_GEMV_SPLIT2 = 2 };
wsg_status wsg_gemv_ex(int32_t w_dtype, int32_t M, int32_t K, int32_t T, int32_t rows_per_wave,
                       int32_t grid_blocks, int32_t flags,
                       const void* d_W, const void* d_X, float* d_Y, void* hip_stream);

/* 4-bit GEMV: symmetric int4 weights in groups of 64 along K with one FP16
 * scale per group (the 4-bit matrix-vector kernel of Our Kernel Benchmark
 * Was Measuring the System Cache, "Summary").
 *   d_Wq uint32 [M][K/8]: nibble j of word w is element 8w+j, two's complement;
 *   d_scales half [M][K/64]; d_X half [T][K]; d_Y float [T][M].
 *   K % 64 == 0, 1 <= T <= 2, rows_per_wave in {1,2,4,8} (0 = default).  */
wsg_status wsg_gemv_q4g64(int32_t M, int32_t K, int32_t T, int32_t rows_per_wave,
                          const uint32_t* d_Wq, const void* d_scales, const void* d_X,
                          float* d_Y, void* hip_stream);
/* wsg_gemv_q4g64 with an explicit launch shape (grid_blocks as for
 * wsg_gemv_ex; flags: WSG_GEMV_NONTEMPORAL only).  A block is 4 waves, except at K = 14336, where the
 * activations staged per block are 28 KiB per row of X and a block is
 * 16 / rows_per_wave waves, at least 4 (one staged copy serves up to four
 * times the rows). */
wsg_status wsg_gemv_q4g64_ex(int32_t M, int32_t K, int32_t T, int32_t rows_per_wave,
                             int32_t grid_blocks, int32_t flags,
                             const uint32_t* d_Wq, const void* d_scales, const void* d_X,
                             float* d_Y, void* hip_stream);

/* FP32 GEMM on the matrix cores: C[M][N] = A[M][K] . B[N][K]^T, or C += that
 * product when accumulate = 1.  Row-major, K-contiguous operands: the batched
 * projection of chunked prefill, with B a packed weight matrix [out][in]
 * (Megakernels, "Chunked prefill for long prompts": projections as ordinary
 * tiled matrix multiplication on the matrix units, FP32 accumulation).
 * M >= 1 (any), N % 64 == 0, K % 32 == 0; all pointers 16-byte aligned.
 * M <= 32 with K in {256, 512, 1024, 2048, 3072} runs the small-M kernel
 * (16-column tiles, K split over the waves of a block); other shapes the
 * tiled one.  Asynchronous on hip_stream. */
wsg_status wsg_gemm_nt_f32(int32_t M, int32_t N, int32_t K, const float* d_A, const float* d_B, float* d_C,
                           int32_t accumulate, void* hip_stream);

/* The gate/up projection of chunked prefill with its SwiGLU:
 * ACT[M][I] = silu(A . Wg^T) * (A . Wu^T), silu(g) = g / (1 + exp(-g)), for
 * d_Wgu = [Wg; Wu], a packed [2I][K] weight (I gate rows, then I up rows),
 * row-major like wsg_gemm_nt_f32's B (Megakernels, "Chunked prefill for long
 * prompts": the MLP's gate and up products as one tiled matrix product; the
 * model's SwiGLU block for the activation).  The activation is applied in the
 * product's epilogue, so the 2I-wide product is never stored.  M >= 1,
 * I % 32 == 0, K % 32 == 0; A is [M][K], ACT [M][I] (caller-owned, not
 * overlapping A or Wgu); all pointers 16-byte aligned.  Asynchronous on
 * hip_stream.  Errors: WSG_ERR_INVALID_ARG for a bad shape, null or misaligned
 * pointer; WSG_ERR_UNSUPPORTED for a shape no compiled kernel takes. */
wsg_status wsg_gemm_swiglu_f32(int32_t M, int32_t I, int32_t K, const float* d_A, const float* d_Wgu, float* d_ACT,
                               void* hip_stream);

/* Read-only streaming reference for the cold-cache GEMV measurements (Our
 * Kernel Benchmark Was Measuring the System Cache, "The fix": the GEMV is
 * judged against what a plain read of the same cycling buffers reaches).
 * Reads all `bytes` of d_buf (16-byte aligned, bytes a positive multiple of
 * 16) once with 16-byte non-temporal loads (the load form of the decode
 * weight streams), one 4 KiB segment per wave; writes nothing
 * in practice (d_out, one float, is written only if the sum equals an
 * improbable constant).  Asynchronous on hip_stream. */
wsg_status wsg_stream_read(const void* d_buf, int64_t bytes, float* d_out, void* hip_stream);

/* Greedy selection over stand-alone logit vectors: d_out[r] = the lowest
 * index i whose logit d_logits[r][i] is maximal, for r < rows (Megakernels,
 * "GPU-wide end-to-end generation": the next token is chosen on the GPU,
 * ties going to the lowest token id; -0.0 and +0.0 tie).  The same ordering
 * as the decode head's argmax, as two ordered launches: one key per 4096
 * logits into d_workspace, then one block per row.
 *   dtype WSG_F32: d_logits float [rows][n]; WSG_F16: half [rows][n];
 *   d_out int32 [rows] (device memory, written by the second launch);
 *   d_workspace at least wsg_argmax_workspace_bytes(rows, n) bytes, 8-byte
 *   aligned, caller-owned scratch (its contents on entry do not matter).
 * Logits must be finite (a NaN is ordered by its bit pattern).  1 <= rows
 * <= 65535, 1 <= n <= 2^30.  Asynchronous on hip_stream.  Errors: a bad dtype or
 * size, a NULL or misaligned pointer, a workspace that is too small
 * (WSG_ERR_INVALID_ARG). */
wsg_status wsg_argmax_workspace_bytes(int32_t rows, int32_t n, size_t* bytes);
wsg_status wsg_argmax(int32_t dtype, int32_t rows, int32_t n, const void* d_logits, int32_t* d_out,
                      void* d_workspace, size_t ws_bytes, void* hip_stream);

/* wsg_argmax for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same result and kernels, with the span keys in a library-owned device
 * array of 16384 keys (128 KiB; each GPU the library runs on holds its own
 * copy until the process ends) instead of a caller workspace.  Allocates
 * nothing; the caller passes the logits and the output.  At most
 * rows * ceil(n / 4096) <= 16384 (WSG_ERR_INVALID_ARG beyond, before any
 * launch).  The current device must be the stream's; the first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress), so
 * make one call outside any graph capture first.  All calls on one GPU share
 * its array: calls that overlap on one GPU (other streams, other host
 * threads) race.  Other arguments and errors as for wsg_argmax. */
wsg_status wsg_argmax_noalloc(int32_t dtype, int32_t rows, int32_t n, const void* d_logits, int32_t* d_out,
                              void* hip_stream);

/* Weight storage the decode path reads: matrices with a packed copy (of
 * 1 + 4 n_layers decode matrices) and the decode weight bytes per token
 * (packed copies count half). */
wsg_status wsg_weight_storage(const wsg_model* m, int32_t* packed_matrices, int32_t* decode_matrices,
                              int64_t* decode_weight_bytes);

/* A JSON text describing the model's launch shapes, for reports (the pages
 * record kernel fingerprints beside their figures: Benchmark methodology,
 * "Long-document chunked prefill"): rows per wave and grids of every decode
 * stage for one- and two-token steps, the attention mode, split count and
 * keys per split at sample context lengths, the prefill chunk, graph use and
 * the library version.  Writes at most n bytes (NUL-terminated) to buf (may be
 * NULL) and the full length + 1 to *needed.  Errors: NULL model or needed. */
wsg_status wsg_describe(const wsg_model* m, char* buf, size_t n, size_t* needed);

/* Message for the last error on this host thread ("" if none).  (Library
 * plumbing: no defining passage.) */
const char* wsg_last_error(void);

/* Library version string.  (Library plumbing: no defining passage.) */
const char* wsg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WSG_H */
