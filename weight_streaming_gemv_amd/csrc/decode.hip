// Decode-step kernels for gfx950: one token through the decoder.
//
// The pages split a layer into eight ordered stages connected by device
// buffers, with no host waits and no cross-workgroup spin barriers
// (Megakernels, "GPU-wide end-to-end generation").  Here the same order is
// kept with fewer, fused launches per layer:
//
//   qkv     input RMSNorm (each wave normalises the 1024-float residual in
//           registers) + fused Q/K/V GEMV; layer 0 also gathers the token's
//           embedding row and writes it to the residual buffer
//   attn_o  (short contexts) per-head Q/K RMSNorm +
//           RoPE + K/V cache write + grouped-query attention, fused with the
//           output GEMV split by KV head: per-head partial sums, the first
//           one carrying the residual
//   attn    (longer contexts) the same attention, split-K over the keys;
//           a merge launch combines the partial softmax states
//   o       (longer contexts) output GEMV + residual add
//   gateup  [sum of the attn_o partials +] post-attention RMSNorm + gate/up
//           GEMV + SwiGLU
//   down    down GEMV + residual add
//   head    final RMSNorm + tied vocabulary GEMV + per-block argmax keys
//   argmax  one block reduces the block keys; writes the token into the
//           token history and advances the position
//
// Every GEMV wave owns R consecutive output rows and streams them with
// 16-byte loads; reductions accumulate in FP32 and are combined with DPP.
#include <type_traits>

#include "common.hpp"
#include "decode.hpp"

namespace wsg {

namespace {

constexpr int kD = 128;          // head_dim
constexpr float kLog2e = 1.4426950408889634f;

__host__ __device__ __forceinline__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Activations of length K in the lane layout the GEMV rows use:
// a[c*VEC + i] = x[c*64*VEC + lane*VEC + i] (VEC consecutive elements per
// lane and chunk, loaded as VEC / Vec16<TS>::N 16-byte vectors).
template <typename TS, int K, int VEC = Vec16<TS>::N>
struct Act {
  static constexpr int V16 = Vec16<TS>::N;
  static constexpr int NV = K / (kWave * VEC);
  static_assert(K % (kWave * VEC) == 0, "K must be a multiple of 64 lane vectors");
  static_assert(VEC % V16 == 0, "whole 16-byte vectors per lane and chunk");
  float a[K / kWave];

  __device__ __forceinline__ void load(const TS* p) {
    const int lane = lane_id();
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
      for (int u = 0; u < VEC / V16; ++u) {
        Vec16<TS> v;
        v.template load<false>(p + c * kWave * VEC + lane * VEC + u * V16);
#pragma unroll
        for (int i = 0; i < V16; ++i) a[c * VEC + u * V16 + i] = v.v[i];
      }
  }
  // Sum of NP FP32 vectors (n-th at p + n * stride) in the same element order,
  // added in order n = 0, 1, ... and rounded as stored: a residual that
  // arrives as partial slices.  16-byte loads (VEC is a multiple of 4).
  template <int NP>
  __device__ __forceinline__ void load_sum_f32(const float* __restrict__ p, size_t stride) {
    static_assert(VEC % 4 == 0, "whole float4 per lane and chunk");
    const int lane = lane_id();
    f4_t v[NP][NV * VEC / 4];
#pragma unroll
    for (int n = 0; n < NP; ++n)
#pragma unroll
      for (int c = 0; c < NV; ++c)
#pragma unroll
        for (int u = 0; u < VEC / 4; ++u)
          v[n][c * VEC / 4 + u] = *reinterpret_cast<const f4_t*>(p + n * stride + c * kWave * VEC + lane * VEC + 4 * u);
#pragma unroll
    for (int i = 0; i < NV * VEC / 4; ++i) {
      f4_t acc = v[0][i];
#pragma unroll
      for (int n = 1; n < NP; ++n) acc += v[n][i];
#pragma unroll
      for (int e = 0; e < 4; ++e) a[4 * i + e] = Store<TS>::to_f(Store<TS>::from_f(acc[e]));
    }
  }
  // From an FP32 array in the same element order (e.g. in LDS).
  __device__ __forceinline__ void load_f32(const float* p) {
    const int lane = lane_id();
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
      for (int i = 0; i < VEC; ++i) a[c * VEC + i] = p[c * kWave * VEC + lane * VEC + i];
  }
  __device__ __forceinline__ void store(TS* p) const {
    const int lane = lane_id();
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
      for (int i = 0; i < VEC; ++i) p[c * kWave * VEC + lane * VEC + i] = Store<TS>::from_f(a[c * VEC + i]);
  }
  // In-register RMSNorm with gain: a = a * (mean(a^2) + eps)^-1/2 * g.
  __device__ __forceinline__ void rms_norm(const TS* gain, float eps) {
    Act<TS, K, VEC> g;
    g.load(gain);
    rms_norm(g, eps);
  }
  // The same with the gain already loaded (its load issued ahead of the
  // weight rows, so that the norm does not wait for them: vector loads
  // return in issue order).
  __device__ __forceinline__ void rms_norm(const Act& g, float eps) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < K / kWave; ++i) ss = fmaf(a[i], a[i], ss);
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)K + eps);
#pragma unroll
    for (int i = 0; i < K / kWave; ++i) a[i] = a[i] * inv * g.a[i];
  }
};

// Weight streams are read once per step and never reused within it, so
// they are loaded non-temporally: on this part a read-only stream of the
// vocabulary matrix runs at 6.8 TB/s with non-temporal loads against 6.2
// TB/s with ordinary ones.  Activations, the K/V cache and partials (reused
// from L2 by many blocks) keep ordinary loads.
constexpr bool kWeightsNT = true;
template <typename V>
__device__ __forceinline__ V weight_load(const V* p) {
  if constexpr (kWeightsNT) return __builtin_nontemporal_load(p);
  else return *p;
}

// R weight rows held in registers (vectors in the lane layout of Act), so a
// wave can put its first rows in flight before its prologue finishes.  TW is
// the weight storage: TS itself, or packed FP32 (bf16w) with FP32
// activations, which gives the same lane layout and products.
template <typename TW, int K, int R>
struct WRows {
  using Vec = typename WVec<TW>::type;
  static constexpr int VEC = Vec::N;
  static constexpr int NV = K / (kWave * VEC);
  Vec v[R][NV];
  // rows row0 .. row0+R-1 (clamped to M-1) of a matrix whose rows are ld
  // elements apart (ld = K for whole rows; a K-slice of wider rows otherwise)
  __device__ __forceinline__ void load(const TW* __restrict__ W, int row0, int M, size_t ld = K) {
    const int lane = lane_id();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const TW* wr = W + (size_t)min(row0 + r, M - 1) * ld + lane * VEC;
#pragma unroll
      for (int c = 0; c < NV; ++c) v[r][c].template load<kWeightsNT>(wr + c * kWave * VEC);
    }
  }
  template <typename A>
  __device__ __forceinline__ void dot(const A& x, float (&acc)[R]) const {
    static_assert(A::NV == NV && A::NV * VEC * kWave == K, "weights and activations share the lane layout");
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < NV; ++c)
#pragma unroll
        for (int i = 0; i < VEC; ++i) a = fmaf(v[r][c].v[i], x.a[c * VEC + i], a);
      acc[r] = a;
    }
  }
};

// ---------------------------------------------------------- int4 weights
// Activations of an int4 GEMV: FP16 pairs in registers, ordered to meet the
// nibble pairs (j, j+4) that one masked 32-bit word yields.  Lane layout:
// chunk c, word i (0, 1), pair j (0..3) holds x[k0 + 8i + j] and
// x[k0 + 8i + j + 4], k0 = c*1024 + 16*lane.  Rounding the FP32 activations
// to FP16 here is the storage rounding of the stage input.
template <int K>
struct Q4Act {
  static constexpr int NV = K / 1024;
  h2_t h[NV][8];
  template <typename TS>
  __device__ __forceinline__ void from(const Act<TS, K, 16>& x) {
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h2_t p;
          p.x = (_Float16)x.a[c * 16 + 8 * i + j];
          p.y = (_Float16)x.a[c * 16 + 8 * i + j + 4];
          h[c][4 * i + j] = p;
        }
  }
};

// Row n of an int4 matrix of width K.
template <int K>
__device__ __forceinline__ const uint8_t* q4_row(const q4w* W, size_t n) {
  return reinterpret_cast<const uint8_t*>(W) + n * Q4Row<K>::kBytes;
}

// The four FP16 pairs of one word: nibbles (j, j+4) of w as exact FP16
// values q = u - 8, from u = q ^ 8 (two's complement to offset binary)
// OR-ed under the exponent of 1024 and reduced by 1032.
__device__ __forceinline__ void q4_pairs(uint32_t w, h2_t (&p)[4]) {
  const h2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  const uint32_t v = w ^ 0x88888888u;
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = as_h2(((v >> (4 * j)) & 0x000F000Fu) | 0x64006400u) - bias;
}

template <int K, int R>
struct WRows<q4w, K, R> {
  static constexpr int NV = K / 1024;
  typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
  u2_t q[R][NV];
  uint16_t s[R][NV];
  __device__ __forceinline__ void load(const q4w* __restrict__ W, int row0, int M) {
    const int lane = lane_id();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint8_t* row = q4_row<K>(W, (size_t)min(row0 + r, M - 1));
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        q[r][c] = weight_load(reinterpret_cast<const u2_t*>(row + c * 512 + lane * 8));
        s[r][c] = weight_load(reinterpret_cast<const uint16_t*>(row + Q4Row<K>::kWordBytes + 2 * (c * 16 + (lane >> 2))));
      }
    }
  }
  // acc[r] = sum over chunks of s * (sum of the chunk's 16 q*x products):
  // products exact, FP32 accumulation.
  __device__ __forceinline__ void dot(const Q4Act<K>& x, float (&acc)[R]) const {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        h2_t p[4];
        float in = 0.f;
        q4_pairs(q[r][c].x, p);
#pragma unroll
        for (int j = 0; j < 4; ++j) in = dot2(p[j], x.h[c][j], in);
        q4_pairs(q[r][c].y, p);
#pragma unroll
        for (int j = 0; j < 4; ++j) in = dot2(p[j], x.h[c][4 + j], in);
        a = fmaf(__half2float(__ushort_as_half(s[r][c])), in, a);
      }
      acc[r] = a;
    }
  }
};

// Row n of the lane's elements of an int4 matrix, dequantised (q * s,
// exact in FP32) and rounded as stored: the embedding gather of an int4
// model.
template <typename TS, int K>
__device__ __forceinline__ void q4_gather(const q4w* __restrict__ E, size_t n, Act<TS, K, 16>& x) {
  const int lane = lane_id();
  const uint8_t* row = q4_row<K>(E, n);
#pragma unroll
  for (int c = 0; c < K / 1024; ++c) {
    typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
    const u2_t w = *reinterpret_cast<const u2_t*>(row + c * 512 + lane * 8);
    const float s = __half2float(
        __ushort_as_half(*reinterpret_cast<const uint16_t*>(row + Q4Row<K>::kWordBytes + 2 * (c * 16 + (lane >> 2)))));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t word = i < 8 ? w.x : w.y;
      const int q = (int)(word << (28 - 4 * (i & 7))) >> 28;   // sign-extended nibble
      x.a[c * 16 + i] = Store<TS>::to_f(Store<TS>::from_f((float)q * s));
    }
  }
}

// Activation operand of a weight storage: the FP32 lane array (plain and
// packed FP32 storage), or FP16 pairs for int4 (built once per wave, after
// the norm).
template <typename TS, typename TW, int K>
struct Operand {
  using act = Act<TS, K, WVec<TW>::type::N>;
  using dot_t = act;
  static __device__ __forceinline__ dot_t prep(const act& a) { return a; }
};
template <typename TS, int K>
struct Operand<TS, q4w, K> {
  using act = Act<TS, K, 16>;
  using dot_t = Q4Act<K>;
  static __device__ __forceinline__ dot_t prep(const act& a) {
    dot_t d;
    d.from(a);
    return d;
  }
};

// Whether the QKV and gate/up launches issue their norm gain ahead of the
// weight rows (so that the norm need not wait for the rows: vector loads
// return in issue order).  Measured: 16-bit storage +2-3 % decode tokens/s;
// FP32 -0.9 % (its weight rows take the registers), so there the gain
// follows the rows.
template <typename TS> constexpr bool kGainAhead = !std::is_same<TS, float>::value;

// Rows [n, ...) of a matrix of width K (the up half of the gate/up matrix).
template <typename TW, int K>
__device__ __forceinline__ const TW* rows_from(const TW* W, size_t n) {
  if constexpr (std::is_same<TW, q4w>::value) return reinterpret_cast<const q4w*>(q4_row<K>(W, n));
  else return W + n * K;
}

__device__ __forceinline__ int wave_row_groups_begin() { return blockIdx.x * kWavesPerBlock + wave_id(); }
__device__ __forceinline__ int wave_row_groups_stride() { return gridDim.x * kWavesPerBlock; }

// Lane r's value of v (r wave-uniform).
__device__ __forceinline__ float lane_value(float v, int r) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), r));
}

// Lane r < R gets base[row0 + r] (rows clamped to M-1): residual values put
// in flight with the operands instead of being loaded after the dot.
template <typename TS, int R>
__device__ __forceinline__ float rows_prefetch(const TS* __restrict__ base, int row0, int M) {
  const int lane = lane_id();
  return Store<TS>::to_f(base[min(row0 + (lane < R ? lane : R - 1), M - 1)]);
}

// ------------------------------------------------------------------ qkv
// T query rows (a T-token step: positions p .. p+T-1) share every weight
// row streamed: activations and outputs are [T][.] arrays.
// NPD > 0: the residual arrives as the previous layer's NPD split-K slices
// of the down projection (FP32, the first carrying that layer's residual) at
// dpart[(t*NPD + s)*H]: every wave sums them in slice order and rounds as
// stored, and block 0 writes the residual x_res for the attention launch.
// Arguments are ordered so that the ones the first loads need fill the 14
// dwords preloaded into SGPRs at wave launch (the rest arrive by a scalar
// load that the first loads then need not wait for).
template <typename TS, typename TW, int H, int R, int T, int NPD>
__global__ __launch_bounds__(kBlock) void k_qkv(const TW* __restrict__ W, TS* __restrict__ x_res,
                                                const TS* __restrict__ in_norm, const float* __restrict__ dpart,
                                                int M, int first_layer, TS* __restrict__ out, float eps, int vocab,
                                                const void* __restrict__ embed, const int32_t* __restrict__ ids,
                                                const int32_t* __restrict__ ctrl, const float* __restrict__ rope_cos,
                                                const float* __restrict__ rope_sin, float* __restrict__ rope_cur) {
  using Op = Operand<TS, TW, H>;
  const int ngroups = ceil_div(M, R);
  int g = wave_row_groups_begin();
  WRows<TW, H, R> w;
  typename Op::act x[T];
  // Vector loads return in issue order: the residual goes out before the
  // first weight rows (so the norm overlaps them); at layer 0 the
  // position -> id -> embedding chain is issued after them.
  if (!first_layer) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if constexpr (NPD > 0) x[t].template load_sum_f32<NPD>(dpart + (size_t)t * NPD * H, H);
      else x[t].load(x_res + t * H);
    }
  }
  typename Op::act gain;
  if constexpr (kGainAhead<TS>) gain.load(in_norm);
  __builtin_amdgcn_sched_barrier(0);
  w.load(W, g * R, M);   // rows clamped into W: no branch around the loads
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NPD > 0) {
    // the summed residual, for the attention launch (a constant index into x:
    // a run-time one would move the array out of registers)
    if (!first_layer && blockIdx.x == 0)
#pragma unroll
      for (int t = 0; t < T; ++t)
        if (wave_id() == t) x[t].store(x_res + t * H);
  }
  if (first_layer) {
    const int pos = ctrl[kCtrlPos];
    const int wave = wave_id();
#pragma unroll
    for (int t = 0; t < T; ++t) {
      int tok = ids[pos + t];
      tok = (tok < 0 || tok >= vocab) ? 0 : tok;   // ids are validated on the host; never read outside E
      if constexpr (std::is_same<TW, q4w>::value) q4_gather<TS, H>(static_cast<const q4w*>(embed), tok, x[t]);
      else x[t].load(static_cast<const TS*>(embed) + (size_t)tok * H);
      if (blockIdx.x == 0 && wave == t) x[t].store(x_res + t * H);
    }
    static_assert(2 * T <= kWavesPerBlock, "a wave per residual row and per rotary row");
    if (blockIdx.x == 0 && wave >= T && wave < 2 * T) {
      // the rotary row of position p + t, for every attention launch of this
      // step (their loads then do not wait for the position)
      static_assert(kD / 2 == kWave, "one rotary pair per lane");
      const int lane = lane_id(), t = wave - T;
      rope_cur[t * kD + lane] = rope_cos[(size_t)(pos + t) * (kD / 2) + lane];
      rope_cur[t * kD + kD / 2 + lane] = rope_sin[(size_t)(pos + t) * (kD / 2) + lane];
    }
  }
  typename Op::dot_t xd[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if constexpr (kGainAhead<TS>) x[t].rms_norm(gain, eps);
    else x[t].rms_norm(in_norm, eps);   // the gain loaded here, after the weight rows
    xd[t] = Op::prep(x[t]);
  }
  const int lane = lane_id();
  for (; g < ngroups; g += wave_row_groups_stride()) {
    float acc[T][R];
#pragma unroll
    for (int t = 0; t < T; ++t) w.dot(xd[t], acc[t]);
    const int next = g + wave_row_groups_stride();
    if (next < ngroups) w.load(W, next * R, M);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float s = wave_sum(acc[t][r]);
        if (lane == 0 && g * R + r < M) out[(size_t)t * M + g * R + r] = Store<TS>::from_f(s);
      }
  }
}

// ------------------------------------------------------------ o / down
// x_out[t][m] = x_in[t][m] + W[m] . in[t]  for m < M (M = hidden), t < T;
// the residual ping-pongs between two buffers, so no kernel rewrites what
// it reads.
template <typename TS, typename TW, int K, int R, int T>
__global__ __launch_bounds__(kBlock) void k_gemv_residual(const TW* __restrict__ W, const TS* __restrict__ in,
                                                          const TS* __restrict__ x_in, TS* __restrict__ x_out, int M,
                                                          int32_t* __restrict__ ctrl, int advance_pos) {
  using Op = Operand<TS, TW, K>;
  const int ngroups = ceil_div(M, R);
  int g = wave_row_groups_begin();
  // operands first, then the weight rows (vector loads return in issue order)
  typename Op::act x[T];
  float xr[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    x[t].load(in + t * K);
    xr[t] = rows_prefetch<TS, R>(x_in + t * M, g * R, M);
  }
  __builtin_amdgcn_sched_barrier(0);
  WRows<TW, K, R> w;
  w.load(W, g * R, M);   // rows clamped into W: no branch around the loads
  __builtin_amdgcn_sched_barrier(0);
  typename Op::dot_t xd[T];
#pragma unroll
  for (int t = 0; t < T; ++t) xd[t] = Op::prep(x[t]);
  const int lane = lane_id();
  for (; g < ngroups; g += wave_row_groups_stride()) {
    float acc[T][R];
#pragma unroll
    for (int t = 0; t < T; ++t) w.dot(xd[t], acc[t]);
    const int next = g + wave_row_groups_stride();
    float xr_next[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xr_next[t] = 0.f;
    if (next < ngroups) {
#pragma unroll
      for (int t = 0; t < T; ++t) xr_next[t] = rows_prefetch<TS, R>(x_in + t * M, next * R, M);
      w.load(W, next * R, M);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float s = wave_sum(acc[t][r]);
        const int m = g * R + r;
        if (lane == 0 && m < M) x_out[(size_t)t * M + m] = Store<TS>::from_f(lane_value(xr[t], r) + s);
      }
      xr[t] = xr_next[t];
    }
  }
  // (no kernel of this launch reads the position)
  if (advance_pos && blockIdx.x == 0 && threadIdx.x == 0) ctrl[kCtrlPos] = ctrl[kCtrlPos] + T;
}

// --------------------------------------------------- down, split over K
// The down projection in S slices of K (more, shorter waves: each streams
// K/S of a row).  Block (b, s): row groups of block b, columns
// [s*K/S, (s+1)*K/S); it writes FP32 slices
//   dpart[(t*S + s)*M + m] = W[m, slice s] . in[t][slice s]  (+ x_in[t][m] for s = 0),
// which the next layer's QKV launch adds up in slice order (rounding once,
// as stored).  One-shot grid: gridDim.x blocks of 4 waves cover every row.
template <typename TS, typename TW, int K, int S, int R, int T>
__global__ __launch_bounds__(kBlock) void k_down_split(const TW* __restrict__ W, const TS* __restrict__ in,
                                                       const TS* __restrict__ x_in, float* __restrict__ dpart, int M) {
  constexpr int KS = K / S;
  using Op = Operand<TS, TW, KS>;
  const int sl = blockIdx.y;
  const int g = wave_row_groups_begin();
  typename Op::act x[T];
  float xr[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    x[t].load(in + (size_t)t * K + sl * KS);
    xr[t] = sl == 0 ? rows_prefetch<TS, R>(x_in + t * M, g * R, M) : 0.f;
  }
  __builtin_amdgcn_sched_barrier(0);
  WRows<TW, KS, R> w;
  w.load(W + (size_t)sl * KS, g * R, M, K);   // rows clamped into W: no branch around the loads
  __builtin_amdgcn_sched_barrier(0);
  typename Op::dot_t xd[T];
#pragma unroll
  for (int t = 0; t < T; ++t) xd[t] = Op::prep(x[t]);
  const int lane = lane_id();
  float acc[T][R];
#pragma unroll
  for (int t = 0; t < T; ++t) w.dot(xd[t], acc[t]);
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = wave_sum(acc[t][r]);
      const int m = g * R + r;
      if (lane == 0 && m < M) dpart[((size_t)t * S + sl) * M + m] = lane_value(xr[t], r) + v;
    }
}

// -------------------------------------------------------------- gate/up
// Partial vectors (float4 loads per thread) the gate/up prologue holds in
// registers: T * ceil(H / 1024) * slots <= kMaxPartVec; other shapes use
// the separate attention and output-projection launches.
constexpr int kMaxPartVec = 16;

// act[t][m] = silu(Wg[m] . b_t) * (Wu[m] . b_t), b_t = rms(x2[t], post_norm);
// Wgu holds the I gate rows followed by the I up rows.  With NP > 0 the
// residual x2[t] arrives as NP FP32 partial vectors (the KV-head split of
// the fused attention/output launch, the first carrying the residual;
// slots past the KV head count hold zeros), at opart[(t*NP + slot)*H]:
// every block sums them in the same order, rounds as stored, and block 0
// writes x2 for the down projection.
template <typename TS, typename TW, int H, int R, int NP, int T>
__global__ __launch_bounds__(kBlock) void k_gateup(const TW* __restrict__ Wgu, const TS* __restrict__ post_norm,
                                                   const TS* __restrict__ x_res, const float* __restrict__ opart,
                                                   float eps, TS* __restrict__ act, int I, TS* __restrict__ x2_out) {
  using Op = Operand<TS, TW, H>;
  const int ngroups = ceil_div(I, R);
  const TW* Wu = rows_from<TW, H>(Wgu, I);
  const int tid = threadIdx.x;
  int g = wave_row_groups_begin();
  typename Op::act x[T], gain;
  WRows<TW, H, R> wg, wu;
  if constexpr (NP > 0) {
    // Vector loads return in issue order, so the partials (this thread's
    // float4 column of every partial, for each 1024-wide slice of x2) go out
    // before the weight rows, and their sum overlaps the weight stream.
    constexpr int NC = ceil_div(H, 4 * kBlock);
    static_assert(T * NC * NP <= kMaxPartVec, "partials held in registers");
    __shared__ float s_x[T][NC * 4 * kBlock];   // padded: every thread writes its column
    f4_t pv[T][NP][NC];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int i = min(4 * (c * kBlock + tid), H - 4);
          pv[t][p][c] = *reinterpret_cast<const f4_t*>(opart + (size_t)(t * NP + p) * H + i);
        }
    if constexpr (kGainAhead<TS>) gain.load(post_norm);
    __builtin_amdgcn_sched_barrier(0);   // partials (and gain) before weights
    wg.load(Wgu, g * R, I);   // rows clamped into W: no branch around the loads
    wu.load(Wu, g * R, I);
    __builtin_amdgcn_sched_barrier(0);   // all loads issued in this order first
    // (the sums are used unconditionally, so the loads are not sunk into a
    // branch below the weight loads)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int i = 4 * (c * kBlock + tid);
        f4_t v = pv[t][0][c];
#pragma unroll
        for (int p = 1; p < NP; ++p) v += pv[t][p][c];
        TS s4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s4[e] = Store<TS>::from_f(v[e]);
          v[e] = Store<TS>::to_f(s4[e]);
        }
        *reinterpret_cast<f4_t*>(&s_x[t][i]) = v;
        if (blockIdx.x == 0 && i < H)
#pragma unroll
          for (int e = 0; e < 4; ++e) x2_out[t * H + i + e] = s4[e];
      }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < T; ++t) x[t].load_f32(s_x[t]);
  } else {
#pragma unroll
    for (int t = 0; t < T; ++t) x[t].load(x_res + t * H);
    if constexpr (kGainAhead<TS>) gain.load(post_norm);
    __builtin_amdgcn_sched_barrier(0);
    wg.load(Wgu, g * R, I);   // rows clamped into W: no branch around the loads
    wu.load(Wu, g * R, I);
    __builtin_amdgcn_sched_barrier(0);
  }
  typename Op::dot_t xd[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if constexpr (kGainAhead<TS>) x[t].rms_norm(gain, eps);
    else x[t].rms_norm(post_norm, eps);   // the gain loaded here, after the weight rows
    xd[t] = Op::prep(x[t]);
  }
  const int lane = lane_id();
  for (; g < ngroups; g += wave_row_groups_stride()) {
    float ga[T][R], ua[T][R];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      wg.dot(xd[t], ga[t]);
      wu.dot(xd[t], ua[t]);
    }
    const int next = g + wave_row_groups_stride();
    if (next < ngroups) { wg.load(Wgu, next * R, I); wu.load(Wu, next * R, I); }
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float gs = wave_sum(ga[t][r]);
        const float us = wave_sum(ua[t][r]);
        const int m = g * R + r;
        if (lane == 0 && m < I) act[(size_t)t * I + m] = Store<TS>::from_f(gs / (1.0f + expf(-gs)) * us);
      }
  }
}

// ---------------------------------------------------------------- head
// (argmax keys: argmax_key / wave_max_u64 in common.hpp)

// The head writes one argmax key per block and row; a one-block kernel then
// reduces them (the pages' two argmax kernels, Megakernels, "GPU-wide
// end-to-end generation").  A single fused launch would need a device-scope
// release fence per block, and on this multi-XCD part each such fence
// writes back the issuing XCD's L2, which costs far more than the extra
// launch.  Row t's logits go to logits[t*V], its block keys to
// am_part[t*gridDim.x].
template <typename TS, typename TW, int H, int R, int WPB, int T>
__global__ __launch_bounds__(WPB * kWave) void k_head(const TW* __restrict__ E, const TS* __restrict__ final_norm,
                                                      const TS* __restrict__ x_res, float eps, TS* __restrict__ logits,
                                                      int V, unsigned long long* __restrict__ am_part) {
  __shared__ unsigned long long best_wave[T][WPB];
  const int lane = lane_id();
  const int ngroups = ceil_div(V, R);
  int g = blockIdx.x * WPB + wave_id();
  const int stride = gridDim.x * WPB;
  using Op = Operand<TS, TW, H>;
  WRows<TW, H, R> w;
  if (g < ngroups) w.load(E, g * R, V);   // first rows in flight before the norm
  typename Op::dot_t xd[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    typename Op::act x;
    x.load(x_res + t * H);
    x.rms_norm(final_norm, eps);
    xd[t] = Op::prep(x);
  }
  unsigned long long best[T];
#pragma unroll
  for (int t = 0; t < T; ++t) best[t] = 0;   // below every real key
  for (; g < ngroups; g += stride) {
    float acc[T][R];
#pragma unroll
    for (int t = 0; t < T; ++t) w.dot(xd[t], acc[t]);
    const int next = g + stride;
    if (next < ngroups) w.load(E, next * R, V);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float s = wave_sum(acc[t][r]);
        const int m = g * R + r;
        if (m < V) {
          const TS stored = Store<TS>::from_f(s);
          if (lane == 0) logits[(size_t)t * V + m] = stored;
          const unsigned long long k = argmax_key(Store<TS>::to_f(stored), m);
          best[t] = k > best[t] ? k : best[t];
        }
      }
  }
  if (lane == 0)
#pragma unroll
    for (int t = 0; t < T; ++t) best_wave[t][wave_id()] = best[t];
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    unsigned long long b = best_wave[t][0];
#pragma unroll
    for (int w2 = 1; w2 < WPB; ++w2) b = best_wave[t][w2] > b ? best_wave[t][w2] : b;
    am_part[(size_t)t * gridDim.x + blockIdx.x] = b;
  }
}

// One block of 1024 threads reads the n block keys of each of the T rows
// (n even: the head grid is rounded up to an even count, a block without
// rows writes key 0) as 16-byte pairs: thread i takes pairs i + 1024k for
// k < PER, all loads issued before the first compare; pair indices past
// the last are clamped to it instead of branched on (a repeated key cannot
// change a maximum).
//
// Every token word written below is also written to the pinned host
// mailbox (MailWord layout), which the host reads after synchronising.
//
// Row t's token goes to ctrl[kCtrlRowTok + t].  One row (a decode step):
// it is also the output token, the next history entry, and the position
// advances by one.  Two rows (a two-token step whose second input is a
// draft of the first row's token): the draft is accepted when it equals
// row 0's greedy token; then both tokens are emitted and the position
// advances by two, else only row 0's token is emitted (slot p + 1 then
// holds the rejected draft's key and value, which the next step
// overwrites) and the position advances by one.  The history receives the
// emitted tokens, so a following step continues from the last one.
template <int PER, int T>
__global__ __launch_bounds__(1024) void k_argmax(const unsigned long long* __restrict__ am_part, int n,
                                                 int32_t* __restrict__ ctrl, int32_t* __restrict__ ids,
                                                 int32_t* __restrict__ mail) {
  static_assert(T == 1 || T == 2, "one- and two-token steps");
  __shared__ unsigned long long red[T][1024 / kWave];
  typedef unsigned long long u64x2_t __attribute__((ext_vector_type(2)));
  const u64x2_t* pairs = reinterpret_cast<const u64x2_t*>(am_part);
  const int half = n / 2, last = half - 1;
  u64x2_t k[T][PER];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < PER; ++i) k[t][i] = pairs[t * half + min((int)threadIdx.x + 1024 * i, last)];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    unsigned long long b = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      b = k[t][i].x > b ? k[t][i].x : b;
      b = k[t][i].y > b ? k[t][i].y : b;
    }
    b = wave_max_u64(b);
    if (lane_id() == 0) red[t][threadIdx.x >> 6] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int tok[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      unsigned long long b = red[t][0];
      for (int w = 1; w < (int)(blockDim.x >> 6); ++w) b = red[t][w] > b ? red[t][w] : b;
      tok[t] = argmax_key_index(b);
      if (b == 0) tok[t] = 0;   // no block key at all (cannot happen with vocab >= 1)
      ctrl[kCtrlRowTok + t] = tok[t];
      mail[kMailRowTok + t] = tok[t];
    }
    const int pos = ctrl[kCtrlPos];
    if constexpr (T == 1) {
      ctrl[kCtrlOutTok] = tok[0];
      mail[kMailOutTok] = tok[0];
      ids[pos + 1] = tok[0];
      mail[kMailHist + pos + 1] = tok[0];
      ctrl[kCtrlPos] = pos + 1;
    } else {
      const int accepted = ids[pos + 1] == tok[0] ? 1 : 0;
      ids[pos + 1] = tok[0];
      mail[kMailHist + pos + 1] = tok[0];
      if (accepted) {
        ids[pos + 2] = tok[1];
        mail[kMailHist + pos + 2] = tok[1];
      }
      ctrl[kCtrlOutTok] = accepted ? tok[1] : tok[0];
      mail[kMailOutTok] = accepted ? tok[1] : tok[0];
      ctrl[kCtrlPos] = pos + 1 + accepted;
    }
  }
}

__global__ void k_set_pos(int32_t* ctrl, int pos) {
  if (threadIdx.x == 0) ctrl[kCtrlPos] = pos;
}

// ------------------------------------------------------------ attention
// Lane layout for one 128-wide head row: a row of 16 lanes covers one key;
// lane sl of the row holds dims [4sl, 4sl+4) and [64+4sl, 64+4sl+4), so both
// members of every rotary pair (i, i+64) sit in the same lane.
// NT: non-temporal loads (cached keys that no other block of the launch reads).
template <typename TS, bool NT = false>
__device__ __forceinline__ void load_head8(const TS* p, int sl, float (&v)[8]) {
  auto ld = [](const auto* q) {
    if constexpr (NT) return __builtin_nontemporal_load(q);
    else return *q;
  };
  if constexpr (sizeof(TS) == 4) {
    const f4_t lo = ld(reinterpret_cast<const f4_t*>(p + 4 * sl));
    const f4_t hi = ld(reinterpret_cast<const f4_t*>(p + 64 + 4 * sl));
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  } else {
    typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
    const u2_t lo = ld(reinterpret_cast<const u2_t*>(p + 4 * sl));
    const u2_t hi = ld(reinterpret_cast<const u2_t*>(p + 64 + 4 * sl));
    const uint32_t w[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __half2float(__ushort_as_half((unsigned short)(w[i] & 0xFFFFu)));
      v[2 * i + 1] = __half2float(__ushort_as_half((unsigned short)(w[i] >> 16)));
    }
  }
}

template <typename TS>
__device__ __forceinline__ void store_head8(TS* p, int sl, const float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[4 * sl + i] = Store<TS>::from_f(v[i]);
    p[64 + 4 * sl + i] = Store<TS>::from_f(v[4 + i]);
  }
}

// Per-head RMSNorm (over the 16 lanes of a row) with gain g, then rotation
// at position p (c, s: this lane's cos/sin of its four pairs).
__device__ __forceinline__ void norm_rope8(float (&v)[8], const float (&g)[8], const float (&c)[4],
                                           const float (&s)[4], float eps) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
  ss = row16_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)kD + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = v[i] * inv * g[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = v[i], hi = v[4 + i];
    v[i] = lo * c[i] - hi * s[i];
    v[4 + i] = hi * c[i] + lo * s[i];
  }
}

template <typename TS>
__device__ __forceinline__ void round_to_store(float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = Store<TS>::to_f(Store<TS>::from_f(v[i]));
}

template <int G>
struct SoftState {
  float m[G], l[G], acc[G][8];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
    }
  }
  // Online softmax update with one key (scores in the log2 domain).
  __device__ __forceinline__ void add(const float (&q)[G][8], const float (&k)[8], const float (&v)[8]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) d = fmaf(q[g][i], k[i], d);
      d = row16_sum(d);
      const float mn = fmaxf(m[g], d);
      const float alpha = exp2f(m[g] - mn);
      const float p = exp2f(d - mn);
      l[g] = fmaf(l[g], alpha, p);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(acc[g][i], alpha, p * v[i]);
      m[g] = mn;
    }
  }
  // Up to four keys at once (key u where use[u]): their scores are
  // independent, so the dot-product reductions and exponentials overlap
  // instead of forming one chain per key.  Same online-softmax state.
  __device__ __forceinline__ void add4(const float (&q)[G][8], const float (&k)[4][8], const float (&v)[4][8],
                                       const bool (&use)[4]) {
    float d[G][4];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaf(q[g][i], k[u][i], a);
        d[g][u] = a;
      }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) d[g][u] = row16_sum(d[g][u]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mn = m[g];
#pragma unroll
      for (int u = 0; u < 4; ++u) mn = use[u] ? fmaxf(mn, d[g][u]) : mn;
      if (mn == -INFINITY) continue;            // no key yet, none added (this lane's key-row)
      const float alpha = exp2f(m[g] - mn);     // exp2(-inf) = 0 before the first key
      float p[4], ls = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        p[u] = use[u] ? exp2f(d[g][u] - mn) : 0.f;
        ls += p[u];
      }
      l[g] = fmaf(l[g], alpha, ls);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a = acc[g][i] * alpha;
#pragma unroll
        for (int u = 0; u < 4; ++u) a = use[u] ? fmaf(p[u], v[u][i], a) : a;   // an unused value may be NaN
        acc[g][i] = a;
      }
      m[g] = mn;
    }
  }
  // Merge with the state of the lane MASK lanes away (another key-row of
  // the wave: MASK 16 or 32), so that after masks 16 and 32 every key-row of
  // the wave holds the merge of its four.  Both lanes of a pair compute the
  // merge from the same (lower lane, upper lane) operands, so they hold the
  // same bits.
  template <int MASK>
  __device__ __forceinline__ void combine_xor() {
    static_assert(MASK == 16 || MASK == 32, "key-rows of a wave");
    auto pair = [](float v) { return MASK == 32 ? lanes_xor32(v) : lanes_xor16(v); };
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const LanePair pm = pair(m[g]), pl = pair(l[g]);
      const float mn = fmaxf(pm.lo, pm.hi);
      const float a = mn == -INFINITY ? 0.f : exp2f(pm.lo - mn);
      const float b = mn == -INFINITY ? 0.f : exp2f(pm.hi - mn);
      l[g] = fmaf(pl.lo, a, pl.hi * b);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const LanePair pa = pair(acc[g][i]);
        acc[g][i] = fmaf(pa.lo, a, pa.hi * b);
      }
      m[g] = mn;
    }
  }
};

// Partial state layout: for each (row, kv head, split, g): [m, l, -, -,
// acc[128]] (kAttnPartStride floats; the accumulators 16-byte aligned).
constexpr int kPartStride = kAttnPartStride;
constexpr int kPartAcc = 4;
static_assert(kPartStride == kPartAcc + kD && kPartStride % 4 == 0, "partial state layout");

// The attention of one KV head j (its G query heads) for one query row at
// position p, over the keys [k_begin, k_end), spread over NR 16-lane rows
// of the block (16 for one query row per block; 8 each when two rows share
// a block): key-row sid takes keys k_begin + sid + NR*u.  prefetch() issues
// every load that does not depend on p (raw queries, the row's current key
// and value, its rotary row, the norm gains, and each key-row's first four
// cached keys, clamped into the cache: keys past p are loaded but never
// used), so they are in flight together with the read of p.  With PREV the
// row is the second of a two-token step and also folds in the first row's
// key and value (slot p - 1, written by another block of the same launch),
// recomputed here from the first row's projections.
template <typename TS, int G, int NR, bool PREV, bool NTKV = false, bool PIPE = false>
struct HeadAttn {
  float q[G][8], kc[8], vc[8], k4[4][8], v4[4][8], c[4], s[4], gq[8], gk[8];
  float kp[PREV ? 8 : 1], vp[PREV ? 8 : 1], cp[PREV ? 4 : 1], sp[PREV ? 4 : 1];

  __device__ __forceinline__ void prefetch(const TS* __restrict__ qkv, const TS* __restrict__ kh,
                                           const TS* __restrict__ vh, const TS* __restrict__ q_norm,
                                           const TS* __restrict__ k_norm, const float* __restrict__ rope,
                                           int j, int Q, int KV, int cap, int k_begin, int sid, int sl) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = min(k_begin + sid + NR * u, cap - 1);
      load_head8<TS, NTKV>(kh + (size_t)kk * kD, sl, k4[u]);
      load_head8<TS, NTKV>(vh + (size_t)kk * kD, sl, v4[u]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) load_head8<TS>(qkv + (size_t)(j * G + g) * kD, sl, q[g]);
    load_head8<TS>(qkv + Q + (size_t)j * kD, sl, kc);
    load_head8<TS>(qkv + Q + KV + (size_t)j * kD, sl, vc);
    load_rope4(rope, sl, c, s);
    load_head8<TS>(q_norm, sl, gq);
    load_head8<TS>(k_norm, sl, gk);
  }
  // The first row's raw key/value and rotary row (PREV only).
  __device__ __forceinline__ void prefetch_prev(const TS* __restrict__ qkv_prev, const float* __restrict__ rope_prev,
                                                int j, int Q, int KV, int sl) {
    if constexpr (PREV) {
      load_head8<TS>(qkv_prev + Q + (size_t)j * kD, sl, kp);
      load_head8<TS>(qkv_prev + Q + KV + (size_t)j * kD, sl, vp);
      load_rope4(rope_prev, sl, cp, sp);
    }
  }
  static __device__ __forceinline__ void load_rope4(const float* rope, int sl, float (&c4)[4], float (&s4)[4]) {
    const float4 cv = *reinterpret_cast<const float4*>(rope + 4 * sl);
    const float4 sv = *reinterpret_cast<const float4*>(rope + kD / 2 + 4 * sl);
    c4[0] = cv.x; c4[1] = cv.y; c4[2] = cv.z; c4[3] = cv.w;
    s4[0] = sv.x; s4[1] = sv.y; s4[2] = sv.z; s4[3] = sv.w;
  }

  // Cached keys [k_begin, k_stop); then, with has_prev, the first row's key
  // (slot p - 1); then, with has_cur, this row's key/value (slot p),
  // normalised, rotated and folded in from registers by key-row 0, which
  // also writes slot p when write_cur is set.
  __device__ __forceinline__ void run(TS* __restrict__ kh, TS* __restrict__ vh, int pos, int k_begin, int k_stop,
                                      bool has_prev, bool has_cur, bool write_cur, float eps, int sid, int sl,
                                      SoftState<G>& st) {
    // queries: normalised, rotated, rounded as stored, then pre-scaled by
    // log2(e)/sqrt(D) so that scores are in the log2 domain
    const float qscale = kLog2e / sqrtf((float)kD);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      norm_rope8(q[g], gq, c, s, eps);
      round_to_store<TS>(q[g]);
#pragma unroll
      for (int i = 0; i < 8; ++i) q[g][i] *= qscale;
    }
    st.init();
    // Keys in groups of 4*NR (four per key-row); the first group is in
    // registers already.
    if constexpr (!PIPE) {
      // Short ranges (the fused launch): each further group's loads are all
      // issued, then folded in.
      // (few keys per key-row: a key slot without a key is skipped, not
      // computed and discarded)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (k_begin + sid + NR * u < k_stop) st.add(q, k4[u], v4[u]);
      for (int key = k_begin + sid + 4 * NR; key < k_stop; key += 4 * NR) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (key + NR * u < k_stop) {
            load_head8<TS, NTKV>(kh + (size_t)(key + NR * u) * kD, sl, k4[u]);
            load_head8<TS, NTKV>(vh + (size_t)(key + NR * u) * kD, sl, v4[u]);
          }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (key + NR * u < k_stop) st.add(q, k4[u], v4[u]);
      }
    } else {
      // Split-K ranges: while a group is folded in, the next one's loads are
      // in flight.  The test for a next group is uniform over the block, so
      // both branches issue a fixed number of loads and the wait before the
      // fold covers only the older group.  Keys of the next group past the
      // range are read at its last key (in bounds, from cache) and not used.
      for (int base = k_begin;; base += 4 * NR) {
        if (base + 4 * NR < k_stop) {
          float kn[4][8], vn[4][8];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int key = min(base + 4 * NR + sid + NR * u, k_stop - 1);
            load_head8<TS, NTKV>(kh + (size_t)key * kD, sl, kn[u]);
            load_head8<TS, NTKV>(vh + (size_t)key * kD, sl, vn[u]);
          }
          const bool all[4] = {true, true, true, true};   // a whole group: base + 4*NR < k_stop
          st.add4(q, k4, v4, all);
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              k4[u][i] = kn[u][i];
              v4[u][i] = vn[u][i];
            }
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (base + sid + NR * u < k_stop) st.add(q, k4[u], v4[u]);
          break;
        }
      }
    }
    if constexpr (PREV) {
      if (has_prev) {
        norm_rope8(kp, gk, cp, sp, eps);
        round_to_store<TS>(kp);
        if (sid == 0) st.add(q, kp, vp);
      }
    }
    if (has_cur) {
      norm_rope8(kc, gk, c, s, eps);
      round_to_store<TS>(kc);
      if (sid == 0) {
        if (write_cur) {
          store_head8<TS>(kh + (size_t)pos * kD, sl, kc);
          store_head8<TS>(vh + (size_t)pos * kD, sl, vc);
        }
        st.add(q, kc, vc);
      }
    }
  }
};

// LDS merge of the NR key-row states of one query row.
template <int G, int NR>
struct RowMerge {
  float m[NR][G], l[NR][G];
  float acc[NR][G][kD];

  __device__ __forceinline__ void put(const SoftState<G>& st, int sid, int sl) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (sl == 0) { m[sid][g] = st.m[g]; l[sid][g] = st.l[g]; }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[sid][g][4 * sl + i] = st.acc[g][i];
        acc[sid][g][64 + 4 * sl + i] = st.acc[g][4 + i];
      }
    }
  }
  // Combined (max, sum, weighted output) of query head g, dim d.
  __device__ __forceinline__ void get(int g, int d, float& mx, float& L, float& A) const {
    mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < NR; ++r) mx = fmaxf(mx, m[r][g]);
    L = 0.f;
    A = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float w = exp2f(m[r][g] - mx);   // rows without keys: exp2(-inf) = 0
      L = fmaf(l[r][g], w, L);
      A = fmaf(acc[r][g][d], w, A);
    }
  }
};

// The fused launch's per-wave attention states, after each wave merged its
// four key-rows (SoftState::combine_xor): maxima and sums per [row][wave of
// the row][g], accumulators as float4 [hi][sl] = dims 64 hi + 4 sl .. +3.
template <int G, int T, int WPR>
struct WaveStates {
  float m[T][WPR][G], l[T][WPR][G];
  f4_t acc[T][WPR][G][2][16];

  // key-row 0 of wave wi of row t writes the wave's state
  __device__ __forceinline__ void put(const SoftState<G>& st, int t, int wi, int lane) {
    if (lane < 16) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        acc[t][wi][g][0][lane] = f4_t{st.acc[g][0], st.acc[g][1], st.acc[g][2], st.acc[g][3]};
        acc[t][wi][g][1][lane] = f4_t{st.acc[g][4], st.acc[g][5], st.acc[g][6], st.acc[g][7]};
        if (lane == 0) {
          m[t][wi][g] = st.m[g];
          l[t][wi][g] = st.l[g];
        }
      }
    }
  }
  // The attention output of query head g of row t, dims 64 hi + 4 sl .. +3:
  // the waves' states merged (a wave without keys has m = -inf, weight 0).
  __device__ __forceinline__ f4_t get4(int t, int g, int hi, int sl) const {
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < WPR; ++w) mx = fmaxf(mx, m[t][w][g]);
    float L = 0.f;
    f4_t A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < WPR; ++w) {
      const float e = exp2f(m[t][w][g] - mx);
      L = fmaf(l[t][w][g], e, L);
      const f4_t a = acc[t][w][g][hi][sl];
#pragma unroll
      for (int i = 0; i < 4; ++i) A[i] = fmaf(a[i], e, A[i]);
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int i = 0; i < 4; ++i) A[i] *= inv;
    return A;
  }
};

// Split-K attention: block (split, j, t) covers the keys of split for query
// row t (position p + t of a T-token step).  With direct set, a context
// within one split writes o itself; otherwise every split writes its
// partial state (for the merge, or the merging output projection).
template <typename TS, int G, int T>
// Arguments as the fused launch's: the first 14 dwords (preloaded into
// SGPRs) hold every address the loads and the position read need (dims =
// n_kv | hidden << 8; qkv from rope_cur, V after K, K-norm after Q-norm).
__global__ __launch_bounds__(kBlock) void k_attn(const float* __restrict__ rope_cur, TS* __restrict__ k_cache,
                                                 const TS* __restrict__ q_norm, const int32_t* __restrict__ ctrl,
                                                 int dims, int cap, int chunk, float eps, int direct,
                                                 float* __restrict__ part, TS* __restrict__ o) {
  constexpr bool PREV = T > 1;
  const int n_kv = dims & 0xFF, n_q = G * n_kv;
  const TS* qkv = reinterpret_cast<const TS*>(reinterpret_cast<const char*>(rope_cur) +
                                              row_block_qkv_offset(dims >> 8, sizeof(TS)));
  TS* v_cache = k_cache + (size_t)n_kv * cap * kD;
  const TS* k_norm = q_norm + kD;
  __shared__ RowMerge<G, 16> sm;
  const int j = blockIdx.y;            // KV head
  const int split = blockIdx.x;
  const int t = blockIdx.z;            // query row
  const int lane = lane_id(), wave = wave_id();
  const int sid = wave * 4 + (lane >> 4), sl = lane & 15;
  const size_t head_off = (size_t)j * cap * kD;
  const int Q = n_q * kD, KV = n_kv * kD, M = Q + 2 * KV;
  TS* kh = k_cache + head_off;
  TS* vh = v_cache + head_off;

  // Every split covers the fixed key range [split*chunk, split*chunk + chunk)
  // (chunk is fixed per captured graph), so its first keys can be loaded before p.
  const int k_begin = split * chunk;
  // one query row: each cached key is read by exactly one block of this
  // launch (two rows read it twice: ordinary loads, so the second may hit L2)
  HeadAttn<TS, G, 16, PREV, (T == 1), true> ha;
  ha.prefetch(qkv + (size_t)t * M, kh, vh, q_norm, k_norm, rope_cur + t * kD, j, Q, KV, cap, k_begin, sid, sl);
  ha.prefetch_prev(qkv, rope_cur, j, Q, KV, sl);   // (unused by row 0; no branch around loads)
  // keep the scheduler from moving work that waits on the first loads
  // (the query norm) above the later ones
  __builtin_amdgcn_sched_barrier(0);
  const int pos0 = ctrl[kCtrlPos];
  const int pos = pos0 + t;
  const int n_keys = pos + 1;
  const int n_splits = ceil_div(n_keys, chunk);
  // Splits past this row's context run on an empty range and write nothing
  // (an early return would let the compiler sink the loads above below the
  // position read).
  const bool active = split < n_splits;
  const int k_end = active ? min(n_keys, k_begin + chunk) : k_begin;
  const bool has_cur = active && k_end == n_keys;
  const bool has_prev = active && t > 0 && k_begin <= pos0 && pos0 < k_end;
  SoftState<G> st;
  ha.run(kh, vh, pos, k_begin, min(k_end, pos0), has_prev, has_cur, true, eps, sid, sl, st);

  sm.put(st, sid, sl);
  __syncthreads();
  if (!active) return;
  float* my_part = part + ((size_t)((t * n_kv + j) * gridDim.x + split) * G) * kPartStride;
  for (int e = threadIdx.x; e < G * kD; e += kBlock) {
    const int g = e / kD, d = e - g * kD;
    float mx, L, A;
    sm.get(g, d, mx, L, A);
    if (n_splits == 1 && direct) {
      o[(size_t)t * Q + (size_t)(j * G + g) * kD + d] = Store<TS>::from_f(A / L);
    } else {
      if (d == 0) { my_part[g * kPartStride] = mx; my_part[g * kPartStride + 1] = L; }
      my_part[g * kPartStride + kPartAcc + d] = A;
    }
  }
}

// ------------------------------------------- attention + output projection
// Blocks of the KV-head-split launches: one linear grid of (row blocks) x
// n_kv, block i serving KV head i % n_kv and row block i / n_kv.  Workgroups
// go to the XCDs round-robin by linear index, so with 8 KV heads all blocks
// of a head run on one XCD and share its L2: the head's K/V prefix (or its
// split states) comes from HBM once instead of once per XCD.
__device__ __forceinline__ int kv_head_of_block(int n_kv) { return (int)blockIdx.x % n_kv; }
__device__ __forceinline__ int row_block_of_block(int n_kv) { return (int)blockIdx.x / n_kv; }

// Short contexts: the output GEMV is split by KV head.  Block (b, j)
// recomputes the attention of KV head j over all keys (a few KiB per key
// range, read from L2 by the blocks of that head), then multiplies its 4R
// rows of W_o restricted to head j's G*128 columns, which it put in flight
// first:
//   part[t][j][m] = W_o[m, cols of head j] . o_j(row t)  (+ x[t][m] for j = 0).
// The gate/up launch sums the partials in a fixed order.  Blocks b = 0
// write the current tokens' keys and values into the cache.  With T = 2
// query rows, waves 0-1 serve row 0 and waves 2-3 row 1 (8 key-rows each).
// Vector type of the W_o slices: the weight format's, except FP16 slices,
// which load four values per lane (Half4Vec) so that every format with a
// 256-wide KV-head slice has four columns per lane.
template <typename TW> struct WoVec { using type = typename WVec<TW>::type; };
template <> struct WoVec<__half> { using type = Half4Vec; };

template <typename TW, int G, int R>
struct WoSlice {
  using Vec = typename WoVec<TW>::type;
  static constexpr int VEC = Vec::N;
  static constexpr int LPR = G * kD / VEC;          // 16-byte vectors per row slice
  static constexpr int NLD = R * LPR / kWave;       // vectors per lane
  static_assert((R * LPR) % kWave == 0, "whole vectors per lane");
  static_assert(LPR == 16 || LPR == 32 || LPR % kWave == 0, "row slice of 16, 32 or a multiple of 64 lanes");
  Vec v[NLD];

  // vector t of this lane: row (64t + lane) / LPR, column vector (64t + lane) % LPR
  __device__ __forceinline__ void load(const TW* __restrict__ Wo, int ld, int col0, int row0, int M) {
    const int lane = lane_id();
#pragma unroll
    for (int t = 0; t < NLD; ++t) {
      const int f = t * kWave + lane;
      const int row = min(row0 + f / LPR, M - 1);
      v[t].template load<kWeightsNT>(Wo + (size_t)row * ld + col0 + (f % LPR) * VEC);
    }
  }
  // apply() for R = 8 with the operand in registers: lane l holds
  // o[VEC l .. VEC l + VEC), the columns of its vector in every row (slices
  // of one vector per lane).  The eight row sums share one transposed
  // butterfly: across lane halves (xor 32), quarters (xor 16) and rows of
  // 16 (mirror) each lane keeps half of its values and adds its partner's
  // other half, so lane l ends with a partial of row l / 8 over 8 lanes,
  // which the 8-lane sum completes.  xb8: row (lane / 8)'s residual.
  __device__ __forceinline__ void apply_regs8(const float (&o)[VEC], int row0, int M, float xb8,
                                              float* __restrict__ out) const {
    static_assert(LPR == kWave && NLD == R && R == 8, "one vector per lane and row, eight rows");
    const int lane = lane_id();
    float d[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) a = fmaf(v[r].v[i], o[i], a);
      d[r] = a;
    }
    const bool b3 = lane & 8;
    float e[4], f[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {   // lower half keeps rows k, upper half rows k + 4
      const LanePair p = swap32(d[k], d[k + 4]);
      e[k] = p.lo + p.hi;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {   // even rows of 16 keep e[k], odd rows e[k + 2]
      const LanePair p = swap16(e[k], e[k + 2]);
      f[k] = p.lo + p.hi;
    }
    // lanes i and 15 - i of a row of 16 differ in bit 3: the partner's
    // other row, then the sum over the 8 lanes of this half-row (quad swaps
    // and the half-row mirror reach all of them)
    const float give = b3 ? f[0] : f[1];
    float a = (b3 ? f[1] : f[0]) + dpp<kDppMirror>(give);
    a = row8_sum(a);
    const int m = row0 + (lane >> 3);
    if ((lane & 7) == 0 && m < M) out[m] = a + xb8;
  }
  // out[row0 + r] = (this slice's row r) . o + lane r's xb
  __device__ __forceinline__ void apply(const float* o, int row0, int M, float xb, float* __restrict__ out) const {
    const int lane = lane_id();
    float d[NLD];
#pragma unroll
    for (int t = 0; t < NLD; ++t) {
      const int f = t * kWave + lane;
      const float* oc = o + (f % LPR) * VEC;
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) a = fmaf(v[t].v[i], oc[i], a);
      d[t] = a;
    }
    if constexpr (LPR % kWave == 0) {
      constexpr int TPR = LPR / kWave;              // vectors per row per lane
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < TPR; ++u) a += d[r * TPR + u];
        a = wave_sum(a);
        const int m = row0 + r;
        if (lane == 0 && m < M) out[m] = a + lane_value(xb, r);
      }
    } else {
#pragma unroll
      for (int t = 0; t < NLD; ++t) {
        float a = row16_sum(d[t]);
        if constexpr (LPR == 32) {
          const LanePair p = lanes_xor16(a);
          a = p.lo + p.hi;
        }
        const int f = t * kWave + lane;
        const int m = row0 + f / LPR;
        const float b = __shfl(xb, f / LPR);
        if (f % LPR == 0 && m < M) out[m] = a + b;
      }
    }
  }
};

// The int4 W_o slice: each lane holds 16 consecutive columns (two words and
// their group's scale) of one row; LPR lanes cover a row's G*128 columns.
// The attention output arrives as FP16 pairs in LDS, ordered as the nibble
// pairs of q4_pairs meet them (8 pairs per 16-column lane chunk).
template <int G, int R>
struct WoSlice<q4w, G, R> {
  static constexpr int LPR = G * kD / 16;           // lanes per row slice: 8, 16 or 32
  static constexpr int NLD = R * LPR / kWave;       // 8-byte loads per lane
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row slice of 8, 16 or 32 lanes");
  static_assert((R * LPR) % kWave == 0, "whole loads per lane");
  typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
  u2_t q[NLD];
  uint16_t s[NLD];

  __device__ __forceinline__ void load(const q4w* __restrict__ Wo, int ld, int col0, int row0, int M) {
    const int lane = lane_id();
    const size_t rb = (size_t)ld / 2 + (size_t)ld / 32;   // int4 row bytes of width ld
#pragma unroll
    for (int t = 0; t < NLD; ++t) {
      const int f = t * kWave + lane;
      const uint8_t* rp = reinterpret_cast<const uint8_t*>(Wo) + (size_t)min(row0 + f / LPR, M - 1) * rb;
      const int k = col0 + (f % LPR) * 16;
      q[t] = weight_load(reinterpret_cast<const u2_t*>(rp + k / 2));
      s[t] = weight_load(reinterpret_cast<const uint16_t*>(rp + ld / 2 + 2 * (k / 64)));
    }
  }
  // out[row0 + r] = (this slice's row r) . o + lane r's xb
  __device__ __forceinline__ void apply(const uint32_t* oh, int row0, int M, float xb, float* __restrict__ out) const {
    const int lane = lane_id();
#pragma unroll
    for (int t = 0; t < NLD; ++t) {
      const int f = t * kWave + lane;
      const uint4 a = *reinterpret_cast<const uint4*>(oh + (f % LPR) * 8);
      const uint4 b = *reinterpret_cast<const uint4*>(oh + (f % LPR) * 8 + 4);
      h2_t p[4];
      float in = 0.f;
      q4_pairs(q[t].x, p);
      in = dot2(p[0], as_h2(a.x), in);
      in = dot2(p[1], as_h2(a.y), in);
      in = dot2(p[2], as_h2(a.z), in);
      in = dot2(p[3], as_h2(a.w), in);
      q4_pairs(q[t].y, p);
      in = dot2(p[0], as_h2(b.x), in);
      in = dot2(p[1], as_h2(b.y), in);
      in = dot2(p[2], as_h2(b.z), in);
      in = dot2(p[3], as_h2(b.w), in);
      float v = __half2float(__ushort_as_half(s[t])) * in;
      if constexpr (LPR == 8) v = row8_sum(v);
      else v = row16_sum(v);
      if constexpr (LPR == 32) {
        const LanePair p = lanes_xor16(v);
        v = p.lo + p.hi;
      }
      const int m = row0 + f / LPR;
      const float xv = __shfl(xb, f / LPR);
      if (f % LPR == 0 && m < M) out[m] = v + xv;
    }
  }
};

// The W_o slice of KV head j times the head's attention output o (T rows,
// in LDS, already rounded as stored), plus the residual rows for j = 0:
// part[t][j][row0 + r] for the wave's rows.  Called by every thread after
// o is complete in LDS.
template <typename TW, int G, int R, int T>
__device__ __forceinline__ void wo_apply(const WoSlice<TW, G, R>& w, const float (&s_o)[T][G * kD], int row0, int H,
                                         const float (&xb)[T], float* __restrict__ opart, int part_row, int j) {
  if constexpr (std::is_same<TW, q4w>::value) {
    // o as FP16 pairs in the int4 slice's order (exact: o is FP16-rounded)
    __shared__ uint32_t s_oh[T][G * kD / 2];
    for (int e = threadIdx.x; e < T * G * kD / 2; e += kBlock) {
      const int r = e / (G * kD / 2), f = e - r * (G * kD / 2);
      const int c = (f / 8) * 16 + 8 * ((f % 8) / 4) + (f % 4);   // chunk, word, pair
      h2_t h;
      h.x = (_Float16)s_o[r][c];
      h.y = (_Float16)s_o[r][c + 4];
      s_oh[r][f] = __builtin_bit_cast(uint32_t, h);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < T; ++r) w.apply(s_oh[r], row0, H, xb[r], opart + (size_t)r * part_row + (size_t)j * H);
  } else {
#pragma unroll
    for (int r = 0; r < T; ++r) w.apply(s_o[r], row0, H, xb[r], opart + (size_t)r * part_row + (size_t)j * H);
  }
}

// Arguments: the first 14 dwords (preloaded into SGPRs at wave launch) hold
// every address the loads and the position read need, so no scalar load
// precedes them.  dims = n_kv | hidden << 8.  Derived from neighbours (the
// runtime checks these layouts before the launch): the residual x and the
// projections qkv from rope_cur (row_block_* offsets), the V cache block of
// a layer from its K block (n_kv * cap * 128 elements on) and the K-norm gain
// from the Q-norm gain (128 elements on).
template <typename TS, typename TW, int G, int R, int T>
__global__ __launch_bounds__(kBlock) void k_attn_o(const float* __restrict__ rope_cur, TS* __restrict__ k_cache,
                                                   const TS* __restrict__ q_norm, const int32_t* __restrict__ ctrl,
                                                   const TW* __restrict__ Wo, int dims, int cap, float eps,
                                                   int part_row, float* __restrict__ opart) {
  const int n_kv = dims & 0xFF, H = dims >> 8, n_q = G * n_kv;
  const char* rb = reinterpret_cast<const char*>(rope_cur);
  const TS* x_res = reinterpret_cast<const TS*>(rb + row_block_x_offset());
  const TS* qkv = reinterpret_cast<const TS*>(rb + row_block_qkv_offset(H, sizeof(TS)));
  TS* v_cache = k_cache + (size_t)n_kv * cap * kD;
  const TS* k_norm = q_norm + kD;
  constexpr int NR = 16 / T;           // key-rows per query row
  constexpr int WPR = kWavesPerBlock / T;
  const int j = kv_head_of_block(n_kv);   // KV head
  const int lane = lane_id(), wave = wave_id();
  const int t = wave / WPR;            // this wave's query row
  const int sid = (wave % WPR) * 4 + (lane >> 4), sl = lane & 15;
  const int row0 = (row_block_of_block(n_kv) * kWavesPerBlock + wave) * R;
  const size_t head_off = (size_t)j * cap * kD;
  const int Q = n_q * kD, KV = n_kv * kD, M = Q + 2 * KV;
  TS* kh = k_cache + head_off;
  TS* vh = v_cache + head_off;
  // Vector loads return in issue order: the attention operands go out
  // first, the W_o rows last, so the attention runs while the weights stream
  // in.  The position (a scalar load) is read after them: scalar loads
  // complete out of order, so any earlier wait on a kernel argument would
  // also wait for it.
  HeadAttn<TS, G, NR, (T > 1)> ha;
  ha.prefetch(qkv + (size_t)t * M, kh, vh, q_norm, k_norm, rope_cur + t * kD, j, Q, KV, cap, 0, sid, sl);
  ha.prefetch_prev(qkv, rope_cur, j, Q, KV, sl);   // (unused by row 0; no branch around loads)
  // the residual rows (carried by the partial of KV head 0): lane r holds
  // row r, or with the register operand path below lane l holds row l / 8
  constexpr bool kRegs = G == 2 && R == 8 &&
                        (std::is_same<TW, float>::value || std::is_same<TW, bf16w>::value ||
                         std::is_same<TW, __half>::value);   // 4 values per lane vector
  float xb[T];
#pragma unroll
  for (int r = 0; r < T; ++r) {
    if constexpr (kRegs)
      xb[r] = j == 0 ? Store<TS>::to_f(x_res[(size_t)r * H + min(row0 + (lane >> 3), H - 1)]) : 0.f;
    else
      xb[r] = j == 0 ? rows_prefetch<TS, R>(x_res + (size_t)r * H, row0, H) : 0.f;
  }
  __builtin_amdgcn_sched_barrier(0);   // attention operands before the weights
  WoSlice<TW, G, R> w;
  w.load(Wo, Q, j * G * kD, row0, H);
  __builtin_amdgcn_sched_barrier(0);   // all loads issued in this order first
  const int pos0 = ctrl[kCtrlPos];
  SoftState<G> st;
  ha.run(kh, vh, pos0 + t, 0, pos0, t > 0, true, row_block_of_block(n_kv) == 0, eps, sid, sl, st);
  if constexpr (kRegs) {
    // the wave's four key-rows merged in registers, then the waves of the
    // row through LDS (one barrier)
    __shared__ WaveStates<G, T, WPR> sw;
    st.template combine_xor<16>();
    st.template combine_xor<32>();
    sw.put(st, t, wave % WPR, lane);
    __syncthreads();
    // FP32, packed FP32 and FP16 slices: lane l's W_o columns (4l .. 4l+3 of the head's 256) are
    // dims 64 hi + 4 sl .. +3 of query head l / 32, hi = l / 16 % 2, sl = l % 16; every wave
    // applies its rows to each query row (two-token steps: the weights loaded once)
#pragma unroll
    for (int r = 0; r < T; ++r) {
      const f4_t o = sw.get4(r, lane >> 5, (lane >> 4) & 1, lane & 15);
      float o4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = Store<TS>::to_f(Store<TS>::from_f(o[i]));   // o rounded as stored
      w.apply_regs8(o4, row0, H, xb[r], opart + (size_t)r * part_row + (size_t)j * H);
    }
  } else {
    // int4 slices and the other shapes: every key-row's state through LDS,
    // one output dim per thread (measured faster for int4 than the register
    // merge with four columns per lane or with a second pass for the LDS
    // operand)
    __shared__ RowMerge<G, NR> sm[T];
    __shared__ float s_o[T][G * kD];
    sm[t].put(st, sid, sl);
    __syncthreads();
    for (int e = threadIdx.x; e < T * G * kD; e += kBlock) {
      const int r = e / (G * kD), f = e - r * G * kD;
      const int g = f / kD, d = f - g * kD;
      float mx, L, A;
      sm[r].get(g, d, mx, L, A);
      s_o[r][f] = Store<TS>::to_f(Store<TS>::from_f(A / L));   // o rounded as stored
    }
    __syncthreads();
    wo_apply<TW, G, R, T>(w, s_o, row0, H, xb, opart, part_row, j);
  }
}

// Merge of the split-K partial states of one query head of row t (one
// block of 256 threads per head and row): the split maxima and sums are
// loaded in parallel, the per-split weights exp2(m_s - max) are kept in LDS,
// and each output dim sums its weighted partials with the loads of two
// halves of the splits in flight.  A separate launch, because a
// last-arriving-block merge needs a device-scope fence per block, and on
// this multi-XCD part each such fence writes back the issuing XCD's L2.
constexpr int kMaxSplits = 128;

template <typename TS, int G>
__global__ __launch_bounds__(kBlock) void k_attn_merge(const float* __restrict__ part,
                                                       const int32_t* __restrict__ ctrl, int n_kv, int splits,
                                                       int chunk, TS* __restrict__ o) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[kWavesPerBlock];
  __shared__ float s_a[2][kD];
  const int h = blockIdx.x, j = h / G, g = h - j * G, t = blockIdx.y, tid = threadIdx.x;
  const int n_keys = ctrl[kCtrlPos] + t + 1;
  const int n_splits = ceil_div(n_keys, chunk);
  if (n_splits == 1) return;   // the attention block wrote o itself
  const float* hp = part + (((size_t)t * n_kv + j) * splits * G + g) * kPartStride;
  const size_t sstride = (size_t)G * kPartStride;
  // split statistics: thread sp < n_splits (n_splits <= kMaxSplits)
  const float m_s = tid < n_splits ? hp[tid * sstride] : -INFINITY;
  const float l_s = tid < n_splits ? hp[tid * sstride + 1] : 0.f;
  float mx = wave_max(m_s);
  if (lane_id() == 0) s_red[wave_id()] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float w = tid < n_splits ? exp2f(m_s - mx) : 0.f;
  if (tid < kMaxSplits) s_w[tid] = w;
  float L = wave_sum(l_s * w);
  __syncthreads();
  if (lane_id() == 0) s_red[wave_id()] = L;
  __syncthreads();
  L = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  // weighted partial outputs: thread (half, d) sums splits half, half+2, ...
  const int d = tid & (kD - 1), half = tid >> 7;
  float A = 0.f;
#pragma unroll 8
  for (int sp = half; sp < n_splits; sp += 2) A = fmaf(s_w[sp], hp[sp * sstride + kPartAcc + d], A);
  s_a[half][d] = A;
  __syncthreads();
  if (tid < kD) o[((size_t)t * n_kv * G + h) * kD + tid] = Store<TS>::from_f((s_a[0][tid] + s_a[1][tid]) / L);
}

// Longer contexts: the split-K merge fused with the output projection.
// Block (b, j) merges KV head j's split states (all its T*G query vectors)
// into o_j in LDS, then multiplies its 4R rows of W_o restricted to head j's
// columns, writing the same per-KV-head partials as the fused short-context
// launch:
//   part[t][j][m] = W_o[m, cols of head j] . o_j(row t)  (+ x[t][m] for j = 0).
// Each of the 32 blocks of a head reads the head's states (a few KiB per
// split, from L2).  Vector loads return in issue order, so the split maxima
// and sums and the first kMergeBatch splits' accumulators of every wave are
// issued before the W_o rows (their latency overlaps the weight stream);
// the loads cover the launch's split count (a kernel argument), clamped,
// and splits past a row's context are dropped by selection, never by a
// multiply (stale memory may hold Inf or NaN).  Wave w sums splits w, w+4,
// ... for every float4 of o_j with the weights exp2(m_s - max); the four
// wave sums are added in LDS in wave order and divided by the weighted sum.
constexpr int kMergeBatch = 16;   // accumulator loads in flight per lane and float4

template <typename TS, typename TW, int G, int R, int T>
__global__ __launch_bounds__(kBlock) void k_merge_o(const float* __restrict__ part, const int32_t* __restrict__ ctrl,
                                                    int n_q, int n_kv, int splits, int chunk,
                                                    const TW* __restrict__ Wo, const TS* __restrict__ x_res, int H,
                                                    float* __restrict__ opart, int part_row) {
  constexpr int TG = T * G;               // query vectors of the head
  constexpr int NE = TG * kD / 4;         // float4 groups of o_j
  constexpr int PL = ceil_div(NE, kWave); // per lane
  constexpr int NST = ceil_div(TG * kMaxSplits, kBlock);   // stat entries per thread
  __shared__ float s_w[TG][kMaxSplits];   // split maxima, then merge weights
  __shared__ float s_l[TG][kMaxSplits];
  __shared__ float s_inv[TG];
  __shared__ f4_t s_acc[kWavesPerBlock][PL * kWave];
  __shared__ float s_o[T][G * kD];
  const int j = kv_head_of_block(n_kv);
  const int lane = lane_id(), wave = wave_id(), tid = threadIdx.x;
  const int row0 = (row_block_of_block(n_kv) * kWavesPerBlock + wave) * R;
  const int Q = n_q * kD;
  const float* hp = part + (size_t)j * splits * G * kPartStride;   // row t adds t * trow
  const size_t trow = (size_t)n_kv * splits * G * kPartStride;
  const size_t sstride = (size_t)G * kPartStride;                  // between splits

  // 1. split statistics (entry e = tg * kMaxSplits + sp), clamped to the launch's splits
  float mv[NST], lv[NST];
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int e = min(tid + kBlock * i, TG * kMaxSplits - 1);
    const int tg = e / kMaxSplits, sp = min(e - tg * kMaxSplits, splits - 1), t = tg / G, g = tg - t * G;
    const float* st = hp + t * trow + (size_t)sp * sstride + (size_t)g * kPartStride;
    mv[i] = st[0];
    lv[i] = st[1];
  }
  // 2. the first batch of accumulators: lane float4 e = lane + 64k of o_j
  // (vector e / 32, dims 4(e % 32)), splits wave + 4b for b < kMergeBatch
  const float* ep[PL];
#pragma unroll
  for (int k = 0; k < PL; ++k) {
    const int e = min(lane + kWave * k, NE - 1);
    const int tg = e / (kD / 4), d4 = e - tg * (kD / 4), t = tg / G, g = tg - t * G;
    ep[k] = hp + t * trow + (size_t)g * kPartStride + kPartAcc + 4 * d4;
  }
  f4_t av[PL][kMergeBatch];
#pragma unroll
  for (int k = 0; k < PL; ++k)
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b)
      av[k][b] = *reinterpret_cast<const f4_t*>(ep[k] + (size_t)min(wave + kWavesPerBlock * b, splits - 1) * sstride);
  // 3. the residual rows and the W_o rows, then the position.  With FP32
  // (or packed) slices of one query row, lane l's W_o columns are exactly
  // o_j's float4 e = l, so each wave finishes o_j in registers and lane l
  // holds row l / 8's residual for the eight-row butterfly; else lane r holds
  // row r.
  constexpr bool kRegs = T == 1 && G == 2 && R == 8 &&
                        (std::is_same<TW, float>::value || std::is_same<TW, bf16w>::value ||
                         std::is_same<TW, __half>::value);
  float xb[T];
#pragma unroll
  for (int r = 0; r < T; ++r) {
    if constexpr (kRegs)
      xb[r] = j == 0 ? Store<TS>::to_f(x_res[min(row0 + (lane >> 3), H - 1)]) : 0.f;
    else
      xb[r] = j == 0 ? rows_prefetch<TS, R>(x_res + (size_t)r * H, row0, H) : 0.f;
  }
  __builtin_amdgcn_sched_barrier(0);
  WoSlice<TW, G, R> w;
  w.load(Wo, Q, j * G * kD, row0, H);
  __builtin_amdgcn_sched_barrier(0);
  const int pos0 = ctrl[kCtrlPos];

  // weights: per query vector the maximum over its splits, exp2(m_s - max), 1 / sum
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int e = tid + kBlock * i;
    if (e < TG * kMaxSplits) {
      const int tg = e / kMaxSplits, sp = e - tg * kMaxSplits, t = tg / G;
      const bool in = sp < ceil_div(pos0 + t + 1, chunk);
      s_w[tg][sp] = in ? mv[i] : -INFINITY;
      s_l[tg][sp] = in ? lv[i] : 0.f;
    }
  }
  __syncthreads();
  for (int tg = wave; tg < TG; tg += kWavesPerBlock) {
    float mx = -INFINITY;
    for (int sp = lane; sp < kMaxSplits; sp += kWave) mx = fmaxf(mx, s_w[tg][sp]);
    mx = wave_max(mx);
    float L = 0.f;
    for (int sp = lane; sp < kMaxSplits; sp += kWave) {
      const float wgt = s_w[tg][sp] == -INFINITY ? 0.f : exp2f(s_w[tg][sp] - mx);
      L = fmaf(s_l[tg][sp], wgt, L);
      s_w[tg][sp] = wgt;
    }
    L = wave_sum(L);
    if (lane == 0) s_inv[tg] = 1.0f / L;
  }
  __syncthreads();
  // weighted sums, batch by batch (later batches only for very long contexts)
  f4_t acc[PL];
#pragma unroll
  for (int k = 0; k < PL; ++k) acc[k] = f4_t{0.f, 0.f, 0.f, 0.f};
  for (int base = 0;; base += kMergeBatch * kWavesPerBlock) {
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      const int tg = min(lane + kWave * k, NE - 1) / (kD / 4);
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b) {
        const int sp = base + wave + kWavesPerBlock * b;
        const float wgt = sp < kMaxSplits ? s_w[tg][sp] : 0.f;   // 0 past the row's context
        acc[k] += wgt == 0.f ? f4_t{0.f, 0.f, 0.f, 0.f} : wgt * av[k][b];
      }
    }
    const int next = base + kMergeBatch * kWavesPerBlock;
    if (next >= splits) break;   // uniform: launch argument
#pragma unroll
    for (int k = 0; k < PL; ++k)
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b)
        av[k][b] = *reinterpret_cast<const f4_t*>(
            ep[k] + (size_t)min(next + wave + kWavesPerBlock * b, splits - 1) * sstride);
  }
#pragma unroll
  for (int k = 0; k < PL; ++k) s_acc[wave][lane + kWave * k] = acc[k];
  __syncthreads();
  if constexpr (kRegs) {
    static_assert(NE == kWave, "one float4 of o_j per lane");
    const f4_t a = ((s_acc[0][lane] + s_acc[1][lane]) + (s_acc[2][lane] + s_acc[3][lane])) * s_inv[lane / (kD / 4)];
    float o4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o4[i] = Store<TS>::to_f(Store<TS>::from_f(a[i]));
    w.apply_regs8(o4, row0, H, xb[0], opart + (size_t)j * H);
  } else {
    for (int e = tid; e < NE; e += kBlock) {
      const int tg = e / (kD / 4), d4 = e - tg * (kD / 4), t = tg / G, g = tg - t * G;
      const f4_t a = ((s_acc[0][e] + s_acc[1][e]) + (s_acc[2][e] + s_acc[3][e])) * s_inv[tg];
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[t][g * kD + 4 * d4 + i] = Store<TS>::to_f(Store<TS>::from_f(a[i]));
    }
    __syncthreads();
    wo_apply<TW, G, R, T>(w, s_o, row0, H, xb, opart, part_row, j);
  }
}

// --------------------------------------------------------------- dispatch
int blocks_for(int M, int R, int grid) {
  const int one_shot = ceil_div(ceil_div(M, R), kWavesPerBlock);
  return (grid > 0 && grid < one_shot) ? grid : one_shot;
}

// Head blocks: one row group per wave unless fewer are asked for, at most
// kHeadMaxBlocks, rounded up to an even count (the argmax reads key pairs).
int head_grid(int V, int R, int waves, int grid) {
  const int one_shot = ceil_div(ceil_div(V, R), waves);
  int b = (grid > 0 && grid < one_shot) ? grid : one_shot;
  b = b < kHeadMaxBlocks ? b : kHeadMaxBlocks;
  return (b + 1) & ~1;
}

// K values compiled in; a K must also be a multiple of 64 lane vectors of
// the weight storage (256 floats, 512 halves, 1024 int4 weights).
template <int V> using IC = std::integral_constant<int, V>;

template <typename TW, int K, typename F>
bool call_k(F& f) {
  if constexpr (K % (kWave * WVec<TW>::type::N) == 0) return f(IC<K>{});
  else return false;
}
template <typename TW, typename F>
bool with_k(int K, F&& f) {
  switch (K) {
    case 256: return call_k<TW, 256>(f);
    case 512: return call_k<TW, 512>(f);
    case 1024: return call_k<TW, 1024>(f);
    case 2048: return call_k<TW, 2048>(f);
    case 3072: return call_k<TW, 3072>(f);
    default: return false;
  }
}
template <typename F>
bool with_t(int T, F&& f) {
  switch (T) {
    case 1: return f(IC<1>{});
    case 2: return f(IC<2>{});
    default: return false;
  }
}
template <typename F>
bool with_r(int R, F&& f) {
  switch (R) {
    case 1: return f(IC<1>{});
    case 2: return f(IC<2>{});
    case 4: return f(IC<4>{});
    default: return false;
  }
}

// Weight storage of one matrix: int4 (FP16 models with int4 weights), its
// lossless packed copy when there is one (FP32 models only), else the
// storage type itself.  f receives the typed pointer.  Launches without an
// int4 kernel pass Q4 = false (the caller never selects them for int4
// weights).
template <typename TS, bool Q4 = true, typename F>
bool with_w(int wfmt, const void* w, const void* packed, F&& f) {
  if (wfmt == kWeightsQ4) {
    if constexpr (Q4 && std::is_same<TS, __half>::value) return f(static_cast<const q4w*>(w));
    else return false;
  }
  if constexpr (std::is_same<TS, float>::value)
    if (packed) return f(static_cast<const bf16w*>(packed));
  return f(static_cast<const TS*>(w));
}
template <typename P> using pointee_t = typename std::remove_cv<typename std::remove_pointer<P>::type>::type;
// The lossless packed copy applies to FP32 storage only.
template <typename TS> const void* TS_packed(const void* p) { return std::is_same<TS, float>::value ? p : nullptr; }

template <typename TS>
bool qkv_t(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool first, int npd, hipStream_t s) {
  const int M = (a.n_q + 2 * a.n_kv) * a.head_dim;
  const int grid = blocks_for(M, sh.rows_qkv, sh.grid_qkv);
  return with_w<TS>(a.wfmt, L.wqkv, L.wqkv_p, [&](auto W) {
    return with_k<pointee_t<decltype(W)>>(a.hidden, [&](auto kc) {
      return with_r(sh.rows_qkv, [&](auto rc) {
        return with_t(sh.tokens, [&](auto tc) {
          auto go = [&](auto nc) {
            hipLaunchKernelGGL((k_qkv<TS, pointee_t<decltype(W)>, decltype(kc)::value, decltype(rc)::value,
                                      decltype(tc)::value, decltype(nc)::value>),
                               dim3(grid), dim3(kBlock), 0, s, W, (TS*)a.x, (const TS*)L.in_norm,
                               (const float*)a.dpart, M, first ? 1 : 0, (TS*)a.qkv, a.eps, a.vocab, a.embed, a.ids,
                               a.ctrl, a.rope_cos, a.rope_sin, a.rope_cur);
            return true;
          };
          switch (first ? 0 : npd) {
            case 0: return go(IC<0>{});
            case 2: return go(IC<2>{});
            case 4: return go(IC<4>{});
            default: return false;
          }
        });
      });
    });
  });
}

// The down projection split over K into S FP32 slices (dense weights; the
// slice width must hold whole lane vectors).
template <typename TS>
bool down_split_t(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, int S, hipStream_t s) {
  if (a.wfmt != kWeightsDense) return false;
  const int grid = blocks_for(a.hidden, sh.rows_down, 0);
  return with_w<TS, false>(a.wfmt, L.wd, TS_packed<TS>(L.wd_p), [&](auto W) {
    using TW = pointee_t<decltype(W)>;
    return with_k<TW>(a.inter, [&](auto kc) {
      return with_t(sh.tokens, [&](auto tc) {
        constexpr int K = decltype(kc)::value, T = decltype(tc)::value;
        auto go = [&](auto sc, auto rc) {
          constexpr int SS = decltype(sc)::value, R = decltype(rc)::value;
          if constexpr (K % SS == 0 && (K / SS) % (kWave * WVec<TW>::type::N) == 0) {
            hipLaunchKernelGGL((k_down_split<TS, TW, K, SS, R, T>), dim3(grid, SS), dim3(kBlock), 0, s, W,
                               (const TS*)a.act, (const TS*)a.x2, a.dpart, a.hidden);
            return true;
          } else {
            return false;
          }
        };
        auto with_s = [&](auto rc) {
          switch (S) {
            case 2: return go(IC<2>{}, rc);
            case 4: return go(IC<4>{}, rc);
            default: return false;
          }
        };
        switch (sh.rows_down) {
          case 1: return with_s(IC<1>{});
          case 2: return with_s(IC<2>{});
          default: return false;
        }
      });
    });
  });
}

template <typename TS>
bool residual_t(const DecodeArgs& a, int T, int K, int R, int grid_req, const void* W, const void* Wp,
                const void* in, const void* x_in, void* x_out, bool adv, hipStream_t s) {
  const int grid = blocks_for(a.hidden, R, grid_req);
  return with_w<TS>(a.wfmt, W, Wp, [&](auto Wt) {
    return with_k<pointee_t<decltype(Wt)>>(K, [&](auto kc) {
      return with_r(R, [&](auto rc) {
        return with_t(T, [&](auto tc) {
          hipLaunchKernelGGL((k_gemv_residual<TS, pointee_t<decltype(Wt)>, decltype(kc)::value, decltype(rc)::value,
                                              decltype(tc)::value>),
                             dim3(grid), dim3(kBlock), 0, s, Wt, (const TS*)in, (const TS*)x_in, (TS*)x_out,
                             a.hidden, a.ctrl, adv ? 1 : 0);
          return true;
        });
      });
    });
  });
}

// Partial slots per row the gate/up prologue sums for a model at T rows:
// the KV head count rounded up to 2, 4 or 8 (the extra slots stay zero),
// or 0 when the partials would not fit its registers.
int parts_slots(int hidden, int n_kv, int T) {
  for (int np : {2, 4, 8})
    if (n_kv <= np) return T * ceil_div(hidden, 4 * kBlock) * np <= kMaxPartVec ? np : 0;
  return 0;
}

template <typename TS>
bool gateup_t(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool from_parts, hipStream_t s) {
  const int grid = blocks_for(a.inter, sh.rows_gu, sh.grid_gu);
  const int np = from_parts ? parts_slots(a.hidden, a.n_kv, sh.tokens) : 0;
  if (from_parts && np == 0) return false;
  return with_w<TS>(a.wfmt, L.wgu, L.wgu_p, [&](auto W) {
    using TW = pointee_t<decltype(W)>;
    return with_k<TW>(a.hidden, [&](auto kc) {
      return with_r(sh.rows_gu, [&](auto rc) {
        return with_t(sh.tokens, [&](auto tc) {
          constexpr int K = decltype(kc)::value, R = decltype(rc)::value, T = decltype(tc)::value;
          auto go = [&](auto npc) {
            constexpr int NP = decltype(npc)::value;
            if constexpr (T * NP * ceil_div(K, 4 * kBlock) <= kMaxPartVec) {
              hipLaunchKernelGGL((k_gateup<TS, TW, K, R, NP, T>), dim3(grid), dim3(kBlock), 0, s, W,
                                 (const TS*)L.post_norm, (const TS*)a.x2, a.opart, a.eps, (TS*)a.act, a.inter,
                                 (TS*)a.x2);
              return true;
            } else {
              return false;
            }
          };
          switch (np) {
            case 0: return go(IC<0>{});
            case 2: return go(IC<2>{});
            case 4: return go(IC<4>{});
            case 8: return go(IC<8>{});
            default: return false;
          }
        });
      });
    });
  });
}

template <typename TS>
bool head_t(const DecodeArgs& a, const DecodeShape& sh, hipStream_t s) {
  const int grid = head_grid(a.vocab, sh.rows_head, sh.head_waves, sh.grid_head);
  return with_w<TS>(a.wfmt, a.embed, a.embed_p, [&](auto E) {
    using TW = pointee_t<decltype(E)>;
    return with_k<TW>(a.hidden, [&](auto kc) {
      return with_r(sh.rows_head, [&](auto rc) {
        return with_t(sh.tokens, [&](auto tc) {
          constexpr int K = decltype(kc)::value, R = decltype(rc)::value, T = decltype(tc)::value;
          auto go = [&](auto wc) {
            constexpr int WPB = decltype(wc)::value;
            hipLaunchKernelGGL((k_head<TS, TW, K, R, WPB, T>), dim3(grid), dim3(WPB * kWave), 0, s, E,
                               (const TS*)a.final_norm, (const TS*)a.x, a.eps, (TS*)a.logits, a.vocab, a.am_part);
            return true;
          };
          switch (sh.head_waves) {
            case 4: return go(IC<4>{});
            case 8: return go(IC<8>{});
            case 16: return go(IC<16>{});
            default: return false;
          }
        });
      });
    });
  });
}

// The layouts the attention launches derive their other addresses from
// (their arguments hold rope_cur, the K block and the Q-norm gain only).
template <typename TS>
bool attn_layout_ok(const DecodeArgs& a, const LayerPtrs& L) {
  const char* rb = reinterpret_cast<const char*>(a.rope_cur);
  return a.n_kv <= 0xFF && a.hidden < (1 << 23) && static_cast<const char*>(a.x) == rb + row_block_x_offset() &&
         static_cast<const char*>(a.qkv) == rb + row_block_qkv_offset(a.hidden, sizeof(TS)) &&
         static_cast<const char*>(L.v_cache) ==
             static_cast<const char*>(L.k_cache) + (size_t)a.n_kv * a.cap * kD * sizeof(TS) &&
         static_cast<const char*>(L.k_norm) == static_cast<const char*>(L.q_norm) + kD * sizeof(TS);
}

template <typename TS>
bool attn_t(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool direct, hipStream_t s) {
  if (!attn_layout_ok<TS>(a, L)) return false;
  const int G = a.n_q / a.n_kv;
  const dim3 grid(sh.attn_splits, a.n_kv, sh.tokens);
  auto go = [&](auto gc) {
    return with_t(sh.tokens, [&](auto tc) {
      hipLaunchKernelGGL((k_attn<TS, decltype(gc)::value, decltype(tc)::value>), grid, dim3(kBlock), 0, s,
                         a.rope_cur, (TS*)L.k_cache, (const TS*)L.q_norm, a.ctrl, a.n_kv | (a.hidden << 8), a.cap,
                         sh.attn_chunk, a.eps, direct ? 1 : 0, a.attn_part, (TS*)a.o);
      return true;
    });
  };
  switch (G) {
    case 1: return go(IC<1>{});
    case 2: return go(IC<2>{});
    case 4: return go(IC<4>{});
    default: return false;
  }
}

template <typename TS>
bool attn_merge_t(const DecodeArgs& a, const DecodeShape& sh, hipStream_t s) {
  const int G = a.n_q / a.n_kv;
  auto go = [&](auto gc) {
    hipLaunchKernelGGL((k_attn_merge<TS, decltype(gc)::value>), dim3(a.n_q, sh.tokens), dim3(kBlock), 0, s,
                       a.attn_part, a.ctrl, a.n_kv, sh.attn_splits, sh.attn_chunk, (TS*)a.o);
    return true;
  };
  switch (G) {
    case 1: return go(IC<1>{});
    case 2: return go(IC<2>{});
    case 4: return go(IC<4>{});
    default: return false;
  }
}

template <typename TS>
bool attn_o_t(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, hipStream_t s) {
  const int G = a.n_q / a.n_kv;
  if (!attn_layout_ok<TS>(a, L)) return false;
  return with_w<TS>(a.wfmt, L.wo, L.wo_p, [&](auto Wo) {
    using TW = pointee_t<decltype(Wo)>;
    // row t's partials start at opart[t * slots * H], as the gate/up
    // prologue reads them
    const int part_row = parts_slots(a.hidden, a.n_kv, sh.tokens) * a.hidden;
    if (part_row == 0) return false;
    auto go = [&](auto gc, auto rc) {
      constexpr int R = decltype(rc)::value, GG = decltype(gc)::value;
      // an int4 slice needs whole 8-byte loads per lane (not G = 1 with 4 rows)
      if constexpr (std::is_same<TW, q4w>::value && (R * GG * kD / 16) % kWave != 0) {
        return false;
      } else {
        const dim3 grid(ceil_div(a.hidden, kWavesPerBlock * R) * a.n_kv);   // KV head = block % n_kv
        return with_t(sh.tokens, [&](auto tc) {
          hipLaunchKernelGGL((k_attn_o<TS, TW, GG, R, decltype(tc)::value>), grid, dim3(kBlock), 0, s,
                             a.rope_cur, (TS*)L.k_cache, (const TS*)L.q_norm, a.ctrl, Wo,
                             a.n_kv | (a.hidden << 8), a.cap, a.eps, part_row, a.opart);
          return true;
        });
      }
    };
    auto with_g = [&](auto rc) {
      switch (G) {
        case 1: return go(IC<1>{}, rc);
        case 2: return go(IC<2>{}, rc);
        case 4: return go(IC<4>{}, rc);
        default: return false;
      }
    };
    switch (sh.rows_attn_o) {
      case 4: return with_g(IC<4>{});
      case 8: return with_g(IC<8>{});
      default: return false;
    }
  });
}

template <typename TS>
bool merge_o_t(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, hipStream_t s) {
  const int G = a.n_q / a.n_kv;
  return with_w<TS>(a.wfmt, L.wo, L.wo_p, [&](auto Wo) {
    using TW = pointee_t<decltype(Wo)>;
    const int part_row = parts_slots(a.hidden, a.n_kv, sh.tokens) * a.hidden;
    if (part_row == 0) return false;
    auto go = [&](auto gc, auto rc) {
      constexpr int R = decltype(rc)::value, GG = decltype(gc)::value;
      if constexpr (std::is_same<TW, q4w>::value && (R * GG * kD / 16) % kWave != 0) {
        return false;
      } else {
        const dim3 grid(ceil_div(a.hidden, kWavesPerBlock * R) * a.n_kv);   // KV head = block % n_kv
        return with_t(sh.tokens, [&](auto tc) {
          hipLaunchKernelGGL((k_merge_o<TS, TW, GG, R, decltype(tc)::value>), grid, dim3(kBlock), 0, s, a.attn_part,
                             a.ctrl, a.n_q, a.n_kv, sh.attn_splits, sh.attn_chunk, Wo, (const TS*)a.x, a.hidden,
                             a.opart, part_row);
          return true;
        });
      }
    };
    auto with_g = [&](auto rc) {
      switch (G) {
        case 1: return go(IC<1>{}, rc);
        case 2: return go(IC<2>{}, rc);
        case 4: return go(IC<4>{}, rc);
        default: return false;
      }
    };
    switch (sh.rows_attn_o) {
      case 4: return with_g(IC<4>{});
      case 8: return with_g(IC<8>{});
      default: return false;
    }
  });
}

}  // namespace

int attn_o_part_slots(int hidden, int n_kv, int tokens) { return parts_slots(hidden, n_kv, tokens); }

int head_blocks(const DecodeArgs& a, const DecodeShape& sh) {
  return head_grid(a.vocab, sh.rows_head, sh.head_waves, sh.grid_head);
}

bool launch_qkv(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool first, int npd, hipStream_t s) {
  return a.dtype == 0 ? qkv_t<float>(a, sh, L, first, npd, s) : qkv_t<__half>(a, sh, L, first, npd, s);
}
bool launch_down_split(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, int S, hipStream_t s) {
  return a.dtype == 0 ? down_split_t<float>(a, sh, L, S, s) : down_split_t<__half>(a, sh, L, S, s);
}
bool launch_attn(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool direct, hipStream_t s) {
  return a.dtype == 0 ? attn_t<float>(a, sh, L, direct, s) : attn_t<__half>(a, sh, L, direct, s);
}
bool launch_merge_o(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, hipStream_t s) {
  return a.dtype == 0 ? merge_o_t<float>(a, sh, L, s) : merge_o_t<__half>(a, sh, L, s);
}
bool launch_attn_merge(const DecodeArgs& a, const DecodeShape& sh, hipStream_t s) {
  return a.dtype == 0 ? attn_merge_t<float>(a, sh, s) : attn_merge_t<__half>(a, sh, s);
}
bool launch_o(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, hipStream_t s) {
  const int K = a.n_q * a.head_dim;
  return a.dtype == 0
             ? residual_t<float>(a, sh.tokens, K, sh.rows_o, sh.grid_o, L.wo, L.wo_p, a.o, a.x, a.x2, false, s)
             : residual_t<__half>(a, sh.tokens, K, sh.rows_o, sh.grid_o, L.wo, nullptr, a.o, a.x, a.x2, false, s);
}
bool launch_attn_o(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, hipStream_t s) {
  return a.dtype == 0 ? attn_o_t<float>(a, sh, L, s) : attn_o_t<__half>(a, sh, L, s);
}
bool launch_gateup(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool from_parts, hipStream_t s) {
  return a.dtype == 0 ? gateup_t<float>(a, sh, L, from_parts, s) : gateup_t<__half>(a, sh, L, from_parts, s);
}
bool launch_down(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs& L, bool adv, hipStream_t s) {
  return a.dtype == 0 ? residual_t<float>(a, sh.tokens, a.inter, sh.rows_down, sh.grid_down, L.wd, L.wd_p, a.act,
                                          a.x2, a.x, adv, s)
                      : residual_t<__half>(a, sh.tokens, a.inter, sh.rows_down, sh.grid_down, L.wd, nullptr, a.act,
                                           a.x2, a.x, adv, s);
}
bool launch_head(const DecodeArgs& a, const DecodeShape& sh, hipStream_t s) {
  return a.dtype == 0 ? head_t<float>(a, sh, s) : head_t<__half>(a, sh, s);
}
bool launch_argmax(const DecodeArgs& a, const DecodeShape& sh, hipStream_t s) {
  const int n = head_blocks(a, sh);
  const int per = ceil_div(n / 2, 1024);
  auto go = [&](auto pc) {
    return with_t(sh.tokens, [&](auto tc) {
      hipLaunchKernelGGL((k_argmax<decltype(pc)::value, decltype(tc)::value>), dim3(1), dim3(1024), 0, s,
                         (const unsigned long long*)a.am_part, n, a.ctrl, a.ids, a.mail);
      return true;
    });
  };
  if (per <= 1) return go(IC<1>{});
  if (per <= 2) return go(IC<2>{});
  if (per <= 4) return go(IC<4>{});
  if (per <= 8) return go(IC<8>{});
  if (per <= 10) return go(IC<10>{});   // the 18992-block FP32 head: 9496 pairs
  static_assert(kHeadMaxBlocks / 2048 == 20, "pairs per thread at the largest head grid");
  return go(IC<20>{});
}
bool launch_set_pos(int32_t* ctrl, int pos, hipStream_t s) {
  hipLaunchKernelGGL(k_set_pos, dim3(1), dim3(64), 0, s, ctrl, pos);
  return true;
}

}  // namespace wsg
