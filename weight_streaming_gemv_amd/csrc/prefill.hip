// Chunked prefill for gfx950: several consecutive prompt rows of one request
// per chunk, every row attending to its whole causal prefix across chunks
// (Megakernels, "Chunked prefill for long prompts").
//
// Per chunk and layer (the pages' 11 ordered stages, here 9 launches):
//   rows_norm   RMSNorm of each row (one wave per row)
//   gemm        QKV projection  [n x H] . W_qkv^T   (FP32 MFMA)
//   rows_qkv    per-head Q/K RMSNorm + RoPE; K/V written to cache rows p0..p0+n-1
//   attn        causal attention of the n rows over keys 0..p0+r (VALU, LDS tiles)
//   gemm+res    O projection, residual added in the epilogue
//   rows_norm   post-attention RMSNorm
//   gemm        gate/up projection [n x 2I]
//   rows_swiglu SwiGLU
//   gemm+res    down projection, residual added in the epilogue
// The projections are the only dense contractions and the only MFMA users.
// The chunk runs exactly n rows: the GEMM masks its ragged last row tile, so
// no padding rows exist.  Within one prefill call the last prompt row goes
// through the decode forward (the only row that reaches the head), so every
// chunk stops its last layer after the K/V write (Benchmark methodology,
// "Long-document chunked prefill": nonterminal chunks prune the final layer).
#include "common.hpp"
#include "prefill.hpp"
#include "status.hpp"

namespace wsg {

namespace {

size_t al(size_t v) { return (v + 255) & ~size_t(255); }
__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;

typedef float f16v_t __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ GEMM
// C[M x N] (+)= A[M x K] . B[N x K]^T, all row-major FP32, K-contiguous
// operands.  Block tile BM x BN x 32, 256 threads = 2 x 2 waves, each wave a
// (BM/2) x (BN/2) sub-tile of 32 x 32 MFMA tiles (v_mfma_f32_32x32x2f32).
//
// MFMA 32x32x2 operand layout (lane l): A element (row l%32, k l/32),
// B element (k l/32, col l%32); accumulator register r holds row
// 8*(r/4) + 4*(l/32) + r%4, col l%32.  The two k slots of every MFMA are
// mapped to k = h*16 + s (h = l/32, s = step 0..15) of the 32-wide K tile,
// so each lane reads 16 consecutive floats of one LDS row per tile.
constexpr int kBK = 32;
constexpr int kLdsPad = 4;                // floats of padding per LDS row
constexpr int kLdsRow = kBK + kLdsPad;

template <int BM, int BN, bool ACC>
__global__ __launch_bounds__(256) void k_gemm_nt(const float* __restrict__ A, const float* __restrict__ B,
                                                 float* __restrict__ C, int M, int N, int K) {
  constexpr int WM = BM / 2, WN = BN / 2;     // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;   // MFMA tiles per wave
  constexpr int A_LOADS = BM * kBK / 4 / 256; // float4 per thread per tile
  constexpr int B_LOADS = BN * kBK / 4 / 256;
  __shared__ float As[BM * kLdsRow];
  __shared__ float Bs[BN * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int li = lane & 31, lh = lane >> 5;

  f16v_t acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // global -> register staging: thread loads float4 #(tid + 256 i) of the
  // tile: row = idx / 8, col4 = idx % 8 (plain loops: arrays captured by a
  // lambda would be forced into scratch memory)
  f4_t ra[A_LOADS], rb[B_LOADS];   // native vectors: HIP's float4 struct arrays end up in scratch
#define WSG_GEMM_LOAD(K0)                                                                           \
  {                                                                                                \
    _Pragma("unroll") for (int i = 0; i < A_LOADS; ++i) {                                          \
      const int idx = tid + 256 * i, row = idx >> 3, c4 = idx & 7;                                 \
      const int gm = min(m0 + row, M - 1);   /* rows past M feed only unstored outputs */        \
      ra[i] = *reinterpret_cast<const f4_t*>(A + (size_t)gm * K + (K0) + 4 * c4);                  \
    }                                                                                              \
    _Pragma("unroll") for (int i = 0; i < B_LOADS; ++i) {                                          \
      const int idx = tid + 256 * i, row = idx >> 3, c4 = idx & 7;                                 \
      rb[i] = *reinterpret_cast<const f4_t*>(B + (size_t)(n0 + row) * K + (K0) + 4 * c4);          \
    }                                                                                              \
  }

  WSG_GEMM_LOAD(0)
  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();          // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, c4 = idx & 7;
      *reinterpret_cast<f4_t*>(&As[row * kLdsRow + 4 * c4]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, c4 = idx & 7;
      *reinterpret_cast<f4_t*>(&Bs[row * kLdsRow + 4 * c4]) = rb[i];
    }
    __syncthreads();
    // next tile in flight during the MFMAs (the last iteration reloads the
    // final tile, in bounds and unused, to keep the loop free of branches)
    WSG_GEMM_LOAD(min(k0 + kBK, K - kBK))
#undef WSG_GEMM_LOAD
    float af[TM][16], bf[TN][16];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f4_t v = *reinterpret_cast<const f4_t*>(&As[(wm + a * 32 + li) * kLdsRow + lh * 16 + 4 * q]);
        af[a][4 * q] = v.x; af[a][4 * q + 1] = v.y; af[a][4 * q + 2] = v.z; af[a][4 * q + 3] = v.w;
      }
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f4_t v = *reinterpret_cast<const f4_t*>(&Bs[(wn + b * 32 + li) * kLdsRow + lh * 16 + 4 * q]);
        bf[b][4 * q] = v.x; bf[b][4 * q + 1] = v.y; bf[b][4 * q + 2] = v.z; bf[b][4 * q + 3] = v.w;
      }
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a][s], bf[b][s], acc[a][b], 0, 0, 0);
  }

#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm + a * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int col = n0 + wn + b * 32 + li;
        if (row < M) {
          float* p = C + (size_t)row * N + col;
          *p = ACC ? *p + acc[a][b][r] : acc[a][b][r];
        }
      }
}

// --------------------------------------------------------------- row kernels
// X[r] = E[ids[r]] for r < n (one block of 256 threads per row).
__global__ __launch_bounds__(256) void k_rows_embed(const float* __restrict__ E, const int32_t* __restrict__ ids,
                                                    int n, int H, int V, float* __restrict__ X) {
  const int r = blockIdx.x;
  if (r >= n) return;
  int tok = ids[r];
  tok = (tok < 0 || tok >= V) ? 0 : tok;   // ids are validated on the host
  for (int c = threadIdx.x * 4; c < H; c += 256 * 4)
    *reinterpret_cast<float4*>(X + (size_t)r * H + c) = *reinterpret_cast<const float4*>(E + (size_t)tok * H + c);
}

// Y[r] = X[r] * (mean(X[r]^2) + eps)^-1/2 * g, one wave per row.
__global__ __launch_bounds__(256) void k_rows_norm(const float* __restrict__ X, const float* __restrict__ g,
                                                   int n, int H, float eps, float* __restrict__ Y) {
  const int r = blockIdx.x * 4 + wave_id();
  if (r >= n) return;
  const int lane = lane_id();
  const float* x = X + (size_t)r * H;
  float ss = 0.f;
  for (int c = lane * 4; c < H; c += 256) {
    const float4 v = *reinterpret_cast<const float4*>(x + c);
    ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
  for (int c = lane * 4; c < H; c += 256) {
    const float4 v = *reinterpret_cast<const float4*>(x + c);
    const float4 w = *reinterpret_cast<const float4*>(g + c);
    *reinterpret_cast<float4*>(Y + (size_t)r * H + c) =
        make_float4(v.x * inv * w.x, v.y * inv * w.y, v.z * inv * w.z, v.w * inv * w.w);
  }
}

// Per (row, head) wave: Q heads normalised + rotated in place; K heads
// normalised + rotated into the K cache at position p0 + r; V heads copied
// into the V cache.  Lane l holds dims l and l + 64 (one rotary pair).
__global__ __launch_bounds__(256) void k_rows_qkv(float* __restrict__ QKV, int n, int n_q, int n_kv, int p0,
                                                  int cap, float eps, const float* __restrict__ q_norm,
                                                  const float* __restrict__ k_norm, const float* __restrict__ rope_cos,
                                                  const float* __restrict__ rope_sin, float* __restrict__ k_cache,
                                                  float* __restrict__ v_cache) {
  const int r = blockIdx.y;
  const int hh = blockIdx.x * 4 + wave_id();
  if (r >= n || hh >= n_q + 2 * n_kv) return;
  const int lane = lane_id();
  const int width = (n_q + 2 * n_kv) * kD;
  float* row = QKV + (size_t)r * width;
  const int pos = p0 + r;
  if (hh >= n_q + n_kv) {   // V head: copy
    const int j = hh - n_q - n_kv;
    const float* v = row + (n_q + n_kv) * kD + j * kD;
    float* dst = v_cache + ((size_t)j * cap + pos) * kD;
    dst[lane] = v[lane];
    dst[lane + 64] = v[lane + 64];
    return;
  }
  float* h = row + hh * kD;
  float lo = h[lane], hi = h[lane + 64];
  float ss = wave_sum(fmaf(lo, lo, hi * hi));
  const float inv = 1.0f / sqrtf(ss / (float)kD + eps);
  const float* g = hh < n_q ? q_norm : k_norm;
  lo = lo * inv * g[lane];
  hi = hi * inv * g[lane + 64];
  const float c = rope_cos[(size_t)pos * (kD / 2) + lane], s = rope_sin[(size_t)pos * (kD / 2) + lane];
  const float o_lo = lo * c - hi * s, o_hi = hi * c + lo * s;
  if (hh < n_q) {
    h[lane] = o_lo;
    h[lane + 64] = o_hi;
  } else {
    float* dst = k_cache + ((size_t)(hh - n_q) * cap + pos) * kD;
    dst[lane] = o_lo;
    dst[lane + 64] = o_hi;
  }
}

// ACT[r][i] = silu(GU[r][i]) * GU[r][I + i]
__global__ __launch_bounds__(256) void k_rows_swiglu(const float* __restrict__ GU, int n, int I,
                                                     float* __restrict__ ACT) {
  const size_t total = (size_t)n * I;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const size_t r = e / I, i = e - r * I;
    const float g = GU[r * 2 * I + i], u = GU[r * 2 * I + I + i];
    ACT[e] = g / (1.0f + expf(-g)) * u;
  }
}

// ------------------------------------------------------------ attention
// Causal attention of chunk rows [0, n) (positions p0 + r) over cached keys
// 0..p0+r of KV head j, for its G query heads.  Block = 16 rows x G heads
// of queries and one KV head; keys stream through LDS in tiles of 32.  The
// query tile shares every K/V tile across its rows (Megakernels, "Chunked
// prefill for long prompts": query-tiled prefill attention), with an
// online softmax per query in the log2 domain.  Thread t owns query t/8 of
// the tile and, for scores, keys t%8 + 8i (i < 4); for the output, dims
// [16 (t%8), 16 (t%8) + 16) of its query.
constexpr int kQR = 16;            // query rows per block
constexpr int kKT = 32;            // keys per tile
constexpr int kRowPad = kD + 4;

template <int G>
__global__ __launch_bounds__(256) void k_prefill_attn(const float* __restrict__ QKV, const float* __restrict__ k_cache,
                                                      const float* __restrict__ v_cache, int n, int n_q, int n_kv,
                                                      int p0, int cap, float* __restrict__ O) {
  constexpr int NQ = kQR * G;       // query vectors per block (32 for G = 2)
  static_assert(NQ * 8 == 256 || NQ * 8 < 256, "one group of 8 threads per query");
  __shared__ float Qs[NQ][kRowPad];
  __shared__ float Ks[kKT][kRowPad];
  __shared__ float Vs[kKT][kRowPad];
  __shared__ float Ps[NQ][kKT + 1];

  const int j = blockIdx.y;
  const int r0 = blockIdx.x * kQR;
  const int tid = threadIdx.x;
  const int width = (n_q + 2 * n_kv) * kD;
  const float qscale = kLog2e / sqrtf((float)kD);

  // stage queries: vector qv = rr * G + g  <->  row r0 + rr, head j*G + g
  for (int e = tid; e < NQ * kD; e += 256) {
    const int qv = e / kD, d = e - qv * kD;
    const int rr = qv / G, g = qv - rr * G;
    const int r = r0 + rr;
    Qs[qv][d] = r < n ? QKV[(size_t)r * width + (j * G + g) * kD + d] * qscale : 0.f;
  }
  const int qv = tid >> 3, sub = tid & 7;
  const bool active = qv < NQ;
  const int rr = qv / G;
  const int my_pos = p0 + r0 + rr;                       // this query's position
  const int last_row = min(n, r0 + kQR) - 1;
  const int n_keys = p0 + last_row + 1;                  // keys any row of the tile needs

  float m = -INFINITY, l = 0.f, acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  const float* kh = k_cache + (size_t)j * cap * kD;
  const float* vh = v_cache + (size_t)j * cap * kD;
  for (int k0 = 0; k0 < n_keys; k0 += kKT) {
    __syncthreads();   // previous tile consumed (and queries staged)
    for (int e = tid * 4; e < kKT * kD; e += 256 * 4) {
      const int kk = e / kD, d = e - kk * kD;
      const int key = k0 + kk;
      float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f), vv4 = kv4;
      if (key < n_keys) {
        kv4 = *reinterpret_cast<const float4*>(kh + (size_t)key * kD + d);
        vv4 = *reinterpret_cast<const float4*>(vh + (size_t)key * kD + d);
      }
      *reinterpret_cast<float4*>(&Ks[kk][d]) = kv4;
      *reinterpret_cast<float4*>(&Vs[kk][d]) = vv4;
    }
    __syncthreads();
    // scores of this thread's query against keys sub + 8i
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = 0.f;
    if (active) {
      for (int d = 0; d < kD; d += 4) {
        const float4 q4 = *reinterpret_cast<const float4*>(&Qs[qv][d]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 k4 = *reinterpret_cast<const float4*>(&Ks[sub + 8 * i][d]);
          s[i] = fmaf(q4.x, k4.x, fmaf(q4.y, k4.y, fmaf(q4.z, k4.z, fmaf(q4.w, k4.w, s[i]))));
        }
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = k0 + sub + 8 * i;
      if (!(active && key <= my_pos)) s[i] = -INFINITY;   // causal mask (and keys past the tile's end)
      tmax = fmaxf(tmax, s[i]);
    }
    // max over the 8 threads of this query (lanes 8q..8q+7 of one wave)
    tmax = fmaxf(tmax, __shfl_xor(tmax, 1));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 2));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 4));
    const float mn = fmaxf(m, tmax);
    // a query with no key yet in this tile keeps m = -inf: guard the rescale
    const float alpha = mn == -INFINITY ? 1.f : exp2f(m - mn);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = mn == -INFINITY ? 0.f : exp2f(s[i] - mn);
      psum += p;
      if (active) Ps[qv][sub + 8 * i] = p;
    }
    psum += __shfl_xor(psum, 1);
    psum += __shfl_xor(psum, 2);
    psum += __shfl_xor(psum, 4);
    l = l * alpha + psum;
    m = mn;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] *= alpha;
    __syncthreads();
    if (active) {
      for (int kk = 0; kk < kKT; ++kk) {
        const float p = Ps[qv][kk];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v4 = *reinterpret_cast<const float4*>(&Vs[kk][16 * sub + 4 * q4]);
          acc[4 * q4] = fmaf(p, v4.x, acc[4 * q4]);
          acc[4 * q4 + 1] = fmaf(p, v4.y, acc[4 * q4 + 1]);
          acc[4 * q4 + 2] = fmaf(p, v4.z, acc[4 * q4 + 2]);
          acc[4 * q4 + 3] = fmaf(p, v4.w, acc[4 * q4 + 3]);
        }
      }
    }
  }
  if (active) {
    const int r = r0 + rr, g = qv - rr * G;
    if (r < n) {
      const float inv = 1.0f / l;
      float* o = O + (size_t)r * n_q * kD + (j * G + g) * kD + 16 * sub;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(o + 4 * q4) =
            make_float4(acc[4 * q4] * inv, acc[4 * q4 + 1] * inv, acc[4 * q4 + 2] * inv, acc[4 * q4 + 3] * inv);
    }
  }
}

// ------------------------------------------------------------ launchers
// Tile choice: the largest tile that still gives >= 256 blocks.
bool launch_gemm(const float* A, const float* B, float* C, int M, int N, int K, bool acc, hipStream_t s) {
  if (M < 1 || N % 64 != 0 || K % kBK != 0) return false;
  const bool big = (N % 128 == 0) && (int64_t)(N / 128) * cdiv(M, 128) >= 256;
  if (big) {
    const dim3 grid(N / 128, cdiv(M, 128));
    if (acc) hipLaunchKernelGGL((k_gemm_nt<128, 128, true>), grid, dim3(256), 0, s, A, B, C, M, N, K);
    else hipLaunchKernelGGL((k_gemm_nt<128, 128, false>), grid, dim3(256), 0, s, A, B, C, M, N, K);
  } else {
    const dim3 grid(N / 64, cdiv(M, 64));
    if (acc) hipLaunchKernelGGL((k_gemm_nt<64, 64, true>), grid, dim3(256), 0, s, A, B, C, M, N, K);
    else hipLaunchKernelGGL((k_gemm_nt<64, 64, false>), grid, dim3(256), 0, s, A, B, C, M, N, K);
  }
  return true;
}

}  // namespace

bool gemm_nt_f32(const float* A, const float* B, float* C, int M, int N, int K, bool accumulate, hipStream_t s) {
  return launch_gemm(A, B, C, M, N, K, accumulate, s);
}

PrefillLayout prefill_layout(int rows, int H, int I, int Q, int KV, size_t es, size_t base) {
  PrefillLayout p;
  p.rows = rows;
  if (rows <= 0) return p;
  (void)es;   // the chunked path computes in FP32
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = base + off; off = al(off + bytes); return o; };
  p.x = take((size_t)rows * H * 4);
  p.a = take((size_t)rows * H * 4);
  p.qkv = take((size_t)rows * (Q + 2 * KV) * 4);
  p.o = take((size_t)rows * Q * 4);
  p.act = take((size_t)rows * I * 4);
  p.gu = take((size_t)rows * 2 * I * 4);
  p.total = off;
  return p;
}

PrefillCtx prefill_ctx(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs* layers, int n_layers,
                       uint8_t* ws, const PrefillLayout& pf, int chunk) {
  PrefillCtx c;
  c.args = a; c.shape = sh; c.layers = layers; c.n_layers = n_layers; c.ws = ws; c.pf = pf; c.chunk = chunk;
  return c;
}

wsg_status run_prefill_chunks(const PrefillCtx& c, int p0, int n, hipStream_t s) {
  const DecodeArgs& a = c.args;
  if (a.dtype != 0) return fail(WSG_ERR_UNSUPPORTED, "chunked prefill runs FP32 models only");
  if (c.chunk < 1 || c.pf.rows < c.chunk) return fail(WSG_ERR_STATE, "prefill chunk scratch too small");
  const int H = a.hidden, I = a.inter, nq = a.n_q, nkv = a.n_kv, Q = nq * kD, KV = nkv * kD;
  const int G = nq / nkv;
  float* X = reinterpret_cast<float*>(c.ws + c.pf.x);
  float* A = reinterpret_cast<float*>(c.ws + c.pf.a);
  float* QKV = reinterpret_cast<float*>(c.ws + c.pf.qkv);
  float* O = reinterpret_cast<float*>(c.ws + c.pf.o);
  float* ACT = reinterpret_cast<float*>(c.ws + c.pf.act);
  float* GU = reinterpret_cast<float*>(c.ws + c.pf.gu);
  const float* E = static_cast<const float*>(a.embed);
  (void)hipGetLastError();
  for (int r0 = 0; r0 < n; r0 += c.chunk) {
    const int rows = min(c.chunk, n - r0);
    const int pc = p0 + r0;   // position of the chunk's first row
    hipLaunchKernelGGL(k_rows_embed, dim3(rows), dim3(256), 0, s, E, a.ids + pc, rows, H, a.vocab, X);
    for (int l = 0; l < c.n_layers; ++l) {
      const LayerPtrs& L = c.layers[l];
      const float* wqkv = static_cast<const float*>(L.wqkv);
      hipLaunchKernelGGL(k_rows_norm, dim3(cdiv(rows, 4)), dim3(256), 0, s, X, (const float*)L.in_norm, rows, H,
                         a.eps, A);
      if (!launch_gemm(A, wqkv, QKV, rows, Q + 2 * KV, H, false, s)) return fail(WSG_ERR_UNSUPPORTED, "gemm shape");
      hipLaunchKernelGGL(k_rows_qkv, dim3(cdiv(nq + 2 * nkv, 4), rows), dim3(256), 0, s, QKV, rows, nq, nkv, pc,
                         a.cap, a.eps, (const float*)L.q_norm, (const float*)L.k_norm, a.rope_cos, a.rope_sin,
                         (float*)L.k_cache, (float*)L.v_cache);
      if (l == c.n_layers - 1) break;   // only the K/V of the last layer has a consumer
      const dim3 ag(cdiv(rows, kQR), nkv);
      switch (G) {
        case 1: hipLaunchKernelGGL((k_prefill_attn<1>), ag, dim3(256), 0, s, QKV, (const float*)L.k_cache,
                                   (const float*)L.v_cache, rows, nq, nkv, pc, a.cap, O); break;
        case 2: hipLaunchKernelGGL((k_prefill_attn<2>), ag, dim3(256), 0, s, QKV, (const float*)L.k_cache,
                                   (const float*)L.v_cache, rows, nq, nkv, pc, a.cap, O); break;
        default: return fail(WSG_ERR_UNSUPPORTED, "chunked prefill supports query groups of 1 or 2");
      }
      if (!launch_gemm(O, static_cast<const float*>(L.wo), X, rows, H, Q, true, s))
        return fail(WSG_ERR_UNSUPPORTED, "gemm shape");
      hipLaunchKernelGGL(k_rows_norm, dim3(cdiv(rows, 4)), dim3(256), 0, s, X, (const float*)L.post_norm, rows, H,
                         a.eps, A);
      if (!launch_gemm(A, static_cast<const float*>(L.wgu), GU, rows, 2 * I, H, false, s))
        return fail(WSG_ERR_UNSUPPORTED, "gemm shape");
      hipLaunchKernelGGL(k_rows_swiglu, dim3(min(cdiv(rows * I, 256), 4096)), dim3(256), 0, s, GU, rows, I, ACT);
      if (!launch_gemm(ACT, static_cast<const float*>(L.wd), X, rows, H, I, true, s))
        return fail(WSG_ERR_UNSUPPORTED, "gemm shape");
    }
  }
  launch_set_pos(a.ctrl, p0 + n, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WSG_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return WSG_OK;
}

}  // namespace wsg
