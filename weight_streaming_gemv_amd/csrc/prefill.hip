// Chunked prefill for gfx950: several consecutive prompt rows of one request
// per chunk, every row attending to its whole causal prefix across chunks
// (Megakernels, "Chunked prefill for long prompts").
//
// Per chunk and layer (the pages' 11 ordered stages, here 8 launches):
//   rows_norm   [residual += pending split-K partials] + RMSNorm, one block per row
//   gemm        QKV projection  [n x H] . W_qkv^T   (FP32 MFMA)
//   rows_qkv    per-head Q/K RMSNorm + RoPE; K/V written to cache rows p0..p0+n-1
//   attn        causal attention of the n rows over keys 0..p0+r (FP32 MFMA)
//   gemm+res    O projection: residual added in the epilogue, or split-K
//               partial slices that the next rows_norm adds
//   rows_norm   post-attention RMSNorm
//   gemm+swiglu gate/up projection [n x 2I] with the SwiGLU in its epilogue
//               (only the [n x I] activation is stored)
//   gemm+res    down projection (as the O projection)
// The projections and attention's two products are the dense contractions
// and the MFMA users: a tiled kernel for many rows, a small-M kernel
// (weights streamed straight into registers, K split over waves and blocks)
// for up to 32 rows.  The chunk runs exactly n rows: the GEMM masks its
// ragged last row tile, so no padding rows exist.  Every chunk stops its last
// layer after the K/V write (Benchmark methodology, "Long-document chunked
// prefill": nonterminal chunks prune the final layer), except that the
// prompt's last row completes it alone (one-row launches of the same
// kernels) and hands its residual to the decode head: the only row that
// reaches the head.
#include <algorithm>
#include <type_traits>

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
typedef float f4v_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ GEMM
// C[M x N] (+)= A[M x K] . B[N x K]^T, all row-major FP32, K-contiguous
// operands.  Block tile BM x BN x BK, 256 threads = 2 x 2 waves, each wave a
// (BM/2) x (BN/2) sub-tile of 32 x 32 MFMA tiles (v_mfma_f32_32x32x2f32).
// Split K: block z covers k in [z*kspan, (z+1)*kspan) and writes its own
// slice C + z*c_split (kspan = K, one slice, when K is not split).
//
// MFMA 32x32x2 operand layout (lane l): A element (row l%32, k l/32),
// B element (k l/32, col l%32); accumulator register r holds row
// 8*(r/4) + 4*(l/32) + r%4, col l%32.  The two k slots of every MFMA are
// mapped to k = 32u + h*16 + s (u = 32-wide part of the K tile, h = l/32,
// s = step 0..15), so each lane reads 16 consecutive floats of one LDS row
// per part.  A 64-wide K tile (K ranges that are multiples of 64) gives
// each wave 32*TM*TN MFMAs (8192 cycles for a 64 x 64 wave tile) between
// barriers, which covers the latency of the next tile's global loads.
// With SWI, B is a packed gate/up matrix (N/2 gate rows, then N/2 up rows):
// tile x takes gate rows [x*BN/2, (x+1)*BN/2) as its first BN/2 columns and
// the matching up rows as the rest, so each gate wave's up partner is the
// wave beside it; the up waves stage their sums in LDS and the gate waves
// write C[M x N/2] = silu(gate) * up (the same per-element sums as without
// SWI).
constexpr int kBK = 32;                   // K granularity of the shapes accepted (and of the small-M kernel)
constexpr int kLdsPad = 4;                // floats of padding per LDS row

template <int BM, int BN, int BK, bool ACC, int WV, bool SWI = false, bool EARLY = false>
__global__ __launch_bounds__(64 * WV) void k_gemm_nt(const float* __restrict__ A, const float* __restrict__ B,
                                                     float* __restrict__ C, int M, int N, int K, int kspan,
                                                     size_t c_split) {
  constexpr int kThreads = 64 * WV;
  constexpr int kLdsRow = BK + kLdsPad;
  constexpr int NU = BK / 32;                  // 32-wide parts per K tile
  constexpr int WM = BM / (WV / 2), WN = BN / 2;   // wave tile: a (WV/2) x 2 grid of waves
  constexpr int TM = WM / 32, TN = WN / 32;    // MFMA tiles per wave
  constexpr int F4_ROW = BK / 4;               // float4 per tile row
  constexpr int A_LOADS = BM * F4_ROW / kThreads;   // float4 per thread per tile
  constexpr int B_LOADS = BN * F4_ROW / kThreads;
  static_assert(TM >= 1 && TN >= 1 && WM % 32 == 0 && WN % 32 == 0, "whole 32 x 32 MFMA tiles per wave");
  static_assert(BM * F4_ROW % kThreads == 0 && BN * F4_ROW % kThreads == 0, "whole float4 per thread");
  static_assert(!SWI || (!ACC && BM * (BN / 2) <= BN * kLdsRow), "SwiGLU: no accumulation, up sums fit in Bs");
  __shared__ float As[BM * kLdsRow];
  __shared__ float Bs[BN * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int nb = blockIdx.x * (BN / 2);   // SWI: the tile's first gate row (output column)
  const int li = lane & 31, lh = lane >> 5;
  A += (size_t)blockIdx.z * kspan;   // this split's K range (row stride stays K)
  B += (size_t)blockIdx.z * kspan;
  C += blockIdx.z * c_split;

  f16v_t acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // global -> register staging: thread loads float4 #(tid + kThreads i) of the
  // tile: row = idx / F4_ROW, col4 = idx % F4_ROW (plain loops: arrays
  // captured by a lambda would be forced into scratch memory)
  f4_t ra[A_LOADS], rb[B_LOADS];   // native vectors: HIP's float4 struct arrays end up in scratch
#define WSG_GEMM_LOAD(K0)                                                                           \
  {                                                                                                \
    _Pragma("unroll") for (int i = 0; i < A_LOADS; ++i) {                                          \
      const int idx = tid + kThreads * i, row = idx / F4_ROW, c4 = idx % F4_ROW;                        \
      const int gm = min(m0 + row, M - 1);   /* rows past M feed only unstored outputs */        \
      ra[i] = *reinterpret_cast<const f4_t*>(A + (size_t)gm * K + (K0) + 4 * c4);                  \
    }                                                                                              \
    _Pragma("unroll") for (int i = 0; i < B_LOADS; ++i) {                                          \
      const int idx = tid + kThreads * i, row = idx / F4_ROW, c4 = idx % F4_ROW;                        \
      const int brow = !SWI ? n0 + row : row < BN / 2 ? nb + row : N / 2 + nb + row - BN / 2;        \
      rb[i] = *reinterpret_cast<const f4_t*>(B + (size_t)brow * K + (K0) + 4 * c4);                \
    }                                                                                              \
  }

  // the operands of one 32-wide part u of the LDS tile
  float af[NU][TM][16], bf[NU][TN][16];
#define WSG_GEMM_FRAGS(U)                                                                          \
  {                                                                                                \
    _Pragma("unroll") for (int a = 0; a < TM; ++a)                                                 \
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                              \
        const f4_t v = *reinterpret_cast<const f4_t*>(                                             \
            &As[(wm + a * 32 + li) * kLdsRow + 32 * (U) + lh * 16 + 4 * q]);                       \
        af[U][a][4 * q] = v.x; af[U][a][4 * q + 1] = v.y; af[U][a][4 * q + 2] = v.z;              \
        af[U][a][4 * q + 3] = v.w;                                                                 \
      }                                                                                            \
    _Pragma("unroll") for (int b = 0; b < TN; ++b)                                                 \
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                              \
        const f4_t v = *reinterpret_cast<const f4_t*>(                                             \
            &Bs[(wn + b * 32 + li) * kLdsRow + 32 * (U) + lh * 16 + 4 * q]);                       \
        bf[U][b][4 * q] = v.x; bf[U][b][4 * q + 1] = v.y; bf[U][b][4 * q + 2] = v.z;              \
        bf[U][b][4 * q + 3] = v.w;                                                                 \
      }                                                                                            \
  }
#define WSG_GEMM_MFMA(U)                                                                           \
  _Pragma("unroll") for (int s = 0; s < 16; ++s)                                                   \
    _Pragma("unroll") for (int a = 0; a < TM; ++a)                                                 \
      _Pragma("unroll") for (int b = 0; b < TN; ++b)                                               \
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[U][a][s], bf[U][b][s], acc[a][b], 0, 0, 0);

  WSG_GEMM_LOAD(0)
  for (int k0 = 0; k0 < kspan; k0 += BK) {
    __syncthreads();          // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int idx = tid + kThreads * i, row = idx / F4_ROW, c4 = idx % F4_ROW;
      *reinterpret_cast<f4_t*>(&As[row * kLdsRow + 4 * c4]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int idx = tid + kThreads * i, row = idx / F4_ROW, c4 = idx % F4_ROW;
      *reinterpret_cast<f4_t*>(&Bs[row * kLdsRow + 4 * c4]) = rb[i];
    }
    __syncthreads();
    // next tile in flight during the MFMAs (the last iteration reloads the
    // final tile, in bounds and unused, to keep the loop free of branches).
    // The scheduler sinks these loads to the end of the loop body; with at
    // most one workgroup per CU (EARLY) nothing else covers their latency
    // there, so they are pinned here, ahead of the MFMAs (with two or more
    // workgroups per CU the sunk placement measured faster)
    WSG_GEMM_LOAD(min(k0 + BK, kspan - BK))
    if constexpr (EARLY) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NU; ++u) WSG_GEMM_FRAGS(u)
#pragma unroll
    for (int u = 0; u < NU; ++u) { WSG_GEMM_MFMA(u) }
  }
#undef WSG_GEMM_LOAD
#undef WSG_GEMM_FRAGS
#undef WSG_GEMM_MFMA

  if constexpr (SWI) {
    constexpr int US = BN / 2;   // row of the staged up sums
    float* s_up = Bs;
    __syncthreads();             // every wave has read its last operands from Bs
    if (wn != 0) {
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s_up[(wm + a * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)) * US + b * 32 + li] = acc[a][b][r];
    }
    __syncthreads();
    if (wn == 0) {
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = wm + a * 32 + 8 * (r >> 2) + 4 * lh + (r & 3), cl = b * 32 + li;
            const float g = acc[a][b][r], u = s_up[rl * US + cl];
            if (m0 + rl < M) C[(size_t)(m0 + rl) * (N / 2) + nb + cl] = g / (1.0f + expf(-g)) * u;
          }
    }
  } else {
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
}

// ------------------------------------------------------- small-M GEMM
// Few rows (M <= 32, short prompts): the tiled kernel above leaves most
// CUs idle and each block waits on its LDS pipeline.  Here a block owns a
// 16-column slice of C (16 weight rows) and splits K over its W waves; each
// wave streams its weight rows straight into registers with up to PD
// 32-wide K tiles in flight and multiplies them on v_mfma_f32_16x16x4f32
// (MT tiles of 16 rows of A).  The W partial tiles are summed in LDS in
// wave order, so the result does not depend on timing.
//
// MFMA 16x16x4 operand layout (lane l): A element (row l%16, k slot l/16),
// B element (k slot l/16, col l%16); accumulator register r holds row
// 4*(l/16) + r, col l%16.  Slot q of step s is k = 8q + s of the 32-wide
// tile, so each lane reads 8 consecutive floats of a row per tile.
typedef float f4v_t __attribute__((ext_vector_type(4)));

//
// Block (x, y) covers columns [16x, 16x + 16) and the K range
// [y*KB, (y+1)*KB) of the ldk-long rows; with several K ranges each writes
// its own partial slice C + y*c_split (summed later by the consumer).
// With SWI, B is a packed gate/up matrix (N/2 gate rows, then N/2 up rows):
// workgroup b takes gate rows [8b, 8b + 8) and the matching up rows, and
// writes C[M x N/2] = silu(gate) * up (the SwiGLU of the MLP) instead of
// the product; the per-element sums are the same as without SWI.
template <int KB, int W, int MT, bool ACC, bool SWI>
__global__ __launch_bounds__(64 * W) void k_gemm_skinny(const float* __restrict__ A, const float* __restrict__ B,
                                                        float* __restrict__ C, int M, int N, int ldk,
                                                        size_t c_split) {
  constexpr int K = KB;
  constexpr int KW = K / W;                       // K range of one wave
  constexpr int NT = KW / kBK;                    // 32-wide tiles per wave
  constexpr int PDM = W >= 16 ? 4 : 8;            // tiles in flight (register budget)
  constexpr int PD = NT < PDM ? NT : PDM;
  constexpr int RS = 17;                          // padded row of the reduction tile
  static_assert(K % (W * kBK) == 0, "whole tiles per wave");
  __shared__ float red[W][MT * 16 * RS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int k0 = blockIdx.y * KB + wave * KW + 8 * lq;
  C += blockIdx.y * c_split;
  const int nrow = SWI ? blockIdx.x * 8 + (li & 7) + (li >= 8 ? N / 2 : 0) : n0 + li;
  const float* bp = B + (size_t)nrow * ldk + k0;
  const float* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)   // rows past M feed only unstored outputs
    ap[mt] = A + (size_t)min(mt * 16 + li, M - 1) * ldk + k0;

  f4_t tb[PD][2], ta[PD][MT][2];
#define WSG_SKINNY_LOAD(T)                                                                        {                                                                                                 const int buf_ = (T) % PD, k_ = (T) * kBK;                                                      tb[buf_][0] = *reinterpret_cast<const f4_t*>(bp + k_);                                          tb[buf_][1] = *reinterpret_cast<const f4_t*>(bp + k_ + 4);                                      _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) {                                               ta[buf_][mt][0] = *reinterpret_cast<const f4_t*>(ap[mt] + k_);                                  ta[buf_][mt][1] = *reinterpret_cast<const f4_t*>(ap[mt] + k_ + 4);                            }                                                                                             }
#pragma unroll
  for (int t = 0; t < PD - 1; ++t) WSG_SKINNY_LOAD(t)
  // keep the scheduler from sinking each load next to its use
  __builtin_amdgcn_sched_barrier(0);
  f4v_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f4v_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t + PD - 1 < NT) WSG_SKINNY_LOAD(t + PD - 1)
    __builtin_amdgcn_sched_barrier(0);
    const int b = t % PD;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float bv = tb[b][s >> 2][s & 3];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[b][mt][s >> 2][s & 3], bv, acc[mt], 0, 0, 0);
    }
  }
#undef WSG_SKINNY_LOAD
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][(mt * 16 + 4 * lq + r) * RS + li] = acc[mt][r];
  __syncthreads();
  if constexpr (SWI) {
    // columns 0-7 of the tile are gate rows, 8-15 the matching up rows
    for (int e = threadIdx.x; e < MT * 128; e += 64 * W) {
      const int row = e >> 3, col = e & 7;
      float g = red[0][row * RS + col], u = red[0][row * RS + col + 8];
#pragma unroll
      for (int w = 1; w < W; ++w) {
        g += red[w][row * RS + col];
        u += red[w][row * RS + col + 8];
      }
      if (row < M) C[(size_t)row * (N / 2) + blockIdx.x * 8 + col] = g / (1.0f + expf(-g)) * u;
    }
  } else {
    for (int e = threadIdx.x; e < MT * 256; e += 64 * W) {
      const int row = e >> 4, col = e & 15;
      float sum = red[0][row * RS + col];
#pragma unroll
      for (int w = 1; w < W; ++w) sum += red[w][row * RS + col];
      if (row < M) {
        float* p = C + (size_t)row * N + n0 + col;
        *p = ACC ? *p + sum : sum;
      }
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

// X[r] += P[0][r] + P[1][r] + ... (NP slices of n x H, added in order),
// then Y[r] = X[r] * (mean(X[r]^2) + eps)^-1/2 * g.  One block of 256
// threads per row (H <= 3072): thread t owns columns 4t + 1024i, with all
// of its loads in flight at once.
template <int NP>
__global__ __launch_bounds__(256) void k_rows_norm(float* __restrict__ X, const float* __restrict__ P,
                                                   const float* __restrict__ g, int n, int H, float eps,
                                                   float* __restrict__ Y) {
  constexpr int kMaxIt = 3;
  __shared__ float s_ss[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  float* x = X + (size_t)r * H;
  f4_t v[kMaxIt], gv[kMaxIt], pv[kMaxIt][NP > 0 ? NP : 1];
#pragma unroll
  for (int i = 0; i < kMaxIt; ++i) {
    const int c = min(4 * tid + 1024 * i, H - 4);   // clamped: columns past H are loaded, never stored
    v[i] = *reinterpret_cast<const f4_t*>(x + c);
    gv[i] = *reinterpret_cast<const f4_t*>(g + c);
#pragma unroll
    for (int p = 0; p < NP; ++p) pv[i][p] = *reinterpret_cast<const f4_t*>(P + ((size_t)p * n + r) * H + c);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxIt; ++i) {
    const int c = 4 * tid + 1024 * i;
#pragma unroll
    for (int p = 0; p < NP; ++p) v[i] += pv[i][p];
    if (c < H) {
      if (NP > 0) *reinterpret_cast<f4_t*>(x + c) = v[i];
      ss = fmaf(v[i].x, v[i].x, fmaf(v[i].y, v[i].y, fmaf(v[i].z, v[i].z, fmaf(v[i].w, v[i].w, ss))));
    }
  }
  ss = wave_sum(ss);
  if (lane_id() == 0) s_ss[wave_id()] = ss;
  __syncthreads();
  ss = (s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3]);
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int i = 0; i < kMaxIt; ++i) {
    const int c = 4 * tid + 1024 * i;
    if (c < H) *reinterpret_cast<f4_t*>(Y + (size_t)r * H + c) = v[i] * inv * gv[i];
  }
}

bool launch_rows_norm(float* X, const float* P, int n_part, const float* g, int n, int H, float eps, float* Y,
                      hipStream_t s) {
  if (H > 3072 || H % 4 != 0) return false;
  switch (n_part) {
    case 0: hipLaunchKernelGGL((k_rows_norm<0>), dim3(n), dim3(256), 0, s, X, P, g, n, H, eps, Y); return true;
    case 2: hipLaunchKernelGGL((k_rows_norm<2>), dim3(n), dim3(256), 0, s, X, P, g, n, H, eps, Y); return true;
    case 4: hipLaunchKernelGGL((k_rows_norm<4>), dim3(n), dim3(256), 0, s, X, P, g, n, H, eps, Y); return true;
    case 8: hipLaunchKernelGGL((k_rows_norm<8>), dim3(n), dim3(256), 0, s, X, P, g, n, H, eps, Y); return true;
    default: return false;
  }
}

// The residual of row r after its last pending split-K slices (added in
// slice order, as k_rows_norm adds them), written to x_out: the input of the
// decode head for a prompt's last row.
__global__ __launch_bounds__(256) void k_row_residual(const float* __restrict__ X, const float* __restrict__ P,
                                                      int n_part, int n, int H, int r, float* __restrict__ x_out) {
  for (int c = 4 * threadIdx.x; c < H; c += 1024) {
    f4_t v = *reinterpret_cast<const f4_t*>(X + (size_t)r * H + c);
    for (int p = 0; p < n_part; ++p) v += *reinterpret_cast<const f4_t*>(P + ((size_t)p * n + r) * H + c);
    *reinterpret_cast<f4_t*>(x_out + c) = v;
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

// ------------------------------------------------------------ attention
// Causal attention of chunk rows [0, n) (positions p0 + r) over cached keys
// 0..p0+r of KV head j, for its G query heads (Megakernels, "Chunked
// prefill for long prompts": query-tiled prefill attention sharing each K/V
// tile across the rows of a query tile, online softmax in the log2 domain).
//
// Both products run on v_mfma_f32_16x16x4f32, in transposed form so the
// probabilities never leave registers.  The chunk's query vectors (vector
// v = row * G + head) are cut into tiles of 32 (32/G rows), and block b
// takes tiles b and n_tiles - 1 - b: under the causal mask a tile's work
// grows with its last row, so every block gets the same total and no CU
// waits for the longest tile (all blocks run at once, one per CU).  The 8
// waves: wave w serves tile w >> 2 (waves w and w + 4 share a SIMD, so
// the later tile's keys past the earlier tile's range keep every SIMD
// busy), key group c = (w >> 1) & 1 (the key tiles 2i + c), and vectors
// [16h, 16h + 16) of its tile, h = w & 1.  Each K/V tile pair is staged once
// per block and serves both query tiles.  Per tile of 32 keys (K row-major
// and V transposed in LDS):
//   S^T[key][v] = sum_d K[key][d] Q[v][d]     (A = K from LDS, B = Q in registers)
//   O^T[d][v]  += sum_key V^T[d][key] P^T[key][v]
// MFMA 16x16x4 layout (lane l): A (row l%16, k slot l/16), B (k slot l/16,
// col l%16), accumulator register r = (row 4(l/16) + r, col l%16).  For the
// first product slot q of step s is d = 32q + s; for the second it is key
// 4q + s of a 16-key half, which is exactly register s of the S^T
// accumulator of lane l: P^T is the B operand as computed.  Every lane owns
// one query vector (column l%16), so its softmax state is per lane; a
// column's 16 keys of a half sit in the 4 lanes l%16 + 16q (xor 16, 32).
// At the end key group 1 hands its (max, sum, O^T) states to key group 0
// through LDS, which merges them and writes O.
constexpr int kAQV = 32;           // query vectors per tile (two tiles per block)
constexpr int kAKT = 32;           // keys per tile
constexpr int kKsRow = kD + 4;     // K tile row (floats): conflict-free 16-byte reads
constexpr int kVtRow = kAKT + 8;   // V^T tile row (+4 measured twice the LDS bank-conflict cycles)
constexpr int kAttnThreads = 512;
constexpr int kStateRow = 34;      // merge record per lane: m, l, O^T[32]

template <int G>
__global__ __launch_bounds__(kAttnThreads) void k_prefill_attn(const float* __restrict__ QKV,
                                                               const float* __restrict__ k_cache,
                                                               const float* __restrict__ v_cache, int n, int n_q,
                                                               int n_kv, int p0, int cap, float* __restrict__ O) {
  constexpr int BR = kAQV / G;       // rows per tile
  __shared__ float Ks[2][kAKT * kKsRow];
  __shared__ float Vt[2][kD * kVtRow];
  static_assert(4 * kWave * kStateRow <= 2 * kD * kVtRow, "merge records fit in the V tiles");
  const int j = blockIdx.y;
  const int n_tiles = (n + BR - 1) / BR;
  const int tile_a = blockIdx.x, tile_b = n_tiles - 1 - blockIdx.x;   // tile_a <= tile_b
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ts = wave >> 2, grp = (wave >> 1) & 1, wh = wave & 1;
  const int li = lane & 15, lq = lane >> 4;
  const int width = (n_q + 2 * n_kv) * kD;
  const float qscale = kLog2e / sqrtf((float)kD);
  // an odd tile count leaves the middle tile to the first half of the block
  const bool tile_on = ts == 0 || tile_b > tile_a;
  const int tile = ts == 0 ? tile_a : tile_b;
  // keys a tile needs: through its last valid row's position
  const int keys_a = p0 + min(n, (tile_a + 1) * BR);
  const int keys_b = p0 + min(n, (tile_b + 1) * BR);
  const int my_keys = tile_on ? (ts == 0 ? keys_a : keys_b) : 0;

  // this lane's query vector
  const int v = wh * 16 + li;
  const int rr = v / G, g = v - rr * G;
  const int row = tile * BR + rr;
  const bool row_ok = tile_on && row < n;
  const int my_pos = p0 + row;
  // the wave's rows: all inside the chunk, and the first one's position
  // (tiles with no key past it need no causal mask)
  const bool wave_rows_ok = tile_on && tile * BR + (wh * 16 + 15) / G < n;
  const int wave_first_pos = p0 + tile * BR + (wh * 16) / G;
  float qf[32];
  {
    const float* q = QKV + (size_t)min(row, n - 1) * width + (j * G + g) * kD + 32 * lq;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const f4_t x = *reinterpret_cast<const f4_t*>(q + 4 * t);
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[4 * t + i] = x[i] * qscale;
    }
  }
  const int n_keys = keys_b;   // keys any row of the block needs (tile b ends last)

  f4v_t oacc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) oacc[mt] = f4v_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  const float* kh = k_cache + (size_t)j * cap * kD;
  const float* vh = v_cache + (size_t)j * cap * kD;
  // tile-pair staging: float4 #idx = tid + 512i of the pair, tile idx/1024;
  // within a tile, K float4 f = (key f/32, dims 4(f%32)) and V float4 f =
  // (key f%32, dims 4(f/32)), so the transposed LDS writes of a wave hit
  // consecutive banks.  Keys at or past n_keys are cache slots no row may
  // see (stale memory): their loads are clamped into the cache and their
  // values replaced by zeros, since a masked key still enters the PV product
  // with weight 0 (and 0 * Inf is NaN).
  f4_t kr[4], vr[4];
#define WSG_ATTN_LOAD(K0)                                                                         \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                 \
    const int idx = tid + kAttnThreads * i, f = idx & 1023;                                       \
    const int kt = (K0) + kAKT * (idx >> 10);                                                     \
    const int k1 = kt + (f >> 5), k2 = kt + (f & 31);                                             \
    const int kk = min(k1, cap - 1), kv = min(k2, cap - 1);                                       \
    kr[i] = *reinterpret_cast<const f4_t*>(kh + (size_t)kk * kD + 4 * (f & 31));                  \
    vr[i] = *reinterpret_cast<const f4_t*>(vh + (size_t)kv * kD + 4 * (f >> 5));                  \
    if (k1 >= n_keys) kr[i] = f4_t{0.f, 0.f, 0.f, 0.f};                                           \
    if (k2 >= n_keys) vr[i] = f4_t{0.f, 0.f, 0.f, 0.f};                                           \
  }
  WSG_ATTN_LOAD(0)
  for (int k0 = 0; k0 < n_keys; k0 += 2 * kAKT) {
    __syncthreads();   // previous tile pair consumed
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kAttnThreads * i, f = idx & 1023, t = idx >> 10;
      *reinterpret_cast<f4_t*>(&Ks[t][(f >> 5) * kKsRow + 4 * (f & 31)]) = kr[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) Vt[t][(4 * (f >> 5) + e) * kVtRow + (f & 31)] = vr[i][e];
    }
    __syncthreads();
    // next pair in flight during the MFMAs (the last iteration reloads an
    // in-bounds pair, unused, to keep the loop free of branches)
    WSG_ATTN_LOAD(min(k0 + 2 * kAKT, n_keys - 1))
#undef WSG_ATTN_LOAD
    const int kt = k0 + kAKT * grp;   // this group's key tile
    if (kt < my_keys) {               // wave-uniform
      const float* ks = Ks[grp];
      const float* vt = Vt[grp];
      // S^T for the two 16-key halves.  Each product reads all of its A
      // operands from LDS first (16 reads in flight), then runs its 64
      // MFMAs, so the waits for the reads overlap the matrix pipe instead of
      // preceding every four MFMAs.
      f4v_t sacc[2];
      {
        f4_t ka[2][8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int t = 0; t < 8; ++t)
            ka[h][t] = *reinterpret_cast<const f4_t*>(&ks[(16 * h + li) * kKsRow + 32 * lq + 4 * t]);
        __builtin_amdgcn_sched_barrier(0);   // (the scheduler would pair each read with its MFMAs)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          sacc[h] = f4v_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sacc[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[h][t][i], qf[4 * t + i], sacc[h], 0, 0, 0);
        }
      }
      // the V^T operands of O^T += V^T P^T, read while the score MFMAs run
      // and the softmax is computed
      f4_t va[2][8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
          va[h][mt] = *reinterpret_cast<const f4_t*>(&vt[(16 * mt + li) * kVtRow + 16 * h + 4 * lq]);
      __builtin_amdgcn_sched_barrier(0);
      // causal mask (only tiles that reach past the wave's first row, or
      // hold rows past the chunk), tile max per query vector
      if (!wave_rows_ok || kt + kAKT - 1 > wave_first_pos) {   // wave-uniform
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kt + 16 * h + 4 * lq + r;
            if (!(row_ok && key <= my_pos)) sacc[h][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[h][r]);
      {
        const LanePair a = lanes_xor16(mx);
        const LanePair b = lanes_xor32(fmaxf(a.lo, a.hi));
        mx = fmaxf(b.lo, b.hi);
      }
      const float mn = fmaxf(m, mx);
      // exponents relative to the new max (0 while a vector has no key yet,
      // so masked scores give exp2(-inf) = 0); alpha = 1 when the max is
      // unchanged.  The hardware exp2: arguments are <= 0, and results below
      // the normal range (weights under 2^-126 against a sum >= 1) may flush.
      const float base = mn == -INFINITY ? 0.f : mn;
      const float alpha = m == mn ? 1.f : __builtin_amdgcn_exp2f(m - base);
      float psum = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(sacc[h][r] - base);
          sacc[h][r] = p;
          psum += p;
        }
      {
        const LanePair a = lanes_xor16(psum);
        const LanePair b = lanes_xor32(a.lo + a.hi);
        psum = b.lo + b.hi;
      }
      l = l * alpha + psum;
      m = mn;
      if (__any(alpha != 1.f)) {   // wave-uniform: rescale only when a max moved
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) oacc[mt] *= alpha;
      }
      // O^T += V^T P^T
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[h][mt][s2], sacc[h][s2], oacc[mt], 0, 0, 0);
    }
  }
  // merge: group 1's states -> group 0 (records in the V tile memory)
  __syncthreads();
  float* rec = &Vt[0][0] + ((ts * 2 + wh) * kWave + lane) * kStateRow;
  if (grp == 1) {
    rec[0] = m;
    rec[1] = l;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) rec[2 + 4 * mt + r] = oacc[mt][r];
  }
  __syncthreads();
  if (grp == 0 && row_ok) {
    const float m2 = rec[0], l2 = rec[1];
    const float mn = fmaxf(m, m2);   // finite: every valid row sees key 0
    const float a1 = m == -INFINITY ? 0.f : exp2f(m - mn);
    const float a2 = m2 == -INFINITY ? 0.f : exp2f(m2 - mn);
    const float inv = 1.0f / (l * a1 + l2 * a2);
    // lane holds O^T[d = 16mt + 4lq + r][its vector]
    float* o = O + (size_t)row * n_q * kD + (j * G + g) * kD + 4 * lq;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f4_t out;
#pragma unroll
      for (int r = 0; r < 4; ++r) out[r] = (oacc[mt][r] * a1 + rec[2 + 4 * mt + r] * a2) * inv;
      *reinterpret_cast<f4_t*>(o + 16 * mt) = out;
    }
  }
}

// ------------------------------------------------------------ launchers
constexpr int kSkinnyMaxM = 32;

// Waves per block: the fewest that give >= 2048 waves in all, with whole
// 32-wide K tiles per wave.
int skinny_waves(int blocks, int KB) {
  int w = 0;
  for (int c : {4, 8, 16}) {
    if (KB % (c * kBK) != 0) continue;
    w = c;
    if ((int64_t)blocks * c >= 2048) break;
  }
  return w;
}

template <int KB>
bool launch_skinny_kb(const float* A, const float* B, float* C, int M, int N, int K, int S, size_t c_split,
                      bool acc, bool swiglu, hipStream_t s) {
  const int W = skinny_waves(N / 16 * S, KB);
  const dim3 grid(N / 16, S);
  auto go = [&](auto wc, auto mc, auto ac, auto sc) {
    constexpr int Wv = decltype(wc)::value, MTv = decltype(mc)::value;
    constexpr bool ACCv = decltype(ac)::value, SWIv = decltype(sc)::value;
    if constexpr (KB % (Wv * kBK) == 0 && !(ACCv && SWIv)) {
      hipLaunchKernelGGL((k_gemm_skinny<KB, Wv, MTv, ACCv, SWIv>), grid, dim3(64 * Wv), 0, s, A, B, C, M, N, K,
                         c_split);
      return true;
    } else {
      return false;
    }
  };
  auto with_m = [&](auto wc) {
    auto with_acc = [&](auto mc) {
      if (swiglu) return go(wc, mc, std::false_type{}, std::true_type{});
      return acc ? go(wc, mc, std::true_type{}, std::false_type{}) : go(wc, mc, std::false_type{}, std::false_type{});
    };
    return M <= 16 ? with_acc(std::integral_constant<int, 1>{}) : with_acc(std::integral_constant<int, 2>{});
  };
  switch (W) {
    case 4: return with_m(std::integral_constant<int, 4>{});
    case 8: return with_m(std::integral_constant<int, 8>{});
    case 16: return with_m(std::integral_constant<int, 16>{});
    default: return false;
  }
}

// K ranges compiled in for the small-M kernel.
bool skinny_kb_ok(int kb) {
  switch (kb) {
    case 128: case 256: case 512: case 768: case 1024: case 2048: case 3072: return true;
    default: return false;
  }
}

bool launch_skinny(const float* A, const float* B, float* C, int M, int N, int K, int S, size_t c_split, bool acc,
                   hipStream_t s, bool swiglu = false) {
  if (K % S != 0 || !skinny_kb_ok(K / S)) return false;
  if (swiglu && (S != 1 || acc || N % 16 != 0)) return false;
  switch (K / S) {
    case 128: return launch_skinny_kb<128>(A, B, C, M, N, K, S, c_split, acc, swiglu, s);
    case 256: return launch_skinny_kb<256>(A, B, C, M, N, K, S, c_split, acc, swiglu, s);
    case 512: return launch_skinny_kb<512>(A, B, C, M, N, K, S, c_split, acc, swiglu, s);
    case 768: return launch_skinny_kb<768>(A, B, C, M, N, K, S, c_split, acc, swiglu, s);
    case 1024: return launch_skinny_kb<1024>(A, B, C, M, N, K, S, c_split, acc, swiglu, s);
    case 2048: return launch_skinny_kb<2048>(A, B, C, M, N, K, S, c_split, acc, swiglu, s);
    case 3072: return launch_skinny_kb<3072>(A, B, C, M, N, K, S, c_split, acc, swiglu, s);
    default: return false;
  }
}

constexpr int kCUs = 256;   // compute units: workgroups of one round at one per CU

// Tiled launch of BM x BN tiles with K split S ways (S slices c_split
// apart): 64-wide K tiles when the split's K range allows, else 32-wide.
// With swi (one slice, no accumulation): the SwiGLU epilogue, C being
// M x N/2; false when the tile cannot stage its up sums in LDS.
template <int BM, int BN>
bool launch_tiled(const float* A, const float* B, float* C, int M, int N, int K, int S, size_t c_split, bool acc,
                  hipStream_t s, bool swi = false) {
  const dim3 grid(N / BN, cdiv(M, BM), S);
  const int kspan = K / S;
  auto go = [&](auto bk) {
    constexpr int BK = decltype(bk)::value;
    // 128-row tiles: 8 waves, two per SIMD (one computes while the other
    // reads its operands from LDS); 64 x 64 tiles: 4 waves
    constexpr int WV = BM == 128 ? 8 : 4;
    // one round of workgroups (at most one per CU): next-tile loads pinned early
    const bool early = (int64_t)grid.x * grid.y * grid.z <= kCUs;
    if (swi) {
      if constexpr (BM / 2 <= BK + kLdsPad) {
        if (S != 1 || acc) return false;
        if (early) {
          hipLaunchKernelGGL((k_gemm_nt<BM, BN, BK, false, WV, true, true>), grid, dim3(64 * WV), 0, s, A, B, C, M,
                             N, K, kspan, c_split);
          return true;
        }
        hipLaunchKernelGGL((k_gemm_nt<BM, BN, BK, false, WV, true>), grid, dim3(64 * WV), 0, s, A, B, C, M, N, K,
                           kspan, c_split);
        return true;
      }
      return false;
    }
    if (early && !acc) {
      hipLaunchKernelGGL((k_gemm_nt<BM, BN, BK, false, WV, false, true>), grid, dim3(64 * WV), 0, s, A, B, C, M, N,
                         K, kspan, c_split);
      return true;
    }
    if (acc)
      hipLaunchKernelGGL((k_gemm_nt<BM, BN, BK, true, WV>), grid, dim3(64 * WV), 0, s, A, B, C, M, N, K, kspan, c_split);
    else
      hipLaunchKernelGGL((k_gemm_nt<BM, BN, BK, false, WV>), grid, dim3(64 * WV), 0, s, A, B, C, M, N, K, kspan, c_split);
    return true;
  };
  if (kspan % 64 == 0) return go(std::integral_constant<int, 64>{});
  return go(std::integral_constant<int, 32>{});
}

// Tile of the tiled kernel for an M x N product: the one with the fewest
// rounds of 256 blocks times tile area (the time of the busiest CU), the
// larger tile on ties; 128 x 192 serves N = 6144-like widths in one round.
struct Tile { int bm, bn; };
Tile pick_tile(int M, int N) {
  Tile best{64, 64};
  int64_t best_cost = -1;
  for (Tile t : {Tile{128, 192}, Tile{128, 128}, Tile{64, 64}}) {
    if (N % t.bn != 0) continue;
    const int64_t blocks = (int64_t)(N / t.bn) * cdiv(M, t.bm);
    const int64_t cost = (blocks + 255) / 256 * t.bm * t.bn;
    if (best_cost < 0 || cost < best_cost) { best = t; best_cost = cost; }
  }
  return best;
}

bool launch_tile(Tile t, const float* A, const float* B, float* C, int M, int N, int K, int S, size_t c_split,
                 bool acc, hipStream_t s, bool swi = false) {
  if (t.bm == 128 && t.bn == 192) return launch_tiled<128, 192>(A, B, C, M, N, K, S, c_split, acc, s, swi);
  if (t.bm == 128) return launch_tiled<128, 128>(A, B, C, M, N, K, S, c_split, acc, s, swi);
  return launch_tiled<64, 64>(A, B, C, M, N, K, S, c_split, acc, s, swi);
}

// M <= 32 with a compiled K: the small-M kernel; otherwise the tiled kernel.
bool launch_gemm(const float* A, const float* B, float* C, int M, int N, int K, bool acc, hipStream_t s) {
  if (M < 1 || N % 64 != 0 || K % kBK != 0) return false;
  if (M <= kSkinnyMaxM && launch_skinny(A, B, C, M, N, K, 1, 0, acc, s)) return true;
  return launch_tile(pick_tile(M, N), A, B, C, M, N, K, 1, 0, acc, s);
}

// ACT[M x I] = silu(A . Wg^T) * (A . Wu^T) for the packed gate/up matrix Wgu
// (I gate rows, then I up rows), the SwiGLU computed in the epilogue of the
// product: up to 32 rows in the small-M kernel, otherwise in the tiled one
// (on the tile the plain product would take, or on 64 x 64 tiles where that
// one cannot stage its up sums).  Same shape rules as launch_gemm for N = 2I.
bool launch_gemm_swiglu(const float* A, const float* Wgu, float* ACT, int M, int I, int K, hipStream_t s) {
  if (M < 1 || I < 1 || (2 * I) % 64 != 0 || K % kBK != 0) return false;
  if (M <= kSkinnyMaxM && launch_skinny(A, Wgu, ACT, M, 2 * I, K, 1, 0, false, s, true)) return true;
  return launch_tile(pick_tile(M, 2 * I), A, Wgu, ACT, M, 2 * I, K, 1, 0, false, s, true) ||
         launch_tile(Tile{64, 64}, A, Wgu, ACT, M, 2 * I, K, 1, 0, false, s, true);
}

// X[M x N] += A . B^T for a residual stream consumed by k_rows_norm.  A
// residual projection has few column tiles (N = hidden), so K is split over
// up to kMaxSplitK blocks per tile (the small-M kernel for up to 32 rows;
// otherwise the larger tiles whose count times the split reaches 1024
// blocks), writing FP32 partial slices to P (M x N each) instead of X;
// returns the slice count (0: added into X), which the following
// k_rows_norm adds to X in slice order.  Returns -1 for an unsupported shape.
constexpr int kMaxSplitK = 8;

int launch_gemm_residual(const float* A, const float* B, float* X, float* P, int M, int N, int K, hipStream_t s) {
  if (M <= kSkinnyMaxM && N % 64 == 0 && N / 16 < 256) {
    int S = 0;   // the fewest K splits (2, 4 or 8, a compiled K range) that give >= 256 blocks
    for (int c = 2; c <= kMaxSplitK; c *= 2) {
      if (K % c != 0 || !skinny_kb_ok(K / c)) continue;
      S = c;
      if ((N / 16) * c >= 256) break;
    }
    if (S > 1 && launch_skinny(A, B, P, M, N, K, S, (size_t)M * N, false, s)) return S;
  }
  if (M > kSkinnyMaxM && N % 64 == 0 && K % kBK == 0) {
    // the fewest splits (64-wide K tiles each) reaching 1024 blocks, 128 x 128
    // tiles first.  Several workgroups share a CU (registers and LDS allow two
    // of 128 x 128, four of 64 x 64), and with more of them resident each
    // hides the others' barriers and operand loads: for 1024-row chunks the
    // 64 x 64 tiles split 4 ways beat 128 x 128 split 4 ways (256 blocks) by
    // 2.7 % of the whole prefill, and 128 x 128 split 8 ways by 1.2 %; a 2048-block
    // target (64 x 64 split 8 ways) measured slower again.
    int bm = 0, S = 0;
    for (int t : {128, 64}) {
      if (N % t != 0) continue;
      const int64_t tiles = (int64_t)(N / t) * cdiv(M, t);
      for (int c = 1; c <= kMaxSplitK && K % (c * 64) == 0; c *= 2)
        if (tiles * c >= 1024) { bm = t; S = c; break; }
      if (bm) break;
    }
    if (bm == 0) {   // too few tiles for 256 blocks: small tiles, the most splits
      bm = 64;
      S = 1;
      while (S < kMaxSplitK && K % (2 * S * 64) == 0) S *= 2;
    }
    if (S > 1 && launch_tile(Tile{bm, bm}, A, B, P, M, N, K, S, (size_t)M * N, false, s)) return S;
  }
  return launch_gemm(A, B, X, M, N, K, true, s) ? 0 : -1;
}

}  // namespace

bool gemm_nt_f32(const float* A, const float* B, float* C, int M, int N, int K, bool accumulate, hipStream_t s) {
  return launch_gemm(A, B, C, M, N, K, accumulate, s);
}

bool gemm_swiglu_f32(const float* A, const float* Wgu, float* ACT, int M, int I, int K, hipStream_t s) {
  return launch_gemm_swiglu(A, Wgu, ACT, M, I, K, s);
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
  p.part = take((size_t)kMaxSplitK * rows * H * 4);   // split-K partial slices of a residual GEMM
  p.total = off;
  return p;
}

PrefillCtx prefill_ctx(const DecodeArgs& a, const DecodeShape& sh, const LayerPtrs* layers, int n_layers,
                       uint8_t* ws, const PrefillLayout& pf, int chunk) {
  PrefillCtx c;
  c.args = a; c.shape = sh; c.layers = layers; c.n_layers = n_layers; c.ws = ws; c.pf = pf; c.chunk = chunk;
  return c;
}

wsg_status run_prefill_chunks(const PrefillCtx& c, int p0, int n, bool to_head, hipStream_t s) {
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
  float* PART = reinterpret_cast<float*>(c.ws + c.pf.part);
  const float* E = static_cast<const float*>(a.embed);
  (void)hipGetLastError();
  for (int r0 = 0; r0 < n; r0 += c.chunk) {
    const int rows = min(c.chunk, n - r0);
    const int pc = p0 + r0;   // position of the chunk's first row
    hipLaunchKernelGGL(k_rows_embed, dim3(rows), dim3(256), 0, s, E, a.ids + pc, rows, H, a.vocab, X);
    int n_part = 0;   // partial slices of the last residual GEMM not yet added to X
    for (int l = 0; l < c.n_layers; ++l) {
      const LayerPtrs& L = c.layers[l];
      const float* wqkv = static_cast<const float*>(L.wqkv);
      if (!launch_rows_norm(X, PART, n_part, (const float*)L.in_norm, rows, H, a.eps, A, s))
        return fail(WSG_ERR_UNSUPPORTED, "row norm shape");
      if (!launch_gemm(A, wqkv, QKV, rows, Q + 2 * KV, H, false, s)) return fail(WSG_ERR_UNSUPPORTED, "gemm shape");
      hipLaunchKernelGGL(k_rows_qkv, dim3(cdiv(nq + 2 * nkv, 4), rows), dim3(256), 0, s, QKV, rows, nq, nkv, pc,
                         a.cap, a.eps, (const float*)L.q_norm, (const float*)L.k_norm, a.rope_cos, a.rope_sin,
                         (float*)L.k_cache, (float*)L.v_cache);
      // The last layer: its K/V is all that later rows need; with to_head
      // the prompt's last row alone also completes it, for the head.
      const bool last_layer = l == c.n_layers - 1;
      if (last_layer && !(to_head && r0 + rows == n)) break;
      const int r_first = last_layer ? rows - 1 : 0, nr = rows - r_first;
      float* Xr = X + (size_t)r_first * H;
      const float* QKVr = QKV + (size_t)r_first * (Q + 2 * KV);
      const dim3 ag(cdiv(cdiv(nr, kAQV / G), 2), nkv);   // pairs of query tiles
      switch (G) {
        case 1: hipLaunchKernelGGL((k_prefill_attn<1>), ag, dim3(kAttnThreads), 0, s, QKVr, (const float*)L.k_cache,
                                   (const float*)L.v_cache, nr, nq, nkv, pc + r_first, a.cap, O); break;
        case 2: hipLaunchKernelGGL((k_prefill_attn<2>), ag, dim3(kAttnThreads), 0, s, QKVr, (const float*)L.k_cache,
                                   (const float*)L.v_cache, nr, nq, nkv, pc + r_first, a.cap, O); break;
        default: return fail(WSG_ERR_UNSUPPORTED, "chunked prefill supports query groups of 1 or 2");
      }
      n_part = launch_gemm_residual(O, static_cast<const float*>(L.wo), Xr, PART, nr, H, Q, s);
      if (n_part < 0) return fail(WSG_ERR_UNSUPPORTED, "gemm shape");
      if (!launch_rows_norm(Xr, PART, n_part, (const float*)L.post_norm, nr, H, a.eps, A, s))
        return fail(WSG_ERR_UNSUPPORTED, "row norm shape");
      if (!launch_gemm_swiglu(A, static_cast<const float*>(L.wgu), ACT, nr, I, H, s))
        return fail(WSG_ERR_UNSUPPORTED, "gemm shape");
      n_part = launch_gemm_residual(ACT, static_cast<const float*>(L.wd), Xr, PART, nr, H, I, s);
      if (n_part < 0) return fail(WSG_ERR_UNSUPPORTED, "gemm shape");
      if (last_layer)   // the last row's final residual, for the head
        hipLaunchKernelGGL(k_row_residual, dim3(1), dim3(256), 0, s, Xr, PART, n_part, 1, H, 0,
                           static_cast<float*>(a.x));
    }
  }
  // the head and argmax that follow a to_head run advance the position past
  // the last row
  launch_set_pos(a.ctrl, to_head ? p0 + n - 1 : p0 + n, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WSG_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return WSG_OK;
}

}  // namespace wsg
