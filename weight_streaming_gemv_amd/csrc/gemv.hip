// Weight-streaming GEMV family for gfx950: FP32 and FP16 weights, int4
// group-64 weights, one or two input vectors, R output rows per wavefront.
//
// One wavefront owns a group of R consecutive output rows and streams those
// rows with 16-byte loads, 64 lanes side by side, so each wave-wide load
// instruction reads 1 KiB of contiguous weights.  Partial sums stay in
// lanes (FP32) and are combined with DPP row operations at the end.  The
// design follows the row-per-SIMD-group GEMV of Megakernels ("GPU-wide
// end-to-end generation") re-shaped for 64-lane waves, with R as the tuning
// constant of Our Kernel Benchmark Was Measuring the System Cache ("Why it
// mattered": fewer rows per group give more loads in flight when the
// weights come from DRAM).
#include "common.hpp"
#include "gemv.hpp"

namespace wsg {

// ------------------------------------------------------------ FP32, fixed K
template <int K, int R, int T, bool NT>
__global__ __launch_bounds__(kBlock) void k_gemv_f32(const float* __restrict__ W,
                                                     const float* __restrict__ X,
                                                     float* __restrict__ Y, int M) {
  constexpr int NV = K / 256;  // float4 chunks per lane per row
  static_assert(K % 256 == 0, "K must be a multiple of 256");
  const int lane = lane_id();
  float4 x[T][NV];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < NV; ++c) x[t][c] = *reinterpret_cast<const float4*>(X + t * K + c * 256 + lane * 4);

  const int ngroups = (M + R - 1) / R;
  for (int g = blockIdx.x * kWavesPerBlock + wave_id(); g < ngroups; g += gridDim.x * kWavesPerBlock) {
    const int row0 = g * R;
    float acc[R][T];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[r][t] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float* wr = W + (size_t)min(row0 + r, M - 1) * K + lane * 4;
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        Vec16<float> w;
        w.load<NT>(wr + c * 256);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          float a = acc[r][t];
          a = fmaf(w.v[0], x[t][c].x, a);
          a = fmaf(w.v[1], x[t][c].y, a);
          a = fmaf(w.v[2], x[t][c].z, a);
          a = fmaf(w.v[3], x[t][c].w, a);
          acc[r][t] = a;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float s = wave_sum(acc[r][t]);
        if (lane == 0 && row0 + r < M) Y[(size_t)t * M + row0 + r] = s;
      }
  }
}

// ------------------------------------------- FP32, two waves per row
// One wave per row holds the lane's K/64 activations and, to keep the row's
// loads in flight, as many weights: at K = 3072 that is 96 registers, and
// the compiler instead held the weight loads back (60 registers, loads
// issued a few at a time).  Here two waves of a workgroup share each row,
// each streaming one half of it (and holding that half of the activations):
// half the registers per wave and twice the waves for the same rows.  The
// two wave sums meet in LDS and are added once, half 0 first.  Workgroup b
// serves rows 2b and 2b + 1 (waves 0, 1 and 2, 3), then b + gridDim.x, ...
template <int K, int T, bool NT>
__global__ __launch_bounds__(kBlock) void k_gemv_f32_split2(const float* __restrict__ W,
                                                            const float* __restrict__ X,
                                                            float* __restrict__ Y, int M) {
  constexpr int KH = K / 2;
  constexpr int NV = KH / 256;  // float4 chunks per lane per half row
  static_assert(KH % 256 == 0, "K must be a multiple of 512");
  const int lane = lane_id();
  const int wv = wave_id();
  const int h = wv & 1;
  float4 x[T][NV];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < NV; ++c)
      x[t][c] = *reinterpret_cast<const float4*>(X + (size_t)t * K + h * KH + c * 256 + lane * 4);
  __shared__ float half_sum[kWavesPerBlock][T];
  const int npairs = (M + 1) / 2;
  // the loop bound depends on the workgroup only, so its barriers are uniform
  for (int b = blockIdx.x; b < npairs; b += gridDim.x) {
    const int row = 2 * b + (wv >> 1);
    const float* wr = W + (size_t)min(row, M - 1) * K + h * KH + lane * 4;
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.f;
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      Vec16<float> w;
      w.load<NT>(wr + c * 256);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float a = acc[t];
        a = fmaf(w.v[0], x[t][c].x, a);
        a = fmaf(w.v[1], x[t][c].y, a);
        a = fmaf(w.v[2], x[t][c].z, a);
        a = fmaf(w.v[3], x[t][c].w, a);
        acc[t] = a;
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float sum = wave_sum(acc[t]);
      if (lane == 0) half_sum[wv][t] = sum;
    }
    __syncthreads();
    if (h == 0 && lane == 0 && row < M)
#pragma unroll
      for (int t = 0; t < T; ++t) Y[(size_t)t * M + row] = half_sum[wv][t] + half_sum[wv + 1][t];
    __syncthreads();  // the next pair rewrites half_sum
  }
}

// ------------------------------------------------------------ FP16, fixed K
// Weights and activations stay packed as half pairs; v_dot2_f32_f16 forms
// the exact FP16 products and adds them into an FP32 accumulator.
template <int K, int R, int T, bool NT>
__global__ __launch_bounds__(kBlock) void k_gemv_f16(const __half* __restrict__ W,
                                                     const __half* __restrict__ X,
                                                     float* __restrict__ Y, int M) {
  constexpr int NV = K / 512;  // 8-half chunks per lane per row
  static_assert(K % 512 == 0, "K must be a multiple of 512");
  const int lane = lane_id();
  uint4 x[T][NV];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < NV; ++c) x[t][c] = *reinterpret_cast<const uint4*>(X + t * K + c * 512 + lane * 8);

  const int ngroups = (M + R - 1) / R;
  for (int g = blockIdx.x * kWavesPerBlock + wave_id(); g < ngroups; g += gridDim.x * kWavesPerBlock) {
    const int row0 = g * R;
    float acc[R][T];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[r][t] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const __half* wr = W + (size_t)min(row0 + r, M - 1) * K + lane * 8;
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        const uint4 w = load_u4<NT>(wr + c * 512);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          float a = acc[r][t];
          a = dot2(as_h2(w.x), as_h2(x[t][c].x), a);
          a = dot2(as_h2(w.y), as_h2(x[t][c].y), a);
          a = dot2(as_h2(w.z), as_h2(x[t][c].z), a);
          a = dot2(as_h2(w.w), as_h2(x[t][c].w), a);
          acc[r][t] = a;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float s = wave_sum(acc[r][t]);
        if (lane == 0 && row0 + r < M) Y[(size_t)t * M + row0 + r] = s;
      }
  }
}

// ------------------------------------------------- any K (multiple of VEC)
// Run-time K: full 64-lane chunks plus a partial last chunk; activations are
// read from global memory (cached) instead of registers.
template <typename TW, int R, int T>
__global__ __launch_bounds__(kBlock) void k_gemv_anyk(const TW* __restrict__ W, const TW* __restrict__ X,
                                                      float* __restrict__ Y, int M, int K) {
  constexpr int VEC = Vec16<TW>::N;
  const int lane = lane_id();
  const int ngroups = (M + R - 1) / R;
  for (int g = blockIdx.x * kWavesPerBlock + wave_id(); g < ngroups; g += gridDim.x * kWavesPerBlock) {
    const int row0 = g * R;
    float acc[R][T];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[r][t] = 0.f;
    for (int k = lane * VEC; k < K; k += kWave * VEC) {
      Vec16<TW> xv[T];
#pragma unroll
      for (int t = 0; t < T; ++t) xv[t].template load<false>(X + (size_t)t * K + k);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        Vec16<TW> w;
        w.template load<false>(W + (size_t)min(row0 + r, M - 1) * K + k);
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[r][t] = fmaf(w.v[i], xv[t].v[i], acc[r][t]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float s = wave_sum(acc[r][t]);
        if (lane == 0 && row0 + r < M) Y[(size_t)t * M + row0 + r] = s;
      }
  }
}

// ------------------------------------------------- scalar fallback (any K)
template <typename TW, int T>
__global__ __launch_bounds__(kBlock) void k_gemv_scalar(const TW* __restrict__ W, const TW* __restrict__ X,
                                                        float* __restrict__ Y, int M, int K) {
  const int lane = lane_id();
  for (int row = blockIdx.x * kWavesPerBlock + wave_id(); row < M; row += gridDim.x * kWavesPerBlock) {
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.f;
    for (int k = lane; k < K; k += kWave) {
      const float w = Store<TW>::to_f(W[(size_t)row * K + k]);
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] = fmaf(w, Store<TW>::to_f(X[(size_t)t * K + k]), acc[t]);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0) Y[(size_t)t * M + row] = s;
    }
  }
}

// ------------------------------------------------------------ int4 group-64
// Each lane reads 16 bytes = 32 consecutive weights = half of one group, so a
// lane needs exactly one scale per chunk.  Nibbles are decoded two at a time
// into FP16 pairs by OR-ing them under the exponent of 1024 and subtracting
// 1032 (after flipping bit 3, which maps two's complement onto offset
// binary); every step is exact.  The activations are staged once per
// workgroup in LDS, permuted so that each FP16 pair lines up with the
// nibble pair (j, j+4) that one 32-bit word yields, and placed so that the
// 64 lanes of a wave read 64 consecutive 16-byte LDS slots (lane l's word i
// of chunk c sits at c*256 + i*64 + l): no bank conflicts.
// Eight FP16 activations (halves 0..7 of one 16-byte word) as the pairs
// (0,4) (1,5) (2,6) (3,7) that the nibble pairs of one weight word meet.
__device__ __forceinline__ uint4 nibble_pair_order(uint4 h) {
  uint4 p;
  p.x = (h.x & 0xFFFFu) | (h.z << 16);
  p.y = (h.x >> 16) | (h.z & 0xFFFF0000u);
  p.z = (h.y & 0xFFFFu) | (h.w << 16);
  p.w = (h.y >> 16) | (h.w & 0xFFFF0000u);
  return p;
}

template <int K, int R, int T, bool NT, int WV = kWavesPerBlock>
__global__ __launch_bounds__(64 * WV) void k_gemv_q4(const uint32_t* __restrict__ Wq,
                                                    const __half* __restrict__ S,
                                                    const __half* __restrict__ X,
                                                    float* __restrict__ Y, int M) {
  constexpr int NV = K / 2048;   // 16-byte chunks per lane per row
  constexpr int W8 = K / 8;      // words per row
  constexpr int G = K / 64;      // groups (scales) per row
  static_assert(K % 2048 == 0, "fixed-K int4 kernel needs K % 2048 == 0");
  __shared__ uint4 xs[T][W8];
  constexpr int kThreads = 64 * WV;
  constexpr int kStage = (T * W8 + kThreads - 1) / kThreads;
  constexpr bool kRagged = (T * W8) % kThreads != 0;   // the last round is partial
  // all staging loads in flight at once, then the permuted LDS stores
  uint4 hx[kStage];
#pragma unroll
  for (int it = 0; it < kStage; ++it) {
    int i = threadIdx.x + it * kThreads;
    if constexpr (kRagged) i = min(i, T * W8 - 1);   // a partial round re-reads the last word
    const int t = i / W8, gi = i - t * W8;
    hx[it] = *reinterpret_cast<const uint4*>(X + (size_t)t * K + gi * 8);
  }
  const int lane = lane_id();
  const int ngroups = (M + R - 1) / R;
  // One row per wave in 4-wave workgroups (two 16-byte chunks per lane at
  // most): the wave's first row is issued before the staging barrier, right
  // after the activation loads, so its latency overlaps the staging instead
  // of following it, and each next row is issued before the current one is
  // reduced.  Larger groups keep chunk-by-chunk loads: holding them costs
  // registers (occupancy) that the measured sweep valued more.
  constexpr bool kPre = R == 1 && WV == kWavesPerBlock && NV <= 2;
  constexpr int PN = kPre ? NV : 1;
  uint4 wq[PN];
  __half ws[PN];
  auto load_row = [&](int row) {
#pragma unroll
    for (int c = 0; c < PN; ++c) {
      wq[c] = load_u4<NT>(Wq + (size_t)row * W8 + c * 256 + lane * 4);
      ws[c] = S[(size_t)row * G + c * 32 + (lane >> 1)];
    }
  };
  int g = blockIdx.x * WV + wave_id();
  // (a wave with no row reads the last row and discards it)
  if constexpr (kPre) {
    load_row(min(g, M - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int it = 0; it < kStage; ++it) {
    const int i = threadIdx.x + it * kThreads;
    if (kRagged && i >= T * W8) break;
    const int t = i / W8, gi = i - t * W8;
    const int c = gi >> 8, w = gi & 255;
    xs[t][(c << 8) + ((w & 3) << 6) + (w >> 2)] = nibble_pair_order(hx[it]);
  }
  __syncthreads();

  const h2_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  if constexpr (kPre) {
    for (; g < M; g += gridDim.x * WV) {
      float acc[T];
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] = 0.f;
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        const uint32_t ww[4] = {wq[c].x, wq[c].y, wq[c].z, wq[c].w};
        float inner[T];
#pragma unroll
        for (int t = 0; t < T; ++t) inner[t] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t v = ww[i] ^ 0x88888888u;
          const h2_t p0 = as_h2((v & 0x000F000Fu) | 0x64006400u) - bias;
          const h2_t p1 = as_h2(((v >> 4) & 0x000F000Fu) | 0x64006400u) - bias;
          const h2_t p2 = as_h2(((v >> 8) & 0x000F000Fu) | 0x64006400u) - bias;
          const h2_t p3 = as_h2(((v >> 12) & 0x000F000Fu) | 0x64006400u) - bias;
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const uint4 xv = xs[t][c * 256 + i * 64 + lane];
            float a = inner[t];
            a = dot2(p0, as_h2(xv.x), a);
            a = dot2(p1, as_h2(xv.y), a);
            a = dot2(p2, as_h2(xv.z), a);
            a = dot2(p3, as_h2(xv.w), a);
            inner[t] = a;
          }
        }
        const float sc = __half2float(ws[c]);
#pragma unroll
        for (int t = 0; t < T; ++t) acc[t] = fmaf(sc, inner[t], acc[t]);
      }
      const int next = g + gridDim.x * WV;
      if (next < M) load_row(next);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float s = wave_sum(acc[t]);
        if (lane == 0) Y[(size_t)t * M + g] = s;
      }
    }
    return;
  }
  for (; g < ngroups; g += gridDim.x * WV) {
    const int row0 = g * R;
    float acc[R][T];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[r][t] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const size_t row = (size_t)min(row0 + r, M - 1);
      // Partial unroll keeps long rows (K = 14336) from using every VGPR;
      // the unroll depth is the number of 16-byte chunks a wave has in
      // flight.  One row per wave: 4 (cold 4096 x 14336, one row of X:
      // 9.44 -> 8.78 us against 2, 9.0 with 3; all 7 spill); larger groups 2.
#pragma unroll(R == 1 ? 4 : 2)
      for (int c = 0; c < NV; ++c) {
        const uint4 w = load_u4<NT>(Wq + row * W8 + c * 256 + lane * 4);
        const float sc = __half2float(S[row * G + c * 32 + (lane >> 1)]);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        float inner[T];
#pragma unroll
        for (int t = 0; t < T; ++t) inner[t] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t v = ww[i] ^ 0x88888888u;
          const h2_t p0 = as_h2((v & 0x000F000Fu) | 0x64006400u) - bias;
          const h2_t p1 = as_h2(((v >> 4) & 0x000F000Fu) | 0x64006400u) - bias;
          const h2_t p2 = as_h2(((v >> 8) & 0x000F000Fu) | 0x64006400u) - bias;
          const h2_t p3 = as_h2(((v >> 12) & 0x000F000Fu) | 0x64006400u) - bias;
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const uint4 xv = xs[t][c * 256 + i * 64 + lane];
            float a = inner[t];
            a = dot2(p0, as_h2(xv.x), a);
            a = dot2(p1, as_h2(xv.y), a);
            a = dot2(p2, as_h2(xv.z), a);
            a = dot2(p3, as_h2(xv.w), a);
            inner[t] = a;
          }
        }
#pragma unroll
        for (int t = 0; t < T; ++t) acc[r][t] = fmaf(sc, inner[t], acc[r][t]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float s = wave_sum(acc[r][t]);
        if (lane == 0 && row0 + r < M) Y[(size_t)t * M + row0 + r] = s;
      }
  }
}

// int4, any K % 64 == 0: one 16-byte chunk per lane per step, run-time loop;
// activations read directly from global memory.
template <int R, int T>
__global__ __launch_bounds__(kBlock) void k_gemv_q4_anyk(const uint32_t* __restrict__ Wq,
                                                         const __half* __restrict__ S,
                                                         const __half* __restrict__ X,
                                                         float* __restrict__ Y, int M, int K) {
  const int lane = lane_id();
  const int W8 = K / 8, G = K / 64;
  const int ngroups = (M + R - 1) / R;
  for (int g = blockIdx.x * kWavesPerBlock + wave_id(); g < ngroups; g += gridDim.x * kWavesPerBlock) {
    const int row0 = g * R;
    float acc[R][T];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[r][t] = 0.f;
    // word index = 4*lane + 256*step; K/8 words per row, multiple of 8
    for (int wi = lane * 4; wi < W8; wi += kWave * 4) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const size_t row = (size_t)min(row0 + r, M - 1);
        const uint4 w = *reinterpret_cast<const uint4*>(Wq + row * W8 + wi);
        const float sc = __half2float(S[row * G + wi / 8]);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int t = 0; t < T; ++t) {
          float inner = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t v = ww[i];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int q = (int)((v >> (4 * j)) & 0xFu);
              const float qf = (float)(q >= 8 ? q - 16 : q);
              inner = fmaf(qf, __half2float(X[(size_t)t * K + (wi + i) * 8 + j]), inner);
            }
          }
          acc[r][t] = fmaf(sc, inner, acc[r][t]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float s = wave_sum(acc[r][t]);
        if (lane == 0 && row0 + r < M) Y[(size_t)t * M + row0 + r] = s;
      }
  }
}

// ------------------------------------------------------------ dispatch
namespace {

int default_grid(int M, int R, int grid_blocks) {
  const int ngroups = (M + R - 1) / R;
  const int one_shot = (ngroups + kWavesPerBlock - 1) / kWavesPerBlock;
  if (grid_blocks > 0) return grid_blocks < one_shot ? grid_blocks : one_shot;
  return one_shot;
}

#define WSG_LAUNCH_FIXED(KERNEL, KK)                                                         \
  if (K == KK) {                                                                             \
    if (nt) hipLaunchKernelGGL((KERNEL<KK, R, T, true>), dim3(grid), dim3(kBlock), 0, s, W, X, Y, M);  \
    else hipLaunchKernelGGL((KERNEL<KK, R, T, false>), dim3(grid), dim3(kBlock), 0, s, W, X, Y, M);    \
    return true;                                                                             \
  }

template <int R, int T>
bool launch_f32_fixed(int M, int K, int grid, bool nt, const float* W, const float* X, float* Y, hipStream_t s) {
  WSG_LAUNCH_FIXED(k_gemv_f32, 1024)
  WSG_LAUNCH_FIXED(k_gemv_f32, 2048)
  WSG_LAUNCH_FIXED(k_gemv_f32, 3072)
  return false;
}
template <int R, int T>
bool launch_f16_fixed(int M, int K, int grid, bool nt, const __half* W, const __half* X, float* Y, hipStream_t s) {
  WSG_LAUNCH_FIXED(k_gemv_f16, 1024)
  WSG_LAUNCH_FIXED(k_gemv_f16, 2048)
  WSG_LAUNCH_FIXED(k_gemv_f16, 3072)
  return false;
}
#undef WSG_LAUNCH_FIXED

// FP32, K = 1024, 2048 or 3072 (checked by the entry point), one row per
// two waves: one workgroup per row pair unless fewer are asked for.
template <int T>
void launch_f32_split2(int M, int K, int grid_req, bool nt, const float* W, const float* X, float* Y,
                       hipStream_t s) {
  const int npairs = (M + 1) / 2;
  const int grid = grid_req > 0 && grid_req < npairs ? grid_req : npairs;
#define WSG_SPLIT2(KK)                                                                                        \
  if (K == KK) {                                                                                              \
    if (nt) hipLaunchKernelGGL((k_gemv_f32_split2<KK, T, true>), dim3(grid), dim3(kBlock), 0, s, W, X, Y, M);  \
    else hipLaunchKernelGGL((k_gemv_f32_split2<KK, T, false>), dim3(grid), dim3(kBlock), 0, s, W, X, Y, M);    \
    return;                                                                                                   \
  }
  WSG_SPLIT2(1024)
  WSG_SPLIT2(2048)
  WSG_SPLIT2(3072)
#undef WSG_SPLIT2
}

template <int R, int T>
void launch_dense(int dtype, int M, int K, int grid_req, bool nt, const void* W, const void* X, float* Y,
                  hipStream_t s) {
  const int grid = default_grid(M, R, grid_req);
  if (dtype == 0) {
    const float* w = static_cast<const float*>(W);
    const float* x = static_cast<const float*>(X);
    if (launch_f32_fixed<R, T>(M, K, grid, nt, w, x, Y, s)) return;
    if (K % 4 == 0) hipLaunchKernelGGL((k_gemv_anyk<float, R, T>), dim3(grid), dim3(kBlock), 0, s, w, x, Y, M, K);
    else hipLaunchKernelGGL((k_gemv_scalar<float, T>), dim3(default_grid(M, 1, grid_req)), dim3(kBlock), 0, s, w, x, Y, M, K);
  } else {
    const __half* w = static_cast<const __half*>(W);
    const __half* x = static_cast<const __half*>(X);
    if (launch_f16_fixed<R, T>(M, K, grid, nt, w, x, Y, s)) return;
    if (K % 8 == 0) hipLaunchKernelGGL((k_gemv_anyk<__half, R, T>), dim3(grid), dim3(kBlock), 0, s, w, x, Y, M, K);
    else hipLaunchKernelGGL((k_gemv_scalar<__half, T>), dim3(default_grid(M, 1, grid_req)), dim3(kBlock), 0, s, w, x, Y, M, K);
  }
}

template <int R, int T>
void launch_q4(int M, int K, int grid_req, bool nt, const uint32_t* Wq, const __half* S, const __half* X,
               float* Y, hipStream_t s) {
  const int grid = default_grid(M, R, grid_req);
#define WSG_Q4(KK)                                                                                         \
  if (K == KK) {                                                                                           \
    if (nt) hipLaunchKernelGGL((k_gemv_q4<KK, R, T, true>), dim3(grid), dim3(kBlock), 0, s, Wq, S, X, Y, M); \
    else hipLaunchKernelGGL((k_gemv_q4<KK, R, T, false>), dim3(grid), dim3(kBlock), 0, s, Wq, S, X, Y, M);  \
    return;                                                                                                \
  }
  WSG_Q4(4096)
#undef WSG_Q4
  if (K == 14336) {
    // long rows: workgroups of 16 / R waves (16 at one row per wave, 8 at
    // two, 4 beyond), so one LDS copy of the 28 KiB (per row of X)
    // activations serves up to four times the waves while a 4096-row matrix
    // still fills 256 workgroups (cold sweep of 4096 x 14336: 16 waves at
    // R = 1, 10.5 -> 9.4 us for one row of X and 15.3 -> 11.0 us for two;
    // 8 and 4 waves instead of 16 at R = 2 and 4, 14.7 -> 13.2 and
    // 25.9 -> 20.9 us)
    constexpr int WV = R == 1 ? 16 : R == 2 ? 8 : 4;
    const int ngroups = (M + R - 1) / R;
    const int one_shot = (ngroups + WV - 1) / WV;
    const int g16 = grid_req > 0 && grid_req < one_shot ? grid_req : one_shot;
    if (nt) hipLaunchKernelGGL((k_gemv_q4<14336, R, T, true, WV>), dim3(g16), dim3(64 * WV), 0, s, Wq, S, X, Y, M);
    else hipLaunchKernelGGL((k_gemv_q4<14336, R, T, false, WV>), dim3(g16), dim3(64 * WV), 0, s, Wq, S, X, Y, M);
    return;
  }
  hipLaunchKernelGGL((k_gemv_q4_anyk<R, T>), dim3(grid), dim3(kBlock), 0, s, Wq, S, X, Y, M, K);
}

}  // namespace

void gemv_dispatch(int dtype, int M, int K, int T, int R, int grid, int flags, const void* W, const void* X,
                   float* Y, hipStream_t s) {
  const bool nt = (flags & 1) != 0;
  if (flags & 2) {
    const float* w = static_cast<const float*>(W);
    const float* x = static_cast<const float*>(X);
    if (T == 1) launch_f32_split2<1>(M, K, grid, nt, w, x, Y, s);
    else launch_f32_split2<2>(M, K, grid, nt, w, x, Y, s);
    return;
  }
#define WSG_DR(RR)                                                             \
  case RR:                                                                     \
    if (T == 1) launch_dense<RR, 1>(dtype, M, K, grid, nt, W, X, Y, s);        \
    else launch_dense<RR, 2>(dtype, M, K, grid, nt, W, X, Y, s);               \
    break;
  switch (R) { WSG_DR(1) WSG_DR(2) WSG_DR(4) WSG_DR(8) default: break; }
#undef WSG_DR
}

void gemv_q4_dispatch(int M, int K, int T, int R, int grid, int flags, const uint32_t* Wq, const void* S,
                      const void* X, float* Y, hipStream_t s) {
  const bool nt = (flags & 1) != 0;
  const __half* sc = static_cast<const __half*>(S);
  const __half* x = static_cast<const __half*>(X);
#define WSG_QR(RR)                                                             \
  case RR:                                                                     \
    if (T == 1) launch_q4<RR, 1>(M, K, grid, nt, Wq, sc, x, Y, s);             \
    else launch_q4<RR, 2>(M, K, grid, nt, Wq, sc, x, Y, s);                    \
    break;
  switch (R) { WSG_QR(1) WSG_QR(2) WSG_QR(4) WSG_QR(8) default: break; }
#undef WSG_QR
}

// ------------------------------------------------------ streaming ceiling
// Read-only streaming reference for the cold-cache sweep: each wave sums
// one contiguous 4 KiB segment of the buffer with 16-byte non-temporal
// loads (the same access size, per-wave footprint and load form as a
// 1024-float decode GEMV row), all loads in flight at once.  The sum is stored only if it equals an improbable value,
// which keeps every load live without writing anything in practice.
namespace {
constexpr int kStreamSeg = 4096;            // bytes per wave
constexpr int kStreamVec = kStreamSeg / (64 * 16);

__global__ __launch_bounds__(256) void k_stream_read(const f4_t* __restrict__ buf, int64_t n_vec,
                                                     float* __restrict__ out) {
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t base = wave * (kStreamSeg / 16) + lane;
  f4_t v[kStreamVec];
#pragma unroll
  for (int i = 0; i < kStreamVec; ++i) v[i] = __builtin_nontemporal_load(buf + min(base + 64 * i, n_vec - 1));
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kStreamVec; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  if (sum == 1.2345678e-30f) out[0] = sum;
}
}  // namespace

void stream_read_dispatch(const void* buf, int64_t bytes, float* out, hipStream_t s) {
  const int64_t seg_per_block = 4 * (int64_t)kStreamSeg;
  const int64_t blocks = (bytes + seg_per_block - 1) / seg_per_block;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const f4_t*>(buf),
                     bytes / 16, out);
}

}  // namespace wsg
