// Device helpers shared by the gfx950 kernels: wave64 reductions, vector
// loads and storage-dtype conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace wsg {

constexpr int kWave = 64;
constexpr int kBlock = 256;          // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;

// ---------------------------------------------------------------- DPP sums
// DPP control words (GFX9 encoding).
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror
constexpr int kDppBcast15 = 0x142;    // row_bcast:15
constexpr int kDppBcast31 = 0x143;    // row_bcast:31

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xF, false));
}

// Sum over each row of 16 lanes; every lane of the row receives the row sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppQuadSwap1>(v);
  v += dpp<kDppQuadSwap2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return v;
}

// Sum over each half-row of 8 lanes (every lane of the half-row gets it).
__device__ __forceinline__ float row8_sum(float v) {
  v += dpp<kDppQuadSwap1>(v);
  v += dpp<kDppQuadSwap2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v;
}

// Sum over the wavefront; the result is wave-uniform (read from lane 63).
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += dpp<kDppBcast15, 0xA>(v);   // rows 1, 3 += last lane of rows 0, 2
  v += dpp<kDppBcast31, 0xC>(v);   // rows 2, 3 += lane 31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppQuadSwap1>(v));
  v = fmaxf(v, dpp<kDppQuadSwap2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

// Cross-lane pairs from the gfx950 lane-swap instructions (VALU only, no
// LDS round trip).  Measured lane layout: swap32(x, y) gives a lane l of the
// lower half of the wave (x(l), x(l + 32)) and a lane of the upper half
// (y(l - 32), y(l)); swap16(x, y) likewise for lanes l and l ^ 16, with x
// paired in the even rows of 16 lanes and y in the odd ones.  Each lane so
// holds one value and its xor partner's, the lower lane's first; with x = y
// that is the plain xor-32 (xor-16) exchange, and with x != y the
// transposed step of a butterfly that halves the values a lane carries.
// Both results are read through one 64-bit value: subscripting the
// builtin's two-element result reads element 0 twice with this compiler.
struct LanePair { float lo, hi; };
__device__ __forceinline__ LanePair swap32(float x, float y) {
  const unsigned long long w = __builtin_bit_cast(
      unsigned long long, __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                           __builtin_bit_cast(unsigned, y), false, false));
  return {__builtin_bit_cast(float, (unsigned)w), __builtin_bit_cast(float, (unsigned)(w >> 32))};
}
__device__ __forceinline__ LanePair swap16(float x, float y) {
  const unsigned long long w = __builtin_bit_cast(
      unsigned long long, __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                           __builtin_bit_cast(unsigned, y), false, false));
  return {__builtin_bit_cast(float, (unsigned)w), __builtin_bit_cast(float, (unsigned)(w >> 32))};
}
__device__ __forceinline__ LanePair lanes_xor32(float x) { return swap32(x, x); }
__device__ __forceinline__ LanePair lanes_xor16(float x) { return swap16(x, x); }

// Maximum over the wavefront, in every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  LanePair p = lanes_xor16(v);
  v = fmaxf(p.lo, p.hi);
  p = lanes_xor32(v);
  return fmaxf(p.lo, p.hi);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ---------------------------------------------------------------- dtypes
template <typename T> struct Store;
template <> struct Store<float> {
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};
template <> struct Store<__half> {
  static __device__ __forceinline__ float to_f(__half v) { return __half2float(v); }
  static __device__ __forceinline__ __half from_f(float v) { return __float2half_rn(v); }
};

typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

// 16-byte vector of storage elements, widened to floats.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  float v[4];
  template <bool NT>
  __device__ __forceinline__ void load(const float* p) {
    f4_t t;
    if constexpr (NT) t = __builtin_nontemporal_load(reinterpret_cast<const f4_t*>(p));
    else t = *reinterpret_cast<const f4_t*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  }
};
template <> struct Vec16<__half> {
  static constexpr int N = 8;
  float v[8];
  template <bool NT>
  __device__ __forceinline__ void load(const __half* p) {
    u4_t t;
    if constexpr (NT) t = __builtin_nontemporal_load(reinterpret_cast<const u4_t*>(p));
    else t = *reinterpret_cast<const u4_t*>(p);
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __half2float(__ushort_as_half((unsigned short)(w[i] & 0xFFFFu)));
      v[2 * i + 1] = __half2float(__ushort_as_half((unsigned short)(w[i] >> 16)));
    }
  }
};

// Raw 16-byte loads (kept packed) for the FP16 dot2 path.
template <bool NT>
__device__ __forceinline__ uint4 load_u4(const void* p) {
  u4_t t;
  if constexpr (NT) t = __builtin_nontemporal_load(reinterpret_cast<const u4_t*>(p));
  else t = *reinterpret_cast<const u4_t*>(p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Lossless packed FP32 weights: an FP32 value whose low 16 bits are zero is
// stored as its high 16 bits (two values per 32-bit word, element 2i in the
// low half; Megakernels, "Lossless decode-weight storage").  Reconstruction
// (a shift or a mask) gives back the exact FP32 bit pattern.
struct bf16w { uint16_t b; };

// Weight vectors: four FP32 values per lane and load, in the same lane
// layout whether they are stored as FP32 (one 16-byte load) or packed (one
// 8-byte load), so the products and their summation order are identical.
template <typename T> struct WVec { using type = Vec16<T>; };
struct PackedVec4 {
  static constexpr int N = 4;
  float v[4];
  template <bool NT>
  __device__ __forceinline__ void load(const bf16w* p) {
    typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
    u2_t t;
    if constexpr (NT) t = __builtin_nontemporal_load(reinterpret_cast<const u2_t*>(p));
    else t = *reinterpret_cast<const u2_t*>(p);
    v[0] = __builtin_bit_cast(float, t.x << 16);
    v[1] = __builtin_bit_cast(float, t.x & 0xFFFF0000u);
    v[2] = __builtin_bit_cast(float, t.y << 16);
    v[3] = __builtin_bit_cast(float, t.y & 0xFFFF0000u);
  }
};
template <> struct WVec<bf16w> { using type = PackedVec4; };

// Four FP16 weights per 8-byte load, widened to FP32: the W_o slice vector
// of FP16 models, so that a lane covers four columns like the FP32 and
// packed slices (the layout the attention's register merge leaves in a lane).
struct Half4Vec {
  static constexpr int N = 4;
  float v[4];
  template <bool NT>
  __device__ __forceinline__ void load(const __half* p) {
    typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
    u2_t t;
    if constexpr (NT) t = __builtin_nontemporal_load(reinterpret_cast<const u2_t*>(p));
    else t = *reinterpret_cast<const u2_t*>(p);
    v[0] = __half2float(__ushort_as_half((unsigned short)(t.x & 0xFFFFu)));
    v[1] = __half2float(__ushort_as_half((unsigned short)(t.x >> 16)));
    v[2] = __half2float(__ushort_as_half((unsigned short)(t.y & 0xFFFFu)));
    v[3] = __half2float(__ushort_as_half((unsigned short)(t.y >> 16)));
  }
};

// int4 group-64 weights (tag type for the decode kernels): each matrix row
// holds K/8 32-bit words (nibble j of word w is k = 8w + j, low nibble
// first, a two's-complement value in [-8, 7]) followed by the row's K/64
// FP16 scales, one per group of 64 consecutive k; the weight is q * s.
// Rows are 16-byte aligned for every K that is a multiple of 1024 (the
// sizes this format supports).
struct q4w { uint32_t w; };
template <int K> struct Q4Row {
  static_assert(K % 1024 == 0, "int4 rows hold a multiple of 1024 weights");
  static constexpr int kWordBytes = K / 2;
  static constexpr int kBytes = K / 2 + K / 32;   // words, then FP16 scales
};
// Lane layout of the int4 decode GEMVs: 16 consecutive k (two words, one
// 8-byte load) per lane per 1024-wide chunk.
struct Q4Vec { static constexpr int N = 16; };
template <> struct WVec<q4w> { using type = Q4Vec; };

// ---------------------------------------------------------------- argmax
// Greedy selection with ties to the lowest token id (Megakernels, "GPU-wide
// end-to-end generation") as a maximum of 64-bit keys: the logit's bits in an
// order-preserving form (negative values complemented, non-negative ones with
// the sign bit set) above the complemented index, so a larger key is a larger
// logit, then a lower index.  -0.0 is folded into +0.0 first, so the two
// zeros tie.  Every key of an index below 2^31 is nonzero, so 0 is below all
// of them.  (A NaN orders by its bit pattern: logits are taken to be finite.)
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  if (v == 0.0f) v = 0.0f;
  uint32_t b = __float_as_uint(v);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)b << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}

// The index a key encodes.
__device__ __forceinline__ int argmax_key_index(unsigned long long k) {
  return (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
}

// Maximum key over the wavefront, in every lane: within rows of 16 by DPP
// (quad swaps, half-row and row mirrors), then across rows by the lane swaps.
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long k) {
  const unsigned lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, 0xF, 0xF, false);
  const unsigned hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
  return ((unsigned long long)hi << 32) | lo;
}
template <bool X32>
__device__ __forceinline__ unsigned long long max_xor_u64(unsigned long long k) {
  const float lo = __uint_as_float((uint32_t)k), hi = __uint_as_float((uint32_t)(k >> 32));
  const LanePair a = X32 ? lanes_xor32(lo) : lanes_xor16(lo);
  const LanePair b = X32 ? lanes_xor32(hi) : lanes_xor16(hi);
  const unsigned long long k0 = ((unsigned long long)__float_as_uint(b.lo) << 32) | __float_as_uint(a.lo);
  const unsigned long long k1 = ((unsigned long long)__float_as_uint(b.hi) << 32) | __float_as_uint(a.hi);
  return k1 > k0 ? k1 : k0;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long k) {
  unsigned long long o = dpp_u64<kDppQuadSwap1>(k);
  k = o > k ? o : k;
  o = dpp_u64<kDppQuadSwap2>(k);
  k = o > k ? o : k;
  o = dpp_u64<kDppHalfMirror>(k);
  k = o > k ? o : k;
  o = dpp_u64<kDppMirror>(k);
  k = o > k ? o : k;
  k = max_xor_u64<false>(k);
  return max_xor_u64<true>(k);
}

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }

// acc + a.x*b.x + a.y*b.y with FP32 accumulation (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(h2_t a, h2_t b, float acc) {
  return __builtin_amdgcn_fdot2(a, b, acc, false);
}

}  // namespace wsg
