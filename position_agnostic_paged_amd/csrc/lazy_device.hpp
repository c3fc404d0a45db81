// Device-side building blocks for gfx950 (CDNA4): fragment types, MFMA
// wrappers, the tile-word unpack and the pairwise rotation.
//
// Wave-level fragment convention used by every attention kernel.  A 64-lane
// wave is split as lane = 16 * g + r (r = lane % 16, g = lane / 16).  One
// "mma32" step computes C[16][16] += A[16][32] * B[32][16] where lane
// (g, r) supplies eight A values of row r and eight B values of column r for
// the eight contraction slots (g, t), t = 0..7.  The result lands as
// C[4g + j][r] in accumulator register j.  bf16 uses one
// v_mfma_f32_16x16x32_bf16 (slot (g,t) = k 8g+t); fp32 uses eight
// v_mfma_f32_16x16x4_f32 (instruction t, slot (g,t) = k 4t+g).  Because both
// operands follow the same slot map, any assignment of the contraction index
// to slots is a valid product; the kernels pick the one that makes every lane's
// eight values contiguous in memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lazy {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kBlock = 16;  // tokens per paged block (= one tile)

// ------------------------------------------------------------------ tile word
// 64-bit word: block id [63:40] | offset [39:16] | valid-slot mask [15:0]
// (bit-packed (block id, offset, mask) metadata split by register shifts,
// LazyAttention notes, "Key designs").
struct TileMeta {
  int32_t block;
  int32_t offset;
  uint32_t mask;
};

__device__ __forceinline__ TileMeta unpack_word(uint64_t w) {
  TileMeta t;
  t.block = (int32_t)(w >> 40);
  t.offset = (int32_t)((w >> 16) & 0xFFFFFFull);
  t.mask = (uint32_t)(w & 0xFFFFull);
  return t;
}

// --------------------------------------------------------------- element types
template <typename T>
struct Elem;

template <>
struct Elem<bf16> {
  using Frag8 = bf16x8;  // 8 contraction values of one lane
  using Frag4 = bf16x4;  // 4 tokens of one V channel
  static __device__ __forceinline__ f32x4 mma(const Frag8& a, const Frag8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
  static __device__ __forceinline__ bf16 from_f(float x) { return (bf16)x; }
};

template <>
struct Elem<float> {
  using Frag8 = f32x8;
  using Frag4 = f32x4;
  static __device__ __forceinline__ f32x4 mma(const Frag8& a, const Frag8& b, f32x4 c) {
#pragma unroll
    for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};

template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag8 load8(const T* p) {
  return *reinterpret_cast<const typename Elem<T>::Frag8*>(p);
}
template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag4 load4(const T* p) {
  return *reinterpret_cast<const typename Elem<T>::Frag4*>(p);
}

// Cache-policy operand of a direct global->LDS copy with the nontemporal
// (streaming) bit.  On MI355X a plain 2 GiB read stream of whole 1 KiB
// wave-contiguous pieces measured 7.1-7.2 TB/s with it against 6.2-6.3
// TB/s with the default policy, for register loads and for these copies
// alike; reads of 64-byte row pieces (the decode kernel's K fragments) drop
// to 5.9 TB/s with it, and data that other workgroups re-read through L2
// loses its hits, so of the copies only the document pass's use it.
constexpr int kCopyAuxStream = 2;

// A V fragment load of the per-wave kernels with the nontemporal hint: each
// instruction reads 16 channel rows x 32 bytes, whole lines, so the hint
// pays (no-sharing 64 x 32K decode 1.335 -> 1.182 ms on MI355X, 6.3 -> 7.1
// TB/s); where many requests re-read the same V through L2 it costs a few
// percent (128 x 16K MQA decode over shared documents 0.142 -> 0.147 ms).
template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag4 load4_stream(const T* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const typename Elem<T>::Frag4*>(p));
}

// -------------------------------------------------------------- misc helpers
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float xor_max16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
__device__ __forceinline__ float xor_sum16_32(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

constexpr float kLog2e = 1.4426950408889634f;

// cos/sin of p * theta for the on-the-fly coefficient path.  The angle is
// formed in fp64 (an fp32 product would be off by up to ulp(p) radians at
// large offsets), reduced into [-pi, pi] by a two-constant Cody-Waite step
// (2 pi = C1 + C2, both fp64), then evaluated in fp32.
__device__ __forceinline__ void sincos_reduced(int p, double theta, float* s, float* c) {
  const double phi = (double)p * theta;
  const double n = rint(phi * 0.15915494309189535);  // 1 / (2 pi)
  double red = fma(-n, 6.283185307179586, phi);      // C1 = fp64(2 pi)
  red = fma(-n, 2.4492935982947064e-16, red);        // C2 = 2 pi - C1
  sincosf((float)red, s, c);
}

}  // namespace lazy
