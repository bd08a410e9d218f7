// Device helpers shared by the gfx950 kernels of libloki: storage-type
// unpacking, RNE rounding to bf16, the order-preserving score key, and
// wave64 reductions built on DPP row operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loki {

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32 bit pattern)

// ---------------------------------------------------------------- storage types

// A 16-byte granule holds 4 fp32 or 8 bf16 elements; element 0 sits in the
// low half of the first dword (little-endian).
template <typename T> struct Gran;

template <> struct Gran<float> {
  static constexpr int N = 4;
  __device__ static __forceinline__ void unpack(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
};

template <> struct Gran<bf16_t> {
  static constexpr int N = 8;
  __device__ static __forceinline__ void unpack(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x << 16); x[1] = __uint_as_float(v.x & 0xffff0000u);
    x[2] = __uint_as_float(v.y << 16); x[3] = __uint_as_float(v.y & 0xffff0000u);
    x[4] = __uint_as_float(v.z << 16); x[5] = __uint_as_float(v.z & 0xffff0000u);
    x[6] = __uint_as_float(v.w << 16); x[7] = __uint_as_float(v.w & 0xffff0000u);
  }
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Round-to-nearest-even fp32 -> bf16: add half an ulp of the kept part minus
// one, plus the kept part's lowest bit, then truncate.  NaNs stay quiet NaNs.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// ---------------------------------------------------------------- ragged batches

// Cached tokens of sequence b: its length clamped into [1, S], or the whole
// capacity S when no lengths are given.
__device__ __forceinline__ int seq_len(const int32_t* lens, int b, int S) {
  return lens ? min(max(lens[b], 1), S) : S;
}

// ---------------------------------------------------------------- score keys

// Order-preserving map fp32 -> uint32: a < b (as reals) iff key(a) < key(b).
// -0.0 is folded onto +0.0 first so equal reals get equal keys.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---------------------------------------------------------------- wave64 reductions

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of L consecutive lanes (L a power of two <= 64).
// Every lane of a group ends with the same bits: each step adds a lane's value
// to that of its partner under an involution (quad swaps, then the half-row
// and row mirrors), and fp addition is commutative.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (L >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (L >= 16) v += dpp_f<0x140>(v); // row_mirror
  if constexpr (L >= 32) v += __shfl_xor(v, 16);
  if constexpr (L >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Number of set bits of a 64-lane mask strictly below this lane.
__device__ __forceinline__ int bits_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace loki
