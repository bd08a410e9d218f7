// MFMA operand helpers shared by the bf16 decode kernels: the operand
// types of v_mfma_f32_16x16x32_bf16, the query operands built from the
// three-part bf16 split of q_rot (q = h + m + l, part 3 zero), and the sums
// that finish a score from its split partial products.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l, element i):
//   A[m][k] : m = l % 16, k = 8 (l / 16) + i
//   B[k][n] : n = l % 16, k = 8 (l / 16) + i
//   D[m][n] : n = l % 16, m = 4 (l / 16) + v   (v = 0..3, one fp32 each)
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace loki {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// Lane n (< 4) of each 16-lane row receives x[n] + x[n+4] + x[n+8] + x[n+12]
// of its row: DPP row_shl:4 then row_shl:8 (lane i reads lane i + k of its
// row; reads past the row's end give 0).
__device__ __forceinline__ float add_split_columns(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x104, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x108, 0xF, 0xF, false));
  return x;
}

// B operand of column group `grp` for the 8 dims starting at dim0 (a
// multiple of 8): column n = head 4 grp + (n % 4), split part n / 4 (part 3
// is the zero row), read with one 16-byte load from qsplit[row][part][d].
// Elements at dims >= r are zeroed.
__device__ __forceinline__ bf16x8_t q_operand(const uint16_t* __restrict__ qsplit, size_t head0, int d,
                                              int G, int r, int grp, int n, int dim0) {
  const int g = 4 * grp + (n & 3), part = n >> 2;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (g < G && dim0 < r) v = ldg16(qsplit + ((head0 + g) * 4 + part) * (size_t)d + dim0);
  const int valid = r - dim0;
  if (valid < 8) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t keep = (2 * e < valid ? 0x0000ffffu : 0u) | (2 * e + 1 < valid ? 0xffff0000u : 0u);
      w[e] &= keep;
    }
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return as_bf16x8(v);
}

// A operand of the transposed product (heads in rows, tokens in columns):
// row m = 4 h + part holds split part `part` of head head0 + h (part 3 is the
// zero row), for the 8 dims starting at dim0; one 16-byte load.  Rows of
// heads >= NH and dims >= r are zero.  Lane l of the result then holds, in
// its four accumulators, the split partial products of head l / 16 for token
// (column) l % 16, so one lane finishes one score with two adds.
__device__ __forceinline__ bf16x8_t q_rows(const uint16_t* __restrict__ qsplit, size_t head0, int d, int NH,
                                           int r, int m, int dim0) {
  const int h = m >> 2, part = m & 3;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (h < NH && dim0 < r) v = ldg16(qsplit + ((head0 + h) * 4 + part) * (size_t)d + dim0);
  const int valid = r - dim0;
  if (valid < 8) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t keep = (2 * e < valid ? 0x0000ffffu : 0u) | (2 * e + 1 < valid ? 0xffff0000u : 0u);
      w[e] &= keep;
    }
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return as_bf16x8(v);
}

// The score of a lane's (head, token) from the split partial products:
// (h + m) + (l + 0), the same grouping as add_split_columns.
__device__ __forceinline__ float sum_split_rows(const floatx4_t& acc) {
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

}  // namespace loki
