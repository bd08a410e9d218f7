// Exact attention of one block's query heads (NH = 1 or 2, one key/value
// head) over a list of kept tokens held in LDS: the last stage of a decode
// step (the AQUA page's eqs. 3-5 on the kept set), shared by the kernels that
// select and attend in one launch.
//
// list[i] = token | kept-by-head-0 << 30 | kept-by-head-1 << 31, i < n, in
// ascending token order (n >= 1), followed by kListPad entries that hold a
// valid token and no head bit (token 0): the tiles past the end read them
// instead of clamping every index.  Wave w takes 16-row tiles w + NWV j of the
// list in one pass, double buffered: for a tile, the K rows (MFMA B operand,
// 64 contiguous bytes of each of 16 rows per load instruction) and the V rows
// (16-byte granules, RL lanes per row) are requested together, one tile
// ahead of the one being used.  Per tile: the exact scores of the heads from
// MFMA (head h's three split rows of the query in A rows 4h .. 4h + 3: lane l
// holds head l / 16's score of row l % 16), scaled to log2 units, -inf where
// the head did not keep the token; an online softmax per head (running max
// and sum; the accumulators are rescaled when the max grows); each lane's V
// granules weighted by the heads' weights of their rows (read from the score
// lanes by lane permutes).  The waves' (max, sum, acc) of each head are then
// merged by log-sum-exp and handed on: as head h's normalised output row at
// out + h D, or as the block's partial when blocks share a head's list.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "common.h"
#include "mfma_common.h"

namespace loki {

// Max over the aligned 16-lane rows of a wave (every lane of a row ends with
// the row's max): quad swaps, then the half-row and row mirrors.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  return v;
}

constexpr uint32_t kListTok = 0x3fffffffu;  // token bits of a list entry
constexpr int kListPad = 16;                 // entries after a list's end that the attention may read

// LDS words of the merge scratch: s_acc [NWV][NH][D] then s_ml [NWV][4].
template <int D, int NH, int NTHR>
constexpr int attend_merge_words() {
  return (NTHR / 64) * NH * D + (NTHR / 64) * 4;
}

// All NTHR threads of the block call it, after a barrier that completes the
// list.  qx: the heads' split query rows in LDS, part 3 zero: with one head,
// the MFMA A rows [16][D] (rows 0..3 the head's parts, rows 4..15 zero, so
// that every lane reads its row with no condition, and the reads leave the
// tile loop); with two, [2][4][D] (read per tile, lanes past row 7 get zero:
// two heads' accumulators leave no registers for the operands); Kx, V: this key/value head's rows [S][D]; scratch: LDS of
// attend_merge_words() floats that no thread reads or writes meanwhile.
// emit(h, c, M, L, A) receives, for head h and dim c, the block's running
// max M (log2 units), weight sum L and weighted sum A of V[.][c]; every
// (h, c) once, by some thread of the block.
template <int D, int NH, int NTHR, typename Emit>
__device__ __forceinline__ void attend_list_core(const uint32_t* list, int n, const uint16_t* qx,
                                                 const bf16_t* __restrict__ Kx, const bf16_t* __restrict__ V,
                                                 float scale_log2, float* scratch, Emit&& emit) {
  static_assert(NH == 1 || NH == 2, "one or two heads per block");
  constexpr int NWV = NTHR / 64;
  constexpr int KSD = D / 32;   // k-steps of the exact dot
  constexpr int RL = D / 8;     // lanes per V row
  constexpr int RPW = 64 / RL;  // V rows per wave pass
  constexpr int VP = 16 / RPW;  // V passes per tile
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, q4 = lane >> 4;
  const int lg = lane / RL, li = lane % RL;
  const int ntile = (n + 15) >> 4;
  auto load_tile = [&](int t, uint4 (&kb)[KSD], uint4 (&vb)[VP]) {
    const uint32_t tk = list[16 * t + m] & kListTok;  // t <= ntile - 1: within the padding
    const bf16_t* kr = Kx + (size_t)tk * D + 8 * q4;
#pragma unroll
    for (int s = 0; s < KSD; ++s) kb[s] = ldg16(kr + 32 * s);
#pragma unroll
    for (int u = 0; u < VP; ++u) {
      const uint32_t tv = list[16 * t + RPW * u + lg] & kListTok;
      vb[u] = ldg16(V + (size_t)tv * D + 8 * li);
    }
  };
  float acc[NH][8];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
  float mr[NH];  // running maxima (the same in every lane)
#pragma unroll
  for (int h = 0; h < NH; ++h) mr[h] = -INFINITY;
  float lp = 0.f;  // this lane's share of its head's weight sum
  auto proc_tile = [&](int t, const uint4 (&kb)[KSD], const uint4 (&vb)[VP]) {
    floatx4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSD; ++s)  // the A operands are read per tile (LDS), not held in registers
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          NH == 1 ? as_bf16x8(*reinterpret_cast<const uint4*>(qx + m * D + 32 * s + 8 * q4))
                  : q_rows(qx, 0, D, NH, D, m, 32 * s + 8 * q4),
          as_bf16x8(kb[s]), sacc, 0, 0, 0);
    const int p = 16 * t + m;
    const uint32_t ent = list[p];  // a padding entry keeps no head
    const bool kept = q4 < NH && ((ent >> (30 + (q4 & 1))) & 1u);
    const float e = kept ? sum_split_rows(sacc) * scale_log2 : -INFINITY;
    const float tm = row16_max(e);
    // the hardware exp2 (no denormal results: a weight below 2^-126 of the
    // running maximum's is 0, which the sums cannot tell apart)
    float c[NH];
    bool grew = false;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const float nm = fmaxf(mr[h], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tm), 16 * h)));
      c[h] = (nm == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mr[h] - nm);
      grew = grew || nm != mr[h];
      mr[h] = nm;
    }
    const float mh = (NH == 1 || q4 == 0) ? mr[0] : mr[NH - 1];
    const float w = kept ? __builtin_amdgcn_exp2f(e - mh) : 0.f;
    lp = fmaf(lp, (NH == 1 || q4 == 0) ? c[0] : c[NH - 1], w);
    float wv[NH][VP];
#pragma unroll
    for (int u = 0; u < VP; ++u)
#pragma unroll
      for (int h = 0; h < NH; ++h) wv[h][u] = __shfl(w, 16 * h + RPW * u + lg);
    if (grew) {  // uniform: the maxima are the same in every lane
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int h = 0; h < NH; ++h) acc[h][i] *= c[h];
    }
#pragma unroll
    for (int u = 0; u < VP; ++u) {
      float x[8];
      Gran<bf16_t>::unpack(vb[u], x);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int h = 0; h < NH; ++h) acc[h][i] = fmaf(wv[h][u], x[i], acc[h][i]);
    }
  };
  {
    uint4 ka[KSD], va[VP], kb2[KSD], vb2[VP];
    load_tile(min(wave, ntile - 1), ka, va);
    for (int t = wave; t < ntile; t += 2 * NWV) {  // unconditional loads: tiles past the end repeat the last
      load_tile(min(t + NWV, ntile - 1), kb2, vb2);
      proc_tile(t, ka, va);
      if (t + NWV >= ntile) break;  // uniform across the wave
      load_tile(min(t + 2 * NWV, ntile - 1), ka, va);
      proc_tile(t + NWV, kb2, vb2);
    }
  }
  // per head: the weight sum over its 16 score lanes; per dim: the sum of
  // the accumulators over the lanes holding other rows of the same dims
  lp = group_sum<16>(lp);
  float l[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) l[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lp), 16 * h));
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = acc[h][i];
      // lane ^ 8 and lane ^ 16 by ds_swizzle (bit-mask mode, no address), lane ^ 32 by bpermute
      if constexpr (RL <= 8) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x201F));
      v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
      v += __shfl_xor(v, 32);
      acc[h][i] = v;
    }
  // merge the waves by log-sum-exp
  float* s_acc = scratch;                   // [NWV][NH][D]
  float* s_ml = scratch + NWV * NH * D;     // [NWV][4] (max, sum per head)
  if (lg == 0) {
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) s_acc[(wave * NH + h) * D + li * 8 + i] = acc[h][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      s_ml[wave * 4 + 2 * h] = mr[h];
      s_ml[wave * 4 + 2 * h + 1] = l[h];
    }
  }
  __syncthreads();
  for (int o = tid; o < NH * D; o += NTHR) {
    const int h = o / D, cdim = o - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, s_ml[w * 4 + 2 * h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float mw = s_ml[w * 4 + 2 * h];
      const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      L = fmaf(s_ml[w * 4 + 2 * h + 1], f, L);
      A = fmaf(s_acc[(w * NH + h) * D + cdim], f, A);
    }
    emit(h, cdim, M, L, A);
  }
}

// The heads' normalised outputs, head h's row at out + h D.
template <int D, int NH, int NTHR>
__device__ __forceinline__ void attend_list(const uint32_t* list, int n, const uint16_t* qx,
                                            const bf16_t* __restrict__ Kx, const bf16_t* __restrict__ V,
                                            float scale_log2, bf16_t* __restrict__ out, float* scratch) {
  attend_list_core<D, NH, NTHR>(list, n, qx, Kx, V, scale_log2, scratch, [&](int h, int c, float, float L, float A) {
    out[(size_t)h * D + c] = f32_to_bf16(L > 0.f ? A / L : 0.f);
  });
}

}  // namespace loki
