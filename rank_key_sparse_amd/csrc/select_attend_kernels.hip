// Top-k selection and exact attention of one query head in one launch (bf16
// caches): one block of 1024 threads per query head takes the head's keys
// from global memory -- all of its approximate-score keys (S <= 32768, the
// register form of the selection) or, for a head selected in two stages, the
// winners of its chunks -- keeps its k best tokens (select_core.h), lists
// them in LDS in ascending order (also written to idx), and runs the exact
// attention over them (attend_core.h), writing the head's output row: the
// selection, attention and merge kernels of the separate path in one.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "attend_core.h"
#include "common.h"
#include "internal.h"
#include "mfma_common.h"
#include "select_core.h"

namespace loki {

constexpr int kSaThreads = 1024;

// MERGE: keys[row][0..S2) are the chunk winners' keys, cidx[row][..] their
// tokens (-1 with key 0 for an empty slot); else keys[row][0..S) are the
// head's keys by token.  ldk: row stride of keys / cidx.  qsplit: the split
// query rows [row][4][D] of the exact stage.  Kx, V: [B][Hkv][Scap][D].
template <int T, int D, bool MERGE>
__global__ __launch_bounds__(kSaThreads, 4) void select_attend_kernel(
    const uint32_t* __restrict__ keys, const int32_t* __restrict__ cidx, int ldk, int S2,
    const uint16_t* __restrict__ qsplit, const bf16_t* __restrict__ Kx, const bf16_t* __restrict__ V,
    bf16_t* __restrict__ out, int32_t* __restrict__ idx, int Hq, int Hkv, int Scap, int k, float scale_log2,
    const int32_t* __restrict__ lens) {
  extern __shared__ __align__(16) uint32_t list[];  // [k] kept tokens, then the attention's merge scratch
  __shared__ uint32_t lds[kNB];
  __shared__ uint32_t take[kSaThreads * T / 32];
  __shared__ SelScratch<kSaThreads> sh;
  __shared__ uint32_t smm[2];
  const int row = blockIdx.x, b = row / Hq, h = row - b * Hq, kv = h / (Hq / Hkv);
  const int S = seq_len(lens, b, Scap);  // this head's tokens
  const int tid = threadIdx.x;
  int32_t* orow = idx + (size_t)row * k;
  int n;
  if (k >= S) {  // every token is kept: dense attention over the sequence
    for (int j = tid; j < k; j += kSaThreads) {
      orow[j] = j < S ? j : -1;
      if (j < S) list[j] = (uint32_t)j;
    }
    n = S;
  } else {
    const int Sx = MERGE ? S2 : S;  // keys of the row
    uint32_t key[T];
    load_regs<T>(keys + (size_t)row * ldk, Sx, key);
    const uint32_t* kmm = nullptr;
    if constexpr (MERGE) {
      // the value bins span the real candidates' keys only (an empty slot's
      // key 0 decodes to NaN); empty slots fall into bin 0
      const int nv = regs_valid<T>(Sx);
      uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
      for (int i = 0; i < T; ++i)
        if (i < nv && key[i] != 0u) {
          mn = min(mn, key[i]);
          mx = max(mx, key[i]);
        }
      uint32_t kmin, kmax;
      block_minmax<kSaThreads>(mn, mx, sh, kmin, kmax);
      if (tid == 0) {
        smm[0] = kmin;
        smm[1] = kmax;
      }
      __syncthreads();  // sh.red is read by every thread before select_regs reuses sh
      kmm = smm;
    }
    select_regs<kSaThreads, T>(key, lds, take, Sx, k, 2 * ((Sx + 63) / 64), reinterpret_cast<int32_t*>(list),
                               nullptr, sh, MERGE ? cidx + (size_t)row * ldk : nullptr, nullptr, 0, kmm);
    __syncthreads();  // the list is complete
    for (int j = tid; j < k; j += kSaThreads) orow[j] = (int32_t)list[j];
    n = k;
  }
  // every entry is kept by the block's one head (bit 30)
  for (int j = tid; j < n; j += kSaThreads) list[j] |= 1u << 30;
  __syncthreads();
  const size_t cb = ((size_t)b * Hkv + kv) * Scap * D;
  attend_list<D, 1, kSaThreads>(list, n, qsplit + (size_t)row * 4 * D, Kx + cb, V + cb, scale_log2,
                                out + (size_t)row * D, reinterpret_cast<float*>(list + k));
}

// ============================================================================
// host side
// ============================================================================
// One CU sustains ~40 GB/s of gathered rows (its outstanding misses, not
// HBM, bound it), so one block per head only pays when the blocks fill the
// chip or a head's kept rows are small; otherwise the attention kernel that
// spreads a group's rows over many blocks is faster.
bool select_attend_fits(const DecodePlan& p) {
  const size_t head_rows_bytes = (size_t)p.k * p.d * 2 * 2;  // K and V rows of one head, bf16
  return p.dt == 1 && (p.d == 64 || p.d == 128) &&
         ((size_t)p.B * p.Hq >= 256 || head_rows_bytes <= ((size_t)256 << 10));
}

hipError_t launch_select_attend(const DecodePlan& p, const uint32_t* keys, const int32_t* cidx, int ldk, int S2,
                                const uint16_t* qsplit, const void* Kx, const void* V, void* out, int32_t* idx,
                                hipStream_t st) {
  if (!select_attend_fits(p)) return hipErrorInvalidValue;
  const bool merge = cidx != nullptr;
  const int Sx = merge ? S2 : p.S;  // keys per row held in registers
  const int rows = p.B * p.Hq;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.d));
  const int mw = p.d == 64 ? attend_merge_words<64, 1, kSaThreads>() : attend_merge_words<128, 1, kSaThreads>();
  const size_t lds = (size_t)(p.k + mw) * sizeof(uint32_t);
  auto go = [&](auto tt, auto dd, auto mg) {
    constexpr int TT = decltype(tt)::value, D = decltype(dd)::value;
    constexpr bool MG = decltype(mg)::value;
    const void* fn = reinterpret_cast<const void*>(&select_attend_kernel<TT, D, MG>);
    hipError_t e = ensure_dynamic_lds(fn, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((select_attend_kernel<TT, D, MG>), dim3(rows), dim3(kSaThreads), lds, st, keys, cidx, ldk,
                       S2, qsplit, static_cast<const bf16_t*>(Kx), static_cast<const bf16_t*>(V),
                       static_cast<bf16_t*>(out), idx, p.Hq, p.Hkv, p.S, p.k, scale_log2, p.lens);
    return hipGetLastError();
  };
  auto by_t = [&](auto dd, auto mg) {
    if (Sx <= kSaThreads * 4) return go(std::integral_constant<int, 4>{}, dd, mg);
    if (Sx <= kSaThreads * 8) return go(std::integral_constant<int, 8>{}, dd, mg);
    if (Sx <= kSaThreads * 16) return go(std::integral_constant<int, 16>{}, dd, mg);
    if (Sx <= kSaThreads * kSelRegMaxT) return go(std::integral_constant<int, kSelRegMaxT>{}, dd, mg);
    return hipErrorInvalidValue;
  };
  auto by_d = [&](auto mg) {
    return p.d == 64 ? by_t(std::integral_constant<int, 64>{}, mg) : by_t(std::integral_constant<int, 128>{}, mg);
  };
  return merge ? by_d(std::true_type{}) : by_d(std::false_type{});
}

}  // namespace loki
