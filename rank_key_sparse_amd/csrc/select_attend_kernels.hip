// Top-k selection and exact attention of one query head in one launch (bf16
// caches): blocks of 1024 threads take a query head's keys from global
// memory -- all of its approximate-score keys (S <= 32768, the register form
// of the selection) or, for a head selected in two stages, the winners of its
// chunks -- keep its k best tokens (select_core.h), list them in LDS in
// ascending order (also written to idx), and run the exact attention over
// them (attend_core.h): the selection, attention and merge kernels of the
// separate path in one.
//
// When the heads alone do not fill the chip, nspl blocks share a head: each
// makes the same selection (its keys are read from L2 after the first block),
// writes its share of idx, attends over its 1/nspl of the kept list and
// stores that partial (max, weight sum, weighted V sum); the last block of
// the head to finish (a device-scope counter, cleared by the query rotation
// of the same call) merges the partials by log-sum-exp into the output row.
// A head's kept rows then come in through nspl CUs instead of one.
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
// nspl > 1: part [rows][nspl][D + 2] partials, cnt [rows] counters (zero on
// entry, left zero).  Block -> (row, split): the nspl blocks of a row get
// block indices that are equal mod 8 (the same XCD, whose L2 then serves
// the keys to all but the first).
template <int T, int D, bool MERGE>
__global__ __launch_bounds__(kSaThreads, 4) void select_attend_kernel(
    const uint32_t* __restrict__ keys, const int32_t* __restrict__ cidx, int ldk, int S2,
    const uint16_t* __restrict__ qsplit, const bf16_t* __restrict__ Kx, const bf16_t* __restrict__ V,
    bf16_t* __restrict__ out, int32_t* __restrict__ idx, int rows, int Hq, int Hkv, int Scap, int k,
    float scale_log2, const int32_t* __restrict__ lens, int nspl, float* part, uint32_t* cnt) {
  extern __shared__ __align__(16) uint32_t list[];  // [k] kept tokens, then the attention's merge scratch
  __shared__ uint32_t lds[kNB];
  __shared__ uint32_t take[kSaThreads * T / 32];
  __shared__ SelScratch<kSaThreads> sh;
  __shared__ uint32_t smm[2];
  __shared__ uint32_t s_last;
  __shared__ __align__(16) uint16_t sq[16 * D];  // the MFMA A rows: the head's split parts, then zeros
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int row = (slot / nspl) * 8 + xcd, j = slot - (slot / nspl) * nspl;
  if (row >= rows) return;  // padding block (uniform)
  const int b = row / Hq, h = row - b * Hq, kv = h / (Hq / Hkv);
  const int S = seq_len(lens, b, Scap);  // this head's tokens
  const int tid = threadIdx.x;
  int32_t* orow = idx + (size_t)row * k;
  // the attention's padding after the list (k or S entries; written by no
  // other step) and its A rows (ordered before it by the barriers below)
  if (tid < kListPad) list[(k >= S ? S : k) + tid] = 0u;
  for (int i = tid; i < 16 * D; i += kSaThreads) sq[i] = i < 4 * D ? qsplit[(size_t)row * 4 * D + i] : (uint16_t)0;
  // this block's share of the idx row
  const int klo = (int)((long long)k * j / nspl), khi = (int)((long long)k * (j + 1) / nspl);
  int n;
  if (k >= S) {  // every token is kept: dense attention over the sequence
    for (int jj = tid; jj < S; jj += kSaThreads) list[jj] = (uint32_t)jj;
    for (int jj = klo + tid; jj < khi; jj += kSaThreads) orow[jj] = jj < S ? jj : -1;
    __syncthreads();  // the list is complete (the marking below touches other threads' entries)
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
    // the list first holds the kept positions in the key row; for chunk
    // winners they become tokens below, every lookup in flight at once
    // (positions ascend with tokens: each chunk lists its winners in order)
    select_regs<kSaThreads, T>(key, lds, take, Sx, k, 2 * ((Sx + 63) / 64),
                                            reinterpret_cast<int32_t*>(list), nullptr, sh, nullptr, nullptr, 0, kmm);
    __syncthreads();  // the list is complete
    if constexpr (MERGE) {
      const int32_t* crow = cidx + (size_t)row * ldk;
#pragma unroll 4
      for (int jj = tid; jj < k; jj += kSaThreads) list[jj] = (uint32_t)crow[list[jj]];
      __syncthreads();
    }
    for (int jj = klo + tid; jj < khi; jj += kSaThreads) orow[jj] = (int32_t)list[jj];
    n = k;
  }
  // this block's share of the kept list, every entry kept by the block's one head (bit 30)
  const int a0 = (int)((long long)n * j / nspl), a1 = (int)((long long)n * (j + 1) / nspl);
  for (int jj = a0 + tid; jj < a1; jj += kSaThreads) list[jj] |= 1u << 30;
  __syncthreads();
  const size_t cb = ((size_t)b * Hkv + kv) * Scap * D;
  const uint16_t* qx = sq;
  float* scratch = reinterpret_cast<float*>(list + k + kListPad);  // n <= k entries and the padding precede it
  if (nspl == 1) {
    attend_list<D, 1, kSaThreads>(list, n, qx, Kx + cb, V + cb, scale_log2, out + (size_t)row * D, scratch);
    return;
  }
  // The partials travel through device-coherent accesses only (agent-scope
  // atomic stores and loads, which bypass the per-XCD L2's non-coherent
  // lines), so no cache-wide fence is needed: each thread waits until its
  // stores are complete, the barrier joins the block, and one thread counts
  // the block; the last block of the row to be counted merges the partials.
  float* prt = part + ((size_t)row * nspl + j) * (D + 2);
  auto st_part = [&](int i, float v) { __hip_atomic_store(prt + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  if (a1 > a0) {
    attend_list_core<D, 1, kSaThreads>(list + a0, a1 - a0, qx, Kx + cb, V + cb, scale_log2, scratch,
                                       [&](int, int c, float M, float L, float A) {
                                         st_part(2 + c, A);
                                         if (c == 0) {
                                           st_part(0, M);
                                           st_part(1, L);
                                         }
                                       });
  } else {  // fewer kept tokens than blocks: an empty partial
    for (int c = tid; c < D; c += kSaThreads) {
      st_part(2 + c, 0.f);
      if (c == 0) {
        st_part(0, -INFINITY);
        st_part(1, 0.f);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&cnt[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(nspl - 1)
                 ? 1u
                 : 0u;
  __syncthreads();
  if (s_last == 0u) return;  // uniform
  // every partial into LDS at once (the merge scratch holds nspl (D + 2) <=
  // kSplitMax (D + 2) words), then the log-sum-exp merge from there
  const float* pr = part + (size_t)row * nspl * (D + 2);
  for (int i = tid; i < nspl * (D + 2); i += kSaThreads)
    scratch[i] = __hip_atomic_load(pr + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  for (int c = tid; c < D; c += kSaThreads) {
    float M = -INFINITY;
    for (int s = 0; s < nspl; ++s) M = fmaxf(M, scratch[s * (D + 2)]);
    float L = 0.f, A = 0.f;
    for (int s = 0; s < nspl; ++s) {
      const float ms = scratch[s * (D + 2)];
      const float f = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
      L = fmaf(scratch[s * (D + 2) + 1], f, L);
      A = fmaf(scratch[s * (D + 2) + 2 + c], f, A);
    }
    out[(size_t)row * D + c] = f32_to_bf16(L > 0.f ? A / L : 0.f);
  }
  if (tid == 0) __hip_atomic_store(&cnt[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ============================================================================
// host side
// ============================================================================
// One CU sustains ~40 GB/s of gathered rows (its outstanding misses, not
// HBM, bound it), so a head's kept rows must come in through several CUs
// unless they are small: this launch pays when a head's K / V rows are at
// most 256 KB, or when p.NSPL >= 2 blocks share each head (<= 128 heads);
// otherwise the attention kernel that spreads a group's rows over many
// blocks is faster.
static_assert(kSplitMax * (64 + 2) <= attend_merge_words<64, 1, kSaThreads>() &&
                  kSplitMax * (128 + 2) <= attend_merge_words<128, 1, kSaThreads>(),
              "the merge scratch holds every partial of a head");
bool select_attend_fits(const DecodePlan& p) {
  const size_t head_rows_bytes = (size_t)p.k * p.d * 2 * 2;  // K and V rows of one head, bf16
  return p.dt == 1 && (p.d == 64 || p.d == 128) && (head_rows_bytes <= ((size_t)256 << 10) || p.NSPL >= 2);
}

hipError_t launch_select_attend(const DecodePlan& p, const uint32_t* keys, const int32_t* cidx, int ldk, int S2,
                                const uint16_t* qsplit, const void* Kx, const void* V, void* out, int32_t* idx,
                                float* part, uint32_t* cnt, hipStream_t st) {
  if (!select_attend_fits(p)) return hipErrorInvalidValue;
  const int nspl = p.NSPL;
  if (nspl < 1 || nspl > kSplitMax || (nspl > 1 && (!part || !cnt))) return hipErrorInvalidValue;
  const bool merge = cidx != nullptr;
  const int Sx = merge ? S2 : p.S;  // keys per row held in registers
  const int rows = p.B * p.Hq;
  const long long nblk = (long long)(rows + 7) / 8 * 8 * nspl;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.d));
  const int mw = p.d == 64 ? attend_merge_words<64, 1, kSaThreads>() : attend_merge_words<128, 1, kSaThreads>();
  const size_t lds = (size_t)(p.k + kListPad + mw) * sizeof(uint32_t);
  auto go = [&](auto tt, auto dd, auto mg) {
    constexpr int TT = decltype(tt)::value, D = decltype(dd)::value;
    constexpr bool MG = decltype(mg)::value;
    const void* fn = reinterpret_cast<const void*>(&select_attend_kernel<TT, D, MG>);
    hipError_t e = ensure_dynamic_lds(fn, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((select_attend_kernel<TT, D, MG>), dim3((unsigned)nblk), dim3(kSaThreads), lds, st, keys,
                       cidx, ldk, S2, qsplit, static_cast<const bf16_t*>(Kx), static_cast<const bf16_t*>(V),
                       static_cast<bf16_t*>(out), idx, rows, p.Hq, p.Hkv, p.S, p.k, scale_log2, p.lens, nspl, part,
                       cnt);
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
