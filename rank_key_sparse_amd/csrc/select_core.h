// Per-query-head top-k selection, shared by the selection kernel (keys from
// the workspace) and the fused score+select kernel (keys computed into LDS).
//
// Given the order-preserving keys of one head (in LDS, or re-read from
// global memory) and their min / max:
// 1. histogram of the scores in kNB equal-width value bins over [min, max]
//    (a monotone map, so bins order like keys);
// 2. scan bins from the top to find the bin t holding the k-th largest;
// 3. resolve the exact k-th key K* inside bin t: rank the (few) candidates
//    of bin t by (key desc, index asc) in LDS; if bin t is too full (heavily
//    tied or degenerate scores) run an exact 11/11/10-bit MSB radix select
//    restricted to bin t instead;
// 4. emit, in index order: key > K*, or key == K* among the first `quota`
//    such tokens (lower index wins).  Each wave owns a 64-aligned token
//    segment, so the kept-token bitmap words are written without atomics.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace loki {

constexpr int kNB = 2048;      // value bins
constexpr int kCap = 1024;     // candidates ranked in LDS (2 * kCap words alias the bins)
constexpr int kRankLds = 256;  // rank limit when the keys themselves are in LDS

template <int NTHR>
struct SelScratch {
  static constexpr int NW = NTHR / 64;
  uint32_t red[2][NW];
  int scan[NW];
  int wgt[NW], weq[NW], selb[NW], eqb[NW];
  uint32_t kmin, kmax, kstar;
  int t, above, quota, ccount;
};

// Inclusive prefix sum over the block in thread order.
template <int NTHR>
__device__ __forceinline__ int block_incl_scan(int v, SelScratch<NTHR>& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  if (lane == 63) sh.scan[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += sh.scan[w];
  __syncthreads();
  return v + add;
}

// Find, scanning bins from the top, the bin holding the `want`-th largest key
// (1-based).  Sets sh.t to that bin and sh.above to the count in higher bins.
// Thread i owns bins kNB-1-BPT*i down to kNB-BPT*(i+1).
template <int NTHR>
__device__ __forceinline__ void find_threshold(const uint32_t* hist, int want, SelScratch<NTHR>& sh) {
  constexpr int BPT = kNB / NTHR;
  const int top = kNB - 1 - BPT * (int)threadIdx.x;
  int h[BPT], mine = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) { h[i] = (int)hist[top - i]; mine += h[i]; }
  int above = block_incl_scan<NTHR>(mine, sh) - mine;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    if (above < want && above + h[i] >= want) { sh.t = top - i; sh.above = above; }
    above += h[i];
  }
  __syncthreads();
}

struct Binner {
  float fmin, scale;
  bool degenerate;
  __device__ __forceinline__ void init(uint32_t kmin, uint32_t kmax) {
    fmin = key_score(kmin);
    const float range = key_score(kmax) - fmin;
    scale = (float)kNB / range;
    degenerate = !(range > 0.f) || !isfinite(range) || !isfinite(scale) || !(scale > 0.f);
  }
  __device__ __forceinline__ int operator()(uint32_t key) const {
    if (degenerate) return 0;
    const int b = (int)((key_score(key) - fmin) * scale);
    return b < kNB - 1 ? b : kNB - 1;
  }
};

// Calls f(j, key) for every token j < S (in no particular order): each thread
// reads 4 consecutive keys per 16-byte load with UB loads in flight.
template <int NTHR, bool IN_LDS, typename F>
__device__ __forceinline__ void for_each_key(const uint32_t* rk, const uint32_t* lk, int S, int Sp,
                                             F&& f) {
  constexpr int UB = IN_LDS ? 4 : 8;
  const uint4* src = reinterpret_cast<const uint4*>(IN_LDS ? lk : rk);
  const int n4 = Sp >> 2, tid = threadIdx.x;
  for (int base = 0; base < n4; base += NTHR * UB) {
    uint4 v[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int i = base + u * NTHR + tid;
      v[u] = (i < n4) ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int j = (base + u * NTHR + tid) << 2;
      if (j < S) f(j, v[u].x);
      if (j + 1 < S) f(j + 1, v[u].y);
      if (j + 2 < S) f(j + 2, v[u].z);
      if (j + 3 < S) f(j + 3, v[u].w);
    }
  }
}

// Writes idx (ascending) and the kept-token bitmap when every token is kept.
template <int NTHR>
__device__ __forceinline__ void keep_all(int S, int W, int32_t* orow, uint32_t* brow) {
  for (int j = threadIdx.x; j < S; j += NTHR) orow[j] = j;
  for (int w = threadIdx.x; w < W; w += NTHR) {
    const int lo = 32 * w;
    brow[w] = (lo + 32 <= S) ? 0xffffffffu : (lo >= S ? 0u : ((1u << (S - lo)) - 1u));
  }
}

// Steps 1-4 for one head with k < S.  `hist` is kNB words of LDS (reused for
// candidates); keys are lk[0..S) in LDS (IN_LDS) or rk[0..S) in global
// memory; kmin / kmax are their extremes.  All threads of the block call it.
template <int NTHR, bool IN_LDS>
__device__ __forceinline__ void select_head(const uint32_t* rk, const uint32_t* lk, uint32_t* hist,
                                            int S, int Sp, int k, uint32_t kmin, uint32_t kmax,
                                            int32_t* orow, uint32_t* brow, SelScratch<NTHR>& sh) {
  constexpr int NW = NTHR / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // 1. value histogram
  for (int i = tid; i < kNB; i += NTHR) hist[i] = 0u;
  __syncthreads();
  Binner bin;
  bin.init(kmin, kmax);
  for_each_key<NTHR, IN_LDS>(rk, lk, S, Sp, [&](int, uint32_t v) { atomicAdd(&hist[bin(v)], 1u); });
  __syncthreads();

  // 2. threshold bin
  find_threshold<NTHR>(hist, k, sh);
  const int tb = sh.t;
  const int need = k - sh.above;  // 1 <= need <= hist[tb]
  const int nc = (int)hist[tb];
  __syncthreads();  // hist is reused below

  // 3. exact k-th key inside bin tb.  Ranking costs nc^2 compares spread over
  // the block; the radix passes cost three sweeps of the keys.
  if (nc <= (IN_LDS ? kRankLds : kCap)) {
    uint32_t* ck = hist;
    uint32_t* ci = hist + kCap;
    if (tid == 0) sh.ccount = 0;
    __syncthreads();
    for_each_key<NTHR, IN_LDS>(rk, lk, S, Sp, [&](int j, uint32_t v) {
      if (bin(v) == tb) {
        const int p = atomicAdd(&sh.ccount, 1);
        ck[p] = v;
        ci[p] = (uint32_t)j;
      }
    });
    __syncthreads();
    for (int i = tid; i < nc; i += NTHR) {
      const uint32_t vi = ck[i], ii = ci[i];
      int gtc = 0, rank = 0;
      for (int c = 0; c < nc; ++c) {
        const uint32_t vc = ck[c], ic = ci[c];
        gtc += (vc > vi);
        rank += (vc > vi) || (vc == vi && ic < ii);
      }
      if (rank == need - 1) { sh.kstar = vi; sh.quota = need - gtc; }
    }
    __syncthreads();
  } else {
    uint32_t prefix = 0u, pmask = 0u;
    int rem = need;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int sft = shifts[pass];
      const uint32_t dm = (1u << widths[pass]) - 1u;
      for (int i = tid; i < kNB; i += NTHR) hist[i] = 0u;
      __syncthreads();
      for_each_key<NTHR, IN_LDS>(rk, lk, S, Sp, [&](int, uint32_t v) {
        if (bin(v) == tb && (v & pmask) == prefix) atomicAdd(&hist[(v >> sft) & dm], 1u);
      });
      __syncthreads();
      find_threshold<NTHR>(hist, rem, sh);
      rem -= sh.above;
      prefix |= (uint32_t)sh.t << sft;
      pmask |= dm << sft;
      __syncthreads();
    }
    if (tid == 0) { sh.kstar = prefix; sh.quota = rem; }
    __syncthreads();
  }
  const uint32_t kstar = sh.kstar;
  const int quota = sh.quota;

  // 4. emit in index order; each wave owns a 64-aligned segment and reads
  // UE 64-token steps ahead
  constexpr int UE = 8;
  const int SEG = (S + NW * 64 - 1) / (NW * 64) * 64;
  const int wb = wave * SEG, we = min(S, wb + SEG);
  auto KEY = [&](int j) -> uint32_t {
    if constexpr (IN_LDS) return lk[j];
    else return rk[j];
  };
  int ngt = 0, neq = 0;
  for (int j0 = wb; j0 < we; j0 += 64 * UE) {
    uint32_t v[UE];
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int j = j0 + 64 * u + lane;
      v[u] = (j < we) ? KEY(j) : 0u;
    }
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const bool ok = j0 + 64 * u + lane < we;
      ngt += __popcll(__ballot(ok && v[u] > kstar));
      neq += __popcll(__ballot(ok && v[u] == kstar));
    }
  }
  if (lane == 0) { sh.wgt[wave] = ngt; sh.weq[wave] = neq; }
  __syncthreads();
  if (tid == 0) {
    int eqb = 0, selb = 0;
    for (int w = 0; w < NW; ++w) {
      sh.eqb[w] = eqb;
      sh.selb[w] = selb;
      const int take = min(max(quota - eqb, 0), sh.weq[w]);
      selb += sh.wgt[w] + take;
      eqb += sh.weq[w];
    }
  }
  __syncthreads();
  int selrun = sh.selb[wave], eqrun = sh.eqb[wave];
  for (int j0 = wb; j0 < we; j0 += 64 * UE) {
    uint32_t v[UE];
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int j = j0 + 64 * u + lane;
      v[u] = (j < we) ? KEY(j) : 0u;
    }
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int js = j0 + 64 * u;  // 64-aligned step start
      if (js >= we) break;         // uniform across the wave
      const int j = js + lane;
      const bool ok = j < we;
      const bool gt = ok && v[u] > kstar, eq = ok && v[u] == kstar;
      const uint64_t eqm = __ballot(eq);
      const bool take = gt || (eq && eqrun + bits_below(eqm) < quota);
      const uint64_t sm = __ballot(take);
      if (take) orow[selrun + bits_below(sm)] = j;
      if (lane == 0) {
        brow[js >> 5] = (uint32_t)sm;
        brow[(js >> 5) + 1] = (uint32_t)(sm >> 32);
      }
      selrun += __popcll(sm);
      eqrun += __popcll(eqm);
    }
  }
}

}  // namespace loki
