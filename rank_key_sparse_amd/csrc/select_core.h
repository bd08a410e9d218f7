// Per-query-head top-k selection, shared by the selection kernels (keys from
// the workspace) and the fused score+select kernel (keys computed on chip).
//
// The scores of a head are mapped to order-preserving uint32 keys.  Then:
// 1. histogram of the keys in kNB equal-width value bins over [min, max] (a
//    monotone map, so bins order like keys); scan the bins from the top for
//    the bin t holding the k-th largest key;
// 2. one pass in index order: per 64-token step, a mask of the tokens above
//    bin t (all kept), and the tokens of bin t (typically a few) collected;
// 3. the need = k - |above| best tokens of bin t by (key desc, index asc)
//    are marked taken: ranked pairwise when bin t is small; when it is
//    crowded (heavy ties, degenerate scores) an exact 11/11/10-bit MSB radix
//    select inside bin t finds the k-th key K* and its tie quota, and a pass
//    in index order takes key > K* and the first `quota` keys equal to K*
//    (lower index wins);
// 4. emit kept = above | taken: the kept-token bitmap words, then per-word
//    counts, a block prefix and the indices listed in ascending order.
//
// Two forms.  select_regs: the head's keys sit in registers (lane l of wave
// w holds tokens w*64T + 64i + l, i < T), so every pass is a register pass
// and each step's mask lives in one lane.  select_head: the keys stay in
// global memory and are streamed once per pass (heads too long for
// registers); the step masks go to global scratch.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace loki {

constexpr int kNB = 2048;      // value bins
constexpr int kCap = 1024;     // candidates collected (2 * kCap words alias the bins)
constexpr int kRankMax = 256;  // candidates ranked pairwise; more go to the radix path

template <int NTHR>
struct SelScratch {
  static constexpr int NW = NTHR / 64;
  uint32_t red[2][NW];
  int scan[NW];
  int wsel[NW], weq[NW];
  int t, above, nt, ccount;
};

template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xF, false);
}

// Inclusive prefix sum over a wave (DPP row shifts, then row broadcasts).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i<0x111, 0xF>(v);  // row_shr:1
  v += dpp_i<0x112, 0xF>(v);  // row_shr:2
  v += dpp_i<0x114, 0xF>(v);  // row_shr:4
  v += dpp_i<0x118, 0xF>(v);  // row_shr:8
  v += dpp_i<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_i<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Sum of part[w] over the waves w below this one.
template <int NTHR>
__device__ __forceinline__ int waves_below(const int* part) {
  const int wave = threadIdx.x >> 6;
  int add = 0;
#pragma unroll
  for (int w = 0; w < NTHR / 64; ++w) add += (w < wave) ? part[w] : 0;
  return add;
}

// Inclusive prefix sum over the block in thread order.  sh.scan may be
// reused only after a later barrier.
template <int NTHR>
__device__ __forceinline__ int block_incl_scan(int v, SelScratch<NTHR>& sh) {
  v = wave_incl_scan(v);
  if ((threadIdx.x & 63) == 63) sh.scan[threadIdx.x >> 6] = v;
  __syncthreads();
  return v + waves_below<NTHR>(sh.scan);
}

// Two inclusive prefix sums over the block at once, one barrier (each one's
// per-wave totals in its own scratch).
template <int NTHR>
__device__ __forceinline__ void block_incl_scan2(int& a, int& b, SelScratch<NTHR>& sa, SelScratch<NTHR>& sb) {
  a = wave_incl_scan(a);
  b = wave_incl_scan(b);
  if ((threadIdx.x & 63) == 63) {
    sa.scan[threadIdx.x >> 6] = a;
    sb.scan[threadIdx.x >> 6] = b;
  }
  __syncthreads();
  a += waves_below<NTHR>(sa.scan);
  b += waves_below<NTHR>(sb.scan);
}

// Find, scanning bins from the top, the bin holding the `want`-th largest key
// (1-based).  Sets sh.t to that bin, sh.above to the count in higher bins and
// sh.nt to the count in bin t (so that callers need not read hist again).
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
    if (above < want && above + h[i] >= want) { sh.t = top - i; sh.above = above; sh.nt = h[i]; }
    above += h[i];
  }
  __syncthreads();
}

struct Binner {
  float fmin, scale;
  // A degenerate range (every key equal, or a range or scale that is not a
  // positive finite number) gets scale 0, which puts every value in bin 0
  // with no branch in of_score.
  __device__ __forceinline__ void init(uint32_t kmin, uint32_t kmax) {
    fmin = key_score(kmin);
    const float range = key_score(kmax) - fmin;
    scale = (float)kNB / range;
    if (!(range > 0.f) || !isfinite(range) || !isfinite(scale) || !(scale > 0.f)) {
      fmin = 0.f;
      scale = 0.f;
    }
  }
  // bin of a score value (the same map as of its key: key_score(score_key(s))
  // is s, with -0 read as +0, which bins alike).  A value below fmin, or the
  // NaN that key 0 (an empty candidate slot) decodes to -- and, under scale
  // 0, every finite value -- goes to bin 0: the max with 0 returns its
  // non-NaN operand.
  __device__ __forceinline__ int of_score(float s) const {
    const int b = (int)fmaxf((s - fmin) * scale, 0.f);
    return b < kNB - 1 ? b : kNB - 1;
  }
  __device__ __forceinline__ int operator()(uint32_t key) const { return of_score(key_score(key)); }
};

// Block-wide min / max of per-thread partial extremes (one barrier: every
// thread then reduces the per-wave values itself).
template <int NTHR>
__device__ __forceinline__ void block_minmax(uint32_t mn, uint32_t mx, SelScratch<NTHR>& sh, uint32_t& kmin,
                                             uint32_t& kmax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  mn = wave_min_u(mn);
  mx = wave_max_u(mx);
  if (lane == 0) { sh.red[0][wave] = mn; sh.red[1][wave] = mx; }
  __syncthreads();
  uint32_t a = sh.red[0][0], b = sh.red[1][0];
#pragma unroll
  for (int w = 1; w < SelScratch<NTHR>::NW; ++w) { a = min(a, sh.red[0][w]); b = max(b, sh.red[1][w]); }
  kmin = a;
  kmax = b;
}

// Writes idx (ascending) and the kept-token bitmap when every one of the S
// tokens is kept (k >= S); idx entries S .. k - 1 are -1.
template <int NTHR>
__device__ __forceinline__ void keep_all(int S, int k, int W, int32_t* orow, uint32_t* brow) {
  for (int j = threadIdx.x; j < k; j += NTHR) orow[j] = j < S ? j : -1;
  for (int w = threadIdx.x; w < W; w += NTHR) {
    const int lo = 32 * w;
    brow[w] = (lo + 32 <= S) ? 0xffffffffu : (lo >= S ? 0u : ((1u << (S - lo)) - 1u));
  }
}

// A copy of x that the compiler cannot match with earlier values, so that
// cheap per-phase quantities (token numbers, validity) are recomputed rather
// than kept live across the whole selection.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Ranks the nc collected candidates (ck, ci; both 16-byte aligned) by (key
// desc, index asc) and calls set(index) for the `need` best.  The candidates
// are read four at a time, eight in flight, so that the loop is not a chain
// of dependent LDS round trips.
template <int NTHR, typename F>
__device__ __forceinline__ void rank_candidates(const uint32_t* ck, const uint32_t* ci, int nc, int need,
                                                F&& set, int t0 = 0) {
  auto beats = [](uint32_t vc, uint32_t ic, uint32_t vi, uint32_t ii) {
    return (int)((vc > vi) || (vc == vi && ic < ii));
  };
  // threads t0 .. t0 + NTHR - 1 take part (NTHR may be a part of the block)
  for (int i = (int)threadIdx.x - t0; i >= 0 && i < nc; i += NTHR) {
    const uint32_t vi = ck[i], ii = ci[i];
    int rank = 0;
    const int n4 = nc & ~3;
#pragma unroll 2
    for (int c = 0; c < n4; c += 4) {
      const uint4 kv = *reinterpret_cast<const uint4*>(ck + c);
      const uint4 iv = *reinterpret_cast<const uint4*>(ci + c);
      rank += beats(kv.x, iv.x, vi, ii) + beats(kv.y, iv.y, vi, ii) + beats(kv.z, iv.z, vi, ii) +
              beats(kv.w, iv.w, vi, ii);
    }
    for (int c = n4; c < nc; ++c) rank += beats(ck[c], ci[c], vi, ii);
    if (rank < need) set(ii);
  }
}

// ============================================================================
// Keys in registers.  Requires S <= NTHR * T and k < S.  lds: kNB words
// (bins, then candidates); take: W words of LDS, W = 2 ceil(S / 64).  All
// threads of the block call it.
// Output: orow[0..k) = the kept positions p, ascending, written as map[p]
// when map is given, else as p + tok_base; with okeys, okeys[i] receives the
// key of orow[i], read from lkeys[p]; with brow, the kept-position bitmap (W
// words).  The block's take holds at least W words.
// kmm: when given, {min, max} of the keys (e.g. gathered while the keys were
// made), readable by every thread after one barrier; the min / max pass is
// then skipped.  KB: keep each key's bin in registers from the histogram to
// the mask pass instead of computing it twice (T more registers).
// ============================================================================

// Token of key[0] of this lane (key[i] is token tok0 + 64 i), and the number
// of this lane's keys that are below S.
template <int T>
__device__ __forceinline__ int regs_tok0() {
  return (int)(threadIdx.x >> 6) * 64 * T + (int)(threadIdx.x & 63);
}
template <int T>
__device__ __forceinline__ int regs_valid(int S) {
  const int left = S - regs_tok0<T>();
  return left <= 0 ? 0 : min(T, (left + 63) >> 6);
}

// Loads a head's keys in the register layout; src[0..S) in LDS or global
// memory.  Lanes past S read token S - 1 (always in bounds; never used).
template <int T>
__device__ __forceinline__ void load_regs(const uint32_t* src, int S, uint32_t (&key)[T]) {
  const int tok0 = regs_tok0<T>();
#pragma unroll
  for (int i = 0; i < T; ++i) key[i] = src[min(tok0 + 64 * i, S - 1)];
}

// The kept positions are listed from the kept-position bitmap: each step's
// mask is stored by its lane, then one block scan over the bitmap words
// (each thread a contiguous run of them) gives every thread its offset.
// okeys[i], when wanted, is read from lkeys (the keys by position, in LDS or
// global memory).
template <int NTHR, int T, bool KB = false>
__device__ __forceinline__ void select_regs(const uint32_t (&key)[T], uint32_t* lds, uint32_t* take,
                                            int S, int k, int W, int32_t* orow, uint32_t* brow,
                                            SelScratch<NTHR>& sh, const int32_t* map = nullptr,
                                            uint32_t* okeys = nullptr, int tok_base = 0,
                                            const uint32_t* kmm = nullptr, const uint32_t* lkeys = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* hist = lds;

  for (int i = tid; i < kNB; i += NTHR) hist[i] = 0u;
  for (int i = tid; i < W; i += NTHR) take[i] = 0u;
  if (tid == 0) sh.ccount = 0;
  int nv = opaque(regs_valid<T>(S));
  uint32_t kmin, kmax;
  if (kmm) {  // uniform
    __syncthreads();  // orders the zeroing
    kmin = kmm[0];
    kmax = kmm[1];
  } else {
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int i = 0; i < T; ++i)
      if (i < nv) { mn = min(mn, key[i]); mx = max(mx, key[i]); }
    block_minmax<NTHR>(mn, mx, sh, kmin, kmax);  // its barrier also orders the zeroing
  }
  Binner bin;
  bin.init(kmin, kmax);

  // 1. histogram and threshold bin
  int kb[KB ? T : 1];
  nv = opaque(nv);
#pragma unroll
  for (int i = 0; i < T; ++i)
    if (i < nv) {
      const int b = bin(key[i]);
      if constexpr (KB) kb[i] = b;
      atomicAdd(&hist[b], 1u);
    }
  __syncthreads();
  find_threshold<NTHR>(hist, k, sh);  // its trailing barrier ends every read of hist
  const int tb = sh.t;
  const int need = k - sh.above;  // 1 <= need <= nc
  const int nc = sh.nt;
  const bool rank_path = nc <= kRankMax;

  // 2. above-masks (lane i keeps step i's) and bin tb's candidates
  uint32_t* ck = lds;
  uint32_t* ci = lds + kCap;
  uint32_t klo = 0u, khi = 0u;
  nv = opaque(nv);
  const int tok0 = opaque(regs_tok0<T>());
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const int j = tok0 + 64 * i;
    int bj = -1;
    if constexpr (KB) {
      if (i < nv) bj = kb[i];
    } else {
      if (i < nv) bj = bin(key[i]);
    }
    const uint64_t mab = __ballot(bj > tb);
    if (lane == i) { klo = (uint32_t)mab; khi = (uint32_t)(mab >> 32); }
    if (rank_path && bj == tb) {
      const int p = atomicAdd(&sh.ccount, 1);
      ck[p] = key[i];
      ci[p] = (uint32_t)j;
    }
  }
  __syncthreads();

  // 3. the need best tokens of bin tb
  if (rank_path) {
    rank_candidates<NTHR>(ck, ci, nc, need, [&](uint32_t ii) { atomicOr(&take[ii >> 5], 1u << (ii & 31)); });
    __syncthreads();
    const int st = wave * T + lane;
    if (lane < T && 2 * st < W) { klo |= take[2 * st]; khi |= take[2 * st + 1]; }
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
      const int nvp = opaque(nv);
#pragma unroll
      for (int i = 0; i < T; ++i)
        if (i < nvp && bin(key[i]) == tb && (key[i] & pmask) == prefix)
          atomicAdd(&hist[(key[i] >> sft) & dm], 1u);
      __syncthreads();
      find_threshold<NTHR>(hist, rem, sh);
      rem -= sh.above;
      prefix |= (uint32_t)sh.t << sft;
      pmask |= dm << sft;
      __syncthreads();
    }
    const uint32_t kstar = prefix;  // a key of bin tb, so key == K* implies bin tb
    const int quota = rem;          // ties at K* to take, lowest indices first
    int neq = 0;
    nv = opaque(nv);
#pragma unroll
    for (int i = 0; i < T; ++i) neq += __popcll(__ballot(i < nv && key[i] == kstar));
    if (lane == 0) sh.weq[wave] = neq;
    __syncthreads();
    int eqrun = waves_below<NTHR>(sh.weq);
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const bool valid = i < nv;
      const bool eq = valid && key[i] == kstar;
      const uint64_t eqm = __ballot(eq);
      const bool tk = (valid && key[i] > kstar && bin(key[i]) == tb) ||
                      (eq && eqrun + bits_below(eqm) < quota);
      const uint64_t tm = __ballot(tk);
      if (lane == i) { klo |= (uint32_t)tm; khi |= (uint32_t)(tm >> 32); }
      eqrun += __popcll(eqm);
    }
  }

  // 4. emit: lane i < T holds the kept mask of step wave * T + i; it goes
  // to take (its lane alone read those words above), then thread t lists
  // words t R .. t R + R - 1 (tokens 32 w ..) at its block-scan offset
  {
    const int st = wave * T + lane;
    if (lane < T && 2 * st < W) *reinterpret_cast<uint2*>(take + 2 * st) = make_uint2(klo, khi);
  }
  __syncthreads();
  const int R = (W + NTHR - 1) / NTHR, w0 = tid * R, w1 = min(w0 + R, W);
  int c = 0;
  for (int w = w0; w < w1; ++w) c += __popc(take[w]);
  int pos = block_incl_scan<NTHR>(c, sh) - c;
  for (int w = w0; w < w1; ++w) {
    const uint32_t wd = take[w];
    for (uint32_t u = wd; u; u &= u - 1u, ++pos) {
      const int t = 32 * w + __ffs(u) - 1;
      orow[pos] = map ? map[t] : t + tok_base;
      if (okeys) okeys[pos] = lkeys[t];
    }
    if (brow) brow[w] = wd;
  }
}

// Both heads' threshold bins in one block scan of (count0 | count1 << 16)
// from the top bin (each head holds fewer than 65536 keys): for head h the
// bin holding its want_h-th largest key (1-based), with sh[h]->above the
// count in higher bins and sh[h]->nt the count in that bin.  A head with
// fewer than want_h keys in all gets bin 0.  Ends with a barrier, after
// which the histograms may be overwritten.
template <int NTHR>
__device__ __forceinline__ void find_thresholds2(const uint32_t* hist0, const uint32_t* hist1, int want0, int want1,
                                                 SelScratch<NTHR>* const (&sh)[2]) {
  constexpr int BPT = kNB / NTHR;
  const int top = kNB - 1 - BPT * (int)threadIdx.x;
  int hv[2][BPT];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    hv[0][i] = (int)hist0[top - i];
    hv[1][i] = (int)hist1[top - i];
    mine += hv[0][i] | (hv[1][i] << 16);
  }
  const int above = block_incl_scan<NTHR>(mine, *sh[0]) - mine;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int want = h ? want1 : want0;
    int a = (above >> (16 * h)) & 0xffff;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (a < want && a + hv[h][i] >= want) { sh[h]->t = top - i; sh[h]->above = a; sh[h]->nt = hv[h][i]; }
      a += hv[h][i];
    }
    // the thread holding bin 0 (the last one) sees every count
    if (threadIdx.x == NTHR - 1 && a < want) { sh[h]->t = 0; sh[h]->above = a - hv[h][BPT - 1]; sh[h]->nt = hv[h][BPT - 1]; }
  }
  __syncthreads();
}

// ============================================================================
// Two heads at once (same S, k, W; the scores as raw fp32 bits in LDS,
// sbits[h][token], read in the register layout of select_regs: bins come
// straight from the value and stay in registers, and the order-preserving
// key is formed only where a total order is needed, for the threshold bin's
// candidates and the radix tie path; sbits must not change during the call):
// every step handles both heads between shared barriers, so a pair costs
// the barriers and latencies of one selection.  Both histograms go through
// one block scan with the two counts packed in 16-bit halves, which needs
// S < 65536.  The caller zeroes hist[h] (kNB words) and take[h] (W words),
// sets sh[h].ccount = 0 and provides kmm[h] = {min, max} of head h's keys,
// all ordered before the call by a barrier.  With prebuilt, lds[h] already
// holds head h's histogram over bins of the range kmm[h] (the caller's own
// range, e.g. of the first keys made; keys outside it fall into the end
// bins, which keeps the map monotone, so the selection stays exact: only the
// threshold bin's size depends on the range).  lds[h] / take[h] / sh[h] are
// separate per head.  Output: head h's kept-token bitmap in brow[h] (W words;
// the caller lists the kept tokens itself).
// ============================================================================
template <int NTHR, int T>
__device__ __forceinline__ void select_regs2(const uint32_t* const (&sbits)[2], uint32_t* const (&lds)[2],
                                             uint32_t* const (&take)[2], int S, int k, int W,
                                             uint32_t* const (&brow)[2],
                                             SelScratch<NTHR>* const (&sh)[2],
                                             const uint32_t* const (&kmm)[2], bool prebuilt = false) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Binner bin[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) bin[h].init(kmm[h][0], kmm[h][1]);
  // the scores stay in LDS (sbits[h][token], fp32 bits) and are read where a
  // key is needed; only each score's bin is held in registers, so the mask
  // pass never recomputes bins
  const int tok0 = opaque(regs_tok0<T>());
  auto key = [&](int h, int i) { return score_key(__uint_as_float(sbits[h][min(tok0 + 64 * i, S - 1)])); };

  // 1. both histograms (unless prebuilt); each score's bin stays in a
  // register for step 2 (-1 for a slot past S: the reads are clamped in
  // bounds, so the bins are computed without a branch)
  int kb[2][T];
  int nv = opaque(regs_valid<T>(S));
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int b = bin[h].of_score(__uint_as_float(sbits[h][min(tok0 + 64 * i, S - 1)]));
      kb[h][i] = i < nv ? b : -1;
      if (!prebuilt && i < nv) atomicAdd(&lds[h][b], 1u);
    }
  if (!prebuilt) __syncthreads();  // uniform

  // threshold bins: one scan of (count0 | count1 << 16) from the top bin
  find_thresholds2<NTHR>(lds[0], lds[1], k, k, sh);  // ends every read of the histograms
  int tb[2], need[2], nc[2];
  bool rank_path[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    tb[h] = sh[h]->t;
    need[h] = k - sh[h]->above;
    nc[h] = sh[h]->nt;
    rank_path[h] = nc[h] <= kRankMax;
  }

  // 2. above-masks and threshold-bin candidates of both heads
  uint32_t klo[2] = {0u, 0u}, khi[2] = {0u, 0u};
  nv = opaque(nv);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t* ck = lds[h];
    uint32_t* ci = lds[h] + kCap;
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int bj = kb[h][i];  // -1 past S
      const uint64_t mab = __ballot(bj > tb[h]);
      if (lane == i) { klo[h] = (uint32_t)mab; khi[h] = (uint32_t)(mab >> 32); }
      if (rank_path[h] && bj == tb[h]) {
        const int p = atomicAdd(&sh[h]->ccount, 1);
        ck[p] = key(h, i);
        ci[p] = (uint32_t)(tok0 + 64 * i);
      }
    }
  }
  __syncthreads();

  // 3. the need best tokens of each threshold bin (head h ranked by the
  // threads of half h of the block: nc <= kRankMax <= NTHR / 2)
  static_assert(kRankMax <= NTHR / 2, "one thread per candidate");
  if (rank_path[0] || rank_path[1]) {  // uniform
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (rank_path[h]) {
        uint32_t* tk = take[h];
        rank_candidates<NTHR / 2>(lds[h], lds[h] + kCap, nc[h], need[h],
                                  [&](uint32_t ii) { atomicOr(&tk[ii >> 5], 1u << (ii & 31)); }, h * (NTHR / 2));
      }
    __syncthreads();
    const int st = wave * T + lane;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (rank_path[h] && lane < T && 2 * st < W) { klo[h] |= take[h][2 * st]; khi[h] |= take[h][2 * st + 1]; }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (rank_path[h]) continue;  // uniform
    // crowded threshold bin: exact radix select inside it (as in select_regs)
    uint32_t* hist = lds[h];
    uint32_t prefix = 0u, pmask = 0u;
    int rem = need[h];
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int sft = shifts[pass];
      const uint32_t dm = (1u << widths[pass]) - 1u;
      for (int i = tid; i < kNB; i += NTHR) hist[i] = 0u;
      __syncthreads();
      const int nvp = opaque(nv);
#pragma unroll
      for (int i = 0; i < T; ++i)
        if (i < nvp && kb[h][i] == tb[h] && (key(h, i) & pmask) == prefix)
          atomicAdd(&hist[(key(h, i) >> sft) & dm], 1u);
      __syncthreads();
      find_threshold<NTHR>(hist, rem, *sh[h]);
      rem -= sh[h]->above;
      prefix |= (uint32_t)sh[h]->t << sft;
      pmask |= dm << sft;
      __syncthreads();
    }
    const uint32_t kstar = prefix;
    const int quota = rem;
    int neq = 0;
    const int nve = opaque(nv);
#pragma unroll
    for (int i = 0; i < T; ++i) neq += __popcll(__ballot(i < nve && key(h, i) == kstar));
    if (lane == 0) sh[h]->weq[wave] = neq;
    __syncthreads();
    int eqrun = waves_below<NTHR>(sh[h]->weq);
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const bool valid = i < nve;
      const bool eq = valid && key(h, i) == kstar;
      const uint64_t eqm = __ballot(eq);
      const bool tk = (valid && key(h, i) > kstar && kb[h][i] == tb[h]) ||
                      (eq && eqrun + bits_below(eqm) < quota);
      const uint64_t tm = __ballot(tk);
      if (lane == i) { klo[h] |= (uint32_t)tm; khi[h] |= (uint32_t)(tm >> 32); }
      eqrun += __popcll(eqm);
    }
  }

  // 4. each step's kept mask to head h's bitmap
  const int st = wave * T + lane;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (lane < T && 2 * st < W) *reinterpret_cast<uint2*>(brow[h] + 2 * st) = make_uint2(klo[h], khi[h]);
}

// ============================================================================
// Two heads whose tokens at or above an estimated bin are already marked: a
// caller that knows, for head h, a bin te[h] and has set bit t of cand[h] for
// every token t whose bin is te[h] or higher (e.g. while the scores were
// made, te[h] estimated from the first keys) lets the final passes visit only
// those tokens instead of all S.  The result is select_regs2's: the same
// histograms give the same threshold bin t_h, every token above it is kept,
// and bin t_h's tokens (all marked, when te[h] <= t_h) are ranked exactly.
// Scores in sbits[h][token] (fp32 bits), histograms in lds[h] over the bins
// of kmm[h], take[h] zero and sh[h]->ccount 0 on entry.  Returns true with
// take[h] = head h's kept-token bitmap (its ranking's bits ordered by the
// caller's next barrier), or false, having changed nothing but sh[h]->t /
// above / nt, when te[h] lies above t_h (the estimate missed) or bin t_h is
// crowded (> kRankMax tokens): then the caller selects with select_regs2.
// Uniform over the block.
// ============================================================================
template <int NTHR>
__device__ __forceinline__ bool select_cands2(const uint32_t* const (&sbits)[2], uint32_t* const (&lds)[2],
                                              uint32_t* const (&take)[2], const uint32_t* const (&cand)[2],
                                              int te0, int te1, int S, int k, SelScratch<NTHR>* const (&sh)[2],
                                              const uint32_t* const (&kmm)[2]) {
  find_thresholds2<NTHR>(lds[0], lds[1], k, k, sh);  // ends every read of the histograms
  int tb[2], need[2], nc[2];
  bool ok = true;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    tb[h] = sh[h]->t;
    need[h] = k - sh[h]->above;
    nc[h] = sh[h]->nt;
    ok = ok && tb[h] >= (h ? te1 : te0) && nc[h] <= kRankMax;
  }
  if (!ok) return false;
  Binner bin[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) bin[h].init(kmm[h][0], kmm[h][1]);
  // one bitmap word of one head per thread (2 ceil(S / 32) <= NTHR words for
  // S <= 16 NTHR): the marked tokens above t_h set the kept word, those of
  // bin t_h join the head's candidates in the space of its histogram
  const int Wh = (S + 31) >> 5;
  for (int i = threadIdx.x; i < 2 * Wh; i += NTHR) {
    const int h = i >= Wh ? 1 : 0, w = i - h * Wh;
    const Binner bh = h ? bin[1] : bin[0];
    const int th = h ? tb[1] : tb[0];
    const uint32_t* sb = h ? sbits[1] : sbits[0];
    uint32_t* ck = h ? lds[1] : lds[0];
    uint32_t c = h ? cand[1][w] : cand[0][w], word = 0u;
    while (c) {
      const int j = __ffs(c) - 1;
      c &= c - 1u;
      const int t = 32 * w + j;
      const float sc = __uint_as_float(sb[t]);
      const int b = bh.of_score(sc);
      if (b > th) {
        word |= 1u << j;
      } else if (b == th) {
        const int p = atomicAdd(&sh[h]->ccount, 1);
        ck[p] = score_key(sc);
        ck[kCap + p] = (uint32_t)t;
      }
    }
    (h ? take[1] : take[0])[w] = word;
  }
  __syncthreads();
  // the need best of each threshold bin (head h ranked by half h of the block)
  static_assert(kRankMax <= NTHR / 2, "one thread per candidate");
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t* tk = take[h];
    rank_candidates<NTHR / 2>(lds[h], lds[h] + kCap, nc[h], need[h],
                              [&](uint32_t ii) { atomicOr(&tk[ii >> 5], 1u << (ii & 31)); }, h * (NTHR / 2));
  }
  return true;
}

// ============================================================================
// Keys in global memory (heads longer than the register form holds).
// ============================================================================

// Calls f(j, key) for every token j < S (in no particular order): each thread
// reads 4 consecutive keys per 16-byte load with 8 loads in flight.
template <int NTHR, typename F>
__device__ __forceinline__ void for_each_key(const uint32_t* rk, int S, int Sp, F&& f) {
  constexpr int UB = 8;
  const uint4* src = reinterpret_cast<const uint4*>(rk);
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

// Steps 1-4 for one head with k < S, keys rk[0..S) in global memory and
// mm[0..nmm) min / max pairs covering them.  hist: kNB words of LDS, zeroed
// by the caller (a barrier inside orders it); masks: Sp / 16 words of global
// scratch, per step {above lo, hi, taken lo, hi}.  All threads call it.
template <int NTHR>
__device__ __forceinline__ void select_head(const uint32_t* rk, const uint2* mm, int nmm, uint32_t* hist,
                                            uint32_t* masks, int S, int Sp, int k, int32_t* orow,
                                            uint32_t* brow, SelScratch<NTHR>& sh) {
  constexpr int NW = NTHR / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int c = tid; c < nmm; c += NTHR) {
    const uint2 v = mm[c];
    mn = min(mn, v.x);
    mx = max(mx, v.y);
  }
  uint32_t kmin, kmax;
  block_minmax<NTHR>(mn, mx, sh, kmin, kmax);  // its barrier also orders the caller's zeroing
  Binner bin;
  bin.init(kmin, kmax);
  for_each_key<NTHR>(rk, S, Sp, [&](int, uint32_t v) { atomicAdd(&hist[bin(v)], 1u); });
  __syncthreads();

  // 1. threshold bin
  find_threshold<NTHR>(hist, k, sh);
  const int tb = sh.t;
  const int need = k - sh.above;  // 1 <= need <= hist[tb]
  const int nc = (int)hist[tb];
  const bool rank_path = nc <= kRankMax;
  if (tid == 0) sh.ccount = 0;
  __syncthreads();  // hist is reused below

  // 2. masks in index order; each wave owns a 64-aligned segment
  constexpr int UE = 8;
  const int SEG = (S + NW * 64 - 1) / (NW * 64) * 64;
  const int wb = wave * SEG, we = min(S, wb + SEG);
  uint32_t* ck = hist;
  uint32_t* ci = hist + kCap;
  for (int j0 = wb; j0 < we; j0 += 64 * UE) {
    uint32_t v[UE];
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int j = j0 + 64 * u + lane;
      v[u] = (j < we) ? rk[j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int js = j0 + 64 * u;
      if (js >= we) break;  // uniform across the wave
      const int j = js + lane;
      const int bj = (j < we) ? bin(v[u]) : -1;
      const uint64_t mab = __ballot(bj > tb);
      if (lane == 0)
        *reinterpret_cast<uint4*>(masks + 4 * (js >> 6)) =
            make_uint4((uint32_t)mab, (uint32_t)(mab >> 32), 0u, 0u);
      if (rank_path && bj == tb) {
        const int p = atomicAdd(&sh.ccount, 1);
        ck[p] = v[u];
        ci[p] = (uint32_t)j;
      }
    }
  }
  __syncthreads();

  // 3. the need best tokens of bin tb
  if (rank_path) {
    rank_candidates<NTHR>(ck, ci, nc, need, [&](uint32_t ii) {
      atomicOr(&masks[4 * (ii >> 6) + 2 + ((ii >> 5) & 1)], 1u << (ii & 31));
    });
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
      for_each_key<NTHR>(rk, S, Sp, [&](int, uint32_t v) {
        if (bin(v) == tb && (v & pmask) == prefix) atomicAdd(&hist[(v >> sft) & dm], 1u);
      });
      __syncthreads();
      find_threshold<NTHR>(hist, rem, sh);
      rem -= sh.above;
      prefix |= (uint32_t)sh.t << sft;
      pmask |= dm << sft;
      __syncthreads();
    }
    const uint32_t kstar = prefix;
    const int quota = rem;
    int neq = 0;
    for (int j0 = wb; j0 < we; j0 += 64) {
      const int j = j0 + lane;
      neq += __popcll(__ballot(j < we && rk[j] == kstar));
    }
    if (lane == 0) sh.weq[wave] = neq;
    __syncthreads();
    int eqrun = waves_below<NTHR>(sh.weq);
    for (int j0 = wb; j0 < we; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t v = (j < we) ? rk[j] : 0u;
      const bool valid = j < we;
      const bool eq = valid && v == kstar;
      const uint64_t eqm = __ballot(eq);
      const bool tk = (valid && v > kstar && bin(v) == tb) || (eq && eqrun + bits_below(eqm) < quota);
      const uint64_t tm = __ballot(tk);
      if (lane == 0)
        *reinterpret_cast<uint2*>(masks + 4 * (j0 >> 6) + 2) = make_uint2((uint32_t)tm, (uint32_t)(tm >> 32));
      eqrun += __popcll(eqm);
    }
  }
  __syncthreads();

  // 4. emit; lane i handles step s0 + 64 c + i of this wave's steps [s0, s1)
  const int s0 = wb >> 6, s1 = (we + 63) >> 6;
  int cnt = 0;
  for (int s = s0 + lane; s < s1; s += 64) {
    const uint4 m = *reinterpret_cast<const uint4*>(masks + 4 * s);
    cnt += __popc(m.x | m.z) + __popc(m.y | m.w);
  }
  cnt = wave_incl_scan(cnt);
  if (lane == 63) sh.wsel[wave] = cnt;
  __syncthreads();
  int pos = waves_below<NTHR>(sh.wsel);
  for (int c = s0; c < s1; c += 64) {
    const int s = c + lane;
    uint32_t lo = 0u, hi = 0u;
    if (s < s1) {
      const uint4 m = *reinterpret_cast<const uint4*>(masks + 4 * s);
      lo = m.x | m.z;
      hi = m.y | m.w;
      *reinterpret_cast<uint2*>(brow + 2 * s) = make_uint2(lo, hi);
    }
    const int n = __popc(lo) + __popc(hi);
    const int incl = wave_incl_scan(n);
    const int o = pos + incl - n;
    const int ns = min(64, s1 - c);
    for (int i = 0; i < ns; ++i) {
      const uint64_t f = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, i) << 32) |
                         (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lo, i);
      const int oi = __builtin_amdgcn_readlane(o, i);
      if ((f >> lane) & 1ull) orow[oi + bits_below(f)] = 64 * (c + i) + lane;
    }
    pos += __builtin_amdgcn_readlane(incl, 63);
  }
}

}  // namespace loki
