// Decode of grouped query heads two at a time (bf16 caches, G even, a
// head's keys fit in LDS): one block of 1024 threads per pair of query heads
// of a (b, kv) group rotates the pair's queries, scores every cached token
// for both heads from one read of the group's score source, selects each
// head's k best tokens and runs the exact attention of
// both heads over their kept tokens and writes the outputs: the whole decode
// step of the pair in one launch.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "attend_core.h"
#include "common.h"
#include "internal.h"
#include "mfma_common.h"
#include "select_core.h"

namespace loki {

// ============================================================================
// Pair kernel: one block of 1024 threads per pair of query heads of a
// (b, kv) group, one block per CU.  A CU's vector-memory path, not HBM,
// limits a kernel in which each query head re-reads its group's source, so
// the pair shares one read: the MFMA A operand carries both heads' split
// rows, the two heads' scores (2 x S words) go to LDS, and one two-head
// selection (select_regs2) keeps the k best of each.  The G / 2 pairs of a
// group get block ids with the same value mod 8 (one XCD) and consecutive
// dispatch order, so their reads of the group's source share L2.
//
// The kept-token bitmaps stay in LDS; the block lists the union of the
// pair's kept tokens in ascending order and runs the exact attention of both
// heads over it (section below), writing the pair's outputs.  Nothing else
// goes to global memory but idx.
// MODE 1: the exact stage takes q_rot against the rotated keys.
// MODE 2: the exact stage takes the query itself against unrotated keys (the
//         asymmetric index: the scores used q A).
// ============================================================================
template <int KS, int U, int D, int MODE>
__global__ __launch_bounds__(kPairThreads, 4) void score_select_pair_kernel(
    const bf16_t* __restrict__ src, int ld, const bf16_t* __restrict__ q, const bf16_t* __restrict__ P, int B,
    int Hq, int Hkv, int Scap, int Sp, int r, int k, int W, int32_t* __restrict__ idx, const bf16_t* __restrict__ Kx,
    const bf16_t* __restrict__ V, bf16_t* __restrict__ out, float scale_log2, const int32_t* __restrict__ lens) {
  static_assert(MODE == 1 || MODE == 2, "exact stage on q_rot or on the query itself");
  constexpr int NWV = kPairThreads / 64;
  constexpr int T = kFusedMaxS / kPairThreads;  // keys per lane in the selection
  constexpr int d = D;
  extern __shared__ __align__(16) uint32_t lk[];  // [2][Sp] fp32 score bits (first: rotation scratch)
  __shared__ __align__(16) uint32_t sel[2][kNB];
  __shared__ __align__(16) uint32_t take[2][kFusedMaxS / 32];
  __shared__ __align__(16) uint32_t cand[2][kFusedMaxS / 32];  // tokens at or above each head's estimated bin
  __shared__ SelScratch<kPairThreads> sh[2];
  __shared__ uint32_t smm[2][2];  // per head {min, max} key
  __shared__ __align__(16) uint16_t sqs[2 * 4 * D];  // the pair's split rows [h][part][d]
  __shared__ __align__(16) uint16_t sqp[MODE == 2 ? 2 * 4 * D : 8];  // the query itself, split
  __shared__ int s_n;
  const int G = Hq / Hkv, NP = G / 2;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int gp = slot % NP, gi = (slot / NP) * 8 + xcd;
  if (gi >= B * Hkv) return;  // padding block (uniform)
  const int b = gi / Hkv, kv = gi - b * Hkv;
  const int S = seq_len(lens, b, Scap);  // this sequence's tokens
  const size_t row0 = (size_t)b * Hq + (size_t)kv * G + 2 * gp;
  const int tid = threadIdx.x, lane = tid & 63;
  const int m = lane & 15, q4 = lane >> 4;
  uint32_t* const brow2[2] = {take[0], take[1]};

  // Wave w takes tiles w + NWV i (16 tokens each) in batches of U, double
  // buffered: the next batch is in flight while this one is multiplied.
  // Loads are unconditional (token clamped to S - 1, dims to the row) so
  // that each tile waits only for its own data; dims >= r are zeroed at the
  // MFMA, tiles past S are dropped at the store.
  const bf16_t* base = src + (size_t)gi * Scap * ld;  // rows of the cache (capacity Scap)
  const int nbat = ((S + 15) / 16 + NWV * U - 1) / (NWV * U);
  // The lane's first token (16 wave + m) is recomputed from the thread id
  // (opaque) wherever the score phase needs it: a copy kept live from the
  // top gets spilled, and reloading it waits for every load in flight.
  auto lane_tok = [&]() {
    const int tt = opaque(tid);
    return 16 * (tt >> 6) + (tt & 15);
  };
  auto load_batch = [&](int bi, uint4 (&a)[U][KS]) {
    const int tl = lane_tok();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(tl + 16 * NWV * (bi * U + u), S - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) a[u][s] = ldg16(base + (size_t)t * ld + min(32 * s + 8 * q4, ld - 8));
    }
  };
  // the pair's query rotation q_rot = q P[kv], with the arithmetic of
  // qrot_kernel (d / 8-term FMA chains over eight j-slices, added in slice
  // order): the split rows go to LDS as this block's A operands.  The P
  // slices and q are requested first, then the first K batch.  Thread
  // js NC4 + c4 of the first 8 NC4 (whole waves) holds rows js J .. js J + J
  // of columns 4 c4 .. 4 c4 + 3 (8-byte loads): a quarter of the block
  // requests P, in a quarter of the load instructions that one column per
  // thread would take (the CU's memory pipe then takes the key batch
  // sooner); every column's chain is unchanged.
  constexpr int J = D / 8, NC4 = D / 4;
  const int c4 = tid % NC4, js = tid / NC4;
  const bool ploader = __builtin_amdgcn_readfirstlane(tid >> 6) < 8 * NC4 / 64;  // uniform per wave
  uint2 pv[J];  // P[kv][js J + jj][4 c4 .. 4 c4 + 3]
  if (ploader) {
    const bf16_t* Pc = P + (size_t)kv * d * d + (size_t)js * J * d + 4 * c4;
#pragma unroll
    for (int jj = 0; jj < J; ++jj) pv[jj] = *reinterpret_cast<const uint2*>(Pc + (size_t)jj * d);
  }
  float* sq = reinterpret_cast<float*>(lk);  // [2][d]
  float* sred = sq + 2 * d;                  // [8][2][d]
  // the pair's heads are adjacent rows of q; the value goes to LDS after the
  // first key batch is requested, so that waiting for it (in order) leaves
  // the batch in flight
  // (q reached through an opaque copy of the pointer and a compiler barrier,
  // which keep its load above the batch's: no instruction is emitted)
  const bf16_t* qp = q + row0 * d;
  asm volatile("" : "+s"(qp));
  using gbf16_t = const __attribute__((address_space(1))) bf16_t;  // a global-memory load, not a flat one
  const bf16_t qv = ((gbf16_t*)qp)[min(tid, 2 * d - 1)];
  asm volatile("" ::: "memory");
  uint4 a0[U][KS], a1[U][KS];
  load_batch(0, a0);  // in flight during the rotation (unused when every token is kept)
  if (tid < 2 * d) sq[tid] = to_f32(qv);
  {
    __syncthreads();
    if (ploader) {
      float r[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int jj = 0; jj < J; ++jj) {
        const int j = js * J + jj;
        const float q0 = sq[j], q1 = sq[d + j];
        const float pj[4] = {__uint_as_float(pv[jj].x << 16), __uint_as_float(pv[jj].x & 0xffff0000u),
                             __uint_as_float(pv[jj].y << 16), __uint_as_float(pv[jj].y & 0xffff0000u)};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          r[0][c] = fmaf(q0, pj[c], r[0][c]);
          r[1][c] = fmaf(q1, pj[c], r[1][c]);
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sred[(2 * js) * d + 4 * c4 + c] = r[0][c];
        sred[(2 * js + 1) * d + 4 * c4 + c] = r[1][c];
      }
    }
    __syncthreads();
    // the thread's row and column are recomputed here (opaque): a copy kept
    // from the top would be spilled, and its reload would wait for every
    // load in flight (the first key batch), not only for the rotation's
    const int tr = opaque(tid);
    if (tr < 2 * d) {
      const int h = tr / d, cc = tr - h * d;
      float v = sred[h * d + cc];
      for (int t = 1; t < 8; ++t) v += sred[(2 * t + h) * d + cc];
      const bf16_t hi = f32_to_bf16(v);
      const float e1 = v - to_f32(hi);
      const bf16_t mid = f32_to_bf16(e1);
      const bf16_t lo = f32_to_bf16(e1 - to_f32(mid));
      const bf16_t part[4] = {hi, mid, lo, 0};
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) sqs[(h * 4 + pt) * d + cc] = part[pt];
      if constexpr (MODE == 2) {
        // the query itself: a bf16 value is its own first split part
        sqp[(h * 4) * d + cc] = q[row0 * d + tr];
#pragma unroll
        for (int pt = 1; pt < 4; ++pt) sqp[(h * 4 + pt) * d + cc] = 0;
      }
    }
    __syncthreads();
  }

  if (k >= S) {
    keep_all<kPairThreads>(S, k, W, idx + row0 * k, brow2[0]);
    keep_all<kPairThreads>(S, k, W, idx + (row0 + 1) * k, brow2[1]);
  } else {
    SelScratch<kPairThreads>* const sh2e[2] = {&sh[0], &sh[1]};
    // A operands: the pair's two heads in rows 0..7 (row 4 h + split)
    bf16x8_t qa[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qa[s] = q_rows(sqs, 0, d, 2, r, m, 32 * s + 8 * q4);

    // Both heads' histograms are built while the keys are made, over value
    // bins fixed by the range of the first batch's keys (later keys outside
    // it fall into the end bins; the map stays monotone, so the selection is
    // exact whatever the range, which only sets how many keys share the
    // threshold bin): the selection then needs no histogram pass of its own.
    uint32_t kmn = 0xffffffffu, kmx = 0u;
    Binner bq;  // this lane's head's bins (set after the first batch)
    int te = kNB;  // this lane's head's estimated bin (set after the first two batches)
    auto score_batch = [&](int bi, const uint4 (&a)[U][KS], auto binning) {
      const int tl = lane_tok();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const uint4 x = 32 * s + 8 * q4 < r ? a[u][s] : make_uint4(0u, 0u, 0u, 0u);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], as_bf16x8(x), acc, 0, 0, 0);
        }
        const int t = tl + 16 * NWV * (bi * U + u);  // this lane's token; its head is q4
        if (q4 < 2 && t < S) {
          const float sc = sum_split_rows(acc);
          lk[q4 * Sp + t] = __float_as_uint(sc);  // the selection bins the value itself
          if constexpr (decltype(binning)::value) {
            const int bn = bq.of_score(sc);
            atomicAdd(&sel[q4][bn], 1u);
            if (bn >= te) atomicOr(&cand[q4][t >> 5], 1u << (t & 31));
          } else {
            const uint32_t key = score_key(sc);
            kmn = min(kmn, key);
            kmx = max(kmx, key);
          }
        }
      }
    };
    // the histograms are cleared now, under the loads in flight
    for (int i = tid; i < 2 * kNB; i += kPairThreads) (&sel[0][0])[i] = 0u;
    for (int i = tid; i < 2 * (kFusedMaxS / 32); i += kPairThreads) (&take[0][0])[i] = 0u;
    for (int i = tid; i < 2 * (kFusedMaxS / 32); i += kPairThreads) (&cand[0][0])[i] = 0u;
    if (tid < 2) {
      smm[tid][0] = 0xffffffffu;
      smm[tid][1] = 0u;
      sh[tid].ccount = 0;
    }
    __syncthreads();  // orders the initialisation before the atomics below
    // the first batch: its keys' range per head fixes the bins
    load_batch(1, a1);
    score_batch(0, a0, std::false_type{});
    load_batch(2, a0);
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) {  // over the 16 lanes of a head's row
      kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, x));
      kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, x));
    }
    if (m == 0 && q4 < 2) {
      atomicMin(&smm[q4][0], kmn);
      atomicMax(&smm[q4][1], kmx);
    }
    __syncthreads();
    bq.init(smm[q4 & 1][0], smm[q4 & 1][1]);
    // this lane's first token, recomputed (opaque) for the read-back passes
    // below: a reload of a spilled copy would wait for the batches in flight
    const int tok_l = lane_tok();
#pragma unroll
    for (int u = 0; u < U; ++u) {  // the first batch's keys, read back
      const int t = tok_l + 16 * NWV * u;
      if (q4 < 2 && t < S) atomicAdd(&sel[q4][bq.of_score(__uint_as_float(lk[q4 * Sp + t]))], 1u);
    }
    // the second batch (a1): counted, not yet marked (te is past every bin);
    // the fourth is requested before the estimate's barriers
    score_batch(1, a1, std::true_type{});
    load_batch(3, a1);
    // A lower bound on each head's final threshold bin, so that
    // the selection visits only the tokens at or above it.  The first two
    // batches (the first n0 tokens) hold about k n0 / S of the head's k best;
    // the bin of their want-th largest key, want a quarter above that plus
    // 32, is then at or below the final threshold bin unless the best tokens
    // crowd the start of the sequence (then the selection falls back to the
    // full passes: the estimate only decides which tokens are marked, never
    // the result).  Computed while the next two batches are in flight.
    int te0 = 0, te1 = 0;
    {
      __syncthreads();  // the first two batches' counts are complete
      const int n0 = min(S, 2 * 16 * NWV * U);
      const int want = (int)min((long long)n0, (5LL * k * n0 + 4LL * S - 1) / (4LL * S) + 32);
      find_thresholds2<kPairThreads>(sel[0], sel[1], want, want, sh2e);
      te0 = sh[0].t;
      te1 = sh[1].t;
      te = (q4 & 1) ? te1 : te0;
#pragma unroll
      for (int u = 0; u < 2 * U; ++u) {  // the first two batches' tokens at or above the estimate
        const int t = tok_l + 16 * NWV * u;
        if (q4 < 2 && t < S && bq.of_score(__uint_as_float(lk[q4 * Sp + t])) >= te)
          atomicOr(&cand[q4][t >> 5], 1u << (t & 31));
      }
    }
    // batch bi is in a0 and bi + 1 in a1 at the top of each step; the steady
    // loop only requests batches that exist, and the last one to three are
    // scored after it, so that no load is left in flight past the scores
    // (batches past the end, here and for nbat <= 4, score no token)
    int bi = 2;
    for (; bi + 3 < nbat; bi += 2) {
      score_batch(bi, a0, std::true_type{});
      load_batch(bi + 2, a0);
      score_batch(bi + 1, a1, std::true_type{});
      load_batch(bi + 3, a1);
    }
    score_batch(bi, a0, std::true_type{});
    if (bi + 2 < nbat) {  // uniform
      load_batch(bi + 2, a0);
      score_batch(bi + 1, a1, std::true_type{});
      score_batch(bi + 2, a0, std::true_type{});
    } else {
      score_batch(bi + 1, a1, std::true_type{});
    }
    __syncthreads();  // every key and histogram count is in LDS
    const uint32_t* const key[2] = {lk, lk + Sp};  // the scores stay in LDS
    uint32_t* const lds2[2] = {sel[0], sel[1]};
    uint32_t* const take2[2] = {take[0], take[1]};
    SelScratch<kPairThreads>* const sh2[2] = {&sh[0], &sh[1]};
    const uint32_t* const kmm2[2] = {smm[0], smm[1]};
    // the selection leaves the kept-token bitmaps in take (idx is written
    // while the kept tokens are listed below); it first tries the marked
    // tokens only (the same result when the estimate holds)
    const uint32_t* const cand2[2] = {cand[0], cand[1]};
    if (!select_cands2<kPairThreads>(key, lds2, take2, cand2, te0, te1, S, k, sh2, kmm2))  // uniform
      select_regs2<kPairThreads, T>(key, lds2, take2, S, k, W, brow2, sh2, kmm2, true);
  }
  {
    // ========================================================================
    // Exact attention of the pair's two heads over their kept tokens.  The
    // union of the two kept sets is listed in ascending token order (entry =
    // token | kept-by-head-0 << 30 | kept-by-head-1 << 31) in the LDS that
    // held the keys; thread w lists bitmap word w, at offsets from block
    // scans of the union's and of each head's counts, and writes each head's
    // kept tokens to its idx row (ascending) at the same time.  attend_list
    // (attend_core.h) then runs both heads' attention in one pass over it.
    // ========================================================================
    __syncthreads();  // the bitmaps (take) are complete
    uint32_t* list = lk;
    {
      uint32_t u0 = 0u, u1 = 0u;
      if (tid < W) {
        u0 = take[0][tid];
        u1 = take[1][tid];
      }
      uint32_t u = u0 | u1;
      const int c = __popc(u), c0 = __popc(u0), c1 = __popc(u1);
      // the union's counts, and both heads' in 16 bits each (a head keeps
      // <= 16384), scanned together
      int incl = c, incl01 = c0 | (c1 << 16);
      block_incl_scan2<kPairThreads>(incl, incl01, sh[0], sh[1]);
      if (tid == kPairThreads - 1) {
        s_n = incl;
        for (int j = 0; j < kListPad; ++j) list[incl + j] = 0u;  // the attention's padding
      }
      int pos = incl - c, p0 = (incl01 & 0xffff) - c0, p1 = (incl01 >> 16) - c1;
      int32_t* const o0 = idx + row0 * k;
      int32_t* const o1 = idx + (row0 + 1) * k;
      const bool wr = k < S;  // else keep_all wrote idx (with the -1 padding)
      while (u) {
        const int j = __ffs(u) - 1;
        u &= u - 1u;
        const uint32_t t = (uint32_t)(32 * tid + j), b0 = (u0 >> j) & 1u, b1 = (u1 >> j) & 1u;
        list[pos++] = t | (b0 << 30) | (b1 << 31);
        if (wr && b0) o0[p0++] = (int32_t)t;
        if (wr && b1) o1[p1++] = (int32_t)t;
      }
    }
    __syncthreads();
    // the attention itself (both heads, one pass over the list); its merge
    // scratch follows the list (<= Sp entries and the padding) in the LDS that held the keys
    const size_t cb = (size_t)gi * Scap * D;  // this group's rows of K and V
    attend_list<D, 2, kPairThreads>(list, s_n, MODE == 2 ? sqp : sqs, Kx + cb, V + cb, scale_log2, out + row0 * D,
                                    reinterpret_cast<float*>(lk + Sp + kListPad));
  }
}

// ============================================================================
// host side
// ============================================================================
bool score_select_pair_fits(const DecodePlan& p) {
  return p.dt == 1 && p.G >= 2 && p.G % 2 == 0 && p.S <= kFusedMaxS && p.r <= 128 && (p.d == 64 || p.d == 128);
}

template <int MODE>
static hipError_t launch_pair(const DecodePlan& p, const void* src, int ld, const void* q, const void* P,
                              int32_t* idx, const void* Kx, const void* V, void* out, hipStream_t st) {
  if (!score_select_pair_fits(p)) return hipErrorInvalidValue;
  // keys [2][Sp] (then the union list, <= Sp entries, and the attention's
  // merge scratch), at least the rotation scratch [2 + 16][d] words
  const int merge = p.d == 64 ? attend_merge_words<64, 2, kPairThreads>() : attend_merge_words<128, 2, kPairThreads>();
  const size_t lds = (size_t)max(max(2 * p.Sp, 18 * p.d), p.Sp + kListPad + merge) * sizeof(uint32_t);
  const int ngroups = p.B * p.Hkv;
  const dim3 grid((unsigned)((ngroups + 7) / 8 * 8 * (p.G / 2))), block(kPairThreads);
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.d));
  const bf16_t* s = static_cast<const bf16_t*>(src);
  auto go = [&](auto ks, auto dd) {
    constexpr int K = decltype(ks)::value, D = decltype(dd)::value;
    const void* fn = reinterpret_cast<const void*>(&score_select_pair_kernel<K, 8 / K, D, MODE>);
    // the limit covers every call of this kernel: keys of the longest head it takes
    hipError_t e = ensure_dynamic_lds(fn, (int)max(lds, (size_t)2 * kFusedMaxS * sizeof(uint32_t)));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((score_select_pair_kernel<K, 8 / K, D, MODE>), grid, block, lds, st, s, ld,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(P), p.B, p.Hq, p.Hkv, p.S, p.Sp,
                       p.r, p.k, p.W, idx, static_cast<const bf16_t*>(Kx),
                       static_cast<const bf16_t*>(V), static_cast<bf16_t*>(out), scale_log2, p.lens);
    return hipGetLastError();
  };
  auto by_d = [&](auto ks) {
    return p.d == 64 ? go(ks, std::integral_constant<int, 64>{}) : go(ks, std::integral_constant<int, 128>{});
  };
  switch ((p.r + 31) / 32) {
    case 1: return by_d(std::integral_constant<int, 1>{});
    case 2: return by_d(std::integral_constant<int, 2>{});
    case 3: return by_d(std::integral_constant<int, 3>{});
    case 4: return by_d(std::integral_constant<int, 4>{});
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_pair(const DecodePlan& p, const void* src, int ld, const void* q, const void* P,
                              const void* Kx, const void* V, void* out, int32_t* idx, bool plain, hipStream_t st) {
  return plain ? launch_pair<2>(p, src, ld, q, P, idx, Kx, V, out, st)
               : launch_pair<1>(p, src, ld, q, P, idx, Kx, V, out, st);
}

}  // namespace loki
