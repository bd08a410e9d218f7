// MFMA forms of the two contractions of a decode step over bf16 caches:
//   scores   s[j, h] = sum_{c<r} K[j, c] q_rot[h, c]   (all tokens j, the G heads of a group)
//   exact    e[j, h] = sum_{c<d} K_rot[j, c] q_rot[h, c] (the kept tokens)
// Both are [tokens x dims] x [dims x heads] products.  With G query heads per
// key row they cost 4G flops per cached element, which on the vector ALUs
// (no packed fp32) would take most of the issue rate at HBM speed; on
// v_mfma_f32_16x16x32_bf16 they cost a few instructions per 16 tokens.
//
// q_rot is fp32 and must not be rounded to bf16: the rotation kernel splits
// it into three bf16 parts q = h + m + l (|q - h - m - l| <= 2^-27 |q|).
// One MFMA yields the three partial products of four heads with exact
// bf16 x bf16 products and fp32 accumulation.  The approximate-score kernels
// put the heads in A rows (row 4 h + split, tokens in B columns): lane l
// ends with head l / 16's three partials for token l % 16 and adds them
// itself, so every lane carries a result.  The exact-score pass of the
// attention kernel puts them in B columns (column n = head (n % 4) + 4 split)
// and adds each head's three columns with two DPP row shifts.  Both add the
// parts as (h + m) + (l + 0), so the two layouts give identical scores.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l, element i):
//   A[m][k] : m = l % 16, k = 8 (l / 16) + i
//   B[k][n] : n = l % 16, k = 8 (l / 16) + i
//   D[m][n] : n = l % 16, m = 4 (l / 16) + v   (v = 0..3, one fp32 each)
// The mapping of k to head dimensions is free as long as A and B agree; each
// kernel picks the one that keeps a lane's loads contiguous.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma_common.h"
#include "select_core.h"

namespace loki {

// ============================================================================
// Approximate scores, bf16 source (K_rot with ld = d, or K_lead with ld = R).
// Block = SC tokens of one (b, kv) group; wave w takes the chunk's 16-token
// tiles w + 4 i in batches of U, double buffered.  For k-step s a lane loads
// dims [32 s + 8 (l/16), +8) of token l % 16 (the B operand), so one load
// instruction covers 16 tokens x 64 contiguous bytes of a dense K_lead;
// loads are unconditional (token clamped into the chunk, dims into the row)
// so that a tile waits only for its own data.  The heads sit in A rows, four
// per MFMA: lane l ends with the score of head 4 grp + l / 16 for token l % 16.
// ============================================================================
template <int GT, int KS, bool KEYS>
__global__ __launch_bounds__(256) void score_mfma_kernel(const bf16_t* __restrict__ src,
                                                         const uint16_t* __restrict__ qsplit,
                                                         void* __restrict__ out, int out_stride,
                                                         uint2* __restrict__ mm, int Hq, int Hkv,
                                                         int S, int d, int ld, int r, int SC,
                                                         const int32_t* __restrict__ lens) {
  constexpr int NGRP = (GT + 3) / 4;
  constexpr int UK = 8 / (KS * NGRP);
  constexpr int U = UK < 1 ? 1 : UK;  // tiles per batch and wave
  const int G = Hq / Hkv;
  const int bk = blockIdx.y, b = bk / Hkv, kv = bk % Hkv;
  // tokens of this chunk that the sequence holds (none past its end: the
  // clamped loads below then repeat its last token and nothing is stored)
  const int t0 = blockIdx.x * SC, t1 = min(seq_len(lens, b, S), t0 + SC);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, q = lane >> 4;
  const size_t head0 = (size_t)b * Hq + (size_t)kv * G;

  bf16x8_t qa[NGRP][KS];
#pragma unroll
  for (int grp = 0; grp < NGRP; ++grp)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qa[grp][s] = q_rows(qsplit, head0 + 4 * grp, d, G - 4 * grp, r, m, 32 * s + 8 * q);
  // k-steps up to the last one where some head's query is non-zero (a query
  // masked to a few dims, as for query-magnitude scoring, may end early):
  // later k-steps re-read the first k-step's columns (cached, no new HBM
  // traffic) and multiply them by zeros, so every load stays unconditional
  int kuse = 0;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    bool nz = false;
#pragma unroll
    for (int grp = 0; grp < NGRP; ++grp) {
      const uint4 v = __builtin_bit_cast(uint4, qa[grp][s]);
      nz = nz || ((v.x | v.y | v.z | v.w) & 0x7fff7fffu) != 0u;
    }
    if (__ballot(nz)) kuse = s + 1;  // the same in every wave: they hold the same operands
  }

  const bf16_t* base = src + (size_t)bk * S * ld;
  __shared__ uint32_t smn[GT], smx[GT];
  if (KEYS && threadIdx.x < GT) { smn[threadIdx.x] = 0xffffffffu; smx[threadIdx.x] = 0u; }
  uint32_t mn[NGRP], mx[NGRP];
#pragma unroll
  for (int grp = 0; grp < NGRP; ++grp) { mn[grp] = 0xffffffffu; mx[grp] = 0u; }
  const int nbat = t1 > t0 ? ((t1 - t0 + 15) / 16 + 4 * U - 1) / (4 * U) : 0;
  auto load_batch = [&](int bi, uint4 (&a)[U][KS]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(t0 + 16 * (wave + 4 * (bi * U + u)) + m, t1 - 1);  // t1 >= 1
#pragma unroll
      for (int s = 0; s < KS; ++s)
        a[u][s] = ldg16(base + (size_t)t * ld + min((s < kuse ? 32 * s : 0) + 8 * q, ld - 8));
    }
  };
  auto score_batch = [&](int bi, const uint4 (&a)[U][KS]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + 16 * (wave + 4 * (bi * U + u)) + m;  // this lane's token
#pragma unroll
      for (int grp = 0; grp < NGRP; ++grp) {
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const uint4 x = 32 * s + 8 * q < r ? a[u][s] : make_uint4(0u, 0u, 0u, 0u);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[grp][s], as_bf16x8(x), acc, 0, 0, 0);
        }
        const float x = sum_split_rows(acc);
        const int g = 4 * grp + q;
        if (g < G && t < t1) {
          const size_t o = (head0 + g) * (size_t)out_stride + t;
          if constexpr (KEYS) {
            const uint32_t key = score_key(x);
            static_cast<uint32_t*>(out)[o] = key;
            mn[grp] = min(mn[grp], key);
            mx[grp] = max(mx[grp], key);
          } else {
            static_cast<float*>(out)[o] = x;
          }
        }
      }
    }
  };
  uint4 a0[U][KS], a1[U][KS];
  load_batch(0, a0);
  for (int bi = 0; bi < nbat; bi += 2) {  // an odd last batch is followed by an empty one
    load_batch(bi + 1, a1);
    score_batch(bi, a0);
    load_batch(bi + 2, a0);
    score_batch(bi + 1, a1);
  }
  if (KEYS && mm) {  // uniform: the chunk's min / max key per head
    __syncthreads();
#pragma unroll
    for (int grp = 0; grp < NGRP; ++grp) {
      const int g = 4 * grp + q;
      if (g < G && mn[grp] <= mx[grp]) { atomicMin(&smn[g], mn[grp]); atomicMax(&smx[g], mx[grp]); }
    }
    __syncthreads();
    if (threadIdx.x < G) mm[(head0 + threadIdx.x) * gridDim.x + blockIdx.x] = make_uint2(smn[threadIdx.x], smx[threadIdx.x]);
  }
}

// ============================================================================
// Fused approximate scores + top-k, one block of 512 threads per query head
// (bf16 source, the head's S keys fit in LDS).  The block streams its group's
// score source (16-token MFMA tiles as in score_mfma_kernel, with only this
// head's three split columns non-zero), writes the order-preserving keys
// straight into LDS while tracking their min / max, and then runs the
// selection of select_core.h in place: no key ever goes to global memory.
// Block -> (group, head) mapping: the G heads of a (b, kv) group get block
// ids with the same value mod 8 (the same XCD under round-robin dispatch)
// and consecutive dispatch order, so their identical reads of the group's
// source hit in L2 / the Infinity Cache.
// ============================================================================
template <int KS>
__global__ __launch_bounds__(kFusedThreads) void score_select_kernel(
    const bf16_t* __restrict__ src, int ld, const uint16_t* __restrict__ qsplit, int B, int Hq,
    int Hkv, int Scap, int Sp, int d, int r, int k, int W, int32_t* __restrict__ idx,
    uint32_t* __restrict__ bitmap, const int32_t* __restrict__ lens) {
  constexpr int NWV = kFusedThreads / 64;
  constexpr int UK = 8 / KS;
  constexpr int U = UK < 1 ? 1 : UK;  // tiles in flight per wave
  constexpr int T = kFusedMaxS / kFusedThreads;  // keys per lane in the selection
  extern __shared__ __align__(16) uint32_t lk[];  // [Sp] keys
  __shared__ uint32_t sel[kNB];
  __shared__ uint32_t take[kFusedMaxS / 32];
  __shared__ SelScratch<kFusedThreads> sh;
  const int G = Hq / Hkv;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int gh = slot % G, gi = (slot / G) * 8 + xcd;
  if (gi >= B * Hkv) return;  // padding block (uniform)
  const int b = gi / Hkv, kv = gi - b * Hkv;
  const int S = seq_len(lens, b, Scap);  // this sequence's tokens
  const size_t row = (size_t)b * Hq + (size_t)kv * G + gh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, q = lane >> 4;
  int32_t* orow = idx + row * k;
  uint32_t* brow = bitmap + row * W;

  if (k >= S) {
    keep_all<kFusedThreads>(S, k, W, orow, brow);
    return;
  }

  // A operands: this head's splits in rows 0..3
  bf16x8_t qa[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qa[s] = q_rows(qsplit, row, d, 1, r, m, 32 * s + 8 * q);

  // tiles of 16 tokens, wave w takes tiles w + NWV i in double-buffered
  // batches of U; unconditional loads as in score_mfma_kernel
  const bf16_t* base = src + (size_t)gi * Scap * ld;  // rows of the cache (capacity Scap)
  const int nbat = ((S + 15) / 16 + NWV * U - 1) / (NWV * U);
  auto load_batch = [&](int bi, uint4 (&a)[U][KS]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(16 * (wave + NWV * (bi * U + u)) + m, S - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) a[u][s] = ldg16(base + (size_t)t * ld + min(32 * s + 8 * q, ld - 8));
    }
  };
  auto score_batch = [&](int bi, const uint4 (&a)[U][KS]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint4 x = 32 * s + 8 * q < r ? a[u][s] : make_uint4(0u, 0u, 0u, 0u);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], as_bf16x8(x), acc, 0, 0, 0);
      }
      const int t = 16 * (wave + NWV * (bi * U + u)) + m;  // this lane's token (lanes 0..15)
      if (q == 0 && t < S) lk[t] = score_key(sum_split_rows(acc));
    }
  };
  uint4 a0[U][KS], a1[U][KS];
  load_batch(0, a0);
  for (int bi = 0; bi < nbat; bi += 2) {  // an odd last batch is followed by an empty one
    load_batch(bi + 1, a1);
    score_batch(bi, a0);
    load_batch(bi + 2, a0);
    score_batch(bi + 1, a1);
  }
  __syncthreads();
  uint32_t key[T];  // the selection's register layout
  load_regs<T>(lk, S, key);
  select_regs<kFusedThreads, T>(key, sel, take, S, k, W, orow, brow, sh);
}

// ============================================================================
// Long heads (bf16): fused approximate scores + the first selection stage, one
// block of 1024 threads per (query head, chunk of kSelChunk tokens).  The
// chunk's keys stay in LDS (they never go to HBM and back), and the block
// keeps the chunk's top-k with their keys in the candidate lists, chunk c at
// offset c k, positions made absolute, exactly as the workspace-key first
// stage does; free slots of a chunk with at most k tokens (or past the
// sequence's end) get index -1 and key 0, below every score's key.  The G
// query heads of a group's chunk get block ids with the same value mod 8 (one
// XCD) and consecutive dispatch order, so they share the chunk's reads in L2.
// ============================================================================
constexpr int kChunkThreads = 1024;

template <int KS>
__global__ __launch_bounds__(kChunkThreads) void score_select_chunk_kernel(
    const bf16_t* __restrict__ src, int ld, const uint16_t* __restrict__ qsplit, int B, int Hq, int Hkv,
    int Scap, int C, int d, int r, int k, int ldc, int32_t* __restrict__ cidx, uint32_t* __restrict__ ckey,
    const int32_t* __restrict__ lens) {
  constexpr int NWV = kChunkThreads / 64;
  constexpr int UK = 8 / KS;
  constexpr int U = UK < 1 ? 1 : UK;  // tiles in flight per wave
  constexpr int T = kSelChunk / kChunkThreads;  // keys per lane in the selection
  extern __shared__ __align__(16) uint32_t lk[];  // [kSelChunk] keys
  __shared__ uint32_t sel[kNB];
  __shared__ uint32_t take[kSelChunk / 32];
  __shared__ SelScratch<kChunkThreads> sh;
  const int G = Hq / Hkv;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int gh = slot % G, unit = (slot / G) * 8 + xcd;  // unit = (group, chunk)
  if (unit >= B * Hkv * C) return;  // padding block (uniform)
  const int gi = unit / C, c = unit - gi * C;
  const int b = gi / Hkv, kv = gi - b * Hkv;
  const int S = seq_len(lens, b, Scap);  // this sequence's tokens
  const int base = c * kSelChunk;
  const int L = min(kSelChunk, S - base);  // <= 0 past the sequence's end
  const size_t row = (size_t)b * Hq + (size_t)kv * G + gh;
  int32_t* oi = cidx + row * ldc + (size_t)c * k;
  uint32_t* ok = ckey + row * ldc + (size_t)c * k;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, q = lane >> 4;
  if (L <= 0) {
    for (int j = tid; j < k; j += kChunkThreads) {
      oi[j] = -1;
      ok[j] = 0u;
    }
    return;
  }

  bf16x8_t qa[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qa[s] = q_rows(qsplit, row, d, 1, r, m, 32 * s + 8 * q);

  // tiles of 16 tokens, wave w takes tiles w + NWV i in double-buffered
  // batches of U; unconditional loads (token clamped into the chunk)
  const bf16_t* cbase = src + ((size_t)gi * Scap + base) * ld;
  const int nbat = ((L + 15) / 16 + NWV * U - 1) / (NWV * U);
  auto load_batch = [&](int bi, uint4 (&a)[U][KS]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(16 * (wave + NWV * (bi * U + u)) + m, L - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) a[u][s] = ldg16(cbase + (size_t)t * ld + min(32 * s + 8 * q, ld - 8));
    }
  };
  auto score_batch = [&](int bi, const uint4 (&a)[U][KS]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint4 x = 32 * s + 8 * q < r ? a[u][s] : make_uint4(0u, 0u, 0u, 0u);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], as_bf16x8(x), acc, 0, 0, 0);
      }
      const int t = 16 * (wave + NWV * (bi * U + u)) + m;  // this lane's token (lanes 0..15)
      if (q == 0 && t < L) lk[t] = score_key(sum_split_rows(acc));
    }
  };
  uint4 a0[U][KS], a1[U][KS];
  load_batch(0, a0);
  for (int bi = 0; bi < nbat; bi += 2) {  // an odd last batch is followed by an empty one
    load_batch(bi + 1, a1);
    score_batch(bi, a0);
    load_batch(bi + 2, a0);
    score_batch(bi + 1, a1);
  }
  __syncthreads();
  if (L <= k) {  // the whole chunk is a candidate
    for (int j = tid; j < k; j += kChunkThreads) {
      oi[j] = j < L ? base + j : -1;
      ok[j] = j < L ? lk[j] : 0u;
    }
    return;
  }
  uint32_t key[T];  // the selection's register layout
  load_regs<T>(lk, L, key);
  // the winners' keys are read back from lk while they are listed
  select_regs<kChunkThreads, T>(key, sel, take, L, k, 2 * ((L + 63) / 64), oi, nullptr, sh, nullptr, ok, base,
                                nullptr, lk);
}

// ============================================================================
// Exact attention over the kept tokens, bf16 caches, G <= 8.
// Wave = a span of up to NT consecutive tokens of one (b, kv) group; four
// waves per block.  A full-length sequence gives every wave NT tokens; a
// shorter one (per-sequence lengths) is cut into the same number of narrower
// spans, whole bitmap words each, so that a block of a short sequence, whose
// kept tokens lie closer together, still sees about as many of them.
// The G heads' bitmap words of the span go through LDS (one load per lane)
// and give the union list (token, head mask).  Then two passes over it:
//   pass 1: 16-row K tiles in MFMA A layout (a load instruction reads 64
//           contiguous bytes of each of 16 rows), up to KT tiles requested
//           before any is used;
//           exact scores of all G heads from MFMA, scaled to log2 units,
//           -inf where a head did not keep the token, into LDS;
//   per head: m = max (kept by the score lanes during pass 1), then one
//           pass over the (token, head) entries: w = 2^(e - m), l = sum w;
//   pass 2: V rows (16-byte granules, RL lanes per row), up to UV row
//           passes in flight; acc += w V on the vector ALUs.
// Each pass holds only its own buffers, which keeps the register file small
// enough for several waves per SIMD.  The block then merges its four waves'
// (m, l, acc) by log-sum-exp and writes one partial per (head, block).
// ============================================================================
template <int D, int GT>
__global__ __launch_bounds__(256, GT <= 4 ? 4 : 2) void attend_mfma_kernel(const bf16_t* __restrict__ K_rot,
                                                          const bf16_t* __restrict__ V,
                                                          const uint16_t* __restrict__ qsplit,
                                                          const uint32_t* __restrict__ bitmap,
                                                          float* __restrict__ part, int Hq, int Hkv,
                                                          int S, int W, int NC, float scale_log2,
                                                          const int32_t* __restrict__ lens) {
  constexpr int NGRP = (GT + 3) / 4;
  constexpr int KS = D / 32;         // 32-dim k-steps of the exact dot
  constexpr int EPL = 8;             // bf16 per 16-byte granule
  constexpr int RL = D / 8;          // lanes per V row
  constexpr int RPW = 64 / RL;       // V rows per wave pass
  constexpr int KT = 16 / KS;        // K tiles in flight (16 loads per lane)
  constexpr int UV = 8;              // V row passes in flight
  constexpr int NT = kAttendMfmaTokens;
  constexpr int NSTEP = NT / 64;
  constexpr int NW = NT / 32;        // bitmap words per head
  static_assert(GT * NW <= 64, "one bitmap word per lane");
  __shared__ uint32_t s_bits[4][GT * NW];
  __shared__ int s_tok[4][NT];
  __shared__ uint16_t s_hm[4][NT];
  __shared__ __align__(16) float s_e[4][NT * GT];
  __shared__ float s_m[4][GT], s_l[4][GT];
  __shared__ float s_mx[4][GT];
  __shared__ __align__(16) float s_acc[4][GT][D];

  const int G = Hq / Hkv;
  const int bk = blockIdx.y, b = bk / Hkv, kv = bk % Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, q = lane >> 4;
  int span = NT, tend = S;
  if (lens) {
    const int L = seq_len(lens, b, S), nwv = 4 * NC;
    span = min(NT, max(32, ((L + nwv - 1) / nwv + 31) & ~31));
    tend = L;
  }
  const int t0 = (blockIdx.x * 4 + wave) * span;
  tend = min(tend, t0 + span);
  const size_t head0 = (size_t)b * Hq + (size_t)kv * G;
  int* tok = s_tok[wave];
  uint16_t* hmk = s_hm[wave];
  float* e = s_e[wave];
  uint32_t* bits = s_bits[wave];

  // A operands of pass 1 (the group's heads in rows), requested together
  // with the bitmap words so that one wait covers both
  bf16x8_t qa[NGRP][KS];
#pragma unroll
  for (int grp = 0; grp < NGRP; ++grp)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qa[grp][s] = q_rows(qsplit, head0 + 4 * grp, D, G - 4 * grp, D, m, 32 * s + 8 * q);

  // union list of the span; tok[0] starts as a valid row so that the clamped
  // V loads below stay in bounds when the list is empty
  if (lane == 0) tok[0] = min(t0, S - 1);
  if (lane < G * NW) {
    const int g = lane / NW, w = lane - g * NW;
    const int t = t0 + 32 * w;
    bits[lane] = (t < tend) ? bitmap[(head0 + g) * W + (t >> 5)] : 0u;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int n = 0;
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    const int t = t0 + 64 * st + lane;
    const int wi = 2 * st + (lane >> 5);
    int hm = 0;
#pragma unroll
    for (int g = 0; g < GT; ++g)
      if (g < G) hm |= (int)((bits[g * NW + wi] >> (t & 31)) & 1u) << g;
    const uint64_t mk = __ballot(hm != 0);
    if (hm) {
      const int pos = n + bits_below(mk);
      tok[pos] = t;
      hmk[pos] = (uint16_t)hm;
    }
    n += __popcll(mk);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const size_t cb = (size_t)bk * S * D;

  // pass 1: exact scores.  k-step s covers dims [32 s, 32 s + 32), lane
  // quarter q the 8 dims from 32 s + 8 q, so one load instruction reads 64
  // contiguous bytes of each of the tile's 16 rows (the B operand; rows past
  // the list repeat its last row and are dropped).  The heads sit in A rows:
  // lane l ends with the score of head 4 grp + l / 16 for row l % 16.
  float mloc[NGRP];
#pragma unroll
  for (int grp = 0; grp < NGRP; ++grp) mloc[grp] = -INFINITY;
  {
    for (int p0 = 0; p0 < n; p0 += 16 * KT) {
      uint4 ka[KT][KS];
#pragma unroll
      for (int tl = 0; tl < KT; ++tl) {
        const int p = min(p0 + 16 * tl + m, n - 1);
        const bf16_t* row = K_rot + cb + (size_t)tok[p] * D + 8 * q;
#pragma unroll
        for (int s = 0; s < KS; ++s) ka[tl][s] = ldg16(row + 32 * s);
      }
#pragma unroll
      for (int tl = 0; tl < KT; ++tl) {
        if (p0 + 16 * tl >= n) break;  // uniform across the wave
        const int p = p0 + 16 * tl + m;
#pragma unroll
        for (int grp = 0; grp < NGRP; ++grp) {
          floatx4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[grp][s], as_bf16x8(ka[tl][s]), sacc, 0, 0, 0);
          const float x = sum_split_rows(sacc);
          const int g = 4 * grp + q;
          if (g < GT && p < n) {
            const float sc = (g < G && ((hmk[p] >> g) & 1)) ? x * scale_log2 : -INFINITY;
            e[p * GT + g] = sc;
            mloc[grp] = fmaxf(mloc[grp], sc);
          }
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // the first batch of V rows is requested now (the K tiles' registers are
  // free), so that the weights pass below runs while the rows travel.  Rows
  // past the list repeat its last row (tok[0] if it is empty; weight 0), so
  // every load is unconditional and waits only where its data is used.
  const int lg = lane / RL, li = lane % RL;
  auto load_v = [&](int p0, uint4 (&vb)[UV]) {
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int p = max(min(p0 + RPW * u + lg, n - 1), 0);
      vb[u] = ldg16(V + cb + (size_t)tok[p] * D + li * EPL);
    }
  };
  uint4 vb[UV];
  __builtin_amdgcn_sched_barrier(0);
  load_v(0, vb);
  __builtin_amdgcn_sched_barrier(0);

  // per-head softmax statistics of the span: the max from the score lanes
  // (the 16 lanes 16 q .. 16 q + 15 hold head 4 grp + q), then one pass over
  // the (token, head) entries in which lane % GT is the head: weights in
  // place, sums
#pragma unroll
  for (int grp = 0; grp < NGRP; ++grp) {
    float v = mloc[grp];
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x041F)));  // lane ^ 1
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x081F)));  // lane ^ 2
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F)));  // lane ^ 4
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x201F)));  // lane ^ 8
    const int g = 4 * grp + q;
    if (m == 0 && g < GT) s_mx[wave][g] = v;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float mreg[GT], lreg[GT];
  {
    const int gl = lane % GT;
    const float mg = s_mx[wave][gl];
    float lp = 0.f;
    for (int i = lane; i < n * GT; i += 64) {
      const float v = e[i];
      const float w = (v == -INFINITY) ? 0.f : exp2f(v - mg);
      e[i] = w;
      lp += w;
    }
#pragma unroll
    for (int o = GT; o < 64; o <<= 1) lp += __shfl_xor(lp, o);
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      mreg[g] = s_mx[wave][g];
      lreg[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lp), g));
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // pass 2: weighted value sum
  float acc[GT][EPL];
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[g][i] = 0.f;
  for (int p0 = 0; p0 < n; p0 += RPW * UV) {
    if (p0 > 0) load_v(p0, vb);
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      if (p0 + RPW * u >= n) break;  // uniform across the wave
      const int p = p0 + RPW * u + lg;
      float x[EPL];
      Gran<bf16_t>::unpack(vb[u], x);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float w = (p < n && g < G) ? e[p * GT + g] : 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[g][i] = fmaf(w, x[i], acc[g][i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      float v = acc[g][i];
      // lane ^ 8 and lane ^ 16 by ds_swizzle (bit-mask mode, no address), lane ^ 32 by bpermute
      if constexpr (RL <= 8) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x201F));
      v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
      v += __shfl_xor(v, 32);
      acc[g][i] = v;
    }

  // merge the four waves' spans by log-sum-exp; one partial per (head, block)
  if (lg == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int i = 0; i < EPL; ++i) s_acc[wave][g][li * EPL + i] = acc[g][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) { s_m[wave][g] = mreg[g]; s_l[wave][g] = lreg[g]; }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < G * D; o += 256) {
    const int g = o / D, c = o - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][g]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (s_m[w][g] == -INFINITY) ? 0.f : exp2f(s_m[w][g] - M);
      L = fmaf(s_l[w][g], f, L);
      A = fmaf(s_acc[w][g][c], f, A);
    }
    float* pr = part + ((head0 + g) * NC + blockIdx.x) * (size_t)(D + 2);
    pr[2 + c] = A;
    if (c == 0) { pr[0] = M; pr[1] = L; }
  }

}

// ============================================================================
// host side
// ============================================================================
template <int GT, bool KEYS>
static hipError_t score_mfma_g(const DecodePlan& p, const void* src, int ld, const uint16_t* qsplit,
                               void* out, int out_stride, uint2* mm, hipStream_t st) {
  const dim3 grid(p.NSC, p.B * p.Hkv), block(256);
  const bf16_t* s = static_cast<const bf16_t*>(src);
  const int ks = (p.r + 31) / 32;
#define LOKI_SM(K)                                                                                 \
  case K:                                                                                          \
    hipLaunchKernelGGL((score_mfma_kernel<GT, K, KEYS>), grid, block, 0, st, s, qsplit, out,       \
                       out_stride, mm, p.Hq, p.Hkv, p.S, p.d, ld, p.r, p.SC, p.lens);              \
    break;
  switch (ks) {
    LOKI_SM(1)
    LOKI_SM(2)
    LOKI_SM(3)
    LOKI_SM(4)
    default: return hipErrorInvalidValue;
  }
#undef LOKI_SM
  return hipGetLastError();
}

hipError_t launch_scores_mfma(const DecodePlan& p, const void* src, int ld, const uint16_t* qsplit,
                              void* out, bool as_keys, int out_stride, uint2* mm, hipStream_t st) {
  if (p.dt != 1 || p.SC % 16 != 0) return hipErrorInvalidValue;
  auto go = [&](auto gt) {
    constexpr int GT = decltype(gt)::value;
    return as_keys ? score_mfma_g<GT, true>(p, src, ld, qsplit, out, out_stride, mm, st)
                   : score_mfma_g<GT, false>(p, src, ld, qsplit, out, out_stride, mm, st);
  };
  if (p.G <= 1) return go(std::integral_constant<int, 1>{});
  if (p.G <= 2) return go(std::integral_constant<int, 2>{});
  if (p.G <= 4) return go(std::integral_constant<int, 4>{});
  if (p.G <= 8) return go(std::integral_constant<int, 8>{});
  return go(std::integral_constant<int, 16>{});
}

size_t score_select_lds_bytes(int Sp) {
  return (size_t)Sp * sizeof(uint32_t);
}

hipError_t launch_score_select(const DecodePlan& p, const void* src, int ld, const uint16_t* qsplit,
                               int32_t* idx, uint32_t* bitmap, hipStream_t st) {
  if (p.dt != 1) return hipErrorInvalidValue;
  const size_t lds = score_select_lds_bytes(p.Sp);
  const int ngroups = p.B * p.Hkv;
  const dim3 grid((unsigned)((ngroups + 7) / 8 * 8 * p.G)), block(kFusedThreads);
  const bf16_t* s = static_cast<const bf16_t*>(src);
  const int ks = (p.r + 31) / 32;
  hipError_t e = hipSuccess;
#define LOKI_SS(K)                                                                                     \
  case K:                                                                                              \
    e = ensure_dynamic_lds(reinterpret_cast<const void*>(&score_select_kernel<K>), (int)lds);        \
    if (e != hipSuccess) return e;                                                                     \
    hipLaunchKernelGGL((score_select_kernel<K>), grid, block, lds, st, s, ld, qsplit, p.B, p.Hq, p.Hkv, \
                       p.S, p.Sp, p.d, p.r, p.k, p.W, idx, bitmap, p.lens);                            \
    break;
  switch (ks) {
    LOKI_SS(1)
    LOKI_SS(2)
    LOKI_SS(3)
    LOKI_SS(4)
    default: return hipErrorInvalidValue;
  }
#undef LOKI_SS
  return hipGetLastError();
}

bool score_select_chunk_fits(const DecodePlan& p) {
  return p.dt == 1 && p.r <= 128 && p.d % 8 == 0;
}

hipError_t launch_score_select_chunk(const DecodePlan& p, const void* src, int ld, const uint16_t* qsplit,
                                     int32_t* cidx, uint32_t* ckey, int ldc, hipStream_t st) {
  if (!score_select_chunk_fits(p)) return hipErrorInvalidValue;
  const int C = (p.S + kSelChunk - 1) / kSelChunk;
  const long long units = (long long)p.B * p.Hkv * C;
  const long long nblk = (units + 7) / 8 * 8 * p.G;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  const size_t lds = (size_t)kSelChunk * sizeof(uint32_t);
  const dim3 grid((unsigned)nblk), block(kChunkThreads);
  const bf16_t* s = static_cast<const bf16_t*>(src);
  const int ks = (p.r + 31) / 32;
  hipError_t e = hipSuccess;
#define LOKI_SC(K)                                                                                       \
  case K:                                                                                                \
    e = ensure_dynamic_lds(reinterpret_cast<const void*>(&score_select_chunk_kernel<K>), (int)lds);    \
    if (e != hipSuccess) return e;                                                                       \
    hipLaunchKernelGGL((score_select_chunk_kernel<K>), grid, block, lds, st, s, ld, qsplit, p.B, p.Hq,   \
                       p.Hkv, p.S, C, p.d, p.r, p.k, ldc, cidx, ckey, p.lens);                           \
    break;
  switch (ks) {
    LOKI_SC(1)
    LOKI_SC(2)
    LOKI_SC(3)
    LOKI_SC(4)
    default: return hipErrorInvalidValue;
  }
#undef LOKI_SC
  return hipGetLastError();
}

hipError_t launch_attend_mfma(const DecodePlan& p, const void* K_rot, const void* V,
                              const uint16_t* qsplit, const uint32_t* bitmap, float* part,
                              hipStream_t st) {
  if (p.dt != 1 || p.G > 8 || p.AC != 4 * kAttendMfmaTokens) return hipErrorInvalidValue;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.d));
  const dim3 grid(p.NAC, p.B * p.Hkv), block(256);
  const bf16_t* k = static_cast<const bf16_t*>(K_rot);
  const bf16_t* v = static_cast<const bf16_t*>(V);
  auto go = [&](auto dd, auto gt) {
    constexpr int D = decltype(dd)::value, GT = decltype(gt)::value;
    hipLaunchKernelGGL((attend_mfma_kernel<D, GT>), grid, block, 0, st, k, v, qsplit, bitmap, part,
                       p.Hq, p.Hkv, p.S, p.W, p.NAC, scale_log2, p.lens);
    return hipGetLastError();
  };
  auto by_g = [&](auto dd) {
    if (p.G <= 1) return go(dd, std::integral_constant<int, 1>{});
    if (p.G <= 2) return go(dd, std::integral_constant<int, 2>{});
    if (p.G <= 4) return go(dd, std::integral_constant<int, 4>{});
    return go(dd, std::integral_constant<int, 8>{});
  };
  return p.d == 64 ? by_g(std::integral_constant<int, 64>{}) : by_g(std::integral_constant<int, 128>{});
}

}  // namespace loki
