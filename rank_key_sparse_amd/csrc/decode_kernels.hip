// gfx950 kernels of one low-rank-key sparse decode step.
//
// Stages (Loki page, abstract; AQUA page, related work on LoKi attention and
// preliminaries eqs. 3-5):
//   qrot     q_rot = q P[kv] in fp32                         (one block per (b, kv))
//   scores   s_j = q_rot[:r] . K_rot[j, :r] for all tokens   (HBM stream of the r-dim prefix)
//   select   per query head, the k largest s_j -> idx, bitmap (radix/bucket select)
//   attend   exact scores, softmax and V-sum over the union of the group's kept
//            tokens, split over token chunks -> (max, sum, acc) partials
//   combine  log-sum-exp merge of the chunk partials -> out
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "select_core.h"

namespace loki {


// ============================================================================
// q rotation: q_rot[b, kv*G+g, c] = sum_j q[b, kv*G+g, j] * P[kv, j, c]
// One block of 8 d threads per (b, kv): P[kv] and the G queries are staged
// in LDS with 16-byte loads; thread (c, js) sums the js-th of 8 contiguous
// slices of j for every head, and the slices are added in slice order.  The
// block also writes the three-way bf16 split of q_rot used as MFMA operands.
// ============================================================================
constexpr int kQrotSlices = 8;

template <typename T, int GT>
__global__ __launch_bounds__(256) void qrot_kernel(const T* __restrict__ q, const T* __restrict__ P,
                                                   float* __restrict__ qrot,
                                                   bf16_t* __restrict__ qsplit, int Hq, int Hkv,
                                                   int d, uint32_t* __restrict__ zero, int nzero) {
  for (int i = (blockIdx.y * gridDim.x + blockIdx.x) * 256 + threadIdx.x; i < nzero; i += gridDim.x * gridDim.y * 256)
    zero[i] = 0u;
  // Block = (b, kv) group x 32 columns of P, staged in LDS with 16-byte
  // loads; thread = (column, j-slice).  Each column is kQrotSlices FMA chains
  // over consecutive j-ranges, added in range order.
  constexpr int CB = 32;
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = CB / EPC;             // chunks per staged row
  __shared__ __align__(16) T sP[128 * CB];
  __shared__ float qs[GT * 128];
  __shared__ float red[kQrotSlices][GT][CB];
  const int G = Hq / Hkv;
  const int bk = blockIdx.x, b = bk / Hkv, kv = bk % Hkv;
  const int c0 = blockIdx.y * CB;
  const size_t qbase = ((size_t)b * Hq + (size_t)kv * G) * d;
  const int tid = threadIdx.x;
  const T* Pk = P + (size_t)kv * d * d + c0;
  for (int i = tid; i < d * CPR; i += 256) {
    const int j = i / CPR, c8 = i - j * CPR;
    *reinterpret_cast<uint4*>(sP + j * CB + c8 * EPC) = ldg16(Pk + (size_t)j * d + c8 * EPC);
  }
  for (int i = tid; i < GT * d; i += 256) qs[i] = (i < G * d) ? to_f32(q[qbase + i]) : 0.f;
  __syncthreads();
  const int cc = tid % CB, js = tid / CB;
  const int J = d / kQrotSlices;
  float acc[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g) acc[g] = 0.f;
  for (int jj = 0; jj < J; ++jj) {
    const int j = js * J + jj;
    const float pj = to_f32(sP[j * CB + cc]);
#pragma unroll
    for (int g = 0; g < GT; ++g) acc[g] = fmaf(qs[g * d + j], pj, acc[g]);
  }
#pragma unroll
  for (int g = 0; g < GT; ++g) red[js][g][cc] = acc[g];
  __syncthreads();
  for (int o = tid; o < GT * CB; o += 256) {
    const int g = o / CB, cl = o - g * CB;
    if (g >= G) continue;
    float v = red[0][g][cl];
    for (int t = 1; t < kQrotSlices; ++t) v += red[t][g][cl];
    const int col = c0 + cl;
    qrot[qbase + (size_t)g * d + col] = v;
    if (qsplit) {
      // three-way bf16 split v = h + m + l (each residual exact in fp32),
      // plus a zero row, as MFMA operands: qsplit[row][part][c]
      bf16_t* o4 = qsplit + (qbase + (size_t)g * d) * 4 + col;
      const bf16_t h = f32_to_bf16(v);
      const float r1 = v - to_f32(h);
      const bf16_t mid = f32_to_bf16(r1);
      const bf16_t lo = f32_to_bf16(r1 - to_f32(mid));
      o4[0] = h;
      o4[d] = mid;
      o4[2 * d] = lo;
      o4[3 * d] = 0;
    }
  }
}

// ============================================================================
// The query itself in the layouts the attention stage reads (fp32 and the
// three-way bf16 split), for an exact stage over keys that are not rotated
// (the asymmetric scoring index keeps the keys as they are).
// ============================================================================
template <typename T>
__global__ __launch_bounds__(256) void qplain_kernel(const T* __restrict__ q, float* __restrict__ qf,
                                                     bf16_t* __restrict__ qsplit, int n, int d) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int row = i / d, c = i - row * d;
  const float v = to_f32(q[i]);
  qf[i] = v;
  bf16_t* o4 = qsplit + (size_t)row * d * 4 + c;
  const bf16_t h = f32_to_bf16(v);
  const float r1 = v - to_f32(h);
  const bf16_t mid = f32_to_bf16(r1);
  o4[0] = h;
  o4[d] = mid;
  o4[2 * d] = f32_to_bf16(r1 - to_f32(mid));
  o4[3 * d] = 0;
}

hipError_t launch_qplain(const DecodePlan& p, const void* q, float* qf, uint16_t* qsplit, hipStream_t st) {
  const int n = p.B * p.Hq * p.d;
  bf16_t* qs = reinterpret_cast<bf16_t*>(qsplit);
  if (p.dt == 1)
    hipLaunchKernelGGL(qplain_kernel<bf16_t>, dim3((n + 255) / 256), dim3(256), 0, st, static_cast<const bf16_t*>(q),
                       qf, qs, n, p.d);
  else
    hipLaunchKernelGGL(qplain_kernel<float>, dim3((n + 255) / 256), dim3(256), 0, st, static_cast<const float*>(q),
                       qf, qs, n, p.d);
  return hipGetLastError();
}

// ============================================================================
// Query-magnitude dimensions (AQUA page, online phase): for each query head,
// the r dims of q_rot with the largest magnitude, ties to the lower index.
// One wave per head (d / 64 elements per lane).  The r-th largest magnitude
// thr is found bit by bit on the magnitudes' bit patterns (non-negative
// floats order as their bits): the largest thr with at least r magnitudes
// >= thr.  The kept dims are those above thr and, of those equal to it, the
// lowest-index ones up to r.
// Writes the masked q_rot (zero outside the chosen dims) and its three-way
// bf16 split for the score stage (a full-width dot product with the masked
// query adds exact zeros for the other dims), and optionally the chosen dims
// in ascending order and the information retention loss
// | ||q|| - ||q_rot[I]|| | / ||q|| (AQUA page, information-retention paragraph).
// ============================================================================
template <typename T, int EPL>
__global__ __launch_bounds__(256) void qdims_kernel(const T* __restrict__ q, const float* __restrict__ qrot,
                                                    float* __restrict__ qrot_m, bf16_t* __restrict__ qsplit_m,
                                                    int32_t* __restrict__ dims, float* __restrict__ info,
                                                    int rows, int r) {
  constexpr int D = 64 * EPL;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;  // the whole wave
  float v[EPL];
  uint32_t a[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    v[e] = qrot[(size_t)row * D + lane + 64 * e];
    a[e] = __float_as_uint(v[e]) & 0x7fffffffu;
  }
  uint32_t thr = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) cnt += __popcll(__ballot(a[e] >= cand));
    if (cnt >= r) thr = cand;
  }
  int above = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) above += __popcll(__ballot(a[e] > thr));
  const int need = r - above;  // dims equal to thr still to take, lowest index first
  const uint64_t lt = (1ull << lane) - 1ull;
  float kept = 0.f, tot = 0.f;
  int before = 0;  // chosen dims below this wave's current 64-block
  int eq_before = 0;  // dims equal to thr below it
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int c = lane + 64 * e;
    const uint64_t eqm = __ballot(a[e] == thr);
    const bool sel = a[e] > thr || (a[e] == thr && eq_before + __popcll(eqm & lt) < need);
    eq_before += __popcll(eqm);
    const float m = sel ? v[e] : 0.f;
    qrot_m[(size_t)row * D + c] = m;
    bf16_t* o4 = qsplit_m + (size_t)row * D * 4 + c;
    const bf16_t h = f32_to_bf16(m);
    const float r1 = m - to_f32(h);
    const bf16_t mid = f32_to_bf16(r1);
    const bf16_t lo = f32_to_bf16(r1 - to_f32(mid));
    o4[0] = h;
    o4[D] = mid;
    o4[2 * D] = lo;
    o4[3 * D] = 0;
    const uint64_t mask = __ballot(sel);
    if (dims && sel) dims[(size_t)row * r + before + __popcll(mask & lt)] = c;
    before += __popcll(mask);
    kept = fmaf(m, m, kept);
    const float x = to_f32(q[(size_t)row * D + c]);
    tot = fmaf(x, x, tot);
  }
  if (info) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      kept += __shfl_xor(kept, o);
      tot += __shfl_xor(tot, o);
    }
    if (lane == 0) {
      const float n = sqrtf(tot);
      info[row] = n > 0.f ? fabsf(n - sqrtf(kept)) / n : 0.f;
    }
  }
}

hipError_t launch_qdims(const DecodePlan& p, const void* q, const float* qrot, float* qrot_m, uint16_t* qsplit_m,
                        int32_t* dims, float* info, int r, hipStream_t st) {
  const int rows = p.B * p.Hq;
  const dim3 grid((rows + 3) / 4), block(256);
  bf16_t* qs = reinterpret_cast<bf16_t*>(qsplit_m);
  auto go = [&](auto ee) {
    constexpr int E = decltype(ee)::value;
    if (p.dt == 1)
      hipLaunchKernelGGL((qdims_kernel<bf16_t, E>), grid, block, 0, st, static_cast<const bf16_t*>(q), qrot, qrot_m,
                         qs, dims, info, rows, r);
    else
      hipLaunchKernelGGL((qdims_kernel<float, E>), grid, block, 0, st, static_cast<const float*>(q), qrot, qrot_m,
                         qs, dims, info, rows, r);
    return hipGetLastError();
  };
  return p.d == 128 ? go(std::integral_constant<int, 2>{}) : go(std::integral_constant<int, 1>{});
}

// ============================================================================
// Approximate scores over the leading r rotated dimensions.
// The source is either K_rot itself (row stride d) or a lead-dims copy
// K_lead holding only the leading R >= r rotated dims of each token (row
// stride R), which turns the strided prefix reads into a dense stream.
// A token's r-dim prefix is LPT 16-byte granules, read by LPT adjacent lanes;
// each lane holds its granule's slice of q_rot for all G heads of the group,
// so the prefix is streamed from HBM once per (b, kv) group.  q_rot entries at
// c >= r are zero, so a partially used granule adds exact zeros.
// Output: order-preserving keys (decode) or the fp32 scores themselves.
// ============================================================================
template <typename T, int LPT, int GT>
__global__ __launch_bounds__(256) void score_kernel(const T* __restrict__ src,
                                                    const float* __restrict__ qrot,
                                                    void* __restrict__ out, int as_keys,
                                                    int out_stride, uint2* __restrict__ mm,
                                                    int Hq, int Hkv, int S, int d, int ld, int r,
                                                    int SC, const int32_t* __restrict__ lens) {
  constexpr int EPL = Gran<T>::N;
  constexpr int TPI = 256 / LPT;  // tokens per block pass
  constexpr int U = 8;            // passes whose loads are in flight together
  const int G = Hq / Hkv;
  const int bk = blockIdx.y, b = bk / Hkv, kv = bk % Hkv;
  const int t0 = blockIdx.x * SC, t1 = min(seq_len(lens, b, S), t0 + SC);  // tokens past the sequence: none
  const int gran = threadIdx.x % LPT, tsub = threadIdx.x / LPT;

  float qv[GT][EPL];
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int c = gran * EPL + i;
      qv[g][i] = (g < G && c < r) ? qrot[((size_t)b * Hq + (size_t)kv * G + g) * d + c] : 0.f;
    }

  const T* base = src + (size_t)bk * S * ld + gran * EPL;
  const size_t orow0 = ((size_t)b * Hq + (size_t)kv * G) * out_stride;
  __shared__ uint32_t smn[GT], smx[GT];
  if (threadIdx.x < GT) { smn[threadIdx.x] = 0xffffffffu; smx[threadIdx.x] = 0u; }
  uint32_t mn[GT], mx[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g) { mn[g] = 0xffffffffu; mx[g] = 0u; }
  for (int tb = t0; tb < t1; tb += TPI * U) {
    uint4 buf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + u * TPI + tsub;
      buf[u] = (t < t1) ? ldg16(base + (size_t)t * ld) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + u * TPI + tsub;
      float x[EPL];
      Gran<T>::unpack(buf[u], x);
      float s[GT];
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) a = fmaf(qv[g][i], x[i], a);
        s[g] = group_sum<LPT>(a);
      }
      if (t < t1) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          if (g % LPT == gran && g < G) {
            const size_t o = orow0 + (size_t)g * out_stride + t;
            if (as_keys) {
              const uint32_t key = score_key(s[g]);
              static_cast<uint32_t*>(out)[o] = key;
              mn[g] = min(mn[g], key);
              mx[g] = max(mx[g], key);
            } else {
              static_cast<float*>(out)[o] = s[g];
            }
          }
        }
      }
    }
  }
  if (as_keys && mm) {  // uniform: the chunk's min / max key per head
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GT; ++g)
      if (g % LPT == gran && g < G && mn[g] <= mx[g]) { atomicMin(&smn[g], mn[g]); atomicMax(&smx[g], mx[g]); }
    __syncthreads();
    if (threadIdx.x < G)
      mm[((size_t)b * Hq + (size_t)kv * G + threadIdx.x) * gridDim.x + blockIdx.x] =
          make_uint2(smn[threadIdx.x], smx[threadIdx.x]);
  }
}

// fp32 scores -> keys, for the stand-alone selection entry point.
__global__ __launch_bounds__(256) void scores_to_keys_kernel(const float* __restrict__ s,
                                                             uint32_t* __restrict__ keys,
                                                             uint2* __restrict__ mm, int S,
                                                             int Sp) {
  __shared__ uint32_t red[2][4];
  const int row = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int j = blockIdx.x * 256 + threadIdx.x; j < S; j += gridDim.x * 256) {
    const uint32_t key = score_key(s[(size_t)row * S + j]);
    keys[(size_t)row * Sp + j] = key;
    mn = min(mn, key);
    mx = max(mx, key);
  }
  mn = wave_min_u(mn);
  mx = wave_max_u(mx);
  if (lane == 0) { red[0][wave] = mn; red[1][wave] = mx; }
  __syncthreads();
  if (threadIdx.x == 0)
    mm[(size_t)row * gridDim.x + blockIdx.x] =
        make_uint2(min(min(red[0][0], red[0][1]), min(red[0][2], red[0][3])),
                   max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3])));
}

// ============================================================================
// Top-k selection from workspace keys, one block of 1024 threads per query
// head (see select_core.h).  Heads of up to 1024 T tokens load their keys
// once into registers (coalesced dword loads, lane l of wave w reading tokens
// w*64T + 64i + l); longer heads stream their keys from global memory with
// min / max from the per-chunk extremes mm and step masks in gmasks.
// ============================================================================
constexpr int kSelThreads = 1024;

// T = 16 is held to 64 VGPRs so that two blocks share a CU.
template <int T>
__global__ __launch_bounds__(kSelThreads, T <= 16 ? 8 : 4) void select_regs_kernel(const uint32_t* __restrict__ keys,
                                                                  int Scap, int Sp, int k, int W,
                                                                  int32_t* __restrict__ idx,
                                                                  uint32_t* __restrict__ bitmap,
                                                                  const int32_t* __restrict__ lens, int Hq) {
  __shared__ uint32_t lds[kNB];
  __shared__ uint32_t take[kSelThreads * T / 32];
  __shared__ SelScratch<kSelThreads> sh;
  const int row = blockIdx.x;
  const int S = seq_len(lens, row / Hq, Scap);  // this head's tokens
  const uint32_t* rk = keys + (size_t)row * Sp;
  int32_t* orow = idx + (size_t)row * k;
  uint32_t* brow = bitmap + (size_t)row * W;
  if (k >= S) {
    keep_all<kSelThreads>(S, k, W, orow, brow);
    return;
  }
  uint32_t key[T];
  load_regs<T>(rk, S, key);
  select_regs<kSelThreads, T>(key, lds, take, S, k, W, orow, brow, sh);
}

// Long heads, two stages (exact: every token of the head's top-k is in the
// top-k of its own chunk).  Stage 1: one block per (chunk of kSelChunk
// tokens, head) keeps the chunk's top-k; its positions (made absolute) and
// keys go to the candidate lists, chunk c at offset c k, ascending.  Stage 2:
// one block per head selects the top-k of its candidate list (position order
// is token order, so ties still go to the lower token), maps positions back
// to tokens and sets the kept tokens' bits in the head's bitmap row (cleared
// while the selection runs).
__global__ __launch_bounds__(kSelThreads) void select_chunk_kernel(const uint32_t* __restrict__ keys, int Scap,
                                                                   int Sp, int k, int ldc,
                                                                   int32_t* __restrict__ cidx,
                                                                   uint32_t* __restrict__ ckey,
                                                                   const int32_t* __restrict__ lens, int Hq) {
  constexpr int T = kSelChunk / kSelThreads;
  __shared__ uint32_t lds[kNB];
  __shared__ uint32_t take[kSelChunk / 32];
  __shared__ SelScratch<kSelThreads> sh;
  const int row = blockIdx.y, c = blockIdx.x, base = c * kSelChunk;
  const int S = seq_len(lens, row / Hq, Scap);  // this head's tokens
  const int L = min(kSelChunk, S - base);        // may be <= 0 past the head's end
  const uint32_t* rk = keys + (size_t)row * Sp + base;
  int32_t* oi = cidx + (size_t)row * ldc + (size_t)c * k;
  uint32_t* ok = ckey + (size_t)row * ldc + (size_t)c * k;
  if (L <= k) {  // the whole chunk is a candidate; free slots get key 0, below every score's key
    for (int j = threadIdx.x; j < k; j += kSelThreads) {
      oi[j] = j < L ? base + j : -1;
      ok[j] = j < L ? rk[j] : 0u;
    }
    return;
  }
  uint32_t key[T];
  load_regs<T>(rk, L, key);
  // the winners' keys are read back from the chunk's row while they are listed
  select_regs<kSelThreads, T>(key, lds, take, L, k, 2 * ((L + 63) / 64), oi, nullptr, sh, nullptr, ok, base, nullptr,
                              rk);
}

template <int T>
__global__ __launch_bounds__(kSelThreads) void select_merge_kernel(const uint32_t* __restrict__ ckey,
                                                                   const int32_t* __restrict__ cidx,
                                                                   int S2, int ldc, int k, int W,
                                                                   int32_t* __restrict__ idx,
                                                                   uint32_t* __restrict__ bitmap,
                                                                   const int32_t* __restrict__ lens, int Hq,
                                                                   int Scap) {
  __shared__ uint32_t lds[kNB];
  __shared__ uint32_t take[kSelThreads * T / 32];
  __shared__ SelScratch<kSelThreads> sh;
  const int row = blockIdx.x;
  const int S = seq_len(lens, row / Hq, Scap);
  int32_t* orow = idx + (size_t)row * k;
  uint32_t* brow = bitmap + (size_t)row * W;
  if (k >= S) {  // a short head keeps all its tokens
    keep_all<kSelThreads>(S, k, W, orow, brow);
    return;
  }
  for (int w = threadIdx.x; w < W; w += kSelThreads) brow[w] = 0u;  // ordered before the bits by the barriers below
  // every chunk filled its k slots (free ones with key 0, below every score's
  // key), and the head has more than k real candidates: none is chosen.  The
  // value bins span the real candidates' keys only (key 0 decodes to NaN and
  // would make the range degenerate); free slots fall into bin 0.
  __shared__ uint32_t smm[2];
  uint32_t key[T];
  load_regs<T>(ckey + (size_t)row * ldc, S2, key);
  {
    const int nv = regs_valid<T>(S2);
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int i = 0; i < T; ++i)
      if (i < nv && key[i] != 0u) { mn = min(mn, key[i]); mx = max(mx, key[i]); }
    uint32_t kmin, kmax;
    block_minmax<kSelThreads>(mn, mx, sh, kmin, kmax);
    if (threadIdx.x == 0) { smm[0] = kmin; smm[1] = kmax; }
    __syncthreads();  // sh.red is read by every thread before select_regs reuses sh
  }
  select_regs<kSelThreads, T>(key, lds, take, S2, k, 2 * ((S2 + 63) / 64), orow, nullptr, sh,
                              cidx + (size_t)row * ldc, nullptr, 0, smm);
  __syncthreads();  // every thread's idx entries written
  for (int i = threadIdx.x; i < k; i += kSelThreads) {
    const int j = orow[i];
    if (j >= 0 && j < S) atomicOr(&brow[j >> 5], 1u << (j & 31));
  }
}

__global__ __launch_bounds__(kSelThreads) void select_global_kernel(const uint32_t* __restrict__ keys,
                                                                    const uint2* __restrict__ mm,
                                                                    int nmm, uint32_t* __restrict__ gmasks,
                                                                    int Scap, int Sp, int k, int W,
                                                                    int32_t* __restrict__ idx,
                                                                    uint32_t* __restrict__ bitmap,
                                                                    const int32_t* __restrict__ lens, int Hq) {
  __shared__ uint32_t hist[kNB];
  __shared__ SelScratch<kSelThreads> sh;
  const int row = blockIdx.x;
  const int S = seq_len(lens, row / Hq, Scap);  // this head's tokens
  int32_t* orow = idx + (size_t)row * k;
  uint32_t* brow = bitmap + (size_t)row * W;
  if (k >= S) {
    keep_all<kSelThreads>(S, k, W, orow, brow);
    return;
  }
  for (int i = threadIdx.x; i < kNB; i += kSelThreads) hist[i] = 0u;
  select_head<kSelThreads>(keys + (size_t)row * Sp, mm + (size_t)row * nmm, nmm, hist,
                           gmasks + (size_t)row * (Sp / 16), S, Sp, k, orow, brow, sh);
  // bitmap words past the head's last 64-token step (a shorter sequence)
  for (int w = 2 * ((S + 63) >> 6) + threadIdx.x; w < W; w += kSelThreads) brow[w] = 0u;
}

// Caller-given kept sets -> bitmap (stand-alone attention entry point).
// One block per query head clears its row, then sets the bits of in-range
// entries (duplicates merge).
__global__ __launch_bounds__(256) void idx_to_bitmap_kernel(const int32_t* __restrict__ idx,
                                                            uint32_t* __restrict__ bitmap, int S,
                                                            int k, int W) {
  const int row = blockIdx.x;
  uint32_t* brow = bitmap + (size_t)row * W;
  for (int w = threadIdx.x; w < W; w += 256) brow[w] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += 256) {
    const int j = idx[(size_t)row * k + i];
    if (j >= 0 && j < S) atomicOr(&brow[j >> 5], 1u << (j & 31));
  }
}

// ============================================================================
// Exact attention over the kept tokens.
// Each wavefront independently owns NT consecutive tokens of one (b, kv)
// group; the four waves of a block own four consecutive spans.  A wave reads
// the G heads' bitmap words for its span, builds the union list (token, head
// mask) in LDS, and reads every listed K_rot row and V row ONCE for all G
// heads (RL lanes per row, 16 bytes each, U row-passes in flight):
//   pass 1: e = q_rot . K_rot[j] * log2(e)/sqrt(d)  (-inf for heads that did
//           not keep j) into LDS;
//   per head: m = max e, w = 2^(e - m), l = sum w;
//   pass 2: acc = sum w V[j].
// No block barrier is needed until the end, where the four waves' (m, l,
// acc) are merged by log-sum-exp and one partial per (head, block) is
// written.  NT shrinks as G grows so the per-wave score buffer stays 4 KB.
// ============================================================================
template <int GT> struct AttendTokens { static constexpr int value = GT <= 4 ? 256 : 1024 / GT; };

template <typename T, int D, int GT>
__global__ __launch_bounds__(256) void attend_kernel(const T* __restrict__ K_rot,
                                                     const T* __restrict__ V,
                                                     const float* __restrict__ qrot,
                                                     const uint32_t* __restrict__ bitmap,
                                                     float* __restrict__ part, int Hq, int Hkv,
                                                     int S, int W, int NC, float scale_log2) {
  constexpr int EPL = Gran<T>::N;
  constexpr int RL = D * (int)sizeof(T) / 16;  // lanes per row
  constexpr int RPW = 64 / RL;                 // rows per wave pass
  constexpr int U = 8;                         // row passes in flight
  constexpr int NT = AttendTokens<GT>::value;  // tokens per wave
  constexpr int NSTEP = NT / 64;
  __shared__ int s_tok[4][NT];
  __shared__ uint16_t s_hm[4][NT];
  __shared__ __align__(16) float s_e[4][NT * GT];
  __shared__ float s_m[4][GT], s_l[4][GT];
  __shared__ __align__(16) float s_acc[4][GT][D];

  const int G = Hq / Hkv;
  const int bk = blockIdx.y, b = bk / Hkv, kv = bk % Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = (blockIdx.x * 4 + wave) * NT;
  const size_t head0 = (size_t)b * Hq + (size_t)kv * G;
  int* tok = s_tok[wave];
  uint16_t* hmk = s_hm[wave];
  float* e = s_e[wave];

  // bitmap words for every step and head, all loads in flight together
  uint32_t words[NSTEP][GT];
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    const int t = t0 + 64 * st + lane;
#pragma unroll
    for (int g = 0; g < GT; ++g)
      words[st][g] = (g < G && t < S) ? bitmap[(head0 + g) * W + (t >> 5)] : 0u;
  }
  int n = 0;
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    const int t = t0 + 64 * st + lane;
    int hm = 0;
#pragma unroll
    for (int g = 0; g < GT; ++g) hm |= (int)((words[st][g] >> (t & 31)) & 1u) << g;
    const uint64_t m = __ballot(hm != 0);
    if (hm) {
      const int pos = n + bits_below(m);
      tok[pos] = t;
      hmk[pos] = (uint16_t)hm;
    }
    n += __popcll(m);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int lg = lane / RL, li = lane % RL;
  float qv[GT][EPL];
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int i = 0; i < EPL; ++i) qv[g][i] = (g < G) ? qrot[(head0 + g) * D + li * EPL + i] : 0.f;
  const size_t cbase = (size_t)bk * S * D + li * EPL;

  // pass 1: exact scores
  for (int p0 = 0; p0 < n; p0 += RPW * U) {
    uint4 buf[U];
    int hms[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * RPW + lg;
      if (p < n) {
        hms[u] = hmk[p];
        buf[u] = ldg16(K_rot + cbase + (size_t)tok[p] * D);
      } else {
        hms[u] = 0;
        buf[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * RPW + lg;
      float x[EPL];
      Gran<T>::unpack(buf[u], x);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) a = fmaf(qv[g][i], x[i], a);
        a = group_sum<RL>(a);
        if (p < n && g % RL == li) e[p * GT + g] = ((hms[u] >> g) & 1) ? a * scale_log2 : -INFINITY;
      }
      __builtin_amdgcn_sched_barrier(0);  // one row's temporaries live at a time
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // per-head softmax statistics of this wave's span
  float mreg[GT], lreg[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    float mx = -INFINITY, sum = 0.f;
    if (g < G) {
      for (int p = lane; p < n; p += 64) mx = fmaxf(mx, e[p * GT + g]);
      mx = wave_max(mx);
      for (int p = lane; p < n; p += 64) {
        const float v = e[p * GT + g];
        const float w = (v == -INFINITY) ? 0.f : exp2f(v - mx);
        e[p * GT + g] = w;
        sum += w;
      }
      sum = wave_sum(sum);
    }
    mreg[g] = mx;
    lreg[g] = sum;
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
  for (int p0 = 0; p0 < n; p0 += RPW * U) {
    uint4 buf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * RPW + lg;
      buf[u] = (p < n) ? ldg16(V + cbase + (size_t)tok[p] * D) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * RPW + lg;
      float x[EPL];
      Gran<T>::unpack(buf[u], x);
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
      for (int o = RL; o < 64; o <<= 1) v += __shfl_xor(v, o);
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

// Log-sum-exp merge of the chunk partials: one block of d threads per head.
// The global max over chunks is reduced first; then chunk scale factors and
// sums are brought into LDS a tile at a time (all loads of a tile in flight)
// and every thread accumulates its output dimension in chunk order.
template <typename T>
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ part,
                                                      T* __restrict__ out, int NC, int d) {
  constexpr int TILE = 1024;
  __shared__ float s_f[TILE];
  __shared__ float s_l[TILE];
  __shared__ float s_red[2];
  const int row = blockIdx.x, c = threadIdx.x;
  const int lane = c & 63, wave = c >> 6;
  const size_t st = (size_t)d + 2;
  const float* pr = part + (size_t)row * NC * st;
  float M = -INFINITY;
  for (int ch = c; ch < NC; ch += blockDim.x) M = fmaxf(M, pr[(size_t)ch * st]);
  M = wave_max(M);
  if (lane == 0) s_red[wave] = M;
  __syncthreads();
  M = s_red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) M = fmaxf(M, s_red[w]);
  float L = 0.f, a = 0.f;
  for (int t0 = 0; t0 < NC; t0 += TILE) {
    const int tn = min(TILE, NC - t0);
    __syncthreads();
    for (int i = c; i < tn; i += blockDim.x) {
      const float m = pr[(size_t)(t0 + i) * st];
      s_f[i] = (m == -INFINITY) ? 0.f : exp2f(m - M);
      s_l[i] = pr[(size_t)(t0 + i) * st + 1];
    }
    __syncthreads();
#pragma unroll 8
    for (int i = 0; i < tn; ++i) {
      const float f = s_f[i];
      L = fmaf(s_l[i], f, L);
      a = fmaf(pr[(size_t)(t0 + i) * st + 2 + c], f, a);
    }
  }
  // a head whose kept set is empty (only possible through loki_attend with
  // no in-range index) gets zeros
  out[(size_t)row * d + c] = from_f32<T>(L > 0.f ? a / L : 0.f);
}

// Heads with 33 to 128 chunk partials (long heads): four waves per head, wave
// w merging partials [w n, (w + 1) n), n = ceil(NC / 4), with every load of
// its share issued up front (the loop above keeps eight in flight, a chain of
// NC / 8 memory round trips); the four waves' (max, sum, acc) are then merged
// by log-sum-exp through LDS.
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_multi_kernel(const float* __restrict__ part,
                                                            T* __restrict__ out, int NC) {
  constexpr int MAXW = 32;     // partials per wave
  constexpr int EPL = D / 64;  // dims per lane
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_a[4][D];
  const int row = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = (NC + 3) / 4;  // <= MAXW for NC <= 128
  const int c0 = wave * n, cn = max(0, min(n, NC - c0));
  const size_t st = (size_t)D + 2;
  const float* pr = part + ((size_t)row * NC + c0) * st;
  float acc[MAXW][EPL];
#pragma unroll
  for (int ch = 0; ch < MAXW; ++ch) {
    if (ch < cn) {
      if constexpr (EPL == 2) {
        const float2 v = *reinterpret_cast<const float2*>(pr + ch * st + 2 + 2 * lane);
        acc[ch][0] = v.x;
        acc[ch][1] = v.y;
      } else {
        acc[ch][0] = pr[ch * st + 2 + lane];
      }
    }
  }
  float m = -INFINITY, l = 0.f;
  if (lane < cn) {
    m = pr[lane * st];
    l = pr[lane * st + 1];
  }
  const float Mw = wave_max(m);
  const float f = (m == -INFINITY) ? 0.f : exp2f(m - Mw);
  float L = 0.f, a[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) a[e] = 0.f;
#pragma unroll
  for (int ch = 0; ch < MAXW; ++ch) {
    if (ch < cn) {
      const float fc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), ch));
      const float lc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), ch));
      L = fmaf(lc, fc, L);
#pragma unroll
      for (int e = 0; e < EPL; ++e) a[e] = fmaf(acc[ch][e], fc, a[e]);
    }
  }
  if (lane == 0) {
    s_m[wave] = Mw;
    s_l[wave] = L;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_a[wave][lane * EPL + e] = a[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float Lt = 0.f, at = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float fw = (s_m[w] == -INFINITY) ? 0.f : exp2f(s_m[w] - M);
      Lt = fmaf(s_l[w], fw, Lt);
      at = fmaf(s_a[w][c], fw, at);
    }
    out[(size_t)row * D + c] = from_f32<T>(Lt > 0.f ? at / Lt : 0.f);
  }
}

template <typename T, int D>
static hipError_t launch_combine(const float* part, T* out, int rows, int NC, hipStream_t st) {
  if (NC > 32 && NC <= 128)
    hipLaunchKernelGGL((combine_multi_kernel<T, D>), dim3(rows), dim3(256), 0, st, part, out, NC);
  else
    hipLaunchKernelGGL((combine_kernel<T>), dim3(rows), dim3(D), 0, st, part, out, NC, D);
  return hipGetLastError();
}

// ============================================================================
// host side
// ============================================================================
static int next_pow2(long long x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

static int chunk_for(long long S, long long groups, int lo, int hi, long long blocks) {
  long long want = (S * groups + blocks - 1) / blocks;  // aim for >= `blocks` blocks
  int c = next_pow2(want < 1 ? 1 : want);
  if (c < lo) c = lo;
  if (c > hi) c = hi;
  return c;
}

bool make_decode_plan(DecodePlan& p, int B, int Hq, int Hkv, int S, int d, int r, int k, int dt) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || Hq % Hkv || (d != 64 && d != 128)) return false;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.S = S; p.d = d; p.r = r; p.k = k; p.dt = dt;
  p.G = Hq / Hkv;
  p.Sp = (S + 63) / 64 * 64;
  p.W = p.Sp / 32;
  const long long groups = (long long)B * Hkv;
  p.SC = chunk_for(S, groups, 256, 8192, 2048);
  p.NSC = (S + p.SC - 1) / p.SC;
  if (dt == 1 && p.G <= 8) {
    p.AC = 4 * kAttendMfmaTokens;  // MFMA attention: four waves per block
  } else {
    const int G = p.G;
    const int nt = G <= 4 ? 256 : (G <= 8 ? 128 : 64);
    p.AC = 4 * nt;  // vector-ALU attention: four waves per block
  }
  p.NAC = (S + p.AC - 1) / p.AC;
  const size_t rows = (size_t)B * Hq;
  // blocks per head of the one-launch selection + attention: as many as
  // one round of blocks on 256 CUs holds (each block repeats the head's
  // selection, so a second round would repeat it again), at most one per
  // 16-row tile of the kept list
  p.NSPL = 1;
  if (rows < 256) {
    long long ns = 256 / (long long)rows;
    ns = std::min(ns, std::min((long long)kSplitMax, std::max(1LL, (long long)(k + 15) / 16)));
    p.NSPL = (int)std::max(1LL, ns);
  }
  size_t off = 0;
  p.off_qrot = off;   off = align_up(off + rows * d * sizeof(float), 256);
  p.off_qsplit = off; off = align_up(off + rows * 4 * d * sizeof(uint16_t), 256);
  p.off_qrot_m = off; off = align_up(off + rows * d * sizeof(float), 256);
  p.off_qsplit_m = off; off = align_up(off + rows * 4 * d * sizeof(uint16_t), 256);
  p.off_keys = off;   off = align_up(off + rows * (size_t)p.Sp * sizeof(uint32_t), 256);
  p.off_mm = off;     off = align_up(off + rows * (size_t)p.NSC * sizeof(uint2), 256);
  p.off_masks = off;  off = align_up(off + rows * (size_t)(p.Sp / 16) * sizeof(uint32_t), 256);
  const size_t ldc = select_chunked_ldc(S, k);
  p.off_cidx = off;   off = align_up(off + rows * ldc * sizeof(int32_t), 256);
  p.off_ckey = off;   off = align_up(off + rows * ldc * sizeof(uint32_t), 256);
  p.off_bitmap = off; off = align_up(off + rows * (size_t)p.W * sizeof(uint32_t), 256);
  p.off_part = off;   off = align_up(off + rows * (size_t)p.NAC * (d + 2) * sizeof(float), 256);
  p.off_spart = off;  off = align_up(off + rows * (size_t)p.NSPL * (d + 2) * sizeof(float), 256);
  p.off_scnt = off;   off = align_up(off + rows * sizeof(uint32_t), 256);
  p.bytes = off;
  return true;
}

bool make_select_plan(SelectPlan& p, int rows, int S, int k) {
  if (rows < 1 || S < 1 || k < 1 || k > S) return false;
  p.rows = rows; p.S = S; p.k = k;
  p.Sp = (S + 63) / 64 * 64;
  p.W = p.Sp / 32;
  p.NMM = (S + 255) / 256 < 1024 ? (S + 255) / 256 : 1024;
  size_t off = 0;
  p.off_keys = off;   off = align_up(off + (size_t)rows * p.Sp * sizeof(uint32_t), 256);
  p.off_mm = off;     off = align_up(off + (size_t)rows * p.NMM * sizeof(uint2), 256);
  p.off_masks = off;  off = align_up(off + (size_t)rows * (p.Sp / 16) * sizeof(uint32_t), 256);
  const size_t ldc = select_chunked_ldc(S, k);
  p.off_cidx = off;   off = align_up(off + (size_t)rows * ldc * sizeof(int32_t), 256);
  p.off_ckey = off;   off = align_up(off + (size_t)rows * ldc * sizeof(uint32_t), 256);
  p.off_bitmap = off; off = align_up(off + (size_t)rows * p.W * sizeof(uint32_t), 256);
  p.bytes = off;
  return true;
}

template <typename F>
static hipError_t dispatch_group(int G, F&& f) {
  if (G <= 1) return f(std::integral_constant<int, 1>{});
  if (G <= 2) return f(std::integral_constant<int, 2>{});
  if (G <= 4) return f(std::integral_constant<int, 4>{});
  if (G <= 8) return f(std::integral_constant<int, 8>{});
  return f(std::integral_constant<int, 16>{});
}

template <typename T>
static hipError_t qrot_t(const DecodePlan& p, const void* q, const void* P, float* qrot,
                         bf16_t* qsplit, hipStream_t st, uint32_t* zero, int nzero) {
  return dispatch_group(p.G, [&](auto gt) {
    constexpr int GT = decltype(gt)::value;
    hipLaunchKernelGGL((qrot_kernel<T, GT>), dim3(p.B * p.Hkv, p.d / 32), dim3(256), 0, st,
                       static_cast<const T*>(q), static_cast<const T*>(P), qrot, qsplit, p.Hq, p.Hkv, p.d,
                       zero, zero ? nzero : 0);
    return hipGetLastError();
  });
}

hipError_t launch_qrot(const DecodePlan& p, const void* q, const void* P, float* qrot,
                       uint16_t* qsplit, hipStream_t st, uint32_t* zero, int nzero) {
  return p.dt == 0 ? qrot_t<float>(p, q, P, qrot, qsplit, st, zero, nzero)
                   : qrot_t<bf16_t>(p, q, P, qrot, qsplit, st, zero, nzero);
}

template <typename T, int GT>
static hipError_t scores_tg(const DecodePlan& p, const void* src, int ld, const float* qrot, void* out,
                            bool as_keys, int out_stride, uint2* mm, hipStream_t st) {
  const int e = (int)sizeof(T);
  const int gran = (p.r * e + 15) / 16;
  const int lpt = next_pow2(gran);
  const dim3 grid(p.NSC, p.B * p.Hkv), block(256);
  const T* K = static_cast<const T*>(src);
  const int ak = as_keys ? 1 : 0;
#define LOKI_SCORE(L)                                                                         \
  case L:                                                                                     \
    hipLaunchKernelGGL((score_kernel<T, L, GT>), grid, block, 0, st, K, qrot, out, ak,       \
                       out_stride, mm, p.Hq, p.Hkv, p.S, p.d, ld, p.r, p.SC, p.lens);             \
    break;
  switch (lpt) {
    LOKI_SCORE(1)
    LOKI_SCORE(2)
    LOKI_SCORE(4)
    LOKI_SCORE(8)
    LOKI_SCORE(16)
    LOKI_SCORE(32)
    default: return hipErrorInvalidValue;
  }
#undef LOKI_SCORE
  return hipGetLastError();
}

hipError_t launch_scores(const DecodePlan& p, const void* src, int ld, const float* qrot,
                         const uint16_t* qsplit, void* out, bool as_keys, int out_stride,
                         uint2* mm, hipStream_t st) {
  if (p.dt == 1) return launch_scores_mfma(p, src, ld, qsplit, out, as_keys, out_stride, mm, st);
  return dispatch_group(p.G, [&](auto gt) {
    constexpr int GT = decltype(gt)::value;
    return p.dt == 0 ? scores_tg<float, GT>(p, src, ld, qrot, out, as_keys, out_stride, mm, st)
                     : scores_tg<bf16_t, GT>(p, src, ld, qrot, out, as_keys, out_stride, mm, st);
  });
}

bool select_needs_minmax(int S) { return S > kSelThreads * kSelRegMaxT; }

size_t select_chunked_ldc(int S, int k) {
  if (S <= kSelThreads * kSelRegMaxT || k > kSelChunk) return 0;
  const int C = (S + kSelChunk - 1) / kSelChunk;
  const long long S2 = (long long)C * k;  // every chunk fills k candidate slots
  if (S2 > (long long)kSelThreads * kSelRegMaxT) return 0;
  return (size_t)S2;
}

// Second stage of the long-head selection over the candidate lists (ldc =
// select_chunked_ldc(S, k) words per row).
hipError_t launch_select_merge(int rows, int S, int k, int W, int ldc, const uint32_t* ckey, const int32_t* cidx,
                               int32_t* idx, uint32_t* bitmap, const int32_t* lens, int Hq, hipStream_t st) {
  if (!lens) Hq = 1;
  if (ldc <= kSelThreads * 16)
    hipLaunchKernelGGL((select_merge_kernel<16>), dim3(rows), dim3(kSelThreads), 0, st, ckey, cidx, ldc, ldc, k,
                       W, idx, bitmap, lens, Hq, S);
  else
    hipLaunchKernelGGL((select_merge_kernel<kSelRegMaxT>), dim3(rows), dim3(kSelThreads), 0, st, ckey, cidx, ldc,
                       ldc, k, W, idx, bitmap, lens, Hq, S);
  return hipGetLastError();
}

hipError_t launch_select(int rows, int S, int Sp, int k, int W, const uint32_t* keys, const uint2* mm,
                         int nmm, uint32_t* gmasks, int32_t* idx, uint32_t* bitmap, hipStream_t st,
                         int32_t* cidx, uint32_t* ckey, const int32_t* lens, int Hq) {
  if (!lens) Hq = 1;  // any divisor: without lengths every row has S tokens
  const size_t ldc = select_chunked_ldc(S, k);
  if (ldc && k < S) {
    if (!cidx || !ckey) return hipErrorInvalidValue;
    const int C = (S + kSelChunk - 1) / kSelChunk;
    const int S2 = (int)ldc;
    hipLaunchKernelGGL(select_chunk_kernel, dim3(C, rows), dim3(kSelThreads), 0, st, keys, S, Sp, k, (int)ldc,
                       cidx, ckey, lens, Hq);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_select_merge(rows, S, k, W, S2, ckey, cidx, idx, bitmap, lens, Hq, st);
  }
  // the fewest keys per lane that hold the head: each wave owns 64 T
  // consecutive tokens, so a larger T than needed leaves whole waves idle
  if (S <= kSelThreads * 4) {
    hipLaunchKernelGGL((select_regs_kernel<4>), dim3(rows), dim3(kSelThreads), 0, st, keys, S, Sp, k, W,
                       idx, bitmap, lens, Hq);
  } else if (S <= kSelThreads * 8) {
    hipLaunchKernelGGL((select_regs_kernel<8>), dim3(rows), dim3(kSelThreads), 0, st, keys, S, Sp, k, W,
                       idx, bitmap, lens, Hq);
  } else if (S <= kSelThreads * 16) {
    hipLaunchKernelGGL((select_regs_kernel<16>), dim3(rows), dim3(kSelThreads), 0, st, keys, S, Sp, k, W,
                       idx, bitmap, lens, Hq);
  } else if (S <= kSelThreads * kSelRegMaxT) {
    hipLaunchKernelGGL((select_regs_kernel<kSelRegMaxT>), dim3(rows), dim3(kSelThreads), 0, st, keys, S,
                       Sp, k, W, idx, bitmap, lens, Hq);
  } else {
    if (!mm || !gmasks) return hipErrorInvalidValue;
    hipLaunchKernelGGL(select_global_kernel, dim3(rows), dim3(kSelThreads), 0, st, keys, mm, nmm, gmasks,
                       S, Sp, k, W, idx, bitmap, lens, Hq);
  }
  return hipGetLastError();
}

hipError_t launch_scores_to_keys(const float* scores, uint32_t* keys, uint2* mm, int nmm, int rows,
                                 int S, int Sp, hipStream_t st) {
  hipLaunchKernelGGL(scores_to_keys_kernel, dim3(nmm, rows), dim3(256), 0, st, scores, keys, mm, S, Sp);
  return hipGetLastError();
}

hipError_t launch_idx_to_bitmap(const DecodePlan& p, const int32_t* idx, uint32_t* bitmap,
                                hipStream_t st) {
  hipLaunchKernelGGL(idx_to_bitmap_kernel, dim3(p.B * p.Hq), dim3(256), 0, st, idx, bitmap, p.S,
                     p.k, p.W);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t attend_td(const DecodePlan& p, const void* K_rot, const void* V, const float* qrot,
                            const uint32_t* bitmap, float* part, void* out, hipStream_t st,
                            hipEvent_t mid) {
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  hipError_t e = dispatch_group(p.G, [&](auto gt) {
    constexpr int GT = decltype(gt)::value;
    if (4 * AttendTokens<GT>::value != p.AC) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attend_kernel<T, D, GT>), dim3(p.NAC, p.B * p.Hkv), dim3(256), 0, st,
                       static_cast<const T*>(K_rot), static_cast<const T*>(V), qrot, bitmap, part,
                       p.Hq, p.Hkv, p.S, p.W, p.NAC, scale_log2);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  if (mid && (e = hipEventRecord(mid, st)) != hipSuccess) return e;
  return launch_combine<T, D>(part, static_cast<T*>(out), p.B * p.Hq, p.NAC, st);
}

hipError_t launch_attend(const DecodePlan& p, const void* K_rot, const void* V, const float* qrot,
                         const uint16_t* qsplit, const uint32_t* bitmap, float* part, void* out,
                         hipStream_t st, hipEvent_t mid) {
  if (p.dt == 1 && p.G <= 8) {
    hipError_t e = launch_attend_mfma(p, K_rot, V, qsplit, bitmap, part, st);
    if (e != hipSuccess) return e;
    if (mid && (e = hipEventRecord(mid, st)) != hipSuccess) return e;
    bf16_t* o = static_cast<bf16_t*>(out);
    return p.d == 64 ? launch_combine<bf16_t, 64>(part, o, p.B * p.Hq, p.NAC, st)
                     : launch_combine<bf16_t, 128>(part, o, p.B * p.Hq, p.NAC, st);
  }
  if (p.dt == 0)
    return p.d == 64 ? attend_td<float, 64>(p, K_rot, V, qrot, bitmap, part, out, st, mid)
                     : attend_td<float, 128>(p, K_rot, V, qrot, bitmap, part, out, st, mid);
  return p.d == 64 ? attend_td<bf16_t, 64>(p, K_rot, V, qrot, bitmap, part, out, st, mid)
                   : attend_td<bf16_t, 128>(p, K_rot, V, qrot, bitmap, part, out, st, mid);
}

}  // namespace loki
