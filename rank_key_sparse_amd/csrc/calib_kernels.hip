// Offline calibration of the projection basis P from sampled keys.
//
// The basis is the set of principal directions of the key matrix A (one row
// per sampled key): the right singular vectors of A, equivalently the
// eigenvectors of the Gram matrix A^T A, ordered by decreasing eigenvalue
// (AQUA page, appendix on the SVD and its complexity; Loki page, abstract:
// the keys' leading principal dimensions; AQUA, related work "LoKi
// Attention": the matrix is computed offline).  No centring: the method only
// uses P in dot products of uncentred queries and keys.
//
// Three launches per call, per key/value head kv:
//   gram_bf16_kernel / gram_f32_kernel - partial Gram matrices of runs of
//       key rows (rows of every batch element of head kv), in fp64:
//       bf16 keys on MFMA (products exact, fp32 sums over 256 rows, then
//       fp64), fp32 keys with fp64 FMAs (products exact);
//   gram_reduce_kernel - the partials of a head summed in a fixed order;
//   jacobi_c_kernel, jacobi_v_kernel, eig_out_kernel - cyclic two-sided
//       Jacobi in fp64 on the Gram matrix held in LDS (all d/2 disjoint
//       rotations of a round at once, round-robin pairing, rotations logged),
//       the eigenvector matrix rebuilt from the log, then eigenvalues ranked
//       in decreasing order, each eigenvector's largest-magnitude entry made
//       positive, P written.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "internal.h"

namespace loki {

typedef __bf16 cbf16x8_t __attribute__((ext_vector_type(8)));
typedef float cfloatx4_t __attribute__((ext_vector_type(4)));

constexpr int kGramTile = 32;       // key rows per tile (one 32-deep MFMA k-step)
constexpr int kGramFlush = 8;       // tiles summed in fp32 before adding into fp64
constexpr int kGramBlocks = 512;    // Gram blocks per call (all heads), before rounding
constexpr int kJacobiThreads = 1024;
constexpr int kJacobiMaxSweeps = 48;
constexpr double kJacobiSmallT = 1e-4;  // a sweep whose rotations all had |tan| below this may end the iteration

// Rounds of the rotation log per head (d - 1 rounds per sweep).
__host__ __device__ constexpr int jacobi_max_rounds(int D) { return kJacobiMaxSweeps * (D - 1); }

bool make_calib_plan(CalibPlan& p, int B, int Hkv, int S, int d, int dt) {
  if (B < 1 || Hkv < 1 || S < 1 || (d != 64 && d != 128)) return false;
  const long long N = (long long)B * S;
  if (N > 0x7fffffffLL) return false;
  p.B = B; p.Hkv = Hkv; p.S = S; p.d = d; p.dt = dt; p.N = (int)N;
  const long long per_head = (kGramBlocks + Hkv - 1) / Hkv;
  long long rows = (N + per_head - 1) / per_head;
  rows = (rows + kGramTile - 1) / kGramTile * kGramTile;
  if (rows < 8 * kGramTile) rows = 8 * kGramTile;
  p.rows = (int)rows;
  p.nblk = (int)((N + rows - 1) / rows);
  const size_t dd = (size_t)d * d * sizeof(double);
  size_t off = 0;
  p.off_part = off; off = align_up(off + (size_t)Hkv * p.nblk * dd, 256);
  p.off_C = off;    off = align_up(off + (size_t)Hkv * dd, 256);
  p.off_V = off;    off = align_up(off + (size_t)Hkv * dd, 256);
  p.off_log = off;  off = align_up(off + (size_t)Hkv * jacobi_max_rounds(d) * (d / 2) * 2 * sizeof(double), 256);
  p.off_nr = off;   off = align_up(off + (size_t)Hkv * sizeof(int), 256);
  p.off_lam = off;  off = align_up(off + (size_t)Hkv * d * sizeof(double), 256);
  p.bytes = off;
  return true;
}

// Address of key row n (0 <= n < B*S) of head kv: batch element n / S.
template <int D, typename T>
__device__ __forceinline__ const T* key_row(const T* K, int n, int kv, int Hkv, int S) {
  const int b = n / S, s = n - b * S;
  return K + (((size_t)b * Hkv + kv) * S + s) * D;
}

// ---------------------------------------------------------------------------
// Gram partials, bf16 keys.  Block = 4 waves over `rows` key rows; wave w
// owns the quadrant (w / 2, w % 2) of the d x d result.  A 32-row tile goes
// through LDS transposed (dim-major), so that both MFMA operands are
// "8 consecutive rows of one dim" per lane, one 16-byte LDS read each:
//   A[m][k] = X[k][16 i + m] and B[k][n] = X[k][16 j + n] (lane l: m or n =
//   l % 16, k = 8 (l / 16) .. +7); D[m][n] lane l: m = 4 (l / 16) + v,
//   n = l % 16.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void gram_bf16_kernel(const bf16_t* __restrict__ K,
                                                          double* __restrict__ part, int Hkv, int S,
                                                          int N, int rows, int nblk) {
  constexpr int TR = kGramTile;
  constexpr int TS = TR + 8;            // LDS stride of a dim's row (elements; 80 B)
  constexpr int GPT = TR * (D / 8) / 256;  // 16-byte granules per thread per tile
  constexpr int Q = D / 2;
  constexpr int NQ = Q / 16;
  static_assert(GPT >= 1, "tile too small for the block");
  __shared__ __align__(16) bf16_t sT[2][D * TS];

  const int kv = blockIdx.y, blk = blockIdx.x;
  const int r0 = blk * rows;
  const int r1 = min(N, r0 + rows);
  const int ntile = (r1 - r0 + TR - 1) / TR;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int I = wave >> 1, J = wave & 1;
  const int m = lane & 15, kq = lane >> 4;

  // granule u of this thread: row id % TR (consecutive lanes, consecutive
  // rows: conflict-free transposed LDS writes), dims 8 (id / TR) .. +7
  auto load_tile = [&](int t, uint4 (&buf)[GPT]) {
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int id = threadIdx.x + 256 * u;
      const int n = r0 + t * TR + id % TR;
      const uint4 v = ldg16(key_row<D>(K, min(n, r1 - 1), kv, Hkv, S) + 8 * (id / TR));
      buf[u] = (n < r1) ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_tile = [&](const uint4 (&buf)[GPT], bf16_t* T) {
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int id = threadIdx.x + 256 * u;
      const int row = id % TR, g = id / TR;
      const uint32_t w[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        T[(8 * g + e) * TS + row] = (bf16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
    }
  };

  cfloatx4_t acc[NQ][NQ];
  double acc64[NQ][NQ][4];
#pragma unroll
  for (int i = 0; i < NQ; ++i)
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      acc[i][j] = cfloatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v) acc64[i][j][v] = 0.0;
    }

  uint4 buf[GPT];
  load_tile(0, buf);
  for (int t = 0; t < ntile; ++t) {
    bf16_t* T = sT[t & 1];
    store_tile(buf, T);
    load_tile(min(t + 1, ntile - 1), buf);  // next tile in flight (the last one repeats)
    __syncthreads();
    cbf16x8_t a[NQ], b[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      a[i] = *reinterpret_cast<const cbf16x8_t*>(T + (I * Q + 16 * i + m) * TS + 8 * kq);
#pragma unroll
    for (int j = 0; j < NQ; ++j)
      b[j] = *reinterpret_cast<const cbf16x8_t*>(T + (J * Q + 16 * j + m) * TS + 8 * kq);
#pragma unroll
    for (int i = 0; i < NQ; ++i)
#pragma unroll
      for (int j = 0; j < NQ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    if (t % kGramFlush == kGramFlush - 1 || t == ntile - 1) {
#pragma unroll
      for (int i = 0; i < NQ; ++i)
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
#pragma unroll
          for (int v = 0; v < 4; ++v) acc64[i][j][v] += (double)acc[i][j][v];
          acc[i][j] = cfloatx4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
  }

  double* out = part + ((size_t)kv * nblk + blk) * D * D;
#pragma unroll
  for (int i = 0; i < NQ; ++i)
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        out[(size_t)(I * Q + 16 * i + 4 * kq + v) * D + J * Q + 16 * j + m] = acc64[i][j][v];
}

// ---------------------------------------------------------------------------
// Gram partials, fp32 keys: fp64 FMAs of exact fp32 products.  Thread t owns
// the E x E block (t / 16, t % 16) of the result; the 32-row tile sits in LDS
// row-major.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void gram_f32_kernel(const float* __restrict__ K,
                                                         double* __restrict__ part, int Hkv, int S,
                                                         int N, int rows, int nblk) {
  constexpr int TR = kGramTile;
  constexpr int RS = D + 4;                // LDS row stride (floats)
  constexpr int GPR = D / 4;               // granules per row
  constexpr int GPT = TR * GPR / 256;
  constexpr int E = D / 16;
  __shared__ __align__(16) float sX[2][TR * RS];

  const int kv = blockIdx.y, blk = blockIdx.x;
  const int r0 = blk * rows;
  const int r1 = min(N, r0 + rows);
  const int ntile = (r1 - r0 + TR - 1) / TR;
  const int ti = threadIdx.x / 16, tj = threadIdx.x % 16;

  auto load_tile = [&](int t, uint4 (&buf)[GPT]) {
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int id = threadIdx.x + 256 * u;
      const int n = r0 + t * TR + id / GPR;
      const uint4 v = ldg16(key_row<D>(K, min(n, r1 - 1), kv, Hkv, S) + 4 * (id % GPR));
      buf[u] = (n < r1) ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  double acc[E][E];
#pragma unroll
  for (int a = 0; a < E; ++a)
#pragma unroll
    for (int b = 0; b < E; ++b) acc[a][b] = 0.0;

  uint4 buf[GPT];
  load_tile(0, buf);
  for (int t = 0; t < ntile; ++t) {
    float* X = sX[t & 1];
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int id = threadIdx.x + 256 * u;
      *reinterpret_cast<uint4*>(X + (id / GPR) * RS + 4 * (id % GPR)) = buf[u];
    }
    load_tile(min(t + 1, ntile - 1), buf);
    __syncthreads();
    for (int n = 0; n < TR; ++n) {
      double xi[E], xj[E];
#pragma unroll
      for (int a = 0; a < E; ++a) {
        xi[a] = (double)X[n * RS + ti * E + a];
        xj[a] = (double)X[n * RS + tj * E + a];
      }
#pragma unroll
      for (int a = 0; a < E; ++a)
#pragma unroll
        for (int b = 0; b < E; ++b) acc[a][b] = fma(xi[a], xj[b], acc[a][b]);
    }
  }

  double* out = part + ((size_t)kv * nblk + blk) * D * D;
#pragma unroll
  for (int a = 0; a < E; ++a)
#pragma unroll
    for (int b = 0; b < E; ++b) out[(size_t)(ti * E + a) * D + tj * E + b] = acc[a][b];
}

// Sum of a head's partials, in block order.
__global__ __launch_bounds__(256) void gram_reduce_kernel(const double* __restrict__ part,
                                                          double* __restrict__ C, int nblk, int DD) {
  const int kv = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= DD) return;
  const double* p = part + (size_t)kv * nblk * DD + e;
  double s = 0.0;
  for (int i = 0; i < nblk; ++i) s += p[(size_t)i * DD];
  C[(size_t)kv * DD + e] = s;
}

// Round r of the round-robin pairing of n indices (n even): pair j is
// (n - 1, r) for j = 0, else ((r + j) mod (n - 1), (r - j) mod (n - 1)).
// Over n - 1 rounds every unordered pair occurs once; within a round the
// pairs are disjoint.
__device__ __forceinline__ void jacobi_pair(int r, int j, int n, int& p, int& q) {
  int a, b;
  if (j == 0) {
    a = n - 1;
    b = r;
  } else {
    a = (r + j) % (n - 1);
    b = (r - j + n - 1) % (n - 1);
  }
  p = min(a, b);
  q = max(a, b);
}

template <typename T> __device__ __forceinline__ T from_f64(double x);
template <> __device__ __forceinline__ float from_f64<float>(double x) { return (float)x; }
template <> __device__ __forceinline__ bf16_t from_f64<bf16_t>(double x) {
  // round the fp64 value to bf16 directly (nearest, ties to even) through the
  // exact fp32 neighbours: fp32 rounding first could double-round
  const float f = (float)x;  // nearest fp32
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  // f is exact or within half an fp32 ulp; on an exact bf16 midpoint after
  // the fp32 rounding, decide by the side of x
  if ((u & 0xffffu) == 0x8000u && back != x) u += (x > back) == (f > 0.f) ? 1u : (uint32_t)-1;
  return f32_to_bf16(__uint_as_float(u));
}

// ---------------------------------------------------------------------------
// Cyclic two-sided Jacobi on the Gram matrix C of one head, in three launches.
//
// jacobi_c_kernel (one block of 1024 threads per head): C (fp64) in LDS, only
// its upper triangle (row stride d + 1, so that a wave's accesses along a row
// or a column fall into different banks).  A round rotates the d/2 disjoint
// pairs (p, q) of the round-robin pairing; for a pair whose C_pq is off the
// diagonal by more than a relative threshold,
//   tau = (C_qq - C_pp) / (2 C_pq), t = sign(tau) / (|tau| + sqrt(1 + tau^2)),
//   c = 1 / sqrt(1 + t^2), s = t c, J = [[c, s], [-s, c]] on (p, q)
// (the symmetric Schur rotation that zeroes C_pq), and C <- J^T C J for all
// pairs at once: one thread per 2 x 2 block between pairs j <= j' (the
// upper triangle of blocks packed densely over the threads).  The
// rotations (c, s) of every round go to a log in the workspace.  Sweeps
// repeat while some pair passes the rotation test (tested on the whole
// matrix before each sweep; at most kJacobiMaxSweeps).
//
// jacobi_v_kernel (one wave per row of V): V = I J_1 J_2 ... from the log,
// partner columns exchanged by lane permutes.
//
// eig_out_kernel (one block per head): eigenvalues ranked in decreasing order
// (equal values by index), each eigenvector's first entry of largest
// magnitude made positive, P and the eigenvalues written.
// ---------------------------------------------------------------------------
constexpr int kJacobiVChunk = 16;  // logged rounds staged in LDS at a time by the rotation-apply kernel

template <int D>
__global__ __launch_bounds__(kJacobiThreads) void jacobi_c_kernel(const double* __restrict__ Cg,
                                                                   double2* __restrict__ rlog,
                                                                   int* __restrict__ nrounds,
                                                                   double* __restrict__ lam_raw) {
  constexpr int NP = D / 2;
  constexpr int DS = D + 1;
  constexpr double kTol = 1e-14;
  constexpr double kTiny = 1e-300;
  constexpr int NOFF = NP * (NP - 1) / 2;  // off-diagonal 2 x 2 blocks j < j2
  constexpr int NDT = NP / 2;              // threads holding the diagonal blocks, two each
  static_assert(NOFF <= 2 * kJacobiThreads, "at most two off-diagonal blocks per thread");
  static_assert(NOFF - kJacobiThreads <= kJacobiThreads - NDT, "diagonal threads hold at most one off-diagonal block");
  extern __shared__ __align__(16) double sC[];
  __shared__ double2 s_cs[NP];  // this round's (c, s) per pair
  __shared__ double s_t[NP];
  __shared__ int2 s_pq[NP];     // this round's pairs (p < q)
  __shared__ int s_rot, s_big;

  const int kv = blockIdx.x, tid = threadIdx.x;
  const double* Ch = Cg + (size_t)kv * D * D;
  double2* lg = rlog + (size_t)kv * jacobi_max_rounds(D) * NP;
  // this thread's blocks (the same every round).  The off-diagonal blocks
  // are packed densely over the threads, at most two each (fold i holds row
  // i, j2 = i+1 .. NP-1, and row NP-1-i, j2 = NP-i .. NP-1); the NP cheap
  // diagonal blocks go two each to the last NP/2 threads, which hold at most
  // one off-diagonal block, so that no thread updates three blocks a round
  // and the block loop has no branch between the two kinds.
  int bj[2], bj2[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int id = tid + u * kJacobiThreads;
    const int fi = id / (NP - 1), fc = id - fi * (NP - 1);
    const bool lo = fc < NP - 1 - fi;
    bj[u] = id < NOFF ? (lo ? fi : NP - 1 - fi) : -1;
    bj2[u] = lo ? fi + 1 + fc : fc + 1;
  }
  const int jd = 2 * (tid - (kJacobiThreads - NDT));  // this thread's diagonal blocks jd, jd + 1 (if >= 0)
  auto U = [&](int x, int y) -> double& { return sC[min(x, y) * DS + max(x, y)]; };
  // the rotation test of a pair (a, b its diagonal entries, g the off-diagonal one)
  auto rotates = [](double a, double b, double g) {
    return fabs(g) > kTiny && fabs(g) > kTol * sqrt(fabs(a)) * sqrt(fabs(b));
  };

  for (int e = tid; e < D * D; e += kJacobiThreads) {
    const int i = e / D, j = e - i * D;
    if (i <= j) sC[i * DS + j] = Ch[e];
  }
  if (tid == 0) {
    s_rot = 0;
    s_big = 0;
  }
  __syncthreads();

  int round = 0;
  double tmax = 0.0;  // lanes tid < NP: the largest |t| this lane applied in the last sweep
  for (int sweep = 0; sweep < kJacobiMaxSweeps; ++sweep) {
    // A sweep rotates nothing exactly when no pair passes the rotation test
    // on the current matrix (then nothing changes during it), so one pass
    // over the pairs decides that instead of running such a sweep.  The pass
    // runs before the first sweep and after a sweep whose rotations were all
    // small (near convergence, where the next sweep may be empty); otherwise
    // the sweep simply runs.
    if (tid < NP && tmax >= kJacobiSmallT) s_big = 1;
    __syncthreads();
    if (s_big == 0) {  // the same value in every thread
      bool any = false;
      for (int e = tid; e < D * D; e += kJacobiThreads) {
        const int x = e / D, y = e - x * D;
        if (x < y && rotates(sC[x * DS + x], sC[y * DS + y], sC[x * DS + y])) any = true;
      }
      if (any) s_rot = 1;
      __syncthreads();
      const bool go = s_rot != 0;  // the same value in every thread
      __syncthreads();
      if (!go) break;
    }
    __syncthreads();  // every thread has read s_big and s_rot
    if (tid == 0) {
      s_big = 0;
      s_rot = 0;
    }
    tmax = 0.0;
    for (int r = 0; r < D - 1; ++r, ++round) {
      if (tid < NP) {
        int p, q;
        jacobi_pair(r, tid, D, p, q);
        const double a = U(p, p), b = U(q, q), g = U(p, q);
        double c = 1.0, s = 0.0, t = 0.0;
        if (rotates(a, b, g)) {
          const double tau = (b - a) / (2.0 * g);
          t = (fabs(tau) > 1e150) ? 0.5 / tau
                                  : (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
          tmax = fmax(tmax, fabs(t));
        }
        s_cs[tid] = make_double2(c, s);
        s_t[tid] = t;
        s_pq[tid] = make_int2(p, q);
        lg[(size_t)round * NP + tid] = make_double2(c, s);
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = bj[u], j2 = bj2[u];
        if (j < 0) break;
        const int2 pq = s_pq[j];
        const int p = pq.x, q = pq.y;
        const double2 cs = s_cs[j];
        const double c = cs.x, s = cs.y;
        const int2 pq2 = s_pq[j2];
        const int p2 = pq2.x, q2 = pq2.y;
        const double2 cs2 = s_cs[j2];
        const double c2 = cs2.x, s2 = cs2.y;
        const double m00 = U(p, p2), m01 = U(p, q2), m10 = U(q, p2), m11 = U(q, q2);
        // rows: J^T M; columns: (J^T M) J'
        const double l00 = c * m00 - s * m10, l01 = c * m01 - s * m11;
        const double l10 = s * m00 + c * m10, l11 = s * m01 + c * m11;
        U(p, p2) = c2 * l00 - s2 * l01;
        U(p, q2) = s2 * l00 + c2 * l01;
        U(q, p2) = c2 * l10 - s2 * l11;
        U(q, q2) = s2 * l10 + c2 * l11;
      }
      if (jd >= 0) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j = jd + e;
          const int2 pq = s_pq[j];
          const int p = pq.x, q = pq.y;
          if (s_cs[j].y != 0.0) {
            const double t = s_t[j], g = U(p, q);
            U(p, p) -= t * g;
            U(q, q) += t * g;
            U(p, q) = 0.0;
          }
        }
      }
      __syncthreads();
    }
  }
  if (tid == 0) nrounds[kv] = round;
  if (tid < D) lam_raw[(size_t)kv * D + tid] = sC[tid * DS + tid];
}

// V = I J_1 J_2 ... from the log.  The rows of V evolve independently (V <- V J
// acts on columns), so one wave owns a row: lane l holds its columns l and
// l + 64 (d = 128) or l (d = 64).  In round r a column's partner and pair
// index follow from the round-robin pairing (col = d-1 pairs with r; col = r
// with d-1; otherwise the partner is 2r - col mod (d-1) and the pair index
// whichever of (col - r), (r - col) mod (d-1) is below d/2); the partner's
// value comes from its lane by a lane permute, the pair's (c, s) from LDS,
// where the block stages the log a chunk at a time (the next chunk travels
// in registers meanwhile), so the only barriers are per chunk.
template <int D>
__global__ __launch_bounds__(256) void jacobi_v_kernel(const double2* __restrict__ rlog,
                                                       const int* __restrict__ nrounds,
                                                       double* __restrict__ V) {
  constexpr int NP = D / 2;
  constexpr int EPL = D / 64;
  constexpr int WPB = 4;                      // rows (waves) per block
  constexpr int CH = kJacobiVChunk;           // logged rounds per chunk
  constexpr int PER = CH * NP / 256;          // log entries per thread per chunk
  static_assert(CH * NP % 256 == 0, "chunk split over the block");
  __shared__ __align__(16) double2 sL[2][CH * NP];

  const int kv = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * WPB + wave;
  const int nr = nrounds[kv];
  const double2* lg = rlog + (size_t)kv * jacobi_max_rounds(D) * NP;
  auto fetch = [&](int c0, double2 (&buf)[PER]) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = threadIdx.x + 256 * u;
      const int rd = c0 + e / NP;
      const double2 v = lg[(size_t)min(rd, max(nr - 1, 0)) * NP + e % NP];
      buf[u] = rd < nr ? v : make_double2(1.0, 0.0);
    }
  };
  double v[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) v[e] = (row == lane + 64 * e) ? 1.0 : 0.0;
  double2 buf[PER];
  if (nr > 0) {
    fetch(0, buf);
#pragma unroll
    for (int u = 0; u < PER; ++u) sL[0][threadIdx.x + 256 * u] = buf[u];
  }
  __syncthreads();
  const int nch = (nr + CH - 1) / CH;
  for (int ch = 0; ch < nch; ++ch) {
    fetch((ch + 1) * CH, buf);  // the next chunk travels while this one is applied
    const double2* L = sL[ch & 1];
    // rounds past the last logged one hold (1, 0), an exact identity, so
    // every chunk runs whole and its index arithmetic is off the chain
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int r = (ch * CH + k) % (D - 1);
      double nv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int col = lane + 64 * e;
        int partner, j;
        if (col == D - 1) {
          partner = r;
          j = 0;
        } else if (col == r) {
          partner = D - 1;
          j = 0;
        } else {
          partner = (2 * r - col + 2 * (D - 1)) % (D - 1);
          const int jj = (col - r + (D - 1)) % (D - 1);
          j = jj < NP ? jj : (r - col + (D - 1)) % (D - 1);
        }
        double pv = __shfl(v[0], partner & 63);
        if constexpr (EPL == 2) {
          const double pv1 = __shfl(v[1], partner & 63);
          pv = partner >= 64 ? pv1 : pv;
        }
        const double2 cs = L[k * NP + j];
        // V'[:, p] = c V[:, p] - s V[:, q],  V'[:, q] = s V[:, p] + c V[:, q]
        nv[e] = col < partner ? cs.x * v[e] - cs.y * pv : cs.y * pv + cs.x * v[e];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[e] = nv[e];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) sL[(ch + 1) & 1][threadIdx.x + 256 * u] = buf[u];
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) V[((size_t)kv * D + row) * D + lane + 64 * e] = v[e];
}

template <int D, typename T>
__global__ __launch_bounds__(kJacobiThreads) void eig_out_kernel(const double* __restrict__ V,
                                                                  const double* __restrict__ lam_raw,
                                                                  T* __restrict__ P, double* __restrict__ eigvals) {
  __shared__ int s_rank[D];
  const int kv = blockIdx.x, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const double* lam = lam_raw + (size_t)kv * D;
  const double* Vh = V + (size_t)kv * D * D;
  if (tid < D) {
    const double li = lam[tid];
    int rank = 0;
    for (int j = 0; j < D; ++j) {
      const double lj = lam[j];
      rank += (lj > li) || (lj == li && j < tid);
    }
    s_rank[tid] = rank;
    if (eigvals) eigvals[(size_t)kv * D + rank] = li;
  }
  __syncthreads();
  T* Ph = P + (size_t)kv * D * D;
  for (int col = wave; col < D; col += kJacobiThreads / 64) {
    double best = -1.0;
    int bi = 0;
    for (int i = lane; i < D; i += 64) {
      const double v = fabs(Vh[(size_t)i * D + col]);
      if (v > best) {
        best = v;
        bi = i;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ob = __shfl_xor(best, off);
      const int oi = __shfl_xor(bi, off);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    const double sg = (Vh[(size_t)bi * D + col] < 0.0) ? -1.0 : 1.0;
    const int rk = s_rank[col];
    for (int i = lane; i < D; i += 64) Ph[(size_t)i * D + rk] = from_f64<T>(sg * Vh[(size_t)i * D + col]);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Gram partials of the plan's rows and their sum into C [Hkv][d][d]; the
// event (may be null) is recorded between the two launches.
static hipError_t launch_gram(const CalibPlan& p, const void* K, double* part, double* C, hipStream_t st,
                              hipEvent_t mid) {
  const int D = p.d, DD = D * D;
  const dim3 ggrid(p.nblk, p.Hkv);
  if (p.dt == 1) {
    const bf16_t* k = static_cast<const bf16_t*>(K);
    if (D == 128)
      hipLaunchKernelGGL((gram_bf16_kernel<128>), ggrid, dim3(256), 0, st, k, part, p.Hkv, p.S, p.N, p.rows,
                         p.nblk);
    else
      hipLaunchKernelGGL((gram_bf16_kernel<64>), ggrid, dim3(256), 0, st, k, part, p.Hkv, p.S, p.N, p.rows,
                         p.nblk);
  } else {
    const float* k = static_cast<const float*>(K);
    if (D == 128)
      hipLaunchKernelGGL((gram_f32_kernel<128>), ggrid, dim3(256), 0, st, k, part, p.Hkv, p.S, p.N, p.rows,
                         p.nblk);
    else
      hipLaunchKernelGGL((gram_f32_kernel<64>), ggrid, dim3(256), 0, st, k, part, p.Hkv, p.S, p.N, p.rows,
                         p.nblk);
  }
  hipError_t e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (mid && (e = hipEventRecord(mid, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(gram_reduce_kernel, dim3((DD + 255) / 256, p.Hkv), dim3(256), 0, st, part, C, p.nblk, DD);
  return hipGetLastError();
}

// Jacobi on the H symmetric matrices C [H][d][d]: unsorted eigenvalues to
// lam_raw [H][d], eigenvectors as the columns of V [H][d][d].
static hipError_t launch_sym_eig(int D, int H, const double* C, double2* rlog, int* nr, double* lam_raw, double* V,
                                 hipStream_t st) {
  const size_t lds = (size_t)D * (D + 1) * sizeof(double);
  hipError_t e;
  auto kc = (D == 128) ? &jacobi_c_kernel<128> : &jacobi_c_kernel<64>;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kc), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(kc, dim3(H), dim3(kJacobiThreads), lds, st, C, rlog, nr, lam_raw);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (D == 128)
    hipLaunchKernelGGL(jacobi_v_kernel<128>, dim3(128 / 4, H), dim3(256), 0, st, rlog, nr, V);
  else
    hipLaunchKernelGGL(jacobi_v_kernel<64>, dim3(64 / 4, H), dim3(256), 0, st, rlog, nr, V);
  return hipGetLastError();
}

hipError_t launch_calibrate(const CalibPlan& p, const void* K, void* P, double* eigvals, void* ws,
                            hipStream_t st, hipEvent_t* ev) {
  char* w = static_cast<char*>(ws);
  double* part = reinterpret_cast<double*>(w + p.off_part);
  double* C = reinterpret_cast<double*>(w + p.off_C);
  double* Vt = reinterpret_cast<double*>(w + p.off_V);
  double2* rlog = reinterpret_cast<double2*>(w + p.off_log);
  int* nr = reinterpret_cast<int*>(w + p.off_nr);
  double* lam_raw = reinterpret_cast<double*>(w + p.off_lam);
  const int D = p.d;
  hipError_t e;
  if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
  if ((e = launch_gram(p, K, part, C, st, ev ? ev[1] : nullptr)) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  if ((e = launch_sym_eig(D, p.Hkv, C, rlog, nr, lam_raw, Vt, st)) != hipSuccess) return e;
  if (p.dt == 1) {
    auto ko = (D == 128) ? &eig_out_kernel<128, bf16_t> : &eig_out_kernel<64, bf16_t>;
    hipLaunchKernelGGL(ko, dim3(p.Hkv), dim3(kJacobiThreads), 0, st, Vt, lam_raw, static_cast<bf16_t*>(P), eigvals);
  } else {
    auto ko = (D == 128) ? &eig_out_kernel<128, float> : &eig_out_kernel<64, float>;
    hipLaunchKernelGGL(ko, dim3(p.Hkv), dim3(kJacobiThreads), 0, st, Vt, lam_raw, static_cast<float*>(P), eigvals);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
  return hipSuccess;
}

// ===========================================================================
// Asymmetric scoring index (page "SAKI: Score-Aware Low-Rank Key Indexing
// with Random-Matrix Noise Correction for KV Retrieval", abstract): the rank-r
// factors minimising the expected squared score error
// || Cq^{1/2} (I - A B^T) Ck^{1/2} ||_F^2, Cq and Ck the query and key second
// moments, are read off the SVD of W = Cq^{1/2} Ck^{1/2} = U S V^T:
// A = Cq^{-1/2} W V_r S_r^{-1/2} (= Cq^{-1/2} U_r S_r^{1/2}), B = Ck^{-1/2} V_r S_r^{1/2}.
// Matrix square roots and inverse square roots come from Jacobi
// eigendecompositions (eigenvalues below 1e-12 of the largest count as zero);
// V and S^2 from the eigendecomposition of W^T W.  All in fp64.
// ===========================================================================
constexpr double kAsymFloor = 1e-12;

// out[h][e] = scale * sum_{g < G} in[h G + g][e]
__global__ __launch_bounds__(256) void pool_kernel(const double* __restrict__ in, double* __restrict__ out, int G,
                                                   int DD, double scale) {
  const int h = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  if (e >= DD) return;
  double s = 0.0;
  for (int g = 0; g < G; ++g) s += in[((size_t)h * G + g) * DD + e];
  out[(size_t)h * DD + e] = s * scale;
}

// out[h] = V[h] diag(f(lam[h])) V[h]^T, f = sqrt (mode 0) or the inverse
// square root above the floor, else 0 (mode 1); negative rounding -> 0.
template <int D>
__global__ __launch_bounds__(D) void psd_fn_kernel(const double* __restrict__ V, const double* __restrict__ lam,
                                                   double* __restrict__ out, int mode) {
  __shared__ double f[D], vi[D], red[D];
  const int h = blockIdx.y, i = blockIdx.x, j = threadIdx.x;
  const double* Vh = V + (size_t)h * D * D;
  const double l = fmax(lam[(size_t)h * D + j], 0.0);
  red[j] = l;
  vi[j] = Vh[(size_t)i * D + j];
  __syncthreads();
  for (int o = D / 2; o > 0; o >>= 1) {
    if (j < o) red[j] = fmax(red[j], red[j + o]);
    __syncthreads();
  }
  const double lmax = red[0];
  f[j] = mode == 0 ? sqrt(l) : (l > kAsymFloor * lmax ? 1.0 / sqrt(l) : 0.0);
  __syncthreads();
  double s = 0.0;
  for (int c = 0; c < D; ++c) s = fma(vi[c] * f[c], Vh[(size_t)j * D + c], s);
  out[((size_t)h * D + i) * D + j] = s;
}

// out[h] = X'[h] Y[h], X' = X or X^T
template <int D>
__global__ __launch_bounds__(D) void matmul_kernel(const double* __restrict__ X, const double* __restrict__ Y,
                                                   double* __restrict__ out, int tx) {
  __shared__ double xr[D];
  const int h = blockIdx.y, i = blockIdx.x, j = threadIdx.x;
  const double* Xh = X + (size_t)h * D * D;
  const double* Yh = Y + (size_t)h * D * D;
  xr[j] = tx ? Xh[(size_t)j * D + i] : Xh[(size_t)i * D + j];
  __syncthreads();
  double s = 0.0;
  for (int c = 0; c < D; ++c) s = fma(xr[c], Yh[(size_t)c * D + j], s);
  out[((size_t)h * D + i) * D + j] = s;
}

// From the eigenpairs (unsorted) of W^T W: the r largest s^2 = lam in
// decreasing order (equal values by index); column k < r of VA / VB is the
// k-th such eigenvector times s^{-1/2} / s^{1/2} (both 0 below the floor),
// columns k >= r are zero.
template <int D>
__global__ __launch_bounds__(D) void asym_cols_kernel(const double* __restrict__ Vw, const double* __restrict__ lam,
                                                      double* __restrict__ VA, double* __restrict__ VB, int r) {
  __shared__ double ls[D];
  const int h = blockIdx.x, c = threadIdx.x;
  const double lc = fmax(lam[(size_t)h * D + c], 0.0);
  ls[c] = lc;
  __syncthreads();
  int rank = 0;
  double lmax = 0.0;
  for (int j = 0; j < D; ++j) {
    rank += (ls[j] > lc) || (ls[j] == lc && j < c);
    lmax = fmax(lmax, ls[j]);
  }
  const double s = sqrt(lc);
  const bool keep = rank < r && lc > kAsymFloor * lmax;
  const double fa = keep ? 1.0 / sqrt(s) : 0.0, fb = keep ? sqrt(s) : 0.0;
  const double* Vh = Vw + (size_t)h * D * D;
  double* A = VA + (size_t)h * D * D;
  double* B = VB + (size_t)h * D * D;
  for (int i = 0; i < D; ++i) {
    const double v = Vh[(size_t)i * D + c];
    A[(size_t)i * D + rank] = v * fa;
    B[(size_t)i * D + rank] = v * fb;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void cast_kernel(const double* __restrict__ in, T* __restrict__ out, int n) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < n) out[e] = from_f64<T>(in[e]);
}

bool make_asym_plan(AsymPlan& p, int N, int Hq, int B, int Hkv, int S, int d, int r, int dt) {
  if (N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || r < 1 || r > d) return false;
  if (!make_calib_plan(p.qp, N, Hq, 1, d, dt) || !make_calib_plan(p.kp, B, Hkv, S, d, dt)) return false;
  p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.d = d; p.r = r; p.dt = dt; p.N = N; p.BS = (long long)B * S;
  const size_t dd = (size_t)d * d * sizeof(double);
  const size_t part = std::max((size_t)Hq * p.qp.nblk, (size_t)Hkv * p.kp.nblk) * dd;
  size_t off = 0;
  auto take = [&](size_t n) { const size_t o = off; off = align_up(off + n, 256); return o; };
  p.off_part = take(part);
  p.off_Cqh = take((size_t)Hq * dd);
  // the eigensolver's scratch for 2 Hkv heads: Cq and Ck are diagonalised in one launch
  p.off_log = take((size_t)2 * Hkv * jacobi_max_rounds(d) * (d / 2) * 2 * sizeof(double));
  p.off_nr = take((size_t)2 * Hkv * sizeof(int));
  p.off_lam = take((size_t)2 * Hkv * d * sizeof(double));
  p.off_V2 = take((size_t)2 * Hkv * dd);
  for (int m = 0; m < kAsymMats; ++m) p.off_mat[m] = take((size_t)Hkv * dd);
  p.bytes = off;
  // that launch reads Cq and Ck as one [2 Hkv, d, d] array
  return p.off_mat[1] == p.off_mat[0] + (size_t)Hkv * dd;
}

hipError_t launch_calibrate_asym(const AsymPlan& p, const void* q_samples, const void* K, void* A, void* Bm, void* ws,
                                 hipStream_t st) {
  char* w = static_cast<char*>(ws);
  double* part = reinterpret_cast<double*>(w + p.off_part);
  double* Cqh = reinterpret_cast<double*>(w + p.off_Cqh);
  double2* rlog = reinterpret_cast<double2*>(w + p.off_log);
  int* nr = reinterpret_cast<int*>(w + p.off_nr);
  double* lam = reinterpret_cast<double*>(w + p.off_lam);
  double* M[kAsymMats];
  for (int m = 0; m < kAsymMats; ++m) M[m] = reinterpret_cast<double*>(w + p.off_mat[m]);
  double *Cq = M[0], *Ck = M[1], *Vq = M[2], *Sq = M[3], *Sqi = M[4], *Sk = M[5], *Ski = M[6], *W = M[7],
         *WtW = M[8], *VA = M[9], *VB = M[10], *T = M[11];
  const int D = p.d, DD = D * D, H = p.Hkv;
  hipError_t e;
  // second moments: queries pooled over each group's heads, keys
  if ((e = launch_gram(p.qp, q_samples, part, Cqh, st, nullptr)) != hipSuccess) return e;
  hipLaunchKernelGGL(pool_kernel, dim3((DD + 255) / 256, H), dim3(256), 0, st, Cqh, Cq, p.G, DD,
                     1.0 / ((double)p.N * p.G));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_gram(p.kp, K, part, Cqh, st, nullptr)) != hipSuccess) return e;
  hipLaunchKernelGGL(pool_kernel, dim3((DD + 255) / 256, H), dim3(256), 0, st, Cqh, Ck, 1, DD, 1.0 / (double)p.BS);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 mg(D, H), mb(D);
  auto psd = [&](const double* Vv, const double* lv, double* out, int mode) {
    if (D == 128) hipLaunchKernelGGL(psd_fn_kernel<128>, mg, mb, 0, st, Vv, lv, out, mode);
    else hipLaunchKernelGGL(psd_fn_kernel<64>, mg, mb, 0, st, Vv, lv, out, mode);
    return hipGetLastError();
  };
  auto mm = [&](const double* X, const double* Y, double* out, int tx) {
    if (D == 128) hipLaunchKernelGGL(matmul_kernel<128>, mg, mb, 0, st, X, Y, out, tx);
    else hipLaunchKernelGGL(matmul_kernel<64>, mg, mb, 0, st, X, Y, out, tx);
    return hipGetLastError();
  };
  // Cq^{1/2}, Cq^{-1/2}, Ck^{1/2}, Ck^{-1/2}: Cq and Ck (adjacent) diagonalised in one launch of
  // 2 H heads, Cq's eigenpairs first
  double* V2 = reinterpret_cast<double*>(w + p.off_V2);
  if ((e = launch_sym_eig(D, 2 * H, Cq, rlog, nr, lam, V2, st)) != hipSuccess) return e;
  const double* Vk = V2 + (size_t)H * DD;
  const double* lamk = lam + (size_t)H * D;
  if ((e = psd(V2, lam, Sq, 0)) != hipSuccess || (e = psd(V2, lam, Sqi, 1)) != hipSuccess) return e;
  if ((e = psd(Vk, lamk, Sk, 0)) != hipSuccess || (e = psd(Vk, lamk, Ski, 1)) != hipSuccess) return e;
  // W = Cq^{1/2} Ck^{1/2}; V, S^2 from W^T W
  if ((e = mm(Sq, Sk, W, 0)) != hipSuccess || (e = mm(W, W, WtW, 1)) != hipSuccess) return e;
  if ((e = launch_sym_eig(D, H, WtW, rlog, nr, lam, Vq, st)) != hipSuccess) return e;
  if (D == 128) hipLaunchKernelGGL(asym_cols_kernel<128>, dim3(H), dim3(128), 0, st, Vq, lam, VA, VB, p.r);
  else hipLaunchKernelGGL(asym_cols_kernel<64>, dim3(H), dim3(64), 0, st, Vq, lam, VA, VB, p.r);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // A = Cq^{-1/2} (W VA), B = Ck^{-1/2} VB
  if ((e = mm(W, VA, T, 0)) != hipSuccess || (e = mm(Sqi, T, VA, 0)) != hipSuccess) return e;
  if ((e = mm(Ski, VB, T, 0)) != hipSuccess) return e;
  const int n = H * DD;
  if (p.dt == 1) {
    hipLaunchKernelGGL(cast_kernel<bf16_t>, dim3((n + 255) / 256), dim3(256), 0, st, VA, static_cast<bf16_t*>(A), n);
    hipLaunchKernelGGL(cast_kernel<bf16_t>, dim3((n + 255) / 256), dim3(256), 0, st, T, static_cast<bf16_t*>(Bm), n);
  } else {
    hipLaunchKernelGGL(cast_kernel<float>, dim3((n + 255) / 256), dim3(256), 0, st, VA, static_cast<float*>(A), n);
    hipLaunchKernelGGL(cast_kernel<float>, dim3((n + 255) / 256), dim3(256), 0, st, T, static_cast<float*>(Bm), n);
  }
  return hipGetLastError();
}

}  // namespace loki
