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
// pairs at once: one thread per 2 x 2 block between pairs j <= j'.  The
// rotations (c, s) of every round go to a log in the workspace.  Sweeps
// repeat until one rotates nothing (at most kJacobiMaxSweeps).
//
// jacobi_v_kernel (one block per 16 rows of V and head): V = I J_1 J_2 ...
// from the log, the rows in LDS, one rotation of one row per thread and round.
//
// eig_out_kernel (one block per head): eigenvalues ranked in decreasing order
// (equal values by index), each eigenvector's first entry of largest
// magnitude made positive, P and the eigenvalues written.
// ---------------------------------------------------------------------------
constexpr int kJacobiVRows = 16;   // rows of V per block of the rotation-apply kernel
constexpr int kJacobiLogChunk = 16;  // logged rounds staged in LDS at a time

template <int D>
__global__ __launch_bounds__(kJacobiThreads) void jacobi_c_kernel(const double* __restrict__ Cg,
                                                                   double2* __restrict__ rlog,
                                                                   int* __restrict__ nrounds,
                                                                   double* __restrict__ lam_raw) {
  constexpr int NP = D / 2;
  constexpr int DS = D + 1;
  constexpr double kTol = 1e-14;
  constexpr double kTiny = 1e-300;
  extern __shared__ __align__(16) double sC[];
  __shared__ double s_c[NP], s_s[NP], s_t[NP];
  __shared__ int s_rot;

  const int kv = blockIdx.x, tid = threadIdx.x;
  const double* Ch = Cg + (size_t)kv * D * D;
  double2* lg = rlog + (size_t)kv * jacobi_max_rounds(D) * NP;
  auto U = [&](int x, int y) -> double& { return sC[min(x, y) * DS + max(x, y)]; };

  for (int e = tid; e < D * D; e += kJacobiThreads) {
    const int i = e / D, j = e - i * D;
    if (i <= j) sC[i * DS + j] = Ch[e];
  }
  if (tid == 0) s_rot = 0;
  __syncthreads();

  int round = 0;
  bool still = true;
  for (int sweep = 0; sweep < kJacobiMaxSweeps && still; ++sweep) {
    for (int r = 0; r < D - 1; ++r, ++round) {
      if (tid < NP) {
        int p, q;
        jacobi_pair(r, tid, D, p, q);
        const double a = U(p, p), b = U(q, q), g = U(p, q);
        double c = 1.0, s = 0.0, t = 0.0;
        if (fabs(g) > kTiny && fabs(g) > kTol * sqrt(fabs(a)) * sqrt(fabs(b))) {
          const double tau = (b - a) / (2.0 * g);
          t = (fabs(tau) > 1e150) ? 0.5 / tau
                                  : (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
          s_rot = 1;
        }
        s_c[tid] = c;
        s_s[tid] = s;
        s_t[tid] = t;
        lg[(size_t)round * NP + tid] = make_double2(c, s);
      }
      __syncthreads();
      for (int id = tid; id < NP * NP; id += kJacobiThreads) {
        const int j = id / NP, j2 = id - j * NP;
        if (j > j2) continue;
        int p, q, p2, q2;
        jacobi_pair(r, j, D, p, q);
        const double c = s_c[j], s = s_s[j];
        if (j == j2) {
          if (s != 0.0) {
            const double t = s_t[j], g = U(p, q);
            U(p, p) -= t * g;
            U(q, q) += t * g;
            U(p, q) = 0.0;
          }
          continue;
        }
        jacobi_pair(r, j2, D, p2, q2);
        const double c2 = s_c[j2], s2 = s_s[j2];
        const double m00 = U(p, p2), m01 = U(p, q2), m10 = U(q, p2), m11 = U(q, q2);
        // rows: J^T M; columns: (J^T M) J'
        const double l00 = c * m00 - s * m10, l01 = c * m01 - s * m11;
        const double l10 = s * m00 + c * m10, l11 = s * m01 + c * m11;
        U(p, p2) = c2 * l00 - s2 * l01;
        U(p, q2) = s2 * l00 + c2 * l01;
        U(q, p2) = c2 * l10 - s2 * l11;
        U(q, q2) = s2 * l10 + c2 * l11;
      }
      __syncthreads();
    }
    still = s_rot != 0;  // the same value in every thread
    __syncthreads();
    if (tid == 0) s_rot = 0;
    __syncthreads();
  }
  if (tid == 0) nrounds[kv] = still ? round : round - (D - 1);  // a last sweep without rotations is not replayed
  if (tid < D) lam_raw[(size_t)kv * D + tid] = sC[tid * DS + tid];
}

template <int D>
__global__ __launch_bounds__(kJacobiThreads) void jacobi_v_kernel(const double2* __restrict__ rlog,
                                                                   const int* __restrict__ nrounds,
                                                                   double* __restrict__ V) {
  constexpr int NP = D / 2;
  constexpr int DS = D + 1;
  constexpr int RB = kJacobiVRows;
  constexpr int CH = kJacobiLogChunk;
  constexpr int NT = NP * RB;  // threads: one (pair, row) each
  static_assert(CH * NP == NT, "one logged rotation per thread per chunk");
  __shared__ __align__(16) double sV[RB * DS];
  __shared__ __align__(16) double2 sL[2][CH * NP];

  const int kv = blockIdx.y, rb = blockIdx.x, tid = threadIdx.x;
  const int j = tid / RB, row = tid - j * RB;
  const int nr = nrounds[kv];
  const double2* lg = rlog + (size_t)kv * jacobi_max_rounds(D) * NP;
  auto fetch = [&](int c0) {
    const int rd = c0 + tid / NP;
    const double2 v = lg[(size_t)min(rd, max(nr - 1, 0)) * NP + tid % NP];
    return rd < nr ? v : make_double2(1.0, 0.0);
  };

  for (int e = tid; e < RB * D; e += NT) {
    const int rr = e / D, c = e - rr * D;
    sV[rr * DS + c] = (rb * RB + rr == c) ? 1.0 : 0.0;
  }
  if (nr > 0) sL[0][tid] = fetch(0);
  __syncthreads();
  const int nch = (nr + CH - 1) / CH;
  for (int ch = 0; ch < nch; ++ch) {
    const double2 nxt = fetch((ch + 1) * CH);  // the next chunk travels while this one is applied
    const double2* L = sL[ch & 1];
    const int kend = min(CH, nr - ch * CH);
    for (int k = 0; k < kend; ++k) {
      int p, q;
      jacobi_pair((ch * CH + k) % (D - 1), j, D, p, q);
      const double2 cs = L[k * NP + j];
      if (cs.y != 0.0) {
        const double vp = sV[row * DS + p], vq = sV[row * DS + q];
        sV[row * DS + p] = cs.x * vp - cs.y * vq;
        sV[row * DS + q] = cs.y * vp + cs.x * vq;
      }
      __syncthreads();
    }
    sL[(ch + 1) & 1][tid] = nxt;
    __syncthreads();
  }
  for (int e = tid; e < RB * D; e += NT) {
    const int rr = e / D, c = e - rr * D;
    V[((size_t)kv * D + rb * RB + rr) * D + c] = sV[rr * DS + c];
  }
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
hipError_t launch_calibrate(const CalibPlan& p, const void* K, void* P, double* eigvals, void* ws,
                            hipStream_t st, hipEvent_t* ev) {
  char* w = static_cast<char*>(ws);
  double* part = reinterpret_cast<double*>(w + p.off_part);
  double* C = reinterpret_cast<double*>(w + p.off_C);
  double* Vt = reinterpret_cast<double*>(w + p.off_V);
  const int D = p.d, DD = D * D;
  hipError_t e;
  if (ev && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
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
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  hipLaunchKernelGGL(gram_reduce_kernel, dim3((DD + 255) / 256, p.Hkv), dim3(256), 0, st, part, C, p.nblk,
                     DD);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  double2* rlog = reinterpret_cast<double2*>(w + p.off_log);
  int* nr = reinterpret_cast<int*>(w + p.off_nr);
  double* lam_raw = reinterpret_cast<double*>(w + p.off_lam);
  const size_t lds = (size_t)D * (D + 1) * sizeof(double);
  {
    auto kc = (D == 128) ? &jacobi_c_kernel<128> : &jacobi_c_kernel<64>;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(kc), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(kc, dim3(p.Hkv), dim3(kJacobiThreads), lds, st, C, rlog, nr, lam_raw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (D == 128)
    hipLaunchKernelGGL(jacobi_v_kernel<128>, dim3(128 / kJacobiVRows, p.Hkv), dim3(64 * kJacobiVRows), 0, st, rlog,
                       nr, Vt);
  else
    hipLaunchKernelGGL(jacobi_v_kernel<64>, dim3(64 / kJacobiVRows, p.Hkv), dim3(32 * kJacobiVRows), 0, st, rlog,
                       nr, Vt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
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

}  // namespace loki
