// Key projection K_rot[b,kv] = K[b,kv] * P[kv] (row-vector convention
// v_hat = v P, AQUA page, information-retention paragraph).
//
// bf16: MFMA v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The product
// is an [S x d] x [d x d] GEMM per (b, kv) whose arithmetic intensity (d/2
// flop per byte moved at d = 128) is far below the MFMA/HBM ridge, so the
// kernel is organised as a stream: P^T is staged once per block in LDS
// (padded rows), each wave owns 32-row tiles whose A operands it loads
// straight from HBM, and results go through a per-wave LDS tile so that
// global stores are full 16-byte row segments.
// fp32: plain VALU FMAs (no fp32 MFMA), P and the K tile in LDS.
// Either kernel can also write the leading R rotated dims of every row into a
// separate dense array K_lead [.., S, R] in the same pass (no extra reads).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace loki {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

// MFMA 32x32x16 operand layout (lane l, element i of the 8-element operand):
//   A[m][k]: m = l % 32, k = 8 * (l / 32) + i
//   B[k][n]: n = l % 32, k = 8 * (l / 32) + i
//   D[m][n] (16 fp32 per lane, element v): n = l % 32,
//            m = 8 * (v / 4) + 4 * (l / 32) + (v % 4)
template <int D>
__global__ __launch_bounds__(256) void project_bf16_kernel(const bf16_t* __restrict__ K,
                                                           const bf16_t* __restrict__ P,
                                                           bf16_t* __restrict__ out,
                                                           bf16_t* __restrict__ lead, int R,
                                                           int Hkv, int S, int tiles, int bpb) {
  constexpr int NT = D / 32;   // 32-column output tiles
  constexpr int KS = D / 16;   // 16-deep k steps
  constexpr int PS = D + 8;    // padded LDS row (elements) of P^T and of the output tile
  constexpr int ROWS = 32;     // rows per wave tile
  __shared__ __align__(16) bf16_t sPT[D * PS];
  __shared__ __align__(16) bf16_t sO[4][ROWS * PS];

  const int bk = blockIdx.x / bpb, part = blockIdx.x % bpb;
  const int kv = bk % Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  // P^T into LDS: sPT[n][k] = P[k][n]
  const bf16_t* Pk = P + (size_t)kv * D * D;
  for (int i = threadIdx.x; i < D * D / 8; i += 256) {
    const int kk = i / (D / 8), n0 = (i % (D / 8)) * 8;
    const uint4 v = ldg16(Pk + (size_t)kk * D + n0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      sPT[(n0 + e) * PS + kk] = (bf16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
  }
  __syncthreads();

  const bf16_t* Kb = K + (size_t)bk * S * D;
  bf16_t* Ob = out ? out + (size_t)bk * S * D : nullptr;  // null: only the lead dims are written
  bf16_t* Lb = lead ? lead + (size_t)bk * S * R : nullptr;
  const int m = lane & 31, half = lane >> 5;
  bf16_t* so = sO[wave];

  // 4 waves x 32 rows = one 128-row tile per block iteration
  for (int tile = part; tile < tiles; tile += bpb) {
    const int row0 = tile * 128 + wave * ROWS;
    const int row = row0 + m;
    bf16x8_t a[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row < S) v = ldg16(Kb + (size_t)row * D + ks * 16 + half * 8);
      a[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
    floatx16_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[nt][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(&sPT[(nt * 32 + m) * PS + ks * 16 + half * 8]);
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], bv, acc[nt], 0, 0, 0);
      }
    }
    // D fragments -> bf16 row-major tile in LDS
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int mm = 8 * (v >> 2) + 4 * half + (v & 3);
        so[mm * PS + nt * 32 + m] = f32_to_bf16(acc[nt][v]);
      }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // tile -> global, 16 bytes per lane, whole rows
    constexpr int LPR = D / 8;             // lanes per row
    constexpr int RPI = 64 / LPR;          // rows per store pass
#pragma unroll
    for (int p = 0; p < ROWS / RPI; ++p) {
      const int rr = p * RPI + lane / LPR, c8 = (lane % LPR) * 8;
      const int grow = row0 + rr;
      const uint4 v = *reinterpret_cast<const uint4*>(&so[rr * PS + c8]);
      if (grow < S) {
        if (out) *reinterpret_cast<uint4*>(Ob + (size_t)grow * D + c8) = v;
        if (Lb && c8 < R) *reinterpret_cast<uint4*>(Lb + (size_t)grow * R + c8) = v;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// fp32 projection on the vector ALUs: 64-row tiles, P[kv] and the tile in LDS;
// thread (row, 4 columns) accumulates over k = 0..D-1 in order.
template <int D>
__global__ __launch_bounds__(256) void project_f32_kernel(const float* __restrict__ K,
                                                          const float* __restrict__ P,
                                                          float* __restrict__ out,
                                                          float* __restrict__ lead, int R, int Hkv,
                                                          int S, int tiles, int bpb) {
  constexpr int TR = 64;
  extern __shared__ __align__(16) float dynf[];
  float* sP = dynf;            // [D][D]
  float* sK = dynf + D * D;    // [TR][D + 1]
  const int bk = blockIdx.x / bpb, part = blockIdx.x % bpb;
  const int kv = bk % Hkv;
  const float* Pk = P + (size_t)kv * D * D;
  for (int i = threadIdx.x; i < D * D; i += 256) sP[i] = Pk[i];
  const float* Kb = K + (size_t)bk * S * D;
  float* Ob = out ? out + (size_t)bk * S * D : nullptr;
  float* Lb = lead ? lead + (size_t)bk * S * R : nullptr;
  constexpr int CPT = D / 4;   // threads per row (4 columns each)
  constexpr int RPP = 256 / CPT;
  for (int tile = part; tile < tiles; tile += bpb) {
    const int row0 = tile * TR;
    __syncthreads();
    for (int i = threadIdx.x; i < TR * D; i += 256) {
      const int rr = i / D, c = i % D;
      sK[rr * (D + 1) + c] = (row0 + rr < S) ? Kb[(size_t)(row0 + rr) * D + c] : 0.f;
    }
    __syncthreads();
    const int c4 = (threadIdx.x % CPT) * 4;
    for (int rr = threadIdx.x / CPT; rr < TR; rr += RPP) {
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      for (int kk = 0; kk < D; ++kk) {
        const float x = sK[rr * (D + 1) + kk];
        const float4 pv = *reinterpret_cast<const float4*>(&sP[kk * D + c4]);
        a0 = fmaf(x, pv.x, a0); a1 = fmaf(x, pv.y, a1);
        a2 = fmaf(x, pv.z, a2); a3 = fmaf(x, pv.w, a3);
      }
      if (row0 + rr < S) {
        const float4 o = make_float4(a0, a1, a2, a3);
        if (out) *reinterpret_cast<float4*>(Ob + (size_t)(row0 + rr) * D + c4) = o;
        if (Lb && c4 < R) *reinterpret_cast<float4*>(Lb + (size_t)(row0 + rr) * R + c4) = o;
      }
    }
  }
}

static int blocks_per_group(long long groups, int tiles) {
  long long want = (1024 + groups - 1) / groups;  // aim for >= 1024 blocks in all
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  return (int)want;
}

// ============================================================================
// Cache append for one decode step: the new key of every (b, kv) is rotated
// into the basis and written at the sequence's position, with its value row
// and lead dims.  One block of 1024 threads per (b, kv): thread (c, js)
// sums k_new[j] P[kv][j][c] over the j-slice js (d / 8 terms, its P loads
// issued together), the eight slice sums of column c are added in order, and
// the row is rounded once.  Rows at other positions are not touched; a
// position outside [0, S) writes nothing.
// ============================================================================
template <typename T>
__global__ __launch_bounds__(1024) void append_kv_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new,
                                                         const T* __restrict__ P, const int32_t* __restrict__ pos,
                                                         T* __restrict__ K_rot, T* __restrict__ V,
                                                         T* __restrict__ K_lead, int R, int Hkv, int S, int d) {
  const int bk = blockIdx.x, b = bk / Hkv, kv = bk - b * Hkv;
  const int p = pos[b];
  if (p < 0 || p >= S) return;  // uniform over the block
  __shared__ float sk[128];
  __shared__ float sred[8][128];
  const int tid = threadIdx.x, c = tid % d, js = tid / d, J = d / 8;
  T pv[16];  // P[kv][js J + jj][c], clamped into the matrix (J <= 16)
  const T* Pc = P + (size_t)kv * d * d + c;
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) pv[jj] = Pc[(size_t)min(js * J + jj, d - 1) * d];
  if (tid < d) sk[tid] = to_f32(k_new[(size_t)bk * d + tid]);
  __syncthreads();
  if (js < 8) {
    float acc = 0.f;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
      if (jj < J) acc = fmaf(sk[js * J + jj], to_f32(pv[jj]), acc);
    sred[js][c] = acc;
  }
  __syncthreads();
  if (tid < d) {
    float v = sred[0][tid];
#pragma unroll
    for (int t = 1; t < 8; ++t) v += sred[t][tid];
    const size_t row = (size_t)bk * S + p;
    const T kr = from_f32<T>(v);
    K_rot[row * d + tid] = kr;
    V[row * d + tid] = v_new[(size_t)bk * d + tid];
    if (K_lead && tid < R) K_lead[row * R + tid] = kr;
  }
}

hipError_t launch_append_kv(const void* k_new, const void* v_new, const void* P, const int32_t* pos, void* K_rot,
                            void* V, void* K_lead, int R, int B, int Hkv, int S, int d, int dt, hipStream_t st) {
  const dim3 grid((unsigned)(B * Hkv)), block(1024);
  if (dt == 1)
    hipLaunchKernelGGL((append_kv_kernel<bf16_t>), grid, block, 0, st, static_cast<const bf16_t*>(k_new),
                       static_cast<const bf16_t*>(v_new), static_cast<const bf16_t*>(P), pos,
                       static_cast<bf16_t*>(K_rot), static_cast<bf16_t*>(V), static_cast<bf16_t*>(K_lead), R, Hkv,
                       S, d);
  else
    hipLaunchKernelGGL((append_kv_kernel<float>), grid, block, 0, st, static_cast<const float*>(k_new),
                       static_cast<const float*>(v_new), static_cast<const float*>(P), pos,
                       static_cast<float*>(K_rot), static_cast<float*>(V), static_cast<float*>(K_lead), R, Hkv, S,
                       d);
  return hipGetLastError();
}

hipError_t launch_project(const void* K, const void* P, void* K_rot, void* K_lead, int R, int B,
                          int Hkv, int S, int d, int dt, hipStream_t st) {
  const long long groups = (long long)B * Hkv;
  if (dt == 1) {
    const int tiles = (S + 127) / 128;
    const int bpb = blocks_per_group(groups, tiles);
    const dim3 grid((unsigned)(groups * bpb));
    const bf16_t* k = static_cast<const bf16_t*>(K);
    const bf16_t* pp = static_cast<const bf16_t*>(P);
    bf16_t* o = static_cast<bf16_t*>(K_rot);
    bf16_t* l = static_cast<bf16_t*>(K_lead);
    if (d == 128)
      hipLaunchKernelGGL((project_bf16_kernel<128>), grid, dim3(256), 0, st, k, pp, o, l, R, Hkv, S, tiles, bpb);
    else
      hipLaunchKernelGGL((project_bf16_kernel<64>), grid, dim3(256), 0, st, k, pp, o, l, R, Hkv, S, tiles, bpb);
  } else {
    const int tiles = (S + 63) / 64;
    const int bpb = blocks_per_group(groups, tiles);
    const dim3 grid((unsigned)(groups * bpb));
    const size_t lds = ((size_t)d * d + 64 * (d + 1)) * sizeof(float);
    const float* k = static_cast<const float*>(K);
    const float* pp = static_cast<const float*>(P);
    float* o = static_cast<float*>(K_rot);
    float* l = static_cast<float*>(K_lead);
    if (d == 128) {
      const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(&project_f32_kernel<128>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (ea != hipSuccess) return ea;
      hipLaunchKernelGGL((project_f32_kernel<128>), grid, dim3(256), lds, st, k, pp, o, l, R, Hkv, S, tiles, bpb);
    } else {
      hipLaunchKernelGGL((project_f32_kernel<64>), grid, dim3(256), lds, st, k, pp, o, l, R, Hkv, S, tiles, bpb);
    }
  }
  return hipGetLastError();
}

}  // namespace loki
