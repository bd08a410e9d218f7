// Host-side plan of a decode call (workspace layout, chunking) and the
// kernel launchers.  Shared by the C ABI and the kernel translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace loki {

constexpr int kMaxGroup = 16;        // largest supported Hq/Hkv
constexpr int kAttendMfmaTokens = 256;  // tokens per wave in the MFMA attention kernel
constexpr int kFusedThreads = 512;      // threads of the fused score+select kernel
constexpr int kFusedMaxS = 16384;       // fused path: a head's keys fit in LDS and in 512 x 32 registers
constexpr int kPairThreads = 1024;      // threads of the fused kernel for pairs of grouped heads
constexpr int kSelRegMaxT = 32;         // selection keeps up to 1024 x 32 keys of a head in registers
constexpr int kSelChunk = 16384;        // long heads: tokens per first-stage selection block
constexpr int kSplitMax = 16;           // most blocks sharing one head's selection + attention

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Raises a kernel's dynamic-LDS limit to at least `bytes` on the current
// device, calling the runtime only the first time a (kernel, device) pair
// needs a larger limit (a decode then makes no attribute call per launch).
hipError_t ensure_dynamic_lds(const void* fn, int bytes);

// Everything a decode-family launch needs, derived from the sizes alone.
struct DecodePlan {
  int B, Hq, Hkv, S, d, r, k, G, dt;  // dt: 0 fp32, 1 bf16
  int Sp;        // key row stride in the workspace: S rounded up to 64
  int W;         // bitmap words per query head: Sp / 32
  int SC, NSC;   // approximate-score kernel: tokens per block, blocks per (b,kv)
  int AC, NAC;   // attention kernel: tokens per block, blocks per (b,kv)
  int NSPL;      // selection + attention in one launch: blocks per query head
  // workspace: q_rot, its bf16 split, keys [row][Sp], per-score-chunk key
  // extremes [row][NSC] (uint2 min, max), selection masks [row][Sp/16] (used
  // when a row's keys do not fit in LDS), bitmap [row][W], attention partials
  size_t off_qrot, off_qsplit, off_keys, off_mm, off_masks, off_cidx, off_ckey, off_bitmap, off_part, bytes;
  // per query head: NSPL attention partials [row][NSPL][d + 2] and the count
  // of its blocks done [row] (cleared by the query rotation)
  size_t off_spart, off_scnt;
  // query-magnitude scoring: q_rot masked to each head's chosen dims, and its split
  size_t off_qrot_m, off_qsplit_m;
  // per-sequence lengths [B] on the device (each clamped into [1, S]), or
  // null: every sequence holds S tokens
  const int32_t* lens = nullptr;
};

// Fills `p` from the sizes; returns false if they are out of the supported range
// (the C ABI validates first, so this only guards internal misuse).
bool make_decode_plan(DecodePlan& p, int B, int Hq, int Hkv, int S, int d, int r, int k, int dt);

// Selection-only plan (loki_select_topk).
struct SelectPlan {
  int rows, S, Sp, W, k;
  int NMM;  // key-conversion blocks per row (one min / max pair each)
  size_t off_keys, off_mm, off_masks, off_cidx, off_ckey, off_bitmap, bytes;
};
bool make_select_plan(SelectPlan& p, int rows, int S, int k);

// ---- launchers: enqueue on `st`; return hipGetLastError() after the launches.
// q_rot in fp32 and, when qsplit is non-null, its three-way bf16 split as
// MFMA operands qsplit[row][part][d] (part 3 is zero).  The same launch sets
// zero[0..nzero) to 0 (the split attention's counters of this call).
hipError_t launch_qrot(const DecodePlan& p, const void* q, const void* P, float* qrot,
                       uint16_t* qsplit, hipStream_t st, uint32_t* zero = nullptr, int nzero = 0);
// Scores from `src` = K_rot (ld = d) or a lead-dims copy K_lead (ld = R >= r).
// With as_keys, `out` receives order-preserving keys and, when mm is not
// null, mm[row][chunk] the min / max key of each of the NSC score chunks.
hipError_t launch_scores(const DecodePlan& p, const void* src, int ld, const float* qrot,
                         const uint16_t* qsplit, void* out, bool as_keys, int out_stride,
                         uint2* mm, hipStream_t st);
// Top-k of each key row.  Rows longer than the register form
// (select_needs_minmax) also need mm[row][0..nmm), min / max pairs covering
// the row, and gmasks (rows * Sp / 16 words of scratch); else both may be null.
// Heads longer than the register form with k <= kSelChunk and a short enough
// candidate list are selected in two stages (per chunk, then over the chunk
// winners) and need candidate lists cidx / ckey of rows * select_chunked_ldc
// entries (0: not this path).
bool select_needs_minmax(int S);
size_t select_chunked_ldc(int S, int k);
hipError_t launch_select(int rows, int S, int Sp, int k, int W, const uint32_t* keys, const uint2* mm,
                         int nmm, uint32_t* gmasks, int32_t* idx, uint32_t* bitmap, hipStream_t st,
                         int32_t* cidx = nullptr, uint32_t* ckey = nullptr, const int32_t* lens = nullptr,
                         int Hq = 1);
// The query itself as fp32 and split (attention over unrotated keys).
hipError_t launch_qplain(const DecodePlan& p, const void* q, float* qf, uint16_t* qsplit, hipStream_t st);
// Query-magnitude dims: the r dims of largest |q_rot| per head; writes the
// masked q_rot and its split, and (when non-null) the dims ascending and the
// information retention loss per head.
hipError_t launch_qdims(const DecodePlan& p, const void* q, const float* qrot, float* qrot_m, uint16_t* qsplit_m,
                        int32_t* dims, float* info, int r, hipStream_t st);
hipError_t launch_scores_to_keys(const float* scores, uint32_t* keys, uint2* mm, int nmm, int rows,
                                 int S, int Sp, hipStream_t st);
hipError_t launch_idx_to_bitmap(const DecodePlan& p, const int32_t* idx, uint32_t* bitmap,
                                hipStream_t st);
// Attention then the partial merge; `mid` (may be null) is recorded between them.
hipError_t launch_attend(const DecodePlan& p, const void* K_rot, const void* V, const float* qrot,
                         const uint16_t* qsplit, const uint32_t* bitmap, float* part, void* out,
                         hipStream_t st, hipEvent_t mid = nullptr);
// K_rot = K P; when K_lead is non-null its rows also receive the leading R dims.
// MFMA paths (bf16 storage).
hipError_t launch_scores_mfma(const DecodePlan& p, const void* src, int ld, const uint16_t* qsplit,
                              void* out, bool as_keys, int out_stride, uint2* mm, hipStream_t st);
// Fused scores + top-k into idx / bitmap (bf16, S <= kFusedMaxS).
size_t score_select_lds_bytes(int Sp);
hipError_t launch_score_select(const DecodePlan& p, const void* src, int ld, const uint16_t* qsplit,
                               int32_t* idx, uint32_t* bitmap, hipStream_t st);
// Pairs of heads of a group in one kernel (bf16, G even, S <= kFusedMaxS).
bool score_select_pair_fits(const DecodePlan& p);
// The whole decode of pairs of heads of a group in one launch (bf16, G even,
// S <= kFusedMaxS, d 64 or 128): rotation, scores, selection into idx, and
// the exact attention of both heads over their kept tokens into out.  With
// plain, the exact stage takes the query itself against Kx = the unrotated
// keys (asymmetric index); else q P against Kx = K_rot.
hipError_t launch_decode_pair(const DecodePlan& p, const void* src, int ld, const void* q, const void* P,
                              const void* Kx, const void* V, void* out, int32_t* idx, bool plain, hipStream_t st);
// Selection and exact attention of each query head in one launch (bf16, d 64
// or 128): p.NSPL blocks per query head over its keys keys[row][0..S) (row
// stride ldk, S <= 32768), or, with cidx, over its chunk winners
// keys / cidx[row][0..S2) (row stride ldk); writes idx and out.  qsplit is
// the exact stage's split query.  With p.NSPL > 1, part and cnt are the
// plan's off_spart / off_scnt regions, cnt zero on entry (launch_qrot).
bool select_attend_fits(const DecodePlan& p);
hipError_t launch_select_attend(const DecodePlan& p, const uint32_t* keys, const int32_t* cidx, int ldk, int S2,
                                const uint16_t* qsplit, const void* Kx, const void* V, void* out, int32_t* idx,
                                float* part, uint32_t* cnt, hipStream_t st);
// Long heads (bf16): fused scores + the first selection stage, one block per
// (query head, chunk of kSelChunk tokens), into the candidate lists cidx /
// ckey (ldc words per row); then launch_select_merge finishes the selection.
bool score_select_chunk_fits(const DecodePlan& p);
hipError_t launch_score_select_chunk(const DecodePlan& p, const void* src, int ld, const uint16_t* qsplit,
                                     int32_t* cidx, uint32_t* ckey, int ldc, hipStream_t st);
hipError_t launch_select_merge(int rows, int S, int k, int W, int ldc, const uint32_t* ckey, const int32_t* cidx,
                               int32_t* idx, uint32_t* bitmap, const int32_t* lens, int Hq, hipStream_t st);
hipError_t launch_attend_mfma(const DecodePlan& p, const void* K_rot, const void* V,
                              const uint16_t* qsplit, const uint32_t* bitmap, float* part,
                              hipStream_t st);
// Cache append: rotated key, value and lead dims of one new token per (b, kv).
hipError_t launch_append_kv(const void* k_new, const void* v_new, const void* P, const int32_t* pos, void* K_rot,
                            void* V, void* K_lead, int R, int B, int Hkv, int S, int d, int dt, hipStream_t st);
hipError_t launch_project(const void* K, const void* P, void* K_rot, void* K_lead, int R, int B,
                          int Hkv, int S, int d, int dt, hipStream_t st);

// Memory-system reference kernels: a copy of `bytes` (a multiple of 16) and a
// streaming read that XORs every 32-bit word of src into *sink.
hipError_t launch_bench_copy(const void* src, void* dst, size_t bytes, hipStream_t st);
hipError_t launch_bench_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);

// Basis calibration (principal directions of the keys of each key head).
struct CalibPlan {
  int B, Hkv, S, d, dt;
  int N;           // key rows per head: B * S
  int rows, nblk;  // Gram kernel: rows per block, blocks per head
  // workspace: Gram partials [Hkv][nblk][d][d], Gram [Hkv][d][d], eigenvectors
  // [Hkv][d][d] (fp64); the eigensolver's rotation log [Hkv][rounds][d/2]
  // (c, s), rounds used per head (int), unsorted eigenvalues [Hkv][d]
  size_t off_part, off_C, off_V, off_log, off_nr, off_lam, bytes;
};
bool make_calib_plan(CalibPlan& p, int B, int Hkv, int S, int d, int dt);
// Gram partials, their sum, Jacobi eigensolver and output; when ev is non-null
// ev[0..3] are recorded before the Gram kernel, after it, after the sum and
// at the end.
hipError_t launch_calibrate(const CalibPlan& p, const void* K, void* P, double* eigvals, void* ws,
                            hipStream_t st, hipEvent_t* ev);

// Asymmetric scoring index calibration: Gram plans of the query samples
// ([N, Hq, 1, d]) and of the keys, and fp64 scratch matrices.
constexpr int kAsymMats = 12;
struct AsymPlan {
  CalibPlan qp, kp;
  int Hq, Hkv, G, d, r, dt, N;
  long long BS;  // key rows per head
  size_t off_part, off_Cqh, off_log, off_nr, off_lam, off_V2, off_mat[kAsymMats], bytes;
};
bool make_asym_plan(AsymPlan& p, int N, int Hq, int B, int Hkv, int S, int d, int r, int dt);
hipError_t launch_calibrate_asym(const AsymPlan& p, const void* q_samples, const void* K, void* A, void* Bm, void* ws,
                                 hipStream_t st);

}  // namespace loki
