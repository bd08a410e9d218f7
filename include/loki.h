/*
 * loki.h -- C ABI of the MI355X (gfx950) low-rank-key sparse decode-attention
 * library (libloki.so).
 *
 * The method (Loki: Low-rank Keys for Efficient Sparse Attention, abstract;
 * AQUA: Attention via QUery mAgnitudes..., related work "LoKi Attention"):
 * cached keys live in an offline orthonormal basis P (K_rot = K P); at each
 * decode step every query head is rotated into the same basis, scores all
 * cached tokens using only the leading r rotated dimensions, keeps its k
 * best tokens for this step (nothing is evicted), and runs exact softmax
 * attention over the full keys and values of just those tokens.  Decode
 * attention itself is eqs. 1-5 of the AQUA page's preliminaries: S = q K^T,
 * A = softmax(S / sqrt(d_head)), c = A V.
 *
 * Entry points, in the order of a deployment:
 *   loki_calibrate_pca               the basis P from sampled keys (offline)
 *   loki_project_keys[_lead]         the rotated cache K P (and its lead dims)
 *   loki_append_kv                   one new token per sequence, in place
 *   loki_decode / _lead / _varlen    one decode step (full or ragged batch)
 *   loki_decode_aqua                 the same with per-query magnitude dims
 *   loki_calibrate_asym, loki_decode_asym
 *                                    an asymmetric (query side A, key side B)
 *                                    scoring index, its calibration and decode
 *   loki_scores, loki_select_topk, loki_attend
 *                                    the decode stages alone
 *   *_profiled                       the same work with stage events
 *   loki_bench_copy, loki_bench_read memory-system reference kernels
 *                                    (measurement; not part of the method)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers (HIP global memory) owned by the
 *    caller; the library never allocates, frees or retains them.  They must
 *    be 16-byte aligned.
 *  - Layouts are contiguous and row-major:
 *      q, out  [B, Hq, d]          K, K_rot, V  [B, Hkv, S, d]
 *      P       [Hkv, d, d]         (K_rot[b,kv] = K[b,kv] * P[kv])
 *      idx     [B, Hq, k] int32    scores  [B, Hq, S] fp32
 *    q, P, K, K_rot, V and out share one storage dtype (fp32 or bf16).
 *  - Grouped-query attention: query head h reads key/value head h / (Hq/Hkv)
 *    (contiguous groups); P belongs to the key/value head.
 *  - All arithmetic accumulates in fp32; the rotated query is kept in fp32
 *    and never rounded to the storage dtype; outputs are rounded once
 *    (round-to-nearest-even for bf16).
 *  - The kept set of a query head is its k largest approximate scores; ties
 *    go to the lower token index; idx lists the kept tokens in ascending
 *    order.  Results are deterministic (bit-identical across runs).
 *  - Every call validates all scalar arguments and pointer alignment on the
 *    host BEFORE any HIP call and returns a status; nothing is enqueued when
 *    the status is not LOKI_OK.  Work is enqueued asynchronously on `stream`
 *    (0 = the null stream); buffers must stay alive until the stream reaches
 *    it.  A failed launch returns LOKI_ERR_HIP.  The library holds no
 *    per-call state, so calls on different streams may run concurrently as
 *    long as they use different workspaces.
 *  - Non-finite inputs (NaN, Inf) are not checked and give unspecified
 *    results.
 *  - Supported: d in {64, 128}; Hq/Hkv <= 16; dtype fp32 or bf16;
 *    1 <= r <= d; 1 <= k <= S <= 2^24; B*Hq <= 65535.
 */
#ifndef LOKI_H
#define LOKI_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOKI_ABI_VERSION 1

typedef enum {
  LOKI_OK = 0,
  LOKI_ERR_NULL = 1,        /* a required pointer is NULL                       */
  LOKI_ERR_SHAPE = 2,       /* a size is < 1, too large, or Hq % Hkv != 0       */
  LOKI_ERR_RANGE = 3,       /* r outside [1, d] or k outside [1, S]             */
  LOKI_ERR_DTYPE = 4,       /* unknown dtype code                               */
  LOKI_ERR_ALIGN = 5,       /* a tensor pointer is not 16-byte aligned          */
  LOKI_ERR_WORKSPACE = 6,   /* workspace smaller than the size function returns */
  LOKI_ERR_UNSUPPORTED = 7, /* valid but not implemented (d, Hq/Hkv)            */
  LOKI_ERR_HIP = 8,         /* a HIP runtime call or kernel launch failed       */
  LOKI_ERR_INTERNAL = 9     /* unexpected internal failure                      */
} loki_status;

/* Storage dtype.  A C caller may pass any integer: C++ gives the enum a
 * fixed 32-bit representation, so an unknown code is a value the library can
 * test (LOKI_ERR_DTYPE) rather than an out-of-range enum. */
#ifdef __cplusplus
typedef enum : int32_t { LOKI_F32 = 0, LOKI_BF16 = 1 } loki_dtype;
#else
typedef enum { LOKI_F32 = 0, LOKI_BF16 = 1 } loki_dtype;
#endif

/* LOKI_ABI_VERSION of the built library. */
int loki_abi_version(void);

/* Static description of a status code (never NULL). */
const char* loki_status_str(int status);

/*
 * Key projection into the offline basis: K_rot[b,kv] = K[b,kv] * P[kv]
 * (row-vector convention v_hat = v P of the AQUA page's information-
 * retention paragraph; with an orthogonal P it preserves every q.k, AQUA
 * appendix on the lossless rotation).  Used when the cache is written
 * (prefill, or a decode step's new key with S = 1).
 *   K      [B, Hkv, S, d]  input keys
 *   P      [Hkv, d, d]     basis per key/value head
 *   K_rot  [B, Hkv, S, d]  output; must not overlap K or P
 * bf16 runs on MFMA matrix cores with fp32 accumulation and one RNE
 * rounding; fp32 runs on the vector ALUs.  No workspace.
 */
loki_status loki_project_keys(const void* K, const void* P, void* K_rot,
                              int32_t B, int32_t Hkv, int32_t S, int32_t d,
                              loki_dtype dt, hipStream_t stream);

/*
 * As loki_project_keys, and in the same pass also writes the leading R
 * rotated dims of every cached key into a separate dense array:
 *   K_lead [B, Hkv, S, R]   K_lead[b,kv,j,c] = K_rot[b,kv,j,c] for c < R
 * K_rot may be NULL: then only K_lead is written (a key index K B for
 * loki_decode_asym, with P = B).
 * K_lead is a second copy of data K_rot already holds (R/d of the key cache
 * in extra memory).  It lets the approximate-score stage of
 * loki_decode_lead stream R*elem bytes per token contiguously instead of a
 * short prefix of every d-wide row, which on HBM costs a full 128-byte line
 * per token whenever R*elem < 128.
 * R: 1 <= R <= d (else LOKI_ERR_RANGE) and R*elem a multiple of 16 bytes
 * (else LOKI_ERR_UNSUPPORTED).
 */
loki_status loki_project_keys_lead(const void* K, const void* P, void* K_rot, void* K_lead,
                                   int32_t R, int32_t B, int32_t Hkv, int32_t S, int32_t d,
                                   loki_dtype dt, hipStream_t stream);

/*
 * Cache append for one decode step, the step before loki_decode in a decode
 * loop (the AQUA page's preliminaries, eqs. 1-2: the new token's key and
 * value join the cache before the scores; the Loki page keeps the cache in
 * the rotated basis).  For every (b, kv) whose position is inside the cache:
 *   K_rot[b,kv,pos[b],:]    = k_new[b,kv,:] P[kv]   (fp32 accumulation, one rounding)
 *   V[b,kv,pos[b],:]        = v_new[b,kv,:]
 *   K_lead[b,kv,pos[b],:R]  = the leading R dims of that K_rot row (if K_lead)
 *   k_new, v_new [B, Hkv, d]; P [Hkv, d, d]; K_rot, V [B, Hkv, S, d];
 *   K_lead [B, Hkv, S, R] or NULL (then R is ignored; else R as for
 *   loki_project_keys_lead).
 *   pos    DEVICE array of B int32 positions, one per sequence, so sequences
 *          of different lengths each append at their own end.  A position
 *          outside [0, S) writes nothing for that sequence (it is read on
 *          the device, so it cannot be reported as an error).
 * No other cache row is touched.  The rotated row equals loki_project_keys's
 * up to the order of the fp32 additions.  No workspace.
 */
loki_status loki_append_kv(const void* k_new, const void* v_new, const void* P, const int32_t* pos,
                           void* K_rot, void* V, void* K_lead, int32_t R,
                           int32_t B, int32_t Hkv, int32_t S, int32_t d, loki_dtype dt,
                           hipStream_t stream);

/*
 * Bytes of device workspace needed by loki_decode, loki_decode_lead, loki_scores and
 * loki_attend for these sizes (0 if the sizes are invalid).  The same
 * workspace may be reused by successive calls on one stream.
 */
size_t loki_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t S,
                                   int32_t d, int32_t r, int32_t k, loki_dtype dt);

/*
 * One Loki decode step for every (batch, query head):
 *   q_rot = q P[kv]                                   (fp32, full d)
 *   s_j   = sum_{c<r} q_rot[c] K_rot[b,kv,j,c]        (all S cached tokens)
 *   idx   = the k tokens with the largest s_j (ties -> lower index), ascending
 *   e_j   = q_rot . K_rot[b,kv,j,:] / sqrt(d),  j in idx
 *   out   = sum_{j in idx} softmax(e)_j V[b,kv,j,:]
 * Every cached token is eligible (no causal mask); V is not rotated.
 *   q [B,Hq,d], P [Hkv,d,d], K_rot [B,Hkv,S,d], V [B,Hkv,S,d]  inputs
 *   out [B,Hq,d] (dtype dt), idx [B,Hq,k] int32                 outputs
 *   workspace: device buffer of >= loki_decode_workspace_bytes(...) bytes,
 *              owned by the caller, contents need no initialisation.
 */
loki_status loki_decode(const void* q, const void* P, const void* K_rot, const void* V,
                        void* out, int32_t* idx,
                        int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d,
                        int32_t r, int32_t k, loki_dtype dt,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * loki_decode with the approximate scores read from the lead-dims copy
 * K_lead [B,Hkv,S,R] (see loki_project_keys_lead) instead of from K_rot's
 * rows.  Needs r <= R (else LOKI_ERR_RANGE); R constraints as for
 * loki_project_keys_lead.  K_lead must hold the leading R dims of K_rot
 * (results are those of loki_decode on the same K_rot).  Exact attention
 * still reads full K_rot and V rows.  Same workspace as loki_decode.
 */
loki_status loki_decode_lead(const void* q, const void* P, const void* K_rot, const void* K_lead,
                             int32_t R, const void* V, void* out, int32_t* idx,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d,
                             int32_t r, int32_t k, loki_dtype dt,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * loki_decode over a ragged batch: sequence b holds only its first lens[b]
 * cached tokens (K_rot / K_lead / V rows past that are unused capacity and
 * are neither read for scores nor kept).  Each sequence is a decode over its
 * own prefix: its query heads keep their min(k, lens[b]) best tokens, and
 * idx rows of sequences shorter than k end with -1 entries.
 *   lens  DEVICE array of B int32 lengths, each clamped into [1, S] (read on
 *         the device, so out-of-range values cannot be reported as errors).
 *   K_lead may be NULL (scores from K_rot's rows; R ignored), else as for
 *   loki_decode_lead.  S is the cache capacity; 1 <= k <= S as for
 *   loki_decode.  Other arguments, workspace and errors as for
 *   loki_decode_lead.  With every lens[b] = S the results are those of
 *   loki_decode_lead (or loki_decode).
 */
loki_status loki_decode_varlen(const void* q, const void* P, const void* K_rot, const void* K_lead,
                               int32_t R, const void* V, const int32_t* lens, void* out, int32_t* idx,
                               int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d,
                               int32_t r, int32_t k, loki_dtype dt,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Instrumented decode for measurement: exactly the work of loki_decode
 * (K_lead == NULL) or loki_decode_lead (lens == NULL) or loki_decode_varlen
 * (lens given), plus hipEventRecord(events[i], stream) at the stage
 * boundaries:
 *   [0] before the query rotation    [1] after it
 *   [2] after the approximate scores [3] after the top-k selection
 *   [4] after exact attention        [5] after the partial merge (the end)
 * events: host array of 6 events created by the caller (LOKI_ERR_NULL if
 * any is NULL).  Other arguments and errors as for loki_decode_lead.
 */
loki_status loki_decode_profiled(const void* q, const void* P, const void* K_rot, const void* K_lead,
                                 int32_t R, const void* V, const int32_t* lens, void* out, int32_t* idx,
                                 int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d,
                                 int32_t r, int32_t k, loki_dtype dt,
                                 void* workspace, size_t workspace_bytes,
                                 hipEvent_t* events, hipStream_t stream);

/*
 * The approximate-score stage alone: scores[b,h,j] = s_j as defined for
 * loki_decode (fp32, unscaled), by the same kernels that loki_decode uses.
 * Workspace as for loki_decode with the same sizes (k = 1 may be passed).
 */
loki_status loki_scores(const void* q, const void* P, const void* K_rot, float* scores,
                        int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d,
                        int32_t r, loki_dtype dt,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace needed by loki_select_topk. */
size_t loki_select_workspace_bytes(int32_t rows, int32_t S, int32_t k);

/*
 * The selection stage alone on caller-given fp32 scores [rows, S]:
 * idx[row] = the k largest scores of the row (ties -> lower index; -0.0
 * equals +0.0), ascending, by the same selection kernel as loki_decode.
 */
loki_status loki_select_topk(const float* scores, int32_t* idx, int32_t rows, int32_t S,
                             int32_t k, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * The exact-attention stage alone over a caller-given kept set idx
 * [B,Hq,k] (int32): out = sum_{j in idx} softmax(e)_j V[b,kv,j,:] with e as
 * for loki_decode, by the same kernels.  Entries outside [0, S) are ignored
 * and repeated entries count once.  Workspace as for loki_decode.
 */
loki_status loki_attend(const void* q, const void* P, const void* K_rot, const void* V,
                        const int32_t* idx, void* out,
                        int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t k,
                        loki_dtype dt, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * Decode step with query-magnitude dimensions for the approximate scores
 * (AQUA page, online phase: the dims kept for the approximate scores are
 * those where the rotated query is largest in magnitude; AQUA page,
 * information-retention paragraph for L_info).  As loki_decode, except that
 * for each query head the approximate score of token j is
 *   s_j = sum_{c in I_h} q_rot[b,h,c] * K_rot[b,kv,j,c],
 *   I_h = the r dims c of largest |q_rot[b,h,c]| (ties -> lower c),
 * computed in fp32 from the fp32 q_rot (decisions on |q_rot| in fp32); the
 * kept tokens and the exact attention over them are as in loki_decode.
 *   lens       DEVICE [B] int32 per-sequence lengths as in loki_decode_varlen,
 *              or NULL (every sequence holds S tokens).
 *   dims       [B, Hq, r] int32 output: I_h ascending, or NULL.
 *   info_loss  [B, Hq] fp32 output: | ||q|| - ||q_rot[I_h]|| | / ||q|| (0 for a
 *              zero query), or NULL.  dims and info_loss 4-byte aligned.
 * The score stage reads every rotated key row in full (the dims differ per
 * head and step), so no lead-dims copy applies.  Sizes, ranges, workspace
 * (loki_decode_workspace_bytes) and errors as for loki_decode.
 */
loki_status loki_decode_aqua(const void* q, const void* P, const void* K_rot, const void* V,
                             const int32_t* lens, void* out, int32_t* idx, int32_t* dims, float* info_loss,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t r, int32_t k,
                             loki_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * loki_decode_aqua plus hipEventRecord(events[i], stream) at the stage
 * boundaries, as loki_decode_profiled: [0] start, [1] after the rotation and
 * the dims, [2] after the scores, [3] after the selection, [4] after the exact
 * attention, [5] end.  events must hold 6 created events (else LOKI_ERR_NULL).
 */
loki_status loki_decode_aqua_profiled(const void* q, const void* P, const void* K_rot, const void* V,
                                      const int32_t* lens, void* out, int32_t* idx, int32_t* dims,
                                      float* info_loss, int32_t B, int32_t Hq, int32_t Hkv, int32_t S,
                                      int32_t d, int32_t r, int32_t k, loki_dtype dt, void* workspace,
                                      size_t workspace_bytes, hipEvent_t* events, hipStream_t stream);

/*
 * Decode step with an asymmetric low-rank scoring index (page "SAKI:
 * Score-Aware Low-Rank Key Indexing with Random-Matrix Noise Correction for
 * KV Retrieval", abstract: approximate scores (q A_r) . (k B_r) with a
 * query-side and a key-side projection).  For each query head h of key head kv:
 *   s_j = sum_{c<r} (q[b,h] A[kv])[c] * K_idx[b,kv,j,c]
 * (fp32 accumulation, the query-side product as for q_rot), the k largest
 * s_j kept (ties -> lower index, idx ascending), and exact attention over
 * them with the query and keys themselves:
 *   out[b,h] = sum_{j in idx} softmax_j(q[b,h] . K[b,kv,j] / sqrt(d)) V[b,kv,j].
 *   A      [Hkv, d, d] in dt: the query-side projection in its first r
 *          columns (the other columns are not used);
 *   K_idx  [B, Hkv, S, R] in dt, r <= R <= d, R*elem a multiple of 16: the key
 *          index K B (loki_project_keys_lead with K_rot = NULL writes it);
 *   K, V   [B, Hkv, S, d] the keys (not rotated) and values;
 *   lens   DEVICE [B] int32 per-sequence lengths or NULL, as in loki_decode_varlen.
 * Other arguments, workspace (loki_decode_workspace_bytes) and errors as for
 * loki_decode_lead (K_idx NULL -> LOKI_ERR_NULL).
 */
loki_status loki_decode_asym(const void* q, const void* A, const void* K_idx, int32_t R, const void* K,
                             const void* V, const int32_t* lens, void* out, int32_t* idx, int32_t B,
                             int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t r, int32_t k,
                             loki_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* loki_decode_asym plus the six stage events of loki_decode_profiled. */
loki_status loki_decode_asym_profiled(const void* q, const void* A, const void* K_idx, int32_t R, const void* K,
                                      const void* V, const int32_t* lens, void* out, int32_t* idx, int32_t B,
                                      int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t r, int32_t k,
                                      loki_dtype dt, void* workspace, size_t workspace_bytes,
                                      hipEvent_t* events, hipStream_t stream);

/*
 * Offline calibration of the basis P, the step that produces the P every
 * other entry point takes (AQUA page, appendix on the SVD: the principal
 * directions of a key matrix A are the right singular vectors of A, i.e. the
 * eigenvectors of A^T A; the Loki page keeps the leading ones; AQUA's related
 * work: the matrix is computed offline).  For each key/value head kv, A is
 * the [B*S, d] matrix of the key rows of all batch elements of that head
 * (uncentred), and
 *   P[kv][:, c]     = the eigenvector of A^T A with the c-th largest
 *                     eigenvalue, scaled by +-1 so that its entry of largest
 *                     magnitude (the first such, on exact ties) is positive;
 *                     equal eigenvalues keep the eigensolver's order;
 *   eigvals[kv][c]  = that eigenvalue (fp64), if eigvals is not NULL.
 *   K       [B, Hkv, S, d] keys in the original basis (the cache layout of
 *           loki_project_keys), dt = LOKI_F32 or LOKI_BF16;
 *   P       [Hkv, d, d] output in dt (fp64 result rounded once, to nearest);
 *   eigvals [Hkv, d] fp64 output or NULL (8-byte aligned).
 * The Gram matrix is accumulated in fp64 (bf16 keys: exact products summed
 * in fp32 over 256 rows, then in fp64; fp32 keys: exact products, fp64
 * sums) and diagonalised by cyclic Jacobi in fp64.  When A has rank below
 * d, the null-space columns are some orthonormal completion.
 * Sizes: B, Hkv, S >= 1 with B*S < 2^31 (else LOKI_ERR_SHAPE); d in {64, 128}
 * (else LOKI_ERR_UNSUPPORTED).  K and P 16-byte aligned.  Workspace of
 * loki_calibrate_workspace_bytes(B, Hkv, S, d) bytes, 16-byte aligned.
 */
size_t loki_calibrate_workspace_bytes(int32_t B, int32_t Hkv, int32_t S, int32_t d);
loki_status loki_calibrate_pca(const void* K, void* P, double* eigvals, int32_t B, int32_t Hkv,
                               int32_t S, int32_t d, loki_dtype dt, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * loki_calibrate_pca plus hipEventRecord(events[i], stream) at the stage
 * boundaries: [0] before the Gram kernel, [1] after it, [2] after the sum of
 * the partials, [3] after the eigensolver and output (the end).  events must
 * hold 4 created events (LOKI_ERR_NULL otherwise).
 */
loki_status loki_calibrate_pca_profiled(const void* K, void* P, double* eigvals, int32_t B, int32_t Hkv,
                                        int32_t S, int32_t d, loki_dtype dt, void* workspace,
                                        size_t workspace_bytes, hipEvent_t* events, hipStream_t stream);

/*
 * Calibration of the asymmetric scoring index taken by loki_decode_asym
 * (page "SAKI: Score-Aware Low-Rank Key Indexing with Random-Matrix Noise
 * Correction for KV Retrieval", abstract: the rank-r query-side and
 * key-side factors that minimise the score error weighted by the query and
 * key second moments come from one SVD, written out below).  Per key/value head kv, with
 *   Cq = mean of q^T q over the query samples of the heads of kv's group,
 *   Ck = mean of k^T k over the key rows of all batch elements of kv,
 *   W  = Cq^{1/2} Ck^{1/2} = U S V^T,
 * the factors minimising || Cq^{1/2} (I - A_r B_r^T) Ck^{1/2} ||_F are
 *   A_r = Cq^{-1/2} U_r S_r^{1/2},  B_r = Ck^{-1/2} V_r S_r^{1/2}
 * (pseudo-inverse roots: eigenvalues below 1e-12 of the largest count as
 * zero).  Written as A [Hkv, d, d] and Bm [Hkv, d, d] in dt with the factors
 * in the first r columns and zeros after (the layout loki_decode_asym and
 * loki_project_keys_lead take).  The columns are unique up to a common sign
 * per column pair (and rotations within equal singular values); A_r B_r^T is
 * unique when S_r > S_{r+1}.  All arithmetic in fp64 (Gram matrices as in
 * loki_calibrate_pca, Jacobi eigendecompositions).
 *   q_samples [N, Hq, d] query samples in dt;  K [B, Hkv, S, d] keys in dt.
 * Sizes: N, Hq, B, Hkv, S >= 1, Hq % Hkv == 0, B*S < 2^31 (LOKI_ERR_SHAPE);
 * d in {64, 128} (LOKI_ERR_UNSUPPORTED); 1 <= r <= d (LOKI_ERR_RANGE).
 * Workspace of loki_calibrate_asym_workspace_bytes bytes.
 */
size_t loki_calibrate_asym_workspace_bytes(int32_t N, int32_t Hq, int32_t B, int32_t Hkv, int32_t S,
                                          int32_t d, int32_t r);
loki_status loki_calibrate_asym(const void* q_samples, const void* K, void* A, void* Bm, int32_t N,
                                int32_t Hq, int32_t B, int32_t Hkv, int32_t S, int32_t d, int32_t r,
                                loki_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): loki_decode_lead (K_lead may be NULL: then loki_decode) with
 * the workspace taken from a fixed device array inside the library,
 * LOKI_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs on
 * holds until the process ends.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).  Sizes whose workspace
 * (loki_decode_workspace_bytes) exceeds LOKI_NOALLOC_SCRATCH_BYTES return
 * LOKI_ERR_WORKSPACE; everything else (arguments, outputs, errors) is as
 * for loki_decode_lead.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (concurrent streams, or host threads) race and
 * give undefined results; calls ordered on one stream are safe.  The array
 * keeps the last call's contents; no decode reads scratch it has not
 * written in the same call.
 */
#define LOKI_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
loki_status loki_decode_noalloc(const void* q, const void* P, const void* K_rot, const void* K_lead, int32_t R,
                                const void* V, void* out, int32_t* idx, int32_t B, int32_t Hq, int32_t Hkv,
                                int32_t S, int32_t d, int32_t r, int32_t k, loki_dtype dt, hipStream_t stream);

/*
 * Memory-system reference kernels (measurement only; no step of the
 * method).  They are the reference points of the decode's HBM figures: the
 * rate a pure stream reaches on this part, and a kernel of known bytes that
 * scales the hardware traffic counters.
 *   loki_bench_copy: dst[0..bytes) = src[0..bytes)  (one read, one write of
 *                    every byte; the ranges must not overlap)
 *   loki_bench_read: reads src[0..bytes) once and XORs every 32-bit word of it
 *                    into *sink (a DEVICE uint32 the caller initialises; the
 *                    XOR keeps every load live)
 * bytes must be a multiple of 16 (LOKI_ERR_SHAPE), src / dst 16-byte aligned
 * (LOKI_ERR_ALIGN), sink 4-byte aligned, pointers non-NULL when bytes > 0
 * (LOKI_ERR_NULL).  Asynchronous on `stream`; no workspace.
 */
loki_status loki_bench_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
loki_status loki_bench_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LOKI_H */
