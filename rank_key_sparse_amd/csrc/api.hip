// C ABI of libloki: argument validation (host only, before any HIP call),
// workspace carving, and the launch sequence of each entry point.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/loki.h"
#include "internal.h"

using namespace loki;

namespace loki {

hipError_t ensure_dynamic_lds(const void* fn, int bytes) {
  struct Entry {
    const void* fn;
    int dev, bytes;
  };
  static std::mutex mu;
  static std::vector<Entry> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (Entry& x : done)
    if (x.fn == fn && x.dev == dev) {
      if (x.bytes >= bytes) return hipSuccess;
      if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) == hipSuccess)
        x.bytes = bytes;
      return e;
    }
  if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) == hipSuccess)
    done.push_back(Entry{fn, dev, bytes});
  return e;
}

}  // namespace loki

namespace {

constexpr int64_t kMaxS = int64_t(1) << 24;
constexpr int64_t kMaxRows = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

loki_status check_dtype(loki_dtype dt) {
  return (dt == LOKI_F32 || dt == LOKI_BF16) ? LOKI_OK : LOKI_ERR_DTYPE;
}

// Sizes shared by the decode family.
loki_status check_sizes(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || d < 1) return LOKI_ERR_SHAPE;
  if (Hq % Hkv != 0) return LOKI_ERR_SHAPE;
  if ((int64_t)S > kMaxS || (int64_t)B * Hq > kMaxRows) return LOKI_ERR_SHAPE;
  if (d != 64 && d != 128) return LOKI_ERR_UNSUPPORTED;
  if (Hq / Hkv > kMaxGroup) return LOKI_ERR_UNSUPPORTED;
  return LOKI_OK;
}

loki_status check_workspace(void* ws, size_t have, size_t need) {
  if (have < need) return LOKI_ERR_WORKSPACE;
  if (need > 0 && ws == nullptr) return LOKI_ERR_NULL;
  if (!aligned16(ws)) return LOKI_ERR_ALIGN;
  return LOKI_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// LOKI_DEBUG=1 in the environment (read once): after every launch step the
// entry point waits for its stream and takes the runtime's last error, so a
// kernel that faults is reported as LOKI_ERR_HIP by the call that launched it
// (slow; not for use under graph capture, where waiting is not allowed).
bool debug_mode() {
  static const bool on = [] {
    const char* v = getenv("LOKI_DEBUG");
    return v && v[0] && !(v[0] == '0' && v[1] == 0);
  }();
  return on;
}

// The status of a launch step (one or more kernels or an event record).
loki_status after_launch(hipError_t e, hipStream_t st) {
  if (e != hipSuccess) return LOKI_ERR_HIP;
  if (debug_mode()) {
    e = hipStreamSynchronize(st);
    const hipError_t last = hipGetLastError();
    if (e != hipSuccess || last != hipSuccess) return LOKI_ERR_HIP;
  }
  return LOKI_OK;
}

#define LOKI_TRY(expr)                          \
  do {                                          \
    const loki_status s_ = (expr);              \
    if (s_ != LOKI_OK) return s_;               \
  } while (0)

#define LOKI_HIP(expr)                                  \
  do {                                                  \
    const loki_status s_ = after_launch((expr), stream); \
    if (s_ != LOKI_OK) return s_;                       \
  } while (0)

}  // namespace

extern "C" {

int loki_abi_version(void) { return LOKI_ABI_VERSION; }

const char* loki_status_str(int s) {
  switch (s) {
    case LOKI_OK: return "ok";
    case LOKI_ERR_NULL: return "a required pointer is NULL";
    case LOKI_ERR_SHAPE: return "invalid sizes (a size < 1, too large, or Hq not a multiple of Hkv)";
    case LOKI_ERR_RANGE: return "r must be in [1, d] and k in [1, S]";
    case LOKI_ERR_DTYPE: return "unknown dtype";
    case LOKI_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case LOKI_ERR_WORKSPACE: return "workspace too small";
    case LOKI_ERR_UNSUPPORTED: return "unsupported configuration (d must be 64 or 128, Hq/Hkv <= 16)";
    case LOKI_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case LOKI_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

static loki_status check_project(const void* K, const void* P, void* K_rot, int32_t B, int32_t Hkv,
                          int32_t S, int32_t d, loki_dtype dt) {
  LOKI_TRY(check_dtype(dt));
  if (!K || !P || !K_rot) return LOKI_ERR_NULL;
  if (B < 1 || Hkv < 1 || S < 1 || d < 1) return LOKI_ERR_SHAPE;
  if ((int64_t)B * Hkv > kMaxRows || (int64_t)S > kMaxS) return LOKI_ERR_SHAPE;
  if (d != 64 && d != 128) return LOKI_ERR_UNSUPPORTED;
  if (!aligned16(K) || !aligned16(P) || !aligned16(K_rot)) return LOKI_ERR_ALIGN;
  return LOKI_OK;
}

// R of a lead-dims copy; r = 0 skips the r <= R check.
static loki_status check_lead(const void* K_lead, int32_t R, int32_t d, int32_t r, loki_dtype dt) {
  if (!K_lead) return LOKI_ERR_NULL;
  if (R < 1 || R > d || r > R) return LOKI_ERR_RANGE;
  if ((R * (dt == LOKI_F32 ? 4 : 2)) % 16 != 0) return LOKI_ERR_UNSUPPORTED;
  if (!aligned16(K_lead)) return LOKI_ERR_ALIGN;
  return LOKI_OK;
}

loki_status loki_project_keys(const void* K, const void* P, void* K_rot, int32_t B, int32_t Hkv,
                              int32_t S, int32_t d, loki_dtype dt, hipStream_t stream) {
  try {
    LOKI_TRY(check_project(K, P, K_rot, B, Hkv, S, d, dt));
    return after_launch(launch_project(K, P, K_rot, nullptr, 0, B, Hkv, S, d, (int)dt, stream), stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_project_keys_lead(const void* K, const void* P, void* K_rot, void* K_lead,
                                   int32_t R, int32_t B, int32_t Hkv, int32_t S, int32_t d,
                                   loki_dtype dt, hipStream_t stream) {
  try {
    // K_rot may be NULL (only the lead dims wanted); K_lead stands in for its checks
    LOKI_TRY(check_project(K, P, K_rot ? K_rot : K_lead, B, Hkv, S, d, dt));
    LOKI_TRY(check_lead(K_lead, R, d, 0, dt));
    return after_launch(launch_project(K, P, K_rot, K_lead, R, B, Hkv, S, d, (int)dt, stream), stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_append_kv(const void* k_new, const void* v_new, const void* P, const int32_t* pos,
                           void* K_rot, void* V, void* K_lead, int32_t R, int32_t B, int32_t Hkv, int32_t S,
                           int32_t d, loki_dtype dt, hipStream_t stream) {
  try {
    LOKI_TRY(check_project(k_new, P, K_rot, B, Hkv, S, d, dt));
    if (!v_new || !pos || !V) return LOKI_ERR_NULL;
    if (!aligned16(v_new) || !aligned16(V)) return LOKI_ERR_ALIGN;
    if (K_lead) LOKI_TRY(check_lead(K_lead, R, d, 0, dt));
    return after_launch(launch_append_kv(k_new, v_new, P, pos, K_rot, V, K_lead, K_lead ? R : 0, B, Hkv, S, d, (int)dt,
                                     stream), stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

size_t loki_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d,
                                   int32_t r, int32_t k, loki_dtype dt) {
  if (check_dtype(dt) != LOKI_OK || check_sizes(B, Hq, Hkv, S, d) != LOKI_OK) return 0;
  if (r < 1 || r > d || k < 1 || k > S) return 0;
  DecodePlan p;
  if (!make_decode_plan(p, B, Hq, Hkv, S, d, r, k, (int)dt)) return 0;
  return p.bytes;
}

static loki_status decode_impl(const void* q, const void* P, const void* K_rot, const void* K_lead,
                               int32_t R, const void* V, void* out, int32_t* idx, int32_t B,
                               int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t r, int32_t k,
                               loki_dtype dt, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, hipEvent_t* ev = nullptr,
                               const int32_t* lens = nullptr, int aqua_r = 0, int32_t* dims = nullptr,
                               float* info = nullptr, bool plain_attn = false) {
  LOKI_TRY(check_dtype(dt));
  if (!q || !P || !K_rot || !V || !out || !idx) return LOKI_ERR_NULL;
  LOKI_TRY(check_sizes(B, Hq, Hkv, S, d));
  if (r < 1 || r > d || k < 1 || k > S) return LOKI_ERR_RANGE;
  if (!aligned16(q) || !aligned16(P) || !aligned16(K_rot) || !aligned16(V) || !aligned16(out) ||
      !aligned16(idx))
    return LOKI_ERR_ALIGN;
  if (K_lead) LOKI_TRY(check_lead(K_lead, R, d, r, dt));
  DecodePlan p;
  if (!make_decode_plan(p, B, Hq, Hkv, S, d, r, k, (int)dt)) return LOKI_ERR_INTERNAL;
  LOKI_TRY(check_workspace(workspace, workspace_bytes, p.bytes));
  p.lens = lens;
  float* qrot = at<float>(workspace, p.off_qrot);
  uint16_t* qsplit = at<uint16_t>(workspace, p.off_qsplit);
  uint32_t* keys = at<uint32_t>(workspace, p.off_keys);
  uint32_t* bitmap = at<uint32_t>(workspace, p.off_bitmap);
  float* part = at<float>(workspace, p.off_part);
  const void* src = K_lead ? K_lead : K_rot;
  int ld = K_lead ? R : d;
  // bf16, a head's keys small enough for LDS and enough blocks to fill the
  // chip: scores and selection in one kernel, one block per query head when
  // each query head has its own key head, one block per pair of query heads
  // of a group otherwise (that kernel also rotates its queries, so the
  // rotation stage is empty); else two kernels with the keys in the workspace
  // query-magnitude dims (aqua_r > 0): each head scores with its own dims of
  // the full rotated rows, so the two-kernel path with a masked query
  const bool aqua = aqua_r > 0;
  const bool fused = !aqua && dt == LOKI_BF16 && Hq == Hkv && S <= kFusedMaxS && (int64_t)B * Hq >= 256;
  const bool pair = !aqua && !fused && score_select_pair_fits(p) && (int64_t)B * Hq >= 2 * 256;
  // long heads selected in two stages: the first stage fused with the scores
  // (one block per query head and 16384-token chunk) when that fills the chip
  const int ldc = (int)select_chunked_ldc(S, k);
  const bool chunk = !aqua && ldc > 0 && k < S && score_select_chunk_fits(p) &&
                     (int64_t)B * Hq * ((S + kSelChunk - 1) / kSelChunk) >= 256;
  float* qrot_s = qrot;
  uint16_t* qsplit_s = qsplit;
  DecodePlan ps = p;  // the score stage's plan
  if (aqua) {
    qrot_s = at<float>(workspace, p.off_qrot_m);
    qsplit_s = at<uint16_t>(workspace, p.off_qsplit_m);
    ps.r = d;
    src = K_rot;
    ld = d;
  }
  if (ev) LOKI_HIP(hipEventRecord(ev[0], stream));
  if (pair) {
    // the whole step of each pair of heads in one kernel (rotation, scores,
    // selection, exact attention); the later stage events follow it
    if (ev) LOKI_HIP(hipEventRecord(ev[1], stream));
    LOKI_HIP(launch_decode_pair(p, src, ld, q, P, K_rot, V, out, idx, plain_attn, stream));
    if (ev)
      for (int i = 2; i < 6; ++i) LOKI_HIP(hipEventRecord(ev[i], stream));
    return LOKI_OK;
  }
  uint32_t* scnt = at<uint32_t>(workspace, p.off_scnt);
  float* spart = at<float>(workspace, p.off_spart);
  // the rotation launch also clears the split attention's counters
  LOKI_HIP(launch_qrot(p, q, P, qrot, qsplit, stream, scnt, p.NSPL > 1 ? B * Hq : 0));
  if (aqua) LOKI_HIP(launch_qdims(p, q, qrot, qrot_s, qsplit_s, dims, info, aqua_r, stream));
  if (ev) LOKI_HIP(hipEventRecord(ev[1], stream));
  if (fused) {
    LOKI_HIP(launch_score_select(p, src, ld, qsplit, idx, bitmap, stream));
    if (ev) LOKI_HIP(hipEventRecord(ev[2], stream));
  } else if (chunk) {
    int32_t* cidx = at<int32_t>(workspace, p.off_cidx);
    uint32_t* ckey = at<uint32_t>(workspace, p.off_ckey);
    LOKI_HIP(launch_score_select_chunk(ps, src, ld, qsplit_s, cidx, ckey, ldc, stream));
    if (ev) LOKI_HIP(hipEventRecord(ev[2], stream));
    if (select_attend_fits(p)) {
      // the second stage and the attention of each head in one launch
      if (plain_attn) LOKI_HIP(launch_qplain(p, q, qrot, qsplit, stream));
      LOKI_HIP(launch_select_attend(p, ckey, cidx, ldc, ldc, qsplit, K_rot, V, out, idx, spart, scnt, stream));
      if (ev)
        for (int i = 3; i < 6; ++i) LOKI_HIP(hipEventRecord(ev[i], stream));
      return LOKI_OK;
    }
    LOKI_HIP(launch_select_merge(B * Hq, S, k, p.W, ldc, ckey, cidx, idx, bitmap, lens, Hq, stream));
  } else {
    uint2* mm = select_needs_minmax(S) ? at<uint2>(workspace, p.off_mm) : nullptr;
    LOKI_HIP(launch_scores(ps, src, ld, qrot_s, qsplit_s, keys, true, p.Sp, mm, stream));
    if (ev) LOKI_HIP(hipEventRecord(ev[2], stream));
    if (select_attend_fits(p) && !select_needs_minmax(S)) {
      // heads whose keys fit the register selection: selection and attention
      // of each head in one launch
      if (plain_attn) LOKI_HIP(launch_qplain(p, q, qrot, qsplit, stream));
      LOKI_HIP(launch_select_attend(p, keys, nullptr, p.Sp, 0, qsplit, K_rot, V, out, idx, spart, scnt, stream));
      if (ev)
        for (int i = 3; i < 6; ++i) LOKI_HIP(hipEventRecord(ev[i], stream));
      return LOKI_OK;
    }
    LOKI_HIP(launch_select(B * Hq, S, p.Sp, k, p.W, keys, mm, p.NSC, at<uint32_t>(workspace, p.off_masks),
                           idx, bitmap, stream, at<int32_t>(workspace, p.off_cidx),
                           at<uint32_t>(workspace, p.off_ckey), lens, Hq));
  }
  if (ev) LOKI_HIP(hipEventRecord(ev[3], stream));
  // asymmetric index: the score stage used q P (P the query-side matrix);
  // the exact stage takes the query itself against the unrotated keys
  if (plain_attn) LOKI_HIP(launch_qplain(p, q, qrot, qsplit, stream));
  LOKI_HIP(launch_attend(p, K_rot, V, qrot, qsplit, bitmap, part, out, stream, ev ? ev[4] : nullptr));
  if (ev) LOKI_HIP(hipEventRecord(ev[5], stream));
  return LOKI_OK;
}

loki_status loki_decode(const void* q, const void* P, const void* K_rot, const void* V, void* out,
                        int32_t* idx, int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d,
                        int32_t r, int32_t k, loki_dtype dt, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  try {
    return decode_impl(q, P, K_rot, nullptr, 0, V, out, idx, B, Hq, Hkv, S, d, r, k, dt, workspace,
                       workspace_bytes, stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_decode_lead(const void* q, const void* P, const void* K_rot, const void* K_lead,
                             int32_t R, const void* V, void* out, int32_t* idx, int32_t B,
                             int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t r, int32_t k,
                             loki_dtype dt, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  try {
    if (!K_lead) return LOKI_ERR_NULL;
    return decode_impl(q, P, K_rot, K_lead, R, V, out, idx, B, Hq, Hkv, S, d, r, k, dt, workspace,
                       workspace_bytes, stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_decode_varlen(const void* q, const void* P, const void* K_rot, const void* K_lead,
                               int32_t R, const void* V, const int32_t* lens, void* out, int32_t* idx,
                               int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t r,
                               int32_t k, loki_dtype dt, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  try {
    if (!lens) return LOKI_ERR_NULL;
    return decode_impl(q, P, K_rot, K_lead, R, V, out, idx, B, Hq, Hkv, S, d, r, k, dt, workspace,
                       workspace_bytes, stream, nullptr, lens);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_decode_profiled(const void* q, const void* P, const void* K_rot, const void* K_lead,
                                 int32_t R, const void* V, const int32_t* lens, void* out, int32_t* idx,
                                 int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t r,
                                 int32_t k, loki_dtype dt, void* workspace, size_t workspace_bytes,
                                 hipEvent_t* events, hipStream_t stream) {
  try {
    if (!events) return LOKI_ERR_NULL;
    for (int i = 0; i < 6; ++i)
      if (!events[i]) return LOKI_ERR_NULL;
    return decode_impl(q, P, K_rot, K_lead, R, V, out, idx, B, Hq, Hkv, S, d, r, k, dt, workspace,
                       workspace_bytes, stream, events, lens);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_scores(const void* q, const void* P, const void* K_rot, float* scores, int32_t B,
                        int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t r, loki_dtype dt,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    LOKI_TRY(check_dtype(dt));
    if (!q || !P || !K_rot || !scores) return LOKI_ERR_NULL;
    LOKI_TRY(check_sizes(B, Hq, Hkv, S, d));
    if (r < 1 || r > d) return LOKI_ERR_RANGE;
    if (!aligned16(q) || !aligned16(P) || !aligned16(K_rot) || !aligned16(scores))
      return LOKI_ERR_ALIGN;
    DecodePlan p;
    if (!make_decode_plan(p, B, Hq, Hkv, S, d, r, 1, (int)dt)) return LOKI_ERR_INTERNAL;
    LOKI_TRY(check_workspace(workspace, workspace_bytes, p.bytes));
    float* qrot = at<float>(workspace, p.off_qrot);
    uint16_t* qsplit = at<uint16_t>(workspace, p.off_qsplit);
    LOKI_HIP(launch_qrot(p, q, P, qrot, qsplit, stream));
    LOKI_HIP(launch_scores(p, K_rot, d, qrot, qsplit, scores, false, S, nullptr, stream));
    return LOKI_OK;
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

size_t loki_select_workspace_bytes(int32_t rows, int32_t S, int32_t k) {
  if (rows < 1 || rows > kMaxRows || S < 1 || (int64_t)S > kMaxS || k < 1 || k > S) return 0;
  SelectPlan p;
  if (!make_select_plan(p, rows, S, k)) return 0;
  return p.bytes;
}

loki_status loki_select_topk(const float* scores, int32_t* idx, int32_t rows, int32_t S, int32_t k,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    if (!scores || !idx) return LOKI_ERR_NULL;
    if (rows < 1 || S < 1 || rows > kMaxRows || (int64_t)S > kMaxS) return LOKI_ERR_SHAPE;
    if (k < 1 || k > S) return LOKI_ERR_RANGE;
    if (!aligned16(scores) || !aligned16(idx)) return LOKI_ERR_ALIGN;
    SelectPlan p;
    if (!make_select_plan(p, rows, S, k)) return LOKI_ERR_INTERNAL;
    LOKI_TRY(check_workspace(workspace, workspace_bytes, p.bytes));
    uint32_t* keys = at<uint32_t>(workspace, p.off_keys);
    uint32_t* bitmap = at<uint32_t>(workspace, p.off_bitmap);
    uint2* mm = at<uint2>(workspace, p.off_mm);
    LOKI_HIP(launch_scores_to_keys(scores, keys, mm, p.NMM, rows, S, p.Sp, stream));
    LOKI_HIP(launch_select(rows, S, p.Sp, k, p.W, keys, mm, p.NMM, at<uint32_t>(workspace, p.off_masks),
                           idx, bitmap, stream, at<int32_t>(workspace, p.off_cidx),
                           at<uint32_t>(workspace, p.off_ckey)));
    return LOKI_OK;
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_attend(const void* q, const void* P, const void* K_rot, const void* V,
                        const int32_t* idx, void* out, int32_t B, int32_t Hq, int32_t Hkv,
                        int32_t S, int32_t d, int32_t k, loki_dtype dt, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  try {
    LOKI_TRY(check_dtype(dt));
    if (!q || !P || !K_rot || !V || !idx || !out) return LOKI_ERR_NULL;
    LOKI_TRY(check_sizes(B, Hq, Hkv, S, d));
    if (k < 1 || k > S) return LOKI_ERR_RANGE;
    if (!aligned16(q) || !aligned16(P) || !aligned16(K_rot) || !aligned16(V) || !aligned16(out) ||
        !aligned16(idx))
      return LOKI_ERR_ALIGN;
    DecodePlan p;
    if (!make_decode_plan(p, B, Hq, Hkv, S, d, d, k, (int)dt)) return LOKI_ERR_INTERNAL;
    LOKI_TRY(check_workspace(workspace, workspace_bytes, p.bytes));
    float* qrot = at<float>(workspace, p.off_qrot);
    uint16_t* qsplit = at<uint16_t>(workspace, p.off_qsplit);
    uint32_t* bitmap = at<uint32_t>(workspace, p.off_bitmap);
    float* part = at<float>(workspace, p.off_part);
    LOKI_HIP(launch_qrot(p, q, P, qrot, qsplit, stream));
    LOKI_HIP(launch_idx_to_bitmap(p, idx, bitmap, stream));
    LOKI_HIP(launch_attend(p, K_rot, V, qrot, qsplit, bitmap, part, out, stream));
    return LOKI_OK;
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_decode_aqua(const void* q, const void* P, const void* K_rot, const void* V, const int32_t* lens,
                             void* out, int32_t* idx, int32_t* dims, float* info_loss, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t S, int32_t d, int32_t r, int32_t k, loki_dtype dt,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    if ((reinterpret_cast<uintptr_t>(dims) & 3u) || (reinterpret_cast<uintptr_t>(info_loss) & 3u))
      return LOKI_ERR_ALIGN;
    return decode_impl(q, P, K_rot, nullptr, 0, V, out, idx, B, Hq, Hkv, S, d, r, k, dt, workspace,
                       workspace_bytes, stream, nullptr, lens, r, dims, info_loss);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_decode_aqua_profiled(const void* q, const void* P, const void* K_rot, const void* V,
                                      const int32_t* lens, void* out, int32_t* idx, int32_t* dims, float* info_loss,
                                      int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t r,
                                      int32_t k, loki_dtype dt, void* workspace, size_t workspace_bytes,
                                      hipEvent_t* events, hipStream_t stream) {
  try {
    if (!events) return LOKI_ERR_NULL;
    for (int i = 0; i < 6; ++i)
      if (!events[i]) return LOKI_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(dims) & 3u) || (reinterpret_cast<uintptr_t>(info_loss) & 3u))
      return LOKI_ERR_ALIGN;
    return decode_impl(q, P, K_rot, nullptr, 0, V, out, idx, B, Hq, Hkv, S, d, r, k, dt, workspace,
                       workspace_bytes, stream, events, lens, r, dims, info_loss);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

static loki_status decode_asym_impl(const void* q, const void* A, const void* K_idx, int32_t R, const void* K,
                                    const void* V, const int32_t* lens, void* out, int32_t* idx, int32_t B,
                                    int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t r, int32_t k,
                                    loki_dtype dt, void* ws, size_t wsb, hipEvent_t* ev, hipStream_t stream) {
  if (!K_idx) return LOKI_ERR_NULL;
  // the decode with A in place of the basis, the key index as the lead-dims
  // source, the keys themselves for the exact stage
  return decode_impl(q, A, K, K_idx, R, V, out, idx, B, Hq, Hkv, S, d, r, k, dt, ws, wsb, stream, ev, lens, 0,
                     nullptr, nullptr, true);
}

loki_status loki_decode_asym(const void* q, const void* A, const void* K_idx, int32_t R, const void* K,
                             const void* V, const int32_t* lens, void* out, int32_t* idx, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t S, int32_t d, int32_t r, int32_t k, loki_dtype dt,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    return decode_asym_impl(q, A, K_idx, R, K, V, lens, out, idx, B, Hq, Hkv, S, d, r, k, dt, workspace,
                            workspace_bytes, nullptr, stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_decode_asym_profiled(const void* q, const void* A, const void* K_idx, int32_t R, const void* K,
                                      const void* V, const int32_t* lens, void* out, int32_t* idx, int32_t B,
                                      int32_t Hq, int32_t Hkv, int32_t S, int32_t d, int32_t r, int32_t k,
                                      loki_dtype dt, void* workspace, size_t workspace_bytes, hipEvent_t* events,
                                      hipStream_t stream) {
  try {
    if (!events) return LOKI_ERR_NULL;
    for (int i = 0; i < 6; ++i)
      if (!events[i]) return LOKI_ERR_NULL;
    return decode_asym_impl(q, A, K_idx, R, K, V, lens, out, idx, B, Hq, Hkv, S, d, r, k, dt, workspace,
                            workspace_bytes, events, stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

static loki_status calibrate_impl(const void* K, void* P, double* eigvals, int32_t B, int32_t Hkv, int32_t S,
                                  int32_t d, loki_dtype dt, void* ws, size_t wsb, hipEvent_t* ev,
                                  hipStream_t stream) {
  LOKI_TRY(check_dtype(dt));
  if (!K || !P) return LOKI_ERR_NULL;
  if (B < 1 || Hkv < 1 || S < 1 || d < 1) return LOKI_ERR_SHAPE;
  if ((int64_t)B * S > 0x7fffffffLL || (int64_t)Hkv > kMaxRows) return LOKI_ERR_SHAPE;
  if (d != 64 && d != 128) return LOKI_ERR_UNSUPPORTED;
  if (!aligned16(K) || !aligned16(P)) return LOKI_ERR_ALIGN;
  if (eigvals && (reinterpret_cast<uintptr_t>(eigvals) & 7u)) return LOKI_ERR_ALIGN;
  CalibPlan p;
  if (!make_calib_plan(p, B, Hkv, S, d, (int)dt)) return LOKI_ERR_INTERNAL;
  LOKI_TRY(check_workspace(ws, wsb, p.bytes));
  return after_launch(launch_calibrate(p, K, P, eigvals, ws, stream, ev), stream);
}

size_t loki_calibrate_workspace_bytes(int32_t B, int32_t Hkv, int32_t S, int32_t d) {
  try {
    CalibPlan p;
    if ((int64_t)B * S > 0x7fffffffLL || !make_calib_plan(p, B, Hkv, S, d, 1)) return 0;
    return p.bytes;
  } catch (...) {
    return 0;
  }
}

loki_status loki_calibrate_pca(const void* K, void* P, double* eigvals, int32_t B, int32_t Hkv, int32_t S,
                               int32_t d, loki_dtype dt, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  try {
    return calibrate_impl(K, P, eigvals, B, Hkv, S, d, dt, workspace, workspace_bytes, nullptr, stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_calibrate_pca_profiled(const void* K, void* P, double* eigvals, int32_t B, int32_t Hkv,
                                        int32_t S, int32_t d, loki_dtype dt, void* workspace,
                                        size_t workspace_bytes, hipEvent_t* events, hipStream_t stream) {
  try {
    if (!events) return LOKI_ERR_NULL;
    for (int i = 0; i < 4; ++i)
      if (!events[i]) return LOKI_ERR_NULL;
    return calibrate_impl(K, P, eigvals, B, Hkv, S, d, dt, workspace, workspace_bytes, events, stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

size_t loki_calibrate_asym_workspace_bytes(int32_t N, int32_t Hq, int32_t B, int32_t Hkv, int32_t S, int32_t d,
                                          int32_t r) {
  try {
    AsymPlan p;
    if ((int64_t)B * S > 0x7fffffffLL || !make_asym_plan(p, N, Hq, B, Hkv, S, d, r, 1)) return 0;
    return p.bytes;
  } catch (...) {
    return 0;
  }
}

loki_status loki_calibrate_asym(const void* q_samples, const void* K, void* A, void* Bm, int32_t N, int32_t Hq,
                                int32_t B, int32_t Hkv, int32_t S, int32_t d, int32_t r, loki_dtype dt,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    LOKI_TRY(check_dtype(dt));
    if (!q_samples || !K || !A || !Bm) return LOKI_ERR_NULL;
    if (N < 1 || Hq < 1 || B < 1 || Hkv < 1 || S < 1 || d < 1 || Hq % Hkv) return LOKI_ERR_SHAPE;
    if ((int64_t)B * S > 0x7fffffffLL || (int64_t)Hq > kMaxRows) return LOKI_ERR_SHAPE;
    if (d != 64 && d != 128) return LOKI_ERR_UNSUPPORTED;
    if (r < 1 || r > d) return LOKI_ERR_RANGE;
    if (!aligned16(q_samples) || !aligned16(K) || !aligned16(A) || !aligned16(Bm)) return LOKI_ERR_ALIGN;
    AsymPlan p;
    if (!make_asym_plan(p, N, Hq, B, Hkv, S, d, r, (int)dt)) return LOKI_ERR_INTERNAL;
    LOKI_TRY(check_workspace(workspace, workspace_bytes, p.bytes));
    return after_launch(launch_calibrate_asym(p, q_samples, K, A, Bm, workspace, stream), stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

// ---------------------------------------------------------------- no-allocation decode

}  // extern "C"

namespace {

// The decode's scratch for callers that cannot allocate: one file-scope
// device array (each GPU the library runs on holds its own copy, at its own
// address, until the process ends).  Host code never uses the array's name
// as an address: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kNoallocScratch = LOKI_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratch];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch address, or a non-success status.
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

loki_status loki_decode_noalloc(const void* q, const void* P, const void* K_rot, const void* K_lead, int32_t R,
                                const void* V, void* out, int32_t* idx, int32_t B, int32_t Hq, int32_t Hkv,
                                int32_t S, int32_t d, int32_t r, int32_t k, loki_dtype dt, hipStream_t stream) {
  try {
    // the sizes are validated first, as for every entry point; then their
    // scratch need against the fixed array
    LOKI_TRY(check_dtype(dt));
    LOKI_TRY(check_sizes(B, Hq, Hkv, S, d));
    if (r < 1 || r > d || k < 1 || k > S) return LOKI_ERR_RANGE;
    DecodePlan p;
    if (!make_decode_plan(p, B, Hq, Hkv, S, d, r, k, (int)dt)) return LOKI_ERR_INTERNAL;
    if (p.bytes > kNoallocScratch) return LOKI_ERR_WORKSPACE;
    void* ws = nullptr;
    LOKI_HIP(scratch_on_current_device(&ws));
    return decode_impl(q, P, K_rot, K_lead, K_lead ? R : 0, V, out, idx, B, Hq, Hkv, S, d, r, k, dt, ws,
                       kNoallocScratch, stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_bench_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  try {
    if (bytes % 16 != 0) return LOKI_ERR_SHAPE;
    if (bytes == 0) return LOKI_OK;
    if (!src || !dst) return LOKI_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst)) return LOKI_ERR_ALIGN;
    return after_launch(launch_bench_copy(src, dst, bytes, stream), stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

loki_status loki_bench_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  try {
    if (bytes % 16 != 0) return LOKI_ERR_SHAPE;
    if (bytes == 0) return LOKI_OK;
    if (!src || !sink) return LOKI_ERR_NULL;
    if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return LOKI_ERR_ALIGN;
    return after_launch(launch_bench_read(src, bytes, sink, stream), stream);
  } catch (...) {
    return LOKI_ERR_INTERNAL;
  }
}

}  // extern "C"
