// C entry points of libvce: argument checks (all on the host, before any HIP
// call), workspace sizing, then the launchers.
#include "../../include/vce.h"

#include <hip/hip_runtime.h>

#include "vce_internal.hpp"

namespace {

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
size_t esize_of(vce_dtype dt) { return dt == VCE_BF16 ? 2 : 4; }
bool dtype_ok(int dt) { return dt == VCE_F32 || dt == VCE_BF16; }

// Shape / shard checks shared by the table-based entry points.
vce_status check_table(int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int32_t n) {
  if (T < 0 || H <= 0 || V_real < 1 || V_real > V_pad) return VCE_ERR_SHAPE;
  if (T > kMaxDim || H > kMaxDim || V_pad > kMaxDim) return VCE_ERR_SHAPE;
  if (n < 1 || n > vce::kMaxShards || V_pad % n != 0) return VCE_ERR_SHARD;
  return VCE_OK;
}

// An explicit layout (shard_rows, num_shards + 1 host values): 0 first,
// V_pad last, nondecreasing.
vce_status check_layout(int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int32_t n,
                        const int64_t* rows) {
  if (T < 0 || H <= 0 || V_real < 1 || V_real > V_pad) return VCE_ERR_SHAPE;
  if (T > kMaxDim || H > kMaxDim || V_pad > kMaxDim) return VCE_ERR_SHAPE;
  if (!rows) return VCE_ERR_NULL;
  if (n < 1 || n > vce::kMaxShards || rows[0] != 0 || rows[n] != V_pad) return VCE_ERR_SHARD;
  for (int32_t k = 0; k < n; ++k)
    if (rows[k + 1] < rows[k]) return VCE_ERR_SHARD;
  return VCE_OK;
}

vce_status check_ignore(int32_t ignore_index, int64_t V_real) {
  return (ignore_index >= 0 && ignore_index < V_real) ? VCE_ERR_SHAPE : VCE_OK;
}

vce_status hip_status(hipError_t e) { return e == hipSuccess ? VCE_OK : VCE_ERR_HIP; }

}  // namespace

extern "C" {

int32_t vce_abi_version(void) { return 1; }

const char* vce_strerror(vce_status s) {
  switch (s) {
    case VCE_OK: return "ok";
    case VCE_ERR_NULL: return "a required pointer is NULL";
    case VCE_ERR_SHAPE: return "invalid size argument (T, H, V_real, V_pad, P, capacity or ignore_index)";
    case VCE_ERR_SHARD:
      return "num_shards must be in [1, 128] and divide V_pad, or shard_rows must run from 0 "
             "to V_pad without decreasing";
    case VCE_ERR_DTYPE: return "unknown element type, reduction or accumulate flag";
    case VCE_ERR_ALIGN: return "pointers must be 16-byte aligned and H a multiple of 8";
    case VCE_ERR_WORKSPACE: return "workspace missing or smaller than the size query";
    case VCE_ERR_HIP: return "a HIP kernel launch failed";
  }
  return "unknown status";
}

size_t vce_fwd_workspace_bytes(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                               int32_t num_shards, vce_dtype dt) {
  if (check_table(T, H, V_real, V_pad, num_shards) != VCE_OK || !dtype_ok(dt)) return 0;
  return vce::plan_fwd(T, H, V_real, V_pad, num_shards, nullptr, nullptr).bytes;
}

size_t vce_fwd_workspace_bytes_ex(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                                  int32_t num_shards, const int64_t* shard_rows, vce_dtype dt) {
  if (check_layout(T, H, V_real, V_pad, num_shards, shard_rows) != VCE_OK || !dtype_ok(dt))
    return 0;
  return vce::plan_fwd(T, H, V_real, V_pad, num_shards, shard_rows, nullptr).bytes;
}

size_t vce_bwd_workspace_bytes(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                               int32_t num_shards, vce_dtype dt) {
  if (check_table(T, H, V_real, V_pad, num_shards) != VCE_OK || !dtype_ok(dt)) return 0;
  return vce::plan_bwd(T, H, V_real, V_pad, num_shards, esize_of(dt), nullptr).bytes;
}

size_t vce_argmax_workspace_bytes(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                                  int32_t num_shards, vce_dtype dt) {
  if (check_table(T, H, V_real, V_pad, num_shards) != VCE_OK || !dtype_ok(dt)) return 0;
  return vce::plan_argmax(T, H, V_real, V_pad, num_shards, nullptr, nullptr).bytes;
}

size_t vce_argmax_workspace_bytes_ex(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                                     int32_t num_shards, const int64_t* shard_rows,
                                     vce_dtype dt) {
  if (check_layout(T, H, V_real, V_pad, num_shards, shard_rows) != VCE_OK || !dtype_ok(dt))
    return 0;
  return vce::plan_argmax(T, H, V_real, V_pad, num_shards, shard_rows, nullptr).bytes;
}

size_t vemb_bwd_workspace_bytes(int64_t T, int64_t H, int64_t V_real, int64_t V_pad) {
  if (check_table(T, H, V_real, V_pad, 1) != VCE_OK) return 0;
  return vce::plan_emb_bwd(T, H, V_real, nullptr).bytes;
}

size_t vss_candidates_workspace_bytes(int64_t T, int64_t V) {
  if (T < 0 || V < 1 || T > kMaxDim || V > kMaxDim) return 0;
  return vce::plan_cand(T, V, nullptr).bytes;
}

static vce_status fwd_impl(const void* h, const void* W, const int32_t* targets, int64_t T,
                           int64_t H, int64_t V_real, int64_t V_pad, int32_t num_shards,
                           const int64_t* shard_rows, int32_t ignore_index, vce_dtype dt,
                           float* lse, float* loss, float* loss_sum, int32_t* n_valid,
                           int32_t* n_bad_target, float* shard_stats, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!dtype_ok(dt)) return VCE_ERR_DTYPE;
  vce_status st = shard_rows ? check_layout(T, H, V_real, V_pad, num_shards, shard_rows)
                             : check_table(T, H, V_real, V_pad, num_shards);
  if (st != VCE_OK) return st;
  if ((st = check_ignore(ignore_index, V_real)) != VCE_OK) return st;
  if (!loss_sum || !n_valid || !n_bad_target) return VCE_ERR_NULL;
  if (T > 0 && (!h || !W || !targets || !lse || !loss)) return VCE_ERR_NULL;
  if (H % 8 != 0) return VCE_ERR_ALIGN;
  if (T > 0 && (!aligned16(h) || !aligned16(W) || !aligned4(targets) || !aligned4(lse) ||
                !aligned4(loss) || (shard_stats && !aligned4(shard_stats))))
    return VCE_ERR_ALIGN;
  if (!aligned4(loss_sum) || !aligned4(n_valid) || !aligned4(n_bad_target)) return VCE_ERR_ALIGN;
  const vce::FwdPlan probe = vce::plan_fwd(T, H, V_real, V_pad, num_shards, shard_rows, nullptr);
  if (T > 0 && (!ws || ws_bytes < probe.bytes)) return VCE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return VCE_ERR_ALIGN;
  const vce::FwdPlan p = vce::plan_fwd(T, H, V_real, V_pad, num_shards, shard_rows, ws);
  return hip_status(vce::run_ce_fwd(h, W, targets, T, H, V_real, V_pad, ignore_index,
                                    dt == VCE_BF16, lse, loss, loss_sum, n_valid, n_bad_target,
                                    shard_stats, p, static_cast<hipStream_t>(stream)));
}

vce_status vce_fwd(const void* h, const void* W, const int32_t* targets, int64_t T, int64_t H,
                   int64_t V_real, int64_t V_pad, int32_t num_shards, int32_t ignore_index,
                   vce_dtype dt, float* lse, float* loss, float* loss_sum, int32_t* n_valid,
                   int32_t* n_bad_target, float* shard_stats, void* ws, size_t ws_bytes,
                   void* stream) {
  return fwd_impl(h, W, targets, T, H, V_real, V_pad, num_shards, nullptr, ignore_index, dt, lse,
                  loss, loss_sum, n_valid, n_bad_target, shard_stats, ws, ws_bytes, stream);
}

vce_status vce_fwd_ex(const void* h, const void* W, const int32_t* targets, int64_t T, int64_t H,
                      int64_t V_real, int64_t V_pad, int32_t num_shards,
                      const int64_t* shard_rows, int32_t ignore_index, vce_dtype dt, float* lse,
                      float* loss, float* loss_sum, int32_t* n_valid, int32_t* n_bad_target,
                      float* shard_stats, void* ws, size_t ws_bytes, void* stream) {
  if (!shard_rows) return VCE_ERR_NULL;
  return fwd_impl(h, W, targets, T, H, V_real, V_pad, num_shards, shard_rows, ignore_index, dt,
                  lse, loss, loss_sum, n_valid, n_bad_target, shard_stats, ws, ws_bytes, stream);
}

vce_status vce_bwd(const void* h, const void* W, const int32_t* targets, const float* lse,
                   const float* grad_loss, const int32_t* n_valid, vce_reduction red, int64_t T,
                   int64_t H, int64_t V_real, int64_t V_pad, int32_t num_shards,
                   int32_t ignore_index, vce_dtype dt, float* dh, float* dW,
                   int32_t accumulate, void* ws, size_t ws_bytes, void* stream) {
  return vce_bwd_timed(h, W, targets, lse, grad_loss, n_valid, red, T, H, V_real, V_pad,
                       num_shards, ignore_index, dt, dh, dW, accumulate, ws, ws_bytes, stream,
                       nullptr, 0);
}

int64_t vce_bwd_event_count(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                            int32_t num_shards, vce_dtype dt) {
  if (!dtype_ok(dt) || check_table(T, H, V_real, V_pad, num_shards) != VCE_OK) return 0;
  const vce::BwdPlan p = vce::plan_bwd(T, H, V_real, V_pad, num_shards, esize_of(dt), nullptr);
  return 1 + 3 * p.n_chunks;
}

vce_status vce_bwd_timed(const void* h, const void* W, const int32_t* targets, const float* lse,
                         const float* grad_loss, const int32_t* n_valid, vce_reduction red,
                         int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int32_t num_shards,
                         int32_t ignore_index, vce_dtype dt, float* dh, float* dW,
                         int32_t accumulate, void* ws, size_t ws_bytes, void* stream,
                         void* const* events, int64_t n_events) {
  if (!dtype_ok(dt) || (red != VCE_REDUCE_MEAN && red != VCE_REDUCE_SUM)) return VCE_ERR_DTYPE;
  if (accumulate & ~(VCE_ACC_DW | VCE_ACC_DH)) return VCE_ERR_DTYPE;
  vce_status st = check_table(T, H, V_real, V_pad, num_shards);
  if (st != VCE_OK) return st;
  if ((st = check_ignore(ignore_index, V_real)) != VCE_OK) return st;
  if (!dW || !grad_loss || (red == VCE_REDUCE_MEAN && !n_valid)) return VCE_ERR_NULL;
  if (T > 0 && (!h || !W || !targets || !lse || !dh)) return VCE_ERR_NULL;
  if (H % 8 != 0) return VCE_ERR_ALIGN;
  if (!aligned16(dW) || !aligned4(grad_loss) || (n_valid && !aligned4(n_valid)))
    return VCE_ERR_ALIGN;
  if (T > 0 && (!aligned16(h) || !aligned16(W) || !aligned4(targets) || !aligned4(lse) ||
                !aligned16(dh)))
    return VCE_ERR_ALIGN;
  const vce::BwdPlan probe = vce::plan_bwd(T, H, V_real, V_pad, num_shards, esize_of(dt), nullptr);
  if (T > 0 && (!ws || ws_bytes < probe.bytes)) return VCE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return VCE_ERR_ALIGN;
  const vce::BwdPlan p = vce::plan_bwd(T, H, V_real, V_pad, num_shards, esize_of(dt), ws);
  if (events && n_events != 1 + 3 * p.n_chunks) return VCE_ERR_SHAPE;
  return hip_status(vce::run_ce_bwd(h, W, targets, lse, grad_loss, n_valid, red, T, H, V_real,
                                    V_pad, num_shards, dt == VCE_BF16, dh, dW, accumulate,
                                    p, static_cast<hipStream_t>(stream), events));
}

// Argument checks of the argmax entry points; on success `need` is the
// workspace the call takes.
static vce_status argmax_check(const void* h, const void* W, int64_t T, int64_t H,
                               int64_t V_real, int64_t V_pad, int32_t num_shards,
                               const int64_t* shard_rows, vce_dtype dt, const int32_t* index,
                               const float* value, const float* shard_value,
                               const int32_t* shard_index, size_t* need) {
  if (!dtype_ok(dt)) return VCE_ERR_DTYPE;
  vce_status st = shard_rows ? check_layout(T, H, V_real, V_pad, num_shards, shard_rows)
                             : check_table(T, H, V_real, V_pad, num_shards);
  if (st != VCE_OK) return st;
  if (T > 0 && (!h || !W || !index || !value)) return VCE_ERR_NULL;
  if (H % 8 != 0) return VCE_ERR_ALIGN;
  if (T > 0 && (!aligned16(h) || !aligned16(W) || !aligned4(index) || !aligned4(value) ||
                (shard_value && !aligned4(shard_value)) ||
                (shard_index && !aligned4(shard_index))))
    return VCE_ERR_ALIGN;
  *need = vce::plan_argmax(T, H, V_real, V_pad, num_shards, shard_rows, nullptr).bytes;
  return VCE_OK;
}

static vce_status argmax_impl(const void* h, const void* W, int64_t T, int64_t H,
                              int64_t V_real, int64_t V_pad, int32_t num_shards,
                              const int64_t* shard_rows, vce_dtype dt, int32_t* index,
                              float* value, float* shard_value, int32_t* shard_index, void* ws,
                              size_t ws_bytes, void* stream) {
  size_t need = 0;
  const vce_status st = argmax_check(h, W, T, H, V_real, V_pad, num_shards, shard_rows, dt,
                                     index, value, shard_value, shard_index, &need);
  if (st != VCE_OK) return st;
  if (T > 0 && (!ws || ws_bytes < need)) return VCE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return VCE_ERR_ALIGN;
  const vce::ArgPlan p = vce::plan_argmax(T, H, V_real, V_pad, num_shards, shard_rows, ws);
  return hip_status(vce::run_argmax(h, W, T, H, V_real, V_pad, dt == VCE_BF16, index,
                                    value, shard_value, shard_index, p,
                                    static_cast<hipStream_t>(stream)));
}

vce_status vce_argmax(const void* h, const void* W, int64_t T, int64_t H, int64_t V_real,
                      int64_t V_pad, int32_t num_shards, vce_dtype dt, int32_t* index,
                      float* value, float* shard_value, int32_t* shard_index, void* ws,
                      size_t ws_bytes, void* stream) {
  return argmax_impl(h, W, T, H, V_real, V_pad, num_shards, nullptr, dt, index, value,
                     shard_value, shard_index, ws, ws_bytes, stream);
}

vce_status vce_argmax_noalloc(const void* h, const void* W, int64_t T, int64_t H,
                              int64_t V_real, int64_t V_pad, int32_t num_shards, vce_dtype dt,
                              int32_t* index, float* value, float* shard_value,
                              int32_t* shard_index, void* stream) {
  size_t need = 0;
  const vce_status st = argmax_check(h, W, T, H, V_real, V_pad, num_shards, nullptr, dt, index,
                                     value, shard_value, shard_index, &need);
  if (st != VCE_OK) return st;
  if (need > vce::kNoAllocScratchBytes) return VCE_ERR_WORKSPACE;
  if (T == 0) return VCE_OK;
  void* ws = nullptr;
  if (vce::noalloc_scratch(&ws) != hipSuccess) return VCE_ERR_HIP;
  return argmax_impl(h, W, T, H, V_real, V_pad, num_shards, nullptr, dt, index, value,
                     shard_value, shard_index, ws, vce::kNoAllocScratchBytes, stream);
}

vce_status vce_argmax_ex(const void* h, const void* W, int64_t T, int64_t H, int64_t V_real,
                         int64_t V_pad, int32_t num_shards, const int64_t* shard_rows,
                         vce_dtype dt, int32_t* index, float* value, float* shard_value,
                         int32_t* shard_index, void* ws, size_t ws_bytes, void* stream) {
  if (!shard_rows) return VCE_ERR_NULL;
  return argmax_impl(h, W, T, H, V_real, V_pad, num_shards, shard_rows, dt, index, value,
                     shard_value, shard_index, ws, ws_bytes, stream);
}

static vce_status emb_fwd_impl(const int32_t* ids, const void* W, int64_t T, int64_t H,
                               int64_t V_real, int64_t V_pad, int32_t num_shards,
                               const int64_t* shard_rows, vce_dtype dt, void* out,
                               int32_t* n_bad_id, void* stream) {
  if (!dtype_ok(dt)) return VCE_ERR_DTYPE;
  vce_status st = shard_rows ? check_layout(T, H, V_real, V_pad, num_shards, shard_rows)
                             : check_table(T, H, V_real, V_pad, num_shards);
  if (st != VCE_OK) return st;
  if (T > 0 && (!ids || !W || !out)) return VCE_ERR_NULL;
  if (H % 8 != 0) return VCE_ERR_ALIGN;
  if (T > 0 && (!aligned4(ids) || !aligned16(W) || !aligned16(out))) return VCE_ERR_ALIGN;
  if (n_bad_id && !aligned4(n_bad_id)) return VCE_ERR_ALIGN;
  return hip_status(vce::run_emb_fwd(ids, W, T, H, V_real,
                                     vce::shard_segments(num_shards, shard_rows, V_pad),
                                     esize_of(dt), out, n_bad_id,
                                     static_cast<hipStream_t>(stream)));
}

vce_status vemb_fwd(const int32_t* ids, const void* W, int64_t T, int64_t H, int64_t V_real,
                    int64_t V_pad, int32_t num_shards, vce_dtype dt, void* out, int32_t* n_bad_id,
                    void* stream) {
  return emb_fwd_impl(ids, W, T, H, V_real, V_pad, num_shards, nullptr, dt, out, n_bad_id,
                      stream);
}

vce_status vemb_fwd_ex(const int32_t* ids, const void* W, int64_t T, int64_t H, int64_t V_real,
                       int64_t V_pad, int32_t num_shards, const int64_t* shard_rows,
                       vce_dtype dt, void* out, int32_t* n_bad_id, void* stream) {
  if (!shard_rows) return VCE_ERR_NULL;
  return emb_fwd_impl(ids, W, T, H, V_real, V_pad, num_shards, shard_rows, dt, out, n_bad_id,
                      stream);
}

vce_status vce_remap(const int32_t* in, int64_t T, const int32_t* map, int64_t V_real,
                     int32_t* out, void* stream) {
  if (T < 0 || T > kMaxDim || V_real < 1 || V_real > kMaxDim) return VCE_ERR_SHAPE;
  if (T > 0 && (!in || !map || !out)) return VCE_ERR_NULL;
  if (T > 0 && (!aligned4(in) || !aligned4(map) || !aligned4(out))) return VCE_ERR_ALIGN;
  return hip_status(vce::run_remap(in, T, map, V_real, out, static_cast<hipStream_t>(stream)));
}

vce_status vngram_fwd(const int32_t* ids, const void* E, const void* E2, const void* E3,
                      int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int64_t rows2,
                      int64_t rows3, int32_t num_shards, vce_dtype dt, void* out,
                      int32_t* ids2, int32_t* ids3, int32_t* n_bad_id, void* stream) {
  if (!dtype_ok(dt)) return VCE_ERR_DTYPE;
  vce_status st = check_table(T, H, V_real, V_pad, num_shards);
  if (st != VCE_OK) return st;
  if (rows2 < 1 || rows3 < 1 || rows2 > kMaxDim || rows3 > kMaxDim) return VCE_ERR_SHAPE;
  if (rows2 % num_shards != 0 || rows3 % num_shards != 0) return VCE_ERR_SHARD;
  if (T > 0 && (!ids || !E || !E2 || !E3 || !out || !ids2 || !ids3)) return VCE_ERR_NULL;
  if (H % 8 != 0) return VCE_ERR_ALIGN;
  if (T > 0 && (!aligned4(ids) || !aligned16(E) || !aligned16(E2) || !aligned16(E3) ||
                !aligned16(out) || !aligned4(ids2) || !aligned4(ids3)))
    return VCE_ERR_ALIGN;
  if (n_bad_id && !aligned4(n_bad_id)) return VCE_ERR_ALIGN;
  return hip_status(vce::run_ngram_fwd(ids, E, E2, E3, T, H, V_real, V_pad, rows2, rows3,
                                       num_shards, dt == VCE_BF16, out, ids2, ids3, n_bad_id,
                                       static_cast<hipStream_t>(stream)));
}

vce_status vemb_bwd(const int32_t* ids, const void* dout, vce_dtype dout_dt, int64_t T, int64_t H,
                    int64_t V_real, int64_t V_pad, int32_t num_shards, float* dW,
                    int32_t accumulate, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dout_dt)) return VCE_ERR_DTYPE;
  vce_status st = check_table(T, H, V_real, V_pad, num_shards);
  if (st != VCE_OK) return st;
  if (!dW) return VCE_ERR_NULL;
  if (T > 0 && (!ids || !dout)) return VCE_ERR_NULL;
  if (H % 8 != 0) return VCE_ERR_ALIGN;
  if (!aligned16(dW)) return VCE_ERR_ALIGN;
  if (T > 0 && (!aligned4(ids) || !aligned16(dout))) return VCE_ERR_ALIGN;
  const vce::EmbBwdPlan probe = vce::plan_emb_bwd(T, H, V_real, nullptr);
  if (T > 0 && (!ws || ws_bytes < probe.bytes)) return VCE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return VCE_ERR_ALIGN;
  const vce::EmbBwdPlan p = vce::plan_emb_bwd(T, H, V_real, ws);
  return hip_status(vce::run_emb_bwd(ids, dout, dout_dt == VCE_BF16, T, H, V_real, V_pad, dW,
                                     accumulate ? 1 : 0, p, static_cast<hipStream_t>(stream)));
}

vce_status vss_candidates(const int32_t* targets, int64_t T, int64_t V, int32_t ignore_index,
                          const int32_t* perm, int64_t P, int32_t* cand, int64_t cand_cap,
                          int32_t* pos, int32_t* n_unique, int32_t* n_cand, void* ws,
                          size_t ws_bytes, void* stream) {
  if (T < 0 || V < 1 || P < 1 || T > kMaxDim || V > kMaxDim || P > kMaxDim) return VCE_ERR_SHAPE;
  // more candidates than table rows cannot all be distinct rows
  if (P > V) return VCE_ERR_SHAPE;
  if (check_ignore(ignore_index, V) != VCE_OK) return VCE_ERR_SHAPE;
  const int64_t need_cap = P > (T < V ? T : V) ? P : (T < V ? T : V);
  if (cand_cap < need_cap) return VCE_ERR_SHAPE;
  if (!perm || !cand || !n_unique || !n_cand) return VCE_ERR_NULL;
  if (T > 0 && (!targets || !pos)) return VCE_ERR_NULL;
  if (!aligned4(perm) || !aligned4(cand) || !aligned4(n_unique) || !aligned4(n_cand))
    return VCE_ERR_ALIGN;
  if (T > 0 && (!aligned4(targets) || !aligned4(pos))) return VCE_ERR_ALIGN;
  const vce::CandPlan probe = vce::plan_cand(T, V, nullptr);
  if (!ws || ws_bytes < probe.bytes) return VCE_ERR_WORKSPACE;
  if (!aligned16(ws)) return VCE_ERR_ALIGN;
  const vce::CandPlan p = vce::plan_cand(T, V, ws);
  return hip_status(vce::run_candidates(targets, T, V, perm, P, cand, pos, n_unique, n_cand, p,
                                        static_cast<hipStream_t>(stream)));
}

vce_status vss_scatter(const int32_t* cand, int64_t P, const float* dWc, int64_t H, int64_t V,
                       float* dW, int32_t accumulate, void* stream) {
  if (P < 0 || V < 1 || H <= 0 || P > kMaxDim || V > kMaxDim || H > kMaxDim) return VCE_ERR_SHAPE;
  if (accumulate != 0 && accumulate != 1) return VCE_ERR_DTYPE;
  if (!dW) return VCE_ERR_NULL;
  if (P > 0 && (!cand || !dWc)) return VCE_ERR_NULL;
  if (H % 8 != 0 || !aligned16(dW)) return VCE_ERR_ALIGN;
  if (P > 0 && (!aligned4(cand) || !aligned16(dWc))) return VCE_ERR_ALIGN;
  return hip_status(
      vce::run_ss_scatter(cand, P, dWc, H, V, dW, accumulate, static_cast<hipStream_t>(stream)));
}

vce_status vss_scatter_replace(const int32_t* prev, int64_t P_prev, const int32_t* cand, int64_t P,
                               const float* dWc, int64_t H, int64_t V, float* dW, void* stream) {
  if (P_prev < 0 || P_prev > kMaxDim) return VCE_ERR_SHAPE;
  if (P < 0 || V < 1 || H <= 0 || P > kMaxDim || V > kMaxDim || H > kMaxDim) return VCE_ERR_SHAPE;
  if (!dW) return VCE_ERR_NULL;
  if (P_prev > 0 && !prev) return VCE_ERR_NULL;
  if (P > 0 && (!cand || !dWc)) return VCE_ERR_NULL;
  if (H % 8 != 0 || !aligned16(dW)) return VCE_ERR_ALIGN;
  if (P_prev > 0 && !aligned4(prev)) return VCE_ERR_ALIGN;
  if (P > 0 && (!aligned4(cand) || !aligned16(dWc))) return VCE_ERR_ALIGN;
  return hip_status(vce::run_ss_scatter_replace(prev, P_prev, cand, P, dWc, H, V, dW,
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"
