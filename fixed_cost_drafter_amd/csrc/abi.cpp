// C ABI of liblongspark: argument validation, then the kernel launchers.
//
// Every check that the host can make runs before anything is enqueued, so a
// rejected call leaves device memory untouched.  No call allocates, frees,
// synchronises or reads device memory from the host.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/longspark.h"
#include "common.hpp"
#include "launch.hpp"

namespace ls {

ls_status check_dims(const ls_dims* d) {
  if (d == nullptr) return LS_ERR_NULL;
  if (d->dtype != LS_F32 && d->dtype != LS_BF16) return LS_ERR_DTYPE;
  // W = 0 (no window view) and S = 0 (no summary view) are allowed: the
  // ablations of one view (Table 5) on the cost side
  if (d->C < 1 || d->Hq < 1 || d->Hkv < 1 || d->d < 1 || d->W < 0 || d->S < 0 || d->B < 1 ||
      d->V < 1)
    return LS_ERR_SHAPE;
  if (d->Hq % d->Hkv != 0) return LS_ERR_SHAPE;
  if (d->B > ls::kMaxBlock || (d->W > 0 && d->B + 1 > d->W)) return LS_ERR_SHAPE;
  if (int64_t(d->C) * (d->B + 1) > 65535) return LS_ERR_SHAPE;
  if (d->V > (1 << 20)) return LS_ERR_SHAPE;  // at most 128 logit chunks per row
  if (int64_t(d->C) * d->Hkv * d->S > (int64_t(1) << 30)) return LS_ERR_SHAPE;
  const int G = d->Hq / d->Hkv;
  if (d->dtype == LS_F32) {
    if (d->d != 16 && d->d != 32 && d->d != 64 && d->d != 128) return LS_ERR_SHAPE;
    if (d->S > 256) return LS_ERR_SHAPE;
  } else {
    if (d->d != 128) return LS_ERR_SHAPE;
    if (d->S != 0 && d->S != 64 && d->S != 128) return LS_ERR_SHAPE;
    if (d->W % 32 != 0) return LS_ERR_SHAPE;  // 32-key chunks never straddle window | slots
    if (d->B * G > 64) return LS_ERR_SHAPE;
  }
  return LS_OK;
}

}  // namespace ls

namespace {

using ls::check_dims;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ls_status check_state(const ls_state* s, const ls_dims& d, int32_t L0) {
  if (s == nullptr) return LS_ERR_NULL;
  if (!s->seq_len || !s->err_flag || !s->workspace) return LS_ERR_NULL;
  // the window arrays may be NULL when W = 0, the summary arrays when S = 0
  if (d.W > 0 && (!s->ring_k || !s->ring_v || !s->ring_pos)) return LS_ERR_NULL;
  if (d.S > 0 && (!s->sum_m || !s->sum_l || !s->sum_n || !s->slot_k || !s->slot_v || !s->u ||
                  !s->log_lambda))
    return LS_ERR_NULL;
  if (!aligned16(s->ring_k) || !aligned16(s->ring_v) || !aligned16(s->sum_n) ||
      !aligned16(s->ring_pos) ||
      !aligned16(s->slot_k) || !aligned16(s->slot_v) || !aligned16(s->u) ||
      !aligned16(s->workspace))
    return LS_ERR_ALIGN;
  if (s->workspace_bytes < size_t(ls::ws_layout(d, L0).total)) return LS_ERR_WORKSPACE;
  return LS_OK;
}

}  // namespace

extern "C" {

int32_t ls_version(void) { return 107; }

const char* ls_status_string(int32_t status) {
  switch (status) {
    case LS_OK: return "ok";
    case LS_ERR_NULL: return "a required pointer is NULL";
    case LS_ERR_SHAPE: return "a size is out of range or not supported";
    case LS_ERR_DTYPE: return "dtype must be LS_F32 or LS_BF16";
    case LS_ERR_WORKSPACE: return "workspace missing or too small";
    case LS_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case LS_ERR_HIP: return "the HIP runtime reported an error at launch";
    case LS_ERR_SCRATCH:
      return "the call needs more scratch than the allocation-free entry point's static buffer";
  }
  return "unknown status";
}

size_t ls_workspace_bytes(const ls_dims* dims, int32_t max_L0) {
  if (check_dims(dims) != LS_OK) return 0;
  return size_t(ls::ws_layout(*dims, max_L0 < 1 ? 1 : max_L0).total);
}

ls_status ls_summary_init(const ls_dims* dims, const ls_state* state, const void* k_prefix,
                          const void* v_prefix, int32_t L0, int64_t prefix_rows_stride,
                          ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  if (L0 < 1 || prefix_rows_stride < L0) return LS_ERR_SHAPE;
  st = check_state(state, *dims, L0);
  if (st != LS_OK) return st;
  if (!k_prefix || !v_prefix) return LS_ERR_NULL;
  if (!aligned16(k_prefix) || !aligned16(v_prefix)) return LS_ERR_ALIGN;
  return ls::launch_init(*dims, *state, k_prefix, v_prefix, L0, prefix_rows_stride,
                         static_cast<hipStream_t>(stream));
}

ls_status ls_verify_greedy(const ls_dims* dims, const void* logits, const int32_t* draft,
                           int32_t* target_tok, int32_t* tau, void* workspace,
                           size_t workspace_bytes, ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  if (!logits || !draft || !target_tok || !tau || !workspace) return LS_ERR_NULL;
  if (!aligned16(workspace)) return LS_ERR_ALIGN;
  if (workspace_bytes < size_t(ls::ws_layout(*dims, 1).total)) return LS_ERR_WORKSPACE;
  return ls::launch_verify(*dims, logits, draft, target_tok, tau, static_cast<char*>(workspace),
                           static_cast<hipStream_t>(stream));
}

ls_status ls_draft_argmax(const ls_dims* dims, const void* logits, int32_t* draft_tok,
                          void* workspace, size_t workspace_bytes, ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  if (!logits || !draft_tok || !workspace) return LS_ERR_NULL;
  if (!aligned16(workspace)) return LS_ERR_ALIGN;
  if (workspace_bytes < size_t(ls::ws_layout(*dims, 1).total)) return LS_ERR_WORKSPACE;
  return ls::launch_argmax(*dims, logits, draft_tok, static_cast<char*>(workspace),
                           static_cast<hipStream_t>(stream));
}

ls_status ls_gather_boundary(const ls_dims* dims, const void* hidden, int32_t H,
                             const int32_t* tau, void* out, int32_t* err_flag, ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  if (!hidden || !tau || !out) return LS_ERR_NULL;
  if (H < 1) return LS_ERR_SHAPE;
  return ls::launch_boundary(*dims, hidden, H, tau, out, err_flag, static_cast<hipStream_t>(stream));
}

ls_status ls_verify_attention(const ls_dims* dims, const void* k_cache, const void* v_cache,
                              int64_t rows_stride, const int32_t* L, int32_t max_rows,
                              const void* q, void* out, void* workspace, size_t workspace_bytes,
                              int32_t* err_flag, ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  if (!k_cache || !v_cache || !L || !q || !out || !workspace) return LS_ERR_NULL;
  if (max_rows < dims->B + 1 || rows_stride < max_rows) return LS_ERR_SHAPE;
  if (dims->dtype == LS_BF16 && ls::attn_query_rows(*dims) > 128) return LS_ERR_SHAPE;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(out) ||
      !aligned16(workspace))
    return LS_ERR_ALIGN;
  if (workspace_bytes < size_t(ls::ws_layout(*dims, max_rows - dims->B - 1).total))
    return LS_ERR_WORKSPACE;
  return ls::launch_verify_attention(*dims, k_cache, v_cache, rows_stride, L, max_rows, q, out,
                                     static_cast<char*>(workspace), err_flag,
                                     static_cast<hipStream_t>(stream));
}

ls_status ls_verify_sampling(const ls_dims* dims, const void* target_logits,
                             const void* draft_logits, const int32_t* draft, float temperature,
                             const float* u_accept, const float* u_sample, int32_t* tokens,
                             int32_t* tau, void* workspace, size_t workspace_bytes,
                             ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  if (!target_logits || !draft_logits || !draft || !u_accept || !u_sample || !tokens || !tau ||
      !workspace)
    return LS_ERR_NULL;
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return LS_ERR_SHAPE;
  if (!aligned16(workspace)) return LS_ERR_ALIGN;
  if (workspace_bytes < size_t(ls::ws_layout(*dims, 1).total)) return LS_ERR_WORKSPACE;
  return ls::launch_sampling(*dims, target_logits, draft_logits, draft, temperature, u_accept,
                             u_sample, tokens, tau, static_cast<char*>(workspace),
                             static_cast<hipStream_t>(stream));
}

ls_status ls_append_accepted(const ls_dims* dims, const ls_state* state, const void* k_new,
                             const void* v_new, const int32_t* tau, ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  st = check_state(state, *dims, 1);
  if (st != LS_OK) return st;
  if (!k_new || !v_new || !tau) return LS_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return LS_ERR_ALIGN;
  return ls::launch_append(*dims, *state, k_new, v_new, tau, static_cast<hipStream_t>(stream));
}

ls_status ls_verify_append(const ls_dims* dims, const ls_state* state, const void* logits,
                           const int32_t* draft, int32_t* target_tok, int32_t* tau,
                           const void* k_new, const void* v_new, ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  st = check_state(state, *dims, 1);
  if (st != LS_OK) return st;
  if (!logits || !draft || !target_tok || !tau || !k_new || !v_new) return LS_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return LS_ERR_ALIGN;
  return ls::launch_verify_append(*dims, *state, logits, draft, target_tok, tau, k_new, v_new,
                                  static_cast<hipStream_t>(stream));
}

ls_status ls_verify_append_draft(const ls_dims* dims, const ls_state* state, const void* logits,
                                 const int32_t* draft, int32_t* target_tok, int32_t* tau,
                                 const void* k_new, const void* v_new, const void* q,
                                 const void* k_blk, const void* v_blk, void* out,
                                 ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  st = check_state(state, *dims, 1);
  if (st != LS_OK) return st;
  if (!logits || !draft || !target_tok || !tau || !k_new || !v_new || !q || !k_blk || !v_blk || !out)
    return LS_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(k_blk) ||
      !aligned16(v_blk) || !aligned16(out))
    return LS_ERR_ALIGN;
  return ls::launch_verify_append_draft(*dims, *state, logits, draft, target_tok, tau, k_new, v_new,
                                        q, k_blk, v_blk, out, static_cast<hipStream_t>(stream));
}

ls_status ls_verify_keys(const ls_dims* dims, const ls_state* state, const void* logits,
                         ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  st = check_state(state, *dims, 1);
  if (st != LS_OK) return st;
  if (!logits) return LS_ERR_NULL;
  return ls::launch_round_keys(*dims, *state, logits, static_cast<hipStream_t>(stream));
}

ls_status ls_update_draft(const ls_dims* dims, const ls_state* state, const int32_t* draft,
                          int32_t* target_tok, int32_t* tau, const void* k_new, const void* v_new,
                          const void* q, const void* k_blk, const void* v_blk, void* out,
                          ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  st = check_state(state, *dims, 1);
  if (st != LS_OK) return st;
  if (!draft || !target_tok || !tau || !k_new || !v_new || !q || !k_blk || !v_blk || !out)
    return LS_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(k_blk) ||
      !aligned16(v_blk) || !aligned16(out))
    return LS_ERR_ALIGN;
  return ls::launch_update_draft(*dims, *state, draft, target_tok, tau, k_new, v_new, q, k_blk, v_blk,
                                 out, static_cast<hipStream_t>(stream));
}

ls_status ls_draft_attention(const ls_dims* dims, const ls_state* state, const void* q,
                             const void* k_blk, const void* v_blk, void* out, ls_stream stream) {
  ls_status st = check_dims(dims);
  if (st != LS_OK) return st;
  st = check_state(state, *dims, 1);
  if (st != LS_OK) return st;
  if (!q || !k_blk || !v_blk || !out) return LS_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(out))
    return LS_ERR_ALIGN;
  return ls::launch_draft(*dims, *state, q, k_blk, v_blk, out, static_cast<hipStream_t>(stream));
}

}  // extern "C"
