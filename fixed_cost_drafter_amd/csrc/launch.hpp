// Internal launchers, one per kernel family.  The C ABI (abi.cpp) validates
// arguments and calls these; they compute launch shapes and enqueue kernels
// on `stream`, never synchronising and never allocating.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/longspark.h"

namespace ls {

// the sizes every entry point validates (abi.cpp): LS_OK or the status to return
ls_status check_dims(const ls_dims* d);

ls_status launch_verify(const ls_dims& d, const void* logits, const int32_t* draft,
                        int32_t* target_tok, int32_t* tau, char* ws, hipStream_t stream);

// the same, with the C*(B+1)*verify_splits(d) partial keys at `keys`
ls_status launch_verify_into(const ls_dims& d, const void* logits, const int32_t* draft,
                             int32_t* target_tok, int32_t* tau, uint64_t* keys,
                             hipStream_t stream);

// the verification's partial argmax keys only (into the workspace's key area);
// the same launch copies seq_len into len_snap when len_snap is not null, and
// then zeroes the arrival counters (arrivals_per_seq per sequence) when
// arrivals is not null
ls_status launch_verify_keys(const ls_dims& d, const void* logits, char* ws,
                             const int32_t* seq_len, int32_t* len_snap, hipStream_t stream,
                             int32_t* arrivals = nullptr);

// greedy verification, then the append of the accepted rows (tau derived by
// the append from the partial keys in st.workspace)
ls_status launch_verify_append(const ls_dims& d, const ls_state& st, const void* logits,
                               const int32_t* draft, int32_t* target_tok, int32_t* tau,
                               const void* k_new, const void* v_new, hipStream_t stream);

// drafter proposal at T = 0: argmax over V of each of the C*B rows
ls_status launch_argmax(const ls_dims& d, const void* logits, int32_t* draft_tok, char* ws,
                        hipStream_t stream);

// boundary state: row tau[c]-1 of each sequence's [B+1, H] states
ls_status launch_boundary(const ls_dims& d, const void* hidden, int32_t H, const int32_t* tau,
                          void* out, int32_t* err_flag, hipStream_t stream);

// target verification attention of the B+1 verified positions over L + B + 1 rows
ls_status launch_verify_attention(const ls_dims& d, const void* k_cache, const void* v_cache,
                                  int64_t rows_stride, const int32_t* L, int32_t max_rows,
                                  const void* q, void* out, char* ws, int32_t* err_flag,
                                  hipStream_t stream);

// sampled (speculative) verification of a drafted block
ls_status launch_sampling(const ls_dims& d, const void* target_logits, const void* draft_logits,
                          const int32_t* draft, float temperature, const float* u_accept,
                          const float* u_sample, int32_t* tokens, int32_t* tau, char* ws,
                          hipStream_t stream);

ls_status launch_append(const ls_dims& d, const ls_state& st, const void* k_new,
                        const void* v_new, const int32_t* tau, hipStream_t stream);

ls_status launch_init(const ls_dims& d, const ls_state& st, const void* k_prefix,
                      const void* v_prefix, int32_t L0, int64_t rows_stride,
                      hipStream_t stream);

ls_status launch_draft(const ls_dims& d, const ls_state& st, const void* q, const void* k_blk,
                       const void* v_blk, void* out, hipStream_t stream);

// the verification's second half over the keys in the workspace
// (target_tok, tau)
ls_status launch_verify_finalize(const ls_dims& d, const int32_t* draft, int32_t* target_tok,
                                 int32_t* tau, const char* ws, hipStream_t stream);
// the update over the keys in the workspace (a key pass took the snapshot):
// tau and target_tok derived on the way, as in launch_verify_append
ls_status launch_append_from_keys(const ls_dims& d, const ls_state& st, const int32_t* draft,
                                  int32_t* target_tok, int32_t* tau, const void* k_new,
                                  const void* v_new, hipStream_t stream);

// a whole round: the key pass (round_keys: partial keys, length snapshot,
// zeroed arrival counters), then update + draft attention (update_draft: one
// launch where round_fusable, else the separate entry points' launches)
bool round_fusable(const ls_dims& d);
ls_status launch_round_keys(const ls_dims& d, const ls_state& st, const void* logits,
                            hipStream_t stream);
ls_status launch_update_draft(const ls_dims& d, const ls_state& st, const int32_t* draft,
                              int32_t* target_tok, int32_t* tau, const void* k_new,
                              const void* v_new, const void* q, const void* k_blk,
                              const void* v_blk, void* out, hipStream_t stream);
ls_status launch_verify_append_draft(const ls_dims& d, const ls_state& st, const void* logits,
                                     const int32_t* draft, int32_t* target_tok, int32_t* tau,
                                     const void* k_new, const void* v_new, const void* q,
                                     const void* k_blk, const void* v_blk, void* out,
                                     hipStream_t stream);

}  // namespace ls
