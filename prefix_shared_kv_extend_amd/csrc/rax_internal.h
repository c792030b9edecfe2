// Declarations shared between librax's host glue (rax_api.cpp) and its device code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rax.h"

namespace raxk {

// Decode-step write-back batch, passed to the kernel by value.
constexpr int kAppendMax = 256;
struct AppendBatch {
  int32_t n;
  int32_t slot[kAppendMax];
  int32_t len[kAppendMax];
};

// A decode step's write-back carried by the first decode-attention kernel (see
// rax_decode_step), passed by value: each new token's K/V row goes to its slot, the slot
// to its req_to_token row at position len - 1, and len to seq_len_dev.
struct AppendJob {
  const void* k_new;
  const void* v_new;
  int32_t* seq_len_dev;
  int64_t chunks_per_row;  // 16-byte chunks per K (or V) row
  int32_t n;               // tokens (0: no append)
  int32_t slot[kAppendMax];
  int32_t len[kAppendMax];  // lengths after the step
};

// Whether decode attention with these sizes starts with the kernel that can carry an
// AppendJob (bf16, D = 128, split decode, batch <= kAppendMax).
bool decode_folds_append(int32_t batch, int32_t h_q, int32_t h_kv, int32_t d, rax_dtype dt);

// Work list of the own-part workgroups (own_stream_kernel), from host copies of the
// lengths and hints: requests by descending own keys, each request's chunks (and in a
// chunk its KV heads) together, so that the longest start first and the shortest fill the
// end of the launch. Request req[i] gets cum[i + 1] - cum[i] chunk items, counted from its
// own keys by the kernels' rule (decode_hint); the kernel flags a request whose own keys
// need more, and items past its count exit at once. n = 0 (or n != batch): none, the
// kernel covers n_chunk items per request in batch order.
struct OwnOrder {
  int32_t n = 0;
  int32_t all_own = 0;  // every request has own keys (the own part then writes every row of O)
  uint16_t req[kAppendMax];
  uint16_t cum[kAppendMax + 1];
};
// What the host knows of a decode batch from host copies of its lengths and hints
// (decode_hint); zeros: nothing, the layout follows the longest sequence.
struct DecodeHint {
  int32_t tiles = 0;  // the most 64-key tiles the shared-prefix part of any row block computes
  int32_t own = 0;    // the most own keys of any request (past its block's or run's shared keys)
  OwnOrder order;     // requests by descending own keys (batch <= kAppendMax); cum set at launch
  int32_t own_keys[kAppendMax];  // per request: its own keys after the step's append
};

// rax_decode_attention, with an optional append carried by its first kernel (seq_len is
// then read from the job, not from memory, by that kernel) and an optional hint that
// sizes the launches (results unchanged).
rax_status decode_attention_impl(const void* q, const void* k_pool, const void* v_pool, int64_t num_slots,
                                 const int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                 const int32_t* req_pool_idx, const int32_t* seq_len, const int32_t* shared_len,
                                 int32_t batch, int32_t max_seq_len, int32_t h_q, int32_t h_kv, int32_t d,
                                 float sm_scale, rax_dtype dt, void* o, rax_dtype o_dt, void* workspace,
                                 size_t ws_bytes, void* stream, const AppendJob* ap, DecodeHint hint = {});

// Workspace bytes of a decode call laid out with the hint.
size_t decode_workspace_bytes(int64_t batch, int32_t h_q, int32_t h_kv, int32_t d, int32_t max_seq_len,
                              DecodeHint hint);

// From host copies of the lengths before a decode step's append (len) and the shared_len
// hints, by the rule of the decode kernels (block shared length, then deeper runs up to
// their per-block cap), for the lengths after the append.
DecodeHint decode_hint(const int32_t* len, const int32_t* shared_len, int32_t batch, int32_t h_q, int32_t h_kv,
                       int32_t max_seq_len);

// One launch of the move kernel: n (src, dst) slot pairs, each dst written once.
constexpr int kMoveMax = 256;
struct MoveBatch {
  int32_t n;
  int32_t src[kMoveMax];
  int32_t dst[kMoveMax];
};

// Device-visible address of pinned host memory; hipErrorInvalidValue-like failures -> false.
bool host_device_ptr(const void* host, void** dev);

// Runs moves (kind 0: device slot -> host slot, 1: host slot -> device slot) in the
// given order: consecutive moves of one kind form one phase; within a phase a later
// move to the same destination supersedes an earlier one.
rax_status launch_kv_moves(const int32_t* kind, const int32_t* src, const int32_t* dst, int64_t n, void* k_pool,
                           void* v_pool, void* k_host_dev, void* v_host_dev, int64_t chunks_per_row, hipStream_t st);

rax_status launch_decode_append(int32_t batch, const int32_t* slots, const int32_t* lens,
                                const int32_t* req_pool_idx, int32_t* seq_len_dev, int32_t* rtt, int64_t stride,
                                int64_t rows, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                int64_t chunks_per_row, hipStream_t st);

}  // namespace raxk
