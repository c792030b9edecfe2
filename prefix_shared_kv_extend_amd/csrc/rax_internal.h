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
