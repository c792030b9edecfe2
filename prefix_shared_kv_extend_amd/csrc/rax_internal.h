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

rax_status launch_decode_append(int32_t batch, const int32_t* slots, const int32_t* lens,
                                const int32_t* req_pool_idx, int32_t* seq_len_dev, int32_t* rtt, int64_t stride,
                                int64_t rows, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                int64_t chunks_per_row, hipStream_t st);

}  // namespace raxk
