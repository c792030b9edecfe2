// KV write-back into the token-granular pool, and req_to_token row fill.
//
// Write-back: the KV computed for new tokens is kept in the pool so that later
// requests sharing the prefix reuse it (bowenzhou SGLang review, "Work loop":
// insert; 2312.07104_SGLang notes, §3, one page per token). Each pool slot holds
// one token's K (or V) for all KV heads: [num_slots, h_kv, d].
//
// Both kernels are pure data movement (HBM-bound): 16-byte vector loads and
// stores, one token row of h_kv*d elements handled by consecutive lanes so reads
// and writes are coalesced.
#include "../../../include/rax.h"
#include "rax_device.h"
#include <unordered_set>
#include <vector>

#include "../rax_internal.h"

namespace raxk {

__device__ int32_t g_rax_err = 0;

// One thread moves one 16-byte chunk of one token row, for K and for V; blocks b of nb
// of a grid-stride loop.
__device__ __forceinline__ void kv_scatter_part(const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                                                const int32_t* __restrict__ out_loc, int64_t n_tok,
                                                uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                                int64_t num_slots, int64_t chunks_per_row, int64_t b, int64_t nb) {
  const int64_t total = n_tok * chunks_per_row;
  for (int64_t i = b * 256 + threadIdx.x; i < total; i += nb * 256) {
    const int64_t tok = i / chunks_per_row;
    const int64_t c = i - tok * chunks_per_row;
    const int32_t slot = out_loc[tok];
    if (slot < 0 || slot >= num_slots) {
      if (c == 0) flag_error(RAX_DEVERR_SLOT);
      continue;
    }
    const int64_t dst = (int64_t)slot * chunks_per_row + c;
    k_pool[dst] = k_new[i];
    v_pool[dst] = v_new[i];
  }
}

// One thread writes one req_to_token entry: entry e of the concatenated sources goes to
// row req_pool_idx[r], column start[r] + e - indptr[r] of its request r; blocks b of nb.
__device__ __forceinline__ void rtt_write_part(int32_t* __restrict__ rtt, int64_t stride, int64_t rows,
                                               const int32_t* __restrict__ req_pool_idx,
                                               const int32_t* __restrict__ start,
                                               const int32_t* __restrict__ indptr, const int32_t* __restrict__ src,
                                               int32_t batch, int64_t total, int64_t b, int64_t nb) {
  for (int64_t e = b * 256 + threadIdx.x; e < total; e += nb * 256) {
    // request owning entry e: last r with indptr[r] <= e
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (indptr[mid] <= e) lo = mid;
      else hi = mid - 1;
    }
    const int64_t row = req_pool_idx[lo];
    const int64_t col = (int64_t)start[lo] + (e - indptr[lo]);
    if (row < 0 || row >= rows || col < 0 || col >= stride) {
      flag_error(RAX_DEVERR_ROW);
      continue;
    }
    rtt[row * stride + col] = src[e];
  }
}

__global__ void __launch_bounds__(256) kv_scatter_kernel(const uint4* __restrict__ k_new,
                                                         const uint4* __restrict__ v_new,
                                                         const int32_t* __restrict__ out_loc, int64_t n_tok,
                                                         uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                                         int64_t num_slots, int64_t chunks_per_row) {
  kv_scatter_part(k_new, v_new, out_loc, n_tok, k_pool, v_pool, num_slots, chunks_per_row, blockIdx.x, gridDim.x);
}

__global__ void __launch_bounds__(256) rtt_write_kernel(int32_t* __restrict__ rtt, int64_t stride, int64_t rows,
                                                        const int32_t* __restrict__ req_pool_idx,
                                                        const int32_t* __restrict__ start,
                                                        const int32_t* __restrict__ indptr,
                                                        const int32_t* __restrict__ src, int32_t batch,
                                                        int64_t total) {
  rtt_write_part(rtt, stride, rows, req_pool_idx, start, indptr, src, batch, total, blockIdx.x, gridDim.x);
}

// An extend call's two write-backs in one launch: the first g_rtt blocks fill the
// requests' req_to_token rows, the others write the new tokens' K/V rows into the pools.
// The two touch different arrays, so their blocks need no order.
__global__ void __launch_bounds__(256) extend_write_kernel(int32_t* __restrict__ rtt, int64_t stride, int64_t rows,
                                                           const int32_t* __restrict__ req_pool_idx,
                                                           const int32_t* __restrict__ start,
                                                           const int32_t* __restrict__ indptr,
                                                           const int32_t* __restrict__ src, int32_t batch,
                                                           int64_t total, int32_t g_rtt,
                                                           const uint4* __restrict__ k_new,
                                                           const uint4* __restrict__ v_new,
                                                           const int32_t* __restrict__ out_loc, int64_t n_tok,
                                                           uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                                           int64_t num_slots, int64_t chunks_per_row) {
  if ((int)blockIdx.x < g_rtt)
    rtt_write_part(rtt, stride, rows, req_pool_idx, start, indptr, src, batch, total, blockIdx.x, g_rtt);
  else
    kv_scatter_part(k_new, v_new, out_loc, n_tok, k_pool, v_pool, num_slots, chunks_per_row, blockIdx.x - g_rtt,
                    gridDim.x - g_rtt);
}

// Decode step write-back: for request i of the batch, its new slot b.slot[i] goes to
// req_to_token[req_pool_idx[i]][b.len[i] - 1], b.len[i] to seq_len_dev[i], and the K/V
// rows of its new token to the pools at that slot. The slots and lengths arrive as kernel
// arguments (host-computed, already validated).
__global__ void __launch_bounds__(256) decode_append_kernel(AppendBatch b, const int32_t* __restrict__ req_pool_idx,
                                                            int32_t* __restrict__ seq_len_dev,
                                                            int32_t* __restrict__ rtt, int64_t stride, int64_t rows,
                                                            const uint4* __restrict__ k_new,
                                                            const uint4* __restrict__ v_new,
                                                            uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                                            int64_t chunks_per_row) {
  const int64_t total = (int64_t)b.n * chunks_per_row;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(e / chunks_per_row);
    const int64_t c = e - (int64_t)i * chunks_per_row;
    const int64_t slot = b.slot[i];
    k_pool[slot * chunks_per_row + c] = k_new[e];
    v_pool[slot * chunks_per_row + c] = v_new[e];
    if (c == 0) {
      const int64_t row = req_pool_idx[i];
      const int32_t len = b.len[i];
      seq_len_dev[i] = len;
      if (row < 0 || row >= rows) flag_error(RAX_DEVERR_ROW);
      else rtt[row * stride + len - 1] = (int32_t)slot;
    }
  }
}

static int grid_for(int64_t work, int64_t per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

// Launch of decode_append_kernel in batches of kAppendMax requests (see rax_decode_append).
rax_status launch_decode_append(int32_t batch, const int32_t* slots, const int32_t* lens,
                                const int32_t* req_pool_idx, int32_t* seq_len_dev, int32_t* rtt, int64_t stride,
                                int64_t rows, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                int64_t chunks_per_row, hipStream_t st) {
  for (int32_t b0 = 0; b0 < batch; b0 += kAppendMax) {
    AppendBatch b;
    b.n = batch - b0 < kAppendMax ? batch - b0 : kAppendMax;
    for (int i = 0; i < b.n; ++i) {
      b.slot[i] = slots[b0 + i];
      b.len[i] = lens[b0 + i];
    }
    const int64_t off = (int64_t)b0 * chunks_per_row;
    hipLaunchKernelGGL(decode_append_kernel, dim3(grid_for(b.n * chunks_per_row, 256)), dim3(256), 0, st, b,
                       req_pool_idx + b0, seq_len_dev + b0, rtt, stride, rows,
                       reinterpret_cast<const uint4*>(k_new) + off, reinterpret_cast<const uint4*>(v_new) + off,
                       reinterpret_cast<uint4*>(k_pool), reinterpret_cast<uint4*>(v_pool), chunks_per_row);
    if (hipGetLastError() != hipSuccess) return RAX_EDEVICE;
  }
  return RAX_OK;
}

// KV moves between the device pool and the host tier (pinned host memory that the
// kernel reads and writes directly over the bus): block (i, kv) copies row src[i] of
// the source into row dst[i] of the destination, 16 bytes per lane.
__global__ void __launch_bounds__(256) kv_move_kernel(MoveBatch b, const uint4* __restrict__ k_src,
                                                      const uint4* __restrict__ v_src, uint4* __restrict__ k_dst,
                                                      uint4* __restrict__ v_dst, int64_t chunks_per_row) {
  const int i = blockIdx.x;
  const uint4* src = blockIdx.y ? v_src : k_src;
  uint4* dst = blockIdx.y ? v_dst : k_dst;
  const int64_t s = (int64_t)b.src[i] * chunks_per_row;
  const int64_t d = (int64_t)b.dst[i] * chunks_per_row;
  for (int64_t c = threadIdx.x; c < chunks_per_row; c += blockDim.x) dst[d + c] = src[s + c];
}

bool host_device_ptr(const void* host, void** dev) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, host) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (a.type != hipMemoryTypeHost || !a.devicePointer) return false;
  *dev = a.devicePointer;
  return true;
}

rax_status launch_kv_moves(const int32_t* kind, const int32_t* src, const int32_t* dst, int64_t n, void* k_pool,
                           void* v_pool, void* k_host_dev, void* v_host_dev, int64_t chunks_per_row,
                           hipStream_t st) {
  std::vector<int32_t> ps, pd;
  std::unordered_set<int32_t> seen;
  for (int64_t a = 0; a < n;) {
    int64_t e = a;
    while (e < n && kind[e] == kind[a]) ++e;
    // the phase [a, e): keep the last move to each destination, in order
    ps.clear();
    pd.clear();
    seen.clear();
    for (int64_t j = e - 1; j >= a; --j) {
      if (seen.insert(dst[j]).second) {
        ps.push_back(src[j]);
        pd.push_back(dst[j]);
      }
    }
    const bool demote = kind[a] == 0;
    const uint4* ks = reinterpret_cast<const uint4*>(demote ? k_pool : k_host_dev);
    const uint4* vs = reinterpret_cast<const uint4*>(demote ? v_pool : v_host_dev);
    uint4* kd = reinterpret_cast<uint4*>(demote ? k_host_dev : k_pool);
    uint4* vd = reinterpret_cast<uint4*>(demote ? v_host_dev : v_pool);
    const int64_t m = static_cast<int64_t>(ps.size());
    for (int64_t b0 = 0; b0 < m; b0 += kMoveMax) {
      MoveBatch b;
      b.n = static_cast<int32_t>(m - b0 < kMoveMax ? m - b0 : kMoveMax);
      for (int i = 0; i < b.n; ++i) {
        b.src[i] = ps[m - 1 - (b0 + i)];  // collected backwards
        b.dst[i] = pd[m - 1 - (b0 + i)];
      }
      hipLaunchKernelGGL(kv_move_kernel, dim3(b.n, 2), dim3(chunks_per_row < 256 ? 128 : 256), 0, st, b, ks, vs,
                         kd, vd, chunks_per_row);
      if (hipGetLastError() != hipSuccess) return RAX_EDEVICE;
    }
    a = e;
  }
  return RAX_OK;
}

}  // namespace raxk

extern "C" rax_status rax_kv_scatter(const void* k_new, const void* v_new, const int32_t* out_loc,
                                     int64_t n_tok, void* k_pool, void* v_pool, int64_t num_slots,
                                     int32_t h_kv, int32_t d, rax_dtype dt, void* stream) {
  if (n_tok < 0 || num_slots < 1 || h_kv < 1 || d < 1 || (dt != RAX_F32 && dt != RAX_BF16)) return RAX_EINVAL;
  if (n_tok == 0) return RAX_OK;
  if (!k_new || !v_new || !out_loc || !k_pool || !v_pool) return RAX_EINVAL;
  const int64_t row_bytes = (int64_t)h_kv * d * (dt == RAX_F32 ? 4 : 2);
  if (row_bytes % 16) return RAX_EINVAL;
  const uintptr_t mis = (uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_pool | (uintptr_t)v_pool;
  if (mis & 15) return RAX_EINVAL;
  const int64_t cpr = row_bytes / 16;
  hipLaunchKernelGGL(raxk::kv_scatter_kernel, dim3(raxk::grid_for(n_tok * cpr, 256)), dim3(256), 0,
                     (hipStream_t)stream, (const uint4*)k_new, (const uint4*)v_new, out_loc, n_tok,
                     (uint4*)k_pool, (uint4*)v_pool, num_slots, cpr);
  return hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
}

extern "C" rax_status rax_req_to_token_write(int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                             const int32_t* req_pool_idx, const int32_t* start,
                                             const int32_t* src_indptr, const int32_t* src_slots, int32_t batch,
                                             int64_t total, void* stream) {
  if (batch < 0 || total < 0 || rtt_stride < 1 || rtt_rows < 1) return RAX_EINVAL;
  if (batch == 0 || total == 0) return RAX_OK;
  if (!req_to_token || !req_pool_idx || !start || !src_indptr || !src_slots) return RAX_EINVAL;
  hipLaunchKernelGGL(raxk::rtt_write_kernel, dim3(raxk::grid_for(total, 256)), dim3(256), 0,
                     (hipStream_t)stream, req_to_token, rtt_stride, rtt_rows, req_pool_idx, start, src_indptr,
                     src_slots, batch, total);
  return hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
}

extern "C" rax_status rax_extend_write(int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                      const int32_t* req_pool_idx, const int32_t* start, const int32_t* src_indptr,
                                      const int32_t* src_slots, int32_t batch, int64_t total, const void* k_new,
                                      const void* v_new, const int32_t* out_loc, int64_t n_tok, void* k_pool,
                                      void* v_pool, int64_t num_slots, int32_t h_kv, int32_t d, rax_dtype dt,
                                      void* stream) {
  // each half checked as its own entry point checks it
  if (batch < 0 || total < 0 || rtt_stride < 1 || rtt_rows < 1) return RAX_EINVAL;
  if (n_tok < 0 || num_slots < 1 || h_kv < 1 || d < 1 || (dt != RAX_F32 && dt != RAX_BF16)) return RAX_EINVAL;
  const bool do_rtt = batch > 0 && total > 0, do_kv = n_tok > 0;
  if (do_rtt && (!req_to_token || !req_pool_idx || !start || !src_indptr || !src_slots)) return RAX_EINVAL;
  const int64_t row_bytes = (int64_t)h_kv * d * (dt == RAX_F32 ? 4 : 2);
  if (do_kv) {
    if (!k_new || !v_new || !out_loc || !k_pool || !v_pool || row_bytes % 16) return RAX_EINVAL;
    if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_pool | (uintptr_t)v_pool) & 15) return RAX_EINVAL;
  }
  if (!do_rtt && !do_kv) return RAX_OK;
  const int64_t cpr = row_bytes / 16;
  const int g_rtt = do_rtt ? raxk::grid_for(total, 256) : 0;
  const int g_kv = do_kv ? raxk::grid_for(n_tok * cpr, 256) : 0;
  hipLaunchKernelGGL(raxk::extend_write_kernel, dim3(g_rtt + g_kv), dim3(256), 0, (hipStream_t)stream, req_to_token,
                     rtt_stride, rtt_rows, req_pool_idx, start, src_indptr, src_slots, batch, total, g_rtt,
                     (const uint4*)k_new, (const uint4*)v_new, out_loc, do_kv ? n_tok : 0, (uint4*)k_pool,
                     (uint4*)v_pool, num_slots, cpr);
  return hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
}

extern "C" rax_status rax_device_errors(void* stream, int32_t* out_mask) {
  if (!out_mask) return RAX_EINVAL;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return RAX_EDEVICE;
  int32_t v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(raxk::g_rax_err), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess)
    return RAX_EDEVICE;
  const int32_t zero = 0;
  if (hipMemcpyToSymbol(HIP_SYMBOL(raxk::g_rax_err), &zero, sizeof(zero), 0, hipMemcpyHostToDevice) != hipSuccess)
    return RAX_EDEVICE;
  *out_mask = v;
  return RAX_OK;
}
