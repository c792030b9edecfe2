// QKV projection of new tokens on MFMA, fused with their KV write-back (bf16, fp32 sums).
//
// The step before attention: every new token's hidden state x (row of [T, hidden]) is
// mapped to its query, key and value, y = x W^T with W [(h_q + 2 h_kv) d, hidden]; the
// output features are Q, then K, then V, head-major (hustzhy SGLang post, §2.3 (2): only
// the unmatched suffix is computed; 2312.07104_SGLang notes, App. A.1: the new tokens'
// KV is what the cache keeps). The epilogue writes Q to q_out, K and V to the
// contiguous suffix buffers that extend attention reads and, optionally, in the same pass
// to the pool slots out_loc[t], in place of the separate write-back (kv_scatter) and its
// re-read of the suffix buffers. Measured on the few-shot batch (3150 tokens, hidden
// 4096, 32 heads x 128), the fused write-back is slower: 430 us against 364 us for the
// projection alone plus 17 us for kv_scatter. The output tiling splits every token's
// pool row into one 256-byte piece per head, written by different workgroups at
// different times, whereas kv_scatter writes each 8 KB row in one go.
//
// Tiling: a workgroup computes a 128-token x 128-feature output tile with 4 waves (each
// 64 x 64 = 2 x 2 MFMA tiles of 32 x 32), k in steps of 64. Both operands are
// k-contiguous rows (tokens of x, features of W), loaded straight into LDS with 16-byte
// global-to-LDS loads, double-buffered; one load instruction fills 8 rows of 128 bytes,
// whose 16-byte chunk positions are XOR-swizzled by (r % 8) ^ ((r / 8) % 2) so that the
// fragment reads (32 rows x 2 chunks) are free of bank conflicts for 128 and 256 bytes
// of banks. C = A B^T on v_mfma_f32_32x32x16_bf16 with A = token rows, B = feature rows.
// Epilogue: the bf16 output tile goes through LDS (rows padded to 272 bytes), then every
// thread writes 16-byte chunks of token rows, looking up each row's slot once: Q chunks
// to q_out, K and V chunks to the contiguous buffers and to the pool rows.
#include "../../../include/rax.h"
#include "rax_device.h"

namespace raxk {

constexpr int kPM = 128, kPN = 128, kPK = 64;

__device__ __forceinline__ int pswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__global__ void __launch_bounds__(256) qkv_kernel(const __bf16* __restrict__ x, const __bf16* __restrict__ w,
                                                  int64_t t_rows, int hidden, int n_q, int n_kv,
                                                  const int32_t* __restrict__ out_loc, int64_t num_slots,
                                                  __bf16* __restrict__ q_out, __bf16* __restrict__ k_ext,
                                                  __bf16* __restrict__ v_ext, __bf16* __restrict__ k_pool,
                                                  __bf16* __restrict__ v_pool) {
  constexpr int kTile = kPM * kPK * 2;  // bytes of one operand tile
  __shared__ __align__(16) char smem[4 * kTile];
  char(*sa)[kTile] = reinterpret_cast<char(*)[kTile]>(smem);              // token rows, 128 B each
  char(*sb)[kTile] = reinterpret_cast<char(*)[kTile]>(smem + 2 * kTile);  // feature rows
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;  // this wave's 64 x 64 quadrant
  const int jrow = lane & 31, half = lane >> 5;
  // feature blocks vary fastest: a token block's rows of x are read by workgroups that run
  // at about the same time (measured 1.13x faster than token blocks fastest)
  const int64_t m0 = (int64_t)blockIdx.y * kPM;
  const int n0 = blockIdx.x * kPN;
  __shared__ int32_t s_slot[kPM];
  // the tile's slot ids, fetched now and parked in LDS by the epilogue (one per thread)
  const int32_t my_slot = out_loc && tid < kPM && m0 + tid < t_rows ? out_loc[m0 + tid] : -1;

  // k-step ks into buffer b: 16 instructions per operand tile, wave w issues w, w + 4, ...
  // (token rows past t_rows read the last row; their results are not stored)
  auto issue = [&](int ks, int b) {
    const int k0 = ks * kPK;
#pragma unroll
    for (int q = wave; q < 16; q += 4) {
      const int r = q * 8 + (lane >> 3);
      const int cs = (lane & 7) ^ pswz(r);
      const int64_t mr = m0 + r < t_rows ? m0 + r : t_rows - 1;
      lds_load16(x + mr * hidden + k0 + cs * 8, uni32(lds_addr(&sa[b][0]) + q * 1024));
      lds_load16(w + (int64_t)(n0 + r) * hidden + k0 + cs * 8, uni32(lds_addr(&sb[b][0]) + q * 1024));
    }
  };
  auto frag = [&](const char* base, int r, int kk) {
    return *reinterpret_cast<const bf16x8*>(base + r * 128 + (((2 * kk + half) ^ pswz(r)) * 16));
  };

  f32x16 c[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) c[i][j] = f32x16{};
  const int nks = hidden / kPK;
  // the loads are asm (see lds_load16): __syncthreads does not wait for them, so each wave
  // waits for its own with s_waitcnt before every barrier
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int b = ks & 1;
    if (ks + 1 < nks) issue(ks + 1, b ^ 1);
#pragma unroll
    for (int kk = 0; kk < kPK / 16; ++kk) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = frag(&sa[b][0], wm * 64 + i * 32 + jrow, kk);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = frag(&sb[b][0], wn * 64 + j * 32 + jrow, kk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], c[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // next buffer loaded by every wave; this one read by every wave
  }

  // register r of tile (i, j): token wm*64 + i*32 + 8*(r/4) + 4*half + r%4, feature
  // wn*64 + j*32 + l%32 of the workgroup's tile; into LDS as bf16 (the operand buffers
  // are free after the loop's last barrier)
  constexpr int kRow = kPN * 2 + 16;  // padded row bytes
  static_assert(kPM * kRow <= (int)sizeof(smem), "output tile");
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const int n = wn * 64 + j * 32 + jrow;
        *reinterpret_cast<__bf16*>(smem + m * kRow + n * 2) = (__bf16)c[i][j][r];
      }
  if (tid < kPM) s_slot[tid] = my_slot;
  __syncthreads();
  // 128 rows x 16 chunks of 8 features; chunk boundaries never straddle Q / K / V (their
  // sizes are multiples of d, and d of 8)
  for (int e = tid; e < kPM * (kPN / 8); e += 256) {
    const int rr = e >> 4, ch = e & 15;
    const int64_t m = m0 + rr;
    if (m >= t_rows) continue;
    const u32x4 val = *reinterpret_cast<const u32x4*>(smem + rr * kRow + ch * 16);
    const int n = n0 + ch * 8;
    if (n < n_q) {
      *reinterpret_cast<u32x4*>(q_out + m * n_q + n) = val;
    } else {
      const bool is_k = n < n_q + n_kv;
      const int f = is_k ? n - n_q : n - n_q - n_kv;
      *reinterpret_cast<u32x4*>((is_k ? k_ext : v_ext) + m * n_kv + f) = val;
      if (out_loc) {
        const int64_t sl = s_slot[rr];
        if (sl >= 0 && sl < num_slots) *reinterpret_cast<u32x4*>((is_k ? k_pool : v_pool) + sl * n_kv + f) = val;
        else if (f == 0) flag_error(RAX_DEVERR_SLOT);
      }
    }
  }
}

}  // namespace raxk

extern "C" rax_status rax_qkv_project(const void* x, const void* w, int64_t n_tok, int32_t hidden, int32_t h_q,
                                      int32_t h_kv, int32_t d, rax_dtype dt, void* q_out, void* k_ext, void* v_ext,
                                      const int32_t* out_loc, void* k_pool, void* v_pool, int64_t num_slots,
                                      void* stream) {
  if (n_tok < 0 || hidden < 1 || h_q < 1 || h_kv < 1 || d < 8 || d % 8 || dt != RAX_BF16) return RAX_EINVAL;
  const int64_t n_out = (int64_t)(h_q + 2 * h_kv) * d;
  if (hidden % raxk::kPK || n_out % raxk::kPN || n_out > INT32_MAX || (int64_t)h_q * d > INT32_MAX) return RAX_EINVAL;
  if (n_tok == 0) return RAX_OK;
  if (!x || !w || !q_out || !k_ext || !v_ext) return RAX_EINVAL;
  if (out_loc && (!k_pool || !v_pool || num_slots < 1)) return RAX_EINVAL;
  if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)q_out | (uintptr_t)k_ext | (uintptr_t)v_ext |
       (uintptr_t)(out_loc ? k_pool : nullptr) | (uintptr_t)(out_loc ? v_pool : nullptr)) & 15)
    return RAX_EINVAL;
  const int64_t m_blocks = (n_tok + raxk::kPM - 1) / raxk::kPM;
  if (m_blocks > 65535) return RAX_EINVAL;
  const dim3 grid((unsigned)(n_out / raxk::kPN), (unsigned)m_blocks);
  hipLaunchKernelGGL(raxk::qkv_kernel, grid, dim3(256), 0, (hipStream_t)stream, (const __bf16*)x, (const __bf16*)w,
                     n_tok, hidden, h_q * d, h_kv * d, out_loc, num_slots, (__bf16*)q_out, (__bf16*)k_ext,
                     (__bf16*)v_ext, (__bf16*)k_pool, (__bf16*)v_pool);
  return hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
}
