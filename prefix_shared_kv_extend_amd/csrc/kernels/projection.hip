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
// 4096, 32 heads x 128): 335 us fused against 318 us for the projection alone plus the
// separate write-back (340 us in all). With 256-feature tiles a token's pool row is
// written in 512-byte pieces (two heads) by different workgroups at different times,
// whereas kv_scatter writes each 8 KB row in one go, so fusing gains little.
//
// Tiling: a workgroup computes a BM-token x BN-feature output tile with WM x WN waves, each
// a (BM / WM) x (BN / WN) block of 32 x 32 MFMA tiles, k in steps of 64. Large batches
// take 256 x 256 tiles (8 waves of 128 x 64, 132 KB of LDS, one workgroup per CU): per
// k step a CU loads 64 KB for 8.4 MFLOP, half the operand traffic per flop of 128 x 128
// tiles, and a wave reads 6 fragments from LDS per 8 MFMAs instead of 4 per 4. Measured
// on the few-shot batch: 307-332 us against 412-448 us for 128 x 128 tiles in id order.
// Batches below 1024 tokens keep 128 x 128 tiles (4 waves of 64 x 64), so that small
// grids still spread over the CUs.
// A grid whose last round of resident workgroups would be at most half full (the
// few-shot batch: 624 tiles, 2.44 rounds of 256 CUs) runs that round's tiles as halves
// of BM / 2 tokens, dispatched last, so it takes about half a round: 1.26x the time of
// the library GEMM of the same shape timed in turn with it (287 against 227 us), against
// 1.33x with whole tiles only (318 against 239 us on another GPU).
// Workgroup ids go round-robin over the 8 XCDs; each XCD takes a contiguous run of the
// tile order, and that order walks groups of 8 token blocks feature block by feature
// block, so the workgroups running at once on one XCD share their operand rows in its
// L2 (128 x 128 tiles: 351 us grouped against 448 us with feature blocks fastest).
// Both operands are k-contiguous rows (tokens of x, features of W), loaded straight into
// LDS with 16-byte global-to-LDS loads, double-buffered; one load instruction fills 8
// rows of 128 bytes, whose 16-byte chunk positions are XOR-swizzled by
// (r % 8) ^ ((r / 8) % 2) so that the fragment reads (32 rows x 2 chunks) are free of bank
// conflicts. C = A B^T on v_mfma_f32_32x32x16_bf16 with A = token rows, B = feature rows.
// Epilogue: the bf16 output tile goes through LDS (rows padded by 16 bytes), then every
// thread writes 16-byte chunks of token rows, looking up each row's slot once: Q chunks
// to q_out, K and V chunks to the contiguous buffers and to the pool rows.
#include "../../../include/rax.h"
#include "rax_device.h"

namespace raxk {

constexpr int kPK = 64;             // k per step
constexpr int kPBigMinTokens = 1024;  // batches from this size take 256 x 256 tiles
constexpr int kPGroup = 8;            // token blocks per group of the tile order

__device__ __forceinline__ int pswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// LDS bytes of a BM x BN tile: two k steps of both operands, reused for the output tile
template <int BM, int BN>
constexpr int qkv_smem() {
  return 2 * (BM + BN) * kPK * 2 > BM * (BN * 2 + 16) ? 2 * (BM + BN) * kPK * 2 : BM * (BN * 2 + 16);
}

// First token and first feature of tile g of the grouped order: groups of kPGroup token
// blocks, each walked feature block by feature block, token blocks fastest.
__device__ __forceinline__ void tile_origin(int g, int tm, int tn, int bm, int bn, int64_t& m0, int& n0) {
  const int grp = g / (kPGroup * tn);
  const int m_first = grp * kPGroup;
  const int gm = min(kPGroup, tm - m_first);
  const int in = g - grp * kPGroup * tn;
  m0 = (int64_t)(m_first + in % gm) * bm;
  n0 = in / gm * bn;
}

// One BM x BN output tile at (m0, n0) computed by the workgroup's WM x WN waves.
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void qkv_tile(const __bf16* __restrict__ x, const __bf16* __restrict__ w,
                                         int64_t t_rows, int hidden, int n_q, int n_kv,
                                         const int32_t* __restrict__ out_loc, int64_t num_slots,
                                         __bf16* __restrict__ q_out, __bf16* __restrict__ k_ext,
                                         __bf16* __restrict__ v_ext, __bf16* __restrict__ k_pool,
                                         __bf16* __restrict__ v_pool, int64_t m0, int n0, char* smem,
                                         int32_t* s_slot) {
  constexpr int NW = WM * WN, NT = NW * 64;
  constexpr int kA = BM * kPK * 2, kStage = kA + BN * kPK * 2;  // operand bytes of one k step
  constexpr int kRow = BN * 2 + 16;                              // padded output row bytes
  constexpr int WTM = BM / WM, WTN = BN / WN, TI = WTM / 32, TJ = WTN / 32;
  static_assert(TI * 32 == WTM && TJ * 32 == WTN && NT >= BM, "tile shape");
  const int n_out = n_q + 2 * n_kv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave % WM, wn = wave / WM;
  const int jrow = lane & 31, half = lane >> 5;
  // the tile's slot ids, fetched now and parked in LDS by the epilogue (one per thread)
  const int32_t my_slot = out_loc && tid < BM && m0 + tid < t_rows ? out_loc[m0 + tid] : -1;

  // k step ks into buffer b: one load instruction per 8 rows, wave w issues w, w + NW, ...
  // (token rows past t_rows and feature rows past n_out read the last row; their results
  // are not stored)
  auto issue = [&](int ks, int b) {
    const int k0 = ks * kPK;
    const uint32_t sa = lds_addr(smem) + b * kStage, sb = sa + kA;
#pragma unroll
    for (int q = wave; q < BM / 8; q += NW) {
      const int r = q * 8 + (lane >> 3);
      const int cs = (lane & 7) ^ pswz(r);
      const int64_t mr = m0 + r < t_rows ? m0 + r : t_rows - 1;
      lds_load16(x + mr * hidden + k0 + cs * 8, uni32(sa + q * 1024));
    }
#pragma unroll
    for (int q = wave; q < BN / 8; q += NW) {
      const int r = q * 8 + (lane >> 3);
      const int cs = (lane & 7) ^ pswz(r);
      const int nr = n0 + r < n_out ? n0 + r : n_out - 1;
      lds_load16(w + (int64_t)nr * hidden + k0 + cs * 8, uni32(sb + q * 1024));
    }
  };
  auto frag = [&](const char* base, int r, int kk) {
    return *reinterpret_cast<const bf16x8*>(base + r * 128 + (((2 * kk + half) ^ pswz(r)) * 16));
  };

  f32x16 c[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) c[i][j] = f32x16{};
  const int nks = hidden / kPK;
  // the loads are asm (see lds_load16): __syncthreads does not wait for them, so each wave
  // waits for its own with s_waitcnt before every barrier
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int b = ks & 1;
    if (ks + 1 < nks) issue(ks + 1, b ^ 1);
    const char* sa = smem + b * kStage;
    const char* sb = sa + kA;
#pragma unroll
    for (int kk = 0; kk < kPK / 16; ++kk) {
      bf16x8 af[TI], bfr[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) af[i] = frag(sa, wm * WTM + i * 32 + jrow, kk);
#pragma unroll
      for (int j = 0; j < TJ; ++j) bfr[j] = frag(sb, wn * WTN + j * 32 + jrow, kk);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], c[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // next buffer loaded by every wave; this one read by every wave
  }

  // register r of tile (i, j): token wm*WTM + i*32 + 8*(r/4) + 4*half + r%4, feature
  // wn*WTN + j*32 + l%32 of the workgroup's tile; into LDS as bf16 (the operand buffers
  // are free after the loop's last barrier)
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const int n = wn * WTN + j * 32 + jrow;
        *reinterpret_cast<__bf16*>(smem + m * kRow + n * 2) = (__bf16)c[i][j][r];
      }
  if (tid < BM) s_slot[tid] = my_slot;
  __syncthreads();
  // BM rows x BN / 8 chunks of 8 features; chunk boundaries never straddle Q / K / V (their
  // sizes are multiples of d, and d of 8); with BN = 256 the last feature block may reach
  // past n_out (a multiple of 128): those features were computed from the last W row and
  // are not stored
  for (int e = tid; e < BM * (BN / 8); e += NT) {
    const int rr = e / (BN / 8), ch = e % (BN / 8);
    const int64_t m = m0 + rr;
    const int n = n0 + ch * 8;
    if (m >= t_rows || n >= n_out) continue;
    const u32x4 val = *reinterpret_cast<const u32x4*>(smem + rr * kRow + ch * 16);
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

// Large tiles, and the last round's tiles in two halves: the ids below 8 * per_xcd take
// whole BM x BN tiles (each XCD a contiguous run of the first n_whole tiles of the
// order); the ids above take the remaining tiles as BM / 2-token halves, dispatched last.
// When the whole tiles fill the CUs some rounds over and a partial round is left, half
// tiles run that round in about half the time (the host sets n_whole and the grid).
template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64)
    qkv_kernel(const __bf16* __restrict__ x, const __bf16* __restrict__ w, int64_t t_rows, int hidden, int n_q,
               int n_kv, const int32_t* __restrict__ out_loc, int64_t num_slots, __bf16* __restrict__ q_out,
               __bf16* __restrict__ k_ext, __bf16* __restrict__ v_ext, __bf16* __restrict__ k_pool,
               __bf16* __restrict__ v_pool, int tm, int tn, int per_xcd, int n_whole) {
  constexpr int kSmem = qkv_smem<BM, BN>() > qkv_smem<BM / 2, BN>() ? qkv_smem<BM, BN>() : qkv_smem<BM / 2, BN>();
  __shared__ __align__(16) char smem[kSmem];
  __shared__ int32_t s_slot[BM];
  const int b = (int)blockIdx.x;
  int64_t m0;
  int n0;
  if (b < 8 * per_xcd) {
    const int g = (b & 7) * per_xcd + (b >> 3);
    if (g >= n_whole) return;
    tile_origin(g, tm, tn, BM, BN, m0, n0);
    qkv_tile<BM, BN, WM, WN>(x, w, t_rows, hidden, n_q, n_kv, out_loc, num_slots, q_out, k_ext, v_ext, k_pool,
                             v_pool, m0, n0, smem, s_slot);
  } else {
    const int h = b - 8 * per_xcd;
    tile_origin(n_whole + h / 2, tm, tn, BM, BN, m0, n0);
    m0 += (h & 1) * (BM / 2);
    if (m0 >= t_rows) return;
    qkv_tile<BM / 2, BN, WM, WN>(x, w, t_rows, hidden, n_q, n_kv, out_loc, num_slots, q_out, k_ext, v_ext, k_pool,
                                 v_pool, m0, n0, smem, s_slot);
  }
}

}  // namespace raxk

extern "C" rax_status rax_qkv_project(const void* x, const void* w, int64_t n_tok, int32_t hidden, int32_t h_q,
                                      int32_t h_kv, int32_t d, rax_dtype dt, void* q_out, void* k_ext, void* v_ext,
                                      const int32_t* out_loc, void* k_pool, void* v_pool, int64_t num_slots,
                                      void* stream) {
  if (n_tok < 0 || hidden < 1 || h_q < 1 || h_kv < 1 || d < 8 || d % 8 || dt != RAX_BF16) return RAX_EINVAL;
  const int64_t n_out = (int64_t)(h_q + 2 * h_kv) * d;
  if (hidden % raxk::kPK || n_out % 128 || n_out > INT32_MAX / 2) return RAX_EINVAL;
  if (n_tok == 0) return RAX_OK;
  if (!x || !w || !q_out || !k_ext || !v_ext) return RAX_EINVAL;
  if (out_loc && (!k_pool || !v_pool || num_slots < 1)) return RAX_EINVAL;
  if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)q_out | (uintptr_t)k_ext | (uintptr_t)v_ext |
       (uintptr_t)(out_loc ? k_pool : nullptr) | (uintptr_t)(out_loc ? v_pool : nullptr)) & 15)
    return RAX_EINVAL;
  const bool big = n_tok >= raxk::kPBigMinTokens;
  const int bm = big ? 256 : 128, bn = big ? 256 : 128;
  const int64_t tm = (n_tok + bm - 1) / bm, tn = (n_out + bn - 1) / bn;
  if (tm * tn > (1 << 28)) return RAX_EINVAL;
  // workgroups resident at once (256 CUs; one 256 x 256 workgroup per CU, two 128 x 128);
  // a last round less than half full runs as half tiles
  const int64_t tiles = tm * tn, slots = big ? 256 : 512, rem = tiles % slots;
  const int64_t whole = tiles > slots && rem > 0 && 2 * rem <= slots ? tiles - rem : tiles;
  const int per = (int)((whole + 7) / 8);  // whole tiles per XCD; 8 * per ids
  const unsigned grid = (unsigned)(8 * (int64_t)per + 2 * (tiles - whole));
  auto go = [&](auto kernel, int threads) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, (hipStream_t)stream, (const __bf16*)x,
                       (const __bf16*)w, n_tok, hidden, h_q * d, h_kv * d, out_loc, num_slots, (__bf16*)q_out,
                       (__bf16*)k_ext, (__bf16*)v_ext, (__bf16*)k_pool, (__bf16*)v_pool, (int)tm, (int)tn, per,
                       (int)whole);
  };
  if (big) go(raxk::qkv_kernel<256, 256, 2, 4>, 512);
  else go(raxk::qkv_kernel<128, 128, 2, 2>, 256);
  return hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
}
