// Extend and decode attention over a radix-cached, token-granular KV pool (gfx950).
//
// What is computed (2312.07104_SGLang notes, §3 and App. A.1; hustzhy SGLang post,
// §2.3 (2)): for a query token at absolute position p of a request, softmax
// attention over the K/V of positions 0..p. Positions below the request's matched
// prefix length are reused from the pool, read through the request's req_to_token
// row (one slot per token); in extend, the new suffix tokens' K/V come from the
// contiguous k_ext / v_ext rows under a causal mask. Decode is the same with one
// query per request and every key read from the pool.
//
// Kernel design (one kernel template for both; MI355X-specific choices):
//  * A workgroup of NW waves owns BM = NW * RT * 32 "MFMA rows"; each wave holds RT
//    row tiles of 32. A row is a (query token, query head) pair; the h_q / h_kv query
//    heads that share a KV head are packed into consecutive rows, so each K/V tile
//    staged in LDS serves all of them (grouped-query attention). Rows of consecutive
//    requests are packed into one block, so a block can span several requests.
//    RT = 2 lets every K/V fragment read from LDS feed two MFMA row tiles, halving
//    LDS traffic per flop.
//  * The block's keys form a list of 64-key tiles: first the positions that all of
//    its requests share (same slots; bounded by the shared_len hint), loaded once for
//    every row; then each request's own remaining prefix positions (only the wave(s)
//    holding that request's rows run the MFMAs); then, in extend, the suffix keys of
//    the block's requests from k_ext under a block-diagonal causal mask.
//  * Software pipeline, one barrier per tile: while the waves run the MFMAs of tile
//    t from one LDS buffer, every thread already has the 16-byte global loads of
//    tile t+1 in flight (slot ids of tile t+2 too); after the MFMAs it writes them to
//    the other LDS buffer. Gathers are slot by slot, 16 lanes per 256-byte token
//    row (coalesced within the row). K is stored row-major with a 16-byte row pad,
//    V transposed (d-major) with an 8-byte pad: MFMA operand reads are free of bank
//    conflicts.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (fp32: v_mfma_f32_32x32x2_f32): each lane
//    owns one query row, so the softmax row max and sum are in-lane reductions plus
//    one cross-half exchange. O^T = V^T P^T accumulates in fp32; P stays in
//    registers (the contraction index is permuted consistently in both operands).
//  * Online softmax in the log2 domain (scale * log2 e folded into the scores);
//    full unmasked tiles skip the mask; the accumulator rescale is skipped when no
//    row's running maximum grew (exactly the same result).
//  * Split-K: the tile list is divided into nsplit ranges (decode needs it to fill
//    256 CUs); partial (m, l, acc) go to a workspace and a merge kernel combines
//    them by log-sum-exp. With nsplit == 1 the block writes O directly.
//  * Workgroup ids are remapped so that the blocks of one KV head run on one XCD and
//    share its L2 for the prefix tiles they all read.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <numeric>
#include <type_traits>
#include <vector>

#include "../../../include/rax.h"
#include "../rax_internal.h"
#include "rax_device.h"

namespace raxk {

constexpr int BN = 64;  // keys per tile
constexpr float kNegInf = -INFINITY;
constexpr float kLazy = 8.f;  // log2 headroom of the lazy softmax rescale

struct AttnArgs {
  const void* q;
  const void* k_ext;
  const void* v_ext;
  const void* k_pool;
  const void* v_pool;
  int64_t num_slots;
  const int32_t* rtt;
  int64_t rtt_stride;
  int64_t rtt_rows;
  const int32_t* req_pool_idx;
  const int32_t* kv_len;      // keys read from the pool per request (prefix_len or seq_len)
  const int32_t* qo_indptr;   // extend only: query rows of request r
  const int32_t* shared_len;  // nullptr: no sharing hint
  int32_t batch;
  int64_t total_q;
  int32_t h_q;
  int32_t h_kv;
  int32_t g;                  // h_q / h_kv
  float scale_log2;           // sm_scale * log2(e)
  void* o;
  int32_t o_bf16;
  float* ws;                  // split-K partials (nsplit > 1)
  int32_t nsplit;
  int32_t n_rb;               // row blocks per KV head
  int32_t bm;                 // MFMA rows per block
  // decode split into a shared part (this kernel) and an own part (own_kernel)
  int32_t shared_only;        // 1: only the keys a block's requests share; always write partials
  float* ws_own;              // own-part partials: [batch * h_kv * n_chunk * g][D], then (m, l)
  int32_t n_chunk;            // most own-part key chunks per (request, KV head)
  int32_t own_fused;          // 0: own_kernel + merge_kernel; 1: own_merge_kernel writes O;
                              // 2: own_stream_kernel + merge_kernel
  int32_t own_min;            // fewest own keys per chunk (own_chunks)
  int32_t sh_small;           // 1: shared part with 4-wave workgroups, 2 tiles per round
  int32_t run_cap;            // split decode: most extra shared-part tiles per row block taken
                              // for deeper runs (block_runs); 0: none
  int32_t* own_cnt;           // own_fold: finished own chunks per (request, KV head), zeroed
                              // by the shared part's kernel; nullptr otherwise
  int32_t own_fold;           // own_fused == 2: own_stream_kernel also merges the requests
                              // with several own chunks (else merge_kernel does)
};

template <typename T, int D, int NW, int RT, int KS>
struct Cfg {
  static constexpr int kThreads = 64 * NW;
  static constexpr int NWR = NW / KS;                   // waves along rows (KS along keys)
  static constexpr int BM = 32 * RT * NWR;
  static constexpr int EPC = 16 / sizeof(T);           // elements per 16-byte chunk
  static constexpr int CHUNKS = D / EPC;                // chunks per token row
  static constexpr int KSTRIDE = D + EPC;               // K row pad: 16 bytes
  static constexpr int VSTRIDE = BN + (sizeof(T) == 2 ? 4 : 1);  // V^T row pad: 8 / 4 bytes
  static constexpr int KPP = kThreads / CHUNKS;         // keys per load pass
  static constexpr int KP = BN / KPP;                   // K load passes
  static constexpr int VP = (BN / 2) / KPP;             // V load passes (key pairs)
  static_assert(KPP > 0 && BN % KPP == 0 && (BN / 2) % KPP == 0, "tile load shape");
};

template <typename T, int D, int NW, int RT, int KS>
struct __align__(16) Smem {
  using C = Cfg<T, D, NW, RT, KS>;
  T k[2][BN * C::KSTRIDE];
  T vt[2][D * C::VSTRIDE];
  int32_t slot[4][BN];
  int32_t req_m[C::BM];
  int32_t req_row[C::BM];
  int32_t req_qo[C::BM + 1];
  int32_t own[C::BM + 1];
  int32_t req_sh[C::BM];
  int32_t hdr[8];
  int32_t cnt[32];
};

struct TileDesc {
  int kind;  // 0 shared prefix, 1 one request's own prefix, 2 suffix (k_ext rows)
  int cnt;   // valid keys in the tile
  int pos0;  // first position (kinds 0, 1)
  int kr0;   // first k_ext row (kind 2)
  int req;   // local request index (kind 1)
  int row;   // req_to_token row (kinds 0, 1)
};

// ---- tiles loaded straight into LDS (bf16, D = 128)
// A tile is row-major [key][D] in LDS, 256 bytes per key, filled by 16-byte global-to-LDS
// loads: one instruction moves 64 x 16 bytes (4 keys) to consecutive LDS bytes, so no
// row padding is possible; instead the 16-byte chunk positions of row r are XORed with a
// swizzle (a lane's global address picks the chunk that belongs at its fixed LDS
// position). K fragment reads take one chunk of 16 consecutive rows per 256 bytes: K
// rows use r % 16, so those rows hit 16 different chunk positions. A transposing V read
// takes two adjacent chunks of 4 consecutive rows per 128 bytes and four of them per 256
// bytes: V rows use 4 (r % 4) + 2 ((r / 2) % 2), which gives those rows different
// 4-chunk blocks and different chunk pairs modulo 8 (no conflict with 128 or 256 bytes
// of banks). The V^T fragments of O^T = V^T P^T come
// from ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of
// the 8-byte pieces addressed by lanes i / 4 + 4e (e = 0..3). Lane p therefore addresses
// key kb + p / 4, dims d0 + 4 (p % 4), and lane i ends up with dim d0 + i of keys
// kb .. kb + 3. Nothing is written to LDS by the threads, so no transposing stores.
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return 4 * (r & 3) + 2 * ((r >> 1) & 1); }

// A operand (K rows kr = 32 keys, dims ks*16 + half*8 .. +8) of S^T = K Q^T.
__device__ __forceinline__ bf16x8 k_frag(const char* kt, int kr, int ks, int half) {
  return *reinterpret_cast<const bf16x8*>(kt + kr * 256 + (((2 * ks + half) ^ swz_k(kr)) * 16));
}

// A operand of O^T = V^T P^T for 32 dims (dt) x 16 keys (kh) of a 32-key half (sub):
// lane l holds dim dt*32 + l%32 of keys sub*32 + kh*16 + 4*(l/32) + {0..3} and the same
// + 8, the key order of the P fragments.
__device__ __forceinline__ bf16x8 vt_frag(const char* vt, int sub, int dt, int kh, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int pl = lane & 15, dsub = (lane >> 4) & 1, half = lane >> 5;
  const int d0 = dt * 32 + dsub * 16 + 4 * (pl & 3);
  const int key = sub * 32 + kh * 16 + 4 * half + (pl >> 2);
  const char* p0 = vt + key * 256 + (((d0 >> 3) ^ swz_v(key)) * 16) + (d0 & 7) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0 + 8 * 256));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Fragment reads through LDS-address-space pointers (the arithmetic stays in the LDS
// address space, so constant parts fold into the instructions' offset fields): k_frag's
// read, and vt_frag's transposing pair (the second 8 keys further)
typedef __attribute__((address_space(3))) const char* lds_cp;
__device__ __forceinline__ lds_cp lds_ptr(uint32_t addr) { return (lds_cp)(uintptr_t)addr; }
__device__ __forceinline__ bf16x8 k_at(lds_cp p) {
  return *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 vt_at(lds_cp p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4* lp;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p + 8 * 256));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// An empty asm that the compiler must treat as changing x: a base formed from it is not
// re-associated with the constant parts of later addresses, which then fold into the
// reads' offset fields (one add per base and tile instead of two per read).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}

// The requests whose extend rows [t0, t1] a block covers: ra = the last r in [0, batch)
// with qo[r] <= t0, rb = the last with qo[r] <= t1. qo rises (never falls) from qo[0] = 0,
// so the last such r is the number of r with qo[r] <= t, minus one: the block counts them
// in one round of loads (a binary search in one thread made about 2 log2(batch) dependent
// loads at every workgroup's start). cnt: 32 ints of LDS; every thread calls; ends with a
// barrier.
__device__ __forceinline__ void block_reqs(const int32_t* qo, int batch, int64_t t0, int64_t t1, int tid,
                                           int nthreads, int* cnt, int& ra, int& rb) {
  const int wave = tid >> 6, lane = tid & 63;
  int c0 = 0, c1 = 0;
  for (int i0 = 0; i0 < batch; i0 += nthreads) {  // the same trip count in every thread
    const int i = i0 + tid;
    const int64_t v = i < batch ? qo[i] : 0;
    c0 += __popcll(__ballot(i < batch && v <= t0));
    c1 += __popcll(__ballot(i < batch && v <= t1));
  }
  if (lane == 0) {
    cnt[wave] = c0;
    cnt[16 + wave] = c1;
  }
  __syncthreads();
  int s0 = 0, s1 = 0;
  for (int w = 0; w < nthreads / 64; ++w) {
    s0 += cnt[w];
    s1 += cnt[16 + w];
  }
  ra = max(s0 - 1, 0);
  rb = max(s1 - 1, 0);
}

// Wave-uniform value (kept in an SGPR): block metadata read from LDS is the same in
// every lane, and saying so keeps tile bookkeeping off the exec mask.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <typename SM>
__device__ __forceinline__ TileDesc describe(int tau, const SM& sm, int L, int n_sh, int n_own, int suf0,
                                             int64_t qb, int nreq) {
  TileDesc d;
  d.pos0 = 0;
  d.kr0 = 0;
  d.req = 0;
  d.row = 0;
  if (tau < n_sh) {
    d.kind = 0;
    d.pos0 = tau * BN;
    d.cnt = min(BN, L - d.pos0);
    d.row = uni(sm.req_row[0]);
  } else if (tau < n_sh + n_own) {
    d.kind = 1;
    const int o = tau - n_sh;
    int lo = 0, hi = nreq - 1;  // last i with own[i] <= o
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (uni(sm.own[mid]) <= o) lo = mid;
      else hi = mid - 1;
    }
    d.req = lo;
    d.pos0 = L + (o - uni(sm.own[lo])) * BN;
    d.cnt = min(BN, uni(sm.req_m[lo]) - d.pos0);
    d.row = uni(sm.req_row[lo]);
  } else {
    d.kind = 2;
    d.kr0 = suf0 + (tau - n_sh - n_own) * BN;
    d.cnt = (int)min((int64_t)BN, qb - d.kr0);
  }
  return d;
}

// Slot ids of a tile are fetched in two halves so the load is unconditional (no branch
// around a memory access, which lets the compiler keep several tiles' loads in flight):
// slot_issue loads req_to_token at a valid index (index 0 for keys that have none) and
// slot_finish turns the raw value into the slot id (pool), the k_ext row (suffix) or -1.
__device__ __forceinline__ int slot_issue(const AttnArgs& a, const TileDesc& d, int i) {
  const bool pool = d.kind != 2 && i < d.cnt;
  const int64_t idx = pool ? (int64_t)d.row * a.rtt_stride + d.pos0 + i : 0;
  return a.rtt[idx];
}

__device__ __forceinline__ int slot_finish(const AttnArgs& a, const TileDesc& d, int i, int raw) {
  if (i >= d.cnt) return -1;
  if (d.kind == 2) return d.kr0 + i;
  if (raw < 0 || raw >= a.num_slots) {
    flag_error(RAX_DEVERR_SLOT);
    return -1;
  }
  return raw;
}

// 16-byte load that always reads valid memory: keys without a slot read row 0 and are
// zeroed when the tile is written to LDS (the mask also removes them from the softmax).
__device__ __forceinline__ u32x4 ld16(const char* base, int s, int64_t row_bytes) {
  return *reinterpret_cast<const u32x4*>(base + (int64_t)(s < 0 ? 0 : s) * row_bytes);
}

__device__ __forceinline__ u32x4 keep_if(bool ok, u32x4 v) {
  u32x4 r;
  r.x = ok ? v.x : 0u;
  r.y = ok ? v.y : 0u;
  r.z = ok ? v.z : 0u;
  r.w = ok ? v.w : 0u;
  return r;
}

__device__ __forceinline__ uint32_t word(u32x4 v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <typename T, int D, bool kDecode, int NW, int RT, int PD, int KS>
__global__ void __launch_bounds__(64 * NW) attn_kernel(AttnArgs a) {
  using C = Cfg<T, D, NW, RT, KS>;
  constexpr int BM = C::BM;
  constexpr bool kBf16 = sizeof(T) == 2;
  // tiles are staged through registers and stored padded / transposed (bf16 extend with
  // D = 128 runs in extend_kernel, which loads them straight into LDS)
  using SM = Smem<T, D, NW, RT, KS>;
  __shared__ SM sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int wrow = wave % C::NWR;  // which RT row tiles
  const int wkey = wave / C::NWR;  // which 32-key half of every tile (KS == 2)
  const int lane = tid & 63;
  const int jrow = lane & 31;  // row within a 32-row tile
  const int half = lane >> 5;  // which half of the key set this lane holds

  // ---- work item: (KV head, row block, split)
  const int64_t item = xcd_remap(blockIdx.x, (int64_t)gridDim.x);
  const int split = (int)(item % a.nsplit);
  int64_t rb = (item / a.nsplit) % a.n_rb;
  const int h = (int)(item / ((int64_t)a.nsplit * a.n_rb));
  // extend: a KV head's row blocks from the last to the first, so that under causal
  // masking the longest blocks are dispatched first and the short ones fill in behind
  if (!kDecode) rb = a.n_rb - 1 - rb;

  const int64_t G0 = rb * BM;   // first MFMA row
  const int64_t qa = G0 / a.g;  // first query row (BM % g == 0)
  int64_t qb = qa + BM / a.g;   // one past the last query row
  if (qb > a.total_q) qb = a.total_q;

  // ---- this lane's rows (RT row tiles) and their Q fragments (B operand of S^T = K Q^T:
  // row jrow, dims [ks*K + half*K/2, +K/2)). They depend on the block index alone, so the
  // Q loads go out first (rows past the block's end read row qa and are zeroed).
  bool row_ok[RT];
  int64_t t_row[RT];
  int hq[RT];
  constexpr int KSTEP = kBf16 ? 16 : 2;
  constexpr int NKS = D / KSTEP;
  typedef typename std::conditional<kBf16, bf16x8, float>::type QFrag;
  QFrag qf[RT][NKS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int R = (wrow * RT + rt) * 32 + jrow;
    const int64_t Gr = G0 + R;
    t_row[rt] = Gr / a.g;
    row_ok[rt] = t_row[rt] < qb;
    hq[rt] = h * a.g + (int)(Gr % a.g);
    const T* qp = reinterpret_cast<const T*>(a.q) + ((row_ok[rt] ? t_row[rt] : qa) * a.h_q + hq[rt]) * (int64_t)D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (kBf16) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + half * 8);
        qf[rt][ks] = row_ok[rt] ? v : bf16x8{};
      } else {
        const float v = qp[ks * 2 + half];
        qf[rt][ks] = row_ok[rt] ? v : 0.f;
      }
    }
  }

  // ---- block metadata (requests covered, shared length, tile list)
  int r0, nreq;
  if constexpr (kDecode) {  // one request per query row
    r0 = (int)qa;
    nreq = (int)(qb - qa);
  } else {
    static_assert(C::kThreads <= 16 * 64, "block_reqs counts per wave");
    int ra, rb_last;
    block_reqs(a.qo_indptr, a.batch, qa, qb - 1, tid, C::kThreads, sm.cnt, ra, rb_last);
    int n = rb_last - ra + 1;
    if (n > BM) {  // only possible with empty requests in between
      if (tid == 0) flag_error(RAX_DEVERR_ROW);
      n = BM;
    }
    r0 = uni(ra);
    nreq = uni(n);
  }
  for (int i = tid; i < nreq; i += C::kThreads) {
    const int r = r0 + i;
    int row = a.req_pool_idx[r];
    int m = a.kv_len[r];
    if (row < 0 || row >= a.rtt_rows || m < 0 || m > a.rtt_stride) {
      flag_error(RAX_DEVERR_ROW);
      row = 0;
      m = 0;
    }
    sm.req_row[i] = row;
    sm.req_m[i] = m;
    sm.req_qo[i] = kDecode ? r : a.qo_indptr[r];
    sm.req_sh[i] = i == 0 ? (1 << 30) : (a.shared_len ? a.shared_len[r] : 0);
  }
  if (tid == 0) sm.req_qo[nreq] = kDecode ? r0 + nreq : a.qo_indptr[r0 + nreq];
  __syncthreads();
  if (wave == 0) {
    // shared length L = min over the block's requests of their key counts (decode: minus
    // one, so the newest key is always the request's own) and of the shared_len hints
    // between neighbours; then an exclusive scan of own-tile counts
    int Lw = 1 << 30;
    for (int i = lane; i < nreq; i += 64) Lw = min(Lw, min(sm.req_m[i] - (kDecode ? 1 : 0), sm.req_sh[i]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) Lw = min(Lw, __shfl_xor(Lw, off));
    const int L = max(Lw, 0);
    int carry = 0;
    for (int base = 0; base < (a.shared_only ? 0 : nreq); base += 64) {
      const int i = base + lane;
      const int rest = i < nreq ? sm.req_m[i] - L : 0;
      const int cnt = rest > 0 ? (rest + BN - 1) / BN : 0;
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      if (i < nreq) sm.own[i] = carry + incl - cnt;
      carry += __shfl(incl, 63);
    }
    if (a.shared_only)
      for (int i = lane; i < nreq; i += 64) sm.own[i] = 0;
    if (lane == 0) {
      sm.own[nreq] = carry;
      const int n_sh = (L + BN - 1) / BN;
      const int n_suf = kDecode ? 0 : (int)((qb - sm.req_qo[0] + BN - 1) / BN);
      const int total = n_sh + carry + n_suf;
      sm.hdr[2] = L;
      sm.hdr[3] = n_sh;
      sm.hdr[4] = carry;
      sm.hdr[5] = (int)(((int64_t)total * split) / a.nsplit);
      sm.hdr[6] = (int)(((int64_t)total * (split + 1)) / a.nsplit);
    }
  }
  __syncthreads();
  const int L = uni(sm.hdr[2]);
  const int n_sh = uni(sm.hdr[3]);
  const int n_own = uni(sm.hdr[4]);
  const int t_begin = uni(sm.hdr[5]);
  const int t_end = uni(sm.hdr[6]);
  const int suf0 = uni(sm.req_qo[0]);

  // ---- the request of each of this lane's rows
  int my_req[RT], my_qo[RT];
  int w_rlo = 1 << 30, w_rhi = -1, w_klo = 1 << 30, w_khi = -1, n_bad = 0;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int req = 0;
    if (row_ok[rt]) {
      int lo = 0, hi = nreq - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sm.req_qo[mid] <= t_row[rt]) lo = mid;
        else hi = mid - 1;
      }
      req = lo;
      w_rlo = min(w_rlo, req);
      w_rhi = max(w_rhi, req);
      w_klo = min(w_klo, sm.req_qo[req]);
      w_khi = max(w_khi, (int)t_row[rt]);
    } else {
      ++n_bad;
    }
    my_req[rt] = req;
    my_qo[rt] = sm.req_qo[req];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    w_rlo = min(w_rlo, __shfl_xor(w_rlo, off));
    w_rhi = max(w_rhi, __shfl_xor(w_rhi, off));
    w_klo = min(w_klo, __shfl_xor(w_klo, off));
    w_khi = max(w_khi, __shfl_xor(w_khi, off));
    n_bad += __shfl_xor(n_bad, off);
  }
  w_rlo = uni(w_rlo);
  w_rhi = uni(w_rhi);
  w_klo = uni(w_klo);
  w_khi = uni(w_khi);
  const bool wave_active = w_rhi >= 0;
  const bool all_rows_ok = uni(n_bad) == 0;

  f32x16 acc[RT][D / 32];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = kNegInf;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[rt][dt] = f32x16{};
  }

  const int64_t row_bytes = (int64_t)a.h_kv * D * sizeof(T);  // bytes per pool slot / k_ext row
  const int64_t head_off = (int64_t)h * D * sizeof(T);
  const int c = tid % C::CHUNKS;
  const int kk = tid / C::CHUNKS;
  const int coff = c * 16;

  // global -> registers for one tile (slot ids already in sm.slot[sb]); PD register sets
  constexpr int NSB = PD + 2;  // slot-id buffers in LDS
  u32x4 kreg[PD][C::KP];
  u32x4 vreg[PD][C::VP][2];
  // Always issues the same number of loads (live == false: row 0, results unused), so the
  // compiler sees one load count on every path and waits only for the tile it consumes.
  auto issue_loads = [&](const TileDesc& d, int sb, bool live, auto set_c) {
    constexpr int set = decltype(set_c)::value;
    const char* kb = reinterpret_cast<const char*>(d.kind == 2 ? a.k_ext : a.k_pool) + head_off + coff;
    const char* vb = reinterpret_cast<const char*>(d.kind == 2 ? a.v_ext : a.v_pool) + head_off + coff;
    // slot buffer sb may hold another tile's ids when !live: read it anyway, then drop
#pragma unroll
    for (int p = 0; p < C::KP; ++p) {
      const int sv = sm.slot[sb][p * C::KPP + kk];
      kreg[set][p] = ld16(kb, live ? sv : -1, row_bytes);
    }
#pragma unroll
    for (int p = 0; p < C::VP; ++p) {
      const int kp = p * C::KPP + kk;
      const int s0 = sm.slot[sb][2 * kp], s1 = sm.slot[sb][2 * kp + 1];
      vreg[set][p][0] = ld16(vb, live ? s0 : -1, row_bytes);
      vreg[set][p][1] = ld16(vb, live ? s1 : -1, row_bytes);
    }
  };
  // registers -> LDS buffer b (K row-major, V transposed); keys without a slot become zeros
  auto store_tile = [&](int b, int sb, auto set_c) {
    constexpr int set = decltype(set_c)::value;
#pragma unroll
    for (int p = 0; p < C::KP; ++p) {
      const int key = p * C::KPP + kk;
      *reinterpret_cast<u32x4*>(&sm.k[b][key * C::KSTRIDE + c * C::EPC]) =
          keep_if(sm.slot[sb][key] >= 0, kreg[set][p]);
    }
#pragma unroll
    for (int p = 0; p < C::VP; ++p) {
      const int kp = p * C::KPP + kk;
      const u32x4 w0 = keep_if(sm.slot[sb][2 * kp] >= 0, vreg[set][p][0]);
      const u32x4 w1 = keep_if(sm.slot[sb][2 * kp + 1] >= 0, vreg[set][p][1]);
      uint32_t* dst = reinterpret_cast<uint32_t*>(&sm.vt[b][(c * C::EPC) * C::VSTRIDE + 2 * kp]);
      constexpr int WSTRIDE = C::VSTRIDE * (int)sizeof(T) / 4;  // V^T row stride in 32-bit words
#pragma unroll
      for (int e = 0; e < C::EPC; ++e) {
        if constexpr (kBf16) {
          // element e of both keys -> one 32-bit word (key 2kp low half, key 2kp+1 high half)
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          dst[e * WSTRIDE] = __builtin_amdgcn_perm(word(w1, e >> 1), word(w0, e >> 1), sel);
        } else {
          float* df = reinterpret_cast<float*>(&sm.vt[b][(c * C::EPC + e) * C::VSTRIDE + 2 * kp]);
          df[0] = __builtin_bit_cast(float, word(w0, e));
          df[1] = __builtin_bit_cast(float, word(w1, e));
        }
      }
    }
  };
  auto desc = [&](int tau) { return describe(tau, sm, L, n_sh, n_own, suf0, qb, nreq); };

  // slot ids of one tile written by the first BN threads (wave 0)
  auto put_slot = [&](int sb, int v) { sm.slot[sb][tid] = v; };

  // ---- prologue: slot ids of tiles t_begin .. t_begin+PD, K/V loads of the first PD tiles
  if (tid < BN && t_begin < t_end) {  // all prologue slot loads in one round trip
    TileDesc di[PD + 1];
    int raw[PD + 1];
#pragma unroll
    for (int i = 0; i <= PD; ++i) {
      di[i] = desc(min(t_begin + i, t_end - 1));
      raw[i] = slot_issue(a, di[i], tid);
    }
#pragma unroll
    for (int i = 0; i <= PD; ++i)
      if (t_begin + i < t_end) put_slot((t_begin + i) % NSB, slot_finish(a, di[i], tid, raw[i]));
  }
  __syncthreads();
  if (t_begin < t_end) {
    issue_loads(desc(t_begin), t_begin % NSB, true, std::integral_constant<int, 0>{});
    if constexpr (PD > 1) {
      const bool live = t_begin + 1 < t_end;
      issue_loads(desc(live ? t_begin + 1 : t_begin), (t_begin + 1) % NSB, live, std::integral_constant<int, 1>{});
    }
    store_tile(0, t_begin % NSB, std::integral_constant<int, 0>{});
  }
  __syncthreads();

  // one pipeline step; ph = (tau - t_begin) % PD selects the register sets at compile time
  auto step = [&](int tau, auto ph_c) {
    constexpr int ph = decltype(ph_c)::value;
    const int buf = (tau - t_begin) & 1;
    const TileDesc d = desc(tau);
    // slot ids of tile tau+PD+1 first: vector loads retire in order, so waiting for this
    // one (end of step) must not also wait for the K/V loads issued after it
    const bool has_next = tau + PD + 1 < t_end;
    const TileDesc dn = desc(has_next ? tau + PD + 1 : tau);
    const int raw_slot = slot_issue(a, dn, tid < BN ? tid : 0);
    const bool live = tau + PD < t_end;
    issue_loads(desc(live ? tau + PD : tau), (tau + PD) % NSB, live, std::integral_constant<int, ph>{});

    // -- does this wave have rows that see any key of the tile?
    bool run = wave_active;
    if (d.kind == 1) run = run && d.req >= w_rlo && d.req <= w_rhi;
    if (d.kind == 2) run = run && d.kr0 <= w_khi && d.kr0 + d.cnt > w_klo;

    if (run) {
      const bool unmasked = d.kind == 0 && d.cnt == BN && all_rows_ok;
      // two 32-key online-softmax steps per 64-key tile (keeps S and P small); with
      // KS == 2 each wave takes one of them and the pair is combined at the end. The S
      // products of all of this wave's halves are issued first, so that the second
      // half's MFMAs run in the matrix pipe while the first half's softmax runs on the VALU
      // (and its P.V MFMAs under the second half's softmax).
      constexpr int NSUB = 2 / KS;
      f32x16 sall[NSUB][RT];
#pragma unroll
      for (int si = 0; si < NSUB; ++si) {
        const int sub = KS == 1 ? si : wkey;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sall[si][rt] = f32x16{};
        const T* kr = &sm.k[buf][(sub * 32 + jrow) * C::KSTRIDE];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if constexpr (kBf16) {
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(kr + ks * 16 + half * 8);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              sall[si][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[rt][ks], sall[si][rt], 0, 0, 0);
          } else {
            const float af = kr[ks * 2 + half];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              sall[si][rt] = __builtin_amdgcn_mfma_f32_32x32x2f32(af, qf[rt][ks], sall[si][rt], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int si = 0; si < NSUB; ++si) {
        const int sub = KS == 1 ? si : wkey;
        f32x16(&s)[RT] = sall[si];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          // mask (raw scores; the scale is positive); key index of register r:
          // sub*32 + 8*(r/4) + 4*half + r%4
          float mx = kNegInf;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float v = s[rt][r];
            if (!unmasked) {
              const int key = sub * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
              bool ok = row_ok[rt] && key < d.cnt;
              if (d.kind == 1) ok = ok && my_req[rt] == d.req;
              if (d.kind == 2) {
                const int kr2 = d.kr0 + key;
                ok = ok && kr2 >= my_qo[rt] && kr2 <= t_row[rt];
              }
              v = ok ? v : kNegInf;
            }
            s[rt][r] = v;
            mx = fmaxf(mx, v);
          }
          mx = max_xor32(mx) * a.scale_log2;
          // Lazy rescale: the reference maximum of a row moves only when some row of the
          // wave sees a score more than 2^kLazy above its reference (also on the first
          // keys, reference -inf). In between, probabilities are up to 2^kLazy; l, acc
          // and the final division all use the same reference, so the result is the
          // same softmax.
          if (__any(mx > m_run[rt] + kLazy)) {
            const float m_new = fmaxf(m_run[rt], mx);
            const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run[rt] - m_new);
            l_run[rt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) acc[rt][dt] *= alpha;
            m_run[rt] = m_new;
          }
          const float neg_m = m_run[rt] == kNegInf ? 0.f : -m_run[rt];
          float psum = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rt][r], a.scale_log2, neg_m));
            s[rt][r] = p;
            psum += p;
          }
          psum = sum_xor32(psum);
          l_run[rt] += psum;
        }

        // O^T += V^T P^T over this sub-step's 32 keys
        if constexpr (kBf16) {
          bf16x8 pb[RT][2];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
              for (int e = 0; e < 8; ++e) pb[rt][kh][e] = (__bf16)s[rt][kh * 8 + e];
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
              const T* vr = &sm.vt[buf][(dt * 32 + jrow) * C::VSTRIDE];
              const int kb0 = sub * 32 + kh * 16 + 4 * half;
              const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr + kb0);
              const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + kb0 + 8);
              const bf16x8 af = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
              for (int rt = 0; rt < RT; ++rt)
                acc[rt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pb[rt][kh], acc[rt][dt], 0, 0, 0);
            }
          }
        } else {
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const T* vr = &sm.vt[buf][(dt * 32 + jrow) * C::VSTRIDE];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = sub * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
              const float af = vr[key];
#pragma unroll
              for (int rt = 0; rt < RT; ++rt)
                acc[rt][dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(af, s[rt][r], acc[rt][dt], 0, 0, 0);
            }
          }
        }
      }
    }

    if (tau + 1 < t_end) store_tile(buf ^ 1, (tau + 1) % NSB, std::integral_constant<int, (ph + 1) % PD>{});
    if (has_next && tid < BN) put_slot((tau + PD + 1) % NSB, slot_finish(a, dn, tid, raw_slot));
    __syncthreads();
  };

  for (int tau = t_begin; tau < t_end; tau += PD) {
    step(tau, std::integral_constant<int, 0>{});
    if constexpr (PD > 1) {
      if (tau + 1 < t_end) step(tau + 1, std::integral_constant<int, 1>{});
    }
  }

  // ---- key-split pairs: the wave of the second key half hands its (m, l, acc) over LDS
  // (the tile buffers are free after the loop's last barrier); the first combines them
  if constexpr (KS == 2) {
    constexpr int NV = (D / 32) * 16 + 2;
    static_assert(C::NWR * RT * NV * 64 * sizeof(float) <= sizeof(sm.k), "key-split exchange area");
    float* xs = reinterpret_cast<float*>(&sm.k[0][0]);
    if (wkey == 1) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int base = (wrow * RT + rt) * NV;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) xs[(base + dt * 16 + r) * 64 + lane] = acc[rt][dt][r];
        xs[(base + NV - 2) * 64 + lane] = m_run[rt];
        xs[(base + NV - 1) * 64 + lane] = l_run[rt];
      }
    }
    __syncthreads();
    if (wkey == 1) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int base = (wrow * RT + rt) * NV;
      const float m1 = xs[(base + NV - 2) * 64 + lane];
      const float l1 = xs[(base + NV - 1) * 64 + lane];
      const float m = fmaxf(m_run[rt], m1);
      if (m != kNegInf) {
        const float a0 = __builtin_amdgcn_exp2f(m_run[rt] - m);
        const float a1 = __builtin_amdgcn_exp2f(m1 - m);
        l_run[rt] = l_run[rt] * a0 + l1 * a1;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[rt][dt][r] = acc[rt][dt][r] * a0 + xs[(base + dt * 16 + r) * 64 + lane] * a1;
        m_run[rt] = m;
      }
    }
  }

  // ---- epilogue: lane holds row jrow of each row tile, dims dt*32 + 8*(r/4) + 4*half + r%4
  // (split partials at the block's own place: extend takes row blocks in reverse order)
  const int64_t item_w = ((int64_t)h * a.n_rb + rb) * a.nsplit + split;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (!row_ok[rt]) continue;
    const int R = (wrow * RT + rt) * 32 + jrow;
    const bool partial = a.nsplit > 1 || a.shared_only;
    if (!partial) {
      const float inv = l_run[rt] > 0.f ? 1.f / l_run[rt] : 0.f;
      const int64_t obase = (t_row[rt] * a.h_q + hq[rt]) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d0 = dt * 32 + 8 * rg + 4 * half;
          const float x0 = acc[rt][dt][rg * 4 + 0] * inv, x1 = acc[rt][dt][rg * 4 + 1] * inv;
          const float x2 = acc[rt][dt][rg * 4 + 2] * inv, x3 = acc[rt][dt][rg * 4 + 3] * inv;
          if (a.o_bf16) {
            *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + obase + d0) =
                bf16x4{(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
          } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + obase + d0) = make_float4(x0, x1, x2, x3);
          }
        }
      }
    } else if (l_run[rt] > 0.f) {
      float* wacc = a.ws + (item_w * BM + R) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d0 = dt * 32 + 8 * rg + 4 * half;
          *reinterpret_cast<float4*>(wacc + d0) = make_float4(acc[rt][dt][rg * 4 + 0], acc[rt][dt][rg * 4 + 1],
                                                              acc[rt][dt][rg * 4 + 2], acc[rt][dt][rg * 4 + 3]);
        }
      }
    }
    if (partial && half == 0) {  // (m, l) of every row; l == 0 means "no keys here"
      const int64_t n_items = (int64_t)a.h_kv * a.n_rb * a.nsplit;
      float* wml = a.ws + n_items * BM * (int64_t)D + (item_w * BM + R) * 2;
      wml[0] = m_run[rt];
      wml[1] = l_run[rt];
    }
  }
}

// ---- extend, bf16, D = 128: the block layout, tile list, masks and softmax of
// attn_kernel's extend form (8 waves of one 32-row tile, 256 rows per block) with a lean
// tile loop. Counters on the few-shot calls showed attn_kernel issuing 10.5 VALU and 8.6
// SALU instructions per MFMA (tile descriptors found by binary search per tile, slot ids
// fetched and checked per tile, mask code on every tile), so the MFMA pipe was busy 16% of
// the time. Here, per segment of up to kExtSeg tiles, the block first builds a table of its
// tiles (kind, key count, source) and stages the source row of every key (pool slot, or
// k_ext row for suffix tiles; past a tile's keys, its first key's row) in LDS, in one
// round of loads. The tile loop then only waits, issues the K/V rows of the tile kExtPD
// ahead straight into LDS (swizzled as above), and computes; full shared-prefix tiles take
// a path without masks. A slot id outside the pool is flagged and read as slot 0.
constexpr int kExtSeg = 128;
constexpr int kExtBuf = 3;  // K/V buffers: kExtBuf - 1 tiles in flight while one is computed

__global__ void __launch_bounds__(512) extend_kernel(AttnArgs a) {
  constexpr int D = 128, NW = 8, BM = 256;
  constexpr int RB = D * 2;              // bytes per row
  constexpr int TB = BN * RB;            // bytes of K (or V) per tile
  constexpr int NKS = D / 16;
  constexpr int NBUF = kExtBuf, PF = NBUF - 1;
  constexpr int IPW = (BN / 4) / NW;     // 1 KB loads per wave per K (or V) tile
  static_assert(IPW == 2, "two K and two V loads per wave and tile");
  struct __align__(16) Sm {
    char k[NBUF][TB];
    char v[NBUF][TB];
    int32_t src[kExtSeg * BN];           // per key of the segment: pool slot or k_ext row
    int32_t t_kind[kExtSeg];             // per tile of the segment: kind | request << 2
    int32_t t_cnt[kExtSeg];              // keys
    int32_t t_row[kExtSeg];              // req_to_token row (kinds 0, 1) or first k_ext row (kind 2)
    int32_t t_pos[kExtSeg];              // first position (kinds 0, 1)
    int32_t req_m[BM];
    int32_t req_row[BM];
    int32_t req_qo[BM + 1];
    int32_t own[BM + 1];
    int32_t req_sh[BM];
    int32_t hdr[8];
    int32_t cnt[32];
  };
  __shared__ Sm sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int jrow = lane & 31;
  const int half = lane >> 5;

  // ---- work item: (KV head, row block, split); a KV head's row blocks from the last to
  // the first, so that under causal masking the longest blocks are dispatched first
  const int64_t item = xcd_remap(blockIdx.x, (int64_t)gridDim.x);
  const int split = (int)(item % a.nsplit);
  const int64_t rb = a.n_rb - 1 - (item / a.nsplit) % a.n_rb;
  const int h = (int)(item / ((int64_t)a.nsplit * a.n_rb));
  const int64_t G0 = rb * BM;
  const int64_t qa = G0 / a.g;
  int64_t qb = qa + BM / a.g;
  if (qb > a.total_q) qb = a.total_q;

  // ---- this lane's row and its Q fragments (B operand of S^T = K Q^T)
  const int R = wave * 32 + jrow;
  const int64_t t_row = (G0 + R) / a.g;
  const bool row_ok = t_row < qb;
  const int hq = h * a.g + (int)((G0 + R) % a.g);
  bf16x8 qf[NKS];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + ((row_ok ? t_row : qa) * a.h_q + hq) * (int64_t)D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + half * 8);
      qf[ks] = row_ok ? v : bf16x8{};
    }
  }

  // ---- block metadata (requests covered, shared length, tile list), as attn_kernel
  int ra, rb_last;
  block_reqs(a.qo_indptr, a.batch, qa, qb - 1, tid, 64 * NW, sm.cnt, ra, rb_last);
  int n_req_blk = rb_last - ra + 1;
  if (n_req_blk > BM) {  // only possible with empty requests in between
    if (tid == 0) flag_error(RAX_DEVERR_ROW);
    n_req_blk = BM;
  }
  const int r0 = uni(ra);
  const int nreq = uni(n_req_blk);
  for (int i = tid; i < nreq; i += 64 * NW) {
    const int r = r0 + i;
    int row = a.req_pool_idx[r];
    int m = a.kv_len[r];
    if (row < 0 || row >= a.rtt_rows || m < 0 || m > a.rtt_stride) {
      flag_error(RAX_DEVERR_ROW);
      row = 0;
      m = 0;
    }
    sm.req_row[i] = row;
    sm.req_m[i] = m;
    sm.req_qo[i] = a.qo_indptr[r];
    sm.req_sh[i] = i == 0 ? (1 << 30) : (a.shared_len ? a.shared_len[r] : 0);
  }
  if (tid == 0) sm.req_qo[nreq] = a.qo_indptr[r0 + nreq];
  __syncthreads();
  if (wave == 0) {
    int Lw = 1 << 30;
    for (int i = lane; i < nreq; i += 64) Lw = min(Lw, min(sm.req_m[i], sm.req_sh[i]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) Lw = min(Lw, __shfl_xor(Lw, off));
    const int L = max(Lw, 0);
    int carry = 0;
    for (int base = 0; base < nreq; base += 64) {
      const int i = base + lane;
      const int rest = i < nreq ? sm.req_m[i] - L : 0;
      const int cnt = rest > 0 ? (rest + BN - 1) / BN : 0;
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      if (i < nreq) sm.own[i] = carry + incl - cnt;
      carry += __shfl(incl, 63);
    }
    if (lane == 0) {
      sm.own[nreq] = carry;
      const int n_sh = (L + BN - 1) / BN;
      const int n_suf = (int)((qb - sm.req_qo[0] + BN - 1) / BN);
      const int total = n_sh + carry + n_suf;
      sm.hdr[2] = L;
      sm.hdr[3] = n_sh;
      sm.hdr[4] = carry;
      sm.hdr[5] = (int)(((int64_t)total * split) / a.nsplit);
      sm.hdr[6] = (int)(((int64_t)total * (split + 1)) / a.nsplit);
    }
  }
  __syncthreads();
  const int L = uni(sm.hdr[2]);
  const int n_sh = uni(sm.hdr[3]);
  const int n_own = uni(sm.hdr[4]);
  const int tb = uni(sm.hdr[5]);
  const int te = uni(sm.hdr[6]);
  const int suf0 = uni(sm.req_qo[0]);

  // ---- the request of this lane's row; the wave's request and suffix-row ranges
  int my_req = 0;
  int w_rlo = 1 << 30, w_rhi = -1, w_klo = 1 << 30, w_khi = -1, n_bad = 0;
  if (row_ok) {
    int lo = 0, hi = nreq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sm.req_qo[mid] <= t_row) lo = mid;
      else hi = mid - 1;
    }
    my_req = lo;
    w_rlo = w_rhi = my_req;
    w_klo = sm.req_qo[my_req];
    w_khi = (int)t_row;
  } else {
    n_bad = 1;
  }
  const int my_qo = sm.req_qo[my_req];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    w_rlo = min(w_rlo, __shfl_xor(w_rlo, off));
    w_rhi = max(w_rhi, __shfl_xor(w_rhi, off));
    w_klo = min(w_klo, __shfl_xor(w_klo, off));
    w_khi = max(w_khi, __shfl_xor(w_khi, off));
    n_bad += __shfl_xor(n_bad, off);
  }
  w_rlo = uni(w_rlo);
  w_rhi = uni(w_rhi);
  w_klo = uni(w_klo);
  w_khi = uni(w_khi);
  const bool wave_active = w_rhi >= 0;
  const bool all_rows_ok = uni(n_bad) == 0;

  const int64_t row_bytes = (int64_t)a.h_kv * RB;
  const int64_t head_off = (int64_t)h * RB;
  const uint32_t k_lds = lds_addr(&sm.k[0][0]), v_lds = lds_addr(&sm.v[0][0]);
  const char* kpool = reinterpret_cast<const char*>(a.k_pool) + head_off;
  const char* vpool = reinterpret_cast<const char*>(a.v_pool) + head_off;
  const char* kext = reinterpret_cast<const char*>(a.k_ext) + head_off;
  const char* vext = reinterpret_cast<const char*>(a.v_ext) + head_off;

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  // LDS byte offsets of this lane's fragment reads within a tile buffer, by k-step (K) and
  // by 32-dim slice (V): the swizzles XOR lane bits into them, so they are formed once here
  // and a tile adds only its buffer's base (k_frag / vt_frag compute the same addresses)
  uint32_t koff[NKS], voff[D / 32];
  {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) koff[ks] = jrow * 256 + (((2 * ks + half) ^ swz_k(jrow)) * 16);
    const int pl = lane & 15, dsub = (lane >> 4) & 1;
    const int kl = 4 * half + (pl >> 2);  // key within a 16-key group
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int d0 = dt * 32 + dsub * 16 + 4 * (pl & 3);
      voff[dt] = kl * 256 + (((d0 >> 3) ^ swz_v(kl)) * 16) + (d0 & 7) * 2;
    }
  }

  // K and V rows of segment tile lt into buffer b (this wave's 2 + 2 loads)
  auto issue = [&](int lt, int b) {
    const bool ext = (uni(sm.t_kind[lt]) & 3) == 2;
    const char* kb = ext ? kext : kpool;
    const char* vb = ext ? vext : vpool;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int q = wave + u * NW;
      const int r = q * 4 + (lane >> 4);
      const int64_t off = (int64_t)sm.src[lt * BN + r] * row_bytes;
      lds_load16(kb + off + (((lane & 15) ^ swz_k(r)) * 16), uni(k_lds + b * TB + q * 1024));
      lds_load16(vb + off + (((lane & 15) ^ swz_v(r)) * 16), uni(v_lds + b * TB + q * 1024));
    }
  };

  // the online softmax of a tile's (masked) scores, both 32-key halves against one running
  // maximum (one wave-uniform branch per tile for the lazy rescale), then O^T += V^T P^T:
  // the first half's PV MFMAs are issued before the second half's probabilities are
  // computed, so that the VALU work of one overlaps the other's MFMAs in the same wave
  auto tile_step = [&](const uint32_t (&va)[D / 32], f32x16 (&sc)[2]) {
    float mx = kNegInf;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[sub][r]);
    mx = max_xor32(mx) * a.scale_log2;
    if (__any(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
      m_run = m_new;
    }
    const float neg_m = m_run == kNegInf ? 0.f : -m_run;
    float psum = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      bf16x8 pb[2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[sub][kh * 8 + e], a.scale_log2, neg_m));
          psum += pv;
          pb[kh][e] = (__bf16)pv;
        }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_at(lds_ptr(va[dt]) + sub * 8192 + kh * 4096),
                                                            pb[kh], acc[dt], 0, 0, 0);
    }
    l_run += sum_xor32(psum);
  };

  for (int seg0 = tb; seg0 < te; seg0 += kExtSeg) {
    const int nt = min(te - seg0, kExtSeg);
    // ---- table of the segment's tiles (one thread per tile, as describe() but per lane)
    for (int i = tid; i < nt; i += 64 * NW) {
      const int tau = seg0 + i;
      int kind, cnt, row = 0, pos0 = 0, req = 0;
      if (tau < n_sh) {
        kind = 0;
        pos0 = tau * BN;
        cnt = min(BN, L - pos0);
        row = sm.req_row[0];
      } else if (tau < n_sh + n_own) {
        kind = 1;
        const int o = tau - n_sh;
        int lo = 0, hi = nreq - 1;  // last request with own[] <= o
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sm.own[mid] <= o) lo = mid;
          else hi = mid - 1;
        }
        req = lo;
        pos0 = L + (o - sm.own[lo]) * BN;
        cnt = min(BN, sm.req_m[lo] - pos0);
        row = sm.req_row[lo];
      } else {
        kind = 2;
        row = suf0 + (tau - n_sh - n_own) * BN;  // first k_ext row
        cnt = (int)min((int64_t)BN, qb - row);
      }
      sm.t_kind[i] = kind | (req << 2);
      sm.t_cnt[i] = cnt;
      sm.t_row[i] = row;
      sm.t_pos[i] = pos0;
    }
    __syncthreads();
    // ---- every key's source row: the slot ids of a pool tile straight into LDS (one 4-byte
    // load per lane, tiles dealt over the waves, all in flight at once), then the suffix
    // tiles' k_ext rows, positions past a tile's keys and slot ids outside the pool fixed up
    // (past the keys: the tile's first key's row, finite data that the masks drop)
    for (int lt = wave; lt < nt; lt += NW) {
      const int tk = uni(sm.t_kind[lt]);
      const int cnt = uni(sm.t_cnt[lt]);
      int64_t idx = 0;
      if ((tk & 3) != 2) idx = (int64_t)uni(sm.t_row[lt]) * a.rtt_stride + uni(sm.t_pos[lt]) + (lane < cnt ? lane : 0);
      lds_load4(a.rtt + idx, uni(lds_addr(&sm.src[lt * BN])));
    }
    wait_vmcnt<0>();
    __syncthreads();
    for (int i = tid; i < nt * BN; i += 64 * NW) {
      const int lt = i / BN, j = i % BN;
      const int kind = sm.t_kind[lt] & 3;
      const bool in = j < sm.t_cnt[lt];
      int sv;
      if (kind == 2) {
        sv = sm.t_row[lt] + (in ? j : 0);
      } else {
        sv = sm.src[i];
        if (sv < 0 || sv >= a.num_slots) {
          if (in) flag_error(RAX_DEVERR_SLOT);
          sv = 0;
        }
      }
      sm.src[i] = sv;
    }
    __syncthreads();

    // ---- the tile loop: PF tiles in flight while one is computed
#pragma unroll
    for (int j = 0; j < PF; ++j)
      if (j < nt) issue(j, j);
    for (int i = 0; i < nt; ++i) {
      // this wave's loads of tile i are done when at most those of the PF - 1 tiles issued
      // after it are in flight
      if (i + PF - 1 < nt) wait_vmcnt<4 * (PF - 1)>();
      else wait_vmcnt<0>();
      __syncthreads();  // every wave's loads of tile i landed; buffer (i - 1) % NBUF is free
      if (i + PF < nt) issue(i + PF, (i + PF) % NBUF);
      const int tk = uni(sm.t_kind[i]);
      const int kind = tk & 3, req = tk >> 2;
      const int cnt = uni(sm.t_cnt[i]);
      const int kr0 = uni(sm.t_row[i]);
      bool run = wave_active;
      if (kind == 1) run = run && req >= w_rlo && req <= w_rhi;
      if (kind == 2) run = run && kr0 <= w_khi && kr0 + cnt > w_klo;
      if (!run) continue;
      const int b = i % NBUF;
      const uint32_t kb = uni(k_lds + b * TB), vb = uni(v_lds + b * TB);
      uint32_t ka[NKS], va[D / 32];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) ka[ks] = opaque(kb + koff[ks]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) va[dt] = opaque(vb + voff[dt]);
      f32x16 sall[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        sall[sub] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          sall[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_at(lds_ptr(ka[ks]) + sub * 8192), qf[ks], sall[sub],
                                                              0, 0, 0);
      }
      if (!(kind == 0 && cnt == BN && all_rows_ok)) {  // masks: full shared tiles have none
        // this lane's row sees keys [lo, hi) of the tile: all of its keys (shared prefix), those
        // of its own request (own prefix), or the causal range of its request's suffix
        int lo = 0, hi = row_ok ? cnt : 0;
        if (kind == 1 && my_req != req) hi = 0;
        if (kind == 2) {
          lo = max(lo, my_qo - kr0);
          hi = min(hi, (int)(t_row - kr0) + 1);
        }
        // nothing to mask when every row of the wave sees the whole tile (interior tiles
        // of a row's own prefix or below its causal diagonal)
        if (!__all(lo <= 0 && hi >= BN)) {
          // key of register r: sub*32 + 8*(r/4) + 4*half + r%4; compare the constant part
          lo -= 4 * half;
          hi -= 4 * half;
#pragma unroll
          for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int c = sub * 32 + 8 * (r >> 2) + (r & 3);
              sall[sub][r] = c >= lo && c < hi ? sall[sub][r] : kNegInf;
            }
        }
      }
      tile_step(va, sall);
    }
    __syncthreads();  // the next segment rewrites the table, the rows and the buffers
  }

  // ---- epilogue: lane holds row jrow, dims dt*32 + 8*(r/4) + 4*half + r%4
  if (!row_ok) return;
  if (a.nsplit == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const int64_t obase = (t_row * a.h_q + hq) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = dt * 32 + 8 * rg + 4 * half;
        const float x0 = acc[dt][rg * 4 + 0] * inv, x1 = acc[dt][rg * 4 + 1] * inv;
        const float x2 = acc[dt][rg * 4 + 2] * inv, x3 = acc[dt][rg * 4 + 3] * inv;
        if (a.o_bf16)
          *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + obase + d0) =
              bf16x4{(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
        else
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + obase + d0) = make_float4(x0, x1, x2, x3);
      }
    }
    return;
  }
  // split partials at the block's own place (merge_kernel's layout)
  const int64_t item_w = ((int64_t)h * a.n_rb + rb) * a.nsplit + split;
  if (l_run > 0.f) {
    float* wacc = a.ws + (item_w * BM + R) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *reinterpret_cast<float4*>(wacc + dt * 32 + 8 * rg + 4 * half) =
            make_float4(acc[dt][rg * 4 + 0], acc[dt][rg * 4 + 1], acc[dt][rg * 4 + 2], acc[dt][rg * 4 + 3]);
  }
  if (half == 0) {
    const int64_t n_items = (int64_t)a.h_kv * a.n_rb * a.nsplit;
    float* wml = a.ws + n_items * BM * (int64_t)D + (item_w * BM + R) * 2;
    wml[0] = m_run;
    wml[1] = l_run;
  }
}

// ---- wavefront lane exchanges: value of lane (l ^ d)
// d = 8, 2, 1 are DPP moves within a 16-lane row (row_ror:8, quad_perm [1,0,3,2] and
// [2,3,0,1]); d = 32, 16, 4 go through ds_bpermute. (gfx950's v_permlane16/32_swap would
// do 32 and 16 in the VALU, but the clang of this toolchain returns the swapped vdst for
// both results of its builtin, dropping the swapped src0.)
template <int d>
__device__ __forceinline__ float xor_get(float x) {
  if constexpr (d == 8 || d == 2 || d == 1) {
    constexpr int ctrl = d == 8 ? 0x128 : d == 2 ? 0x4E : 0xB1;
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xf, 0xf, false));
  } else {
    return __shfl_xor(x, d);
  }
}

// Sum over lanes that differ only in bit d.
template <int d>
__device__ __forceinline__ float xor_sum(float x) {
  return x + xor_get<d>(x);
}

// One transposing butterfly step at distance d over the pair (x, y): lanes with bit d
// clear return x + x(l ^ d), lanes with bit d set return y + y(l ^ d).
template <int d>
__device__ __forceinline__ float xor_pair(float x, float y, int lane) {
  const bool up = lane & d;
  return (up ? y : x) + xor_get<d>(up ? x : y);
}

// Wave reduction of P partial sums per lane: on return, v[0] of lane l is the sum over
// all 64 lanes of v[l % P]. Distances >= P are plain sums (the lanes that differ there
// hold the same pairs); below P each step halves the values a lane keeps.
template <int P>
__device__ __forceinline__ void wave_reduce_pairs(float (&v)[P], int lane) {
#define RAX_SUM_STEP(dd)                                                   \
  if constexpr (dd >= P) {                                                 \
    _Pragma("unroll") for (int i = 0; i < P; ++i) v[i] = xor_sum<dd>(v[i]); \
  } else {                                                                 \
    _Pragma("unroll") for (int i = 0; i < dd; ++i) v[i] = xor_pair<dd>(v[i], v[i + dd], lane); \
  }
  RAX_SUM_STEP(32)
  RAX_SUM_STEP(16)
  RAX_SUM_STEP(8)
  RAX_SUM_STEP(4)
  RAX_SUM_STEP(2)
  RAX_SUM_STEP(1)
#undef RAX_SUM_STEP
}

template <int d>
__device__ __forceinline__ float xor_max(float x) {
  return fmaxf(x, xor_get<d>(x));
}

// Maximum over lanes that agree in the bits below g (g a power of two).
__device__ __forceinline__ float group_max(float x, int g) {
  x = xor_max<32>(x);
  if (g <= 16) x = xor_max<16>(x);
  if (g <= 8) x = xor_max<8>(x);
  if (g <= 4) x = xor_max<4>(x);
  if (g <= 2) x = xor_max<2>(x);
  if (g <= 1) x = xor_max<1>(x);
  return x;
}

__device__ __forceinline__ float group_sum(float x, int g) {
  x = xor_sum<32>(x);
  if (g <= 16) x = xor_sum<16>(x);
  if (g <= 8) x = xor_sum<8>(x);
  if (g <= 4) x = xor_sum<4>(x);
  if (g <= 2) x = xor_sum<2>(x);
  if (g <= 1) x = xor_sum<1>(x);
  return x;
}

// Raw bits of E consecutive elements of a K/V row.
template <typename T, int E>
using piece_t = std::conditional_t<E * sizeof(T) == 2, uint16_t,
                                   std::conditional_t<E * sizeof(T) == 4, uint32_t, uint64_t>>;

template <typename T, int E>
__device__ __forceinline__ float piece_elem(piece_t<T, E> r, int e) {
  if constexpr (sizeof(T) == 2) return __builtin_bit_cast(float, (uint32_t)((r >> (16 * e)) & 0xffffu) << 16);
  else return __builtin_bit_cast(float, (uint32_t)(r >> (32 * e)));
}

// Decode row-block metadata from one round of loads, one lane per request of the block
// (a block holds at most 64): the request's req_to_token row and key count, raw, and its
// shared_len hint to the previous request. Issued first and reduced later, so that other
// loads can be in flight in between.
struct BlockMeta {
  int row, len, sh;
  bool in;  // the lane holds a request of the block
};
__device__ __forceinline__ BlockMeta block_meta_load(const AttnArgs& a, int64_t rb, int lane, bool load_len = true) {
  // 32-bit index math (rows < 2^31): 64-bit divisions cost hundreds of instructions here
  const int qa = (int)rb * a.bm / a.g;
  const int qb = min(qa + a.bm / a.g, a.batch);
  const int r = qa + lane;
  const bool in = r < qb;
  const int rr = in ? r : qa;  // unconditional loads
  BlockMeta m;
  m.row = a.req_pool_idx[rr];
  m.len = load_len ? a.kv_len[rr] : 0;
  m.sh = a.shared_len ? a.shared_len[rr] : 0;
  m.in = in;
  return m;
}

// Shared length L of the block, by the rule every decode kernel applies: the minimum over
// its requests of their key counts minus one (0 for a request whose row or length is
// invalid) and of the shared_len hints between neighbours (the block's first request has
// none). The minus one keeps every request's newest key in its own part, so the shared
// part never reads a key that this step's append writes (rax_decode_step folds the
// append into the shared-part kernel). Wave-uniform.
__device__ __forceinline__ int block_shared_len(const AttnArgs& a, const BlockMeta& m, int lane) {
  int v = 1 << 30;
  if (m.in) {
    const bool ok = m.row >= 0 && m.row < a.rtt_rows && m.len >= 0 && m.len <= a.rtt_stride;
    v = min(ok ? m.len - 1 : 0, lane == 0 ? (1 << 30) : m.sh);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off));
  return uni(max(v, 0));
}

__device__ __forceinline__ int block_shared_len(const AttnArgs& a, int64_t rb, int lane) {
  return block_shared_len(a, block_meta_load(a, rb, lane), lane);
}

// Deeper runs inside a row block. A request whose shared_len hint to its predecessor
// exceeds the block's shared length L0 joins the predecessor's run: the runs are the
// subtrees of the radix tree below the block's common prefix, contiguous when a batch is
// in tree order (a system prompt branching into few-shot blocks puts a whole block of
// questions in one run). A run of two or more requests shares keys [L0, L1) of its first
// request's slot row, L1 by block_shared_len's rule over the run alone (so the newest key
// of each request stays its own). Runs are taken in request order while their extra
// 64-key tiles add up to at most a.run_cap: the shared-part kernel computes a taken run's
// tiles once for the run's rows, and the own parts of its requests start at L1. Every
// decode kernel derives the same runs from the same block metadata. Wave-uniform except
// where noted.
struct BlockRuns {
  int L0;          // shared length of the whole block
  int l1;          // per lane: where the lane's request's own keys start (L0, or its run's L1)
  int end;         // per lane: one past the last request of the lane's run (block-relative)
  int excl;        // per lane: extra tiles of the taken runs before the lane's run
  uint64_t heads;  // lanes whose request is the first of a taken run
  int tiles;       // extra tiles of all taken runs
};
__device__ __forceinline__ BlockRuns block_runs(const AttnArgs& a, const BlockMeta& m, int lane) {
  BlockRuns b;
  b.L0 = block_shared_len(a, m, lane);
  b.l1 = b.L0;
  b.end = lane + 1;
  b.excl = 0;
  b.heads = 0;
  b.tiles = 0;
  if (a.run_cap <= 0) return b;
  const bool join = m.in && lane > 0 && m.sh > b.L0;
  if (!__ballot(join)) return b;  // no deeper run: the common case costs one ballot
  const bool ok = m.in && m.row >= 0 && m.row < a.rtt_rows && m.len >= 0 && m.len <= a.rtt_stride;
  const int own_v = ok ? m.len - 1 : 0;
  const uint64_t starts = __ballot(m.in && !join);  // bit 0 set: a block holds request 0
  const int nb = __popcll(__ballot(m.in));
  const uint64_t upto = lane == 63 ? ~0ull : (2ull << lane) - 1;  // lanes 0 .. lane
  const int head = 63 - __builtin_clzll((starts & upto) | 1ull);
  const uint64_t later = starts & ~upto;
  const int end = later ? __builtin_ctzll(later) : nb;
  // segmented minimum over [head, lane] of the rule's terms, then the run's at its last lane
  int w = m.in ? (lane == head ? own_v : min(own_v, m.sh)) : (1 << 30);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(w, off);
    if (lane - off >= head) w = min(w, y);
  }
  const int l1 = __shfl(w, end > 0 ? end - 1 : 0);
  const bool cand = m.in && lane == head && end - head >= 2 && l1 > b.L0;
  const int nt = cand ? (l1 - b.L0 + BN - 1) / BN : 0;
  int incl = nt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  const bool take = cand && incl <= a.run_cap;
  b.heads = __ballot(take);
  b.excl = incl - nt;
  b.tiles = b.heads ? __builtin_amdgcn_readlane(incl, 63 - __builtin_clzll(b.heads)) : 0;
  const bool run_taken = __shfl(take ? 1 : 0, head) != 0;
  if (m.in && run_taken) b.l1 = l1;
  b.end = end;
  return b;
}

// Where the own keys of request rl of the block (block-relative, wave-uniform) start.
__device__ __forceinline__ int row_shared_len(const AttnArgs& a, const BlockMeta& m, int lane, int rl) {
  if (a.run_cap <= 0) return block_shared_len(a, m, lane);
  return __builtin_amdgcn_readlane(block_runs(a, m, lane).l1, rl);
}

// Own keys of request r in split decode: positions [L, seq_len), L the shared length of the
// request's row block. They are cut into n_act <= n_chunk chunks of about equal size, each
// at least a.own_min keys. Returns n_act (0: nothing of its own, or an invalid row) and
// sets the first own position and the chunk size.
constexpr int kOwnMin = 32;       // own_kernel / own_merge_kernel
// own_stream_kernel: chunks of at least 1024 keys, at most 4 per (request, KV head) unless
// more keep each within 1024 keys (or one chunk per request, see decode_layout). Measured
// (with the tile-round form it replaced)
// on GQA decode (self-consistency 64/8, multi-turn 32/8) from 128/8 to 1024/4: fewer,
// longer chunks win (275 -> 225 us, 204 -> 159 us); idle workgroups (chunks past a
// request's keys) and partials to merge cost more than the parallelism they add.
constexpr int kOwnTileMin = 1024;
constexpr int64_t kOneChunkItems = 1024;  // (request, KV head) pairs for one chunk per request
constexpr int kOwnTileChunks = 4;
__device__ __forceinline__ int own_chunks(const AttnArgs& a, int row, int end, int L, int& first, int& per) {
  first = L;
  per = 0;
  if (row < 0 || row >= a.rtt_rows || end < 0 || end > a.rtt_stride) return 0;
  const int n = end - L;
  if (n <= 0) return 0;
  const int n_act = min(a.n_chunk, (n + a.own_min - 1) / a.own_min);
  per = (n + n_act - 1) / n_act;
  return n_act;
}
__device__ __forceinline__ int own_chunks(const AttnArgs& a, int r, int L, int& first, int& per) {
  return own_chunks(a, a.req_pool_idx[r], a.kv_len[r], L, first, per);
}

// Own part of decode: the keys of one request that its row block does not share (see
// own_chunks). No LDS in the key loop and no barriers: an HBM-bound gather with wavefront
// reductions. Lane l holds dims [l*E, l*E+E) (E = D/64) of the G query heads of the KV
// head. A batch of KB keys: the slot ids are one load per lane, then every K and V row
// piece of the batch is loaded at once (addresses of keys without a slot are clamped to
// slot 0 and their values dropped), giving P = KB*G (key, head) partial dot products per
// lane; wave_reduce_pairs leaves the score of pair l in lane l. Softmax state per head is
// wave-uniform; P.V takes each key's probability with v_readlane and accumulates in fp32.
// own_chunk runs one wave over keys [start, stop) of request r, KV head h.
// This lane's dims of the G query heads of (request r, KV head h), in fp32.
template <typename T, int D, int G>
__device__ __forceinline__ void load_q_heads(const AttnArgs& a, int r, int h, int lane, float (&q)[G][D / 64]) {
  constexpr int E = D / 64;
  const T* qp = reinterpret_cast<const T*>(a.q) + ((int64_t)r * a.h_q + (int64_t)h * G) * D + lane * E;
#pragma unroll
  for (int hl = 0; hl < G; ++hl)
#pragma unroll
    for (int e = 0; e < E; ++e) q[hl][e] = (float)qp[hl * D + e];
}

template <typename T, int D, int G>
__device__ __forceinline__ void own_chunk(const AttnArgs& a, int h, int row, int start, int stop, int lane,
                                          const float (&q)[G][D / 64], float (&acc)[G][D / 64], float (&m_run)[G],
                                          float (&l_run)[G]) {
  constexpr int E = D / 64;
  constexpr int KB = 32 / G > 0 ? 32 / G : 1;  // 32 (key, head) pairs per batch
  constexpr int P = KB * G;
  using Raw = piece_t<T, E>;
#pragma unroll
  for (int hl = 0; hl < G; ++hl) {
    m_run[hl] = kNegInf;
    l_run[hl] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[hl][e] = 0.f;
  }
  const int64_t row_elems = (int64_t)a.h_kv * D;
  const T* kb = reinterpret_cast<const T*>(a.k_pool) + (int64_t)h * D + lane * E;
  const T* vb = reinterpret_cast<const T*>(a.v_pool) + (int64_t)h * D + lane * E;
  const int32_t* rtt_row = a.rtt + (int64_t)row * a.rtt_stride;
  const int my_key = (lane % P) / G;
  const int my_hl = lane % G;

  // Load rounds of KL keys: one slot-id load, then every K and V piece of the round in
  // flight at once; the round's keys are then scored in batches of KB keys (P pairs). With
  // query-head groups (G > 1) a batch has fewer keys, but a round still fetches 32, so the
  // number of dependent round trips does not grow with G.
  constexpr int KL = sizeof(Raw) <= 4 && KB < 32 ? 32 : KB;
  constexpr int NSUB = KL / KB;
  static_assert(KL % KB == 0 && KL <= 64, "load round");
  for (int j0 = start; j0 < stop; j0 += KL) {
    const int nk = min(KL, stop - j0);
    const int raw_slot = rtt_row[j0 + min(lane, nk - 1)];
    int slot = -1;
    if (lane < nk) {
      if (raw_slot >= 0 && raw_slot < a.num_slots) slot = raw_slot;
      else flag_error(RAX_DEVERR_SLOT);
    }
    const uint64_t valid_all = __ballot(slot >= 0);
    Raw kr[KL], vr[KL];
#pragma unroll
    for (int kk = 0; kk < KL; ++kk) {
      const int s = __builtin_amdgcn_readlane(slot, kk);
      const int64_t off = (int64_t)(s < 0 ? 0 : s) * row_elems;
      kr[kk] = *reinterpret_cast<const Raw*>(kb + off);
      vr[kk] = *reinterpret_cast<const Raw*>(vb + off);
    }
#pragma unroll
    for (int kk = 0; kk < KL; ++kk) vr[kk] = ((valid_all >> kk) & 1) ? vr[kk] : (Raw)0;
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
    if (sb * KB >= nk) break;  // no keys left in this round
    const uint64_t valid = valid_all >> (sb * KB);
    float v[P];
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int hl = 0; hl < G; ++hl) {
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) x += q[hl][e] * piece_elem<T, E>(kr[sb * KB + kk], e);
        v[kk * G + hl] = x;
      }
    wave_reduce_pairs<P>(v, lane);
    const bool ok = lane < P && ((valid >> my_key) & 1);
    const float sc = ok ? v[0] * a.scale_log2 : kNegInf;
    const float mx = group_max(sc, G);  // lane hl < G holds head hl's batch maximum
    float mu_lane = 0.f;
#pragma unroll
    for (int hl = 0; hl < G; ++hl) {
      const float bmax = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), hl));
      const float m_new = fmaxf(m_run[hl], bmax);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[hl] - m_use);
      l_run[hl] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[hl][e] *= alpha;
      m_run[hl] = m_new;
      if (my_hl == hl) mu_lane = m_use;
    }
    const float pr = __builtin_amdgcn_exp2f(sc - mu_lane);
    const float ps = group_sum(pr, G);
#pragma unroll
    for (int hl = 0; hl < G; ++hl)
      l_run[hl] += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ps), hl));
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int hl = 0; hl < G; ++hl) {
        const float pk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr), kk * G + hl));
#pragma unroll
        for (int e = 0; e < E; ++e) acc[hl][e] += pk * piece_elem<T, E>(vr[sb * KB + kk], e);
      }
    }
  }
}

// Own part, general form: one wave per (chunk, request, KV head), chunk index slowest so
// that chunks past every request's own keys are whole workgroups that exit at once;
// partials go to the workspace and merge_kernel combines them with the shared part's.
template <typename T, int D, int G>
__global__ void __launch_bounds__(256) own_kernel(AttnArgs a) {
  constexpr int E = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n_rh = (int64_t)a.batch * a.h_kv;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= n_rh * a.n_chunk) return;
  const int c = (int)(w / n_rh);
  const int64_t rh = w % n_rh;
  const int r = (int)(rh / a.h_kv);
  const int h = (int)(rh % a.h_kv);
  float q[G][E];
  load_q_heads<T, D, G>(a, r, h, lane, q);  // issued first: it depends on nothing else
  int first, per;
  const int rbk = r * G / a.bm;
  const int L = row_shared_len(a, block_meta_load(a, rbk, lane), lane, r - rbk * a.bm / G);
  const int n_act = own_chunks(a, r, L, first, per);
  if (c >= n_act) return;  // the merge reads only chunks [0, n_act)
  const int start = first + c * per;
  const int stop = min(start + per, (int)a.kv_len[r]);
  float acc[G][E], m_run[G], l_run[G];
  own_chunk<T, D, G>(a, h, a.req_pool_idx[r], start, stop, lane, q, acc, m_run, l_run);
  const int64_t item = rh * a.n_chunk + c;
  float* out_acc = a.ws_own + item * G * (int64_t)D;
  float* out_ml = a.ws_own + n_rh * a.n_chunk * G * (int64_t)D + item * G * 2;
#pragma unroll
  for (int hl = 0; hl < G; ++hl) {
#pragma unroll
    for (int e = 0; e < E; ++e) out_acc[(int64_t)hl * D + lane * E + e] = acc[hl][e];
  }
#pragma unroll
  for (int hl = 0; hl < G; ++hl)
    if (lane == hl) {
      out_ml[hl * 2] = m_run[hl];
      out_ml[hl * 2 + 1] = l_run[hl];
    }
}

// Own part with the merge folded in: one workgroup per (request, KV head), wave c runs own
// chunk c (W = n_chunk waves). The chunk states meet in LDS; after one barrier, wave w
// merges query heads w, w + W, ... : the shared part's split partials of the head's row
// (written by the previous kernel) and the W chunk states, by log-sum-exp, then writes O.
// Dynamic LDS: W*G*D floats of accumulators, then W*G (m, l) pairs.
// Leading scalar arguments: preloaded copies of fields of `a` (see shared_kernel).
template <typename T, int D, int G>
__global__ void __launch_bounds__(512) own_merge_kernel(const void* p_q, float* p_ws, const int32_t* p_rpi,
                                                        const int32_t* p_len, const int32_t* p_sh, int32_t h_kv,
                                                        int32_t bm, int32_t batch, int32_t split_rb, AttnArgs a) {
  a.q = p_q;
  a.ws = p_ws;
  a.req_pool_idx = p_rpi;
  a.kv_len = p_len;
  a.shared_len = p_sh;
  a.h_kv = h_kv;
  a.h_q = h_kv * G;
  a.g = G;
  a.bm = bm;
  a.batch = batch;
  a.nsplit = split_rb & 255;  // nsplit <= 32, n_rb < 2^23 (checked on the host)
  a.n_rb = split_rb >> 8;
  constexpr int E = D / 64;
  constexpr int PER = D / 64;
  extern __shared__ float own_lds[];
  const int W = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rh = blockIdx.x;
  const int r = rh / a.h_kv;
  const int h = rh - r * a.h_kv;
  float* s_acc = own_lds;
  float* s_ml = own_lds + (int64_t)W * G * D;
  const int nsplit = a.nsplit;
  const int64_t n_items = (int64_t)a.h_kv * a.n_rb * nsplit;
  // the split partials' (m, l) of this wave's first merged head, fetched now so that the
  // load overlaps the own-key work (they come from the previous kernel)
  // the Q heads and, for this wave's first merged head, the split partials' (m, l) and the
  // accumulator rows of the first kPre splits: all fetched now, so the loads overlap the
  // own-key work (the partials come from the previous kernel)
  constexpr int kPre = 8;
  // block metadata first: the own-key work waits for it, and loads complete in order
  const int rb0 = r * G / a.bm;
  const BlockMeta meta = block_meta_load(a, rb0, lane);
  float q[G][E];
  load_q_heads<T, D, G>(a, r, h, lane, q);
  float2 pre_ml = make_float2(kNegInf, 0.f);
  float pre_acc[kPre][PER];
  if (wave < G) {
    const int Grow = r * G + wave;
    const int rbw = Grow / a.bm, Rw = Grow - rbw * a.bm;
    const int64_t item0 = ((int64_t)h * a.n_rb + rbw) * nsplit;
    const float* sh_ml = a.ws + n_items * a.bm * (int64_t)D + (item0 * a.bm + Rw) * 2;
    pre_ml = *reinterpret_cast<const float2*>(sh_ml + (int64_t)(lane < nsplit ? lane : 0) * a.bm * 2);
    const float* sh_acc = a.ws + (item0 * a.bm + Rw) * (int64_t)D;
#pragma unroll
    for (int j = 0; j < kPre; ++j)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        pre_acc[j][i] = sh_acc[(int64_t)(j < nsplit ? j : 0) * a.bm * D + lane + 64 * i];
  }
  {
    // row and key count of request r from the block metadata's lanes
    const int rl = r - rb0 * a.bm / G;
    const int L = row_shared_len(a, meta, lane, rl);
    const int row = __builtin_amdgcn_readlane(meta.row, rl);
    const int end = __builtin_amdgcn_readlane(meta.len, rl);
    int first, per;
    const int n_act = own_chunks(a, row, end, L, first, per);
    float acc[G][E], m_run[G], l_run[G];
    if (wave < n_act) {
      const int start = first + wave * per;
      const int stop = min(start + per, end);
      own_chunk<T, D, G>(a, h, row, start, stop, lane, q, acc, m_run, l_run);
    } else {
#pragma unroll
      for (int hl = 0; hl < G; ++hl) {
        m_run[hl] = kNegInf;
        l_run[hl] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[hl][e] = 0.f;
      }
    }
#pragma unroll
    for (int hl = 0; hl < G; ++hl) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[(wave * G + hl) * D + lane * E + e] = acc[hl][e];
      if (lane == 0) {
        s_ml[(wave * G + hl) * 2] = m_run[hl];
        s_ml[(wave * G + hl) * 2 + 1] = l_run[hl];
      }
    }
  }
  __syncthreads();

  for (int hl = wave; hl < G; hl += W) {
    const int Grow = r * G + hl;  // MFMA row of (request r, query head h*G + hl)
    const int rb = Grow / a.bm;
    const int R = Grow - rb * a.bm;
    const int64_t item0 = ((int64_t)h * a.n_rb + rb) * nsplit;
    const float* sh_acc = a.ws + (item0 * a.bm + R) * (int64_t)D;
    const int64_t sh_stride = (int64_t)a.bm * D;
    const float* sh_ml = a.ws + n_items * a.bm * (int64_t)D + (item0 * a.bm + R) * 2;
    // lane s < nsplit: split partial s; nsplit <= s < nsplit + W: own chunk s - nsplit
    const int sl = lane < nsplit ? lane : 0;
    const float2 gml = hl == wave ? pre_ml : *reinterpret_cast<const float2*>(sh_ml + (int64_t)sl * a.bm * 2);
    const int oc = lane - nsplit;
    const bool own_lane = oc >= 0 && oc < W;
    const float om = own_lane ? s_ml[(oc * G + hl) * 2] : kNegInf;
    const float ol = own_lane ? s_ml[(oc * G + hl) * 2 + 1] : 0.f;
    const float my_m = lane < nsplit ? gml.x : om;
    const float my_l = lane < nsplit ? gml.y : ol;
    float M = my_l > 0.f ? my_m : kNegInf;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float Mu = M == kNegInf ? 0.f : M;
    const float my_w = my_l > 0.f ? exp2f(my_m - Mu) : 0.f;
    float lsum = my_w * my_l;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
    float o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    // split partials with nonzero weight: the prefetched ones (first head of this wave; a
    // partial that saw no key may hold stale data, hence the select), then the rest up
    // to 32 per round trip
    uint64_t nz = __ballot(lane < nsplit && my_w != 0.f);
    if (hl == wave) {
#pragma unroll
      for (int j = 0; j < kPre; ++j) {
        const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j));
        const bool use = j < nsplit && wj != 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] += use ? wj * pre_acc[j][i] : 0.f;
      }
      nz &= ~(uint64_t)((1u << kPre) - 1);
    }
    constexpr int U = 32;
    const int s_first = nz ? __builtin_ctzll(nz) : 0;
    while (nz) {
      float x[U][PER], wt[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int sp = nz ? __builtin_ctzll(nz) : s_first;
        wt[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), sp));
        if (!nz) wt[j] = 0.f;
        nz &= nz - 1;
        const float* pp = sh_acc + sp * sh_stride;
#pragma unroll
        for (int i = 0; i < PER; ++i) x[j][i] = pp[lane + 64 * i];
      }
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] += wt[j] * x[j][i];
    }
    // own chunks (LDS)
    for (int c = 0; c < W; ++c) {
      const float wc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), nsplit + c));
      if (wc != 0.f) {
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] += wc * s_acc[(c * G + hl) * D + lane + 64 * i];
      }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int64_t obase = ((int64_t)r * a.h_q + (int64_t)h * G + hl) * (int64_t)D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (a.o_bf16) reinterpret_cast<__bf16*>(a.o)[obase + lane + 64 * i] = (__bf16)(o[i] * inv);
      else reinterpret_cast<float*>(a.o)[obase + lane + 64 * i] = o[i] * inv;
    }
  }
}

// Log-sum-exp merge of partials: one wave per (MFMA row, KV head). Inputs are the split
// partials of the row's block and, for split decode, the own-part chunks of the row's
// request. Lane s fetches partial s's (m, l) for every partial that may exist, in the same
// round trip as the request's own-chunk count; then only partials with nonzero weight are
// visited, up to 32 per round trip, with unconditional loads (spare load slots read the
// first such partial and get weight 0).
template <int D>
__global__ void __launch_bounds__(256) merge_kernel(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t G = (int64_t)blockIdx.x * 4 + wave;
  const int h = blockIdx.y;
  const int64_t t = G / a.g;
  if (t >= a.total_q) return;
  const int hl = (int)(G % a.g);
  const int hq = h * a.g + hl;
  const int64_t rb = G / a.bm;
  const int R = (int)(G % a.bm);
  const int nsplit = a.nsplit;
  const int64_t n_items = (int64_t)a.h_kv * a.n_rb * nsplit;
  const int64_t item0 = ((int64_t)h * a.n_rb + rb) * nsplit;
  const int64_t own_items = (int64_t)a.batch * a.h_kv * a.n_chunk;
  const int64_t own0 = (t * a.h_kv + h) * a.n_chunk;  // own items of (request t, KV head h)
  // partial s < nsplit: split s of the block; otherwise own chunk s - nsplit
  const float* sh_acc = a.ws + (item0 * a.bm + R) * (int64_t)D;
  const int64_t sh_stride = (int64_t)a.bm * D;
  const float* sh_ml = a.ws + n_items * a.bm * (int64_t)D + (item0 * a.bm + R) * 2;
  const float* own_base = a.shared_only ? a.ws_own : a.ws;  // no own partials: never read
  const float* own_acc = own_base + (own0 * a.g + hl) * (int64_t)D - (int64_t)nsplit * a.g * D;
  const int64_t own_stride = (int64_t)a.g * D;
  const float* own_ml = own_base + own_items * a.g * (int64_t)D + (own0 * a.g + hl) * 2 - (int64_t)nsplit * a.g * 2;
  const int n_max = nsplit + (a.shared_only ? a.n_chunk : 0);  // <= 64
  const int sl = lane < n_max ? lane : 0;
  const float2 mlv = *reinterpret_cast<const float2*>(sl < nsplit ? sh_ml + (int64_t)sl * a.bm * 2
                                                                  : own_ml + (int64_t)sl * a.g * 2);
  const float my_m = mlv.x;
  float my_l = lane < n_max ? mlv.y : 0.f;
  int n_own = 0, first = 0, per = 0;
  if (a.shared_only) {
    const int rl = (int)(t - rb * a.bm / a.g);  // request t's lane in its block's metadata
    n_own = own_chunks(a, (int)t, row_shared_len(a, block_meta_load(a, rb, lane), lane, rl), first, per);
  }
  // own_stream_kernel merged this row and wrote O
  if (a.own_fused == 2 && (n_own == 1 || (n_own > 1 && a.own_fold))) return;
  if (lane >= nsplit + n_own) my_l = 0.f;  // own chunks past n_own were not written
  float M = my_l > 0.f ? my_m : kNegInf;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float Mu = M == kNegInf ? 0.f : M;
  const float my_w = my_l > 0.f ? exp2f(my_m - Mu) : 0.f;
  float lsum = my_w * my_l;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
  constexpr int PER = D / 64;
  constexpr int U = 32;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  uint64_t nz = __ballot(my_w != 0.f);
  const int s_first = nz ? __builtin_ctzll(nz) : 0;
  while (nz) {
    float x[U][PER], w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int s = nz ? __builtin_ctzll(nz) : s_first;
      w[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), s));
      if (!nz) w[j] = 0.f;
      nz &= nz - 1;
      const float* p = s < nsplit ? sh_acc + s * sh_stride : own_acc + s * own_stride;
#pragma unroll
      for (int i = 0; i < PER; ++i) x[j][i] = p[lane + 64 * i];
    }
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] += w[j] * x[j][i];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int64_t obase = (t * a.h_q + hq) * (int64_t)D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (a.o_bf16) reinterpret_cast<__bf16*>(a.o)[obase + lane + 64 * i] = (__bf16)(o[i] * inv);
    else reinterpret_cast<float*>(a.o)[obase + lane + 64 * i] = o[i] * inv;
  }
}

// Shared-prefix part of split decode, bf16 with D = 128: the keys every request of a
// 64-row block shares (positions [0, L) of the block's first request's slot row), then
// the keys [L, L1) that each taken run of the block shares beyond them (block_runs: from
// the run's first request's row, scores masked to the run's rows), all cut into nsplit
// ranges of whole tiles; partials in attn_kernel's layout (a row that saw no key of a
// split gets l = 0 there, which the merges skip). attn_kernel
// stages one tile at a time through registers, so each tile costs a full memory round
// trip, and with one workgroup per CU nothing hides it. Here a workgroup issues the K
// and V rows of a round of ST tiles at once straight into LDS (16-byte global-to-LDS
// loads that hold no registers), then computes the first half of the round while the
// second half may still be arriving. 2 x NKG waves: two 32-row tiles x NKG key groups;
// the 32-key halves of a round's tiles go round-robin to the key groups, whose softmax
// states combine in LDS at the end. Two forms: NKG = 4, ST = kShTiles (8 waves, 128 KB of
// LDS, one workgroup per CU), and, when a split holds many tiles, NKG = 2, ST = 2 (4
// waves, 64 KB, two workgroups per CU), which runs its tiles through a ring of two slots
// (tile_loop). (Running the requests' own
// keys in the same workgroups, while the tiles arrive, measured slower: with eight waves
// per CU each own-key stream is a chain of round trips that the separate own-part
// kernel's 16 waves per CU hide.) LDS layout and fragment reads: see "tiles loaded
// straight into LDS" above.
constexpr int kShTiles = 4;

// The leading scalar arguments repeat fields of `a`: the compiler preloads the first 14
// argument dwords into SGPRs at wave launch (kernel-argument preloading), so the loads
// of the block metadata and Q are issued without first waiting for an argument fetch.
template <int D, int NKG, int ST>
__global__ void __launch_bounds__(128 * NKG) __attribute__((amdgpu_waves_per_eu(NKG == 2 ? 2 : 1)))
shared_kernel(const int32_t* p_rpi, const int32_t* p_len, const int32_t* p_sh,
                                                     const void* p_q, int32_t n_items, int32_t nsplit, int32_t n_rb,
                                                     int32_t g, int32_t batch, int32_t h_q, AttnArgs a, AppendJob ap) {
  static_assert(D == 128, "the swizzle assumes 16 chunks per row");
  a.req_pool_idx = p_rpi;
  a.kv_len = p_len;
  a.shared_len = p_sh;
  a.q = p_q;
  a.nsplit = nsplit;
  a.n_rb = n_rb;
  a.g = g;
  a.batch = batch;
  a.h_q = h_q;
  constexpr int NW = 2 * NKG;          // waves: two row tiles x NKG key groups
  constexpr int BM = 64;
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int RB = D * 2;            // bytes per row
  constexpr int TB = BN * RB;          // bytes per K (or V) tile
  constexpr int RPI = 1024 / RB;       // rows per 1 KB global-to-LDS instruction
  constexpr int NI = BN / RPI;         // instructions per tile
  constexpr int NKS = D / 16;
  __shared__ __align__(16) char kv[2 * ST * TB];  // ST K tiles, then ST V tiles
  __shared__ int32_t slot[ST * BN];
  const uint32_t kv_lds = lds_addr(kv);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wrow = wave & 1, wkey = wave >> 1;  // 32-row tile, key group
  const int jrow = lane & 31, half = lane >> 5;
  // 32-bit index math (grid and rows < 2^31): 64-bit divisions cost hundreds of
  // instructions before the first load could issue
  const int item = (int)xcd_remap(blockIdx.x, n_items);
  const int isp = item / nsplit;
  const int split = item - isp * nsplit;
  const int h = isp / n_rb;
  const int rb = isp - h * n_rb;
  const int G0 = rb * BM;
  const int qa = G0 / g;
  const int qb = min(qa + BM / g, batch);

  // block metadata and Q fragments of this lane's row (B operand of S^T = K Q^T) first:
  // their addresses need only the preloaded arguments. Lengths are loaded from memory
  // even when the job carries them (the value is then replaced below: this launch's
  // append may be rewriting it).
  a.bm = BM;
  BlockMeta bmeta = block_meta_load(a, rb, lane, true);
  const int R = wrow * 32 + jrow;
  const int Gr = G0 + R;
  const int t_row = Gr / g;
  const bool row_ok = t_row < qb;
  const int hq = h * g + (Gr - t_row * g);
  bf16x8 qf[NKS];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + ((int64_t)(row_ok ? t_row : qa) * a.h_q + hq) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + half * 8);
      qf[ks] = row_ok ? v : bf16x8{};
    }
  }

  if (a.own_cnt) {  // the own part's chunk counters start at zero (this launch precedes it)
    const int n_cnt = batch * a.h_kv;
    for (int i = (int)blockIdx.x * NW * 64 + tid; i < n_cnt; i += (int)gridDim.x * NW * 64) a.own_cnt[i] = 0;
  }

  // A decode step's append carried by this launch (rax_decode_step): token i's K/V row to
  // its slot, the slot into its row at len - 1, len to seq_len_dev (what
  // decode_append_kernel does). This kernel reads none of it: its keys end before every
  // request's newest position, and it takes the lengths from the job. The workgroup's
  // first token is loaded into registers now and stored after the tiles are computed, so
  // that no wait for it sits on the path to the tile loads; further tokens (more tokens
  // than workgroups) and row chunks past kApR per thread are copied at the end.
  constexpr int kApR = 2;
  const bool ap_mine = (int)blockIdx.x < ap.n;
  const int64_t ap_cpr = ap.chunks_per_row;
  u32x4 ap_k[kApR], ap_v[kApR];
  if (ap_mine) {
    const u32x4* kn = reinterpret_cast<const u32x4*>(ap.k_new) + (int64_t)blockIdx.x * ap_cpr;
    const u32x4* vn = reinterpret_cast<const u32x4*>(ap.v_new) + (int64_t)blockIdx.x * ap_cpr;
#pragma unroll
    for (int j = 0; j < kApR; ++j) {
      const int64_t c = tid + (int64_t)j * 64 * NW;
      ap_k[j] = c < ap_cpr ? kn[c] : u32x4{};
      ap_v[j] = c < ap_cpr ? vn[c] : u32x4{};
    }
  }
  if (ap.n > 0) {  // lengths after this step's append: from the job, not memory
    const int r = qa + lane;
    bmeta.len = ap.len[r < ap.n ? r : qa];
  }
  const bool all_rows_ok = __all(row_ok);

  const BlockRuns br = block_runs(a, bmeta, lane);
  const int L = br.L0;  // 0 if the first request's row is invalid
  const int row0 = __builtin_amdgcn_readfirstlane(bmeta.row);
  const int n_sh = (L + BN - 1) / BN;
  // the block's tiles: its shared keys [0, L), then each taken run's keys [L, L1)
  // (block_runs), cut into nsplit ranges of whole tiles
  const int n_vt = n_sh + br.tiles;
  const int t_begin = (int)(((int64_t)n_vt * split) / a.nsplit);
  const int t_end = (int)(((int64_t)n_vt * (split + 1)) / a.nsplit);
  const int rq = t_row - qa;  // request of this lane's row, block-relative
  const int64_t row_bytes = (int64_t)a.h_kv * RB;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (int64_t)h * RB;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (int64_t)h * RB;

  // Tile v of the block: positions [k0, k1) of slot row `row`, seen by the rows of the
  // block's requests [ra, rb) (wave-uniform)
  struct TileRef {
    int k0, k1, row, ra, rb;
  };
  auto tile_ref = [&](int v) {
    TileRef r;
    if (v < n_sh) {
      r.k0 = v * BN;
      r.k1 = L;
      r.row = row0;
      r.ra = 0;
      r.rb = 64;
      return r;
    }
    const int u = v - n_sh;  // run tiles: the last taken run starting at or before u
    const uint64_t at = __ballot(((br.heads >> lane) & 1ull) && br.excl <= u);
    const int hd = 63 - __builtin_clzll(at | 1ull);
    r.k0 = L + (u - __builtin_amdgcn_readlane(br.excl, hd)) * BN;
    r.k1 = __builtin_amdgcn_readlane(br.l1, hd);
    r.row = __builtin_amdgcn_readlane(bmeta.row, hd);
    r.ra = hd;
    r.rb = __builtin_amdgcn_readlane(br.end, hd);
    return r;
  };
  // the round's tiles as named values, picked by selects (an array indexed by a
  // variable tile number would live in scratch memory)
  static_assert(ST == 2 || ST == 4, "tiles per round");
  TileRef tr0, tr1, tr2, tr3;
  auto tile_of = [&](int t) {
    auto pick = [t](int x0, int x1, int x2, int x3) { return t == 0 ? x0 : t == 1 ? x1 : t == 2 ? x2 : x3; };
    TileRef r;
    r.k0 = pick(tr0.k0, tr1.k0, tr2.k0, tr3.k0);
    r.k1 = pick(tr0.k1, tr1.k1, tr2.k1, tr3.k1);
    r.row = pick(tr0.row, tr1.row, tr2.row, tr3.row);
    r.ra = pick(tr0.ra, tr1.ra, tr2.ra, tr3.ra);
    r.rb = pick(tr0.rb, tr1.rb, tr2.rb, tr3.rb);
    return r;
  };

  // slot ids, then every K and V row of the round's tiles into LDS
  auto issue = [&](int nt, auto tile) {
    for (int i = tid; i < nt * BN; i += 64 * NW) {
      const TileRef r = tile(i / BN);
      const int pos = r.k0 + i % BN;
      const bool in = pos < r.k1;
      int sv = a.rtt[in ? (int64_t)r.row * a.rtt_stride + pos : 0];
      if (in && (sv < 0 || sv >= a.num_slots)) {
        flag_error(RAX_DEVERR_SLOT);
        sv = -1;
      }
      slot[i] = in ? sv : -1;
    }
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
#pragma unroll
      for (int q = wave; q < NI; q += NW) {
        const int r = q * RPI + lane / CH;
        const int sv = slot[t * BN + r];
        const int64_t off = (int64_t)(sv < 0 ? 0 : sv) * row_bytes;
        lds_load16(kbase + off + (((lane % CH) ^ swz_k(r)) * 16), uni(kv_lds + t * TB + q * 1024));
        lds_load16(vbase + off + (((lane % CH) ^ swz_v(r)) * 16), uni(kv_lds + (ST + t) * TB + q * 1024));
      }
    }
  };
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  // One 32-key half (sub) of a tile in LDS (kt, vt) for this wave's rows: S^T on MFMA,
  // online softmax, O^T += V^T P^T.
  auto half_step = [&](const char* kt, const char* vt, const TileRef& tt, int sub) {
    const int cnt = min(BN, tt.k1 - tt.k0);
    const bool rows_in = rq >= tt.ra && rq < tt.rb;  // run tiles: the run's rows only
    // S^T over this wave's 32 keys: row kr of the tile, dims ks*16 + half*8
    f32x16 sc = f32x16{};
    const int kr = sub * 32 + jrow;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(kt, kr, ks, half), qf[ks], sc, 0, 0, 0);
    }
    // register r holds key sub*32 + 8*(r/4) + 4*half + r%4 of this lane's row
    const bool unmasked = cnt == BN && all_rows_ok && tt.ra == 0 && tt.rb == 64;
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = sc[r];
      if (!unmasked) {
        const int key = sub * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        v = row_ok && rows_in && key < cnt ? v : kNegInf;
      }
      sc[r] = v;
      mx = fmaxf(mx, v);
    }
    mx = max_xor32(mx) * a.scale_log2;
    // lazy rescale, as in attn_kernel: the reference moves only when a row's maximum
    // exceeds it by more than 2^kLazy
    if (__any(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
      m_run = m_new;
    }
    const float neg_m = m_run == kNegInf ? 0.f : -m_run;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], a.scale_log2, neg_m));
      sc[r] = p;
      psum += p;
    }
    psum = sum_xor32(psum);
    l_run += psum;
    bf16x8 pb[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[kh][e] = (__bf16)sc[kh * 8 + e];
    // O^T += V^T P^T (V^T fragments by transposing LDS reads)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_frag(vt, sub, dt, kh, lane), pb[kh], acc[dt], 0, 0, 0);
  };

  // The tile loop in two forms: blocks with taken runs, and blocks without (every tile
  // from the block's row for all rows, whose code stays that of the plain loop).
  auto tile_loop = [&](auto with_runs) {
  constexpr bool kRuns = decltype(with_runs)::value;
  if constexpr (ST == 2) {
    // Two-tile form: a ring of two tile slots, one tile at a time. While tile v is
    // computed, tile v + 1's K/V rows and tile v + 2's slot ids (into registers) are in
    // flight, so a tile's ids never wait in front of its loads and each tile takes one
    // barrier. The slot-id list holds the ids of the ring's two tiles.
    auto tref = [&](int v) {
      if constexpr (kRuns) {
        return tile_ref(v);
      } else {
        TileRef r;
        r.k0 = v * BN;
        r.k1 = L;
        r.row = row0;
        r.ra = 0;
        r.rb = 64;
        return r;
      }
    };
    int id_raw = 0;
    bool id_in = false;
    auto load_ids = [&](int v) {  // threads < BN: the id of key tid of tile v, into a register
      const TileRef r = tref(v);
      const int pos = r.k0 + tid;
      id_in = tid < BN && pos < r.k1;
      id_raw = id_in ? a.rtt[(int64_t)r.row * a.rtt_stride + pos] : 0;
    };
    auto put_ids = [&](int v) {  // ... into tile v's half of the list (out of range: -1)
      if (tid < BN) {
        int sv = id_raw;
        if (id_in && (sv < 0 || sv >= a.num_slots)) {
          flag_error(RAX_DEVERR_SLOT);
          sv = -1;
        }
        slot[((v - t_begin) & 1) * BN + tid] = id_in ? sv : -1;
      }
    };
    auto issue_kv = [&](int v) {  // every K and V row of tile v into its ring slot
      const int t = (v - t_begin) & 1;
#pragma unroll
      for (int q = wave; q < NI; q += NW) {
        const int r = q * RPI + lane / CH;
        const int sv = slot[t * BN + r];
        const int64_t off = (int64_t)(sv < 0 ? 0 : sv) * row_bytes;
        lds_load16(kbase + off + (((lane % CH) ^ swz_k(r)) * 16), uni(kv_lds + t * TB + q * 1024));
        lds_load16(vbase + off + (((lane % CH) ^ swz_v(r)) * 16), uni(kv_lds + (ST + t) * TB + q * 1024));
      }
    };
    if (t_begin < t_end) {
      load_ids(t_begin);
      put_ids(t_begin);
      if (t_begin + 1 < t_end) load_ids(t_begin + 1);
      __syncthreads();
      issue_kv(t_begin);
    }
    for (int v = t_begin; v < t_end; ++v) {
      const int t = (v - t_begin) & 1;
      // tile v's rows and tile v + 1's ids (issued during tile v - 1) have arrived
      __builtin_amdgcn_s_waitcnt(0);
      if (v + 1 < t_end) put_ids(v + 1);
      // every wave's rows of tile v in LDS, tile v + 1's ids written, and every wave done
      // with tile v - 1, whose ring slot tile v + 1 takes (a plain barrier after the LDS
      // writes: __syncthreads' release fence would also wait for loads in flight)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (v + 1 < t_end) issue_kv(v + 1);
      if (v + 2 < t_end) load_ids(v + 2);
      const TileRef tv = tref(v);
      const int cnt = tv.k1 - tv.k0;
      if (cnt < BN) {
        // rows past the tile's last key read slot 0: zero them (their scores are masked;
        // zeros keep P.V finite)
        for (int i = tid; i < (BN - cnt) * CH; i += 64 * NW) {
          const int off = t * TB + (cnt + i / CH) * RB + (i % CH) * 16;
          *reinterpret_cast<u32x4*>(kv + off) = u32x4{0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(kv + ST * TB + off) = u32x4{0u, 0u, 0u, 0u};
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
      for (int sub = wkey; sub < 2; sub += NKG) half_step(kv + t * TB, kv + (ST + t) * TB, tv, sub);
    }
    __syncthreads();  // the epilogue reuses the tile area
    return;
  }
  for (int tb = t_begin; tb < t_end; tb += ST) {
    const int nt = min(ST, t_end - tb);
    if constexpr (kRuns) {
      tr0 = tile_ref(tb);
      tr1 = tile_ref(min(tb + 1, t_end - 1));
      if constexpr (ST == 4) {
        tr2 = tile_ref(min(tb + 2, t_end - 1));
        tr3 = tile_ref(min(tb + 3, t_end - 1));
      } else {
        tr2 = tr3 = tr1;
      }
    }
    auto tile = [&](int t) {
      if constexpr (kRuns) {
        return tile_of(t);
      } else {
        TileRef r;
        r.k0 = (tb + t) * BN;
        r.k1 = L;
        r.row = row0;
        r.ra = 0;
        r.rb = 64;
        return r;
      }
    };
    issue(nt, tile);
    // each wave issued LPT = 2 * NI / NW loads per tile, in tile order, and they retire in
    // order; the round is computed in two parts of ST / 2 tiles, the second part's loads
    // may still fly during the first
    constexpr int PT = ST / 2, LPT = 2 * NI / NW;
    static_assert(ST % 2 == 0 && PT * LPT <= 15, "vmcnt immediates below (bits [3:0])");
    for (int part = 0; part < 2; ++part) {
      const int t0 = part * PT, t1 = min(nt, t0 + PT);  // tiles of this part
      if (t0 >= nt) break;
      const int fly = part == 0 ? (nt - t1) * LPT : 0;  // loads of later tiles that may fly
      if (fly == 8) __builtin_amdgcn_s_waitcnt(0x0F78);       // vmcnt(8)
      else if (fly == 4) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
      else __builtin_amdgcn_s_waitcnt(0);
      // a plain barrier: __syncthreads' release fence would wait for every load in flight
      asm volatile("s_barrier" ::: "memory");
      // rows past a tile's last key read slot 0: zero them (their scores are masked; zeros
      // keep P.V finite)
      bool zeroed = false;
      for (int t = t0; t < t1; ++t) {
        const TileRef tz = tile(t);
        const int cnt = tz.k1 - tz.k0;
        if (cnt < BN) {
          for (int i = tid; i < (BN - cnt) * CH; i += 64 * NW) {
            const int off = t * TB + (cnt + i / CH) * RB + (i % CH) * 16;
            *reinterpret_cast<u32x4*>(kv + off) = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(kv + ST * TB + off) = u32x4{0u, 0u, 0u, 0u};
          }
          zeroed = true;
        }
      }
      if (zeroed) __syncthreads();
      // 32-key halves 2 t0 .. 2 t1 - 1 of the round, round-robin over the key groups
      for (int j = 2 * t0 + wkey; j < 2 * t1; j += NKG) {
        const int t = j >> 1;
        half_step(kv + t * TB, kv + (ST + t) * TB, tile(t), j & 1);
      }
    }
    __syncthreads();  // the next round overwrites the tiles
  }
  };
  if (br.tiles > 0) tile_loop(std::true_type{});
  else tile_loop(std::false_type{});

  // the carried append (see above): this workgroup's first token from registers, then the
  // rest
  auto append_token = [&](int i, bool from_regs) {
    const int64_t slot = ap.slot[i];
    const u32x4* kn = reinterpret_cast<const u32x4*>(ap.k_new) + (int64_t)i * ap_cpr;
    const u32x4* vn = reinterpret_cast<const u32x4*>(ap.v_new) + (int64_t)i * ap_cpr;
    u32x4* kp = reinterpret_cast<u32x4*>(const_cast<void*>(a.k_pool)) + slot * ap_cpr;
    u32x4* vp = reinterpret_cast<u32x4*>(const_cast<void*>(a.v_pool)) + slot * ap_cpr;
    int64_t c0 = tid;
    if (from_regs) {
#pragma unroll
      for (int j = 0; j < kApR; ++j) {
        const int64_t c = tid + (int64_t)j * 64 * NW;
        if (c < ap_cpr) {
          kp[c] = ap_k[j];
          vp[c] = ap_v[j];
        }
      }
      c0 = tid + (int64_t)kApR * 64 * NW;
    }
    for (int64_t c = c0; c < ap_cpr; c += 64 * NW) {
      kp[c] = kn[c];
      vp[c] = vn[c];
    }
    if (tid == 0) {
      const int64_t row = a.req_pool_idx[i];
      const int32_t len = ap.len[i];
      ap.seq_len_dev[i] = len;
      if (row < 0 || row >= a.rtt_rows) flag_error(RAX_DEVERR_ROW);
      else const_cast<int32_t*>(a.rtt)[row * a.rtt_stride + len - 1] = (int32_t)slot;
    }
  };
  if (ap_mine) {
    append_token(blockIdx.x, true);
    for (int i = blockIdx.x + n_items; i < ap.n; i += n_items) append_token(i, false);
  }

  // The key groups combine their states over LDS, the work split by dims: slice dt (32
  // dims) belongs to group dt % NKG. Every wave hands the owners of the other slices its
  // parts of them and its (m, l); then each wave merges its own slices from all groups and
  // writes them. (Merging everything in one wave per row tile made that wave read every
  // other state and write every dim alone.)
  constexpr int NDT = D / 32;
  static_assert(NDT % NKG == 0, "whole 32-dim slices per key group");
  constexpr int SPG = NDT / NKG;                // slices per group
  constexpr int NX = 2 * NDT * (NKG - 1) * 16;  // floats per lane handed over
  static_assert((NX + 2 * NKG * 2) * 64 * sizeof(float) <= sizeof(kv), "key-split exchange area");
  float* xs = reinterpret_cast<float*>(kv);       // [wrow][dt][group other than dt's owner][16][64]
  float* xml = xs + NX * 64;                      // [wrow][group][m, l][64]
  auto xacc = [&](int row_tile, int dt, int grp, int r) -> float& {
    const int own = dt % NKG;
    const int g3 = grp < own ? grp : grp - 1;
    return xs[(((row_tile * NDT + dt) * (NKG - 1) + g3) * 16 + r) * 64 + lane];
  };
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    if (dt % NKG == wkey) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) xacc(wrow, dt, wkey, r) = acc[dt][r];
  }
  xml[((wrow * NKG + wkey) * 2 + 0) * 64 + lane] = m_run;
  xml[((wrow * NKG + wkey) * 2 + 1) * 64 + lane] = l_run;
  __syncthreads();
  float mk[NKG], ak[NKG];
  float m = kNegInf;
#pragma unroll
  for (int kg = 0; kg < NKG; ++kg) {
    mk[kg] = xml[((wrow * NKG + kg) * 2 + 0) * 64 + lane];
    m = fmaxf(m, mk[kg]);
  }
  float l = 0.f;
#pragma unroll
  for (int kg = 0; kg < NKG; ++kg) {
    ak[kg] = m == kNegInf || mk[kg] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mk[kg] - m);
    l += xml[((wrow * NKG + kg) * 2 + 1) * 64 + lane] * ak[kg];
  }
  // slices dt = wkey + sp * NKG: group kg's part is this wave's registers for kg == wkey,
  // else LDS
  f32x16 o[SPG];
#pragma unroll
  for (int sp = 0; sp < SPG; ++sp) {
    o[sp] = f32x16{};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if (dt != wkey + sp * NKG) continue;
#pragma unroll
      for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[sp][r] += (kg == wkey ? acc[dt][r] : xacc(wrow, dt, kg, r)) * ak[kg];
    }
  }
  if (!row_ok) return;
  // partials go out as non-temporal stores: the next kernel reads them from memory
  // anyway, and dirty L2 lines left here are written back at the kernel boundary, which
  // measured 0.5-0.8 µs longer per decode call. (Non-temporal stores of O in extend or
  // of the appended rows measured slower.)
  if (l > 0.f) {
    float* wacc = a.ws + ((int64_t)item * BM + R) * D;
#pragma unroll
    for (int sp = 0; sp < SPG; ++sp)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = (wkey + sp * NKG) * 32 + 8 * rg + 4 * half;
        __builtin_nontemporal_store(f32x4{o[sp][rg * 4 + 0], o[sp][rg * 4 + 1], o[sp][rg * 4 + 2], o[sp][rg * 4 + 3]},
                                    reinterpret_cast<f32x4*>(wacc + d0));
      }
  }
  if (wkey == 0 && half == 0) {  // (m, l) of the row; l == 0 means "no keys here"
    float* wml = a.ws + (int64_t)n_items * BM * D + ((int64_t)item * BM + R) * 2;
    __builtin_nontemporal_store(m, wml);
    __builtin_nontemporal_store(l, wml + 1);
  }
}

// End of an own-part workgroup with query-head groups (bf16, D = 128): wave w holds dims
// [32w, 32w + 32) of the chunk's output for query head l % 16 (lane l: dims 32w + 16j +
// 4*(l/16) + {0..3} in o[j]) with the running (m, l), the same in every wave. Either the
// request's only own chunk is merged in place with the shared part's split partials and
// O written, or the chunk's partial goes to the workspace in own_kernel's layout.
// The shared part's split partials of one row of an own-chunk workgroup (this lane's dims
// in own_chunk_epilogue's layout), when there are at most kShPre splits and the host's
// list gives the request one chunk: loaded at the workgroup's start, next to the block
// metadata, so that the in-place merge at its end waits for no load. (They are written
// by the launch before.)
constexpr int kShPre = 2;
struct ShPre {
  float2 ml[kShPre];
  f32x4 acc[kShPre][2];
};
template <int D>
__device__ __forceinline__ void sh_partials_load(const AttnArgs& a, int t, int h, int r16, int wq, int g4, ShPre& p) {
  const int Grow = t * a.g + r16;
  const int rbr = Grow / a.bm, Rr = Grow - rbr * a.bm;
  const int64_t n_items = (int64_t)a.h_kv * a.n_rb * a.nsplit;
  const int64_t item0 = ((int64_t)h * a.n_rb + rbr) * a.nsplit;
  const float* sh_ml = a.ws + n_items * a.bm * (int64_t)D + (item0 * a.bm + Rr) * 2;
  const float* sh_acc = a.ws + (item0 * a.bm + Rr) * (int64_t)D + wq * 32 + 4 * g4;
#pragma unroll
  for (int sp = 0; sp < kShPre; ++sp) {
    if (sp < a.nsplit) {
      p.ml[sp] = *reinterpret_cast<const float2*>(sh_ml + (int64_t)sp * a.bm * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) p.acc[sp][j] = *reinterpret_cast<const f32x4*>(sh_acc + (int64_t)sp * a.bm * D + 16 * j);
    } else {
      p.ml[sp] = make_float2(0.f, 0.f);  // l = 0: weight 0
    }
  }
}

template <int D>
__device__ __forceinline__ void own_chunk_epilogue(const AttnArgs& a, const f32x4 (&o)[2], float m, float l,
                                                   int wq, int lane, bool row_ok, int t, int h, int rh, int c,
                                                   int n_act, int n_rh, bool pre_on, const ShPre& pre) {
  static_assert(D == 128, "four 32-dim quarters, one per wave");
  const int G = a.g;
  const int r16 = lane & 15, g4 = lane >> 4;
  if (!row_ok) return;
  if (n_act == 1) {
    // the request's only own chunk: merge here with the shared part's split partials of
    // this row (written by the previous kernel) by log-sum-exp and write this wave's
    // dims of O; merge_kernel skips such rows. A split that saw no key (l == 0) may hold
    // stale data, hence the selects.
    const int Grow = t * G + r16;
    const int rbr = Grow / a.bm, Rr = Grow - rbr * a.bm;
    const int nsplit = a.nsplit;
    const int64_t n_items = (int64_t)a.h_kv * a.n_rb * nsplit;
    const int64_t item0 = ((int64_t)h * a.n_rb + rbr) * nsplit;
    const float* sh_ml = a.ws + n_items * a.bm * (int64_t)D + (item0 * a.bm + Rr) * 2;
    const float* sh_acc = a.ws + (item0 * a.bm + Rr) * (int64_t)D;
    float M = l > 0.f ? m : kNegInf;
    f32x4 fin[2];
    float lsum;
    if (pre_on) {  // the splits' partials are in registers already
#pragma unroll
      for (int sp = 0; sp < kShPre; ++sp)
        if (pre.ml[sp].y > 0.f) M = fmaxf(M, pre.ml[sp].x);
      const float Mu = M == kNegInf ? 0.f : M;
      const float w_own = l > 0.f ? __builtin_amdgcn_exp2f(m - Mu) : 0.f;
      lsum = w_own * l;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) fin[j][e] = w_own != 0.f ? w_own * o[j][e] : 0.f;
#pragma unroll
      for (int sp = 0; sp < kShPre; ++sp) {
        const float2 ml = pre.ml[sp];
        const float w = ml.y > 0.f ? __builtin_amdgcn_exp2f(ml.x - Mu) : 0.f;
        lsum += w * ml.y;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) fin[j][e] += w != 0.f ? w * pre.acc[sp][j][e] : 0.f;
      }
    } else {
    for (int sp = 0; sp < nsplit; ++sp) {
      const float2 ml = *reinterpret_cast<const float2*>(sh_ml + (int64_t)sp * a.bm * 2);
      if (ml.y > 0.f) M = fmaxf(M, ml.x);
    }
    const float Mu = M == kNegInf ? 0.f : M;
    const float w_own = l > 0.f ? __builtin_amdgcn_exp2f(m - Mu) : 0.f;
    lsum = w_own * l;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) fin[j][e] = w_own != 0.f ? w_own * o[j][e] : 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float2 ml = *reinterpret_cast<const float2*>(sh_ml + (int64_t)sp * a.bm * 2);
      const float w = ml.y > 0.f ? __builtin_amdgcn_exp2f(ml.x - Mu) : 0.f;
      lsum += w * ml.y;
      const float* pa = sh_acc + (int64_t)sp * a.bm * D;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(pa + wq * 32 + 16 * j + 4 * g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) fin[j][e] += w != 0.f ? w * x[e] : 0.f;
      }
    }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int64_t obase = ((int64_t)t * a.h_q + h * G + r16) * D;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int d0 = wq * 32 + 16 * j + 4 * g4;
      if (a.o_bf16)
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + obase + d0) =
            bf16x4{(__bf16)(fin[j][0] * inv), (__bf16)(fin[j][1] * inv), (__bf16)(fin[j][2] * inv),
                   (__bf16)(fin[j][3] * inv)};
      else
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + obase + d0) =
            make_float4(fin[j][0] * inv, fin[j][1] * inv, fin[j][2] * inv, fin[j][3] * inv);
    }
    return;
  }
  // partial of (request t, KV head h, chunk c), query head r16, in own_kernel's layout.
  // With own_fold another workgroup of the same launch (own_rows_merge), possibly on
  // another XCD, reads it: stored coherent at device scope (through this XCD's L2), one
  // dword at a time. Otherwise for the merge kernel: 16-byte non-temporal stores (dword
  // device-scope stores here took multi-turn decode 218.5 -> 224 us per call).
  const int64_t item = (int64_t)rh * a.n_chunk + c;
  float* wacc = a.ws_own + (item * G + r16) * D;
  float* wml = a.ws_own + (int64_t)n_rh * a.n_chunk * G * D + (item * G + r16) * 2;
  if (a.own_fold) {
    if (l > 0.f) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) store_dev(wacc + wq * 32 + 16 * j + 4 * g4 + e, o[j][e]);
    }
    if (wq == 0 && g4 == 0) {
      store_dev(wml, m);
      store_dev(wml + 1, l);
    }
    return;
  }
  if (l > 0.f) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_nontemporal_store(o[j], reinterpret_cast<f32x4*>(wacc + wq * 32 + 16 * j + 4 * g4));
  }
  if (wq == 0 && g4 == 0) {
    __builtin_nontemporal_store(m, wml);
    __builtin_nontemporal_store(l, wml + 1);
  }
}

// 16x16x32 MFMA fragments of a stage (32 keys x 128 dims of K, and of V, swizzled as above).
// A operand of S^T = K Q^T: key 16*kh + l%16, dims 32*ks + 8*(l/16) .. +8.
__device__ __forceinline__ bf16x8 k_frag16(const char* kt, int kh, int ks, int lane) {
  const int key = 16 * kh + (lane & 15);
  return *reinterpret_cast<const bf16x8*>(kt + key * 256 + (((4 * ks + (lane >> 4)) ^ swz_k(key)) * 16));
}
// A operand of O^T = V^T P^T for dims 16*dt .. +16: lane l holds dim 16*dt + l%16 of keys
// 4*(l/16) + {0..3} and 16 + 4*(l/16) + {0..3}, the key order of the P fragment (the two
// 16-key score tiles of a lane, one after the other). Each transposing read takes 4 keys x
// 16 dims over 16 lanes (lane i: key i/4, dims 4*(i%4) .. +4) and hands lane i dim i.
__device__ __forceinline__ bf16x8 vt_frag16(const char* vt, int dt, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int i = lane & 15;
  const int d0 = dt * 16 + 4 * (i & 3);
  const int key = 4 * (lane >> 4) + (i >> 2);
  const char* p0 = vt + key * 256 + (((d0 >> 3) ^ swz_v(key)) * 16) + (d0 & 7) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0 + 16 * 256));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One 32-key stage of the own part on 16x16x32 MFMA (K at kt, V at vt, swizzled as
// above): scores of this lane's query head r16 (row_ok: r16 < g) against the stage's first
// cnt keys, the online softmax update of (m_run, l_run) shared by every wave, and this
// wave's quarter of the output dims (acc[j]: dims 32*wave + 16*j + 4*(l/16) + e).
__device__ __forceinline__ void own_stage16(const char* kt, const char* vt, const bf16x8 (&qf)[4], int cnt,
                                            bool row_ok, int wave, int lane, float scale_log2, float& m_run,
                                            float& l_run, f32x4 (&acc)[2]) {
  const int g4 = lane >> 4;
  f32x4 sc[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    sc[kh] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      sc[kh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag16(kt, kh, ks, lane), qf[ks], sc[kh], 0, 0, 0);
  }
  // sc[kh][e] is the score of key 16*kh + 4*g4 + e of the stage for query head r16
  float mx = kNegInf;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = 16 * kh + 4 * g4 + e;
      const float v = row_ok && key < cnt ? sc[kh][e] : kNegInf;
      sc[kh][e] = v;
      mx = fmaxf(mx, v);
    }
  mx = max_xor16(max_xor32(mx)) * scale_log2;
  if (__any(mx > m_run + kLazy)) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[j] *= alpha;
    m_run = m_new;
  }
  const float neg_m = m_run == kNegInf ? 0.f : -m_run;
  float psum = 0.f;
  bf16x8 pb;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kh][e], scale_log2, neg_m));
      psum += pv;
      pb[kh * 4 + e] = (__bf16)pv;
    }
  psum = sum_xor16(sum_xor32(psum));
  l_run += psum;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt_frag16(vt, 2 * wave + j, lane), pb, acc[j], 0, 0, 0);
}

// Final merge of (request t, KV head h) when its own keys took several chunks: each row
// (query head r16 < g of the group) combines the shared part's split partials of its row
// block and the request's n_act own-chunk partials by log-sum-exp, and this wave writes
// its quarter of the row's dims of O (own_chunk_epilogue's lane layout). Partials with
// l = 0 saw no key and get weight 0 (their accumulators may be stale, hence the selects).
template <int D>
__device__ __forceinline__ void own_rows_merge(const AttnArgs& a, int wq, int lane, int t, int h, int rh, int n_act,
                                               int n_rh) {
  const int G = a.g;
  const int r16 = lane & 15, g4 = lane >> 4;
  if (r16 >= G) return;
  const int Grow = t * G + r16;
  const int rbr = Grow / a.bm, Rr = Grow - rbr * a.bm;
  const int nsplit = a.nsplit;
  const int64_t n_items = (int64_t)a.h_kv * a.n_rb * nsplit;
  const int64_t item0 = ((int64_t)h * a.n_rb + rbr) * nsplit;
  const float* sh_ml = a.ws + n_items * a.bm * (int64_t)D + (item0 * a.bm + Rr) * 2;
  const float* sh_acc = a.ws + (item0 * a.bm + Rr) * (int64_t)D;
  const int64_t own0 = (int64_t)rh * a.n_chunk;  // chunk c: item own0 + c
  const float* ow_ml = a.ws_own + (int64_t)n_rh * a.n_chunk * G * D + (own0 * G + r16) * 2;
  const float* ow_acc = a.ws_own + (own0 * G + r16) * (int64_t)D;
  // Partial s < nsplit: split s of the shared part (the previous launch's), else own chunk
  // s - nsplit (this launch's); all read with device-coherent loads, U partials per round
  // trip (indices past the last repeat it and are dropped), combined by an online
  // log-sum-exp (running maximum M, rescaled sums).
  constexpr int U = 4;
  const int n_all = nsplit + n_act;
  float M = kNegInf, lsum = 0.f;
  f32x4 fin[2] = {f32x4{}, f32x4{}};
  for (int s0 = 0; s0 < n_all; s0 += U) {
    float mv[U], lv[U];
    f32x4 x[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(s0 + u, n_all - 1);
      const bool sh = s < nsplit;
      const float* pml = sh ? sh_ml + (int64_t)s * a.bm * 2 : ow_ml + (int64_t)(s - nsplit) * G * 2;
      const float* pa = (sh ? sh_acc + (int64_t)s * a.bm * D : ow_acc + (int64_t)(s - nsplit) * G * D) + wq * 32 + 4 * g4;
      mv[u] = load_dev(pml);
      lv[u] = load_dev(pml + 1);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[u][j][e] = load_dev(pa + 16 * j + e);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u >= n_all || !(lv[u] > 0.f)) continue;  // no keys: weight 0 (stale accumulators)
      const float m_new = fmaxf(M, mv[u]);
      const float keep = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - m_new);
      const float w = __builtin_amdgcn_exp2f(mv[u] - m_new);
      lsum = lsum * keep + w * lv[u];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) fin[j][e] = fin[j][e] * keep + w * x[u][j][e];
      M = m_new;
    }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int64_t obase = ((int64_t)t * a.h_q + h * G + r16) * D;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int d0 = wq * 32 + 16 * j + 4 * g4;
    if (a.o_bf16)
      *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + obase + d0) =
          bf16x4{(__bf16)(fin[j][0] * inv), (__bf16)(fin[j][1] * inv), (__bf16)(fin[j][2] * inv),
                 (__bf16)(fin[j][3] * inv)};
    else
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + obase + d0) =
          make_float4(fin[j][0] * inv, fin[j][1] * inv, fin[j][2] * inv, fin[j][3] * inv);
  }
}

// Own part of split decode with query-head groups (bf16, D = 128), as one continuous
// stream per workgroup, on MFMA: the VALU own part (own_chunk) scores 32 / g keys per
// batch through chains of cross-lane reductions, which for g > 1 bound it rather than
// memory (0.56 ms per GQA 64/8 self-consistency call for 0.59 GB). A workgroup takes one
// own chunk of request t for HP adjacent KV heads (below), at most kStreamCap keys; four
// waves per head. Its slot ids go to LDS
// first (one round of loads); then the chunk's keys stream through a ring of S stages of
// 32 keys (8 KB of K and 8 KB of V per head) filled straight from global memory: while stage i
// is computed, the loads of the next S - 1 stages are in flight. One barrier per stage.
// A stage is S^T = K Q^T and O^T = V^T P^T on 16x16x32 MFMA, the g <= 16 query heads as
// the columns of one 16-wide tile (columns past g masked). Every wave computes every
// stage's scores and softmax (the same instructions on the same data, so the same values
// in every wave) and O^T for its own quarter of the dims: the stage's critical path is
// one wave's QK^T, softmax and a quarter of PV, with no end-of-chunk exchange between
// waves. (Per-workgroup timestamps of the form where one wave computed a whole stage
// while the others waited at the barrier: ~0.8 us per stage with the GPU nearly idle,
// against ~0.37 us for the loads alone.) Keys past the chunk in its last stage read the
// chunk's first slot (a key it attends, so finite) and are masked.
constexpr int kStreamCap = 2048;  // most keys per own chunk of own_stream_kernel (slot ids in LDS)
constexpr int kStreamTK = 32;     // keys per stage
// Two stages (one in flight while one is computed). Measured with one head per workgroup
// (36 KB of LDS with the slot ids, four workgroups per CU), faster than three stages
// (three per CU) or four (two per CU): multi-turn decode 221.6, 223.0 and 224.3 us per
// call; six stages (one per CU) 262.7 us. With more workgroups per CU, one's start
// (metadata, slot ids, first stage: ~5 us) runs while the others stream. With two heads
// per workgroup and a 2048-key slot-id list: 72 KB, two workgroups (16 waves) per CU.
constexpr int kStreamStages = 2;

// Heads per workgroup: HP adjacent KV heads of the same (request, chunk), four waves each,
// one slot-id list. A key's rows of adjacent heads are adjacent 256-byte pieces of its
// slot's K (and V) row, and the waves of the heads load them in the same stage: a gather
// probe (random slots, non-temporal 16-byte loads) read 512 contiguous bytes per slot at
// 6.7 TB/s, against 6.3-6.4 TB/s for one 256-byte piece per slot; 1 KB or 2 KB pieces were
// no faster than 512 bytes.
constexpr int kStreamHeads = 2;
// Most (chunk, KV head) items of requests with several own chunks for which the own part
// merges such requests itself
constexpr int64_t kOwnFoldMaxItems = 256;

template <int D, int S, int HP>
__global__ void __launch_bounds__(256 * HP) own_stream_kernel(AttnArgs a, OwnOrder ord) {
  static_assert(D == 128, "the swizzle assumes 16 chunks per row");
  static_assert(S >= 2 && 2 * (S - 2) < 64, "stages");
  static_assert(HP >= 1 && HP <= 2, "heads per workgroup");
  constexpr int NW = 4;                  // waves per head
  constexpr int TK = kStreamTK;
  constexpr int RB = D * 2;              // bytes per row
  constexpr int TB = TK * RB;            // bytes of K (or V) per stage and head
  constexpr int RPI = 1024 / RB;         // rows per 1 KB global-to-LDS instruction
  constexpr int NI = TK / RPI;           // instructions per K (or V) stage and head
  constexpr int IPW = NI / NW;           // of them per wave
  constexpr int NKS = D / 32;
  constexpr int KV_BYTES = S * HP * 2 * TB;
  static_assert(NI % NW == 0 && (HP == 1 || IPW % HP == 0), "loads per wave");
  static_assert(D == 32 * NW, "a 32-dim quarter per wave");
  __shared__ __align__(16) char kv[KV_BYTES];  // per stage: K then V of head 0, then of head 1, ...
  __shared__ int32_t slot[kStreamCap];
  const uint32_t kv_lds = lds_addr(kv);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = wave / NW, wq = wave - hh * NW;  // this wave's head of the group, dim quarter
  const int r16 = lane & 15, g4 = lane >> 4;
  const int G = a.g;
  const int n_rh = a.batch * a.h_kv;
  const int n_hg = a.h_kv / HP;  // head groups per (request, chunk)
  // Workgroup order. The hardware hands out workgroups in id order, round-robin over the
  // XCDs and their shader engines, and waits for room on the next one's engine: work items
  // that exit at once must come in contiguous runs, not at a fixed stride (interleaving
  // one live item with three exiting ones put every live one on one engine in four and
  // measured 2x slower). With the host's work list (requests by descending own keys,
  // each request's chunks and a chunk's head groups together): exactly the live items,
  // the longest requests first. Without it: rows of batch x n_hg ids, one chunk index per
  // row, chunk 0 first, in batch order; ids past a request's chunks exit at once.
  const bool ordered = ord.n == a.batch;
  int c, hg, t, n_host = 0;
  if (ordered) {
    // item blockIdx / n_hg of the list, head group blockIdx % n_hg. The list's cumulative
    // counts rise strictly, so the item's entry is the number of entries that start at or
    // before it, minus one: lane l reads entries 4l .. 4l + 3 of the counts and of the
    // requests in one round of loads and ballots count them. (A binary search made eight
    // dependent loads from the argument memory at every workgroup's start.)
    static_assert(kAppendMax == 256, "four list entries per lane");
    const int item = (int)(blockIdx.x / (unsigned)n_hg);
    hg = (int)(blockIdx.x - (unsigned)item * n_hg);
    int cv[4], rv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cv[k] = ord.cum[4 * lane + k];
      rv[k] = ord.req[4 * lane + k];
    }
    const int cum_end = ord.cum[kAppendMax];
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) cnt += __popcll(__ballot(4 * lane + k < ord.n && cv[k] <= item));
    const int lo = cnt - 1;  // cum[0] = 0 <= item
    auto pick = [](const int (&v)[4], int k) { return k == 0 ? v[0] : k == 1 ? v[1] : k == 2 ? v[2] : v[3]; };
    const int c_lo = __builtin_amdgcn_readlane(pick(cv, lo & 3), lo >> 2);
    const int c_hi =
        lo + 1 < kAppendMax ? __builtin_amdgcn_readlane(pick(cv, (lo + 1) & 3), (lo + 1) >> 2) : cum_end;
    t = __builtin_amdgcn_readlane(pick(rv, lo & 3), lo >> 2);
    c = item - c_lo;
    n_host = c_hi - c_lo;
  } else {
    const int n_row = a.batch * n_hg;
    const int row_i = blockIdx.x / n_row;
    const int in_row = blockIdx.x - row_i * n_row;
    c = row_i;
    t = in_row / n_hg;
    hg = in_row - t * n_hg;
  }
  const int h = hg * HP + hh;  // this wave's KV head
  const int rh = t * a.h_kv + h;

  const int rb0 = t * G / a.bm;
  const BlockMeta meta = block_meta_load(a, rb0, lane);
  const bool row_ok = r16 < G;
  bf16x8 qf[NKS];  // B operand: query head r16 of the group of KV head h, dims 32*ks + 8*g4 .. +8
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + ((int64_t)t * a.h_q + h * G + (row_ok ? r16 : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + ks * 32 + g4 * 8);
      qf[ks] = row_ok ? v : bf16x8{};
    }
  }
  ShPre pre;
  const bool pre_on = a.nsplit <= kShPre && ordered && n_host == 1;  // merges in place (the host's count)
  if (pre_on) sh_partials_load<D>(a, t, h, row_ok ? r16 : 0, wq, g4, pre);
  const int rl = t - rb0 * a.bm / G;
  const int L = row_shared_len(a, meta, lane, rl);
  const int row_t = __builtin_amdgcn_readlane(meta.row, rl);
  const int end = __builtin_amdgcn_readlane(meta.len, rl);
  int first, per;
  const int n_act = own_chunks(a, row_t, end, L, first, per);
  // the host's item count bounds the kernel's (else chunks past it would be missed)
  if (ordered && c == n_host - 1 && n_act > n_host && tid == 0) flag_error(RAX_DEVERR_ROW);
  if (c >= n_act) return;  // the same for the whole workgroup
  const int start = first + c * per;
  int stop = min(start + per, end);
  if (stop - start > kStreamCap) {  // the layout bounds every chunk; never taken
    flag_error(RAX_DEVERR_ROW);
    stop = start + kStreamCap;
  }
  const int n = stop - start;
  const int n_tiles = (n + TK - 1) / TK;
  const int64_t row_bytes = (int64_t)a.h_kv * RB;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (int64_t)hg * HP * RB;  // the group's first head
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (int64_t)hg * HP * RB;
  const int32_t* rtt_row = a.rtt + (int64_t)row_t * a.rtt_stride;  // row_t valid: n_act > 0

  // every slot id of the chunk into LDS in one round of loads (positions past the chunk
  // take the chunk's first slot)
  {
    constexpr int PER_T = kStreamCap / (64 * NW * HP);
    int raw[PER_T];
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const int i = tid + k * 64 * NW * HP;
      raw[k] = k * 64 * NW * HP < n ? rtt_row[start + (i < n ? i : 0)] : 0;  // (uniform: rounds past n skipped)
    }
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const int i = tid + k * 64 * NW * HP;
      int sv = raw[k];
      if (sv < 0 || sv >= a.num_slots) {
        if (i < n) flag_error(RAX_DEVERR_SLOT);
        sv = 0;
      }
      if (i < n_tiles * TK) slot[i] = sv;
    }
  }
  __syncthreads();

  // this wave's share of the K and V rows of stage j's keys into ring slot j % S: IPW of
  // the stage's NI x HP 1 KB pieces (NI groups of RPI keys, one head each) per K and V;
  // with a group of heads, one wave loads every head of its key group, one after another
  // (adjacent pieces of the same slot rows)
  auto issue = [&](int j) {
    const uint32_t kl = kv_lds + (j % S) * HP * 2 * TB;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      int q, hx;
      if constexpr (HP == 1) {
        q = wave + u * NW;
        hx = 0;
      } else {
        const int x = wave * IPW + u;
        q = x / HP;
        hx = x % HP;
      }
      const int r = q * RPI + (lane >> 4);
      const int64_t off = (int64_t)slot[j * TK + r] * row_bytes + hx * RB;
      // read once per call: non-temporal (multi-turn decode 300 -> 241 us per call)
      lds_load16_nt(kbase + off + (((lane & 15) ^ swz_k(r)) * 16), uni(kl + hx * 2 * TB + q * 1024));
      lds_load16_nt(vbase + off + (((lane & 15) ^ swz_v(r)) * 16), uni(kl + hx * 2 * TB + TB + q * 1024));
    }
  };

  f32x4 acc[2] = {f32x4{}, f32x4{}};  // this wave's dims 32*wq + 16*j + 4*g4 + e
  float m_run = kNegInf, l_run = 0.f;

  for (int j = 0; j < S - 1 && j < n_tiles; ++j) issue(j);
  for (int i = 0; i < n_tiles; ++i) {
    // this wave's loads of stage i are done when at most those of the stages issued after
    // it (up to S - 2, each 2 * IPW loads) are in flight; the barrier makes every wave's
    // loads of stage i visible and frees ring slot (i - 1) % S for stage i + S - 1
    if (i + S - 2 < n_tiles) wait_vmcnt<2 * IPW * (S - 2)>();
    else wait_vmcnt<0>();
    asm volatile("s_barrier" ::: "memory");
    if (i + S - 1 < n_tiles) issue(i + S - 1);
    const char* kt = kv + ((i % S) * HP + hh) * 2 * TB;
    own_stage16(kt, kt + TB, qf, min(TK, n - i * TK), row_ok, wq, lane, a.scale_log2, m_run, l_run, acc);
  }
  own_chunk_epilogue<D>(a, acc, m_run, l_run, wq, lane, row_ok, t, h, rh, c, n_act, n_rh, pre_on, pre);
  if (n_act > 1 && a.own_fold) {
    // the workgroup that finishes the last of the request's chunks (per KV head) merges
    // them. Its partial stores are device-coherent: once every wave has seen them
    // complete (vmcnt 0), the count that follows is ordered after them, and the last
    // workgroup's device-coherent loads see every chunk's partial. (Device-scope fences
    // instead, which write back and invalidate a whole L2, made the multi-turn decode
    // call 4x slower.)
    __shared__ int32_t last[HP];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (wq == 0 && lane == 0)
      last[hh] = __hip_atomic_fetch_add(a.own_cnt + rh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_act - 1;
    __syncthreads();
    if (last[hh]) own_rows_merge<D>(a, wq, lane, t, h, rh, n_act, n_rh);
  }
}

// ------------------------------------------------------------------ host side
struct Shape {
  int nw, rt, pd, ks;
  int bm() const { return 32 * (nw / ks) * rt; }
};

// Work shape per call. Extend (bf16, D = 128): 8 waves x one 32-row tile; at under 256
// VGPRs two such workgroups share a CU, so every SIMD has two waves and one wave's softmax
// runs under the other's MFMAs. (4 waves x two row tiles reads half the LDS fragments per
// flop but needs 350 VGPRs, one wave per SIMD, and measured 1.6x slower.) D = 64 has too
// few 16-byte chunks per key row for 512 loaders and keeps 4 x 2. Decode: 4 waves as two
// 32-row tiles x two 32-key halves of every tile (KS = 2), one tile of loads in flight:
// the same 64 rows per block as 2 waves x 1 tile, half the MFMA chain per wave and twice
// the waves per CU; the key halves combine their softmax states in LDS at the end.
// Every decode shape has 64 rows per block: the decode kernels read a block's requests
// with one lane each (block_meta_load), so a block may hold at most 64 requests.
static Shape pick_shape(bool decode, rax_dtype dt, int d) {
  if (decode) return {4, 1, 1, 2};
  if (dt != RAX_BF16) return {4, 1, 1, 1};
  return d == 128 ? Shape{8, 1, 1, 1} : Shape{4, 2, 1, 1};
}

static int choose_nsplit(int64_t blocks, int32_t max_kv_len) {
  // about one workgroup per CU (256 CUs): measured as fast as two per CU for the shared
  // prefix of decode, with half the split partials to write and merge
  int64_t want = (256 + blocks - 1) / blocks;
  const int64_t tiles = (int64_t)(max_kv_len + BN - 1) / BN;
  int64_t cap = tiles;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want > 32) want = 32;
  if (want < 1) want = 1;
  return (int)want;
}

// Key splits of an extend call: up to one workgroup per CU (the extend shape runs one per
// CU), never more, so the grid stays one round. A call of few long requests has few row
// blocks (a multi-turn turn of 500 new tokens over a 2000-token history: 8 blocks per KV
// head), so without splits most CUs would idle. Each split keeps at least 4 tiles of the
// longest key range; 0 = unknown length, no split.
constexpr int64_t kExtendWGs = 256;
static int32_t extend_nsplit(int64_t blocks, int32_t max_kv_len) {
  if (max_kv_len <= 0 || blocks <= 0) return 1;
  const int64_t tiles = ((int64_t)max_kv_len + BN - 1) / BN;
  int64_t want = kExtendWGs / blocks;
  want = std::min<int64_t>({want, tiles / 4, 32});
  return (int32_t)std::max<int64_t>(want, 1);
}

static size_t ws_bytes_for(int64_t items, int bm, int d) {
  return (size_t)items * bm * (size_t)(d + 2) * sizeof(float);
}

template <typename T, int D, bool kDecode, int NW, int RT, int PD, int KS>
static rax_status launch_one(AttnArgs& a, hipStream_t st) {
  const int64_t items = (int64_t)a.h_kv * a.n_rb * a.nsplit;
  hipLaunchKernelGGL((attn_kernel<T, D, kDecode, NW, RT, PD, KS>), dim3((unsigned)items), dim3(64 * NW), 0, st, a);
  return hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
}

template <int D>
static rax_status launch_merge(AttnArgs& a, hipStream_t st) {
  const int64_t rows = a.total_q * a.g;
  hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)((rows + 3) / 4), (unsigned)a.h_kv), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
}

constexpr int kOwnFusedMaxWaves = 8;
constexpr size_t kOwnFusedMaxLds = 48 * 1024;
static size_t own_fused_lds_bytes(int n_chunk, int g, int d) {
  return (size_t)n_chunk * g * (d + 2) * sizeof(float);
}

template <typename T, int D>
static rax_status launch_own(AttnArgs& a, hipStream_t st) {
  const int64_t own_items = (int64_t)a.batch * a.h_kv * a.n_chunk;
  const unsigned blocks = (unsigned)((own_items + 3) / 4);
  switch (a.g) {
    case 1: hipLaunchKernelGGL((own_kernel<T, D, 1>), dim3(blocks), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((own_kernel<T, D, 2>), dim3(blocks), dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((own_kernel<T, D, 4>), dim3(blocks), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((own_kernel<T, D, 8>), dim3(blocks), dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL((own_kernel<T, D, 16>), dim3(blocks), dim3(256), 0, st, a); break;
    default: return RAX_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
}

template <typename T, int D, bool kDecode>
static rax_status launch_attn(AttnArgs& a, Shape s, hipStream_t st, const AppendJob* ap) {
  rax_status rc = RAX_EINVAL;
  if constexpr (sizeof(T) == 2 && !kDecode) {
    if constexpr (D == 128) {
      if (s.nw == 8 && s.rt == 1 && s.pd == 1 && s.ks == 1) {
        const int64_t items = (int64_t)a.h_kv * a.n_rb * a.nsplit;
        hipLaunchKernelGGL(extend_kernel, dim3((unsigned)items), dim3(512), 0, st, a);
        rc = hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
      }
    } else {
      if (s.nw == 4 && s.rt == 2 && s.pd == 1 && s.ks == 1) rc = launch_one<T, D, kDecode, 4, 2, 1, 1>(a, st);
    }
  }
  if constexpr (sizeof(T) == 2 && kDecode) {
    if constexpr (D == 128) {
      if (a.shared_only) {  // shared part of split decode
        const int64_t items = (int64_t)a.h_kv * a.n_rb * a.nsplit;
        AppendJob none;
        none.n = 0;
        if (a.sh_small)
          hipLaunchKernelGGL((shared_kernel<D, 2, 2>), dim3((unsigned)items), dim3(256), 0, st, a.req_pool_idx,
                             a.kv_len, a.shared_len, a.q, (int32_t)items, a.nsplit, a.n_rb, a.g, a.batch, a.h_q, a,
                             ap ? *ap : none);
        else
          hipLaunchKernelGGL((shared_kernel<D, 4, kShTiles>), dim3((unsigned)items), dim3(512), 0, st,
                             a.req_pool_idx, a.kv_len, a.shared_len, a.q, (int32_t)items, a.nsplit, a.n_rb, a.g,
                             a.batch, a.h_q, a, ap ? *ap : none);
        return hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
      }
    }
  }
  if constexpr (kDecode) {
    if (s.nw == 4 && s.rt == 1 && s.pd == 1 && s.ks == 2) rc = launch_one<T, D, kDecode, 4, 1, 1, 2>(a, st);
  }
  if constexpr (!kDecode) {
    if (rc == RAX_EINVAL && s.nw == 4 && s.rt == 1 && s.pd == 1 && s.ks == 1)
      rc = launch_one<T, D, kDecode, 4, 1, 1, 1>(a, st);
  }
  return rc;
}

template <typename T, int D, bool kDecode>
static rax_status launch_shape(AttnArgs& a, Shape s, hipStream_t st, const AppendJob* ap, const OwnOrder* ord) {
  rax_status rc = launch_attn<T, D, kDecode>(a, s, st, ap);
  if (rc != RAX_OK) return rc;
  if constexpr (kDecode) {
    if (a.shared_only && a.own_fused == 1) {
      // one workgroup per (request, KV head), n_chunk waves; writes O (no merge kernel)
      if (a.nsplit > 255 || a.n_rb >= (1 << 23)) return RAX_EINVAL;  // packed in one argument
      const unsigned blocks = (unsigned)((int64_t)a.batch * a.h_kv);
      const dim3 block((unsigned)(64 * a.n_chunk));
      const size_t lds = own_fused_lds_bytes(a.n_chunk, a.g, D);
#define OWN_ARGS a.q, a.ws, a.req_pool_idx, a.kv_len, a.shared_len, a.h_kv, a.bm, a.batch, a.nsplit | a.n_rb << 8, a
      switch (a.g) {
        case 1: hipLaunchKernelGGL((own_merge_kernel<T, D, 1>), dim3(blocks), block, lds, st, OWN_ARGS); break;
        case 2: hipLaunchKernelGGL((own_merge_kernel<T, D, 2>), dim3(blocks), block, lds, st, OWN_ARGS); break;
        case 4: hipLaunchKernelGGL((own_merge_kernel<T, D, 4>), dim3(blocks), block, lds, st, OWN_ARGS); break;
        case 8: hipLaunchKernelGGL((own_merge_kernel<T, D, 8>), dim3(blocks), block, lds, st, OWN_ARGS); break;
        case 16: hipLaunchKernelGGL((own_merge_kernel<T, D, 16>), dim3(blocks), block, lds, st, OWN_ARGS); break;
        default: return RAX_EINVAL;
      }
#undef OWN_ARGS
      return hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
    }
    if (a.shared_only && a.own_fused == 0) {
      // more chunks per (request, KV head) than one workgroup takes: partials, then merge
      rc = launch_own<T, D>(a, st);
      if (rc != RAX_OK) return rc;
    }
    if (a.shared_only && a.own_fused == 2) {
      if constexpr (sizeof(T) == 2 && D == 128) {
        static const OwnOrder none{};
        const bool ordered = ord && ord->n == a.batch;
        const int64_t items = ordered ? (int64_t)ord->cum[ord->n] * a.h_kv : (int64_t)a.batch * a.h_kv * a.n_chunk;
        if (items > INT32_MAX || a.g > 16) return RAX_EINVAL;  // one 16-wide tile of query heads
        // a group of kStreamHeads KV heads per workgroup where they divide h_kv
        if (items > 0 && a.h_kv % kStreamHeads == 0)
          hipLaunchKernelGGL((own_stream_kernel<D, kStreamStages, kStreamHeads>), dim3((unsigned)(items / kStreamHeads)),
                             dim3(256 * kStreamHeads), 0, st, a, ordered ? *ord : none);
        else if (items > 0)
          hipLaunchKernelGGL((own_stream_kernel<D, kStreamStages, 1>), dim3((unsigned)items), dim3(256), 0, st, a,
                             ordered ? *ord : none);
        rc = hipGetLastError() == hipSuccess ? RAX_OK : RAX_EDEVICE;
        if (rc != RAX_OK) return rc;
      } else {
        return RAX_EINVAL;
      }
    }
  }
  // split decode with the own part on own_stream_kernel merging in its own launch
  // (own_fold): it writes every row with own keys, the merge kernel only rows without any
  // (none when the host's list says so)
  if (a.shared_only && a.own_fused == 2 && a.own_fold && ord && ord->n == a.batch && ord->all_own) return RAX_OK;
  if (a.nsplit > 1 || a.shared_only) return launch_merge<D>(a, st);
  return RAX_OK;
}

template <bool kDecode>
static rax_status dispatch(AttnArgs& a, rax_dtype dt, int d, Shape s, hipStream_t st,
                           const AppendJob* ap = nullptr, const OwnOrder* ord = nullptr) {
  if (dt == RAX_BF16) {
    if (d == 128) return launch_shape<__bf16, 128, kDecode>(a, s, st, ap, ord);
    if (d == 64) return launch_shape<__bf16, 64, kDecode>(a, s, st, ap, ord);
  } else {
    if (d == 128) return launch_shape<float, 128, kDecode>(a, s, st, ap, ord);
    if (d == 64) return launch_shape<float, 64, kDecode>(a, s, st, ap, ord);
  }
  return RAX_EINVAL;
}

// Workspace of a decode call, in 4-byte words: shared-part partials (accumulators, then
// m/l), own-part partials (accumulators, then m/l), own-part chunk counters (own_mode 2).
struct DecodeLayout {
  int64_t sh_acc, sh_ml, own_acc, own_ml, own_cnt, total;
  int32_t nsplit, n_rb, n_chunk, bm;
  bool split_decode;
  int32_t own_mode;  // 0: own_kernel + merge_kernel, 1: own_merge_kernel, 2: own_stream_kernel + merge_kernel
  int32_t own_min;   // fewest keys per own chunk
  int32_t sh_small;  // shared part: 4-wave workgroups, 2 tiles per round (two per CU)
  int32_t run_cap;   // most extra shared-part tiles per row block for deeper runs
};

static DecodeLayout decode_layout(int64_t batch, int32_t h_q, int32_t h_kv, int32_t d, int32_t max_seq_len,
                                  rax_dtype dt, DecodeHint hint = {}) {
  DecodeLayout l{};
  const int g = h_q / h_kv;
  const Shape s = pick_shape(true, dt, d);
  l.bm = s.bm();
  l.n_rb = (int32_t)((batch * g + l.bm - 1) / l.bm);
  l.nsplit = choose_nsplit((int64_t)l.n_rb * h_kv, max_seq_len);
  l.split_decode = g == 1 || g == 2 || g == 4 || g == 8 || g == 16;
  // Many prefix tiles per workgroup (many row blocks, long prefixes): the shared part runs
  // in 4-wave workgroups with 2 tiles per round, two per CU, over twice the workgroups, so
  // that two chains of rounds overlap on each CU.
  {
    const int64_t blocks = (int64_t)l.n_rb * h_kv;
    // the most tiles a row block's shared part holds: known from the hints (deeper runs
    // included), else bounded by the longest sequence
    const int64_t tiles = std::max<int64_t>(1, hint.tiles > 0 ? hint.tiles : (max_seq_len + BN - 1) / BN);
    if (l.split_decode && dt == RAX_BF16 && d == 128 && tiles > 8 * (int64_t)l.nsplit) {
      l.sh_small = 1;
      l.nsplit = (int32_t)std::max<int64_t>(1, std::min<int64_t>({(512 + blocks - 1) / blocks, tiles, 32}));
    } else if (hint.tiles > 0 && l.split_decode && dt == RAX_BF16 && d == 128) {
      // the 8-wave form takes a round of kShTiles tiles at once: with the hints' tile
      // count known, no split takes less than a round (a short shared prefix, such as a
      // system prompt under many blocks, then runs in one workgroup per block, with one
      // partial per row to write and merge)
      l.nsplit = (int32_t)std::max<int64_t>(
          1, std::min<int64_t>(l.nsplit, (hint.tiles + kShTiles - 1) / kShTiles));
    }
  }
  // Deeper runs (block_runs) where the shared part runs in shared_kernel: up to four
  // times the longest sequence's tiles per row block, so that a block whose requests
  // form many deep runs cannot make its shared part more than ~5x longer than the rest.
  if (l.split_decode && dt == RAX_BF16 && d == 128)
    l.run_cap = (int32_t)std::min<int64_t>(4 * (((int64_t)max_seq_len + BN - 1) / BN), 1 << 24);
  if (!l.split_decode) {
    l.sh_acc = l.nsplit > 1 ? (int64_t)h_kv * l.n_rb * l.nsplit * l.bm * d : 0;
    l.sh_ml = l.nsplit > 1 ? (int64_t)h_kv * l.n_rb * l.nsplit * l.bm * 2 : 0;
    l.total = l.sh_acc + l.sh_ml;
    return l;
  }
  // own part: chunks per (request, KV head) so that about kOwnWaves waves exist in total,
  // at most one per kOwnMin keys of the longest sequence and at most 64 - nsplit partials
  // per row; the kernel uses fewer when a request has fewer own keys. kOwnWaves is one
  // round of residency (256 CUs x 4 SIMDs x 4 waves at ~120 VGPRs): with more waves the
  // latency chain of each (slots, then K/V, then merge) runs twice; measured on the
  // few-shot decode, 4096 waves 15.4 us, 8192 waves 20.2 us, 2048 waves 16.7 us.
  constexpr int64_t kOwnWaves = 4096;
  const int64_t pairs = std::max<int64_t>(1, batch * h_kv);
  // query-head groups: own keys on MFMA (own_stream_kernel), chunks of at least
  // kOwnTileMin keys, at most kOwnTileChunks per (request, KV head) unless more are needed
  // to keep every chunk within kOwnTileMin keys. Knowing that no request has more than
  // kStreamCap own keys and that the batch fills the GPU (kOneChunkItems (request, KV head)
  // pairs), every request takes one chunk instead: no request then needs a merge.
  // Measured on self-consistency decode (256 requests, at most ~1100 own keys): 180.3 ->
  // 173.1 us per call; on multi-turn, whose longest requests hold thousands of own keys,
  // chunks of up to 1536 or 2048 keys made the longest workgroups the tail (216.7 -> 220.6
  // and 227.0 us), so there the chunks stay at 1024 keys.
  const int64_t cap_chunks = ((int64_t)max_seq_len + kOwnTileMin - 1) / kOwnTileMin;
  if (dt == RAX_BF16 && d == 128 && g >= 2 && cap_chunks <= 64 - l.nsplit) {
    l.own_mode = 2;
    if (hint.own > 0 && hint.own <= kStreamCap && batch * h_kv >= kOneChunkItems) {
      l.own_min = kStreamCap;
      l.n_chunk = 1;
    } else {
      l.own_min = kOwnTileMin;
      l.n_chunk = (int32_t)std::max<int64_t>(
          {1, cap_chunks,
           std::min<int64_t>({64 - l.nsplit, (max_seq_len + kOwnTileMin - 1) / kOwnTileMin, kOwnTileChunks})});
    }
  } else {
    l.own_min = kOwnMin;
    const int64_t by_len = (max_seq_len + kOwnMin - 1) / kOwnMin;
    l.n_chunk = (int32_t)std::max<int64_t>(1, std::min<int64_t>({64 - l.nsplit, by_len, (kOwnWaves + pairs - 1) / pairs}));
    // Knowing the most own keys: enough chunks that each takes one round of keys
    // (kOwnMin), when that stays within 1.5x the wave budget. A chunk's second round costs
    // a whole K/V round trip: few-shot steps with 65..83 own keys measured 36.9 -> 34.8 us
    // at 3 chunks instead of 2, while at most 64 own keys 2 chunks stay faster.
    if (hint.own > 0) {
      const int64_t one_round = (hint.own + kOwnMin - 1) / kOwnMin;
      const int64_t roomy = std::max<int64_t>((kOwnWaves + pairs - 1) / pairs, (3 * kOwnWaves / 2) / pairs);
      l.n_chunk = (int32_t)std::max<int64_t>(
          1, std::min<int64_t>({64 - l.nsplit, by_len, std::max<int64_t>(l.n_chunk, std::min(one_round, roomy))}));
    }
    // the chunks of one (request, KV head) fit one workgroup: merge in LDS, no own partials
    l.own_mode = l.n_chunk <= kOwnFusedMaxWaves && own_fused_lds_bytes(l.n_chunk, g, d) <= kOwnFusedMaxLds ? 1 : 0;
  }
  const int64_t sh_items = (int64_t)h_kv * l.n_rb * l.nsplit;
  const int64_t own_rows = l.own_mode == 1 ? 0 : batch * h_kv * l.n_chunk * g;
  l.sh_acc = sh_items * l.bm * d;
  l.sh_ml = sh_items * l.bm * 2;
  l.own_acc = own_rows * d;
  l.own_ml = own_rows * 2;
  l.own_cnt = l.own_mode == 2 ? batch * h_kv : 0;  // int32 chunk counters
  l.total = l.sh_acc + l.sh_ml + l.own_acc + l.own_ml + l.own_cnt;
  return l;
}

static bool common_ok(int32_t h_q, int32_t h_kv, int32_t d, rax_dtype dt, rax_dtype o_dt) {
  if (h_q < 1 || h_kv < 1 || h_q % h_kv) return false;
  const int g = h_q / h_kv;
  if (g > 64 || 64 % g) return false;  // query-head groups tile every block shape exactly
  if (d != 64 && d != 128) return false;
  if ((dt != RAX_F32 && dt != RAX_BF16) || (o_dt != RAX_F32 && o_dt != RAX_BF16)) return false;
  return true;
}

}  // namespace raxk

using namespace raxk;

extern "C" size_t rax_attention_workspace_bytes(int32_t is_decode, int64_t rows, int32_t h_q, int32_t h_kv,
                                                int32_t d, int32_t max_kv_len) {
  if (rows <= 0 || h_kv < 1 || h_q < h_kv || h_q % h_kv || (d != 64 && d != 128) || max_kv_len < 0) return 0;
  size_t need = 0;  // the larger need of the two input dtypes' block shapes
  if (!is_decode) {  // key-split partials of extend (none without splits)
    for (rax_dtype dt : {RAX_BF16, RAX_F32}) {
      const Shape s = pick_shape(false, dt, d);
      const int64_t n_rb = (rows * (h_q / h_kv) + s.bm() - 1) / s.bm();
      const int32_t nsplit = extend_nsplit(n_rb * h_kv, max_kv_len);
      if (nsplit > 1) need = max(need, ws_bytes_for((int64_t)h_kv * n_rb * nsplit, s.bm(), d));
    }
    return need;
  }
  for (rax_dtype dt : {RAX_BF16, RAX_F32}) {
    const DecodeLayout l = decode_layout(rows, h_q, h_kv, d, max_kv_len, dt);
    need = max(need, (size_t)l.total * sizeof(float));
  }
  return need;
}

extern "C" rax_status rax_extend_attention(const void* q, const void* k_ext, const void* v_ext,
                                           const void* k_pool, const void* v_pool, int64_t num_slots,
                                           const int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                           const int32_t* req_pool_idx, const int32_t* prefix_len,
                                           const int32_t* qo_indptr, const int32_t* shared_len, int32_t batch,
                                           int64_t total_q, int32_t max_kv_len, int32_t h_q, int32_t h_kv,
                                           int32_t d, float sm_scale, rax_dtype dt, void* o, rax_dtype o_dt,
                                           void* workspace, size_t ws_bytes, void* stream) {
  if (!common_ok(h_q, h_kv, d, dt, o_dt) || batch < 0 || total_q < 0 || num_slots < 1 || rtt_stride < 1 ||
      rtt_rows < 1 || rtt_stride > INT32_MAX || max_kv_len < 0)
    return RAX_EINVAL;
  if (batch == 0 || total_q == 0) return RAX_OK;
  if (!q || !k_ext || !v_ext || !k_pool || !v_pool || !req_to_token || !req_pool_idx || !prefix_len ||
      !qo_indptr || !o)
    return RAX_EINVAL;
  const Shape s = pick_shape(false, dt, d);
  AttnArgs a{};
  a.q = q;
  a.k_ext = k_ext;
  a.v_ext = v_ext;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_slots = num_slots;
  a.rtt = req_to_token;
  a.rtt_stride = rtt_stride;
  a.rtt_rows = rtt_rows;
  a.req_pool_idx = req_pool_idx;
  a.kv_len = prefix_len;
  a.qo_indptr = qo_indptr;
  a.shared_len = shared_len;
  a.batch = batch;
  a.total_q = total_q;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.g = h_q / h_kv;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.o = o;
  a.o_bf16 = o_dt == RAX_BF16;
  a.ws = nullptr;
  a.bm = s.bm();
  a.n_rb = (int32_t)((total_q * a.g + a.bm - 1) / a.bm);
  // key splits, as many as the workspace holds (none without one)
  int32_t nsplit = extend_nsplit((int64_t)a.n_rb * h_kv, max_kv_len);
  while (nsplit > 1 && (!workspace || ws_bytes < ws_bytes_for((int64_t)h_kv * a.n_rb * nsplit, a.bm, d))) --nsplit;
  a.nsplit = nsplit;
  if (nsplit > 1) a.ws = reinterpret_cast<float*>(workspace);
  return dispatch<false>(a, dt, d, s, (hipStream_t)stream);
}

size_t raxk::decode_workspace_bytes(int64_t batch, int32_t h_q, int32_t h_kv, int32_t d, int32_t max_seq_len,
                                    DecodeHint hint) {
  if (batch <= 0 || h_kv < 1 || h_q < h_kv || h_q % h_kv || (d != 64 && d != 128) || max_seq_len < 0) return 0;
  size_t need = 0;
  for (rax_dtype dt : {RAX_BF16, RAX_F32}) {
    const DecodeLayout l = decode_layout(batch, h_q, h_kv, d, max_seq_len, dt, hint);
    need = max(need, (size_t)l.total * sizeof(float));
  }
  return need;
}

DecodeHint raxk::decode_hint(const int32_t* len, const int32_t* shared_len, int32_t batch, int32_t h_q,
                             int32_t h_kv, int32_t max_seq_len) {
  DecodeHint hint;
  if (!len || !shared_len || batch < 1 || h_kv < 1 || h_q % h_kv || 64 % (h_q / h_kv)) return hint;
  const int32_t per_block = 64 / (h_q / h_kv);  // requests per 64-row block
  const int64_t cap = 4 * (((int64_t)max_seq_len + BN - 1) / BN);  // as decode_layout's run_cap
  int64_t most = 0, own = 0;
  std::vector<int64_t> own_r(static_cast<size_t>(batch), 0);
  for (int32_t b0 = 0; b0 < batch; b0 += per_block) {
    const int32_t b1 = std::min(batch, b0 + per_block);
    // the block rule: lengths after the append minus one (len here), hints to the predecessor
    int64_t L0 = 1 << 30;
    for (int32_t i = b0; i < b1; ++i) L0 = std::min<int64_t>(L0, i > b0 ? std::min(len[i], shared_len[i]) : len[i]);
    L0 = std::max<int64_t>(L0, 0);
    // deeper runs, taken in order while their tiles stay within the cap
    int64_t extra = 0;
    bool full = false;
    for (int32_t i = b0; i < b1;) {
      int32_t j = i + 1;
      int64_t L1 = len[i];
      while (j < b1 && shared_len[j] > L0) {
        L1 = std::min<int64_t>(L1, std::min(len[j], shared_len[j]));
        ++j;
      }
      int64_t start = L0;  // where the run's own keys start
      if (!full && j - i >= 2 && L1 > L0) {
        const int64_t nt = (L1 - L0 + BN - 1) / BN;
        if (extra + nt > cap) {
          full = true;
        } else {
          extra += nt;
          start = L1;
        }
      }
      for (int32_t r = i; r < j; ++r) {
        own_r[r] = (int64_t)len[r] + 1 - start;
        own = std::max<int64_t>(own, own_r[r]);
      }
      i = j;
    }
    most = std::max(most, (L0 + BN - 1) / BN + extra);
  }
  hint.tiles = (int32_t)std::min<int64_t>(most, 1 << 24);
  hint.own = (int32_t)std::min<int64_t>(std::max<int64_t>(own, 0), 1 << 30);
  if (batch <= kAppendMax) {
    std::vector<int32_t> ord(static_cast<size_t>(batch));
    std::iota(ord.begin(), ord.end(), 0);
    std::stable_sort(ord.begin(), ord.end(), [&](int32_t x, int32_t y) { return own_r[x] > own_r[y]; });
    for (int32_t i = 0; i < batch; ++i) {
      hint.order.req[i] = (uint16_t)ord[i];
      hint.own_keys[i] = (int32_t)std::min<int64_t>(std::max<int64_t>(own_r[i], 0), 1 << 30);
    }
    hint.order.n = batch;
  }
  return hint;
}

bool raxk::decode_folds_append(int32_t batch, int32_t h_q, int32_t h_kv, int32_t d, rax_dtype dt) {
  if (dt != RAX_BF16 || d != 128 || batch < 1 || batch > kAppendMax || h_kv < 1 || h_q % h_kv) return false;
  const int g = h_q / h_kv;
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16;  // split decode: shared_kernel runs first
}

extern "C" rax_status rax_decode_attention(const void* q, const void* k_pool, const void* v_pool,
                                           int64_t num_slots, const int32_t* req_to_token, int64_t rtt_stride,
                                           int64_t rtt_rows, const int32_t* req_pool_idx, const int32_t* seq_len,
                                           const int32_t* shared_len, int32_t batch, int32_t max_seq_len,
                                           int32_t h_q, int32_t h_kv, int32_t d, float sm_scale, rax_dtype dt,
                                           void* o, rax_dtype o_dt, void* workspace, size_t ws_bytes,
                                           void* stream) {
  return raxk::decode_attention_impl(q, k_pool, v_pool, num_slots, req_to_token, rtt_stride, rtt_rows, req_pool_idx,
                                     seq_len, shared_len, batch, max_seq_len, h_q, h_kv, d, sm_scale, dt, o, o_dt,
                                     workspace, ws_bytes, stream, nullptr);
}

rax_status raxk::decode_attention_impl(const void* q, const void* k_pool, const void* v_pool, int64_t num_slots,
                                       const int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                       const int32_t* req_pool_idx, const int32_t* seq_len,
                                       const int32_t* shared_len, int32_t batch, int32_t max_seq_len, int32_t h_q,
                                       int32_t h_kv, int32_t d, float sm_scale, rax_dtype dt, void* o,
                                       rax_dtype o_dt, void* workspace, size_t ws_bytes, void* stream,
                                       const AppendJob* ap, DecodeHint hint) {
  if (!common_ok(h_q, h_kv, d, dt, o_dt) || batch < 0 || max_seq_len < 0 || num_slots < 1 || rtt_stride < 1 ||
      rtt_rows < 1 || rtt_stride > INT32_MAX)
    return RAX_EINVAL;
  if (batch == 0) return RAX_OK;
  if (!q || !k_pool || !v_pool || !req_to_token || !req_pool_idx || !seq_len || !o) return RAX_EINVAL;
  const Shape s = pick_shape(true, dt, d);
  AttnArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_slots = num_slots;
  a.rtt = req_to_token;
  a.rtt_stride = rtt_stride;
  a.rtt_rows = rtt_rows;
  a.req_pool_idx = req_pool_idx;
  a.kv_len = seq_len;
  a.qo_indptr = nullptr;
  a.shared_len = shared_len;
  a.batch = batch;
  a.total_q = batch;
  a.h_q = h_q;
  a.h_kv = h_kv;
  a.g = h_q / h_kv;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.o = o;
  a.o_bf16 = o_dt == RAX_BF16;
  const DecodeLayout l = decode_layout(batch, h_q, h_kv, d, max_seq_len, dt, hint);
  if (l.bm / a.g > 64) return RAX_EINVAL;  // one lane per request of a block (block_meta_load)
  a.bm = l.bm;
  a.n_rb = l.n_rb;
  a.nsplit = l.nsplit;
  if (l.total > 0) {
    if (!workspace || ws_bytes < (size_t)l.total * sizeof(float)) return RAX_EINVAL;
    float* w = reinterpret_cast<float*>(workspace);
    a.ws = w;
    if (l.split_decode) {
      a.shared_only = 1;
      a.ws_own = w + l.sh_acc + l.sh_ml;
      a.n_chunk = l.n_chunk;
      a.own_fused = l.own_mode;
      a.own_min = l.own_min;
      a.sh_small = l.sh_small;
      a.run_cap = l.run_cap;
    }
  }
  if (ap && !(l.split_decode && dt == RAX_BF16 && d == 128)) return RAX_EINVAL;  // see decode_folds_append
  if (hint.order.n == batch && l.own_mode == 2) {
    // the own part's work list: per request, the chunks of its own keys (own_chunks)
    int32_t acc_items = 0;
    hint.order.all_own = 1;
    for (int32_t i = 0; i < batch; ++i) {
      hint.order.cum[i] = (uint16_t)acc_items;
      const int64_t own = hint.own_keys[hint.order.req[i]];
      if (own < 1) hint.order.all_own = 0;
      acc_items += (int32_t)std::min<int64_t>(l.n_chunk, std::max<int64_t>(1, (own + l.own_min - 1) / l.own_min));
    }
    hint.order.cum[batch] = (uint16_t)acc_items;  // <= 256 x 64
    // Requests with several own chunks merge in the own part's launch when few: each of
    // their workgroups then ends with a device-scope count (and the last one with the
    // merge), a few microseconds in which it holds its CU slot. Measured: self-consistency
    // decode (nearly every request one chunk) 195.8 -> 182.9 us per call without the merge
    // launch; multi-turn (most requests 2-4 chunks, ~3000 such items) 218.5 -> 242.8 us.
    int64_t multi = 0;
    for (int32_t i = 0; i < batch; ++i) {
      const int32_t n_i = hint.order.cum[i + 1] - hint.order.cum[i];
      if (n_i > 1) multi += (int64_t)n_i * h_kv;
    }
    if (multi <= kOwnFoldMaxItems) {
      a.own_fold = 1;
      a.own_cnt = reinterpret_cast<int32_t*>(a.ws_own + l.own_acc + l.own_ml);
    }
  } else {
    hint.order.n = 0;
  }
  return dispatch<true>(a, dt, d, s, (hipStream_t)stream, ap, &hint.order);
}

// ---- decode attention that allocates nothing: for callers that cannot allocate device
// memory (code under graph capture, tight serving loops). Its workspace is this file-scope
// device array, which every GPU the library runs on holds until the process ends; calls
// on one GPU share it, so calls that overlap on one GPU race. Nothing in it has to start
// at zero (every kernel writes its partials before the merge reads them; the own part's
// chunk counters, used only with host lengths, are zeroed by the call's first kernel).
// 64 MiB covers 256 requests x 64 query heads x 128 dims for MHA at any length and for
// query-head groups (2 to 16 per KV head) up to 5120 keys per request; larger layouts are
// refused.
constexpr size_t kScratchBytes = 64ull << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of `scratch` on each device, taken once per device with that device
// current (the name itself is a host-side stand-in, never passed to a kernel).
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];
static rax_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return RAX_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RAX_EDEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RAX_OK;
}

extern "C" rax_status rax_decode_attention_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                                   int64_t num_slots, const int32_t* req_to_token,
                                                   int64_t rtt_stride, int64_t rtt_rows,
                                                   const int32_t* req_pool_idx, const int32_t* seq_len,
                                                   const int32_t* shared_len, int32_t batch, int32_t max_seq_len,
                                                   int32_t h_q, int32_t h_kv, int32_t d, float sm_scale,
                                                   rax_dtype dt, void* o, rax_dtype o_dt, void* stream) {
  if (!common_ok(h_q, h_kv, d, dt, o_dt) || batch < 0 || max_seq_len < 0) return RAX_EINVAL;
  if (batch == 0) return RAX_OK;
  const size_t need = raxk::decode_workspace_bytes(batch, h_q, h_kv, d, max_seq_len, DecodeHint{});
  if (need > kScratchBytes) return RAX_ENOMEM;  // beyond the static workspace
  void* ws = nullptr;
  if (need > 0) {
    const rax_status rc = scratch_on_current_device(&ws);
    if (rc != RAX_OK) return rc;
  }
  return raxk::decode_attention_impl(q, k_pool, v_pool, num_slots, req_to_token, rtt_stride, rtt_rows, req_pool_idx,
                                     seq_len, shared_len, batch, max_seq_len, h_q, h_kv, d, sm_scale, dt, o, o_dt, ws,
                                     need > 0 ? kScratchBytes : 0, stream, nullptr);
}
