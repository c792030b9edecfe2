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
// Kernel design (one kernel for both; MI355X-specific choices):
//  * A workgroup (4 waves of 64) owns a block of BM = 128 "MFMA rows". A row is a
//    (query token, query head) pair; the h_q / h_kv query heads that share a KV head
//    are packed into consecutive rows, so each K/V tile staged in LDS serves all of
//    them (grouped-query attention). Rows of consecutive requests are packed into
//    one block, so a block can span several requests.
//  * The block's keys form a list of 64-key tiles: first the positions that all of
//    its requests share (same slots; bounded by the shared_len hint), loaded once for
//    every row; then each request's own remaining prefix positions (only the wave(s)
//    holding that request's rows run the MFMAs); then, in extend, the suffix keys of
//    the block's requests from k_ext under a block-diagonal causal mask.
//  * Each tile is gathered slot by slot from HBM with 16-byte loads (16 lanes per
//    token row: coalesced within the row) into LDS: K row-major with a 16-byte row
//    pad, V transposed (d-major) with an 8-byte pad, so the MFMA operand reads are
//    free of bank conflicts.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (fp32: v_mfma_f32_32x32x2_f32): each lane
//    owns one query row, so the softmax row max and sum are in-lane reductions plus
//    one cross-half exchange. O^T = V^T P^T accumulates in fp32; P stays in
//    registers (the contraction index is permuted consistently in both operands).
//  * Online softmax in the log2 domain (scale * log2 e folded into the scores).
//  * Split-K: the tile list is divided into nsplit ranges (decode needs it to fill
//    256 CUs); partial (m, l, acc) go to a workspace and a merge kernel combines
//    them by log-sum-exp. With nsplit == 1 the block writes O directly.
//  * Workgroup ids are remapped so that all blocks of one KV head run on one XCD and
//    share its L2 for the prefix tiles they all read.
#include <math.h>

#include <type_traits>

#include "../../../include/rax.h"
#include "rax_device.h"

namespace raxk {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 128;  // MFMA rows per workgroup (32 per wave)
constexpr int BN = 64;   // keys per tile
constexpr float kNegInf = -INFINITY;

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
  const int32_t* qo_indptr;   // nullptr: request r owns query row r (decode)
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
};

template <typename T, int D>
struct Tile {
  static constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
  static constexpr int CHUNKS = D / EPC;           // chunks per token row
  static constexpr int KPAD = EPC;                 // K row pad: 16 bytes
  static constexpr int VPAD = sizeof(T) == 2 ? 4 : 1;  // V^T row pad: 8 (bf16) / 4 (fp32) bytes
  static constexpr int KSTRIDE = D + KPAD;
  static constexpr int VSTRIDE = BN + VPAD;
};

template <typename T, int D>
struct __align__(16) Smem {
  T k[BN * Tile<T, D>::KSTRIDE];
  T vt[D * Tile<T, D>::VSTRIDE];
  int32_t slot[BN];
  int32_t req_m[BM];
  int32_t req_row[BM];
  int32_t req_qo[BM + 1];
  int32_t own[BM + 1];
  int32_t hdr[8];
};

__device__ __forceinline__ int upper_req(const int32_t* qo, int batch, int64_t t) {
  // last r in [0, batch) with qo[r] <= t
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qo[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Load one 16-byte chunk (or zeros).
__device__ __forceinline__ uint4 ld16(const void* base, int64_t elem_off, int esize, bool ok) {
  if (!ok) return make_uint4(0, 0, 0, 0);
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + elem_off * esize);
}

template <typename T, int D, bool kDecode>
__global__ void __launch_bounds__(kThreads) attn_kernel(AttnArgs a) {
  using TL = Tile<T, D>;
  constexpr bool kBf16 = sizeof(T) == 2;
  __shared__ Smem<T, D> sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int jrow = lane & 31;  // row within the wave's 32
  const int half = lane >> 5;  // which half of the key set this lane holds

  // ---- work item: (KV head, row block, split)
  const int64_t nblocks = (int64_t)gridDim.x;
  const int64_t item = xcd_remap(blockIdx.x, nblocks);
  const int split = (int)(item % a.nsplit);
  const int64_t rb = (item / a.nsplit) % a.n_rb;
  const int h = (int)(item / ((int64_t)a.nsplit * a.n_rb));

  const int64_t G0 = rb * BM;                 // first MFMA row
  const int64_t qa = G0 / a.g;                // first query row (BM % g == 0)
  int64_t qb = qa + BM / a.g;                 // one past the last query row
  if (qb > a.total_q) qb = a.total_q;

  // ---- block metadata (requests covered, shared length, tile list)
  if (tid == 0) {
    int r0, r1;
    if (!kDecode) {
      r0 = upper_req(a.qo_indptr, a.batch, qa);
      r1 = upper_req(a.qo_indptr, a.batch, qb - 1);
    } else {
      r0 = (int)qa;
      r1 = (int)(qb - 1);
    }
    int nreq = r1 - r0 + 1;
    if (nreq > BM) {  // only possible with empty requests in between
      flag_error(RAX_DEVERR_ROW);
      nreq = BM;
    }
    sm.hdr[0] = r0;
    sm.hdr[1] = nreq;
  }
  __syncthreads();
  const int r0 = sm.hdr[0];
  const int nreq = sm.hdr[1];
  for (int i = tid; i < nreq; i += kThreads) {
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
  }
  if (tid == 0) sm.req_qo[nreq] = kDecode ? r0 + nreq : a.qo_indptr[r0 + nreq];
  __syncthreads();
  if (tid == 0) {
    int L;
    if (nreq == 1) {
      L = sm.req_m[0];
    } else {
      L = sm.req_m[0];
      for (int i = 1; i < nreq; ++i) {
        const int sh = a.shared_len ? a.shared_len[r0 + i] : 0;
        L = min(L, min(sm.req_m[i], sh));
      }
      if (L < 0) L = 0;
    }
    int acc = 0;
    for (int i = 0; i < nreq; ++i) {
      sm.own[i] = acc;
      const int rest = sm.req_m[i] - L;
      acc += rest > 0 ? (rest + BN - 1) / BN : 0;
    }
    sm.own[nreq] = acc;
    const int n_sh = (L + BN - 1) / BN;
    int n_suf = 0;
    if (!kDecode) n_suf = (int)((qb - sm.req_qo[0] + BN - 1) / BN);
    const int total = n_sh + acc + n_suf;
    sm.hdr[2] = L;
    sm.hdr[3] = n_sh;
    sm.hdr[4] = acc;
    sm.hdr[5] = (int)(((int64_t)total * split) / a.nsplit);
    sm.hdr[6] = (int)(((int64_t)total * (split + 1)) / a.nsplit);
  }
  __syncthreads();
  const int L = sm.hdr[2];
  const int n_sh = sm.hdr[3];
  const int n_own = sm.hdr[4];
  const int t_begin = sm.hdr[5];
  const int t_end = sm.hdr[6];
  const int suf0 = sm.req_qo[0];

  // ---- this lane's row
  const int R = wave * 32 + jrow;
  const int64_t Gr = G0 + R;
  const int64_t t_row = Gr / a.g;
  const bool row_ok = t_row < qb;
  const int hq = h * a.g + (int)(Gr % a.g);
  int my_req = 0;  // local request index
  if (row_ok) {
    int lo = 0, hi = nreq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sm.req_qo[mid] <= t_row) lo = mid;
      else hi = mid - 1;
    }
    my_req = lo;
  }
  const int my_qo = sm.req_qo[my_req];
  // wave's request range and suffix-key interest range (uniform across the wave)
  int w_rlo = row_ok ? my_req : 1 << 30, w_rhi = row_ok ? my_req : -1;
  int w_klo = row_ok ? my_qo : 1 << 30, w_khi = row_ok ? (int)t_row : -1;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    w_rlo = min(w_rlo, __shfl_xor(w_rlo, off));
    w_rhi = max(w_rhi, __shfl_xor(w_rhi, off));
    w_klo = min(w_klo, __shfl_xor(w_klo, off));
    w_khi = max(w_khi, __shfl_xor(w_khi, off));
  }
  const bool wave_active = w_rhi >= 0;

  // ---- Q fragments (B operand of S^T = K Q^T): row jrow, dims [ks*K + half*K/2, +K/2)
  constexpr int KSTEP = kBf16 ? 16 : 2;
  constexpr int NKS = D / KSTEP;
  typedef typename std::conditional<kBf16, bf16x8, float>::type QFrag;
  QFrag qf[NKS];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + (t_row * a.h_q + hq) * (int64_t)D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (kBf16) {
        if (row_ok) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + half * 8);
        else qf[ks] = bf16x8{};
      } else {
        qf[ks] = row_ok ? qp[ks * 2 + half] : 0.f;
      }
    }
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  const int64_t row_elems = (int64_t)a.h_kv * D;  // elements per pool slot / k_ext row
  int own_i = 0;                                  // request of the current own tile

  for (int tau = t_begin; tau < t_end; ++tau) {
    // -- decode tile
    int kind, cnt, pos0 = 0, kr0 = 0, req_i = 0, row = 0;
    if (tau < n_sh) {
      kind = 0;
      pos0 = tau * BN;
      cnt = min(BN, L - pos0);
      row = sm.req_row[0];
    } else if (tau < n_sh + n_own) {
      kind = 1;
      const int o = tau - n_sh;
      while (sm.own[own_i + 1] <= o) ++own_i;
      req_i = own_i;
      pos0 = L + (o - sm.own[own_i]) * BN;
      cnt = min(BN, sm.req_m[own_i] - pos0);
      row = sm.req_row[own_i];
    } else {
      kind = 2;
      kr0 = suf0 + (tau - n_sh - n_own) * BN;
      cnt = (int)min((int64_t)BN, qb - kr0);
    }

    // -- slot ids of the tile's keys
    if (tid < BN) {
      int s = -1;
      if (kind != 2 && tid < cnt) {
        s = a.rtt[(int64_t)row * a.rtt_stride + pos0 + tid];
        if (s < 0 || s >= a.num_slots) {
          flag_error(RAX_DEVERR_SLOT);
          s = -1;
        }
      } else if (kind == 2 && tid < cnt) {
        s = kr0 + tid;
      }
      sm.slot[tid] = s;
    }
    __syncthreads();

    // -- gather K (row-major) and V (transposed) into LDS
    {
      const void* kb = kind == 2 ? a.k_ext : a.k_pool;
      const void* vb = kind == 2 ? a.v_ext : a.v_pool;
      constexpr int KPP = kThreads / TL::CHUNKS;  // keys per pass
      const int c = tid % TL::CHUNKS;
      const int kk = tid / TL::CHUNKS;
#pragma unroll
      for (int p = 0; p < BN / KPP; ++p) {
        const int key = p * KPP + kk;
        const int s = sm.slot[key];
        const uint4 v = ld16(kb, ((int64_t)s * row_elems + (int64_t)h * D) + c * TL::EPC, sizeof(T), s >= 0);
        *reinterpret_cast<uint4*>(&sm.k[key * TL::KSTRIDE + c * TL::EPC]) = v;
      }
      constexpr int PPP = kThreads / TL::CHUNKS;  // key pairs per pass
#pragma unroll
      for (int p = 0; p < (BN / 2) / PPP; ++p) {
        const int kp = p * PPP + kk;
        const int s0 = sm.slot[2 * kp], s1 = sm.slot[2 * kp + 1];
        const uint4 v0 = ld16(vb, ((int64_t)s0 * row_elems + (int64_t)h * D) + c * TL::EPC, sizeof(T), s0 >= 0);
        const uint4 v1 = ld16(vb, ((int64_t)s1 * row_elems + (int64_t)h * D) + c * TL::EPC, sizeof(T), s1 >= 0);
        const T* e0 = reinterpret_cast<const T*>(&v0);
        const T* e1 = reinterpret_cast<const T*>(&v1);
#pragma unroll
        for (int e = 0; e < TL::EPC; ++e) {
          T* dst = &sm.vt[(c * TL::EPC + e) * TL::VSTRIDE + 2 * kp];
          if constexpr (kBf16) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            *reinterpret_cast<bf16x2*>(dst) = bf16x2{e0[e], e1[e]};
          } else {
            dst[0] = e0[e];
            dst[1] = e1[e];
          }
        }
      }
    }
    __syncthreads();

    // -- does this wave have rows that see any key of the tile?
    bool run = wave_active;
    if (kind == 1) run = run && req_i >= w_rlo && req_i <= w_rhi;
    if (kind == 2) run = run && kr0 <= w_khi && kr0 + cnt > w_klo;

    if (run) {
      f32x16 s[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        f32x16 c16 = f32x16{};
        const T* kr = &sm.k[(sub * 32 + jrow) * TL::KSTRIDE];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if constexpr (kBf16) {
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(kr + ks * 16 + half * 8);
            c16 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], c16, 0, 0, 0);
          } else {
            c16 = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[ks * 2 + half], qf[ks], c16, 0, 0, 0);
          }
        }
        s[sub] = c16;
      }
      // scale + mask; key index of register r: sub*32 + 8*(r/4) + 4*half + r%4
      float mx = kNegInf;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = sub * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          bool ok = row_ok && key < cnt;
          if (kind == 1) ok = ok && my_req == req_i;
          if (kind == 2) {
            const int kr = kr0 + key;
            ok = ok && kr >= my_qo && kr <= t_row;
          }
          const float v = ok ? s[sub][r] * a.scale_log2 : kNegInf;
          s[sub][r] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(s[sub][r] - m_use);
          s[sub][r] = p;
          psum += p;
        }
      }
      psum += __shfl_xor(psum, 32);
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;

      // O^T += V^T P^T
      if constexpr (kBf16) {
        bf16x8 pb[2][2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[sub][kh][e] = (__bf16)s[sub][kh * 8 + e];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const T* vr = &sm.vt[(dt * 32 + jrow) * TL::VSTRIDE];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
              const int kb0 = sub * 32 + kh * 16 + 4 * half;
              const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr + kb0);
              const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + kb0 + 8);
              const bf16x8 af = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
              acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pb[sub][kh], acc[dt], 0, 0, 0);
            }
          }
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const T* vr = &sm.vt[(dt * 32 + jrow) * TL::VSTRIDE];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = sub * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
              acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[key], s[sub][r], acc[dt], 0, 0, 0);
            }
          }
        }
      }
    }
    __syncthreads();
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
        if (a.o_bf16) {
          *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + obase + d0) =
              bf16x4{(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + obase + d0) = make_float4(x0, x1, x2, x3);
        }
      }
    }
  } else {
    float* wacc = a.ws + (item * BM + R) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = dt * 32 + 8 * rg + 4 * half;
        *reinterpret_cast<float4*>(wacc + d0) =
            make_float4(acc[dt][rg * 4 + 0], acc[dt][rg * 4 + 1], acc[dt][rg * 4 + 2], acc[dt][rg * 4 + 3]);
      }
    }
    if (half == 0) {
      const int64_t n_items = (int64_t)a.h_kv * a.n_rb * a.nsplit;
      float* wml = a.ws + n_items * BM * (int64_t)D + (item * BM + R) * 2;
      wml[0] = m_run;
      wml[1] = l_run;
    }
  }
}

// Log-sum-exp merge of split-K partials: one wave per (MFMA row, KV head).
template <int D>
__global__ void __launch_bounds__(256) merge_kernel(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t G = (int64_t)blockIdx.x * 4 + wave;
  const int h = blockIdx.y;
  const int64_t t = G / a.g;
  if (t >= a.total_q) return;
  const int hq = h * a.g + (int)(G % a.g);
  const int64_t rb = G / BM;
  const int R = (int)(G % BM);
  const int64_t n_items = (int64_t)a.h_kv * a.n_rb * a.nsplit;
  const int64_t item0 = ((int64_t)h * a.n_rb + rb) * a.nsplit;
  const float* ml = a.ws + n_items * BM * (int64_t)D;
  float M = kNegInf;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, ml[((item0 + s) * BM + R) * 2]);
  const float Mu = M == kNegInf ? 0.f : M;
  float lsum = 0.f;
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float* e = ml + ((item0 + s) * BM + R) * 2;
    const float w = exp2f(e[0] - Mu);
    if (e[1] == 0.f) continue;
    lsum += w * e[1];
    const float* acc = a.ws + ((item0 + s) * BM + R) * (int64_t)D;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] += w * acc[lane + 64 * i];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int64_t obase = (t * a.h_q + hq) * (int64_t)D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (a.o_bf16) reinterpret_cast<__bf16*>(a.o)[obase + lane + 64 * i] = (__bf16)(o[i] * inv);
    else reinterpret_cast<float*>(a.o)[obase + lane + 64 * i] = o[i] * inv;
  }
}

// ------------------------------------------------------------------ host side
static int choose_nsplit(int64_t blocks, int32_t max_kv_len) {
  // enough workgroups for 256 CUs x 2 resident, but at least ~4 tiles per split
  int64_t want = (512 + blocks - 1) / blocks;
  const int64_t tiles = (int64_t)(max_kv_len + BN - 1) / BN;
  int64_t cap = tiles / 4;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want > 32) want = 32;
  if (want < 1) want = 1;
  return (int)want;
}

static size_t ws_bytes_for(int64_t items, int d) {
  return (size_t)items * BM * (size_t)(d + 2) * sizeof(float);
}

template <typename T, int D>
static rax_status launch(AttnArgs& a, hipStream_t st) {
  const int64_t items = (int64_t)a.h_kv * a.n_rb * a.nsplit;
  if (a.qo_indptr)
    hipLaunchKernelGGL((attn_kernel<T, D, false>), dim3((unsigned)items), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<T, D, true>), dim3((unsigned)items), dim3(kThreads), 0, st, a);
  if (hipGetLastError() != hipSuccess) return RAX_EDEVICE;
  if (a.nsplit > 1) {
    const int64_t rows = a.total_q * a.g;
    hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)((rows + 3) / 4), (unsigned)a.h_kv), dim3(256), 0, st, a);
    if (hipGetLastError() != hipSuccess) return RAX_EDEVICE;
  }
  return RAX_OK;
}

static rax_status dispatch(AttnArgs& a, rax_dtype dt, int d, hipStream_t st) {
  if (dt == RAX_BF16) {
    if (d == 128) return launch<__bf16, 128>(a, st);
    if (d == 64) return launch<__bf16, 64>(a, st);
  } else {
    if (d == 128) return launch<float, 128>(a, st);
    if (d == 64) return launch<float, 64>(a, st);
  }
  return RAX_EINVAL;
}

static bool common_ok(int32_t h_q, int32_t h_kv, int32_t d, rax_dtype dt, rax_dtype o_dt) {
  if (h_q < 1 || h_kv < 1 || h_q % h_kv) return false;
  const int g = h_q / h_kv;
  if (g > BM || BM % g) return false;  // query-head groups tile a block exactly
  if (d != 64 && d != 128) return false;
  if ((dt != RAX_F32 && dt != RAX_BF16) || (o_dt != RAX_F32 && o_dt != RAX_BF16)) return false;
  return true;
}

}  // namespace raxk

using namespace raxk;

extern "C" size_t rax_attention_workspace_bytes(int32_t is_decode, int64_t rows, int32_t h_q, int32_t h_kv,
                                                int32_t d, int32_t max_kv_len) {
  if (rows <= 0 || h_kv < 1 || h_q < h_kv || h_q % h_kv || (d != 64 && d != 128)) return 0;
  if (!is_decode) return 0;  // extend writes O directly
  const int64_t n_rb = (rows * (h_q / h_kv) + BM - 1) / BM;
  const int ns = choose_nsplit(n_rb * h_kv, max_kv_len);
  return ns > 1 ? ws_bytes_for((int64_t)h_kv * n_rb * ns, d) : 0;
}

extern "C" rax_status rax_extend_attention(const void* q, const void* k_ext, const void* v_ext,
                                           const void* k_pool, const void* v_pool, int64_t num_slots,
                                           const int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                           const int32_t* req_pool_idx, const int32_t* prefix_len,
                                           const int32_t* qo_indptr, const int32_t* shared_len, int32_t batch,
                                           int64_t total_q, int32_t h_q, int32_t h_kv, int32_t d,
                                           float sm_scale, rax_dtype dt, void* o, rax_dtype o_dt,
                                           void* workspace, size_t ws_bytes, void* stream) {
  (void)workspace;
  (void)ws_bytes;
  if (!common_ok(h_q, h_kv, d, dt, o_dt) || batch < 0 || total_q < 0 || num_slots < 1 || rtt_stride < 1 ||
      rtt_rows < 1 || rtt_stride > INT32_MAX)
    return RAX_EINVAL;
  if (batch == 0 || total_q == 0) return RAX_OK;
  if (!q || !k_ext || !v_ext || !k_pool || !v_pool || !req_to_token || !req_pool_idx || !prefix_len ||
      !qo_indptr || !o)
    return RAX_EINVAL;
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
  a.nsplit = 1;
  a.n_rb = (int32_t)((total_q * a.g + BM - 1) / BM);
  return dispatch(a, dt, d, (hipStream_t)stream);
}

extern "C" rax_status rax_decode_attention(const void* q, const void* k_pool, const void* v_pool,
                                           int64_t num_slots, const int32_t* req_to_token, int64_t rtt_stride,
                                           int64_t rtt_rows, const int32_t* req_pool_idx, const int32_t* seq_len,
                                           const int32_t* shared_len, int32_t batch, int32_t max_seq_len,
                                           int32_t h_q, int32_t h_kv, int32_t d, float sm_scale, rax_dtype dt,
                                           void* o, rax_dtype o_dt, void* workspace, size_t ws_bytes,
                                           void* stream) {
  if (!common_ok(h_q, h_kv, d, dt, o_dt) || batch < 0 || max_seq_len < 0 || num_slots < 1 || rtt_stride < 1 ||
      rtt_rows < 1 || rtt_stride > INT32_MAX)
    return RAX_EINVAL;
  if (batch == 0) return RAX_OK;
  if (!q || !k_pool || !v_pool || !req_to_token || !req_pool_idx || !seq_len || !o) return RAX_EINVAL;
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
  a.n_rb = (int32_t)(((int64_t)batch * a.g + BM - 1) / BM);
  a.nsplit = choose_nsplit((int64_t)a.n_rb * h_kv, max_seq_len);
  if (a.nsplit > 1) {
    const size_t need = ws_bytes_for((int64_t)h_kv * a.n_rb * a.nsplit, d);
    if (!workspace || ws_bytes < need) return RAX_EINVAL;
    a.ws = reinterpret_cast<float*>(workspace);
  }
  return dispatch(a, dt, d, (hipStream_t)stream);
}
