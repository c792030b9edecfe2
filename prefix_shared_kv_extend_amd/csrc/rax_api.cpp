// C ABI: host radix-tree entry points of librax (declared in include/rax.h).
#include <algorithm>
#include <new>
#include <numeric>
#include <vector>

#include "../../include/rax.h"
#include "radix_tree.h"
#include "rax_internal.h"

struct rax_tree {
  explicit rax_tree(int64_t n) : t(n) {}
  rax::RadixTree t;
  void* k_host = nullptr;  // device-visible addresses of the host tier's K and V rows
  void* v_host = nullptr;
};

// Launches and drains the tree's pending moves (no-op when none).
static rax_status run_pending(rax_tree* t, void* k_pool, void* v_pool, int64_t chunks_per_row, hipStream_t st) {
  rax::Moves& mv = t->t.pending();
  if (mv.kind.empty()) return RAX_OK;
  if (!t->k_host || !t->v_host) return RAX_ESTATE;
  const rax_status s = raxk::launch_kv_moves(mv.kind.data(), mv.src.data(), mv.dst.data(),
                                             static_cast<int64_t>(mv.kind.size()), k_pool, v_pool, t->k_host,
                                             t->v_host, chunks_per_row, st);
  mv.clear();
  return s;
}

#define RAX_GUARD_BEGIN try {
#define RAX_GUARD_END                 \
  }                                   \
  catch (const std::bad_alloc&) {     \
    return RAX_ENOMEM;                \
  }                                   \
  catch (...) {                       \
    return RAX_EINVAL;                \
  }

extern "C" {

const char* rax_status_str(rax_status s) {
  switch (s) {
    case RAX_OK: return "ok";
    case RAX_EINVAL: return "invalid argument";
    case RAX_ENOMEM: return "not enough free slots or memory";
    case RAX_ESTATE: return "unknown node or ref count below zero";
    case RAX_EDEVICE: return "HIP device error";
    default: return "unknown status";
  }
}

int32_t rax_abi_version(void) { return 4; }

rax_status rax_tree_create(int64_t num_slots, rax_tree** out) {
  if (!out || num_slots < 1 || num_slots >= (int64_t(1) << 31)) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  *out = new rax_tree(num_slots);
  return RAX_OK;
  RAX_GUARD_END
}

void rax_tree_destroy(rax_tree* t) { delete t; }

rax_status rax_match_prefix(rax_tree* t, const int32_t* tokens, int64_t n, int32_t* out_slots,
                            int64_t* out_len, rax_node* out_node) {
  if (!t || n < 0 || !out_len || !out_node || (n > 0 && (!tokens || !out_slots))) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  *out_len = t->t.match(tokens, n, out_slots, out_node);
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_insert(rax_tree* t, const int32_t* tokens, const int32_t* slots, int64_t n,
                      int32_t* out_slots, int64_t* out_existing, rax_node* out_node) {
  if (!t || n < 0 || !out_existing || !out_node || (n > 0 && (!tokens || !slots))) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  if (!t->t.insert(tokens, slots, n, out_slots, out_existing, out_node)) return RAX_EINVAL;
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_lock_ref(rax_tree* t, rax_node node, int32_t delta) {
  if (!t || (delta != 1 && delta != -1)) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  return t->t.lock_ref(node, delta) == 0 ? RAX_OK : RAX_ESTATE;
  RAX_GUARD_END
}

rax_status rax_evict_lru(rax_tree* t, int64_t num_tokens, int32_t* out_freed, int64_t cap,
                         int64_t* out_num_freed) {
  if (!t || num_tokens < 0 || cap < 0 || !out_num_freed || (cap > 0 && !out_freed)) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  *out_num_freed = t->t.evict(num_tokens, out_freed, cap);
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_alloc_slots(rax_tree* t, int64_t n, int32_t* out_slots) {
  if (!t || n < 0 || (n > 0 && !out_slots)) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  return t->t.alloc().alloc(n, out_slots) ? RAX_OK : RAX_ENOMEM;
  RAX_GUARD_END
}

rax_status rax_free_slots(rax_tree* t, const int32_t* slots, int64_t n) {
  if (!t || n < 0 || (n > 0 && !slots)) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  const rax::SlotAllocator& a = t->t.alloc();
  std::vector<uint8_t> seen;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t s = slots[i];
    if (s < 0 || s >= a.num_slots() || a.is_free(s)) return RAX_EINVAL;
  }
  if (n > 1) {
    seen.assign(static_cast<size_t>(a.num_slots()), 0);
    for (int64_t i = 0; i < n; ++i) {
      if (seen[slots[i]]) return RAX_EINVAL;
      seen[slots[i]] = 1;
    }
  }
  t->t.alloc().release(slots, n);
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_lca_depth(const rax_tree* t, rax_node a, rax_node b, int64_t* out_depth) {
  if (!t || !out_depth) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  return t->t.lca_depth(a, b, out_depth) ? RAX_OK : RAX_ESTATE;
  RAX_GUARD_END
}

rax_status rax_tree_stats(const rax_tree* t, rax_stats* out) {
  if (!t || !out) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  const rax::RadixTree& r = t->t;
  out->num_slots = r.alloc().num_slots();
  out->free_slots = r.alloc().num_free();
  r.totals(&out->cached_tokens, &out->locked_tokens);
  out->evictable_tokens = out->cached_tokens - out->locked_tokens;
  out->num_nodes = r.num_nodes();
  out->clock = r.clock();
  out->matched_tokens = r.matched_total;
  out->inserted_tokens = r.inserted_total;
  out->evicted_tokens = r.evicted_total;
  out->host_slots = r.host_alloc().num_slots();
  out->host_free_slots = r.host_alloc().num_free();
  out->host_tokens = r.host_tokens;
  out->demoted_tokens = r.demoted_total;
  out->promoted_tokens = r.promoted_total;
  out->pending_moves = static_cast<int64_t>(r.pending().kind.size());
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_tree_dump(const rax_tree* t, int64_t* buf, int64_t cap, int64_t* out_len) {
  if (!t || !out_len || cap < 0) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  const int64_t need = t->t.dump(buf, buf ? cap : 0);
  *out_len = need;
  if (buf && need > cap) return RAX_EINVAL;
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_match_prefix_batch(rax_tree* t, const int32_t* tokens, const int64_t* indptr, int32_t batch,
                                  int32_t cut_full, int32_t lock, int32_t* out_slots, int64_t* out_len,
                                  rax_node* out_node) {
  if (!t || batch < 0 || (batch > 0 && (!indptr || !out_len || !out_node))) return RAX_EINVAL;
  if (batch > 0 && indptr[0] != 0) return RAX_EINVAL;
  for (int32_t r = 0; r < batch; ++r)
    if (indptr[r + 1] < indptr[r]) return RAX_EINVAL;
  if (batch > 0 && indptr[batch] > 0 && (!tokens || !out_slots)) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t n = indptr[r + 1] - indptr[r];
    int64_t m = t->t.match(tokens + indptr[r], n, out_slots + indptr[r], &out_node[r]);
    if (cut_full && n > 0 && m == n) --m;
    out_len[r] = m;
    if (lock) t->t.lock_ref(out_node[r], +1);
  }
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_insert_batch(rax_tree* t, const int32_t* tokens, const int32_t* slots, const int64_t* indptr,
                            int32_t batch, int32_t* out_slots, int64_t* out_existing, rax_node* out_node,
                            int32_t* out_done) {
  if (out_done) *out_done = 0;
  if (!t || batch < 0 || (batch > 0 && (!indptr || !out_existing || !out_node))) return RAX_EINVAL;
  if (batch > 0 && indptr[0] != 0) return RAX_EINVAL;
  for (int32_t r = 0; r < batch; ++r)
    if (indptr[r + 1] < indptr[r]) return RAX_EINVAL;
  if (batch > 0 && indptr[batch] > 0 && (!tokens || !slots)) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t o = indptr[r], n = indptr[r + 1] - o;
    if (!t->t.insert(tokens + o, slots + o, n, out_slots ? out_slots + o : nullptr, &out_existing[r],
                     &out_node[r]))
      return RAX_EINVAL;
    if (out_done) *out_done = r + 1;
  }
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_insert_batch_from(rax_tree* t, const rax_node* start, const int64_t* trusted, const int32_t* tokens,
                                 const int32_t* slots, const int64_t* indptr, int32_t batch, int32_t* out_slots,
                                 int64_t* out_existing, rax_node* out_node, int32_t* out_done) {
  if (out_done) *out_done = 0;
  if (!t || batch < 0 || (batch > 0 && (!indptr || !start || !trusted || !out_existing || !out_node)))
    return RAX_EINVAL;
  if (batch > 0 && indptr[0] != 0) return RAX_EINVAL;
  for (int32_t r = 0; r < batch; ++r)
    if (indptr[r + 1] < indptr[r]) return RAX_EINVAL;
  if (batch > 0 && indptr[batch] > 0 && (!tokens || !slots)) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t o = indptr[r], n = indptr[r + 1] - o;
    const int rc = t->t.insert_from(start[r], trusted[r], tokens + o, slots + o, n,
                                    out_slots ? out_slots + o : nullptr, &out_existing[r], &out_node[r]);
    if (rc == 1) return RAX_ESTATE;
    if (rc == 2) return RAX_EINVAL;
    if (out_done) *out_done = r + 1;
  }
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_lock_ref_batch(rax_tree* t, const rax_node* nodes, int32_t n, int32_t delta) {
  if (!t || n < 0 || (n > 0 && !nodes) || (delta != 1 && delta != -1)) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  for (int32_t i = 0; i < n; ++i) {
    const int rc = t->t.lock_ref(nodes[i], delta);
    if (rc != 0) {  // undo the ones already applied
      for (int32_t j = 0; j < i; ++j) t->t.lock_ref(nodes[j], -delta);
      return RAX_ESTATE;
    }
  }
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_lca_depths(const rax_tree* t, const rax_node* nodes, int32_t n, int32_t* out) {
  if (!t || n < 0 || (n > 0 && (!nodes || !out))) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  if (!t->t.lca_depths(nodes, n, out)) return RAX_ESTATE;
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_free_count(const rax_tree* t, int64_t* out) {
  if (!t || !out) return RAX_EINVAL;
  *out = t->t.alloc().num_free();
  return RAX_OK;
}

rax_status rax_alloc_slots_evict(rax_tree* t, int64_t n, int32_t* out_slots, int32_t* out_freed,
                                 int64_t cap, int64_t* out_num_freed) {
  if (!t || n < 0 || cap < 0 || !out_num_freed || (n > 0 && !out_slots) || (cap > 0 && !out_freed))
    return RAX_EINVAL;
  RAX_GUARD_BEGIN
  rax::RadixTree& r = t->t;
  *out_num_freed = 0;
  const int64_t short_by = n - r.alloc().num_free();
  if (short_by > 0) *out_num_freed = r.evict(short_by, out_freed, cap);
  return r.alloc().alloc(n, out_slots) ? RAX_OK : RAX_ENOMEM;
  RAX_GUARD_END
}

// The host part of a decode append: checks, one slot per request (evicting when short),
// lengths + 1, and pending host-tier moves launched on the stream, which read their slots
// before anything writes the new tokens. *cpr = 16-byte chunks per K row.
static rax_status append_host(rax_tree* t, int32_t batch, int32_t* seq_len, int32_t* out_slots, int32_t* out_freed,
                              int64_t cap, int64_t* out_num_freed, const int32_t* req_pool_idx,
                              int32_t* seq_len_dev, int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                              const void* k_new, const void* v_new, void* k_pool, void* v_pool, int32_t h_kv,
                              int32_t d, rax_dtype dt, void* stream, int64_t* cpr) {
  if (!t || batch < 0 || cap < 0 || !out_num_freed || (cap > 0 && !out_freed) || rtt_stride < 1 || rtt_rows < 1 ||
      h_kv < 1 || d < 1 || (dt != RAX_F32 && dt != RAX_BF16))
    return RAX_EINVAL;
  *out_num_freed = 0;
  if (batch == 0) return RAX_OK;
  if (!seq_len || !out_slots || !req_pool_idx || !seq_len_dev || !req_to_token || !k_new || !v_new || !k_pool ||
      !v_pool)
    return RAX_EINVAL;
  const int64_t row_bytes = (int64_t)h_kv * d * (dt == RAX_F32 ? 4 : 2);
  const uintptr_t mis = (uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_pool | (uintptr_t)v_pool;
  if (row_bytes % 16 || (mis & 15)) return RAX_EINVAL;
  for (int32_t i = 0; i < batch; ++i)
    if (seq_len[i] < 0 || (int64_t)seq_len[i] + 1 > rtt_stride) return RAX_EINVAL;
  if (t->t.host_alloc().num_slots() > 0 && !t->k_host) return RAX_ESTATE;  // demotions would have nowhere to run
  RAX_GUARD_BEGIN
  rax::RadixTree& r = t->t;
  const int64_t short_by = batch - r.alloc().num_free();
  if (short_by > 0) *out_num_freed = r.evict(short_by, out_freed, cap);
  if (!r.alloc().alloc(batch, out_slots)) return RAX_ENOMEM;
  for (int32_t i = 0; i < batch; ++i) seq_len[i] += 1;
  *cpr = row_bytes / 16;
  return run_pending(t, k_pool, v_pool, row_bytes / 16, (hipStream_t)stream);
  RAX_GUARD_END
}

rax_status rax_decode_append(rax_tree* t, int32_t batch, int32_t* seq_len, int32_t* out_slots, int32_t* out_freed,
                             int64_t cap, int64_t* out_num_freed, const int32_t* req_pool_idx, int32_t* seq_len_dev,
                             int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows, const void* k_new,
                             const void* v_new, void* k_pool, void* v_pool, int32_t h_kv, int32_t d, rax_dtype dt,
                             void* stream) {
  int64_t cpr = 0;
  const rax_status s = append_host(t, batch, seq_len, out_slots, out_freed, cap, out_num_freed, req_pool_idx,
                                   seq_len_dev, req_to_token, rtt_stride, rtt_rows, k_new, v_new, k_pool, v_pool, h_kv,
                                   d, dt, stream, &cpr);
  if (s != RAX_OK || batch == 0) return s;
  return raxk::launch_decode_append(batch, out_slots, seq_len, req_pool_idx, seq_len_dev, req_to_token, rtt_stride,
                                    rtt_rows, k_new, v_new, k_pool, v_pool, cpr, (hipStream_t)stream);
}

rax_status rax_prefix_len_batch(const rax_tree* t, const int32_t* tokens, const int64_t* indptr, int32_t batch,
                                int64_t* out_len) {
  if (!t || batch < 0 || (batch > 0 && (!indptr || !out_len))) return RAX_EINVAL;
  for (int32_t r = 0; r < batch; ++r)
    if (indptr[r + 1] < indptr[r] || (indptr[r + 1] > indptr[r] && !tokens)) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  for (int32_t r = 0; r < batch; ++r) out_len[r] = t->t.prefix_len(tokens + indptr[r], indptr[r + 1] - indptr[r]);
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_schedule_order(const rax_tree* t, int32_t policy, const int32_t* tokens, const int64_t* indptr,
                              int32_t batch, uint64_t seed, int32_t* out_order, int64_t* out_len) {
  if (!t || batch < 0 || policy < RAX_SCHED_FCFS || policy > RAX_SCHED_RANDOM) return RAX_EINVAL;
  if (batch == 0) return RAX_OK;
  if (!out_order || !out_len) return RAX_EINVAL;
  rax_status st = rax_prefix_len_batch(t, tokens, indptr, batch, out_len);
  if (st != RAX_OK) return st;
  RAX_GUARD_BEGIN
  std::vector<int32_t> order(static_cast<size_t>(batch));
  std::iota(order.begin(), order.end(), 0);
  if (policy == RAX_SCHED_LPM) {
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return out_len[a] > out_len[b]; });
  } else if (policy == RAX_SCHED_DFS) {
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      return std::lexicographical_compare(tokens + indptr[a], tokens + indptr[a + 1], tokens + indptr[b],
                                          tokens + indptr[b + 1]);
    });
  } else if (policy == RAX_SCHED_RANDOM) {
    // Fisher-Yates, draws from SplitMix64 (Steele, Lea, Flood 2014) started at seed
    uint64_t state = seed;
    auto next = [&state]() {
      state += 0x9E3779B97F4A7C15ull;
      uint64_t z = state;
      z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
      z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
      return z ^ (z >> 31);
    };
    for (int32_t i = batch - 1; i > 0; --i) {
      const int32_t j = static_cast<int32_t>(next() % static_cast<uint64_t>(i + 1));
      std::swap(order[i], order[j]);
    }
  }
  std::copy(order.begin(), order.end(), out_order);
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_decode_attention_hinted(const void* q, const void* k_pool, const void* v_pool, int64_t num_slots,
                                       const int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                       const int32_t* req_pool_idx, const int32_t* seq_len,
                                       const int32_t* shared_len, int32_t batch, int32_t max_seq_len, int32_t h_q,
                                       int32_t h_kv, int32_t d, float sm_scale, rax_dtype dt, void* o,
                                       rax_dtype o_dt, void* workspace, size_t ws_bytes, void* stream,
                                       const int32_t* seq_len_host, const int32_t* shared_len_host,
                                       size_t* out_ws_needed) {
  if (out_ws_needed) *out_ws_needed = 0;
  if (batch < 0 || (batch > 0 && (!seq_len_host || !shared_len_host))) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  // the hint counts from the lengths before a step's append: one less than these
  std::vector<int32_t> before(static_cast<size_t>(batch));
  for (int32_t i = 0; i < batch; ++i) before[i] = std::max(seq_len_host[i] - 1, 0);
  const raxk::DecodeHint hint =
      batch > 0 ? raxk::decode_hint(before.data(), shared_len_host, batch, h_q, h_kv, max_seq_len)
                : raxk::DecodeHint{};
  const size_t need = batch > 0 ? raxk::decode_workspace_bytes(batch, h_q, h_kv, d, max_seq_len, hint) : 0;
  if (out_ws_needed) *out_ws_needed = need;
  if (need > ws_bytes) return RAX_EINVAL;
  return raxk::decode_attention_impl(q, k_pool, v_pool, num_slots, req_to_token, rtt_stride, rtt_rows, req_pool_idx,
                                     seq_len, shared_len, batch, max_seq_len, h_q, h_kv, d, sm_scale, dt, o, o_dt,
                                     workspace, ws_bytes, stream, nullptr, hint);
  RAX_GUARD_END
}

rax_status rax_decode_step(rax_tree* t, rax_decode_step_args* a) {
  if (!t || !a || a->batch < 0) return RAX_EINVAL;
  a->num_freed = 0;
  a->ws_needed = 0;
  if (a->batch == 0) return RAX_OK;
  if (!a->seq_len) return RAX_EINVAL;
  int32_t max_len = 0;
  for (int32_t i = 0; i < a->batch; ++i) max_len = std::max(max_len, a->seq_len[i] + 1);
  // with host hints, the launches are sized for the tiles the row blocks' shared parts
  // hold and for the longest own part
  const raxk::DecodeHint hint = a->shared_len_host ? raxk::decode_hint(a->seq_len, a->shared_len_host, a->batch,
                                                                      a->h_q, a->h_kv, max_len)
                                                   : raxk::DecodeHint{};
  a->ws_needed = a->shared_len_host ? raxk::decode_workspace_bytes(a->batch, a->h_q, a->h_kv, a->d, max_len, hint)
                                    : rax_attention_workspace_bytes(1, a->batch, a->h_q, a->h_kv, a->d, max_len);
  if (a->ws_needed > a->ws_bytes) return RAX_EINVAL;  // nothing done yet
  // the attention's argument checks first (a zero-row call checks shapes and types only)
  if (!a->q || !a->o ||
      rax_decode_attention(a->q, a->k_pool, a->v_pool, t->t.alloc().num_slots(), a->req_to_token, a->rtt_stride,
                           a->rtt_rows, a->req_pool_idx, a->seq_len_dev, a->shared_len, 0, max_len, a->h_q, a->h_kv,
                           a->d, a->sm_scale, a->dt, a->o, a->o_dt, a->workspace, a->ws_bytes, a->stream) != RAX_OK)
    return RAX_EINVAL;
  if (!raxk::decode_folds_append(a->batch, a->h_q, a->h_kv, a->d, a->dt)) {
    const rax_status s = rax_decode_append(t, a->batch, a->seq_len, a->out_slots, a->out_freed, a->cap, &a->num_freed,
                                           a->req_pool_idx, a->seq_len_dev, a->req_to_token, a->rtt_stride,
                                           a->rtt_rows, a->k_new, a->v_new, a->k_pool, a->v_pool, a->h_kv, a->d, a->dt,
                                           a->stream);
    if (s != RAX_OK) return s;
    return raxk::decode_attention_impl(a->q, a->k_pool, a->v_pool, t->t.alloc().num_slots(), a->req_to_token,
                                       a->rtt_stride, a->rtt_rows, a->req_pool_idx, a->seq_len_dev, a->shared_len,
                                       a->batch, max_len, a->h_q, a->h_kv, a->d, a->sm_scale, a->dt, a->o, a->o_dt,
                                       a->workspace, a->ws_bytes, a->stream, nullptr, hint);
  }
  // the append rides in the first attention kernel's launch (one launch less per step)
  raxk::AppendJob job;
  const rax_status s = append_host(t, a->batch, a->seq_len, a->out_slots, a->out_freed, a->cap, &a->num_freed,
                                   a->req_pool_idx, a->seq_len_dev, a->req_to_token, a->rtt_stride, a->rtt_rows,
                                   a->k_new, a->v_new, a->k_pool, a->v_pool, a->h_kv, a->d, a->dt, a->stream,
                                   &job.chunks_per_row);
  if (s != RAX_OK) return s;
  job.k_new = a->k_new;
  job.v_new = a->v_new;
  job.seq_len_dev = a->seq_len_dev;
  job.n = a->batch;
  for (int32_t i = 0; i < a->batch; ++i) {
    job.slot[i] = a->out_slots[i];
    job.len[i] = a->seq_len[i];
  }
  return raxk::decode_attention_impl(a->q, a->k_pool, a->v_pool, t->t.alloc().num_slots(), a->req_to_token,
                                     a->rtt_stride, a->rtt_rows, a->req_pool_idx, a->seq_len_dev, a->shared_len,
                                     a->batch, max_len, a->h_q, a->h_kv, a->d, a->sm_scale, a->dt, a->o, a->o_dt,
                                     a->workspace, a->ws_bytes, a->stream, &job, hint);
}

rax_status rax_set_host_tier(rax_tree* t, int64_t host_slots, void* k_host, void* v_host) {
  if (!t || host_slots < 0 || host_slots >= (int64_t(1) << 31) || (k_host == nullptr) != (v_host == nullptr) ||
      (host_slots == 0 && k_host))
    return RAX_EINVAL;
  void* kd = nullptr;
  void* vd = nullptr;
  if (k_host && (!raxk::host_device_ptr(k_host, &kd) || !raxk::host_device_ptr(v_host, &vd) ||
                 (((uintptr_t)kd | (uintptr_t)vd) & 15)))
    return RAX_EINVAL;
  RAX_GUARD_BEGIN
  if (!t->t.set_host_tier(host_slots)) return RAX_ESTATE;
  t->k_host = kd;
  t->v_host = vd;
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_promote_batch(rax_tree* t, const int32_t* tokens, const int64_t* indptr, int32_t batch,
                             int64_t* out_promoted, int32_t* out_freed, int64_t cap, int64_t* out_num_freed) {
  if (!t || batch < 0 || cap < 0 || !out_num_freed || (cap > 0 && !out_freed) ||
      (batch > 0 && (!indptr || !out_promoted)))
    return RAX_EINVAL;
  for (int32_t i = 0; i < batch; ++i)
    if (indptr[i + 1] < indptr[i] || indptr[0] != 0) return RAX_EINVAL;
  if (batch > 0 && indptr[batch] > 0 && !tokens) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  rax::RadixTree& r = t->t;
  std::vector<int32_t> freed;
  for (int32_t i = 0; i < batch; ++i)
    out_promoted[i] = r.promote(tokens + indptr[i], indptr[i + 1] - indptr[i], &freed);
  *out_num_freed = static_cast<int64_t>(freed.size());
  const int64_t k = std::min<int64_t>(cap, *out_num_freed);
  if (k > 0) std::copy(freed.begin(), freed.begin() + k, out_freed);
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_take_moves(rax_tree* t, int32_t* kind, int32_t* src, int32_t* dst, int64_t cap, int64_t* out_len) {
  if (!t || !out_len || cap < 0 || (kind == nullptr) != (src == nullptr) || (kind == nullptr) != (dst == nullptr))
    return RAX_EINVAL;
  RAX_GUARD_BEGIN
  rax::Moves& mv = t->t.pending();
  const int64_t n = static_cast<int64_t>(mv.kind.size());
  *out_len = n;
  if (!kind) return RAX_OK;  // count only
  if (n > cap) return RAX_EINVAL;
  std::copy(mv.kind.begin(), mv.kind.end(), kind);
  std::copy(mv.src.begin(), mv.src.end(), src);
  std::copy(mv.dst.begin(), mv.dst.end(), dst);
  mv.clear();
  return RAX_OK;
  RAX_GUARD_END
}

rax_status rax_run_moves(rax_tree* t, void* k_pool, void* v_pool, int32_t h_kv, int32_t d, rax_dtype dt,
                         void* stream) {
  if (!t || !k_pool || !v_pool || h_kv < 1 || d < 1 || (dt != RAX_F32 && dt != RAX_BF16)) return RAX_EINVAL;
  const int64_t row_bytes = (int64_t)h_kv * d * (dt == RAX_F32 ? 4 : 2);
  if (row_bytes % 16 || (((uintptr_t)k_pool | (uintptr_t)v_pool) & 15)) return RAX_EINVAL;
  RAX_GUARD_BEGIN
  return run_pending(t, k_pool, v_pool, row_bytes / 16, (hipStream_t)stream);
  RAX_GUARD_END
}

}  // extern "C"
