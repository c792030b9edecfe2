/*
 * rax.h -- C ABI of librax, the MI355X (gfx950) implementation of RadixAttention's
 * data-parallel hot path: attention over a token-granular KV pool whose prefix
 * entries are reused through a radix tree.
 *
 * Sources for the operations (cited by page title and section):
 *   [notes]  "2312.07104_SGLang: Efficient Execution of Structured Language Model
 *            Programs" (paper notes), §3 RadixAttention, App. A.1-A.3, Figure 3.
 *   [lqhl]   "SGLang: Efficient Execution of Structured Language Model Programs
 *            (NeurIPS 2024)" review, "Core method".
 *   [hustzhy] "SGLang: the structured-program revolution in LLM inference" post,
 *            §2.2-2.5 (RadixAttention).
 *   [bowen]  "SGLang: managing the KV cache as a cache for the first time" review,
 *            "How RadixAttention works".
 *
 * Conventions for every entry point:
 *   - Returns rax_status: RAX_OK (0) or a negative code. Nothing throws across the ABI.
 *   - Arrays are caller-owned; capacities are explicit. The library keeps no pointer
 *     to a caller array after the call returns (device calls: until the stream
 *     reaches the launched work).
 *   - Host tree calls are single-threaded: one rax_tree must not be used from two
 *     threads at once. Different trees are independent.
 *   - Device calls take device pointers (e.g. a torch tensor's data_ptr) and a
 *     hipStream_t passed as void*; they only enqueue work and never synchronise.
 *     Arguments are validated on the host before any launch (RAX_EINVAL, nothing
 *     launched). A launch failure is RAX_EDEVICE. Kernels never dereference an
 *     index outside the sizes given here: out-of-range slot ids, request rows or
 *     positions are skipped and recorded in a device error word that
 *     rax_device_errors() reads back.
 *   - Layouts are row-major and dense. The KV pool is K and V arrays of shape
 *     [num_slots, h_kv, d]: one slot holds one token's K (or V) for every KV head
 *     (token-granular paging, [notes] §3: one page per token).
 */
#ifndef RAX_H
#define RAX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t rax_status;
#define RAX_OK 0
#define RAX_EINVAL (-1)  /* bad argument; nothing changed, nothing launched */
#define RAX_ENOMEM (-2)  /* not enough free slots (or host memory); nothing taken */
#define RAX_ESTATE (-3)  /* unknown node, or a ref count would drop below zero */
#define RAX_EDEVICE (-4) /* a HIP call or kernel launch failed */

typedef enum { RAX_F32 = 0, RAX_BF16 = 1 } rax_dtype;

/* Opaque host radix tree that also owns the slot free set of one KV pool. */
typedef struct rax_tree rax_tree;
/* Node handle. 0 is the root; every new node takes the next integer. A handle stays
 * valid until its node is evicted; a node split keeps its handle on the lower part. */
typedef int64_t rax_node;

typedef struct {
  int64_t num_slots;        /* pool size */
  int64_t free_slots;       /* slots in the free set */
  int64_t cached_tokens;    /* tokens held by tree nodes */
  int64_t locked_tokens;    /* tokens in nodes with ref count > 0 */
  int64_t evictable_tokens; /* cached_tokens - locked_tokens */
  int64_t num_nodes;        /* excluding the root */
  int64_t clock;            /* logical LRU clock (one tick per match or insert) */
  int64_t matched_tokens;   /* cumulative over rax_match_prefix calls */
  int64_t inserted_tokens;  /* cumulative new tokens adopted by rax_insert */
  int64_t evicted_tokens;   /* cumulative (device slots freed, demoted or dropped) */
  int64_t host_slots;       /* host tier size (0 = no tier) */
  int64_t host_free_slots;
  int64_t host_tokens;      /* tokens whose KV sits in the host tier (not in cached_tokens) */
  int64_t demoted_tokens;   /* cumulative device -> host */
  int64_t promoted_tokens;  /* cumulative host -> device */
  int64_t pending_moves;    /* moves recorded and not yet run or taken */
} rax_stats;

const char* rax_status_str(rax_status s);
int32_t rax_abi_version(void);

/* ======================================================================== host: tree
 * Semantics ([notes] §3; [bowen] "Work loop: insert, match, split, evict";
 * [hustzhy] §2.3):
 *  - match: longest cached prefix of the request ("traverse"); its KV is reused.
 *  - a node shared only up to a divergence point splits in two (Figure 3 steps 4, 7).
 *  - ref counts pin nodes that running requests depend on; only ref 0 may be freed.
 *  - eviction is LRU over leaves; parents become candidates once they are leaves.
 *  - cached and running KV share one pool of slots.
 * Choices where the pages are silent (fixed so results are reproducible bit for bit):
 *  - a match ending inside a node splits it immediately; the upper part is a new
 *    node with the same ref count and tick; the lower part keeps its handle.
 *  - one logical clock tick per match or insert call; every node on the matched /
 *    inserted path takes it; ties between leaves break by the smaller handle.
 *  - eviction removes whole leaves until at least the requested count is freed
 *    (it may overshoot by part of one leaf) or nothing is evictable.
 *  - the allocator hands out the lowest free slot ids, ascending.
 */

/* Create a tree over a pool of num_slots slots, all free. num_slots in [1, 2^31). */
rax_status rax_tree_create(int64_t num_slots, rax_tree** out);
void rax_tree_destroy(rax_tree* t);

/* Longest cached prefix of tokens[0..n). Writes its slots to out_slots (capacity n,
 * may be NULL when n == 0), the matched length to *out_len and the node where the
 * match ends to *out_node (0 if nothing matched). Splits and ticks as above. */
rax_status rax_match_prefix(rax_tree* t, const int32_t* tokens, int64_t n, int32_t* out_slots,
                            int64_t* out_len, rax_node* out_node);

/* Cache tokens[0..n) with the caller's slots[0..n) (request finished or prefilled;
 * [bowen] "insert"). Positions already cached keep the tree's slot; a caller slot
 * there that differs is returned to the free set. New positions adopt the caller's
 * slots as one new leaf. out_slots (capacity n, or NULL) receives the slot the tree
 * holds for every position afterwards; *out_existing the number of positions that
 * were already cached; *out_node the node ending at position n. Slots must lie in
 * [0, num_slots) and must not be free. */
rax_status rax_insert(rax_tree* t, const int32_t* tokens, const int32_t* slots, int64_t n,
                      int32_t* out_slots, int64_t* out_existing, rax_node* out_node);

/* Add delta (+1 or -1) to the ref count of every node from `node` up to the root.
 * RAX_ESTATE if the node is unknown, is in the host tier, or a count would go below
 * zero (nothing changed). */
rax_status rax_lock_ref(rax_tree* t, rax_node node, int32_t delta);

/* Evict least-recently-used leaves with ref 0 until >= num_tokens slots are freed or
 * nothing is evictable; freed slots go back to the free set. *out_num_freed is the
 * total freed; the first min(cap, total) slot ids, leaf by leaf in eviction order and
 * each leaf in token order, are written to out_freed (may be NULL when cap == 0).
 * With a host tier (rax_set_host_tier) a "leaf" is a device node with ref 0 and no
 * device child, and its KV is demoted to host slots instead of dropped, which records
 * moves that must run (rax_run_moves) before the freed slots are written. */
rax_status rax_evict_lru(rax_tree* t, int64_t num_tokens, int32_t* out_freed, int64_t cap,
                         int64_t* out_num_freed);

/* Take the n lowest free slots (ascending) into out_slots. RAX_ENOMEM: nothing taken. */
rax_status rax_alloc_slots(rax_tree* t, int64_t n, int32_t* out_slots);
/* Allocation as a scheduler does it before running a batch ([notes] App. A.2: form the
 * batch, evicting when memory is short): if fewer than n slots are free, first evict
 * LRU leaves for the shortfall (as rax_evict_lru, reporting into out_freed / cap /
 * *out_num_freed), then take the n lowest free slots. RAX_ENOMEM if still short
 * (evicted slots stay free, nothing is taken). */
rax_status rax_alloc_slots_evict(rax_tree* t, int64_t n, int32_t* out_slots, int32_t* out_freed,
                                 int64_t cap, int64_t* out_num_freed);
/* Number of free slots (O(1)). */
rax_status rax_free_count(const rax_tree* t, int64_t* out);
/* Return slots to the free set. RAX_EINVAL (nothing changed) if one is out of range,
 * already free, or repeated. */
rax_status rax_free_slots(rax_tree* t, const int32_t* slots, int64_t n);

/* Token depth of the deepest common ancestor of nodes a and b (0 = root). Two running
 * requests holding nodes a and b have identical slots on exactly these positions. */
rax_status rax_lca_depth(const rax_tree* t, rax_node a, rax_node b, int64_t* out_depth);

/* Batched forms for a scheduler that handles a whole batch per call ([notes] App. A.2:
 * match every waiting request, then form the batch). Request r's tokens are
 * tokens[indptr[r] .. indptr[r+1]) (indptr: batch + 1 int64 entries, indptr[0] = 0).
 *
 * rax_match_prefix_batch: rax_match_prefix on each request in order; its slots go to
 * out_slots[indptr[r] ..] (capacity indptr[batch]). cut_full != 0: a match covering a
 * whole non-empty request is reported as n - 1 (the node stays the one covering all n).
 * lock != 0: rax_lock_ref(node, +1) after each match. */
rax_status rax_match_prefix_batch(rax_tree* t, const int32_t* tokens, const int64_t* indptr, int32_t batch,
                                  int32_t cut_full, int32_t lock, int32_t* out_slots, int64_t* out_len,
                                  rax_node* out_node);
/* rax_insert on each request in order, with slots[indptr[r] ..]; out_slots (nullable,
 * capacity indptr[batch]) receives the tree's slots. On RAX_EINVAL (a bad slot) the
 * requests before the failing one stay inserted; *out_done (nullable) counts them. */
rax_status rax_insert_batch(rax_tree* t, const int32_t* tokens, const int32_t* slots, const int64_t* indptr,
                            int32_t batch, int32_t* out_slots, int64_t* out_existing, rax_node* out_node,
                            int32_t* out_done);
/* rax_insert_batch without walking and checking each request's cached prefix again
 * ([hustzhy] §2.3 (3): the request's KV is inserted once computed; here from where its
 * prefix matched). start[r] must be a device node whose root path spells the request's
 * first tokens (the node rax_match_prefix(_batch) returned for them, locked since,
 * qualifies: locking keeps it on the device, and splits leave its path and depth as they
 * are), and the request's slots for positions [0, trusted[r]) must be the tree's. The
 * walk starts at the deepest of start[r] and its ancestors that ends at or before
 * trusted[r]; from there on everything is as in rax_insert_batch (same results, same
 * returns). A start node that is unknown, a host node, deeper than the request or whose
 * label differs from the request's tokens gives RAX_ESTATE; a bad slot past the walk's
 * start gives RAX_EINVAL; in both cases the requests before the failing one stay
 * inserted and *out_done (nullable) counts them. */
rax_status rax_insert_batch_from(rax_tree* t, const rax_node* start, const int64_t* trusted, const int32_t* tokens,
                                 const int32_t* slots, const int64_t* indptr, int32_t batch, int32_t* out_slots,
                                 int64_t* out_existing, rax_node* out_node, int32_t* out_done);
/* rax_lock_ref on nodes[0..n) in order. All-or-nothing: RAX_ESTATE changes nothing. */
rax_status rax_lock_ref_batch(rax_tree* t, const rax_node* nodes, int32_t n, int32_t delta);
/* out[0] = 0 and out[i] = rax_lca_depth(nodes[i-1], nodes[i]) for 0 < i < n: the
 * shared_len hint of consecutive requests for the attention kernels. */
rax_status rax_lca_depths(const rax_tree* t, const rax_node* nodes, int32_t n, int32_t* out);

/* out_len[r] = length of the longest cached prefix of request r's tokens
 * tokens[indptr[r] .. indptr[r+1]), for r < batch. Read-only: nothing splits, no clock
 * tick (a scheduler's look at the cache, not a match). */
rax_status rax_prefix_len_batch(const rax_tree* t, const int32_t* tokens, const int64_t* indptr, int32_t batch,
                                int64_t* out_len);

/* Cache-aware scheduling ([notes] §3 and App. A.2; [lqhl] "Cache-aware scheduling"): the
 * order in which waiting requests should be admitted. out_order receives a permutation of
 * [0, batch) (request indices in arrival order); out_len the read-only prefix lengths as
 * rax_prefix_len_batch. Policies:
 *   RAX_SCHED_FCFS    arrival order;
 *   RAX_SCHED_LPM     longest cached prefix first (ties: arrival order) -- the pages' policy;
 *   RAX_SCHED_DFS     token sequences in lexicographic order (ties: arrival order): a
 *                     depth-first order of the requests' own radix tree, the offline
 *                     optimum of Theorem 3.1;
 *   RAX_SCHED_RANDOM  a uniform shuffle (Fisher-Yates with SplitMix64 draws from `seed`:
 *                     for i = batch-1 .. 1, j = next() % (i+1), swap). */
#define RAX_SCHED_FCFS 0
#define RAX_SCHED_LPM 1
#define RAX_SCHED_DFS 2
#define RAX_SCHED_RANDOM 3
rax_status rax_schedule_order(const rax_tree* t, int32_t policy, const int32_t* tokens, const int64_t* indptr,
                              int32_t batch, uint64_t seed, int32_t* out_order, int64_t* out_len);

rax_status rax_tree_stats(const rax_tree* t, rax_stats* out);

/* Serialise the tree in preorder (children by ascending first token), as int64 words:
 * per node [handle, parent handle, length L, ref, tick, tokens[L], slots[L]] (a host
 * node's slots as -1 - host slot id). With
 * buf == NULL (or cap too small) *out_len receives the word count; too small a
 * non-NULL buffer is RAX_EINVAL. */
rax_status rax_tree_dump(const rax_tree* t, int64_t* buf, int64_t cap, int64_t* out_len);

/* ================================================================ host-memory KV tier
 * A second level below the device pool ([hustzhy] §6.1, HiCache: GPU memory holds the
 * hottest KV, host memory the next; the pages' third level, distributed storage, is not
 * built). The tier is a pinned host buffer of host_slots token rows laid out like the
 * pool ([host_slots, h_kv, d], K and V apart); kernels read and write it directly over
 * the bus. Rules (choices where the pages are silent):
 *  - eviction demotes: the LRU device leaf's KV moves to the lowest free host slots and
 *    the node stays in the tree as a host node. If the tier is short, LRU host leaves
 *    are dropped first; if it is still short the node and its host subtree are dropped.
 *  - host nodes only ever have host descendants. Matching (and rax_prefix_len_batch,
 *    the scheduler's ordering) stops at the first host node: reuse needs device KV.
 *  - rax_promote_batch moves the host continuation of each request's cached device
 *    prefix back to device slots (evicting, hence demoting, when short), node by node,
 *    splitting where the request diverges inside a host node; it stops at the first
 *    node that does not fit.
 *  - rax_insert adopts host nodes on the inserted path: the caller's fresh device slots
 *    become the node's slots and its host slots are released (nothing to move).
 *  - every demotion and promotion appends a move (kind 0: device src -> host dst, 1:
 *    host src -> device dst) to the tree's pending list, in decision order. Run in that
 *    order the moves are correct even when a slot freed by one is taken by a later one;
 *    they must run before the caller writes any slot the same calls handed out.
 *  - rax_tree_dump writes a host node's slots as -1 - host slot id. */

/* Enable the tier with host_slots rows (or 0 to disable), at most once while no node is
 * on the host. k_host, v_host: pinned host memory (allocated pinned, e.g.
 * hipHostMalloc), host_slots * h_kv * d elements each, 16-byte aligned, caller-owned and
 * alive while the tree is; both NULL (host-only use: moves are collected with
 * rax_take_moves) or both set. RAX_EINVAL: bad size or memory the device cannot reach;
 * RAX_ESTATE: host nodes exist. */
rax_status rax_set_host_tier(rax_tree* t, int64_t host_slots, void* k_host, void* v_host);

/* For each request i (tokens[indptr[i] .. indptr[i+1]), host int32/int64 arrays), promote
 * its host-resident continuation as described above; out_promoted[i] = tokens promoted.
 * Device slots freed by evictions are reported as by rax_alloc_slots_evict (first cap into
 * out_freed, *out_num_freed = total). Promotions record moves; run them before use. */
rax_status rax_promote_batch(rax_tree* t, const int32_t* tokens, const int64_t* indptr, int32_t batch,
                             int64_t* out_promoted, int32_t* out_freed, int64_t cap, int64_t* out_num_freed);

/* Copy the pending moves (host int32 arrays of cap entries) and clear the list; with
 * kind == src == dst == NULL only *out_len = number pending. RAX_EINVAL if cap is short
 * (nothing taken). */
rax_status rax_take_moves(rax_tree* t, int32_t* kind, int32_t* src, int32_t* dst, int64_t cap, int64_t* out_len);

/* Run the pending moves on `stream` between the device pools ([num_slots, h_kv, d],
 * dtype dt) and the tier's buffers, then clear the list: one kernel launch per 256
 * moves of a phase (a run of one kind), phases in order, a later move to the same
 * destination within a phase superseding an earlier one. RAX_ESTATE if moves are pending
 * and the tier has no buffers. Host arrays are consumed before the call returns. */
rax_status rax_run_moves(rax_tree* t, void* k_pool, void* v_pool, int32_t h_kv, int32_t d, rax_dtype dt,
                         void* stream);

/* ====================================================================== device calls */

/* KV write-back ([bowen] "insert": computed KV is kept for reuse; [notes] App. A.1):
 *   k_pool[out_loc[i], h, :] = k_new[i, h, :] and v_pool[...] = v_new[...] for i < n_tok.
 * k_new, v_new: [n_tok, h_kv, d] of dtype dt. out_loc: device int32 [n_tok].
 * Rows whose slot is outside [0, num_slots) are skipped and flagged. */
rax_status rax_kv_scatter(const void* k_new, const void* v_new, const int32_t* out_loc, int64_t n_tok,
                          void* k_pool, void* v_pool, int64_t num_slots, int32_t h_kv, int32_t d,
                          rax_dtype dt, void* stream);

/* req_to_token row fill: for request r < batch and i < src_indptr[r+1] - src_indptr[r],
 *   req_to_token[req_pool_idx[r] * rtt_stride + start[r] + i] = src_slots[src_indptr[r] + i].
 * All pointers are device int32 arrays; total = src_indptr[batch] (host copy).
 * Entries that would fall outside [0, rtt_rows) x [0, rtt_stride) are skipped and flagged. */
rax_status rax_req_to_token_write(int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                  const int32_t* req_pool_idx, const int32_t* start,
                                  const int32_t* src_indptr, const int32_t* src_slots, int32_t batch,
                                  int64_t total, void* stream);

/* An extend call's two write-backs in one launch: rax_req_to_token_write(req_to_token, ...,
 * total) and rax_kv_scatter(k_new, ..., dt), with the same arguments, checks and flagged
 * errors; either half may be empty (batch or total 0: no rows; n_tok 0: no K/V). The two
 * write different arrays, so nothing orders them within the launch. For a runtime that
 * fills a batch's rows and writes its suffix K/V in the same step (one launch fewer per
 * extend call). */
rax_status rax_extend_write(int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                            const int32_t* req_pool_idx, const int32_t* start, const int32_t* src_indptr,
                            const int32_t* src_slots, int32_t batch, int64_t total, const void* k_new,
                            const void* v_new, const int32_t* out_loc, int64_t n_tok, void* k_pool, void* v_pool,
                            int64_t num_slots, int32_t h_kv, int32_t d, rax_dtype dt, void* stream);

/* One decode step's bookkeeping and write-back for a batch of running requests, in one
 * call: the work a scheduler does between two decode attention calls ([notes] App. A.2:
 * take memory for the batch, evicting LRU leaves when short; [bowen] "insert": keep the
 * new tokens' KV in the pool).
 *  1. Host: one new slot per request, exactly as rax_alloc_slots_evict(t, batch, ...)
 *     (eviction report into out_freed / cap / *out_num_freed); out_slots[i] receives
 *     request i's slot and seq_len[i] is incremented.
 *  2. Device, one kernel on `stream`: req_to_token[req_pool_idx[i], seq_len[i] - 1] =
 *     out_slots[i], seq_len_dev[i] = seq_len[i], and the K/V rows k_new[i], v_new[i]
 *     ([batch, h_kv, d] of dtype dt) go to the pools at out_slots[i].
 * seq_len (in/out) and out_slots are host int32 [batch]; req_pool_idx and seq_len_dev are
 * device int32 [batch]. Slots and lengths travel as kernel arguments, so the host arrays
 * may be reused as soon as the call returns; device arrays must stay alive until the
 * stream passes the call. RAX_EINVAL (nothing changed): bad argument, or a length that
 * would exceed rtt_stride. RAX_ENOMEM: fewer than batch slots even after evicting (the
 * evicted slots stay free, nothing else changes). A req_pool_idx outside [0, rtt_rows)
 * is skipped on the device and flagged (RAX_DEVERR_ROW). With a host tier, moves that
 * step 1's eviction records (and any still pending) run first, on the same stream;
 * RAX_ESTATE up front if the tier has no buffers. */
rax_status rax_decode_append(rax_tree* t, int32_t batch, int32_t* seq_len, int32_t* out_slots,
                             int32_t* out_freed, int64_t cap, int64_t* out_num_freed,
                             const int32_t* req_pool_idx, int32_t* seq_len_dev, int32_t* req_to_token,
                             int64_t rtt_stride, int64_t rtt_rows, const void* k_new, const void* v_new,
                             void* k_pool, void* v_pool, int32_t h_kv, int32_t d, rax_dtype dt, void* stream);

/* Extend (prefill) attention over radix-cached KV ([hustzhy] §2.3 (2): reuse the matched
 * prefix's KV and compute only the unmatched suffix; [lqhl] "Core method").
 * Request r (r < batch) has prefix_len[r] = m_r cached tokens and q_len_r =
 * qo_indptr[r+1] - qo_indptr[r] new tokens. Query row t = qo_indptr[r] + i is the token
 * at absolute position p = m_r + i; for query head h (KV head g = h / (h_q / h_kv)):
 *   keys j <  m_r : K/V from the pool at slot req_to_token[req_pool_idx[r], j]
 *   keys m_r <= j <= p : K/V rows qo_indptr[r] + (j - m_r) of k_ext / v_ext (causal)
 *   o[t, h, :] = softmax_j(sm_scale * q[t,h,:] . k_j) V_j
 * Shapes: q [total_q, h_q, d], k_ext/v_ext [total_q, h_kv, d], o [total_q, h_q, d];
 * metadata arrays are device int32. shared_len (optional, may be NULL) is a hint:
 * shared_len[r] (r >= 1) promises that requests r-1 and r have identical slots at
 * positions [0, shared_len[r]) -- the kernel then loads those K/V tiles once for the
 * query rows of both requests. d in {64, 128}; h_q % h_kv == 0; dt RAX_F32 or RAX_BF16
 * (pools, q, k_ext, v_ext); o_dt RAX_F32 or RAX_BF16; fp32 accumulation throughout.
 * max_kv_len: the most keys any query row of the call sees (max over r of prefix_len[r] +
 * q_len_r), or 0 if unknown. It only sizes the work: when the call has few row blocks
 * (few long requests), each block's key range is split over several workgroups whose
 * partial softmax states go to `workspace` and are merged by log-sum-exp (results equal
 * up to summation order). The split uses at most what ws_bytes holds (size from
 * rax_attention_workspace_bytes(0, total_q, ..., max_kv_len)); with no workspace or
 * max_kv_len 0 there is no split. RAX_EINVAL: bad sizes, dtypes or null pointers. */
rax_status rax_extend_attention(const void* q, const void* k_ext, const void* v_ext,
                                const void* k_pool, const void* v_pool, int64_t num_slots,
                                const int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                const int32_t* req_pool_idx, const int32_t* prefix_len,
                                const int32_t* qo_indptr, const int32_t* shared_len, int32_t batch,
                                int64_t total_q, int32_t max_kv_len, int32_t h_q, int32_t h_kv, int32_t d,
                                float sm_scale, rax_dtype dt, void* o, rax_dtype o_dt, void* workspace,
                                size_t ws_bytes, void* stream);

/* Batched decode attention ([notes] App. A.1: a decoding step attends over the KV of
 * all previous tokens and itself). Request r's new token is already in the pool: its
 * keys are positions 0..seq_len[r]-1, all read through req_to_token. q [batch, h_q, d],
 * o [batch, h_q, d]. The key range is split (split-K) so that enough workgroups run;
 * partial softmax states go to `workspace` (size from rax_attention_workspace_bytes)
 * and are merged by log-sum-exp. shared_len as in rax_extend_attention. */
rax_status rax_decode_attention(const void* q, const void* k_pool, const void* v_pool, int64_t num_slots,
                                const int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                const int32_t* req_pool_idx, const int32_t* seq_len,
                                const int32_t* shared_len, int32_t batch, int32_t max_seq_len,
                                int32_t h_q, int32_t h_kv, int32_t d, float sm_scale, rax_dtype dt,
                                void* o, rax_dtype o_dt, void* workspace, size_t ws_bytes, void* stream);

/* rax_decode_attention that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory (code under graph capture, tight serving loops). Its
 * split-K partials live in a 64 MiB device array of the library (each GPU it runs on
 * holds one until the process ends), whose device address is taken on the first call
 * on each device: make the device of the pools and stream current before calling. Calls
 * on one GPU share that array, so calls that overlap on one GPU (other streams, other
 * host threads) race; calls on one stream do not. Results as rax_decode_attention's.
 * RAX_EINVAL: bad sizes or pointers; RAX_ENOMEM: the call's layout needs more than
 * 64 MiB (rax_attention_workspace_bytes(1, ...) > 64 MiB; nothing runs); RAX_EDEVICE:
 * no device address for the array. */
rax_status rax_decode_attention_noalloc(const void* q, const void* k_pool, const void* v_pool, int64_t num_slots,
                                        const int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                        const int32_t* req_pool_idx, const int32_t* seq_len,
                                        const int32_t* shared_len, int32_t batch, int32_t max_seq_len,
                                        int32_t h_q, int32_t h_kv, int32_t d, float sm_scale, rax_dtype dt,
                                        void* o, rax_dtype o_dt, void* stream);

/* rax_decode_attention with host copies of seq_len and shared_len (seq_len_host,
 * shared_len_host: [batch] each, as the device arrays): the launches are sized from them
 * as rax_decode_step sizes its attention (the tiles each row block's shared part holds,
 * deeper runs included, and the longest own part); results as rax_decode_attention's up
 * to summation order. The workspace this layout needs goes to *out_ws_needed (nullable);
 * if ws_bytes is smaller, nothing is launched and RAX_EINVAL is returned. */
rax_status rax_decode_attention_hinted(const void* q, const void* k_pool, const void* v_pool, int64_t num_slots,
                                       const int32_t* req_to_token, int64_t rtt_stride, int64_t rtt_rows,
                                       const int32_t* req_pool_idx, const int32_t* seq_len,
                                       const int32_t* shared_len, int32_t batch, int32_t max_seq_len, int32_t h_q,
                                       int32_t h_kv, int32_t d, float sm_scale, rax_dtype dt, void* o,
                                       rax_dtype o_dt, void* workspace, size_t ws_bytes, void* stream,
                                       const int32_t* seq_len_host, const int32_t* shared_len_host,
                                       size_t* out_ws_needed);

/* One whole decode step in one call: rax_decode_append (slots, row append, K/V
 * write-back, with any host-tier moves) followed by rax_decode_attention over the rows
 * as they are after the append, on the same stream; max_seq_len is taken from the host
 * lengths. For dt = RAX_BF16, d = 128, h_q / h_kv in {1, 2, 4, 8, 16} and batch <= 256
 * the append is done by the attention's first kernel (one launch less); the results are
 * the same bit for bit. Meant for serving loops, where the per-call argument marshalling of two
 * entry points costs as much host time as the GPU spends on the step: the caller keeps
 * one argument block per decode batch and updates only what changes (q, k_new, v_new, o,
 * stream). Fields are as in the two calls; the pool holds the tree's num_slots rows.
 * Outputs: seq_len (host, incremented), out_slots, out_freed / num_freed, and ws_needed,
 * the workspace bytes the attention needs. If ws_bytes is smaller, nothing is done and
 * RAX_EINVAL is returned with ws_needed set (grow the workspace and call again). Other
 * errors are those of the two calls; an attention error after a successful append leaves
 * the append done. */
typedef struct {
  int32_t batch;
  int32_t* seq_len;           /* host [batch], in/out */
  int32_t* out_slots;         /* host [batch] */
  int32_t* out_freed;         /* host [cap] */
  int64_t cap;
  int64_t num_freed;          /* out */
  size_t ws_needed;           /* out */
  const int32_t* req_pool_idx; /* device [batch] */
  int32_t* seq_len_dev;       /* device [batch] */
  const int32_t* shared_len;  /* device [batch] or NULL */
  int32_t* req_to_token;      /* device [rtt_rows, rtt_stride] */
  int64_t rtt_stride;
  int64_t rtt_rows;
  const void* q;              /* device [batch, h_q, d] */
  const void* k_new;          /* device [batch, h_kv, d] */
  const void* v_new;
  void* k_pool;               /* device [num_slots, h_kv, d] */
  void* v_pool;
  int32_t h_q, h_kv, d;
  float sm_scale;
  rax_dtype dt;
  rax_dtype o_dt;
  void* o;                    /* device [batch, h_q, d] */
  void* workspace;
  size_t ws_bytes;
  void* stream;
  const int32_t* shared_len_host; /* NULL, or a host copy of shared_len [batch]: then the
                                   * shared-prefix part's key splits are sized for the
                                   * deeper runs the hints form (results unchanged) */
} rax_decode_step_args;
rax_status rax_decode_step(rax_tree* t, rax_decode_step_args* args);

/* Workspace bytes that an extend (is_decode = 0, rows = total_q) or decode (is_decode =
 * 1, rows = batch) call with these sizes may use. 0 means the call needs none. */
size_t rax_attention_workspace_bytes(int32_t is_decode, int64_t rows, int32_t h_q, int32_t h_kv,
                                     int32_t d, int32_t max_kv_len);

/* QKV projection of new tokens, fused with their KV write-back (the step before the
 * path; [hustzhy] §2.3 (2): the suffix is computed; [notes] App. A.1: its KV is kept).
 * y = x W^T for x [n_tok, hidden] and W [(h_q + 2 h_kv) d, hidden] (device, row-major,
 * dtype dt = RAX_BF16 only, 16-byte aligned), fp32 sums rounded once to bf16. Output
 * features: Q (first h_q d) -> q_out [n_tok, h_q, d]; K (next h_kv d) -> k_ext
 * [n_tok, h_kv, d]; V (last h_kv d) -> v_ext. With out_loc (device int32 [n_tok]) K and V
 * also go to k_pool / v_pool [num_slots, h_kv, d] at slot out_loc[t] (the write-back of
 * rax_kv_scatter, done by the same kernel); slots outside [0, num_slots) are skipped and
 * flagged. RAX_EINVAL: bad sizes (hidden % 64, (h_q + 2 h_kv) d % 128 and d % 8 must be
 * 0), pointers (all 16-byte aligned) or dtype. Asynchronous on `stream`. */
rax_status rax_qkv_project(const void* x, const void* w, int64_t n_tok, int32_t hidden, int32_t h_q,
                           int32_t h_kv, int32_t d, rax_dtype dt, void* q_out, void* k_ext, void* v_ext,
                           const int32_t* out_loc, void* k_pool, void* v_pool, int64_t num_slots, void* stream);

/* Synchronise `stream`, return (and clear) the device error word: a bit mask of
 * RAX_DEVERR_* for indices the kernels skipped since the last call. */
#define RAX_DEVERR_SLOT 1   /* slot id outside [0, num_slots) */
#define RAX_DEVERR_ROW 2    /* req_to_token row or column outside its bounds */
rax_status rax_device_errors(void* stream, int32_t* out_mask);

#ifdef __cplusplus
}
#endif
#endif /* RAX_H */
