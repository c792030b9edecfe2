"""ctypes binding of librax (include/rax.h): argument marshalling only.

Host tree calls take numpy int32 arrays; device calls take torch tensors that
already live on the GPU and enqueue work on the current (or given) HIP stream.
Every computation happens inside librax. There is no fallback: if the library
is missing, importing anything that needs it raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# RAX_LIB_PATH selects another build of the same library (the sanitized host build of
# prefix_shared_kv_extend_amd.sanitize_check)
LIB_PATH = os.environ.get("RAX_LIB_PATH") or os.path.join(_HERE, "librax.so")

OK, EINVAL, ENOMEM, ESTATE, EDEVICE = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
DEVERR_SLOT, DEVERR_ROW = 1, 2
SCHED_FCFS, SCHED_LPM, SCHED_DFS, SCHED_RANDOM = 0, 1, 2, 3

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class RaxStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_slots", "free_slots", "cached_tokens", "locked_tokens", "evictable_tokens",
        "num_nodes", "clock", "matched_tokens", "inserted_tokens", "evicted_tokens",
        "host_slots", "host_free_slots", "host_tokens", "demoted_tokens", "promoted_tokens", "pending_moves")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class DecodeStepArgs(ctypes.Structure):
    """rax_decode_step_args (include/rax.h)."""
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", _c_i32p), ("out_slots", _c_i32p), ("out_freed", _c_i32p),
                ("cap", ctypes.c_int64), ("num_freed", ctypes.c_int64), ("ws_needed", ctypes.c_size_t),
                ("req_pool_idx", _vp), ("seq_len_dev", _vp), ("shared_len", _vp), ("req_to_token", _vp),
                ("rtt_stride", ctypes.c_int64), ("rtt_rows", ctypes.c_int64), ("q", _vp), ("k_new", _vp),
                ("v_new", _vp), ("k_pool", _vp), ("v_pool", _vp), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("sm_scale", ctypes.c_float), ("dt", ctypes.c_int32), ("o_dt", ctypes.c_int32),
                ("o", _vp), ("workspace", _vp), ("ws_bytes", ctypes.c_size_t), ("stream", _vp),
                ("shared_len_host", _c_i32p)]


_SIGS = {
    "rax_status_str": (ctypes.c_char_p, [_i32]),
    "rax_abi_version": (_i32, []),
    "rax_tree_create": (_i32, [_i64, ctypes.POINTER(_vp)]),
    "rax_tree_destroy": (None, [_vp]),
    "rax_match_prefix": (_i32, [_vp, _c_i32p, _i64, _c_i32p, _c_i64p, _c_i64p]),
    "rax_insert": (_i32, [_vp, _c_i32p, _c_i32p, _i64, _c_i32p, _c_i64p, _c_i64p]),
    "rax_lock_ref": (_i32, [_vp, _i64, _i32]),
    "rax_evict_lru": (_i32, [_vp, _i64, _c_i32p, _i64, _c_i64p]),
    "rax_alloc_slots": (_i32, [_vp, _i64, _c_i32p]),
    "rax_alloc_slots_evict": (_i32, [_vp, _i64, _c_i32p, _c_i32p, _i64, _c_i64p]),
    "rax_free_count": (_i32, [_vp, _c_i64p]),
    "rax_free_slots": (_i32, [_vp, _c_i32p, _i64]),
    "rax_lca_depth": (_i32, [_vp, _i64, _i64, _c_i64p]),
    "rax_match_prefix_batch": (_i32, [_vp, _c_i32p, _c_i64p, _i32, _i32, _i32, _c_i32p, _c_i64p, _c_i64p]),
    "rax_insert_batch": (_i32, [_vp, _c_i32p, _c_i32p, _c_i64p, _i32, _c_i32p, _c_i64p, _c_i64p, _c_i32p]),
    "rax_insert_batch_from": (_i32, [_vp, _c_i64p, _c_i64p, _c_i32p, _c_i32p, _c_i64p, _i32, _c_i32p, _c_i64p,
                                     _c_i64p, _c_i32p]),
    "rax_lock_ref_batch": (_i32, [_vp, _c_i64p, _i32, _i32]),
    "rax_lca_depths": (_i32, [_vp, _c_i64p, _i32, _c_i32p]),
    "rax_prefix_len_batch": (_i32, [_vp, _c_i32p, _c_i64p, _i32, _c_i64p]),
    "rax_schedule_order": (_i32, [_vp, _i32, _c_i32p, _c_i64p, _i32, ctypes.c_uint64, _c_i32p, _c_i64p]),
    "rax_tree_stats": (_i32, [_vp, ctypes.POINTER(RaxStats)]),
    "rax_decode_step": (_i32, [_vp, ctypes.POINTER(DecodeStepArgs)]),
    "rax_set_host_tier": (_i32, [_vp, _i64, _vp, _vp]),
    "rax_promote_batch": (_i32, [_vp, _c_i32p, _c_i64p, _i32, _c_i64p, _c_i32p, _i64, _c_i64p]),
    "rax_take_moves": (_i32, [_vp, _c_i32p, _c_i32p, _c_i32p, _i64, _c_i64p]),
    "rax_run_moves": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _vp]),
    "rax_tree_dump": (_i32, [_vp, _c_i64p, _i64, _c_i64p]),
    "rax_kv_scatter": (_i32, [_vp, _vp, _vp, _i64, _vp, _vp, _i64, _i32, _i32, _i32, _vp]),
    "rax_decode_append": (_i32, [_vp, _i32, _c_i32p, _c_i32p, _c_i32p, _i64, _c_i64p, _vp, _vp, _vp, _i64, _i64,
                                 _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]),
    "rax_req_to_token_write": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _i32, _i64, _vp]),
    "rax_extend_write": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _i64, _vp, _vp,
                                _i64, _i32, _i32, _i32, _vp]),
    "rax_extend_attention": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp,
                                    _i32, _i64, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _i32, _vp, _sz, _vp]),
    "rax_decode_attention": (_i32, [_vp, _vp, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _i32, _i32,
                                    _i32, _i32, _i32, _f32, _i32, _vp, _i32, _vp, _sz, _vp]),
    "rax_decode_attention_noalloc": (_i32, [_vp, _vp, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _i32, _i32,
                                            _i32, _i32, _i32, _f32, _i32, _vp, _i32, _vp]),
    "rax_decode_attention_hinted": (_i32, [_vp, _vp, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _i32, _i32,
                                           _i32, _i32, _i32, _f32, _i32, _vp, _i32, _vp, _sz, _vp, _c_i32p,
                                           _c_i32p, ctypes.POINTER(_sz)]),
    "rax_attention_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32]),
    "rax_device_errors": (_i32, [_vp, _c_i32p]),
    "rax_qkv_project": (_i32, [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
}

EXPORTS = tuple(_SIGS)
_lib = None


def lib() -> ctypes.CDLL:
    """Load librax.so (built in-tree). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m prefix_shared_kv_extend_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            # array pointers as void pointers: they take addresses as ints (_ptr) as well as
            # ctypes pointer objects; the table keeps the element types for the reader
            f.argtypes = [_vp if t in (_c_i32p, _c_i64p) else t for t in args]
        _lib = L
    return _lib


class RaxError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib().rax_status_str(status).decode()
        super().__init__(f"{what}: {msg} ({status})")
        self.status = status


def _check(st: int, what: str) -> None:
    if st != OK:
        raise RaxError(st, what)


def _i32arr(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(_c_i32p)


def _ptr(a: np.ndarray) -> int:
    """Address of a contiguous host array, for an entry point's pointer argument (the
    argument types are void pointers, so the int goes straight through; several times
    cheaper than building a ctypes pointer object)."""
    return a.__array_interface__["data"][0]


def status_str(st: int) -> str:
    return lib().rax_status_str(st).decode()


# --------------------------------------------------------------------- host tree
class Tree:
    """Owner of one rax_tree (radix tree + slot allocator of one KV pool)."""

    def __init__(self, num_slots: int):
        self._L = lib()
        h = _vp()
        _check(self._L.rax_tree_create(int(num_slots), ctypes.byref(h)), "rax_tree_create")
        self._h = h
        self.num_slots = int(num_slots)
        self._freed = np.empty(self.num_slots, dtype=np.int32)  # eviction report buffer

    def close(self):
        if getattr(self, "_h", None):
            self._L.rax_tree_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def match_prefix(self, tokens):
        t = _i32arr(tokens)
        out = np.empty(len(t), dtype=np.int32)
        m, node = _i64(), _i64()
        _check(self._L.rax_match_prefix(self._h, _ptr(t), len(t), _ptr(out), ctypes.byref(m),
                                        ctypes.byref(node)), "rax_match_prefix")
        return int(m.value), out[: m.value], int(node.value)

    def insert(self, tokens, slots):
        t, s = _i32arr(tokens), _i32arr(slots)
        if len(t) != len(s):
            raise ValueError("tokens and slots differ in length")
        out = np.empty(len(t), dtype=np.int32)
        ex, node = _i64(), _i64()
        _check(self._L.rax_insert(self._h, _ptr(t), _ptr(s), len(t), _ptr(out), ctypes.byref(ex),
                                  ctypes.byref(node)), "rax_insert")
        return int(ex.value), int(node.value), out

    def lock_ref(self, node: int, delta: int) -> None:
        _check(self._L.rax_lock_ref(self._h, int(node), int(delta)), "rax_lock_ref")

    def evict_lru(self, num_tokens: int) -> np.ndarray:
        n = _i64()
        _check(self._L.rax_evict_lru(self._h, int(num_tokens), _ptr(self._freed), self.num_slots,
                                     ctypes.byref(n)), "rax_evict_lru")
        return self._freed[: n.value].copy()

    def alloc_slots(self, n: int) -> np.ndarray:
        out = np.empty(int(n), dtype=np.int32)
        _check(self._L.rax_alloc_slots(self._h, int(n), _ptr(out)), "rax_alloc_slots")
        return out

    def alloc_slots_evict(self, n: int):
        """(slots, freed) -- evicts LRU leaves first when the free set is short."""
        out = np.empty(int(n), dtype=np.int32)
        nf = _i64()
        st = self._L.rax_alloc_slots_evict(self._h, int(n), _ptr(out), _ptr(self._freed), self.num_slots,
                                           ctypes.byref(nf))
        _check(st, "rax_alloc_slots_evict")
        return out, self._freed[: nf.value].copy()

    def decode_append(self, seq_len, req_to_token, req_pool_idx, seq_len_dev, k_new, v_new, k_pool, v_pool,
                      stream=None):
        """One decode step's slot allocation (evicting LRU leaves when short) and write-back
        (rax_decode_append). seq_len: host int32 [batch], incremented in place; req_pool_idx,
        seq_len_dev: device int32 [batch]. Returns (new slots, freed slots)."""
        n = len(seq_len)
        _need(isinstance(seq_len, np.ndarray) and seq_len.dtype == np.int32 and seq_len.flags.c_contiguous,
              "seq_len: contiguous host int32 array")
        _need(k_new.shape == v_new.shape and k_new.shape[0] == n and k_pool.shape == v_pool.shape
              and k_pool.shape[1:] == k_new.shape[1:], "k_new/v_new [batch, h_kv, d], pools [slots, h_kv, d]")
        _need(k_new.dtype == v_new.dtype == k_pool.dtype == v_pool.dtype, "dtypes must agree")
        _need(all(t.is_contiguous() and t.is_cuda for t in (k_new, v_new, k_pool, v_pool)), "contiguous cuda")
        _cuda_i32(req_to_token, req_pool_idx, seq_len_dev)
        _need(req_pool_idx.numel() == n and seq_len_dev.numel() == n, "req_pool_idx, seq_len_dev: [batch]")
        out = np.empty(n, dtype=np.int32)
        nf = _i64()
        st = self._L.rax_decode_append(
            self._h, n, _ptr(seq_len), _ptr(out), _ptr(self._freed), self.num_slots, ctypes.byref(nf),
            _dev(req_pool_idx), _dev(seq_len_dev), _dev(req_to_token), req_to_token.shape[1], req_to_token.shape[0],
            _dev(k_new), _dev(v_new), _dev(k_pool), _dev(v_pool), k_pool.shape[1], k_pool.shape[2],
            _dtype_code(k_pool), _stream(stream, k_pool))
        _check(st, "rax_decode_append")
        return out, self._freed[: nf.value].copy()

    def decode_step_prepare(self, seq_len, req_to_token, req_pool_idx, seq_len_dev, k_pool, v_pool, h_q,
                            shared_len=None, sm_scale=None, o_dtype=None, shared_len_host=None):
        """Argument block of rax_decode_step for one decode batch: everything except the
        per-step tensors, checked once. seq_len: host int32 [batch] (kept and updated in place);
        shared_len_host: optional host copy of shared_len (sizes the shared part's splits)."""
        import torch
        n = len(seq_len)
        _need(isinstance(seq_len, np.ndarray) and seq_len.dtype == np.int32 and seq_len.flags.c_contiguous,
              "seq_len: contiguous host int32 array")
        _need(k_pool.shape == v_pool.shape and k_pool.dtype == v_pool.dtype and k_pool.is_cuda
              and k_pool.is_contiguous() and v_pool.is_contiguous() and k_pool.shape[0] == self.num_slots,
              "pools: contiguous cuda [num_slots, h_kv, d]")
        _cuda_i32(req_to_token, req_pool_idx, seq_len_dev)
        _need(req_pool_idx.numel() == n and seq_len_dev.numel() == n, "req_pool_idx, seq_len_dev: [batch]")
        if shared_len is not None:
            _cuda_i32(shared_len)
            _need(shared_len.numel() == n, "shared_len: [batch]")
        h_kv, d = k_pool.shape[1], k_pool.shape[2]
        a = DecodeStepArgs()
        # evicted slots land in the tree's report buffer (num_slots entries, allocated once)
        keep = {"seq_len": seq_len, "out": np.empty(max(n, 1), dtype=np.int32), "freed": self._freed}
        if shared_len_host is not None:
            _need(shared_len is not None and len(shared_len_host) == n, "shared_len_host: [batch], with shared_len")
            keep["sh_host"] = _i32arr(shared_len_host)
        a.batch = n
        a.seq_len = _p32(seq_len)
        a.out_slots = _p32(keep["out"])
        a.out_freed = _p32(keep["freed"])
        a.cap = self.num_slots
        a.req_pool_idx, a.seq_len_dev = req_pool_idx.data_ptr(), seq_len_dev.data_ptr()
        a.shared_len = shared_len.data_ptr() if shared_len is not None else None
        a.shared_len_host = _p32(keep["sh_host"]) if "sh_host" in keep else None
        a.req_to_token = req_to_token.data_ptr()
        a.rtt_stride, a.rtt_rows = req_to_token.shape[1], req_to_token.shape[0]
        a.k_pool, a.v_pool = k_pool.data_ptr(), v_pool.data_ptr()
        a.h_q, a.h_kv, a.d = int(h_q), int(h_kv), int(d)
        a.sm_scale = float(sm_scale) if sm_scale is not None else 1.0 / float(d) ** 0.5
        a.dt = _dtype_code(k_pool)
        a.o_dt = F32 if o_dtype == torch.float32 else BF16 if o_dtype == torch.bfloat16 else a.dt
        return a, keep, (n, int(h_q), d), (n, h_kv, d), k_pool.dtype, k_pool.get_device()

    def decode_step(self, prep, q, k_new, v_new, o, workspace, stream=None):
        """rax_decode_step with a block from decode_step_prepare; sets the per-step tensors.
        Returns (new slots, freed slots, the workspace bytes the call needed)."""
        a, keep, qshape, kshape, dtype, dev = prep
        _need(tuple(q.shape) == qshape and tuple(k_new.shape) == kshape and tuple(v_new.shape) == kshape
              and tuple(o.shape) == qshape and q.dtype == dtype and k_new.dtype == dtype and v_new.dtype == dtype,
              "q, o: [batch, h_q, d]; k_new, v_new: [batch, h_kv, d], the pool dtype")
        _need(all(t.is_contiguous() and t.is_cuda and t.get_device() == dev for t in (q, k_new, v_new, o)),
              "q, k_new, v_new, o: contiguous tensors on the pools' device")
        _need(workspace is None or (workspace.is_contiguous() and workspace.is_cuda and workspace.get_device() == dev),
              "workspace: contiguous, on the pools' device")
        a.q, a.k_new, a.v_new, a.o = q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), o.data_ptr()
        a.o_dt = _dtype_code(o)
        a.workspace = workspace.data_ptr() if workspace is not None else None
        a.ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        a.stream = _stream(stream, q).value
        st = self._L.rax_decode_step(self._h, ctypes.byref(a))
        if st == EINVAL and a.ws_needed > a.ws_bytes:
            return None, None, int(a.ws_needed)
        _check(st, "rax_decode_step")
        return keep["out"][: a.batch], keep["freed"][: a.num_freed].copy(), int(a.ws_needed)

    # ------------------------------------------------------------ host tier
    def set_host_tier(self, host_slots: int, k_host=None, v_host=None) -> None:
        """Enable the host tier (rax_set_host_tier): host_slots token rows; k_host, v_host pinned
        CPU tensors [host_slots, h_kv, d] (or None for host-only use, moves taken by take_moves)."""
        if k_host is not None:
            _need(k_host.shape == v_host.shape and k_host.shape[0] == host_slots and k_host.dtype == v_host.dtype
                  and k_host.is_pinned() and v_host.is_pinned() and k_host.is_contiguous() and v_host.is_contiguous(),
                  "k_host/v_host: pinned contiguous [host_slots, h_kv, d]")
        _check(self._L.rax_set_host_tier(self._h, int(host_slots), _dev(k_host), _dev(v_host)), "rax_set_host_tier")

    def promote_batch(self, tokens, indptr):
        """Promote each request's host-resident continuation (rax_promote_batch).
        Returns (promoted tokens per request, device slots freed by evictions)."""
        t = _i32arr(tokens)
        ip = np.ascontiguousarray(np.asarray(indptr, dtype=np.int64))
        b = len(ip) - 1
        out = np.zeros(max(b, 0), dtype=np.int64)
        cap = 2 * self.num_slots + len(t)
        freed = np.empty(cap, dtype=np.int32)
        nf = _i64()
        _check(self._L.rax_promote_batch(self._h, _ptr(t), _ptr(ip), b,
                                         _ptr(out), _ptr(freed), cap, ctypes.byref(nf)),
               "rax_promote_batch")
        if nf.value > cap:
            raise RuntimeError("rax_promote_batch: eviction report truncated")
        return out, freed[: nf.value].copy()

    def take_moves(self):
        """Pending moves as (kind, src, dst) int32 arrays; clears the list (rax_take_moves)."""
        n = _i64()
        _check(self._L.rax_take_moves(self._h, None, None, None, 0, ctypes.byref(n)), "rax_take_moves")
        k, s, d = (np.empty(max(n.value, 1), dtype=np.int32) for _ in range(3))
        _check(self._L.rax_take_moves(self._h, _ptr(k), _ptr(s), _ptr(d), len(k), ctypes.byref(n)),
               "rax_take_moves")
        return k[: n.value].copy(), s[: n.value].copy(), d[: n.value].copy()

    def run_moves(self, k_pool, v_pool, stream=None) -> None:
        """Launch the pending moves between the pools and the host tier (rax_run_moves)."""
        _need(k_pool.shape == v_pool.shape and k_pool.is_cuda and k_pool.is_contiguous() and v_pool.is_contiguous(),
              "pools: contiguous cuda [slots, h_kv, d]")
        _check(self._L.rax_run_moves(self._h, _dev(k_pool), _dev(v_pool), k_pool.shape[1], k_pool.shape[2],
                                     _dtype_code(k_pool), _stream(stream, k_pool)), "rax_run_moves")

    def free_count(self) -> int:
        n = _i64()
        _check(self._L.rax_free_count(self._h, ctypes.byref(n)), "rax_free_count")
        return int(n.value)

    def free_slots(self, slots) -> None:
        s = _i32arr(slots)
        _check(self._L.rax_free_slots(self._h, _ptr(s), len(s)), "rax_free_slots")

    def match_prefix_batch(self, tokens_flat, indptr, cut_full=True, lock=True):
        """Batched match (and lock) of requests tokens_flat[indptr[r]:indptr[r+1]].
        Returns (slots_flat, m[batch], node[batch])."""
        t = _i32arr(tokens_flat)
        ip = np.ascontiguousarray(indptr, dtype=np.int64)
        b = len(ip) - 1
        out = np.empty(max(len(t), 1), dtype=np.int32)
        m = np.empty(b, dtype=np.int64)
        nodes = np.empty(b, dtype=np.int64)
        _check(self._L.rax_match_prefix_batch(self._h, _ptr(t), _ptr(ip), b, int(cut_full),
                                              int(lock), _ptr(out), _ptr(m),
                                              _ptr(nodes)), "rax_match_prefix_batch")
        return out[: len(t)], m, nodes

    def prefix_len_batch(self, tokens_flat, indptr) -> np.ndarray:
        """Read-only longest cached prefix of each request (no split, no clock tick)."""
        t = _i32arr(tokens_flat)
        ip = np.ascontiguousarray(indptr, dtype=np.int64)
        out = np.empty(len(ip) - 1, dtype=np.int64)
        _check(self._L.rax_prefix_len_batch(self._h, _ptr(t), _ptr(ip), len(ip) - 1,
                                            _ptr(out)), "rax_prefix_len_batch")
        return out

    def schedule_order(self, policy: int, tokens_flat, indptr, seed: int = 0):
        """Admission order of waiting requests under a SCHED_* policy (rax_schedule_order).
        Returns (order[batch] of request indices, cached prefix length[batch])."""
        t = _i32arr(tokens_flat)
        ip = np.ascontiguousarray(indptr, dtype=np.int64)
        b = len(ip) - 1
        order = np.empty(b, dtype=np.int32)
        m = np.empty(b, dtype=np.int64)
        _check(self._L.rax_schedule_order(self._h, int(policy), _ptr(t), _ptr(ip), b,
                                          int(seed) & (2 ** 64 - 1), _ptr(order), _ptr(m)),
               "rax_schedule_order")
        return order, m

    def insert_batch(self, tokens_flat, slots_flat, indptr):
        """Batched insert. Returns (tree_slots_flat, existing[batch], node[batch])."""
        t, sl = _i32arr(tokens_flat), _i32arr(slots_flat)
        ip = np.ascontiguousarray(indptr, dtype=np.int64)
        b = len(ip) - 1
        out = np.empty(max(len(t), 1), dtype=np.int32)
        ex = np.empty(b, dtype=np.int64)
        nodes = np.empty(b, dtype=np.int64)
        done = ctypes.c_int32()
        _check(self._L.rax_insert_batch(self._h, _ptr(t), _ptr(sl), _ptr(ip), b, _ptr(out),
                                        _ptr(ex), _ptr(nodes),
                                        ctypes.byref(done)), "rax_insert_batch")
        return out[: len(t)], ex, nodes

    def insert_batch_from(self, start_nodes, trusted, tokens_flat, slots_flat, indptr):
        """insert_batch with each walk starting at start_nodes[r] (rax_insert_batch_from):
        a node matched for the request's tokens and locked since; slots before trusted[r]
        are the tree's. Same returns."""
        t, sl = _i32arr(tokens_flat), _i32arr(slots_flat)
        ip = np.ascontiguousarray(indptr, dtype=np.int64)
        st = np.ascontiguousarray(start_nodes, dtype=np.int64)
        tr = np.ascontiguousarray(trusted, dtype=np.int64)
        b = len(ip) - 1
        _need(len(st) == b and len(tr) == b, "start_nodes, trusted: one per request")
        out = np.empty(max(len(t), 1), dtype=np.int32)
        ex = np.empty(b, dtype=np.int64)
        nodes = np.empty(b, dtype=np.int64)
        done = ctypes.c_int32()
        _check(self._L.rax_insert_batch_from(self._h, _ptr(st), _ptr(tr),
                                             _ptr(t), _ptr(sl),
                                             _ptr(ip), b, _ptr(out), _ptr(ex),
                                             _ptr(nodes), ctypes.byref(done)),
               "rax_insert_batch_from")
        return out[: len(t)], ex, nodes

    def lock_ref_batch(self, nodes, delta: int) -> None:
        nd = np.ascontiguousarray(nodes, dtype=np.int64)
        _check(self._L.rax_lock_ref_batch(self._h, _ptr(nd), len(nd), int(delta)),
               "rax_lock_ref_batch")

    def lca_depths(self, nodes) -> np.ndarray:
        nd = np.ascontiguousarray(nodes, dtype=np.int64)
        out = np.zeros(len(nd), dtype=np.int32)
        _check(self._L.rax_lca_depths(self._h, _ptr(nd), len(nd), _ptr(out)), "rax_lca_depths")
        return out

    def lca_depth(self, a: int, b: int) -> int:
        d = _i64()
        _check(self._L.rax_lca_depth(self._h, int(a), int(b), ctypes.byref(d)), "rax_lca_depth")
        return int(d.value)

    def stats(self) -> dict:
        s = RaxStats()
        _check(self._L.rax_tree_stats(self._h, ctypes.byref(s)), "rax_tree_stats")
        return s.as_dict()

    def dump(self) -> list:
        """Preorder list of (id, parent, length, ref, tick, tokens, slots)."""
        n = _i64()
        _check(self._L.rax_tree_dump(self._h, None, 0, ctypes.byref(n)), "rax_tree_dump")
        buf = np.empty(max(1, n.value), dtype=np.int64)
        _check(self._L.rax_tree_dump(self._h, _ptr(buf), len(buf), ctypes.byref(n)),
               "rax_tree_dump")
        out, i, words = [], 0, buf[: n.value].tolist()
        while i < len(words):
            nid, par, ln, ref, tick = words[i: i + 5]
            toks = tuple(words[i + 5: i + 5 + ln])
            sl = tuple(words[i + 5 + ln: i + 5 + 2 * ln])
            out.append((nid, par, ln, ref, tick, toks, sl))
            i += 5 + 2 * ln
        return out


# ----------------------------------------------------------------- device calls
def _dev(t):
    return _vp(t.data_ptr()) if t is not None else _vp(0)


def _stream(stream, like=None):
    """hipStream_t of `stream`; None means the current stream of like's device (else of the
    current device). torch.cuda.current_stream() costs ~10 us per call, the raw query ~1 us."""
    if stream is None:
        import torch
        dev = like.get_device() if like is not None else torch._C._cuda_getDevice()
        return _vp(torch._C._cuda_getCurrentRawStream(dev))
    return _vp(getattr(stream, "cuda_stream", stream))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _cuda_i32(*ts):
    import torch
    for t in ts:
        if t is not None:
            _need(t.is_cuda and t.dtype == torch.int32 and t.is_contiguous(), "index arrays: contiguous cuda int32")


def kv_scatter(k_new, v_new, out_loc, k_pool, v_pool, stream=None) -> None:
    _need(k_new.shape == v_new.shape and k_new.dim() == 3, "k_new/v_new: [n_tok, h_kv, d]")
    _need(k_pool.shape == v_pool.shape and k_pool.shape[1:] == k_new.shape[1:], "pool: [num_slots, h_kv, d]")
    _need(k_new.dtype == k_pool.dtype == v_new.dtype == v_pool.dtype, "dtypes must agree")
    _need(all(t.is_contiguous() and t.is_cuda for t in (k_new, v_new, k_pool, v_pool)), "contiguous cuda tensors")
    _cuda_i32(out_loc)
    _need(out_loc.numel() == k_new.shape[0], "out_loc: [n_tok]")
    _check(lib().rax_kv_scatter(_dev(k_new), _dev(v_new), _dev(out_loc), k_new.shape[0], _dev(k_pool),
                                _dev(v_pool), k_pool.shape[0], k_pool.shape[1], k_pool.shape[2],
                                _dtype_code(k_pool), _stream(stream, k_pool)), "rax_kv_scatter")


def req_to_token_write(req_to_token, req_pool_idx, start, src_indptr, src_slots, total: int, stream=None) -> None:
    _cuda_i32(req_to_token, req_pool_idx, start, src_indptr, src_slots)
    _need(req_to_token.dim() == 2, "req_to_token: [rows, stride]")
    b = req_pool_idx.numel()
    _need(start.numel() == b and src_indptr.numel() == b + 1 and src_slots.numel() >= total, "shapes")
    _check(lib().rax_req_to_token_write(_dev(req_to_token), req_to_token.shape[1], req_to_token.shape[0],
                                        _dev(req_pool_idx), _dev(start), _dev(src_indptr), _dev(src_slots),
                                        b, int(total), _stream(stream, req_to_token)), "rax_req_to_token_write")


def extend_write(req_to_token, req_pool_idx, start, src_indptr, src_slots, total: int, k_new, v_new, out_loc,
                 k_pool, v_pool, stream=None) -> None:
    """rax_extend_write: req_to_token_write and kv_scatter (the same arguments) in one launch."""
    _cuda_i32(req_to_token, req_pool_idx, start, src_indptr, src_slots, out_loc)
    _need(req_to_token.dim() == 2, "req_to_token: [rows, stride]")
    b = req_pool_idx.numel()
    _need(start.numel() == b and src_indptr.numel() == b + 1 and src_slots.numel() >= total, "shapes")
    _need(k_new.shape == v_new.shape and k_new.dim() == 3, "k_new/v_new: [n_tok, h_kv, d]")
    _need(k_pool.shape == v_pool.shape and k_pool.shape[1:] == k_new.shape[1:], "pool: [num_slots, h_kv, d]")
    _need(k_new.dtype == k_pool.dtype == v_new.dtype == v_pool.dtype, "dtypes must agree")
    _need(all(t.is_contiguous() and t.is_cuda for t in (k_new, v_new, k_pool, v_pool)), "contiguous cuda tensors")
    _need(out_loc.numel() == k_new.shape[0], "out_loc: [n_tok]")
    _check(lib().rax_extend_write(_dev(req_to_token), req_to_token.shape[1], req_to_token.shape[0],
                                  _dev(req_pool_idx), _dev(start), _dev(src_indptr), _dev(src_slots), b, int(total),
                                  _dev(k_new), _dev(v_new), _dev(out_loc), k_new.shape[0], _dev(k_pool), _dev(v_pool),
                                  k_pool.shape[0], k_pool.shape[1], k_pool.shape[2], _dtype_code(k_pool),
                                  _stream(stream, k_pool)), "rax_extend_write")


def attention_workspace_bytes(is_decode: bool, rows: int, h_q: int, h_kv: int, d: int, max_kv_len: int) -> int:
    return int(lib().rax_attention_workspace_bytes(int(bool(is_decode)), int(rows), h_q, h_kv, d, int(max_kv_len)))


def extend_attention(q, k_ext, v_ext, k_pool, v_pool, req_to_token, req_pool_idx, prefix_len, qo_indptr,
                     o, shared_len=None, sm_scale=None, workspace=None, stream=None, max_kv_len: int = 0) -> None:
    """rax_extend_attention. max_kv_len (the most keys a query row sees, 0 = unknown) and a
    workspace of rax_attention_workspace_bytes(False, total_q, ..., max_kv_len) bytes let a
    call of few long requests split its key ranges over more workgroups."""
    _need(q.dim() == 3 and k_ext.dim() == 3 and q.shape[0] == k_ext.shape[0], "q [T,h_q,d], k_ext [T,h_kv,d]")
    _need(k_ext.shape == v_ext.shape and k_pool.shape == v_pool.shape, "k/v shapes")
    _need(k_pool.shape[1:] == k_ext.shape[1:] and q.shape[2] == k_pool.shape[2], "head shapes")
    _need(o.shape == q.shape and o.is_contiguous() and o.is_cuda, "o like q")
    _need(q.dtype == k_ext.dtype == v_ext.dtype == k_pool.dtype == v_pool.dtype, "input dtypes agree")
    _need(all(t.is_contiguous() and t.is_cuda for t in (q, k_ext, v_ext, k_pool, v_pool)), "contiguous cuda")
    _cuda_i32(req_to_token, req_pool_idx, prefix_len, qo_indptr, shared_len)
    b = req_pool_idx.numel()
    _need(prefix_len.numel() == b and qo_indptr.numel() == b + 1, "metadata shapes")
    _need(shared_len is None or shared_len.numel() == b, "shared_len: [batch]")
    _need(workspace is None or (workspace.is_cuda and workspace.is_contiguous()), "workspace: contiguous cuda")
    d = q.shape[2]
    scale = float(sm_scale if sm_scale is not None else d ** -0.5)
    ws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().rax_extend_attention(
        _dev(q), _dev(k_ext), _dev(v_ext), _dev(k_pool), _dev(v_pool), k_pool.shape[0],
        _dev(req_to_token), req_to_token.shape[1], req_to_token.shape[0], _dev(req_pool_idx), _dev(prefix_len),
        _dev(qo_indptr), _dev(shared_len), b, q.shape[0], int(max_kv_len), q.shape[1], k_pool.shape[1], d, scale,
        _dtype_code(q), _dev(o), _dtype_code(o), _dev(workspace), ws, _stream(stream, q)), "rax_extend_attention")


def decode_attention(q, k_pool, v_pool, req_to_token, req_pool_idx, seq_len, max_seq_len: int, o,
                     workspace=None, shared_len=None, sm_scale=None, stream=None) -> None:
    _need(q.dim() == 3 and q.shape[2] == k_pool.shape[2] and k_pool.shape == v_pool.shape, "shapes")
    _need(o.shape == q.shape and o.is_contiguous() and o.is_cuda, "o like q")
    _need(q.dtype == k_pool.dtype == v_pool.dtype, "input dtypes agree")
    _need(all(t.is_contiguous() and t.is_cuda for t in (q, k_pool, v_pool)), "contiguous cuda")
    _cuda_i32(req_to_token, req_pool_idx, seq_len, shared_len)
    b = q.shape[0]
    _need(req_pool_idx.numel() == b and seq_len.numel() == b, "metadata shapes")
    d = q.shape[2]
    scale = float(sm_scale if sm_scale is not None else d ** -0.5)
    ws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().rax_decode_attention(
        _dev(q), _dev(k_pool), _dev(v_pool), k_pool.shape[0], _dev(req_to_token), req_to_token.shape[1],
        req_to_token.shape[0], _dev(req_pool_idx), _dev(seq_len), _dev(shared_len), b, int(max_seq_len),
        q.shape[1], k_pool.shape[1], d, scale, _dtype_code(q), _dev(o), _dtype_code(o), _dev(workspace), ws,
        _stream(stream, q)), "rax_decode_attention")


def decode_attention_noalloc(q, k_pool, v_pool, req_to_token, req_pool_idx, seq_len, max_seq_len: int, o,
                             shared_len=None, sm_scale=None, stream=None) -> None:
    """rax_decode_attention_noalloc: decode_attention with the library's static workspace."""
    _need(q.dim() == 3 and q.shape[2] == k_pool.shape[2] and k_pool.shape == v_pool.shape, "shapes")
    _need(o.shape == q.shape and o.is_contiguous() and o.is_cuda, "o like q")
    _need(q.dtype == k_pool.dtype == v_pool.dtype, "input dtypes agree")
    _need(all(t.is_contiguous() and t.is_cuda for t in (q, k_pool, v_pool)), "contiguous cuda")
    _cuda_i32(req_to_token, req_pool_idx, seq_len, shared_len)
    b = q.shape[0]
    _need(req_pool_idx.numel() == b and seq_len.numel() == b, "metadata shapes")
    d = q.shape[2]
    scale = float(sm_scale if sm_scale is not None else d ** -0.5)
    _check(lib().rax_decode_attention_noalloc(
        _dev(q), _dev(k_pool), _dev(v_pool), k_pool.shape[0], _dev(req_to_token), req_to_token.shape[1],
        req_to_token.shape[0], _dev(req_pool_idx), _dev(seq_len), _dev(shared_len), b, int(max_seq_len),
        q.shape[1], k_pool.shape[1], d, scale, _dtype_code(q), _dev(o), _dtype_code(o), _stream(stream, q)),
        "rax_decode_attention_noalloc")


def decode_attention_hinted(q, k_pool, v_pool, req_to_token, req_pool_idx, seq_len, max_seq_len: int, o,
                            seq_len_host, shared_len_host, workspace=None, shared_len=None, sm_scale=None,
                            stream=None) -> int:
    """rax_decode_attention_hinted: decode_attention with host copies of seq_len and
    shared_len sizing the launches. Returns the workspace bytes the layout needs; when
    `workspace` is smaller nothing runs (grow it and call again)."""
    _need(q.dim() == 3 and q.shape[2] == k_pool.shape[2] and k_pool.shape == v_pool.shape, "shapes")
    _need(o.shape == q.shape and o.is_contiguous() and o.is_cuda, "o like q")
    _need(q.dtype == k_pool.dtype == v_pool.dtype, "input dtypes agree")
    _need(all(t.is_contiguous() and t.is_cuda for t in (q, k_pool, v_pool)), "contiguous cuda")
    _cuda_i32(req_to_token, req_pool_idx, seq_len, shared_len)
    b = q.shape[0]
    _need(req_pool_idx.numel() == b and seq_len.numel() == b, "metadata shapes")
    sl, sh = _i32arr(seq_len_host), _i32arr(shared_len_host)
    _need(len(sl) == b and len(sh) == b, "host copies: [batch]")
    d = q.shape[2]
    scale = float(sm_scale if sm_scale is not None else d ** -0.5)
    ws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    need = _sz()
    st = lib().rax_decode_attention_hinted(
        _dev(q), _dev(k_pool), _dev(v_pool), k_pool.shape[0], _dev(req_to_token), req_to_token.shape[1],
        req_to_token.shape[0], _dev(req_pool_idx), _dev(seq_len), _dev(shared_len), b, int(max_seq_len),
        q.shape[1], k_pool.shape[1], d, scale, _dtype_code(q), _dev(o), _dtype_code(o), _dev(workspace), ws,
        _stream(stream, q), _ptr(sl), _ptr(sh), ctypes.byref(need))
    if st == EINVAL and need.value > ws:
        return int(need.value)
    _check(st, "rax_decode_attention_hinted")
    return int(need.value)


def device_errors(stream=None) -> int:
    m = _i32()
    _check(lib().rax_device_errors(_stream(stream), ctypes.byref(m)), "rax_device_errors")
    return int(m.value)


def qkv_project(x, w, h_q: int, h_kv: int, out_loc=None, k_pool=None, v_pool=None, q_out=None, k_ext=None,
                v_ext=None, stream=None):
    """rax_qkv_project: x [T, hidden] bf16, w [(h_q + 2 h_kv) d, hidden] bf16 (cuda,
    contiguous). Returns (q [T, h_q, d], k_ext [T, h_kv, d], v_ext [T, h_kv, d]); with
    out_loc (cuda int32 [T]) K and V also go to the pools at those slots."""
    import torch
    _need(x.dim() == 2 and w.dim() == 2 and x.shape[1] == w.shape[1], "x [T, hidden], w [n_out, hidden]")
    _need(x.is_cuda and w.is_cuda and x.is_contiguous() and w.is_contiguous()
          and x.dtype == w.dtype == torch.bfloat16, "x, w: contiguous cuda bf16")
    t, n_out = x.shape[0], w.shape[0]
    _need(n_out % (h_q + 2 * h_kv) == 0, "w rows: (h_q + 2 h_kv) * d")
    d = n_out // (h_q + 2 * h_kv)
    if q_out is None:
        q_out = torch.empty((t, h_q, d), dtype=x.dtype, device=x.device)
    if k_ext is None:
        k_ext = torch.empty((t, h_kv, d), dtype=x.dtype, device=x.device)
    if v_ext is None:
        v_ext = torch.empty((t, h_kv, d), dtype=x.dtype, device=x.device)
    for o, h in ((q_out, h_q), (k_ext, h_kv), (v_ext, h_kv)):
        _need(tuple(o.shape) == (t, h, d) and o.dtype == x.dtype and o.is_cuda and o.is_contiguous(),
              "outputs: contiguous cuda [T, heads, d] of x's dtype")
    slots = 0
    if out_loc is not None:
        _cuda_i32(out_loc)
        _need(out_loc.numel() == t and k_pool is not None and v_pool is not None
              and k_pool.shape == v_pool.shape and tuple(k_pool.shape[1:]) == (h_kv, d)
              and k_pool.dtype == x.dtype and k_pool.is_contiguous() and v_pool.is_contiguous(),
              "out_loc [T]; pools [slots, h_kv, d] of x's dtype")
        slots = k_pool.shape[0]
    _check(lib().rax_qkv_project(_dev(x), _dev(w), t, x.shape[1], h_q, h_kv, d, BF16, _dev(q_out), _dev(k_ext),
                                 _dev(v_ext), _dev(out_loc), _dev(k_pool), _dev(v_pool), slots,
                                 _stream(stream, x)), "rax_qkv_project")
    return q_out, k_ext, v_ext
