"""ctypes binding of libkvhier.so (include/kv_hier.h).

Argument marshalling only: every step of the verification path runs in the
library's HIP kernels.  Device arguments are torch CUDA tensors (or raw
integer device addresses); the stream defaults to torch's current stream.
There is no fallback: if the library cannot be loaded, every entry point
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVHIER_LIBRARY names another build of the same sources (the host-sanitizer
# build that the CPU sanitizer run loads); by default the in-tree library
LIB_PATH = os.environ.get("KVHIER_LIBRARY") or os.path.join(_HERE, "libkvhier.so")

KV_OK, KV_EINVAL, KV_ENOMEM, KV_EHIP, KV_ESTATE, KV_EUNSUPPORTED, KV_EWAIT = 0, -1, -2, -3, -4, -5, -6
KV_TIER_HOT, KV_TIER_STAGED, KV_TIER_RESIDENT, KV_TIER_RING = 0, 1, 2, 3
KV_FLAG_TIMING, KV_FLAG_POISON, KV_FLAG_TIMING_ATTN, KV_FLAG_SERIAL, KV_FLAG_SYNC_BACKUP = 1, 2, 4, 8, 16
KV_FLAG_TEST_FAIL_ATTN = 32
TIER_SHIFT = 29

_ERRNAMES = {KV_EINVAL: "KV_EINVAL", KV_ENOMEM: "KV_ENOMEM", KV_EHIP: "KV_EHIP",
             KV_ESTATE: "KV_ESTATE", KV_EUNSUPPORTED: "KV_EUNSUPPORTED", KV_EWAIT: "KV_EWAIT"}

EXPORTED = [
    "kv_hier_create", "kv_hier_destroy", "kv_hier_last_error", "kv_hier_info_get",
    "kv_hier_host_rows", "kv_hier_set_hist_len", "kv_hier_hist_len", "kv_hier_set_hot",
    "kv_hier_set_resident", "kv_hier_clear_resident", "kv_hier_ring_load",
    "kv_hier_verify_step", "kv_hier_commit", "kv_hier_stats", "kv_hier_reset_stats",
    "kv_hier_last_lists", "kv_hier_slot_table", "kv_hier_read_rows", "kv_hier_sync",
    "kv_hier_set_flags", "kv_hier_cache_snapshot", "kv_hier_opt_admit", "kv_hier_opt_complete",
    "kv_hier_opt_populate", "kv_hier_opt_publish", "kv_hier_opt_query", "kv_hier_verify_reuse",
    "kv_hier_set_compression", "kv_hier_commit_src", "kv_hier_verify_step_static",
]


class KVHierError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (%d): %s" % (_ERRNAMES.get(code, "KV_E?"), code, msg))
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_req", "n_groups", "n_arenas", "hist_cap", "n_prefix", "prefix_len", "row_elems",
        "d_qk", "v_off", "d_v", "n_heads", "q_max", "topk", "hot_slots", "ring_window",
        "ring_page", "ring_block_only", "n_chunks")] + [
        ("resident_cap", ctypes.c_int64), ("softmax_scale", ctypes.c_float), ("flags", ctypes.c_int32),
        ("fetch_cus", ctypes.c_int32), ("fetch_wgs", ctypes.c_int32), ("plan_share", ctypes.c_int32),
        ("opt_page_rows", ctypes.c_int32), ("opt_reserve", ctypes.c_int32)]


COUNTER_FIELDS = ("calls", "active_requests", "active_queries", "selections", "pads", "invalid",
                  "union_rows", "union_resident", "union_hot", "union_miss", "fetched_bytes",
                  "promoted", "overflow", "sel_resident", "sel_hot", "sel_miss")
TIMING_FIELDS = ("ms_ring", "ms_plan", "ms_gather", "ms_attn", "ms_combine", "ms_promote", "ms_victims")
TIMING_COUNTS = ("n_ring", "n_plan", "n_gather", "n_attn", "n_combine", "n_promote", "n_victims")


TAIL_FIELDS = ("union_tail", "sel_tail")


class Counters(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_int64) for n in COUNTER_FIELDS] +
                [(n, ctypes.c_double) for n in TIMING_FIELDS] +
                [(n, ctypes.c_int64) for n in TIMING_COUNTS] +
                [(n, ctypes.c_int64) for n in TAIL_FIELDS] +
                [("ms_order", ctypes.c_double), ("n_order", ctypes.c_int64)])

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_i32p = ctypes.POINTER(ctypes.c_int32)


class Lists(ctypes.Structure):
    _fields_ = [("union_rows", _i32p), ("union_loc", _i32p), ("miss_rows", _i32p),
                ("victims", _i32p), ("loc", _i32p), ("n_union", ctypes.c_int32),
                ("n_miss", ctypes.c_int32), ("n_promote", ctypes.c_int32), ("n_active", ctypes.c_int32)]


class Info(ctypes.Structure):
    _fields_ = [("ring_rows", ctypes.c_int32), ("n_chunks", ctypes.c_int32)] + \
               [(n, ctypes.c_int64) for n in ("bytes_hot", "bytes_staging", "bytes_ring", "bytes_maps",
                                              "bytes_resident", "bytes_host")] + \
               [("attn_splits", ctypes.c_int32), ("attn_head_groups", ctypes.c_int32),
                ("plan_rows_per_pass", ctypes.c_int32), ("attn_reuse_head_groups", ctypes.c_int32),
                ("attn_row_order", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


OPT_INFO_FIELDS = ("admitted", "required_pages", "held_pages", "ready_pages", "pending_pages", "free_pages",
                   "eligible_pages", "pages_populated", "pages_published", "pages_reclaimed",
                   "requests_reclaimed", "admissions_waited", "bytes_populated")


class OptInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("pool_pages", "page_rows", "reserve", "cursor")] + \
               [(n, ctypes.c_int64) for n in OPT_INFO_FIELDS]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads libkvhier.so (built in-tree by ``build.py``); raises if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libkvhier.so not found at %s: build it with "
                           "`python -m hierarchical_sparse_kv_verify_amd.build`" % p)
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7).
    # Loading torch first makes the library bind to that runtime, so torch's
    # allocations and stream handles belong to the runtime the library uses;
    # loading the library first would put a second runtime in the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    sig = {
        "kv_hier_create": ([ctypes.POINTER(Config), ctypes.POINTER(vp)], i32),
        "kv_hier_destroy": ([vp], None),
        "kv_hier_last_error": ([vp], ctypes.c_char_p),
        "kv_hier_info_get": ([vp, ctypes.POINTER(Info)], i32),
        "kv_hier_host_rows": ([vp, i32, i32, i32, ctypes.POINTER(vp), ctypes.POINTER(i64)], i32),
        "kv_hier_set_hist_len": ([vp, vp], i32),
        "kv_hier_hist_len": ([vp, vp], i32),
        "kv_hier_set_hot": ([vp, i32, i32, vp, vp, i32], i32),
        "kv_hier_set_resident": ([vp, i32, i32, vp], i32),
        "kv_hier_clear_resident": ([vp, i32], i32),
        "kv_hier_ring_load": ([vp, i32, i32, ctypes.c_int32, vp, i32], i32),
        "kv_hier_verify_step": ([vp, i32, vp, vp, vp, vp, vp, vp], i32),
        "kv_hier_verify_step_static": ([vp, i32, vp, vp, vp, vp, vp, vp], i32),
        "kv_hier_verify_reuse": ([vp, i32, vp, vp, vp, vp], i32),
        "kv_hier_commit": ([vp, vp, vp], i32),
        "kv_hier_commit_src": ([vp, vp, vp, vp], i32),
        "kv_hier_set_compression": ([vp, i32, ctypes.c_int32], i32),
        "kv_hier_stats": ([vp, i32, ctypes.POINTER(Counters), ctypes.POINTER(Counters)], i32),
        "kv_hier_reset_stats": ([vp], i32),
        "kv_hier_last_lists": ([vp, i32, i32, ctypes.POINTER(Lists)], i32),
        "kv_hier_slot_table": ([vp, i32, i32, vp, vp], i32),
        "kv_hier_read_rows": ([vp, i32, vp, i32, vp], i32),
        "kv_hier_sync": ([vp], i32),
        "kv_hier_set_flags": ([vp, ctypes.c_int32], i32),
        "kv_hier_cache_snapshot": ([vp, i32, i32], i32),
        "kv_hier_opt_admit": ([vp, i32, ctypes.c_int32, vp, i32, vp], i32),
        "kv_hier_opt_complete": ([vp, i32], i32),
        "kv_hier_opt_populate": ([vp, ctypes.c_int32, vp], i32),
        "kv_hier_opt_publish": ([vp, i32], i32),
        "kv_hier_opt_query": ([vp, i32, ctypes.c_int32, vp, vp, ctypes.POINTER(OptInfo)], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = L
    return L


def _dev_ptr(x) -> int:
    """Device address of a torch CUDA tensor (contiguous) or a raw int."""
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise TypeError("expected a CUDA (HIP) tensor for a device argument")
    if not x.is_contiguous():
        raise ValueError("device tensors must be contiguous")
    return int(x.data_ptr())


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


class KVHier:
    """One handle of the library (see include/kv_hier.h for every call)."""

    def __init__(self, **cfg):
        self._lib = load_library()
        c = Config()
        defaults = dict(n_arenas=1, n_prefix=0, prefix_len=0, ring_block_only=0, n_chunks=0,
                        resident_cap=0, softmax_scale=0.0, flags=0, fetch_cus=0, fetch_wgs=0, plan_share=0,
                        opt_page_rows=0, opt_reserve=0)
        defaults.update(cfg)
        for name, _ in Config._fields_:
            if name not in defaults:
                raise TypeError("missing config field %s" % name)
            setattr(c, name, defaults[name])
        self.cfg = {n: getattr(c, n) for n, _ in Config._fields_}
        h = ctypes.c_void_p()
        rc = self._lib.kv_hier_create(ctypes.byref(c), ctypes.byref(h))
        if rc != KV_OK:
            msg = self._lib.kv_hier_last_error(None)
            raise KVHierError(rc, "kv_hier_create: " + (msg.decode() if msg else ""))
        self._h = h
        self.info = self._info()

    # -------------------------------------------------------------- plumbing
    def _check(self, rc):
        if rc != KV_OK:
            msg = self._lib.kv_hier_last_error(self._h)
            raise KVHierError(rc, msg.decode() if msg else "")

    def close(self):
        if getattr(self, "_h", None):
            self._lib.kv_hier_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _info(self):
        inf = Info()
        self._check(self._lib.kv_hier_info_get(self._h, ctypes.byref(inf)))
        return inf.as_dict()

    # -------------------------------------------------------------- set-up
    def host_rows(self, g: int, kind: int, index: int) -> np.ndarray:
        """numpy view (uint16 [rows, row_elems]) of pinned host backing."""
        p = ctypes.c_void_p()
        n = ctypes.c_int64()
        self._check(self._lib.kv_hier_host_rows(self._h, g, kind, index, ctypes.byref(p), ctypes.byref(n)))
        re = self.cfg["row_elems"]
        if n.value == 0 or not p.value:
            return np.zeros((0, re), dtype=np.uint16)
        buf = (ctypes.c_uint16 * (n.value * re)).from_address(p.value)
        return np.frombuffer(buf, dtype=np.uint16).reshape(n.value, re)

    def set_hist_len(self, hist_len):
        a = _i32(hist_len)
        self._check(self._lib.kv_hier_set_hist_len(self._h, a.ctypes.data))

    def hist_len(self) -> np.ndarray:
        a = np.zeros(self.cfg["n_req"], dtype=np.int32)
        self._check(self._lib.kv_hier_hist_len(self._h, a.ctypes.data))
        return a

    def set_hot(self, g: int, r: int, rows, last_used):
        rows, lu = _i32(rows), _i32(last_used)
        self._check(self._lib.kv_hier_set_hot(self._h, g, r, rows.ctypes.data, lu.ctypes.data, rows.size))

    def set_resident(self, g: int, r: int, bitmap):
        bm = np.ascontiguousarray(bitmap, dtype=np.uint8)
        if bm.size < self.cfg["hist_cap"]:
            raise ValueError("resident bitmap needs hist_cap entries")
        self._check(self._lib.kv_hier_set_resident(self._h, g, r, bm.ctypes.data))

    def clear_resident(self, g: int):
        self._check(self._lib.kv_hier_clear_resident(self._h, g))

    def ring_load(self, g: int, r: int, first_pos: int, rows):
        rows = np.ascontiguousarray(rows, dtype=np.uint16)
        n = rows.shape[0] if rows.ndim == 2 else 0
        self._check(self._lib.kv_hier_ring_load(self._h, g, r, int(first_pos),
                                                rows.ctypes.data if n else None, n))

    # -------------------------------------------------------------- the step
    def verify_step(self, g: int, queries, topk_idx, causal_pos, ring_rows, out, stream=None):
        """ring_rows None: a Reindex consumer of a shared source (the ring already
        holds this step's rows); topk_idx None only for a follower layer."""
        self._check(self._lib.kv_hier_verify_step(
            self._h, g, _dev_ptr(queries), None if topk_idx is None else _dev_ptr(topk_idx),
            _dev_ptr(causal_pos), None if ring_rows is None else _dev_ptr(ring_rows), _dev_ptr(out),
            _stream_handle(stream)))

    def verify_step_static(self, g: int, queries, topk_idx, causal_pos, ring_rows, out, stream=None):
        """kv_hier_verify_step_static: the same step, allocating nothing during
        the call (split-key partials in the library's static device array)."""
        self._check(self._lib.kv_hier_verify_step_static(
            self._h, g, _dev_ptr(queries), None if topk_idx is None else _dev_ptr(topk_idx),
            _dev_ptr(causal_pos), None if ring_rows is None else _dev_ptr(ring_rows), _dev_ptr(out),
            _stream_handle(stream)))

    def verify_reuse(self, g: int, queries, causal_pos, out, stream=None):
        """A Reuse consumer: new queries over the latest selection of source g."""
        self._check(self._lib.kv_hier_verify_reuse(self._h, g, _dev_ptr(queries), _dev_ptr(causal_pos),
                                                   _dev_ptr(out), _stream_handle(stream)))

    def commit(self, accepted, stream=None, src_rows=None):
        """src_rows: per group a device tensor of completed stored rows (compressed
        sources) or None."""
        a = _i32(accepted)
        if src_rows is None:
            self._check(self._lib.kv_hier_commit(self._h, a.ctypes.data, _stream_handle(stream)))
            return
        ptrs = (ctypes.c_void_p * len(src_rows))(*[None if x is None else _dev_ptr(x) for x in src_rows])
        self._check(self._lib.kv_hier_commit_src(self._h, a.ctypes.data, ptrs, _stream_handle(stream)))

    def set_compression(self, g: int, m: int):
        self._check(self._lib.kv_hier_set_compression(self._h, g, int(m)))

    # -------------------------------------------------------------- read-back
    def stats(self, g: int):
        cum, last = Counters(), Counters()
        self._check(self._lib.kv_hier_stats(self._h, g, ctypes.byref(cum), ctypes.byref(last)))
        return cum.as_dict(), last.as_dict()

    def reset_stats(self):
        self._check(self._lib.kv_hier_reset_stats(self._h))

    def last_lists(self, g: int, r: int) -> dict:
        qk = self.cfg["q_max"] * self.cfg["topk"]
        bufs = {n: np.zeros(qk, dtype=np.int32) for n in ("union_rows", "union_loc", "miss_rows", "victims", "loc")}
        ls = Lists()
        for n, a in bufs.items():
            setattr(ls, n, a.ctypes.data_as(_i32p))
        self._check(self._lib.kv_hier_last_lists(self._h, g, r, ctypes.byref(ls)))
        return dict(union_rows=bufs["union_rows"][: ls.n_union].copy(),
                    union_loc=bufs["union_loc"][: ls.n_union].copy(),
                    miss_rows=bufs["miss_rows"][: ls.n_miss].copy(),
                    victims=bufs["victims"][: ls.n_promote].copy(),
                    loc=bufs["loc"].reshape(self.cfg["q_max"], self.cfg["topk"]).copy(),
                    n_union=ls.n_union, n_miss=ls.n_miss, n_promote=ls.n_promote, n_active=ls.n_active)

    def slot_table(self, g: int, r: int):
        B = self.cfg["hot_slots"]
        rows, lu = np.zeros(B, np.int32), np.zeros(B, np.int32)
        self._check(self._lib.kv_hier_slot_table(self._h, g, r, rows.ctypes.data, lu.ctypes.data))
        return rows, lu

    def read_rows(self, g: int, locs) -> np.ndarray:
        locs = _i32(locs).ravel()
        out = np.zeros((locs.size, self.cfg["row_elems"]), dtype=np.uint16)
        self._check(self._lib.kv_hier_read_rows(self._h, g, locs.ctypes.data if locs.size else None,
                                                locs.size, out.ctypes.data if locs.size else None))
        return out

    def sync(self):
        self._check(self._lib.kv_hier_sync(self._h))

    def set_flags(self, flags: int):
        self._check(self._lib.kv_hier_set_flags(self._h, int(flags)))
        self.cfg["flags"] = int(flags)

    def save_cache(self, g: int):
        self._check(self._lib.kv_hier_cache_snapshot(self._h, g, 0))

    def restore_cache(self, g: int):
        self._check(self._lib.kv_hier_cache_snapshot(self._h, g, 1))

    # -------------------------------------------------------------- dynamic optional residency
    def opt_admit(self, r: int, required_pages: int, order=()):
        """Returns the number of reclaimed requests, or None when the
        admission has to wait (KV_EWAIT)."""
        o = _i32(list(order))
        q = ctypes.c_int32(0)
        rc = self._lib.kv_hier_opt_admit(self._h, r, int(required_pages), o.ctypes.data if o.size else None,
                                         o.size, ctypes.byref(q))
        if rc == KV_EWAIT:
            return None
        self._check(rc)
        return q.value

    def opt_complete(self, r: int):
        self._check(self._lib.kv_hier_opt_complete(self._h, r))

    def opt_populate(self, max_pages: int) -> int:
        n = ctypes.c_int32(0)
        self._check(self._lib.kv_hier_opt_populate(self._h, int(max_pages), ctypes.byref(n)))
        return n.value

    def opt_publish(self, wait: bool = False):
        self._check(self._lib.kv_hier_opt_publish(self._h, 1 if wait else 0))

    def opt_info(self) -> dict:
        inf = OptInfo()
        self._check(self._lib.kv_hier_opt_query(self._h, -1, 0, None, None, ctypes.byref(inf)))
        return inf.as_dict()

    def opt_pages(self, r: int, n_pages: int):
        """Pool page held for each page index of request r (-1 none) and its ready flag."""
        held = np.zeros(n_pages, np.int32)
        ready = np.zeros(n_pages, np.uint8)
        self._check(self._lib.kv_hier_opt_query(self._h, r, n_pages, held.ctypes.data, ready.ctypes.data, None))
        return held, ready


def loc_code(tier: int, index: int) -> int:
    return (tier << TIER_SHIFT) | index
