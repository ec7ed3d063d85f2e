"""Loads a generated workload into a library handle.

The host rows, committed frontiers, hot-cache warm sets, resident rows and
ring prefill drawn by ``workloads.gen`` are handed to the library through its
own set-up calls.  Argument marshalling only: nothing here resolves, places
or attends, and nothing here imports the oracle.  The benchmark and the tests
build their handles here; the tests give the same generated state to the
oracle.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .gen import (History, Workload, make_hist_len, make_history, make_hot_warm_set, make_resident_bitmaps,
                  make_step_inputs)


def lib_config(w: Workload, **kw) -> dict:
    """kv_hier_config fields of a workload (keyword overrides win)."""
    cfg = dict(n_req=w.n_req, n_groups=w.n_groups, n_arenas=w.n_arenas, hist_cap=w.hist_cap,
               n_prefix=w.n_prefix, prefix_len=w.prefix_len if w.n_prefix > 0 else 0,
               row_elems=w.row_elems, d_qk=w.d_qk, v_off=w.v_off, d_v=w.d_v, n_heads=w.n_heads,
               q_max=w.q_max, topk=w.topk, hot_slots=w.hot_slots, ring_window=w.ring_window,
               ring_page=w.ring_page, ring_block_only=0, n_chunks=0, resident_cap=0,
               softmax_scale=0.0, flags=0, fetch_cus=0, fetch_wgs=0, plan_share=w.plan_share)
    cfg.update(kw)
    return cfg


def resident_capacity(w: Workload, rho: float) -> int:
    """Resident-pool rows for a resident fraction rho (with a little slack)."""
    return int(w.n_req * w.hist_cap * min(1.0, rho + 0.05)) + 1024


def prefill_rows(hist: History, w: Workload, r: int, n_r: int):
    """The committed positions max(0, n_r - W + 1) .. n_r - 1 of request r (the
    ring's content below the frontier): (first position, rows)."""
    first = max(0, n_r - w.ring_window + 1)
    plen = w.prefix_len if w.n_prefix > 0 else 0
    rows = [hist.prefix[r % max(w.n_prefix, 1), s] if s < plen else hist.tails[r, s - plen]
            for s in range(first, n_r)]
    return first, (np.stack(rows) if rows else np.zeros((0, w.row_elems), np.uint16))


@dataclass
class Loaded:
    """A handle with a workload's generated state, and that state."""
    w: Workload
    lib: object
    hist_len: np.ndarray
    hists: List[History]
    warm_sets: List[Optional[list]] = field(default_factory=list)   # [g][r] = (rows, ages) or None
    res_bitmaps: List[Optional[np.ndarray]] = field(default_factory=list)


def load_library(w: Workload, *, warm: bool = True, rho: float = 0.0, block_only: bool = False,
                 lib_kw: Optional[dict] = None, histories: Optional[List[History]] = None,
                 step_for_warm: int = 0, hist_len: Optional[np.ndarray] = None) -> Loaded:
    """Creates a KVHier handle for ``w`` and loads the generated state into it."""
    from hierarchical_sparse_kv_verify_amd import KVHier
    hl = make_hist_len(w) if hist_len is None else np.asarray(hist_len, dtype=np.int32)
    hists = histories if histories is not None else [make_history(w, g, hl) for g in range(w.n_groups)]
    kw = dict(ring_block_only=1 if block_only else 0)
    if rho > 0:
        kw["resident_cap"] = resident_capacity(w, rho)
    kw.update(lib_kw or {})
    lib = KVHier(**lib_config(w, **kw))
    for g in range(w.n_groups):
        for p in range(w.n_prefix):
            lib.host_rows(g, 0, p)[:] = hists[g].prefix[p]
        for r in range(w.n_req):
            lib.host_rows(g, 1, r)[:] = hists[g].tails[r]
    lib.set_hist_len(hl)
    out = Loaded(w=w, lib=lib, hist_len=hl, hists=hists)
    for g in range(w.n_groups):
        ws = None
        if warm:
            si = make_step_inputs(w, g, step_for_warm, hl)
            ws = make_hot_warm_set(w, g, hl, si)
            for r, hs in enumerate(ws):
                lib.set_hot(g, r, hs[0], hs[1])
        out.warm_sets.append(ws)
        bm = None
        if rho > 0:
            bm = make_resident_bitmaps(w, g, hl, rho)
            for r in range(w.n_req):
                lib.set_resident(g, r, bm[r])
        out.res_bitmaps.append(bm)
        if w.ring_prefill:
            for r in range(w.n_req):
                first, rows = prefill_rows(hists[g], w, r, int(hl[r]))
                lib.ring_load(g, r, first, rows)
    return out


def device_inputs(si) -> dict:
    """The step inputs of ``make_step_inputs`` as device tensors (bf16 as int16
    bit patterns): queries, topk, causal positions, new ring rows."""
    import torch
    dev = torch.device("cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return dict(queries=t(si.queries.view(np.int16)), topk=t(si.topk), causal=t(si.causal_pos),
                ring=t(si.block_rows.view(np.int16)))
