"""Builds the library handle and the oracle from the same seeded workload.

Both sides receive identical inputs from ``workloads``; they share nothing
else.  Used by the GPU parity tests and the smoke check.  The benchmark builds
its handle here with ``with_oracle=False``, which never imports the oracle;
only its CPU-baseline leg runs the oracle.
"""
from __future__ import annotations

import copy
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from workloads import (History, Workload, f32_from_bf16_bits, make_history, make_hot_warm_set,
                       make_resident_bitmaps, make_step_inputs)
from workloads.gen import make_hist_len

TOL_ABS, TOL_REL = 2e-2, 1e-2


def lib_config(w: Workload, **kw) -> dict:
    cfg = dict(n_req=w.n_req, n_groups=w.n_groups, n_arenas=w.n_arenas, hist_cap=w.hist_cap,
               n_prefix=w.n_prefix, prefix_len=w.prefix_len if w.n_prefix > 0 else 0,
               row_elems=w.row_elems, d_qk=w.d_qk, v_off=w.v_off, d_v=w.d_v, n_heads=w.n_heads,
               q_max=w.q_max, topk=w.topk, hot_slots=w.hot_slots, ring_window=w.ring_window,
               ring_page=w.ring_page, ring_block_only=0, n_chunks=0, resident_cap=0,
               softmax_scale=0.0, flags=0, fetch_cus=0, fetch_wgs=0, plan_share=w.plan_share)
    cfg.update(kw)
    return cfg


def oracle_config(w: Workload, block_only: bool = False) -> "oracle.OracleConfig":
    import oracle
    return oracle.OracleConfig(
        n_req=w.n_req, n_groups=w.n_groups, hist_cap=w.hist_cap, n_prefix=w.n_prefix,
        prefix_len=w.prefix_len, row_elems=w.row_elems, d_qk=w.d_qk, v_off=w.v_off, d_v=w.d_v,
        n_heads=w.n_heads, q_max=w.q_max, topk=w.topk, hot_slots=w.hot_slots,
        ring_window=w.ring_window, ring_page=w.ring_page, ring_block_only=block_only)


def prefill_rows(hist: History, w: Workload, r: int, n_r: int):
    first = max(0, n_r - w.ring_window + 1)
    plen = w.prefix_len if w.n_prefix > 0 else 0
    rows = [hist.prefix[r % max(w.n_prefix, 1), s] if s < plen else hist.tails[r, s - plen]
            for s in range(first, n_r)]
    return first, (np.stack(rows) if rows else np.zeros((0, w.row_elems), np.uint16))


@dataclass
class Pair:
    w: Workload
    lib: object
    orc: Optional["oracle.HierOracle"]
    hist_len: np.ndarray
    lib_hists: List[History] = field(default_factory=list)


def build_pair(w: Workload, *, warm: bool = True, rho: float = 0.0, with_oracle: bool = True,
               oracle_requests=None, block_only: bool = False, lib_kw: Optional[dict] = None,
               histories: Optional[List[History]] = None, step_for_warm: int = 0) -> Pair:
    """Library handle (and oracle) with host rows, frontier, hot-cache warm set,
    resident map and ring prefill applied identically."""
    from hierarchical_sparse_kv_verify_amd import KVHier
    hl = make_hist_len(w)
    hists = histories if histories is not None else [make_history(w, g, hl) for g in range(w.n_groups)]
    kw = dict(ring_block_only=1 if block_only else 0)
    if rho > 0:
        kw["resident_cap"] = int(w.n_req * w.hist_cap * min(1.0, rho + 0.05)) + 1024
    kw.update(lib_kw or {})
    lib = KVHier(**lib_config(w, **kw))
    for g in range(w.n_groups):
        for p in range(w.n_prefix):
            lib.host_rows(g, 0, p)[:] = hists[g].prefix[p]
        for r in range(w.n_req):
            lib.host_rows(g, 1, r)[:] = hists[g].tails[r]
    lib.set_hist_len(hl)
    orc = None
    if with_oracle:
        import oracle   # only here: the benchmark's timed path builds its handle without it
        ohists = [History(prefix=h.prefix, tails=h.tails.copy(), hist_len=h.hist_len.copy()) for h in hists]
        orc = oracle.HierOracle(oracle_config(w, block_only), ohists, hl, requests=oracle_requests)
    oreq = set(orc.requests) if orc else set()
    for g in range(w.n_groups):
        if warm:
            si = make_step_inputs(w, g, step_for_warm, hl)
            for r, hs in enumerate(make_hot_warm_set(w, g, hl, si)):
                lib.set_hot(g, r, hs[0], hs[1])
                if orc is not None:
                    orc.set_hot(g, r, hs[0], hs[1])
        if rho > 0:
            bm = make_resident_bitmaps(w, g, hl, rho)
            for r in range(w.n_req):
                lib.set_resident(g, r, bm[r])
                if orc is not None:
                    orc.set_resident(g, r, bm[r])
        if w.ring_prefill:
            for r in range(w.n_req):
                first, rows = prefill_rows(hists[g], w, r, int(hl[r]))
                lib.ring_load(g, r, first, rows)
                if r in oreq:
                    orc.ring_load(g, r, first, rows)
    return Pair(w=w, lib=lib, orc=orc, hist_len=hl, lib_hists=hists)


def to_device(si):
    import torch
    dev = torch.device("cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return dict(queries=t(si.queries.view(np.int16)), topk=t(si.topk), causal=t(si.causal_pos),
                ring=t(si.block_rows.view(np.int16)))


def run_lib_step(pair: Pair, g: int, si):
    import torch
    w = pair.w
    d = to_device(si)
    out = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
    pair.lib.verify_step(g, d["queries"], d["topk"], d["causal"], d["ring"], out)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def assert_close(gpu_bits: np.ndarray, ref: np.ndarray, what: str = ""):
    got = f32_from_bf16_bits(gpu_bits).astype(np.float64)
    err = np.abs(got - ref)
    lim = TOL_ABS + TOL_REL * np.abs(ref)
    bad = ~(err <= lim)          # NaN fails too
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d outputs outside 2e-2 + 1e-2*|ref|; first at %s: got %r ref %r"
                             % (what, int(bad.sum()), bad.size, tuple(i), got[tuple(i)], ref[tuple(i)]))
