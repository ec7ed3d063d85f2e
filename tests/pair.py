"""Builds the library handle and the oracle from the same seeded workload.

Both sides receive identical inputs from ``workloads``; they share nothing
else.  The library side is ``workloads.load.load_library`` (also what the
benchmark uses); the oracle is given the same generated state here.  Used by
the GPU parity tests and the smoke check.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from workloads import History, Workload, f32_from_bf16_bits
from workloads.load import device_inputs, lib_config, load_library, prefill_rows  # noqa: F401

TOL_ABS, TOL_REL = 2e-2, 1e-2


@dataclass
class Pair:
    w: Workload
    lib: object
    orc: Optional["oracle.HierOracle"]
    hist_len: np.ndarray
    lib_hists: List[History] = field(default_factory=list)


def build_pair(w: Workload, *, warm: bool = True, rho: float = 0.0, with_oracle: bool = True,
               oracle_requests=None, block_only: bool = False, lib_kw: Optional[dict] = None,
               histories: Optional[List[History]] = None, step_for_warm: int = 0,
               hist_len: Optional[np.ndarray] = None) -> Pair:
    """Library handle (and oracle) with host rows, frontier, hot-cache warm set,
    resident map and ring prefill applied identically."""
    ld = load_library(w, warm=warm, rho=rho, block_only=block_only, lib_kw=lib_kw, histories=histories,
                      step_for_warm=step_for_warm, hist_len=hist_len)
    hl, hists = ld.hist_len, ld.hists
    orc = None
    if with_oracle:
        import oracle   # only here: building the library handle never imports it
        from tests.oracle_helpers import oracle_config
        ohists = [History(prefix=h.prefix, tails=h.tails.copy(), hist_len=h.hist_len.copy()) for h in hists]
        orc = oracle.HierOracle(oracle_config(w, ring_block_only=block_only), ohists, hl,
                                requests=oracle_requests)
        oreq = set(orc.requests)
        for g in range(w.n_groups):
            if ld.warm_sets[g] is not None:
                for r, hs in enumerate(ld.warm_sets[g]):
                    orc.set_hot(g, r, hs[0], hs[1])
            if ld.res_bitmaps[g] is not None:
                for r in range(w.n_req):
                    orc.set_resident(g, r, ld.res_bitmaps[g][r])
            if w.ring_prefill:
                for r in range(w.n_req):
                    if r in oreq:
                        first, rows = prefill_rows(hists[g], w, r, int(hl[r]))
                        orc.ring_load(g, r, first, rows)
    return Pair(w=w, lib=ld.lib, orc=orc, hist_len=hl, lib_hists=hists)


def to_device(si):
    return device_inputs(si)


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
