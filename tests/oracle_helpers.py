"""Glue between the seeded workloads and the oracle, for tests only."""
import numpy as np

import oracle
from workloads import Workload


def oracle_config(w: Workload, **kw) -> "oracle.OracleConfig":
    base = dict(n_req=w.n_req, n_groups=w.n_groups, hist_cap=w.hist_cap, n_prefix=w.n_prefix,
                prefix_len=w.prefix_len, row_elems=w.row_elems, d_qk=w.d_qk, v_off=w.v_off,
                d_v=w.d_v, n_heads=w.n_heads, q_max=w.q_max, topk=w.topk,
                hot_slots=w.hot_slots, ring_window=w.ring_window, ring_page=w.ring_page)
    base.update(kw)
    return oracle.OracleConfig(**base)


def ring_prefill_rows(hist, r: int, n_r: int, window: int, plen: int, n_prefix: int):
    """Committed positions max(0, n_r-W+1) .. n_r-1, taken from the host rows."""
    first = max(0, n_r - window + 1)
    rows = []
    for s in range(first, n_r):
        if s < plen:
            rows.append(hist.prefix[r % n_prefix, s])
        else:
            rows.append(hist.tails[r, s - plen])
    return first, (np.stack(rows) if rows else np.zeros((0, hist.tails.shape[2]), np.uint16))
