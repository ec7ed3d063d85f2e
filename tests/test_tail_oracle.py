"""Pins of the oracle's tail resolution and host backup ("Adaptive DHiSparse"
Figure 2 callout 1, §3.1 "mutable tail", Figure 3 callout 4, eq. 7, eq. 10).

A selected history row that the ring still holds resolves there directly;
the ring holds a committed position until a later block's rows take its slot
(eq. 10), which bounds the tail from below by n_r + K_max - R_d.  Checked by
brute force over the ring addresses, and over random rounds with commits
whose selections favour recently generated rows: every tail location holds
the selected row, rows committed one round earlier are never fetched, rows
below the bound are never given a ring location.
"""
import numpy as np
import pytest

import oracle
from oracle import CLS_TAIL, HierOracle
from tests.oracle_helpers import oracle_config, ring_prefill_rows
from tests.test_oracle_pins import _tiny_case
from workloads import make_accepted, make_history, make_step_inputs


@pytest.mark.parametrize("window,page,k_max", [(6, 4, 4), (8, 4, 4), (128, 64, 8), (2048, 64, 8), (5, 1, 3)])
def test_tail_bound_is_the_last_position_the_block_cannot_overwrite(window, page, k_max):
    """Eq. (10) by brute force: while a block of K_max rows is written at
    n .. n+K_max-1, the positions n+K_max-R_d .. n-1 keep their slots and the
    position just below that range shares a slot with the block."""
    r_d = oracle.ring_rows(window, page, k_max)
    for n in (r_d, r_d + 1, 3 * r_d + 7):
        block = {oracle.ring_addr(0, p, r_d) for p in range(n, n + k_max)}
        lo = n + k_max - r_d
        assert all(oracle.ring_addr(0, u, r_d) not in block for u in range(lo, n))
        assert oracle.ring_addr(0, lo - 1, r_d) in block


def _rounds(n_rounds=8, seed=3):
    w = _tiny_case(n_req=3, ring_window=8, ring_page=4, q_max=4, topk=24, hot_slots=16, var_k=True,
                   recent_frac=0.3, recent_span=24, pad_frac=0.0, invalid_frac=0.0)
    hist = make_history(w, 0)
    hl = hist.hist_len.copy()
    cfg = oracle_config(w)
    o = HierOracle(cfg, [hist], hl)
    for r in range(w.n_req):
        first, rows = ring_prefill_rows(hist, r, int(hl[r]), w.ring_window, cfg.plen, max(w.n_prefix, 1))
        o.ring_load(0, r, first, rows)
    return w, hist, o


def test_tail_rows_resolve_from_the_ring_over_rounds():
    w, hist, o = _rounds()
    r_d = o.r_d
    assert r_d == 16
    n = [int(x) for x in hist.hist_len]
    prev_commit = {r: set() for r in range(w.n_req)}
    seen_tail = seen_recent_fetch = 0
    for step in range(8):
        si = make_step_inputs(w, 0, step, np.array(n, np.int32))
        res = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
        for r in range(w.n_req):
            rr = res.req[r]
            lo = max(o.st[0][r].ring_lo, n[r] + w.q_max - r_d)
            cls = dict(zip(rr.union, rr.cls))
            for u, c in cls.items():
                assert (c == CLS_TAIL) == (u >= lo)
                if u < lo and u >= n[r] - w.recent_span:
                    seen_recent_fetch += c == oracle.CLS_MISS
            assert not (set(rr.miss) & prev_commit[r])           # committed last round: never fetched
            assert all(cls[u] == CLS_TAIL for u in prev_commit[r] if u in cls)
            for j in range(w.q_max):
                for i in range(w.topk):
                    code = int(rr.loc[j, i])
                    if code < 0 or code >> 29 != oracle.RING:
                        continue
                    e = int(si.topk[r, j, i])
                    idx = code & ((1 << 29) - 1)
                    assert idx == r * r_d + e % r_d
                    # the ring row there is the selected history row (eq. 12)
                    assert np.array_equal(o.st[0][r].ring[e], hist.row(r, e))
                    seen_tail += 1
        acc = make_accepted(w, step, si.k_active)
        o.commit(acc)
        for r in range(w.n_req):
            prev_commit[r] = set(range(n[r], n[r] + 1 + int(acc[r])))
            n[r] += 1 + int(acc[r])
    assert seen_tail >= 20 and seen_recent_fetch >= 1


def test_tail_rows_are_never_cached():
    w, hist, o = _rounds()
    n = [int(x) for x in hist.hist_len]
    for step in range(4):
        si = make_step_inputs(w, 0, step, np.array(n, np.int32))
        res = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
        for r in range(w.n_req):
            rr = res.req[r]
            tail = {u for u, c in zip(rr.union, rr.cls) if c == CLS_TAIL}
            assert not (tail & set(rr.miss))
            rows, _ = o.slot_table(0, r)
            assert not (tail & set(int(x) for x in rows))      # not inserted in the hot cache
            assert rr.counts["union_tail"] == len(tail)
        acc = make_accepted(w, step, si.k_active)
        o.commit(acc)
        for r in range(w.n_req):
            n[r] += 1 + int(acc[r])
