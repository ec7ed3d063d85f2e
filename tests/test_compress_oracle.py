"""Pins of the oracle's compressed sources ("Adaptive DHiSparse" §3.3 eq. 8
and the text around it): a stored row packs m consecutive positions; only
complete rows are history; a commit completes the rows eq. (8) names.

Eq. (8) is checked by brute force over positions; the compressed step's
attention against the dense masked formulation over the stored rows plus the
position ring; commits over rounds against the test's own record of which
rows exist.
"""
import numpy as np
import pytest

import oracle
from oracle import HierOracle
from tests.oracle_helpers import oracle_config, ring_prefill_rows
from tests.test_oracle_pins import _dense_reference, _tiny_case
from workloads import (bf16_bits_from_f32, f32_from_bf16_bits, make_accepted, make_history, make_source_rows,
                       make_step_inputs)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 7])
def test_eq8_completed_rows_by_brute_force(m):
    rng = np.random.default_rng(m)
    for _ in range(200):
        n = int(rng.integers(0, 60))
        n2 = n + int(rng.integers(1, 9))
        # row s is complete once all of its positions s*m .. s*m+m-1 are below the frontier
        done = lambda front: {s for s in range(0, 80) if s * m + m - 1 < front}
        want = sorted(done(n2) - done(n))
        assert list(oracle.completed_rows(n, n2, m)) == want


def _compressed_case(m=4, **kw):
    w = _tiny_case(n_req=3, compress=m, compress_groups=(0,), pad_frac=0.05, invalid_frac=0.05, **kw)
    hist = make_history(w, 0)
    hl = hist.hist_len.copy()
    cfg = oracle_config(w)
    o = HierOracle(cfg, [hist], hl)
    o.set_compression(0, m)
    prefill = {}
    for r in range(w.n_req):
        first, rows = ring_prefill_rows(hist, r, int(hl[r]), w.ring_window, cfg.plen, max(w.n_prefix, 1))
        # the ring holds positions: the test's own per-position rows (history rows are stored rows)
        rows = bf16_bits_from_f32(np.random.default_rng(r).standard_normal(rows.shape).astype(np.float32))
        o.ring_load(0, r, first, rows)
        prefill[r] = (first, rows.copy())
    return w, hist, hl, cfg, o, prefill


def test_compressed_step_selects_complete_rows_and_attends_exactly():
    m = 4
    w, hist, hl, cfg, o, prefill = _compressed_case(m)
    si = make_step_inputs(w, 0, 0, hl)
    res = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows)
    checked = 0
    for r in range(w.n_req):
        n_pos = int(hl[r])
        n_src = n_pos // m
        act = si.causal_pos[r] >= 0
        ent = si.topk[r][act]
        valid = ent[(ent >= 0) & (ent < n_src)]
        assert res.req[r].counts["selections"] == valid.size
        assert res.req[r].counts["invalid"] == ent.size - valid.size - int((ent == -1).sum())
        assert res.req[r].counts["union_tail"] == 0             # the ring holds positions, not rows
        hist_rows = f32_from_bf16_bits(hist.tails[r, :n_src]).astype(np.float64)
        first, pre = prefill[r]
        for j in range(w.q_max):
            p_j = int(si.causal_pos[r, j])
            if p_j < 0:
                continue
            lst = si.topk[r, j]
            good = lst[(lst >= 0) & (lst < n_src)]
            mult = np.bincount(good, minlength=n_src)
            lo = max(first, p_j - w.ring_window + 1, 0)
            ring = [pre[pos - first] if pos < n_pos else si.block_rows[r, pos - n_pos] for pos in range(lo, p_j + 1)]
            ring = f32_from_bf16_bits(np.stack(ring)).astype(np.float64)
            q = f32_from_bf16_bits(si.queries[r, j]).astype(np.float64)
            ref = _dense_reference(q, hist_rows, mult, ring, cfg.scale, w.d_qk, w.v_off, w.d_v)
            np.testing.assert_allclose(res.out[(r, j)], ref, rtol=1e-11, atol=1e-12)
            checked += 1
    assert checked >= 3


def test_compressed_commits_add_the_completed_rows():
    m = 3
    w, hist, hl, cfg, o, prefill = _compressed_case(m, var_k=True)
    n = [int(x) for x in hl]
    record = {r: {} for r in range(w.n_req)}       # row -> bytes the test handed over
    for step in range(6):
        si = make_step_inputs(w, 0, step, np.array(n, np.int32))
        o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
        acc = make_accepted(w, step, si.k_active)
        src = make_source_rows(w, 0, step)
        o.commit(acc, src_rows=[src])
        for r in range(w.n_req):
            n2 = n[r] + 1 + int(acc[r])
            new = [s for s in range(n2 // m + 2) if s * m + m - 1 < n2 and not s * m + m - 1 < n[r]]
            for i, s in enumerate(new):
                record[r][s] = src[r, i].copy()
            n[r] = n2
    for r in range(w.n_req):
        assert record[r]
        for s, row in record[r].items():
            assert np.array_equal(hist.tails[r, s - cfg.plen], row)
        # the incomplete group is not a row yet: its index still holds the generator's bytes
        s_inc = n[r] // m
        assert s_inc not in record[r]
