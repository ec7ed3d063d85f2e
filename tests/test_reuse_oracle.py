"""Pins of the oracle's shared-source consumers ("Adaptive DHiSparse" §2,
physical-source sharing; §3.2; Table 3): a Reuse consumer attends with its
own queries over the latest selection of the source; a Reindex consumer
selects again from the same source, resolving against the cache state the
earlier selection left.

Reuse outputs are checked against the dense masked formulation over every
history row; Reindex misses against set algebra over the slot table the
earlier selection left; neither kind may change state it does not own.
"""
import numpy as np

from oracle import HierOracle
from tests.oracle_helpers import oracle_config, ring_prefill_rows
from tests.test_oracle_pins import _dense_reference, _tiny_case
from workloads import f32_from_bf16_bits, make_history, make_hot_warm_set, make_step_inputs


def _source(n_req=3, **kw):
    w = _tiny_case(n_req=n_req, **kw)
    hist = make_history(w, 0)
    hl = hist.hist_len
    cfg = oracle_config(w)
    o = HierOracle(cfg, [hist], hl)
    si = make_step_inputs(w, 0, 0, hl)
    for r, (rows, ages) in enumerate(make_hot_warm_set(w, 0, hl, si)):
        o.set_hot(0, r, rows, ages)
    prefill = {}
    for r in range(w.n_req):
        first, rows = ring_prefill_rows(hist, r, int(hl[r]), w.ring_window, cfg.plen, max(w.n_prefix, 1))
        o.ring_load(0, r, first, rows)
        prefill[r] = (first, rows.copy())
    return w, hist, hl, cfg, o, si, prefill


def test_reuse_is_attention_over_the_latest_selection():
    w, hist, hl, cfg, o, si, prefill = _source()
    o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
    before = [o.slot_table(0, r) for r in range(w.n_req)]
    t0 = o.t[0]
    q2 = make_step_inputs(w, 0, 7, hl).queries           # the Reuse layer's own queries
    out = o.verify_reuse(0, q2)
    assert o.t[0] == t0                                   # no resolution happened
    for r in range(w.n_req):
        rows, ages = o.slot_table(0, r)
        assert np.array_equal(rows, before[r][0]) and np.array_equal(ages, before[r][1])
    checked = 0
    for r in range(w.n_req):
        n_r = int(hl[r])
        hist_rows = f32_from_bf16_bits(hist.tails[r, :n_r]).astype(np.float64)
        first, pre = prefill[r]
        for j in range(w.q_max):
            p_j = int(si.causal_pos[r, j])
            if p_j < 0:
                assert (r, j) not in out
                continue
            lst = si.topk[r, j]
            good = lst[(lst >= 0) & (lst < n_r)]
            mult = np.bincount(good, minlength=n_r)
            lo = max(first, p_j - w.ring_window + 1, 0)
            ring = [pre[pos - first] if pos < n_r else si.block_rows[r, pos - n_r] for pos in range(lo, p_j + 1)]
            ring = f32_from_bf16_bits(np.stack(ring)).astype(np.float64)
            q = f32_from_bf16_bits(q2[r, j]).astype(np.float64)
            ref = _dense_reference(q, hist_rows, mult, ring, cfg.scale, w.d_qk, w.v_off, w.d_v)
            np.testing.assert_allclose(out[(r, j)], ref, rtol=1e-11, atol=1e-12)
            checked += 1
    assert checked >= 3


def test_reindex_adds_only_rows_absent_from_the_source_state():
    """A fresh selection from the shared source fetches exactly its union
    rows that neither the hot cache (as the earlier selection left it) nor
    the resident map holds; rows the earlier selection promoted are hits."""
    w, hist, hl, cfg, o, si, prefill = _source(n_req=4, hot_slots=40)
    res_a = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
    state = {r: set(int(x) for x in o.slot_table(0, r)[0] if x >= 0) for r in range(w.n_req)}
    ring_before = [dict((p, v.copy()) for p, v in o.st[0][r].ring.items()) for r in range(w.n_req)]
    sb = make_step_inputs(w, 0, 3, hl)                   # the Reindex layer's fresh top-k:
    topk_b = si.topk.copy()                              # half of it new, half as before
    topk_b[:, :, ::2] = sb.topk[:, :, ::2]
    res_b = o.verify_step(0, topk_b, si.causal_pos, sb.queries, None, attend=None)
    overlap = 0
    for r in range(w.n_req):
        a, b = res_a.req[r], res_b.req[r]
        if not b.active:
            continue
        # rows the test loaded into the ring below n_r are the tail (resolved
        # directly); everything else absent from the slot table is fetched
        tail = set(range(prefill[r][0], int(hl[r])))
        assert set(b.miss) == set(b.union) - state[r] - tail
        promoted_a = set(a.miss[: len(a.victims)])
        assert not (set(b.miss) & promoted_a)             # fetched once for the earlier layer
        assert set(b.union) & promoted_a <= {u for u, c in zip(b.union, b.cls) if c == 1}
        overlap += len(set(b.union) & promoted_a)
        # the ring still holds what the producer wrote (no rows passed)
        ring = o.st[0][r].ring
        assert set(ring) == set(ring_before[r])
        for p in ring:
            assert np.array_equal(ring[p], ring_before[r][p])
    assert overlap >= 10


def test_reindex_then_reuse_reads_the_fresh_selection():
    w, hist, hl, cfg, o, si, prefill = _source(n_req=2)
    o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
    sb = make_step_inputs(w, 0, 5, hl)
    res_b = o.verify_step(0, sb.topk, si.causal_pos, sb.queries, None)
    # a Reuse with the Reindex layer's own queries reproduces the Reindex outputs
    out = o.verify_reuse(0, sb.queries)
    assert set(out) == set(res_b.out)
    for key in out:
        assert np.array_equal(out[key], res_b.out[key])


def test_commit_ends_the_reusable_selection():
    w, hist, hl, cfg, o, si, prefill = _source(n_req=2)
    o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
    o.commit(np.zeros(w.n_req, np.int32))
    try:
        o.verify_reuse(0, si.queries)
    except RuntimeError:
        return
    raise AssertionError("a selection survived its step's commit")
