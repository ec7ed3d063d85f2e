"""Pins of the oracle against what the pages and the mathematics fix.

Nothing here re-implements the oracle's own formula: attention is checked
against a dense masked formulation over every history row (multiplicities as
weights), against closed forms and against worked examples; resolution against
hand-worked fixtures, structural invariants and the pages' printed figures.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import CLS_HOT, CLS_MISS, CLS_RESIDENT, HierOracle
from tests.oracle_helpers import oracle_config, ring_prefill_rows
from workloads import (WORKLOADS, f32_from_bf16_bits, make_history, make_hot_warm_set,
                       make_resident_bitmaps, make_step_inputs, shrink, bf16_bits_from_f32)

GIB = float(1 << 30)


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- closed forms

def test_ring_rows_closed_form(golden_dir):
    g = _golden(golden_dir, "closed_forms.json")
    for case in g["ring_rows"]:
        r_d = oracle.ring_rows(case["window"], case["page"], case["k_max"])
        assert r_d == case["expected"], case
        for kb in case.get("covers_blocks", []):
            # the live span of a smaller block (window plus block) still fits the ring
            assert case["window"] + kb - 1 <= r_d


def test_ring_and_staging_memory(golden_dir):
    g = _golden(golden_dir, "closed_forms.json")
    rm = g["ring_memory"]
    r_d = oracle.ring_rows(2048, 64, 8)
    assert r_d == rm["r_d"]
    assert abs(rm["slots"] * r_d * rm["row_bytes"] / GIB - rm["expected_gib"]) <= rm["tol_gib"]
    for case in g["staging"]:
        b = oracle.staging_bytes(case["chi"], case["slots"], case["k_max"], case["k"], case["d_kv"])
        assert abs(b / GIB - case["expected_gib"]) <= case["tol_gib"], case
    ps = g["per_session_state"]
    ring_sess = r_d * rm["row_bytes"] / GIB
    assert abs(ring_sess - ps["ring_gib_per_session"]) < 5e-4
    assert abs(ring_sess + ps["staging_gib_total"] / ps["slots"] - ps["expected_gib"]) <= ps["tol_gib"]


def test_fetch_volume_closed_form(golden_dir):
    fv = _golden(golden_dir, "closed_forms.json")["fetch_volume"]
    one = fv["requests"] * fv["k"] * fv["d_kv"] / 1e6
    assert abs(one - fv["one_query_mb"]) < 0.01
    assert abs(fv["q"] * one - fv["disjoint_mb"]) < 0.5


@pytest.mark.parametrize("window,page,k_max", [(2048, 64, 8), (128, 64, 8), (64, 64, 4), (5, 4, 3),
                                               (1, 1, 1), (17, 8, 6)])
def test_ring_addr_no_collision(window, page, k_max):
    """Eq. (10): positions live together (the window below the frontier plus the
    block above it) never share a ring row, and request slots are disjoint."""
    r_d = oracle.ring_rows(window, page, k_max)
    assert r_d >= window + k_max - 1 and r_d % page == 0
    for n in range(0, 3 * r_d + 5, max(1, r_d // 37)):
        lo = max(0, n - window + 1)
        live = list(range(lo, n + k_max))
        for slot in (0, 1, 7):
            addrs = [oracle.ring_addr(slot, t, r_d) for t in live]
            assert len(set(addrs)) == len(addrs)
            assert all(slot * r_d <= a < (slot + 1) * r_d for a in addrs)


# ---------------------------------------------------------------- resolution examples

def _example_oracle(ex, d=4, heads=1):
    n_r = ex["n_r"]
    cfg = oracle.OracleConfig(n_req=1, n_groups=1, hist_cap=n_r + ex["q_max"] + 1, n_prefix=0,
                              prefix_len=0, row_elems=2 * d, d_qk=d, v_off=d, d_v=d,
                              n_heads=heads, q_max=ex["q_max"], topk=ex["topk"],
                              hot_slots=ex["hot_slots"], ring_window=4, ring_page=4)
    rng = np.random.default_rng(5)
    from workloads.gen import History
    hist = History(prefix=np.zeros((1, 0, 2 * d), np.uint16),
                   tails=bf16_bits_from_f32(rng.standard_normal((1, cfg.hist_cap, 2 * d)).astype(np.float32)),
                   hist_len=np.array([n_r], np.int32))
    o = HierOracle(cfg, [hist], [n_r])
    if ex["resident_rows"]:
        bm = np.zeros(cfg.hist_cap, np.uint8)
        bm[ex["resident_rows"]] = 1
        o.set_resident(0, 0, bm)
    o.set_hot(0, 0, ex["hot_rows"], ex["hot_ages"])
    Q, k = ex["q_max"], ex["topk"]
    topk = np.array([ex["lists"]], np.int32)
    cp = np.array([ex["causal_pos"]], np.int32)
    qs = np.zeros((1, Q, heads, d), np.uint16)
    blk = bf16_bits_from_f32(rng.standard_normal((1, Q, 2 * d)).astype(np.float32))
    return o, topk, cp, qs, blk


def test_resolve_worked_examples(golden_dir):
    g = _golden(golden_dir, "resolve_examples.json")
    for ex in g["examples"]:
        o, topk, cp, qs, blk = _example_oracle(ex)
        res = o.verify_step(0, topk, cp, qs, blk, attend=None)
        e = ex["expected"]
        rr = res.req[0]
        assert res.step == e["step"], ex["name"]
        assert rr.union == e["union"], ex["name"]
        assert rr.cls == e["cls"], ex["name"]
        assert rr.miss == e["miss"], ex["name"]
        assert rr.victims == e["victims"], ex["name"]
        assert rr.overflow == e["overflow"], ex["name"]
        assert rr.loc.tolist() == e["loc"], ex["name"]
        rows, ages = o.slot_table(0, 0)
        assert rows.tolist() == e["slot_rows_after"], ex["name"]
        assert ages.tolist() == e["slot_ages_after"], ex["name"]
        for key, val in e["counts"].items():
            assert rr.counts[key] == val, (ex["name"], key)


def test_figure3_each_shared_miss_fetched_once(golden_dir):
    """§3.3 / Figure 3 callout 2: a (3 selectors) and b (2 selectors) are each
    copied once: 2 fetched rows for 5 missing selections."""
    ex = [e for e in _golden(golden_dir, "resolve_examples.json")["examples"]
          if e["name"] == "figure3_shared_misses"][0]
    o, topk, cp, qs, blk = _example_oracle(ex)
    rr = o.verify_step(0, topk, cp, qs, blk, attend=None).req[0]
    assert rr.counts["union_miss"] == 2 and rr.counts["sel_miss"] == 5
    assert sorted(rr.miss) == [10, 20]


# ---------------------------------------------------------------- attention pins

def _dense_reference(q, hist_rows, mult, ring_rows, scale, d_qk, v_off, d_v):
    """Masked dense attention over *every* history row, each weighted by how
    many times the query's list holds it, plus the ring rows with weight 1."""
    rows = np.concatenate([hist_rows, ring_rows], axis=0)
    w = np.concatenate([mult.astype(np.float64), np.ones(ring_rows.shape[0])])
    K = rows[:, :d_qk]
    V = rows[:, v_off:v_off + d_v]
    S = scale * (q @ K.T)
    S = np.where(w[None, :] > 0, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    P = w[None, :] * np.exp(S - m)
    return (P @ V) / P.sum(axis=1, keepdims=True)


def _tiny_case(seed_name="tiny", **kw):
    base = shrink(WORKLOADS["tiny"], hist_lo=300, hist_hi=300, hist_cap=340, row_elems=48,
                  d_qk=32, v_off=16, d_v=32, n_heads=3, q_max=4, topk=24, hot_slots=16,
                  ring_window=6, ring_page=4, pad_frac=0.1, invalid_frac=0.05,
                  empty_slot_frac=0.2, var_k=True)
    return shrink(base, **kw)


def _run_with_history_views(w, block_only=False, rho=0.0, step=0, warm=True):
    hist = make_history(w, 0)
    hl = hist.hist_len
    cfg = oracle_config(w, ring_block_only=block_only)
    o = HierOracle(cfg, [hist], hl)
    si = make_step_inputs(w, 0, step, hl)
    if warm:
        for r, (rows, ages) in enumerate(make_hot_warm_set(w, 0, hl, si)):
            o.set_hot(0, r, rows, ages)
    if rho > 0:
        bm = make_resident_bitmaps(w, 0, hl, rho)
        for r in range(w.n_req):
            o.set_resident(0, r, bm[r])
    prefill = {}
    for r in range(w.n_req):
        first, rows = ring_prefill_rows(hist, r, int(hl[r]), w.ring_window, cfg.plen, max(w.n_prefix, 1))
        o.ring_load(0, r, first, rows)
        prefill[r] = (first, rows.copy())
    res = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows)
    return o, hist, si, res, prefill, cfg


@pytest.mark.parametrize("block_only", [False, True])
def test_attention_matches_dense_bruteforce(block_only):
    w = _tiny_case(n_req=3)
    o, hist, si, res, prefill, cfg = _run_with_history_views(w, block_only=block_only)
    checked = 0
    for r in range(w.n_req):
        n_r = int(hist.hist_len[r])
        hist_rows = f32_from_bf16_bits(hist.tails[r, :n_r]).astype(np.float64)
        first, pre = prefill[r]
        for j in range(w.q_max):
            p_j = int(si.causal_pos[r, j])
            if p_j < 0:
                continue
            lst = si.topk[r, j]
            good = lst[(lst >= 0) & (lst < n_r)]
            mult = np.bincount(good, minlength=n_r)
            # ring content from the test's own record: prefill below n_r, block rows above
            lo = max(first, p_j - w.ring_window + 1, 0)
            if block_only:
                lo = max(lo, n_r)
            ring = []
            for pos in range(lo, p_j + 1):
                ring.append(pre[pos - first] if pos < n_r else si.block_rows[r, pos - n_r])
            ring = f32_from_bf16_bits(np.stack(ring)).astype(np.float64)
            q = f32_from_bf16_bits(si.queries[r, j]).astype(np.float64)
            ref = _dense_reference(q, hist_rows, mult, ring, cfg.scale, w.d_qk, w.v_off, w.d_v)
            got = res.out[(r, j)]
            np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)
            checked += 1
    assert checked >= 3


def _single_query_oracle(n_r, rows_f32, lst, W, q_f32, d_qk, v_off, d_v, ring_rows_f32=None):
    """One request, one query at p = n_r, history rows given, ring = its own block row."""
    rows_elems = rows_f32.shape[1]
    cfg = oracle.OracleConfig(n_req=1, n_groups=1, hist_cap=n_r + 2, n_prefix=0, prefix_len=0,
                              row_elems=rows_elems, d_qk=d_qk, v_off=v_off, d_v=d_v,
                              n_heads=q_f32.shape[0], q_max=1, topk=len(lst), hot_slots=2,
                              ring_window=W, ring_page=1)
    from workloads.gen import History
    tails = np.zeros((1, n_r + 2, rows_elems), np.uint16)
    tails[0, :n_r] = bf16_bits_from_f32(rows_f32)
    hist = History(prefix=np.zeros((1, 0, rows_elems), np.uint16), tails=tails,
                   hist_len=np.array([n_r], np.int32))
    o = HierOracle(cfg, [hist], [n_r])
    blk = np.zeros((1, 1, rows_elems), np.uint16)
    if ring_rows_f32 is not None:
        blk[0, 0] = bf16_bits_from_f32(ring_rows_f32)
    res = o.verify_step(0, np.array([[lst]], np.int32), np.array([[n_r]], np.int32),
                        bf16_bits_from_f32(q_f32)[None, None], blk)
    return res.out[(0, 0)]


def test_attention_single_visible_row_is_its_value():
    rng = np.random.default_rng(1)
    row = rng.standard_normal(24).astype(np.float32)
    q = rng.standard_normal((2, 16)).astype(np.float32)
    # every list entry is a pad and the window holds only the query's own row
    out = _single_query_oracle(5, np.zeros((5, 24), np.float32), [-1, -1, -1], 1, q, 16, 8, 16,
                               ring_rows_f32=row)
    v = f32_from_bf16_bits(bf16_bits_from_f32(row))[8:24].astype(np.float64)
    assert np.array_equal(out, np.stack([v, v]))


def test_attention_identical_rows_give_their_value():
    rng = np.random.default_rng(2)
    row = rng.standard_normal(24).astype(np.float32)
    rows = np.stack([row] * 9)
    q = rng.standard_normal((3, 16)).astype(np.float32)
    out = _single_query_oracle(9, rows, [0, 3, 5, 8, 8], 1, q, 16, 8, 16, ring_rows_f32=row)
    v = f32_from_bf16_bits(bf16_bits_from_f32(row))[8:24].astype(np.float64)
    np.testing.assert_allclose(out, np.stack([v] * 3), rtol=0, atol=1e-14)


def test_attention_zero_query_is_multiplicity_weighted_mean():
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((12, 20)).astype(np.float32)
    own = rng.standard_normal(20).astype(np.float32)
    lst = [4, 7, 4, -1, 11, 30]       # 30 is out of range -> skipped; 4 counts twice
    out = _single_query_oracle(12, rows, lst, 1, np.zeros((2, 10), np.float32), 10, 10, 10,
                               ring_rows_f32=own)
    vb = f32_from_bf16_bits(bf16_bits_from_f32(rows)).astype(np.float64)[:, 10:20]
    ob = f32_from_bf16_bits(bf16_bits_from_f32(own)).astype(np.float64)[10:20]
    want = (2 * vb[4] + vb[7] + vb[11] + ob) / 5.0
    np.testing.assert_allclose(out[0], want, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out[1], want, rtol=1e-13, atol=1e-14)


def test_attention_duplicate_entry_has_double_weight():
    """Two distinct rows a, b; list [a, a, b]; window empty of history, own row
    orthogonal: closed form (2 e^sa Va + e^sb Vb + e^so Vo) / (2 e^sa + e^sb + e^so)."""
    K = np.zeros((3, 8), np.float32)
    K[0, 0] = 1.0        # a
    K[1, 1] = 1.0        # b
    rows = np.concatenate([K, np.arange(24, dtype=np.float32).reshape(3, 8) / 8.0], axis=1)
    own = np.zeros(16, np.float32)
    own[8:] = -1.0
    q = np.zeros((1, 8), np.float32)
    q[0, 0], q[0, 1] = 2.0, -1.0
    out = _single_query_oracle(3, rows, [0, 0, 1], 1, q, 8, 8, 8, ring_rows_f32=own)
    s = 1.0 / math.sqrt(8)
    ea, eb, eo = math.exp(2.0 * s), math.exp(-1.0 * s), 1.0
    Va, Vb, Vo = rows[0, 8:].astype(np.float64), rows[1, 8:].astype(np.float64), own[8:].astype(np.float64)
    want = (2 * ea * Va + eb * Vb + eo * Vo) / (2 * ea + eb + eo)
    np.testing.assert_allclose(out[0], want, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- invariants

def test_resolution_invariants_random():
    w = _tiny_case(n_req=4, hot_slots=20)
    hist = make_history(w, 0)
    hl = hist.hist_len
    cfg = oracle_config(w)
    o = HierOracle(cfg, [hist], hl)
    si = make_step_inputs(w, 0, 0, hl)
    warm = make_hot_warm_set(w, 0, hl, si)
    bm = make_resident_bitmaps(w, 0, hl, 0.2)
    pool_of = {}
    cursor = 0
    for r in range(w.n_req):
        o.set_hot(0, r, *warm[r])
        o.set_resident(0, r, bm[r])
        for s in np.flatnonzero(bm[r][: hl[r]]):
            pool_of[cursor] = (r, int(s))
            cursor += 1
    before = {r: o.slot_table(0, r) for r in range(w.n_req)}
    res = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
    B, Q, k = w.hot_slots, w.q_max, w.topk
    for r in range(w.n_req):
        rr = res.req[r]
        n_r = int(hl[r])
        act = si.causal_pos[r] >= 0
        ent = si.topk[r][act]
        valid = ent[(ent >= 0) & (ent < n_r)]
        assert rr.union == np.unique(valid).tolist()
        assert rr.counts["selections"] == valid.size
        assert rr.counts["pads"] == int((ent == -1).sum())
        assert rr.counts["invalid"] == ent.size - valid.size - int((ent == -1).sum())
        # each distinct missing row is fetched once and is a member of the union
        assert len(set(rr.miss)) == len(rr.miss) and set(rr.miss) <= set(rr.union)
        assert rr.miss == sorted(rr.miss)
        # D = U minus ready rows (eq. 6); ready = resident or hot before the step
        rows0, ages0 = before[r]
        ready = set(np.flatnonzero(bm[r][:n_r]).tolist()) | set(int(x) for x in rows0 if x >= 0)
        assert set(rr.miss) == set(rr.union) - ready
        # D subset of H: every missing row has a host copy (rows below the frontier)
        assert all(0 <= u < n_r for u in rr.miss)
        # eq. (12): every location decodes to the selected row's place
        for j in range(Q):
            for i in range(k):
                e = int(si.topk[r, j, i])
                code = int(rr.loc[j, i])
                if not act[j] or not (0 <= e < n_r):
                    assert code == -1
                    continue
                tier, idx = code >> 29, code & ((1 << 29) - 1)
                if tier == oracle.HOT:
                    assert idx // B == r and rows0[idx % B] == e
                elif tier == oracle.STAGED:
                    assert idx // (Q * k) == r and rr.miss[idx % (Q * k)] == e
                else:
                    assert tier == oracle.RESIDENT and pool_of[idx] == (r, e)
        # LRU: every evicted slot precedes every kept unselected slot in (age, slot) order
        rows1, ages1 = o.slot_table(0, r)
        uset = set(rr.union)
        key = lambda s: (-1 if rows0[s] == -1 else ages0[s], s)
        unsel = [s for s in range(B) if rows0[s] == -1 or rows0[s] not in uset]
        ev = set(rr.victims)
        kept = [s for s in unsel if s not in ev]
        if ev and kept:
            assert max(key(s) for s in ev) < min(key(s) for s in kept)
        # selected rows in the cache are never evicted
        for s in range(B):
            if rows0[s] != -1 and rows0[s] in uset:
                assert rows1[s] == rows0[s]
        # promoted rows now sit in their victim slots with the step's stamp
        for i, s in enumerate(rr.victims):
            assert rows1[s] == rr.miss[i] and ages1[s] == res.step
        assert rr.overflow == len(rr.miss) - len(rr.victims)
        assert len(rr.victims) == min(len(rr.miss), len(unsel))


def test_outputs_independent_of_cache_state():
    w = _tiny_case(n_req=2)
    outs = []
    unions = []
    misses = []
    for warm, rho in ((False, 0.0), (True, 0.0), (True, 0.5)):
        o, hist, si, res, prefill, cfg = _run_with_history_views(w, rho=rho, warm=warm)
        outs.append(res.out)
        unions.append({r: res.req[r].union for r in range(w.n_req)})
        misses.append(sum(len(res.req[r].miss) for r in range(w.n_req)))
    for key in outs[0]:
        assert np.array_equal(outs[0][key], outs[1][key])
        assert np.array_equal(outs[0][key], outs[2][key])
    assert unions[0] == unions[1] == unions[2]
    assert misses[0] > misses[1] > misses[2]


def test_multi_step_ring_preserves_accepted_prefix(golden_dir):
    """Eq. (7) over random rounds: after commit(A) the committed rows are the
    anchor and accepted drafts (host copy written), the rejected rows are never
    visible again, and every later window reads the committed rows."""
    w = _tiny_case(n_req=3, ring_window=5, pad_frac=0.0, invalid_frac=0.0)
    hist = make_history(w, 0)
    hl = hist.hist_len.copy()
    cfg = oracle_config(w)
    o = HierOracle(cfg, [hist], hl)
    committed = {r: {} for r in range(w.n_req)}      # position -> row, the test's own record
    for r in range(w.n_req):
        first, rows = ring_prefill_rows(hist, r, int(hl[r]), w.ring_window, 0, 1)
        o.ring_load(0, r, first, rows)
        for i in range(rows.shape[0]):
            committed[r][first + i] = rows[i].copy()
    n = [int(x) for x in hl]
    rng = np.random.default_rng(11)
    for step in range(6):
        si = make_step_inputs(w, 0, step, np.array(n, np.int32))
        res = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
        for r in range(w.n_req):
            kr = int(si.k_active[r])
            for j in range(kr):
                p = n[r] + j
                lo = max(p - w.ring_window + 1, 0)
                for pos in range(lo, p + 1):
                    want = committed[r][pos] if pos < n[r] else si.block_rows[r, pos - n[r]]
                    if pos >= min(committed[r]):
                        assert np.array_equal(o.st[0][r].ring[pos], want)
        acc = np.array([rng.integers(0, int(si.k_active[r])) for r in range(w.n_req)], np.int32)
        o.commit(acc)
        for r in range(w.n_req):
            for a in range(int(acc[r]) + 1):
                committed[r][n[r] + a] = si.block_rows[r, a].copy()
                assert np.array_equal(hist.tails[r, n[r] + a], si.block_rows[r, a])
            n[r] += 1 + int(acc[r])
            assert o.n[r] == n[r]
            assert all(p < n[r] for p in o.st[0][r].ring)


def test_acceptance_example(golden_dir):
    """Figure 3 callout 4: D,E,F,G computed, E and F accepted (A=2): the
    frontier advances by 3 and G's row is not visible to the next round."""
    acc = _golden(golden_dir, "closed_forms.json")["acceptance"]
    w = _tiny_case(n_req=1, q_max=acc["k_active"], var_k=False, pad_frac=0.0, invalid_frac=0.0)
    hist = make_history(w, 0)
    hl = hist.hist_len.copy()
    o = HierOracle(oracle_config(w), [hist], hl)
    si = make_step_inputs(w, 0, 0, hl)
    o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
    n0 = int(hl[0])
    o.commit(np.array([acc["accepted"]], np.int32))
    assert o.n[0] == n0 + acc["frontier_advance"]
    g_pos = n0 + 3                                  # G, the rejected draft
    assert g_pos not in o.st[0][0].ring
    si2 = make_step_inputs(w, 0, 1, np.array([o.n[0]], np.int32))
    o.verify_step(0, si2.topk, si2.causal_pos, si2.queries, si2.block_rows, attend=None)
    # G's position now holds the new anchor G* of the next round
    assert np.array_equal(o.st[0][0].ring[g_pos], si2.block_rows[0, 0])


@pytest.mark.slow
def test_residency_sweep_cuts_host_fetch_share():
    """§4.3.1 / Table A1: optional residency cut the host-fetched share of
    selected rows from 14.21% to 1.38% (about 10x).  With a static resident
    fraction rho = 0.9 of rows the share falls by 1/(1-rho) = 10x."""
    w = shrink(WORKLOADS["mla128"], n_req=3, n_groups=1, hist_lo=20_000, hist_hi=20_000,
               hist_cap=20_100, prefix_len=16_384, row_elems=8, d_qk=8, v_off=0, d_v=8,
               n_heads=1)
    shares = {}
    for rho in (0.0, 0.9):
        hist = make_history(w, 0)
        hl = hist.hist_len
        o = HierOracle(oracle_config(w), [hist], hl)
        si = make_step_inputs(w, 0, 0, hl)
        for r, (rows, ages) in enumerate(make_hot_warm_set(w, 0, hl, si)):
            o.set_hot(0, r, rows, ages)
        if rho > 0:
            bm = make_resident_bitmaps(w, 0, hl, rho)
            for r in range(w.n_req):
                o.set_resident(0, r, bm[r])
        res = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
        sel = sum(res.req[r].counts["selections"] for r in range(w.n_req))
        dist = sum(res.req[r].counts["union"] for r in range(w.n_req))
        miss = sum(res.req[r].counts["union_miss"] for r in range(w.n_req))
        shares[rho] = miss / dist
        assert sel > 0
    assert 0.12 < shares[0.0] < 0.16
    assert 7.0 < shares[0.0] / shares[0.9] < 14.0
