"""Pins of the dynamic optional-residency oracle ("Adaptive DHiSparse" §3.1,
eqs. 3-4; Figure 2; §4.3.1 with Figure 6 and Table A1).

The eq. (4) walk is checked against a hand-worked fixture and, on random
operation sequences, against properties that any correct implementation has:
the capacity bound of eq. (3), a minimal reclaimed prefix of the reclaim order,
untouched pages of the other requests, an unchanged state when an admission
waits, ascending page fill, round-robin fairness and the bound per attempt,
unique pool pages, and pending pages invisible to resolution.
"""
import copy
import json
import os

import numpy as np
import pytest

import oracle
from oracle import HierOracle, OptResidency
from tests.oracle_helpers import oracle_config
from workloads import WORKLOADS, make_history, make_hot_warm_set, make_step_inputs, shrink


def _fixture(golden_dir):
    with open(os.path.join(golden_dir, "residency_examples.json")) as f:
        return json.load(f)


def _state(o: OptResidency):
    return (list(o.admitted), list(o.required), list(o.eligible), copy.deepcopy(o.held),
            copy.deepcopy(o.ready), set(o.free), o.cursor)


def _check_pool(o: OptResidency):
    pools = [p for h in o.held for p in h.values()]
    assert len(pools) == len(set(pools))
    assert set(pools).isdisjoint(o.free)
    assert set(pools) | o.free == set(range(o.M))
    for r in range(o.N):
        assert o.ready[r] <= set(o.held[r])
        assert set(o.held[r]) == set(range(len(o.held[r])))    # pages fill in ascending order
        assert len(o.held[r]) <= o.eligible[r]
        if not o.admitted[r]:
            assert not o.held[r] and o.required[r] == 0


def test_eq4_worked_examples(golden_dir):
    """Hand-worked walks of eq. (4) on one admitted set (fixture)."""
    fx = _fixture(golden_dir)
    n_old = len(fx["admitted"])
    for case in fx["cases"]:
        o = OptResidency(n_old + 1, fx["pool_pages"], fx["page_rows"], fx["reserve"])
        for r, (n_r, req) in enumerate(fx["admitted"]):
            assert o.admit(r, n_r, req, []) == []
        o.populate(1000)
        o.publish()
        assert [len(h) for h in o.held[:n_old]] == fx["held_before"]
        deficit = o.sum_required() + case["admit_required"] + o.sum_held() + o.reserve - o.M
        assert deficit == case["deficit"], case["name"]
        got = o.admit(n_old, 0, case["admit_required"], case["order"])
        assert got == case["expected_reclaimed"], case["name"]
        assert [len(h) for h in o.held[:n_old]] == case["held_after"], case["name"]
        assert o.admitted[n_old] == (got is not None)


def _random_ops(seed, n_req=6, pool=40, page_rows=4, reserve=3, n_ops=300):
    rng = np.random.default_rng(seed)
    o = OptResidency(n_req, pool, page_rows, reserve)
    admit_seq = []
    for _ in range(n_ops):
        op = rng.integers(0, 4)
        if op == 0:
            cand = [r for r in range(n_req) if not o.admitted[r]]
            if not cand:
                continue
            r = int(rng.choice(cand))
            n_r = int(rng.integers(0, 9 * page_rows))
            need = int(rng.integers(0, 12))
            adm = [x for x in range(n_req) if o.admitted[x]]
            order = [int(x) for x in rng.permutation(adm)][: int(rng.integers(0, len(adm) + 1))]
            before = _state(o)
            held_before = [dict(h) for h in o.held]
            deficit = o.sum_required() + need + o.sum_held() + reserve - pool
            got = o.admit(r, n_r, need, order)
            if got is None:
                assert deficit > 0
                assert sum(len(held_before[x]) for x in order) < deficit
                assert _state(o) == before                      # waiting changes nothing
            else:
                q = len(got)
                assert got == order[:q]                          # a prefix of the reclaim order
                if deficit > 0:
                    cov = [len(held_before[x]) for x in got]
                    assert sum(cov) >= deficit
                    assert sum(cov[:-1]) < deficit               # eq. (4): the smallest such q
                else:
                    assert q == 0
                for x in range(n_req):
                    if x in got:
                        assert not o.held[x] and o.admitted[x]   # whole request reclaimed, still admitted
                    elif x != r:
                        assert o.held[x] == held_before[x]       # the others keep their pages
                assert o.eligible[r] == n_r // page_rows         # complete pages only
                admit_seq.append(r)
        elif op == 1:
            adm = [x for x in range(n_req) if o.admitted[x]]
            if adm:
                o.complete(int(rng.choice(adm)))
        elif op == 2:
            m = int(rng.integers(0, 10))
            need0 = {x: o.eligible[x] - len(o.held[x]) for x in range(n_req) if o.admitted[x]}
            budget0 = o.budget()
            new = o.populate(m)
            assert len(new) <= m and len(new) <= max(0, budget0)
            per = {x: sum(1 for (y, _, _) in new if y == x) for x in need0}
            for x, k in per.items():
                assert k <= need0[x]
            still = [x for x in need0 if per[x] < need0[x]]
            if still and per:
                # round robin: a request still needing pages got at most one fewer than any other
                assert max(per.values()) - min(per[x] for x in still) <= 1
            if len(new) < min(m, budget0):
                assert all(per[x] == need0[x] for x in need0)   # stopped only when no one needs more
            for (x, idx, pool_page) in new:
                for row in (idx * page_rows, idx * page_rows + page_rows - 1):
                    assert o.lookup(x, row) is None              # pending: invisible to resolution
        else:
            o.publish()
            for x in range(n_req):
                for idx, pp in o.held[x].items():
                    row = idx * page_rows + 1
                    assert o.lookup(x, row) == pp * page_rows + 1
        assert o.sum_required() + o.sum_held() + reserve <= pool   # eq. (3)
        _check_pool(o)
    return o, admit_seq


@pytest.mark.parametrize("seed", range(8))
def test_residency_random_sequences(seed):
    _random_ops(seed)


def test_eq3_holds_after_every_successful_admission():
    rng = np.random.default_rng(3)
    o = OptResidency(8, 50, 2, 4)
    for step in range(400):
        r = int(rng.integers(0, 8))
        if o.admitted[r]:
            o.complete(r)
            continue
        order = [x for x in range(8) if o.admitted[x]]
        got = o.admit(r, int(rng.integers(0, 40)), int(rng.integers(0, 10)), order)
        if got is not None:
            assert o.sum_required() + o.sum_held() + o.reserve <= o.M
        o.populate(int(rng.integers(0, 20)))
        assert o.sum_required() + o.sum_held() + o.reserve <= o.M


def test_round_robin_cursor_persists_between_attempts():
    o = OptResidency(3, 100, 1, 0)
    for r in range(3):
        o.admit(r, 5, 0, [])
    a = o.populate(2)
    b = o.populate(2)
    assert [x[0] for x in a] == [0, 1] and [x[0] for x in b] == [2, 0]
    assert [x[1] for x in a + b] == [0, 0, 0, 1]
    assert [x[2] for x in a + b] == [0, 1, 2, 3]                 # lowest free pool page first


def test_partial_boundary_page_is_never_optional():
    o = OptResidency(1, 10, 8, 0)
    o.admit(0, 8 * 3 + 5, 0, [])
    assert o.eligible[0] == 3
    o.populate(10)
    o.publish()
    assert len(o.held[0]) == 3
    assert o.lookup(0, 23) is not None and o.lookup(0, 24) is None


def _load_step_case():
    return shrink(WORKLOADS["mla128"], n_req=6, n_groups=1, hist_lo=6_000, hist_hi=6_000,
                  hist_cap=6_100, prefix_len=4_096, row_elems=8, d_qk=8, v_off=0, d_v=8,
                  n_heads=1, topk=256, hot_slots=512)


def test_dynamic_residency_resolves_ready_rows_and_keeps_outputs():
    """Figure 2 callout 1: exactly the union rows of ready pages resolve as
    resident, rows of pending pages do not, and outputs equal the run with
    no residency (the method is exact)."""
    w = shrink(_load_step_case(), n_req=3, hist_lo=900, hist_hi=900, hist_cap=960,
               prefix_len=512, topk=48, hot_slots=64, q_max=4, n_heads=2)
    outs = []
    for mode in ("off", "dyn"):
        hist = make_history(w, 0)
        hl = hist.hist_len
        o = HierOracle(oracle_config(w), [hist], hl)
        si = make_step_inputs(w, 0, 0, hl)
        for r, (rows, ages) in enumerate(make_hot_warm_set(w, 0, hl, si)):
            o.set_hot(0, r, rows, ages)
        opt = None
        if mode == "dyn":
            opt = OptResidency(w.n_req, 12, 32, 0)
            o.attach_residency(opt)
            for r in range(w.n_req):
                assert opt.admit(r, int(hl[r]), 0, []) == []
            opt.populate(7)
            opt.publish()
            pend = opt.populate(3)                       # pending, not yet published
            assert pend
        res = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
        if mode == "dyn":
            for r in range(w.n_req):
                rr = res.req[r]
                ready_rows = {u for u in rr.union if (u // 32) in opt.ready[r]}
                got = {u for u, c in zip(rr.union, rr.cls) if c == oracle.CLS_RESIDENT}
                assert got == ready_rows
                for (x, idx, _) in pend:
                    if x == r:
                        assert not any(u // 32 == idx for u in got)
                for j in range(w.q_max):
                    for i in range(w.topk):
                        code = int(rr.loc[j, i])
                        e = int(si.topk[r, j, i])
                        if code >= 0 and code >> 29 == oracle.RESIDENT:
                            idx = code & ((1 << 29) - 1)
                            assert idx == opt.held[r][e // 32] * 32 + e % 32
        res2 = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows)
        outs.append(res2.out)
    for key in outs[0]:
        assert np.array_equal(outs[0][key], outs[1][key])


@pytest.mark.slow
def test_load_step_host_share_follows_coverage():
    """§4.3.1 / Figure 6 / Table A1: with residency on, low load keeps most of
    the eligible history on the device and cuts the host-fetched share by an
    order of magnitude; a load rise reclaims it (coverage near zero, the share
    of the arm without residency); after completion, population restores it."""
    w = _load_step_case()
    hist = make_history(w, 0)
    hl = hist.hist_len
    P = 64
    eligible = int(hl[0]) // P
    required = 8
    pool = 2 * (eligible + required) + 4                 # two requests' history fits, not six
    opt = OptResidency(w.n_req, pool, P, 4)
    o = HierOracle(oracle_config(w), [hist], hl)
    o.attach_residency(opt)
    si = make_step_inputs(w, 0, 0, hl)
    warm = make_hot_warm_set(w, 0, hl, si)

    def share(active):
        for r in active:
            o.set_hot(0, r, *warm[r])
        o.requests = sorted(active)
        res = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
        u = sum(res.req[r].counts["union"] for r in active)
        m = sum(res.req[r].counts["union_miss"] for r in active)
        return m / u

    low = [0, 1]
    off = share(low)
    for r in low:
        assert opt.admit(r, int(hl[r]), required, []) == []
    while opt.populate(64):
        opt.publish()
    opt.publish()
    ready, elig = opt.coverage()
    assert ready == elig
    on_low = share(low)
    assert off > 0.1 and on_low < off / 10
    for r in range(2, w.n_req):                          # the load step
        got = opt.admit(r, int(hl[r]), required, [x for x in range(w.n_req) if opt.admitted[x]])
        assert got is not None
        opt.populate(64)
        opt.publish()
    ready, elig = opt.coverage()
    assert ready < 0.45 * elig                           # most history reclaimed
    for r in range(2, w.n_req):                          # load falls
        opt.complete(r)
    while opt.populate(64):
        opt.publish()
    opt.publish()
    ready, elig = opt.coverage()
    assert ready == elig
    assert share(low) < off / 10
