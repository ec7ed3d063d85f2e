"""Selection patterns of the resolver-cost measurement ("Adaptive DHiSparse"
§4.3.3, Fig. 8a: shared, partial and disjoint selections across a request's
verification queries) and what the oracle's resolution makes of them.

Identical lists need one payload (|U| = k, every union row fetched once from
a cold cache); disjoint lists need Q payloads (|U| = Q k); a retained cache
holding every row of an earlier identical call fetches nothing when the union
fits the B slots, and |U| - B rows when it does not (§3.2: misses deduplicated
within the request, a union larger than the hot cache overflows to staging).
"""
import pytest

from oracle import HierOracle
from tests.oracle_helpers import oracle_config
from tests.test_oracle_pins import _tiny_case
from workloads import make_history, make_step_inputs


def _case(**kw):
    return _tiny_case(n_req=2, q_max=4, topk=24, hot_slots=40, pad_frac=0.0, invalid_frac=0.0, var_k=False,
                      empty_slot_frac=0.0, **kw)


@pytest.mark.parametrize("pattern", ["shared", "partial", "disjoint"])
def test_pattern_union_sizes(pattern):
    kw = dict(shared=dict(f_sh=1.0), partial=dict(f_sh=0.5), disjoint=dict(f_sh=0.0, disjoint=True))[pattern]
    w = _case(**kw)
    hist = make_history(w, 0)
    si = make_step_inputs(w, 0, 0, hist.hist_len)
    for r in range(w.n_req):
        lists = [set(int(x) for x in si.topk[r, j]) for j in range(w.q_max)]
        assert all(len(s) == w.topk for s in lists)               # distinct entries within a list
        union = set().union(*lists)
        if pattern == "shared":
            assert all(s == lists[0] for s in lists) and len(union) == w.topk
        elif pattern == "disjoint":
            assert len(union) == w.q_max * w.topk
            for a in range(w.q_max):
                for b in range(a + 1, w.q_max):
                    assert not (lists[a] & lists[b])
        else:
            core = set.intersection(*lists)
            assert len(core) >= w.topk // 2 and w.topk < len(union) < w.q_max * w.topk


@pytest.mark.parametrize("pattern,expect_cold,expect_retained", [
    ("shared", lambda w: w.topk, lambda w: 0),
    ("disjoint", lambda w: w.q_max * w.topk, lambda w: w.q_max * w.topk - w.hot_slots),
])
def test_cold_and_retained_fetch_counts(pattern, expect_cold, expect_retained):
    kw = dict(shared=dict(f_sh=1.0), disjoint=dict(f_sh=0.0, disjoint=True))[pattern]
    w = _case(**kw)
    assert w.topk <= w.hot_slots < w.q_max * w.topk
    hist = make_history(w, 0)
    hl = hist.hist_len
    o = HierOracle(oracle_config(w), [hist], hl)                 # empty hot caches
    si = make_step_inputs(w, 0, 0, hl)
    cold = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
    warm = o.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=None)
    for r in range(w.n_req):
        assert len(cold.req[r].miss) == expect_cold(w)
        assert len(set(cold.req[r].miss)) == len(cold.req[r].miss)   # each row fetched once
        assert len(warm.req[r].miss) == expect_retained(w)
        # the rows the first call promoted are hits now; nothing else is
        promoted = set(int(u) for u in cold.req[r].miss[: len(cold.req[r].victims)])
        hits = set(warm.req[r].union) - set(warm.req[r].miss)
        assert hits == promoted
