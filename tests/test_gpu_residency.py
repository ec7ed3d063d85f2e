"""Dynamic optional residency on the GPU vs the oracle ("Adaptive DHiSparse"
§3.1, eqs. 3-4; Figure 2), through the C ABI.

With every population copy published before a step, the library's page
tables (held pool page and ready flag per page index) equal the oracle's
exactly, and the step's lists, locations, slot tables and counters are
bit-exact, outputs within tolerance.  The pool starts poisoned with NaN, so a
location published before its copy completed would show in the outputs.
With publication left to the library (copies running beside the steps),
which rows resolve through the pool depends on timing, but outputs must
still equal the oracle's and every returned location must hold its row.
"""
import numpy as np
import pytest

import oracle
from tests.pair import assert_close, build_pair, run_lib_step
from tests.test_gpu_parity import _mla_small, compare_counts, compare_step
from workloads import make_step_inputs

pytestmark = pytest.mark.gpu

P = 64


def _dyn_pair(w, pool_pages, reserve, flags=2):
    pair = build_pair(w, lib_kw=dict(resident_cap=pool_pages * P, opt_page_rows=P, opt_reserve=reserve,
                                     flags=flags))
    opt = oracle.OptResidency(w.n_req, pool_pages, P, reserve)
    pair.orc.attach_residency(opt)
    return pair, opt


def _compare_pages(pair, opt, w):
    n_pages = w.hist_cap // P
    for r in range(w.n_req):
        held, ready = pair.lib.opt_pages(r, n_pages)
        oh, orr = opt.page_table(r, n_pages)
        assert held.tolist() == oh, ("held pages", r)
        assert ready.tolist() == orr, ("ready pages", r)
    info = pair.lib.opt_info()
    assert info["held_pages"] == opt.sum_held()
    assert info["required_pages"] == opt.sum_required()
    assert info["free_pages"] == len(opt.free)
    assert info["cursor"] == opt.cursor


def _exact_resident_hot(pair, g, r, topk_r):
    """Eqs. (11)-(12) for the pool and hot-cache locations: the row stored
    there is the selected original row.  (Staged rows are not read back: the
    arena is poisoned once the step's readers are done.)"""
    L = pair.lib.last_lists(g, r)
    loc = L["loc"].ravel()
    sel = np.flatnonzero((loc >= 0) & ((loc >> 29) != 1))
    if sel.size == 0:
        return 0
    rows = pair.lib.read_rows(g, loc[sel])
    hist = pair.lib_hists[g]
    plen = pair.w.prefix_len if pair.w.n_prefix > 0 else 0
    for x, e in zip(rows, topk_r.ravel()[sel]):
        e = int(e)
        want = hist.prefix[r % max(pair.w.n_prefix, 1), e] if e < plen else hist.tails[r, e - plen]
        assert np.array_equal(x, want), ("row at location differs", r, e)
    return int(((loc[sel] >> 29) == 2).sum())


def _step_all(pair, w, step, check_exact=False):
    for g in range(w.n_groups):
        si = make_step_inputs(w, g, step, pair.hist_len)
        res = pair.orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
        out = run_lib_step(pair, g, si)
        compare_step(pair, g, si, res, out)
        compare_counts(pair, g, res)
        if check_exact:
            for r in range(w.n_req):
                _exact_resident_hot(pair, g, r, si.topk[r])
        yield g, res


def test_dynamic_residency_parity():
    w = _mla_small()
    pair, opt = _dyn_pair(w, pool_pages=300, reserve=2)
    hl = pair.hist_len
    lib = pair.lib
    # low load: three requests admitted, their whole eligible history populated
    for r in range(3):
        assert lib.opt_admit(r, 4) == 0
        assert opt.admit(r, int(hl[r]), 4, []) == []
    for _ in range(3):
        assert lib.opt_populate(100) == len(opt.populate(100))
    lib.opt_publish(wait=True)
    opt.publish()
    _compare_pages(pair, opt, w)
    ready, elig = opt.coverage()
    assert ready == elig > 0
    list(_step_all(pair, w, 0, check_exact=True))
    _, last = lib.stats(0)
    assert last["union_resident"] > 0
    # a request with a large required allocation: deficit, whole-request reclaim (eq. 4)
    order = [1, 0, 2]
    q = lib.opt_admit(3, 40, order)
    got = opt.admit(3, int(hl[3]), 40, order)
    assert got is not None and q == len(got) >= 1
    _compare_pages(pair, opt, w)
    # an admission nothing can cover waits and changes nothing
    assert lib.opt_admit(4, 10_000, [0, 1, 2, 3]) is None
    assert opt.admit(4, int(hl[4]), 10_000, [0, 1, 2, 3]) is None
    assert lib.opt_info()["admissions_waited"] == 1
    # bounded round-robin repopulation, then a step over the new state
    for bound in (7, 60, 1):
        assert lib.opt_populate(bound) == len(opt.populate(bound))
    lib.opt_publish(wait=True)
    opt.publish()
    _compare_pages(pair, opt, w)
    list(_step_all(pair, w, 1, check_exact=True))
    # completion releases capacity; repopulation reuses the withdrawn pages
    lib.opt_complete(0)
    opt.complete(0)
    _compare_pages(pair, opt, w)
    while True:
        n = lib.opt_populate(50)
        assert n == len(opt.populate(50))
        if n == 0:
            break
    lib.opt_publish(wait=True)
    opt.publish()
    _compare_pages(pair, opt, w)
    list(_step_all(pair, w, 2, check_exact=True))
    info = lib.opt_info()
    assert info["pages_reclaimed"] > 0 and info["requests_reclaimed"] == q
    assert info["bytes_populated"] == info["pages_populated"] * P * 2 * w.row_elems * w.n_groups
    lib.close()


def test_dynamic_residency_with_follower_layers():
    """One selection feeding two payload layers: the follower reads its own
    pool through the leader's resident locations."""
    w = _mla_small(n_groups=2, plan_share=2, n_arenas=2)
    pair, opt = _dyn_pair(w, pool_pages=200, reserve=0)
    hl = pair.hist_len
    for r in range(w.n_req):
        assert pair.lib.opt_admit(r, 0) == 0
        opt.admit(r, int(hl[r]), 0, [])
    assert pair.lib.opt_populate(150) == len(opt.populate(150))
    pair.lib.opt_publish(wait=True)
    opt.publish()
    _compare_pages(pair, opt, w)
    list(_step_all(pair, w, 0))
    pair.lib.close()


def test_dynamic_residency_async_publication():
    """Copies run beside the steps and are published by the steps themselves:
    outputs equal the oracle's (placement never changes the result) and every
    location holds its row.  Pages withdrawn while a step that resolved them
    is still in flight are rewritten only after that step's attention."""
    import torch
    from tests.pair import to_device
    w = _mla_small(n_groups=1)
    pair = build_pair(w, lib_kw=dict(resident_cap=260 * P, opt_page_rows=P, opt_reserve=0, flags=2))
    lib, orc = pair.lib, pair.orc
    hl = pair.hist_len
    for r in range(w.n_req):
        assert lib.opt_admit(r, 0) == 0
    seen_resident = 0
    for step in range(6):
        lib.opt_populate(40)
        si = make_step_inputs(w, 0, step, hl)
        res = orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
        d = to_device(si)
        out_t = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
        lib.verify_step(0, d["queries"], d["topk"], d["causal"], d["ring"], out_t)
        if step == 3:
            # withdraw request 2's pages while this step may still read them, and
            # hand the same pool pages (lowest free first) to other requests
            lib.opt_complete(2)
            lib.opt_populate(40)
        torch.cuda.synchronize()
        out = out_t.cpu().numpy().view(np.uint16)
        for (r, j), ref in res.out.items():
            assert_close(out[r, j], ref, "out step=%d r=%d j=%d" % (step, r, j))
        if step != 3:
            for r in range(w.n_req):
                L = lib.last_lists(0, r)
                assert L["union_rows"].tolist() == res.req[r].union
                _exact_resident_hot(pair, 0, r, si.topk[r])
        _, last = lib.stats(0)
        seen_resident += last["union_resident"]
    lib.opt_publish(wait=True)
    info = lib.opt_info()
    assert info["pending_pages"] == 0 and info["ready_pages"] == info["held_pages"]
    assert seen_resident > 0
    lib.close()
