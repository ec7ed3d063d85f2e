"""GPU parity at the full shapes the benchmark runs, through the C ABI.

Each test builds the workload at its configured size, runs the library in
the launch configuration ``bench.py`` times (automatic request chunks), and
compares sampled requests with the oracle: one request from every request
chunk, lists, classes, victims, locations and slot tables bit-exact, sampled
queries within |gpu - ref| <= 2e-2 + 1e-2 |ref|; whole-step counters are
checked for consistency.  Host generation of the largest workload takes
seconds per prefix, so these tests carry their own time limits.
"""
import numpy as np
import pytest

from tests.pair import build_pair, run_lib_step
from tests.test_gpu_parity import _exact_vs_topk, compare_step
from workloads import WORKLOADS, make_step_inputs, shrink

pytestmark = pytest.mark.gpu


def _check_layout(pair, bounds):
    """The handle's request chunks are the expected ones (their count through
    kv_hier_info; the automatic layout rule is pinned in the parity suite),
    and the sampled requests cover every chunk."""
    assert pair.lib.info["n_chunks"] == len(bounds) - 1, (pair.lib.info, bounds)
    reqs = pair.orc.requests
    for a, b in zip(bounds, bounds[1:]):
        assert any(a <= r < b for r in reqs), (a, b, reqs)


def _check_group(pair, g, si, reqs, queries_per_req, n_threads=16):
    w = pair.w
    attend = {(r, j) for r in reqs for j in queries_per_req}
    res = pair.orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows, attend=attend,
                               n_threads=n_threads)
    out = run_lib_step(pair, g, si)
    compare_step(pair, g, si, res, out, requests=reqs)
    for r in reqs:
        _exact_vs_topk(pair, g, r, si.topk[r])
    _, last = pair.lib.stats(g)
    assert last["active_queries"] == int(si.k_active.sum())
    assert last["fetched_bytes"] == last["union_miss"] * 2 * w.row_elems
    assert last["union_miss"] == last["promoted"] + last["overflow"]
    return last


@pytest.mark.timeout(400)
def test_full_size_mla32_sampled():
    """32 requests x 32,768 rows, one group, 64 heads, Q = 8, k = 2048, B = 4096
    at 80% hits: two request chunks whose keys are split and merged."""
    w = WORKLOADS["mla32"]
    reqs = [0, 8, 16, 24, 31]
    pair = build_pair(w, oracle_requests=reqs)
    _check_layout(pair, [0, 16, 32])
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    last = _check_group(pair, 0, si, reqs, (0, 4, 7))
    assert last["selections"] == w.n_req * w.q_max * w.topk
    assert 0.15 < last["union_miss"] / last["union_rows"] < 0.25
    pair.lib.close()


@pytest.mark.timeout(600)
def test_full_size_mla128_resident_rho09_sampled():
    """The residency sweep's last point: 128 requests x ~100K rows, 4 layer
    groups, 90% of every request's rows resident (static map): the resident
    tier takes most union rows and the host fetch shrinks ~10x; sampled
    requests of every chunk exact against the oracle in every group."""
    w = shrink(WORKLOADS["mla128_res"], rho=0.9)
    reqs = [0, 16, 48, 80, 112, 127]
    pair = build_pair(w, rho=0.9, oracle_requests=reqs)
    _check_layout(pair, [0, 32, 64, 96, 128])
    for g in range(w.n_groups):
        si = make_step_inputs(w, g, 0, pair.hist_len)
        last = _check_group(pair, g, si, reqs, (0, 7))
        assert last["union_resident"] > 0.8 * last["union_rows"]
        assert last["union_miss"] < 0.03 * last["union_rows"]
    pair.lib.close()


@pytest.mark.timeout(900)
def test_full_size_mla512_sampled():
    """512 requests x ~500K rows over 16 shared host prefixes, 128 heads (two
    64-head workgroups per query), Q = 4, k = 2048, B = 2048, W = 64, only the
    shared core warm (~38% of distinct rows miss, most overflow the 2048
    slots): the five-chunk layout (128, 128, 128, 64, 64) without key splits.
    One request of every chunk and both ends, from different prefixes."""
    w = WORKLOADS["mla512"]
    reqs = [0, 65, 194, 323, 420, 485, 511]       # prefixes 0-5 and 15
    pair = build_pair(w, oracle_requests=reqs)
    info = pair.lib.info
    _check_layout(pair, [0, 128, 256, 384, 448, 512])
    assert info["attn_splits"] == 1 and info["attn_head_groups"] == 2, info
    assert len({r % w.n_prefix for r in reqs}) == len(reqs)
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    last = _check_group(pair, 0, si, reqs, (0, 3))
    assert last["overflow"] > last["promoted"]
    assert 0.3 < last["union_miss"] / last["union_rows"] < 0.45
    pair.lib.close()


@pytest.mark.timeout(600)
def test_full_size_ds_shared_select_and_reuse_sampled():
    """The shared-source measurement's shape: 128 requests x ~100K rows of 288 B
    (one prefix), 128 heads, Q = 4, k = 512, B = 2048, W = 64.  A selecting
    layer over four 32-request chunks (64 heads per attention workgroup, 256
    workgroups per chunk) and a Reuse layer over all 128 requests (128 heads
    per workgroup, each row gathered once per query), sampled requests of
    every chunk against the oracle."""
    from tests.pair import assert_close
    from tests.test_gpu_reuse import _reuse
    w = shrink(WORKLOADS["ds_shared"], n_groups=1, n_arenas=1)
    reqs = [0, 40, 77, 101, 127]
    pair = build_pair(w, oracle_requests=reqs)
    info = pair.lib.info
    _check_layout(pair, [0, 32, 64, 96, 128])
    assert info["attn_splits"] == 1 and info["attn_head_groups"] == 2 and info["attn_reuse_head_groups"] == 1, info
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    _check_group(pair, 0, si, reqs, (0, 3))
    q = make_step_inputs(w, 0, 1, pair.hist_len).queries
    ref = pair.orc.verify_reuse(0, q, attend={(r, j) for r in reqs for j in (0, 1, 3)}, n_threads=16)
    got = _reuse(pair, 0, q, si.causal_pos)
    for (r, j), v in ref.items():
        assert_close(got[r, j], v, "ds_shared reuse r=%d j=%d" % (r, j))
    pair.lib.close()
