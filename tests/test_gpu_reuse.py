"""Shared KV sources on the GPU vs the oracle ("Adaptive DHiSparse" §2,
physical-source sharing; §3.2), through the C ABI.

One layer group is one physical source.  Per step: the producing (Full)
layer resolves and attends; a Reuse layer attends with its own queries over
that selection (kv_hier_verify_reuse); a Reindex layer resolves a fresh top-k
against the state the earlier layer left (verify_step without ring rows);
another Reuse layer reads the fresh selection.  Lists, slot tables and
counters are bit-exact, outputs within tolerance, over two steps with a
commit; the arena is poisoned between its last reader and its next fetch.
"""
import numpy as np
import pytest

from tests.pair import assert_close, build_pair, to_device
from tests.test_gpu_parity import _mla_small, compare_counts, compare_step
from workloads import make_accepted, make_step_inputs

pytestmark = pytest.mark.gpu


def _out(w):
    import torch
    return torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")


def _bits(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint16)


def _resolve(pair, g, queries, topk, causal, ring):
    import torch
    w = pair.w
    dev = torch.device("cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = _out(w)
    pair.lib.verify_step(g, t(queries.view(np.int16)), t(topk), t(causal),
                         None if ring is None else t(ring.view(np.int16)), out)
    return _bits(out)


def _reuse(pair, g, queries, causal):
    import torch
    dev = torch.device("cuda")
    out = _out(pair.w)
    pair.lib.verify_reuse(g, torch.from_numpy(np.ascontiguousarray(queries.view(np.int16))).to(dev),
                          torch.from_numpy(np.ascontiguousarray(causal)).to(dev), out)
    return _bits(out)


class _Sel:
    def __init__(self, topk, causal_pos):
        self.topk, self.causal_pos = topk, causal_pos


def _check_reuse(pair, g, q, causal, what):
    ref = pair.orc.verify_reuse(g, q, n_threads=8)
    got = _reuse(pair, g, q, causal)
    for (r, j), v in ref.items():
        assert_close(got[r, j], v, "%s r=%d j=%d" % (what, r, j))
    for r in range(pair.w.n_req):
        for j in range(pair.w.q_max):
            if int(causal[r, j]) < 0:
                assert (got[r, j] == 0).all()


@pytest.mark.parametrize("rows", ["mla576", "rows288"])
def test_shared_source_full_reuse_reindex_reuse(rows):
    from hierarchical_sparse_kv_verify_amd import KVHierError
    if rows == "mla576":
        w = _mla_small(n_groups=1)
    else:  # the 288-B rows of the shared-source measurement, 128 heads
        w = _mla_small(n_groups=1, row_elems=144, d_qk=144, v_off=0, d_v=128, n_heads=128)
    pair = build_pair(w, lib_kw=dict(flags=2, n_chunks=2))
    orc, lib = pair.orc, pair.lib
    with pytest.raises(KVHierError) as ei:            # nothing to reuse yet
        _reuse(pair, 0, make_step_inputs(w, 0, 0, pair.hist_len).queries,
               make_step_inputs(w, 0, 0, pair.hist_len).causal_pos)
    assert ei.value.code == -4
    n = pair.hist_len.copy()
    for step in range(2):
        si = make_step_inputs(w, 0, 10 * step, n)                 # Full: produces the rows, selects
        res = orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
        out = _resolve(pair, 0, si.queries, si.topk, si.causal_pos, si.block_rows)
        compare_step(pair, 0, si, res, out)
        compare_counts(pair, 0, res)
        _check_reuse(pair, 0, make_step_inputs(w, 0, 10 * step + 1, n).queries, si.causal_pos, "reuse A")
        sb = make_step_inputs(w, 0, 10 * step + 2, n)             # Reindex: half of it new
        topk_b = si.topk.copy()
        topk_b[:, :, ::2] = sb.topk[:, :, ::2]
        res_b = orc.verify_step(0, topk_b, si.causal_pos, sb.queries, None, n_threads=8)
        out_b = _resolve(pair, 0, sb.queries, topk_b, si.causal_pos, None)
        compare_step(pair, 0, _Sel(topk_b, si.causal_pos), res_b, out_b)
        compare_counts(pair, 0, res_b)
        _, last = lib.stats(0)
        assert last["union_miss"] < 0.5 * last["union_rows"]         # only rows absent from the state
        _check_reuse(pair, 0, make_step_inputs(w, 0, 10 * step + 3, n).queries, si.causal_pos, "reuse B")
        acc = make_accepted(w, step, si.k_active)
        orc.commit(acc)
        lib.commit(acc)
        n = n + 1 + acc
        with pytest.raises(KVHierError) as ei:                    # the step's selections ended
            _reuse(pair, 0, si.queries, si.causal_pos)
        assert ei.value.code == -4
    lib.close()


def test_reuse_needs_its_staged_payload():
    """Two sources staging into one arena: once the second source has fetched,
    the first one's staged rows are gone and its Reuse is refused; the second
    source's Reuse matches the oracle."""
    from hierarchical_sparse_kv_verify_amd import KVHierError
    w = _mla_small(n_groups=2, n_arenas=1)
    pair = build_pair(w, lib_kw=dict(flags=2))
    sis = []
    for g in range(2):
        si = make_step_inputs(w, g, 0, pair.hist_len)
        res = pair.orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
        out = _resolve(pair, g, si.queries, si.topk, si.causal_pos, si.block_rows)
        compare_step(pair, g, si, res, out)
        sis.append(si)
    with pytest.raises(KVHierError) as ei:
        _reuse(pair, 0, sis[0].queries, sis[0].causal_pos)
    assert ei.value.code == -4
    _check_reuse(pair, 1, make_step_inputs(w, 1, 5, pair.hist_len).queries, sis[1].causal_pos, "reuse g1")
    pair.lib.close()


def test_reuse_on_follower_layers():
    """A follower layer of a plan-sharing set reuses its own payload through
    the leader's locations."""
    w = _mla_small(n_groups=2, plan_share=2, n_arenas=2)
    pair = build_pair(w)
    sis = []
    for g in range(2):
        si = make_step_inputs(w, g, 0, pair.hist_len)
        res = pair.orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
        out = _resolve(pair, g, si.queries, si.topk, si.causal_pos, si.block_rows)
        compare_step(pair, g, si, res, out)
        sis.append(si)
    for g in (1, 0):
        _check_reuse(pair, g, make_step_inputs(w, g, 9, pair.hist_len).queries, sis[g].causal_pos,
                     "reuse g%d" % g)
    pair.lib.close()


@pytest.mark.parametrize("n_heads", [128, 96])
def test_rows288_128_head_workgroups_step_and_reuse(n_heads):
    """Launches of at least 256 workgroups over 288-B rows take one workgroup
    of 128 heads per query (four head blocks x two row halves, each row
    gathered once; 96 heads leave the last block masked): 32 requests x 8
    queries as one request chunk, a resolving step and a Reuse layer over its
    selection, against the oracle; pads, invalid entries and ragged tiles."""
    w = _mla_small(n_req=32, n_groups=1, row_elems=144, d_qk=144, v_off=0, d_v=128, n_heads=n_heads,
                   hist_lo=1500, hist_hi=2000, hist_cap=2100, prefix_len=1024, topk=256, hot_slots=512,
                   ring_window=48)
    pair = build_pair(w, lib_kw=dict(n_chunks=1))
    info = pair.lib.info
    assert info["attn_head_groups"] == 1 and info["attn_reuse_head_groups"] == 1, info
    assert info["attn_splits"] == 1, info
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
    out = _resolve(pair, 0, si.queries, si.topk, si.causal_pos, si.block_rows)
    compare_step(pair, 0, si, res, out)
    compare_counts(pair, 0, res)
    _check_reuse(pair, 0, make_step_inputs(w, 0, 1, pair.hist_len).queries, si.causal_pos, "reuse 128-head")
    pair.lib.close()
