"""GPU path vs oracle, element by element, through the C ABI.

Integer results (union, classes, missing rows, victims, locations, slot
tables, counters, committed host rows) must be bit-exact; attention outputs
within |gpu - ref| <= 2e-2 + 1e-2 |ref| (bf16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest

from tests.pair import assert_close, build_pair, run_lib_step
from workloads import WORKLOADS, make_accepted, make_step_inputs, shrink

pytestmark = pytest.mark.gpu

TIER_TO_CLS = {2: 0, 0: 1, 1: 2, 3: 3}     # resident, hot, staged(miss), ring(tail) -> oracle class


def _cls_of(codes):
    return [TIER_TO_CLS[int(c) >> 29] for c in codes]


def compare_step(pair, g, si, res, out_bits, requests=None, check_out=True):
    lib = pair.lib
    w = pair.w
    reqs = requests if requests is not None else pair.orc.requests
    for r in reqs:
        L = lib.last_lists(g, r)
        rr = res.req[r]
        if not rr.active:
            assert L["n_union"] == 0 and (L["loc"] == -1).all(), r
            continue
        assert L["union_rows"].tolist() == rr.union, ("union", r)
        assert _cls_of(L["union_loc"]) == rr.cls, ("classes", r)
        assert L["miss_rows"].tolist() == rr.miss, ("miss", r)
        assert L["victims"].tolist() == rr.victims, ("victims", r)
        np.testing.assert_array_equal(L["loc"], rr.loc, err_msg="loc r=%d" % r)
        rows, lu = lib.slot_table(g, r)
        orows, olu = pair.orc.slot_table(g, r)
        np.testing.assert_array_equal(rows, orows, err_msg="slot rows r=%d" % r)
        np.testing.assert_array_equal(lu, olu, err_msg="slot stamps r=%d" % r)
    if check_out:
        for (r, j), ref in res.out.items():
            assert_close(out_bits[r, j], ref, "out r=%d j=%d" % (r, j))
        for r in reqs:
            for j in range(w.q_max):
                if int(si.causal_pos[r, j]) < 0:
                    assert (out_bits[r, j] == 0).all(), ("inactive query output", r, j)


def compare_counts(pair, g, res):
    _, last = pair.lib.stats(g)
    tot = {}
    for rr in res.req.values():
        for k2, v in rr.counts.items():
            tot[k2] = tot.get(k2, 0) + v
    for key, lk in (("selections", "selections"), ("pads", "pads"), ("invalid", "invalid"),
                    ("union", "union_rows"), ("union_resident", "union_resident"),
                    ("union_hot", "union_hot"), ("union_miss", "union_miss"),
                    ("promoted", "promoted"), ("overflow", "overflow"),
                    ("sel_resident", "sel_resident"), ("sel_hot", "sel_hot"), ("sel_miss", "sel_miss"),
                    ("union_tail", "union_tail"), ("sel_tail", "sel_tail"),
                    ("queries", "active_queries")):
        assert last[lk] == tot.get(key, 0), (key, last[lk], tot.get(key, 0))
    assert last["fetched_bytes"] == last["union_miss"] * 2 * pair.w.row_elems


def check_exactness(pair, g, r):
    """Eq. (11)-(12): the row at every returned location is the selected original row."""
    L = pair.lib.last_lists(g, r)
    loc = L["loc"].ravel()
    sel = np.flatnonzero(loc >= 0)
    if sel.size == 0:
        return
    rows = pair.lib.read_rows(g, loc[sel])
    hist = pair.lib_hists[g]
    plen = pair.w.prefix_len if pair.w.n_prefix > 0 else 0
    # the list entries themselves come from the oracle's inputs (topk); rebuild them
    return rows, sel, hist, plen


def _exact_vs_topk(pair, g, r, topk_r):
    out = check_exactness(pair, g, r)
    if out is None:
        return
    rows, sel, hist, plen = out
    ent = topk_r.ravel()[sel]
    for x, e in zip(rows, ent):
        e = int(e)
        want = hist.prefix[r % max(pair.w.n_prefix, 1), e] if e < plen else hist.tails[r, e - plen]
        assert np.array_equal(x, want), ("row at location differs", r, e)


def _tiny(**kw):
    base = shrink(WORKLOADS["tiny"], pad_frac=0.02, invalid_frac=0.01, empty_slot_frac=0.05)
    return shrink(base, **kw)


def test_tiny_parity_and_exactness():
    w = _tiny()
    pair = build_pair(w)
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows)
    out = run_lib_step(pair, 0, si)
    compare_step(pair, 0, si, res, out)
    compare_counts(pair, 0, res)
    _exact_vs_topk(pair, 0, 0, si.topk[0])
    pair.lib.close()


def test_tiny_multi_step_with_commits():
    w = _tiny(var_k=True)
    pair = build_pair(w)
    n = pair.hist_len.copy()
    for step in range(5):
        si = make_step_inputs(w, 0, step + 1, n)
        res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows)
        out = run_lib_step(pair, 0, si)
        compare_step(pair, 0, si, res, out)
        compare_counts(pair, 0, res)
        acc = make_accepted(w, step, si.k_active)
        pair.orc.commit(acc)
        pair.lib.commit(acc)
        pair.lib.sync()
        n = n + 1 + acc
        assert pair.lib.hist_len().tolist() == n.tolist()
        # the committed rows now have their host copy, identical on both sides
        for r in range(w.n_req):
            np.testing.assert_array_equal(pair.lib.host_rows(0, 1, r)[: n[r]], pair.orc.hist[0].tails[r, : n[r]])
    pair.lib.close()


def _mla_small(**kw):
    base = shrink(WORKLOADS["mla32"], n_req=6, n_groups=2, hist_lo=5000, hist_hi=6000, hist_cap=6100,
                  n_prefix=1, prefix_len=4096, topk=512, hot_slots=1024, ring_window=128,
                  q_max=8, f_sh=0.75, hit_rate=0.8, pad_frac=0.02, invalid_frac=0.01,
                  empty_slot_frac=0.03, var_k=True)
    return shrink(base, **kw)


@pytest.mark.parametrize("n_chunks,fetch_cus", [(1, 0), (2, 0), (3, 0), (2, 16)])
def test_mla_two_groups_two_steps(n_chunks, fetch_cus):
    w = _mla_small()
    pair = build_pair(w, lib_kw=dict(n_chunks=n_chunks, fetch_cus=fetch_cus))
    assert pair.lib.info["attn_row_order"] == 0, pair.lib.info    # 512-entry lists keep selection order
    n = pair.hist_len.copy()
    for step in range(2):
        sis = []
        for g in range(w.n_groups):
            si = make_step_inputs(w, g, step, n)
            res = pair.orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
            out = run_lib_step(pair, g, si)
            compare_step(pair, g, si, res, out)
            compare_counts(pair, g, res)
            sis.append(si)
        acc = make_accepted(w, step, sis[0].k_active)
        pair.orc.commit(acc)
        pair.lib.commit(acc)
        n = n + 1 + acc
    pair.lib.close()


@pytest.mark.parametrize("n_heads,n_chunks,head_groups", [(128, 2, 2), (16, 1, 1), (64, 3, 1), (96, 2, 2),
                                                          (256, 2, 4), (48, 1, 1)])
def test_288_byte_rows_two_groups_two_steps(n_heads, n_chunks, head_groups):
    """Rows of 144 bf16 (288 B, the bytes per missed selection of the pages'
    DeepSeek configuration, Table 3): K = all 144 elements, V = the first 128.
    Up to 32 heads the four waves of a head block split the key width (nine
    16-dim k-steps: the last wave takes none) and a row's 18 chunks leave
    gather lanes idle; above, the narrow-row kernel takes 64 heads per
    workgroup at this size (two head blocks x two row halves, the last block
    partly masked at 48 and 96 heads), rows moved by DMA in the chunk-major
    layout, pads and the ragged last tile masked.  Two groups, two steps with
    a commit, key splits at this size."""
    w = _mla_small(row_elems=144, d_qk=144, v_off=0, d_v=128, n_heads=n_heads)
    pair = build_pair(w, lib_kw=dict(n_chunks=n_chunks))
    assert pair.lib.info["attn_splits"] > 1
    assert pair.lib.info["attn_head_groups"] == head_groups, pair.lib.info
    n = pair.hist_len.copy()
    for step in range(2):
        sis = []
        for g in range(w.n_groups):
            si = make_step_inputs(w, g, step, n)
            res = pair.orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
            out = run_lib_step(pair, g, si)
            compare_step(pair, g, si, res, out)
            compare_counts(pair, g, res)
            sis.append(si)
        acc = make_accepted(w, step, sis[0].k_active)
        pair.orc.commit(acc)
        pair.lib.commit(acc)
        n = n + 1 + acc
    pair.lib.close()


def test_plan_shared_by_follower_layers():
    """Follower-layer reuse of one plan: groups 0-1 and 2-3 each form a set fed
    by one selection.  The leader resolves once and fetches for both layers;
    the follower attends over its own payload through the leader's locations.
    Every layer matches the oracle, which resolves each group on its own from
    identical selections and warm sets, over two steps with a commit."""
    from hierarchical_sparse_kv_verify_amd import KVHierError
    w = _mla_small(n_groups=4, plan_share=2, n_arenas=2)
    pair = build_pair(w)
    n = pair.hist_len.copy()
    for step in range(2):
        sis = []
        for g in range(w.n_groups):
            si = make_step_inputs(w, g, step, n)
            res = pair.orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
            out = run_lib_step(pair, g, si)
            compare_step(pair, g, si, res, out)
            compare_counts(pair, g, res)
            sis.append(si)
        if step == 0:
            # a follower whose leader has not stepped again is refused
            with pytest.raises(KVHierError) as ei:
                run_lib_step(pair, 1, sis[1])
            assert ei.value.code == -4
        acc = make_accepted(w, step, sis[0].k_active)
        pair.orc.commit(acc)
        pair.lib.commit(acc)
        n = n + 1 + acc
    pair.lib.close()


@pytest.mark.parametrize("n_heads,groups", [(128, 2), (256, 4), (96, 2)])
def test_mla_many_heads_split_keys(n_heads, groups):
    """Head groups of 64 (the last one partly masked at 96 heads) and key
    splits merged by the combine pass."""
    w = _mla_small(n_req=2, n_groups=1, n_heads=n_heads, q_max=4, topk=1024, ring_window=64,
                   n_prefix=2, hot_slots=2048, var_k=False)
    pair = build_pair(w)
    assert pair.lib.info["attn_head_groups"] == groups and pair.lib.info["attn_splits"] > 1, pair.lib.info
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
    out = run_lib_step(pair, 0, si)
    compare_step(pair, 0, si, res, out)
    pair.lib.close()


@pytest.mark.parametrize("n_heads", [32, 16, 8, 48])
def test_mla_one_head_block_split_keys(n_heads):
    """Absorbed-MLA rows with few heads: at most 32 heads take one 32-head
    block per workgroup (four waves, eight rows of every tile per wave), 48
    heads two blocks; heads past H masked, key splits merged by the combine
    pass."""
    w = _mla_small(n_req=2, n_groups=1, n_heads=n_heads, q_max=4, topk=1024, ring_window=64,
                   n_prefix=2, hot_slots=2048, var_k=True)
    pair = build_pair(w)
    assert pair.lib.info["attn_head_groups"] == 1 and pair.lib.info["attn_splits"] > 1
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
    out = run_lib_step(pair, 0, si)
    compare_step(pair, 0, si, res, out)
    pair.lib.close()


@pytest.mark.parametrize("topk,window,rows,n_req", [(8, 8, 576, 3), (40, 16, 576, 3), (3, 64, 576, 3),
                                                    (8, 8, 144, 3), (40, 16, 144, 3), (3, 64, 144, 3),
                                                    (50, 20, 144, 32), (3, 64, 144, 32)])
def test_mla_short_lists(topk, window, rows, n_req):
    """Lists and windows that fill one partial tile, or two with a ragged
    second one: the tile pipeline's first tiles are also its last (DMA of
    tiles past the range reads the zero row).  Absorbed-MLA rows, and 288-B
    rows at 128 heads (64-head workgroups with key splits at 3 requests;
    128-head workgroups at 32 requests x 8 queries)."""
    lay = {} if rows == 576 else dict(row_elems=144, d_qk=144, v_off=0, d_v=128, n_heads=128)
    w = _mla_small(n_req=n_req, n_groups=1, q_max=2 if n_req == 3 else 8, topk=topk, ring_window=window,
                   ring_page=8, hot_slots=64, var_k=True, **lay)
    pair = build_pair(w, lib_kw=dict(n_chunks=1) if n_req == 32 else None)
    if n_req == 32:
        assert pair.lib.info["attn_head_groups"] == 1, pair.lib.info
    for step in range(2):
        si = make_step_inputs(w, 0, step, pair.hist_len)
        res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
        out = run_lib_step(pair, 0, si)
        compare_step(pair, 0, si, res, out)
        compare_counts(pair, 0, res)
    pair.lib.close()


@pytest.mark.parametrize("n_req,n_heads,q_max,chunks,splits", [
    (128, 64, 8, [0, 32, 64, 96, 128], 1),            # quarters of one GPU wave each
    (128, 128, 8, [0, 32, 64, 96, 112, 128], 1),      # halves of the last quarter still fill the GPU
    (256, 64, 8, [0, 64, 128, 192, 224, 256], 1),     # the same with 64 heads and twice the requests
    (64, 64, 4, [0, 16, 32, 48, 64], 4),              # quarters under a wave: key splits (17 tiles)
    (32, 64, 8, [0, 16, 32], 2),                      # fewer than 64 requests: two chunks
])
def test_automatic_chunk_layout(n_req, n_heads, q_max, chunks, splits):
    """The automatic request chunks of the fetch/attention pipeline, read back
    through kv_hier_info, and one step over them against the oracle."""
    from hierarchical_sparse_kv_verify_amd import KVHier
    from tests.pair import lib_config
    w = _mla_small(n_req=n_req, n_groups=1, n_heads=n_heads, q_max=q_max, topk=512, ring_window=32,
                   hot_slots=1024, hist_lo=900, hist_hi=1000, hist_cap=1100, prefix_len=256, var_k=True)
    lib = KVHier(**lib_config(w))
    info = lib.info
    lib.close()
    assert info["n_chunks"] == len(chunks) - 1
    assert info["attn_splits"] == splits
    assert info["attn_head_groups"] == (n_heads + 63) // 64
    # the first and last request of every chunk against the oracle
    reqs = sorted({x for a, b in zip(chunks, chunks[1:]) for x in (a, b - 1)})
    pair = build_pair(w, oracle_requests=reqs)
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
    out = run_lib_step(pair, 0, si)
    compare_step(pair, 0, si, res, out, requests=reqs)
    pair.lib.close()


def test_maximum_queries_hot_slots_and_plan_passes():
    """The largest shapes create accepts: Q = 32 verification queries, B = 16384
    hot slots, and Q*k = 38,400 list entries, whose location codes leave the
    resolution's LDS row bitmap about 38K rows, so a ~100K-row history is
    resolved in three passes over row ranges (union ranks, probe and staging
    order carried across passes); the victim choice sorts 16384 slots."""
    w = _tiny(n_req=2, q_max=32, topk=1200, hot_slots=16384, hist_lo=99000, hist_hi=100000,
              hist_cap=100100, var_k=False)
    pair = build_pair(w)
    info = pair.lib.info
    n_r = int(pair.hist_len.min())
    assert 2 * info["plan_rows_per_pass"] < n_r <= 3 * info["plan_rows_per_pass"], info
    for step in range(2):
        si = make_step_inputs(w, 0, step, pair.hist_len)
        res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
        out = run_lib_step(pair, 0, si)
        compare_step(pair, 0, si, res, out)
        compare_counts(pair, 0, res)
        # rows from every pass were resolved, and misses were staged and promoted
        assert any(len(rr.union) and max(rr.union) >= 2 * info["plan_rows_per_pass"] for rr in res.req.values())
        assert sum(len(rr.victims) for rr in res.req.values()) > 0
    _exact_vs_topk(pair, 0, 1, si.topk[1])
    pair.lib.close()


def test_two_handles_on_two_streams():
    """Two handles in one process (the 256-element layout and the absorbed-MLA
    layout), each driven on its own non-default caller stream, steps and
    commits interleaved: each matches its own oracle, so no launch setting or
    device state leaks between handles, and the library orders its work after
    whatever the caller enqueued on the stream it is given."""
    import torch
    from tests.pair import to_device
    pairs = [build_pair(_tiny(n_req=2, var_k=True)), build_pair(_mla_small(n_req=3, n_groups=1))]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    n = [p.hist_len.copy() for p in pairs]
    for step in range(3):
        pending = []
        for p, s, nn in zip(pairs, streams, n):
            w = p.w
            si = make_step_inputs(w, 0, step + 1, nn)
            with torch.cuda.stream(s):
                d = to_device(si)
                out = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
                p.lib.verify_step(0, d["queries"], d["topk"], d["causal"], d["ring"], out, stream=s)
            pending.append((p, si, out, d))
        torch.cuda.synchronize()
        for k, (p, si, out, d) in enumerate(pending):
            res = p.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
            compare_step(p, 0, si, res, out.cpu().numpy().view(np.uint16))
            compare_counts(p, 0, res)
            acc = make_accepted(p.w, step, si.k_active)
            p.orc.commit(acc)
            p.lib.commit(acc, stream=streams[k])
            n[k] = n[k] + 1 + acc
        torch.cuda.synchronize()
    for p, nn in zip(pairs, n):
        assert p.lib.hist_len().tolist() == nn.tolist()
        p.lib.close()


def test_invalid_calls_are_rejected_and_change_nothing():
    """Host-side argument checks of the entry points (a null device pointer, a
    group or request outside the handle, a bad hot set, a ring load that does
    not end at the frontier, an acceptance outside [-1, q_max)): each returns
    its error code before any device work, and the next valid step still
    matches the oracle exactly."""
    import torch
    from hierarchical_sparse_kv_verify_amd import KVHierError
    from tests.pair import to_device
    w = _tiny(n_req=2)
    pair = build_pair(w)
    lib = pair.lib
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    d = to_device(si)
    out = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
    B, L = w.hot_slots, w.hist_cap
    bad = [
        (lambda: lib.verify_step(0, 0, d["topk"], d["causal"], d["ring"], out), -1),       # null queries
        (lambda: lib.verify_step(0, d["queries"], 0, d["causal"], d["ring"], out), -1),    # null list
        (lambda: lib.verify_step(1, d["queries"], d["topk"], d["causal"], d["ring"], out), -1),   # no group 1
        (lambda: lib.set_hot(0, w.n_req, [1], [0]), -1),                                    # no such request
        (lambda: lib.set_hot(0, 0, list(range(B + 1)), [0] * (B + 1)), -1),                 # more rows than slots
        (lambda: lib.set_hot(0, 0, [3, 3], [0, 0]), -1),                                    # repeated row
        (lambda: lib.set_hot(0, 0, [L], [0]), -1),                                          # row outside the history
        (lambda: lib.set_hot(0, 0, [3], [-1]), -1),                                         # negative stamp
        (lambda: lib.ring_load(0, 0, int(pair.hist_len[0]) - 2, np.zeros((1, w.row_elems), np.uint16)), -1),
        (lambda: lib.commit(np.full(w.n_req, w.q_max, np.int32)), -1),                      # A_r >= q_max
        (lambda: lib.last_lists(0, w.n_req), -1),
    ]
    for i, (call, code) in enumerate(bad):
        with pytest.raises(KVHierError) as ei:
            call()
        assert ei.value.code == code, (i, ei.value.code, str(ei.value))
    torch.cuda.synchronize()
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows)
    lib.verify_step(0, d["queries"], d["topk"], d["causal"], d["ring"], out)
    torch.cuda.synchronize()
    compare_step(pair, 0, si, res, out.cpu().numpy().view(np.uint16))
    compare_counts(pair, 0, res)
    assert lib.hist_len().tolist() == pair.hist_len.tolist()
    lib.close()


def test_ring_block_only_reading():
    w = _tiny()
    pair = build_pair(w, block_only=True)
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows)
    out = run_lib_step(pair, 0, si)
    compare_step(pair, 0, si, res, out)
    pair.lib.close()


@pytest.mark.parametrize("n_chunks", [1, 3])
def test_outputs_bitwise_identical_across_cache_states(n_chunks):
    """The sum order depends only on the lists: cold, warm and resident caches
    give bitwise identical outputs, also where the attention walks the
    row-ordered lists (every request chunk but the first)."""
    w = _mla_small(n_groups=1, var_k=False, topk=1024)
    outs, misses, unions = [], [], []
    for warm, rho in ((False, 0.0), (True, 0.0), (True, 0.5)):
        pair = build_pair(w, warm=warm, rho=rho, with_oracle=False, lib_kw=dict(n_chunks=n_chunks))
        assert pair.lib.info["attn_row_order"] == (1 if n_chunks > 1 else 0), pair.lib.info
        si = make_step_inputs(w, 0, 0, pair.hist_len)
        outs.append(run_lib_step(pair, 0, si))
        _, last = pair.lib.stats(0)
        misses.append(last["union_miss"])
        unions.append(last["union_rows"])
        pair.lib.close()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    assert unions[0] == unions[1] == unions[2]
    assert misses[0] > misses[1] > misses[2]


def test_resident_tier_parity():
    w = _mla_small(n_groups=1)
    pair = build_pair(w, rho=0.3)
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
    out = run_lib_step(pair, 0, si)
    compare_step(pair, 0, si, res, out)
    compare_counts(pair, 0, res)
    for r in range(w.n_req):
        _exact_vs_topk(pair, 0, r, si.topk[r])
    pair.lib.close()


def test_inactive_requests_and_queries():
    w = _mla_small(n_groups=1)
    pair = build_pair(w)
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    si.causal_pos[1, :] = -1                  # whole request inactive
    si.causal_pos[2, 3:] = -1                 # inactive suffix
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
    out = run_lib_step(pair, 0, si)
    compare_step(pair, 0, si, res, out)
    compare_counts(pair, 0, res)
    assert (out[1] == 0).all()
    pair.lib.close()


def test_poisoned_arena_after_readers():
    """With arena poisoning (NaN between a chunk's last readers and its next
    fetch) the outputs of two groups sharing one arena are unchanged: every
    fetch waits for the previous readers and every attention for its fetch.
    The staged rows stay readable after the step (a Reuse consumer may still
    read them).  Timing events and the serialised attention leave the outputs
    unchanged too."""
    w = _mla_small(n_groups=2, n_arenas=1, var_k=False)
    outs = []
    for flags in (0, 2, 1, 4 | 8):
        pair = build_pair(w, with_oracle=False, lib_kw=dict(flags=flags, n_chunks=2))
        outs.append([run_lib_step(pair, g, make_step_inputs(w, g, 0, pair.hist_len)) for g in range(2)])
        if flags == 2:
            L = pair.lib.last_lists(1, 0)
            sel = np.flatnonzero((L["loc"].ravel() >= 0) & ((L["loc"].ravel() >> 29) == 1))[:8]
            if sel.size:
                rows = pair.lib.read_rows(1, L["loc"].ravel()[sel])
                assert not (rows == 0x7fc0).all(axis=1).any()
        pair.lib.close()
    for o in outs[1:]:
        for g in range(2):
            assert np.array_equal(outs[0][g], o[g])


def test_full_size_mla128_sampled():
    """The benchmarked shape (128 requests x ~100K rows, 4 layer groups, the
    default chunked launch): sampled requests bit-exact, sampled queries within
    tolerance; whole-step counters consistent."""
    w = WORKLOADS["mla128"]
    reqs = [0, 37, 70, 126, 127]          # every chunk of (0, 32, 64, 96, 128)
    pair = build_pair(w, oracle_requests=reqs)
    assert pair.lib.info["n_chunks"] > 1
    attend = {(r, j) for r in reqs for j in (0, 3, 7)}
    assert pair.lib.info["n_chunks"] == 4
    for g in range(w.n_groups):
        si = make_step_inputs(w, g, 0, pair.hist_len)
        res = pair.orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows,
                                   attend=attend, n_threads=16)
        out = run_lib_step(pair, g, si)
        compare_step(pair, g, si, res, out, requests=reqs)
        _, last = pair.lib.stats(g)
        assert last["active_queries"] == w.n_req * w.q_max
        assert last["selections"] == w.n_req * w.q_max * w.topk
        assert last["fetched_bytes"] == last["union_miss"] * 2 * w.row_elems
        assert last["union_miss"] == last["promoted"] + last["overflow"]
        assert 0.12 < last["union_miss"] / last["union_rows"] < 0.16
        for r in reqs:
            _exact_vs_topk(pair, g, r, si.topk[r])
    pair.lib.close()


def test_full_request_shape_mla512_sampled():
    """The 512-request, 500K-row shape at its full per-request size (~500K-row
    histories, 128 heads in two 64-head workgroups per query, Q = 4, k = 2048,
    B = 2048, W = 64, the shared core as the only warm rows, so ~38% of
    distinct rows miss and most misses overflow the 2048 slots), with 128
    requests over two host prefixes: four chunks of 32 requests, each one wave of
    256 attention workgroups without key splits.  Sampled requests of both
    prefixes bit-exact, sampled queries within tolerance."""
    w = shrink(WORKLOADS["mla512"], n_req=128, n_prefix=2)
    reqs = [0, 1, 64, 127]
    pair = build_pair(w, oracle_requests=reqs)
    info = pair.lib.info
    assert info["n_chunks"] == 4 and info["attn_splits"] == 1 and info["attn_head_groups"] == 2, info
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    attend = {(r, j) for r in reqs for j in (0, 3)}
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, attend=attend, n_threads=16)
    out = run_lib_step(pair, 0, si)
    compare_step(pair, 0, si, res, out, requests=reqs)
    _, last = pair.lib.stats(0)
    assert last["active_queries"] == w.n_req * w.q_max
    assert last["union_miss"] == last["promoted"] + last["overflow"] and last["overflow"] > last["promoted"]
    assert 0.3 < last["union_miss"] / last["union_rows"] < 0.45
    for r in reqs:
        _exact_vs_topk(pair, 0, r, si.topk[r])
    pair.lib.close()


@pytest.mark.parametrize("window,page", [(8, 4), (2, 1)])
def test_tail_rows_and_async_backup_over_rounds(window, page):
    """Selections favour recently generated rows: rows still in the ring
    resolve from it (tail), rows that left it are fetched from the host copy
    that the asynchronous backup wrote.  R_d = 16 >= 2 K_max runs the backup
    beside the next step; R_d = 6 < 2 K_max runs it ahead of it."""
    w = _tiny(n_req=3, ring_window=window, ring_page=page, q_max=4, var_k=True, recent_frac=0.3,
              recent_span=24)
    pair = build_pair(w)
    n = pair.hist_len.copy()
    tail_seen = 0
    for step in range(8):
        si = make_step_inputs(w, 0, step + 1, n)
        res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows)
        out = run_lib_step(pair, 0, si)
        compare_step(pair, 0, si, res, out)
        compare_counts(pair, 0, res)
        for r in range(w.n_req):
            # every location holds its row; rows committed in earlier rounds are
            # compared with the oracle's history, which its commits extended
            L = pair.lib.last_lists(0, r)
            loc = L["loc"].ravel()
            sel = np.flatnonzero(loc >= 0)
            rows = pair.lib.read_rows(0, loc[sel])
            for x, e in zip(rows, si.topk[r].ravel()[sel]):
                assert np.array_equal(x, pair.orc.hist[0].row(r, int(e))), ("row at location", r, int(e))
        tail_seen += pair.lib.stats(0)[1]["union_tail"]
        acc = make_accepted(w, step, si.k_active)
        pair.orc.commit(acc)
        pair.lib.commit(acc)
        n = n + 1 + acc
    pair.lib.sync()
    for r in range(w.n_req):
        np.testing.assert_array_equal(pair.lib.host_rows(0, 1, r)[: n[r]], pair.orc.hist[0].tails[r, : n[r]])
    assert tail_seen > 0
    pair.lib.close()


def test_mla_recent_rows_two_groups():
    w = _mla_small(recent_frac=0.05, recent_span=256)
    pair = build_pair(w)
    n = pair.hist_len.copy()
    for step in range(3):
        sis = []
        for g in range(w.n_groups):
            si = make_step_inputs(w, g, step, n)
            res = pair.orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
            out = run_lib_step(pair, g, si)
            compare_step(pair, g, si, res, out)
            compare_counts(pair, g, res)
            sis.append(si)
        acc = make_accepted(w, step, sis[0].k_active)
        pair.orc.commit(acc)
        pair.lib.commit(acc)
        n = n + 1 + acc
    _, last = pair.lib.stats(0)
    assert last["union_tail"] > 0
    pair.lib.close()


def test_compressed_source_rounds():
    """Eq. (8): group 1 stores one row per 4 positions.  Its selections name
    complete stored rows, its ring holds positions, and each commit adds the
    stored rows the new frontier completes (the caller's compressed rows).
    Group 0 (uncompressed) runs beside it with the asynchronous backup."""
    import torch
    from hierarchical_sparse_kv_verify_amd import KVHierError
    from workloads import make_source_rows
    w = _mla_small(compress=4, compress_groups=(1,), var_k=True, n_prefix=0, prefix_len=0)
    pair = build_pair(w)
    pair.lib.set_compression(1, 4)
    pair.orc.set_compression(1, 4)
    n = pair.hist_len.copy()
    for step in range(4):
        sis = []
        for g in range(w.n_groups):
            si = make_step_inputs(w, g, step, n)
            res = pair.orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
            out = run_lib_step(pair, g, si)
            compare_step(pair, g, si, res, out)
            compare_counts(pair, g, res)
            sis.append(si)
        _, last = pair.lib.stats(1)
        assert last["union_tail"] == 0 and last["selections"] > 0
        acc = make_accepted(w, step, sis[0].k_active)
        src = make_source_rows(w, 1, step)
        if step == 0:
            with pytest.raises(KVHierError):                   # compressed rows are required
                pair.lib.commit(acc)
        pair.orc.commit(acc, src_rows=[None, src])
        pair.lib.commit(acc, src_rows=[None, torch.from_numpy(src.view(np.int16)).cuda()])
        n = n + 1 + acc
    pair.lib.sync()
    for g in range(2):
        for r in range(w.n_req):
            np.testing.assert_array_equal(pair.lib.host_rows(g, 1, r), pair.orc.hist[g].tails[r],
                                          err_msg="host rows g=%d r=%d" % (g, r))
    with pytest.raises(KVHierError) as ei:                      # only before the group's first step
        pair.lib.set_compression(1, 2)
    assert ei.value.code == -4
    pair.lib.close()


@pytest.mark.parametrize("layout", ["tiny", "mla", "mla_chunks"])
def test_repeated_entries_within_a_list(layout):
    """Reading R2: a row selected twice by one query is two terms of its
    softmax (eq. 12 gives every entry a location), while the union holds it
    once and the host fetch copies it once.  Repeats are planted in the
    generated lists (the generator draws distinct entries): within a query,
    across the two halves of one list and at both ends.  With three request
    chunks the attention of chunks 1 and 2 walks the row-ordered lists, and a
    query with repeats keeps its selection order (repeats planted in every
    other query there, so both kinds meet in one step)."""
    w = (_tiny(n_req=2) if layout == "tiny" else
         _mla_small(n_groups=1, n_req=3, topk=1024) if layout == "mla_chunks" else _mla_small(n_groups=1, n_req=3))
    pair = build_pair(w, lib_kw=dict(n_chunks=3) if layout == "mla_chunks" else None)
    if layout == "mla_chunks":
        assert pair.lib.info["attn_row_order"] == 1, pair.lib.info
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    rng = np.random.default_rng(7)
    planted = 0
    for r in range(w.n_req):
        for j in range(int(si.k_active[r])):
            if layout == "mla_chunks" and j % 2 == 1:
                continue
            lst = si.topk[r, j]
            valid = np.flatnonzero((lst >= 0) & (lst < int(pair.hist_len[r])))
            src = rng.choice(valid, size=min(12, valid.size // 2), replace=False)
            dst = rng.choice(np.setdiff1d(np.arange(w.topk), src), size=src.size, replace=False)
            lst[dst] = lst[src]
            lst[-1] = lst[0] if lst[0] >= 0 else lst[-1]
            planted += src.size
    assert planted > 0
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
    out = run_lib_step(pair, 0, si)
    compare_step(pair, 0, si, res, out)
    compare_counts(pair, 0, res)
    for r in range(w.n_req):
        L = pair.lib.last_lists(0, r)
        assert len(set(L["union_rows"].tolist())) == L["n_union"]        # the union holds each row once
        assert len(set(L["miss_rows"].tolist())) == L["n_miss"]          # each missing row fetched once
        _exact_vs_topk(pair, 0, r, si.topk[r])
    pair.lib.close()


def test_request_with_no_history():
    """A request whose committed history is empty (n_r = 0, a fresh request
    before any commit): every list entry is a pad or invalid (R1: valid iff
    0 <= e < n_r), its union is empty, nothing is fetched or evicted, and its
    queries attend over their ring window only (this step's block rows).  The
    other requests of the step are unaffected."""
    w = _mla_small(n_groups=1, n_req=4, var_k=False, n_prefix=0, prefix_len=0)
    from workloads.gen import make_hist_len
    hl = make_hist_len(w)
    hl[1] = 0
    pair = build_pair(w, hist_len=hl)
    si = make_step_inputs(w, 0, 0, hl)                 # request 1: nothing to draw from, p_j = j
    assert (si.causal_pos[1] == np.arange(w.q_max)).all()
    rng = np.random.default_rng(3)
    si.topk[1] = rng.integers(-1, 40, size=si.topk[1].shape).astype(np.int32)   # pads and invalid entries
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
    assert res.req[1].union == [] and res.req[1].miss == []
    out = run_lib_step(pair, 0, si)
    compare_step(pair, 0, si, res, out)
    compare_counts(pair, 0, res)
    L = pair.lib.last_lists(0, 1)
    assert L["n_union"] == 0 and L["n_miss"] == 0 and (L["loc"] == -1).all()
    pair.lib.close()


def test_failed_launch_latches_the_handle():
    """A HIP error after a step has started its device work leaves the handle
    latched: that call returns KV_EHIP, every later call that changes state or
    enqueues work returns KV_ESTATE naming the first failure, reads still
    work.  The failure is forced from the host (the attention launch reports an
    error without launching anything), so no kernel faults."""
    import torch
    from hierarchical_sparse_kv_verify_amd import KV_FLAG_TEST_FAIL_ATTN, KVHierError
    from tests.pair import to_device
    w = _tiny(n_req=2)
    pair = build_pair(w)
    lib = pair.lib
    si = make_step_inputs(w, 0, 0, pair.hist_len)
    d = to_device(si)
    out = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
    res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows)
    lib.verify_step(0, d["queries"], d["topk"], d["causal"], d["ring"], out)
    torch.cuda.synchronize()
    compare_step(pair, 0, si, res, out.cpu().numpy().view(np.uint16))
    lib.set_flags(KV_FLAG_TEST_FAIL_ATTN)
    with pytest.raises(KVHierError) as ei:
        lib.verify_step(0, d["queries"], d["topk"], d["causal"], d["ring"], out)
    assert ei.value.code == -3, str(ei.value)
    lib.set_flags(0)
    later = [
        lambda: lib.verify_step(0, d["queries"], d["topk"], d["causal"], d["ring"], out),
        lambda: lib.commit(np.zeros(w.n_req, np.int32)),
        lambda: lib.set_hot(0, 0, [1], [0]),
        lambda: lib.save_cache(0),
        lambda: lib.set_hist_len(pair.hist_len),
    ]
    for call in later:
        with pytest.raises(KVHierError) as ei:
            call()
        assert ei.value.code == -4 and "unusable" in str(ei.value), str(ei.value)
    lib.sync()
    _, last = lib.stats(0)                     # reads still work
    assert last["calls"] >= 1
    assert lib.hist_len().tolist() == pair.hist_len.tolist()
    lib.close()


def test_reuse_on_another_stream_without_host_sync():
    """A Reuse layer issued on a second caller stream right after the selecting
    step (no host synchronisation in between) reads that step's ring rows,
    staged rows and locations: the library orders it after the step.  Two
    rounds with commits; outputs match the oracle."""
    import torch
    from tests.pair import to_device
    w = _mla_small(n_groups=1, n_req=4, var_k=False)
    pair = build_pair(w, lib_kw=dict(n_chunks=2))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    n = pair.hist_len.copy()
    for step in range(2):
        si = make_step_inputs(w, 0, step, n)
        q2 = make_step_inputs(w, 0, 100 + step, n).queries
        with torch.cuda.stream(s1):
            d = to_device(si)
            out1 = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
        with torch.cuda.stream(s2):
            dq2 = torch.from_numpy(np.ascontiguousarray(q2.view(np.int16))).cuda()
            dc2 = torch.from_numpy(np.ascontiguousarray(si.causal_pos)).cuda()
            out2 = torch.zeros_like(out1)
        torch.cuda.synchronize()
        pair.lib.verify_step(0, d["queries"], d["topk"], d["causal"], d["ring"], out1, stream=s1)
        pair.lib.verify_reuse(0, dq2, dc2, out2, stream=s2)
        torch.cuda.synchronize()
        res = pair.orc.verify_step(0, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
        compare_step(pair, 0, si, res, out1.cpu().numpy().view(np.uint16))
        ref2 = pair.orc.verify_reuse(0, q2, n_threads=8)
        got2 = out2.cpu().numpy().view(np.uint16)
        for (r, j), v in ref2.items():
            assert_close(got2[r, j], v, "reuse r=%d j=%d" % (r, j))
        acc = make_accepted(w, step, si.k_active)
        pair.orc.commit(acc)
        pair.lib.commit(acc, stream=s1)
        n = n + 1 + acc
    pair.lib.close()


def test_follower_sets_over_rounds_without_host_sync():
    """Plan-sharing sets (two sets of two layers) over four rounds with
    commits, every call issued without host synchronisation and the two layers
    of each set on two different caller streams: the leader's next plan waits
    for the follower's previous readers, so the final slot tables of every
    layer and every round's outputs match the oracle."""
    import torch
    from tests.pair import to_device
    w = _mla_small(n_groups=4, plan_share=2, n_arenas=2, var_k=True)
    pair = build_pair(w)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    n = pair.hist_len.copy()
    rounds = []
    for step in range(4):
        sis, outs = [], []
        for g in range(w.n_groups):
            si = make_step_inputs(w, g, step, n)
            s = streams[g % 2]
            with torch.cuda.stream(s):
                d = to_device(si)
                out = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
            # the inputs were copied on the stream the step is issued on
            pair.lib.verify_step(g, d["queries"], d["topk"], d["causal"], d["ring"], out, stream=s)
            sis.append((si, d))
            outs.append(out)
        acc = make_accepted(w, step, sis[0][0].k_active)
        pair.lib.commit(acc, stream=streams[0])
        rounds.append((sis, outs, acc))
        n = n + 1 + acc
    torch.cuda.synchronize()
    for step, (sis, outs, acc) in enumerate(rounds):
        for g in range(w.n_groups):
            si = sis[g][0]
            res = pair.orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=8)
            got = outs[g].cpu().numpy().view(np.uint16)
            for (r, j), ref in res.out.items():
                assert_close(got[r, j], ref, "round %d group %d r=%d j=%d" % (step, g, r, j))
        pair.orc.commit(acc)
    for g in range(w.n_groups):
        for r in range(w.n_req):
            rows, lu = pair.lib.slot_table(g, r)
            orows, olu = pair.orc.slot_table(g, r)
            np.testing.assert_array_equal(rows, orows, err_msg="slot rows g=%d r=%d" % (g, r))
            np.testing.assert_array_equal(lu, olu, err_msg="slot stamps g=%d r=%d" % (g, r))
    assert pair.lib.hist_len().tolist() == n.tolist()
    pair.lib.close()
