"""kv_hier_verify_step_static (the entry point that allocates nothing during
a call: its split-key partials live in the library's static device array)
against kv_hier_verify_step, through the C ABI.

Two handles are built with identical state; each call runs the regular entry
point on one and the static one on the other, and the lists, slot tables,
counters and outputs must be identical (the same kernels run on the same
inputs; only the partials' memory differs).  Two calls in a row, the second
on a smaller input (fewer requests and queries, so fewer partial blocks), so
what the first call left in the shared array cannot leak into the second.
"""
import numpy as np
import pytest

from tests.pair import build_pair, to_device
from workloads import WORKLOADS, make_step_inputs, shrink

pytestmark = pytest.mark.gpu


def _workload(**kw):
    base = shrink(WORKLOADS["mla32"], n_req=4, n_groups=1, hist_lo=5000, hist_hi=6000, hist_cap=6100,
                  n_prefix=1, prefix_len=4096, topk=512, hot_slots=1024, ring_window=128, q_max=8,
                  f_sh=0.75, hit_rate=0.8, pad_frac=0.02, invalid_frac=0.01, var_k=True)
    return shrink(base, **kw)


def _both(w):
    import torch
    a = build_pair(w, with_oracle=False)
    b = build_pair(w, with_oracle=False)
    assert a.lib.info["attn_splits"] > 1, a.lib.info          # the partials are used
    si = make_step_inputs(w, 0, 0, a.hist_len)
    d = to_device(si)
    outs = []
    for p, static in ((a, False), (b, True)):
        out = torch.full((w.n_req, w.q_max, w.n_heads, w.d_v), 0x7fc0, dtype=torch.int16, device="cuda")
        fn = p.lib.verify_step_static if static else p.lib.verify_step
        fn(0, d["queries"], d["topk"], d["causal"], d["ring"], out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().view(np.uint16))
    np.testing.assert_array_equal(outs[0], outs[1])
    for r in range(w.n_req):
        la, lb = a.lib.last_lists(0, r), b.lib.last_lists(0, r)
        for key in ("union_rows", "union_loc", "miss_rows", "victims", "loc"):
            np.testing.assert_array_equal(la[key], lb[key], err_msg="%s r=%d" % (key, r))
        for x, y in zip(a.lib.slot_table(0, r), b.lib.slot_table(0, r)):
            np.testing.assert_array_equal(x, y)
    ca, cb = a.lib.stats(0)[1], b.lib.stats(0)[1]
    for key in ("selections", "union_rows", "union_miss", "promoted", "overflow", "sel_miss"):
        assert ca[key] == cb[key], key
    a.lib.close()
    b.lib.close()
    return outs[1]


def test_static_scratch_step_matches_the_regular_step():
    big = _both(_workload())
    small = _both(_workload(n_req=2, q_max=4))
    assert big.shape[0] > small.shape[0]


def test_static_scratch_rejects_partials_over_the_array():
    """32 requests of 8 queries (64 heads) in two 16-request chunks split their
    keys in two: 256 partial blocks x 64 heads x (512 + 2) floats = 33.7 MB,
    over the 32 MiB array.  The static step is refused before any device work
    (KV_EINVAL, the handle stays usable) and the regular step runs."""
    import torch
    from hierarchical_sparse_kv_verify_amd import KVHierError
    w = _workload(n_req=32, var_k=False)
    p = build_pair(w, with_oracle=False)
    assert p.lib.info["n_chunks"] == 2 and p.lib.info["attn_splits"] == 2, p.lib.info
    si = make_step_inputs(w, 0, 0, p.hist_len)
    d = to_device(si)
    out = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
    with pytest.raises(KVHierError) as ei:
        p.lib.verify_step_static(0, d["queries"], d["topk"], d["causal"], d["ring"], out)
    assert ei.value.code == -1 and "static scratch" in str(ei.value), str(ei.value)
    p.lib.verify_step(0, d["queries"], d["topk"], d["causal"], d["ring"], out)
    torch.cuda.synchronize()
    _, last = p.lib.stats(0)
    assert last["calls"] == 1
    p.lib.close()
