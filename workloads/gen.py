"""Seeded workload generator.

Everything here is drawn from ``numpy.random`` with seeds derived from
``SeedSequence([20261009, config_id, group, purpose, ...])`` and spawned per
request, so a (workload, group, step) triple always yields the same bytes.

Value recipe: every KV row, query and new block row is N(0, 1) rounded to
bf16 (round to nearest even).  Selections follow a "core + Zipf" recipe: a
shared core of round(f_sh * k) rows drawn uniformly without replacement from
the request's history, plus, for every query, k - core distinct rows drawn
from a Zipf(s) law over a seeded permutation of the remaining rows; each list
is then shuffled.  Optionally a share of each list is replaced by distinct
rows among the most recent ones (recently generated history).  Correctness suites may replace a fraction of entries by the
pad value -1 or by out-of-range values.

The module holds no step of the verified method: it never resolves, places or
attends; the hot-cache warm set is chosen from the rows this module itself
drew.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED = 20261009

# purposes, the 4th word of every SeedSequence
_P_HISTORY, _P_STEP, _P_WARM, _P_RESIDENT, _P_ACCEPT = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    n_req: int
    n_groups: int
    n_arenas: int
    hist_lo: int              # committed rows n_r drawn uniformly in [hist_lo, hist_hi]
    hist_hi: int
    hist_cap: int             # host rows reserved per request (room for commits)
    n_prefix: int             # shared host prefixes (0 = every request owns its history)
    prefix_len: int           # rows [0, prefix_len) come from prefix r % n_prefix
    row_elems: int
    d_qk: int
    v_off: int
    d_v: int
    n_heads: int
    q_max: int
    topk: int
    hot_slots: int
    ring_window: int
    ring_page: int
    f_sh: float               # shared-core fraction of each list
    zipf_s: float
    hit_rate: Optional[float]  # None: warm set = core rows + unselected filler
    rho: float = 0.0          # resident (optional-history) fraction of rows
    pad_frac: float = 0.0
    invalid_frac: float = 0.0
    empty_slot_frac: float = 0.0
    var_k: bool = False       # draw K_r in [1, q_max] per request
    ring_prefill: bool = True  # load the W-1 committed positions below n_r into the ring
    plan_share: int = 1       # payload layers per index producer: consecutive groups of this
                              # size share one selection (and warm set / resident map)
    recent_frac: float = 0.0  # share of each list replaced by distinct rows of the last
    recent_span: int = 0      # recent_span history rows (recently generated rows)
    compress: int = 1         # positions per stored row of the groups in compress_groups
    compress_groups: tuple = ()
    disjoint: bool = False    # private parts drawn from disjoint uniform ranges of one
                              # permutation (no overlap between a request's queries)
    note: str = ""

    @property
    def row_bytes(self) -> int:
        return 2 * self.row_elems


def _tiny() -> Workload:
    return Workload(
        name="tiny", config_id=1, n_req=1, n_groups=1, n_arenas=1,
        hist_lo=4096, hist_hi=4096, hist_cap=4096 + 64, n_prefix=0, prefix_len=0,
        row_elems=256, d_qk=128, v_off=128, d_v=128, n_heads=8,
        q_max=4, topk=256, hot_slots=512, ring_window=64, ring_page=64,
        f_sh=0.5, zipf_s=1.1, hit_rate=0.8,
        note="1 request, MQA row K128|V128, 8 heads of 128, Q=4, k=256, B=512, W=64")


def _mla32() -> Workload:
    return Workload(
        name="mla32", config_id=2, n_req=32, n_groups=1, n_arenas=1,
        hist_lo=32768, hist_hi=32768, hist_cap=32768 + 256, n_prefix=0, prefix_len=0,
        row_elems=576, d_qk=576, v_off=0, d_v=512, n_heads=64,
        q_max=8, topk=2048, hot_slots=4096, ring_window=128, ring_page=64,
        f_sh=0.75, zipf_s=1.0, hit_rate=0.8,
        note="32 requests x 32768 rows, MLA latent 576 bf16, 64 heads, Q=8, k=2048, "
             "B=4096 at 80% hits, W=128")


def _mla128() -> Workload:
    return Workload(
        name="mla128", config_id=3, n_req=128, n_groups=4, n_arenas=1,
        hist_lo=99_000, hist_hi=100_000, hist_cap=100_512, n_prefix=1, prefix_len=98_304,
        row_elems=576, d_qk=576, v_off=0, d_v=512, n_heads=64,
        q_max=8, topk=2048, hot_slots=4096, ring_window=128, ring_page=64,
        f_sh=0.85, zipf_s=1.0, hit_rate=0.86,
        note="128 requests x ~100K rows (one shared host prefix + per-request tail), "
             "MLA 576 bf16, 64 heads, Q=8, k=2048, ~14% distinct-row misses, B=4096, "
             "W=128, 4 layer groups over one staging arena")


def _mla128_res() -> Workload:
    return dataclasses.replace(_mla128(), name="mla128_res", config_id=4,
                               note="mla128 plus a static resident fraction rho of each "
                                    "request's rows")


def _mla512() -> Workload:
    return Workload(
        name="mla512", config_id=5, n_req=512, n_groups=1, n_arenas=1,
        hist_lo=499_000, hist_hi=500_000, hist_cap=500_512, n_prefix=16, prefix_len=498_688,
        row_elems=576, d_qk=576, v_off=0, d_v=512, n_heads=128,
        q_max=4, topk=2048, hot_slots=2048, ring_window=64, ring_page=64,
        f_sh=0.85, zipf_s=1.0, hit_rate=None,
        note="512 requests x ~500K rows over 16 shared host prefixes, MLA 576 bf16, "
             "128 heads, Q=4, k=2048, B=2048, W=64")


def _mla128_shared() -> Workload:
    return dataclasses.replace(
        _mla128(), name="mla128_shared", n_arenas=4, plan_share=4,
        note="mla128 with its 4 layer groups fed by one index producer: one selection, "
             "four payload layers (follower-layer reuse of one plan)")


def _ds_shared() -> Workload:
    return Workload(
        name="ds_shared", config_id=6, n_req=128, n_groups=4, n_arenas=4,
        hist_lo=99_000, hist_hi=100_000, hist_cap=100_512, n_prefix=1, prefix_len=98_304,
        row_elems=144, d_qk=144, v_off=0, d_v=128, n_heads=128,
        q_max=4, topk=512, hot_slots=2048, ring_window=64, ring_page=64,
        f_sh=0.85, zipf_s=1.0, hit_rate=0.82,
        note="4 shared KV sources (one staging arena each) read by several layers: per source "
             "a selecting layer, a re-selecting layer and layers reusing the latest selection; "
             "128 requests x ~100K rows of 144 bf16 (288 B: K = all 144, V = the first 128), "
             "128 heads, Q=4, k=512, B=2048, W=64, ~18% distinct-row misses")


WORKLOADS = {w.name: w for w in (_tiny(), _mla32(), _mla128(), _mla128_res(), _mla512(), _mla128_shared(),
                                 _ds_shared())}


def _leader(w: Workload, group: int) -> int:
    return group - group % max(1, w.plan_share)


def positions_per_row(w: Workload, group: int) -> int:
    """m of a compressed source, 1 otherwise."""
    return w.compress if group in w.compress_groups else 1


def shrink(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with fields replaced (smaller sizes for fast tests)."""
    return dataclasses.replace(w, **kw)


# ---------------------------------------------------------------------------
# bf16 helpers (bit patterns stored as uint16)

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (no NaN inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))


def _fill_normal_bf16(rng: np.random.Generator, out: np.ndarray, block_rows: int = 8192) -> None:
    """out[:] = N(0, 1) rounded to bf16, drawn in blocks of rows: the same
    values as one draw of the whole array (the generator fills sequentially),
    without a full-size float32 temporary."""
    for i in range(0, out.shape[0], block_rows):
        n = min(block_rows, out.shape[0] - i)
        out[i:i + n] = _normal_bf16(rng, (n,) + out.shape[1:])


def _pool_map(fn, items) -> None:
    """Runs fn over independent items (each with its own generator and its own
    output slice) on up to 16 threads; the results do not depend on the order."""
    items = list(items)
    workers = max(1, min(16, os.cpu_count() or 1, len(items)))
    if workers == 1:
        for x in items:
            fn(x)
        return
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        for _ in ex.map(fn, items):
            pass


def _seeds(w: Workload, group: int, purpose: int, *extra: int, n: int):
    ss = np.random.SeedSequence([SEED, w.config_id, group, purpose, *extra])
    return [np.random.default_rng(s) for s in ss.spawn(n)]


# ---------------------------------------------------------------------------
# host history

@dataclass
class History:
    """Original KV rows of one layer group (the host backing).

    ``prefix[p]`` holds rows [0, prefix_len) shared by requests r with
    r % n_prefix == p; ``tails[r]`` holds rows [prefix_len, hist_cap) of request r
    (rows at or above hist_len[r] are zero until committed)."""
    prefix: np.ndarray        # uint16 [n_prefix, prefix_len, row_elems]
    tails: np.ndarray         # uint16 [n_req, hist_cap - prefix_len, row_elems]
    hist_len: np.ndarray      # int32 [n_req]

    def row(self, r: int, s: int) -> np.ndarray:
        n_prefix, plen = self.prefix.shape[0], self.prefix.shape[1]
        if s < plen:
            return self.prefix[r % n_prefix, s]
        return self.tails[r, s - plen]


def make_hist_len(w: Workload) -> np.ndarray:
    rng = _seeds(w, 0, _P_HISTORY, 7, n=1)[0]
    return rng.integers(w.hist_lo, w.hist_hi + 1, size=w.n_req).astype(np.int32)


def make_history(w: Workload, group: int, hist_len: Optional[np.ndarray] = None,
                 progress=None) -> History:
    """Host rows of one layer group; ``progress`` (optional callable) receives a
    line after each shared prefix (large prefixes take seconds each)."""
    if hist_len is None:
        hist_len = make_hist_len(w)
    assert w.n_prefix == 0 or w.prefix_len <= int(hist_len.min())
    assert int(hist_len.max()) <= w.hist_cap
    plen = w.prefix_len if w.n_prefix > 0 else 0
    npfx = w.n_prefix if w.n_prefix > 0 else 0
    rngs = _seeds(w, group, _P_HISTORY, n=npfx + w.n_req)
    prefix = np.empty((max(npfx, 1), plen, w.row_elems), dtype=np.uint16)

    def one_prefix(p):
        _fill_normal_bf16(rngs[p], prefix[p])
        if progress is not None:
            progress("history of group %d: prefix %d of %d ready" % (group, p + 1, npfx))

    _pool_map(one_prefix, range(npfx))
    tails = np.zeros((w.n_req, w.hist_cap - plen, w.row_elems), dtype=np.uint16)

    def one_tail(r):
        n_own = int(hist_len[r]) - plen
        _fill_normal_bf16(rngs[npfx + r], tails[r, :n_own])

    _pool_map(one_tail, range(w.n_req))
    return History(prefix=prefix, tails=tails, hist_len=hist_len.astype(np.int32).copy())


# ---------------------------------------------------------------------------
# selections and per-step tensors

def _zipf_cdf(m: int, s: float) -> np.ndarray:
    cdf = np.cumsum(1.0 / np.arange(1, m + 1, dtype=np.float64) ** s)
    return cdf / cdf[-1]


def _zipf_distinct(rng: np.random.Generator, cdf: np.ndarray, need: int) -> np.ndarray:
    """``need`` distinct ranks in [0, m) drawn from P(rank) ~ (rank+1)^-s, in draw order."""
    m = cdf.size
    if need <= 0:
        return np.zeros(0, dtype=np.int64)
    assert need <= m
    out = np.zeros(0, dtype=np.int64)
    seen = np.zeros(m, dtype=bool)
    while out.size < need:
        draw = np.searchsorted(cdf, rng.random(4 * (need - out.size) + 64), side="right")
        draw = np.minimum(draw, m - 1)
        _, first = np.unique(draw, return_index=True)
        draw = draw[np.sort(first)]
        draw = draw[~seen[draw]]
        seen[draw] = True
        out = np.concatenate([out, draw[: need - out.size]])
    return out


@dataclass
class StepInputs:
    topk: np.ndarray          # int32 [N, Q, k]; -1 = pad
    causal_pos: np.ndarray    # int32 [N, Q]; n_r + j for active j, -1 for the inactive suffix
    queries: np.ndarray       # uint16 (bf16) [N, Q, H, d_qk]
    block_rows: np.ndarray    # uint16 (bf16) [N, Q, row_elems]: new KV row of each query position
    k_active: np.ndarray      # int32 [N]
    drawn: list = field(default_factory=list)   # per request: (core rows, [private rows per query])


def make_step_inputs(w: Workload, group: int, step: int, hist_len: np.ndarray,
                     k_active: Optional[np.ndarray] = None,
                     requests: Optional[np.ndarray] = None) -> StepInputs:
    """Inputs of one verification step of one layer group.

    ``requests`` restricts generation to a subset (other rows of the outputs are
    left as pads / inactive), which the full-size parity tests use to sample."""
    N, Q, k = w.n_req, w.q_max, w.topk
    if w.plan_share > 1:
        # one selection per index producer; each payload layer has its own
        # queries and new rows
        lead = make_step_inputs(dataclasses.replace(w, plan_share=1), _leader(w, group), step, hist_len,
                                k_active, requests)
        if group == _leader(w, group):
            return lead
        rngs = _seeds(w, group, _P_STEP, step, 1, n=N)
        queries = np.zeros_like(lead.queries)
        block = np.zeros_like(lead.block_rows)
        for r in (range(N) if requests is None else [int(x) for x in requests]):
            for j in range(Q):
                queries[r, j] = _normal_bf16(rngs[r], (w.n_heads, w.d_qk))
                block[r, j] = _normal_bf16(rngs[r], (w.row_elems,))
        return StepInputs(topk=lead.topk, causal_pos=lead.causal_pos, queries=queries, block_rows=block,
                          k_active=lead.k_active, drawn=lead.drawn)
    rngs = _seeds(w, group, _P_STEP, step, n=N)
    topk = np.full((N, Q, k), -1, dtype=np.int32)
    causal = np.full((N, Q), -1, dtype=np.int32)
    queries = np.zeros((N, Q, w.n_heads, w.d_qk), dtype=np.uint16)
    block = np.zeros((N, Q, w.row_elems), dtype=np.uint16)
    if k_active is None:
        k_active = np.full(N, Q, dtype=np.int32)
        if w.var_k:
            # K_r belongs to the request, not to a layer group
            kr = _seeds(w, 0, _P_STEP, step, 99, n=1)[0]
            k_active = kr.integers(1, Q + 1, size=N).astype(np.int32)
    drawn = [None] * N
    req_iter = range(N) if requests is None else [int(x) for x in requests]
    m = positions_per_row(w, group)

    def one_request(r):
        rng = rngs[r]
        n_pos = int(hist_len[r])
        n_r = n_pos // m                  # stored rows the selections draw from
        kr = int(k_active[r])
        core_n = min(int(round(w.f_sh * k)), n_r)
        core = rng.choice(n_r, size=core_n, replace=False)
        rest_mask = np.ones(n_r, dtype=bool)
        rest_mask[core] = False
        rest = np.flatnonzero(rest_mask)
        perm = rest[rng.permutation(rest.size)]
        priv_n = min(k - core_n, rest.size)
        cdf = _zipf_cdf(rest.size, w.zipf_s) if rest.size else np.zeros(0)
        if w.disjoint:
            priv_n = min(priv_n, rest.size // Q)
        privs = []
        for j in range(Q):
            if w.disjoint:
                priv = perm[j * priv_n:(j + 1) * priv_n]
            else:
                ranks = _zipf_distinct(rng, cdf, priv_n)
                priv = perm[ranks]
            lst = np.concatenate([core, priv]).astype(np.int64)
            lst = lst[rng.permutation(lst.size)]
            row = np.full(k, -1, dtype=np.int64)
            row[: lst.size] = lst
            if w.recent_frac > 0:
                cand = np.setdiff1d(np.arange(max(0, n_r - w.recent_span), n_r), row)
                n_rec = min(int(round(w.recent_frac * k)), cand.size)
                if n_rec:
                    at = rng.choice(k, size=n_rec, replace=False)
                    row[at] = rng.choice(cand, size=n_rec, replace=False)
            if w.pad_frac > 0 or w.invalid_frac > 0:
                u = rng.random(k)
                row[u < w.pad_frac] = -1
                bad = (u >= w.pad_frac) & (u < w.pad_frac + w.invalid_frac)
                nb = int(bad.sum())
                # out-of-range values: at or above the frontier, or negative below -1
                choices = np.array([n_r, n_r + 1, n_r + 7, 1 << 30, -2, -100], dtype=np.int64)
                row[bad] = choices[rng.integers(0, choices.size, size=nb)]
            if j < kr:
                topk[r, j] = row.astype(np.int32)
                causal[r, j] = n_pos + j
                privs.append(priv)
            queries[r, j] = _normal_bf16(rng, (w.n_heads, w.d_qk))
            block[r, j] = _normal_bf16(rng, (w.row_elems,))
        drawn[r] = (core, privs)

    _pool_map(one_request, req_iter)
    return StepInputs(topk=topk, causal_pos=causal, queries=queries, block_rows=block,
                      k_active=k_active.astype(np.int32), drawn=drawn)


def make_hot_warm_set(w: Workload, group: int, hist_len: np.ndarray, step_in: StepInputs,
                      requests: Optional[np.ndarray] = None):
    """Initial hot-cache contents per request: (rows int32[B], last_used int32[B]).

    With a hit-rate target h: the request's core rows first, then randomly chosen
    rows among those this generator drew for the queries, up to round(h * drawn
    distinct rows) (capped at B); remaining slots get random rows that the
    generator did not draw (the future victims), minus an optional fraction of
    empty slots (-1).  Without a target: core rows plus undrawn filler.  Ages are
    uniform in {0..7}."""
    B = w.hot_slots
    rngs = _seeds(w, _leader(w, group), _P_WARM, n=w.n_req)
    out = [None] * w.n_req
    req_iter = range(w.n_req) if requests is None else [int(x) for x in requests]
    m = positions_per_row(w, group)
    for r in req_iter:
        rng = rngs[r]
        n_r = int(hist_len[r]) // m
        core, privs = step_in.drawn[r]
        drawn_all = np.unique(np.concatenate([core] + list(privs))) if privs else np.unique(core)
        core_sh = core[rng.permutation(core.size)]
        priv_only = np.setdiff1d(drawn_all, core, assume_unique=False)
        priv_only = priv_only[rng.permutation(priv_only.size)]
        if w.hit_rate is None:
            hot = core_sh[:B]
        else:
            want = min(int(round(w.hit_rate * drawn_all.size)), B)
            hot = np.concatenate([core_sh, priv_only])[:want]
        n_fill = B - hot.size
        n_empty = int(round(w.empty_slot_frac * n_fill))
        n_fill -= n_empty
        taken = np.zeros(n_r, dtype=bool)
        taken[drawn_all] = True
        free = np.flatnonzero(~taken)
        filler = free[rng.choice(free.size, size=min(n_fill, free.size), replace=False)]
        rows = np.concatenate([hot, filler, np.full(B - hot.size - filler.size, -1)])
        rows = rows[rng.permutation(B)].astype(np.int32)
        ages = rng.integers(0, 8, size=B).astype(np.int32)
        out[r] = (rows, ages)
    return out


def make_resident_bitmaps(w: Workload, group: int, hist_len: np.ndarray, rho: float,
                          requests: Optional[np.ndarray] = None) -> np.ndarray:
    """uint8 [N, hist_cap]: row s of request r is resident with probability rho (s < n_r)."""
    bm = np.zeros((w.n_req, w.hist_cap), dtype=np.uint8)
    if rho <= 0:
        return bm
    rngs = _seeds(w, _leader(w, group), _P_RESIDENT, int(round(rho * 1000)), n=w.n_req)
    req_iter = range(w.n_req) if requests is None else [int(x) for x in requests]
    for r in req_iter:
        n_r = int(hist_len[r])
        bm[r, :n_r] = (rngs[r].random(n_r) < rho).astype(np.uint8)
    return bm


def make_source_rows(w: Workload, group: int, step: int) -> np.ndarray:
    """Stored rows a commit completes in a compressed source (the model's
    compressed KV of each completed group of m positions): bf16
    [N, ceil(q_max / m), row_elems], N(0, 1)."""
    m = positions_per_row(w, group)
    cmax = -(-w.q_max // m)
    rng = _seeds(w, group, _P_ACCEPT, step, 5, n=1)[0]
    return _normal_bf16(rng, (w.n_req, cmax, w.row_elems))


def make_accepted(w: Workload, step: int, k_active: np.ndarray) -> np.ndarray:
    """Accepted draft count A_r uniform in [0, K_r - 1] (host int32 [N])."""
    rng = _seeds(w, 0, _P_ACCEPT, step, n=1)[0]
    hi = np.maximum(k_active.astype(np.int64), 1)
    return (rng.integers(0, 1 << 30, size=w.n_req) % hi).astype(np.int32)
