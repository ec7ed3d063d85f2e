"""TEST INFRASTRUCTURE ONLY.  Reference (oracle) model of one speculative
verification step of sparse attention over a hierarchical KV cache.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module; the product library never calls it and shares no code,
table or constant with it.

Source: "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
Hierarchy" (arXiv 2610.13708), referred to below as "the paper":
  - §2.1 eqs. (1)-(2): selected list S_t, attention over it, ready set R_t and
    host-recovery set D_t = S_t minus R_t.
  - §2.2 "Fixed-cache offloading": per request and source a B-entry GPU cache;
    hits, protection of useful rows, LRU victims, fetch of misses, locations.
  - §3.2 and Figure 2: resolution order (1) direct (tail / ready optional
    history), (2) hot cache, (3) host copy; locations in selection order.
  - §3.3 eqs. (5)-(7): visible positions, retrieval union U_r and missing set
    D_r = U_r minus R_r, one copy per distinct missing row, overflow staging
    bounded by K_max*k, acceptance and the new frontier n' = n + 1 + A.
  - §3.4 eqs. (9)-(10): draft-ring size and address; staging reservation,
    promoted rows copied back before an arena is released.
  - §3.5 eqs. (11)-(12): location l_{r,j,i} = pi_r(s_{r,j,i}) and
    KV[l] = c_{r,s}; a row held in two places has one of them chosen.

Everything is plain Python containers (sets, dicts, sorted lists) walked in
the paper's order; attention is the C reference in ``attn_ref.c``.

Readings where the pages leave a step open.  One numbering R1-R27 covers
every reading taken of the pages; the ones the oracle follows are listed here and
in ``residency.py`` (R17-R21, dynamic residency):
  R1 a list entry e of query j is a valid history selection iff 0 <= e < n_r
     (n_r = causal position of the anchor); -1 is a pad; anything else is
     counted invalid and skipped.  Rows of the current block reach attention
     through the ring branch, not through the list.
  R2 Attn of eq. (1) is per-head scaled dot-product softmax; every list entry
     is one term (a repeated entry counts twice: eq. 12 gives every entry a
     location).
  R3 absorbed-MLA rows of 576 elements: K = all 576, V = the first 512;
     256-element rows: K = row[0:128], V = row[128:256].  (R27: the 288-B
     rows of Table 3 are 144 elements, K = all 144, V = the first 128; the
     attention here reads K = row[0:d_qk], V = row[v_off:v_off+d_v] for any
     layout the configuration names.)
  R4 the ring is a separate local branch joined in one softmax: query j also
     attends positions max(ring_lo, p_j - W + 1) .. p_j of its ring (and, with
     ring_block_only, only those >= n_r); no positional dedup against the list.
  R5 a row that is both resident and in the hot cache resolves as resident
     (probe order of Figure 2).
  R6 LRU: per-step timestamps; the step counter of a group starts above every
     age given to set_hot; hits are stamped with the step counter t; victims
     are slots whose row is not in U_r, ordered by (last_used, slot) with
     empty slots first.
  R7 the i-th missing row (ascending) takes the i-th victim; missing rows
     beyond the victims overflow (staged only).
  R8 staging order: missing rows ascending, dense, in the request's segment
     of K_max*k rows of the arena.
  R9 location codes: tier in bits 30..29 (0 hot slot r*B+slot, 1 staged
     r*K_max*k+i, 2 resident pool index, 3 ring row r*R_d + (u mod R_d) of a
     tail row, R24), index in bits 28..0, -1 for pads and invalid entries;
     every valid code is a non-negative int32.
  R10 resident pool indices are handed out per layer group in call order of
     set_resident, ascending row order within a call.
  R24 the tail (Figure 2 callout 1; §3.1 "mutable tail"; Figure 3 callout 4):
     a selected history row still held by the request's ring resolves there
     directly, before the optional map and the hot cache.  The ring holds
     position u while u >= ring_lo and u >= n_r + K_max - R_d (slots of
     older positions may already carry this step's new rows, eq. 10);
     location tier 3, index r*R_d + (u mod R_d).  Tail rows are never
     inserted in the hot cache.
  R26 compressed sources, below.

Compressed sources (§3.3 eq. 8, R26): a group whose stored rows each pack m
consecutive token positions.  Its history rows are source rows; a list entry
s is valid iff 0 <= s < floor(n_r / m) (complete rows only: the incomplete
group stays in the tail as positions, reached by the ring branch); a commit
from n to n' completes the source rows floor(n/m) <= s < floor(n'/m), whose
bytes (the model's compressed rows) the caller supplies.  Selections of such
a source never resolve from the tail (the ring holds positions, not source
rows).

Dynamic optional residency (§3.1, eqs. 3-4) is modelled in ``residency.py``;
once attached, its ready map (shared by every group) is what step (1) of the
resolution order consults, in place of the static resident sets.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from . import native

HOT, STAGED, RESIDENT, RING = 0, 1, 2, 3  # tiers of a location code (R9)
CLS_RESIDENT, CLS_HOT, CLS_MISS, CLS_TAIL = 0, 1, 2, 3  # class of a union row


def loc_code(tier: int, index: int) -> int:
    return (tier << 29) | index


# ---------------------------------------------------------------------------
# closed forms of §3.4

def ring_rows(window: int, page: int, k_max: int) -> int:
    """Eq. (9): R_d = p * ceil((W + p - 1 + K_max) / p)."""
    return page * math.ceil((window + page - 1 + k_max) / page)


def ring_addr(slot: int, pos: int, r_d: int) -> int:
    """Eq. (10): phi(i, t) = i * R_d + (t mod R_d)."""
    return slot * r_d + (pos % r_d)


def completed_rows(n: int, n_new: int, m: int) -> range:
    """Eq. (8): source rows completed when the frontier moves from n to n_new,
    floor(n/m) <= s < floor(n_new/m) (complete rows only)."""
    return range(n // m, n_new // m)


def staging_bytes(chi: int, n_slots: int, k_max: int, k: int, d_kv: int) -> int:
    """§3.4: M_stage = chi * N * K_max * k * d_KV."""
    return chi * n_slots * k_max * k * d_kv


# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class OracleConfig:
    n_req: int
    n_groups: int
    hist_cap: int
    n_prefix: int
    prefix_len: int
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
    softmax_scale: float = 0.0      # <= 0: 1/sqrt(d_qk)
    ring_block_only: bool = False

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.d_qk)

    @property
    def plen(self) -> int:
        return self.prefix_len if self.n_prefix > 0 else 0


@dataclass
class _Req:
    slot_row: List[int]
    slot_lu: List[int]
    slot_of: Dict[int, int]
    res_idx: Dict[int, int]
    ring: Dict[int, np.ndarray]
    ring_lo: int
    resident_set: bool = False


@dataclass
class ReqResult:
    active: bool
    k_active: int = 0
    union: List[int] = field(default_factory=list)
    cls: List[int] = field(default_factory=list)
    miss: List[int] = field(default_factory=list)
    victims: List[int] = field(default_factory=list)   # victim slot of miss i, i < n_promote
    overflow: int = 0
    loc: Optional[np.ndarray] = None                    # int32 [Q, k]
    counts: Dict[str, int] = field(default_factory=dict)


@dataclass
class StepResult:
    step: int
    req: Dict[int, ReqResult]
    out: Dict[tuple, np.ndarray]                        # (r, j) -> double [H, d_v]


class HierOracle:
    """Per layer group g and request r: hot-cache slot table, resident map and
    ring, exactly as the paper's state; host rows are ``histories[g]``
    (a ``workloads.History``), written in place by ``commit``."""

    def __init__(self, cfg: OracleConfig, histories, hist_len, requests=None):
        self.cfg = cfg
        self.hist = histories
        self.n = [int(x) for x in hist_len]
        self.requests = list(range(cfg.n_req)) if requests is None else sorted(int(r) for r in requests)
        self.t = [0] * cfg.n_groups
        self.res_cursor = [0] * cfg.n_groups
        self.r_d = ring_rows(cfg.ring_window, cfg.ring_page, cfg.q_max)
        self.last_k = {r: 0 for r in self.requests}
        self.opt = None                                   # dynamic optional residency (residency.py)
        self.last_sel = [None] * cfg.n_groups             # (topk, causal_pos, per-request activity)
        self.m = [1] * cfg.n_groups                       # positions per stored row (eq. 8)
        self.st = [{r: _Req(slot_row=[-1] * cfg.hot_slots, slot_lu=[0] * cfg.hot_slots,
                            slot_of={}, res_idx={}, ring={}, ring_lo=self.n[r])
                    for r in self.requests} for _ in range(cfg.n_groups)]

    # ------------------------------------------------------------- set-up
    def set_hot(self, g: int, r: int, rows, ages):
        B = self.cfg.hot_slots
        rows = [int(x) for x in rows]
        ages = [int(x) for x in ages]
        if len(rows) != len(ages) or len(rows) > B:
            raise ValueError("bad hot set size")
        live = [x for x in rows if x >= 0]
        if len(set(live)) != len(live) or any(x >= self.cfg.hist_cap for x in live) \
                or any(x < -1 for x in rows) or any(a < 0 for a in ages):
            raise ValueError("bad hot set")
        if ages:
            self.t[g] = max(self.t[g], max(ages))          # R6 (every request counts)
        if r not in self.st[g]:
            return                                        # request not modelled here
        st = self.st[g][r]
        st.slot_row = rows + [-1] * (B - len(rows))
        st.slot_lu = ages + [0] * (B - len(ages))
        st.slot_of = {x: s for s, x in enumerate(st.slot_row) if x >= 0}

    def set_resident(self, g: int, r: int, bitmap):
        bm = np.asarray(bitmap)
        rows = [s for s in range(min(bm.size, self.n[r])) if bm[s]]
        if self.opt is not None:
            raise RuntimeError("static resident sets and dynamic residency do not mix")
        if r not in self.st[g]:                           # not modelled: only the cursor moves (R10)
            self.res_cursor[g] += len(rows)
            return
        st = self.st[g][r]
        if st.resident_set:
            raise RuntimeError("resident set already given for this request and group")
        for s in rows:                                    # R10
            st.res_idx[s] = self.res_cursor[g]
            self.res_cursor[g] += 1
        st.resident_set = True

    def set_compression(self, g: int, m: int):
        """Group g stores one row per m consecutive positions (eq. 8)."""
        if m < 1:
            raise ValueError("m must be >= 1")
        self.m[g] = int(m)

    def attach_residency(self, opt):
        """Dynamic optional residency: the ready map of `opt` (shared by every
        group) replaces the static resident sets."""
        if any(st.resident_set for grp in self.st for st in grp.values()):
            raise RuntimeError("static resident sets and dynamic residency do not mix")
        self.opt = opt

    def _resident(self, g: int, r: int, u: int):
        """Resident pool row of history row u, or None (Figure 2 callout 1)."""
        if self.opt is not None:
            return self.opt.lookup(r, u)
        return self.st[g][r].res_idx.get(u)

    def clear_resident(self, g: int):
        self.res_cursor[g] = 0
        for st in self.st[g].values():
            st.res_idx = {}
            st.resident_set = False

    def ring_load(self, g: int, r: int, first_pos: int, rows: np.ndarray):
        """Committed positions first_pos .. n_r-1 enter the ring (eq. 10)."""
        n = rows.shape[0]
        if first_pos < 0 or first_pos + n != self.n[r] or n > self.r_d:
            raise ValueError("ring_load must end at the frontier and fit the ring")
        st = self.st[g][r]
        for i in range(n):
            st.ring[first_pos + i] = np.array(rows[i], dtype=np.uint16)
        st.ring_lo = first_pos

    # ------------------------------------------------------------- helpers
    def host_row(self, g: int, r: int, s: int) -> np.ndarray:
        h = self.hist[g]
        plen = self.cfg.plen
        if s < plen:
            return h.prefix[r % self.cfg.n_prefix, s]
        return h.tails[r, s - plen]

    def window(self, g: int, r: int, n_r: int, p_j: int) -> range:
        st = self.st[g][r]
        lo = max(st.ring_lo, p_j - self.cfg.ring_window + 1, 0)   # R4
        if self.cfg.ring_block_only:
            lo = max(lo, n_r)
        return range(lo, p_j + 1)

    # ------------------------------------------------------------- the step
    def verify_step(self, g: int, topk, causal_pos, queries, block_rows,
                    attend="all", n_threads: int = 1) -> StepResult:
        cfg = self.cfg
        Q, k, B = cfg.q_max, cfg.topk, cfg.hot_slots
        self.t[g] += 1
        t = self.t[g]
        res: Dict[int, ReqResult] = {}
        for r in self.requests:
            st = self.st[g][r]
            cp = [int(x) for x in causal_pos[r]]
            if cp[0] < 0:
                res[r] = ReqResult(active=False, loc=np.full((Q, k), -1, dtype=np.int32))
                self.last_k[r] = 0
                continue
            J = [j for j in range(Q) if cp[j] >= 0]
            self.last_k[r] = len(J)
            m = self.m[g]
            n_r = cp[0] // m                              # complete stored rows (eq. 8)
            # Figure 3 callout 4: the rows of all K queries are written; eq. (10) places them.
            # A Reindex consumer of a shared source passes no rows: the source's
            # producer already wrote this step's block (§2, physical-source sharing).
            if block_rows is not None:
                for j in J:
                    st.ring[cp[j]] = np.array(block_rows[r][j], dtype=np.uint16)

            # eq. (6): U_r is the union of the K_r selections (R1 for validity)
            n_sel = n_pad = n_bad = 0
            valid = set()
            for j in J:
                for e in topk[r][j]:
                    e = int(e)
                    if e == -1:
                        n_pad += 1
                    elif 0 <= e < n_r:
                        n_sel += 1
                        valid.add(e)
                    else:
                        n_bad += 1
            U = sorted(valid)

            # Figure 2 / §3.2: (1) direct map, (2) hot cache, (3) host; R5
            cls = {}
            res_at = {}
            tail_lo = max(st.ring_lo, n_r + Q - self.r_d) if m == 1 else n_r   # R24
            for u in U:
                ri = self._resident(g, r, u)
                if u >= tail_lo:
                    if u not in st.ring:
                        raise RuntimeError("tail row %d of request %d not in the ring" % (u, r))
                    cls[u] = CLS_TAIL
                elif ri is not None:
                    res_at[u] = ri
                    cls[u] = CLS_RESIDENT
                elif u in st.slot_of:
                    cls[u] = CLS_HOT
                else:
                    cls[u] = CLS_MISS
            D = [u for u in U if cls[u] == CLS_MISS]          # eq. (6): D_r = U_r \ R_r
            stage = {u: i for i, u in enumerate(D)}          # R8

            # §3.5 eq. (12): one location per list entry, in selection order (R9)
            seg = r * Q * k
            loc = np.full((Q, k), -1, dtype=np.int32)
            sel_cls = [0, 0, 0, 0]
            for j in J:
                for i, e in enumerate(topk[r][j]):
                    e = int(e)
                    if not (0 <= e < n_r):
                        continue
                    c = cls[e]
                    sel_cls[c] += 1
                    if c == CLS_TAIL:
                        loc[j, i] = loc_code(RING, r * self.r_d + e % self.r_d)
                    elif c == CLS_RESIDENT:
                        loc[j, i] = loc_code(RESIDENT, res_at[e])
                    elif c == CLS_HOT:
                        loc[j, i] = loc_code(HOT, r * B + st.slot_of[e])
                    else:
                        loc[j, i] = loc_code(STAGED, seg + stage[e])

            # §2.2: hits refresh recency, selected rows are protected, LRU victims (R6, R7)
            in_u = set(U)
            for u in U:
                if cls[u] == CLS_HOT:
                    st.slot_lu[st.slot_of[u]] = t
            cand = [s for s in range(B) if st.slot_row[s] == -1 or st.slot_row[s] not in in_u]
            cand.sort(key=lambda s: (-1 if st.slot_row[s] == -1 else st.slot_lu[s], s))
            n_prom = min(len(D), len(cand))
            victims = cand[:n_prom]
            # §3.4: promoted rows take their victim slots (copied back after attention)
            for i, s in enumerate(victims):
                old = st.slot_row[s]
                if old != -1:
                    del st.slot_of[old]
                st.slot_row[s] = D[i]
                st.slot_lu[s] = t
                st.slot_of[D[i]] = s

            counts = dict(selections=n_sel, pads=n_pad, invalid=n_bad, union=len(U),
                          union_resident=sum(1 for u in U if cls[u] == CLS_RESIDENT),
                          union_hot=sum(1 for u in U if cls[u] == CLS_HOT),
                          union_miss=len(D), promoted=n_prom, overflow=len(D) - n_prom,
                          sel_resident=sel_cls[0], sel_hot=sel_cls[1], sel_miss=sel_cls[2],
                          union_tail=sum(1 for u in U if cls[u] == CLS_TAIL), sel_tail=sel_cls[3],
                          queries=len(J))
            res[r] = ReqResult(active=True, k_active=len(J), union=U,
                               cls=[cls[u] for u in U], miss=D, victims=victims,
                               overflow=len(D) - n_prom, loc=loc, counts=counts)

        out = self._attend(g, topk, causal_pos, queries, res, attend, n_threads)
        self.last_sel[g] = (np.array(topk, dtype=np.int32, copy=True), np.array(causal_pos, dtype=np.int32, copy=True),
                            {r: res[r].active for r in self.requests})
        return StepResult(step=t, req=res, out=out)

    def verify_reuse(self, g: int, queries, attend="all", n_threads: int = 1) -> Dict[tuple, np.ndarray]:
        """A Reuse consumer (§2 "physical-source sharing"; §3.2): new queries
        attend over the latest selection of source g through its location
        vector and payload.  Placement never changes the result (eqs. 11-12),
        so this is eq. (1) over that selection's lists plus the ring window;
        no resolution, fetch or cache update happens."""
        if self.last_sel[g] is None:
            raise RuntimeError("no selection of this source to reuse")
        topk, causal_pos, active = self.last_sel[g]
        res = {r: ReqResult(active=active[r]) for r in self.requests}
        return self._attend(g, topk, causal_pos, queries, res, attend, n_threads)

    def _attend(self, g, topk, causal_pos, queries, res, attend, n_threads):
        """Eq. (1) over each query's own list (read from the original rows,
        eqs. 11-12) plus its ring window (R4)."""
        cfg = self.cfg
        pairs = []
        for r in self.requests:
            if not res[r].active:
                continue
            for j in range(cfg.q_max):
                if int(causal_pos[r][j]) < 0:
                    continue
                if attend == "all" or (attend is not None and (r, j) in attend):
                    pairs.append((r, j))
        if not pairs:
            return {}
        keep = []
        q_ptrs = np.zeros(len(pairs), dtype=np.uint64)
        row_begin = np.zeros(len(pairs) + 1, dtype=np.int64)
        ptrs = []
        for qi, (r, j) in enumerate(pairs):
            st = self.st[g][r]
            n_r = int(causal_pos[r][0])
            n_src = n_r // self.m[g]
            p_j = int(causal_pos[r][j])
            qa = np.ascontiguousarray(queries[r][j], dtype=np.uint16)
            keep.append(qa)
            q_ptrs[qi] = qa.ctypes.data
            for e in topk[r][j]:
                e = int(e)
                if 0 <= e < n_src:
                    ptrs.append(self.host_row(g, r, e).ctypes.data)
            for pos in self.window(g, r, n_r, p_j):
                if pos not in st.ring:
                    raise RuntimeError("ring position %d of request %d was never written" % (pos, r))
                ptrs.append(st.ring[pos].ctypes.data)
            row_begin[qi + 1] = len(ptrs)
        row_ptrs = np.array(ptrs, dtype=np.uint64)
        out = native.attend_batch(cfg.n_heads, cfg.d_qk, cfg.v_off, cfg.d_v, cfg.row_elems,
                                  cfg.scale, q_ptrs, row_begin, row_ptrs, n_threads)
        return {pr: out[i] for i, pr in enumerate(pairs)}

    # ------------------------------------------------------------- acceptance
    def commit(self, accepted, src_rows=None):
        """Eq. (7): the anchor and A_r accepted drafts join history,
        n' = n + 1 + A; committed rows get their host copy and rejected rows
        are never published (§3.3, after eq. 8).  A compressed group (m > 1)
        instead gains the source rows floor(n/m) <= s < floor(n'/m) (eq. 8),
        taken from src_rows[g][r][s - floor(n/m)].  The step's selections end
        with it: nothing is left to reuse."""
        self.last_sel = [None] * self.cfg.n_groups
        for r in self.requests:
            a = int(accepted[r])
            if a < 0:
                continue
            if self.last_k[r] == 0 or a >= self.last_k[r]:
                raise ValueError("accepted count beyond the verified block")
            n = self.n[r]
            new_n = n + 1 + a
            if new_n > self.cfg.hist_cap:
                raise ValueError("history capacity exceeded")
            for g in range(self.cfg.n_groups):
                st = self.st[g][r]
                m = self.m[g]
                if m == 1:
                    for pos in range(n, new_n):
                        assert pos >= self.cfg.plen
                        self.hist[g].tails[r, pos - self.cfg.plen] = st.ring[pos]
                else:
                    for i, s_row in enumerate(completed_rows(n, new_n, m)):
                        assert s_row >= self.cfg.plen
                        self.hist[g].tails[r, s_row - self.cfg.plen] = np.asarray(src_rows[g][r][i], np.uint16)
                for pos in [p for p in st.ring if p >= new_n]:
                    del st.ring[pos]
            self.n[r] = new_n

    # ------------------------------------------------------------- views
    def slot_table(self, g: int, r: int):
        st = self.st[g][r]
        return np.array(st.slot_row, dtype=np.int32), np.array(st.slot_lu, dtype=np.int32)

