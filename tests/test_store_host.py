"""Prefix-cache store bookkeeping on the CPU (no device calls): the store runs
over a host-memory arena, and every reserve / commit / abort / lookup /
release / erase / stats result is compared with a Python model of the policy
that include/skv.h states -- 256-byte granules, the lowest free offset that
fits, coalescing of freed runs, least-recently-used eviction of unpinned
committed entries only when evicting all of them would make room, lookups by
the longest verified leading run of block hashes with the most recently used
entry winning ties, pins held by lookups."""
import os

import numpy as np
import pytest
import torch

GRAN = 256


@pytest.fixture(scope="module")
def skv():
    from lossless_kv_cache_amd import skv as m
    if not os.path.exists(m.LIB_PATH):
        from lossless_kv_cache_amd import build
        build.build()
    m.lib()
    return m


def host_arena(nbytes: int, misalign: int = 0) -> torch.Tensor:
    """A uint8 host tensor of nbytes whose first byte sits `misalign` bytes past a 256-byte boundary."""
    raw = torch.empty(nbytes + 2 * GRAN, dtype=torch.uint8)
    off = (-raw.data_ptr()) % GRAN + misalign
    return raw[off:off + nbytes]


# ------------------------------------------------------------------ model
class Model:
    def __init__(self, size):
        self.size = size
        self.free = {0: size}
        self.ent = {}
        self.lru = []
        self.next_id = 1
        self.tick = 0
        self.c = dict(inserts=0, evictions=0, hits=0, misses=0, hit_blocks=0)

    def _take(self, span):
        for off in sorted(self.free):
            if self.free[off] >= span:
                rest = self.free.pop(off) - span
                if rest:
                    self.free[off + span] = rest
                return off
        return None

    def _give(self, off, n):
        if not n:
            return
        self.free[off] = n
        runs = sorted(self.free.items())
        merged = []
        for o, l in runs:
            if merged and merged[-1][0] + merged[-1][1] == o:
                merged[-1][1] += l
            else:
                merged.append([o, l])
        self.free = {o: l for o, l in merged}

    def _possible(self):
        fixed = sorted((e["off"], e["span"]) for e in self.ent.values() if not e["committed"] or e["pins"])
        at, m = 0, 0
        for o, s in fixed:
            m = max(m, o - at)
            at = o + s
        return max(m, self.size - at)

    def _drop(self, i):
        e = self.ent.pop(i)
        if e["committed"]:
            self.lru.remove(i)
        self._give(e["off"], e["span"])

    def reserve(self, hashes, nbytes):
        if len(hashes) == 0 or nbytes == 0:
            return -1, None
        span = -(-nbytes // GRAN) * GRAN
        if span > self.size:
            return -3, None
        off = self._take(span)
        if off is None:
            if self._possible() < span:
                return -3, None
            for i in list(self.lru):
                if self.ent[i]["pins"]:
                    continue
                self._drop(i)
                self.c["evictions"] += 1
                off = self._take(span)
                if off is not None:
                    break
        i = self.next_id
        self.next_id += 1
        self.ent[i] = dict(off=off, span=span, bytes=0, hashes=list(hashes), pins=0, committed=False, tick=0)
        return 0, (i, off)

    def commit(self, i, nbytes):
        e = self.ent.get(i)
        if e is None or e["committed"] or nbytes == 0 or nbytes > e["span"]:
            return -1
        span = -(-nbytes // GRAN) * GRAN
        self._give(e["off"] + span, e["span"] - span)
        e.update(span=span, bytes=nbytes, committed=True)
        self.lru.append(i)
        self.tick += 1
        e["tick"] = self.tick
        self.c["inserts"] += 1
        return 0

    def abort(self, i):
        e = self.ent.get(i)
        if e is None or e["committed"]:
            return -1
        self._drop(i)
        return 0

    def lookup(self, q):
        for b in range(len(q) - 1, -1, -1):
            best = None
            for i, e in self.ent.items():
                if e["committed"] and len(e["hashes"]) > b and e["hashes"][:b + 1] == list(q[:b + 1]):
                    if best is None or e["tick"] > self.ent[best]["tick"]:
                        best = i
            if best is not None:
                e = self.ent[best]
                e["pins"] += 1
                self.tick += 1
                e["tick"] = self.tick
                self.lru.remove(best)
                self.lru.append(best)
                self.c["hits"] += 1
                self.c["hit_blocks"] += b + 1
                return (best, b + 1, len(e["hashes"]), e["off"], e["bytes"])
        self.c["misses"] += 1
        return (0, 0, 0, None, 0)

    def release(self, i):
        e = self.ent.get(i)
        if e is None or not e["committed"] or e["pins"] == 0:
            return -1
        e["pins"] -= 1
        return 0

    def erase(self, i):
        e = self.ent.get(i)
        if e is None or not e["committed"]:
            return -1
        if e["pins"]:
            return -8
        self._drop(i)
        return 0

    def stats(self):
        com = [e for e in self.ent.values() if e["committed"]]
        return dict(arena_bytes=self.size, used_bytes=self.size - sum(self.free.values()),
                    largest_free=max(self.free.values(), default=0),
                    container_bytes=sum(e["bytes"] for e in com), entries=len(com),
                    pinned=sum(1 for e in com if e["pins"]), **self.c)


def call(skv, fn, *args):
    try:
        return 0, fn(*args)
    except skv.SkvError as e:
        return e.status, None


# ------------------------------------------------------------------ tests
def test_create_rules(skv):
    for arena in (host_arena(4096, misalign=16), host_arena(4000), host_arena(128)):
        with pytest.raises(skv.SkvError) as ei:
            skv.Store(arena=arena)
        assert ei.value.status == skv.ERR_ARG
    st = skv.Store(arena=host_arena(4096))
    assert st.stats()["arena_bytes"] == 4096 and st.stats()["largest_free"] == 4096
    st.close()
    with pytest.raises(ValueError):
        st.stats()


def test_first_fit_shrink_and_coalesce(skv):
    base = host_arena(8 * GRAN)
    st = skv.Store(arena=base)
    p0 = base.data_ptr()
    a, va = st.reserve(3 * GRAN, [1])
    assert va.data_ptr() == p0 and va.numel() == 3 * GRAN
    st.commit(a, 300)                                    # shrinks to 2 granules
    b, vb = st.reserve(GRAN, [2])
    assert vb.data_ptr() == p0 + 2 * GRAN
    st.commit(b, GRAN)
    c, vc = st.reserve(2 * GRAN, [3])
    assert vc.data_ptr() == p0 + 3 * GRAN
    st.commit(c, 2 * GRAN)
    s = st.stats()
    assert (s["used_bytes"], s["container_bytes"], s["entries"], s["largest_free"]) == (5 * GRAN, 300 + 3 * GRAN, 3,
                                                                                       3 * GRAN)
    st.erase(a)
    st.erase(b)                                          # [0, 3 granules) coalesced
    d, vd = st.reserve(3 * GRAN, [4])
    assert vd.data_ptr() == p0
    st.abort(d)
    assert st.stats()["largest_free"] == 3 * GRAN and st.stats()["evictions"] == 0


def test_lru_eviction_respects_pins_and_feasibility(skv):
    st = skv.Store(arena=host_arena(4 * GRAN))
    ids = []
    for k in range(4):
        i, _ = st.reserve(GRAN, [100 + k])
        st.commit(i, GRAN)
        ids.append(i)
    hit = st.lookup([100])                               # entry 0 pinned and most recent
    assert hit.entry == ids[0] and hit.matched_blocks == 1
    i, v = st.reserve(2 * GRAN, [200])                   # evicts ids[1] then ids[2] (least recent, adjacent)
    assert v.data_ptr() == st.arena.data_ptr() + GRAN
    s = st.stats()
    assert s["evictions"] == 2 and s["entries"] == 2
    assert st.lookup([101]).entry == 0 and st.lookup([102]).entry == 0
    st.commit(i, 2 * GRAN)
    # 4 granules can only come from evicting the pinned entry: refused, nothing evicted
    with pytest.raises(skv.SkvError) as ei:
        st.reserve(4 * GRAN, [300])
    assert ei.value.status == skv.ERR_CAPACITY
    assert st.stats()["evictions"] == 2 and st.stats()["entries"] == 3
    with pytest.raises(skv.SkvError) as ei:
        st.erase(ids[0])
    assert ei.value.status == skv.ERR_BUSY
    st.release(ids[0])
    st.erase(ids[0])
    with pytest.raises(skv.SkvError) as ei:
        st.release(ids[0])
    assert ei.value.status == skv.ERR_ARG
    with pytest.raises(skv.SkvError) as ei:
        st.reserve(5 * GRAN, [400])                      # larger than the arena
    assert ei.value.status == skv.ERR_CAPACITY


def test_lookup_longest_verified_prefix(skv):
    st = skv.Store(arena=host_arena(64 * GRAN))
    a = [11, 12, 13, 14]
    b = [11, 12, 23]
    c = [91, 12, 13]                                     # same later hashes, different first block
    ia, _ = st.reserve(GRAN, a)
    st.commit(ia, 10)
    ib, _ = st.reserve(GRAN, b)
    st.commit(ib, 10)
    ic, _ = st.reserve(GRAN, c)
    st.commit(ic, 10)
    h = st.lookup([11, 12, 13, 99, 5])
    assert (h.entry, h.matched_blocks, h.entry_blocks) == (ia, 3, 4)
    st.release(ia)
    h = st.lookup([11, 12, 77])                          # a and b both hold 2 blocks: a was used last
    assert (h.entry, h.matched_blocks) == (ia, 2)
    st.release(ia)
    h = st.lookup([11, 12, 23])
    assert (h.entry, h.matched_blocks, h.entry_blocks) == (ib, 3, 3)
    st.release(ib)
    h = st.lookup([11, 12, 88])                          # now b was used last
    assert (h.entry, h.matched_blocks) == (ib, 2)
    st.release(ib)
    h = st.lookup([55, 12, 13])                          # 12, 13 at the right positions, first block differs
    assert (h.entry, h.matched_blocks) == (0, 0)
    h = st.lookup([])
    assert h.entry == 0
    s = st.stats()
    assert (s["hits"], s["misses"], s["hit_blocks"], s["pinned"]) == (4, 2, 10, 0)


def test_block_hashes_chain(skv):
    rng = np.random.default_rng(7)
    x = rng.integers(0, 50000, 1000)
    y = x.copy()
    y[700] += 1
    hx, hy = skv.block_hashes(x), skv.block_hashes(y)
    assert len(hx) == 7 and hx.dtype == np.uint64
    assert (hx[:5] == hy[:5]).all() and (hx[5:] != hy[5:]).all()
    assert len(set(hx.tolist())) == 7
    z = np.concatenate([x[:128], x[:128]])               # equal blocks at different positions differ
    hz = skv.block_hashes(z)
    assert hz[0] != hz[1]


@pytest.mark.parametrize("seed", range(6))
def test_random_sequences_match_model(skv, seed):
    rng = np.random.default_rng(seed)
    size = int(rng.integers(8, 40)) * GRAN
    arena = host_arena(size)
    st = skv.Store(arena=arena)
    m = Model(size)
    # hash chains sharing prefixes: each new chain copies a prefix of an earlier one
    chains = []
    for _ in range(12):
        n = int(rng.integers(1, 9))
        if chains and rng.random() < 0.7:
            par = chains[int(rng.integers(len(chains)))]
            k = int(rng.integers(0, len(par) + 1))
            ch = par[:k] + [int(v) for v in rng.integers(1, 2**63, n)]
        else:
            ch = [int(v) for v in rng.integers(1, 2**63, n)]
        chains.append(ch[:12])
    open_res = {}
    for step in range(400):
        op = rng.choice(["reserve", "commit", "abort", "lookup", "release", "erase"], p=[.3, .2, .05, .25, .12, .08])
        ids = list(m.ent)
        if op == "reserve":
            ch = chains[int(rng.integers(len(chains)))]
            nb = int(rng.integers(1, 6 * GRAN))
            want, res = m.reserve(ch, nb)
            rc, got = call(skv, st.reserve, nb, ch)
            assert rc == want, (step, op)
            if rc == 0:
                assert got[0] == res[0] and got[1].data_ptr() - arena.data_ptr() == res[1], step
                open_res[got[0]] = nb
        elif op == "commit" and open_res:
            i = list(open_res)[int(rng.integers(len(open_res)))]
            nb = int(rng.integers(1, open_res[i] + 1)) if rng.random() < 0.9 else open_res[i] + GRAN
            want = m.commit(i, nb)
            rc, _ = call(skv, st.commit, i, nb)
            assert rc == want, (step, op)
            if rc == 0:
                del open_res[i]
        elif op == "abort" and open_res:
            i = list(open_res)[0]
            assert call(skv, st.abort, i)[0] == m.abort(i) == 0
            del open_res[i]
        elif op == "lookup":
            ch = chains[int(rng.integers(len(chains)))]
            q = ch[:int(rng.integers(0, len(ch) + 1))] + [int(v) for v in rng.integers(1, 2**63, int(rng.integers(0, 3)))]
            want = m.lookup(q)
            h = st.lookup(q)
            got = (h.entry, h.matched_blocks, h.entry_blocks,
                   (h.container - arena.data_ptr()) if h.entry else None, h.container_bytes)
            assert got == want, (step, op)
        elif op == "release" and ids:
            i = ids[int(rng.integers(len(ids)))]
            assert call(skv, st.release, i)[0] == m.release(i), (step, op)
        elif op == "erase" and ids:
            i = ids[int(rng.integers(len(ids)))] if rng.random() < 0.9 else 10**9
            assert call(skv, st.erase, i)[0] == m.erase(i), (step, op)
        assert st.stats() == m.stats(), (step, op)
