"""A CPU model of the fused forward's hand-off protocol (the persistent kernel of mok_layer_fwd and
mok_layer_fwd_macro), for testing its ordering logic with threads and random delays.

Each thread plays one workgroup of the kernel and follows the kernel's control flow: it
registers on an XCD; the XCD's first `lag` row tiles are gathered by all of its workgroups; then
the first C workgroups of the XCD are dispatch workers (they take the XCD's next row tile from one
global counter once its gather slot and activation slot are free, gather it, and count
themselves in landed[t]) and the others are GEMM workers (they take the XCD's next item number
from the XCD's item counter: gate/up items of the first `lag` tiles, then blocks [gate/up of tile
q + lag, down of tile q]). Waits: gate/up of tile t waits for landed[t], and before it stores h
for dn_done of the XCD's (q - caph)-th tile (the last reader of its h slot); down of tile t for
gu_done[t]; the dispatch of the XCD's q-th tile for gu_done of its (q - capx)-th tile (gather
slot) and dn_done of its (q - capa)-th (activation slot). Counters and the per-XCD tile list
are shared integers under one lock (the kernel's atomics).

Slot contents are tracked explicitly: a gather writes "tile t" into its gather slot; a gate/up
item checks that the gather slot still holds its tile when it starts and when it ends, writes
"tile t" into the activation slot (g|u, read only by the backward) and then into the h slot; a
down item checks that the h slot holds its tile when it starts and when it ends. A protocol
error (a slot overwritten while an item of the previous tile still reads or writes it, an item
run twice, a wait that never ends) raises in the thread that sees it.

Test infrastructure only: nothing in the library imports it.
"""
from __future__ import annotations

import random
import threading
import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple


class ProtocolError(AssertionError):
    pass


@dataclass
class Params:
    xcds: int = 2               # XCDs (each its own ring share)
    wgs_per_xcd: int = 5        # workgroups registered on each XCD
    comm: int = 1               # dispatch workers per XCD (C)
    ngu: int = 3                # gate/up items per row tile
    ndn: int = 2                # down items per row tile
    capx: int = 3               # gather slots per XCD
    capa: int = 3               # activation slots per XCD
    caph: int = 3               # h slots per XCD
    tiles: Tuple[int, ...] = (11,)   # row tiles per macrobatch
    max_delay: float = 0.0005   # random sleep per step (seconds)
    timeout: float = 20.0       # a wait longer than this is a deadlock


@dataclass
class State:
    p: Params
    lock: threading.Lock = field(default_factory=threading.Lock)
    reg: List[int] = field(default_factory=list)
    arrived: int = 0
    next_tile: int = 0
    item: List[int] = field(default_factory=list)
    xend: List[int] = field(default_factory=list)
    xq: List[List[int]] = field(default_factory=list)
    landed: Dict[int, int] = field(default_factory=dict)
    gu_done: Dict[int, int] = field(default_factory=dict)
    dn_done: Dict[int, int] = field(default_factory=dict)
    gather_slot: Dict[Tuple[int, int], int] = field(default_factory=dict)   # (x, s) -> tile
    act_slot: Dict[Tuple[int, int], int] = field(default_factory=dict)
    h_slot: Dict[Tuple[int, int], int] = field(default_factory=dict)
    done_items: Dict[Tuple[int, str, int], int] = field(default_factory=dict)
    rowner: Dict[Tuple[int, int], Tuple[int, int]] = field(default_factory=dict)  # slot -> (b, t)
    failures: List[str] = field(default_factory=list)

    def __post_init__(self):
        n = self.p.xcds
        self.reg = [0] * n
        self.item = [0] * n
        self.xend = [-1] * n
        self.xq = [[] for _ in range(n)]

    @property
    def nt(self) -> int:
        return sum(self.p.tiles)

    def macro_of(self, g: int) -> Tuple[int, int]:
        first = 0
        for b, n in enumerate(self.p.tiles):
            if g < first + n:
                return b, g - first
            first += n
        raise ProtocolError(f"tile {g} beyond the list")


def _nap(p: Params):
    if p.max_delay > 0:
        time.sleep(random.random() * p.max_delay)


def _wait(st: State, cond, what: str):
    t0 = time.monotonic()
    while True:
        with st.lock:
            if st.failures:
                raise ProtocolError("another worker failed")
            if cond():
                return
        if time.monotonic() - t0 > st.p.timeout:
            raise ProtocolError(f"wait never ended: {what}")
        time.sleep(0.0001)


def _workgroup(st: State, wid: int):
    p = st.p
    x = wid % p.xcds                                   # blockIdx % xcds, as on the device
    with st.lock:
        local = st.reg[x]
        st.reg[x] += 1
        st.arrived += 1
    _wait(st, lambda: st.arrived == p.xcds * p.wgs_per_xcd, "registration")
    nx = p.wgs_per_xcd
    C = min(p.comm, nx - 1)
    lag = 2 if p.capa > 2 else 1
    gmax = 1 << 20

    def tile_of(q: int) -> int:
        """The XCD's q-th tile once published, or nt (none)."""
        out = []

        def ready():
            if q < len(st.xq[x]):
                out.append(st.xq[x][q])
                return True
            if st.xend[x] >= 0 and q >= st.xend[x]:
                out.append(st.nt)
                return True
            return False
        _wait(st, ready, f"xcd {x} tile {q}")
        return out[0]

    def take_tile(q: int) -> int:
        if local != 0:
            return tile_of(q)
        with st.lock:
            t = st.next_tile
            st.next_tile += 1
            if t >= st.nt:
                st.xend[x] = q
                return st.nt
            if len(st.xq[x]) != q:
                raise ProtocolError(f"xcd {x} took tile index {q} out of order")
            slot = (x, q % p.capa)
            st.rowner[slot] = st.macro_of(t)
            st.xq[x].append(t)
            return t

    def gather(q: int, t: int):
        s = (x, q % p.capx)
        with st.lock:
            prev = st.gather_slot.get(s)
            if prev is not None and prev != t and st.gu_done.get(prev, 0) < p.ngu:
                st.failures.append(f"gather slot {s} overwritten while tile {prev} in use")
                raise ProtocolError(st.failures[-1])
            st.gather_slot[s] = t
        _nap(p)
        with st.lock:
            st.landed[t] = st.landed.get(t, 0) + 1

    # prologue: the first lag tiles, gathered by every workgroup of the XCD
    ended = False
    for q in range(lag):
        t = take_tile(q)
        if t >= st.nt:
            ended = True
            break
        gather(q, t)

    if local < C:
        q = lag
        while not ended:
            if q >= p.capx:
                tq = st.xq[x][q - p.capx]
                _wait(st, lambda: st.gu_done.get(tq, 0) >= p.ngu, f"gather slot of tile {tq}")
            if q >= p.capa:
                ta = st.xq[x][q - p.capa]
                _wait(st, lambda: st.dn_done.get(ta, 0) >= p.ndn, f"act slot of tile {ta}")
            t = take_tile(q)
            if t >= st.nt:
                break
            gather(q, t)
            q += 1
        return

    per_tile = p.ngu + p.ndn
    while True:
        with st.lock:
            it = st.item[x]
            st.item[x] += 1
        if it < lag * p.ngu:
            q, k = it // p.ngu, it % p.ngu
        else:
            blk, off = divmod(it - lag * p.ngu, per_tile)
            if tile_of(blk) >= st.nt:
                break
            q, k = (blk + lag, off) if off < p.ngu else (blk, off)
        t = tile_of(q)
        if t >= st.nt:
            if q == 0:
                break
            continue
        kind = "gu" if k < p.ngu else "dn"
        key = (t, kind, k)
        with st.lock:
            if key in st.done_items:
                st.failures.append(f"item {key} run twice")
                raise ProtocolError(st.failures[-1])
            st.done_items[key] = it
        if kind == "gu":
            _wait(st, lambda: st.landed.get(t, 0) >= (nx if q < lag else C), f"landed {t}")
            gs, as_, hs = (x, q % p.capx), (x, q % p.capa), (x, q % p.caph)
            with st.lock:
                if st.gather_slot.get(gs) != t:
                    st.failures.append(f"gate/up of tile {t} found slot {gs} holding "
                                       f"{st.gather_slot.get(gs)}")
                    raise ProtocolError(st.failures[-1])
                # g|u: the slot's previous tile must have finished writing it
                prev = st.act_slot.get(as_)
                if prev is not None and prev != t and st.gu_done.get(prev, 0) < p.ngu:
                    st.failures.append(f"act slot {as_} overwritten while tile {prev} writes it")
                    raise ProtocolError(st.failures[-1])
                st.act_slot[as_] = t
            _nap(p)
            # before h: the down items of the tile that used the h slot before are done
            if q >= p.caph:
                th = tile_of(q - p.caph)
                _wait(st, lambda: st.dn_done.get(th, 0) >= p.ndn, f"h slot of tile {th}")
            with st.lock:
                prev = st.h_slot.get(hs)
                if prev is not None and prev != t and st.dn_done.get(prev, 0) < p.ndn:
                    st.failures.append(f"h slot {hs} overwritten while tile {prev} in use")
                    raise ProtocolError(st.failures[-1])
                st.h_slot[hs] = t
                if st.gather_slot.get(gs) != t:
                    st.failures.append(f"gather slot {gs} changed under gate/up of tile {t}")
                    raise ProtocolError(st.failures[-1])
                st.gu_done[t] = st.gu_done.get(t, 0) + 1
        else:
            _wait(st, lambda: st.gu_done.get(t, 0) >= p.ngu, f"gu_done {t}")
            hs = (x, q % p.caph)
            with st.lock:
                if st.h_slot.get(hs) != t:
                    st.failures.append(f"down of tile {t} found h slot {hs} holding "
                                       f"{st.h_slot.get(hs)}")
                    raise ProtocolError(st.failures[-1])
            _nap(p)
            with st.lock:
                if st.h_slot.get(hs) != t:
                    st.failures.append(f"h slot {hs} changed under down of tile {t}")
                    raise ProtocolError(st.failures[-1])
                st.dn_done[t] = st.dn_done.get(t, 0) + 1


def run(p: Params, seed: int = 0) -> State:
    """Run the protocol once with random delays; raises ProtocolError on a violation."""
    random.seed(seed)
    st = State(p)
    errors: List[BaseException] = []

    def body(w):
        try:
            _workgroup(st, w)
        except BaseException as e:  # noqa: BLE001 - reported below
            errors.append(e)
            with st.lock:
                if not st.failures:
                    st.failures.append(str(e))

    threads = [threading.Thread(target=body, args=(w,)) for w in range(p.xcds * p.wgs_per_xcd)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(p.timeout * 4)
        if t.is_alive():
            raise ProtocolError("a workgroup never finished")
    if errors:
        raise errors[0]
    return st


def item_waits(ngu: int, ndn: int, lag: int, blocks: int, caph: int = 3):
    """The waits of the GEMM items in item-number order, for the static check that every item
    waits only on lower-numbered items: returns [(item, waited item)]. Gate/up of tile q waits
    for the gather of tile q, which (for q >= capx or capa) waits for items of earlier tiles,
    and, before it stores h, for the down items of tile q - caph; down of tile q waits for the
    gate/up items of tile q."""
    number = {}
    it = 0
    for q in range(lag):
        for k in range(ngu):
            number[("gu", q, k)] = it
            it += 1
    for blk in range(blocks):
        for k in range(ngu):
            number[("gu", blk + lag, k)] = it
            it += 1
        for k in range(ndn):
            number[("dn", blk, k)] = it
            it += 1
    out = []
    for (kind, q, k), n in number.items():
        if kind == "dn":
            out.append((n, max(number[("gu", q, j)] for j in range(ngu))))
        elif q >= caph and ("dn", q - caph, 0) in number:
            out.append((n, max(number[("dn", q - caph, j)] for j in range(ndn))))
    return out
