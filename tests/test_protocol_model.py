"""The fused forward's hand-off protocol, run on the CPU model of tests/protocol_model.py with
threads and random delays: no slot is overwritten while an item of its previous tile may still
read or write it, every item runs once, every wait ends, and the ring record names each
activation slot's last tile (per macrobatch). Planted mistakes (the dispatch worker not waiting
for its gather slot; a gate/up item not waiting for its h slot) are caught."""
import itertools

import pytest

from tests import protocol_model as pm


CASES = [
    # (capx, capa, comm per XCD, tiles per macrobatch)
    (3, 2, 1, (9,)),            # the smallest ring: lag 1
    (3, 3, 1, (13,)),           # lag 2
    (3, 5, 2, (17,)),           # two dispatch workers per XCD
    (3, 4, 1, (5, 7, 3)),       # three macrobatches in one launch
]


@pytest.mark.parametrize("capx,capa,comm,tiles", CASES)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_protocol_runs_clean(capx, capa, comm, tiles, seed):
    p = pm.Params(capx=capx, capa=capa, comm=comm, tiles=tiles)
    st = pm.run(p, seed)
    nt = sum(tiles)
    # every item of every tile ran exactly once (the model raises on a second run)
    assert len(st.done_items) == nt * (p.ngu + p.ndn)
    assert all(st.gu_done[t] == p.ngu and st.dn_done[t] == p.ndn for t in range(nt))
    assert sorted(itertools.chain(*st.xq)) == list(range(nt))
    # the ring record: each activation slot is owned by the last tile its XCD put there, and
    # that tile's data is what the slot holds
    for x in range(p.xcds):
        for s in range(p.capa):
            mine = [t for q, t in enumerate(st.xq[x]) if q % p.capa == s]
            if mine:
                assert st.rowner[(x, s)] == st.macro_of(mine[-1])
                assert st.act_slot[(x, s)] == mine[-1]


def test_item_order_waits_only_on_earlier_items():
    for ngu, ndn, lag, capx, capa in [(3, 2, 1, 3, 2), (16, 28, 2, 3, 7), (4, 4, 2, 3, 6)]:
        caph = 3
        assert capa > lag and capx > lag and caph > lag
        for item, waited in pm.item_waits(ngu, ndn, lag, blocks=12, caph=caph):
            assert waited < item
        # gate/up of tile q (numbered in block q - lag) waits, through its gather, for the
        # gate/up items of tile q - capx and the down items of tile q - capa: both in earlier
        # blocks because capx > lag and capa > lag
        for q in range(max(capx, capa), 14):
            block = q - lag
            assert (q - capx) - lag < block and q - capa < block


def test_model_catches_a_gather_slot_reused_too_early(monkeypatch):
    """Plant a protocol mistake in the model: the dispatch worker takes its next tile without
    waiting for the gate/up items of the tile that last used the gather slot."""
    real_wait = pm._wait

    def skip_gather_wait(st, cond, what):
        if what.startswith("gather slot"):
            return
        return real_wait(st, cond, what)

    monkeypatch.setattr(pm, "_wait", skip_gather_wait)
    caught = 0
    for seed in range(6):
        p = pm.Params(capx=3, capa=5, comm=1, tiles=(17,), max_delay=0.002, timeout=5.0)
        try:
            pm.run(p, seed)
        except pm.ProtocolError:
            caught += 1
    assert caught > 0


def test_model_catches_an_h_slot_reused_too_early(monkeypatch):
    """Plant a protocol mistake in the model: a gate/up item stores h without waiting for the
    down items of the tile that used the h slot before."""
    real_wait = pm._wait

    def skip_h_wait(st, cond, what):
        if what.startswith("h slot"):
            return
        return real_wait(st, cond, what)

    monkeypatch.setattr(pm, "_wait", skip_h_wait)
    caught = 0
    for seed in range(6):
        p = pm.Params(capx=3, capa=5, comm=1, tiles=(17,), max_delay=0.002, timeout=5.0)
        try:
            pm.run(p, seed)
        except pm.ProtocolError:
            caught += 1
    assert caught > 0
