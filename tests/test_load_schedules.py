"""The load/wait schedules of the direct-to-LDS kernels, checked on the CPU.

A wave's vector-memory loads complete in issue order, and `s_waitcnt
vmcnt(X)` returns once at most X of its loads are still outstanding.  The
kernels wait with counts derived from the ring depth (loads issued AHEAD
k-tiles ahead, PER loads per wave and k-tile).  These models replay each
kernel's issue and wait sequence for every k-tile count up to 300 and check
that (1) every load of a k-tile has completed, in every wave, before any
wave reads that k-tile's stage, and (2) a stage is refilled only after every
read of its previous k-tile.  The sequences follow k_skinny_shared
(and k_skinny_split, whose K loop it shares), k_skinny and the steady state
of the 256 x 256 engine in kernels.hip.
"""
import pytest


class Wave:
    def __init__(self):
        self.issued = []          # tile of each load, in issue order
        self.done = 0             # loads completed (a prefix of `issued`)

    def issue(self, tile, per):
        self.issued += [tile] * per

    def wait(self, outstanding):
        self.done = max(self.done, len(self.issued) - outstanding)

    def landed(self, tile):
        return tile not in self.issued[self.done:] and tile in self.issued[:self.done]


def shared_ring(nk, ahead, per, waves=4):
    """k_skinny_shared: all waves load every stage together (PER loads each);
    top of k-tile t: wait until min(nk-1-t, AHEAD-1) k-tiles may be in flight,
    barrier, issue k-tile t+AHEAD into the stage of t-1, read stage t."""
    nst = ahead + 1
    ws = [Wave() for _ in range(waves)]
    stage_of = {}
    last_read = {}               # stage -> k-tile step of its last read
    for w in ws:
        for u in range(min(ahead, nk)):
            w.issue(u, per)
    for u in range(min(ahead, nk)):
        stage_of[u] = u % nst
    for t in range(nk):
        for w in ws:
            w.wait(min(nk - 1 - t, ahead - 1) * per)
        # barrier: every wave's loads of tile t have landed
        assert all(w.landed(t) for w in ws), (nk, ahead, t)
        if t + ahead < nk:
            s = (t + ahead) % nst
            # the stage's previous tile was read at an earlier step (before this barrier)
            assert last_read.get(s, -1) < t, (nk, ahead, t)
            for w in ws:
                w.issue(t + ahead, per)
            stage_of[t + ahead] = s
        last_read[stage_of[t]] = t


def private_rings(nk, ahead, per, waves):
    """k_skinny: wave v owns k-tiles v, v+W, ...; before its u-th tile it waits
    until min(nu-1-u, AHEAD-1) of its tiles may be in flight, reads, then
    refills the stage of its tile u-1 with its tile u+AHEAD (no barrier)."""
    nst = ahead + 1
    for v in range(waves):
        nu = (nk - v + waves - 1) // waves if nk > v else 0
        w = Wave()
        last_read = {}
        for u in range(min(ahead, nu)):
            w.issue(u, per)
        for u in range(nu):
            w.wait(min(nu - 1 - u, ahead - 1) * per)
            assert w.landed(u), (nk, ahead, v, u)
            last_read[u % nst] = u
            if u + ahead < nu:
                s = (u + ahead) % nst
                assert s != u % nst and last_read.get(s, -1) < u, (nk, ahead, v, u)
                w.issue(u + ahead, per)


def engine_steady(nk, ahead, per, waves=8):
    """256 x 256 engine: fragments of k-tile t+1 are read during k-tile t, so
    at the top of k-tile t (wait, barrier) tile t+1 must have landed while
    tiles t+2 .. t+AHEAD-1 may still be in flight; tile t+AHEAD then goes into
    the stage of tile t-1.  Prologue: tiles 0..AHEAD-1, then wait for tile 0."""
    nst = ahead + 1
    ws = [Wave() for _ in range(waves)]
    for w in ws:
        for u in range(min(ahead, nk)):
            w.issue(u, per)
        w.wait((min(nk, ahead) - 1) * per)
    assert nk == 0 or all(w.landed(0) for w in ws)
    read_step = {0: -1}           # tile -> step during which its fragments are read
    for t in range(nk):
        if t + 1 < nk:
            # steady state waits (AHEAD-2)*PER; the tail waits for what it issued
            issued_after = min(nk - 2 - t, ahead - 2)
            for w in ws:
                w.wait(issued_after * per)
            assert all(w.landed(t + 1) for w in ws), (nk, ahead, t)
            read_step[t + 1] = t
        if t + ahead < nk:
            victim = t + ahead - nst            # = t - 1, read during step t - 2
            assert read_step.get(victim, -1) < t, (nk, ahead, t)
            for w in ws:
                w.issue(t + ahead, per)


@pytest.mark.parametrize("ahead,per,waves", [(4, 4, 4), (4, 6, 2), (4, 6, 4), (4, 10, 2), (2, 4, 4), (9, 4, 4)])
def test_shared_ring_schedule(ahead, per, waves):
    # (4, 4, 4): 64 rows, 5-stage ring; (4, 6, 2): 32 rows; (4, 6, 4) and (4, 10, 2): the K-split
    # kernel's 128-column strips of 64 and 32 rows; 3 and 10 stages: the depths measured around it
    for nk in range(0, 301):
        shared_ring(nk, ahead, per, waves)


@pytest.mark.parametrize("ahead,per,waves", [(4, 12, 2), (4, 6, 4)])
def test_private_ring_schedule(ahead, per, waves):
    # (4, 12, 2): 32 rows, 64-k stages on two waves; (4, 6, 4): 32-k stages on four waves
    for nk in range(0, 301):
        private_rings(nk, ahead, per, waves)


@pytest.mark.parametrize("ahead,per", [(3, 4), (7, 2)])
def test_engine_schedule(ahead, per):
    # 256 x 256 tiles (3 ahead, 4 loads per wave and k-tile); 128 x 128 tiles for long K (7 ahead, 2)
    for nk in range(0, 301):
        engine_steady(nk, ahead, per)


def test_the_models_catch_a_wait_that_is_one_tile_short():
    # the same shared-ring sequence with the wait allowing one more tile in flight fails
    def short(nk, ahead, per):
        w = Wave()
        for u in range(min(ahead, nk)):
            w.issue(u, per)
        for t in range(nk):
            w.wait(min(nk - 1 - t, ahead - 1) * per + per)
            if not w.landed(t):
                return True
            if t + ahead < nk:
                w.issue(t + ahead, per)
        return False
    assert short(20, 4, 4)
