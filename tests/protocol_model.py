"""Host-side model of the single-pass look-back scan's inter-workgroup protocol.

The decoupled look-back ("Selective-scan CUDA kernels", the paragraph on the
synchronisation between thread blocks) is correct only if every tile folds
exactly the tiles before it, in order, from words of the current launch; a
missing wait or a stale word gives a kernel that is right almost every time.
This model replays the protocol of the gfx950 kernel step by step, with
every global memory access a scheduling point and a seeded random scheduler
choosing which workgroup runs next, so that the interleavings a GPU could
take are explored on the CPU:

* claims: one 64-bit word, ((epoch - 1) << 32) | claims made; a workgroup
  claims tiles one at a time until its first failed claim, and the launch's
  last claim (number ntiles + grid - 1) stores the next launch's epoch;
* status words: two per aggregate (multiplier, offset), each tagged with the
  launch's epoch and written separately (so a reader may see one new and one
  old), at three levels (tiles, superblocks of `fan` tiles, blocks of `fan`
  superblocks);
* look-back windows as the kernel forms them: the level-2 words of earlier
  blocks, the level-1 words of the earlier superblocks of the block, and the
  level-0 words of the `recent` most recent superblocks, the last one cut at
  the tile;
* the last tile of a superblock publishes the superblock's aggregate once its
  own superblock's window is complete, and the last tile of a block the
  block's aggregate once its level-1 and recent windows are complete, before
  the level-2 words arrive;
* a workgroup's pipeline as the kernel runs it: a control part (the first
  three claims, then one look-back per iteration) and a data part (one claim
  and one level-0 publication per iteration) meeting at barriers;
* epochs cycling through 1 .. cycle, the launch holding the last epoch
  counting its waves out and the last one clearing every status word.

Payloads are not numbers but the interval of tiles an aggregate covers and
the launch it belongs to; composing two aggregates asserts that they belong
to the current launch and are adjacent, so a word read too early, read from
an earlier launch, or folded in the wrong order fails at once, and every
tile's incoming prefix must cover exactly the tiles before it.

Test infrastructure: the kernels never use this module.
"""
import random
from dataclasses import dataclass, field


class ProtocolError(AssertionError):
    """The protocol produced a wrong fold, a stale read or a hang."""


@dataclass(frozen=True)
class Agg:
    launch: int
    lo: int  # first tile covered
    hi: int  # last tile covered


def compose(x, y, launch):
    """x then y; None is the identity."""
    if x is None:
        return y
    if y is None:
        return x
    if x.launch != launch or y.launch != launch:
        raise ProtocolError(f"aggregate of launch {x.launch}/{y.launch} used in launch {launch}")
    if x.hi + 1 != y.lo:
        raise ProtocolError(f"fold of [{x.lo},{x.hi}] and [{y.lo},{y.hi}] is not in order")
    return Agg(launch, x.lo, y.hi)


@dataclass
class Word:
    tag: int = 0  # epoch of the launch that wrote it (0: cleared, never current)
    payload: object = None


@dataclass
class Faults:
    """Protocol mistakes that the tests plant in the model (all off: the
    kernel's protocol)."""
    check_a_only: bool = False          # accept a pair when only the multiplier word is current
    no_cycle_clear: bool = False        # the cycle's last launch does not clear the words
    handoff_one_early: bool = False     # the next epoch is stored one claim too early
    publish_without_wait: bool = False  # superblock aggregate published before its window is complete
    lvl1_window_one_short: bool = False  # the level-1 window leaves out its last superblock
    block_needs_only_own: bool = False   # block aggregate published once the own window is complete


@dataclass
class Status:
    max_tiles: int
    fan: int
    cycle: int
    claims_hi: int = 0
    claims_count: int = 0
    done: int = 0
    lvl: list = field(default_factory=list)

    def __post_init__(self):
        nsb = -(-self.max_tiles // self.fan)
        nblk = -(-nsb // self.fan)
        self.lvl = [[(Word(), Word()) for _ in range(n)] for n in (self.max_tiles, nsb, nblk)]


class Launch:
    """One kernel launch on a workspace: `grid` workgroups over `ntiles`
    tiles, at most `resident` of them running at a time (workgroups start in
    index order as running ones finish)."""

    def __init__(self, st, launch_id, ntiles, grid, resident, recent, rng, faults):
        assert st.fan >= recent >= 1 and ntiles <= st.max_tiles
        self.st, self.id, self.ntiles, self.grid = st, launch_id, ntiles, grid
        self.resident, self.recent, self.rng, self.f = resident, recent, rng, faults
        self.h_in = {}       # tile -> the prefix its look-back formed
        self.published = {}  # (level, index) -> aggregate, as published
        self.events = 0      # claims and stores so far (progress)

    # -- global memory: every access is a scheduling point -------------------
    def claim(self):
        yield
        st = self.st
        count, hi = st.claims_count, st.claims_hi
        st.claims_count += 1
        self.events += 1
        last = self.ntiles + self.grid - 1 - (1 if self.f.handoff_one_early else 0)
        if count == last:
            yield
            st.claims_hi = 0 if hi + 1 >= st.cycle else hi + 1
            st.claims_count = 0
        return (count if count < self.ntiles else self.ntiles), hi + 1

    def successor(self, t):
        if t >= self.ntiles:
            return self.ntiles
        tile, _ = yield from self.claim()
        return tile

    def store_pair(self, level, index, agg, epoch):
        pair = self.st.lvl[level][index]
        order = [0, 1] if self.rng.random() < 0.5 else [1, 0]  # relaxed stores: either order
        for k in order:
            yield
            pair[k].tag, pair[k].payload = epoch, agg
        self.published[(level, index)] = agg
        self.events += 1

    def load_pair(self, level, index, epoch):
        """Reads both words (in either order); returns the aggregate if the
        pair is current, else a marker that it is not."""
        pair = self.st.lvl[level][index]
        order = [0, 1] if self.rng.random() < 0.5 else [1, 0]
        got = [None, None]
        for k in order:
            yield
            got[k] = (pair[k].tag, pair[k].payload)
        ready_a = got[0][0] == epoch
        ready_b = got[1][0] == epoch
        if ready_a and (ready_b or self.f.check_a_only):
            if got[0][1] != got[1][1] and not self.f.check_a_only:
                raise ProtocolError("current pair with two different payloads")
            return True, got[1][1]
        return False, None

    # -- the look-back --------------------------------------------------------
    def windows(self, tile):
        """The kernel's windows for a tile: a list of (level, first index,
        count, role) in sequence order."""
        fan = self.st.fan
        sb = tile // fan
        n0 = tile - sb * fan
        sb0 = sb - (self.recent - 1) if sb >= self.recent - 1 else 0
        nw = sb - sb0 + 1
        blk1 = sb0 // fan
        n1 = sb0 - blk1 * fan
        if self.f.lvl1_window_one_short and n1 > 0:
            n1 -= 1
        n2 = blk1
        out = [(2, 0, n2, "lvl2"), (1, blk1 * fan, n1, "lvl1")]
        for q in range(nw):
            cnt = fan if q < nw - 1 else n0
            out.append((0, (sb0 + q) * fan, cnt, "own" if q == nw - 1 else "recent"))
        return out

    def wait_words(self, tile, epoch, roles, have):
        """Reads the words of the windows whose role is in `roles` until every
        one is current (each round rereads the words not yet complete)."""
        wins = [w for w in self.windows(tile) if w[3] in roles]
        pending = [(lv, first + i) for lv, first, cnt, _ in wins for i in range(cnt)
                   if (lv, first + i) not in have]
        while pending:
            still = []
            for key in pending:
                ok, agg = yield from self.load_pair(key[0], key[1], epoch)
                if ok:
                    have[key] = agg
                else:
                    still.append(key)
            pending = still
            if pending:
                yield  # s_sleep

    def fold(self, tile, have, roles):
        """Composes the windows' words in sequence order, as read (a word
        never waited for is taken as it stands, here the identity: the fold
        then misses its tiles, which compose or verify reports)."""
        total = None
        for lv, first, cnt, role in self.windows(tile):
            if role in roles:
                for i in range(cnt):
                    total = compose(total, have.get((lv, first + i)), self.id)
        return total

    def lookback(self, tile, epoch):
        fan = self.st.fan
        have = {}
        sb = tile // fan
        own = Agg(self.id, tile, tile)
        if tile % fan == fan - 1:  # closes a superblock: publish early
            closes_block = sb % fan == fan - 1 and not self.f.block_needs_only_own
            need = {"own", "recent", "lvl1"} if closes_block else {"own"}
            if not self.f.publish_without_wait:
                yield from self.wait_words(tile, epoch, need, have)
            sbm = compose(self.fold(tile, have, {"own"}), own, self.id)
            yield from self.store_pair(1, sb, sbm, epoch)
            if sb % fan == fan - 1:
                pb = self.fold(tile, have, {"lvl1", "recent"})
                yield from self.store_pair(2, sb // fan, compose(pb, sbm, self.id), epoch)
        yield from self.wait_words(tile, epoch, {"lvl2", "lvl1", "recent", "own"}, have)
        self.h_in[tile] = self.fold(tile, have, {"lvl2", "lvl1", "recent", "own"})

    # -- one workgroup --------------------------------------------------------
    def workgroup(self, wg):
        ids = [None] * 4
        bar = {"count": 0}

        def barrier():
            bar["count"] += 1
            target = -(-bar["count"] // 2) * 2
            while bar["count"] < target:
                yield

        def check_out(epoch):
            if epoch < self.st.cycle or self.f.no_cycle_clear:
                return
            yield
            self.st.done += 1
            if self.st.done == 2 * self.grid:  # two waves per workgroup in this model
                for level in self.st.lvl:
                    for pair in level:
                        for w in pair:
                            yield
                            w.tag, w.payload = 0, None
                self.st.done = 0

        state = {}

        def control():
            t0, epoch = yield from self.claim()
            t0 = min(t0, self.ntiles)
            state["epoch"] = epoch
            ids[0] = t0
            yield from barrier()  # A0
            t1 = yield from self.successor(t0)
            ids[1] = t1
            yield from barrier()  # A1
            t2 = yield from self.successor(t1)
            ids[2] = t2
            yield from barrier()  # A
            yield from barrier()  # B
            tp, j = self.ntiles, 0
            while True:
                tn = ids[j & 3]
                if tp < self.ntiles:
                    yield from self.lookback(tp, epoch)
                tp = tn
                yield from barrier()  # C_j
                j += 1
                if tp >= self.ntiles:
                    break
            yield from check_out(epoch)

        def data():
            yield from barrier()  # A0
            epoch = state["epoch"]
            t0 = ids[0]
            yield from barrier()  # A1
            t1 = ids[1]
            yield from barrier()  # A
            t2 = ids[2]
            if t0 < self.ntiles:
                yield from self.store_pair(0, t0, Agg(self.id, t0, t0), epoch)
            yield from barrier()  # B
            tp, j = self.ntiles, 0
            while j == 0 or tp < self.ntiles:
                claimed = self.ntiles
                if t2 < self.ntiles:
                    claimed = yield from self.successor(t2)
                if t1 < self.ntiles:
                    yield from self.store_pair(0, t1, Agg(self.id, t1, t1), epoch)
                ids[(j + 3) & 3] = claimed
                yield from barrier()  # C_j
                tp, t0, t1, t2 = t0, t1, t2, ids[(j + 3) & 3]
                j += 1
            yield from check_out(epoch)

        return [control(), data()]

    def run(self, idle_steps):
        """Runs the launch to its end. Each workgroup gets a speed drawn from a
        heavy-tailed set when it starts, so that stragglers hold their tiles
        while others run far ahead (the skews that expose a missing wait)."""
        waiting = list(range(self.grid))
        running = []  # (wg, [coroutines])
        speed = []
        steps = last_event = seen = 0
        while waiting or running:
            while waiting and len(running) < self.resident:
                wg = waiting.pop(0)
                running.append((wg, self.workgroup(wg)))
                speed.append(self.rng.choice((1.0, 1.0, 0.25, 0.02)))
            k = self.rng.choices(range(len(running)), weights=speed)[0]
            wg, cos = running[k]
            c = self.rng.randrange(len(cos))
            try:
                next(cos[c])
            except StopIteration:
                cos.pop(c)
                if not cos:
                    running.pop(k)
                    speed.pop(k)
            steps += 1
            if self.events != seen:
                seen, last_event = self.events, steps
            elif steps - last_event > idle_steps:
                raise ProtocolError(f"no claim or store in {idle_steps} steps (a hang)")
        return steps

    def verify(self):
        for t in range(self.ntiles):
            want = Agg(self.id, 0, t - 1) if t > 0 else None
            if self.h_in.get(t, "missing") != want:
                raise ProtocolError(f"tile {t}: prefix {self.h_in.get(t, 'missing')}, want {want}")
        fan = self.st.fan
        for (level, i), agg in self.published.items():
            span = fan ** level
            want = Agg(self.id, i * span, min((i + 1) * span, self.ntiles) - 1)
            if level > 0 and agg != want:
                raise ProtocolError(f"level {level} aggregate {i}: {agg}, want {want}")
        if self.st.claims_count != 0:
            raise ProtocolError(f"{self.st.claims_count} claims after the epoch hand-over")


def run_launches(launches, fan=4, recent=3, cycle=3, seed=0, faults=None, max_tiles=None):
    """Runs launches = [(ntiles, grid, resident), ...] one after another on
    one workspace, each under a random schedule, and checks every one."""
    faults = faults or Faults()
    rng = random.Random(seed)
    st = Status(max_tiles or max(n for n, _, _ in launches), fan, cycle)
    for lid, (ntiles, grid, resident) in enumerate(launches, start=1):
        la = Launch(st, lid, ntiles, grid, resident, recent, rng, faults)
        # Every wait ends within a few rounds of reads once its words are
        # written; a slow workgroup (speed 0.02) takes about 50 picks a step.
        la.run(idle_steps=200000)
        la.verify()
    return st
