"""CPU model of the column kernels' LDS progress-counter protocol.

The column kernels (csrc/cols.hip: 4 producer and 12 consumer waves that also exchange
partial block-scale maxima; csrc/fp8q_cols.hip: 8 producer and 8 consumer waves, the
producer waves in two blocks of four that exchange partial column maxima within the
block, and one `produced` counter per producer wave) split each workgroup into producer
and consumer waves that share a
four-slot LDS ring and synchronise only through monotonic counters: `published`
(partial block-scale maxima), `produced` (strips converted) and `drained[slot]`
(strips written out).  This model replays the kernel's waits, with the
same targets, as agents under a deterministic random scheduler, and checks every
shared access:

  * a consumer reads ring slot t % 4 only once all producers wrote strip t, and the
    carry bytes of strip t - 1 (slot (t - 1) % 4) are still strip t - 1;
  * a producer overwrites ring slot t % 4 only after every consumer finished strip
    t - 4 (its own reader) and strip t - 3 (which reads strip t - 4 as carry);
  * a producer reads the partial maxima of strip t only once all producer waves
    published them, and no wave overwrites them while another still needs them;
  * the slot's strip info (written by producer wave 0) is the strip a consumer expects;
  * with the block exchange (fp8q_cols.hip, where a wave holds a 128-column block over
    32 rows), a producer reads the partial column maxima of strip t from the other three
    waves of its block only once they published them, before converting the strip's
    columns, and no wave overwrites its slot while a block member still needs the
    previous strip's maxima.

Every wait is bounded in the kernels: a wave that polls a counter `polls` times in vain
sets the device's status word and leaves.  With a poll budget the model checks that
every wave then leaves (no deadlock), that the accesses made on the way out are still
in order, and that a run whose column output is incomplete always has a wave that gave
up, so an incomplete output is never reported as success.

It checks the protocol design (the wait targets), not the compiled kernel; the GPU
parity tests check the kernel.
"""
import random

import pytest

SLOTS = 4
# (producer waves, consumer waves, partial-maximum slots or None, block exchange) of the
# kernels: cols.hip, and fp8q_cols.hip (both instances)
CONFIGS = [(4, 12, 4, False), (8, 8, None, True)]


class Violation(AssertionError):
    pass


def _run(n, seed, carry=True, drain_lag=3, PW=4, CW=12, PMAX=4, per_wave=None, blocks=False, blocks_wait=True,
         polls=None):
    """PMAX None: no partial maxima.  per_wave (default: PMAX is None): one produced
    counter per producer wave, the consumers wait for the smallest.  blocks: the
    backward quantizer's exchange (per-wave partial column maxima exchanged within blocks
    of four waves before the strip's columns are converted); blocks_wait False drops the
    wait for the block (the model must catch that).  polls:
    the bound of every wait (None: unbounded).  Returns (column output complete, some
    wave gave up)."""
    if per_wave is None:
        per_wave = PMAX is None
    rnd = random.Random(seed)
    cnt = {"published": 0, "produced": 0}
    for w in range(PW):
        cnt[f"produced{w}"] = 0
    for k in range(SLOTS):
        cnt[f"drained{k}"] = 0
    ring = [None] * SLOTS          # slot -> [strip, set of producer waves written]
    pmax = [None] * (PMAX or 1)    # slot -> [strip, set of waves published]
    info = [None] * SLOTS          # slot -> strip
    done_prod = [[False] * n for _ in range(PW)]       # producer w finished produce(t)
    done_cons = [[False] * n for _ in range(CW)]       # consumer v finished strip t
    cmax = [[None] * PW for _ in range(SLOTS)]         # slot -> wave -> strip published there
    read_done = [[False] * n for _ in range(PW)]       # producer w read its block's maxima of strip t
    for w in range(PW):
        cnt[f"colpub{w}"] = 0

    def need(cond, msg):
        if not cond:
            raise Violation(msg)

    gave_up = []

    def wait(agent, cond):
        # the kernel's bounded wait: cond is polled at most `polls` times; a wave that
        # runs out sets the status word (recorded here) and leaves the kernel
        k = 0
        while polls is None or k < polls:
            if cond():
                return True
            k += 1
            yield "wait"
        gave_up.append(agent)
        return False

    def publish(w, t):
        s = t % PMAX
        e = pmax[s]
        if e is not None and e[0] != t:
            # the slot held strip t - PMAX: every producer must have read it
            need(e[0] == t - PMAX, f"P{w} publishes {t} over pmax of strip {e[0]}")
            need(all(done_prod[x][t - PMAX] for x in range(PW)),
                 f"P{w} publishes {t} while strip {t - PMAX}'s maxima are still needed")
            e = None
        pmax[s] = [t, (e[1] if e else set()) | {w}]

    def producer(w):
        if PMAX:
            publish(w, 0)
            cnt["published"] += 1
        yield None
        for t in range(n):
            # the kernel waits until strip t - 3 is drained (drain_lag = 3)
            if t >= drain_lag:
                k = (t - drain_lag) % SLOTS
                if not (yield from wait(f"P{w}", lambda: cnt[f"drained{k}"] >= CW * ((t - drain_lag) // SLOTS + 1))):
                    return
            if PMAX:
                if not (yield from wait(f"P{w}", lambda: cnt["published"] >= PW * (t + 1))):
                    return
                e = pmax[t % PMAX]
                need(e is not None and e[0] == t and len(e[1]) == PW, f"P{w} reads pmax {e} for strip {t}")
            if blocks:
                # publish this wave's partial column maxima of strip t into slot t % 4, then
                # wait for the other three waves of its block and read theirs: the block's
                # maxima are needed before the strip's columns are converted into the ring
                old = cmax[t % SLOTS][w]
                blk = range(w & ~3, (w & ~3) + 4)
                if old is not None:
                    need(old == t - SLOTS, f"P{w} maxima of {t} over strip {old}")
                    need(all(read_done[x][old] for x in blk),
                         f"P{w} overwrites the maxima of strip {old} while its block still needs them")
                cmax[t % SLOTS][w] = t
                yield None
                cnt[f"colpub{w}"] += 1
                yield None
                if blocks_wait:
                    if not (yield from wait(f"P{w}", lambda: min(cnt[f"colpub{x}"] for x in blk) >= t + 1)):
                        return
                for x in blk:
                    need(cmax[t % SLOTS][x] == t, f"P{w} reads maxima {cmax[t % SLOTS][x]} of P{x} for strip {t}")
                    yield None
                read_done[w][t] = True
            s = t % SLOTS
            if w == 0:
                info[s] = t
            e = ring[s]
            if e is not None and e[0] != t:
                need(e[0] == t - SLOTS, f"P{w} writes strip {t} over strip {e[0]}")
                need(all(done_cons[v][t - SLOTS] for v in range(CW)),
                     f"P{w} overwrites strip {t - SLOTS} before it is written out")
                if carry and t - SLOTS + 1 < n:
                    need(all(done_cons[v][t - SLOTS + 1] for v in range(CW)),
                         f"P{w} overwrites strip {t - SLOTS} before strip {t - SLOTS + 1} took its carry")
                e = None
            ring[s] = [t, (e[1] if e else set()) | {w}]
            done_prod[w][t] = True
            yield None
            cnt["produced"] += 1
            cnt[f"produced{w}"] += 1
            if t + 1 >= n:
                return
            if PMAX:
                yield None
                publish(w, t + 1)
                yield None
                cnt["published"] += 1

    def consumer(v):
        for t in range(n):
            if per_wave:
                ok = yield from wait(f"C{v}", lambda: min(cnt[f"produced{w}"] for w in range(PW)) >= t + 1)
            else:
                ok = yield from wait(f"C{v}", lambda: cnt["produced"] >= PW * (t + 1))
            if not ok:
                return
            s = t % SLOTS
            need(info[s] == t, f"C{v} expects strip {t}, slot info says {info[s]}")
            e = ring[s]
            need(e is not None and e[0] == t and len(e[1]) == PW, f"C{v} reads {e} for strip {t}")
            if carry and t >= 1:
                e = ring[(t - 1) % SLOTS]
                need(e is not None and e[0] == t - 1, f"C{v} carry of strip {t - 1} is {e}")
            yield None
            done_cons[v][t] = True
            cnt[f"drained{s}"] += 1

    agents = [producer(w) for w in range(PW)] + [consumer(v) for v in range(CW)]
    live = list(range(len(agents)))
    # a slow agent makes the interesting orders (one wave far behind the rest) likely
    slow = rnd.randrange(len(agents))
    steps = 0
    stalled = 0
    while live:
        i = rnd.choice(live)
        if i == slow and rnd.random() < 0.8:
            continue
        try:
            r = next(agents[i])
        except StopIteration:
            live.remove(i)
            stalled = 0
            continue
        steps += 1
        stalled = stalled + 1 if r == "wait" else 0
        if stalled > 100000:
            raise Violation(f"deadlock at n={n}: counters {cnt}")
    complete = all(all(done_cons[v]) for v in range(CW))
    if not gave_up:
        for v in range(CW):
            need(all(done_cons[v]), f"C{v} did not write every strip")
    return complete, bool(gave_up)


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 9, 13])
def test_protocol_random_schedules(n, cfg):
    pw, cw, pm, bl = cfg
    for seed in range(60 if cfg == CONFIGS[0] else 30):
        _run(n, seed, PW=pw, CW=cw, PMAX=pm, blocks=bl)


@pytest.mark.parametrize("n", [1, 2, 4, 5, 9, 13])
def test_protocol_both_layouts_random_schedules(n):
    """fp8q_cols.hip: 8 producer waves in two blocks of four (more schedules)."""
    for seed in range(30):
        _run(n, seed, PW=8, CW=8, PMAX=None, blocks=True)


def test_model_catches_a_missing_row_block_wait():
    """Without the wait for the block's other waves, some schedule reads another wave's
    partial column maxima before that wave published the strip."""
    caught = 0
    for seed in range(40):
        try:
            _run(6, seed, PW=8, CW=8, PMAX=None, blocks=True, blocks_wait=False)
        except Violation:
            caught += 1
    assert caught > 0


def test_model_catches_a_weaker_wait():
    """The model is not vacuous: a producer that only waits for strip t - 4 to be
    drained (ignoring that strip t - 3 still reads strip t - 4 as carry) is caught on
    some schedule, and so is one that does not wait for the drain at all."""
    for lag in (4, 99):
        caught = False
        for seed in range(300):
            try:
                _run(9, seed, drain_lag=lag)
            except Violation:
                caught = True
                break
        assert caught, f"drain lag {lag} not caught"


def test_model_catches_a_summed_produced_counter_without_lockstep():
    """Without a lockstep exchange over all producer waves (fp8q_cols.hip's two blocks
    exchange only within themselves; here none at all), producer waves drift apart, so a
    single summed `produced` counter no longer shows that every wave wrote strip t."""
    caught = False
    for seed in range(300):
        try:
            _run(9, seed, PW=8, CW=8, PMAX=None, per_wave=False)
        except Violation:
            caught = True
            break
    assert caught


def test_model_catches_a_summed_produced_counter_across_two_blocks():
    """fp8q_cols.hip's two blocks of four producer waves exchange maxima only within the
    block, so the blocks drift apart and the consumers need one counter per wave."""
    caught = False
    for seed in range(300):
        try:
            _run(9, seed, PW=8, CW=8, PMAX=None, per_wave=False, blocks=True)
        except Violation:
            caught = True
            break
    assert caught


def test_model_catches_a_single_partial_maximum_slot():
    """The partial-maximum check is not vacuous: with one slot, a wave publishing strip
    t + 1 overwrites strip t's maxima while another wave still converts strip t."""
    caught = False
    for seed in range(300):
        try:
            _run(9, seed, PW=4, CW=12, PMAX=1)
        except Violation:
            caught = True
            break
    assert caught


@pytest.mark.parametrize("cfg", CONFIGS + ["both"])
def test_give_up_leaves_every_wave_and_is_reported(cfg):
    """With a tiny poll budget (the host's wait-limit hook), waves give up: every wave
    still leaves (the scheduler would flag a deadlock), the accesses made before they
    leave stay in order (the model's checks hold), and every run whose column output
    is incomplete has a wave that gave up, so the status word reports it."""
    kw = dict(PW=8, CW=8, PMAX=None, blocks=True) if cfg == "both" else dict(PW=cfg[0], CW=cfg[1], PMAX=cfg[2],
                                                                               blocks=cfg[3])
    outcomes = set()
    for polls in (1, 2, 3, 8, 40, 400):
        for seed in range(20):
            complete, gave_up = _run(9, seed, polls=polls, **kw)
            assert complete or gave_up, f"incomplete output with no give-up (polls {polls}, seed {seed})"
            outcomes.add((complete, gave_up))
    # both sides are exercised: runs that gave up and runs that finished
    assert (False, True) in outcomes and (True, False) in outcomes, outcomes


def test_give_up_budget_does_not_change_a_run_that_finishes():
    """A budget large enough for the schedule changes nothing: the run completes."""
    for seed in range(20):
        assert _run(6, seed, polls=10 ** 6) == (True, False)
