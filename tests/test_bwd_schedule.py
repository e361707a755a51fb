"""Host-side check of the backward kernel's phase schedule (no GPU).

m2rnn_bwd runs three wave roles in lock step, one barrier per phase:
* forward role: recomputes chunk cF = nch - 1 - k (S steps) in period k, reads
  its start state from the chunk-start buffer (phase 0) or the state ring,
  writes each step's state and tanh term into LDS rings of 2 S entries, and
  forms dv of the reverse role's previous step from the D buffer;
* reverse role: walks the previously recomputed chunk backwards one phase
  behind, reading the rings and the staging slots, publishing D;
* side role: dW from the previous phase's D and the A operands read in the
  same phase as the reverse role's state read; stages the next chunk's inputs
  and start state at the period's last phase.
This test replays, phase by phase, every buffer position and slot exactly as
the kernel computes them (same expressions as m2rnn_bwd.hip) and checks that

* every read finds the item it needs, written in an earlier phase;
* no location is read and written in the same phase (no barrier between);
* the forward role recomputes, and the reverse role reverses, every step of
  the padded sequence exactly once, in the required orders.
"""
import pytest


def slots(S):
    """Staging slots of the kernel for chunk length S."""
    return 3 if S >= 4 else (4 if S == 2 else 5)


def replay(S, nch, nslot=None):
    M = 2 * S
    NSLOT = nslot or slots(S)
    jlast = nch * S + S + 1
    nper = jlast // S + 1
    store = {}          # (buffer, position) -> (item, phase written)
    errors = []
    fwd_steps, rev_steps = [], []
    rstep = lambda j: nch * S + S - j            # noqa: E731
    ractive = lambda j: S + 1 <= j <= nch * S + S  # noqa: E731

    # prologue (side role): staging and start state of the last chunk
    store[("st", (nch - 1) % NSLOT)] = (("chunk", nch - 1), -1)
    store[("ck", (nch - 1) & 1)] = (("start", nch - 1), -1)
    for k in range(nper):
        cF = nch - 1 - k
        rec = cF >= 0
        slot = cF % NSLOT if rec else 0
        hbase = (cF & 1) * S if rec else 0
        slotA = (cF + 1) % NSLOT if cF + 1 >= 0 else 0
        slotB = (cF + 2) % NSLOT if cF + 2 >= 0 else 0
        slotC = (cF + 3) % NSLOT if cF + 3 >= 0 else 0
        par = (cF + 2) & 1
        for I in range(S):
            j = k * S + I
            jp = j & 1
            reads, writes = [], []
            # ---------------- forward role
            if rec:
                t = cF * S + I
                fwd_steps.append(t)
                reads.append(("st", slot, ("chunk", t // S)))
                if I == 0:
                    reads.append(("ck", cF & 1, ("start", cF)))
                else:
                    reads.append(("hr", hbase + I, ("S", t)))
                writes.append(("hr", (hbase + I + 1) & (M - 1), ("S", t + 1)))
                writes.append(("zr", hbase + I, ("Z", t)))
            if j == nch * S:
                writes.append(("hr", 0, ("S", 0)))
            if ractive(j - 1):   # dv of the reverse role's previous step
                tp = (cF + 2) * S - I + 1
                if tp != rstep(j - 1):
                    errors.append(f"j={j}: previous reverse step {tp} != {rstep(j - 1)}")
                tq = (1 - I + S) % S
                sl = slotC if S == 1 else (slotB if I <= 1 else slotA)
                if tq != tp % S:
                    errors.append(f"j={j}: staged index {tq} != {tp % S}")
                reads.append(("st", sl, ("chunk", tp // S)))
                reads.append(("xd", jp ^ 1, ("D", tp)))
            # ---------------- reverse role
            t = rstep(j)
            act = ractive(j)
            fin = j == jlast
            if act or fin:
                reads.append(("xd", jp ^ 1, ("D", t + 1) if j > S + 1 else ("D", "zero")))
            if act:
                rev_steps.append(t)
                tt = S - I if I >= 1 else 0
                sl = slotA if I >= 1 else slotB
                if tt != t % S:
                    errors.append(f"j={j}: staged step index {tt} != {t % S}")
                reads.append(("st", sl, ("chunk", t // S)))
                pos = (par * S - I) & (M - 1)
                if pos != t % M:
                    errors.append(f"j={j}: ring position {pos} != {t % M}")
                reads.append(("hr", pos, ("S", t)))
                writes.append(("xd", jp, ("D", t)))
                if t >= 1:
                    reads.append(("zr", (pos - 1) & (M - 1), ("Z", t - 1)))
            if j == S:
                reads.append(("zr", (nch * S - 1) & (M - 1), ("Z", nch * S - 1)))
            # ---------------- side role
            if ractive(j - 1):   # dW B operands: the previous step's D
                reads.append(("xd", jp ^ 1, ("D", rstep(j - 1))))
            if act:              # dW A operands: this phase's reverse step's state
                reads.append(("hr", (par * S - I) & (M - 1), ("S", t)))
            if I == S - 1 and cF >= 1:
                writes.append(("st", (cF - 1) % NSLOT, ("chunk", cF - 1)))
                writes.append(("ck", (cF - 1) & 1, ("start", cF - 1)))
            # ---------------- checks
            wpos = {(b, p) for b, p, _ in writes}
            for b, p, item in reads:
                if (b, p) in wpos:
                    errors.append(f"j={j}: {b}[{p}] read ({item}) and written in one phase")
                have = store.get((b, p))
                if item == ("D", "zero"):
                    if have is not None:
                        errors.append(f"j={j}: {b}[{p}] should still hold zeros")
                    continue
                if have is None or have[0] != item or have[1] >= j:
                    errors.append(f"j={j}: {b}[{p}] wants {item}, holds {have}")
            for b, p, item in writes:
                store[(b, p)] = (item, j)
    return errors, fwd_steps, rev_steps


@pytest.mark.parametrize("S", [1, 2, 4, 8])
@pytest.mark.parametrize("nch", [1, 2, 3, 4, 5, 9, 16])
def test_backward_phase_schedule(S, nch):
    errors, fwd, rev = replay(S, nch)
    assert not errors, errors[:5]
    Tp = nch * S
    # forward role: chunks last to first, each chunk's steps in time order
    assert fwd == [c * S + i for c in range(nch - 1, -1, -1) for i in range(S)]
    # reverse role: every step once, from the last to the first
    assert rev == list(range(Tp - 1, -1, -1))


@pytest.mark.parametrize("S", [1, 2])
def test_schedule_replay_detects_too_few_slots(S):
    """With one staging slot fewer than the kernel uses, the replay must fail
    (the side role's store would meet a read of the same slot)."""
    assert any(replay(S, n, nslot=slots(S) - 1)[0] for n in range(2, 9))


def test_schedule_replay_detects_short_rings():
    """The replay must catch rings one chunk long (too short) and pass 2 S."""
    for S in (2, 4, 8):
        assert replay_with_ring(S, 5, ring=S)
        assert not replay_with_ring(S, 5, ring=2 * S)


def replay_with_ring(S, nch, ring):
    """The state and tanh-term rings alone, with positions taken mod `ring`."""
    errors = []
    store = {}
    jlast = nch * S + S + 1
    for j in range(jlast + 1):
        k, I = divmod(j, S)
        cF = nch - 1 - k
        reads, writes = [], []
        if cF >= 0:
            t = cF * S + I
            if I > 0:
                reads.append(("hr", t % ring, ("S", t)))
            writes.append(("hr", (t + 1) % ring, ("S", t + 1)))
            writes.append(("zr", t % ring, ("Z", t)))
        t = nch * S + S - j
        if S + 1 <= j <= nch * S + S:
            reads.append(("hr", t % ring, ("S", t)))
            if t >= 1:
                reads.append(("zr", (t - 1) % ring, ("Z", t - 1)))
        if j == nch * S:
            writes.append(("hr", 0, ("S", 0)))
        wpos = {(b, p) for b, p, _ in writes}
        for b, p, item in reads:
            have = store.get((b, p))
            if (b, p) in wpos or have is None or have[0] != item:
                errors.append((j, b, p, item))
        for b, p, item in writes:
            store[(b, p)] = (item, j)
    return errors


# ---------------------------------------------------------------- interval sweep
#
# With checkpoints every C steps (C a multiple of S, C > S) the forward role
# sweeps each checkpoint interval forward in time once and keeps its states
# (and rc) in a per-unit ring of two interval slots; the LDS rings of a chunk
# are filled from there.  Each ring element is written and read by the same
# lane, so within a phase program order decides: the fill's load for its next
# step is issued at the end of the phase, after the sweep's store.  The replay below uses
# the sweep's definitions (sweep order, slot (t / C) & 1, position t mod C,
# C / S sweep-only periods first, one more when S = 1, where the fill's load of
# the next chunk shares its phase with that chunk's sweep) and checks that every
# fill load finds the item it needs, stored in an earlier phase and not yet
# overwritten, and that the sweep covers every step once.  The kernel walks the
# same order with counters instead of divisions; a test below checks that the
# counters reproduce the definitions.

def sweep_chunk(s, nch, CS, S):
    J = -(-nch // CS)
    n_last = nch - (J - 1) * CS
    if s < n_last:
        return ((J - 1) * CS + s) * S
    m, r = divmod(s - n_last, CS)
    return ((J - 2 - m) * CS + r) * S


def replay_sweep(S, C, nch, slots_=2):
    CS = C // S
    P0 = CS + (1 if S == 1 else 0)
    jlast = nch * S + S + 1
    nper = jlast // S + 1
    ring = {}
    errors, swept = [], []

    def rix(t):
        i = t // C
        return ((i % slots_) if slots_ != 2 else (i & 1), t - i * C)

    def fill_load(t, ph):
        have = ring.get(rix(t))
        if have is None or have[0] != ("S", t + 1) or have[1] >= ph:
            errors.append(f"phase {ph}: fill load of step {t} finds {have}")

    for kt in range(P0 + nper):
        for I in range(S):
            ph = kt * S + I
            k = kt - P0
            if kt == P0 and I == 0 and nch > 0:
                pass  # the first fill load happens after the prologue (below)
            # sweep: stores S_{x+1} (and rc_x)
            if kt < nch:
                x = sweep_chunk(kt, nch, CS, S) + I
                swept.append(x)
                ring[rix(x)] = (("S", x + 1), ph)
            # fill: uses step t (loaded in the phase before) and loads the next
            # step at the end of the phase, after the sweep's stores
            if k >= 0:
                cF = nch - 1 - k
                if cF >= 0:
                    if I + 1 < S or cF >= 1:
                        fill_load(cF * S + I + 1 if I + 1 < S else (cF - 1) * S, ph)
            if kt == P0 - 1 and I == S - 1 and nch > 0:
                fill_load((nch - 1) * S, ph + 0.5)   # after the prologue's last barrier
    return errors, swept


@pytest.mark.parametrize("S,C", [(2, 4), (2, 64), (4, 8), (4, 16), (1, 3), (2, 6), (4, 12)])
@pytest.mark.parametrize("nch", [1, 2, 3, 5, 7, 16, 33, 64])
def test_interval_sweep_schedule(S, C, nch):
    errors, swept = replay_sweep(S, C, nch)
    assert not errors, errors[:5]
    assert sorted(swept) == list(range(nch * S))


def sweep_cursor_walk(S, C, nch):
    """The kernel's sweep cursor (interval, chunk position, interval length,
    chunks left), advanced once per chunk with no division: per sweep step
    (x, ring slot, ring position, next step, interval that the next step starts)."""
    CS = C // S
    J = -(-nch // CS)
    n_last = nch - (J - 1) * CS
    s_i, s_pos, s_len, s_left = J - 1, 0, n_last * S, nch
    out = []
    while s_left > 0:
        for I in range(S):
            x = s_i * C + s_pos + I
            nx, nck = x + 1, -1
            last = I + 1 == S and s_pos + S == s_len
            if last:
                nck = s_i - 1
                nx = nck * C if nck >= 0 else -1
            out.append((x, s_i & 1, s_pos + I, nx, nck))
            if I + 1 == S:
                s_left -= 1
                if last:
                    s_i, s_pos, s_len = s_i - 1, 0, C
                else:
                    s_pos += S
    return out


def fill_cursor_walk(S, C, nch):
    """The kernel's fill cursor (interval and first step within it of the chunk
    filled in the period), moved back one chunk per period: per fill load
    (step, ring slot, ring position), in the kernel's order."""
    CS = C // S
    J = -(-nch // CS)
    n_last = nch - (J - 1) * CS
    f_i, f_pos = J - 1, (n_last - 1) * S
    out = [((nch - 1) * S, f_i & 1, f_pos)]
    for cF in range(nch - 1, -1, -1):
        for I in range(S):
            if I + 1 < S:
                out.append((cF * S + I + 1, f_i & 1, f_pos + I + 1))
            elif cF >= 1:
                out.append(((cF - 1) * S, f_i & 1, f_pos - S) if f_pos > 0
                           else ((cF - 1) * S, (f_i - 1) & 1, C - S))
        if f_pos > 0:
            f_pos -= S
        else:
            f_i, f_pos = f_i - 1, C - S
    return out


@pytest.mark.parametrize("S,C", [(2, 4), (2, 64), (4, 8), (4, 16), (2, 6), (4, 12), (2, 1024)])
@pytest.mark.parametrize("nch", [1, 2, 3, 5, 7, 16, 33, 64, 700])
def test_interval_sweep_cursors_match_the_division_form(S, C, nch):
    """The counters that replace every division in the kernel's sweep and fill
    give the same steps, ring slots and positions as the definitions (sweep
    order from sweep_chunk, slot (t / C) & 1, position t mod C)."""
    CS = C // S
    ref = []
    for kt in range(nch):
        for I in range(S):
            x = sweep_chunk(kt, nch, CS, S) + I
            nx = x + 1 if I + 1 < S else (sweep_chunk(kt + 1, nch, CS, S) if kt + 1 < nch else -1)
            nck = nx // C if nx >= 0 and nx % C == 0 else -1
            ref.append((x, (x // C) & 1, x % C, nx, nck))
    assert sweep_cursor_walk(S, C, nch) == ref
    fill_ref = [((nch - 1) * S, ((nch - 1) * S // C) & 1, (nch - 1) * S % C)]
    for cF in range(nch - 1, -1, -1):
        for I in range(S):
            if I + 1 < S or cF >= 1:
                t = cF * S + I + 1 if I + 1 < S else (cF - 1) * S
                fill_ref.append((t, (t // C) & 1, t % C))
    assert fill_cursor_walk(S, C, nch) == fill_ref


def test_interval_sweep_replay_detects_one_slot():
    """With a single interval slot the sweep overwrites states the fill still needs."""
    assert any(replay_sweep(S, C, n, slots_=1)[0]
               for S, C in [(2, 4), (4, 8)] for n in range(3, 12))
