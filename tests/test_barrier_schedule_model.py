"""Schedule model of the plain-barrier baseline's per-wave-index counter
(CPU only).

The simulator keeps the baseline's top and bottom barriers among the waves
of one wave index, one in every rank, with one counter: per op it takes the
N producers' arrivals, then the C consumers' completions.  A producer of op
i (i >= 1) waits until the counter reaches i*(N + C); a consumer of op i
waits until it reaches i*(N + C) + N.  In system mode every rank's wave
produces and then consumes each op; in share mode (C = 1) ranks 1..N-1 only
produce and rank 0 does both.

This model runs those wait rules over random interleavings of the waves'
steps and checks the two properties the barriers exist for, on one buffer:
a consumer reads a slot only after its producer wrote the same op into it
(top barrier), and no producer overwrites a slot before every consumer has
read the previous op from it (bottom barrier).  It also checks that every
schedule ends with all ops done (no wait can block forever).
"""
import random

import pytest


def _run(nranks, share, nops, rng):
    consumers = [0] if share else list(range(nranks))
    K = nranks + len(consumers)
    counter = 0
    # slot[c][g]: the op producer g last wrote into consumer c's slot g
    slot = {c: {g: None for g in range(nranks) if g != c} for c in consumers}
    # reads[c][g]: the last op consumer c read from slot g
    reads = {c: {g: -1 for g in slot[c]} for c in consumers}

    def program(g):
        for op in range(nops):
            if op >= 1:
                yield ("wait", op * K)
            for c in consumers:
                if c == g:
                    continue
                # bottom barrier: every consumer read op - 1 from this slot
                assert reads[c][g] == op - 1, (g, c, op, reads[c][g])
                slot[c][g] = op
                yield ("step", None)
            yield ("arrive", None)
            if g in consumers:
                yield ("wait", op * K + nranks)
                for p in slot[g]:
                    # top barrier: the producer's op is in place
                    assert slot[g][p] == op, (g, p, op, slot[g][p])
                    reads[g][p] = op
                    yield ("step", None)
                yield ("arrive", None)

    waves = {g: program(g) for g in range(nranks)}
    pending = {g: next(waves[g]) for g in range(nranks)}
    while pending:
        runnable = [g for g, (kind, arg) in pending.items()
                    if kind != "wait" or counter >= arg]
        assert runnable, f"deadlock at counter {counter}: {pending}"
        g = rng.choice(runnable)
        kind, _ = pending[g]
        if kind == "arrive":
            counter += 1
        try:
            pending[g] = next(waves[g])
        except StopIteration:
            del pending[g]
    assert counter == nops * K
    for c in consumers:
        assert all(v == nops - 1 for v in reads[c].values())


@pytest.mark.parametrize("share", [False, True])
@pytest.mark.parametrize("nranks", [1, 2, 3, 8, 16])
def test_counter_thresholds_keep_both_barriers(nranks, share):
    rng = random.Random(1000 * nranks + share)
    for _ in range(200):
        _run(nranks, share, nops=5, rng=rng)


def test_model_catches_a_missing_bottom_barrier():
    """The model is not vacuous: with the producers' wait one arrival short
    of the consumers' completions, some schedule overwrites a slot that a
    consumer has not read yet."""
    rng = random.Random(7)
    nranks, nops = 4, 4
    K = 2 * nranks
    counter = 0
    slot = {c: {g: None for g in range(nranks) if g != c} for c in range(nranks)}
    reads = {c: {g: -1 for g in slot[c]} for c in range(nranks)}
    failures = 0

    def program(g):
        for op in range(nops):
            if op >= 1:
                yield ("wait", op * K - 1)          # one completion short
            for c in range(nranks):
                if c != g:
                    if reads[c][g] != op - 1:
                        raise AssertionError("overwrite before read")
                    slot[c][g] = op
                    yield ("step", None)
            yield ("arrive", None)
            yield ("wait", op * K + nranks)
            for p in slot[g]:
                reads[g][p] = op
                yield ("step", None)
            yield ("arrive", None)

    for _ in range(300):
        counter = 0
        for c in slot:
            for g in slot[c]:
                slot[c][g] = None
                reads[c][g] = -1
        waves = {g: program(g) for g in range(nranks)}
        pending = {g: next(waves[g]) for g in range(nranks)}
        try:
            while pending:
                runnable = [g for g, (kind, arg) in pending.items()
                            if kind != "wait" or counter >= arg]
                g = rng.choice(runnable)
                if pending[g][0] == "arrive":
                    counter += 1
                try:
                    pending[g] = next(waves[g])
                except StopIteration:
                    del pending[g]
        except AssertionError:
            failures += 1
    assert failures > 0
