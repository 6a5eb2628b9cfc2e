"""Model check of the single-pass encode's in-workgroup handshake (host
logic, no GPU).

The kernel's key waves (the "workers" below) and its coordinator wave
exchange, through LDS, each round's key maxima (wg_max), a count of key
waves done with the round (done) and the number of rounds whose layer
maxima are ready (ready). The key waves park round r, then quantise round
r-lag once ready > r-lag (the kernel's lag is 3); the coordinator waits
until every key wave is done with round r, takes and clears
its entries, publishes, and marks round r-1 ready. This model runs those
steps under random interleavings and checks that no count or maximum is
lost and every round is quantised with its own maxima. With the entries
indexed by round % (lag + 1) (as in the kernel: % 4) every schedule
passes; indexed by round % lag, a worker can reach round r+lag before the
coordinator has cleared round r, and the count it adds is lost (the
kernel's bounded wait would then give up and mark the pool invalid)."""

import random

import pytest


def run(buffers, rounds, seed, workers=8, lag=2):
    rng = random.Random(seed)
    done = [0] * buffers
    wg_max = [[] for _ in range(buffers)]
    layer_max = [None] * buffers
    ready = 0

    def worker():
        for r in range(rounds + lag):
            if r < rounds:
                yield ("encode", r)
            if r >= lag:
                yield ("quantise", r - lag)

    def coordinator():
        for k in range(rounds + 1):
            if k < rounds:
                yield ("take", k)
            if k >= 1:
                yield ("ready", k - 1)

    ws = [worker() for _ in range(workers)]
    wstep = [next(g) for g in ws]
    cg = coordinator()
    cstep = next(cg)
    errors = []
    while True:
        runnable = [("w", i) for i, st in enumerate(wstep)
                    if st is not None and not (st[0] == "quantise" and ready <= st[1])]
        if cstep is not None and not (cstep[0] == "take" and done[cstep[1] % buffers] < workers):
            runnable.append(("c", 0))
        if not runnable:
            if cstep is None and all(st is None for st in wstep):
                return errors
            return errors + ["stuck"]
        who, i = rng.choice(runnable)
        if who == "w":
            kind, r = wstep[i]
            if kind == "encode":
                wg_max[r % buffers].append(r)
                done[r % buffers] += 1
            elif layer_max[r % buffers] != r:
                errors.append(f"round {r} quantised with the maxima of round {layer_max[r % buffers]}")
            wstep[i] = next(ws[i], None)
        else:
            kind, k = cstep
            if kind == "take":
                if sorted(wg_max[k % buffers]) != [k] * workers:
                    errors.append(f"round {k}: maxima from rounds {sorted(wg_max[k % buffers])}")
                wg_max[k % buffers] = []
                done[k % buffers] = 0
            else:
                layer_max[k % buffers] = k
                ready = k + 1
            cstep = next(cg, None)


@pytest.mark.parametrize("workers", [4, 8])
@pytest.mark.parametrize("lag", [2, 3])
def test_entries_by_round_mod_lag_plus_1_survive_every_schedule(workers, lag):
    """Entries indexed by round % (lag + 1): the kernel quantises round r-3
    with 4 buffers and 4 key waves (lag 2 with 3 buffers is the earlier
    build's, kept as a case); 8 workers: the count does not matter."""
    for seed in range(400):
        assert run(lag + 1, 9, seed, workers, lag) == [], seed


@pytest.mark.parametrize("workers", [4, 8])
@pytest.mark.parametrize("lag", [2, 3])
def test_entries_by_round_mod_lag_lose_counts(workers, lag):
    """One buffer fewer than lag + 1 and some schedule loses a count."""
    failures = sum(1 for seed in range(200) if run(lag, 9, seed, workers, lag))
    assert failures > 0
