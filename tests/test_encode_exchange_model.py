"""Model check of the single-pass encode's exchange across workgroups over a
sequence of calls on one workspace (host logic, no GPU).

Each workgroup's coordinator, for layer l = 0, 1, ...: publishes its maximum
of layer l in its word of the layer, tagged with the call's number, then
reads every workgroup's word of the layer until all carry this call's
number - or gives up (a bounded wait) and takes the layer's maximum from the
keys directly. Nothing is ever cleared. Under random interleavings (any
workgroup may run late, any wait may give up) every maximum a workgroup
uses must be this call's true maximum, also when the calls have different
layer counts. Without the tag (a plain "published" flag) the words a call
leaves behind are taken for the next call's, and some schedule uses a stale
maximum."""

import random

import pytest


def run_call(ws, call, G, L, maxima, rng, tagged=True, give_up=0.1):
    """One encode: ws maps (layer, workgroup) to (tag, value); maxima[g][l]
    is workgroup g's local maximum. Returns the errors found."""
    true = [max(maxima[g][l] for g in range(G)) for l in range(L)]
    tag = call if tagged else 1
    errors = []

    def coordinator(g):
        for l in range(L):
            ws[(l, g)] = (tag, maxima[g][l])
            yield
            while True:
                seen = []
                for h in range(G):
                    seen.append(ws.get((l, h), (0, 0)))
                    yield
                if all(t == tag for t, _ in seen):
                    used = max(x for _, x in seen)
                    break
                if rng.random() < give_up:
                    used = true[l]   # read from the keys directly: exact
                    break
            if used != true[l]:
                errors.append(f"call {call} wg {g} layer {l}: used {used}, true {true[l]}")

    procs = [coordinator(g) for g in range(G)]
    live = list(range(G))
    steps = 0
    while live:
        g = rng.choice(live)
        try:
            next(procs[g])
        except StopIteration:
            live.remove(g)
        steps += 1
        if steps > 400 * G * G * L:
            return errors + ["stuck: a wait that never ends without its bound"]
    return errors


@pytest.mark.parametrize("give_up", [0.0, 0.1])
@pytest.mark.parametrize("G", [3, 4, 6])
def test_tagged_words_give_exact_maxima_over_calls(G, give_up):
    """Calls 1..5 on one workspace with layer counts that change from call to
    call: every maximum used is the call's own; with every workgroup
    resident (no wait gives up) no poll depends on its bound."""
    for seed in range(200):
        rng = random.Random(seed)
        ws = {}
        for call in range(1, 6):
            L = rng.choice([1, 2, 3])
            maxima = [[rng.randrange(1, 1000) for _ in range(L)] for _ in range(G)]
            errs = run_call(ws, call, G, L, maxima, rng, give_up=give_up)
            assert errs == [], (seed, errs)


def test_untagged_flags_leak_stale_maxima():
    """The same protocol with a plain flag instead of the call's number:
    some schedule has a workgroup take a word left by the previous call."""
    bad = 0
    for seed in range(200):
        rng = random.Random(seed)
        ws = {}
        for call in range(1, 4):
            maxima = [[rng.randrange(1, 1000) for _ in range(2)] for _ in range(4)]
            if run_call(ws, call, 4, 2, maxima, rng, tagged=False):
                bad += 1
                break
    assert bad > 0
