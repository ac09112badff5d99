"""A CPU model of the split-K slot protocol shared by the batch-1 and grouped kernels.

Output block c of a call with S splits takes its tickets from counter c, which advances by
2^16 per call, and its partials travel in slots (c*S + s, lane) for s < S, each tagged with
the call number (the counter's high 16 bits) and S. A reducer must never find, before the
call's own writers have stored, a slot of its layout that already holds the tag it waits
for. The model replays random sequences of layers with different block and split counts on
one workspace and checks that rule, and checks that it catches the weaker tag made of the
call number alone, so the test is not vacuous."""
import numpy as np


def _replay(calls, tag_of):
    counters, slots = {}, {}
    stale_matches = 0
    for ob, S in calls:
        for c in range(ob):
            call = counters.get(c, 0) >> 16
            want = tag_of(call, S)
            stale_matches += sum(slots.get(c * S + s) == want for s in range(S))
        for c in range(ob):
            call = counters.get(c, 0) >> 16
            for s in range(S):
                slots[c * S + s] = tag_of(call, S)
            counters[c] = counters.get(c, 0) + (1 << 16)
    return stale_matches


def _tag_with_splits(call, S):
    return ((call & 0xFFFF) << 16) | S


def _tag_call_only(call, S):
    return (call & 0xFFFF) + 1


def _random_calls(rng, n_layers, n_calls):
    layers = [(int(rng.integers(1, 65)), int(rng.integers(2, 33))) for _ in range(n_layers)]
    return [layers[int(rng.integers(0, n_layers))] for _ in range(n_calls)]


def test_no_stale_slot_carries_the_expected_tag():
    rng = np.random.default_rng(7)
    for _ in range(40):
        calls = _random_calls(rng, n_layers=int(rng.integers(2, 6)), n_calls=300)
        assert _replay(calls, _tag_with_splits) == 0


def test_model_catches_a_tag_of_the_call_number_alone():
    # The two layers of the GPU test: 1024 x 4096 (8 blocks, 8 splits) and 512 x 8192
    # (4 blocks, 16 splits), called a, b, a: the third call's blocks 4..7 meet b's slots.
    assert _replay([(8, 8), (4, 16), (8, 8)], _tag_call_only) > 0
    assert _replay([(8, 8), (4, 16), (8, 8)], _tag_with_splits) == 0
    rng = np.random.default_rng(8)
    hits = sum(_replay(_random_calls(rng, 3, 200), _tag_call_only) > 0 for _ in range(20))
    assert hits > 0


def test_one_layer_repeated_wraps_harmlessly():
    # A single layer never meets a stale tag, through the 16-bit wrap of the call number.
    assert _replay([(2, 4)] * 70_000, _tag_with_splits) == 0
