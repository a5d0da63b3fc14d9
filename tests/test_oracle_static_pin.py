"""Pin of the hindsight static pin: it is the best fixed set, by brute force over all subsets."""
import itertools

import numpy as np

from oracle import static_pin, static_pin_hit_rate


def test_static_pin_is_optimal_over_all_subsets():
    rng = np.random.default_rng(8)
    for trial in range(20):
        E, S = 7, int(rng.integers(1, 6))
        steps = [set(rng.choice(E, size=int(rng.integers(1, 4)), replace=False).tolist()) for _ in range(40)]
        tot = sum(len(u) for u in steps)
        best = max(sum(len(u & set(c)) for u in steps) for c in itertools.combinations(range(E), S))
        assert abs(static_pin_hit_rate(steps, E, S) - best / tot) < 1e-15
        pin = static_pin(steps, E, S)
        assert len(pin) == S and sum(len(u & set(pin)) for u in steps) == best
