"""Host-side mirror of the streaming GQA kernel's work partition (CPU only):
wave w of the n waves in use runs tiles [floor(w T / n), floor((w+1) T / n)),
and the combine finds the wave of tile x as ceil((x + 1) n / T) - 1."""
import numpy as np


def test_gqa_tile_split_invariants():
    """Ranges cover 0 .. T once in wave order, every wave in use gets at least
    one tile and at most one more than any other, and the combine's closed
    form finds the wave that holds each tile."""
    rng = np.random.default_rng(0)
    for _ in range(300):
        n = int(rng.integers(1, 2049))
        T = int(rng.integers(n, 40 * n))
        lo = np.array([w * T // n for w in range(n + 1)])
        assert lo[0] == 0 and lo[-1] == T
        cnt = np.diff(lo)
        assert cnt.min() >= 1 and cnt.max() - cnt.min() <= 1
        x = rng.integers(0, T, 50)
        w = -(-(x + 1) * n // T) - 1
        assert ((lo[w] <= x) & (x < lo[w + 1])).all()
