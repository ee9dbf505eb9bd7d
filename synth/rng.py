"""SplitMix64, written from its published definition (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014; the constants
are those of Vigna's reference ``splitmix64.c``).

Every random draw in the synthetic generators comes from this stream, so the
inputs do not drift with numpy's own generator versions.  Output ``i`` of a
stream with seed ``s`` is ``mix(s + (i + 1) * GAMMA)`` and can be computed in
bulk.
"""
import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK = (1 << 64) - 1


def _mix(z):
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


class SplitMix64:
    """A SplitMix64 stream with bulk draws.  ``state`` advances by GAMMA per
    output, exactly as the scalar definition does."""

    def __init__(self, seed: int):
        self.state = int(seed) & _MASK

    def u64(self, n: int) -> np.ndarray:
        idx = np.arange(1, n + 1, dtype=np.uint64)
        with np.errstate(over="ignore"):
            z = np.uint64(self.state) + idx * GAMMA
            out = _mix(z)
        self.state = (self.state + n * int(GAMMA)) & _MASK
        return out

    def uniform(self, n: int) -> np.ndarray:
        """Doubles in [0, 1) from the top 53 bits."""
        return (self.u64(n) >> np.uint64(11)).astype(np.float64) * (1.0 / (1 << 53))

    def integers(self, lo: int, hi: int, n: int) -> np.ndarray:
        """Integers in [lo, hi] (inclusive), by multiply-shift on 53-bit
        uniforms; the bias is below 2^-40 for the ranges used here."""
        span = hi - lo + 1
        return lo + np.floor(self.uniform(n) * span).astype(np.int64)

    def choice_cdf(self, cdf: np.ndarray, n: int) -> np.ndarray:
        """Indices drawn from a discrete distribution given its CDF."""
        u = self.uniform(n) * cdf[-1]
        return np.searchsorted(cdf, u, side="right").astype(np.int64)

    def u64_scalar(self) -> int:
        return int(self.u64(1)[0])

    def fork(self, tag: int) -> "SplitMix64":
        """An independent child stream, seeded from this one and a tag."""
        return SplitMix64((self.u64_scalar() ^ (tag * 0xD1B54A32D192ED03)) & _MASK)


def zipf_cdf(n: int, s: float) -> np.ndarray:
    """CDF of Zipf(s) over ranks 1..n (unnormalised; choice_cdf scales)."""
    w = 1.0 / np.power(np.arange(1, n + 1, dtype=np.float64), s)
    return np.cumsum(w)
