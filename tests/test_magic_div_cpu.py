"""CPU pins of the launch-invariant divisions the step kernels use.

The kernels divide work-item indices by launch constants (heads, column slices,
chunks per row slice) with a multiply-high by a multiplier the host computes
once per launch (Granlund and Montgomery's division by invariant integers):

  div_magic   q = floor(n m / 2^32),  m = floor(2^32 / d) + 1  (m = 0: q = n for d = 1),
              exact for n d < 2^32;
  div_small   q = floor(n m / 2^20),  m = ceil(2^20 / d),  exact for n < 2^20 / d,
              with n < 4096 so that the 24-bit product fits 32 bits.

Checked here exhaustively or at the domain boundaries for every divisor the kernels
can meet, and the host's shape limit (batch * heads * max(heads, 256) < 2^32) is
checked to keep every tile index inside div_magic's domain.
"""
import numpy as np


def magic(d):
    return 0 if d == 1 else (1 << 32) // d + 1


def div_magic(n, m):
    return n if m == 0 else (n * m) >> 32


def test_div_magic_exact_on_its_domain():
    rng = np.random.default_rng(0)
    for d in range(1, 4097):
        m = magic(d)
        nmax = ((1 << 32) - 1) // d                  # largest n with n d < 2^32
        ns = {0, 1, d - 1, d, d + 1, nmax, nmax - 1, max(nmax - d, 0), max(nmax - d - 1, 0)}
        ns.update(int(x) for x in rng.integers(0, nmax + 1, 64))
        for n in ns:
            assert div_magic(n, m) == n // d, (n, d)


def test_div_magic_domain_is_not_vacuous():
    """Just past the domain the multiplier can be off by one (so the host limit matters)."""
    failures = 0
    for d in (3, 7, 100, 129, 255, 4095):
        m = magic(d)
        for n in range(((1 << 32) // d) * d, ((1 << 32) // d) * d + 64 * d):
            failures += div_magic(n, m) != n // d
    assert failures > 0


def test_div_small_exact_on_its_domain():
    for d in range(1, 4097):
        m = -(-(1 << 20) // d)
        n = np.arange(min(4096, -(-(1 << 20) // d)), dtype=np.int64)
        n = n[n * d < (1 << 20)]
        assert ((n * m) < (1 << 32)).all()
        assert np.array_equal((n * m) >> 20, n // d), d


def test_tile_indices_stay_in_the_domain():
    """tile_of divides item < B H nsplit by nsplit and then b h < B H by H; the host accepts
    a shape only if B H max(H, 256) < 2^32, and nsplit <= 16."""
    for H in (1, 4, 32, 128, 256, 1024):
        Bmax = ((1 << 32) - 1) // (H * max(H, 256))
        for nsplit in (1, 2, 4, 8, 16):
            items = Bmax * H * nsplit
            assert (items - 1) * nsplit < (1 << 32)
            assert (Bmax * H - 1) * H < (1 << 32)
