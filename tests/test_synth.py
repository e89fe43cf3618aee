"""The seeded input generators draw what they are documented to draw.

The 13B-class training workload asks for many near-ties in the master
magnitudes.  `synth.plant_ties` puts them on the n:m keep boundary: in 25% of
the groups the n-th and (n+1)-th largest magnitudes are equal, and in a
disjoint 25% they differ by at most one BF16 ulp.  Gaussian masters alone put
an exact tie there in only about 0.5% of the 6:8 groups.
"""

import numpy as np
import pytest

import synth


def boundary_gap(bits, n, m):
    """Per group: (n-th largest - (n+1)-th largest) magnitude, in BF16 ulps
    of the bit pattern (consecutive finite magnitudes differ by 1)."""
    mag = np.sort((bits & 0x7FFF).reshape(-1, m).astype(np.int32), axis=1)[:, ::-1]
    return mag[:, n - 1] - mag[:, n]


@pytest.mark.parametrize("n,m", [(6, 8), (2, 4)])
def test_planted_ties_sit_on_the_keep_boundary(n, m):
    rng = np.random.default_rng(11)
    bits = synth.gaussian_masters(rng, 512, 4096)
    planted = synth.plant_ties(bits, np.random.default_rng(12), m=m, n=n)
    gap0, gap = boundary_gap(bits, n, m), boundary_gap(planted, n, m)
    assert (gap0 == 0).mean() < 0.01                  # natural exact ties are rare
    assert 0.24 <= (gap == 0).mean() <= 0.27          # 25% exact + natural
    assert 0.49 <= (gap <= 1).mean() <= 0.53          # + 25% near ties
    assert np.array_equal(planted & 0x8000, bits & 0x8000)   # signs kept
    changed = (planted != bits).reshape(-1, m).sum(1)
    assert changed.max() <= 3


def test_planted_groups_follow_the_recipe():
    """Exact groups hold the boundary magnitude at 4 positions (or more, with
    natural ties), at least one of them below the boundary of the original
    order; near groups change exactly the documented two positions by one ulp
    around the boundary magnitude."""
    rng = np.random.default_rng(13)
    bits = synth.gaussian_masters(rng, 64, 1024)
    planted = synth.plant_ties(bits, np.random.default_rng(14))
    g0 = (bits & 0x7FFF).reshape(-1, 8).astype(np.int32)
    g1 = (planted & 0x7FFF).reshape(-1, 8).astype(np.int32)
    order = np.argsort(-g0, axis=1, kind="stable")
    bmag = g0[np.arange(len(g0)), order[:, 5]]
    for i in range(len(g0)):
        diff = np.nonzero(g0[i] != g1[i])[0]
        if diff.size == 0:
            continue
        new = g1[i, diff]
        if np.all(new == bmag[i]):
            assert (g1[i] == bmag[i]).sum() >= 4 - (3 - diff.size)
            assert set(order[i, 6:]) & set(np.nonzero(g1[i] == bmag[i])[0])
        else:
            assert diff.size <= 2 and np.all(np.abs(new - bmag[i]) <= 1)


def test_workload_13b_has_planted_ties():
    bits = synth.workload_masters("b13", 0, 256, 5120)
    gap = boundary_gap(bits, 6, 8)
    assert 0.24 <= (gap == 0).mean() <= 0.28
    assert 0.48 <= (gap <= 1).mean() <= 0.54
