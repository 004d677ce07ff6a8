"""Pins of the oracle's densify/prune step: brute-force selection, the fp32
key, the output order, and the edge fractions."""
import numpy as np
import pytest

import oracle


def _params(rng, N, deg=1):
    K = (deg + 1) ** 2
    f = np.float32
    return (rng.normal(size=(N, 3)).astype(f), rng.uniform(0.01, 1, size=(N, 3)).astype(f),
            rng.normal(size=(N, 4)).astype(f), rng.uniform(size=N).astype(f),
            rng.normal(size=(N, K, 3)).astype(f))


def _brute(g, opac, frac, min_opac):
    """Select by repeatedly taking the largest remaining fp32 key (lowest index
    first among equals), then filter."""
    N = len(g)
    key = [float(np.float32(np.float32(x * x) + np.float32(y * y)) + np.float32(z * z))
           for x, y, z in g.astype(np.float32)]
    key = [np.inf if np.isnan(k) else k for k in key]
    n = int(np.floor(float(np.float32(frac)) * N + 0.5))
    left, chosen = list(range(N)), []
    for _ in range(n):
        best = left[0]
        for i in left:
            if key[i] > key[best]:
                best = i
        chosen.append(best)
        left.remove(best)
    cand = list(range(N)) + sorted(chosen)
    return [i for i in cand if opac[i] >= np.float32(min_opac)]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_brute_force_with_ties_and_nan(seed):
    rng = np.random.default_rng(seed)
    N = 200
    m, s, q, o, sh = _params(rng, N)
    g = rng.normal(size=(N, 3)).astype(np.float32)
    g[10] = g[20] = g[30]                       # exact ties
    g[40, 1] = np.nan                           # ranks with +inf
    g[41] = [np.inf, 0, 0]
    o[::7] = 0.001                              # pruned
    for frac in (0.0, 0.02, 0.1, 0.5, 1.0):
        r = oracle.densify_prune(m, s, q, o, sh, g, frac, 0.005)
        want = _brute(g, o, frac, 0.005)
        np.testing.assert_array_equal(r["src"], want)
        np.testing.assert_array_equal(r["means"], m[want])
        np.testing.assert_array_equal(r["sh"], sh[want])
        assert np.all(r["opacities"] >= np.float32(0.005))


def test_key_is_taken_in_fp32():
    """(1, 2^-13, 0) and (1, 0, 0) tie in fp32 (1 + 2^-26 rounds to 1), so the
    lower index wins; in fp64 the first vector would rank higher."""
    N = 4
    g = np.array([[0.5, 0, 0], [1, 0, 0], [1, 2.0 ** -13, 0], [0.1, 0, 0]], np.float32)
    m, s, q, o, sh = _params(np.random.default_rng(3), N)
    o[:] = 1.0
    r = oracle.densify_prune(m, s, q, o, sh, g, 0.25, 0.0)   # one clone
    assert r["src"].tolist() == [0, 1, 2, 3, 1]


def test_clone_count_rounding_and_edges():
    rng = np.random.default_rng(4)
    m, s, q, o, sh = _params(rng, 50)
    g = rng.normal(size=(50, 3)).astype(np.float32)
    o[:] = 0.5
    assert len(oracle.densify_prune(m, s, q, o, sh, g, 0.0, 0.0)["src"]) == 50
    assert len(oracle.densify_prune(m, s, q, o, sh, g, 1.0, 0.0)["src"]) == 100
    assert len(oracle.densify_prune(m, s, q, o, sh, g, 0.25, 0.0)["src"]) == 63   # 12.5 -> 13
    assert len(oracle.densify_prune(m, s, q, o, sh, g, 0.5, 0.9)["src"]) == 0
    # clones are exact copies appended in index order after every original
    r = oracle.densify_prune(m, s, q, o, sh, g, 0.2, 0.0)
    assert r["src"][:50].tolist() == list(range(50))
    assert np.all(np.diff(r["src"][50:]) > 0)
    assert int(np.floor(float(np.float32(0.02)) * 6_000_000 + 0.5)) == 120_000
