"""Expected path rates of the sampled selector on rows of exchangeable scores.

A sizing and calibration model, not part of the selection. The pages give the sample
stride and the candidate targets (page "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确
Top-K", section "采样不是处处都该开"), not a model of how often each path is taken; this is
one derived from the order statistics of the sample.

A row of L scores is sampled at offsets 0, s, 2s, ... (n_s = ceil(L / s) samples), and tau
is the r-th largest sample key. For exchangeable continuous scores (i.i.d. per element, no
ties), the share of the row above tau is distributed as the r-th largest of n_s uniforms,
Beta(r, n_s - r + 1). Given that share, each of the other L - n_s elements lies above tau
independently, so the count of keys >= tau is

    C(tau) = r + X,   X ~ BetaBinomial(L - n_s, r, n_s - r + 1).

The selector certifies a row at tau0 when C(tau0) >= K and falls back to tau1 (and, on rows
sampled one element per period, to the deeper rank tau_a) otherwise. The targets follow
the library's host rules: T = ceil(rho * K / 1000) with rho0 = 1500 and rho1 = 1750 per
mille, clamped to [12 s, 5 CAP / 8] and [16 s, 3 CAP / 4], T1 >= T0; the rank of a target
is r = ceil(T * n_s / L), within [1, n_s].

The synthetic FP32 workloads draw every element independently, so the model applies to
them; the bf16-rounded ones have ties and it does not.
"""
from typing import Iterable, Tuple

from scipy.stats import betabinom

CAP = 8192  # candidate slots of the selector's LDS buffer


def targets(K: int, stride: int = 128, rho0: int = 1500, rho1: int = 1750) -> Tuple[int, int]:
    """(T0, T1): the candidate targets of the first and second thresholds."""
    t0 = (rho0 * K + 999) // 1000
    t1 = (rho1 * K + 999) // 1000
    t0 = min(max(t0, 12 * stride), 5 * CAP // 8)
    t1 = min(max(t1, 16 * stride), 3 * CAP // 4)
    return t0, max(t1, t0)


def sample_rank(target: int, n_s: int, L: int) -> int:
    """Rank (1 = largest) of the sample key that aims at `target` keys above it."""
    r = -(-target * n_s // L)
    return max(1, min(n_s, r))


def p_short(L: int, K: int, target: int, stride: int = 128) -> float:
    """P(C(tau) < K) for the threshold at the rank of `target` on one row of length L."""
    n_s = -(-L // stride)
    r = sample_rank(target, n_s, L)
    if K - r - 1 < 0:
        return 0.0
    return float(betabinom.cdf(K - r - 1, L - n_s, r, n_s - r + 1))


def expected_short_rows(lengths: Iterable[int], K: int, stride: int = 128, rho0: int = 1500,
                        rho1: int = 1750) -> Tuple[float, float]:
    """Expected numbers of rows (of those longer than K) with C(tau0) < K and with
    C(tau1) < K."""
    t0, t1 = targets(K, stride, rho0, rho1)
    e0 = e1 = 0.0
    cache = {}
    for L in lengths:
        L = int(L)
        if L <= K:
            continue
        if L not in cache:
            cache[L] = (p_short(L, K, t0, stride), p_short(L, K, t1, stride))
        a, b = cache[L]
        e0 += a
        e1 += b
    return e0, e1
