"""CPU pins of the path-rate model (exact_top_selection_stride_amd.path_model): a closed
form, a brute-force simulation, and the ranks the library documents."""
import numpy as np

from exact_top_selection_stride_amd import path_model as PM


def test_rank_one_closed_form():
    # With tau the largest sample (r = 1), C(tau) = 1 exactly when the row's maximum is one of
    # the n_s samples, which for exchangeable scores happens with probability n_s / L.
    for L, s in ((1000, 10), (4096, 128), (131072, 128)):
        n_s = -(-L // s)
        p = PM.betabinom.pmf(0, L - n_s, 1, n_s)
        assert abs(p - n_s / L) < 1e-9 * (n_s / L)


def test_documented_ranks():
    # K = 2048 on a 128K row (1024 samples): tau0 at rank 24, tau1 at 28, tau_a (2.25 K) at 36.
    t0, t1 = PM.targets(2048)
    assert (t0, t1) == (3072, 3584)
    assert PM.sample_rank(t0, 1024, 131072) == 24
    assert PM.sample_rank(t1, 1024, 131072) == 28
    assert PM.sample_rank((2250 * 2048 + 999) // 1000, 1024, 131072) == 36


def test_matches_simulation():
    # Rows of i.i.d. uniforms, sampled every s-th element: the share with C(tau) < K agrees
    # with the beta-binomial law within four binomial standard deviations.
    rng = np.random.default_rng(11)
    L, s, K, T = 2000, 16, 200, 300
    rows = 20000
    x = rng.random((rows, L), dtype=np.float32)
    n_s = -(-L // s)
    r = PM.sample_rank(T, n_s, L)
    samples = np.sort(x[:, ::s], axis=1)[:, ::-1]
    tau = samples[:, r - 1]
    c = (x >= tau[:, None]).sum(axis=1)
    rate = float((c < K).mean())
    p = PM.p_short(L, K, T, s)
    sigma = np.sqrt(p * (1 - p) / rows)
    assert 0.01 < p < 0.5
    assert abs(rate - p) < 4 * sigma, (rate, p)


def test_expected_counts_sum_rows():
    # Rows no longer than K take no threshold; the others add their probabilities.
    e0, e1 = PM.expected_short_rows([100, 2048, 131072, 131072], 2048)
    p0 = PM.p_short(131072, 2048, 3072)
    p1 = PM.p_short(131072, 2048, 3584)
    assert abs(e0 - 2 * p0) < 1e-12 and abs(e1 - 2 * p1) < 1e-12
    assert 0 < p1 < p0 < 0.05
