"""CPU check of the worker-pool oracle used by the full-size GPU tests: on
small matrices whose "GPU results" are produced by the oracle's own step, the
check passes, and a wrong index or a wrong momentum bit is reported."""

import numpy as np

import oracle as O
import oracle_pool as P


def _case(seed, n=24, m=40, k=6, mu=0.95):
    rng = np.random.default_rng(seed)
    g1 = O.round_to(rng.standard_normal((n, m)) * np.exp(rng.standard_normal((n, 1))), "bf16")
    g2 = O.round_to(rng.standard_normal((n, m)) * np.exp(rng.standard_normal((n, 1))), "bf16")
    W = np.zeros((n, m))
    s1 = O.dion3_step(W, np.zeros((n, m)), g1, k=k, mu=mu, eta=0.0, fmt="bf16", sel_axis=0)
    s2 = O.dion3_step(W, s1["M"], g2, k=k, mu=mu, eta=0.0, fmt="bf16", sel_axis=0)
    return ("m", P.f64_to_bf16_bits(g1), P.f64_to_bf16_bits(g2), P.f64_to_bf16_bits(s2["M"]),
            s1["idx"], s2["idx"], k, mu)


def test_pool_check_passes_and_catches_mistakes():
    good = [_case(s) for s in range(3)]
    bad_idx = list(good[0])
    bad_idx[5] = np.sort(np.r_[bad_idx[5][:-1], [np.setdiff1d(np.arange(24), bad_idx[5])[0]]])
    bad_m = list(good[1])
    bad_m[3] = bad_m[3].copy()
    bad_m[3][0, 0] ^= 1
    with P.pool(2) as pool:
        res = pool.map(P.check_two_steps, good + [tuple(bad_idx), tuple(bad_m)])
    assert [w for _, w in res[:3]] == [None, None, None]
    assert res[3][1] == "idx step 2" and res[4][1] == "M after step 2"


def test_exact_l1_matches_oracle_keys():
    rng = np.random.default_rng(7)
    M = O.round_to(rng.standard_normal((30, 200)) * np.exp(4 * rng.standard_normal((30, 200))), "bf16")
    M[4] = 0.0
    M[9, :3] = [2.0 ** 40, 2.0 ** -60, -2.0 ** -100]      # a row past the exact-sum span
    assert np.array_equal(P.exact_l1(M), O.l1_row_norms(M))
