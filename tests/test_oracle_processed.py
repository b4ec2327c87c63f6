"""Pins for the oracle's processed target distribution: temperature, top-k,
top-p and the renormalisation that "Why speculative decoding preserves
distributions but may not be faster" (Sec. 1) requires of p, and that
"Speculative Decoding: Draft, Then Verify" ("Production gotchas", "The same
sampling settings") requires the test and the residual to use.

The pages name the filters but leave their ties open; the readings are the
oracle's (every token tied with the k-th largest logit is kept; a token is in
the nucleus iff the renormalised mass of the strictly larger tokens is below
top_p).  The tests hold the oracle to independent formulations of the same
sets (counts of strictly larger tokens, brute-force mass sums, a sorted
cumulative sum on distinct logits), to library routines (softmax,
logsumexp), to the greedy contract, and to the output-follows-p property.
"""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from tests._oracle_cases import chi2_pvalue, identity_problem


def _tie_heavy_logits(rng, V):
    # small integers: many exact ties, including at the filter boundaries
    return rng.integers(-3, 4, size=V).astype(np.float64)


def test_no_filter_is_the_softmax():
    rng = np.random.default_rng(1)
    for V in (1, 2, 7, 300):
        l = rng.standard_normal(V) * 3
        for k, p in ((0, 0.0), (V, 1.0), (V + 5, 1.5)):
            pr, cnt, lz, _ = oracle.processed(l, k, p)
            assert cnt == V
            np.testing.assert_allclose(pr, softmax(l), rtol=1e-14, atol=1e-300)
            assert abs(lz - logsumexp(l)) < 1e-12


def test_top_k_keeps_tokens_with_fewer_than_k_strictly_larger():
    rng = np.random.default_rng(2)
    for trial in range(200):
        V = int(rng.integers(1, 9))
        l = _tie_heavy_logits(rng, V)
        for k in range(1, V + 1):
            pr, cnt, lz, _ = oracle.processed(l, k, 0.0)
            keep = np.array([(l > l[v]).sum() < k for v in range(V)])
            assert cnt == keep.sum()
            np.testing.assert_array_equal(pr > 0, keep)
            np.testing.assert_allclose(pr[keep], softmax(l[keep]), rtol=1e-14)
            assert abs(lz - logsumexp(l[keep])) < 1e-12


def test_top_p_brute_force_mass_of_strictly_larger_tokens():
    rng = np.random.default_rng(3)
    for trial in range(300):
        V = int(rng.integers(1, 9))
        l = _tie_heavy_logits(rng, V) if trial % 2 else rng.standard_normal(V)
        k = int(rng.integers(0, V + 1))
        top_p = float(rng.choice([0.05, 0.3, 0.5, 0.77, 0.95]))
        pr, cnt, _, margin = oracle.processed(l, k, top_p)
        in_k = np.array([k == 0 or (l > l[v]).sum() < k for v in range(V)])
        pk = np.where(in_k, np.exp(l - l.max()), 0.0)
        pk /= pk.sum()
        larger_mass = np.array([pk[(l > l[v]) & in_k].sum() for v in range(V)])
        keep = in_k & (larger_mass < top_p)
        if np.min(np.abs(larger_mass[in_k] - top_p)) < 1e-12:
            continue  # an exact tie with top_p: rounding decides
        assert cnt == keep.sum(), (l, k, top_p)
        np.testing.assert_array_equal(pr > 0, keep)
        np.testing.assert_allclose(pr[keep], softmax(l[keep]), rtol=1e-13)
        assert margin <= np.min(np.abs(larger_mass[in_k] - top_p)) + 1e-12


def test_top_p_matches_the_sorted_cumulative_sum_on_distinct_logits():
    """With distinct logits the nucleus is the shortest prefix (in order of
    probability) whose mass reaches top_p."""
    rng = np.random.default_rng(4)
    for trial in range(200):
        V = int(rng.integers(2, 60))
        l = rng.standard_normal(V) * 2
        top_p = float(rng.uniform(0.01, 0.99))
        order = np.argsort(-l)
        cs = np.cumsum(softmax(l)[order])
        n_keep = int(np.searchsorted(cs, top_p) + 1)  # first prefix with mass >= top_p
        if np.min(np.abs(cs - top_p)) < 1e-12:
            continue
        pr, cnt, _, _ = oracle.processed(l, 0, top_p)
        assert cnt == n_keep
        assert set(np.flatnonzero(pr)) == set(order[:n_keep])


def test_filters_nest():
    rng = np.random.default_rng(5)
    for trial in range(100):
        V = int(rng.integers(2, 30))
        l = _tie_heavy_logits(rng, V) if trial % 2 else rng.standard_normal(V)
        sets_k = [set(np.flatnonzero(oracle.processed(l, k, 0.0)[0])) for k in range(1, V + 1)]
        for a, b in zip(sets_k, sets_k[1:]):
            assert a <= b
        sets_p = [set(np.flatnonzero(oracle.processed(l, 0, p)[0])) for p in (0.1, 0.4, 0.7, 0.9, 0.99)]
        for a, b in zip(sets_p, sets_p[1:]):
            assert a <= b
        # the argmax group is always kept
        amax = set(np.flatnonzero(l == l.max()))
        assert amax <= sets_k[0] and amax <= sets_p[0]


def test_margins_measure_the_distance_to_a_flip():
    l = np.array([3.0, 1.0, 2.0, 2.0, 0.0])
    z = np.exp(l - 3).sum()
    # top_p = 0.5: the group {3} alone (mass 0.5206 reaches 0.5); margin 0.0206
    pr, cnt, _, m = oracle.processed(l, 0, 0.5)
    assert cnt == 1 and abs(m - (1 / z - 0.5)) < 1e-12
    # top_k = 2: the 2nd largest logit is 2, tied twice -> three tokens; the gap to 1 is 1
    pr, cnt, _, m = oracle.processed(l, 2, 0.0)
    assert cnt == 3 and m == 1.0


# ------------------------------------------------------------ in the verify step
def _row_problem(p_rows, q_rows, drafts):
    W, h, d, q = identity_problem(p_rows, q_rows, drafts)
    return W, h, d, q


def test_temperature_divides_every_logit_row():
    """softmax(l / T): the logits are divided exactly (a power of two here),
    argmaxes are unchanged, log-partitions follow logsumexp(l / T)."""
    rng = np.random.default_rng(6)
    B, G, V = 3, 2, 40
    p = rng.dirichlet(np.ones(V) * 0.5, size=(B, G + 1))
    q = rng.dirichlet(np.ones(V), size=(B, G))
    W, h, d, qh = _row_problem(p, q, rng.integers(0, V, (B, G)))
    modes = np.array([0, 1, 2], np.uint8)
    r1 = oracle.run(W, h, d, qh, modes, 3, 0.1, 11, want_logits=True, n_threads=1)
    r2 = oracle.run(W, h, d, qh, modes, 3, 0.1, 11, want_logits=True, n_threads=1, temperature=2.0)
    ok = ~np.isnan(r1["logits"])
    np.testing.assert_array_equal(r2["logits"][ok], r1["logits"][ok] / 2)
    np.testing.assert_array_equal(r2["head_argmax"], r1["head_argmax"])
    np.testing.assert_array_equal(r2["centroid_argmax"], r1["centroid_argmax"])
    for b in range(B):
        for t in range(G + 1):
            rows = 3 if modes[b] else 1
            for i in range(rows):
                assert abs(r2["head_logz"][b, t, i] - logsumexp(r1["logits"][b, t, i] / 2)) < 1e-9
    # T = 0 is read as 1
    r0 = oracle.run(W, h, d, qh, modes, 3, 0.1, 11, want_logits=True, n_threads=1, temperature=0.0)
    np.testing.assert_array_equal(r0["logits"][ok], r1["logits"][ok])


def test_top_k_one_is_the_greedy_contract():
    """With top_k = 1 and a unique largest logit the processed target is a
    point mass at the argmax: the lossless test keeps x iff it is the target
    argmax, and the round emits the argmax at the first mismatch (greedy
    decoding, "Speculative Decoding: Draft, Then Verify").  (Ties at the max
    are all kept by the top-k reading, so they share the mass.)"""
    rng = np.random.default_rng(7)
    B, G, V = 64, 4, 12
    logits = rng.standard_normal((B, G + 1, V)) * 2  # no ties at the max: the point mass is one token
    p = softmax(logits, axis=-1)
    q = rng.dirichlet(np.ones(V), size=(B, G))
    target = p.argmax(-1)  # numpy: first index of the max
    drafts = np.where(rng.random((B, G)) < 0.6, target[:, :-1], rng.integers(0, V, (B, G)))
    W, h, d, qh = _row_problem(p, q, drafts)
    r = oracle.run(W, h, d, qh, np.zeros(B, np.uint8), 1, 0.0, 3, n_threads=1, top_k=1)
    match = drafts == target[:, :-1]
    np.testing.assert_array_equal(r["accept_flags"].astype(bool), match)
    A = np.where(match.all(1), G, np.argmin(match, axis=1))
    np.testing.assert_array_equal(r["accept_len"], A)
    np.testing.assert_array_equal(r["out_token"], target[np.arange(B), A])
    np.testing.assert_array_equal(r["filter_count"], np.ones((B, G + 1), np.int32))


@pytest.mark.parametrize("k,top_p,seed", [(3, 0.0, 41), (0, 0.8, 42), (4, 0.7, 43)])
def test_committed_token_follows_the_processed_p(k, top_p, seed):
    """Probability budget Sec. 1-2 with processed distributions: drafts drawn
    from q, the first committed token follows the processed p."""
    rng = np.random.default_rng(seed)
    V = 7
    l = rng.standard_normal(V) * 1.5
    p_proc = oracle.processed(l, k, top_p)[0]
    q = rng.dirichlet(np.ones(V) * 0.8)
    n = 60_000
    drafts = rng.choice(V, size=(n, 1), p=q)
    P = np.broadcast_to(softmax(l), (n, 2, V))
    Q = np.broadcast_to(q, (n, 1, V))
    W, h, d, qh = identity_problem(P, Q, drafts)
    r = oracle.run(W, h, d, qh, np.zeros(n, np.uint8), 1, 0.0, seed, n_threads=1, top_k=k, top_p=top_p)
    first = np.where(r["accept_len"] >= 1, drafts[:, 0], r["out_token"])
    counts = np.bincount(first, minlength=V)
    assert chi2_pvalue(counts, p_proc) > 1e-3
    # the filters remove real mass here, and the unprocessed p is rejected
    assert np.any(p_proc == 0) and softmax(l)[p_proc == 0].sum() > 0.05
    assert chi2_pvalue(counts, softmax(l)) < 1e-6
