"""Pins of the oracle's sampling path (temperature sampling of the drafter, lossless
rejection-sampling verification) against things other than itself: the published
splitmix64 vectors, the distribution Gumbel-max sampling must reproduce, the target
distribution a lossless verifier must emit, and the greedy limit at small temperature."""
import numpy as np
from scipy import stats

import oracle as O


def test_splitmix64_matches_published_vectors():
    # Vigna's splitmix64 from seed 1234567: the first five outputs
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    seed = 1234567
    got = [int(O.splitmix64_mix(np.uint64((seed + k * 0x9E3779B97F4A7C15) % 2 ** 64))) for k in range(1, 6)]
    assert got == want


def test_uniforms_are_uniform_in_the_open_interval():
    u = O.uniform01(7, 3, 0, 2, 5, np.arange(200000))
    assert u.dtype == np.float32 and u.min() > 0 and u.max() < 1
    # the extreme draws stay strictly inside (0, 1) in float32
    top = (np.float32(2 ** 23 - 1) + np.float32(0.5)) * np.float32(2.0 ** -23)
    low = np.float32(0.5) * np.float32(2.0 ** -23)
    assert 0 < low and top < 1 and np.isfinite(-np.log(-np.log(np.array([low, top], np.float32)))).all()
    counts, _ = np.histogram(u, bins=32, range=(0, 1))
    assert stats.chisquare(counts).pvalue > 1e-3
    # different fields give different streams
    assert not np.array_equal(u[:1000], O.uniform01(7, 3, 1, 2, 5, np.arange(1000)))
    assert not np.array_equal(u[:1000], O.uniform01(8, 3, 0, 2, 5, np.arange(1000)))


def test_gumbel_max_samples_the_tempered_softmax():
    rng = np.random.default_rng(0)
    z = rng.normal(0, 1.5, 8).astype(np.float32)
    for T in (0.5, 1.0, 2.0):
        n = 30000
        draws = np.array([int(O.argmax_lowest(O.sample_keys(z, T, 11, c, 0, 0, 1))) for c in range(n)])
        p = np.exp(O.log_softmax_t(z, T))
        counts = np.bincount(draws, minlength=8)
        assert stats.chisquare(counts, p * n).pvalue > 1e-3, T


def test_small_temperature_sampling_is_greedy():
    rng = np.random.default_rng(1)
    z = rng.normal(0, 1, (20, 50)).astype(np.float32)
    for i in range(20):
        assert int(O.argmax_lowest(O.sample_keys(z[i], 1e-4, 3, 0, 0, 0, i))) == int(np.argmax(z[i]))


def _emitted_first_token(zq, zp, T, c):
    """One block of B = 2 (one draft): draft d ~ q, verify against p_0; the first token the
    cycle emits is d when accepted, else the residual draw."""
    d = int(O.argmax_lowest(O.sample_keys(zq, T, 5, c, 0, 0, 1)))
    zt = np.stack([zp, zp])          # row 0 checks d; row 1 would give the bonus
    a, tau, tok, _, _, _ = O.accept_sampled(np.array([d]), zq[None], zt, T, 5, c, 0)
    return d if a == 1 else tok


def test_rejection_sampling_emits_the_target_distribution():
    """Whatever the drafter proposes, the first emitted token is distributed as p_0: the
    verifier is lossless."""
    rng = np.random.default_rng(2)
    for T in (1.0, 0.7):
        zq = rng.normal(0, 1.2, 6).astype(np.float32)
        zp = rng.normal(0, 1.2, 6).astype(np.float32)
        n = 30000
        got = np.bincount([_emitted_first_token(zq, zp, T, c) for c in range(n)], minlength=6)
        p = np.exp(O.log_softmax_t(zp, T))
        assert stats.chisquare(got, p * n).pvalue > 1e-3, T
        # and it is not the drafter's distribution (the test can tell the two apart)
        q = np.exp(O.log_softmax_t(zq, T))
        assert stats.chisquare(got, q * n).pvalue < 1e-6


def test_bonus_after_full_acceptance_follows_the_last_target_row():
    """With the drafter equal to the target every draft passes (ratio 1 > u), tau = B, and
    the emitted token is a draw from the last target row."""
    rng = np.random.default_rng(3)
    B, V, T = 4, 7, 1.0
    zp = rng.normal(0, 1, (B, V)).astype(np.float32)
    n = 20000
    toks = []
    for c in range(n):
        drafts = np.array([int(O.argmax_lowest(O.sample_keys(zp[i - 1], T, 9, c, 0, 0, i))) for i in range(1, B)])
        a, tau, tok, ratios, us, _ = O.accept_sampled(drafts, zp[:B - 1], zp, T, 9, c, 0)
        assert a == B - 1 and tau == B and np.allclose(ratios, 1.0)
        toks.append(tok)
    p = np.exp(O.log_softmax_t(zp[B - 1], T))
    assert stats.chisquare(np.bincount(toks, minlength=V), p * n).pvalue > 1e-3


def test_rejection_uses_the_previous_target_row():
    """A draft at position i is judged by the target's row i-1: with p_0 putting no mass on
    the draft it is always rejected, whatever row 1 says."""
    V, T = 5, 1.0
    zq = np.array([[4.0, 0, 0, 0, 0]], np.float32)      # the drafter proposes token 0
    zt = np.array([[-60.0, 0, 0, 0, 0], [60.0, 0, 0, 0, 0]], np.float32)   # row 0 rules 0 out
    for c in range(200):
        a, tau, tok, r, u, _ = O.accept_sampled(np.array([0]), zq, zt, T, 1, c, 0)
        assert a == 0 and tau == 1 and tok != 0 and r[0] < 1e-20
