"""Pins for the oracle's score (CPU only).

Each test ties the oracle to something other than itself: closed forms the
mathematics fixes, the textbook rotation-matrix statement of RoPE, invariants
the pages state, and agreement of three independently written evaluations
(definition, trigonometric series, angle-addition fold).
"""
import itertools
import math

import numpy as np
import pytest

from oracle import (band_frequencies, fold_coefficients, rope_rotate, score_folded,
                    score_literal, score_series)
from workloads import rng

FORMS = [score_literal, score_series, score_folded]


# --------------------------------------------------------------------------
# closed forms (values fixed by trigonometry, not by the oracle)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("form", FORMS)
def test_d2_unit_vectors_give_cos_of_distance(form):
    # d=2: one band with omega_0 = theta^0 = 1, so the logit is cos(Delta + phi).
    K = np.array([[1.0, 0.0]])
    assert form(K, [0], [1.0, 0.0], 3, 1e4, [0])[0] == pytest.approx(math.cos(3.0), abs=1e-14)
    # q has phase +pi/2, k phase 0: cos(Delta + pi/2) = -sin(Delta).  Pins the sign convention
    # phi = arg q - arg k and the direction of rotation.
    assert form(K, [4], [0.0, 1.0], 5, 1e6, [0])[0] == pytest.approx(-math.sin(1.0), abs=1e-14)
    # averaging over the offsets D = {1, 2} with t = p
    assert form(K, [7], [1.0, 0.0], 7, 1e4, [1, 2])[0] == pytest.approx(
        (math.cos(1.0) + math.cos(2.0)) / 2, abs=1e-14)


@pytest.mark.parametrize("form", FORMS)
def test_band_frequency_and_interleaving(form):
    # d=4, theta=1e4: omega_1 = 1e4^(-2/4) = 0.01.  Band 1 is coordinates (2, 3).
    K = np.array([[0.0, 0.0, 1.0, 0.0]])
    assert form(K, [0], [0.0, 0.0, 1.0, 0.0], 100, 1e4, [0])[0] == pytest.approx(math.cos(1.0), abs=1e-13)
    # coordinate 0 pairs with 1, not with 2: different bands never interact.
    for dist in (0, 1, 17, 1000):
        assert form(np.array([[0.0, 0.0, 1.0, 0.0]]), [0], [1.0, 0.0, 0.0, 0.0], dist, 1e4, [0])[0] == \
            pytest.approx(0.0, abs=1e-14)
    # q=(1,0,0,0), k=(0,1,0,0): phi = 0 - pi/2, so cos(1 - pi/2) = sin(1) at Delta = 1.
    assert form(np.array([[0.0, 1.0, 0.0, 0.0]]), [0], [1.0, 0.0, 0.0, 0.0], 1, 1e4, [0])[0] == \
        pytest.approx(math.sin(1.0), abs=1e-14)


@pytest.mark.parametrize("form", FORMS)
def test_magnitudes_enter_as_product(form):
    # |q|=5, |k|=2, angle between them: atan2(4,3) - pi/2 -> logit = 10*sin(atan2(4,3)) = 8 = <q,k>.
    assert form(np.array([[0.0, 2.0]]), [9], [3.0, 4.0], 9, 1e4, [0])[0] == pytest.approx(8.0, abs=1e-13)


def test_band_frequencies_values():
    w = band_frequencies(8, 1e4)
    assert w[0] == 1.0
    np.testing.assert_allclose(w, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    np.testing.assert_allclose(band_frequencies(128, 1e6)[64 - 1], 1e6 ** (-126 / 128), rtol=1e-15)


# --------------------------------------------------------------------------
# textbook statement of RoPE as a block-diagonal rotation matrix
# --------------------------------------------------------------------------
def _rope_matrix(d, p, theta):
    R = np.zeros((d, d))
    for f in range(d // 2):
        a = p * theta ** (-2.0 * f / d)
        R[2 * f:2 * f + 2, 2 * f:2 * f + 2] = [[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]]
    return R


@pytest.mark.parametrize("d,theta", [(2, 1e4), (4, 1e4), (8, 1e6), (16, 500.0)])
def test_rotation_matrix_brute_force(d, theta):
    r = rng(100, d)
    T = 7
    K = r.standard_normal((T, d))
    q = r.standard_normal(d)
    pos = r.integers(0, 300, T)
    t = 311
    D = [1, 3, 8, 64]
    ref = np.array([np.mean([(_rope_matrix(d, t + dl, theta) @ q) @ (_rope_matrix(d, p, theta) @ k)
                             for dl in D]) for k, p in zip(K, pos)])
    for form in FORMS:
        np.testing.assert_allclose(form(K, pos, q, t, theta, D), ref, rtol=0, atol=1e-12)
    # and rope_rotate itself equals the matrix action
    np.testing.assert_allclose(rope_rotate(K, pos, theta),
                               np.stack([_rope_matrix(d, p, theta) @ k for k, p in zip(K, pos)]), atol=1e-13)


def test_relative_position_property_of_rotation():
    # R(a)^T R(b) = R(b - a): the logit depends on positions only through their difference.
    d, theta = 8, 1e4
    for a, b in [(0, 5), (100, 37), (32768, 65536 + 32768)]:
        np.testing.assert_allclose(_rope_matrix(d, a, theta).T @ _rope_matrix(d, b, theta),
                                   _rope_matrix(d, b - a, theta), atol=1e-9)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def _rand_head(seed, T=33, d=16):
    r = rng(101, seed)
    return r.standard_normal((T, d)), r.integers(0, 5000, T), r.standard_normal(d)


@pytest.mark.parametrize("d", [2, 4, 8, 64, 128])
@pytest.mark.parametrize("theta", [1e4, 1e6])
def test_three_forms_agree(d, theta):
    r = rng(102, d, int(theta))
    K, pos, q = r.standard_normal((40, d)), r.integers(0, 40000, 40), r.standard_normal(d)
    D = sorted(set(int(x) for x in r.integers(0, 70000, 9)))
    t = 40000
    lit = score_literal(K, pos, q, t, theta, D)
    amp = np.abs(q[0::2] + 1j * q[1::2]) @ np.abs(K[:, 0::2] + 1j * K[:, 1::2]).T
    # fp64 evaluation of cos at phase angles up to ~1.1e5 rad carries ~eps*angle absolute error
    tol = 8 * np.finfo(np.float64).eps * (t + max(D)) + 1e-14
    for form in (score_series, score_folded):
        assert np.max(np.abs(form(K, pos, q, t, theta, D) - lit) / amp) < tol


def test_shift_invariance():
    # a common shift of the current position and every key position leaves the score unchanged
    K, pos, q = _rand_head(1)
    D = [2 ** i for i in range(17)]
    a = score_literal(K, pos, q, 6000, 1e6, D)
    for c in (1, 977, 123456):
        np.testing.assert_allclose(score_literal(K, pos + c, q, 6000 + c, 1e6, D), a, atol=1e-9, rtol=0)


def test_zero_offset_at_same_position_is_plain_dot_product():
    # D = {0} and p = t: both vectors rotate by the same angle; the real dot product is unchanged
    K, pos, q = _rand_head(2)
    np.testing.assert_allclose(score_literal(K, np.full(len(K), 4242), q, 4242, 1e4, [0]), K @ q, atol=1e-12)


def test_linearity_in_query_centre():
    # the mean of G query centres scores as the mean of the G scores
    K, pos, _ = _rand_head(3)
    r = rng(103)
    qs = r.standard_normal((4, K.shape[1]))
    D = [1, 2, 4, 8]
    mean_q = score_literal(K, pos, qs.mean(0), 5100, 1e6, D)
    np.testing.assert_allclose(mean_q, np.mean([score_literal(K, pos, qg, 5100, 1e6, D) for qg in qs], 0),
                               atol=1e-12)


def test_bilinear_scaling():
    K, pos, q = _rand_head(4)
    D = [1, 16, 256]
    base = score_literal(K, pos, q, 5000, 1e4, D)
    np.testing.assert_allclose(score_literal(2.5 * K, pos, -0.5 * q, 5000, 1e4, D), -1.25 * base, atol=1e-12)


def test_offset_average_is_mean_of_single_offsets():
    K, pos, q = _rand_head(5)
    D = [1, 2, 4, 8, 16]
    singles = [score_literal(K, pos, q, 5001, 1e6, [dl]) for dl in D]
    np.testing.assert_allclose(score_literal(K, pos, q, 5001, 1e6, D), np.mean(singles, 0), atol=1e-12)


def test_fold_coefficients_limits():
    # low-frequency bands barely turn over D, so A_f -> 1; D = {0} gives A_f = 1 exactly
    A = fold_coefficients(128, 1e6, [2 ** i for i in range(17)])
    assert abs(A[-1] - 1.0) < 0.02        # omega_63 * mean(D) ~ 1.2e-6 * 7710
    assert np.all(np.abs(A) <= 1.0 + 1e-15)
    np.testing.assert_allclose(fold_coefficients(16, 1e4, [0]), np.ones(8))


def test_post_rope_formulation_of_blog_agrees():
    # TriAttention blog (implementation walkthrough): with keys stored post-RoPE, the score is
    # Re(q_centre * conj(k_rot) * exp(i * omega * t_query)) summed over bands.  Averaged over the
    # offsets it must equal the pre-RoPE definition.
    K, pos, q = _rand_head(6, d=32)
    theta, t, D = 1e6, 5200, [1, 4, 64, 4096]
    k_rot = rope_rotate(K, pos, theta)
    omega = band_frequencies(32, theta)
    kr, ki = k_rot[:, 0::2], k_rot[:, 1::2]
    qr, qi = q[0::2], q[1::2]
    prod_real = qr * kr + qi * ki
    prod_imag = qi * kr - qr * ki
    blog = np.mean([np.sum(prod_real * np.cos((t + dl) * omega) - prod_imag * np.sin((t + dl) * omega), 1)
                    for dl in D], 0)
    np.testing.assert_allclose(score_literal(K, pos, q, t, theta, D), blog, atol=1e-11)


def test_bad_inputs_raise():
    with pytest.raises(ValueError):
        score_literal(np.zeros((3, 5)), None, np.zeros(5), 0, 1e4, [1])
    with pytest.raises(ValueError):
        score_literal(np.zeros((3, 4)), None, np.zeros(4), 0, 1e4, [])


# --------------------------------------------------------------------------
# the norm-based term (TriAttention summary 3.4, "The Norm-Based Term")
# --------------------------------------------------------------------------
from oracle import norm_term, score_full  # noqa: E402


def test_norm_term_hand_example():
    # |q_bar| = 5, E|q| = 7 (R = 5/7), |k| = 2: (1 - 5/7) * 7 * 2 = 4
    assert norm_term(np.array([[0.0, 2.0]]), [3.0, 4.0], [7.0])[0] == pytest.approx(4.0, abs=1e-14)
    # two bands: only band 1 is dispersed; band 0 has R = 1 and contributes nothing
    K = np.array([[3.0, 4.0, 1.0, 0.0]])
    assert norm_term(K, [1.0, 0.0, 0.0, 2.0], [1.0, 3.0])[0] == pytest.approx((3.0 - 2.0) * 1.0, abs=1e-14)


def test_norm_term_limits():
    r = rng(110)
    K, q = r.standard_normal((9, 16)), r.standard_normal(16)
    centre = np.abs(q[0::2] + 1j * q[1::2])
    # perfect concentration (R_f = 1): the norm term vanishes and the full score is S_trig
    np.testing.assert_allclose(norm_term(K, q, centre), 0.0, atol=1e-14)
    np.testing.assert_allclose(score_full(K, None, q, centre, 500, 1e4, [1, 2]),
                               score_literal(K, None, q, 500, 1e4, [1, 2]), atol=1e-12)
    # no directional signal (q_bar = 0, R_f = 0): the basic form sum_f E|q_f| |k_f|
    qa = np.abs(r.standard_normal(8)) + 0.1
    kabs = np.hypot(K[:, 0::2], K[:, 1::2])
    np.testing.assert_allclose(norm_term(K, np.zeros(16), qa), kabs @ qa, atol=1e-12)
    # the dispersion form stated beside it: sum_f (E|q_f| - |q_bar_f|) |k_f|
    qa2 = centre + np.abs(r.standard_normal(8))
    np.testing.assert_allclose(norm_term(K, q, qa2), kabs @ (qa2 - centre), atol=1e-12)


def test_norm_term_is_distance_free_and_scales():
    r = rng(111)
    K, q = r.standard_normal((7, 8)), r.standard_normal(8)
    qa = np.abs(q[0::2] + 1j * q[1::2]) * 1.3
    a = score_full(K, np.arange(7), q, qa, 100, 1e4, [1, 4])
    b = score_full(K, np.arange(7) + 50, q, qa, 150, 1e4, [1, 4])
    np.testing.assert_allclose(a, b, atol=1e-10)
    np.testing.assert_allclose(norm_term(3 * K, 2 * q, 2 * qa), 6 * norm_term(K, q, qa), atol=1e-12)


# --------------------------------------------------------------------------
# keys stored after RoPE (TriAttention blog, implementation walkthrough)
# --------------------------------------------------------------------------
from oracle import score_rotated  # noqa: E402


@pytest.mark.parametrize("d", [2, 8, 64])
def test_rotated_keys_score_like_pre_rope_keys(d):
    # scoring the stored rotated key directly gives the pre-RoPE score (the blog's two routes agree)
    r = rng(120, d)
    K, pos, q = r.standard_normal((11, d)), r.integers(0, 30000, 11), r.standard_normal(d)
    qa = np.abs(q[0::2] + 1j * q[1::2]) * 1.2
    D = [1, 4, 64, 1024]
    np.testing.assert_allclose(score_rotated(rope_rotate(K, pos, 1e6), q, 31000, 1e6, D),
                               score_literal(K, pos, q, 31000, 1e6, D), atol=1e-10)
    np.testing.assert_allclose(score_rotated(rope_rotate(K, pos, 1e6), q, 31000, 1e6, D, qabs=qa),
                               score_full(K, pos, q, qa, 31000, 1e6, D), atol=1e-10)


def test_half_split_style_is_a_coordinate_permutation():
    # the half-split layout is the interleaved one with coordinates permuted (band f at f and f+d/2)
    d = 16
    r = rng(121)
    K, q = r.standard_normal((6, d)), r.standard_normal(d)
    perm = np.empty(d, np.int64)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2          # interleaved[i] = half[perm[i]]
    D = [1, 2, 3]
    np.testing.assert_allclose(score_rotated(K, q, 777, 1e4, D, style="half"),
                               score_rotated(K[:, perm], q[perm], 777, 1e4, D), atol=1e-12)
    np.testing.assert_allclose(rope_rotate(K, 5, 1e4, "half")[:, perm], rope_rotate(K[:, perm], 5, 1e4), atol=1e-12)
    # d=2: both styles pair the same two coordinates
    np.testing.assert_allclose(rope_rotate(K[:, :2], 9, 1e4, "half"), rope_rotate(K[:, :2], 9, 1e4), atol=1e-15)


def test_rotated_closed_form():
    # d=2, stored key = RoPE((1,0), p) at p = 2, query centre (1,0), t = 5, D={0}: cos(5 - 2)
    k = rope_rotate(np.array([[1.0, 0.0]]), 2, 1e4)
    assert score_rotated(k, [1.0, 0.0], 5, 1e4, [0])[0] == pytest.approx(np.cos(3.0), abs=1e-14)


# --------------------------------------------------------------------------
# GQA: z-score per query head, then max (TriAttention summary 3.4, GQA)
# --------------------------------------------------------------------------
from oracle import score_gqa, zscore  # noqa: E402


def test_zscore_hand_example():
    z = zscore([1.0, 2.0, 3.0])                      # mean 2, population std sqrt(2/3)
    np.testing.assert_allclose(z, [-np.sqrt(1.5), 0.0, np.sqrt(1.5)], atol=1e-15)
    assert np.all(zscore([4.0, 4.0, 4.0]) == 0.0)     # no spread: no preference


def test_gqa_single_query_head_keeps_the_ranking():
    r = rng(130)
    K, q = r.standard_normal((50, 16)), r.standard_normal((1, 16))
    final, per = score_gqa(K, None, q, 60, 1e4, [1, 8])
    assert np.array_equal(np.argsort(final, kind="stable"), np.argsort(per[0], kind="stable"))
    np.testing.assert_allclose(per[0], score_literal(K, None, q[0], 60, 1e4, [1, 8]), atol=1e-12)


def test_gqa_is_scale_free_per_query_head():
    # each query head is normalised separately: rescaling one head's centre changes nothing
    r = rng(131)
    K, q = r.standard_normal((40, 8)), r.standard_normal((3, 8))
    a, _ = score_gqa(K, None, q, 90, 1e4, [1, 2, 4])
    q2 = q * np.array([[10.0], [0.01], [3.0]])
    b, _ = score_gqa(K, None, q2, 90, 1e4, [1, 2, 4])
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_gqa_max_over_heads():
    r = rng(132)
    K, q = r.standard_normal((30, 8)), r.standard_normal((4, 8))
    final, per = score_gqa(K, None, q, 40, 1e4, [1])
    z = np.stack([(p - p.mean()) / p.std() for p in per])
    np.testing.assert_allclose(final, z.max(0), atol=1e-12)
    # duplicating a query head changes nothing
    f2, _ = score_gqa(K, None, np.concatenate([q, q[:1]]), 40, 1e4, [1])
    np.testing.assert_allclose(final, f2, atol=1e-15)


from oracle import score_gqa_rotated  # noqa: E402


@pytest.mark.parametrize("with_norm", [False, True])
def test_gqa_over_rotated_keys_equals_gqa_over_pre_rope_keys(with_norm):
    # the grouped-query rule over stored rotated keys reproduces the rule over the pre-RoPE keys at
    # their positions (relative-position identity), per query head and after the z-score + max
    d, G = 16, 3
    r = rng(125, int(with_norm))
    K, pos = r.standard_normal((40, d)), np.sort(r.integers(0, 5000, 40))
    qg = r.standard_normal((G, d))
    qa = np.abs(qg[:, 0::2] + 1j * qg[:, 1::2]) * 1.3 if with_norm else None
    D = [1, 8, 512]
    z_rot, s_rot = score_gqa_rotated(rope_rotate(K, pos, 1e4), qg, 5100, 1e4, D, qabs_g=qa)
    z_pre, s_pre = score_gqa(K, pos, qg, 5100, 1e4, D, qabs_g=qa)
    np.testing.assert_allclose(s_rot, s_pre, atol=1e-10)
    np.testing.assert_allclose(z_rot, z_pre, atol=1e-9)


def test_gqa_over_rotated_keys_half_split_is_a_permutation():
    d, G = 12, 2
    r = rng(126)
    K, qg = r.standard_normal((25, d)), r.standard_normal((G, d))
    perm = np.empty(d, np.int64)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    zh, sh = score_gqa_rotated(K, qg, 300, 1e6, [1, 2], style="half")
    zi, si = score_gqa_rotated(K[:, perm], qg[:, perm], 300, 1e6, [1, 2])
    np.testing.assert_allclose(sh, si, atol=1e-12)
    np.testing.assert_allclose(zh, zi, atol=1e-12)
