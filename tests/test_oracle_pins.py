"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every check is a closed form, a
library routine (numpy / scipy), brute force, or an invariant the nystrom.rs
source page states in prose.  The numbered checks (1)-(5) are:
  (1) with no far keys the output is exact softmax attention;
  (2) sink = 0 gives the sink-free operator (near = last w keys, far = the rest);
  (3) far_len of each head equals the number of evictions, never a multiple;
  (4) when every far key is one of the landmark keys and lambda -> 0 the far
      field reproduces the exact exp weights (F M A = F), pinning M's
      [key landmark][query landmark] orientation;
  (5) the shifted streaming form equals the unshifted formula of the module doc.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers --

def rand_prompt(rng, hpk, T, d, dv, qstd=1.0, kstd=1.0):
    qs = (qstd * rng.standard_normal((hpk, T, d))).astype(np.float32)
    ks = (kstd * rng.standard_normal((T, d))).astype(np.float32)
    vs = rng.standard_normal((T, dv)).astype(np.float32)
    return qs, ks, vs


def softmax_attention(q, K, V, scale):
    """Exact attention from scipy's softmax (library routine), f64."""
    w = softmax(K.astype(np.float64) @ q.astype(np.float64) * scale)
    return w @ V.astype(np.float64)


def direct_output(q, K, V, p, S, w, kt, qt, mu, scale, rect):
    """The module-doc formula of the nystrom.rs source page evaluated directly,
    with raw (unshifted) exponentials, for the query at absolute position p
    after keys 0..p have been seen:
        near = {j : p - j < w} u {j < S},  far = {S <= j <= p - w}
        out  = (sum_near e_j v_j + FM . T_far) / (sum_near e_j + FM . Z_far)
    with FM = F M, the far field dropped when FM . Z_far < 0 (Aggregate) or
    FM clamped at 0 first (Fm)."""
    q = q.astype(np.float64)
    K = K[: p + 1].astype(np.float64)
    V = V[: p + 1].astype(np.float64)
    j = np.arange(p + 1)
    near = (p - j < w) | (j < S)
    far = (j >= S) & (p - j >= w)
    e = np.exp(K[near] @ q * scale)
    num = e @ V[near]
    den = e.sum()
    if far.any():
        F = np.exp(kt.astype(np.float64) @ q * scale)
        FM = F @ mu.astype(np.float64)
        if rect == O.RECT_FM:
            FM = np.maximum(FM, 0.0)
        E = np.exp(qt.astype(np.float64) @ K[far].T * scale)
        far_den = FM @ E.sum(axis=1)
        if far_den >= 0:
            num = num + FM @ (E @ V[far])
            den = den + far_den
    return num / den


def run_group(rng, hpk, T, d, dv, m, w, S, steps, rect=O.RECT_AGGREGATE, qstd=1.0, kstd=1.0):
    """Prefill + `steps` decode steps; returns (group, all q, all K, all V, outputs)."""
    qs, ks, vs = rand_prompt(rng, hpk, T, d, dv, qstd, kstd)
    g = O.Group(m, w, S, hpk, rect)
    g.prefill(qs, ks, vs)
    Q = [qs[:, j, :] for j in range(T)]
    K, V, outs = list(ks), list(vs), []
    for _ in range(steps):
        q = (qstd * rng.standard_normal((hpk, d))).astype(np.float32)
        k = (kstd * rng.standard_normal(d)).astype(np.float32)
        v = rng.standard_normal(dv).astype(np.float32)
        outs.append(g.step(q, k, v))
        Q.append(q)
        K.append(k)
        V.append(v)
    return g, np.array(Q), np.array(K), np.array(V), np.array(outs)


def rel_err(a, b):
    return np.max(np.abs(a - b)) / np.linalg.norm(b)


# ------------------------------------------------------------- constants --

def test_constants_match_pages():
    c = json.load(open(os.path.join(GOLDEN, "constants.json")))
    assert O.RIDGE_REL == c["RIDGE_REL"]
    assert O.DEN_EPS == c["DEN_EPS"]
    assert O.EXACT_SLACK == c["EXACT_SLACK"]
    assert O.RIDGE_TRIES == c["RIDGE_TRIES"]


def test_m_eff_and_exact_only_rule():
    c = json.load(open(os.path.join(GOLDEN, "constants.json")))
    rng = np.random.default_rng(3)
    for t, m, expect in c["m_eff_examples"]:
        qs, ks, vs = rand_prompt(rng, 1, t, 8, 8)
        g = O.Group(m, 4, 0, 1)
        g.prefill(qs, ks, vs)
        assert not g.exact_only
        assert g.m_eff == expect, (t, m)
    # exact-only exactly when t <= w + sink + EXACT_SLACK
    for w, S in [(16, 2), (4, 0), (128, 4)]:
        for t, expect in [(w + S + 8, True), (w + S + 9, False)]:
            qs, ks, vs = rand_prompt(rng, 1, t, 8, 8)
            g = O.Group(8, w, S, 1)
            g.prefill(qs, ks, vs)
            assert g.exact_only == expect


def test_invalid_settings_rejected():
    for args in [(3, 16, 2, 1), (8, 0, 2, 1), (8, 16, 2, 0), (8, 16, -1, 1)]:
        with pytest.raises(ValueError):
            O.Group(*args)


# -------------------------------------------------------------- seg_means --

def test_seg_means_ramp_closed_form():
    # t = 10, m = 4: segments [0,2) [2,5) [5,7) [7,10) by floor(i*t/m);
    # row j holds j + 100 c, so segment means are (lo + hi - 1)/2 + 100 c.
    t, d = 10, 3
    xs = (np.arange(t)[:, None] + 100.0 * np.arange(d)[None, :]).astype(np.float32)
    got = O.seg_means(xs, 4)
    expect = np.array([0.5, 3.0, 5.5, 8.0])[:, None] + 100.0 * np.arange(d)[None, :]
    np.testing.assert_array_equal(got, expect)


def test_seg_means_mass_and_constant_segments():
    rng = np.random.default_rng(1)
    for t, m in [(37, 5), (256, 32), (64, 8), (101, 12)]:
        xs = rng.standard_normal((t, 4)).astype(np.float32)
        got = O.seg_means(xs, m)
        sizes = np.array([(i + 1) * t // m - i * t // m for i in range(m)])
        assert sizes.sum() == t and sizes.min() >= 1
        np.testing.assert_allclose((sizes[:, None] * got).sum(0), xs.astype(np.float64).sum(0),
                                   rtol=0, atol=1e-12)
        # piecewise-constant rows give back the constants
        consts = rng.standard_normal((m, 4)).astype(np.float32)
        rows = np.repeat(consts, sizes, axis=0)
        np.testing.assert_allclose(O.seg_means(rows, m), consts.astype(np.float64), rtol=1e-15)


# --------------------------------------------------------------- cholesky --

def test_cholesky_matches_numpy():
    rng = np.random.default_rng(2)
    for n in (4, 8, 32, 64):
        a = rng.standard_normal((n, n))
        g = a.T @ a + n * np.eye(n)
        L = O.cholesky(g)
        np.testing.assert_allclose(L, np.linalg.cholesky(g), rtol=1e-12, atol=1e-12)


def test_cholesky_rejects_non_pd():
    assert O.cholesky(np.array([[1.0, 2.0], [2.0, 1.0]])) is None        # indefinite
    assert O.cholesky(np.zeros((3, 3))) is None                           # zero pivot
    assert O.cholesky(np.array([[np.nan, 0.0], [0.0, 1.0]])) is None      # not finite
    assert O.cholesky(np.array([[1.0, 0.0], [0.0, 0.0]])) is None


# ------------------------------------------------------------- ridge_pinv --

def _exp_gram(rng, m, d, std):
    qt = std * rng.standard_normal((m, d))
    kt = std * rng.standard_normal((m, d))
    return np.exp(qt @ kt.T / np.sqrt(d))


@pytest.mark.parametrize("m,std", [(8, 0.3), (32, 0.25), (64, 0.2)])
def test_ridge_pinv_matches_library(m, std):
    rng = np.random.default_rng(m)
    a = _exp_gram(rng, m, 128, std)
    M, lam, tries = O.ridge_pinv(a)
    G = a.T @ a
    lam_ref = O.RIDGE_REL * np.mean(np.diag(G))
    assert tries == 1
    assert lam == pytest.approx(lam_ref, rel=1e-14)
    # normal equations (library solve) and the SVD form of the same operator
    ref = np.linalg.solve(G + lam_ref * np.eye(m), a.T)
    U, s, Vt = np.linalg.svd(a)
    ref_svd = Vt.T @ np.diag(s / (s * s + lam_ref)) @ U.T
    scale = np.linalg.norm(ref)
    assert np.linalg.norm(M - ref) / scale < 1e-8
    assert np.linalg.norm(M - ref_svd) / scale < 1e-8
    # residual bound in exact arithmetic: ||AMA - A||_F <= sqrt(RIDGE_REL)/2 ||A||_F
    res = np.linalg.norm(a @ M @ a - a) / np.linalg.norm(a)
    assert res <= 0.5 * np.sqrt(O.RIDGE_REL) * (1 + 1e-6)


def test_ridge_pinv_fallback_paths():
    # An exactly zero pivot with no ridge never factors: all 12 attempts fail
    # and the result is diag(1 / mean diag(A^T A)).
    a = np.array([[1.0, 0.0], [0.0, 0.0]])
    M, lam, tries = O.ridge_pinv(a, ridge_rel=0.0)
    assert tries == O.RIDGE_TRIES + 1
    np.testing.assert_array_equal(M, np.diag([2.0, 2.0]))
    # A non-finite matrix: mean diag falls back to DBL_MIN as well.
    a = np.array([[np.nan, 1.0], [1.0, 1.0]])
    M, lam, tries = O.ridge_pinv(a)
    assert tries == O.RIDGE_TRIES + 1
    np.testing.assert_array_equal(np.diag(M), [1.0 / np.finfo(np.float64).tiny] * 2)


def test_ridge_pinv_grows_lambda_tenfold():
    # Rank-1 A: the pivots of A^T A after the first are rounding noise, some
    # negative; a ridge far below the noise fails until it has grown past it.
    found = False
    for seed in range(200):
        rng = np.random.default_rng(seed)
        u, v = rng.standard_normal(6), rng.standard_normal(6)
        a = np.outer(u, v)
        M, lam, tries = O.ridge_pinv(a, ridge_rel=1e-22)
        if not (1 < tries <= O.RIDGE_TRIES):
            continue
        found = True
        G = a.T @ a
        lam_ref = 1e-22 * np.mean(np.diag(G))
        for _ in range(tries - 1):
            lam_ref *= 10.0
        assert lam == lam_ref
        assert O.cholesky(G + (lam / 10.0) * np.eye(6)) is None       # the attempt before failed
        assert O.cholesky(G + lam * np.eye(6)) is not None
        r = (G + lam * np.eye(6)) @ M - a.T
        assert np.linalg.norm(r) / np.linalg.norm(a) < 1e-6
        break
    assert found, "no seed exercised the ridge growth"


def zero_one_gram_case(m=16):
    """A 0/1 matrix A (m = 16) whose A^T A has a rank-deficient 2x2 block: columns
    0 and 1 of A are both e_0, row 1 is empty, and column j >= 2 is e_j.  Then
    A^T A has ones on the diagonal, ones at (0, 1) and (1, 0), zeros elsewhere,
    and tr(A^T A) / m = 1 exactly."""
    a = np.zeros((m, m))
    a[0, 0] = a[0, 1] = 1.0
    for j in range(2, m):
        a[j, j] = 1.0
    return a


def test_ridge_pinv_retry_fixed_by_rounding():
    # IEEE arithmetic fixes the attempt: while lambda <= 2^-53, 1 + lambda rounds
    # to 1, so the second pivot of the block [[1, 1], [1, 1]] is 1 - 1*1 = 0
    # exactly and the factorisation fails.  With ridge_rel = 8e-19 the ridges are
    # 8e-19, 8e-18, 8e-17 (all below 2^-53 ~ 1.11e-16), then 8e-16: attempt 4
    # factors, with a pivot of about 2 * 4 * 2^-52.
    a = zero_one_gram_case()
    M, lam, tries = O.ridge_pinv(a, ridge_rel=8e-19)
    assert tries == 4
    assert lam == 8e-19 * 10.0 * 10.0 * 10.0
    G = a.T @ a + lam * np.eye(16)
    ref = np.linalg.solve(G, a.T)
    assert np.linalg.norm(M - ref) / np.linalg.norm(ref) < 1e-9
    # the ridge of attempt 3 is lost when added to 1, that of attempt 4 is not
    assert 1.0 + lam / 10.0 == 1.0 and 1.0 + lam > 1.0
    assert O.cholesky(a.T @ a + (lam / 10.0) * np.eye(16)) is None


# ------------------------------------------------------------ memory_bytes --

def _state_words(st):
    return sum(int(np.asarray(st[k]).size) for k in
               ("sink_k", "sink_v", "win_k", "win_v", "k_tilde", "q_tilde", "mu", "t_hat",
                "z_hat", "m_max") if k in st)


@pytest.mark.parametrize("hpk,T,d,dv,m,w,S", [(2, 256, 128, 128, 32, 128, 4),
                                             (3, 100, 64, 32, 16, 24, 0),
                                             (1, 64, 64, 64, 8, 16, 2)])
def test_memory_bytes_skeleton_counts_state_vectors(hpk, T, d, dv, m, w, S):
    # NystromState::memory_bytes counts f32 words of the window (w rows), sinks,
    # K~, and per head T^, Z^, running max, Q~, M plus the score scratch (sink + w)
    # and three m-vectors of scratch.  The state arrays' own sizes give all but
    # the scratch; the count does not change while stepping.
    rng = np.random.default_rng(T + hpk)
    g, *_ = run_group(rng, hpk, T, d, dv, m, w, S, steps=0)
    st = g.state()
    me = st["m_eff"]
    expect = 4 * (_state_words(st) + hpk * ((S + w) + 3 * me))
    assert g.memory_bytes() == expect
    for _ in range(3):
        g.step(rng.standard_normal((hpk, d)).astype(np.float32),
               rng.standard_normal(d).astype(np.float32), rng.standard_normal(dv).astype(np.float32))
        assert g.memory_bytes() == expect


def test_memory_bytes_qwen3_layer_group_by_hand():
    # One group of the Qwen3-0.6B-shaped layer (d = dv = 128, m = 32, w = 128,
    # sink = 4, two query heads), counted field by field from the page's lists:
    #   shared  128*256 (window) + 4*256 (sinks) + 32*128 (K~)        = 37 888 words
    #   head    32*128 (T^) + 32 (Z^) + 32 (max) + 32*128 (Q~) + 32*32 (M)
    #           + 132 (score scratch) + 3*32 (other scratch)           =  9 508 words
    #   total   37 888 + 2 * 9 508 = 56 904 words = 227 616 bytes
    rng = np.random.default_rng(5)
    g, *_ = run_group(rng, 2, 256, 128, 128, 32, 128, 4, steps=2)
    assert g.memory_bytes() == 227_616


def test_memory_bytes_exact_only_counts_lengths():
    # Exact-only (seal_exact): the window holds every key by length (not by the
    # capacity reserved for growth); each head's score scratch is reserved but
    # empty until the first step, then holds one entry per key.  No sinks, K~ or
    # skeleton vectors.  A group never prefilled holds nothing.
    hpk, T, d, dv, w, S = 3, 20, 64, 32, 16, 2
    rng = np.random.default_rng(9)
    g = O.Group(8, w, S, hpk)
    assert g.memory_bytes() == 0
    qs, ks, vs = rand_prompt(rng, hpk, T, d, dv)
    g.prefill(qs, ks, vs)
    assert g.exact_only
    assert g.memory_bytes() == 4 * T * (d + dv)
    for s in range(1, 40):  # the window grows past its first reserved capacity
        g.step(rng.standard_normal((hpk, d)).astype(np.float32),
               rng.standard_normal(d).astype(np.float32), rng.standard_normal(dv).astype(np.float32))
        n = T + s
        assert g.win_len == n
        assert g.memory_bytes() == 4 * (n * (d + dv) + hpk * n)


# ------------------------------------------------------- exact attention --

def test_exact_attention_matches_scipy():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(16).astype(np.float32)
    K = (3 * rng.standard_normal((50, 16))).astype(np.float32)
    V = rng.standard_normal((50, 8)).astype(np.float32)
    got = O.exact_attention(q, K, V, 0.25)
    np.testing.assert_allclose(got, softmax_attention(q, K, V, 0.25), rtol=1e-12, atol=1e-14)


# --------------------------------------------------------- (1) no far keys --

def test_check1_exact_only_prompt_is_exact_softmax():
    rng = np.random.default_rng(10)
    hpk, d, dv, m, w, S = 2, 16, 8, 8, 16, 2
    T = w + S + 8                       # exact-only: every key stays exact
    g, Q, K, V, outs = run_group(rng, hpk, T, d, dv, m, w, S, steps=40)
    assert g.exact_only and g.far_len(0) == 0
    for i in range(40):
        p = T + i
        for h in range(hpk):
            ref = softmax_attention(Q[p][h], K[: p + 1], V[: p + 1], g.scale)
            assert rel_err(outs[i][h], ref) < 1e-13


def test_check1_replay_before_first_eviction_is_exact_softmax():
    rng = np.random.default_rng(11)
    hpk, T, d, dv, m, w, S = 2, 64, 16, 8, 8, 16, 2
    qs, ks, vs = rand_prompt(rng, hpk, T, d, dv)
    g = O.Group(m, w, S, hpk)
    rep = g.prefill(qs, ks, vs, replay_outputs=True)
    assert not g.exact_only
    for j in range(S, S + w):           # ring not yet full: no far key exists
        for h in range(hpk):
            ref = softmax_attention(qs[h, j], ks[: j + 1], vs[: j + 1], g.scale)
            assert rel_err(rep[j, h], ref) < 1e-13
    # the first eviction makes the output differ from exact attention
    j = S + w
    assert rel_err(rep[j, 0], softmax_attention(qs[0, j], ks[: j + 1], vs[: j + 1], g.scale)) > 1e-6


# ------------------------------------------------- (2) sink=0, (5) shifts --

@pytest.mark.parametrize("S", [0, 4])
@pytest.mark.parametrize("rect", [O.RECT_AGGREGATE, O.RECT_FM])
def test_check2_check5_streaming_equals_direct_formula(S, rect):
    rng = np.random.default_rng(20 + S + 7 * rect)
    hpk, T, d, dv, m, w = 2, 96, 32, 16, 8, 16
    g, Q, K, V, outs = run_group(rng, hpk, T, d, dv, m, w, S, steps=60, rect=rect)
    st = g.state()
    worst = 0.0
    for i in range(60):
        p = T + i
        for h in range(hpk):
            ref = direct_output(Q[p][h], K, V, p, S, w, st["k_tilde"], st["q_tilde"][h],
                                st["mu"][h], g.scale, rect)
            worst = max(worst, rel_err(outs[i][h], ref))
    assert worst < 1e-9, worst


def test_check5_larger_logits_still_match_direct():
    # std-3 queries and keys: far logits reach tens, running maxima grow often.
    rng = np.random.default_rng(25)
    hpk, T, d, dv, m, w, S = 2, 128, 32, 16, 16, 32, 4
    g, Q, K, V, outs = run_group(rng, hpk, T, d, dv, m, w, S, steps=50, qstd=2.0, kstd=2.0)
    st = g.state()
    worst = 0.0
    for i in range(50):
        p = T + i
        for h in range(hpk):
            ref = direct_output(Q[p][h], K, V, p, S, w, st["k_tilde"], st["q_tilde"][h],
                                st["mu"][h], g.scale, O.RECT_AGGREGATE)
            worst = max(worst, rel_err(outs[i][h], ref))
    assert worst < 1e-8, worst


# ----------------------------------------------------------- (3) far_len --

def test_check3_far_len_counts_evictions_once_per_head():
    rng = np.random.default_rng(30)
    hpk, T, d, dv, m, w, S = 3, 80, 16, 8, 8, 16, 2
    qs, ks, vs = rand_prompt(rng, hpk, T, d, dv)
    g = O.Group(m, w, S, hpk)
    g.prefill(qs, ks, vs)
    E = T - S - w
    assert [g.far_len(h) for h in range(hpk)] == [E] * hpk
    assert g.win_head == E % w and g.win_len == w
    for i in range(1, 41):
        g.step(rng.standard_normal((hpk, d)).astype(np.float32),
               rng.standard_normal(d).astype(np.float32), rng.standard_normal(dv).astype(np.float32))
        assert [g.far_len(h) for h in range(hpk)] == [E + i] * hpk
        assert g.win_head == (E + i) % w


# ------------------------------------------------- ring and sink placement --

def test_ring_and_sink_contents_bit_exact():
    rng = np.random.default_rng(31)
    hpk, T, d, dv, m, w, S = 2, 100, 16, 8, 8, 24, 3
    g, Q, K, V, outs = run_group(rng, hpk, T, d, dv, m, w, S, steps=37)
    st = g.state()
    p_last = T + 37 - 1
    np.testing.assert_array_equal(st["sink_k"], K[:S])
    np.testing.assert_array_equal(st["sink_v"], V[:S])
    for p in range(p_last - w + 1, p_last + 1):
        slot = (p - S) % w
        np.testing.assert_array_equal(st["win_k"][slot], K[p])
        np.testing.assert_array_equal(st["win_v"][slot], V[p])


# ------------------------------------------------------- prefill landmarks --

def test_prefill_landmarks_and_gram():
    rng = np.random.default_rng(32)
    hpk, T, d, dv, m, w, S = 2, 200, 16, 8, 32, 32, 4
    qs, ks, vs = rand_prompt(rng, hpk, T, d, dv)
    g = O.Group(m, w, S, hpk)
    g.prefill(qs, ks, vs)
    st = g.state()
    me = g.m_eff
    assert me == 25
    bounds = [(i * T // me, (i + 1) * T // me) for i in range(me)]
    kt_ref = np.array([ks[lo:hi].astype(np.float64).mean(0) for lo, hi in bounds])
    np.testing.assert_allclose(st["k_tilde"], kt_ref.astype(np.float32), rtol=1e-6, atol=1e-7)
    kt64, qt64 = g.landmarks64()
    np.testing.assert_allclose(kt64, kt_ref, rtol=1e-13, atol=1e-15)
    for h in range(hpk):
        qt_ref = np.array([qs[h, lo:hi].astype(np.float64).mean(0) for lo, hi in bounds])
        np.testing.assert_allclose(qt64[h], qt_ref, rtol=1e-13, atol=1e-15)
        au_ref = np.exp(qt64[h] @ kt64.T * g.scale)
        np.testing.assert_allclose(st["au"][h], au_ref, rtol=1e-13)


# ------------------------------------------------- far state after replay --

def test_replayed_far_state_equals_batched_closed_form():
    rng = np.random.default_rng(33)
    hpk, T, d, dv, m, w, S = 2, 300, 16, 8, 16, 32, 4
    qs, ks, vs = rand_prompt(rng, hpk, T, d, dv, qstd=2.0, kstd=2.0)
    g = O.Group(m, w, S, hpk)
    g.prefill(qs, ks, vs)
    st = g.state()
    far = np.arange(S, T - w)
    for h in range(hpk):
        L = st["q_tilde"][h].astype(np.float64) @ ks[far].astype(np.float64).T * g.scale
        mx = L.max(axis=1)
        E = np.exp(L - mx[:, None])
        np.testing.assert_allclose(st["m_max"][h], mx, rtol=1e-14)
        np.testing.assert_allclose(st["z_hat"][h], E.sum(1), rtol=1e-12)
        np.testing.assert_allclose(st["t_hat"][h], E @ vs[far].astype(np.float64), rtol=1e-10,
                                   atol=1e-12)
        assert g.far_len(h) == len(far)


# ------------------------------------------------------------- rectifier --

def test_rectifier_negative_mixing_drops_far_field():
    rng = np.random.default_rng(40)
    hpk, T, d, dv, m, w, S = 1, 64, 16, 8, 8, 16, 2
    qs, ks, vs = rand_prompt(rng, hpk, T, d, dv)
    me = 8
    for rect in (O.RECT_AGGREGATE, O.RECT_FM):
        g = O.Group(m, w, S, hpk, rect)
        g.prefill(qs, ks, vs, frozen=O.Frozen(mu=-np.eye(me, dtype=np.float32)[None]))
        q = rng.standard_normal((1, d)).astype(np.float32)
        k = rng.standard_normal(d).astype(np.float32)
        v = rng.standard_normal(dv).astype(np.float32)
        out, alt, diags = g.step(q, k, v, with_alt=True)
        st = g.state()
        near_k = np.concatenate([st["sink_k"], st["win_k"]])
        near_v = np.concatenate([st["sink_v"], st["win_v"]])
        ref = softmax_attention(q[0], near_k, near_v, g.scale)
        assert rel_err(out[0], ref) < 1e-13
        if rect == O.RECT_AGGREGATE:
            assert diags[0].far_den < 0 and diags[0].keep == 0
        else:                               # Fm clamps u to 0: far_den = 0 keeps (R5)
            assert diags[0].far_den == 0.0 and diags[0].keep == 1


# ------------------------------------------------------ (4) Nystrom identity --

def _identity_case(rng, m=8, d=8, hpk=2, w=8, S=0, std=0.9):
    T = 8 * m                              # segments of 8 rows: exact f64 means
    kappa = (std * rng.standard_normal((m, d))).astype(np.float32)
    rho = (std * rng.standard_normal((hpk, m, d))).astype(np.float32)
    ks = np.repeat(kappa, 8, axis=0)
    qs = np.repeat(rho, 8, axis=1)
    vs = rng.standard_normal((T, 4)).astype(np.float32)
    return T, kappa, rho, qs, ks, vs


def _identity_error(ridge_rel, transpose_mu=False, seed=50):
    rng = np.random.default_rng(seed)
    m, hpk, w, S = 8, 2, 8, 0
    T, kappa, rho, qs, ks, vs = _identity_case(rng, m=m, hpk=hpk, w=w, S=S)
    g = O.Group(m, w, S, hpk)
    g.set_ridge_rel(ridge_rel)
    g.prefill(qs, ks, vs)
    st = g.state()
    assert g.m_eff == m
    np.testing.assert_array_equal(st["k_tilde"], kappa)
    np.testing.assert_array_equal(st["q_tilde"], rho)
    for h in range(hpk):
        assert np.linalg.cond(st["au"][h]) < 1e3
        assert np.abs(st["au"][h] - st["au"][h].T).max() > 0.1   # non-symmetric
    if transpose_mu:
        g2 = O.Group(m, w, S, hpk)
        g2.prefill(qs, ks, vs, frozen=O.Frozen(mu=np.ascontiguousarray(st["mu"].transpose(0, 2, 1))))
        g = g2
    K, V = list(ks), list(vs)
    worst = 0.0
    for i in range(30):
        k = kappa[rng.integers(m)]               # every later key is a landmark key
        v = rng.standard_normal(4).astype(np.float32)
        q = (0.9 * rng.standard_normal((hpk, 8))).astype(np.float32)
        out = g.step(q, k, v)
        K.append(k)
        V.append(v)
        for h in range(hpk):
            ref = softmax_attention(q[h], np.array(K), np.array(V), g.scale)
            worst = max(worst, rel_err(out[h], ref))
    return worst


def test_check4_nystrom_identity_reproduces_exact_weights():
    e6, e10, e0 = _identity_error(1e-6), _identity_error(1e-10), _identity_error(0.0)
    # M is stored in f32, which floors the error near cond(A) * 2^-24.
    assert e0 < 2e-5 and e10 < 2e-5
    assert e6 < 5e-3
    assert e6 > 2 * e10                         # the error shrinks with lambda


def test_check4_transposed_mixing_matrix_fails():
    # A planted orientation mistake (M^T in place of M) must be caught.
    assert _identity_error(0.0, transpose_mu=True) > 1e-2


# --------------------------------------------------------------- GQA split --

def test_gqa_group_equals_single_head_groups_bitwise():
    rng = np.random.default_rng(60)
    hpk, T, d, dv, m, w, S = 3, 90, 16, 8, 8, 16, 2
    qs, ks, vs = rand_prompt(rng, hpk, T, d, dv)
    grp = O.Group(m, w, S, hpk)
    grp.prefill(qs, ks, vs)
    singles = []
    for h in range(hpk):
        s = O.Group(m, w, S, 1)
        s.prefill(qs[h:h + 1], ks, vs)
        singles.append(s)
    for _ in range(20):
        q = rng.standard_normal((hpk, d)).astype(np.float32)
        k = rng.standard_normal(d).astype(np.float32)
        v = rng.standard_normal(dv).astype(np.float32)
        out = grp.step(q, k, v)
        for h in range(hpk):
            np.testing.assert_array_equal(out[h], singles[h].step(q[h:h + 1], k, v)[0])


def test_reading_r7_dropped_far_uses_near_shift():
    # Far logits near 1000 and near logits near 0: the joint shift c_all sits
    # ~1000 above every near logit, beyond the f64 exp range.  When the
    # rectifier drops the far field, the output must still be the near softmax
    # (the module-doc formula is shift-invariant); shifting the near weights by
    # c_all would underflow all of them and return 0.
    rng = np.random.default_rng(70)
    d, dv, m, w, S, T = 16, 8, 8, 16, 2, 64
    kappa = np.ones(d, np.float32)
    ks = np.tile(kappa, (T, 1))
    vs = rng.standard_normal((T, dv)).astype(np.float32)
    qs = rng.standard_normal((1, T, d)).astype(np.float32)
    g = O.Group(m, w, S, 1)
    g.prefill(qs, ks, vs, frozen=O.Frozen(q_tilde=np.full((1, 8, d), 250.0, np.float32),
                                          mu=-np.eye(8, dtype=np.float32)[None]))
    st = g.state()
    assert st["m_max"].min() > 900.0
    q = (0.5 * rng.standard_normal((1, d))).astype(np.float32)
    k = rng.standard_normal(d).astype(np.float32)
    v = rng.standard_normal(dv).astype(np.float32)
    out, alt, diags = g.step(q, k, v, with_alt=True)
    assert diags[0].keep == 0
    st = g.state()
    near_k = np.concatenate([st["sink_k"], st["win_k"]])
    near_v = np.concatenate([st["sink_v"], st["win_v"]])
    ref = softmax_attention(q[0], near_k, near_v, g.scale)
    assert rel_err(out[0], ref) < 1e-13
