"""Pins of the Video Delta Attention oracle (oracle/vda.py).

FreeVideo page, section "Where Video DeltaNet comes in": each frame's write is
the solution of a joint least-squares problem, S_t = (Sbar_t + B_t)(I + A_t)^-1;
forward and reverse scans seeded with S_text / 2; the carried-over part cannot
grow (||Diag(alpha)(I + A)^-1|| <= 1).
"""

import numpy as np
import pytest
from scipy.optimize import minimize

import oracle
from oracle import vda as D


def unit_rows(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def small_problem(seed, n=5, dv=3, dk=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((dv, dk)), rng.standard_normal((n, dk)), rng.standard_normal((n, dv)),
            rng.uniform(0.1, 0.9, n), rng.uniform(0.5, 1.0, dk))


def objective(s, sbar, k, v, beta):
    """1/2 ||S - Sbar||^2 + 1/2 sum_u beta_u ||S k_u - v_u||^2, token by token."""
    j = 0.5 * float(np.sum((s - sbar) ** 2))
    for u in range(k.shape[0]):
        r = s @ k[u] - v[u]
        j += 0.5 * beta[u] * float(r @ r)
    return j


def check_least_squares(update):
    for seed in range(4):
        s_prev, k, v, beta, alpha = small_problem(seed)
        sbar = s_prev * alpha[None, :]
        s = update(s_prev, k, v, beta, alpha)
        # stationarity, written token by token
        grad = s - sbar
        for u in range(k.shape[0]):
            grad = grad + beta[u] * np.outer(s @ k[u] - v[u], k[u])
        assert np.abs(grad).max() < 1e-12
        # an independent minimizer agrees
        res = minimize(lambda x: objective(x.reshape(s.shape), sbar, k, v, beta), np.zeros(s.size),
                       method="BFGS", options={"gtol": 1e-12})
        np.testing.assert_allclose(res.x.reshape(s.shape), s, rtol=0, atol=1e-6)


def check_delta_rule(update):
    """One unit key: (I + b k k^T)^-1 = I - b/(1+b) k k^T, the classic delta rule."""
    rng = np.random.default_rng(5)
    for _ in range(3):
        s_prev = rng.standard_normal((6, 8))
        k = unit_rows(rng, 1, 8)
        v = rng.standard_normal((1, 6))
        b = rng.uniform(0.1, 2.0)
        alpha = rng.uniform(0.5, 1.0, 8)
        sbar = s_prev * alpha[None, :]
        want = sbar + (b / (1 + b)) * np.outer(v[0] - sbar @ k[0], k[0])
        np.testing.assert_allclose(update(s_prev, k, v, np.array([b]), alpha), want, rtol=0, atol=1e-12)


def check_contraction(update):
    rng = np.random.default_rng(6)
    for _ in range(5):
        s_prev = rng.standard_normal((16, 16))
        k = unit_rows(rng, 40, 16)
        s = update(s_prev, k, np.zeros((40, 16)), rng.uniform(0, 1, 40), rng.uniform(0.3, 1.0, 16))
        assert np.linalg.norm(s, 2) <= np.linalg.norm(s_prev, 2) * (1 + 1e-12)


def check_order_invariance(update):
    s_prev, k, v, beta, alpha = small_problem(7, n=9)
    p = np.random.default_rng(8).permutation(9)
    np.testing.assert_allclose(update(s_prev, k[p], v[p], beta[p], alpha),
                               update(s_prev, k, v, beta, alpha), rtol=0, atol=1e-13)


def scan_case(seed, F=7, ft=6, d=8):
    rng = np.random.default_rng(seed)
    k = unit_rows(rng, F * ft, d)
    v = rng.standard_normal((F * ft, d))
    beta = rng.uniform(0.05, 0.95, F * ft)
    alpha = rng.uniform(0.8, 1.0, (F, d))
    s_text = 0.3 * rng.standard_normal((d, d))
    return k, v, beta, alpha, s_text, ft


def check_scans(scan):
    k, v, beta, alpha, s_text, ft = scan_case(9)
    F = alpha.shape[0]
    fwd, rev = scan(k, v, beta, alpha, s_text, ft)
    assert np.array_equal(fwd[0], s_text / 2) and np.array_equal(rev[F], s_text / 2)
    # explicit recurrences
    s = s_text / 2
    for t in range(F):
        if 1 <= t <= F - 2:
            sl = slice(t * ft, (t + 1) * ft)
            s = D.frame_update(s, k[sl], v[sl], beta[sl], alpha[t])
        np.testing.assert_allclose(fwd[t + 1], s, rtol=0, atol=1e-13)
    # the reverse scan is the forward scan of the time-reversed frames
    order = np.concatenate([np.arange(t * ft, (t + 1) * ft) for t in range(F - 1, -1, -1)])
    fr, _ = scan(k[order], v[order], beta[order], alpha[::-1], s_text, ft)
    for t in range(F + 1):
        np.testing.assert_allclose(rev[t], fr[F - t], rtol=0, atol=1e-13)
    # anchor frames are never written
    k2, v2 = k.copy(), v.copy()
    k2[:ft] = unit_rows(np.random.default_rng(10), ft, k.shape[1])
    v2[-ft:] += 5.0
    f2, r2 = scan(k2, v2, beta, alpha, s_text, ft)
    np.testing.assert_allclose(f2, fwd, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r2, rev, rtol=0, atol=1e-13)


def check_readout_complement(positions):
    """The frames a query's two states have absorbed are exactly the frames its
    softmax window does not reach, anchors excepted."""
    for F, ch, nb in [(72, 5, 1), (42, 5, 1), (13, 2, 1), (9, 3, 0), (20, 5, 2)]:
        lo, hi = positions(F, ch, nb)
        allowed = oracle.window_frames_allowed(F, ch, nb)
        for f in range(F):
            absorbed = set(range(1, lo[f])) | set(range(hi[f], F - 1))
            want = {g for g in range(1, F - 1) if not allowed[f, g]}
            assert absorbed == want, (F, ch, nb, f)


def check_readout(attn):
    rng = np.random.default_rng(11)
    H, F, ft, d = 2, 12, 5, 8
    q = np.stack([unit_rows(rng, F * ft, d) for _ in range(H)])
    k = np.stack([unit_rows(rng, F * ft, d) for _ in range(H)])
    v = rng.standard_normal((H, F * ft, d))
    beta = rng.uniform(0.05, 0.95, (H, F * ft))
    alpha = rng.uniform(0.8, 1.0, (H, F, d))
    s_text = 0.3 * rng.standard_normal((H, d, d))
    out = attn(q, k, v, beta, alpha, s_text, ft, 3, 1)
    # anchor-frame queries read the two seeds: S_text q
    for f in (0, F - 1):
        sl = slice(f * ft, (f + 1) * ft)
        for h in range(H):
            np.testing.assert_allclose(out[h, sl], q[h, sl] @ s_text[h].T, rtol=0, atol=1e-13)
    # no writes and no decay: every query reads S_text q
    still = attn(q, k, v, np.zeros_like(beta), np.ones_like(alpha), s_text, ft, 3, 1)
    for h in range(H):
        np.testing.assert_allclose(still[h], q[h] @ s_text[h].T, rtol=0, atol=1e-13)
    # explicit readout of one interior query
    fwd, rev = D.scan_states(k[1], v[1], beta[1], alpha[1], s_text[1], ft)
    f = 7                        # chunk 2 of 3-frame chunks: window frames 3..11, reads fwd[3], rev[12]
    i = f * ft + 2
    np.testing.assert_allclose(out[1, i], fwd[3] @ q[1, i] + rev[12] @ q[1, i], rtol=0, atol=1e-13)


def test_update_solves_least_squares():
    check_least_squares(D.frame_update)


def test_single_token_is_delta_rule():
    check_delta_rule(D.frame_update)


def test_carried_state_does_not_grow():
    check_contraction(D.frame_update)


def test_token_order_within_frame_is_irrelevant():
    check_order_invariance(D.frame_update)


def test_scans():
    check_scans(D.scan_states)


def test_readout_covers_complement_of_window():
    check_readout_complement(D.read_positions)


def test_readout():
    check_readout(D.vda_attention)


# ---------------------------------------------------------------- mutants

def _update_no_decay(s_prev, k, v, beta, alpha):
    return D.frame_update(s_prev, k, v, beta, np.ones_like(alpha))


def _update_left_decay(s_prev, k, v, beta, alpha):
    dv = s_prev.shape[0]          # decay on the value side instead of the key side
    return D.frame_update(alpha[:dv, None] * s_prev, k, v, beta, np.ones_like(alpha))


def _update_no_inverse(s_prev, k, v, beta, alpha):
    return s_prev * alpha[None, :] + (v * beta[:, None]).T @ k


@pytest.mark.parametrize("mut", [_update_no_decay, _update_left_decay, _update_no_inverse],
                         ids=lambda f: f.__name__)
def test_update_mutants_caught(mut):
    caught = 0
    for check in (check_least_squares, check_delta_rule, check_contraction):
        try:
            check(mut)
        except AssertionError:
            caught += 1
    assert caught >= 1


def _scan_absorbs_anchors(k, v, beta, alpha, s_text, ft):
    N, d = k.shape
    F = N // ft
    fwd = np.empty((F + 1, d, d))
    rev = np.empty((F + 1, d, d))
    fwd[0] = s_text / 2
    for t in range(F):
        sl = slice(t * ft, (t + 1) * ft)
        fwd[t + 1] = D.frame_update(fwd[t], k[sl], v[sl], beta[sl], alpha[t])
    rev[F] = s_text / 2
    for t in range(F - 1, -1, -1):
        sl = slice(t * ft, (t + 1) * ft)
        rev[t] = D.frame_update(rev[t + 1], k[sl], v[sl], beta[sl], alpha[t])
    return fwd, rev


def _scan_full_seed(k, v, beta, alpha, s_text, ft):
    return D.scan_states(k, v, beta, alpha, 2 * s_text, ft)


@pytest.mark.parametrize("mut", [_scan_absorbs_anchors, _scan_full_seed], ids=lambda f: f.__name__)
def test_scan_mutants_caught(mut):
    with pytest.raises(AssertionError):
        check_scans(mut)


def _positions_window_not_widened(frames, chunk_frames=5, neighbours=1):
    return D.read_positions(frames, chunk_frames, 0)


def _positions_anchor_rows_read_states(frames, chunk_frames=5, neighbours=1):
    lo, hi = D.read_positions(frames, chunk_frames, neighbours)
    lo[0], hi[0] = 0, min(frames, (neighbours + 1) * chunk_frames)
    return lo, hi


@pytest.mark.parametrize("mut", [_positions_window_not_widened, _positions_anchor_rows_read_states],
                         ids=lambda f: f.__name__)
def test_position_mutants_caught(mut):
    with pytest.raises(AssertionError):
        check_readout_complement(mut)
