"""Planted mistakes in copies of the oracle must fail the pins (CPU only).

Each mutant is a plausible slip (a dropped term, a wrong axis, sign, index or
divisor, a transposed operand, the wrong tie rule).  The pins in
test_oracle_pins.py are only worth something if they catch these.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import attention as A
import test_oracle_pins as P


# ---------------------------------------------------------------- dense mutants

def _dense_from_rows(rows_fn):
    def dense(q, k, v, scale, rows=None):
        H, N, d = q.shape
        return np.stack([rows_fn(q[h], k[h], v[h], scale) for h in range(H)])
    return dense


def _rows_wrong_axis(q, k, v, scale):          # softmax over queries instead of keys
    s = scale * (q @ k.T)
    p = np.exp(s - s.max(axis=0, keepdims=True))
    return (p / p.sum(axis=0, keepdims=True)) @ v


def _rows_no_scale(q, k, v, scale):
    return A.attention_rows(q, k, v, 1.0)


def _rows_k_as_v(q, k, v, scale):              # wrong operand in PV
    return A.attention_rows(q, k, k, scale)


def _rows_no_max(q, k, v, scale):              # forgets the normalizer
    s = scale * (q @ k.T)
    return np.exp(s - s.max(axis=1, keepdims=True)) @ v


def _rows_transposed_scores(q, k, v, scale):  # K Q^T used as Q K^T (only square cases)
    s = scale * (k @ q.T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)) @ v


DENSE_MUTANTS = [_rows_wrong_axis, _rows_no_scale, _rows_k_as_v, _rows_no_max, _rows_transposed_scores]


@pytest.mark.parametrize("mut", DENSE_MUTANTS, ids=lambda f: f.__name__)
def test_dense_mutants_caught(mut):
    fn = _dense_from_rows(mut)
    caught = 0
    for check in (P.check_dense_brute_force, P.check_dense_invariants):
        try:
            check(fn)
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1


# ---------------------------------------------------------------- selection mutants

def _means_div_tile(x):
    N, d = x.shape
    T = A.tile_count(N)
    out = np.zeros((T, d))
    for t in range(T):
        out[t] = x[t * 128:min(t * 128 + 128, N)].sum(0) / 128.0
    return out


def _means_skip_first(x):
    N, d = x.shape
    T = A.tile_count(N)
    out = np.zeros((T, d))
    for t in range(T):
        rows = x[t * 128 + 1:min(t * 128 + 128, N)]
        out[t] = rows.sum(0) / max(1, len(rows))
    return out


@pytest.mark.parametrize("mut", [_means_div_tile, _means_skip_first], ids=lambda f: f.__name__)
def test_means_mutants_caught(mut):
    with pytest.raises(AssertionError):
        P.check_tile_means_exact(mut)


def _scores_blas(qm, km):       # blocked / fused summation order
    return qm @ km.T


def _scores_reversed(qm, km):   # same rounding rules, wrong order
    acc = np.zeros((qm.shape[0], km.shape[0]))
    for c in reversed(range(qm.shape[1])):
        acc = acc + np.multiply.outer(qm[:, c], km[:, c])
    return acc


def _scores_transposed(qm, km):
    return A.tile_scores(km, qm)


@pytest.mark.parametrize("mut", [_scores_blas, _scores_reversed, _scores_transposed],
                         ids=lambda f: f.__name__)
def test_scores_mutants_caught(mut):
    with pytest.raises(AssertionError):
        P.check_tile_scores_canonical(mut)


def _top_ties_high(sigma, k):
    T = sigma.shape[0]
    out = np.empty((T, k), dtype=np.int32)
    for i in range(T):
        order = (T - 1) - np.argsort(-sigma[i][::-1], kind="stable")
        out[i] = np.sort(order[:k])
    return out


def _top_unsorted(sigma, k):
    T = sigma.shape[0]
    out = np.empty((T, k), dtype=np.int32)
    for i in range(T):
        out[i] = np.argsort(-sigma[i], kind="stable")[:k]
    return out


def _top_smallest(sigma, k):
    return A.top_tiles(-sigma, k)


@pytest.mark.parametrize("mut", [_top_ties_high, _top_unsorted, _top_smallest], ids=lambda f: f.__name__)
def test_topk_mutants_caught(mut):
    with pytest.raises(AssertionError):
        P.check_top_tiles_brute_force(mut)


def _select_with(means=A.tile_means, scores=A.tile_scores, top=A.top_tiles, count=A.keep_count):
    def select(q, k, keep_frac):
        H, N, _ = q.shape
        T = A.tile_count(N)
        kk = count(T, keep_frac)
        return np.stack([top(scores(means(q[h]), means(k[h])), kk) for h in range(H)])
    return select


SELECT_MUTANTS = {
    "floor_count": _select_with(count=lambda T, f: max(1, min(math.floor(f * T), T))),
    "div_tile": _select_with(means=_means_div_tile),
    "ties_high": _select_with(top=_top_ties_high),
    "smallest": _select_with(top=_top_smallest),
}


@pytest.mark.parametrize("name", sorted(SELECT_MUTANTS))
def test_select_mutants_caught(name):
    with pytest.raises(AssertionError):
        P.check_select_closed_forms(SELECT_MUTANTS[name])


def test_select_reference_passes_checks():
    P.check_select_closed_forms(_select_with())


# ---------------------------------------------------------------- sparse mutants

def _sparse_ignores_idx(q, k, v, scale, idx, rows=None):
    return oracle.dense(q, k, v, scale, rows=rows)


def _sparse_wrong_head(q, k, v, scale, idx, rows=None):
    return oracle.sparse(q, k, v, scale, idx[::-1].copy(), rows=rows)


def _sparse_tile_of_row_off(q, k, v, scale, idx, rows=None):
    H, N, d = q.shape
    out = np.empty((H, N, d))
    for h in range(H):
        for i in range(N):
            t = min(i // 128 + 1, idx.shape[1] - 1)
            keys = oracle.kept_keys(idx[h, t], N)
            out[h, i] = A.attention_rows(q[h, i:i + 1], k[h, keys], v[h, keys], scale)[0]
    return out


@pytest.mark.parametrize("mut", [_sparse_ignores_idx, _sparse_wrong_head, _sparse_tile_of_row_off],
                         ids=lambda f: f.__name__)
def test_sparse_mutants_caught(mut):
    with pytest.raises(AssertionError):
        P.check_sparse_pins(mut, oracle.dense)
