"""fp64 CPU oracle for Video Delta Attention, the linear branch of Video DeltaNet.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It shares no code with
the HIP library and imports nothing from it.

What is computed (FreeVideo page, "FreeVideo: a 66 GB video transformer on an
8 GB card...", section "Where Video DeltaNet comes in"):

* The state is a d_v x d_k matrix per head.  A latent frame's tokens are
  written at once: with the decayed state Sbar_t, keys k_u, values v_u and
  write strengths beta_u of the frame's tokens, the new state minimizes
  1/2 ||S - Sbar_t||_F^2 + 1/2 sum_u beta_u ||S k_u - v_u||^2, whose closed
  form is S_t = (Sbar_t + B_t)(I + A_t)^-1 with A_t = sum_u beta_u k_u k_u^T
  and B_t = sum_u beta_u v_u k_u^T (the page's equations).
* The decay is Sbar_t = S_prev Diag(alpha_t), alpha_t in (0, 1]^d_k per frame
  and head: the page's bound on ||Diag(alpha_t)(I + A_t)^-1|| names this form.
* Two scans, forward over the frames and reverse, both seeded with S_text / 2,
  so that the two readouts together count the text state once.
* A query reads the forward state of the frames before its softmax window and
  the reverse state of the frames after it.

Readings taken where the page is silent:

* The softmax window is the frame window of ``attention.window_frames_allowed``
  (chunks of ``chunk_frames`` frames, ``neighbours`` chunks on each side, first
  and last frame as anchors).  The linear branch covers what that window does
  not: the anchor frames are never written into a state (the forward scan
  absorbs frames 1..F-2 in order, the reverse scan F-2..1), a query of chunk c
  reads the forward state after the frames before frame (c - neighbours) *
  chunk_frames and the reverse state after the frames from (c + neighbours + 1)
  * chunk_frames on, and a query of an anchor frame (which sees every frame by
  softmax) reads only the two seeds.
* The readout is o = S_fwd q + S_rev q, before the branch's learned gate,
  normalization and projection (out of scope: they need trained weights).
"""

from __future__ import annotations

import numpy as np


def frame_update(s_prev: np.ndarray, k: np.ndarray, v: np.ndarray, beta: np.ndarray,
                 alpha: np.ndarray) -> np.ndarray:
    """One Video Delta Attention write.

    s_prev: [dv, dk]; k: [n, dk]; v: [n, dv]; beta: [n]; alpha: [dk].
    Returns (s_prev Diag(alpha) + B)(I + A)^-1 in float64.
    """
    dk = k.shape[1]
    a = (k * beta[:, None]).T @ k                 # sum_u beta_u k_u k_u^T
    b = (v * beta[:, None]).T @ k                 # sum_u beta_u v_u k_u^T
    x = s_prev * alpha[None, :] + b
    # S (I + A) = x  <=>  (I + A) S^T = x^T  (I + A is symmetric)
    return np.linalg.solve(np.eye(dk) + a, x.T).T


def scan_states(k: np.ndarray, v: np.ndarray, beta: np.ndarray, alpha: np.ndarray,
                s_text: np.ndarray, frame_tokens: int):
    """Forward and reverse states of one head.

    k, v: [N, d]; beta: [N]; alpha: [F, d]; s_text: [d, d]; N = F * frame_tokens.
    Returns (fwd, rev), each [F + 1, d, d]: fwd[t] has absorbed the non-anchor
    frames before t, rev[t] the non-anchor frames from t on; fwd[0] = rev[F] =
    s_text / 2.
    """
    N, d = k.shape
    F = N // frame_tokens
    assert F * frame_tokens == N
    fwd = np.empty((F + 1, d, d))
    rev = np.empty((F + 1, d, d))
    fwd[0] = s_text / 2.0
    for t in range(F):
        sl = slice(t * frame_tokens, (t + 1) * frame_tokens)
        if 1 <= t <= F - 2:
            fwd[t + 1] = frame_update(fwd[t], k[sl], v[sl], beta[sl], alpha[t])
        else:
            fwd[t + 1] = fwd[t]
    rev[F] = s_text / 2.0
    for t in range(F - 1, -1, -1):
        sl = slice(t * frame_tokens, (t + 1) * frame_tokens)
        if 1 <= t <= F - 2:
            rev[t] = frame_update(rev[t + 1], k[sl], v[sl], beta[sl], alpha[t])
        else:
            rev[t] = rev[t + 1]
    return fwd, rev


def read_positions(frames: int, chunk_frames: int = 5, neighbours: int = 1):
    """(lo, hi) per query frame: it reads fwd[lo] and rev[hi]."""
    lo = np.empty(frames, dtype=np.int64)
    hi = np.empty(frames, dtype=np.int64)
    for f in range(frames):
        if f == 0 or f == frames - 1:
            lo[f], hi[f] = 0, frames
        else:
            c = f // chunk_frames
            lo[f] = min(max((c - neighbours) * chunk_frames, 0), frames)
            hi[f] = min(max((c + neighbours + 1) * chunk_frames, 0), frames)
    return lo, hi


def vda_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, beta: np.ndarray,
                  alpha: np.ndarray, s_text: np.ndarray, frame_tokens: int,
                  chunk_frames: int = 5, neighbours: int = 1) -> np.ndarray:
    """Linear-branch readout of every head: o_i = fwd[lo] q_i + rev[hi] q_i.

    q, k, v: [H, N, d]; beta: [H, N]; alpha: [H, F, d]; s_text: [H, d, d].
    Returns [H, N, d] float64.
    """
    H, N, d = q.shape
    F = N // frame_tokens
    lo, hi = read_positions(F, chunk_frames, neighbours)
    out = np.empty((H, N, d))
    for h in range(H):
        fwd, rev = scan_states(k[h], v[h], beta[h], alpha[h], s_text[h], frame_tokens)
        for f in range(F):
            sl = slice(f * frame_tokens, (f + 1) * frame_tokens)
            out[h, sl] = q[h, sl] @ (fwd[lo[f]] + rev[hi[f]]).T
    return out
