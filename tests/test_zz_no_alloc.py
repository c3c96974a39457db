"""The allocation-free sparse entry point (fvattn_forward_sparse_noalloc)
against fvattn_forward in block-sparse mode, through the C ABI: bit for bit,
on two calls in a row (the second with a smaller input, so stale contents of
the static scratch from the first call would show), and the smaller one also
against the fp64 oracle."""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_amd as fv
from video_diffusion_transformer_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[no-alloc]", *a, file=sys.stderr, flush=True)


def test_noalloc_sparse_matches_allocating_entry_twice():
    scale = 1 / math.sqrt(128)
    cases = [(72576, 16, "frame", 3, 0.1), (5040 + 37, 3, "iid", 8, 0.25)]
    for N, H, dist, seed, frac in cases:
        say("case", N, "tokens x", H, "heads, keep", frac)
        q, k, v = inputs.make_qkv(N, H, dist, seed)
        qd, kd, vd = (t.to(DEV) for t in (q, k, v))
        ref = fv.forward(qd, kd, vd, scale=scale, mode="sparse", keep_frac=frac)
        out = torch.full_like(qd, float("nan"))
        fv.forward_sparse_noalloc(qd, kd, vd, scale=scale, keep_frac=frac, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (N, H)
        say("bitwise equal to fvattn_forward (sparse)")
        if N < 10000:
            qw, kw, vw = (oracle.widen(t) for t in (q, k, v))
            idx = oracle.select_tiles(qw, kw, frac)
            want = oracle.sparse(qw, kw, vw, scale, idx)
            err = np.abs(oracle.widen(out.cpu()) - want)
            rel = np.linalg.norm(oracle.widen(out.cpu()) - want) / np.linalg.norm(want)
            say(f"against the oracle: max_abs={err.max():.3e} mean_abs={err.mean():.3e} rel_fro={rel:.3e}")
            assert err.max() <= 2e-2 and err.mean() <= 2e-3 and rel <= 1e-2


def test_noalloc_rejects_inputs_beyond_its_scratch():
    q = torch.zeros((64, 72576, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fv.FvattnError) as e:
        fv.forward_sparse_noalloc(q, q, q, keep_frac=0.1, out=torch.empty_like(q))
    assert e.value.status == fv.FVATTN_ERR_UNSUPPORTED
