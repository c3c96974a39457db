"""Host-side tests of the C ABI: the library loads, exports what include/fvattn.h
declares, and checks its arguments on the host.  No compute runs here."""

import ctypes
import math
import os
import re

import pytest
import torch

import oracle
import video_diffusion_transformer_amd as fv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fvattn.h")

# never dereferenced: every call below fails its host checks first
BOGUS = ctypes.c_void_p(0x1000)
NULL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fvattn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return fv.load()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(fv.SIGNATURES)


def test_library_resolves_every_symbol_at_load():
    # a kernel whose host stub was not emitted shows up as an unresolved symbol;
    # RTLD_NOW makes the loader resolve everything instead of on first call
    ctypes.CDLL(fv.LIB_PATH, mode=os.RTLD_NOW)


def test_status_strings(lib):
    for s in range(0, 6):
        assert fv.status_string(s)
    assert "INVALID" in fv.status_string(fv.FVATTN_ERR_INVALID_ARG)
    assert "unknown" in fv.status_string(99)


def test_keep_count_matches_oracle(lib):
    for tokens in [1, 127, 128, 129, 1008, 5040, 72576, 102816, 262144, 300000]:
        for f in [1e-9, 0.01, 0.07, 0.1, 1 - 0.9, 0.14, 0.25, 0.3, 0.5, 0.99, 1.0]:
            T = oracle.tile_count(tokens)
            assert fv.keep_count(tokens, f) == oracle.keep_count(T, f), (tokens, f)
    assert fv.keep_count(72576, 0.1) == 57
    assert fv.keep_count(102816, 0.1) == 81
    assert fv.keep_count(0, 0.1) == 0


@pytest.mark.parametrize("frac", [0.0, -0.1, 1.5, float("nan"), float("inf")])
def test_keep_count_rejects_bad_fraction(lib, frac):
    assert lib.fvattn_keep_count(1008, frac) == -fv.FVATTN_ERR_INVALID_ARG


def test_keep_count_rejects_negative_tokens(lib):
    assert lib.fvattn_keep_count(-1, 0.1) == -fv.FVATTN_ERR_INVALID_ARG


def _fwd(lib, q=BOGUS, k=BOGUS, v=BOGUS, o=BOGUS, heads=4, tokens=1008, hd=128, scale=0.088,
         mode=0, frac=0.1):
    return lib.fvattn_forward(q, k, v, o, heads, tokens, hd, scale, mode, frac, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(q=NULL), fv.FVATTN_ERR_INVALID_ARG),
    (dict(k=NULL), fv.FVATTN_ERR_INVALID_ARG),
    (dict(v=NULL), fv.FVATTN_ERR_INVALID_ARG),
    (dict(o=NULL), fv.FVATTN_ERR_INVALID_ARG),
    (dict(heads=-1), fv.FVATTN_ERR_INVALID_ARG),
    (dict(tokens=-5), fv.FVATTN_ERR_INVALID_ARG),
    (dict(hd=64), fv.FVATTN_ERR_UNSUPPORTED),
    (dict(hd=256), fv.FVATTN_ERR_UNSUPPORTED),
    (dict(scale=0.0), fv.FVATTN_ERR_INVALID_ARG),
    (dict(scale=-1.0), fv.FVATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fv.FVATTN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fv.FVATTN_ERR_INVALID_ARG),
    (dict(mode=7), fv.FVATTN_ERR_INVALID_ARG),
    (dict(mode=-1), fv.FVATTN_ERR_INVALID_ARG),
    (dict(mode=1, frac=0.0), fv.FVATTN_ERR_INVALID_ARG),
    (dict(mode=1, frac=1.01), fv.FVATTN_ERR_INVALID_ARG),
    (dict(mode=1, frac=float("nan")), fv.FVATTN_ERR_INVALID_ARG),
    (dict(mode=1, tokens=2048 * 128 + 1), fv.FVATTN_ERR_UNSUPPORTED),
    (dict(tokens=(1 << 31) // 128 + 1), fv.FVATTN_ERR_UNSUPPORTED),
])
def test_forward_rejects_bad_arguments(lib, kw, want):
    assert _fwd(lib, **kw) == want


@pytest.mark.parametrize("sink,floats,iters", [(NULL, fv.PROBE_SINK, 10), (BOGUS, fv.PROBE_SINK - 1, 10),
                                               (BOGUS, fv.PROBE_SINK, 0), (BOGUS, 0, 10)])
def test_mfma_probe_rejects_bad_arguments(lib, sink, floats, iters):
    assert lib.fvattn_mfma_probe(sink, floats, iters, NULL) == fv.FVATTN_ERR_INVALID_ARG


def test_dense_ignores_keep_frac_checks(lib):
    # keep_frac is not looked at in dense mode: a bad one plus a NULL pointer
    # still reports the pointer
    assert _fwd(lib, q=NULL, frac=float("nan")) == fv.FVATTN_ERR_INVALID_ARG


def test_empty_inputs_are_noops(lib):
    # nothing to do: OK without touching any pointer or the device
    assert _fwd(lib, q=NULL, k=NULL, v=NULL, o=NULL, tokens=0) == fv.FVATTN_OK
    assert _fwd(lib, q=NULL, k=NULL, v=NULL, o=NULL, heads=0) == fv.FVATTN_OK
    assert _fwd(lib, q=NULL, k=NULL, v=NULL, o=NULL, tokens=0, mode=1) == fv.FVATTN_OK
    assert lib.fvattn_select_tiles(NULL, NULL, 0, 1008, 128, 0.1, NULL, NULL) == fv.FVATTN_OK
    assert lib.fvattn_forward_indexed(NULL, NULL, NULL, NULL, 1, NULL, 4, 0, 128, 0.1, NULL) == 0
    assert lib.fvattn_forward_heads(NULL, NULL, NULL, NULL, 0, 16, 1008, 128, 0.1, 0, 0.1, NULL) == 0
    assert lib.fvattn_tile_means(NULL, 0, 10, 128, NULL, NULL) == fv.FVATTN_OK
    assert lib.fvattn_tile_scores(NULL, NULL, 3, 0, 128, NULL, NULL) == fv.FVATTN_OK


def test_select_tiles_rejects_bad_arguments(lib):
    st = lib.fvattn_select_tiles
    assert st(NULL, BOGUS, 4, 1008, 128, 0.1, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert st(BOGUS, BOGUS, 4, 1008, 128, 0.1, NULL, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert st(BOGUS, BOGUS, 4, 1008, 128, 0.0, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert st(BOGUS, BOGUS, 4, 1008, 120, 0.1, BOGUS, NULL) == fv.FVATTN_ERR_UNSUPPORTED
    assert st(BOGUS, BOGUS, 4, 2049 * 128, 128, 0.1, BOGUS, NULL) == fv.FVATTN_ERR_UNSUPPORTED
    assert st(BOGUS, BOGUS, -4, 1008, 128, 0.1, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG


def test_forward_indexed_rejects_bad_keep(lib):
    fi = lib.fvattn_forward_indexed
    # 1008 tokens = 8 tiles: keep must be in [1, 8]
    assert fi(BOGUS, BOGUS, BOGUS, BOGUS, 0, BOGUS, 4, 1008, 128, 0.1, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert fi(BOGUS, BOGUS, BOGUS, BOGUS, 9, BOGUS, 4, 1008, 128, 0.1, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert fi(BOGUS, BOGUS, BOGUS, NULL, 2, BOGUS, 4, 1008, 128, 0.1, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert fi(BOGUS, BOGUS, BOGUS, BOGUS, 2, BOGUS, 4, 1008, 128, 0.0, NULL) == fv.FVATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("group", [0, 1, 2, 3, 5, 12, 32, 56])
def test_forward_heads_rejects_bad_group(lib, group):
    assert lib.fvattn_forward_heads(BOGUS, BOGUS, BOGUS, BOGUS, 56, group, 1008, 128, 0.088, 0, 0.1,
                                    NULL) == fv.FVATTN_ERR_UNSUPPORTED


def test_tile_scores_rejects_bad_arguments(lib):
    ts = lib.fvattn_tile_scores
    assert ts(NULL, BOGUS, 2, 8, 128, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert ts(BOGUS, BOGUS, 2, 8, 64, BOGUS, NULL) == fv.FVATTN_ERR_UNSUPPORTED
    assert ts(BOGUS, BOGUS, 2, 4096, 128, BOGUS, NULL) == fv.FVATTN_ERR_UNSUPPORTED


def test_alloc_failure_hook_launches_nothing(lib, monkeypatch):
    monkeypatch.setenv("FVATTN_TEST_FAIL_ALLOC", "1")
    assert _fwd(lib, mode=1) == fv.FVATTN_ERR_ALLOC
    assert lib.fvattn_select_tiles(BOGUS, BOGUS, 4, 1008, 128, 0.1, BOGUS, NULL) == fv.FVATTN_ERR_ALLOC
    assert lib.fvattn_forward_heads(BOGUS, BOGUS, BOGUS, BOGUS, 56, 16, 1008, 128, 0.088, 1, 0.1,
                                    NULL) == fv.FVATTN_ERR_ALLOC
    assert lib.fvattn_tile_scores(BOGUS, BOGUS, 2, 8, 128, BOGUS, NULL) == fv.FVATTN_ERR_ALLOC
    # argument errors still come first
    assert _fwd(lib, mode=1, q=NULL) == fv.FVATTN_ERR_INVALID_ARG


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful on a host without a GPU")
def test_no_device_reports_hip_error(lib):
    # valid arguments but no GPU: the device check fails before any launch
    assert _fwd(lib) == fv.FVATTN_ERR_HIP


def test_binding_rejects_cpu_tensors():
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fv.forward(q, q, q)
    with pytest.raises(TypeError):
        fv.forward(q.float(), q.float(), q.float())


def _win(lib, q=BOGUS, k=BOGUS, v=BOGUS, o=BOGUS, heads=4, tokens=1008 * 12, hd=128, scale=0.088,
         ft=1008, chunk=5, nb=1, prefix=0):
    return lib.fvattn_forward_window(q, k, v, o, heads, tokens, hd, scale, prefix, ft, chunk, nb, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(q=NULL), fv.FVATTN_ERR_INVALID_ARG),
    (dict(o=NULL), fv.FVATTN_ERR_INVALID_ARG),
    (dict(heads=-1), fv.FVATTN_ERR_INVALID_ARG),
    (dict(tokens=-5), fv.FVATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), fv.FVATTN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fv.FVATTN_ERR_INVALID_ARG),
    (dict(chunk=0), fv.FVATTN_ERR_INVALID_ARG),
    (dict(nb=-1), fv.FVATTN_ERR_INVALID_ARG),
    (dict(hd=64), fv.FVATTN_ERR_UNSUPPORTED),
    (dict(ft=63), fv.FVATTN_ERR_UNSUPPORTED),
    (dict(ft=0), fv.FVATTN_ERR_UNSUPPORTED),
    (dict(tokens=2049 * 128), fv.FVATTN_ERR_UNSUPPORTED),
    (dict(prefix=-1), fv.FVATTN_ERR_INVALID_ARG),
    (dict(prefix=1008 * 12 + 1), fv.FVATTN_ERR_INVALID_ARG),
])
def test_forward_window_rejects_bad_arguments(lib, kw, want):
    assert _win(lib, **kw) == want


def test_window_entry_points_empty_and_bad(lib):
    assert _win(lib, q=NULL, k=NULL, v=NULL, o=NULL, heads=0) == fv.FVATTN_OK
    assert _win(lib, q=NULL, k=NULL, v=NULL, o=NULL, tokens=0) == fv.FVATTN_OK
    wt = lib.fvattn_window_tiles
    assert wt(0, 0, 1008, 5, 1, NULL, NULL, NULL) == fv.FVATTN_OK
    assert wt(-1, 0, 1008, 5, 1, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert wt(5000, 0, 1008, 0, 1, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert wt(5000, 0, 1008, 5, -1, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert wt(5000, -1, 1008, 5, 1, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert wt(5000, 5001, 1008, 5, 1, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert wt(5000, 0, 32, 5, 1, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_UNSUPPORTED
    assert wt(5000, 0, 1008, 5, 1, NULL, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert wt(5000, 0, 1008, 5, 1, BOGUS, NULL, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert wt(2049 * 128, 0, 1008, 5, 1, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_UNSUPPORTED


def test_window_alloc_failure_hook(lib, monkeypatch):
    monkeypatch.setenv("FVATTN_TEST_FAIL_ALLOC", "1")
    assert _win(lib) == fv.FVATTN_ERR_ALLOC
    assert _win(lib, q=NULL) == fv.FVATTN_ERR_INVALID_ARG


def _vsa(lib, q=BOGUS, k=BOGUS, v=BOGUS, o=BOGUS, heads=4, prefix=37, grid=(5, 24, 42),
         tile=(4, 4, 4), frac=0.1, scale=0.088, hd=128, tokens=None):
    if tokens is None:
        tokens = prefix + grid[0] * grid[1] * grid[2]
    return lib.fvattn_forward_vsa(q, k, v, o, heads, tokens, hd, scale, prefix, *grid, *tile, frac, NULL)


@pytest.mark.parametrize("kw,want", [
    (dict(q=NULL), fv.FVATTN_ERR_INVALID_ARG),
    (dict(o=NULL), fv.FVATTN_ERR_INVALID_ARG),
    (dict(heads=-1), fv.FVATTN_ERR_INVALID_ARG),
    (dict(prefix=-1), fv.FVATTN_ERR_INVALID_ARG),
    (dict(grid=(0, 24, 42)), fv.FVATTN_ERR_INVALID_ARG),
    (dict(tile=(4, 0, 4)), fv.FVATTN_ERR_INVALID_ARG),
    (dict(tokens=5078), fv.FVATTN_ERR_INVALID_ARG),
    (dict(frac=0.0), fv.FVATTN_ERR_INVALID_ARG),
    (dict(frac=1.5), fv.FVATTN_ERR_INVALID_ARG),
    (dict(scale=-1.0), fv.FVATTN_ERR_INVALID_ARG),
    (dict(hd=64), fv.FVATTN_ERR_UNSUPPORTED),
    (dict(tile=(2, 4, 4)), fv.FVATTN_ERR_UNSUPPORTED),
    (dict(tile=(4, 8, 16)), fv.FVATTN_ERR_UNSUPPORTED),
    (dict(grid=(400, 24, 42)), fv.FVATTN_ERR_UNSUPPORTED),      # 100 x 66 tiles > 2048
])
def test_forward_vsa_rejects_bad_arguments(lib, kw, want):
    assert _vsa(lib, **kw) == want


def test_vsa_entry_points_empty_and_counts(lib):
    assert _vsa(lib, q=NULL, k=NULL, v=NULL, o=NULL, heads=0) == fv.FVATTN_OK
    sel = lib.fvattn_vsa_select
    assert sel(NULL, NULL, 0, 5077, 128, 37, 5, 24, 42, 4, 4, 4, 0.1, NULL, NULL) == fv.FVATTN_OK
    assert sel(BOGUS, BOGUS, 2, 5077, 128, 37, 5, 24, 42, 4, 4, 4, 0.1, NULL, NULL) == \
        fv.FVATTN_ERR_INVALID_ARG
    assert sel(BOGUS, BOGUS, 2, 5078, 128, 37, 5, 24, 42, 4, 4, 4, 0.1, BOGUS, NULL) == \
        fv.FVATTN_ERR_INVALID_ARG
    tc = lib.fvattn_vsa_tile_count
    assert tc(72, 24, 42, 4, 4, 4) == 1188
    assert tc(102, 24, 42, 4, 4, 4) == 1716
    assert tc(72, 24, 42, 4, 8, 8) == 324
    assert tc(0, 24, 42, 4, 4, 4) == -fv.FVATTN_ERR_INVALID_ARG
    for grid, tile in [((5, 24, 42), (4, 4, 4)), ((9, 7, 11), (2, 3, 5))]:
        assert tc(*grid, *tile) == len(oracle.video_tiles(*grid, tile))


def test_vsa_alloc_failure_hook(lib, monkeypatch):
    monkeypatch.setenv("FVATTN_TEST_FAIL_ALLOC", "1")
    assert _vsa(lib) == fv.FVATTN_ERR_ALLOC
    assert _vsa(lib, q=NULL) == fv.FVATTN_ERR_INVALID_ARG


def test_int8_mode_argument_checks(lib, monkeypatch):
    # mode 2 (dense, INT8 query-key scores): keep_frac is not looked at
    assert _fwd(lib, q=NULL, mode=2, frac=float("nan")) == fv.FVATTN_ERR_INVALID_ARG
    assert _fwd(lib, mode=2, hd=64) == fv.FVATTN_ERR_UNSUPPORTED
    assert _fwd(lib, q=NULL, k=NULL, v=NULL, o=NULL, tokens=0, mode=2) == fv.FVATTN_OK
    assert _fwd(lib, mode=4) == fv.FVATTN_ERR_INVALID_ARG
    assert _fwd(lib, mode=-1) == fv.FVATTN_ERR_INVALID_ARG
    # mode 3 (dense, FP8 query-key scores) takes the same checks
    assert _fwd(lib, q=NULL, mode=3, frac=float("nan")) == fv.FVATTN_ERR_INVALID_ARG
    assert _fwd(lib, mode=3, hd=64) == fv.FVATTN_ERR_UNSUPPORTED
    assert _fwd(lib, q=NULL, k=NULL, v=NULL, o=NULL, tokens=0, mode=3) == fv.FVATTN_OK
    for qk in (lib.fvattn_quantize_k, lib.fvattn_quantize_k_fp8):
        assert qk(NULL, 0, 100, 128, NULL, NULL, NULL) == fv.FVATTN_OK
        assert qk(BOGUS, 2, 100, 128, NULL, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
        assert qk(BOGUS, 2, 100, 96, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_UNSUPPORTED
    qk = lib.fvattn_quantize_k
    assert qk(NULL, 0, 100, 128, NULL, NULL, NULL) == fv.FVATTN_OK
    assert qk(BOGUS, 2, 100, 128, NULL, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert qk(BOGUS, 2, 100, 128, BOGUS, NULL, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert qk(BOGUS, 2, 100, 96, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_UNSUPPORTED
    assert qk(BOGUS, -2, 100, 128, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    monkeypatch.setenv("FVATTN_TEST_FAIL_ALLOC", "1")
    assert _fwd(lib, mode=2) == fv.FVATTN_ERR_ALLOC
    assert _fwd(lib, mode=3) == fv.FVATTN_ERR_ALLOC
    assert lib.fvattn_forward_heads(BOGUS, BOGUS, BOGUS, BOGUS, 56, 16, 1008, 128, 0.088, 2, 0.1,
                                    NULL) == fv.FVATTN_ERR_ALLOC


def test_vda_argument_checks(lib, monkeypatch):
    fw, st = lib.fvattn_vda_forward, lib.fvattn_vda_states
    args = lambda **kw: [kw.get(n, d) for n, d in [("q", BOGUS), ("k", BOGUS), ("v", BOGUS), ("b", BOGUS),
                                                  ("a", BOGUS), ("s", BOGUS), ("o", BOGUS), ("h", 2),
                                                  ("f", 7), ("ft", 64), ("hd", 128), ("ch", 5), ("nb", 1)]]
    assert fw(*args(q=NULL), NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert fw(*args(o=NULL), NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert fw(*args(b=NULL), NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert fw(*args(h=-1), NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert fw(*args(ch=0), NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert fw(*args(nb=-1), NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert fw(*args(ft=0), NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert fw(*args(hd=64), NULL) == fv.FVATTN_ERR_UNSUPPORTED
    assert fw(*args(q=NULL, k=NULL, v=NULL, h=0), NULL) == fv.FVATTN_OK
    assert fw(*args(q=NULL, k=NULL, v=NULL, f=0), NULL) == fv.FVATTN_OK
    assert st(BOGUS, BOGUS, BOGUS, BOGUS, BOGUS, 2, 7, 64, 128, NULL, BOGUS, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert st(BOGUS, BOGUS, BOGUS, BOGUS, BOGUS, 2, 7, 64, 96, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_UNSUPPORTED
    assert st(NULL, NULL, NULL, NULL, NULL, 0, 7, 64, 128, NULL, NULL, NULL) == fv.FVATTN_OK
    monkeypatch.setenv("FVATTN_TEST_FAIL_ALLOC", "1")
    assert fw(*args(), NULL) == fv.FVATTN_ERR_ALLOC
    assert st(BOGUS, BOGUS, BOGUS, BOGUS, BOGUS, 2, 7, 64, 128, BOGUS, BOGUS, NULL) == fv.FVATTN_ERR_ALLOC


def test_vda_frame_size_limit(lib):
    fw = lib.fvattn_vda_forward
    # one frame's bf16 rows must stay below 2^31 bytes (8,388,608 x 256 B is 2^31)
    assert fw(BOGUS, BOGUS, BOGUS, BOGUS, BOGUS, BOGUS, BOGUS, 1, 1, 8388608, 128, 5, 1,
              NULL) == fv.FVATTN_ERR_UNSUPPORTED


def test_token_limit_is_per_head_elements(lib):
    # one head's tensor must hold fewer than 2^31 elements: 2^24 tokens x 128 is 2^31
    for mode in (0, 1, 2):
        assert _fwd(lib, heads=1, tokens=1 << 24, mode=mode) == fv.FVATTN_ERR_UNSUPPORTED
    assert lib.fvattn_forward_indexed(BOGUS, BOGUS, BOGUS, BOGUS, 1, BOGUS, 1, 1 << 24, 128, 0.088,
                                      NULL) == fv.FVATTN_ERR_UNSUPPORTED
    # 2^23 tokens (2^31 bytes of one head) pass the argument checks; without a
    # GPU the call then fails at the device check, not at the size check
    assert _fwd(lib, heads=1, tokens=1 << 23, mode=0) == fv.FVATTN_ERR_HIP


@pytest.mark.parametrize("tokens,rows,count,stride,ok", [
    (72576, 128, 567, 567, True),        # the layout the window entry point allocates
    (72576, 128, 600, 700, True),        # more room than needed
    (72576, 256, 567, 567, False),       # lists built for another block height
    (72576, 128, 566, 567, False),       # one list short
    (72576, 128, 567, 566, False),       # rows too narrow for every key tile
    (1, 128, 1, 1, True),
    (129, 128, 1, 2, False),
])
def test_window_list_layout_check(lib, tokens, rows, count, stride, ok):
    fn = lib.fvattn_internal_window_lists_fit
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int] * 4
    want = fv.FVATTN_OK if ok else fv.FVATTN_ERR_INVALID_ARG
    assert fn(tokens, rows, count, stride) == want


def test_vda_binding_checks_shapes_before_use():
    H, F, ft = 2, 3, 8
    N = F * ft
    bf, f32 = torch.bfloat16, torch.float32
    good = dict(q=torch.zeros(H, N, 128, dtype=bf), k=torch.zeros(H, N, 128, dtype=bf),
                v=torch.zeros(H, N, 128, dtype=bf), beta=torch.zeros(H, N, dtype=f32),
                alpha=torch.ones(H, F, 128, dtype=f32), s_text=torch.zeros(H, 128, 128, dtype=f32))
    bad = [("beta", torch.zeros(H, N - 1, dtype=f32)), ("alpha", torch.ones(H, F + 1, 128, dtype=f32)),
           ("s_text", torch.zeros(H, 128, 64, dtype=f32)), ("v", torch.zeros(H, N, 128, dtype=f32)),
           ("beta", torch.zeros(H, 2 * N, dtype=f32)[:, ::2])]
    for name, t in bad:
        a = dict(good, **{name: t})
        with pytest.raises(ValueError, match=name):
            fv.vda_forward(a["q"], a["k"], a["v"], a["beta"], a["alpha"], a["s_text"], ft)
        with pytest.raises(ValueError, match=name):
            fv.vda_states(a["k"], a["v"], a["beta"], a["alpha"], a["s_text"], ft)
    with pytest.raises(ValueError, match="out"):
        fv.vda_forward(*good.values(), ft, out=torch.zeros(H, N, 64, dtype=f32))
    # right shapes on the CPU: refused as host tensors, before any library call
    with pytest.raises(ValueError, match="device"):
        fv.vda_forward(*good.values(), ft)
    with pytest.raises(ValueError, match="frame"):
        fv.vda_states(good["k"], good["v"], good["beta"], good["alpha"], good["s_text"], 7)


def _noalloc_bytes(heads, tokens, frac):
    al = lambda n: (n + 255) // 256 * 256
    T = oracle.tile_count(tokens)
    k = oracle.keep_count(T, frac)
    return 2 * al(8 * heads * T * 128) + al(8 * heads * T * T) + al(4 * heads * T * k)


def test_noalloc_limit_is_checked_on_the_host(lib):
    f = lib.fvattn_forward_sparse_noalloc
    limit = 64 * 1024 * 1024
    for heads, tokens in [(16, 72576), (8, 102816), (17, 72576), (9, 102816), (1, 262144), (64, 72576)]:
        fits = _noalloc_bytes(heads, tokens, 0.1) <= limit
        rc = f(BOGUS, BOGUS, BOGUS, BOGUS, heads, tokens, 128, 0.088, 0.1, NULL)
        # within the limit the call goes on to the device check (no GPU here)
        assert rc == (fv.FVATTN_ERR_HIP if fits else fv.FVATTN_ERR_UNSUPPORTED), (heads, tokens)
    assert _noalloc_bytes(16, 72576, 0.1) <= limit and _noalloc_bytes(8, 102816, 0.1) <= limit
    assert f(NULL, BOGUS, BOGUS, BOGUS, 1, 100, 128, 0.088, 0.1, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert f(BOGUS, BOGUS, BOGUS, BOGUS, 1, 100, 128, 0.088, 0.0, NULL) == fv.FVATTN_ERR_INVALID_ARG
    assert f(BOGUS, BOGUS, BOGUS, BOGUS, 1, 100, 64, 0.088, 0.1, NULL) == fv.FVATTN_ERR_UNSUPPORTED
    assert f(NULL, NULL, NULL, NULL, 0, 100, 128, 0.088, 0.1, NULL) == fv.FVATTN_OK
