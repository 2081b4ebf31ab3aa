"""C-ABI contract tests that need no GPU: the library loads, exports every
entry point the header declares, validates arguments before touching the
device (each invalid call returns its error code and message), and the host
helpers agree with the oracle's table and layer pattern."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(HERE), "include", "fa.h")

fa = pytest.importorskip("causal_attention_fa_amd.fa",
                         reason="libfa.so not built (python -m causal_attention_fa_amd.build)")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported():
    names = header_functions()
    assert set(names) == set(fa.EXPORTS), names
    lib = ctypes.CDLL(fa.library_path())
    for n in names:
        assert hasattr(lib, n), n


# A fake, aligned, non-null pointer: validation fails before it is used.
P = 1 << 20


def _fwd(**kw):
    a = dict(q=P, k=2 * P, v=3 * P, o=4 * P, lse=5 * P, B=1, H=2, Hkv=1, T=8, d=64,
             scale=0.125, window=0, global_every=0, softcap=0.0)
    a.update(kw)
    return fa._lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"],
                          a["T"], a["d"], a["scale"], a["window"], a["global_every"],
                          a["softcap"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=0), -1, "null pointer q"),
    (dict(lse=0), -1, "null pointer lse"),
    (dict(B=0), -1, "positive"),
    (dict(T=-3), -1, "positive"),
    (dict(H=3, Hkv=2), -1, "multiple of Hkv"),
    (dict(d=63), -1, "even"),
    (dict(d=96), -2, "64, 128 or 256"),
    (dict(window=-1), -1, "window"),
    (dict(global_every=-2), -1, "global_every"),
    (dict(softcap=-1.0), -1, "softcap"),
    (dict(softcap=float("nan")), -1, "softcap"),
    (dict(scale=0.0), -1, "scale"),
    (dict(scale=float("inf")), -1, "scale"),
    (dict(q=P + 8), -1, "aligned"),
    (dict(o=P), -1, "overlaps"),
    # one head's [T, d] slice is addressed through a 32-bit buffer range
    (dict(B=1, H=1, Hkv=1, T=9_000_000, d=128), -1, "exceeds 2 GiB"),
])
def test_fwd_validation(kw, code, msg):
    assert _fwd(**kw) == code
    assert msg in fa.fa_last_error()


def test_bwd_validation_and_overlap():
    lib = fa._lib
    args = [P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P, 7 * P, 8 * P, 9 * P]
    rc = lib.fa_bwd(*args, 1, 2, 2, 8, 64, 0.125, 0, 0, 0.0, None)
    # all ranges are 1 MiB apart and small: valid up to the device call, so
    # only check invalid variants here
    bad = list(args)
    bad[7] = bad[0]  # dk aliases q
    assert lib.fa_bwd(*bad, 1, 2, 2, 8, 64, 0.125, 0, 0, 0.0, None) == -1
    assert "overlaps" in fa.fa_last_error()
    assert lib.fa_bwd(*args, 1, 2, 2, 8, 64, 0.125, -5, 0, 0.0, None) == -1
    assert lib.fa_bwd_f32(*args, 1, 2, 2, 8, 32, 0.125, 0, 0, 0.0, None) == -2
    del rc


def test_sink_validation():
    lib = fa._lib
    fwd = [P, 2 * P, 3 * P, 4 * P, 5 * P]
    assert lib.fa_fwd_sink(*fwd, 6 * P, 4 * P + 64, 1, 2, 2, 8, 64, 0.125, 0, 0, 0.0, None) == -1
    assert "max_logit overlaps o" in fa.fa_last_error()
    assert lib.fa_fwd_sink(*fwd, 6 * P, 7 * P + 4, 1, 2, 2, 8, 64, 0.125, 0, 0, 0.0, None) == -1
    assert "aligned" in fa.fa_last_error()
    assert lib.fa_fwd_sink(*fwd, 6 * P + 4, None, 1, 2, 2, 8, 64, 0.125, 0, 0, 0.0, None) == -1
    assert "sinks not 16-byte aligned" in fa.fa_last_error()
    bwd = [P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P]
    outs = [8 * P, 9 * P, 10 * P]
    assert lib.fa_bwd_sink(*bwd, 7 * P, *outs, None, 1, 2, 2, 8, 64, 0.125, 0, 0, 0.0,
                           None) == -1
    assert "both" in fa.fa_last_error()
    assert lib.fa_bwd_sink(*bwd, 7 * P, *outs, 8 * P, 1, 2, 2, 8, 64, 0.125, 0, 0, 0.0,
                           None) == -1
    assert "dsinks overlaps" in fa.fa_last_error()
    assert lib.fa_bwd_sink(*bwd, 7 * P, *outs, 7 * P, 1, 2, 2, 8, 64, 0.125, 0, 0, 0.0,
                           None) == -1
    assert "dsinks overlaps sinks" in fa.fa_last_error()


def test_rope_validation():
    lib = fa._lib
    assert lib.rope_apply(0, P, 2 * P, 1, 1, 4, 64, None) == -1
    assert lib.rope_apply(P, 2 * P, 3 * P, 1, 1, 4, 7, None) == -1
    assert lib.rope_apply(P, P + 16, 3 * P, 1, 1, 4, 64, None) == -1
    assert "overlaps" in fa.fa_last_error()
    assert lib.rope_apply_bwd_f32(P, 2 * P, 3 * P, 0, 1, 4, 64, None) == -1


def test_layer_window_matches_oracle():
    from oracle import attention as OA
    for ge in (0, 1, 2, 6):
        for w in (0, 1, 1024, 4096):
            for layer in range(13):
                assert fa.fa_layer_window(layer, w, ge) == OA.layer_window(layer, w, ge)
    with pytest.raises(fa.FAError):
        fa.fa_layer_window(0, -1, 0)


@pytest.mark.parametrize("d,theta", [(64, 1e4), (128, 1e6), (256, 1e4), (2, 5.0)])
def test_inv_freq_matches_oracle(d, theta):
    from oracle import rope as OR
    got = fa.fa_rope_inv_freq(d, theta)
    want = OR.inv_freq(d, theta)
    # both round theta^(-2i/d) from double; allow one float32 ulp
    np.testing.assert_array_max_ulp(got, want, maxulp=1)
    with pytest.raises(fa.FAError):
        fa.fa_rope_inv_freq(5, theta)


@pytest.mark.parametrize("d,theta,factor", [(128, 5e5, 32.0), (64, 1e4, 8.0), (128, 5e5, 0.0),
                                            (256, 1e6, 1.0)])
def test_llama3_table_matches_oracle(d, theta, factor):
    from oracle import rope as OR
    got = fa.fa_rope_inv_freq_llama3(d, theta, factor, 1.0, 4.0, 8192.0)
    want = OR.inv_freq_llama3(d, theta, factor, 1.0, 4.0, 8192.0)
    np.testing.assert_array_max_ulp(got, want, maxulp=1)
    with pytest.raises(fa.FAError):
        fa.fa_rope_inv_freq_llama3(d, theta, 8.0, 4.0, 1.0, 8192.0)


def test_layer_rope_theta_matches_oracle():
    from oracle import rope as OR
    for ge in (0, 2, 6):
        for tg in (0.0, 1e6):
            for layer in range(13):
                assert fa.fa_layer_rope_theta(layer, 1e4, tg, ge) == OR.layer_rope_theta(layer, 1e4, tg, ge)


def test_bwd_kernel_plan():
    """Every supported head-size pair covers dK and dV in one pass and dQ
    once: by the recomputing dQ pass first, or from the dS the dK/dV pass
    stores, after the D prologue.  Mode 0 (default) stores dS at d = 256
    only, mode 1 never, mode 2 wherever supported (d = 128, 256); other
    modes and unsupported sizes raise."""
    sizes = ((64, 64), (128, 128), (256, 256), (192, 128))
    stored = {0: {(256, 256)}, 1: set(), 2: {(128, 128), (256, 256)}}
    prev = fa.fa_set_dq_mode(0)
    try:
        for mode in (0, 1, 2, 0):
            fa.fa_set_dq_mode(mode)
            for d, dv in sizes:
                plan = fa.fa_bwd_kernels(d, dv)
                want = ["rowdot", "dkdv", "dq_ds"] if (d, dv) in stored[mode] else ["dq", "dkdv"]
                assert plan == want, (mode, d, dv, plan)
        for bad in (-1, 3):
            with pytest.raises(fa.FAError):
                fa.fa_set_dq_mode(bad)
        assert fa.fa_set_dq_mode(2) == 0 and fa.fa_set_dq_mode(0) == 2
    finally:
        fa.fa_set_dq_mode(prev)
    for d, dv in ((96, 96), (128, 64), (0, 0)):
        with pytest.raises(fa.FAError):
            fa.fa_bwd_kernels(d, dv)


def test_bwd_noalloc_rejects_oversize_before_device_work():
    """fa_bwd_noalloc's fixed scratch holds B*H*T <= 4,194,304 rows; a larger
    call is rejected with its own message before any HIP call."""
    lib = fa._lib
    args = [P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P, 7 * P, 8 * P, 9 * P]
    # 1 * 2 * 2,097,153 rows: one past the limit (tiny fake buffers: the size
    # check comes first)
    assert lib.fa_bwd_noalloc(*args, 1, 2, 2, 2_097_153, 64, 0.125, 0, 0, 0.0, None) == -1
    assert "exceeds its fixed scratch" in fa.fa_last_error()
    bad = list(args)
    bad[6] = bad[0]  # dq aliases q: the shared validation still applies
    assert lib.fa_bwd_noalloc(*bad, 1, 2, 2, 8, 64, 0.125, 0, 0, 0.0, None) == -1
    assert "overlaps" in fa.fa_last_error()


@pytest.mark.parametrize("T,W", [(1, 0), (31, 0), (33, 1), (100, 31), (100, 32), (100, 33),
                                 (257, 64), (300, 97), (640, 257), (1000, 999), (1000, 1000),
                                 (130, 5000)])
def test_bwd_workspace_band_covers_exactly_the_visible_tiles(T, W):
    """The dS workspace shape against the oracle's mask (q - W < k <= q),
    brute force over every (query, key) pair: each visible pair's key tile
    lands in a slot of its query tile's band (slot kt - qt + band - 1 in
    [0, band)), and each slot of a query tile's band that names a real key
    tile holds at least one visible pair of it (no slot is wasted on a tile
    the query tile cannot see).  Bytes: 2 KB per slot for B*H heads at
    d = 256 in the default mode and at d = 128 only in mode 2."""
    from oracle import attention as OA
    _, nqt, band = fa.fa_bwd_workspace(1, 1, T, 256, 256, W)
    assert nqt == (T + 31) // 32
    vis = OA.visibility(np.arange(T), np.arange(T), W if W < T else 0)
    qi, kj = np.nonzero(vis)
    slot = kj // 32 - qi // 32 + band - 1
    assert slot.min() >= 0 and slot.max() < band
    seen = np.zeros((nqt, band), dtype=bool)
    seen[qi // 32, slot] = True
    for qt in range(nqt):
        for j in range(band):
            kt = qt - band + 1 + j
            assert seen[qt, j] == (kt >= 0), (qt, j, kt)
    prev = fa.fa_set_dq_mode(0)
    try:
        assert fa.fa_bwd_workspace(2, 3, T, 256, 256, W)[0] == 2 * 3 * nqt * band * 2048
        assert fa.fa_bwd_workspace(2, 3, T, 128, 128, W)[0] == 0
        fa.fa_set_dq_mode(2)
        assert fa.fa_bwd_workspace(2, 3, T, 128, 128, W)[0] == 2 * 3 * nqt * band * 2048
        assert fa.fa_bwd_workspace(2, 3, T, 64, 64, W)[0] == 0
        fa.fa_set_dq_mode(1)
        assert fa.fa_bwd_workspace(2, 3, T, 256, 256, W)[0] == 0
    finally:
        fa.fa_set_dq_mode(prev)
    with pytest.raises(fa.FAError):
        fa.fa_bwd_workspace(1, 1, T, 96, 96, W)
