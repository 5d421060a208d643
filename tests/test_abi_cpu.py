"""Host-side checks of the C ABI (no GPU needed).

* liboscar.so loads and exports every function ``include/oscar.h`` declares;
* argument validation rejects bad calls before any device work;
* host calibration (``oscar_calibrate_rotation``) agrees with the oracle.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from bit_rotated_kv_int2_amd import oscar as O
from bit_rotated_kv_int2_amd import synth
from oracle import oscar_ref as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar.h")

pytestmark = pytest.mark.skipif(not os.path.exists(O.LIB_PATH), reason="liboscar.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oscar_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(O.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(O.EXPORTED)


def test_header_layout_constants_match_binding():
    text = open(HEADER).read()
    for macro, val in [("OSCAR_PAGE_BYTES", O.PAGE_BYTES), ("OSCAR_PAGE_VCODES", O.PAGE_VCODES),
                       ("OSCAR_PAGE_KMETA", O.PAGE_KMETA), ("OSCAR_PAGE_VMETA", O.PAGE_VMETA),
                       ("OSCAR_HEAD_DIM", O.HEAD_DIM), ("OSCAR_PAGE_TOKENS", O.PAGE_TOKENS)]:
        m = re.search(rf"#define {macro} (\d+)", text)
        assert m and int(m.group(1)) == val, macro
    # 64 tokens x (2 x 32 code bytes + 2 x 8 metadata bytes) per page
    assert O.PAGE_BYTES == 64 * (32 + 32 + 4 + 4)


def _fake_pool(batch=1):
    # non-NULL but never dereferenced: validation fails first
    return O.KVPoolC(*([0x1000] * 10), batch, 4, 4, batch)


def _call_decode(params, pool=None, ws_bytes=1 << 30, opts=None):
    L = O.lib()
    rot = O.Rotation(0x1000, 0x1000, 0x1000, 0x1000)
    pool = pool or _fake_pool()
    return L.oscar_decode_attention(ctypes.byref(params), ctypes.byref(rot), ctypes.byref(pool),
                                    0x1000, 0x1000, None if opts is None else ctypes.byref(opts),
                                    0x1000, ws_bytes, None)


def test_validation_errors():
    L = O.lib()
    assert _call_decode(O.make_params(8, 32, head_dim=64)) == O.OSCAR_ENOTSUP
    assert _call_decode(O.make_params(8, 30)) == O.OSCAR_EINVAL
    assert _call_decode(O.make_params(1, 32)) == O.OSCAR_ENOTSUP        # G = 32 > 16
    assert _call_decode(O.make_params(8, 32, sink=32)) == O.OSCAR_ENOTSUP
    assert _call_decode(O.make_params(8, 32, sm_scale=-1.0)) == O.OSCAR_EINVAL
    assert _call_decode(O.make_params(8, 32), ws_bytes=16) == O.OSCAR_EWORKSPACE
    assert b"workspace" in L.oscar_last_error()
    bad = _fake_pool()
    bad.seq_lens = None
    assert _call_decode(O.make_params(8, 32), pool=bad) == O.OSCAR_EINVAL
    p = O.make_params(8, 32)
    rot = O.Rotation(0x1000, 0x1000, 0x1000, 0x1000)
    pool = _fake_pool()
    assert L.oscar_quantize_append(ctypes.byref(p), ctypes.byref(rot), ctypes.byref(pool),
                                   0x1000, 0x1000, 0, None) == O.OSCAR_EINVAL
    assert L.oscar_quantize_append(ctypes.byref(p), None, ctypes.byref(pool),
                                   0x1000, 0x1000, 1, None) == O.OSCAR_EINVAL
    # device tensors read 16 bytes at a time must be 16-byte aligned
    assert L.oscar_decode_attention(ctypes.byref(p), ctypes.byref(rot), ctypes.byref(pool),
                                    0x1008, 0x1000, None, 0x1000, 1 << 30, None) == O.OSCAR_EINVAL
    assert b"aligned" in L.oscar_last_error()
    assert L.oscar_decode_attention(ctypes.byref(p), ctypes.byref(O.Rotation(0x1004, 0x1000, 0x1000, 0x1000)),
                                    ctypes.byref(pool), 0x1000, 0x1000, None, 0x1000, 1 << 30, None) == O.OSCAR_EINVAL
    bad = _fake_pool()
    bad.pages = 0x1002
    assert _call_decode(p, pool=bad) == O.OSCAR_EINVAL
    assert L.oscar_quantize_append(ctypes.byref(p), ctypes.byref(rot), ctypes.byref(pool),
                                   0x1000, 0x1010 + 2, 1, None) == O.OSCAR_EINVAL
    # per-call decode options: checked before anything else is looked at
    for bad_opts in (O.decode_options(2, 0), O.decode_options(7, 0), O.decode_options(-1, 0), O.decode_options(0, -1),
                     O.decode_options(0, 65537)):
        assert _call_decode(p, opts=bad_opts) == O.OSCAR_EINVAL
        assert b"options" in L.oscar_last_error()
    p8 = O.make_params(8, 32)
    ws = lambda opts: L.oscar_decode_workspace_size(ctypes.byref(p8), 1, 1600,
                                                    None if opts is None else ctypes.byref(opts))
    default_ws = ws(None)
    assert default_ws == ws(O.decode_options(0, 0)) == ws(O.decode_options(0, 256))
    assert 0 < ws(O.decode_options(0, 8)) < default_ws       # one split per (sequence, KV head): fewer partials
    assert ws(O.decode_options(0, -1)) == 0 and ws(O.decode_options(3, 0)) == 0
    assert ws(None) == default_ws                           # nothing is kept between calls
    # shared-prefix decode: MFMA variant, at most max_pages prefix pages
    p12 = O.make_params(8, 96)
    ws12 = lambda opts, mp=1600: L.oscar_decode_workspace_size(ctypes.byref(p12), 16, mp, ctypes.byref(opts))
    assert ws12(O.decode_options(0, 0, 1535)) > ws12(O.decode_options(0, 0, 0)) > 0   # prefix partials + operands
    assert ws12(O.decode_options(0, 0, 1600)) > 0
    assert ws12(O.decode_options(0, 0, 1601)) == 0
    assert ws12(O.decode_options(1, 0, 10)) == 0
    assert ws12(O.decode_options(0, 0, -1)) == 0
    assert ws(O.decode_options(0, 0, 10)) > default_ws      # G = 4: prefix partials and query operands
    for bad_opts, what in ((O.decode_options(0, 0, -1), b"prefix_pages"), (O.decode_options(1, 0, 4), b"variant 0")):
        assert _call_decode(p12, opts=bad_opts) == O.OSCAR_EINVAL
        assert what in L.oscar_last_error()
    assert _call_decode(p, opts=O.decode_options(0, 0, 5)) == O.OSCAR_EINVAL   # more than max_pages = 4
    assert b"max_pages" in L.oscar_last_error()
    assert L.oscar_decode_workspace_size(ctypes.byref(O.make_params(8, 30)), 1, 10, None) == 0
    with pytest.raises(O.OscarError):
        O.calibrate_rotation(O.make_params(1, 1), np.zeros((1, 8, 128), np.float32),
                             np.zeros((1, 8, 128), np.float32), np.zeros((1, 8, 128), np.float32))


def test_workspace_size_monotone():
    p = O.make_params(8, 32)
    a = O.decode_workspace_size(p, 1, 100)
    b = O.decode_workspace_size(p, 32, 1600)
    assert 0 < a < b and a % 256 == 0


@pytest.mark.slow
def test_calibration_matches_oracle():
    wl = synth.WORKLOADS["tiny-4k"]
    q, k, v = synth.calibration_set(wl, 0, n_cal=256)
    qf, kf, vf = (synth.bf16_bits_to_f32(x) for x in (q, k, v))
    p = O.make_params(1, 4)
    UK, UV, tK, tV = O.calibrate_rotation(p, qf, kf, vf)
    ref = R.calibrate_head(qf, kf[0], vf[0], 1 / np.sqrt(128))
    # float32 bases agree to rounding of the float64 eigenvectors
    assert np.max(np.abs(UK[0] - ref.U_K)) <= 2e-7
    assert np.max(np.abs(UV[0] - ref.U_V)) <= 2e-7
    assert abs(float(tK[0]) - float(ref.tau_K)) <= 2 * np.spacing(np.float32(ref.tau_K))
    assert abs(float(tV[0]) - float(ref.tau_V)) <= 2 * np.spacing(np.float32(ref.tau_V))


@pytest.mark.slow
def test_codebook_calibration_matches_oracle():
    """oscar_calibrate_codebook (host C++) against the oracle's Lloyd-Max
    codebook on the same rotation artifact and calibration tokens."""
    wl = synth.WORKLOADS["tiny-4k"]
    q, k, v = synth.calibration_set(wl, 0, n_cal=512)
    f = synth.bf16_bits_to_f32
    qf, kf, vf = f(q), f(k), f(v)
    cal = R.calibrate_head(qf, kf[0], vf[0], 1 / np.sqrt(128))
    cb = R.calibrate_codebook(cal, kf[0], vf[0])
    p = O.make_params(1, 4)
    wk = O.calibrate_codebook(p, cal.U_K[None], np.array([cal.tau_K], np.float32), kf)
    wv = O.calibrate_codebook(p, cal.U_V[None], np.array([cal.tau_V], np.float32), vf)
    assert int(wk[0]) == O.levels_word(cb.levels_K), (hex(int(wk[0])), cb.levels_K)
    assert int(wv[0]) == O.levels_word(cb.levels_V), (hex(int(wv[0])), cb.levels_V)
    with pytest.raises(O.OscarError):
        O.calibrate_codebook(p, cal.U_K[None], np.array([cal.tau_K], np.float32), kf[:, :0])
