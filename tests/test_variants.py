"""Quantiser variants (naive INT2, clip only, Hadamard only, OSCAR) as
diagnostics through the oracle: their rotation factors and thresholds, the
error measures, and the pages' qualitative claim that rotating spreads
outlier channels and so beats plain INT2 on data with outliers."""
import numpy as np
import pytest

from bit_rotated_kv_int2_amd import synth
from oracle import oscar_ref as R
from oracle import variants as V

D = 128


@pytest.fixture(scope="module")
def tiny_head():
    """tiny-4k: one KV head, 4 query heads, 4 outlier channels x20."""
    wl = synth.WORKLOADS["tiny-4k"]
    q, k, v = synth.calibration_set(wl, 0, n_cal=512)
    qf, kf, vf = (synth.bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v))
    cal = R.calibrate_head(qf, kf[0], vf[0], 1 / np.sqrt(D))
    kb, vb = synth.kv_tokens(wl, 0, 0, 0, 2048)
    kt = synth.bf16_bits_to_f32(kb[:, 0]).astype(np.float64)
    vt = synth.bf16_bits_to_f32(vb[:, 0]).astype(np.float64)
    qd = synth.bf16_bits_to_f32(synth.decode_queries(wl, 0)[0]).astype(np.float64)
    qs = np.concatenate([qd, qf[:, :60].reshape(-1, D)])   # 4 decode + 240 calibration queries
    return cal, kf[0], vf[0], kt, vt, qs


def test_variant_rotations(tiny_head):
    cal, kc, vc, *_ = tiny_head
    naive = V.variant_calibration("naive", cal, kc, vc)
    clip = V.variant_calibration("clip", cal, kc, vc)
    had = V.variant_calibration("hadamard", cal, kc, vc)
    assert np.abs(R.composite_rotation(naive.U_K) - np.eye(D)).max() < 1e-6
    assert np.abs(R.composite_rotation(clip.U_V) - np.eye(D)).max() < 1e-6
    HP = R.hadamard_matrix(D) @ R.bitrev_matrix(D)
    assert np.abs(R.composite_rotation(had.U_K) - HP).max() < 1e-12
    assert V.variant_calibration("oscar", cal, kc, vc) is cal
    # naive: no clipping inside the calibration range; clip: the calibrated quantile
    assert abs(float(naive.tau_K) - np.abs(kc).max()) <= 1e-5 * np.abs(kc).max()
    assert abs(float(clip.tau_V) - np.quantile(np.abs(vc), 0.92)) <= 1e-5 * float(clip.tau_V)
    assert float(clip.tau_K) < float(naive.tau_K)
    with pytest.raises(ValueError):
        V.variant_calibration("other", cal, kc, vc)


def test_error_measures_basic():
    """KL of a distribution with itself is 0, and positive otherwise; with
    a clip threshold above every value and inputs on the metadata grid the
    quantised cache equals the input, so both errors vanish."""
    g = np.random.default_rng(1)
    s = g.standard_normal((5, 9))
    lp = V._log_softmax(s)
    assert np.allclose(V.kl_rows(lp, lp), 0.0, atol=1e-15)
    assert np.all(V.kl_rows(lp, V._log_softmax(s + g.standard_normal((5, 9)))) > 0)
    # tau = 382.5: zero step 3, scale step 1 (oracle pin); R = I
    U = V.identity_rotation_factor(D)
    z8 = g.integers(0, 200, size=(64, 2))
    s8 = np.minimum(g.integers(1, 86, size=(64, 2)), (255 - z8) // 3)
    c = g.integers(0, 4, size=(64, 2, 64))
    c[:, :, 0], c[:, :, 1] = 0, 3
    x = (3.0 * z8[..., None] - 382.5 + c * s8[..., None]).reshape(64, D)
    cal = R.HeadCalibration(U_K=U, U_V=U, tau_K=np.float32(382.5), tau_V=np.float32(382.5))
    # the write rotation with R = I is exact only up to float32 rounding of U
    xr = V.quantised_values(x, U, np.float32(382.5))
    assert np.abs(xr - x).max() < 1e-3
    kl, mse = V.attention_errors(g.standard_normal((6, D)) * 1e-3, x, x, cal, 1 / np.sqrt(D))
    assert kl < 1e-9 and mse < 1e-9


def test_rotation_beats_naive_int2_on_outliers(tiny_head):
    """[B] "为什么 INT2 KV 缓存量化很难" / "OSCAR 有何不同做法": outlier channels make
    plain INT2 fail; a rotation spreads them over all channels.  On the tiny
    workload (4 channels x20) every rotated variant beats naive and clip-only
    INT2 on the attention scores (KL), and naive INT2 on the output.  (With
    isotropic synthetic data and diffuse attention the output is small and
    its error is dominated by the clipping bias of V, shared by clip-only and
    the rotated variants, so that comparison is not pinned.)"""
    cal, kc, vc, kt, vt, qs = tiny_head
    errs = {kind: V.attention_errors(qs, kt, vt, V.variant_calibration(kind, cal, kc, vc), 1 / np.sqrt(D))
            for kind in V.KINDS}
    for rotated in ("hadamard", "oscar"):
        for plain in ("naive", "clip"):
            assert errs[rotated][0] < errs[plain][0], (rotated, plain, errs)
        assert errs[rotated][1] < errs["naive"][1], (rotated, errs)
    assert all(e[0] >= 0 and e[1] >= 0 for e in errs.values())
