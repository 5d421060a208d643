"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a closed
form, a textbook/library routine, an exhaustive enumeration, a hand-computed
value or a number printed by the pages (``tests/golden``).  They are chosen
so that a dropped term, a wrong sign or index, or a transposed operand in
``oracle/oscar_ref.py`` fails at least one of them.
"""
import json
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import oscar_ref as O
from bit_rotated_kv_int2_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")
D = 128


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rand_orthogonal(d, seed):
    g = np.random.default_rng(seed)
    q, r = np.linalg.qr(g.standard_normal((d, d)))
    return q * np.sign(np.diag(r))[None, :]


@pytest.fixture(scope="module")
def small_cal():
    """A calibrated head from a reduced calibration set (G = 2, N = 384)."""
    wl = synth.WORKLOADS["tiny-4k"]
    q, k, v = synth.calibration_set(wl, 0, n_cal=384)
    qf = synth.bf16_bits_to_f32(q)[:2]
    kf = synth.bf16_bits_to_f32(k)[0]
    vf = synth.bf16_bits_to_f32(v)[0]
    cal = O.calibrate_head(qf, kf, vf, 1.0 / np.sqrt(D))
    return cal, qf, kf, vf


# --- page constants -------------------------------------------------------

def test_defaults_match_pages():
    g = _golden()
    assert O.SINK_TOKENS == g["sink_tokens"]["value"]
    assert O.RECENT_TOKENS == g["recent_tokens"]["value"]
    assert O.GROUP_CHANNELS == g["group_channels"]["value"]
    assert O.CLIP_QUANTILE_K == g["clip_quantile_k"]["value"]
    assert O.CLIP_QUANTILE_V == g["clip_quantile_v"]["value"]
    assert O.CODES_PER_BYTE == g["codes_per_byte"]["value"]


def test_bit_accounting_reproduces_page_figures():
    """P-m: 2.25 history bits + BF16 windows gives the pages' 2.28 and 2.38."""
    g = _golden()
    hb = O.history_bits_per_element(metadata_bits_per_group=16)
    assert hb == g["rotation_int2_baselines_bpe"]["value"]
    for key in ("bpe_main", "bpe_aime_32k"):
        L = g[key]["context_tokens"]
        bpe = O.effective_bits_per_element(L, hb)
        assert round(bpe, 2) == g[key]["value"], (key, bpe)
    share = 100.0 * (O.SINK_TOKENS + O.RECENT_TOKENS) / g["bf16_window_share_percent_128k"]["context_tokens"]
    assert round(share, 2) == g["bf16_window_share_percent_128k"]["value"]
    # the stored format: 8-bit zero + 8-bit scale per 64-channel group
    assert O.history_bits_per_element() == 2.25
    assert abs(O.effective_bits_per_element(102400, 2.25) - (320 * 16 + 102080 * 2.25) / 102400) < 1e-12
    qt = O.quantize_int2(np.zeros((3, D), np.float32), np.float32(1.0))
    assert qt.s8.dtype == np.uint8 and qt.z8.dtype == np.uint8 and qt.s8.shape == (3, D // 64)


# --- Hadamard and butterfly (P-c) and Lemma 1 (P-b) -------------------------

def test_hadamard_matches_scipy_sylvester():
    for d in (2, 8, 64, 128):
        H = O.hadamard_matrix(d) * np.sqrt(d)
        assert np.array_equal(H, scipy.linalg.hadamard(d).astype(float))


def test_hadamard_orthogonal_involution():
    H = O.hadamard_matrix(D)
    assert np.max(np.abs(H @ H - np.eye(D))) < 1e-14
    assert np.array_equal(H, H.T)


def test_butterfly_equals_matrix():
    g = np.random.default_rng(1)
    x = g.standard_normal((5, D))
    a = O.fwht_butterfly(x) * O.inv_sqrt_dim(D)
    b = x @ O.hadamard_matrix(D)
    assert np.max(np.abs(a - b)) < 1e-13
    # unit vector e_j transforms to row j of the unnormalised matrix
    e = np.eye(D)[[0, 1, 37, 127]]
    assert np.array_equal(O.fwht_butterfly(e), scipy.linalg.hadamard(D)[[0, 1, 37, 127]].astype(float))


def test_inv_sqrt_dim_correctly_rounded():
    getcontext().prec = 60
    for d in (64, 128, 2, 32):
        exact = Decimal(1) / Decimal(d).sqrt()
        got = O.inv_sqrt_dim(d)
        # nearest double: error at most half an ulp
        err = abs(Fraction(got) - Fraction(exact))
        assert err <= Fraction(np.spacing(got)) / 2
    assert O.inv_sqrt_dim(128) == float.fromhex("0x1.6a09e667f3bcdp-4")


def test_lemma1_constant_diagonal():
    """[B] method, Lemma 1: diag(H^T Λ H) = tr(Λ)/d for any diagonal Λ."""
    g = np.random.default_rng(2)
    lam = np.sort(g.exponential(size=D))[::-1] * 10
    lam[:3] *= 100.0                         # spiked spectrum
    H = O.hadamard_matrix(D)
    M = H.T @ np.diag(lam) @ H
    assert np.max(np.abs(np.diag(M) - lam.sum() / D)) < 1e-12 * lam.sum()


def test_rotated_query_covariance_equalised(small_cal):
    """U diagonalises C_Q (descending); R = U H P equalises its diagonal."""
    cal, qf, _, _ = small_cal
    CQ = O.query_covariance(qf.reshape(-1, D))
    w, U = O.sorted_eigenbasis(CQ)
    Dg = U.T @ CQ @ U
    off = Dg - np.diag(np.diag(Dg))
    assert np.max(np.abs(off)) < 1e-12 * np.trace(CQ)
    assert np.all(np.diff(np.diag(Dg)) <= 1e-12)
    R = O.composite_rotation(U)
    diag = np.diag(R.T @ CQ @ R)
    assert np.max(np.abs(diag - np.trace(CQ) / D)) < 1e-12 * np.trace(CQ)
    # with the stored float32 basis the equalisation holds to float32 accuracy
    R32 = O.composite_rotation(cal.U_K)
    diag32 = np.diag(R32.T @ CQ @ R32)
    assert np.max(np.abs(diag32 - np.trace(CQ) / D)) < 1e-6 * np.trace(CQ)


# --- rotation orthogonality (P-a) -----------------------------------------

def test_rotation_orthogonal(small_cal):
    cal = small_cal[0]
    for U in (cal.U_K, cal.U_V):
        R = O.composite_rotation(U)
        assert np.max(np.abs(R.T @ R - np.eye(D))) < 2e-7
    U64 = _rand_orthogonal(D, 3)
    R = O.composite_rotation(U64)
    assert np.max(np.abs(R.T @ R - np.eye(D))) < 1e-13


# --- bit reversal (P-d) ----------------------------------------------------

def test_bitrev_values_and_involution():
    idx = O.bitrev_indices(D)
    assert idx[0] == 0 and idx[1] == 64 and idx[2] == 32 and idx[3] == 96 and idx[127] == 127
    assert idx[5] == 0b1010000
    assert np.array_equal(idx[idx], np.arange(D))
    P = O.bitrev_matrix(D)
    assert np.array_equal(P @ P, np.eye(D)) and np.array_equal(P, P.T)
    y = np.arange(D, dtype=float)
    assert np.array_equal(y @ P, y[idx])


def test_bitrev_balances_every_power_of_two_group():
    """[B] method: each power-of-two group of consecutive output channels takes
    one channel from every level of the input ordering (exhaustive)."""
    idx = O.bitrev_indices(D)
    size = 1
    while size <= D:
        levels = D // size                    # input channels per level
        for g0 in range(0, D, size):
            got = sorted(int(idx[p]) // levels for p in range(g0, g0 + size))
            assert got == list(range(size)), (size, g0)
        size *= 2


# --- packing (P-e) ----------------------------------------------------------

def test_pack_unpack_exhaustive():
    allb = np.arange(256, dtype=np.uint8)[None, :]
    codes = O.unpack_codes(allb)
    assert codes.shape == (1, 1024) and codes.max() == 3
    assert np.array_equal(O.pack_codes(codes), allb)
    assert O.pack_codes(np.array([[1, 0, 0, 0]]))[0, 0] == 1
    assert O.pack_codes(np.array([[0, 1, 0, 0]]))[0, 0] == 4
    assert O.pack_codes(np.array([[0, 0, 0, 2]]))[0, 0] == 128
    assert O.pack_codes(np.array([[3, 3, 3, 3, 2, 0, 1, 0]]))[0].tolist() == [255, 18]


# --- quantiser (P-f) ----------------------------------------------------------

def test_quantizer_grid_values_exact():
    """tau = 382.5: the zero grid (255 steps over [-tau, tau]) has step 3 and
    the scale grid (255 steps over [0, 2 tau / 3]) step 1, both exact, so
    zero = 3 z8 - 382.5 and scale = s8.  Values z + k s with the group's
    minimum and maximum present come back with codes k, metadata (z8, s8)
    and exact dequantised values."""
    g = np.random.default_rng(4)
    tau = np.float32(382.5)
    n = 64
    z8 = g.integers(0, 200, size=(n, 2))
    s8 = np.minimum(g.integers(1, 86, size=(n, 2)), (255 - z8) // 3)   # z + 3 s <= tau
    k = g.integers(0, 4, size=(n, 2, 64))
    k[:, :, 0] = 0
    k[:, :, 1] = 3
    x = (3.0 * z8[..., None] - 382.5 + k * s8[..., None]).reshape(n, D)
    assert np.all(np.abs(x) <= 382.5)
    qt = O.quantize_int2(x.astype(np.float32), tau)
    assert np.array_equal(qt.z8, z8) and np.array_equal(qt.s8, s8)
    assert np.array_equal(qt.codes, k.reshape(n, D))
    assert np.array_equal(O.dequantize_int2(qt.codes, qt.scale, qt.zero), x)


def test_quantizer_hand_example():
    """Hand-worked, tau = 382.5 (zero step 3, scale step 1):
    group 0 = {-351.1, -320, -337, -331, -306.1, rest -330}: min -351.1 ->
    (min + tau) / 3 = 10.467 -> z8 = 10, zero -352.5; range 45 -> s = 15 ->
    s8 = 15.  Codes: (-351.1 + 352.5) / 15 = 0.093 -> 0; -320 -> 2.167 -> 2;
    -337 -> 1.033 -> 1; -331 -> 1.433 -> 1; -306.1 -> 3.093 -> 3; -330 ->
    1.5, a tie, to the even code 2.
    group 1: every value 500 is clipped to tau: range 0 -> s8 = 0, all codes
    0; (tau + tau) / 3 = 255 -> z8 = 255."""
    x = np.full((1, D), -330.0, dtype=np.float32)
    x[0, :5] = [-351.1, -320.0, -337.0, -331.0, -306.1]
    x[0, 64:] = 500.0
    qt = O.quantize_int2(x, np.float32(382.5))
    assert qt.z8[0].tolist() == [10, 255] and qt.s8[0].tolist() == [15, 0]
    assert qt.zero[0, 0] == np.float32(-352.5) and qt.scale[0, 0] == np.float32(15.0)
    assert qt.codes[0, :6].tolist() == [0, 2, 1, 1, 3, 2]
    assert np.all(qt.codes[0, 64:] == 0) and qt.scale[0, 1] == 0


def test_quantizer_degenerate():
    """tau = 0 clips everything to 0: all metadata and codes are 0.  A constant
    group has scale code 0 and its zero within half a zero step."""
    qt = O.quantize_int2(np.random.default_rng(9).standard_normal((4, D)).astype(np.float32), np.float32(0.0))
    assert not qt.codes.any() and not qt.s8.any() and not qt.z8.any()
    assert np.all(qt.zero == 0) and np.all(qt.scale == 0)
    x = np.full((1, D), 0.37, dtype=np.float32)
    qt = O.quantize_int2(x, np.float32(2.0))
    assert np.all(qt.s8 == 0) and not qt.codes.any()
    assert np.all(np.abs(qt.zero.astype(np.float64) - 0.37) <= 0.5 * 4.0 / 255 + 1e-6)


def test_quantizer_properties():
    """Random tokens: codes in [0, 3], group min -> code 0, group max -> code 3
    (up to the metadata rounding), and every dequantised value within half a
    scale step plus the metadata rounding (half a zero step 2 tau / 255, and
    three times half a scale step 2 tau / 765) of the clipped value."""
    g = np.random.default_rng(5)
    x = (g.standard_normal((200, D)) * 3).astype(np.float32)
    tau = np.float32(4.0)
    qt = O.quantize_int2(x, tau)
    xc = np.clip(x, -tau, tau).reshape(200, 2, 64).astype(np.float64)
    c = qt.codes.reshape(200, 2, 64)
    assert c.max() <= 3
    zs, ss = 2 * 4.0 / 255, 2 * 4.0 / 765
    z = qt.zero.astype(np.float64)[..., None]
    s = qt.scale.astype(np.float64)[..., None]
    assert np.all(np.abs(z - xc.min(-1, keepdims=True)) <= zs / 2 * (1 + 1e-5))
    assert np.all(np.abs(s - (xc.max(-1, keepdims=True) - xc.min(-1, keepdims=True)) / 3) <= ss / 2 * (1 + 1e-5))
    xh = O.dequantize_int2(qt.codes, qt.scale, qt.zero).reshape(200, 2, 64)
    bound = s / 2 + zs / 2 + 3 * ss / 2 + 1e-5
    assert np.all(np.abs(xh - xc) <= bound)


# --- write-path rotation ------------------------------------------------------

def test_rotate_for_write_matches_dense_rotation(small_cal):
    """The fixed-order write rotation equals x @ (U H P) computed by BLAS."""
    cal = small_cal[0]
    g = np.random.default_rng(7)
    x = synth.bf16_round(g.standard_normal((64, D)).astype(np.float32))[1].astype(np.float64)
    a = O.rotate_for_write(x, cal.U_K).astype(np.float64)
    b = x @ O.composite_rotation(cal.U_K)
    assert np.max(np.abs(a - b)) <= 2.0 ** -23 * np.max(np.abs(b))
    # and the forward rotation inverts with R^T
    assert np.max(np.abs(a @ O.composite_rotation(cal.U_K).T - x)) < 1e-5


def test_rotate_for_write_identity_basis():
    """U = I: the write rotation is the normalised Hadamard followed by bit
    reversal; for x = e_0 every output is +1/sqrt(d) exactly (float32)."""
    x = np.zeros((1, D))
    x[0, 0] = 1.0
    y = O.rotate_for_write(x, np.eye(D, dtype=np.float32))
    assert np.all(y == np.float32(1 / np.sqrt(D)))
    x = np.zeros((1, D))
    x[0, 1] = 2.0                          # row 1 of H alternates sign
    y = O.rotate_for_write(x, np.eye(D, dtype=np.float32))
    idx = O.bitrev_indices(D)
    want = np.where(idx % 2 == 0, 2.0, -2.0) / np.sqrt(D)
    assert np.array_equal(y[0], want.astype(np.float32))


# --- softmax merge (P-g), attention (P-i, P-j), logit identity (P-h) ------------

def test_lse_merge_equals_single_softmax():
    g = np.random.default_rng(8)
    q = g.standard_normal((3, 16))
    K = g.standard_normal((50, 16)) * 2
    V = g.standard_normal((50, 16))
    full = O.attention_dense(q, K, V, 0.3)
    cuts = [0, 0, 7, 7, 20, 49, 50, 50]
    parts = [O.segment_partial(q, K[a:b], V[a:b], 0.3) for a, b in zip(cuts[:-1], cuts[1:])]
    m = O.lse_merge(parts)
    assert np.max(np.abs(m.o / m.l[:, None] - full)) < 1e-13


def test_attention_dense_matches_torch_sdpa():
    g = np.random.default_rng(9)
    q = g.standard_normal((4, D))
    K = g.standard_normal((300, D))
    V = g.standard_normal((300, D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(K)[None, None].expand(1, 4, 300, D),
        torch.from_numpy(V)[None, None].expand(1, 4, 300, D), scale=1 / np.sqrt(D))[0, :, 0]
    assert np.max(np.abs(O.attention_dense(q, K, V, 1 / np.sqrt(D)) - ref.numpy())) < 1e-12


def test_logit_error_identity(small_cal):
    """[B] method: ||QK^T - QK^^T||_F^2 = tr((K - K^) Q^T Q (K - K^)^T), with K^
    the oracle's dequantised, inverse-rotated keys."""
    cal, qf, kf, _ = small_cal
    Q = qf[0, :7].astype(np.float64)
    K = kf[:5].astype(np.float64)
    qt = O.write_history(K, cal.U_K, cal.tau_K)
    Kh = O.dequantize_int2(qt.codes, qt.scale, qt.zero) @ O.composite_rotation(cal.U_K).T
    lhs = np.sum((Q @ K.T - Q @ Kh.T) ** 2)
    E = K - Kh
    rhs = np.trace(E @ Q.T @ Q @ E.T)
    assert abs(lhs - rhs) <= 1e-12 * abs(lhs)
    assert lhs > 0


def _tiny_pool(L, seed=10):
    wl = synth.WORKLOADS["tiny-4k"]
    q, k, v = synth.calibration_set(wl, 0, n_cal=256)
    cal = O.calibrate_head(synth.bf16_bits_to_f32(q), synth.bf16_bits_to_f32(k)[0],
                           synth.bf16_bits_to_f32(v)[0], 1 / np.sqrt(D))
    kb, vb = synth.kv_tokens(wl, 0, 0, 0, L)
    K = synth.bf16_bits_to_f32(kb)[:, 0].astype(np.float64)
    V = synth.bf16_bits_to_f32(vb)[:, 0].astype(np.float64)
    pool = O.build_head_pool(K, V, cal)
    qd = synth.bf16_bits_to_f32(synth.decode_queries(wl, 0))[0].astype(np.float64)
    return pool, cal, qd, K, V


def test_segmented_equals_dense_decode():
    pool, cal, q, _, _ = _tiny_pool(1000)
    a = O.decode_head_dense(q, pool, cal, 1 / np.sqrt(D))
    b = O.decode_head_segmented(q, pool, cal, 1 / np.sqrt(D))
    assert np.max(np.abs(a - b)) < 1e-12


def test_decode_brute_force_loop():
    """Token-by-token loop with math.exp over the dequantised cache (P-i)."""
    import math
    pool, cal, q, _, _ = _tiny_pool(400)
    Kh, Vh = O.dequantized_head_cache(pool, cal)
    ref = O.decode_head_dense(q, pool, cal, 1 / np.sqrt(D))
    sm = 1 / math.sqrt(D)
    for h in range(q.shape[0]):
        logits = [sm * sum(float(q[h, c]) * float(Kh[t, c]) for c in range(D)) for t in range(Kh.shape[0])]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        tot = sum(w)
        for c in (0, 5, 77, 127):
            o = sum(w[t] * float(Vh[t, c]) for t in range(len(w))) / tot
            assert abs(o - ref[h, c]) < 1e-12


def test_short_sequences_reduce_to_bf16_attention():
    """P-j: L <= S0 + W has no history, so decode is plain attention on bf16."""
    for L in (1, 64, 65, 320):
        pool, cal, q, K, V = _tiny_pool(L)
        assert pool.hist_k.codes.shape[0] == 0
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[:, None, :], torch.from_numpy(K)[None].expand(4, L, D),
            torch.from_numpy(V)[None].expand(4, L, D), scale=1 / np.sqrt(D))[:, 0]
        assert np.max(np.abs(O.decode_head_dense(q, pool, cal, 1 / np.sqrt(D)) - ref.numpy())) < 1e-12


def test_pool_regions():
    assert O.pool_regions(10) == ((0, 10), (10, 10), (10, 10))
    assert O.pool_regions(64) == ((0, 64), (64, 64), (64, 64))
    assert O.pool_regions(300) == ((0, 64), (64, 64), (64, 300))
    assert O.pool_regions(320) == ((0, 64), (64, 64), (64, 320))
    assert O.pool_regions(321) == ((0, 64), (64, 65), (65, 321))
    assert O.pool_regions(4096) == ((0, 64), (64, 3840), (3840, 4096))   # 64 + 3776 + 256


# --- calibration (P-l) --------------------------------------------------------

def test_eigenbasis_recovers_known_basis():
    Q = _rand_orthogonal(D, 11)
    lam = np.linspace(100.0, 1.0, D)
    C = Q @ np.diag(lam) @ Q.T
    w, U = O.sorted_eigenbasis(C)
    assert np.max(np.abs(w - lam)) < 1e-10
    for j in range(D):
        col = Q[:, j] * (1 if Q[np.argmax(np.abs(Q[:, j])), j] > 0 else -1)
        assert np.max(np.abs(U[:, j] - col)) < 1e-9


def test_eigenbasis_rejects_degenerate():
    with pytest.raises(ValueError):
        O.sorted_eigenbasis(np.eye(8))


def test_query_covariance_closed_form():
    q = np.zeros((4, 8))
    q[0, 0], q[1, 1], q[2, 1], q[3, 7] = 2.0, 1.0, -3.0, 1.0
    C = O.query_covariance(q)
    assert np.array_equal(C, np.diag([4, 10, 0, 0, 0, 0, 0, 1]) / 4.0)


def test_score_weighted_covariance_special_cases():
    g = np.random.default_rng(12)
    q = g.standard_normal((2, 5, 8))
    V = g.standard_normal((6, 8))
    # identical keys: every score row is uniform, S V = mean(V) for every row
    K = np.tile(g.standard_normal((1, 8)), (6, 1))
    mu = V.mean(axis=0)
    assert np.max(np.abs(O.score_weighted_value_covariance(q, K, V, 0.7) - np.outer(mu, mu))) < 1e-13
    # one key: C_S = v^T v
    C1 = O.score_weighted_value_covariance(q, K[:1], V[:1], 0.7)
    assert np.max(np.abs(C1 - np.outer(V[0], V[0]))) < 1e-13
    # very peaked scores (keys = scaled queries' directions) pick single values
    Kp = np.eye(8)[:6] * 1e3
    qp = np.zeros((1, 6, 8))
    qp[0, np.arange(6), np.arange(6)] = 1.0
    Cp = O.score_weighted_value_covariance(qp, Kp, V, 1.0)
    assert np.max(np.abs(Cp - V.T @ V / 6)) < 1e-12


def test_clip_threshold_uses_rotated_values():
    """x = diag(a) R^T makes |x R| = diag(a): the quantile is over those
    d^2 values (d^2 - d zeros and the a's), linear interpolation."""
    U = _rand_orthogonal(D, 13).astype(np.float32)
    R = O.composite_rotation(U)
    a = np.arange(1, D + 1, dtype=np.float64)
    x = np.diag(a) @ R.T
    n = D * D
    qv = 0.9995
    pos = qv * (n - 1)                      # sorted: zeros first, then 1..128
    lo = int(np.floor(pos))
    frac = pos - lo
    def val(i):
        return 0.0 if i < n - D else float(i - (n - D) + 1)
    want = val(lo) + frac * (val(lo + 1) - val(lo))
    got = O.clip_threshold(x, U, qv)
    assert abs(float(got) - want) <= 1e-4 * want


def test_calibration_thresholds_reasonable(small_cal):
    cal, _, kf, vf = small_cal
    assert 0 < cal.tau_K and 0 < cal.tau_V
    rk = np.abs(kf.astype(np.float64) @ O.composite_rotation(cal.U_K))
    assert abs(np.mean(rk <= cal.tau_K) - 0.96) < 1e-3
    rv = np.abs(vf.astype(np.float64) @ O.composite_rotation(cal.U_V))
    assert abs(np.mean(rv <= cal.tau_V) - 0.92) < 1e-3


# --- calibration wiring: which covariance feeds which basis -----------------

def _one_hot_calibration_set(seed=21, n=256, G=2, scale=1e4):
    """Queries that are large multiples of the calibration keys, one key per
    query (a permutation per head): every softmax score row is exactly one-hot
    in float64, so S V selects value rows and C_S = V^T V / n, while
    C_Q = scale^2 K^T K / n."""
    g = np.random.default_rng(seed)
    K = g.standard_normal((n, D))
    V = g.standard_normal((n, D)) * np.linspace(3.0, 0.5, D)[None, :]
    q = np.stack([scale * K[g.permutation(n)] for _ in range(G)])
    return q, K, V


def _basis_matches(U, C, tol):
    """True if the columns of U are the eigenvectors of C by descending
    eigenvalue, up to sign (scipy's symmetric eigensolver as the reference)."""
    w, E = scipy.linalg.eigh(C)
    E = E[:, ::-1]
    dots = np.abs(np.sum(E * np.asarray(U, dtype=np.float64), axis=0))
    return bool(np.all(dots > 1.0 - tol))


def test_calibrate_head_value_basis_from_score_weighted_values():
    """[B] method: R_V comes from C_S = V^T S^T S V and R_K from C_Q.  With
    one-hot scores C_S reduces to V^T V / n, so U_V must be the eigenbasis of
    the value Gram matrix and U_K that of the key Gram matrix; a basis built
    from the wrong operand (keys for values, or the query covariance) fails."""
    q, K, V = _one_hot_calibration_set()
    n = K.shape[0]
    cal = O.calibrate_head(q, K, V, 1 / np.sqrt(D))
    assert _basis_matches(cal.U_V, V.T @ V / n, 1e-5)
    assert _basis_matches(cal.U_K, K.T @ K / n, 1e-5)
    w = scipy.linalg.eigh(V.T @ V / n, eigvals_only=True)[::-1]
    assert np.max(np.abs(cal.eig_V - w)) < 1e-10 * w[0]
    # the plausible wiring mistakes would not pass the same check
    assert not _basis_matches(cal.U_K, V.T @ V / n, 1e-5)
    swapped = O.calibrate_head(q, V, K, 1 / np.sqrt(D))      # keys and values exchanged
    assert not _basis_matches(swapped.U_V, V.T @ V / n, 1e-5)


def test_lemma1_on_calibrated_value_rotation(small_cal):
    """Lemma 1 ([B] method) on the calibrated value rotation: R_V^T C_S R_V has
    the constant diagonal tr(C_S) / d only if U_V diagonalises the C_S of the
    same calibration data.  The basis a key/value swap would give does not."""
    cal, qf, kf, vf = small_cal
    CS = O.score_weighted_value_covariance(qf, kf, vf, 1 / np.sqrt(D))
    tr = np.trace(CS)
    R = O.composite_rotation(cal.U_V)
    assert np.max(np.abs(np.diag(R.T @ CS @ R) - tr / D)) < 1e-6 * tr
    Dg = cal.U_V.astype(np.float64).T @ CS @ cal.U_V.astype(np.float64)
    assert np.all(np.diff(np.diag(Dg)) <= 1e-6 * tr)          # descending eigenvalues
    _, Uw = O.sorted_eigenbasis(O.score_weighted_value_covariance(qf, vf, kf, 1 / np.sqrt(D)))
    Rw = O.composite_rotation(Uw.astype(np.float32))
    assert np.max(np.abs(np.diag(Rw.T @ CS @ Rw) - tr / D)) > 1e-3 * tr


# --- decode_sequence: query head h reads KV head h // G ----------------------

def test_decode_sequence_gqa_head_mapping():
    """Query head h reads KV head h // (Hq / Hkv) (grouped-query attention):
    checked against torch SDPA's grouped-query mode over the oracle's
    dequantised caches, with two KV heads holding different data."""
    wl = synth.WORKLOADS["tiny-4k"]
    qc, kc, vc = synth.calibration_set(wl, 0, n_cal=256)
    f = synth.bf16_bits_to_f32
    Hkv, G, L = 2, 3, 700
    pools, cals = [], []
    for kv in range(Hkv):
        cal = O.calibrate_head(f(qc)[:G] * (1 + kv), f(kc)[0] * (1 - 0.4 * kv), f(vc)[0], 1 / np.sqrt(D))
        kb, vb = synth.kv_tokens(wl, kv, kv, 0, L)      # layer / sequence index as a different seed
        K = f(kb)[:, 0].astype(np.float64) * (1 + 2 * kv)
        V = f(vb)[:, 0].astype(np.float64) + 3.0 * kv
        pools.append(O.build_head_pool(K, V, cal))
        cals.append(cal)
    g = np.random.default_rng(22)
    q = g.standard_normal((Hkv * G, D))
    out = O.decode_sequence(q, pools, cals, 1 / np.sqrt(D))
    caches = [O.dequantized_head_cache(p, c) for p, c in zip(pools, cals)]
    Kt = torch.from_numpy(np.stack([c[0] for c in caches]))[None]
    Vt = torch.from_numpy(np.stack([c[1] for c in caches]))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], Kt, Vt, scale=1 / np.sqrt(D), enable_gqa=True)[0, :, 0]
    assert np.max(np.abs(out - ref.numpy())) < 1e-12
    # the interleaved mapping h % Hkv gives a different answer on these heads
    wrong = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], Kt.repeat(1, G, 1, 1), Vt.repeat(1, G, 1, 1),
        scale=1 / np.sqrt(D))[0, :, 0]
    assert np.max(np.abs(out - wrong.numpy())) > 0.1


# --- Lloyd-Max codebook -------------------------------------------------------

def test_lloyd_max_gaussian_fixed_point():
    """On the unit Gaussian the 4-level Lloyd-Max quantiser converges to the
    textbook levels +-0.4528, +-1.5104 with thresholds 0, +-0.9816 (Max's
    table).  The distribution is a fine deterministic quantile grid."""
    from scipy.stats import norm
    N = 400_000
    x = norm.ppf((np.arange(N) + 0.5) / N)
    c = O.lloyd_max(x, [-1.5, -0.5, 0.5, 1.5])
    assert np.max(np.abs(c - np.array([-1.5104, -0.4528, 0.4528, 1.5104]))) < 3e-4
    t = (c[:-1] + c[1:]) / 2
    assert np.max(np.abs(t - np.array([-0.9816, 0.0, 0.9816]))) < 3e-4


def test_lloyd_max_uniform_equally_spaced():
    """On a uniform distribution over [0, 3] the optimum is the four cell
    centres 3/8, 9/8, 15/8, 21/8 (equal cells of width 3/4)."""
    N = 120_000
    x = (np.arange(N) + 0.5) / N * 3.0
    c = O.lloyd_max(x, [0.0, 1.0, 2.0, 3.0])
    assert np.max(np.abs(c - np.array([3, 9, 15, 21]) / 8.0)) < 1e-4


def test_uniform_codebook_is_the_rounding_quantiser():
    """The codebook (0, 32, 64, 96) / 32 reproduces the plain quantiser bit for
    bit: its thresholds 0.5, 1.5, 2.5 with the tie rule (middle up, outer
    down) equal clamp(rint(u), 0, 3) with rounding half to even, exact
    half-way values included; end to end on random tokens too."""
    t = O.level_thresholds(O.UNIFORM_LEVELS)
    assert np.array_equal(t, np.array([0.5, 1.5, 2.5], np.float32))
    u = np.concatenate([np.arange(-8, 40, dtype=np.float32) / 8,
                        np.nextafter(np.float32([0.5, 1.5, 2.5]), np.float32(9)),
                        np.nextafter(np.float32([0.5, 1.5, 2.5]), np.float32(-9))])
    by_threshold = (u > t[0]).astype(int) + (u >= t[1]).astype(int) + (u > t[2]).astype(int)
    assert np.array_equal(by_threshold, np.clip(np.rint(u), 0, 3).astype(int))
    g = np.random.default_rng(30)
    x = g.standard_normal((300, D)).astype(np.float32) * 2
    tau = np.float32(4.0)
    base = O.quantize_int2(x, tau)
    a = O.quantize_int2(x, tau, levels=O.UNIFORM_LEVELS)
    assert np.array_equal(a.codes, base.codes) and np.array_equal(a.s8, base.s8) and np.array_equal(a.z8, base.z8)
    assert np.array_equal(O.dequantize_int2(a.codes, a.scale, a.zero, levels=a.levels),
                          O.dequantize_int2(base.codes, base.scale, base.zero))


def test_codebook_code_choice_by_hand():
    """Levels (0, 20, 50, 96) / 32: thresholds 0.3125, 1.09375, 2.28125; a tie
    at the middle threshold goes up, at the outer ones down; the decoded value
    is z^ + s^ n[code] / 32."""
    lv = np.array([0, 20, 50, 96], np.uint8)
    t = O.level_thresholds(lv)
    assert np.array_equal(t, np.array([0.3125, 1.09375, 2.28125], np.float32))
    # one group with z^ = -2 (z8 = 0 at tau = 2... grid a = 4/255) and a value per probe
    tau = np.float32(2.0)
    a, b = O.metadata_steps(tau)
    x = np.full((1, D), -2.0, np.float32)
    x[0, 1] = 2.0                       # group 0 spans [-2, 2]: z8 = 0, s = 4/3
    probes = [0.0, 0.3125, 0.4, 1.09375, 1.2, 2.28125, 2.5, 3.0]
    qt0 = O.quantize_int2(x, tau)
    zf, sf = qt0.zero[0, 0], qt0.scale[0, 0]
    for i, u in enumerate(probes):
        x[0, 2 + i] = zf + sf * np.float32(u)
    qt = O.quantize_int2(x, tau, levels=lv)
    zf, sf = qt.zero[0, 0], qt.scale[0, 0]
    for i, u in enumerate(probes):
        uu = (x[0, 2 + i] - zf) / sf                          # float32, as the quantiser sees it
        want = int(uu > t[0]) + int(uu >= t[1]) + int(uu > t[2])
        assert qt.codes[0, 2 + i] == want, (u, uu)
    deq = O.dequantize_int2(qt.codes, qt.scale, qt.zero, levels=lv)
    assert deq[0, 1] == float(zf) + float(sf) * 96 / 32


def test_codebook_levels_calibrated():
    """Calibrated levels are strictly increasing integers in [0, 96] and, being
    the Lloyd-Max levels of the calibration values, lower the reconstruction
    error of those values below the uniform grid's."""
    wl = synth.WORKLOADS["tiny-4k"]
    q, k, v = synth.calibration_set(wl, 0, n_cal=1024)
    f = synth.bf16_bits_to_f32
    cal = O.calibrate_head(f(q), f(k)[0], f(v)[0], 1 / np.sqrt(D))
    cb = O.calibrate_codebook(cal, f(k)[0], f(v)[0])
    for lv in (cb.levels_K, cb.levels_V):
        assert lv.dtype == np.uint8 and np.all(np.diff(lv.astype(int)) >= 1) and lv[-1] <= 96
    for x, U, tau, lv in ((f(k)[0], cal.U_K, cal.tau_K, cb.levels_K), (f(v)[0], cal.U_V, cal.tau_V, cb.levels_V)):
        xr = O.rotate_for_write(x.astype(np.float64), U).astype(np.float64)
        xc = np.clip(xr, -float(tau), float(tau))
        errs = []
        for levels in (None, lv):
            qt = O.quantize_int2(xr.astype(np.float32), tau, levels=levels)
            errs.append(np.mean((O.dequantize_int2(qt.codes, qt.scale, qt.zero, levels=levels) - xc) ** 2))
        assert errs[1] < 0.95 * errs[0], errs


def test_codebook_levels_degenerate_samples():
    """All samples equal: every cell but one stays at its start, and the
    stored levels are still strictly increasing inside [0, 96]."""
    lv = O.codebook_levels(np.full(1000, 3.0))
    assert np.all(np.diff(lv.astype(int)) >= 1) and lv[0] >= 0 and lv[-1] <= 96
    lv = O.codebook_levels(np.zeros(1000))
    assert np.all(np.diff(lv.astype(int)) >= 1) and lv[0] == 0
