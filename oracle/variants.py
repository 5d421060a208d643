"""Quantiser variants of the rotated-INT2 cache, as diagnostics.

TEST INFRASTRUCTURE ONLY, under the same rules as ``oscar_ref``: only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it, and the library never does.

The pages compare OSCAR against plain INT2 quantisation, against a Hadamard
rotation alone, and against clipping alone ([B] "为什么 INT2 KV 缓存量化很难" and
"OSCAR 有何不同做法"; [A] the comparison under "OSCAR 的设计思路"), by how far the
quantised cache moves the attention scores and the attention output.  Every
variant here is the same write path (``oscar_ref.write_history``) with another
rotation factor U and clip threshold tau, so the library runs them unchanged:

  naive     R = I (U = P H, the inverse of H P); tau = the largest |value|
            of the calibration set (quantile 1.0): no clipping inside the
            calibration range.  (An infinite tau has no 8-bit metadata grid.)
  clip      R = I; tau = the calibrated quantile (0.96 for K, 0.92 for V).
  hadamard  R = H P (U = I); tau = the same quantile of |x H P|.
  oscar     the calibrated eigenbasis U and its tau.

Error measures ([A]/[B]: attention-score distortion and output error), with
every token of the head quantised so that only the quantiser is measured:
  score KL   mean over queries of KL(p || p^), p = softmax(sm q K^T) with the
             bf16 keys, p^ with the dequantised, inverse-rotated keys;
  output     sum ||o - o^||^2 / sum ||o||^2 with o = p V, o^ = p^ V^.
"""
from __future__ import annotations

import numpy as np

from . import oscar_ref as R

KINDS = ("naive", "clip", "hadamard", "oscar")


def identity_rotation_factor(d: int = 128) -> np.ndarray:
    """U with U H P = I: U = (H P)^-1 = P H (H and P are involutions)."""
    return (R.bitrev_matrix(d) @ R.hadamard_matrix(d)).astype(np.float32)


def variant_calibration(kind: str, cal: R.HeadCalibration, k_cal: np.ndarray,
                        v_cal: np.ndarray) -> R.HeadCalibration:
    """The calibration of one KV head for quantiser variant ``kind``, from
    the OSCAR calibration ``cal`` and the head's calibration keys/values."""
    d = cal.U_K.shape[0]
    if kind == "oscar":
        return cal
    if kind in ("naive", "clip"):
        U = identity_rotation_factor(d)
    elif kind == "hadamard":
        U = np.eye(d, dtype=np.float32)
    else:
        raise ValueError(f"unknown variant {kind!r}")
    qk, qv = (1.0, 1.0) if kind == "naive" else (R.CLIP_QUANTILE_K, R.CLIP_QUANTILE_V)
    return R.HeadCalibration(U_K=U, U_V=U.copy(), tau_K=R.clip_threshold(k_cal, U, qk),
                             tau_V=R.clip_threshold(v_cal, U, qv))


def quantised_values(x: np.ndarray, U32: np.ndarray, tau: np.float32) -> np.ndarray:
    """Tokens x [n, d] (bf16 values) through the write path, dequantised and
    rotated back to the original basis (float64)."""
    qt = R.write_history(x, U32, tau)
    return R.dequantize_int2(qt.codes, qt.scale, qt.zero) @ R.composite_rotation(U32).T


def _log_softmax(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=1, keepdims=True)
    return s - m - np.log(np.sum(np.exp(s - m), axis=1, keepdims=True))


def kl_rows(logp: np.ndarray, logq: np.ndarray) -> np.ndarray:
    """KL(p || q) per row, from log-probabilities."""
    return np.sum(np.exp(logp) * (logp - logq), axis=1)


def attention_errors(q: np.ndarray, k: np.ndarray, v: np.ndarray, cal: R.HeadCalibration,
                     sm_scale: float):
    """(mean score KL, relative output MSE) of one head: queries q [nq, d],
    keys and values k, v [n, d], every token quantised with ``cal``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    kh = quantised_values(k, cal.U_K, cal.tau_K)
    vh = quantised_values(v, cal.U_V, cal.tau_V)
    logp = _log_softmax(sm_scale * (q @ k.T))
    logph = _log_softmax(sm_scale * (q @ kh.T))
    o = np.exp(logp) @ v
    oh = np.exp(logph) @ vh
    return float(np.mean(kl_rows(logp, logph))), float(np.sum((o - oh) ** 2) / np.sum(o ** 2))
