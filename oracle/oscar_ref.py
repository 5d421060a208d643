"""Plain CPU oracle for OSCAR rotated-INT2 KV-cache decode attention.

TEST INFRASTRUCTURE ONLY.  This module is the independent checker of the HIP
library.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The library (``include/``, the package's
``csrc/`` and its Python binding) never imports, links or calls anything here,
and this module shares no code, tables or constants generator with it.

Everything is numpy, float64 unless a step fixes another precision.  Each
function names the passage it follows.  Source pages (cited by title and
section, never by line):

  [A]  youleyou.com news article "超越 TurboQuant，显存压力终于得到缓解！Together AI
       最新论文 OSCAR 直接挑战 TurboQuant …" -- sections "OSCAR 的设计思路"
       (design) and the token-pool paragraphs that follow it.
  [B]  MarkTechPost article in Chinese translation, "Together AI 开源 OSCAR：一种用于
       长上下文 LLM 服务的注意力感知 2 位 KV 缓存量化系统" -- sections
       "为什么 INT2 KV 缓存量化很难", "OSCAR 有何不同做法" (method),
       "服务系统：混合精度缓存布局" (serving), "结果" (results) and the visual
       guide's step 04 (calibration) and step 06 (key parameters table).

Where the pages leave a step open, the reading taken is stated next to the
code (the full list of readings lives in the repository's design document).

What the oracle computes
------------------------
1. Calibration per KV head ([B] method): uncentred query covariance C_Q,
   score-weighted value covariance C_S, their eigenbases U_Q / U_S (sorted by
   descending eigenvalue, sign fixed), stored as float32; composite rotation
   R = U · H · P with the normalised Sylvester-Hadamard H and the
   bit-reversal permutation P; clipping thresholds tau = quantile of
   |rotated calibration values| (0.96 for K, 0.92 for V; [B] serving and
   guide step 06).
2. The write path ([A] token pool paragraph, [B] serving): rotate a bf16
   token by R (fp64 U-projection with k ascending, fp64 butterfly, fp64
   scale, bit-reversal, round to float32), clip to +-tau, per-token
   asymmetric INT2 over groups of 64 channels with an 8-bit zero and an
   8-bit scale per group (fixed-point fractions of tau), pack four 2-bit
   codes per byte.
3. The pool ([A], [B] serving): BF16 sink (first 64 tokens), rotated INT2
   history, BF16 recent window (last 256 tokens).
4. Decode attention over the pool: the literal form (each history token is
   dequantised and inverse-rotated, then one softmax over all tokens) and a
   segmented form (per-segment partial softmax, merged by log-sum-exp, [A]).

Parity pins for all of this live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Constants printed by the pages ([B] serving; guide step 06 table).
SINK_TOKENS = 64          # S0: first tokens kept in BF16
RECENT_TOKENS = 256       # W: last tokens before the current position kept in BF16
GROUP_CHANNELS = 64       # G_K: channels per INT2 quantisation group
CLIP_QUANTILE_K = 0.96    # c_K
CLIP_QUANTILE_V = 0.92    # c_V
CODES_PER_BYTE = 4        # [A] token-pool paragraph: four 2-bit values per byte
PAGE_TOKENS = 64          # history page size of the synthetic workloads
INT2_LEVELS = 4


# ---------------------------------------------------------------------------
# Rotation factors ([B] method: R_K = U_Q · H_Had · P_br, R_V = U_S · H_Had · P_br)
# ---------------------------------------------------------------------------

def _log2_exact(d: int) -> int:
    k = int(d).bit_length() - 1
    if d <= 0 or (1 << k) != d:
        raise ValueError(f"dimension {d} is not a power of two")
    return k


def inv_sqrt_dim(d: int) -> float:
    """float64 nearest to 1/sqrt(d) for a power of two d.

    For even log2(d) it is an exact power of two; for odd log2(d) it is
    RN(sqrt(2)) scaled by a power of two, which is still the correctly rounded
    value because scaling by 2^k is exact.
    """
    k = _log2_exact(d)
    if k % 2 == 0:
        return math.ldexp(1.0, -k // 2)
    return math.ldexp(float(np.sqrt(np.float64(2.0))), -(k + 1) // 2)


def hadamard_matrix(d: int) -> np.ndarray:
    """Normalised Walsh-Hadamard matrix in Sylvester (natural) order.

    [B] method names the Walsh-Hadamard transform; the reading taken is the
    Sylvester order H[i, j] = (-1)^popcount(i & j) / sqrt(d), which is the
    order the radix-2 butterfly produces.  Symmetric and its own inverse.
    """
    _log2_exact(d)
    i = np.arange(d)[:, None]
    j = np.arange(d)[None, :]
    bits = np.bitwise_and(i, j)
    parity = np.zeros_like(bits)
    while np.any(bits):
        parity ^= bits & 1
        bits = bits >> 1
    return np.where(parity == 1, -1.0, 1.0) / math.sqrt(d)


def fwht_butterfly(y: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis (fp64).

    Stage h = 1, 2, 4, ..., d/2 maps each pair (i, i + h) with (i & h) == 0 to
    (a + b, a - b).  Every add/sub is one fp64 rounding, so two
    implementations that follow the same stage order agree bit for bit.
    """
    y = np.array(y, dtype=np.float64, copy=True)
    n, d = y.reshape(-1, y.shape[-1]).shape
    _log2_exact(d)
    out = y.reshape(n, d)
    h = 1
    while h < d:
        v = out.reshape(n, d // (2 * h), 2, h)
        a = v[:, :, 0, :].copy()
        b = v[:, :, 1, :].copy()
        v[:, :, 0, :] = a + b
        v[:, :, 1, :] = a - b
        h *= 2
    return out.reshape(y.shape)


def bit_reverse(p: int, bits: int) -> int:
    r = 0
    for _ in range(bits):
        r = (r << 1) | (p & 1)
        p >>= 1
    return r


def bitrev_indices(d: int) -> np.ndarray:
    """idx[p] = bitrev(p): output position p takes input channel bitrev(p)."""
    k = _log2_exact(d)
    return np.array([bit_reverse(p, k) for p in range(d)], dtype=np.int64)


def bitrev_matrix(d: int) -> np.ndarray:
    """Permutation matrix P with (y @ P)[p] = y[bitrev(p)] ([B] method, P_br)."""
    idx = bitrev_indices(d)
    P = np.zeros((d, d))
    P[idx, np.arange(d)] = 1.0
    return P


def composite_rotation(U: np.ndarray) -> np.ndarray:
    """R = U · H · P in float64 from the stored basis U ([A] design, [B] method).

    Tokens are row vectors: the forward rotation is x -> x @ R and the inverse
    is x~ -> x~ @ R.T.
    """
    U = np.asarray(U, dtype=np.float64)
    d = U.shape[-1]
    return U @ hadamard_matrix(d) @ bitrev_matrix(d)


# ---------------------------------------------------------------------------
# Calibration ([B] method; [B] guide step 04; [A] design)
# ---------------------------------------------------------------------------

def softmax_rows(x: np.ndarray) -> np.ndarray:
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def query_covariance(q_rows: np.ndarray) -> np.ndarray:
    """C_Q = (1/N) sum_n q_n^T q_n over row vectors, uncentred ([B] method).

    Reading: the query heads that share one KV head are pooled, N counts
    (query, head) rows.
    """
    q = np.asarray(q_rows, dtype=np.float64)
    return (q.T @ q) / q.shape[0]


def score_weighted_value_covariance(q_heads: np.ndarray, k_cal: np.ndarray,
                                    v_cal: np.ndarray, sm_scale: float) -> np.ndarray:
    """C_S = (1/N) V^T S^T S V ([B] method).

    Reading: S is the post-softmax score matrix of the calibration queries
    over the calibration keys (scale sm_scale, no mask), one S per query head
    of the group; the G products are pooled and N counts (query, head) rows.
    ``q_heads`` is [G, Nq, d].
    """
    k = np.asarray(k_cal, dtype=np.float64)
    v = np.asarray(v_cal, dtype=np.float64)
    acc = np.zeros((k.shape[1], k.shape[1]))
    rows = 0
    for qh in np.asarray(q_heads, dtype=np.float64):
        S = softmax_rows((qh @ k.T) * sm_scale)
        SV = S @ v
        acc += SV.T @ SV
        rows += qh.shape[0]
    return acc / rows


def sorted_eigenbasis(C: np.ndarray, min_rel_gap: float = 1e-10):
    """Eigenvectors of a symmetric C as columns, by descending eigenvalue.

    Readings: index 0 is the most important direction (matching the
    importance hierarchy the bit-reversal step balances, [B] method); each
    column's largest-magnitude entry is made positive (lowest index on ties);
    near-degenerate spectra (relative gap below ``min_rel_gap``) are refused
    because the basis would not be unique.
    """
    C = np.asarray(C, dtype=np.float64)
    w, U = np.linalg.eigh(0.5 * (C + C.T))
    order = np.argsort(-w, kind="stable")
    w = w[order]
    U = U[:, order]
    scale = max(abs(w[0]), np.finfo(np.float64).tiny)
    gaps = np.abs(np.diff(w)) / scale
    if gaps.size and np.min(gaps) < min_rel_gap:
        raise ValueError("degenerate spectrum: eigenbasis not unique")
    for j in range(U.shape[1]):
        col = U[:, j]
        i = int(np.argmax(np.abs(col)))   # first index of the maximum
        if col[i] < 0:
            U[:, j] = -col
    return w, U


def clip_threshold(x_cal: np.ndarray, U32: np.ndarray, quantile: float) -> np.float32:
    """tau = quantile of |x @ R| over all calibration values of one head.

    Reading ([B] serving: clipping to a calibration-derived percentile
    threshold; guide step 06: c_K 0.96 / c_V 0.92 as percentile clipping):
    the quantile is over all rotated calibration entries of the KV head,
    linear interpolation in float64, stored as float32.
    """
    R = composite_rotation(U32)
    vals = np.abs(np.asarray(x_cal, dtype=np.float64) @ R).ravel()
    return np.float32(np.quantile(vals, quantile, method="linear"))


@dataclass
class HeadCalibration:
    U_K: np.ndarray        # float32 [d, d], columns = eigenvectors of C_Q
    U_V: np.ndarray        # float32 [d, d], columns = eigenvectors of C_S
    tau_K: np.float32
    tau_V: np.float32
    eig_K: np.ndarray = field(repr=False, default=None)
    eig_V: np.ndarray = field(repr=False, default=None)
    levels_K: np.ndarray = None   # uint8 [4] reconstruction levels n / 32 (None: the uniform grid)
    levels_V: np.ndarray = None


def calibrate_head(q_heads: np.ndarray, k_cal: np.ndarray, v_cal: np.ndarray,
                   sm_scale: float, quantile_k: float = CLIP_QUANTILE_K,
                   quantile_v: float = CLIP_QUANTILE_V) -> HeadCalibration:
    """Offline calibration of one KV head ([B] method and guide step 04).

    ``q_heads`` [G, Nq, d] are the calibration queries of the G query heads
    that read this KV head; ``k_cal``/``v_cal`` [Nkv, d] its calibration keys
    and values (bf16-valued).
    """
    q_heads = np.asarray(q_heads, dtype=np.float64)
    d = q_heads.shape[-1]
    CQ = query_covariance(q_heads.reshape(-1, d))
    CS = score_weighted_value_covariance(q_heads, k_cal, v_cal, sm_scale)
    wK, UK = sorted_eigenbasis(CQ)
    wV, UV = sorted_eigenbasis(CS)
    UK32 = UK.astype(np.float32)
    UV32 = UV.astype(np.float32)
    return HeadCalibration(U_K=UK32, U_V=UV32,
                           tau_K=clip_threshold(k_cal, UK32, quantile_k),
                           tau_V=clip_threshold(v_cal, UV32, quantile_v),
                           eig_K=wK, eig_V=wV)


# ---------------------------------------------------------------------------
# Write path: rotate, clip, quantise, pack ([A] token pool; [B] serving)
# ---------------------------------------------------------------------------

def rotate_for_write(x: np.ndarray, U32: np.ndarray) -> np.ndarray:
    """x~ = bitrev(FWHT(x · U) / sqrt(d)), rounded to float32.

    The arithmetic order is fixed so that an independent implementation can
    reproduce every bit:
      S1  y_j = sum_k x_k U[k, j] in float64 with k ascending (each bf16 x
          float32 product is exact in float64, so a fused multiply-add gives
          the same value as multiply-then-add);
      S2  unnormalised butterfly of ``fwht_butterfly``;
      S3  multiply by the float64 nearest to 1/sqrt(d);
      S4  bit-reversal permutation;
      S5  round to float32 (nearest-even).
    ``x`` [n, d] holds bf16 values (exact in float64).
    """
    x = np.asarray(x, dtype=np.float64)
    U = np.asarray(U32, dtype=np.float32).astype(np.float64)
    n, d = x.shape
    out = np.empty((n, d), dtype=np.float32)
    idx = bitrev_indices(d)
    c = inv_sqrt_dim(d)
    for r0 in range(0, n, 2048):               # row blocks only bound memory use
        xb = x[r0:r0 + 2048]
        y = np.zeros((xb.shape[0], d))
        for k in range(d):
            y += xb[:, k:k + 1] * U[k:k + 1, :]
        y = fwht_butterfly(y) * c
        out[r0:r0 + 2048] = y[:, idx].astype(np.float32)
    return out


@dataclass
class QuantizedTokens:
    codes: np.ndarray      # uint8 [n, d], values 0..3
    s8: np.ndarray         # uint8 [n, d // group]: scale code
    z8: np.ndarray         # uint8 [n, d // group]: zero code
    scale: np.ndarray      # float32 [n, d // group]: decoded scale  s8 * b
    zero: np.ndarray       # float32 [n, d // group]: decoded zero   z8 * a - tau
    levels: np.ndarray = None   # uint8 [4]: code k stands for levels[k] / 32 (None: k)


META_LEVELS = 255          # largest 8-bit zero / scale code


def metadata_steps(tau: np.float32):
    """Grid steps of the 8-bit zero and scale codes of one head.

    After the clip every group lies in [-tau, tau]: its minimum in that
    interval and its INT2 step s = (max - min) / 3 in [0, 2 tau / 3].  The
    zero code z8 in 0..255 stands for z8 * a - tau with a = 2 tau / 255; the
    scale code s8 for s8 * b with b = 2 tau / 765.  Each step is one float32
    division of 2 tau (exact) by the integer, correctly rounded.
    """
    t = np.float32(tau)
    a = np.float32((t + t) / np.float32(255.0))
    b = np.float32((t + t) / np.float32(765.0))
    return a, b


def quantize_int2(xr: np.ndarray, tau: np.float32, group: int = GROUP_CHANNELS, levels=None) -> QuantizedTokens:
    """Clip to +-tau and quantise per token, per group of ``group`` channels.

    [B] serving: per-token asymmetric INT2 with G_K = 64 channels per group,
    after clipping to the calibration threshold.  Readings: groups are
    consecutive channels of the rotated, permuted vector; min-max range after
    the clip; s = (max - min) / 3; the zero point is the group minimum
    (x^ = code * s + z).  Metadata: 16 bits per group, the density that the
    pages' 2.28 bits per element at 128K implies (2 code bits + 16 / 64 per
    element, plus the BF16 windows).  Zero and scale are stored as 8-bit
    codes on grids spanning [-tau, tau] and [0, 2 tau / 3] (see
    ``metadata_steps``): z8 = rint((min + tau) / a), s8 = rint(s / b), each
    clamped to [0, 255] (0 when tau is 0).  The codes are computed against
    the decoded values z^ = z8 a - tau and s^ = s8 b: code = rint((x - z^) /
    s^) clamped to [0, 3], all codes 0 if s^ == 0.  All steps in float32
    (IEEE add, subtract, multiply and divide; round half to even).

    With ``levels`` (a Lloyd-Max codebook, see ``codebook_levels``) code k
    stands for the value z^ + s^ levels[k] / 32 instead of z^ + s^ k: the
    code of u = (x - z^) / s^ is the nearest level, the thresholds being the
    midpoints t_k = (levels[k] + levels[k+1]) / 64, with a tie at the middle
    threshold going up and at the outer ones down.  For the uniform grid
    levels = (0, 32, 64, 96) that is exactly the rounding above.
    """
    xr = np.asarray(xr, dtype=np.float32)
    n, d = xr.shape
    if d % group:
        raise ValueError("group must divide the head dimension")
    t = np.float32(tau)
    xc = np.clip(xr, -t, t).reshape(n, d // group, group)
    mx = np.max(xc, axis=-1)
    mn = np.min(xc, axis=-1)
    s = (mx - mn) / np.float32(3.0)
    a, b = metadata_steps(t)
    lev = np.float32(META_LEVELS)
    z8 = np.clip(np.rint((mn + t) / a), 0, lev) if a > 0 else np.zeros_like(mn)
    s8 = np.clip(np.rint(s / b), 0, lev) if b > 0 else np.zeros_like(s)
    z8 = z8.astype(np.uint8)
    s8 = s8.astype(np.uint8)
    zf = z8.astype(np.float32) * a - t
    sf = s8.astype(np.float32) * b
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (xc - zf[..., None]) / sf[..., None]
    if levels is None:
        q = np.rint(u)
    else:
        t = level_thresholds(levels)
        q = ((u > t[0]).astype(np.int32) + (u >= t[1]).astype(np.int32) + (u > t[2]).astype(np.int32)).astype(np.float32)
    q = np.where(sf[..., None] == 0, np.float32(0), q)
    codes = np.clip(q, 0, INT2_LEVELS - 1).astype(np.uint8).reshape(n, d)
    return QuantizedTokens(codes=codes, s8=s8, z8=z8, scale=sf, zero=zf,
                           levels=None if levels is None else np.asarray(levels, np.uint8).copy())


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Four 2-bit codes per byte ([A] token-pool paragraph).

    Reading: byte j of a token row holds channels 4j..4j+3, channel 4j+i in
    bits [2i, 2i+2) (least significant first).
    """
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % CODES_PER_BYTE:
        raise ValueError("channel count must be a multiple of 4")
    c = c.reshape(*c.shape[:-1], -1, CODES_PER_BYTE).astype(np.uint16)
    b = c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)
    return b.astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.stack([(p >> (2 * i)) & 3 for i in range(CODES_PER_BYTE)], axis=-1)
    return out.reshape(*p.shape[:-1], -1).astype(np.uint8)


def dequantize_int2(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray,
                    group: int = GROUP_CHANNELS, levels=None) -> np.ndarray:
    """x^ = code * s + z per group, in float64 from the decoded float32 s, z
    (with a codebook: levels[code] / 32 in place of the code)."""
    c = np.asarray(codes, dtype=np.float64)
    if levels is not None:
        c = np.asarray(levels, dtype=np.float64)[np.asarray(codes, dtype=np.int64)] / LEVEL_DENOM
    n, d = c.shape
    s = np.asarray(scale, dtype=np.float64)[..., None]
    z = np.asarray(zero, dtype=np.float64)[..., None]
    return (c.reshape(n, d // group, group) * s + z).reshape(n, d)


def write_history(x: np.ndarray, U32: np.ndarray, tau: np.float32, levels=None) -> QuantizedTokens:
    """Whole write path for history tokens: rotate, clip, quantise."""
    return quantize_int2(rotate_for_write(x, U32), tau, levels=levels)


# ---------------------------------------------------------------------------
# Lloyd-Max codebook ([A] summary and outlook: the latest code base adds a
# Lloyd-Max codebook for the 2-bit codes; the pages say nothing more)
# ---------------------------------------------------------------------------
#
# Reading taken: rotation, clip and the per-token, per-group zero and scale
# (with their 8-bit codes) stay as they are; only the four reconstruction
# levels of a code change.  On the uniform grid code k stands for
# z^ + s^ k.  With a codebook it stands for z^ + s^ c_k, where c_0..c_3 are
# the Lloyd-Max levels of the normalised values u = (x - z^) / s^ in [0, 3]
# of one head's calibration tokens (keys and values separately).  The levels
# are stored as integers n_k = c_k * 32 in [0, 96], strictly increasing
# (8 bits each, 32 bits per head and tensor), so that the grid stays exact
# in float32 and in the integer products of the decode kernels.

LEVEL_DENOM = 32
UNIFORM_LEVELS = np.array([0, 32, 64, 96], dtype=np.uint8)


def level_thresholds(levels) -> np.ndarray:
    """Midpoints between consecutive levels, in float32 (exact: integers / 64)."""
    n = np.asarray(levels, dtype=np.float64)
    return ((n[:-1] + n[1:]) / (2 * LEVEL_DENOM)).astype(np.float32)


def lloyd_max(samples: np.ndarray, levels0, iters: int = 1000, tol: float = 1e-12) -> np.ndarray:
    """Lloyd-Max scalar quantiser of 1-D samples (float64): alternately assign
    each sample to the nearest level (cells bounded by the midpoints) and move
    each level to the mean of its cell, from the ascending levels0, until no
    level moves by more than tol.  A cell without samples keeps its level."""
    x = np.sort(np.asarray(samples, dtype=np.float64).ravel())
    c = np.array(levels0, dtype=np.float64)
    csum = np.concatenate([[0.0], np.cumsum(x)])
    for _ in range(iters):
        t = (c[:-1] + c[1:]) / 2
        edges = np.concatenate([[0], np.searchsorted(x, t, side="left"), [x.size]])
        new = c.copy()
        for k in range(c.size):
            lo, hi = edges[k], edges[k + 1]
            if hi > lo:
                new[k] = (csum[hi] - csum[lo]) / (hi - lo)
        done = np.max(np.abs(new - c)) <= tol
        c = new
        if done:
            break
    return c


def codebook_levels(u: np.ndarray) -> np.ndarray:
    """Stored levels (uint8 [4]) of the normalised values u in [0, 3]: the
    Lloyd-Max levels from the uniform start (0, 1, 2, 3), each rounded to the
    nearest 1/32 (half to even) and clamped to [0, 96], then made strictly
    increasing by raising each level to at least one step above the one
    below it and lowering it to leave room for the ones above."""
    c = lloyd_max(u, [0.0, 1.0, 2.0, 3.0])
    n = np.clip(np.rint(c * LEVEL_DENOM), 0, 3 * LEVEL_DENOM).astype(np.int64)
    for k in range(1, 4):
        n[k] = max(n[k], n[k - 1] + 1)
    for k in range(3, -1, -1):
        n[k] = min(n[k], 3 * LEVEL_DENOM - (3 - k))
        if k < 3:
            n[k] = min(n[k], n[k + 1] - 1)
    return n.astype(np.uint8)


def normalised_values(x: np.ndarray, U32: np.ndarray, tau: np.float32, group: int = GROUP_CHANNELS) -> np.ndarray:
    """u = (x~ - z^) / s^ (float32) of every element of tokens x [n, d]
    through the write path up to the code (rotate, clip, group metadata),
    for the groups whose decoded scale is not zero."""
    xr = rotate_for_write(x, U32)
    qt = quantize_int2(xr, tau, group)
    t = np.float32(tau)
    n, d = xr.shape
    xc = np.clip(xr, -t, t).reshape(n, d // group, group)
    keep = qt.scale > 0
    u = (xc - qt.zero[..., None]) / np.where(keep, qt.scale, np.float32(1))[..., None]
    return u[keep].ravel()


def calibrate_codebook(cal: HeadCalibration, k_cal: np.ndarray, v_cal: np.ndarray) -> HeadCalibration:
    """``cal`` with Lloyd-Max levels for keys and values, from the head's
    calibration tokens (the same ones that set tau)."""
    import dataclasses
    return dataclasses.replace(cal, levels_K=codebook_levels(normalised_values(k_cal, cal.U_K, cal.tau_K)),
                               levels_V=codebook_levels(normalised_values(v_cal, cal.U_V, cal.tau_V)))


# ---------------------------------------------------------------------------
# Pool regions ([A] token pool; [B] serving)
# ---------------------------------------------------------------------------

def pool_regions(L: int, sink: int = SINK_TOKENS, recent: int = RECENT_TOKENS):
    """Token ranges (sink, history, recent) of a sequence of L tokens.

    Reading: positions [0, S0) are sink; the last W positions are recent
    unless they overlap the sink; everything between is history.  L <= S0:
    all sink; S0 < L <= S0 + W: sink + recent; otherwise history = L - S0 - W.
    """
    s_end = min(L, sink)
    r_start = max(s_end, L - recent)
    return (0, s_end), (s_end, r_start), (r_start, L)


@dataclass
class HeadPool:
    """One KV head of one sequence, as the oracle stores it."""
    sink_k: np.ndarray     # float64 [n_sink, d] (bf16 values)
    sink_v: np.ndarray
    hist_k: QuantizedTokens
    hist_v: QuantizedTokens
    recent_k: np.ndarray   # float64 [n_recent, d], in position order
    recent_v: np.ndarray


def build_head_pool(k: np.ndarray, v: np.ndarray, cal: HeadCalibration,
                    sink: int = SINK_TOKENS, recent: int = RECENT_TOKENS) -> HeadPool:
    """Place L bf16 tokens of one KV head into the three regions.

    History tokens go through ``write_history`` from their bf16 values
    (reading: tokens enter the BF16 recent window before demotion, so the
    quantiser sees bf16 inputs).
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L = k.shape[0]
    (s0, s1), (h0, h1), (r0, r1) = pool_regions(L, sink, recent)
    return HeadPool(sink_k=k[s0:s1], sink_v=v[s0:s1],
                    hist_k=write_history(k[h0:h1], cal.U_K, cal.tau_K, cal.levels_K),
                    hist_v=write_history(v[h0:h1], cal.U_V, cal.tau_V, cal.levels_V),
                    recent_k=k[r0:r1], recent_v=v[r0:r1])


def dequantized_head_cache(pool: HeadPool, cal: HeadCalibration):
    """Full L x d float64 K^ and V^ with history inverse-rotated (x~ @ R^T)."""
    RK = composite_rotation(cal.U_K)
    RV = composite_rotation(cal.U_V)
    hk = dequantize_int2(pool.hist_k.codes, pool.hist_k.scale, pool.hist_k.zero, levels=pool.hist_k.levels) @ RK.T
    hv = dequantize_int2(pool.hist_v.codes, pool.hist_v.scale, pool.hist_v.zero, levels=pool.hist_v.levels) @ RV.T
    K = np.concatenate([pool.sink_k, hk, pool.recent_k], axis=0)
    V = np.concatenate([pool.sink_v, hv, pool.recent_v], axis=0)
    return K, V


# ---------------------------------------------------------------------------
# Decode attention ([A] token-pool paragraph: INT2 and BF16 segments merged by
# online softmax; [B] serving: read path unpacks, dequantises, inverse-rotates)
# ---------------------------------------------------------------------------

def attention_dense(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """softmax(sm_scale * q K^T) V for query rows q [G, d] (float64)."""
    logits = (np.asarray(q, dtype=np.float64) @ K.T) * sm_scale
    return softmax_rows(logits) @ V


def decode_head_dense(q: np.ndarray, pool: HeadPool, cal: HeadCalibration,
                      sm_scale: float) -> np.ndarray:
    """Literal read path: inverse-rotate every history token, one softmax.

    Reading: the decode query attends to every token in the pool, no mask.
    """
    K, V = dequantized_head_cache(pool, cal)
    return attention_dense(q, K, V, sm_scale)


@dataclass
class Partial:
    """Unnormalised softmax partial of one segment: m = max logit,
    l = sum exp(logit - m), o = sum exp(logit - m) v."""
    m: np.ndarray      # [G]
    l: np.ndarray      # [G]
    o: np.ndarray      # [G, d]


def segment_partial(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> Partial:
    q = np.asarray(q, dtype=np.float64)
    G, d = q.shape
    if K.shape[0] == 0:
        return Partial(m=np.full(G, -np.inf), l=np.zeros(G), o=np.zeros((G, d)))
    logits = (q @ K.T) * sm_scale
    m = np.max(logits, axis=1)
    e = np.exp(logits - m[:, None])
    return Partial(m=m, l=e.sum(axis=1), o=e @ V)


def lse_merge(parts) -> Partial:
    """Online-softmax merge of partials ([A]: segments merged by online softmax).

    Empty segments carry m = -inf and contribute nothing.
    """
    parts = list(parts)
    m = np.max(np.stack([p.m for p in parts]), axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    l = np.zeros_like(m)
    o = np.zeros_like(parts[0].o)
    for p in parts:
        w = np.where(np.isfinite(p.m), np.exp(p.m - safe_m), 0.0)
        l = l + w * p.l
        o = o + w[:, None] * p.o
    return Partial(m=m, l=l, o=o)


def decode_head_segmented(q: np.ndarray, pool: HeadPool, cal: HeadCalibration,
                          sm_scale: float, page_tokens: int = PAGE_TOKENS) -> np.ndarray:
    """Segmented read path: sink, one partial per history page, recent; merged."""
    RK = composite_rotation(cal.U_K)
    RV = composite_rotation(cal.U_V)
    parts = [segment_partial(q, pool.sink_k, pool.sink_v, sm_scale)]
    n_hist = pool.hist_k.codes.shape[0]
    for start in range(0, n_hist, page_tokens):
        sl = slice(start, min(n_hist, start + page_tokens))
        hk = dequantize_int2(pool.hist_k.codes[sl], pool.hist_k.scale[sl], pool.hist_k.zero[sl],
                             levels=pool.hist_k.levels) @ RK.T
        hv = dequantize_int2(pool.hist_v.codes[sl], pool.hist_v.scale[sl], pool.hist_v.zero[sl],
                             levels=pool.hist_v.levels) @ RV.T
        parts.append(segment_partial(q, hk, hv, sm_scale))
    parts.append(segment_partial(q, pool.recent_k, pool.recent_v, sm_scale))
    merged = lse_merge(parts)
    return merged.o / merged.l[:, None]


def decode_sequence(q: np.ndarray, pools, cals, sm_scale: float) -> np.ndarray:
    """Decode output [Hq, d] for one sequence; query head h reads KV head h // G."""
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape
    Hkv = len(pools)
    G = Hq // Hkv
    out = np.zeros((Hq, d))
    for kv in range(Hkv):
        out[kv * G:(kv + 1) * G] = decode_head_dense(q[kv * G:(kv + 1) * G], pools[kv], cals[kv], sm_scale)
    return out


# ---------------------------------------------------------------------------
# Accounting ([A] summary figures; [B] serving and results)
# ---------------------------------------------------------------------------

def effective_bits_per_element(L: int, history_bits: float, sink: int = SINK_TOKENS,
                               recent: int = RECENT_TOKENS, window_bits: float = 16.0) -> float:
    """Average stored bits per KV element of an L-token sequence."""
    (s0, s1), (h0, h1), (r0, r1) = pool_regions(L, sink, recent)
    n_win = (s1 - s0) + (r1 - r0)
    return (n_win * window_bits + (h1 - h0) * history_bits) / L


def history_bits_per_element(d: int = 128, group: int = GROUP_CHANNELS,
                             metadata_bits_per_group: int = 16) -> float:
    """2 code bits plus the per-group metadata spread over the group."""
    return 2.0 + metadata_bits_per_group / group
