"""Test-side helpers: read the page layout documented in include/oscar.h back
into plain arrays, and build matching GPU / oracle pools from synth inputs.

The layout readers are written from the header's description alone; they
share nothing with the HIP kernels or the oracle.
"""
from __future__ import annotations

import numpy as np

from bit_rotated_kv_int2_amd import oscar as O
from bit_rotated_kv_int2_amd import synth
from oracle import oscar_ref as R

D = 128


def page_kcodes(page: np.ndarray) -> np.ndarray:
    """[64 tokens, 128 channels] codes of a page's K block (token-major)."""
    rows = page[O.PAGE_KCODES:O.PAGE_KCODES + 2048].reshape(64, 32)
    out = np.zeros((64, D), np.uint8)
    for i in range(4):
        out[:, i::4] = (rows >> (2 * i)) & 3
    return out


def page_vcodes(page: np.ndarray) -> np.ndarray:
    """[64 tokens, 128 channels] codes of a page's V block (channel-major)."""
    rows = page[O.PAGE_VCODES:O.PAGE_VCODES + 2048].reshape(D, 16)
    out = np.zeros((64, D), np.uint8)
    for t in range(64):
        byte = 4 * ((t >> 2) & 3) + (t >> 4)
        out[t] = (rows[:, byte] >> (2 * (t & 3))) & 3
    return out


def page_meta(page: np.ndarray, off: int):
    """(s8 [64, 2], z8 [64, 2]) uint8 metadata codes of a metadata block:
    64 entries of 4 bytes {s8_0, z8_0, s8_1, z8_1}, slot t at entry
    4 (t % 16) + t / 16."""
    ent = page[off:off + 256].reshape(64, 4)
    idx = np.array([4 * (t & 15) + (t >> 4) for t in range(64)])
    e = ent[idx]
    return e[:, [0, 2]].copy(), e[:, [1, 3]].copy()


def gather_history(pages: np.ndarray, block_row: np.ndarray, kv: int, n_hist: int):
    """Canonical codes and metadata codes (s8, z8) of the first n_hist
    history tokens of one sequence and KV head, read from the device page
    buffer copy."""
    kc, vc = np.zeros((n_hist, D), np.uint8), np.zeros((n_hist, D), np.uint8)
    ks, kz = np.zeros((n_hist, 2), np.uint8), np.zeros((n_hist, 2), np.uint8)
    vs, vz = np.zeros((n_hist, 2), np.uint8), np.zeros((n_hist, 2), np.uint8)
    for pg in range((n_hist + 63) // 64):
        page = pages[block_row[pg], kv]
        a, b = pg * 64, min(n_hist, pg * 64 + 64)
        n = b - a
        kc[a:b] = page_kcodes(page)[:n]
        vc[a:b] = page_vcodes(page)[:n]
        s, z = page_meta(page, O.PAGE_KMETA)
        ks[a:b], kz[a:b] = s[:n], z[:n]
        s, z = page_meta(page, O.PAGE_VMETA)
        vs[a:b], vz[a:b] = s[:n], z[:n]
    return (kc, ks, kz), (vc, vs, vz)


def oracle_calibration(wl: synth.Workload, layer: int = 0, n_cal: int = 512):
    """Per-KV-head oracle calibration (float32 U and tau) from synth data."""
    q, k, v = synth.calibration_set(wl, layer, n_cal=n_cal)
    qf, kf, vf = (synth.bf16_bits_to_f32(x) for x in (q, k, v))
    G = wl.n_q // wl.n_kv
    cals = []
    for h in range(wl.n_kv):
        cals.append(R.calibrate_head(qf[h * G:(h + 1) * G], kf[h], vf[h], 1 / np.sqrt(D)))
    return cals


def rotation_tensors(cals, device="cuda"):
    """Device rotation artifact of per-head oracle calibrations; their
    codebooks, when they have them, as the library's level words."""
    UK = np.stack([c.U_K for c in cals])
    UV = np.stack([c.U_V for c in cals])
    tK = np.array([c.tau_K for c in cals], np.float32)
    tV = np.array([c.tau_V for c in cals], np.float32)
    lk = lv = None
    if cals[0].levels_K is not None:
        lk = np.array([O.levels_word(c.levels_K) for c in cals], np.uint32)
        lv = np.array([O.levels_word(c.levels_V) for c in cals], np.uint32)
    return O.RotationTensors.from_numpy(UK, UV, tK, tV, device, levels_K=lk, levels_V=lv)


def pool_view(pool: O.KVPool, b: int) -> O.KVPoolC:
    """C struct addressing sequence b of ``pool`` alone (batch 1)."""
    c = pool.c()
    p = pool.params
    rs = pool.recent_k[b].element_size() * p.num_kv_heads * p.recent * p.head_dim
    c.recent_k = c.recent_k + b * rs
    c.recent_v = c.recent_v + b * rs
    c.block_table = c.block_table + b * pool.max_pages * 4
    c.sink_slot = c.sink_slot + b * 4
    c.seq_lens = c.seq_lens + b * 4
    c.batch = 1
    return c


def append_sequence(params, rot, pool: O.KVPool, b: int, k_bits: np.ndarray, v_bits: np.ndarray,
                    chunks=None):
    """Append tokens [T, Hkv, d] (bf16 bits) to sequence b in the given chunk sizes."""
    import ctypes
    import torch
    T = k_bits.shape[0]
    chunks = chunks or [T]
    assert sum(chunks) == T
    kt = torch.from_numpy(k_bits.view(np.int16)).cuda()
    vt = torch.from_numpy(v_bits.view(np.int16)).cuda()
    pos = 0
    r = rot.c()
    view = pool_view(pool, b)
    stream = torch.cuda.current_stream().cuda_stream
    for n in chunks:
        kc = kt[pos:pos + n][None].contiguous()
        vc = vt[pos:pos + n][None].contiguous()
        rc = O.lib().oscar_quantize_append(ctypes.byref(params), ctypes.byref(r), ctypes.byref(view),
                                           kc.data_ptr(), vc.data_ptr(), n, stream)
        O._check(rc)
        pos += n
        torch.cuda.synchronize()


def decode_check(out_gpu: np.ndarray, out_ref: np.ndarray, tol: float = 2e-3):
    """max-abs error per (sequence, head) relative to the reference output norm."""
    err = np.max(np.abs(out_gpu - out_ref), axis=-1)
    nrm = np.linalg.norm(out_ref, axis=-1)
    ratio = err / np.maximum(nrm, 1e-30)
    return float(np.max(ratio))
