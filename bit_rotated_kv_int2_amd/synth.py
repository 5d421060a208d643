"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds no arithmetic of the method (no rotation, clipping,
quantisation or attention).  It only draws random tensors with the shapes and
value structure of the workloads, rounds them to bf16 and lays out block
tables.

Recipe
------
* Keys and values: N(0, 1) float32, with a few outlier channels multiplied by
  20, rounded to bf16 (nearest-even).  Tiny workload: 4 outlier channels per
  KV head, drawn without replacement, independently for K and V.  Larger
  workloads: 10 (head, channel) pairs out of n_kv_heads * head_dim per tensor
  (the whole count nearest to 1 %).  A layer's calibration tokens and cache
  tokens share its outlier channels.
* Queries (decode and calibration): N(0, 1) rounded to bf16.
* Calibration set: ``n_cal`` queries per query head and ``n_cal`` keys/values
  per KV head.
* Block tables: contiguous, or pages scattered by a seeded permutation.
* Lengths: fixed, or integers uniform on an inclusive range.

Small tensors come from ``numpy.random.default_rng([workload_id, layer,
stream, ...])``.  Cache contents of the 100K-token workloads are drawn on the
GPU with a seeded ``torch.Generator`` (same distributions), because host
generation of gigabytes per layer would dominate the benchmark.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

STREAM_K, STREAM_V, STREAM_Q, STREAM_CAL_Q, STREAM_CAL_K, STREAM_CAL_V = 0, 1, 2, 3, 4, 5
STREAM_OUTLIER, STREAM_PERM, STREAM_LEN = 6, 7, 8
OUTLIER_FACTOR = 20.0


@dataclass(frozen=True)
class Workload:
    wid: int                 # seed component
    name: str
    batch: int
    n_kv: int
    n_q: int
    head_dim: int
    min_len: int
    max_len: int
    layers: int = 1
    n_cal: int = 2048
    outliers: str = "per_head4"     # or "pairs10"
    scattered_pages: bool = False
    shared_prefix: int = 0          # tokens shared by every sequence (sink + whole pages)
    page_tokens: int = 64
    sink: int = 64
    recent: int = 256

    @property
    def group_size(self) -> int:
        return self.n_q // self.n_kv

    def max_pages(self, extra_tokens: int = 0) -> int:
        hist = max(0, self.max_len + extra_tokens - self.sink - self.recent)
        return (hist + self.page_tokens - 1) // self.page_tokens


WORKLOADS = {
    w.name: w for w in [
        Workload(0, "tiny-4k", 1, 1, 4, 128, 4096, 4096),
        Workload(1, "qwen3-8b-32k-b1", 1, 8, 32, 128, 32768, 32768, outliers="pairs10"),
        Workload(2, "qwen3-8b-100k-b1-36l", 1, 8, 32, 128, 102400, 102400, layers=36,
                 outliers="pairs10"),
        Workload(3, "qwen3-8b-100k-b32-36l", 32, 8, 32, 128, 92160, 102400, layers=36,
                 outliers="pairs10", scattered_pages=True),
        Workload(4, "prefix-128k-b16-gqa12", 16, 8, 96, 128, 131072, 131072,
                 outliers="pairs10", shared_prefix=98304),
    ]
}


def bf16_round(x: np.ndarray):
    """Round float32 to bf16 (nearest-even).  Returns (uint16 bits, float32 values)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r = np.where(nan, np.uint16(0x7FC0), r)
    vals = (r.astype(np.uint32) << 16).view(np.float32)
    return r, vals


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rng(wl: Workload, layer: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([wl.wid, layer, stream, *extra])


def outlier_scale(wl: Workload, layer: int, tensor: int) -> np.ndarray:
    """Per-(kv head, channel) multiplier, 1 or OUTLIER_FACTOR.  tensor 0 = K, 1 = V."""
    g = rng(wl, layer, STREAM_OUTLIER, tensor)
    scale = np.ones((wl.n_kv, wl.head_dim), dtype=np.float32)
    if wl.outliers == "per_head4":
        for h in range(wl.n_kv):
            ch = g.choice(wl.head_dim, size=4, replace=False)
            scale[h, ch] = OUTLIER_FACTOR
    elif wl.outliers == "pairs10":
        flat = g.choice(wl.n_kv * wl.head_dim, size=10, replace=False)
        scale.reshape(-1)[flat] = OUTLIER_FACTOR
    else:
        raise ValueError(wl.outliers)
    return scale


def kv_tokens(wl: Workload, layer: int, seq: int, start: int, count: int):
    """bf16 K and V of tokens [start, start+count) of one sequence, numpy.

    Returns (k_bits, v_bits) uint16 [count, n_kv, head_dim].  Tokens are drawn
    in fixed blocks of 1024 positions so any sub-range is reproducible.
    """
    if count <= 0:
        empty = np.zeros((0, wl.n_kv, wl.head_dim), np.uint16)
        return empty, empty.copy()
    out = []
    for tensor, stream in ((0, STREAM_K), (1, STREAM_V)):
        sc = outlier_scale(wl, layer, tensor)
        blocks = []
        b0, b1 = start // 1024, (start + count + 1023) // 1024
        for blk in range(b0, b1):
            g = rng(wl, layer, stream, seq, blk)
            blocks.append(g.standard_normal((1024, wl.n_kv, wl.head_dim), dtype=np.float32))
        x = np.concatenate(blocks, axis=0)[start - b0 * 1024: start - b0 * 1024 + count] * sc
        out.append(bf16_round(x)[0])
    return out[0], out[1]


def decode_queries(wl: Workload, layer: int, step: int = 0) -> np.ndarray:
    """bf16 bits [batch, n_q, head_dim]."""
    g = rng(wl, layer, STREAM_Q, step)
    return bf16_round(g.standard_normal((wl.batch, wl.n_q, wl.head_dim), dtype=np.float32))[0]


def calibration_set(wl: Workload, layer: int, n_cal: Optional[int] = None):
    """Calibration queries [n_q, n, d] and keys/values [n_kv, n, d] as bf16 bits."""
    n = wl.n_cal if n_cal is None else n_cal
    q = bf16_round(rng(wl, layer, STREAM_CAL_Q).standard_normal((wl.n_q, n, wl.head_dim), dtype=np.float32))[0]
    ks = outlier_scale(wl, layer, 0)[:, None, :]
    vs = outlier_scale(wl, layer, 1)[:, None, :]
    k = bf16_round(rng(wl, layer, STREAM_CAL_K).standard_normal((wl.n_kv, n, wl.head_dim), dtype=np.float32) * ks)[0]
    v = bf16_round(rng(wl, layer, STREAM_CAL_V).standard_normal((wl.n_kv, n, wl.head_dim), dtype=np.float32) * vs)[0]
    return q, k, v


def sequence_lengths(wl: Workload) -> np.ndarray:
    if wl.min_len == wl.max_len:
        return np.full(wl.batch, wl.max_len, dtype=np.int32)
    g = rng(wl, 0, STREAM_LEN)
    return g.integers(wl.min_len, wl.max_len, size=wl.batch, endpoint=True).astype(np.int32)


def block_table(wl: Workload, lengths: np.ndarray, extra_tokens: int = 0):
    """int32 [batch, max_pages] page ids (-1 = unused) and the page count.

    Pages are reserved for ``extra_tokens`` more tokens per sequence.  With
    ``shared_prefix`` every sequence maps its first prefix pages to the same
    physical pages.  With ``scattered_pages`` physical ids are a seeded
    permutation of the pool.
    """
    mp = wl.max_pages(extra_tokens)
    need = [max(0, int(L) + extra_tokens - wl.sink - wl.recent) for L in lengths]
    need = [(n + wl.page_tokens - 1) // wl.page_tokens for n in need]
    shared = 0
    if wl.shared_prefix:
        shared = (wl.shared_prefix - wl.sink) // wl.page_tokens
    total = shared + sum(n - shared for n in need)
    ids = np.arange(total, dtype=np.int32)
    if wl.scattered_pages:
        ids = rng(wl, 0, STREAM_PERM).permutation(total).astype(np.int32)
    bt = np.full((wl.batch, max(mp, 1)), -1, dtype=np.int32)
    nxt = shared
    for b, n in enumerate(need):
        bt[b, :shared] = ids[:shared]
        bt[b, shared:n] = ids[nxt:nxt + n - shared]
        nxt += n - shared
    return bt, total


def torch_kv_generator(wl: Workload, layer: int, seq: int, device):
    """Seeded torch.Generator for GPU-side cache contents of one sequence."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(((wl.wid * 1000 + layer) * 100000 + seq) * 7 + 1)
    return g


def _gpu_kv_block(wl: Workload, layer: int, stream_seq: int, count: int, device):
    import torch
    g = torch_kv_generator(wl, layer, stream_seq, device)
    out = []
    for tensor in (0, 1):
        sc = torch.from_numpy(outlier_scale(wl, layer, tensor)).to(device)
        x = torch.randn((count, wl.n_kv, wl.head_dim), generator=g, device=device, dtype=torch.float32) * sc
        out.append(x.to(torch.bfloat16).view(torch.int16).contiguous())
        del x
    return out[0], out[1]


def gpu_sequence_kv(wl: Workload, layer: int, seq: int, L: int, device="cuda"):
    """Seeded bf16 K and V bit patterns (int16 tensors [L, Hkv, d]) of one
    sequence, generated on the device: N(0, 1) float32 times the layer's
    outlier scale, rounded to bf16.  With ``shared_prefix`` the first
    shared_prefix tokens come from one stream common to every sequence (seq
    id = batch), the rest from the sequence's own stream."""
    import torch
    P = min(L, wl.shared_prefix)
    if P == 0:
        return _gpu_kv_block(wl, layer, seq, L, device)
    kp, vp = _gpu_kv_block(wl, layer, wl.batch, P, device)
    if L == P:
        return kp, vp
    ks, vs = _gpu_kv_block(wl, layer, seq, L - P, device)
    return torch.cat([kp, ks]).contiguous(), torch.cat([vp, vs]).contiguous()
