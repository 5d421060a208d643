"""ctypes binding of liboscar.so (argument marshalling only).

Every computation happens in the library's HIP kernels (or, for offline
calibration, its host C++).  This module converts torch tensors to device
pointers, fills the C structs of ``include/oscar.h`` and raises on non-zero
status.  PyTorch only provides device memory and streams.

The library must have been built (``python -m bit_rotated_kv_int2_amd.build``);
there is no fallback: a missing library raises ``OscarLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboscar.so")

OSCAR_OK, OSCAR_EINVAL, OSCAR_ENOTSUP, OSCAR_EWORKSPACE, OSCAR_EHIP = 0, -1, -2, -3, -4
DEVERR_PAGE, DEVERR_LENGTH, DEVERR_SINKSLOT = 1, 2, 4
HEAD_DIM, PAGE_TOKENS, GROUP, PAGE_BYTES = 128, 64, 64, 4608
PAGE_KCODES, PAGE_VCODES, PAGE_KMETA, PAGE_VMETA = 0, 2048, 4096, 4352

EXPORTED = [
    "oscar_calibrate_rotation", "oscar_quantize_append", "oscar_decode_attention",
    "oscar_decode_workspace_size", "oscar_bf16_decode_attention",
    "oscar_bf16_decode_workspace_size", "oscar_last_error", "oscar_version",
    "oscar_decode_attention_noalloc", "oscar_calibrate_codebook",
]
UNIFORM_LEVELS = 0x60402000


class OscarLibraryMissing(RuntimeError):
    pass


class OscarError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"oscar error {code}: {msg}")
        self.code = code


class Params(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("sink", ctypes.c_int32),
                ("recent", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("group", ctypes.c_int32), ("sm_scale", ctypes.c_float)]


class Rotation(ctypes.Structure):
    _fields_ = [("U_K", ctypes.c_void_p), ("U_V", ctypes.c_void_p),
                ("tau_K", ctypes.c_void_p), ("tau_V", ctypes.c_void_p),
                ("levels_K", ctypes.c_void_p), ("levels_V", ctypes.c_void_p)]


class KVPoolC(ctypes.Structure):
    _fields_ = [("sink_k", ctypes.c_void_p), ("sink_v", ctypes.c_void_p),
                ("recent_k", ctypes.c_void_p), ("recent_v", ctypes.c_void_p),
                ("pages", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("sink_slot", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("error_flags", ctypes.c_void_p), ("append_counters", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32), ("n_pages", ctypes.c_int32),
                ("n_sink_slots", ctypes.c_int32)]


class DecodeOptions(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("blocks", ctypes.c_int32), ("prefix_pages", ctypes.c_int32)]


class Bf16CacheC(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("error_flags", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


_lib = None


def lib():
    """Load liboscar.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OscarLibraryMissing(
            f"{LIB_PATH} not found: build it with `python -m bit_rotated_kv_int2_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i32, i64, f64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
    L.oscar_calibrate_rotation.argtypes = [P(Params), vp, i64, vp, vp, i64, f64, f64, vp, vp, vp, vp]
    L.oscar_calibrate_rotation.restype = i32
    L.oscar_calibrate_codebook.argtypes = [P(Params), vp, vp, vp, i64, vp]
    L.oscar_calibrate_codebook.restype = i32
    L.oscar_quantize_append.argtypes = [P(Params), P(Rotation), P(KVPoolC), vp, vp, i32, vp]
    L.oscar_quantize_append.restype = i32
    L.oscar_decode_attention.argtypes = [P(Params), P(Rotation), P(KVPoolC), vp, vp, P(DecodeOptions), vp, sz, vp]
    L.oscar_decode_attention.restype = i32
    L.oscar_decode_workspace_size.argtypes = [P(Params), i32, i32, P(DecodeOptions)]
    L.oscar_decode_attention_noalloc.argtypes = [P(Params), P(Rotation), P(KVPoolC), vp, vp, P(DecodeOptions), vp]
    L.oscar_decode_attention_noalloc.restype = i32
    L.oscar_decode_workspace_size.restype = sz
    L.oscar_bf16_decode_attention.argtypes = [P(Params), P(Bf16CacheC), vp, vp, vp, sz, vp]
    L.oscar_bf16_decode_attention.restype = i32
    L.oscar_bf16_decode_workspace_size.argtypes = [P(Params), i32, i32]
    L.oscar_bf16_decode_workspace_size.restype = sz
    L.oscar_last_error.argtypes = []
    L.oscar_last_error.restype = ctypes.c_char_p
    L.oscar_version.argtypes = []
    L.oscar_version.restype = i32
    _lib = L
    return L


def _check(rc):
    if rc != OSCAR_OK:
        raise OscarError(rc, lib().oscar_last_error().decode())


def make_params(num_kv_heads, num_q_heads, head_dim=HEAD_DIM, sink=64, recent=256,
                page_tokens=PAGE_TOKENS, group=GROUP, sm_scale=None) -> Params:
    if sm_scale is None:
        sm_scale = 1.0 / float(np.sqrt(head_dim))
    return Params(head_dim, num_kv_heads, num_q_heads, sink, recent, page_tokens, group, sm_scale)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def version() -> int:
    return int(lib().oscar_version())


# ---------------------------------------------------------------------------
# Calibration (host)
# ---------------------------------------------------------------------------

def calibrate_rotation(params: Params, q_cal: np.ndarray, k_cal: np.ndarray, v_cal: np.ndarray,
                       quantile_k: float = 0.96, quantile_v: float = 0.92):
    """q_cal float32 [Hq][n_q][d]; k_cal, v_cal float32 [Hkv][n_kv][d] (host).

    Returns (U_K, U_V, tau_K, tau_V) as numpy float32 arrays.
    """
    q = np.ascontiguousarray(q_cal, dtype=np.float32)
    k = np.ascontiguousarray(k_cal, dtype=np.float32)
    v = np.ascontiguousarray(v_cal, dtype=np.float32)
    hkv, d = params.num_kv_heads, params.head_dim
    UK = np.zeros((hkv, d, d), np.float32)
    UV = np.zeros((hkv, d, d), np.float32)
    tK = np.zeros(hkv, np.float32)
    tV = np.zeros(hkv, np.float32)
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check(lib().oscar_calibrate_rotation(ctypes.byref(params), vp(q), q.shape[1], vp(k), vp(v), k.shape[1],
                                          float(quantile_k), float(quantile_v), vp(UK), vp(UV), vp(tK), vp(tV)))
    return UK, UV, tK, tV


def calibrate_codebook(params: Params, U: np.ndarray, tau: np.ndarray, x_cal: np.ndarray) -> np.ndarray:
    """Lloyd-Max codebook words (uint32 [Hkv]) of one tensor: U float32
    [Hkv][d][d], tau float32 [Hkv], x_cal float32 [Hkv][n][d] (host)."""
    Uc = np.ascontiguousarray(U, dtype=np.float32)
    tc = np.ascontiguousarray(tau, dtype=np.float32)
    xc = np.ascontiguousarray(x_cal, dtype=np.float32)
    out = np.zeros(params.num_kv_heads, np.uint32)
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check(lib().oscar_calibrate_codebook(ctypes.byref(params), vp(Uc), vp(tc), vp(xc), xc.shape[1], vp(out)))
    return out


def levels_word(levels) -> int:
    """Four level integers n_k (code k stands for n_k / 32) as the codebook word."""
    n = [int(x) for x in levels]
    return n[0] | (n[1] << 8) | (n[2] << 16) | (n[3] << 24)


# ---------------------------------------------------------------------------
# Device-side pool and calls
# ---------------------------------------------------------------------------

@dataclass
class RotationTensors:
    U_K: "torch.Tensor"      # float32 [Hkv, d, d]
    U_V: "torch.Tensor"
    tau_K: "torch.Tensor"    # float32 [Hkv]
    tau_V: "torch.Tensor"
    levels_K: Optional["torch.Tensor"] = None   # int32 [Hkv] codebook words, None = uniform grid
    levels_V: Optional["torch.Tensor"] = None

    def c(self) -> Rotation:
        return Rotation(_ptr(self.U_K), _ptr(self.U_V), _ptr(self.tau_K), _ptr(self.tau_V),
                        _ptr(self.levels_K), _ptr(self.levels_V))

    @staticmethod
    def from_numpy(UK, UV, tK, tV, device, levels_K=None, levels_V=None):
        import torch
        f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
        w = lambda a: None if a is None else torch.from_numpy(
            np.ascontiguousarray(np.asarray(a, dtype=np.uint32).view(np.int32))).to(device)
        return RotationTensors(f(UK), f(UV), f(tK), f(tV), w(levels_K), w(levels_V))


class KVPool:
    """Device tensors of one layer's mixed-precision pool (caller-owned memory).

    Layout and meaning of every field: ``include/oscar.h`` (oscar_kv_pool).
    """

    def __init__(self, params: Params, batch: int, n_pages: int, block_table, sink_slot=None,
                 n_sink_slots: Optional[int] = None, device="cuda", zero_pages=True):
        import torch
        hkv, d = params.num_kv_heads, params.head_dim
        bt = torch.as_tensor(np.asarray(block_table, dtype=np.int32)).to(device)
        assert bt.dim() == 2 and bt.shape[0] == batch
        if sink_slot is None:
            sink_slot = np.arange(batch, dtype=np.int32)
        self.sink_slot = torch.as_tensor(np.asarray(sink_slot, dtype=np.int32)).to(device)
        self.n_sink_slots = int(n_sink_slots if n_sink_slots is not None else batch)
        self.params = params
        self.batch = batch
        self.block_table = bt.contiguous()
        self.max_pages = int(bt.shape[1])
        self.n_pages = int(n_pages)
        self.sink_k = torch.zeros((self.n_sink_slots, hkv, params.sink, d), dtype=torch.int16, device=device)
        self.sink_v = torch.zeros_like(self.sink_k)
        self.recent_k = torch.zeros((batch, hkv, params.recent, d), dtype=torch.int16, device=device)
        self.recent_v = torch.zeros_like(self.recent_k)
        alloc = torch.zeros if zero_pages else torch.empty
        self.pages = alloc((max(self.n_pages, 1), hkv, PAGE_BYTES), dtype=torch.uint8, device=device)
        self.seq_lens = torch.zeros(batch, dtype=torch.int32, device=device)
        self.error_flags = torch.zeros(1, dtype=torch.int32, device=device)
        self.append_counters = torch.zeros(batch, dtype=torch.int32, device=device)

    def c(self) -> KVPoolC:
        return KVPoolC(_ptr(self.sink_k), _ptr(self.sink_v), _ptr(self.recent_k), _ptr(self.recent_v),
                       _ptr(self.pages), _ptr(self.block_table), _ptr(self.sink_slot), _ptr(self.seq_lens),
                       _ptr(self.error_flags), _ptr(self.append_counters), self.batch, self.max_pages,
                       self.n_pages, self.n_sink_slots)

    def c_seq(self, b: int) -> KVPoolC:
        """The same pool seen as a batch of one: sequence b alone."""
        c = self.c()
        c.recent_k = _ptr(self.recent_k[b])
        c.recent_v = _ptr(self.recent_v[b])
        c.block_table = _ptr(self.block_table[b])
        c.sink_slot = _ptr(self.sink_slot[b:b + 1])
        c.seq_lens = _ptr(self.seq_lens[b:b + 1])
        c.append_counters = _ptr(self.append_counters[b:b + 1])
        c.batch = 1
        return c


def quantize_append(params: Params, rot: RotationTensors, pool: KVPool, k_new, v_new, stream=None,
                    seq: Optional[int] = None):
    """k_new, v_new: bf16 bit patterns (int16/uint16 tensor) [B, n_new, Hkv, d] on the device.

    With ``seq`` set, appends to that sequence only and k_new/v_new have batch 1.
    """
    assert k_new.is_contiguous() and v_new.is_contiguous() and k_new.shape == v_new.shape
    assert k_new.dim() == 4 and k_new.element_size() == 2
    assert k_new.shape[0] == (1 if seq is not None else pool.batch)
    n_new = int(k_new.shape[1])
    r, pc = rot.c(), (pool.c() if seq is None else pool.c_seq(seq))
    _check(lib().oscar_quantize_append(ctypes.byref(params), ctypes.byref(r), ctypes.byref(pc),
                                       _ptr(k_new), _ptr(v_new), n_new, _stream_ptr(stream)))


def decode_options(variant: int = 0, blocks: int = 0, prefix_pages: int = 0) -> DecodeOptions:
    """Per-call decode choices (see oscar_decode_options in include/oscar.h)."""
    return DecodeOptions(int(variant), int(blocks), int(prefix_pages))


def decode_workspace_size(params: Params, batch: int, max_pages: int, variant: int = 0, blocks: int = 0,
                          prefix_pages: int = 0) -> int:
    opts = decode_options(variant, blocks, prefix_pages)
    return int(lib().oscar_decode_workspace_size(ctypes.byref(params), batch, max_pages, ctypes.byref(opts)))


def alloc_workspace(nbytes: int, device="cuda"):
    """Zero-filled device workspace (the decode's completion counters start at zero)."""
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def decode_attention(params: Params, rot: RotationTensors, pool: KVPool, q, out, workspace, stream=None,
                     variant: int = 0, blocks: int = 0, prefix_pages: int = 0):
    """q: bf16 bits [B, Hq, d]; out: float32 [B, Hq, d]; workspace: uint8 device tensor
    sized by decode_workspace_size with the same options."""
    assert q.is_contiguous() and out.is_contiguous() and q.element_size() == 2
    r, pc = rot.c(), pool.c()
    opts = decode_options(variant, blocks, prefix_pages)
    _check(lib().oscar_decode_attention(ctypes.byref(params), ctypes.byref(r), ctypes.byref(pc), _ptr(q),
                                        _ptr(out), ctypes.byref(opts), _ptr(workspace), workspace.numel(),
                                        _stream_ptr(stream)))


def decode_attention_noalloc(params: Params, rot: RotationTensors, pool: KVPool, q, out, stream=None,
                             variant: int = 0, blocks: int = 0, prefix_pages: int = 0):
    """As decode_attention, on the library's own per-GPU buffer instead of a
    workspace (no allocation; calls that overlap on one GPU race)."""
    assert q.is_contiguous() and out.is_contiguous() and q.element_size() == 2
    r, pc = rot.c(), pool.c()
    opts = decode_options(variant, blocks, prefix_pages)
    _check(lib().oscar_decode_attention_noalloc(ctypes.byref(params), ctypes.byref(r), ctypes.byref(pc), _ptr(q),
                                                _ptr(out), ctypes.byref(opts), _stream_ptr(stream)))


class Bf16Cache:
    """Paged all-BF16 cache for the baseline decode (bf16 bits as int16)."""

    def __init__(self, params: Params, batch: int, n_pages: int, block_table, device="cuda"):
        import torch
        hkv, d = params.num_kv_heads, params.head_dim
        self.batch = batch
        self.block_table = torch.as_tensor(np.asarray(block_table, dtype=np.int32)).to(device).contiguous()
        self.max_pages = int(self.block_table.shape[1])
        self.n_pages = int(n_pages)
        self.k_pages = torch.zeros((max(n_pages, 1), hkv, PAGE_TOKENS, d), dtype=torch.int16, device=device)
        self.v_pages = torch.zeros_like(self.k_pages)
        self.seq_lens = torch.zeros(batch, dtype=torch.int32, device=device)
        self.error_flags = torch.zeros(1, dtype=torch.int32, device=device)

    def c(self) -> Bf16CacheC:
        return Bf16CacheC(_ptr(self.k_pages), _ptr(self.v_pages), _ptr(self.block_table), _ptr(self.seq_lens),
                          _ptr(self.error_flags), self.batch, self.max_pages, self.n_pages)


def bf16_workspace_size(params: Params, batch: int, max_pages: int) -> int:
    return int(lib().oscar_bf16_decode_workspace_size(ctypes.byref(params), batch, max_pages))


def bf16_decode_attention(params: Params, cache: Bf16Cache, q, out, workspace, stream=None):
    cc = cache.c()
    _check(lib().oscar_bf16_decode_attention(ctypes.byref(params), ctypes.byref(cc), _ptr(q), _ptr(out),
                                             _ptr(workspace), workspace.numel(), _stream_ptr(stream)))
