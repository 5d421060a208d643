"""oscar_decode_attention_noalloc (the decode entry point that allocates
nothing) against oscar_decode_attention with a caller's workspace, through
the C ABI: the same kernels on the same inputs agree up to summation order
(the BF16 tiles go to the waves of a workgroup in the order they finish),
also on a second call in a row with a smaller input; both stay within the
2e-3 tolerance of the oracle.  Shapes past the library's buffer are refused
before any launch."""
import ctypes

import numpy as np
import pytest

from bit_rotated_kv_int2_amd import oscar as O
from bit_rotated_kv_int2_amd import synth
from oracle import oscar_ref as R
from pool_helpers import append_sequence, decode_check, oracle_calibration, rotation_tensors

pytestmark = pytest.mark.gpu
D = 128
TOL = 2e-3


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _pool(wl, lens, layer=0):
    cals = oracle_calibration(wl, layer, n_cal=256)
    rot = rotation_tensors(cals)
    params = O.make_params(wl.n_kv, wl.n_q)
    bt, total = synth.block_table(wl, lens)
    pool = O.KVPool(params, wl.batch, total, bt)
    toks = []
    for b in range(wl.batch):
        kb, vb = synth.kv_tokens(wl, layer, b, 0, int(lens[b]))
        toks.append((kb, vb))
        append_sequence(params, rot, pool, b, kb, vb)
    return cals, rot, params, pool, toks


def _both(params, rot, pool, q_bits, variant):
    import torch
    q = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).cuda()
    ws = O.alloc_workspace(O.decode_workspace_size(params, pool.batch, pool.max_pages, variant))
    a = torch.full((pool.batch, params.num_q_heads, D), float("nan"), device="cuda")
    b = torch.full_like(a, float("nan"))
    O.decode_attention(params, rot, pool, q, a, ws, variant=variant)
    O.decode_attention_noalloc(params, rot, pool, q, b, variant=variant)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


@pytest.mark.parametrize("variant", [0, 1])
def test_noalloc_matches_workspace_decode(variant):
    big = synth.Workload(130, "test-noalloc-big", 3, 2, 8, 128, 0, 5000, n_cal=256, outliers="pairs10",
                         scattered_pages=True)
    small = synth.Workload(131, "test-noalloc-small", 1, 2, 8, 128, 0, 900, n_cal=256, outliers="pairs10")
    for wl, lens in ((big, np.array([5000, 321, 2900], np.int32)), (small, np.array([900], np.int32))):
        cals, rot, params, pool, toks = _pool(wl, lens)
        q = synth.decode_queries(wl, 0)
        a, b = _both(params, rot, pool, q, variant)
        for s in range(wl.batch):
            assert decode_check(b[s], a[s]) <= 1e-5, (wl.name, variant, s)
        for s in range(wl.batch):
            pools = [R.build_head_pool(_f64(toks[s][0][:, h]), _f64(toks[s][1][:, h]), cals[h])
                     for h in range(wl.n_kv)]
            want = R.decode_sequence(_f64(q[s]), pools, cals, 1 / np.sqrt(D))
            err = decode_check(b[s], want)
            print(f"{wl.name} seq {s} variant {variant}: no-alloc err/||o|| = {err:.3e}", flush=True)
            assert err <= TOL


def test_noalloc_rejects_oversized_shapes():
    """A batch whose partials exceed the library's buffer is refused with
    OSCAR_EWORKSPACE on the host (nothing launched)."""
    params = O.make_params(8, 32)
    rot = O.Rotation(0x1000, 0x1000, 0x1000, 0x1000)
    pool = O.KVPoolC(*([0x1000] * 10), 4096, 1600, 1600, 4096)
    rc = O.lib().oscar_decode_attention_noalloc(ctypes.byref(params), ctypes.byref(rot), ctypes.byref(pool),
                                                0x1000, 0x1000, None, None)
    assert rc == O.OSCAR_EWORKSPACE
    assert b"no-alloc" in O.lib().oscar_last_error()
