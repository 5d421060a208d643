"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (MFMA history scan, default grid).

The oracle cannot redo a whole 100K-token batch, so it recomputes sampled
(sequence, KV head) pairs one by one from the same seeded tokens:

- their INT2 history codes and 8-bit scale/zero codes must be bit-exact;
- the outputs of the pair's G query heads must be within
  2e-3 * ||o||_2 (max-abs).

The rotation artifact fed to both sides comes from the oracle's own
calibration (2048 calibration tokens per head).
"""
import numpy as np
import pytest

from bit_rotated_kv_int2_amd import oscar as O
from bit_rotated_kv_int2_amd import synth
from oracle import oscar_ref as R
from pool_helpers import decode_check, gather_history, oracle_calibration, rotation_tensors

pytestmark = pytest.mark.gpu
D = 128
TOL = 2e-3


def _f64(t):
    """int16 torch tensor of bf16 bits -> float64 numpy."""
    return synth.bf16_bits_to_f32(t.cpu().numpy().view(np.uint16)).astype(np.float64)


def _build_pool(wl, lengths, cals, extra_tokens=0):
    """GPU pool of one layer, filled by one bulk append per sequence."""
    import torch
    params = O.make_params(wl.n_kv, wl.n_q)
    rot = rotation_tensors(cals)
    bt, total = synth.block_table(wl, lengths, extra_tokens)
    if wl.shared_prefix:
        pool = O.KVPool(params, wl.batch, total, bt, sink_slot=np.zeros(wl.batch, np.int32), n_sink_slots=1)
    else:
        pool = O.KVPool(params, wl.batch, total, bt)
    for b in range(wl.batch):
        k, v = synth.gpu_sequence_kv(wl, 0, b, int(lengths[b]))
        O.quantize_append(params, rot, pool, k[None], v[None], seq=b)
        del k, v
    torch.cuda.synchronize()
    assert int(pool.error_flags.item()) == 0
    return params, rot, pool, bt


def _decode(params, rot, pool, q_bits, prefix_pages=0):
    import torch
    ws = O.alloc_workspace(O.decode_workspace_size(params, pool.batch, pool.max_pages, prefix_pages=prefix_pages))
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().contiguous()
    out = torch.zeros((pool.batch, params.num_q_heads, D), dtype=torch.float32, device="cuda")
    O.decode_attention(params, rot, pool, q, out, ws, prefix_pages=prefix_pages)
    torch.cuda.synchronize()
    assert int(pool.error_flags.item()) == 0
    return out.cpu().numpy()


def _check_pair(wl, cals, pool, bt, b, h, L, q_bits, out_gpu, k_all=None, v_all=None):
    """Oracle recomputation of sequence b, KV head h (L tokens)."""
    G = wl.n_q // wl.n_kv
    if k_all is None:
        k_all, v_all = synth.gpu_sequence_kv(wl, 0, b, L)
    kh, vh = _f64(k_all[:, h]), _f64(v_all[:, h])
    ref_pool = R.build_head_pool(kh, vh, cals[h])
    n_hist = max(0, L - wl.sink - wl.recent)
    if n_hist:
        n_pg = (n_hist + 63) // 64
        ids = bt[b, :n_pg].astype(np.int64)
        import torch
        pages = pool.pages[torch.from_numpy(ids).cuda(), h].cpu().numpy()[:, None]   # [n_pg, 1, 4608]
        (kc, ks, kz), (vc, vs, vz) = gather_history(pages, np.arange(n_pg), 0, n_hist)
        assert np.array_equal(kc, ref_pool.hist_k.codes), (b, h, "K codes")
        assert np.array_equal(vc, ref_pool.hist_v.codes), (b, h, "V codes")
        for got, want, what in ((ks, ref_pool.hist_k.s8, "K scale code"), (kz, ref_pool.hist_k.z8, "K zero code"),
                                (vs, ref_pool.hist_v.s8, "V scale code"), (vz, ref_pool.hist_v.z8, "V zero code")):
            assert np.array_equal(got, want), (b, h, what)
    q = synth.bf16_bits_to_f32(q_bits[b, h * G:(h + 1) * G]).astype(np.float64)
    ref = R.decode_head_dense(q, ref_pool, cals[h], 1 / np.sqrt(D))
    err = decode_check(out_gpu[b, h * G:(h + 1) * G], ref, TOL)
    assert err <= TOL, (b, h, err)
    return err


def test_qwen3_32k_one_append_one_decode():
    """Single layer, batch 1, 8 KV / 32 query heads, 32768 tokens: the pool
    holds 32767 tokens from a bulk append; the last token arrives through
    the single-token fused write (demoting one ring token); then one decode
    step.  Every KV head is checked."""
    import torch
    wl = synth.WORKLOADS["qwen3-8b-32k-b1"]
    L = wl.max_len
    cals = oracle_calibration(wl, n_cal=2048)
    params, rot, pool, bt = _build_pool(wl, np.array([L - 1], np.int32), cals, extra_tokens=1)
    k, v = synth.gpu_sequence_kv(wl, 0, 0, L)
    O.quantize_append(params, rot, pool, k[L - 1:L][None].contiguous(), v[L - 1:L][None].contiguous())
    torch.cuda.synchronize()
    assert int(pool.seq_lens[0].item()) == L and int(pool.error_flags.item()) == 0
    q = synth.decode_queries(wl, 0)
    out = _decode(params, rot, pool, q)
    errs = [_check_pair(wl, cals, pool, bt, 0, h, L, q, out, k, v) for h in range(wl.n_kv)]
    print(f"32K: max err/||o|| = {max(errs):.3e}")


def test_qwen3_100k_batch32_scattered_sampled():
    """Batch 32, lengths U[92160, 102400], pages scattered by a seeded
    permutation: three sampled (sequence, KV head) pairs."""
    wl = synth.WORKLOADS["qwen3-8b-100k-b32-36l"]
    lengths = synth.sequence_lengths(wl)
    cals = oracle_calibration(wl, n_cal=2048)
    params, rot, pool, bt = _build_pool(wl, lengths, cals)
    q = synth.decode_queries(wl, 0)
    out = _decode(params, rot, pool, q)
    assert np.all(np.isfinite(out))
    for b, h in ((0, 0), (17, 5), (31, 7)):
        err = _check_pair(wl, cals, pool, bt, b, h, int(lengths[b]), q, out)
        print(f"batch32 seq {b} kv {h} L {int(lengths[b])}: err/||o|| = {err:.3e}")


def test_qwen3_100k_batch1_sampled():
    """Batch 1 at 102400 tokens, contiguous pages: two sampled KV heads."""
    wl = synth.WORKLOADS["qwen3-8b-100k-b1-36l"]
    lengths = synth.sequence_lengths(wl)
    cals = oracle_calibration(wl, n_cal=2048)
    params, rot, pool, bt = _build_pool(wl, lengths, cals)
    q = synth.decode_queries(wl, 0)
    out = _decode(params, rot, pool, q)
    k, v = synth.gpu_sequence_kv(wl, 0, 0, int(lengths[0]))
    for h in (2, 6):
        err = _check_pair(wl, cals, pool, bt, 0, h, int(lengths[0]), q, out, k, v)
        print(f"batch1 kv {h}: err/||o|| = {err:.3e}")


def test_prefix_128k_gqa12_sampled():
    """Batch 16 at 131072 tokens, GQA 12 (96 query heads), one shared
    98304-token prefix on shared pages and sink slot: two sequences that
    share the prefix are checked, for the plain decode and for the
    shared-prefix decode (prefix_pages = 1535, as the benchmark times it),
    which must also agree with the plain one within summation order."""
    wl = synth.WORKLOADS["prefix-128k-b16-gqa12"]
    lengths = synth.sequence_lengths(wl)
    cals = oracle_calibration(wl, n_cal=2048)
    params, rot, pool, bt = _build_pool(wl, lengths, cals)
    shared = (wl.shared_prefix - wl.sink) // 64
    assert np.array_equal(bt[0, :shared], bt[9, :shared]) and shared == 1535
    q = synth.decode_queries(wl, 0)
    out = _decode(params, rot, pool, q)
    out_sh = _decode(params, rot, pool, q, prefix_pages=shared)
    for b, h in ((0, 1), (9, 4)):
        err = _check_pair(wl, cals, pool, bt, b, h, int(lengths[b]), q, out)
        print(f"prefix seq {b} kv {h}: err/||o|| = {err:.3e}")
        err = _check_pair(wl, cals, pool, bt, b, h, int(lengths[b]), q, out_sh)
        print(f"shared-prefix decode, seq {b} kv {h}: err/||o|| = {err:.3e}")
    assert decode_check(out_sh, out) <= 1e-4


def test_qwen3_100k_batch1_codebook_sampled():
    """Batch 1 at 102400 tokens with Lloyd-Max codebooks (levels calibrated
    by the oracle on the calibration tokens): the write kernels' threshold
    codes bit-exact and the level-lookup scan within tolerance, two KV
    heads."""
    wl = synth.WORKLOADS["qwen3-8b-100k-b1-36l"]
    lengths = synth.sequence_lengths(wl)
    cals = oracle_calibration(wl, n_cal=2048)
    _, kc, vc = synth.calibration_set(wl, 0, n_cal=2048)
    f = synth.bf16_bits_to_f32
    cals = [R.calibrate_codebook(c, f(kc)[h], f(vc)[h]) for h, c in enumerate(cals)]
    assert any(not np.array_equal(c.levels_K, R.UNIFORM_LEVELS) for c in cals)
    params, rot, pool, bt = _build_pool(wl, lengths, cals)
    q = synth.decode_queries(wl, 0)
    out = _decode(params, rot, pool, q)
    k, v = synth.gpu_sequence_kv(wl, 0, 0, int(lengths[0]))
    for h in (1, 5):
        err = _check_pair(wl, cals, pool, bt, 0, h, int(lengths[0]), q, out, k, v)
        print(f"batch1 codebook kv {h} levels K {cals[h].levels_K} V {cals[h].levels_V}: err/||o|| = {err:.3e}")
